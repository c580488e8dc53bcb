// Kernel instances of the 1024-thread layout (kLayW1024): fp32 scores, every
// load width.
#include "topk_instances.hpp"

namespace rrt {

const void* kernels_w1024_l0(int lay, int path, int vec, bool vals, bool bf16) {
  constexpr int L = kLayW1024;
  return lay == L ? pick<L, false>(path, vec, vals, bf16) : nullptr;
}

}  // namespace rrt
