// Kernel instances of the 256-thread layout (0): every load width, fp32
// and bf16 scores, with and without values.
#include "topk_instances.hpp"

namespace rrt {

const void* kernels_w256_l0(int lay, int path, int vec, bool vals, bool bf16) {
  constexpr int L = 0;
  return lay == L ? pick<L, true>(path, vec, vals, bf16) : nullptr;
}

}  // namespace rrt
