// Kernel instances of the 512-thread layouts with 32-bit candidate indices
// (K up to 2048 and up to 4096): every load width, fp32 and bf16 scores.
#include "topk_instances.hpp"

namespace rrt {

const void* kernels_w512_i32(int lay, int path, int vec, bool vals, bool bf16) {
  constexpr int A = kLayW512, B = kLayW512 | kLayBigK;
  if (lay == A) return pick<A, true>(path, vec, vals, bf16);
  if (lay == B) return pick<B, true>(path, vec, vals, bf16);
  return nullptr;
}

}  // namespace rrt
