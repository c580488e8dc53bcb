// Kernel instance tables: each instance file includes this header and
// compiles the kernels of a few buffer layouts, so that the files build in
// parallel.  pick<LAY, BF16>() returns the instance for a path, load width
// and values flag, or nullptr when the combination is not compiled.
#pragma once

#include "topk_kernels.hpp"

namespace rrt {

template <int VEC, int LAY, typename T>
static const void* pick_vec(int path, bool vals) {
  if (path == 2) return reinterpret_cast<const void*>(&topk_multi_kernel<VEC, LAY, T>);
  if (path != 1) return nullptr;
  if (vals) return reinterpret_cast<const void*>(&topk_single_kernel<VEC, LAY, true, T>);
  return reinterpret_cast<const void*>(&topk_single_kernel<VEC, LAY, false, T>);
}

// BF16: whether this file also compiles the bf16 instances of the layout.
template <int LAY, bool BF16>
static const void* pick(int path, int vec, bool vals, bool bf16) {
  if (bf16) {
    if constexpr (BF16)
      return vec == 8 ? pick_vec<8, LAY, uint16_t>(path, vals) : vec == 1 ? pick_vec<1, LAY, uint16_t>(path, vals)
                                                                          : nullptr;
    return nullptr;
  }
  if (vec == 4) return pick_vec<4, LAY, float>(path, vals);
  if (vec == 2) return pick_vec<2, LAY, float>(path, vals);
  if (vec == 1) return pick_vec<1, LAY, float>(path, vals);
  return nullptr;
}

}  // namespace rrt
