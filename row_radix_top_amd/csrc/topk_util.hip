// Utility kernels (workspace fill, key probe, strided packing), the
// streaming-read reference used for measurement, and the host-side lookup of
// kernel instances across the instance files.

#include "topk_kernels.hpp"

namespace rrt {

// ---------------------------------------------------------------------------
// Streaming-read reference (measurement only): the largest key of each row's
// valid prefix, read with the same tiles, load width and prefetch ring as the
// selection kernels, and no filtering.  Its rate is the ceiling the streaming
// filter can approach on the same bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t tile_max(const float (&x)[kElems], uint32_t m) {
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    const uint32_t k = ord_key(__float_as_uint(x[e]));
    m = k > m ? k : m;
  }
  return m;
}

constexpr int kRefBlock = 256;  // threads per workgroup of the read reference

template <int VEC, typename T>
__global__ void __launch_bounds__(kRefBlock) read_ref_kernel(KernelParams p) {
  constexpr int NT = kRefBlock;
  constexpr int kWaves = NT / 64;
  constexpr uint32_t kTile = NT * kElems;
  __shared__ uint32_t wmax[kWaves];
  constexpr int PF = kPrefetch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int row = blockIdx.x; row < p.num_rows; row += gridDim.x) {
    const uint32_t n = (uint32_t)clamp_len(p, row);
    const T* rowp = row_of<T>(p, row);
    const uint32_t F = n / kTile;
    uint32_t m = 0;
    if (F > 0) {
      float buf[PF][kElems];
#pragma unroll
      for (int s = 0; s < PF - 1; ++s) {
        load_full<VEC>(rowp + ((uint32_t)s < F ? (uint32_t)s : F - 1) * kTile, buf[s]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t Fr = F - F % PF;
      for (uint32_t j0 = 0; j0 < Fr; j0 += PF) {
#pragma unroll
        for (int slot = 0; slot < PF; ++slot) {
          const uint32_t j = j0 + slot;
          const uint32_t jn = j + PF - 1 < F ? j + PF - 1 : F - 1;
          load_full<VEC>(rowp + jn * kTile, buf[(slot + PF - 1) % PF]);
          __builtin_amdgcn_sched_barrier(0);
          m = tile_max(buf[slot], m);
        }
      }
#pragma unroll
      for (int slot = 0; slot < PF - 1; ++slot)
        if (Fr + slot < F) m = tile_max(buf[slot], m);
    }
    const uint32_t pt = F * kTile;
    if (pt < n) {
      float x[kElems];
      load_tail<VEC>(rowp, n, pt, x);
#pragma unroll
      for (int u = 0; u < kElems / VEC; ++u)
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
          const uint32_t pos = tile_pbase(pt, VEC) + (uint32_t)u * (64u * VEC) + c;
          const uint32_t k = ord_key(__float_as_uint(x[u * VEC + c]));
          if (pos < n && k > m) m = k;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, off);
      m = o > m ? o : m;
    }
    if (lane == 0) wmax[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t r = wmax[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) r = wmax[i] > r ? wmax[i] : r;
      reinterpret_cast<uint32_t*>(p.out)[row] = r;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Small utility kernels
// ---------------------------------------------------------------------------

__global__ void zero_kernel(uint32_t* p, uint64_t words) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

// Packs rows with a column stride into contiguous rows of num_cols:
// packed[r * num_cols + c] = scores[r * row_stride + c * col_stride] for
// c < clamp(lengths[r], 0, num_cols).  Nothing at or past a length is read
// or written.  Tiles of 64 rows x 64 columns go through LDS: loaded with the
// lanes along whichever of rows and columns is closer in memory (a
// transposed view reads consecutive addresses), written with the lanes
// along the packed rows.
constexpr int kPackTile = 64;

__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                   int64_t col_stride, int64_t num_cols,
                                                   const int32_t* __restrict__ lengths, int32_t num_rows,
                                                   float* __restrict__ packed) {
  __shared__ float tile[kPackTile][kPackTile + 1];  // [column][row]
  __shared__ int32_t len[kPackTile];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t tiles_r = (num_rows + kPackTile - 1) / kPackTile;
  const int64_t tiles_c = (num_cols + kPackTile - 1) / kPackTile;
  const bool rows_close = row_stride < col_stride;
  for (int64_t tt = blockIdx.x; tt < tiles_r * tiles_c; tt += gridDim.x) {
    const int64_t r0 = (tt % tiles_r) * kPackTile, c0 = (tt / tiles_r) * kPackTile;
    if (threadIdx.x < kPackTile) {
      const int64_t r = r0 + threadIdx.x;
      int64_t n = r < num_rows ? lengths[r] : 0;
      n = n < 0 ? 0 : (n > num_cols ? num_cols : n);
      len[threadIdx.x] = (int32_t)(n > c0 ? (n - c0 < kPackTile ? n - c0 : kPackTile) : 0);
    }
    __syncthreads();
    if (rows_close) {
      for (int cc = w; cc < kPackTile; cc += 4)
        if (cc < len[lane]) tile[cc][lane] = scores[(r0 + lane) * row_stride + (c0 + cc) * col_stride];
    } else {
      for (int rr = w; rr < kPackTile; rr += 4)
        if (lane < len[rr]) tile[lane][rr] = scores[(r0 + rr) * row_stride + (c0 + lane) * col_stride];
    }
    __syncthreads();
    for (int rr = w; rr < kPackTile; rr += 4)
      if (lane < len[rr]) packed[(r0 + rr) * num_cols + c0 + lane] = tile[lane][rr];
    __syncthreads();  // the tile and lengths are reused
  }
}

__global__ void keys_kernel(const uint32_t* bits, uint32_t* keys, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) keys[i] = ord_key(bits[i]);
}


// ---------------------------------------------------------------------------
// Instance lookup
// ---------------------------------------------------------------------------

const void* read_ref_kernel_ptr(int vec) {
  if (vec == 4) return reinterpret_cast<const void*>(&read_ref_kernel<4, float>);
  if (vec == 2) return reinterpret_cast<const void*>(&read_ref_kernel<2, float>);
  return reinterpret_cast<const void*>(&read_ref_kernel<1, float>);
}

const void* kernel_ptr(int path, int vec, bool idx16, bool vals, bool bf16, bool big_k, int block) {
  if (path == 3) return read_ref_kernel_ptr(vec);
  if (!has_block(block, bf16)) return nullptr;
  const int lay = layout_of(idx16, big_k, block);
  switch (block) {
    case 1024:
      switch (lay & (kLayIdx16 | kLayBigK)) {
        case kLayIdx16: return kernels_w1024_l1(lay, path, vec, vals, bf16);
        case kLayBigK: return kernels_w1024_l2(lay, path, vec, vals, bf16);
        case kLayIdx16 | kLayBigK: return kernels_w1024_l3(lay, path, vec, vals, bf16);
        default: return kernels_w1024_l0(lay, path, vec, vals, bf16);
      }
    case 512: return idx16 ? kernels_w512_i16(lay, path, vec, vals, bf16) : kernels_w512_i32(lay, path, vec, vals, bf16);
    default:
      switch (lay) {
        case kLayIdx16: return kernels_w256_l1(lay, path, vec, vals, bf16);
        case kLayBigK: return kernels_w256_l2(lay, path, vec, vals, bf16);
        case kLayIdx16 | kLayBigK: return kernels_w256_l3(lay, path, vec, vals, bf16);
        default: return kernels_w256_l0(lay, path, vec, vals, bf16);
      }
  }
}

template <int LAY>
static int lds_of() {
  return (int)sizeof(Smem<LAY>);
}

int lds_bytes_of(bool idx16, bool big_k, int block) {
  switch (layout_of(idx16, big_k, block)) {
    case 0: return lds_of<0>();
    case kLayIdx16: return lds_of<kLayIdx16>();
    case kLayBigK: return lds_of<kLayBigK>();
    case kLayIdx16 | kLayBigK: return lds_of<kLayIdx16 | kLayBigK>();
    case kLayW512: return lds_of<kLayW512>();
    case kLayW512 | kLayIdx16: return lds_of<kLayW512 | kLayIdx16>();
    case kLayW512 | kLayBigK: return lds_of<kLayW512 | kLayBigK>();
    case kLayW512 | kLayIdx16 | kLayBigK: return lds_of<kLayW512 | kLayIdx16 | kLayBigK>();
    case kLayW1024: return lds_of<kLayW1024>();
    case kLayW1024 | kLayIdx16: return lds_of<kLayW1024 | kLayIdx16>();
    case kLayW1024 | kLayBigK: return lds_of<kLayW1024 | kLayBigK>();
    default: return lds_of<kLayW1024 | kLayIdx16 | kLayBigK>();
  }
}

const void* zero_kernel_ptr() { return reinterpret_cast<const void*>(&zero_kernel); }
const void* keys_kernel_ptr() { return reinterpret_cast<const void*>(&keys_kernel); }
const void* pack_kernel_ptr() { return reinterpret_cast<const void*>(&pack_kernel); }

}  // namespace rrt
