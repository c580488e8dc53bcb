// gfx950 kernels for ragged per-row top-K.
//
// What is computed (vLLM persistent_topk pages; PR #54110 page, topk.cu
// excerpt; PR #41189 page, topk.cu excerpt): for each row, the indices of the
// K largest fp32 scores among the first lengths[row] entries, ties to the
// lower index, written in ascending index order, -1 padded.
//
// Design (not the pages' CUDA design, which is prior art):
//
// * Streaming filter.  A workgroup walks its row (or its chunk of a row) once,
//   in 2048-element tiles of coalesced vector loads.  It keeps an
//   index-ordered candidate buffer in LDS and a lower bound L on the key of
//   the K-th best element seen so far; an element is appended only if its key
//   is >= L.  When a tile would overflow the buffer, the buffer is compacted
//   to exactly its K best entries (radix select below) and L rises to just
//   above the K-th best key.  Later elements equal to that key can never win
//   (every kept entry has a lower index), so the buffer never fills with
//   ties.  Each score is read from HBM exactly once.
//
// * Radix select in LDS.  The buffer is held in registers (cap/256 entries per
//   thread) while 11/11/10-bit digit histograms are built with LDS atomics;
//   one wavefront scans each histogram from the top with a lane prefix scan
//   to find the threshold digit.  Ties at the final 32-bit key go to the
//   lower buffer position, which is the lower index.
//
// * Ordered emit.  Wavefront ballots and mbcnt give each lane its rank inside
//   the wave; per-wave counts exchanged through LDS give the rest.  Output is
//   written in ascending index order with no sort.
//
// * Multi-workgroup rows.  G workgroups each filter a contiguous chunk, then
//   merge digit histograms in the workspace with agent-scope atomics across
//   three cooperative rounds (an arrival-counter barrier each), publish the
//   few keys left undecided after 22 bits, and derive their output offsets
//   from per-workgroup counts.  The last workgroup to leave zeroes everything
//   the row touched, so the workspace is all-zero when the kernel ends (the
//   in-kernel cleanup of the PR #41748 page, without the race its review
//   describes: nothing is reset while another workgroup can still read it).
//
// The key function maps fp32 bits to uint32 so that unsigned order equals
// IEEE order for non-NaN values, with -0.0 and +0.0 mapped to the same key.
// Everything on the selection path is integer or bit manipulation except the
// streaming compare x >= f(L), an exact IEEE comparison (denormals are kept:
// the library is built without flush-to-zero).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_internal.h"

namespace rrt {

// ---------------------------------------------------------------------------
// Bit-level helpers
// ---------------------------------------------------------------------------

// Order-preserving key: negative floats -> ~bits, non-negative -> bits | sign.
// -0.0 (0x80000000) is first mapped to +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t ord_key(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose key is L: {x : x >= key_floor(L)} == {x : key(x) >= L} for
// non-NaN x and any L >= 0x00800000 (below that the float is a NaN and the
// caller accepts everything instead).
__device__ __forceinline__ float key_floor(uint32_t L) {
  const uint32_t u = (L & 0x80000000u) ? (L & 0x7fffffffu) : ~L;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Shared memory of one workgroup
// ---------------------------------------------------------------------------

template <int KMAX>
struct Shape {
  static constexpr int kCap = cap_of(KMAX);
  static constexpr int kSlots = kCap / kBlock;  // buffer entries per thread in registers
  static_assert(kCap % kBlock == 0, "capacity must tile the workgroup");
  static_assert(kCap < 65536, "packed 16-bit counts");
};

template <int KMAX>
struct __align__(16) Smem {
  uint32_t key[Shape<KMAX>::kCap];
  uint32_t idx[Shape<KMAX>::kCap];
  uint32_t hist[kBins];
  uint32_t tile_cnt[2][kElems][kWaves];
  uint32_t rank_cnt[Shape<KMAX>::kSlots][kWaves];
  uint32_t res[4];
  uint32_t acc[8];
};

// ---------------------------------------------------------------------------
// Threshold search: wavefront 0 finds the bin holding the krem-th largest
// entry, counting down from the top bin, then leaves the histogram zeroed.
// res = {bin, entries in bins above it, entries in the bin, ok}.  Kept out of
// line: inlined, its rotated LDS addresses are hoisted out of the row loop
// and pinned in registers for the whole kernel.
// ---------------------------------------------------------------------------
template <int NB>
__device__ __noinline__ void wave_search(uint32_t* hist, uint32_t krem, uint32_t* res) {
  constexpr int kPer = NB / 64;
  const int lane = threadIdx.x & 63;
  const int q = 63 - lane;  // lane 0 owns the highest group of bins
  uint32_t* grp = hist + q * kPer;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) s += grp[(i + lane) & (kPer - 1)];  // rotated: no bank conflicts
  const uint32_t incl = wave_incl_scan(s);
  const uint32_t excl = incl - s;
  if (incl >= krem && excl < krem) {
    uint32_t acc = excl;
    for (int i = kPer - 1; i >= 0; --i) {
      const uint32_t v = grp[i];
      if (acc + v >= krem) {
        res[0] = (uint32_t)(q * kPer + i);
        res[1] = acc;
        res[2] = v;
        res[3] = 1u;
        break;
      }
      acc += v;
    }
  }
  const uint32_t total = __shfl(incl, 63, 64);
  if (lane == 0 && total < krem) {
    res[0] = 0u;
    res[1] = 0u;
    res[2] = total;
    res[3] = 0u;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) grp[(i + lane) & (kPer - 1)] = 0u;
}

struct Sel {
  uint32_t prefix;  // decided key bits
  uint32_t pmask;   // which bits are decided
  uint32_t krem;    // entries equal to prefix (under pmask) still to take, lowest position first
  uint32_t ok;
};

// Radix select over the register-held buffer: the keep best entries are those
// with (key & pmask) > prefix, plus the first krem (by position) with
// (key & pmask) == prefix.  Requires keep <= number of valid entries.
template <int KMAX>
__device__ Sel radix_select(Smem<KMAX>& sm, const uint32_t (&k)[Shape<KMAX>::kSlots], uint32_t cnt,
                            uint32_t keep) {
  constexpr int S = Shape<KMAX>::kSlots;
  const int t = threadIdx.x;
  Sel r{0u, 0u, keep, 1u};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const uint32_t p = (uint32_t)(t + j * kBlock);
      if (p < cnt && (k[j] & r.pmask) == r.prefix) atomicAdd(&sm.hist[(k[j] >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (t < 64) {
      if (pass == 2)
        wave_search<1024>(sm.hist, r.krem, sm.res);
      else
        wave_search<2048>(sm.hist, r.krem, sm.res);
    }
    __syncthreads();
    const uint32_t b = sm.res[0], above = sm.res[1], in_bin = sm.res[2];
    r.ok &= sm.res[3];
    r.krem -= above;
    r.prefix |= b << shift;
    r.pmask |= dmask << shift;
    if (in_bin == r.krem) break;  // every entry of the bin is taken: no further digit needed
  }
  return r;
}

// Ordered emit of the entries chosen by s.  An entry's rank counts chosen
// entries before it in buffer order; gt_base / eq_base add counts from
// earlier chunks of the row (multi path); take_eq bounds the row-wide number
// of entries equal to the prefix that are taken.  Writes idx to out[rank]
// when out != nullptr, otherwise (key, idx) back to the LDS buffer.  Ranks at
// or above limit are dropped (only reachable with an inconsistent workspace).
// Flags are recomputed after the barrier rather than kept live across it.
template <int KMAX>
__device__ void ordered_emit(Smem<KMAX>& sm, const uint32_t (&k)[Shape<KMAX>::kSlots],
                             const uint32_t (&ix)[Shape<KMAX>::kSlots], uint32_t cnt, const Sel& s,
                             uint32_t gt_base, uint32_t eq_base, uint32_t take_eq, int32_t* out,
                             uint32_t limit) {
  constexpr int S = Shape<KMAX>::kSlots;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = (uint32_t)(t + j * kBlock) < cnt;
    const uint32_t km = k[j] & s.pmask;
    const uint32_t cg = popc64(ballot(valid && km > s.prefix));
    const uint32_t ce = popc64(ballot(valid && km == s.prefix));
    if (lane == 0) sm.rank_cnt[j][w] = cg | (ce << 16);
  }
  __syncthreads();
  uint32_t run = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = (uint32_t)(t + j * kBlock) < cnt;
    const uint32_t km = k[j] & s.pmask;
    const bool gt = valid && km > s.prefix;
    const bool eq = valid && km == s.prefix;
    const uint32_t pg = lanes_below(ballot(gt));
    const uint32_t pe = lanes_below(ballot(eq));
    const uint4 v = *reinterpret_cast<const uint4*>(sm.rank_cnt[j]);
    const uint32_t before = (w > 0 ? v.x : 0u) + (w > 1 ? v.y : 0u) + (w > 2 ? v.z : 0u);
    const uint32_t base = run + before;
    run += v.x + v.y + v.z + v.w;
    const uint32_t gtb = gt_base + (base & 0xffffu) + pg;
    const uint32_t eqb = eq_base + (base >> 16) + pe;
    if (gt || (eq && eqb < take_eq)) {
      const uint32_t pos = gtb + (eqb < take_eq ? eqb : take_eq);
      if (pos < limit) {
        if (out != nullptr) {
          out[pos] = (int32_t)ix[j];
        } else {
          sm.key[pos] = k[j];
          sm.idx[pos] = ix[j];
        }
      }
    }
  }
}

template <int KMAX>
__device__ __forceinline__ void load_buffer(const Smem<KMAX>& sm, uint32_t cnt,
                                            uint32_t (&k)[Shape<KMAX>::kSlots],
                                            uint32_t (&ix)[Shape<KMAX>::kSlots]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < Shape<KMAX>::kSlots; ++j) {
    const uint32_t p = (uint32_t)(t + j * kBlock);
    k[j] = p < cnt ? sm.key[p] : 0u;
    ix[j] = p < cnt ? sm.idx[p] : 0u;
  }
}

// Compacts the LDS buffer to its keep best entries (index order kept) and
// raises the acceptance bound L.
template <int KMAX>
__device__ void compact(Smem<KMAX>& sm, uint32_t& cnt, uint32_t keep, uint32_t& L) {
  constexpr int S = Shape<KMAX>::kSlots;
  uint32_t k[S], ix[S];
  load_buffer<KMAX>(sm, cnt, k, ix);
  const Sel s = radix_select<KMAX>(sm, k, cnt, keep);
  ordered_emit<KMAX>(sm, k, ix, cnt, s, 0u, 0u, s.krem, nullptr, (uint32_t)Shape<KMAX>::kCap);
  __syncthreads();
  cnt = keep;
  // Every element still to come has a higher index than all kept entries, so
  // it must beat the K-th best key strictly to matter.  When the K-th best key
  // is known only to its top bits, accept anything from that prefix up.
  uint32_t Ln;
  if (s.pmask == 0xffffffffu)
    Ln = s.prefix == 0xffffffffu ? 0xffffffffu : s.prefix + 1u;
  else
    Ln = s.prefix;
  L = Ln > L ? Ln : L;
}

// ---------------------------------------------------------------------------
// Streaming filter over [c0, c1) of one row
// ---------------------------------------------------------------------------

template <int VEC>
__device__ __forceinline__ void load_tile(const float* __restrict__ rowp, uint32_t c1, uint32_t p0,
                                          float (&x)[kElems]) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
    const uint32_t pos = p0 + (uint32_t)u * (kBlock * VEC) + t * VEC;
    if (pos + VEC <= c1) {
      if constexpr (VEC == 4) {
        const float4 v = *reinterpret_cast<const float4*>(rowp + pos);
        x[u * 4 + 0] = v.x;
        x[u * 4 + 1] = v.y;
        x[u * 4 + 2] = v.z;
        x[u * 4 + 3] = v.w;
      } else if constexpr (VEC == 2) {
        const float2 v = *reinterpret_cast<const float2*>(rowp + pos);
        x[u * 2 + 0] = v.x;
        x[u * 2 + 1] = v.y;
      } else {
        x[u] = rowp[pos];
      }
    } else {
#pragma unroll
      for (int c = 0; c < VEC; ++c) x[u * VEC + c] = (pos + c < c1) ? rowp[pos + c] : 0.0f;
    }
  }
}

// Bit e of the result: element e of this thread's tile slice is in range and
// passes the acceptance bound (key >= L, evaluated as an IEEE compare).
template <int VEC>
__device__ __forceinline__ uint32_t tile_flags(const float (&x)[kElems], uint32_t p0, uint32_t c1,
                                               uint32_t L) {
  const uint32_t t = threadIdx.x;
  const bool on = L >= 0x00800000u;
  const float bf = key_floor(L);
  uint32_t f = 0;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const uint32_t pos = p0 + (uint32_t)u * (kBlock * VEC) + t * VEC + c;
      const bool a = pos < c1 && (!on || x[u * VEC + c] >= bf);
      f |= (a ? 1u : 0u) << (u * VEC + c);
    }
  }
  return f;
}

// Per-wave counts of accepted elements for each load slot go through LDS
// (double-buffered by par); returns the tile total and each slot's offset for
// this wave.
template <int KMAX, int VEC>
__device__ __forceinline__ uint32_t tile_exchange(Smem<KMAX>& sm, uint32_t f, int& par,
                                                  uint32_t (&off)[kElems / VEC]) {
  constexpr int NL = kElems / VEC;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    uint32_t c = 0;
#pragma unroll
    for (int cc = 0; cc < VEC; ++cc) c += popc64(ballot((f >> (u * VEC + cc)) & 1u));
    if (lane == 0) sm.tile_cnt[par][u][w] = c;
  }
  __syncthreads();
  uint32_t total = 0;
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const uint4 v = *reinterpret_cast<const uint4*>(sm.tile_cnt[par][u]);
    const uint32_t before = (w > 0 ? v.x : 0u) + (w > 1 ? v.y : 0u) + (w > 2 ? v.z : 0u);
    off[u] = total + before;
    total += v.x + v.y + v.z + v.w;
  }
  par ^= 1;
  return total;
}

template <int KMAX, int VEC>
__device__ void stream_chunk(Smem<KMAX>& sm, const float* __restrict__ rowp, uint32_t c0, uint32_t c1,
                             uint32_t keep, uint32_t& cnt, uint32_t& L) {
  constexpr int NL = kElems / VEC;
  const uint32_t t = threadIdx.x;
  int par = 0;
  float xa[kElems], xb[kElems];
  load_tile<VEC>(rowp, c1, c0, xa);
  for (uint32_t p0 = c0; p0 < c1; p0 += kTile) {
    const bool more = p0 + kTile < c1;
    if (more) load_tile<VEC>(rowp, c1, p0 + kTile, xb);
    uint32_t off[NL];
    uint32_t f = tile_flags<VEC>(xa, p0, c1, L);
    uint32_t total = tile_exchange<KMAX, VEC>(sm, f, par, off);
    if (cnt + total > (uint32_t)Shape<KMAX>::kCap) {
      compact<KMAX>(sm, cnt, keep, L);
      f = tile_flags<VEC>(xa, p0, c1, L);
      total = tile_exchange<KMAX, VEC>(sm, f, par, off);
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      uint32_t r = cnt + off[u];
#pragma unroll
      for (int c = 0; c < VEC; ++c) r += lanes_below(ballot((f >> (u * VEC + c)) & 1u));
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const int e = u * VEC + c;
        if ((f >> e) & 1u) {
          sm.key[r] = ord_key(__float_as_uint(xa[e]));
          sm.idx[r] = p0 + (uint32_t)u * (kBlock * VEC) + t * VEC + c;
          ++r;
        }
      }
    }
    cnt += total;
    if (more) {
#pragma unroll
      for (int e = 0; e < kElems; ++e) xa[e] = xb[e];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int64_t clamp_len(const KernelParams& p, int row) {
  int64_t n = p.lengths[row];
  n = n < 0 ? 0 : n;
  return n > p.row_stride ? p.row_stride : n;
}

// n <= K: every valid index, then -1.  Reads no scores.
__device__ __forceinline__ void write_all_then_pad(int32_t* out, int64_t n, int K) {
  for (int i = threadIdx.x; i < K; i += kBlock) out[i] = i < n ? i : -1;
}

// ---------------------------------------------------------------------------
// One workgroup per row, persistent over rows.
// ---------------------------------------------------------------------------
template <int KMAX, int VEC>
__global__ void __launch_bounds__(kBlock) topk_single_kernel(KernelParams p) {
  __shared__ Smem<KMAX> sm;
  constexpr int S = Shape<KMAX>::kSlots;
  const int t = threadIdx.x;
  for (int i = t; i < kBins; i += kBlock) sm.hist[i] = 0u;
  __syncthreads();
  const uint32_t K = (uint32_t)p.K;
  for (int row = blockIdx.x; row < p.num_rows; row += gridDim.x) {
    const int64_t n = clamp_len(p, row);
    int32_t* out = p.out + (int64_t)row * p.K;
    if (n <= (int64_t)K) {
      write_all_then_pad(out, n, p.K);
      continue;
    }
    const float* rowp = p.scores + (int64_t)row * p.row_stride;
    uint32_t cnt = 0, L = 0;
    stream_chunk<KMAX, VEC>(sm, rowp, 0u, (uint32_t)n, K, cnt, L);
    uint32_t k[S], ix[S];
    load_buffer<KMAX>(sm, cnt, k, ix);
    const Sel s = radix_select<KMAX>(sm, k, cnt, K);
    ordered_emit<KMAX>(sm, k, ix, cnt, s, 0u, 0u, s.krem, out, K);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Several workgroups per row, cooperating through the workspace.
// ---------------------------------------------------------------------------

// Arrival barrier of the workgroups sharing a row.  Every thread publishes
// its global writes at agent scope, one thread arrives and polls, everyone
// acquires.  A wait that exceeds spin_limit polls sets an error bit and
// returns, so no wave can wait forever.
__device__ void group_barrier(uint32_t* ctr, uint32_t target, uint32_t spin_limit, uint32_t* err) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t polls = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++polls > spin_limit) {
        __hip_atomic_fetch_or(err, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Adds the LDS histogram into a workspace histogram (non-zero bins only) and
// zeroes the LDS copy.
__device__ __forceinline__ void merge_hist(uint32_t* lds_hist, uint32_t* gh) {
  for (int i = threadIdx.x; i < kBins; i += kBlock) {
    const uint32_t v = lds_hist[i];
    if (v) {
      __hip_atomic_fetch_add(gh + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_hist[i] = 0u;
    }
  }
}

__device__ __forceinline__ void load_hist(uint32_t* lds_hist, const uint32_t* gh) {
  for (int i = threadIdx.x; i < kBins; i += kBlock) lds_hist[i] = gh[i];
}

// Adds a wave-uniform count into an LDS accumulator (one lane per wave).
__device__ __forceinline__ void wave_add(uint32_t* acc, uint32_t v) {
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(acc, v);
}

template <int KMAX, int VEC>
__global__ void __launch_bounds__(kBlock) topk_multi_kernel(KernelParams p) {
  __shared__ Smem<KMAX> sm;
  constexpr int S = Shape<KMAX>::kSlots;
  constexpr int CAP = Shape<KMAX>::kCap;
  const int t = threadIdx.x, lane = t & 63;
  const int G = p.wg_per_row;
  const int row = blockIdx.x / G;
  const int g = blockIdx.x - row * G;
  if (row >= p.num_rows) return;
  const uint32_t K = (uint32_t)p.K;
  const int64_t n = clamp_len(p, row);
  int32_t* out = p.out + (int64_t)row * p.K;
  if (n <= (int64_t)K) {
    if (g == 0) write_all_then_pad(out, n, p.K);
    return;
  }
  const int grow = (int)((n + p.chunk - 1) / p.chunk);  // workgroups with data in this row
  if (g >= grow) return;

  uint32_t* err = reinterpret_cast<uint32_t*>(p.ws);
  const GroupLayout lay = group_layout(G, CAP);
  uint8_t* blk = p.ws + kWsHeader + (uint64_t)row * p.group_bytes;
  uint32_t* ctr = reinterpret_cast<uint32_t*>(blk);
  uint32_t* exit_ctr = reinterpret_cast<uint32_t*>(blk + 128);
  uint32_t* slots = reinterpret_cast<uint32_t*>(blk + lay.slots);
  uint32_t* h1 = reinterpret_cast<uint32_t*>(blk + lay.h1);
  uint32_t* h2 = reinterpret_cast<uint32_t*>(blk + lay.h2);
  uint32_t* lists = reinterpret_cast<uint32_t*>(blk + lay.lists);

  for (int i = t; i < kBins; i += kBlock) sm.hist[i] = 0u;
  if (t < 8) sm.acc[t] = 0u;
  __syncthreads();

  const int64_t c0 = (int64_t)g * p.chunk;
  const int64_t c1 = c0 + p.chunk < n ? c0 + p.chunk : n;
  const float* rowp = p.scores + (int64_t)row * p.row_stride;
  uint32_t cnt = 0, L = 0;
  stream_chunk<KMAX, VEC>(sm, rowp, (uint32_t)c0, (uint32_t)c1, K, cnt, L);

  uint32_t k[S], ix[S];
  load_buffer<KMAX>(sm, cnt, k, ix);

  // Round 1: top 11 bits.
#pragma unroll
  for (int j = 0; j < S; ++j)
    if ((uint32_t)(t + j * kBlock) < cnt) atomicAdd(&sm.hist[k[j] >> 21], 1u);
  __syncthreads();
  merge_hist(sm.hist, h1);
  group_barrier(ctr, 1u * grow, p.spin_limit, err);
  load_hist(sm.hist, h1);
  __syncthreads();
  if (t < 64) wave_search<2048>(sm.hist, K, sm.res);
  __syncthreads();
  uint32_t ok = sm.res[3];
  uint32_t krem = K - sm.res[1];
  uint32_t prefix = sm.res[0] << 21;
  uint32_t pmask = 0xffe00000u;

  // Round 2: next 11 bits of the entries in the threshold bin; publish how
  // many of this chunk's entries lie above it.
  uint32_t n_above1 = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = (uint32_t)(t + j * kBlock) < cnt;
    const uint32_t km = k[j] & pmask;
    if (valid && km == prefix) atomicAdd(&sm.hist[(k[j] >> 10) & 2047u], 1u);
    n_above1 += popc64(ballot(valid && km > prefix));
  }
  wave_add(&sm.acc[0], n_above1);
  __syncthreads();
  merge_hist(sm.hist, h2);
  if (t == 0) slots[4 * g + 0] = sm.acc[0];
  group_barrier(ctr, 2u * grow, p.spin_limit, err);
  load_hist(sm.hist, h2);
  __syncthreads();
  if (t < 64) wave_search<2048>(sm.hist, krem, sm.res);
  __syncthreads();
  ok &= sm.res[3];
  krem -= sm.res[1];
  prefix |= sm.res[0] << 10;
  pmask = 0xfffffc00u;

  // Round 3: publish the keys still undecided after 22 bits, in index order,
  // and the count above them.
  {
    uint32_t n_above2 = 0;
    uint32_t pm[S];
    bool m[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool valid = (uint32_t)(t + j * kBlock) < cnt;
      const uint32_t km = k[j] & pmask;
      n_above2 += popc64(ballot(valid && km > prefix));
      m[j] = valid && km == prefix;
      const uint64_t mm = ballot(m[j]);
      pm[j] = lanes_below(mm);
      if (lane == 0) sm.rank_cnt[j][t >> 6] = popc64(mm);
    }
    wave_add(&sm.acc[1], n_above2);
    __syncthreads();
    const int w = t >> 6;
    uint32_t run = 0;
    uint32_t* my_list = lists + (uint64_t)g * CAP;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(sm.rank_cnt[j]);
      const uint32_t before = (w > 0 ? v.x : 0u) + (w > 1 ? v.y : 0u) + (w > 2 ? v.z : 0u);
      if (m[j]) my_list[run + before + pm[j]] = k[j];
      run += v.x + v.y + v.z + v.w;
    }
    if (t == 0) {
      slots[4 * g + 1] = sm.acc[1] - sm.acc[0];
      slots[4 * g + 2] = run;
    }
  }
  group_barrier(ctr, 3u * grow, p.spin_limit, err);

  // Last 10 bits over every chunk's list; then this chunk's offsets.
  for (int gg = 0; gg < grow; ++gg) {
    uint32_t len = slots[4 * gg + 2];
    len = len < (uint32_t)CAP ? len : (uint32_t)CAP;
    const uint32_t* lst = lists + (uint64_t)gg * CAP;
    for (uint32_t i = t; i < len; i += kBlock) atomicAdd(&sm.hist[lst[i] & 1023u], 1u);
  }
  __syncthreads();
  if (t < 64) wave_search<1024>(sm.hist, krem, sm.res);
  __syncthreads();
  ok &= sm.res[3];
  const uint32_t T = prefix | sm.res[0];
  const uint32_t take_eq = krem - sm.res[1];
  {
    uint32_t gt_b = 0, eq_b = 0;
    for (int gg = 0; gg < g; ++gg) {
      uint32_t len = slots[4 * gg + 2];
      len = len < (uint32_t)CAP ? len : (uint32_t)CAP;
      const uint32_t* lst = lists + (uint64_t)gg * CAP;
      for (uint32_t i0 = 0; i0 < len; i0 += kBlock) {
        const uint32_t i = i0 + t;
        const uint32_t v = i < len ? lst[i] : 0u;
        gt_b += popc64(ballot(i < len && v > T));
        eq_b += popc64(ballot(i < len && v == T));
      }
      if (t == 0) gt_b += slots[4 * gg + 0] + slots[4 * gg + 1];
    }
    // gt_b from lists is wave-uniform; slot counts were added on thread 0 only.
    if (lane == 0) {
      if (gt_b) atomicAdd(&sm.acc[2], gt_b);
      if (eq_b) atomicAdd(&sm.acc[3], eq_b);
    }
  }
  __syncthreads();
  const uint32_t gt_base = sm.acc[2];
  const uint32_t eq_base = sm.acc[3];

  // Leave: the last workgroup out zeroes what this row used in the workspace.
  if (t == 0) {
    const uint32_t old = __hip_atomic_fetch_add(exit_ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sm.res[0] = (old == (uint32_t)grow - 1u) ? 1u : 0u;
    if (!ok) __hip_atomic_fetch_or(err, kErrSearch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sm.res[0]) {
    for (int i = t; i < kBins; i += kBlock) {
      h1[i] = 0u;
      h2[i] = 0u;
    }
    if (t == 0) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exit_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  const Sel s{T, 0xffffffffu, take_eq, ok};
  ordered_emit<KMAX>(sm, k, ix, cnt, s, gt_base, eq_base, take_eq, out, K);
}

// ---------------------------------------------------------------------------
// Small utility kernels
// ---------------------------------------------------------------------------

__global__ void zero_kernel(uint32_t* p, uint64_t words) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

__global__ void keys_kernel(const uint32_t* bits, uint32_t* keys, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) keys[i] = ord_key(bits[i]);
}

// ---------------------------------------------------------------------------
// Instance table
// ---------------------------------------------------------------------------

template <int KMAX>
static const void* pick(int path, int vec) {
  if (path == 1) {
    if (vec == 4) return reinterpret_cast<const void*>(&topk_single_kernel<KMAX, 4>);
    if (vec == 2) return reinterpret_cast<const void*>(&topk_single_kernel<KMAX, 2>);
    return reinterpret_cast<const void*>(&topk_single_kernel<KMAX, 1>);
  }
  if (vec == 4) return reinterpret_cast<const void*>(&topk_multi_kernel<KMAX, 4>);
  if (vec == 2) return reinterpret_cast<const void*>(&topk_multi_kernel<KMAX, 2>);
  return reinterpret_cast<const void*>(&topk_multi_kernel<KMAX, 1>);
}

const void* kernel_ptr(int path, int kmax, int vec) {
  switch (kmax) {
    case 256: return pick<256>(path, vec);
    case 512: return pick<512>(path, vec);
    case 1024: return pick<1024>(path, vec);
    case 2048: return pick<2048>(path, vec);
    default: return nullptr;
  }
}

int lds_bytes_of(int path, int kmax) {
  (void)path;
  switch (kmax) {
    case 256: return (int)sizeof(Smem<256>);
    case 512: return (int)sizeof(Smem<512>);
    case 1024: return (int)sizeof(Smem<1024>);
    case 2048: return (int)sizeof(Smem<2048>);
    default: return 0;
  }
}

const void* zero_kernel_ptr() { return reinterpret_cast<const void*>(&zero_kernel); }
const void* keys_kernel_ptr() { return reinterpret_cast<const void*>(&keys_kernel); }

}  // namespace rrt
