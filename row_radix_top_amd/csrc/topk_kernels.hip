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
//   in 2048-element tiles of coalesced vector loads kept in flight by a
//   register ring.  It keeps an index-ordered candidate buffer in LDS and a
//   lower bound L on the key of the K-th best element seen so far; an element
//   is appended only if its key is >= L, which costs one IEEE compare per
//   element.  When a tile would overflow the buffer, the buffer is compacted
//   to exactly its K best entries and L rises to just above the K-th best key.
//   Later elements equal to that key can never win (every kept entry has a
//   lower index), so the buffer never fills with ties.  Each score is read
//   from HBM exactly once.
//
// * Running histogram.  Every appended key also bumps an 11-bit (top digit)
//   LDS histogram of the buffer, so the first radix pass of every selection
//   is already done; after a compaction the histogram is corrected bin-wise
//   (bins below the threshold digit empty, the threshold bin holds the number
//   of entries kept from it).
//
// * Radix select.  Later digits (11 then 10 bits) are histogrammed with LDS
//   atomics over the register-held buffer; one wavefront scans a histogram
//   from the top with DPP prefix sums to find the threshold digit.  Ties at
//   the final 32-bit key go to the lower buffer position, the lower index.
//
// * Ordered emit.  Each thread owns a contiguous slice of the buffer; one
//   workgroup prefix sum of the per-thread (greater, equal) counts gives every
//   chosen entry its output rank, so output is written in ascending index
//   order with no sort.
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
// Bit-level and wavefront helpers
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

// Acceptance threshold as a float: x >= accept_floor(L) <=> key(x) >= L.
__device__ __forceinline__ float accept_floor(uint32_t L) {
  return L >= 0x00800000u ? key_floor(L) : -__builtin_inff();
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Pointers into LDS (address space 3), so out-of-line helpers address it with
// ds_* instructions directly.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4 lds_u4;

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS traffic).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// ---------------------------------------------------------------------------
// Shared memory of one workgroup
// ---------------------------------------------------------------------------

template <int KMAX>
struct Shape {
  static constexpr int kCap = cap_of(KMAX);
  static constexpr int kSlots = kCap / kBlock;  // buffer entries owned per thread
  static_assert(kCap % kBlock == 0 && kSlots % 4 == 0, "capacity must tile the workgroup in uint4s");
  static_assert(kCap < 65536, "packed 16-bit counts");
};

template <int KMAX>
struct __align__(16) Smem {
  uint32_t key[Shape<KMAX>::kCap];  // candidate keys, index order
  uint32_t idx[Shape<KMAX>::kCap];  // their column indices
  uint32_t hist1[kBins];            // top-digit histogram of the buffer, kept current
  uint32_t hist2[kBins];            // scratch histogram for later digits (zero between uses)
  uint32_t tile_cnt[2][kElems][kWaves];
  uint32_t wsum[kWaves];
  uint32_t res[4];
  uint32_t acc[8];
};

// ---------------------------------------------------------------------------
// Threshold search: wavefront 0 finds the bin holding the krem-th largest
// entry, counting down from the top bin; with ZERO it leaves the histogram
// zeroed.  res = {bin, entries in bins above it, entries in the bin, ok}.
// Kept out of line: inlined, its per-lane LDS addresses are hoisted out of
// the row loop and pinned in registers for the whole kernel.
// ---------------------------------------------------------------------------
template <int NB, bool ZERO>
__device__ __noinline__ void wave_search(lds_u32* hist, uint32_t krem, lds_u32* res) {
  constexpr int kPer = NB / 64;  // bins per lane-group: 32 or 16
  constexpr int kVec = kPer / 4;
  const int lane = threadIdx.x & 63;
  // Lane l owns group 63 - l, so lane order is descending bin order.
  lds_u4* grp = (lds_u4*)(hist + (63 - lane) * kPer);
  uint32_t s = 0;
#pragma unroll
  for (int c = 0; c < kVec; ++c) {
    const u32x4 v = grp[(c + lane) & (kVec - 1)];  // rotated start: spreads the banks
    s += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_incl_scan(s);
  const uint64_t reach = ballot(incl >= krem);
  if (reach == 0) {  // fewer than krem entries: inconsistent histogram
    if (lane == 0) {
      res[0] = 0u;
      res[1] = 0u;
      res[2] = lane_value(incl, 63);
      res[3] = 0u;
    }
  } else {
    // The first lane whose running count reaches krem owns the threshold
    // group; its bins are scanned by as many lanes, top bin first.
    const int lc = __builtin_ctzll(reach);
    const uint32_t before = lane_value(incl, lc) - lane_value(s, lc);
    const int qc = 63 - lc;
    const uint32_t v = lane < kPer ? hist[qc * kPer + (kPer - 1 - lane)] : 0u;
    const uint32_t in2 = wave_incl_scan(v) + before;
    const uint64_t reach2 = ballot(lane < kPer && in2 >= krem);
    const int l2 = __builtin_ctzll(reach2);
    if (lane == l2) {
      res[0] = (uint32_t)(qc * kPer + (kPer - 1 - l2));
      res[1] = in2 - v;
      res[2] = v;
      res[3] = 1u;
    }
  }
  if (ZERO) {
#pragma unroll
    for (int c = 0; c < kVec; ++c) grp[(c + lane) & (kVec - 1)] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int NB, bool ZERO>
__device__ __forceinline__ void search(uint32_t* hist, uint32_t krem, uint32_t* res) {
  if (threadIdx.x < 64) wave_search<NB, ZERO>((lds_u32*)hist, krem, (lds_u32*)res);
}

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum.  Contains one barrier.
template <int KMAX>
__device__ __forceinline__ uint32_t block_excl_scan(Smem<KMAX>& sm, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sm.wsum[w] = incl;
  __syncthreads();
  const uint4 ws = *reinterpret_cast<const uint4*>(sm.wsum);
  *total = ws.x + ws.y + ws.z + ws.w;
  const uint32_t before = (w > 0 ? ws.x : 0u) + (w > 1 ? ws.y : 0u) + (w > 2 ? ws.z : 0u);
  return before + incl - v;
}

// ---------------------------------------------------------------------------
// Selection over the candidate buffer
// ---------------------------------------------------------------------------

struct Sel {
  uint32_t prefix;  // decided key bits
  uint32_t pmask;   // which bits are decided
  uint32_t krem;    // entries equal to prefix (under pmask) to take, lowest position first
  uint32_t ok;
  uint32_t b1;      // threshold top digit
  uint32_t krem1;   // entries taken from bin b1
};

// Thread t owns buffer positions [t*S, t*S + S); loads keys and indices.
template <int KMAX>
__device__ __forceinline__ void load_owned(const Smem<KMAX>& sm, uint32_t (&k)[Shape<KMAX>::kSlots],
                                           uint32_t (&ix)[Shape<KMAX>::kSlots]) {
  constexpr int S = Shape<KMAX>::kSlots;
  const uint32_t base = threadIdx.x * S;
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(&sm.key[base + 4 * q]);
    const u32x4 b = *reinterpret_cast<const u32x4*>(&sm.idx[base + 4 * q]);
    k[4 * q + 0] = a.x;
    k[4 * q + 1] = a.y;
    k[4 * q + 2] = a.z;
    k[4 * q + 3] = a.w;
    ix[4 * q + 0] = b.x;
    ix[4 * q + 1] = b.y;
    ix[4 * q + 2] = b.z;
    ix[4 * q + 3] = b.w;
  }
}

// The keep best of the cnt buffer entries (keys in registers, contiguous
// ownership): those with (key & pmask) > prefix plus the first krem with
// (key & pmask) == prefix.  hist1 must be the top-digit histogram of the
// buffer; it is read, not changed.  hist2 is left zeroed.  keep <= cnt.
template <int KMAX>
__device__ Sel select_keep(Smem<KMAX>& sm, const uint32_t (&k)[Shape<KMAX>::kSlots], uint32_t cnt,
                           uint32_t keep) {
  constexpr int S = Shape<KMAX>::kSlots;
  const uint32_t base = threadIdx.x * S;
  Sel r;
  search<2048, false>(sm.hist1, keep, sm.res);
  __syncthreads();
  r.b1 = sm.res[0];
  r.ok = sm.res[3];
  r.krem = keep - sm.res[1];
  r.krem1 = r.krem;
  r.prefix = r.b1 << 21;
  r.pmask = 0xffe00000u;
  uint32_t in_bin = sm.res[2];
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    if (in_bin == r.krem) break;  // every entry of the bin is taken
    const int shift = pass == 1 ? 10 : 0;
    const uint32_t dmask = pass == 1 ? 2047u : 1023u;
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (base + j < cnt && (k[j] & r.pmask) == r.prefix) atomicAdd(&sm.hist2[(k[j] >> shift) & dmask], 1u);
    __syncthreads();
    if (pass == 1)
      search<2048, true>(sm.hist2, r.krem, sm.res);
    else
      search<1024, true>(sm.hist2, r.krem, sm.res);
    __syncthreads();
    r.ok &= sm.res[3];
    r.krem -= sm.res[1];
    r.prefix |= sm.res[0] << shift;
    r.pmask |= dmask << shift;
    in_bin = sm.res[2];
  }
  return r;
}

// Writes the chosen entries in buffer order.  An entry is chosen if
// (key & pmask) > prefix, or if it equals prefix and fewer than take_eq
// equal entries precede it (gt_base / eq_base count greater / equal entries
// of earlier chunks of the row).  Its rank = earlier greater entries +
// min(earlier equal entries, take_eq).  Ranks >= limit are dropped (only
// reachable with an inconsistent workspace).  To LDS (key, idx) when out is
// null, else idx to out[rank].  Contains one barrier.
template <int KMAX>
__device__ __forceinline__ void emit_chosen(Smem<KMAX>& sm, const uint32_t (&k)[Shape<KMAX>::kSlots],
                                            const uint32_t (&ix)[Shape<KMAX>::kSlots], uint32_t cnt,
                                            uint32_t prefix, uint32_t pmask, uint32_t gt_base,
                                            uint32_t eq_base, uint32_t take_eq, int32_t* out,
                                            uint32_t limit) {
  constexpr int S = Shape<KMAX>::kSlots;
  const uint32_t base = threadIdx.x * S;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = base + j < cnt;
    const uint32_t km = k[j] & pmask;
    packed += (valid && km > prefix) ? 1u : 0u;
    packed += (valid && km == prefix) ? 0x10000u : 0u;
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan(sm, packed, &total);
  uint32_t g = gt_base + (excl & 0xffffu);
  uint32_t e = eq_base + (excl >> 16);
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = base + j < cnt;
    const uint32_t km = k[j] & pmask;
    const bool gt = valid && km > prefix;
    const bool eq = valid && km == prefix;
    const bool take = gt || (eq && e < take_eq);
    const uint32_t pos = g + (e < take_eq ? e : take_eq);
    if (take && pos < limit) {
      if (out != nullptr) {
        out[pos] = (int32_t)ix[j];
      } else {
        sm.key[pos] = k[j];
        sm.idx[pos] = ix[j];
      }
    }
    g += gt ? 1u : 0u;
    e += eq ? 1u : 0u;
  }
}

// Compacts the buffer (cnt > keep entries) to its keep best, index order
// kept, corrects the running histogram and returns the raised acceptance
// bound.  Arguments and result go by value: as an out-of-line call, a
// by-reference counter would live in scratch, and every scratch reload waits
// on all outstanding prefetches.
template <int KMAX>
__device__ __noinline__ uint32_t compact(Smem<KMAX>& sm, uint32_t cnt, uint32_t keep, uint32_t L) {
  constexpr int S = Shape<KMAX>::kSlots;
  uint32_t k[S], ix[S];
  load_owned<KMAX>(sm, k, ix);
  const Sel s = select_keep<KMAX>(sm, k, cnt, keep);
  emit_chosen<KMAX>(sm, k, ix, cnt, s.prefix, s.pmask, 0u, 0u, s.krem, nullptr,
                    (uint32_t)Shape<KMAX>::kCap);
  // Kept entries: bins above b1 unchanged, krem1 from bin b1, none below.
  for (uint32_t i = threadIdx.x; i < (uint32_t)kBins; i += kBlock) {
    if (i < s.b1) sm.hist1[i] = 0u;
    if (i == s.b1) sm.hist1[i] = s.krem1;
  }
  __syncthreads();
  // Every element still to come has a higher index than all kept entries, so
  // it must beat the K-th best key strictly to matter.  When the K-th best key
  // is known only to its top bits, accept anything from that prefix up.
  uint32_t Ln;
  if (s.pmask == 0xffffffffu)
    Ln = s.prefix == 0xffffffffu ? 0xffffffffu : s.prefix + 1u;
  else
    Ln = s.prefix;
  return Ln > L ? Ln : L;
}

// The K best of the buffer, written to out in index order; the running
// histogram is cleared for the next row.
template <int KMAX>
__device__ __noinline__ void final_select(Smem<KMAX>& sm, uint32_t cnt, uint32_t K, int32_t* out) {
  constexpr int S = Shape<KMAX>::kSlots;
  uint32_t k[S], ix[S];
  load_owned<KMAX>(sm, k, ix);
  const Sel s = select_keep<KMAX>(sm, k, cnt, K);
  emit_chosen<KMAX>(sm, k, ix, cnt, s.prefix, s.pmask, 0u, 0u, s.krem, out, K);
  for (uint32_t i = threadIdx.x; i < (uint32_t)kBins; i += kBlock) sm.hist1[i] = 0u;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Streaming filter over [c0, c1) of one row
// ---------------------------------------------------------------------------

template <int VEC>
__device__ __forceinline__ void load_full(const float* __restrict__ rowp, uint32_t p0, float (&x)[kElems]) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
    const uint32_t pos = p0 + (uint32_t)u * (kBlock * VEC) + t * VEC;
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
  }
}

// The partial last tile: per-element bounds checks, nothing read at or past c1.
template <int VEC>
__device__ __forceinline__ void load_tail(const float* __restrict__ rowp, uint32_t c1, uint32_t p0,
                                          float (&x)[kElems]) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
    const uint32_t pos = p0 + (uint32_t)u * (kBlock * VEC) + t * VEC;
#pragma unroll
    for (int c = 0; c < VEC; ++c) x[u * VEC + c] = (pos + c < c1) ? rowp[pos + c] : 0.0f;
  }
}

// Per-wave counts of accepted elements for each load slot go through LDS
// (double-buffered by par); returns the tile total and this wave's offset
// for each slot.
template <int KMAX, int VEC>
__device__ __forceinline__ uint32_t tile_exchange(Smem<KMAX>& sm, const bool (&a)[kElems], int& par,
                                                  uint32_t (&off)[kElems / VEC]) {
  constexpr int NL = kElems / VEC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    uint32_t c = 0;
#pragma unroll
    for (int cc = 0; cc < VEC; ++cc) c += popc64(ballot(a[u * VEC + cc]));
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

template <int VEC, bool FULL>
__device__ __forceinline__ void tile_accept(const float (&x)[kElems], uint32_t pbase, uint32_t c1, float bf,
                                            bool (&a)[kElems]) {
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const int e = u * VEC + c;
      const bool in = FULL || pbase + (uint32_t)u * (kBlock * VEC) + c < c1;
      a[e] = in && x[e] >= bf;
    }
  }
}

// Filters one tile into the candidate buffer, compacting first if the
// tile's accepted elements would not fit.
template <int KMAX, int VEC, bool FULL>
__device__ __forceinline__ void process_tile(Smem<KMAX>& sm, const float (&x)[kElems], uint32_t p0, uint32_t c1,
                                             uint32_t keep, uint32_t& cnt, uint32_t& L, int& par) {
  constexpr int NL = kElems / VEC;
  const uint32_t pbase = p0 + threadIdx.x * VEC;
  bool a[kElems];
  uint32_t off[NL];
  tile_accept<VEC, FULL>(x, pbase, c1, accept_floor(L), a);
  uint32_t total = tile_exchange<KMAX, VEC>(sm, a, par, off);
  if (cnt + total > (uint32_t)Shape<KMAX>::kCap) {
    L = compact<KMAX>(sm, cnt, keep, L);
    cnt = keep;
    tile_accept<VEC, FULL>(x, pbase, c1, accept_floor(L), a);
    total = tile_exchange<KMAX, VEC>(sm, a, par, off);
  }
  if (total != 0) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      uint32_t r = cnt + off[u];
#pragma unroll
      for (int c = 0; c < VEC; ++c) r += lanes_below(ballot(a[u * VEC + c]));
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const int e = u * VEC + c;
        if (a[e]) {
          const uint32_t key = ord_key(__float_as_uint(x[e]));
          sm.key[r] = key;
          sm.idx[r] = pbase + (uint32_t)u * (kBlock * VEC) + c;
          atomicAdd(&sm.hist1[key >> 21], 1u);
        }
        r += a[e] ? 1u : 0u;
      }
    }
  }
  cnt += total;
}

// Streams [c0, c1) through the filter.  Full tiles come through a ring of
// kPrefetch register buffers: the load for tile j + kPrefetch - 1 is issued
// before tile j is processed, so about (kPrefetch - 1) tiles per workgroup
// are in flight.  Prefetch addresses past the last full tile are clamped to
// it (a cache hit), which keeps the load pattern identical every iteration.
// The partial last tile is loaded with per-element bounds checks.
template <int KMAX, int VEC>
__device__ void stream_chunk(Smem<KMAX>& sm, const float* __restrict__ rowp, uint32_t c0, uint32_t c1,
                             uint32_t keep, uint32_t& cnt, uint32_t& L) {
  constexpr int PF = kPrefetch;
  const uint32_t F = (c1 - c0) / kTile;  // full tiles
  int par = 0;
  if (F > 0) {
    float buf[PF][kElems];
#pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
      load_full<VEC>(rowp, c0 + ((uint32_t)s < F ? (uint32_t)s : F - 1) * kTile, buf[s]);
      __builtin_amdgcn_sched_barrier(0);  // keep tiles in issue order: waits then retire oldest first
    }
    // Whole rounds of PF tiles: one uniform back edge, so the compiler's
    // load-counter waits stay exact (retire only the tile about to be used).
    const uint32_t Fr = F - F % PF;
    for (uint32_t j0 = 0; j0 < Fr; j0 += PF) {
#pragma unroll
      for (int slot = 0; slot < PF; ++slot) {
        const uint32_t j = j0 + slot;
        const uint32_t jn = j + PF - 1 < F ? j + PF - 1 : F - 1;
        load_full<VEC>(rowp, c0 + jn * kTile, buf[(slot + PF - 1) % PF]);
        __builtin_amdgcn_sched_barrier(0);
        process_tile<KMAX, VEC, true>(sm, buf[slot], c0 + j * kTile, c1, keep, cnt, L, par);
      }
    }
    // The last F % PF full tiles are already in buf[0..]: no more loads.
#pragma unroll
    for (int slot = 0; slot < PF - 1; ++slot) {
      const uint32_t j = Fr + slot;
      if (j < F) process_tile<KMAX, VEC, true>(sm, buf[slot], c0 + j * kTile, c1, keep, cnt, L, par);
    }
  }
  const uint32_t pt = c0 + F * kTile;
  if (pt < c1) {
    float x[kElems];
    load_tail<VEC>(rowp, c1, pt, x);
    process_tile<KMAX, VEC, false>(sm, x, pt, c1, keep, cnt, L, par);
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

template <int KMAX>
__device__ __forceinline__ void zero_histograms(Smem<KMAX>& sm) {
  for (int i = threadIdx.x; i < kBins; i += kBlock) {
    sm.hist1[i] = 0u;
    sm.hist2[i] = 0u;
  }
}

// ---------------------------------------------------------------------------
// One workgroup per row, persistent over rows.
// ---------------------------------------------------------------------------
template <int KMAX, int VEC>
__global__ void __launch_bounds__(kBlock) topk_single_kernel(KernelParams p) {
  __shared__ Smem<KMAX> sm;
  zero_histograms(sm);
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
    final_select<KMAX>(sm, cnt, K, out);
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

// Adds an LDS histogram into a workspace histogram (non-zero bins only) and
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
  const int t = threadIdx.x;
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

  zero_histograms(sm);
  if (t < 8) sm.acc[t] = 0u;
  __syncthreads();

  const int64_t c0 = (int64_t)g * p.chunk;
  const int64_t c1 = c0 + p.chunk < n ? c0 + p.chunk : n;
  const float* rowp = p.scores + (int64_t)row * p.row_stride;
  uint32_t cnt = 0, L = 0;
  stream_chunk<KMAX, VEC>(sm, rowp, (uint32_t)c0, (uint32_t)c1, K, cnt, L);

  uint32_t k[S], ix[S];
  load_owned<KMAX>(sm, k, ix);
  const uint32_t base = (uint32_t)t * S;

  // Round 1: the chunk's top-digit histogram (already in hist1) into the
  // row's, then the row-wide threshold digit.
  merge_hist(sm.hist1, h1);
  group_barrier(ctr, 1u * grow, p.spin_limit, err);
  load_hist(sm.hist2, h1);
  __syncthreads();
  search<2048, true>(sm.hist2, K, sm.res);
  __syncthreads();
  uint32_t ok = sm.res[3];
  uint32_t krem = K - sm.res[1];
  uint32_t prefix = sm.res[0] << 21;
  uint32_t pmask = 0xffe00000u;

  // Round 2: next 11 bits of the entries in the threshold bin; publish how
  // many of this chunk's entries lie above it.
  uint32_t n_above = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool valid = base + j < cnt;
    const uint32_t km = k[j] & pmask;
    if (valid && km == prefix) atomicAdd(&sm.hist2[(k[j] >> 10) & 2047u], 1u);
    n_above += popc64(ballot(valid && km > prefix));
  }
  wave_add(&sm.acc[0], n_above);
  __syncthreads();
  merge_hist(sm.hist2, h2);
  if (t == 0) slots[4 * g + 0] = sm.acc[0];
  group_barrier(ctr, 2u * grow, p.spin_limit, err);
  load_hist(sm.hist2, h2);
  __syncthreads();
  search<2048, true>(sm.hist2, krem, sm.res);
  __syncthreads();
  ok &= sm.res[3];
  krem -= sm.res[1];
  prefix |= sm.res[0] << 10;
  pmask = 0xfffffc00u;

  // Round 3: publish the keys still undecided after 22 bits, in index order,
  // and the count above them.
  {
    uint32_t mine = 0;
    n_above = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool valid = base + j < cnt;
      const uint32_t km = k[j] & pmask;
      mine += (valid && km == prefix) ? 1u : 0u;
      n_above += popc64(ballot(valid && km > prefix));
    }
    wave_add(&sm.acc[1], n_above);
    uint32_t len;
    uint32_t at = block_excl_scan(sm, mine, &len);
    uint32_t* my_list = lists + (uint64_t)g * CAP;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool valid = base + j < cnt;
      if (valid && (k[j] & pmask) == prefix) my_list[at++] = k[j];
    }
    if (t == 0) {
      slots[4 * g + 1] = sm.acc[1] - sm.acc[0];
      slots[4 * g + 2] = len;
    }
  }
  group_barrier(ctr, 3u * grow, p.spin_limit, err);

  // Last 10 bits over every chunk's list; then this chunk's offsets.
  for (int gg = 0; gg < grow; ++gg) {
    uint32_t len = slots[4 * gg + 2];
    len = len < (uint32_t)CAP ? len : (uint32_t)CAP;
    const uint32_t* lst = lists + (uint64_t)gg * CAP;
    for (uint32_t i = t; i < len; i += kBlock) atomicAdd(&sm.hist2[lst[i] & 1023u], 1u);
  }
  __syncthreads();
  search<1024, true>(sm.hist2, krem, sm.res);
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
    // List counts are wave-uniform; the slot counts were added on thread 0 only.
    if ((t & 63) == 0) {
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
    for (int gg = 0; gg < grow; ++gg) {
      uint32_t len = slots[4 * gg + 2];
      len = len < (uint32_t)CAP ? len : (uint32_t)CAP;
      uint32_t* lst = lists + (uint64_t)gg * CAP;
      for (uint32_t i = t; i < len; i += kBlock) lst[i] = 0u;
    }
    __syncthreads();  // every list length has been read before the slots are cleared
    if (t < 4 * grow) slots[t] = 0u;
    if (t == 0) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exit_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  emit_chosen<KMAX>(sm, k, ix, cnt, T, 0xffffffffu, gt_base, eq_base, take_eq, out, K);
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
