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
//   in tiles of coalesced loads kept in flight by a register ring.  It keeps
//   an index-ordered candidate buffer in LDS (fp32 bits and indices) and a
//   lower bound L on the key of the K-th best element seen so far; an
//   element is appended only if it reaches L, one IEEE compare per element,
//   and its position comes from ballots and mbcnt ranks.  When a tile would
//   overflow the buffer, the buffer is compacted and L rises (see compact()).
//   Each score is read from HBM once.
//
// * Speculative bound.  On long rows the bound starts at (about) the key of
//   the ceil(1.5 K M / n)-th best of an M-element sample (the first two wave
//   tiles of every wavefront's segment), so only ~1.5 K elements reach the
//   buffer; each wavefront then streams its own segment of the row into its
//   own part of the buffer, with no per-tile barrier.  A row whose bound
//   proves too high (fewer than K reached it), or whose part of the buffer
//   would overflow, is streamed again without one.
//
// * Range select.  Over the register-held keys: passes histogram the keys of
//   the current interval [lo, hi] into 2048 or 256 LDS bins, starting from
//   the keys' exact range or, after a speculative stream, from [bound, the
//   sample's largest key] with an open top bin.  Every wavefront scans a
//   histogram from the top with DPP prefix sums and finds the threshold bin
//   itself, so a search costs no barrier.  Ties at the final 32-bit key go
//   to the lower buffer position, the lower index.
//
// * Ordered emit.  Each wavefront owns a contiguous, index-ordered part of
//   the buffer; one exchange of per-wavefront counts gives every chosen
//   entry its output rank by ballots, so output is written in ascending
//   index order with no sort.
//
// * Multi-workgroup rows.  G workgroups each stream a chunk of the row from
//   the same speculative bound (the same sample, the same selection), publish
//   the elements that reach it to the workspace and arrive once; the last to
//   arrive gathers the union in chunk order and selects.  If the bound fails
//   for the row, every workgroup falls back to three cooperative rounds that
//   merge digit histograms in the workspace.  All workspace traffic is
//   agent-scope atomic, ordered by waits and barriers, so no cache-wide
//   fences are needed.  The last workgroup to leave zeroes everything the
//   row touched, so the workspace is all-zero when the kernel ends (the
//   in-kernel cleanup of the PR #41748 page, without the race its review
//   describes: nothing is reset while another workgroup can still read it).
//
// Instances differ in the workgroup width (256, 512 or 1024 threads: 4, 8 or
// 16 wavefronts share a row), the buffer layout (16-bit or 32-bit candidate
// indices; room for K up to 2048 or 4096), the load width, the score type
// (fp32, or bf16 widened exactly at the load), and whether the launch writes
// the chosen scores (compiled out otherwise, to keep the row loop's
// registers).  This header holds the templates; the instance
// files compile groups of them in parallel.
//
// The key function maps fp32 bits to uint32 so that unsigned order equals
// IEEE order for non-NaN values, with -0.0 and +0.0 mapped to the same key.
// Everything on the selection path is integer or bit manipulation except the
// streaming compare x >= f(L), an exact IEEE comparison (denormals are kept:
// the library is built without flush-to-zero).

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// The same order without folding -0.0 into +0.0 (-0.0 sorts just below it),
// exactly reversible by key_bits; for transforms that must give the bits back.
__device__ __forceinline__ uint32_t raw_key(uint32_t u) {
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ord_key (up to the sign of zero) and of raw_key: fp32 bits.
__device__ __forceinline__ uint32_t key_bits(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// threadIdx.x laundered through an empty asm statement: values computed
// from it cannot be hoisted out of the row loop and kept live (in registers
// or spilled) across the whole kernel.  Used on the selection paths, which
// run once per row.
__device__ __forceinline__ uint32_t tid() {
  uint32_t t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Wave-uniform copy of a value that is the same in every lane, so that the
// compiler keeps it (and what is computed from it) in scalar registers.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// ---------------------------------------------------------------------------
// Shared memory of one workgroup
// ---------------------------------------------------------------------------

template <int LAY>
struct Shape {
  static constexpr int kBlock = block_of(LAY);   // threads per workgroup
  static constexpr int kWaves = kBlock / 64;
  static constexpr int kTile = kBlock * kElems;  // elements one general-path tile covers
  static constexpr bool kIdx16 = (LAY & kLayIdx16) != 0;
  static constexpr int kMaxK = kmax_of(LAY);
  static constexpr int kCap = cap_of(LAY);
  static constexpr int kSlots = kCap / kBlock;  // buffer entries owned per thread
  // Candidate index type in LDS.  16 bits only for the 256-thread layouts,
  // where they let a fourth workgroup share the CU.  The wide layouts keep 32
  // bits: the value and the index of a kept element then go out as one
  // paired store (the two arrays sit a multiple of 256 bytes apart), where a
  // 16-bit index costs a second store and its own address arithmetic, on a
  // streaming loop that a lone workgroup runs as fast as it can issue it
  // (multi-token rows 16.2 -> 15.3 us, decode 14.0 -> 13.7 us, measured on
  // MI355X).
  using Idx = typename std::conditional<kIdx16 && kWaves == 4, uint16_t, uint32_t>::type;
  static_assert(kCap % kBlock == 0 && kSlots % 4 == 0, "capacity must tile the workgroup in aligned runs");
  static_assert(kCap % (kWaves * 64) == 0 && kCap / kWaves <= 64 * kSlots, "a wavefront's part fits its slices");
  static_assert(kWaves % 4 == 0 && kWaves <= 16, "per-wave partials are read four at a time");
  static_assert(kCap < 65536, "packed 16-bit counts");
  static_assert(kCap >= kMaxK + kTile, "a tile must fit after a compaction");
  // Workgroups per CU the LDS footprint allows (160 KB per CU); the register
  // budget is held to match (at most 16 wavefronts per CU: 128 VGPRs).
  static constexpr int kResident = resident_of(LAY);
  // HIP's second launch bound is waves per SIMD (four SIMDs per CU): the
  // register budget that lets kResident workgroups share a CU.
  static constexpr int kWavesPerSimd = kResident * kWaves / 4;
};

template <int LAY>
struct __align__(16) Smem {
  // Wide workgroups append without a branch per element: a lane with nothing
  // to keep writes to its own word past the capacity (never read).
  static constexpr int kDiscard = Shape<LAY>::kWaves > 4 ? 64 : 0;
  uint32_t val[Shape<LAY>::kCap + kDiscard];                 // candidate fp32 bits, index order
  typename Shape<LAY>::Idx idx[Shape<LAY>::kCap + kDiscard];  // their indices, relative to the chunk start
  uint32_t hist1[kBins];                          // digit histogram; all-zero outside a selection
  uint32_t hs[kSmallBins];                        // second digit histogram; all-zero outside a selection
  uint32_t red[2 * Shape<LAY>::kWaves];           // per-wave partial results
  uint32_t tile_cnt[2][kElems][Shape<LAY>::kWaves];
  uint32_t wsum[Shape<LAY>::kWaves];
  uint32_t acc[16];
  uint32_t bnd[2 * Shape<LAY>::kWaves];  // per-wave bounds and sample maxima of a speculative sample
  uint32_t wcnt[2 * Shape<LAY>::kWaves]; // per-wave candidate counts and overflow flags of a stream
  // Target of histogram adds that count nothing: one word per lane, so the
  // lanes of one add never collide on it (never read).
  uint32_t sink[64];
};

// ---------------------------------------------------------------------------
// Threshold search.  Every wavefront of the workgroup runs it on the same
// histogram and gets the same wave-uniform answer: the bin holding the
// krem-th largest entry, counting down from the top bin, the number of
// entries in bins above it and in the bin.  No barrier is needed to share the
// result.  The lane id goes through an empty asm statement so the compiler
// cannot hoist the per-lane LDS addresses out of the row loop and pin them in
// registers for the whole kernel.
// ---------------------------------------------------------------------------
struct Found {
  uint32_t bin, above, in_bin, ok;
};

template <int NB>
__device__ __forceinline__ Found wave_find(const uint32_t* hist, uint32_t krem) {
  constexpr int kPer = NB / 64;  // bins per lane-group: 32 or 16
  constexpr int kVec = kPer / 4;
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  // Lane l owns group 63 - l, so lane order is descending bin order.
  const u32x4* grp = reinterpret_cast<const u32x4*>(hist + (63 - lane) * kPer);
  // Loads go out four at a time (rotated start: spreads the banks), so their
  // latencies overlap without holding the whole group in registers.
  constexpr int kB = kVec < 4 ? kVec : 4;
  static_assert(kVec % kB == 0, "whole batches");
  uint32_t s = 0;
#pragma unroll
  for (int c0 = 0; c0 < kVec; c0 += kB) {
    u32x4 g[kB];
#pragma unroll
    for (int c = 0; c < kB; ++c) g[c] = grp[(c0 + c + lane) & (kVec - 1)];
#pragma unroll
    for (int c = 0; c < kB; ++c) s += (g[c].x + g[c].y) + (g[c].z + g[c].w);
  }
  const uint32_t incl = wave_incl_scan(s);
  const uint64_t reach = ballot(incl >= krem);
  Found f;
  if (reach == 0) {  // fewer than krem entries: inconsistent histogram
    f.bin = 0u;
    f.above = 0u;
    f.in_bin = lane_value(incl, 63);
    f.ok = 0u;
    return f;
  }
  // The first lane whose running count reaches krem owns the threshold group;
  // its bins are scanned by as many lanes, top bin first.
  const int lc = __builtin_ctzll(reach);
  const uint32_t before = lane_value(incl, lc) - lane_value(s, lc);
  const int qc = 63 - lc;
  const uint32_t v = lane < kPer ? hist[qc * kPer + (kPer - 1 - lane)] : 0u;
  const uint32_t in2 = wave_incl_scan(v) + before;
  const uint64_t reach2 = ballot(lane < kPer && in2 >= krem);
  const int l2 = __builtin_ctzll(reach2);
  f.bin = (uint32_t)(qc * kPer + (kPer - 1 - l2));
  f.in_bin = lane_value(v, l2);
  f.above = lane_value(in2, l2) - f.in_bin;
  f.ok = 1u;
  return f;
}

// Sum of v over the wavefront (every lane gets it), by DPP row shifts and
// broadcasts.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return lane_value(wave_incl_scan(v), 63); }

// Exclusive prefix over the wavefronts of the workgroup of a wave-uniform
// value v (this wavefront's share): the sum of v over the lower wavefronts,
// with the sum over all of them in *total.  One barrier; sm.wsum is free
// again after the next barrier.
template <int LAY>
__device__ __forceinline__ uint32_t wave_exclusive(Smem<LAY>& sm, uint32_t v, uint32_t* total) {
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t t = tid();
  const uint32_t w = t >> 6;
  if ((t & 63) == 0) sm.wsum[w] = v;
  __syncthreads();
  uint32_t tot = 0, before = 0;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const uint4 ws = *reinterpret_cast<const uint4*>(&sm.wsum[4 * q]);
    const uint32_t a[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      before += ((uint32_t)(4 * q + c) < w) ? a[c] : 0u;
      tot += a[c];
    }
  }
  *total = uni(tot);
  return uni(before);
}

// ---------------------------------------------------------------------------
// Selection over the candidate buffer
//
// Each wavefront owns a contiguous range of the buffer, in index order, and
// its lanes hold that range interleaved: slot j of lane l is position
// ws + 64 j + l.  The keys of a lane's slots sit in registers k[0..sp).  A
// wavefront's slot j thus covers 64 consecutive positions, so ranks come from
// one ballot per slot and every lane of a slot reads and writes neighbouring
// words (no LDS bank conflicts, coalesced output stores).  Work per selection
// scales with the entries present, not with the buffer's capacity.
//
// A selection narrows a key interval [lo, hi] known to hold the wanted
// entry.  Each pass histograms the keys inside it by (key - lo) >> s, with s
// chosen so the interval fills at most 2048 (even passes) or 256 (odd
// passes) bins, finds the bin holding the krem-th largest, and continues in
// that bin.  Starting from the exact range of the keys, the first pass
// usually leaves a handful of entries, whatever the data's scale; 32 bits
// take at most four passes.  Passes alternate between two histograms, so
// the second pass needs no clearing barrier.
// ---------------------------------------------------------------------------

// Chosen set of a selection: every key > hi, plus the first `take` entries
// (in buffer order, i.e. lowest index first) with lo <= key <= hi.
struct Sel {
  uint32_t lo, hi, take;
  uint32_t above;   // entries with key > hi
  uint32_t in_bin;  // entries with lo <= key <= hi
  uint32_t ok;      // 0 if a histogram was inconsistent
  bool all_in;      // take covers every entry inside [lo, hi]: the set is key >= lo
};

// A wavefront's share of the buffer during a selection: positions [ws, ws +
// wn) in index order, lane l holding slots j at ws + 64 j + l; sp slots are
// visited (a multiple of 4, wave-uniform), of which this lane's first nv hold
// entries.  Loops over the slots test sp once per group of 4: a test per slot
// would split the unrolled loop into one basic block per slot, and a lone
// wavefront then waits out each block's dependent chain in turn.
struct Slice {
  uint32_t ws, sp, nv;
};

template <int LAY>
__device__ __forceinline__ Slice make_slice(uint32_t ws, uint32_t wn) {
  constexpr uint32_t S = (uint32_t)Shape<LAY>::kSlots;
  ws = uni(ws);
  wn = uni(wn);
  uint32_t sp = (wn + 63u) / 64u;
  sp = (sp + 3u) & ~3u;
  sp = sp < S ? sp : S;
  const uint32_t lane = tid() & 63u;
  Slice sl;
  sl.ws = ws;
  sl.sp = sp;
  sl.nv = wn > lane ? (wn - lane + 63u) / 64u : 0u;
  return sl;
}

// The buffer as filled by the general path: cnt entries in positions [0,
// cnt), cut into one contiguous range per wavefront (whole groups of 64).
template <int LAY>
__device__ __forceinline__ Slice plain_slice(uint32_t cnt) {
  constexpr uint32_t W = (uint32_t)Shape<LAY>::kWaves;
  cnt = uni(cnt);
  const uint32_t seg = ((cnt + W - 1u) / W + 63u) / 64u * 64u;
  const uint32_t ws = uni(tid() >> 6) * seg;
  const uint32_t rest = cnt > ws ? cnt - ws : 0u;
  return make_slice<LAY>(ws, rest < seg ? rest : seg);
}

// The buffer as filled wave by wave: this wavefront's cw entries in
// positions [w * SUB, w * SUB + cw).
template <int LAY>
__device__ __forceinline__ Slice wave_slice(uint32_t cw) {
  constexpr uint32_t SUB = (uint32_t)Shape<LAY>::kCap / Shape<LAY>::kWaves;
  return make_slice<LAY>(uni(tid() >> 6) * SUB, cw);
}

// Position of this lane's slot j.
__device__ __forceinline__ uint32_t slot_pos(const Slice& sl, int j) { return sl.ws + 64u * (uint32_t)j + (tid() & 63u); }

// Keys of this lane's slots (every visited slot is read: positions past the
// entries stay inside the buffer and their keys are never counted).
template <int LAY>
__device__ __forceinline__ void load_keys(const Smem<LAY>& sm, uint32_t (&k)[Shape<LAY>::kSlots], const Slice& sl) {
  constexpr int S = Shape<LAY>::kSlots;
  const uint32_t p0 = slot_pos(sl, 0);
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) k[4 * q + c] = ord_key(sm.val[p0 + 64u * (uint32_t)(4 * q + c)]);
    }
  }
}

// The fp32 bits of this lane's slots, as stored.
template <int LAY>
__device__ __forceinline__ void load_bits(const Smem<LAY>& sm, uint32_t (&v)[Shape<LAY>::kSlots], const Slice& sl) {
  constexpr int S = Shape<LAY>::kSlots;
  const uint32_t p0 = slot_pos(sl, 0);
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = sm.val[p0 + 64u * (uint32_t)(4 * q + c)];
    }
  }
}

template <int LAY>
__device__ __forceinline__ void load_idx(const Smem<LAY>& sm, uint32_t (&ix)[Shape<LAY>::kSlots], const Slice& sl) {
  constexpr int S = Shape<LAY>::kSlots;
  const uint32_t p0 = slot_pos(sl, 0);
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ix[4 * q + c] = (uint32_t)sm.idx[p0 + 64u * (uint32_t)(4 * q + c)];
    }
  }
}

// The second-pass histogram is cleared by the first kSmallBins threads.
template <int LAY>
__device__ __forceinline__ void clear_small(Smem<LAY>& sm) {
  static_assert(Shape<LAY>::kBlock >= kSmallBins, "one second-pass bin per thread at most");
  const uint32_t t = tid();
  if (Shape<LAY>::kBlock == kSmallBins || t < (uint32_t)kSmallBins) sm.hs[t] = 0u;
}

template <int LAY>
__device__ __forceinline__ void clear_hists(Smem<LAY>& sm) {
  for (int i = tid(); i < kBins; i += Shape<LAY>::kBlock) sm.hist1[i] = 0u;
  clear_small(sm);
}

// Maximum over the wavefront by DPP row shifts and row broadcasts; every
// lane gets the result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  uint32_t x = v;
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return lane_value(x, 63);
}

// Minimum over the wavefront (lanes without a DPP source keep the identity).
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  const int id = -1;
  uint32_t x = v;
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return lane_value(x, 63);
}

// [lo, hi]: the smallest and largest key of the entries (both uniform).
// Contains one barrier.
template <int LAY, int S>
__device__ __forceinline__ void key_range(Smem<LAY>& sm, const uint32_t (&k)[S], const Slice& sl, uint32_t& lo,
                                          uint32_t& hi) {
  // Two independent chains (even and odd slots) halve the dependent latency.
  uint32_t mn0 = 0xffffffffu, mx0 = 0, mn1 = 0xffffffffu, mx1 = 0;
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        const bool v = (uint32_t)j < sl.nv;
        const uint32_t a = v ? k[j] : 0xffffffffu;
        const uint32_t b = v ? k[j] : 0u;
        if (c & 1) {
          mn1 = min(mn1, a);
          mx1 = max(mx1, b);
        } else {
          mn0 = min(mn0, a);
          mx0 = max(mx0, b);
        }
      }
    }
  }
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t mn = wave_min(min(mn0, mn1));
  const uint32_t mx = wave_max(max(mx0, mx1));
  const int w = tid() >> 6;
  if ((tid() & 63) == 0) {
    sm.red[w] = mn;
    sm.red[W + w] = mx;
  }
  __syncthreads();
  uint32_t l = 0xffffffffu, h = 0u;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(&sm.red[4 * q]);
    const u32x4 b = *reinterpret_cast<const u32x4*>(&sm.red[W + 4 * q]);
    l = min(l, min(min(a.x, a.y), min(a.z, a.w)));
    h = max(h, max(max(b.x, b.y), max(b.z, b.w)));
  }
  lo = uni(l);
  hi = uni(h);
}

// [mn, mx]: the smallest and largest key inside [lo, hi] (both uniform; mn >
// mx when none is).  One barrier, as key_range.
template <int LAY, int S>
__device__ __forceinline__ void interval_range(Smem<LAY>& sm, const uint32_t (&k)[S], const Slice& sl, uint32_t lo,
                                               uint32_t hi, uint32_t& mn, uint32_t& mx) {
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t range = hi - lo;
  uint32_t a0 = 0xffffffffu, b0 = 0u, a1 = 0xffffffffu, b1 = 0u;
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        const bool in = (uint32_t)j < sl.nv && k[j] - lo <= range;
        if (c & 1) {
          a1 = min(a1, in ? k[j] : 0xffffffffu);
          b1 = max(b1, in ? k[j] : 0u);
        } else {
          a0 = min(a0, in ? k[j] : 0xffffffffu);
          b0 = max(b0, in ? k[j] : 0u);
        }
      }
    }
  }
  const uint32_t wa = wave_min(min(a0, a1));
  const uint32_t wb = wave_max(max(b0, b1));
  const int w = tid() >> 6;
  if ((tid() & 63) == 0) {
    sm.red[w] = wa;
    sm.red[W + w] = wb;
  }
  __syncthreads();
  uint32_t l = 0xffffffffu, h = 0u;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.red[4 * q]);
    const u32x4 y = *reinterpret_cast<const u32x4*>(&sm.red[W + 4 * q]);
    l = min(l, min(min(x.x, x.y), min(x.z, x.w)));
    h = max(h, max(max(y.x, y.y), max(y.z, y.w)));
  }
  mn = uni(l);
  mx = uni(h);
  __syncthreads();  // sm.red is free again
}

// A threshold bin holding more entries than this after a pass is checked
// for being one key (ties), and otherwise narrowed to its exact range: with
// many equal keys every further pass would send most lanes of a wavefront to
// the same histogram word.  A selection with a stop total (a bound that may
// take its bin whole) checks from kTieCheckSoft: a tied bin there would
// otherwise take a pass per 8 bits of key until the bins are single keys.
constexpr uint32_t kTieCheck = 128;
constexpr uint32_t kTieCheckSoft = 8;

// Narrows [lo, hi] (which holds every entry at or above the keep-th largest;
// entries below lo are not counted) to the bin holding the keep-th largest
// entry.  Stops when that bin is taken whole (its entries are
// exactly the ones still needed, or entries above plus the bin number at
// most stop_total) or holds a single key; the result's take is then the
// whole bin or the entries still needed.  stop_total = 0 asks for an exact
// selection of keep entries.  With open_top, hi is only an estimate of the
// largest key: the first pass counts the keys above it in its top bin, and
// if the wanted entry lies there the search goes on from that bin's exact
// key range.  Both histograms are zero on entry and hold garbage on return.
template <int LAY, int S>
__device__ Sel range_select(Smem<LAY>& sm, const uint32_t (&k)[S], const Slice& sl, uint32_t lo, uint32_t hi,
                            uint32_t keep, uint32_t stop_total, bool open_top = false) {
  Sel r;
  r.ok = 1u;
  r.above = 0u;
  r.in_bin = 0u;
  uint32_t krem = keep;
  bool whole = false;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const bool big = (pass & 1) == 0;
    uint32_t* h = big ? sm.hist1 : sm.hs;
    const uint32_t bits = big ? 11u : 8u;
    if (pass >= 2) {  // this histogram was used two passes ago
      __syncthreads();
      if (big) {
        for (int i = tid(); i < kBins; i += Shape<LAY>::kBlock) h[i] = 0u;
      } else {
        clear_small(sm);
      }
      __syncthreads();
    }
    const uint32_t range = hi - lo;
    const uint32_t nb = range != 0u ? 32u - (uint32_t)__builtin_clz(range) : 0u;
    const uint32_t sh = nb > bits ? nb - bits : 0u;
    // One LDS add per slot and no per-slot branch: entries outside the
    // interval (and empty slots) add to the lane's own sink word instead of a
    // bin.  (Adding 0 to some bin would let every such lane of a wave hit the
    // same bin when the keys share their low bits, as bf16 scores do.)
    uint32_t* const sink = &sm.sink[tid() & 63];
    if (open_top) {
#pragma unroll
      for (int q = 0; q < S / 4; ++q) {
        if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = 4 * q + c;
            const uint32_t d = k[j] - lo;
            const bool in = (uint32_t)j < sl.nv && k[j] >= lo;
            atomicAdd(in ? &h[min(d, range) >> sh] : sink, 1u);
          }
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < S / 4; ++q) {
        if ((uint32_t)(4 * q) < sl.sp) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = 4 * q + c;
            const uint32_t d = k[j] - lo;
            const bool in = (uint32_t)j < sl.nv && d <= range;
            atomicAdd(in ? &h[d >> sh] : sink, 1u);
          }
        }
      }
    }
    __syncthreads();
    const Found f = big ? wave_find<kBins>(h, krem) : wave_find<kSmallBins>(h, krem);
    r.ok &= f.ok;
    krem -= f.above;
    r.above += f.above;
    r.in_bin = f.in_bin;
    // The top bin of an open first pass holds every key from its start up.
    const bool top = open_top && f.bin == range >> sh;
    open_top = false;
    lo += f.bin << sh;
    const uint32_t width = (1u << sh) - 1u;
    hi = top ? 0xffffffffu : (hi - lo > width ? lo + width : hi);
    whole = f.in_bin == krem || r.above + f.in_bin <= stop_total;
    if (whole || (sh == 0u && !top) || !f.ok) break;
    if (top || f.in_bin > (stop_total != 0u ? kTieCheckSoft : kTieCheck)) {
      uint32_t mn, mx;
      interval_range<LAY, S>(sm, k, sl, lo, hi, mn, mx);
      if (mn <= mx) {
        lo = mn;
        hi = mx;
        if (mn == mx) break;  // one key: take krem of its entries, lowest index first
      }
    }
  }
  r.lo = lo;
  r.hi = hi;
  r.take = whole ? r.in_bin : krem;
  r.all_in = whole;
  return r;
}

// Where the emit goes: kToBuffer (a compaction) or kToOut (the output).
// Either way both histograms are all-zero afterwards.
enum EmitMode { kToBuffer = 0, kToOut = 1 };

// Writes the chosen entries (of Sel s, see above) in buffer order.  gt_base
// / eq_base count the entries above / inside [lo, hi] of earlier chunks of
// the row; an entry's rank = earlier entries above + min(earlier entries
// inside, take).  Ranks >= limit are dropped (only reachable with an
// inconsistent workspace).
//
// Ranks come from ballots: a wavefront's slot j covers 64 consecutive
// buffer positions, so the rank of an entry is its wavefront's base (the
// counts of the lower wavefronts, one exchange), plus the counts of the
// wavefront's earlier slots, plus the lanes below it in its slot.  The
// chosen entries of one slot get consecutive ranks, so their stores are
// coalesced.  To the buffer (fp32 bits and index at position rank) for
// kToBuffer; otherwise ibase + index goes straight to out[rank], and with
// vout the entry's exact fp32 bits to vout[rank].  Every wavefront has read
// its slots and finished with the histograms before any entry moves (the
// exchange's barrier); the histograms are cleared after it.
template <int LAY, int MODE>
__device__ __forceinline__ void emit_chosen(Smem<LAY>& sm, const uint32_t (&k)[Shape<LAY>::kSlots], const Slice& sl,
                                            const Sel& s, uint32_t gt_base, uint32_t eq_base, int32_t* out,
                                            uint32_t limit, uint32_t ibase, float* vout = nullptr) {
  constexpr int S = Shape<LAY>::kSlots;
  static_assert(S <= 32, "slot flags fit one word");
  const uint32_t sp = sl.sp, nv = sl.nv;
  const uint32_t width = s.hi - s.lo;
  const uint32_t take = s.take;
  // Whole interval taken: the chosen set is every key >= lo (eqm stays 0).
  // Otherwise flags for above / inside the interval.
  const bool whole = s.all_in && gt_base == 0u && eq_base == 0u;
  uint32_t gtm = 0, eqm = 0;
  if (whole) {
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      if ((uint32_t)(4 * q) < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * q + c;
          gtm |= ((uint32_t)j < nv && k[j] >= s.lo) ? (1u << j) : 0u;
        }
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      if ((uint32_t)(4 * q) < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * q + c;
          const bool valid = (uint32_t)j < nv;
          gtm |= (valid && k[j] > s.hi) ? (1u << j) : 0u;
          eqm |= (valid && k[j] - s.lo <= width) ? (1u << j) : 0u;
        }
      }
    }
  }
  // Indices (and, for a compaction, the fp32 bits) are read before the
  // exchange's barrier: a compaction then moves entries down into other
  // wavefronts' ranges.  The bits are kept rather than rebuilt from the
  // keys, which fold -0.0 into +0.0.
  uint32_t ix[S];
  load_idx<LAY>(sm, ix, sl);
  uint32_t rv[MODE == kToBuffer ? S : 1];
  if constexpr (MODE == kToBuffer) load_bits<LAY>(sm, rv, sl);
  uint32_t total;
  const uint32_t before =
      wave_exclusive(sm, wave_sum((uint32_t)__popc(gtm) | ((uint32_t)__popc(eqm) << 16)), &total);
  (void)total;
  if constexpr (MODE != kToBuffer) clear_hists(sm);  // every wavefront is past its searches
  uint32_t g = gt_base + (before & 0xffffu);
  uint32_t e = eq_base + (before >> 16);
  const uint32_t p0 = slot_pos(sl, 0);
  if (whole) {
    // Every key >= lo is chosen: one ballot per slot.
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      if ((uint32_t)(4 * q) < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * q + c;
          const bool gt = (gtm >> j) & 1u;
          const uint64_t bg = ballot(gt);
          const uint32_t pos = g + lanes_below(bg);
          if (gt && pos < limit) {
            if constexpr (MODE != kToBuffer) {
              out[pos] = (int32_t)(ibase + ix[j]);
              if (vout != nullptr) vout[pos] = __uint_as_float(sm.val[p0 + 64u * (uint32_t)j]);
            } else {
              sm.val[pos] = rv[j];
              sm.idx[pos] = (typename Shape<LAY>::Idx)ix[j];
            }
          }
          g += popc64(bg);
        }
      }
    }
    if constexpr (MODE == kToBuffer) clear_hists(sm);
    return;
  }
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        const bool gt = (gtm >> j) & 1u;
        const bool eq = (eqm >> j) & 1u;
        const uint64_t bg = ballot(gt), be = ballot(eq);
        const uint32_t gr = g + lanes_below(bg);
        const uint32_t er = e + lanes_below(be);
        const bool pick = gt || (eq && er < take);
        const uint32_t pos = gr + (er < take ? er : take);
        if (pick && pos < limit) {
          if constexpr (MODE != kToBuffer) {
            out[pos] = (int32_t)(ibase + ix[j]);
            if (vout != nullptr) vout[pos] = __uint_as_float(sm.val[p0 + 64u * (uint32_t)j]);
          } else {
            sm.val[pos] = rv[j];
            sm.idx[pos] = (typename Shape<LAY>::Idx)ix[j];
          }
        }
        g += popc64(bg);
        e += popc64(be);
      }
    }
  }
  if constexpr (MODE == kToBuffer) clear_hists(sm);
}

// Frees buffer space when a tile would not fit (cnt > keep entries), keeping
// index order; returns (new count << 32) | new bound.  Keeps the bin holding
// the keep-th best whole, with everything above it, as soon as that leaves
// room for a tile; the bound becomes the bin's lowest key.  Failing that
// (ties crowding one key) keeps exactly the keep best: every element still
// to come has a higher index than all kept entries, so it must beat the
// keep-th best key strictly to matter.
//
// Out of line: inlined into each slot of the unrolled streaming loop it
// would multiply the register demand.  Arguments and result go by value: a
// by-reference counter would live in scratch, and every scratch reload waits
// on all outstanding prefetches.  The caller's next barrier orders the
// rewritten buffer before its next use.
template <int LAY>
__device__ __noinline__ uint64_t compact(Smem<LAY>& sm, uint32_t cnt, uint32_t keep, uint32_t L) {
  constexpr int S = Shape<LAY>::kSlots;
  constexpr uint32_t CAP = (uint32_t)Shape<LAY>::kCap;
  keep = uni(keep);
  L = uni(L);
  const Slice sl = plain_slice<LAY>(cnt);
  uint32_t k[S];
  load_keys<LAY>(sm, k, sl);
  uint32_t lo, hi;
  key_range<LAY, S>(sm, k, sl, lo, hi);
  const Sel s = range_select<LAY, S>(sm, k, sl, lo, hi, keep, CAP - (uint32_t)Shape<LAY>::kTile);
  emit_chosen<LAY, kToBuffer>(sm, k, sl, s, 0u, 0u, nullptr, CAP, 0u);
  uint32_t Ln;
  if (s.all_in) {
    Ln = s.lo;  // the bin was kept whole
  } else {
    Ln = s.lo == 0xffffffffu ? 0xffffffffu : s.lo + 1u;  // exact split at the single key lo
  }
  Ln = Ln > L ? Ln : L;
  return ((uint64_t)(s.above + s.take) << 32) | Ln;
}

// Where the candidates of a speculative stream lie, in ord_key terms: every
// one at or above lo (they passed the bound), the largest usually at most hi
// (the sample's largest key), so the final selection can skip its key range.
struct Hint {
  uint32_t lo, hi;
  bool on;
};

// The hint of a stream from bound L (a raw_key, > 0) and the sample's largest
// raw key top.
__device__ __forceinline__ Hint stream_hint(uint32_t L, uint32_t top) {
  Hint h;
  h.lo = ord_key(__float_as_uint(accept_floor(L)));
  h.hi = ord_key(key_bits(top));
  h.hi = h.hi > h.lo ? h.hi : h.lo;
  h.on = true;
  return h;
}

// The K best of the buffer, written to out in index order as ibase + index.
// Inline, so that loads issued before it (the next row's first tiles) stay
// in flight.  With a hint the first pass spans [hint.lo, hint.hi] with an
// open top instead of the entries' exact key range, saving a reduction and
// its barrier.
template <int LAY>
__device__ __forceinline__ void final_select(Smem<LAY>& sm, const Slice& sl, uint32_t K, int32_t* out,
                                             uint32_t ibase, float* vout = nullptr, Hint hint = Hint{0u, 0u, false}) {
  constexpr int S = Shape<LAY>::kSlots;
  K = uni(K);
  uint32_t k[S];
  load_keys<LAY>(sm, k, sl);
  uint32_t lo, hi;
  if (hint.on) {
    lo = uni(hint.lo);
    hi = uni(hint.hi);
  } else {
    key_range<LAY, S>(sm, k, sl, lo, hi);
  }
  const Sel s = range_select<LAY, S>(sm, k, sl, lo, hi, K, 0u, hint.on);
  emit_chosen<LAY, kToOut>(sm, k, sl, s, 0u, 0u, out, K, ibase, vout);
}

// ---------------------------------------------------------------------------
// Streaming filter over [c0, c1) of one row
// ---------------------------------------------------------------------------

// Scores are fp32 or bf16 (kept as its 16 bits).  Either way they enter the
// registers as fp32: widening bf16 shifts its bits up, which is exact, so
// every later step sees the same values and keys.
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// VEC consecutive elements at p (aligned to VEC elements) into x[o .. o + VEC).
// Scores are read once and never again by this launch, so the loads carry
// the nontemporal hint: they stream through the caches without displacing
// anything (measured on the prefill-shaped batch: 211.6 -> 198.1 us, and
// the streaming-read reference 168 -> 149 us).  A sample that several
// workgroups of one row read (NT = false) goes through the caches as usual,
// so that the row's other workgroups find it in L2.
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int VEC, bool NT = true, typename T>
__device__ __forceinline__ void load_run(const T* __restrict__ p, float (&x)[kElems], int o) {
  if constexpr (std::is_same<T, float>::value) {
    static_assert(VEC == 4 || VEC == 2 || VEC == 1, "fp32 loads of 16, 8 or 4 bytes");
    if constexpr (VEC == 4) {
      const f32x4 v = ld<NT>(reinterpret_cast<const f32x4*>(p));
      x[o + 0] = v.x;
      x[o + 1] = v.y;
      x[o + 2] = v.z;
      x[o + 3] = v.w;
    } else if constexpr (VEC == 2) {
      const f32x2 v = ld<NT>(reinterpret_cast<const f32x2*>(p));
      x[o + 0] = v.x;
      x[o + 1] = v.y;
    } else {
      x[o] = ld<NT>(p);
    }
  } else {
    static_assert(std::is_same<T, uint16_t>::value && (VEC == 8 || VEC == 1), "bf16 loads of 16 or 2 bytes");
    if constexpr (VEC == 8) {
      const u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(p));
      x[o + 0] = __uint_as_float(v.x << 16);
      x[o + 1] = __uint_as_float(v.x & 0xffff0000u);
      x[o + 2] = __uint_as_float(v.y << 16);
      x[o + 3] = __uint_as_float(v.y & 0xffff0000u);
      x[o + 4] = __uint_as_float(v.z << 16);
      x[o + 5] = __uint_as_float(v.z & 0xffff0000u);
      x[o + 6] = __uint_as_float(v.w << 16);
      x[o + 7] = __uint_as_float(v.w & 0xffff0000u);
    } else {
      x[o] = widen(ld<NT>(p));
    }
  }
}

// Tiles are wave-major: wavefront w of the workgroup covers elements
// [w * kWaveTile, (w + 1) * kWaveTile) of a tile, and lane l of it loads
// elements u * 64 * VEC + l * VEC .. + VEC - 1 of that range (u < kElems /
// VEC).  Each load instruction of a wave covers one contiguous run of 64 * VEC
// elements, and a wavefront's elements all precede the next one's in index
// order, so wavefronts only need each other's totals to place candidates.
constexpr uint32_t kWaveTile = 64u * kElems;  // elements one wavefront covers per tile

// One full tile starting at `tile` (a wave-uniform pointer).
template <int VEC, typename T>
__device__ __forceinline__ void load_full(const T* __restrict__ tile, float (&x)[kElems]) {
  const uint32_t w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u)
    load_run<VEC>(tile + w * kWaveTile + (uint32_t)u * (64u * VEC) + l * VEC, x, u * VEC);
}

// The partial last tile [p0, c1): per-element bounds checks, nothing read at
// or past c1.
template <int VEC, typename T>
__device__ __forceinline__ void load_tail(const T* __restrict__ rowp, uint32_t c1, uint32_t p0, float (&x)[kElems]) {
  const uint32_t w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
    const uint32_t pos = p0 + w * kWaveTile + (uint32_t)u * (64u * VEC) + l * VEC;
#pragma unroll
    for (int c = 0; c < VEC; ++c) x[u * VEC + c] = (pos + c < c1) ? widen(rowp[pos + c]) : 0.0f;
  }
}

// Row position of this thread's first element in the tile at p0.
__device__ __forceinline__ uint32_t tile_pbase(uint32_t p0, int vec) {
  return p0 + (threadIdx.x >> 6) * kWaveTile + (threadIdx.x & 63) * (uint32_t)vec;
}

// Whether element e of this thread's share of a tile is accepted: inside
// the chunk and at least the bound's float bf.  Evaluated where it is used
// (a compare is one instruction; a stored per-lane flag would cost more to
// keep and unpack).
template <int VEC, bool FULL>
__device__ __forceinline__ bool accepted(const float (&x)[kElems], int e, uint32_t pbase, uint32_t c1, float bf) {
  const int u = e / VEC, c = e % VEC;
  const bool in = FULL || pbase + (uint32_t)u * (64u * VEC) + c < c1;
  return in && x[e] >= bf;
}

// The wave's ballot of each element's acceptance.
template <int VEC, bool FULL>
__device__ __forceinline__ void tile_accept(const float (&x)[kElems], uint32_t pbase, uint32_t c1, float bf,
                                            uint64_t (&bal)[kElems]) {
#pragma unroll
  for (int e = 0; e < kElems; ++e) bal[e] = ballot(accepted<VEC, FULL>(x, e, pbase, c1, bf));
}

// Every wavefront's count of accepted elements goes through LDS
// (double-buffered by par); returns the tile total, and in before the
// counts of the lower wavefronts, both wave-uniform.
template <int LAY>
__device__ __forceinline__ uint32_t tile_exchange(Smem<LAY>& sm, const uint64_t (&bal)[kElems], int& par,
                                                  uint32_t& before) {
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t w = uni(threadIdx.x >> 6);
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kElems; ++e) mine += popc64(bal[e]);
  if ((threadIdx.x & 63) == 0) sm.tile_cnt[par][0][w] = mine;
  __syncthreads();
  uint32_t b = 0, all = 0;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.tile_cnt[par][0][4 * q]);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      b += ((uint32_t)(4 * q + c) < w) ? a[c] : 0u;
      all += a[c];
    }
  }
  before = uni(b);
  par ^= 1;
  return uni(all);
}

// Appends this wavefront's accepted elements of one tile, in index order,
// at cnt + before + their rank in the wavefront's part: fp32 bits and the
// index relative to the chunk start.
template <int LAY, int VEC, bool FULL>
__device__ __forceinline__ void tile_append(Smem<LAY>& sm, const float (&x)[kElems], const uint64_t (&bal)[kElems],
                                            uint32_t before, uint32_t cnt, uint32_t pbase, uint32_t c1, float bf,
                                            uint32_t rel) {
  constexpr int NL = kElems / VEC;
  uint32_t r0 = cnt + before;
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    uint32_t r = r0;
#pragma unroll
    for (int c = 0; c < VEC; ++c) r = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u * VEC + c] >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u * VEC + c], r));
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const int e = u * VEC + c;
      const bool take = accepted<VEC, FULL>(x, e, pbase, c1, bf);
      if (take) {
        sm.val[r] = __float_as_uint(x[e]);
        sm.idx[r] = (typename Shape<LAY>::Idx)(rel + (uint32_t)u * (64u * VEC) + c);
      }
      r += take ? 1u : 0u;
    }
#pragma unroll
    for (int c = 0; c < VEC; ++c) r0 += popc64(bal[u * VEC + c]);
  }
}

// Stream state of one workgroup, all wave-uniform: buffer count, bound (as a
// key and as the float every accepted element must reach), the pending
// speculation (row length, or 0), and the tile-count parity.
struct Stream {
  uint32_t cnt, L;
  float bf;
  int par;
};

// Filters one tile into the candidate buffer, compacting first if the
// tile's accepted elements would not fit.  p0 and c1 are absolute row
// positions; indices are stored relative to ibase.
template <int LAY, int VEC, bool FULL>
__device__ __forceinline__ void process_tile(Smem<LAY>& sm, const float (&x)[kElems], uint32_t p0, uint32_t c1,
                                             uint32_t ibase, uint32_t keep, Stream& st) {
  const uint32_t pbase = tile_pbase(p0, VEC);
  uint64_t bal[kElems];
  uint32_t before = 0;
  tile_accept<VEC, FULL>(x, pbase, c1, st.bf, bal);
  uint32_t total = tile_exchange<LAY>(sm, bal, st.par, before);
  if (st.cnt + total > (uint32_t)Shape<LAY>::kCap) {
    const uint64_t r = compact<LAY>(sm, st.cnt, keep, st.L);
    st.L = uni((uint32_t)r);
    st.cnt = uni((uint32_t)(r >> 32));
    st.bf = accept_floor(st.L);
    tile_accept<VEC, FULL>(x, pbase, c1, st.bf, bal);
    total = tile_exchange<LAY>(sm, bal, st.par, before);
  }
  if (total != 0) tile_append<LAY, VEC, FULL>(sm, x, bal, before, st.cnt, pbase, c1, st.bf, pbase - ibase);
  st.cnt += total;
}

// Per lane, the largest and the KK-th largest of its first nk sample keys
// (uniform nk of 2 * kElems; the others count as key 0, below every key):
// an insertion network over a descending list of the KK largest so far.
template <int KK>
__device__ __forceinline__ void lane_top(const uint32_t (&k)[2 * kElems], uint32_t nk, uint32_t& kth,
                                         uint32_t& top) {
  uint32_t t[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) t[i] = 0u;
#pragma unroll
  for (int j = 0; j < 2 * kElems; ++j) {
    const uint32_t v = (uint32_t)j < nk ? k[j] : 0u;
#pragma unroll
    for (int i = KK - 1; i > 0; --i) t[i] = max(t[i], min(t[i - 1], v));
    t[0] = max(t[0], v);
  }
  kth = t[KK - 1];
  top = t[0];
}

// The q-th largest of the wavefront's 64 values v (uniform; 1 <= q <= 64):
// the largest t that at least q lanes reach, found bit by bit from the top
// with one ballot per bit.  Used for q up to kKthLanes only: nearer to 64
// it is little above the smallest value and its 32 steps do not pay
// (decode and multi-token rows, q = 48: 13.0 -> 13.3 and 14.6 -> 15.3 us).
constexpr uint32_t kKthLanes = 32;
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, uint32_t q) {
  uint32_t t = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    t = popc64(ballot(v >= c)) >= q ? c : t;
  }
  return t;
}

// The interval the speculative bound's selection starts from (both ends
// uniform), over the first nk keys of every lane (all of them sample keys,
// so kk <= nk below).  hi is the largest sample key.  lo is a key that at
// least r sample keys reach, found without a selection.  Every lane takes
// its kk-th largest key a (kk = ceil(r / threads) at most 4; else its
// smallest key, kk = nk): it holds kk keys at or above a.  Every wavefront
// then takes the q-th largest a over its lanes, q = ceil(r / (W kk)) (the
// smallest when q > kKthLanes), and lo is the smallest of those: each wavefront holds
// q lanes with kk keys at or above it, W q kk >= r in all.  The r-th best
// key is therefore at least lo.  Keys below lo go to the sink, so the first
// pass spends its bins on the upper part of the sample, where the r-th best
// lies; taking the q-th largest lane instead of the smallest keeps the
// lanes whose keys happen to be low from widening the interval (an N(0, 1)
// sample at r = 192 keeps about 4% of its keys inside instead of 38%, and a
// quantised one no longer crowds its adds onto a few levels).  Contains one
// barrier.
template <int LAY>
__device__ __forceinline__ void sample_range(Smem<LAY>& sm, const uint32_t (&k)[2 * kElems], uint32_t nk,
                                             uint32_t r, uint32_t& lo, uint32_t& hi) {
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t kk = (r + (uint32_t)Shape<LAY>::kBlock - 1u) / (uint32_t)Shape<LAY>::kBlock;
  uint32_t a, b, kq;
  if (kk == 1u) {
    lane_top<1>(k, nk, a, b);
    kq = 1u;
  } else if (kk == 2u) {
    lane_top<2>(k, nk, a, b);
    kq = 2u;
  } else if (kk <= 4u) {
    lane_top<4>(k, nk, a, b);  // kk = 3 takes the 4th largest: a lower key that qualifies too
    kq = 4u;
  } else {
    a = 0xffffffffu;
    b = 0u;
#pragma unroll
    for (int j = 0; j < 2 * kElems; ++j) {
      if ((uint32_t)j < nk) {
        a = min(a, k[j]);
        b = max(b, k[j]);
      }
    }
    kq = nk;
  }
  const uint32_t q = (r + (uint32_t)W * kq - 1u) / ((uint32_t)W * kq);
  const uint32_t mn = q > kKthLanes ? wave_min(a) : wave_kth_largest(a, q);
  const uint32_t mx = wave_max(b);
  const int w = tid() >> 6;
  if ((tid() & 63) == 0) {
    sm.red[w] = mn;
    sm.red[W + w] = mx;
  }
  __syncthreads();
  uint32_t l = 0xffffffffu, h = 0u;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.red[4 * q]);
    const u32x4 y = *reinterpret_cast<const u32x4*>(&sm.red[W + 4 * q]);
    l = min(l, min(min(x.x, x.y), min(x.z, x.w)));
    h = max(h, max(max(y.x, y.y), max(y.z, y.w)));
  }
  lo = uni(l);
  hi = uni(h);
}

// Rank of the speculative bound in a sample of M elements of a row of n:
// r = max(kSpecMinRank, ceil(kSpecNum / kSpecDen * K * M / n)).
__device__ __forceinline__ uint32_t spec_rank(uint32_t K, uint32_t M, uint32_t n) {
  const uint64_t want = ((uint64_t)kSpecNum * K * M + (uint64_t)kSpecDen * n - 1) / ((uint64_t)kSpecDen * n);
  return want > kSpecMinRank ? (uint32_t)want : kSpecMinRank;
}

// One wavefront's part of a speculative bound: a key t that at least rw of
// its first nk sample keys per lane (k, all lanes) reach, and the largest of
// those keys (both uniform).  Everything stays inside the wavefront, with no
// workgroup barrier.  The interval starts at the q-th largest over lanes of
// each lane's kk-th largest key (kk = ceil(rw / 64), at most 4; else the
// smallest key, kk = nk; q = ceil(rw / kk)) and ends at the largest key;
// each pass histograms it into this
// wavefront's own kBins / W bins of hist1 and narrows it to the bin holding
// the rw-th best, until that bin may be taken whole (at most rw + rw / 8 + 8
// keys from it up) or holds one key; t is then the bin's lowest key.  The
// LDS serves one wavefront's instructions in order, so its reads see its
// adds; the bins are zero again on return.
template <int LAY>
__device__ __forceinline__ uint32_t wave_sample_bound(Smem<LAY>& sm, const uint32_t (&k)[2 * kElems], uint32_t nk,
                                                      uint32_t rw, uint32_t& wmax) {
  constexpr int W = Shape<LAY>::kWaves;
  constexpr int NB = kBins / W;
  constexpr uint32_t BITS = NB == 512 ? 9u : 8u;
  static_assert(NB == 512 || NB == 256, "four or eight wavefronts");
  const uint32_t kk = (rw + 63u) / 64u;
  uint32_t a, b, kq;
  if (kk == 1u) {
    lane_top<1>(k, nk, a, b);
    kq = 1u;
  } else if (kk == 2u) {
    lane_top<2>(k, nk, a, b);
    kq = 2u;
  } else if (kk <= 4u) {
    lane_top<4>(k, nk, a, b);
    kq = 4u;
  } else {
    a = 0xffffffffu;
    b = 0u;
#pragma unroll
    for (int j = 0; j < 2 * kElems; ++j) {
      if ((uint32_t)j < nk) {
        a = min(a, k[j]);
        b = max(b, k[j]);
      }
    }
    kq = nk;
  }
  // q lanes holding kq keys each at or above lo: q kq >= rw.
  const uint32_t q = (rw + kq - 1u) / kq;
  uint32_t lo = uni(q > kKthLanes ? wave_min(a) : wave_kth_largest(a, q));
  uint32_t hi = uni(wave_max(b));
  wmax = hi;
  uint32_t* const h = sm.hist1 + uni(tid() >> 6) * (uint32_t)NB;
  uint32_t* const sink = &sm.sink[tid() & 63];
  const uint32_t stop = rw + rw / 8u + 8u;
  uint32_t krem = rw, above = 0u;
  bool ok = true;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const uint32_t range = hi - lo;
    const uint32_t nbit = range != 0u ? 32u - (uint32_t)__builtin_clz(range) : 0u;
    const uint32_t sh = nbit > BITS ? nbit - BITS : 0u;
#pragma unroll
    for (int j = 0; j < 2 * kElems; ++j) {
      const uint32_t d = k[j] - lo;
      const bool in = (uint32_t)j < nk && d <= range;
      atomicAdd(in ? &h[d >> sh] : sink, 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const Found f = wave_find<NB>(h, krem);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (uint32_t i = tid() & 63u; i < (uint32_t)NB; i += 64u) h[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    ok = ok && f.ok != 0u;
    lo += f.bin << sh;
    const uint32_t width = (1u << sh) - 1u;
    hi = hi - lo > width ? lo + width : hi;
    if (!ok || sh == 0u || above + f.above + f.in_bin <= stop) break;
    above += f.above;
    krem -= f.above;
  }
  return ok ? lo : 0u;
}

// The speculative bound for a row of n elements whose first two tiles are
// in x0 and x1 (n >= kSpecMinLen): the key of (about) the r-th best of those
// M = 2 * kTile elements (4096, 8192 or 16384 by workgroup width), r =
// spec_rank(K, M, n).  When that r reaches K (the two tiles are too large a
// share of the row) the sample is the first tile alone, M = kTile, and if r
// still reaches K there is no bound (0).  The bin holding the r-th best is taken whole
// when it is small, which only lowers the bound.  The caller checks at the
// end of the row that at least K elements reached the bound and streams the
// row again without it if not; when the check passes, every element below
// the bound is beaten by at least K others.  Runs on register-held keys
// while the next tiles' loads are in flight.  Leaves the histograms zero.
// With top, also gives the sample's largest raw_key (uniform).
//
// WAVES (a row streamed wave by wave by one 512-thread workgroup): each
// wavefront takes a bound from its own part of the sample instead, with no
// workgroup barrier but the one that combines them (a lone row's decode and
// multi-token rows 13.6 -> 13.3 us and 15.0 -> 14.8 us on MI355X).  The
// lowest of the per-wave bounds admits about a fifth more candidates than
// the shared selection; where rows share a CU (256 threads: prefill-shaped
// batch 190 -> 224 us) or rows have heavy ties (cooperative long rows
// 18.0 -> 19.7 us) that cost more than the barriers it saves.
template <int LAY, bool WAVES = false>
__device__ __forceinline__ uint32_t spec_bound(Smem<LAY>& sm, float (&x0)[kElems], float (&x1)[kElems], uint32_t n,
                                               uint32_t K, uint32_t* top = nullptr) {
  constexpr uint32_t M = 2u * (uint32_t)Shape<LAY>::kTile;
  uint32_t r = spec_rank(K, M, n);
  const bool one = r >= K;
  if (one) r = spec_rank(K, M / 2u, n);
  if (r >= K) return 0u;
  // The keys replace the values in place (registers are scarce here) and
  // are turned back afterwards, bit for bit: raw_key keeps -0.0 apart from
  // +0.0 (just below it), which only a bound of exactly zero can see, and
  // both floats of that bound accept both zeros.
  uint32_t k[2 * kElems];
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    k[e] = raw_key(__float_as_uint(x0[e]));
    k[kElems + e] = raw_key(__float_as_uint(x1[e]));
  }
  if constexpr (WAVES && Shape<LAY>::kWaves == 8) {
    // Every wavefront finds a bound on its own part of the sample, reached
    // by ceil(r / W) of its keys; the row's bound is the lowest of them, so
    // at least r sample keys reach it.  One barrier in all; each wavefront
    // cleared its own bins.
    constexpr int W = Shape<LAY>::kWaves;
    uint32_t wmax = 0u;
    const uint32_t t = wave_sample_bound<LAY>(sm, k, one ? kElems : 2u * kElems, (r + W - 1u) / W, wmax);
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
      x0[e] = __uint_as_float(key_bits(k[e]));
      x1[e] = __uint_as_float(key_bits(k[kElems + e]));
    }
    const uint32_t w = tid() >> 6;
    if ((tid() & 63) == 0) {
      sm.bnd[w] = t;
      sm.bnd[W + w] = wmax;
    }
    __syncthreads();
    uint32_t l = 0xffffffffu, h = 0u;
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.bnd[4 * q]);
      const u32x4 y = *reinterpret_cast<const u32x4*>(&sm.bnd[W + 4 * q]);
      l = min(l, min(min(x.x, x.y), min(x.z, x.w)));
      h = max(h, max(max(y.x, y.y), max(y.z, y.w)));
    }
    if (top != nullptr) *top = uni(h);
    return uni(l);
  }
  Slice sl;  // the keys live only in registers: every lane holds 16 slots, 8 or 16 of them sample keys
  sl.ws = 0u;
  sl.sp = 2u * kElems;
  sl.nv = one ? kElems : 2u * kElems;
  uint32_t lo, hi;
  sample_range<LAY>(sm, k, sl.nv, r, lo, hi);
  const Sel s = range_select<LAY, 2 * kElems>(sm, k, sl, lo, hi, r, r + r / 8u + 8u);
  if (top != nullptr) *top = hi;
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    x0[e] = __uint_as_float(key_bits(k[e]));
    x1[e] = __uint_as_float(key_bits(k[kElems + e]));
  }
  __syncthreads();  // every wave is done with the histograms
  clear_hists(sm);
  return s.ok ? s.lo : 0u;
}

// Streams [c0, c1) through the filter.  Full tiles come through a ring of
// kPrefetch register buffers: the load for tile j + kPrefetch - 1 is issued
// before tile j is processed, so about (kPrefetch - 1) tiles per workgroup
// are in flight.  Prefetch addresses past the last full tile are clamped to
// it (a cache hit), which keeps the load pattern identical every iteration.
// The partial last tile is loaded with per-element bounds checks.
//
// spec = the row length (>= kSpecMinLen) to start from a speculative bound
// taken from the first two tiles (see spec_bound), else 0.  Those two tiles
// go through x0 and x1 ahead of the ring, which starts at tile 2 with its
// loads issued before the bound is computed; with preloaded they were
// already loaded by the caller.
template <int LAY, int VEC, typename T>
__device__ __forceinline__ void stream_chunk(Smem<LAY>& sm, const T* __restrict__ rowp, uint32_t c0,
                                             uint32_t c1, uint32_t keep, uint32_t& cnt, uint32_t& L,
                                             uint32_t spec, float (&x0)[kElems], float (&x1)[kElems],
                                             bool preloaded) {
  constexpr int PF = kPrefetch;
  constexpr int NT = Shape<LAY>::kBlock;
  constexpr uint32_t kTile = (uint32_t)Shape<LAY>::kTile;
  c0 = uni(c0);
  c1 = uni(c1);
  Stream st;
  st.cnt = uni(cnt);
  st.L = uni(L);
  st.bf = accept_floor(st.L);
  st.par = 0;
  const uint32_t F = (c1 - c0) / kTile;  // full tiles
  const T* base = rowp + c0;
  const bool pre = uni(spec) != 0u && F >= 2u;
  const uint32_t j1 = pre ? 2u : 0u;  // first tile of the ring
  if (pre && !preloaded) {
    load_full<VEC>(base, x0);
    load_full<VEC>(base + kTile, x1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (F > j1) {
    float buf[PF][kElems];
#pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
      load_full<VEC>(base + (j1 + (uint32_t)s < F ? j1 + (uint32_t)s : F - 1) * kTile, buf[s]);
      __builtin_amdgcn_sched_barrier(0);  // keep tiles in issue order: waits then retire oldest first
    }
    if (pre) {
      st.L = uni(spec_bound<LAY>(sm, x0, x1, uni(spec), keep));
      st.bf = accept_floor(st.L);
      process_tile<LAY, VEC, true>(sm, x0, c0, c1, c0, keep, st);
      process_tile<LAY, VEC, true>(sm, x1, c0 + kTile, c1, c0, keep, st);
    }
    // Whole rounds of PF tiles: one uniform back edge, so the compiler's
    // load-counter waits stay exact (retire only the tile about to be used).
    const uint32_t Fr = j1 + (F - j1) - (F - j1) % PF;
    for (uint32_t j0 = j1; j0 < Fr; j0 += PF) {
#pragma unroll
      for (int slot = 0; slot < PF; ++slot) {
        const uint32_t j = j0 + slot;
        const uint32_t jn = j + PF - 1 < F ? j + PF - 1 : F - 1;
        load_full<VEC>(base + jn * kTile, buf[(slot + PF - 1) % PF]);
        __builtin_amdgcn_sched_barrier(0);
        process_tile<LAY, VEC, true>(sm, buf[slot], c0 + j * kTile, c1, c0, keep, st);
      }
    }
    // The last (F - j1) % PF full tiles are already in buf[0..]: no more loads.
#pragma unroll
    for (int slot = 0; slot < PF - 1; ++slot) {
      const uint32_t j = Fr + slot;
      if (j < F) process_tile<LAY, VEC, true>(sm, buf[slot], c0 + j * kTile, c1, c0, keep, st);
    }
  } else if (pre) {
    // Exactly two full tiles: no ring, no bound worth taking.
    process_tile<LAY, VEC, true>(sm, x0, c0, c1, c0, keep, st);
    process_tile<LAY, VEC, true>(sm, x1, c0 + kTile, c1, c0, keep, st);
  }
  const uint32_t pt = c0 + F * kTile;
  if (pt < c1) {
    float x[kElems];
    load_tail<VEC>(rowp, c1, pt, x);
    process_tile<LAY, VEC, false>(sm, x, pt, c1, c0, keep, st);
  }
  __syncthreads();
  cnt = st.cnt;
  L = st.L;
}

// ---------------------------------------------------------------------------
// Wave-by-wave streaming of a row with a speculative bound
//
// Rows long enough to speculate (see spec_bound) usually end with a few
// thousand candidates.  Each of the W wavefronts then streams its own
// contiguous segment (a quarter of the row for W = 4) into its own part of
// the buffer, with positions from its own ballots: no per-tile exchange
// between wavefronts and no per-tile barrier.  The segments are contiguous in
// index order, so the buffer read part by part is in index order too.  If a wavefront's quarter of the
// buffer would overflow (or the bound turns out too high) the row is
// streamed again on the general path.
// ---------------------------------------------------------------------------


// Elements per wavefront segment of a chunk of n, W wavefronts: whole wave
// tiles (the cooperative chunks; the last segments may be short or empty).
template <int W>
__device__ __forceinline__ uint32_t segment_of(uint32_t n) {
  const uint32_t q = (n + W - 1) / W;
  return (q + kWaveTile - 1) / kWaveTile * kWaveTile;
}

// Wave segments of a whole row of n elements.  Normally every wavefront but
// the last takes segment_of(n) elements (whole wave tiles, rounded up) and
// the last takes the rest: the last wavefront, issued last, gets the least
// work, which evens out finishing times since the oldest waves of a SIMD win
// its issue slots.  When that would leave the last segment without the two
// full wave tiles of the sample, the row's T = n / kWaveTile full tiles are
// dealt out evenly instead (wavefront w starts at tile ceil(w T / W)), with
// the partial tile at the end going to the last wavefront: every segment
// then holds at least floor(T / W) full tiles.
template <int W>
__device__ __forceinline__ bool even_segments(uint32_t n) {
  return n < (uint32_t)(W - 1) * segment_of<W>(n) + 2u * kWaveTile;
}
template <int W>
__device__ __forceinline__ uint32_t seg_begin(uint32_t n, uint32_t w) {
  if (even_segments<W>(n)) return ((w * (n / kWaveTile) + (uint32_t)W - 1u) / (uint32_t)W) * kWaveTile;
  return w * segment_of<W>(n);
}
template <int W>
__device__ __forceinline__ uint32_t seg_end(uint32_t n, uint32_t w) {
  return w + 1u == (uint32_t)W ? n : seg_begin<W>(n, w + 1u);
}

// Whether a row of n elements (n > K) goes wave by wave: long enough to
// speculate, every segment holding the two full wave tiles of the sample
// (at least 2W full wave tiles in all), and a speculative rank below K.
template <int LAY>
__device__ __forceinline__ bool wave_mode(uint32_t n, uint32_t K) {
  constexpr uint32_t W = (uint32_t)Shape<LAY>::kWaves;
  if (n < kSpecMinLen) return false;
  if (n / kWaveTile < 2u * W) return false;
  return spec_rank(K, (uint32_t)Shape<LAY>::kTile, n) < K;  // a bound from one or two tiles
}

// One full wave tile at `tile` (wave-uniform): lane l loads elements
// u * 64 * VEC + l * VEC .. + VEC - 1.
template <int VEC, bool NT = true, typename T>
__device__ __forceinline__ void load_wave_full(const T* __restrict__ tile, float (&x)[kElems]) {
  const uint32_t l = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u)
    load_run<VEC, NT>(tile + (uint32_t)u * (64u * VEC) + l * VEC, x, u * VEC);
}

// The partial last wave tile [p0, end): nothing read at or past end.
template <int VEC, typename T>
__device__ __forceinline__ void load_wave_tail(const T* __restrict__ rowp, uint32_t end, uint32_t p0,
                                               float (&x)[kElems]) {
  const uint32_t l = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kElems / VEC; ++u) {
    const uint32_t pos = p0 + (uint32_t)u * (64u * VEC) + l * VEC;
#pragma unroll
    for (int c = 0; c < VEC; ++c) x[u * VEC + c] = (pos + c < end) ? widen(rowp[pos + c]) : 0.0f;
  }
}

// Filters one wave tile (row positions p0 + ...) into this wavefront's part
// of the buffer, slots sub0 + [0, SUB), after its cnt entries.  If the tile's
// accepted elements would not fit, sets ovf and appends nothing from then on.
template <int LAY, int VEC, bool FULL>
__device__ __forceinline__ void wave_tile(Smem<LAY>& sm, const float (&x)[kElems], uint32_t p0, uint32_t end, float bf,
                                          uint32_t sub0, uint32_t& cnt, bool& ovf) {
  constexpr uint32_t SUB = (uint32_t)Shape<LAY>::kCap / Shape<LAY>::kWaves;
  constexpr int NL = kElems / VEC;
  const uint32_t pbase = p0 + (threadIdx.x & 63) * VEC;
  uint64_t bal[kElems];
  uint32_t total = 0;
#pragma unroll
  for (int e = 0; e < kElems; ++e) {
    const int u = e / VEC, c = e % VEC;
    const bool in = FULL || pbase + (uint32_t)u * (64u * VEC) + c < end;
    bal[e] = ballot(in && x[e] >= bf);
    total += popc64(bal[e]);
  }
  if (ovf || cnt + total > SUB) {
    ovf = true;
    return;
  }
  uint32_t r0 = sub0 + cnt;
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    uint32_t r = r0;
#pragma unroll
    for (int c = 0; c < VEC; ++c) r = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[u * VEC + c] >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal[u * VEC + c], r));
    if constexpr (Smem<LAY>::kDiscard != 0) {
      // Wide workgroups: every lane stores every element, the ones it does
      // not keep to its own discard word.  Positions are kept as byte
      // offsets, which both arrays share (32-bit entries), so an element
      // costs a select, its index, one paired store and the running add.
      static_assert(sizeof(typename Shape<LAY>::Idx) == 4, "wide layouts keep 32-bit indices");
      uint32_t rb = r * 4u;
      const uint32_t db = ((uint32_t)Shape<LAY>::kCap + (threadIdx.x & 63)) * 4u;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const int e = u * VEC + c;
        const uint32_t pos = pbase + (uint32_t)u * (64u * VEC) + c;
        const bool take = (FULL || pos < end) && x[e] >= bf;
        const uint32_t d = take ? rb : db;
        *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(sm.val) + d) = __float_as_uint(x[e]);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(sm.idx) + d) = pos;
        rb += take ? 4u : 0u;
      }
    } else {
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const int e = u * VEC + c;
        const uint32_t pos = pbase + (uint32_t)u * (64u * VEC) + c;
        const bool take = (FULL || pos < end) && x[e] >= bf;
        if (take) {
          sm.val[r] = __float_as_uint(x[e]);
          sm.idx[r] = (typename Shape<LAY>::Idx)pos;
        }
        r += take ? 1u : 0u;
      }
    }
#pragma unroll
    for (int c = 0; c < VEC; ++c) r0 += popc64(bal[u * VEC + c]);
  }
  cnt += total;
}

// After a wave-by-wave stream: every wavefront's candidate count and overflow
// flag are shared; returns whether any wavefront overflowed, with the sum of
// the counts in all and the counts of lower wavefronts in before (all
// wave-uniform).  pre() runs before the exchange's barrier, so what it
// writes to LDS is shared by the same barrier.  One barrier: sm.wcnt is
// written again only by the next row's stream, after the barriers between.
struct NoPre {
  __device__ void operator()() const {}
};

template <int LAY, typename Pre = NoPre>
__device__ __forceinline__ bool wave_counts(Smem<LAY>& sm, uint32_t w, uint32_t cnt, bool ovf, uint32_t& all,
                                            uint32_t& before, const Pre& pre = Pre{}) {
  constexpr int W = Shape<LAY>::kWaves;
  if ((threadIdx.x & 63) == 0) {
    sm.wcnt[w] = cnt;
    sm.wcnt[W + w] = ovf ? 1u : 0u;
  }
  pre();
  __syncthreads();
  uint32_t a = 0, b = 0, o = 0;
#pragma unroll
  for (int q = 0; q < W / 4; ++q) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(&sm.wcnt[4 * q]);
    const u32x4 f = *reinterpret_cast<const u32x4*>(&sm.wcnt[W + 4 * q]);
    const uint32_t v[4] = {uni(c.x), uni(c.y), uni(c.z), uni(c.w)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a += v[i];
      b += ((uint32_t)(4 * q + i) < w) ? v[i] : 0u;
    }
    o |= uni(f.x | f.y | f.z | f.w);
  }
  all = a;
  before = b;
  return o != 0u;
}

// Streams row [0, n) wave by wave (wave_mode(n, K) holds; indices fit the
// buffer's index type).  x0 / x1 carry each wavefront's first two wave tiles
// (already loaded when preloaded); together they sample 2 * kTile elements
// from the W segments for the speculative bound.  Returns false if the row must
// be streamed again on the general path; otherwise mine is this
// wavefront's number of candidates (in slots [w * SUB, w * SUB + mine)) and
// hint says where their keys lie.  pre() runs before the closing exchange's
// barrier (see wave_counts).
template <int LAY, int VEC, typename T, typename Pre>
__device__ __forceinline__ bool stream_row_waves(Smem<LAY>& sm, const T* __restrict__ rowp, uint32_t n,
                                                 uint32_t K, float (&x0)[kElems], float (&x1)[kElems],
                                                 bool preloaded, uint32_t& mine, Hint& hint, const Pre& pre) {
  constexpr int PF = kPrefetch;
  constexpr uint32_t WT = kWaveTile;
  constexpr int W = Shape<LAY>::kWaves;
  constexpr uint32_t SUB = (uint32_t)Shape<LAY>::kCap / W;
  n = uni(n);
  K = uni(K);
  const uint32_t w = uni(threadIdx.x >> 6);
  const uint32_t qs = uni(seg_begin<W>(n, w));
  const uint32_t qe = uni(seg_end<W>(n, w));
  const T* qp = rowp + qs;
  if (!preloaded) {
    load_wave_full<VEC>(qp, x0);
    load_wave_full<VEC>(qp + WT, x1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // wave_mode(n, K): every segment holds at least two full wave tiles, F >= 2.
  const uint32_t F = (qe - qs) / WT;
  float buf[PF][kElems];
#pragma unroll
  for (int s = 0; s < PF - 1; ++s) {
    load_wave_full<VEC>(qp + (2u + (uint32_t)s < F ? 2u + (uint32_t)s : F - 1) * WT, buf[s]);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t top = 0u;
  const uint32_t L = uni(spec_bound<LAY, true>(sm, x0, x1, n, K, &top));
  hint = stream_hint(L, uni(top));
  const float bf = accept_floor(L);
  const uint32_t sub0 = w * SUB;
  uint32_t cnt = 0;
  bool ovf = L == 0u;  // no bound: the quarters of the buffer could not hold the row
  wave_tile<LAY, VEC, true>(sm, x0, qs, qe, bf, sub0, cnt, ovf);
  wave_tile<LAY, VEC, true>(sm, x1, qs + WT, qe, bf, sub0, cnt, ovf);
  const uint32_t Fr = F - (F - 2u) % PF;
  for (uint32_t j0 = 2; j0 < Fr; j0 += PF) {
#pragma unroll
    for (int slot = 0; slot < PF; ++slot) {
      const uint32_t j = j0 + slot;
      const uint32_t jn = j + PF - 1 < F ? j + PF - 1 : F - 1;
      load_wave_full<VEC>(qp + jn * WT, buf[(slot + PF - 1) % PF]);
      __builtin_amdgcn_sched_barrier(0);
      wave_tile<LAY, VEC, true>(sm, buf[slot], qs + j * WT, qe, bf, sub0, cnt, ovf);
    }
  }
#pragma unroll
  for (int slot = 0; slot < PF - 1; ++slot) {
    const uint32_t j = Fr + slot;
    if (j < F) wave_tile<LAY, VEC, true>(sm, buf[slot], qs + j * WT, qe, bf, sub0, cnt, ovf);
  }
  const uint32_t pt = qs + F * WT;
  if (pt < qe) {
    float x[kElems];
    load_wave_tail<VEC>(rowp, qe, pt, x);
    wave_tile<LAY, VEC, false>(sm, x, pt, qe, bf, sub0, cnt, ovf);
  }
  uint32_t all = 0, before = 0;
  const bool bad = wave_counts<LAY>(sm, w, cnt, ovf, all, before, pre);
  mine = cnt;
  return !bad && all >= K;
}

// Workspace traffic between the workgroups of a row goes only through
// agent-scope atomic operations (loads, stores, adds), which are coherent at
// device scope on their own; no cache-wide write-back or invalidate is
// needed.  Ordering: a writer wave waits until all its atomics have completed
// before the workgroup arrives at the barrier, and readers issue their loads
// only after seeing the arrival count.
__device__ __forceinline__ uint32_t ws_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// A chunk of a row, wave by wave (the cooperative kernel's first pass)
//
// Every workgroup of a row takes the same speculative bound: from the same
// sample (the first two wave tiles of each wave segment of the whole row,
// the sample a row streamed wave by wave in one workgroup uses) through the
// same integer selection.  A chunk keeps every element of its range at or
// above the bound, wave by wave.
// ---------------------------------------------------------------------------

// Streams [c0, c1) of a row of n elements wave by wave, each wavefront its
// own quarter of the range, from the row's speculative bound (returned in
// L; 0 if none could be taken).  x0 / x1 hold the row's sample (loaded here
// unless preloaded).  Returns false if a wavefront's part of the buffer
// overflowed; otherwise mine / off are this wavefront's candidate count and
// its offset among the chunk's total (in slots [w * SUB, w * SUB + mine)).
// hint says where the keys of the row's candidates lie.
template <int LAY, int VEC, typename T>
__device__ __forceinline__ bool stream_range_waves(Smem<LAY>& sm, const T* __restrict__ rowp, uint32_t n,
                                                   uint32_t K, uint32_t c0, uint32_t c1, float (&x0)[kElems],
                                                   float (&x1)[kElems], bool preloaded, uint32_t& mine,
                                                   uint32_t& off, uint32_t& total, uint32_t& L, Hint& hint) {
  constexpr int PF = kPrefetch;
  constexpr uint32_t WT = kWaveTile;
  constexpr int W = Shape<LAY>::kWaves;
  constexpr uint32_t SUB = (uint32_t)Shape<LAY>::kCap / W;
  n = uni(n);
  K = uni(K);
  c0 = uni(c0);
  c1 = uni(c1);
  const uint32_t w = uni(threadIdx.x >> 6);
  if (!preloaded) {
    // Every workgroup of the row reads this sample: through L2.
    const T* sp = rowp + seg_begin<W>(n, w);
    load_wave_full<VEC, false>(sp, x0);
    load_wave_full<VEC, false>(sp + WT, x1);
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t q = segment_of<W>(c1 - c0);
  const uint32_t qs = c0 + w * q;  // at or past c1 when the range has fewer segments
  const uint32_t qe = qs + q < c1 ? qs + q : c1;
  const uint32_t F = qe > qs ? (qe - qs) / WT : 0u;
  const T* qp = rowp + qs;
  float buf[PF][kElems];
  if (F > 0u) {
#pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
      load_wave_full<VEC>(qp + ((uint32_t)s < F ? (uint32_t)s : F - 1) * WT, buf[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  uint32_t top = 0u;
  L = uni(spec_bound<LAY>(sm, x0, x1, n, K, &top));
  hint = stream_hint(L, uni(top));
  const float bf = accept_floor(L);
  const uint32_t sub0 = w * SUB;
  uint32_t cnt = 0;
  bool ovf = L == 0u;
  const uint32_t Fr = F - F % PF;
  for (uint32_t j0 = 0; j0 < Fr; j0 += PF) {
#pragma unroll
    for (int slot = 0; slot < PF; ++slot) {
      const uint32_t j = j0 + slot;
      const uint32_t jn = j + PF - 1 < F ? j + PF - 1 : F - 1;
      load_wave_full<VEC>(qp + jn * WT, buf[(slot + PF - 1) % PF]);
      __builtin_amdgcn_sched_barrier(0);
      wave_tile<LAY, VEC, true>(sm, buf[slot], qs + j * WT, qe, bf, sub0, cnt, ovf);
    }
  }
#pragma unroll
  for (int slot = 0; slot < PF - 1; ++slot) {
    const uint32_t j = Fr + slot;
    if (j < F) wave_tile<LAY, VEC, true>(sm, buf[slot], qs + j * WT, qe, bf, sub0, cnt, ovf);
  }
  const uint32_t pt = qs + F * WT;
  if (pt < qe) {
    float x[kElems];
    load_wave_tail<VEC>(rowp, qe, pt, x);
    wave_tile<LAY, VEC, false>(sm, x, pt, qe, bf, sub0, cnt, ovf);
  }
  const bool bad = wave_counts<LAY>(sm, w, cnt, ovf, total, off);
  mine = cnt;
  return !bad;
}

// Row r of the scores, as elements of type T.
template <typename T>
__device__ __forceinline__ const T* row_of(const KernelParams& p, int64_t r) {
  return static_cast<const T*>(p.scores) + r * p.row_stride;
}

__device__ __forceinline__ int64_t clamp_len(const KernelParams& p, int row) {
  int64_t n = p.lengths[row];
  n = n < 0 ? 0 : n;
  return n > p.row_stride ? p.row_stride : n;
}

// n <= K: every valid index (plus the row's offset), then -1.  Reads no scores.
// With vout, the n scores themselves (read from rowp, as fp32) and -inf after them.
template <int NT, typename T = float>
__device__ __forceinline__ void write_all_then_pad(int32_t* out, int64_t n, int K, uint32_t off,
                                                   float* vout = nullptr, const T* rowp = nullptr) {
  for (int i = threadIdx.x; i < K; i += NT) {
    out[i] = i < n ? (int32_t)(off + (uint32_t)i) : -1;
    if (vout != nullptr) vout[i] = i < n ? widen(rowp[i]) : -__builtin_huge_valf();
  }
}

// What a row's chosen indices are shifted by in the output: its offset in a
// flat ragged layout when the caller gives row offsets, else 0.
__device__ __forceinline__ uint32_t offset_of(const KernelParams& p, int row) {
  return p.row_offsets != nullptr ? (uint32_t)p.row_offsets[row] : 0u;
}

template <int LAY>
__device__ __forceinline__ void zero_histograms(Smem<LAY>& sm) {
  clear_hists(sm);
}

// ---------------------------------------------------------------------------
// One workgroup per row, persistent over rows.
//
// Workgroup b takes row b first.  With a workspace every later row comes
// from a ticket counter, so workgroups that run faster -- the hardware
// favours the oldest waves -- take more rows, evening out the end of the
// launch.  Each workgroup draws its next ticket when it starts a row, hiding
// the atomic's latency behind the row, and stops at the first ticket past
// the last row.  Without a workspace row b + k * gridDim.x is taken in turn.
// ---------------------------------------------------------------------------

// VALS: the launch also writes the chosen scores (compiled out otherwise: it
// costs registers the row loop needs).
// T: the score type (float, or uint16_t holding bf16).
template <int VEC, int LAY, bool VALS, typename T>
__global__ void __launch_bounds__(Shape<LAY>::kBlock, Shape<LAY>::kWavesPerSimd) topk_single_kernel(KernelParams p) {
  constexpr int NT = Shape<LAY>::kBlock;
  constexpr int W = Shape<LAY>::kWaves;
  __shared__ Smem<LAY> sm;
  zero_histograms(sm);
  __syncthreads();
  const uint32_t K = (uint32_t)p.K;
  const uint32_t U = (uint32_t)p.num_rows;
  uint32_t* ticket = p.ws != nullptr ? reinterpret_cast<uint32_t*>(p.ws + kTicketOff) : nullptr;
  uint32_t redo = 0u;  // 1 while a row is streamed again after a failed speculation
  uint32_t next = 0u;  // thread 0: the row after this one
  bool drawn = false;  // thread 0: next is set for the current row
  uint32_t row = blockIdx.x;
  bool first_row = true;
  // Every row draws its successor when it starts, so the atomic's latency
  // hides behind the row.  The first row's successor is fixed (row + grid):
  // at launch every workgroup would hit the counter at once, and at the end
  // of the first rows, which end close together, nearly as many.  Tickets
  // therefore start at two grids; U - grid draws are made in all (each
  // workgroup with a second row draws until it gets no row), and the last
  // one resets the counter.
  auto draw = [&]() {
    if (threadIdx.x == 0 && !drawn) {
      if (ticket != nullptr && !first_row) {
        const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t == U - gridDim.x - 1u) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        next = 2u * gridDim.x + t;
      } else {
        next = row + gridDim.x;
      }
      drawn = true;
    }
  };
  // The next row's first tiles (or its sample) are loaded before this row's
  // final selection, so that their latency hides behind it.
  bool have_pre = false;
  float x0[kElems], x1[kElems];
  int64_t n = row < U ? clamp_len(p, (int)row) : 0;
  uint32_t off = row < U ? uni(offset_of(p, (int)row)) : 0u;
  // Thread 0 shares the next row, its length and offset through LDS.
  auto publish_next = [&]() {
    draw();
    if (threadIdx.x == 0) {
      uint32_t nn = 0u;
      if (next < U) {
        nn = (uint32_t)clamp_len(p, (int)next);
        sm.acc[13] = offset_of(p, (int)next);
      }
      sm.acc[8] = next < U ? next : U;
      sm.acc[9] = nn;
    }
  };
  while (row < U) {
    draw();
    int32_t* out = p.out + (int64_t)row * p.K;
    uint32_t cnt = 0;
    bool waved = false;  // the candidates sit wave by wave
    bool shared = false;  // the next row went out with the stream's closing exchange
    Hint hint{0u, 0u, false};
    bool select = false;
    if (n <= (int64_t)K) {
      if constexpr (VALS)
        write_all_then_pad<NT, T>(out, n, p.K, off, p.out_val + (int64_t)row * p.K, row_of<T>(p, row));
      else
        write_all_then_pad<NT>(out, n, p.K, off);
    } else {
      const T* rowp = row_of<T>(p, row);
      uint32_t gL = 0;  // general path: starting bound
      if (!redo && wave_mode<LAY>((uint32_t)n, K)) {
        waved = stream_row_waves<LAY, VEC>(sm, rowp, (uint32_t)n, K, x0, x1, have_pre, cnt, hint, publish_next);
        shared = true;
        have_pre = false;
        if (!waved) {
          // A wavefront's part of the buffer overflowed, or fewer than K
          // elements reached the speculative bound: stream the row again on
          // the general path, without speculating.
          redo = 1u;
          continue;
        }
      } else {
        const uint32_t spec = (redo || n < (int64_t)kSpecMinLen) ? 0u : (uint32_t)n;
        stream_chunk<LAY, VEC>(sm, rowp, 0u, (uint32_t)n, K, cnt, gL, spec, x0, x1, have_pre);
        have_pre = false;
        if (cnt < K && !redo) {
          // Fewer than K elements reached the speculative bound: it was above
          // the K-th best.  Stream the same row again without speculating.
          redo = 1u;
          __syncthreads();
          continue;
        }
      }
      select = true;
      redo = 0u;
    }
    if (!shared) {
      publish_next();
      __syncthreads();
    }
    const uint32_t nrow = uni(sm.acc[8]);
    const int64_t nn = (int64_t)uni(sm.acc[9]);
    const uint32_t noff = uni(sm.acc[13]);
    if (nrow < U && nn >= (int64_t)kSpecMinLen && nn > (int64_t)K) {
      // The next row's first two tiles: per wave segment (the row's sample)
      // when it will go wave by wave, else the row's first two tiles.
      const T* nrowp = row_of<T>(p, nrow);
      if (wave_mode<LAY>((uint32_t)nn, K)) {
        const T* qp = nrowp + seg_begin<W>((uint32_t)nn, uni(threadIdx.x >> 6));
        load_wave_full<VEC>(qp, x0);
        load_wave_full<VEC>(qp + kWaveTile, x1);
      } else {
        load_full<VEC>(nrowp, x0);
        load_full<VEC>(nrowp + Shape<LAY>::kTile, x1);
      }
      have_pre = true;
    }
    if (select) {
      // The hint only for the wide workgroups: the 256-thread instances are
      // held to 128 VGPRs, and carrying it spills there.
      final_select<LAY>(sm, waved ? wave_slice<LAY>(cnt) : plain_slice<LAY>(cnt), K, out, off,
                        VALS ? p.out_val + (int64_t)row * p.K : nullptr,
                        W > 4 ? hint : Hint{0u, 0u, false});
    }
    first_row = false;
    drawn = false;
    row = nrow;
    n = nn;
    off = noff;
    __syncthreads();  // every thread has read the next row before it is overwritten
  }
}

// ---------------------------------------------------------------------------
// Several workgroups per row, cooperating through the workspace.
// ---------------------------------------------------------------------------

// Arrival barrier of the workgroups sharing a row: every wave drains its
// outstanding memory operations, one thread arrives and polls.  A wait that
// exceeds spin_limit polls sets an error bit and returns, so no wave can
// wait forever.
__device__ void group_barrier(uint32_t* ctr, uint32_t target, uint32_t spin_limit, uint32_t* err) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    ws_add(ctr, 1u);
    uint32_t polls = 0;
    while (ws_load(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls > spin_limit) {
        __hip_atomic_fetch_or(err, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// The waiting half of group_barrier, for a workgroup that has already
// arrived: one thread polls until the count reaches target (bounded as
// above), then the workgroup proceeds.
__device__ void group_wait(const uint32_t* ctr, uint32_t target, uint32_t spin_limit, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t polls = 0;
    while (ws_load(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls > spin_limit) {
        __hip_atomic_fetch_or(err, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Gathers the chunks' published candidates of a row, in chunk order (so in
// index order), into buffer positions [0, total): chunk gg's entries sit at
// lists + gg * CAP (fp32 bits) and + pub (row indices), and go to merged
// positions [s_off[gg], s_off[gg + 1]) (s_off ascending, s_off[0] = 0, grow
// chunks, total = s_off[grow] <= the buffer capacity).  First every merged
// position's source offset is written into the buffer (wavefront w takes
// chunks w, w + W, ..., its lanes 64 positions at a time; the chunk bounds
// come from registers, so nothing waits on LDS); then each thread reads its
// positions' offsets and issues all its workspace loads back to back, with
// no branch between them, so the gather costs about one round trip; the
// values go to the buffer last.
template <int LAY>
__device__ __forceinline__ void gather_union(Smem<LAY>& sm, const uint32_t* lists, uint32_t pub, const uint32_t* s_off,
                                             int grow, uint32_t total) {
  constexpr int S = Shape<LAY>::kSlots;
  constexpr uint32_t NT = (uint32_t)Shape<LAY>::kBlock;
  constexpr uint32_t CAP = (uint32_t)Shape<LAY>::kCap;
  using Idx = typename Shape<LAY>::Idx;
  constexpr int W = Shape<LAY>::kWaves;
  const uint32_t t = tid();
  // Every merged position's source word goes into the buffer's value array
  // first (it is overwritten last).  The chunk bounds are read once, lane gg
  // of each wavefront holding s_off[gg], so the loop waits on nothing.
  const uint32_t lane = t & 63u;
  const int w = (int)uni(t >> 6);
  const uint32_t bound = lane < (uint32_t)grow ? s_off[lane] : 0u;  // grow <= 64 chunk starts
  for (int gg = w; gg < grow; gg += W) {
    const uint32_t o = lane_value(bound, gg);
    const uint32_t e = gg + 1 < grow ? lane_value(bound, gg + 1) : total;
    const uint32_t src = (uint32_t)gg * CAP - o;
    for (uint32_t i = o + lane; i < e; i += 64u) sm.val[i] = src + i;
  }
  __syncthreads();
  uint32_t vb[S], vi[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const uint32_t i = t + (uint32_t)j * NT;
    const uint32_t a = i < total ? sm.val[i] : 0u;
    vb[j] = ws_load(lists + a);
    vi[j] = ws_load(lists + a + pub);
  }
  __syncthreads();  // every position's address has been read before the buffer is overwritten
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const uint32_t i = t + (uint32_t)j * NT;
    if (i < total) {
      sm.val[i] = vb[j];
      sm.idx[i] = (Idx)vi[j];
    }
  }
}

// Zeroes the published candidates of a row's grow chunks (positions as in
// gather_union): wavefront w takes chunks w, w + W, ..., with the chunk
// bounds in registers as in gather_union.
template <int NT>
__device__ __forceinline__ void clear_union(uint32_t* lists, uint32_t cap, uint32_t pub, const uint32_t* s_off,
                                            int grow) {
  constexpr int W = NT / 64;
  const uint32_t lane = threadIdx.x & 63u;
  const int w = (int)uni(threadIdx.x >> 6);
  const uint32_t bound = lane < (uint32_t)grow ? s_off[lane] : 0u;  // grow <= 64 chunk starts
  const uint32_t last = s_off[grow];
  for (int gg = w; gg < grow; gg += W) {
    const uint32_t o = lane_value(bound, gg);
    const uint32_t e = gg + 1 < grow ? lane_value(bound, gg + 1) : last;
    uint32_t* l = lists + (uint32_t)gg * cap;
    for (uint32_t i = lane; i < e - o; i += 64u) {
      ws_store(l + i, 0u);
      ws_store(l + pub + i, 0u);
    }
  }
}

// Adds a complete LDS histogram into a workspace histogram (non-zero bins
// only) and its sums over groups of 32 bins into the workspace's group sums
// gc.  The LDS copy is left as it is.  NT threads.
template <int NT>
__device__ __forceinline__ void merge_hist(const uint32_t* lds_hist, uint32_t* gh, uint32_t* gc) {
  const int t = threadIdx.x;
  if (t < kBins / 32) {
    const u32x4* grp = reinterpret_cast<const u32x4*>(lds_hist + t * 32);
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 v = grp[(c + t) & 7];  // rotated start: spreads the banks
      s += (v.x + v.y) + (v.z + v.w);
    }
    if (s) ws_add(gc + t, s);
  }
  for (int i = t; i < kBins; i += NT) {
    const uint32_t v = lds_hist[i];
    if (v) ws_add(gh + i, v);
  }
}

// The threshold search of wave_find<2048> run straight on a merged workspace
// histogram: the 64 group sums first, then the 32 bins of the group holding
// the krem-th largest entry (96 loads per wavefront instead of copying 2048
// bins to LDS).  Wave-uniform result; every wavefront runs it itself.
__device__ Found ws_find(const uint32_t* gh, const uint32_t* gc, uint32_t krem) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const uint32_t s = ws_load(gc + (63 - lane));  // lane order is descending group order
  const uint32_t incl = wave_incl_scan(s);
  const uint64_t reach = ballot(incl >= krem);
  Found f;
  if (reach == 0) {  // fewer than krem entries: inconsistent histogram
    f.bin = 0u;
    f.above = 0u;
    f.in_bin = lane_value(incl, 63);
    f.ok = 0u;
    return f;
  }
  const int lc = __builtin_ctzll(reach);
  const uint32_t before = lane_value(incl, lc) - lane_value(s, lc);
  const int qc = 63 - lc;
  const uint32_t v = lane < 32 ? ws_load(gh + qc * 32 + (31 - lane)) : 0u;
  const uint32_t in2 = wave_incl_scan(v) + before;
  const uint64_t reach2 = ballot(lane < 32 && in2 >= krem);
  if (reach2 == 0) {  // the group's bins disagree with its sum: inconsistent
    f.bin = (uint32_t)qc * 32u;
    f.above = before;
    f.in_bin = 0u;
    f.ok = 0u;
    return f;
  }
  const int l2 = __builtin_ctzll(reach2);
  f.bin = (uint32_t)(qc * 32 + (31 - l2));
  f.in_bin = lane_value(v, l2);
  f.above = lane_value(in2, l2) - f.in_bin;
  f.ok = 1u;
  return f;
}

// Adds a wave-uniform count into an LDS accumulator (one lane per wave).
__device__ __forceinline__ void wave_add(uint32_t* acc, uint32_t v) {
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(acc, v);
}

// Index of the list holding flattened position i: the last gg with
// off[gg] <= i (off ascending, off[0] = 0, n lists).
__device__ __forceinline__ int list_of(const uint32_t* off, int n, uint32_t i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <int VEC, int LAY, typename E>
__global__ void __launch_bounds__(Shape<LAY>::kBlock, Shape<LAY>::kWavesPerSimd) topk_multi_kernel(KernelParams p) {
  __shared__ Smem<LAY> sm;
  __shared__ uint32_t s_off[kMaxGroup + 1];
  __shared__ uint32_t s_above[kMaxGroup];
  constexpr int S = Shape<LAY>::kSlots;
  constexpr int CAP = Shape<LAY>::kCap;
  constexpr int NT = Shape<LAY>::kBlock;
  const int t = threadIdx.x;
  const int G = p.wg_per_row;
  // Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
  // that consecutive logical ids -- the G workgroups of one row -- share an
  // XCD and its L2 (performance only; any mapping is correct).
  const int W = (int)gridDim.x;
  const int l = (W & 7) == 0 ? (int)(blockIdx.x & 7) * (W >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int row = l / G;
  const int g = l - row * G;
  if (row >= p.num_rows) return;
  const uint32_t K = (uint32_t)p.K;
  const int64_t n = clamp_len(p, row);
  // The row's offset is read here, beside its length, and kept uniform: read
  // at the emit, its load would still be outstanding there, and the wait for
  // it (for all vector memory operations) would then sit before every store
  // of the output, each waiting for the previous one.
  const uint32_t roff = uni(offset_of(p, row));
  int32_t* out = p.out + (int64_t)row * p.K;
  if (n <= (int64_t)K) {
    if (g == 0)
      write_all_then_pad<NT, E>(out, n, p.K, roff,
                            p.out_val != nullptr ? p.out_val + (int64_t)row * p.K : nullptr, row_of<E>(p, row));
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
  uint32_t* gs1 = reinterpret_cast<uint32_t*>(blk + lay.c1);
  uint32_t* gs2 = reinterpret_cast<uint32_t*>(blk + lay.c2);
  uint32_t* lists = reinterpret_cast<uint32_t*>(blk + lay.lists);

  zero_histograms(sm);
  if (t < 16) sm.acc[t] = 0u;
  __syncthreads();

  const int64_t c0 = (int64_t)g * p.chunk;
  const int64_t c1 = c0 + p.chunk < n ? c0 + p.chunk : n;
  const E* rowp = row_of<E>(p, row);
  float* vout = p.out_val != nullptr ? p.out_val + (int64_t)row * p.K : nullptr;
  uint32_t* my_list = lists + (uint64_t)g * CAP;
  uint32_t base = 0;  // arrivals counted on ctr before the rounds below

  // One round.  Every workgroup of the row takes the same speculative bound
  // from the same sample (the first two wave tiles of each wavefront segment
  // of the whole row, through the same integer selection), streams its chunk
  // wave by wave keeping the elements that reach it, publishes them with
  // their row indices, and arrives once.  When every chunk published and at
  // least K and at most the buffer's capacity reached the bound in all, the
  // union holds every element of the row's K best (each is at least the K-th
  // best key, which is at least the bound); the last workgroup to arrive
  // gathers it and selects, and no workgroup waits for a second round.
  // Otherwise (the bound was above the K-th best, a wavefront's part of the
  // buffer overflowed, or too many elements passed) every workgroup falls
  // back to the three rounds below, which need nothing from the bound.
  if (wave_mode<LAY>((uint32_t)n, K)) {
    constexpr uint32_t PUB = (uint32_t)CAP / 2u;  // published entries a chunk may hold
    constexpr uint32_t SUB = (uint32_t)CAP / Shape<LAY>::kWaves;
    uint32_t mine = 0, woff = 0, total = 0, Lr = 0;
    float x0[kElems], x1[kElems];
    Hint hint{0u, 0u, false};
    const bool ok = stream_range_waves<LAY, VEC>(sm, rowp, (uint32_t)n, K, (uint32_t)c0, (uint32_t)c1, x0, x1, false,
                                                mine, woff, total, Lr, hint);
    const bool pub = ok && Lr != 0u && total <= PUB;
    if (pub) {
      const uint32_t lane = t & 63, s0 = ((uint32_t)t >> 6) * SUB;
      for (uint32_t i = lane; i < mine; i += 64u) {
        ws_store(my_list + woff + i, sm.val[s0 + i]);
        ws_store(my_list + PUB + woff + i, (uint32_t)sm.idx[s0 + i]);  // row positions already
      }
    }
    if (t == 0) ws_store(&slots[4 * g + 3], pub ? total : (0x80000000u | (total & 0x7fffffffu)));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) sm.acc[5] = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool last = uni(sm.acc[5]) == (uint32_t)grow - 1u;
    if (!last) group_wait(ctr, (uint32_t)grow + p.wait_extra, p.spin_limit, err);
    // Every workgroup reads the same published counts and decides alike.
    if (t < 64) {  // the whole of wavefront 0
      const uint32_t v = t < grow ? ws_load(&slots[4 * t + 3]) : 0u;
      const uint32_t c = (v & 0x80000000u) ? 0u : (v < PUB ? v : PUB);
      const uint32_t incl = wave_incl_scan(c);
      const uint64_t unpublished = ballot(t < grow && (v & 0x80000000u) != 0u);
      if (t < grow) s_off[t + 1] = incl;
      if (t == 0) {
        s_off[0] = 0u;
        sm.acc[6] = unpublished != 0u ? 1u : 0u;
      }
    }
    __syncthreads();
    const uint32_t sum = uni(s_off[grow]);
    const bool fast = uni(sm.acc[6]) == 0u && sum >= K && sum <= (uint32_t)CAP;
    if (fast) {
      if (last) gather_union<LAY>(sm, lists, PUB, s_off, grow, sum);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every gather load has completed
      // Leave.  The last workgroup out zeroes the slots and both counters
      // (every workgroup has read the slots by then).  The workgroup that
      // selects issues its exit before the selection and looks at the
      // answer after it, so the atomic's round trip is off its critical
      // path.
      uint32_t old = 0u;
      if (t == 0) old = __hip_atomic_fetch_add(exit_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (last) {
        final_select<LAY>(sm, plain_slice<LAY>(sum), K, out, roff, vout, hint);
        // The gatherer was the lists' only reader: it zeroes them.
        clear_union<NT>(lists, (uint32_t)CAP, PUB, s_off, grow);
      }
      if (t == 0) sm.acc[4] = (old == (uint32_t)grow - 1u) ? 1u : 0u;
      __syncthreads();
      const bool clean = uni(sm.acc[4]) != 0u;
      if (clean) {
        if (t < 4 * grow) ws_store(&slots[t], 0u);
        if (t == 0) {
          ws_store(ctr, 0u);
          ws_store(exit_ctr, 0u);
        }
      }
      return;
    }
    // Fallback: this chunk's published entries are nobody's input any more.
    if (pub) {
      for (uint32_t i = t; i < total; i += NT) {
        ws_store(my_list + i, 0u);
        ws_store(my_list + PUB + i, 0u);
      }
    }
    __syncthreads();  // s_off and sm.acc are reused below
    base = (uint32_t)grow;
  }

  uint32_t cnt = 0, L = 0;
  float x0[kElems], x1[kElems];
  // The chunk speculates from its first two tiles, as a general-path row
  // does: the bound keeps its candidates below the buffer's capacity, so no
  // compaction runs.  Every chunk element below the bound is beaten by the
  // cnt >= K kept ones; if fewer than K reached it, the chunk is streamed
  // again without one.
  const uint32_t clen = (uint32_t)(c1 - c0);
  stream_chunk<LAY, VEC>(sm, rowp, (uint32_t)c0, (uint32_t)c1, K, cnt, L,
                         clen >= 2u * (uint32_t)Shape<LAY>::kTile ? clen : 0u, x0, x1, false);
  if (cnt < K && clen > K) {
    cnt = 0u;
    L = 0u;
    stream_chunk<LAY, VEC>(sm, rowp, (uint32_t)c0, (uint32_t)c1, K, cnt, L, 0u, x0, x1, false);
  }

  const Slice sl = plain_slice<LAY>(cnt);
  const uint32_t sp = sl.sp, nv = sl.nv;
  uint32_t k[S];
  load_keys<LAY>(sm, k, sl);

  // Round 1: the chunk's top-digit (11-bit) histogram into the row's, then
  // the row-wide threshold digit from a copy of the row's.  (Loops over the
  // slice test it once per group of 4 slots, and adds that count nothing go
  // to the lane's sink word, as in range_select.)
  uint32_t* const sink = &sm.sink[t & 63];
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        atomicAdd((uint32_t)j < nv ? &sm.hist1[k[j] >> 21] : sink, 1u);
      }
    }
  }
  __syncthreads();
  merge_hist<NT>(sm.hist1, h1, gs1);
  group_barrier(ctr, base + 1u * grow + p.wait_extra, p.spin_limit, err);
  const Found f1 = ws_find(h1, gs1, K);
  uint32_t ok = f1.ok;
  uint32_t krem = K - f1.above;
  uint32_t prefix = f1.bin << 21;
  uint32_t pmask = 0xffe00000u;

  // Round 2: next 11 bits of the entries in the threshold bin; publish how
  // many of this chunk's entries lie above it.
  __syncthreads();  // every wave has read the row's copy
  for (int i = t; i < kBins; i += NT) sm.hist1[i] = 0u;
  __syncthreads();
  uint32_t n_above = 0;
#pragma unroll
  for (int q = 0; q < S / 4; ++q) {
    if ((uint32_t)(4 * q) < sp) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * q + c;
        const bool valid = (uint32_t)j < nv;
        const uint32_t km = k[j] & pmask;
        atomicAdd(valid && km == prefix ? &sm.hist1[(k[j] >> 10) & 2047u] : sink, 1u);
        n_above += popc64(ballot(valid && km > prefix));
      }
    }
  }
  wave_add(&sm.acc[0], n_above);
  __syncthreads();
  merge_hist<NT>(sm.hist1, h2, gs2);
  if (t == 0) ws_store(&slots[4 * g + 0], sm.acc[0]);
  group_barrier(ctr, base + 2u * grow + p.wait_extra, p.spin_limit, err);
  const Found f2 = ws_find(h2, gs2, krem);
  ok &= f2.ok;
  krem -= f2.above;
  prefix |= f2.bin << 10;
  pmask = 0xfffffc00u;

  // Round 3: publish the keys still undecided after 22 bits, in index order
  // (positions from ballots, as in emit_chosen), and the count above them.
  {
    uint32_t mine = 0;
    n_above = 0;
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      if ((uint32_t)(4 * q) < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * q + c;
          const bool valid = (uint32_t)j < nv;
          const uint32_t km = k[j] & pmask;
          mine += popc64(ballot(valid && km == prefix));
          n_above += popc64(ballot(valid && km > prefix));
        }
      }
    }
    wave_add(&sm.acc[1], n_above);
    uint32_t len;
    uint32_t at = wave_exclusive(sm, mine, &len);
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {
      if ((uint32_t)(4 * q) < sp) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * q + c;
          const bool und = (uint32_t)j < nv && (k[j] & pmask) == prefix;
          const uint64_t b = ballot(und);
          if (und) ws_store(&my_list[at + lanes_below(b)], k[j]);
          at += popc64(b);
        }
      }
    }
    if (t == 0) {
      ws_store(&slots[4 * g + 1], sm.acc[1] - sm.acc[0]);
      ws_store(&slots[4 * g + 2], len);
    }
  }
  group_barrier(ctr, base + 3u * grow + p.wait_extra, p.spin_limit, err);
  for (int i = t; i < kBins; i += NT) sm.hist1[i] = 0u;  // round 2's local histogram was merged before the barrier

  // Every chunk's list, flattened: offsets by a prefix sum over the lengths.
  if (t < 64) {
    uint32_t len = 0, above = 0;
    if (t < grow) {
      len = ws_load(&slots[4 * t + 2]);
      len = len < (uint32_t)CAP ? len : (uint32_t)CAP;
      above = ws_load(&slots[4 * t + 0]) + ws_load(&slots[4 * t + 1]);
    }
    const uint32_t incl = wave_incl_scan(len);
    if (t < grow) {
      s_off[t + 1] = incl;
      s_above[t] = above;
    }
    if (t == 0) s_off[0] = 0u;
  }
  __syncthreads();
  const uint32_t total = s_off[grow];
  // Last 10 bits over all lists.
  for (uint32_t i = t; i < total; i += NT) {
    const int gg = list_of(s_off, grow, i);
    const uint32_t v = ws_load(&lists[(uint64_t)gg * CAP + (i - s_off[gg])]);
    atomicAdd(&sm.hist1[v & 1023u], 1u);
  }
  __syncthreads();
  const Found f3 = wave_find<1024>(sm.hist1, krem);
  ok &= f3.ok;
  const uint32_t T = prefix | f3.bin;
  const uint32_t take_eq = krem - f3.above;
  // Entries of earlier chunks: above the 22-bit prefix (slots), and in the
  // lists above / equal to T.
  {
    uint32_t gt_b = 0, eq_b = 0;
    const uint32_t lim = s_off[g];
    for (uint32_t i0 = 0; i0 < lim; i0 += NT) {
      const uint32_t i = i0 + t;
      uint32_t v = 0;
      if (i < lim) {
        const int gg = list_of(s_off, grow, i);
        v = ws_load(&lists[(uint64_t)gg * CAP + (i - s_off[gg])]);
      }
      gt_b += popc64(ballot(i < lim && v > T));
      eq_b += popc64(ballot(i < lim && v == T));
    }
    wave_add(&sm.acc[2], gt_b);
    wave_add(&sm.acc[3], eq_b);
    if (t == 0) {
      uint32_t a = 0;
      for (int gg = 0; gg < g; ++gg) a += s_above[gg];
      if (a) atomicAdd(&sm.acc[2], a);
    }
  }
  __syncthreads();
  const uint32_t gt_base = sm.acc[2];
  const uint32_t eq_base = sm.acc[3];

  // Leave: the last workgroup out zeroes what this row used in the workspace.
  if (t == 0) {
    const uint32_t old = __hip_atomic_fetch_add(exit_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.acc[4] = (old == (uint32_t)grow - 1u) ? 1u : 0u;
    if (!ok) __hip_atomic_fetch_or(err, kErrSearch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sm.acc[4]) {
    for (int i = t; i < kBins; i += NT) {
      ws_store(&h1[i], 0u);
      ws_store(&h2[i], 0u);
    }
    if (t < kBins / 32) {
      ws_store(&gs1[t], 0u);
      ws_store(&gs2[t], 0u);
    }
    for (uint32_t i = t; i < total; i += NT) {
      const int gg = list_of(s_off, grow, i);
      ws_store(&lists[(uint64_t)gg * CAP + (i - s_off[gg])], 0u);
    }
    if (t < 4 * grow) ws_store(&slots[t], 0u);
    if (t == 0) {
      ws_store(ctr, 0u);
      ws_store(exit_ctr, 0u);
    }
  }

  Sel s;
  s.lo = T;
  s.hi = T;
  s.take = take_eq;
  s.above = 0u;
  s.in_bin = 0u;
  s.ok = ok;
  s.all_in = false;
  emit_chosen<LAY, kToOut>(sm, k, sl, s, gt_base, eq_base, out, K, (uint32_t)c0 + roff, vout);
}

}  // namespace rrt
