// Internal constants and launch parameters shared by the host launcher and
// the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rrt {

constexpr int kBlock = 256;                 // threads per workgroup of the base instances (4 wave64)
constexpr int kElems = 8;                   // fp32 elements per thread per tile
constexpr int kTile = kBlock * kElems;      // 2048 elements per tile of the base instances
constexpr int kBins = 2048;                 // bins of a first-pass histogram
constexpr int kSmallBins = 256;             // bins of a second-pass histogram
constexpr int kPrefetch = 4;                // register ring of tiles per thread
constexpr int kMaxGroup = 64;               // most workgroups that may share a row
constexpr int kMaxK = 2048;
constexpr uint32_t kDefaultSpin = 1u << 24; // polls before a cooperative wait gives up

// Speculative bound (one-workgroup rows of at least kSpecMinLen elements):
// before the first two tiles are filtered, the bound is raised to (about) the
// key of the r-th best of their 4096 elements, with
// r = max(kSpecMinRank, ceil(kSpecNum / kSpecDen * K * 4096 / n)), when that
// r is below K.  kSpecNum / kSpecDen is the safety factor over the expected
// rank of the K-th best of the row; kSpecMinRank keeps the sample quantile
// from resting on too few elements.  From 8192 elements on, speculating
// beats the general path's compactions (alone on a CU, rows of 12288 and
// 16383 elements took 20.6 and 24.2 us on the general path, 16384 took 13.4
// wave by wave); below it the sample would be more than half the row.
constexpr uint32_t kSpecNum = 3, kSpecDen = 2;
constexpr uint32_t kSpecMinRank = 128;
constexpr uint32_t kSpecMinLen = 8192;

// Candidate buffer capacity: 5120 entries.  It must hold K = 2048 kept
// entries plus one full tile, so a tile always fits after a compaction; the
// slack lets most compactions keep a whole bin, and gives each of the four
// wavefronts 1280 slots when a row streams wave by wave.  With 16-bit
// indices (rows or chunks of at most 65536 elements) an entry takes 6 bytes
// and four workgroups fit in a CU's 160 KB of LDS; with 32-bit indices,
// three.  The wider workgroups keep 32-bit indices in LDS whatever the row
// length (8 bytes per entry); their layouts with the 16-bit flag differ from
// the others only in capacity and residency.
constexpr int kIdx16Limit = 65536;

// Buffer layout of a kernel instance (a bit set): 16-bit candidate indices,
// room for K up to kMaxKBig, and the workgroup width (256 threads, or 512 /
// 1024: 8 or 16 wavefronts on one row).  The capacity holds K plus one tile
// (kElems per thread) for the general path, and about twice the ~1.5 K that
// pass a speculative bound, split between the wavefronts.  256 threads:
// 5120 (7168 for the large K), four workgroups per CU with 16-bit indices,
// three with 32-bit ones, two for the large K.  512 threads (32-bit
// indices in LDS either way): 8192 with the 16-bit flag (a row of up to two
// tiles then never compacts), 6144 without it (8192 for the large K), two
// per CU, except one for the large K without the flag (LDS) and one with the
// flag below the large K: the rows that layout serves are fewer than the
// CUs, and at one workgroup per CU its instances keep up to 256 VGPRs
// instead of spilling at 128.
// 1024 threads: 12288, one per CU.  At most 16 wavefronts per CU in every
// case, so each keeps 128 VGPRs (more where fewer fit).
constexpr int kLayIdx16 = 1;
constexpr int kLayBigK = 2;
constexpr int kLayW512 = 4;
constexpr int kLayW1024 = 8;
constexpr int kMaxKBig = 4096;
constexpr int layout_of(bool idx16, bool big_k, int block = kBlock) {
  return (idx16 ? kLayIdx16 : 0) | (big_k ? kLayBigK : 0) | (block == 1024 ? kLayW1024 : block == 512 ? kLayW512 : 0);
}
constexpr int block_of(int lay) { return (lay & kLayW1024) ? 1024 : (lay & kLayW512) ? 512 : kBlock; }
constexpr int tile_of(int lay) { return block_of(lay) * kElems; }
constexpr int cap_of(int lay) {
  return block_of(lay) == 1024 ? 12288 : block_of(lay) == 512 ? ((lay & (kLayBigK | kLayIdx16)) ? 8192 : 6144)
                                                              : ((lay & kLayBigK) ? 7168 : 5120);
}
constexpr int kmax_of(int lay) { return (lay & kLayBigK) ? kMaxKBig : kMaxK; }
constexpr int resident_of(int lay) {
  return block_of(lay) == 1024 ? 1
       : block_of(lay) == 512 ? (((lay & kLayBigK) != 0) != ((lay & kLayIdx16) != 0) ? 1 : 2)
                              : ((lay & kLayBigK) ? 2 : ((lay & kLayIdx16) ? 4 : 3));
}
// Workgroup widths with instances: 256 and 512 for every load width of fp32
// and bf16 scores; 1024 for fp32 scores only.
constexpr bool has_block(int block, bool bf16) {
  return block == kBlock || block == 512 || (block == 1024 && !bf16);
}

// The planner gives a row several workgroups only when rows are longer than
// this (the one-workgroup path streams shorter rows wave by wave faster) and
// only with at least kMinGroup workgroups per row.
constexpr int64_t kMultiMinStride = 65536;
constexpr int64_t kMinGroup = 4;

// Workspace: a 256-byte header followed by one block per row of the
// multi-workgroup path.  Header word 0: error bits; the word at byte
// kTicketOff: the next-row ticket of the one-workgroup-per-row path when
// rows outnumber its grid (zero between launches).
constexpr uint64_t kWsHeader = 256;
constexpr uint64_t kTicketOff = 128;
constexpr uint32_t kErrSpin = 1u;
constexpr uint32_t kErrSearch = 2u;

// Per-row block layout (bytes from the block start):
//   0    arrival counter (u32)
//   128  exit counter (u32)
//   256  per-workgroup slots, 4 x u32 each: [above digit 1, above digit 2,
//        list length, published count (bit 31: nothing published)]
//   ...  digit-1 histogram, 2048 x u32
//   ...  digit-2 histogram, 2048 x u32
//   ...  their sums over groups of 32 bins, 64 x u32 each (digit 1, digit 2)
//   ...  per-workgroup lists, cap x u32 each: the one-round path publishes
//        up to cap / 2 candidates there (fp32 bits in the first half, row
//        indices in the second); the three rounds write undecided keys.
struct GroupLayout {
  uint64_t slots, h1, h2, c1, c2, lists, bytes;
};

inline constexpr uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

inline constexpr GroupLayout group_layout(int wg_per_row, int cap) {
  GroupLayout L{};
  L.slots = 256;
  L.h1 = L.slots + round_up(16ull * (uint64_t)wg_per_row, 256);
  L.h2 = L.h1 + 4ull * kBins;
  L.c1 = L.h2 + 4ull * kBins;
  L.c2 = L.c1 + 256;
  L.lists = L.c2 + 256;
  L.bytes = round_up(L.lists + 4ull * (uint64_t)cap * (uint64_t)wg_per_row, 256);
  return L;
}

struct KernelParams {
  const void* scores;          // fp32, or bf16 as uint16_t bits (the kernel instance says which)
  const int32_t* lengths;
  const int32_t* row_offsets;  // nullable: added to each row's chosen indices
  float* out_val;              // nullable: the chosen scores, [num_rows, K]
  int32_t* out;
  uint8_t* ws;
  int64_t row_stride;
  int64_t chunk;         // multi path: row elements per workgroup (multiple of 4)
  uint64_t group_bytes;  // multi path: bytes per row block in the workspace
  int32_t num_rows;
  int32_t K;
  int32_t wg_per_row;    // multi path: G
  uint32_t spin_limit;
  uint32_t wait_extra;  // added to every cooperative wait's target: 0, or 1 to force timeouts (testing)
};

// Kernel lookup for the host side.  path: 1 single, 2 multi, 3 the
// streaming-read reference (idx16, big_k and block ignored).  vals: the one-workgroup instance that also writes the chosen
// scores (the multi-workgroup kernel always can).  bf16: the instance that
// reads bf16 scores (vec 8 or 1); big_k: the large layout (K up to
// kMaxKBig); block: threads per workgroup.  nullptr if no such instance.
const void* kernel_ptr(int path, int vec, bool idx16, bool vals = false, bool bf16 = false, bool big_k = false,
                       int block = kBlock);
// Per instance file: the kernels of the layouts it compiles (nullptr for
// others), and static LDS bytes per workgroup of a layout.
const void* kernels_w256_l0(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w256_l1(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w256_l2(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w256_l3(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w512_i16(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w512_i32(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w1024_l0(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w1024_l1(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w1024_l2(int lay, int path, int vec, bool vals, bool bf16);
const void* kernels_w1024_l3(int lay, int path, int vec, bool vals, bool bf16);
const void* read_ref_kernel_ptr(int vec);
const void* zero_kernel_ptr();

// Allocation-free launches (topk_ragged_noalloc) take their workspace from a
// static device array of this many bytes per device (topk_noalloc.hip).
constexpr uint64_t kNoallocScratchBytes = 8ull << 20;
// Device address of dev's scratch array (set up on first use, zeroed by a
// fill kernel on stream); 0 or a HIP error code, *msg naming the step.
int noalloc_scratch(int dev, hipStream_t stream, void** out, const char** msg);
const void* keys_kernel_ptr();
const void* pack_kernel_ptr();
int lds_bytes_of(bool idx16, bool big_k = false, int block = kBlock);

}  // namespace rrt
