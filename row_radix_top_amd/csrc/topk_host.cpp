// Host side of the C ABI: argument checks, the launch planner, cached device
// facts and kernel launches.  No allocation, no memset and no synchronisation
// on the launch path, so a call can be captured in a hipGraph.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <string>

#include "topk_internal.h"
#include "topk_ragged.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr int64_t kDefaultMinChunk = 8192;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool verbose() {
  static const bool v = [] {
    const char* e = std::getenv("TOPK_RAGGED_VERBOSE");
    return e != nullptr && e[0] == '1';
  }();
  return v;
}

std::string describe(const topk_plan& p) {
  char buf[512];
  std::snprintf(buf, sizeof(buf),
                "path=%d idx16=%d vec=%d block=%d grid=%d wg_per_row=%d chunk=%lld "
                "resident_cap=%d headroom=%d lds=%d fell_back=%d workspace=%llu",
                p.path, p.idx16, p.vec, p.block, p.grid, p.wg_per_row, (long long)p.chunk,
                p.resident_cap, p.headroom, p.lds_bytes, p.fell_back,
                (unsigned long long)p.workspace_bytes);
  return buf;
}

// ---------------------------------------------------------------------------
// Device facts, cached per device (the stream's device, looked up per call,
// so a cached value can never belong to another device).  After the first
// call on a device every lookup is a plain array read: the entries are
// atomics filled once (a query is deterministic, so two threads filling the
// same entry store the same value) and no lock is taken.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

// Occupancy entries: (path single / multi / read reference) x (vec 1, 2, 4,
// 8) x idx16 x bf16 x big K x (block 256, 512, 1024).
constexpr int kOccEntries = 3 * 4 * 2 * 2 * 2 * 3;

struct DevCache {
  std::atomic<int> num_cus{0};  // 0 until the attributes were read
  std::atomic<int> max_lds_block{0};
  std::atomic<int> occ[kOccEntries];  // -1 unknown, else workgroups per CU (0: no such instance)
  DevCache() {
    for (auto& o : occ) o.store(-1, std::memory_order_relaxed);
  }
};

DevCache g_dev[kMaxDevices];

int stream_device(hipStream_t stream, int* dev) {
  hipError_t e = stream == nullptr ? hipGetDevice(dev) : hipStreamGetDevice(stream, dev);
  if (e != hipSuccess)
    return fail(TOPK_EDEVICE, std::string("cannot find the stream's device: ") + hipGetErrorString(e));
  if (*dev < 0 || *dev >= kMaxDevices) return fail(TOPK_EDEVICE, "device ordinal beyond the library's table");
  return TOPK_OK;
}

int device_info(int dev, DevCache** out) {
  DevCache& d = g_dev[dev];
  if (d.num_cus.load(std::memory_order_acquire) == 0) {
    int cus = 0, lds = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess)
      return fail(TOPK_EDEVICE, std::string("device attribute query failed: ") + hipGetErrorString(e));
    if (cus < 1) return fail(TOPK_EDEVICE, "device reports no compute units");
    d.max_lds_block.store(lds, std::memory_order_relaxed);
    d.num_cus.store(cus, std::memory_order_release);
  }
  *out = &d;
  return TOPK_OK;
}

int occ_slot(int path, int vec, bool idx16, bool bf16, bool big_k, int block) {
  const int v = vec == 8 ? 3 : vec == 4 ? 2 : vec == 2 ? 1 : 0;
  const int b = block == 1024 ? 2 : block == 512 ? 1 : 0;
  const int pi = path == 2 ? 1 : path == 3 ? 2 : 0;
  return (((((pi * 4 + v) * 2 + (idx16 ? 1 : 0)) * 2 + (bf16 ? 1 : 0)) * 2 + (big_k ? 1 : 0)) * 3) + b;
}

// Occupancy of the exact instance that will be launched (0 when the library
// has no such instance).
int occupancy(int dev, DevCache* d, int path, int vec, bool idx16, int* occ, bool bf16 = false, bool big_k = false,
              int block = rrt::kBlock) {
  std::atomic<int>& slot = d->occ[occ_slot(path, vec, idx16, bf16, big_k, block)];
  const int cached = slot.load(std::memory_order_acquire);
  if (cached >= 0) {
    *occ = cached;
    return TOPK_OK;
  }
  const void* fn = rrt::kernel_ptr(path, vec, idx16, false, bf16, big_k, block);
  int o = 0;
  if (fn != nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, fn, block, 0);
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      char buf[256];
      std::snprintf(buf, sizeof(buf), "occupancy query failed (path=%d vec=%d idx16=%d block=%d): %s", path, vec,
                    idx16 ? 1 : 0, block, hipGetErrorString(e));
      return fail(TOPK_EDEVICE, buf);
    }
  }
  slot.store(o, std::memory_order_release);
  *occ = o;
  return TOPK_OK;
}

// Widest load, in elements, that the pointer and stride alignment allow:
// fp32 rows take 16-, 8- or 4-byte loads, bf16 rows 16- or 2-byte loads.
int vec_allowed_for(const void* scores, int64_t row_stride, bool bf16 = false) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(scores);
  if (bf16) return (a % 16 == 0 && row_stride % 8 == 0) ? 8 : 1;
  if (a % 16 == 0 && row_stride % 4 == 0) return 4;
  if (a % 8 == 0 && row_stride % 2 == 0) return 2;
  return 1;
}

int chosen_vec(int vec_allowed, const topk_overrides* ov, int* vec) {
  int v = vec_allowed;
  if (ov != nullptr && ov->force_vec != 0) {
    if (ov->force_vec != 1 && ov->force_vec != 2 && ov->force_vec != 4 && ov->force_vec != 8)
      return fail(TOPK_EINVAL, "force_vec must be 1, 2, 4 or 8");
    if (ov->force_vec > vec_allowed)
      return fail(TOPK_EINVAL, "force_vec is wider than the scores pointer/stride alignment allows");
    v = ov->force_vec;
  }
  *vec = v;
  return TOPK_OK;
}

// Fills props for the load width vec of every kernel instance on device dev:
// the 256-thread instances and the wider ones (0 where none exists).
// big_k: the instances of the large layout (K above 2048).
int real_props(int dev, int vec, topk_device_props* props, bool bf16 = false, bool big_k = false) {
  DevCache* d = nullptr;
  int rc = device_info(dev, &d);
  if (rc != TOPK_OK) return rc;
  std::memset(props, 0, sizeof(*props));
  props->num_cus = d->num_cus.load(std::memory_order_relaxed);
  props->max_lds_per_block = d->max_lds_block.load(std::memory_order_relaxed);
  int32_t* base[4] = {&props->occupancy_single, &props->occupancy_multi, &props->occupancy_single16,
                      &props->occupancy_multi16};
  for (int i = 0; i < 4 && rc == TOPK_OK; ++i)
    rc = occupancy(dev, d, (i & 1) ? 2 : 1, vec, i >= 2, base[i], bf16, big_k, rrt::kBlock);
  for (int i = 0; i < 4 && rc == TOPK_OK; ++i)
    rc = occupancy(dev, d, (i & 1) ? 2 : 1, vec, i >= 2, &props->occupancy_w512[i], bf16, big_k, 512);
  for (int i = 0; i < 4 && rc == TOPK_OK; ++i)
    rc = occupancy(dev, d, (i & 1) ? 2 : 1, vec, i >= 2, &props->occupancy_w1024[i], bf16, big_k, 1024);
  return rc;
}

int check_common(int32_t num_rows, int64_t row_stride, int32_t K) {
  if (num_rows < 0) return fail(TOPK_EINVAL, "num_rows must be >= 0");
  if (row_stride < 1 || row_stride > INT32_MAX)
    return fail(TOPK_EINVAL, "row_stride must be in [1, 2^31 - 1]");
  if (K < 1 || K > TOPK_RAGGED_MAX_K) {
    char buf[128];
    std::snprintf(buf, sizeof(buf), "K=%d outside [1, %d]", K, TOPK_RAGGED_MAX_K);
    return fail(TOPK_EUNSUPPORTED_K, buf);
  }
  return TOPK_OK;
}

// The four occupancies of the instances of one workgroup width.
struct OccSet {
  int single, multi, single16, multi16;
};

OccSet occ_for(const topk_device_props* p, int block) {
  if (block == 512) return {p->occupancy_w512[0], p->occupancy_w512[1], p->occupancy_w512[2], p->occupancy_w512[3]};
  if (block == 1024)
    return {p->occupancy_w1024[0], p->occupancy_w1024[1], p->occupancy_w1024[2], p->occupancy_w1024[3]};
  return {p->occupancy_single, p->occupancy_multi, p->occupancy_single16, p->occupancy_multi16};
}

// Whether a row of n elements streams wave by wave on an instance of
// `block` threads: long enough to speculate, every wavefront segment holding
// the two wave tiles of the sample, and a speculative rank below K (the
// sample is 2 * block * kElems elements).  Mirrors the kernels' rule.
bool waves_on(int block, int64_t n, int32_t K) {
  const int64_t W = block / 64, wave_tile = 64 * rrt::kElems;
  if (n < (int64_t)rrt::kSpecMinLen) return false;
  const int64_t seg = (ceil_div(n, W) + wave_tile - 1) / wave_tile * wave_tile;
  if (n < (W - 1) * seg + 2 * wave_tile) return false;
  const int64_t M = 2 * (int64_t)block * rrt::kElems;
  const int64_t want = ((int64_t)rrt::kSpecNum * K * M + (int64_t)rrt::kSpecDen * n - 1) / ((int64_t)rrt::kSpecDen * n);
  return std::max<int64_t>(want, rrt::kSpecMinRank) < K;
}

// Workgroup width of the one-workgroup path when the caller does not force
// one.  512 threads (8 wavefronts per row) when every row gets a resident
// workgroup of its own and rows of row_stride elements still speculate with
// the 512-thread sample: a row's streaming is then spread over twice the
// wavefronts.  Measured on MI355X, 64 rows: multi-token rows 22.3 -> 18.4
// us, decode 17.8 -> 17.3 us; 4 x 8192 rows at K = 512 cannot speculate on
// 512 threads and stay on 256 (9.7 us against 11.5).  Batches that fill the
// GPU stay on 256 threads: four workgroups per CU overlap one row's
// selection with other rows' streaming (prefill-shaped batch 191-201 us on
// 256, 210 us on 512).  1024 threads measured slower everywhere.
int auto_block_single(const topk_device_props* p, int32_t num_rows, int64_t row_stride, int32_t K) {
  const int occ512 = std::min(p->occupancy_w512[0], p->occupancy_w512[2]);
  if (occ512 >= 1 && (int64_t)num_rows <= (int64_t)p->num_cus * occ512 && waves_on(512, row_stride, K))
    return 512;
  return rrt::kBlock;
}

// Workgroup width of the multi-workgroup path when the caller does not
// force one: 512 threads when that instance can be resident.  Each chunk is
// then streamed by 8 wavefronts, and the workgroup that merges a row selects
// with twice the lanes.  Measured on MI355X, 16 rows of up to 131072
// elements: 26.0 -> 20.4 us (K = 1024) and 26.0 -> 22.4 us (K = 2048);
// 1024 threads measured 28-29 us.
int auto_block_multi(const topk_device_props* p, int32_t num_rows, int64_t row_stride, int32_t K) {
  (void)num_rows;
  (void)row_stride;
  (void)K;
  return std::min(p->occupancy_w512[1], p->occupancy_w512[3]) >= 1 ? 512 : rrt::kBlock;
}

int plan_for_call(const void* scores, int32_t num_rows, int64_t row_stride, int32_t K,
                  const topk_overrides* ov, hipStream_t stream, int* dev_out, topk_plan* plan, bool bf16 = false) {
  int rc = check_common(num_rows, row_stride, K);
  if (rc != TOPK_OK) return rc;
  const int va = vec_allowed_for(scores, row_stride, bf16);
  int vec = 4;
  rc = chosen_vec(va, ov, &vec);
  if (rc != TOPK_OK) return rc;
  if (bf16 && vec != 8 && vec != 1) return fail(TOPK_EINVAL, "bf16 rows load 8 elements or 1 (force_vec 8 or 1)");
  int dev = 0;
  rc = stream_device(stream, &dev);
  if (rc != TOPK_OK) return rc;
  topk_device_props props;
  rc = real_props(dev, vec, &props, bf16, K > rrt::kMaxK);
  if (rc != TOPK_OK) return rc;
  if (dev_out) *dev_out = dev;
  return topk_ragged_plan(&props, num_rows, row_stride, K, va, ov, plan);
}

// Elements per load of a plan: the widest the alignment allows, except for
// fp32 rows on the wide workgroups (512 or 1024 threads) when the caller
// forces no width.  Those load one element per lane and instruction: with
// lane l holding elements l, l + 64, ... of a wave tile every element's
// buffer position is one rank (mbcnt) with no running count per lane, which
// shortens the streaming loop a lone workgroup runs.  Measured on MI355X: decode 13.3 ->
// 12.9 us, multi-token rows 14.8 -> 14.7 us, long rows 0.1-0.2 us less.
int plan_vec(int vec, int vec_allowed, const topk_overrides* ov, int block) {
  if (vec_allowed == 8 || (ov != nullptr && ov->force_vec != 0) || block == rrt::kBlock) return vec;
  return 1;
}

}  // namespace

extern "C" {

int topk_ragged_plan(const topk_device_props* props_in, int32_t num_rows, int64_t row_stride, int32_t K,
                     int32_t vec_allowed, const topk_overrides* ov, topk_plan* plan) {
  if (props_in == nullptr || plan == nullptr) return fail(TOPK_EINVAL, "null props or plan");
  // A smaller device, for testing the residency rules on this one: every
  // instance keeps at most max_occupancy workgroups per CU.
  topk_device_props capped = *props_in;
  if (ov != nullptr && ov->max_occupancy != 0) {
    if (ov->max_occupancy < 0) return fail(TOPK_EINVAL, "max_occupancy must be >= 0");
    for (int32_t* o : {&capped.occupancy_single, &capped.occupancy_multi, &capped.occupancy_single16,
                       &capped.occupancy_multi16})
      *o = std::min(*o, ov->max_occupancy);
    for (int i = 0; i < 4; ++i) {
      capped.occupancy_w512[i] = std::min(capped.occupancy_w512[i], ov->max_occupancy);
      capped.occupancy_w1024[i] = std::min(capped.occupancy_w1024[i], ov->max_occupancy);
    }
  }
  const topk_device_props* props = &capped;
  std::memset(plan, 0, sizeof(*plan));
  int rc = check_common(num_rows, row_stride, K);
  if (rc != TOPK_OK) return rc;
  if (vec_allowed != 1 && vec_allowed != 2 && vec_allowed != 4 && vec_allowed != 8)
    return fail(TOPK_EINVAL, "vec_allowed must be 1, 2, 4 or 8");
  if (props->num_cus < 1) return fail(TOPK_EDEVICE, "device reports no compute units");
  int vec = 4;
  rc = chosen_vec(vec_allowed, ov, &vec);
  if (rc != TOPK_OK) return rc;
  const int want_block = ov != nullptr ? ov->force_block : 0;
  if (want_block != 0 && want_block != 256 && want_block != 512 && want_block != 1024)
    return fail(TOPK_EINVAL, "force_block must be 0, 256, 512 or 1024");

  // K above 2048 takes the large layout (more candidates, fewer workgroups
  // per CU); props must then describe those instances.
  const bool big = K > rrt::kMaxK;
  const bool idx32_only = ov != nullptr && ov->force_idx32 != 0;
  plan->kmax = rrt::kmax_of(rrt::layout_of(false, big));
  plan->vec = vec;
  plan->block = rrt::kBlock;
  plan->wg_per_row = 1;
  if (num_rows == 0) {
    plan->path = TOPK_PATH_NONE;
    return TOPK_OK;
  }
  const int want = ov != nullptr ? ov->force_path : 0;
  if (want != 0 && want != TOPK_PATH_SINGLE && want != TOPK_PATH_MULTI)
    return fail(TOPK_EINVAL, "force_path must be 0, 1 or 2");

  // Several workgroups per row only pay off when rows are long and too few
  // to occupy the GPU one per workgroup.  The pages share rows above their
  // 32K radix threshold; here the one-workgroup path streams rows of up to
  // 64K elements wave by wave faster than several workgroups do, so rows are
  // shared automatically only above that, and only by at least kMinGroup
  // workgroups.  row_stride stands in for the longest length, which lives
  // on the device.
  const bool long_rows = row_stride > TOPK_RAGGED_RADIX_THRESHOLD && row_stride > rrt::kMultiMinStride;
  if (want == TOPK_PATH_MULTI || (want == 0 && long_rows)) {
    int block = want_block != 0 ? want_block : auto_block_multi(props, num_rows, row_stride, K);
    OccSet os = occ_for(props, block);
    if (want_block == 0 && std::min(os.multi, os.multi16) < 1) {
      block = rrt::kBlock;  // no wider instance resident: the base one
      os = occ_for(props, block);
    }
    // Size with the less resident of the two instances; the chunk length then
    // picks the instance (16-bit indices when a chunk fits them).
    const int occ = std::min(os.multi, os.multi16);
    if (occ < 1) {
      if (want == TOPK_PATH_MULTI) return fail(TOPK_EDEVICE, "multi-workgroup kernel cannot be resident");
    } else {
      // Workgroups of one row wait for each other, so all of them must be
      // resident at once.  Keep headroom for slots another kernel may hold
      // (PR #41189 page: a CU's worth when occupancy > 1, else one slot).
      const int64_t cap = (int64_t)props->num_cus * occ;
      int64_t headroom = occ > 1 ? props->num_cus : 1;
      int64_t avail = cap;
      if (avail >= headroom + 2)
        avail -= headroom;
      else
        headroom = 0;
      const int64_t tile = rrt::tile_of(rrt::layout_of(false, false, block));
      const int64_t min_chunk =
          (ov != nullptr && ov->min_chunk > 0) ? ov->min_chunk : std::max<int64_t>(kDefaultMinChunk, 2 * tile);
      int64_t G = 0, chunk = 0;
      if (ov != nullptr && ov->force_chunk > 0) {
        if (ov->force_chunk % 4 != 0) return fail(TOPK_EINVAL, "force_chunk must be a multiple of 4");
        chunk = ov->force_chunk;
        G = ceil_div(row_stride, chunk);
      } else {
        if (ov != nullptr && ov->force_wg_per_row > 0) {
          G = ov->force_wg_per_row;
        } else {
          G = ceil_div(row_stride, min_chunk);
          const int64_t by_slots = avail / num_rows;
          if (by_slots < G) G = by_slots;
          if (G > rrt::kMaxGroup) G = rrt::kMaxGroup;
        }
        if (G >= 1) {
          // Automatic chunks are whole tiles; a requested G keeps its count
          // (chunks only need 4-element alignment).
          const uint64_t align = (ov != nullptr && ov->force_wg_per_row > 0) ? 4 : (uint64_t)tile;
          chunk = (int64_t)rrt::round_up((uint64_t)ceil_div(row_stride, G), align);
          G = ceil_div(row_stride, chunk);
        }
      }
      if (G > rrt::kMaxGroup) {
        char buf[160];
        std::snprintf(buf, sizeof(buf), "wg_per_row=%lld exceeds %d", (long long)G, rrt::kMaxGroup);
        return fail(TOPK_EINVAL, buf);
      }
      const bool usable = want == TOPK_PATH_MULTI ? G >= 1 : G >= rrt::kMinGroup;
      if (usable) {
        const int64_t grid = (int64_t)num_rows * G;
        if (grid <= avail) {
          // 16-bit candidate indices only when every row index fits them:
          // the workgroup that merges a row's chunks holds row indices.
          const bool i16 = row_stride <= rrt::kIdx16Limit && !idx32_only;
          const rrt::GroupLayout lay = rrt::group_layout((int)G, rrt::cap_of(rrt::layout_of(i16, big, block)));
          plan->path = TOPK_PATH_MULTI;
          plan->block = block;
          plan->idx16 = i16 ? 1 : 0;
          plan->wg_per_row = (int)G;
          plan->chunk = chunk;
          plan->grid = (int)grid;
          plan->resident_cap = (int)cap;
          plan->headroom = (int)headroom;
          plan->lds_bytes = rrt::lds_bytes_of(i16, big, block);
          plan->workspace_bytes = rrt::kWsHeader + (uint64_t)num_rows * lay.bytes;
          plan->vec = plan_vec(vec, vec_allowed, ov, block);
          return TOPK_OK;
        }
        // Not co-resident: waiting workgroups could deadlock.  Fall back to
        // one workgroup per row, which never waits (PR #41189 page).
        plan->fell_back = 1;
      } else if (want == TOPK_PATH_MULTI) {
        plan->fell_back = 1;
      }
    }
  }

  const bool i16 = row_stride <= rrt::kIdx16Limit && !idx32_only;
  int block = want_block != 0 ? want_block : auto_block_single(props, num_rows, row_stride, K);
  int occ = i16 ? occ_for(props, block).single16 : occ_for(props, block).single;
  if (occ < 1 && want_block == 0 && block != rrt::kBlock) {
    block = rrt::kBlock;  // no wider instance resident: the base one
    occ = i16 ? props->occupancy_single16 : props->occupancy_single;
  }
  if (occ < 1) return fail(TOPK_EDEVICE, "single-workgroup kernel cannot be resident");
  const int64_t cap = (int64_t)props->num_cus * occ;
  int64_t grid = num_rows < cap ? num_rows : cap;
  if (ov != nullptr && ov->max_grid > 0 && grid > ov->max_grid) grid = ov->max_grid;
  plan->path = TOPK_PATH_SINGLE;
  plan->block = block;
  plan->wg_per_row = 1;
  plan->chunk = row_stride;
  plan->grid = (int)grid;
  plan->resident_cap = (int)cap;
  plan->headroom = 0;
  plan->idx16 = i16 ? 1 : 0;
  plan->lds_bytes = rrt::lds_bytes_of(i16, big, block);
  // More rows than workgroups: later rows are handed out by a ticket
  // counter in the workspace header.
  plan->workspace_bytes = num_rows > grid ? rrt::kWsHeader : 0;
  plan->vec = plan_vec(vec, vec_allowed, ov, block);
  return TOPK_OK;
}

int topk_ragged_query_plan(const float* scores, int32_t num_rows, int64_t row_stride, int32_t K,
                           const topk_overrides* ov, hipStream_t stream, topk_plan* plan) {
  if (plan == nullptr) return fail(TOPK_EINVAL, "null plan");
  return plan_for_call(scores, num_rows, row_stride, K, ov, stream, nullptr, plan);
}

int topk_ragged_workspace_size_ex(const float* scores, int32_t num_rows, int64_t row_stride, int32_t K,
                                  const topk_overrides* ov, hipStream_t stream, size_t* bytes) {
  if (bytes == nullptr) return fail(TOPK_EINVAL, "null bytes");
  topk_plan plan;
  const int rc = plan_for_call(scores, num_rows, row_stride, K, ov, stream, nullptr, &plan);
  if (rc != TOPK_OK) return rc;
  *bytes = (size_t)plan.workspace_bytes;
  return TOPK_OK;
}

int topk_ragged_workspace_size(int32_t num_rows, int64_t row_stride, int32_t K, hipStream_t stream,
                               size_t* bytes) {
  // The workspace size does not depend on load width; plan as if 16-byte aligned.
  return topk_ragged_workspace_size_ex(reinterpret_cast<const float*>(uintptr_t(256)), num_rows, row_stride,
                                       K, nullptr, stream, bytes);
}

int topk_ragged_workspace_init(void* workspace, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return TOPK_OK;
  if (workspace == nullptr) return fail(TOPK_EINVAL, "null workspace with nonzero size");
  if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0 || bytes % 4 != 0)
    return fail(TOPK_EINVAL, "workspace must be 4-byte aligned and a multiple of 4 bytes");
  const uint64_t words = bytes / 4;
  uint32_t* p = static_cast<uint32_t*>(workspace);
  uint64_t w = words;
  void* args[] = {&p, &w};
  const uint64_t blocks64 = (words + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? blocks64 : 4096);
  hipError_t e = hipLaunchKernel(rrt::zero_kernel_ptr(), dim3(blocks), dim3(256), args, 0, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ELAUNCH, std::string("workspace init: ") + hipGetErrorString(e));
  return TOPK_OK;
}

}  // extern "C"

namespace {

int launch(const void* scores, int64_t row_stride, const int32_t* lengths, const int32_t* row_offsets,
           int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx, void* workspace, hipStream_t stream,
           const topk_overrides* ov, float* out_val = nullptr, bool bf16 = false, bool noalloc = false) {
  if (num_rows < 0) return fail(TOPK_EINVAL, "num_rows must be >= 0");
  if (next_n < 1) return fail(TOPK_EINVAL, "next_n must be >= 1");
  if (num_rows % next_n != 0) return fail(TOPK_EINVAL, "num_rows must be a multiple of next_n");
  int rc = check_common(num_rows, row_stride, K);
  if (rc != TOPK_OK) return rc;
  if (num_rows == 0) return TOPK_OK;
  if (scores == nullptr || lengths == nullptr || out_idx == nullptr)
    return fail(TOPK_EINVAL, "null scores, lengths or out_idx");
  if (reinterpret_cast<uintptr_t>(out_idx) % 4 != 0 || reinterpret_cast<uintptr_t>(lengths) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(scores) % (bf16 ? 2 : 4) != 0 || reinterpret_cast<uintptr_t>(row_offsets) % 4 != 0)
    return fail(TOPK_EINVAL, "scores must be aligned to their element; lengths, row_offsets and out_idx to 4 bytes");
  const bool big = K > rrt::kMaxK;
  topk_plan plan;
  int dev = 0;
  rc = plan_for_call(scores, num_rows, row_stride, K, ov, stream, &dev, &plan, bf16);
  if (rc != TOPK_OK) return rc;
  if (noalloc && plan.workspace_bytes > 0) {
    // The library's static scratch array stands in for the workspace.
    if (plan.workspace_bytes > rrt::kNoallocScratchBytes)
      return fail(TOPK_EWORKSPACE, "this launch needs " + std::to_string(plan.workspace_bytes) +
                                       " bytes of workspace; the allocation-free entry point's scratch holds " +
                                       std::to_string(rrt::kNoallocScratchBytes) + " (" + describe(plan) + ")");
    const char* what = "";
    const int e = rrt::noalloc_scratch(dev, stream, &workspace, &what);
    if (e != 0)
      return fail(TOPK_EDEVICE, std::string(what) + ": " + hipGetErrorString(static_cast<hipError_t>(e)));
  }
  if (plan.workspace_bytes > 0 && workspace == nullptr)
    return fail(TOPK_EWORKSPACE, "this launch needs a workspace of " + std::to_string(plan.workspace_bytes) +
                                     " bytes (" + describe(plan) + ")");
  if (plan.workspace_bytes > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TOPK_EINVAL, "workspace must be 256-byte aligned");

  rrt::KernelParams kp{};
  kp.scores = scores;
  kp.lengths = lengths;
  kp.row_offsets = row_offsets;
  kp.out_val = out_val;
  kp.out = out_idx;
  kp.ws = plan.workspace_bytes > 0 ? static_cast<uint8_t*>(workspace) : nullptr;
  kp.row_stride = row_stride;
  kp.chunk = plan.chunk;
  kp.group_bytes = plan.path == TOPK_PATH_MULTI
                       ? rrt::group_layout(plan.wg_per_row, rrt::cap_of(rrt::layout_of(plan.idx16 != 0, big, plan.block)))
                             .bytes
                       : 0;
  kp.num_rows = num_rows;
  kp.K = K;
  kp.wg_per_row = plan.wg_per_row;
  kp.spin_limit = (ov != nullptr && ov->spin_limit > 0) ? ov->spin_limit : rrt::kDefaultSpin;
  kp.wait_extra = (ov != nullptr && ov->force_wait_timeout != 0) ? 1u : 0u;

  if (verbose()) std::fprintf(stderr, "[topk_ragged] rows=%d stride=%lld K=%d %s\n", num_rows,
                              (long long)row_stride, K, describe(plan).c_str());
  void* args[] = {&kp};
  const void* fn = rrt::kernel_ptr(plan.path, plan.vec, plan.idx16 != 0, out_val != nullptr, bf16, big, plan.block);
  if (fn == nullptr) return fail(TOPK_EINVAL, "no kernel instance for this plan (" + describe(plan) + ")");
  hipError_t e = hipLaunchKernel(fn, dim3(plan.grid), dim3(plan.block), args, 0, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    char buf[640];
    std::snprintf(buf, sizeof(buf), "kernel launch failed: %s (K=%d %s)", hipGetErrorString(e), K,
                  describe(plan).c_str());
    return fail(TOPK_ELAUNCH, buf);
  }
  return TOPK_OK;
}

}  // namespace

extern "C" {

int topk_ragged_ex(const float* scores, int64_t row_stride, const int32_t* lengths, int32_t num_rows,
                   int32_t next_n, int32_t K, int32_t* out_idx, void* workspace, hipStream_t stream,
                   const topk_overrides* ov) {
  return launch(scores, row_stride, lengths, nullptr, num_rows, next_n, K, out_idx, workspace, stream, ov);
}

int topk_ragged(const float* scores, int64_t row_stride, const int32_t* lengths, int32_t num_rows,
                int32_t next_n, int32_t K, int32_t* out_idx, void* workspace, hipStream_t stream) {
  return launch(scores, row_stride, lengths, nullptr, num_rows, next_n, K, out_idx, workspace, stream, nullptr);
}

int topk_ragged_noalloc(const float* scores, int64_t row_stride, const int32_t* lengths, int32_t num_rows,
                        int32_t next_n, int32_t K, int32_t* out_idx, hipStream_t stream) {
  return launch(scores, row_stride, lengths, nullptr, num_rows, next_n, K, out_idx, nullptr, stream, nullptr,
                nullptr, false, true);
}

int topk_ragged_offsets(const float* scores, int64_t row_stride, const int32_t* lengths,
                        const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                        int32_t* out_idx, void* workspace, hipStream_t stream) {
  if (num_rows > 0 && row_offsets == nullptr) return fail(TOPK_EINVAL, "null row_offsets");
  return launch(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, workspace, stream,
                nullptr);
}

int topk_ragged_strided_workspace_size(int32_t num_rows, int64_t num_cols, int32_t K, hipStream_t stream,
                                       size_t* bytes) {
  if (bytes == nullptr) return fail(TOPK_EINVAL, "null bytes");
  if (num_cols < 1 || num_cols > INT32_MAX) return fail(TOPK_EINVAL, "num_cols must be in [1, 2^31 - 1]");
  size_t plan_bytes = 0;
  const int rc = topk_ragged_workspace_size(num_rows, num_cols, K, stream, &plan_bytes);
  if (rc != TOPK_OK) return rc;
  *bytes = num_rows == 0 ? 0 : rrt::round_up(plan_bytes, 256) + 4ull * (uint64_t)num_rows * (uint64_t)num_cols;
  return TOPK_OK;
}

int topk_ragged_strided(const float* scores, int64_t row_stride, int64_t col_stride, int64_t num_cols,
                        const int32_t* lengths, const int32_t* row_offsets, int32_t num_rows, int32_t next_n,
                        int32_t K, int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream) {
  if (num_rows < 0) return fail(TOPK_EINVAL, "num_rows must be >= 0");
  if (col_stride < 1) return fail(TOPK_EINVAL, "col_stride must be >= 1");
  if (row_stride < 0) return fail(TOPK_EINVAL, "row_stride must be >= 0");
  size_t need = 0;
  int rc = topk_ragged_strided_workspace_size(num_rows, num_cols, K, stream, &need);
  if (rc != TOPK_OK) return rc;
  if (num_rows == 0) return TOPK_OK;
  if (scores == nullptr || lengths == nullptr) return fail(TOPK_EINVAL, "null scores or lengths");
  if (workspace == nullptr) return fail(TOPK_EWORKSPACE, "strided rows need a workspace of " + std::to_string(need) +
                                                             " bytes (topk_ragged_strided_workspace_size)");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(TOPK_EINVAL, "workspace must be 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(scores) % 4 != 0 || reinterpret_cast<uintptr_t>(lengths) % 4 != 0)
    return fail(TOPK_EINVAL, "scores and lengths must be 4-byte aligned");
  size_t plan_bytes = 0;
  rc = topk_ragged_workspace_size(num_rows, num_cols, K, stream, &plan_bytes);
  if (rc != TOPK_OK) return rc;
  float* packed = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + rrt::round_up(plan_bytes, 256));
  {
    const int64_t tiles = ((num_rows + 63) / 64) * ((num_cols + 63) / 64);
    const unsigned blocks = (unsigned)std::min<int64_t>(tiles, 4096);
    void* args[] = {&scores, &row_stride, &col_stride, &num_cols, &lengths, &num_rows, &packed};
    hipError_t e = hipLaunchKernel(rrt::pack_kernel_ptr(), dim3(blocks), dim3(256), args, 0, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(TOPK_ELAUNCH, std::string("pack kernel: ") + hipGetErrorString(e));
  }
  void* plan_ws = plan_bytes > 0 ? workspace : nullptr;
  if (out_val != nullptr)
    return topk_ragged_values_ex(packed, num_cols, lengths, row_offsets, num_rows, next_n, K, out_idx, out_val,
                                 plan_ws, stream, nullptr);
  return launch(packed, num_cols, lengths, row_offsets, num_rows, next_n, K, out_idx, plan_ws, stream, nullptr);
}

int topk_ragged_values_ex(const float* scores, int64_t row_stride, const int32_t* lengths,
                          const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                          int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream,
                          const topk_overrides* ov) {
  if (num_rows > 0 && out_val == nullptr) return fail(TOPK_EINVAL, "null out_val");
  if (reinterpret_cast<uintptr_t>(out_val) % 4 != 0) return fail(TOPK_EINVAL, "out_val must be 4-byte aligned");
  return launch(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, workspace, stream, ov,
                out_val);
}

int topk_ragged_values(const float* scores, int64_t row_stride, const int32_t* lengths, const int32_t* row_offsets,
                       int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx, float* out_val,
                       void* workspace, hipStream_t stream) {
  return topk_ragged_values_ex(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, out_val,
                               workspace, stream, nullptr);
}

int topk_ragged_bf16_ex(const uint16_t* scores, int64_t row_stride, const int32_t* lengths,
                        const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx,
                        float* out_val, void* workspace, hipStream_t stream, const topk_overrides* ov) {
  if (reinterpret_cast<uintptr_t>(scores) % 2 != 0) return fail(TOPK_EINVAL, "bf16 scores must be 2-byte aligned");
  if (reinterpret_cast<uintptr_t>(out_val) % 4 != 0) return fail(TOPK_EINVAL, "out_val must be 4-byte aligned");
  return launch(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, workspace, stream, ov,
                out_val, true);
}

int topk_ragged_bf16(const uint16_t* scores, int64_t row_stride, const int32_t* lengths, const int32_t* row_offsets,
                     int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx, float* out_val,
                     void* workspace, hipStream_t stream) {
  return topk_ragged_bf16_ex(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, out_val,
                             workspace, stream, nullptr);
}

int topk_ragged_offsets_ex(const float* scores, int64_t row_stride, const int32_t* lengths,
                           const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                           int32_t* out_idx, void* workspace, hipStream_t stream, const topk_overrides* ov) {
  if (num_rows > 0 && row_offsets == nullptr) return fail(TOPK_EINVAL, "null row_offsets");
  return launch(scores, row_stride, lengths, row_offsets, num_rows, next_n, K, out_idx, workspace, stream, ov);
}

const char* topk_ragged_last_error(void) { return g_last_error.c_str(); }

int topk_ragged_workspace_status(const void* workspace, hipStream_t stream, uint32_t* flags) {
  if (flags == nullptr) return fail(TOPK_EINVAL, "null flags");
  *flags = 0;
  if (workspace == nullptr) return TOPK_OK;
  hipError_t e = hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(TOPK_EDEVICE, std::string("workspace status: ") + hipGetErrorString(e));
  return TOPK_OK;
}

int topk_ragged_debug_keys(const uint32_t* bits, uint32_t* keys, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(TOPK_EINVAL, "n must be >= 0");
  if (n == 0) return TOPK_OK;
  if (bits == nullptr || keys == nullptr) return fail(TOPK_EINVAL, "null bits or keys");
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return fail(TOPK_EINVAL, "n too large");
  void* args[] = {&bits, &keys, &n};
  hipError_t e = hipLaunchKernel(rrt::keys_kernel_ptr(), dim3((unsigned)blocks), dim3(256), args, 0, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ELAUNCH, std::string("keys kernel: ") + hipGetErrorString(e));
  return TOPK_OK;
}

int topk_ragged_read_reference(const float* scores, int64_t row_stride, const int32_t* lengths,
                               int32_t num_rows, uint32_t* row_max_keys, hipStream_t stream) {
  if (num_rows < 0) return fail(TOPK_EINVAL, "num_rows must be >= 0");
  if (row_stride < 1 || row_stride > INT32_MAX) return fail(TOPK_EINVAL, "row_stride must be in [1, 2^31 - 1]");
  if (num_rows == 0) return TOPK_OK;
  if (scores == nullptr || lengths == nullptr || row_max_keys == nullptr)
    return fail(TOPK_EINVAL, "null scores, lengths or row_max_keys");
  if (reinterpret_cast<uintptr_t>(scores) % 4 != 0 || reinterpret_cast<uintptr_t>(lengths) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(row_max_keys) % 4 != 0)
    return fail(TOPK_EINVAL, "scores, lengths and row_max_keys must be 4-byte aligned");
  int dev = 0;
  int rc = stream_device(stream, &dev);
  if (rc != TOPK_OK) return rc;
  DevCache* d = nullptr;
  rc = device_info(dev, &d);
  if (rc != TOPK_OK) return rc;
  const int vec = vec_allowed_for(scores, row_stride);
  int occ = 0;
  rc = occupancy(dev, d, 3, vec, false, &occ);
  if (rc != TOPK_OK) return rc;
  if (occ < 1) return fail(TOPK_EDEVICE, "read reference kernel cannot be resident");
  const int64_t cap = (int64_t)d->num_cus.load(std::memory_order_relaxed) * occ;
  const int64_t grid = num_rows < cap ? num_rows : cap;
  rrt::KernelParams kp{};
  kp.scores = scores;
  kp.lengths = lengths;
  kp.out = reinterpret_cast<int32_t*>(row_max_keys);
  kp.row_stride = row_stride;
  kp.num_rows = num_rows;
  void* args[] = {&kp};
  hipError_t e = hipLaunchKernel(rrt::kernel_ptr(3, vec, false), dim3((unsigned)grid), dim3(rrt::kBlock), args,
                                 0, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(TOPK_ELAUNCH, std::string("read reference: ") + hipGetErrorString(e));
  return TOPK_OK;
}

int topk_ragged_version(void) { return 100; }

}  // extern "C"
