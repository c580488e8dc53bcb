/*
 * topk_ragged.h -- ragged per-row top-K on AMD Instinct MI355X (gfx950).
 *
 * The operation (vLLM persistent_topk pages: PR #54110 "low shared memory
 * fallback", its csrc/libtorch_stable/topk.cu excerpt, which passes logits,
 * next_n, lengths, the output and both logits strides to the per-row decode
 * top-K; PR #41189 "cooperative barrier deadlock fix", its csrc/topk.cu
 * excerpt, which hands fp32 logits to the top-K and gets int32 indices back):
 *
 *   for every row r of an fp32 score matrix, return the int32 column indices
 *   of the K largest scores among the first lengths[r] entries.
 *
 * The pages leave three things open; this library fixes them so that exactly
 * one output is correct:
 *   - ties: of two equal scores the lower index wins (IEEE equality, so -0.0
 *     and +0.0 are equal);
 *   - order: the chosen indices are written in ascending index order;
 *   - short rows: when lengths[r] < K the row is padded with -1.
 *
 * All pointers given to topk_ragged are DEVICE pointers owned by the caller.
 * The library never allocates device memory, never synchronises and never
 * issues a host memset on the launch path, so a launch can be captured in a
 * hipGraph and replayed.  Every call is asynchronous on `stream`; the device
 * is the stream's device.  Device properties and kernel occupancies are
 * queried once per device and cached.
 *
 * Return values are topk_status codes.  On failure a description is
 * available from topk_ragged_last_error() (thread-local).  A kernel that
 * faults reports at the caller's next synchronisation, like any HIP op.
 *
 * Scores are ordinary IEEE fp32 values (or bf16, widened exactly).  A NaN in
 * a row's valid prefix is outside the contract: NaNs are never selected, so
 * a row with fewer than K non-NaN values among its first lengths[r] entries
 * gets undefined output.  Entries at or past lengths[r] are never read and
 * may hold anything, NaN included.
 */
#ifndef TOPK_RAGGED_H
#define TOPK_RAGGED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TOPK_OK = 0,
  TOPK_EINVAL = -1,          /* bad pointer, size, stride, next_n or alignment */
  TOPK_EUNSUPPORTED_K = -2,  /* K outside [1, TOPK_RAGGED_MAX_K] */
  TOPK_EWORKSPACE = -3,      /* the plan needs a workspace and none was given */
  TOPK_EDEVICE = -4,         /* a HIP runtime query failed */
  TOPK_ELAUNCH = -5          /* the kernel launch reported an error */
} topk_status;

#define TOPK_RAGGED_MAX_K 4096
/* Rows whose stride exceeds this may be split over several workgroups that
 * cooperate through the workspace (the pages' RADIX_THRESHOLD of 32K with a
 * strict comparison: PR #41189 page, csrc/topk.cu excerpt and review notes). */
#define TOPK_RAGGED_RADIX_THRESHOLD 32768

/*
 * topk_ragged -- the hot path.
 *
 *   scores     fp32, row r starts at scores + r * row_stride (elements), column
 *              stride 1.  Only entries [0, lengths[r]) of row r are read.
 *   row_stride elements between row starts, >= 1.
 *   lengths    int32, num_rows entries, one per row.  Multi-token layouts
 *              ([batch, next_n] row-major, PR #54110 page, topk.cu excerpt)
 *              are passed flattened: row b*next_n + j belongs to batch b.
 *              A length outside [0, row_stride] is clamped into it.
 *   num_rows   >= 0; 0 is a successful no-op.
 *   next_n     >= 1 and divides num_rows.  It groups rows and never changes
 *              which indices are chosen.
 *   K          1 <= K <= TOPK_RAGGED_MAX_K.
 *   out_idx    int32 [num_rows, K] contiguous, 4-byte aligned.  Row r gets
 *              min(K, n_r) ascending indices then -1s.
 *   workspace  device memory of at least topk_ragged_workspace_size() bytes
 *              for the same (num_rows, row_stride, K) and device, zeroed once
 *              by topk_ragged_workspace_init().  Every launch returns it to
 *              all-zero before it ends (in-kernel cleanup), so no per-call
 *              memset is needed.  May be NULL when the size is 0.
 *   stream     HIP stream (NULL = the current device's null stream).
 *
 * Concurrent launches that share a workspace race; give each stream its own.
 * If a launch fails or a cooperative wait times out (see
 * topk_ragged_workspace_status) the workspace contents are undefined:
 * initialise it again before reuse.
 */
int topk_ragged(const float* scores, int64_t row_stride, const int32_t* lengths,
                int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx,
                void* workspace, hipStream_t stream);

/*
 * topk_ragged_offsets -- the same selection, with each row's chosen indices
 * shifted into a flat ragged layout.  The PR #41189 page calls a
 * "RaggedTransform" variant of the ragged top-K without defining it; this
 * library reads it as: a row r whose scores start at row_offsets[r] in a
 * flat (concatenated) layout reports positions in that layout.
 *
 *   row_offsets  int32 device array, num_rows entries, 4-byte aligned.
 *   out_idx[r, i] = row_offsets[r] + (the i-th chosen index) for
 *                   i < min(K, n_r), and -1 after that (unchanged).
 *
 * The sum is formed in 32-bit two's complement; the caller keeps
 * row_offsets[r] + n_r - 1 within int32 (not checked on the device).  Every
 * other argument, the workspace and the errors are as for topk_ragged; a
 * null row_offsets with num_rows > 0 is TOPK_EINVAL.
 */
int topk_ragged_offsets(const float* scores, int64_t row_stride, const int32_t* lengths,
                        const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                        int32_t* out_idx, void* workspace, hipStream_t stream);

/*
 * topk_ragged_values -- the selection (with or without row offsets) plus the
 * chosen scores.  Not on the pages, which return indices only.
 *
 *   row_offsets  NULL, or as for topk_ragged_offsets.
 *   out_val      float device array [num_rows, K], 4-byte aligned:
 *                out_val[r, i] = the fp32 score at out_idx[r, i] (its exact
 *                bits, -0.0 included) for i < min(K, n_r), -inf after that.
 *
 * The selection writes the values itself, in the same single launch: each
 * chosen entry's stored fp32 bits go out beside its index, so no score is
 * read twice and -0.0 stays -0.0.  Other arguments and errors as for
 * topk_ragged; a null out_val with num_rows > 0 is TOPK_EINVAL.
 */
int topk_ragged_values(const float* scores, int64_t row_stride, const int32_t* lengths,
                       const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                       int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream);

/*
 * topk_ragged_strided -- rows with any column stride (the pages' op takes
 * both logits strides: PR #54110 page, the top_k_per_row_decode call).
 *
 *   scores       element (r, c) at scores + r * row_stride + c * col_stride;
 *                row_stride >= 0, col_stride >= 1 (elements).
 *   num_cols     columns of the matrix (>= 1): lengths are clamped to
 *                [0, num_cols], since row_stride no longer bounds a row.
 *   row_offsets  NULL or as for topk_ragged_offsets; out_val NULL or as for
 *                topk_ragged_values.
 *   workspace    at least topk_ragged_strided_workspace_size() bytes,
 *                256-byte aligned, zeroed once by topk_ragged_workspace_init.
 *                Its first part is the ordinary workspace of
 *                (num_rows, num_cols, K), returned to zero by every launch;
 *                after it, each row's valid prefix is packed contiguously
 *                (contents undefined between launches).
 *
 * Each row's valid prefix is first copied into the workspace (nothing past a
 * length is read), then selected as contiguous rows of stride num_cols.  A
 * slow path for unusual layouts: it reads the valid scores once strided and
 * once packed.  Asynchronous, graph-capturable; errors as for topk_ragged.
 */
int topk_ragged_strided_workspace_size(int32_t num_rows, int64_t num_cols, int32_t K,
                                       hipStream_t stream, size_t* bytes);
int topk_ragged_strided(const float* scores, int64_t row_stride, int64_t col_stride, int64_t num_cols,
                        const int32_t* lengths, const int32_t* row_offsets, int32_t num_rows,
                        int32_t next_n, int32_t K, int32_t* out_idx, float* out_val,
                        void* workspace, hipStream_t stream);

/*
 * topk_ragged_bf16 -- the same selection over bf16 scores (not on the pages,
 * whose logits are fp32).
 *
 *   scores       bf16 values as their 16 bits, row r at scores + r * row_stride
 *                (elements), 2-byte aligned; rows with a 16-byte-aligned start
 *                and row_stride % 8 == 0 load 8 elements at a time.
 *   row_offsets  NULL or as for topk_ragged_offsets.
 *   out_val      NULL or as for topk_ragged_values: the chosen scores widened
 *                to fp32 (exact).
 *
 * Each score is widened to fp32 by shifting its bits up, which is exact, so
 * the order, the ties and the chosen indices are those of the fp32 values.
 * Workspace and errors as for topk_ragged (topk_ragged_workspace_size gives
 * the size for the same shape).
 */
int topk_ragged_bf16(const uint16_t* scores, int64_t row_stride, const int32_t* lengths,
                     const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                     int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream);

/* Bytes of workspace topk_ragged needs for this shape on the stream's device.
 * The PR #41444 page (risk section) relies on the workspace being large
 * enough and on a check that it is; here the size is a function of the
 * launch plan, and a launch that needs one and is given NULL fails with
 * TOPK_EWORKSPACE.
 *
 *   num_rows, row_stride, K  as for topk_ragged (same ranges and errors).
 *   stream                   selects the device whose properties the plan uses.
 *   bytes                    host pointer, receives the size; must not be NULL
 *                            (TOPK_EINVAL).
 *
 * *bytes = 0 means no workspace is used: one workgroup per row and no more
 * rows than resident workgroups (the PR #41748 page, Motivation: rows up to
 * the radix threshold need no workspace).  With more rows than that, a
 * 256-byte workspace holds the counter that hands rows to workgroups as they
 * finish; rows that several workgroups share need a block per row on top. */
int topk_ragged_workspace_size(int32_t num_rows, int64_t row_stride, int32_t K,
                               hipStream_t stream, size_t* bytes);

/* One-time zeroing of a freshly allocated workspace.  The PR #41748 page
 * (Motivation) replaces a per-call memset of the workspace with cleanup at
 * the end of the kernel; this call is the zeroing that remains, once per
 * allocation.  Every launch leaves the workspace all-zero again, so it is
 * not needed between launches, only after a failed launch.
 *
 *   workspace  device pointer, 4-byte aligned; may be NULL when bytes == 0.
 *   bytes      a multiple of 4.
 *   stream     the fill runs asynchronously on it, as a small kernel (not a
 *              memset node, so it can be captured in a graph).
 *
 * Errors: TOPK_EINVAL for a NULL or misaligned workspace with bytes > 0;
 * TOPK_ELAUNCH if the fill kernel cannot be launched.  The caller owns the
 * memory. */
int topk_ragged_workspace_init(void* workspace, size_t bytes, hipStream_t stream);

/* Diagnostic text for the last failing call on this host thread ("" if none):
 * the counterpart of the checks with messages that the PR #41189 page's
 * topk.cu excerpt raises (for example when the occupancy query fails, with
 * the HIP error string, or when a launch would oversubscribe, with the plan's
 * numbers).  The pointer stays valid until the next failing call on the same
 * thread; the library owns it. */
const char* topk_ragged_last_error(void);

/* ---------------------------------------------------------------------------
 * Planning, overrides and diagnostics.  These expose the launch decision so
 * that it can be tested without a GPU and forced down each code path.
 * ------------------------------------------------------------------------- */

/* Device facts the planner uses.  occupancy_* are workgroups per CU of the
 * exact kernel instance that would run (PR #41189 page, implementation
 * notes: query the instance actually launched, not a sibling).  The "16"
 * instances serve rows or chunks of at most 65536 elements: at 256 threads
 * they keep 16-bit candidate indices, at 512 and 1024 threads 32-bit ones in
 * a larger candidate buffer (one workgroup per CU at 512 threads below the
 * large K). */
typedef struct {
  int32_t num_cus;
  int32_t occupancy_single;    /* one workgroup per row kernel, 32-bit indices */
  int32_t occupancy_multi;     /* several workgroups per row kernel, 32-bit indices */
  int32_t max_lds_per_block;
  int32_t occupancy_single16;  /* one workgroup per row kernel, 16-bit indices */
  int32_t occupancy_multi16;   /* several workgroups per row kernel, 16-bit indices */
  /* The same four occupancies (single, multi, single16, multi16) of the
   * 512- and 1024-thread instances; 0 where the library has no such
   * instance or it cannot be resident.  The fields above describe the
   * 256-thread instances. */
  int32_t occupancy_w512[4];
  int32_t occupancy_w1024[4];
} topk_device_props;

typedef enum {
  TOPK_PATH_NONE = 0,    /* num_rows == 0 */
  TOPK_PATH_SINGLE = 1,  /* one workgroup owns a row; persistent grid over rows */
  TOPK_PATH_MULTI = 2    /* wg_per_row workgroups split a row, merge through the workspace */
} topk_path;

typedef struct {
  int32_t path;           /* topk_path */
  int32_t kmax;           /* largest K the kernel instance handles: 2048, or 4096 for the
                             large layout that K above 2048 takes */
  int32_t vec;            /* elements per load: 4, 2 or 1 (fp32), 8 or 1 (bf16); fp32 rows on 512- or
                             1024-thread workgroups load 1 unless force_vec says otherwise */
  int32_t block;          /* threads per workgroup: 256, or 512 / 1024 (8 or 16 wavefronts per row) */
  int32_t grid;           /* workgroups launched */
  int32_t wg_per_row;     /* G (1 on the single path) */
  int64_t chunk;          /* elements of a row per workgroup (multi path) */
  int32_t resident_cap;   /* num_cus * occupancy of the chosen kernel */
  int32_t headroom;       /* slots left free when workgroups wait on each other */
  int32_t lds_bytes;      /* static LDS per workgroup */
  int32_t fell_back;      /* 1 if a requested multi plan could not be made co-resident */
  int32_t idx16;          /* 1 if the instance serves rows or chunks of at most 65536 elements (16-bit
                             candidate indices at 256 threads) */
  uint64_t workspace_bytes;
} topk_plan;

typedef struct {
  int32_t force_path;        /* 0 auto, TOPK_PATH_SINGLE or TOPK_PATH_MULTI */
  int32_t force_wg_per_row;  /* 0 auto, else G for the multi path */
  int32_t max_grid;          /* 0 auto, else cap on the single path's persistent grid */
  int32_t force_vec;         /* 0 auto, else 1, 2 or 4 for fp32, 1 or 8 for bf16 (must suit the alignment) */
  int64_t force_chunk;       /* 0 auto, else elements per workgroup (multiple of 4) */
  uint32_t spin_limit;       /* 0 default; bound on a cooperative wait (polls) */
  int32_t min_chunk;         /* 0 default; smallest per-workgroup chunk the planner picks */
  int32_t max_occupancy;     /* 0 the device's, else plan as if no instance could keep more
                                workgroups per CU resident (emulates a smaller device) */
  int32_t force_idx32;       /* 1: never keep 16-bit candidate indices (testing) */
  int32_t force_block;       /* 0 auto, else threads per workgroup: 256, 512 or 1024 */
  int32_t force_wait_timeout; /* 1: every cooperative wait waits for one arrival more than can come, so it
                                 gives up after spin_limit polls and sets error bit 0 (testing the bound
                                 on waits; the results of such a launch are undefined) */
} topk_overrides;

/* Pure planning function (host only, no GPU needed).  vec_allowed is the
 * widest load, in elements, the pointer/stride alignment permits (1, 2, 4
 * or 8).  ov may be NULL. */
int topk_ragged_plan(const topk_device_props* props, int32_t num_rows, int64_t row_stride,
                     int32_t K, int32_t vec_allowed, const topk_overrides* ov,
                     topk_plan* plan);

/* The plan topk_ragged / topk_ragged_ex would use for these arguments on the
 * stream's device (queries and caches occupancy). */
int topk_ragged_query_plan(const float* scores, int32_t num_rows, int64_t row_stride,
                           int32_t K, const topk_overrides* ov, hipStream_t stream,
                           topk_plan* plan);

/* Workspace bytes for the plan chosen under overrides ov. */
int topk_ragged_workspace_size_ex(const float* scores, int32_t num_rows, int64_t row_stride,
                                  int32_t K, const topk_overrides* ov, hipStream_t stream,
                                  size_t* bytes);

/* topk_ragged / topk_ragged_offsets with planner overrides (testing and
 * benchmarking). */
int topk_ragged_ex(const float* scores, int64_t row_stride, const int32_t* lengths,
                   int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx,
                   void* workspace, hipStream_t stream, const topk_overrides* ov);
int topk_ragged_offsets_ex(const float* scores, int64_t row_stride, const int32_t* lengths,
                           const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                           int32_t* out_idx, void* workspace, hipStream_t stream,
                           const topk_overrides* ov);
int topk_ragged_values_ex(const float* scores, int64_t row_stride, const int32_t* lengths,
                          const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                          int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream,
                          const topk_overrides* ov);
int topk_ragged_bf16_ex(const uint16_t* scores, int64_t row_stride, const int32_t* lengths,
                        const int32_t* row_offsets, int32_t num_rows, int32_t next_n, int32_t K,
                        int32_t* out_idx, float* out_val, void* workspace, hipStream_t stream,
                        const topk_overrides* ov);

/* Error bits a kernel left in the workspace header (synchronises stream):
 * bit 0: a cooperative wait hit its spin limit; bit 1: a threshold search
 * found the histogram inconsistent.  0 = healthy. */
int topk_ragged_workspace_status(const void* workspace, hipStream_t stream, uint32_t* flags);

/* Key-transform probe (testing only): keys[i] = the device's order-preserving
 * uint32 key of the fp32 bit pattern bits[i], for i < n.  Both arrays are
 * device memory; asynchronous on stream. */
int topk_ragged_debug_keys(const uint32_t* bits, uint32_t* keys, int64_t n, hipStream_t stream);

/* Streaming-read reference (measurement only): row_max_keys[r] = the
 * order-preserving uint32 key of the largest of the first lengths[r] scores of
 * row r (0 for an empty row).  It reads exactly the bytes topk_ragged reads,
 * with the same tiles, load width and prefetch depth, and does no selection,
 * so its rate bounds what the selection can reach on the same input.
 * Arguments as for topk_ragged; row_max_keys is a device array of num_rows
 * entries.  Asynchronous on stream. */
int topk_ragged_read_reference(const float* scores, int64_t row_stride, const int32_t* lengths,
                               int32_t num_rows, uint32_t* row_max_keys, hipStream_t stream);

/*
 * topk_ragged_noalloc -- topk_ragged without a workspace argument, for
 * callers that cannot allocate device memory: code under hipGraph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results and errors are those of topk_ragged.  Where a launch
 * needs a workspace it uses a library-owned static device array of
 * TOPK_RAGGED_NOALLOC_SCRATCH_BYTES (8 MiB) instead: one per GPU, held
 * from the first call on that GPU until the process ends.  The call never
 * allocates or frees device memory.
 *   - A launch whose plan needs more than that fails with TOPK_EWORKSPACE
 *     and launches nothing (topk_ragged_workspace_size gives the need: the
 *     prefill-shaped batches need 256 bytes, rows of 131072 elements at
 *     K = 2048 about 0.41 MB per row, more for K above 2048).
 *   - The first call on a GPU also queues a fill kernel on `stream` that
 *     zeroes the array, ahead of its own launch; every launch leaves the
 *     array all-zero again (in-kernel cleanup).
 *   - Every call on a GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, or different host threads without
 *     ordering) race and give undefined results.  Serialise them.
 */
#define TOPK_RAGGED_NOALLOC_SCRATCH_BYTES (8u << 20)
int topk_ragged_noalloc(const float* scores, int64_t row_stride, const int32_t* lengths,
                        int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx,
                        hipStream_t stream);

/* Library version: major * 10000 + minor * 100 + patch. */
int topk_ragged_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_RAGGED_H */
