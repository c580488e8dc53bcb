// CPU oracle for ragged per-row top-K.  TEST INFRASTRUCTURE ONLY.
//
// Only the tests, the package's smoke check and the benchmark's CPU-baseline
// leg may load this library.  The product path (the HIP library) shares no
// code, header or table with it and never calls it.
//
// What it computes.  The pages (vLLM persistent_topk; PR #54110 "low shared
// memory fallback", the top_k_per_row_decode call; PR #41189, the
// FilteredTopKRaggedTransform<float, int32_t, TopK> call) describe one op: for
// each row of an fp32 logits matrix, the int32 indices of the TopK largest
// entries among the first lengths[row] entries.  The pages fix neither the tie
// rule, the output order nor what fills a short row; this oracle uses the
// readings adopted for this library:
//
//   n   = clamp(lengths[r], 0, row_stride)
//   m   = min(K, n)
//   c beats d  <=>  v(c) > v(d)  or  (v(c) == v(d) and c < d)
//       (IEEE comparison, so -0.0 == +0.0; a strict total order when the
//       valid prefix holds no NaN)
//   S_r = the m positions beaten by fewer than K others (unique)
//   out[r, 0:m) = S_r in ascending index order, out[r, m:K) = -1
//
// Algorithm: per row, std::nth_element on the index array with the "beats"
// order puts the m best positions first (a strict total order makes that set
// unique), std::sort orders them by index, the rest is -1.  Rows are split
// over std::thread workers.  No fast-math: build with plain -O2/-O3.
//
// Error codes: 0 ok; -1 invalid arguments; -2 a NaN inside some row's valid
// prefix (out of contract: the order above is not total there).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <thread>
#include <vector>

namespace {

struct Beats {
  const float* v;
  bool operator()(int32_t c, int32_t d) const {
    if (v[c] > v[d]) return true;
    if (v[c] == v[d]) return c < d;
    return false;
  }
};

int one_row(const float* row, int64_t n, int32_t K, int32_t* out,
            std::vector<int32_t>& idx) {
  for (int64_t c = 0; c < n; ++c)
    if (std::isnan(row[c])) return -2;
  const int64_t m = std::min<int64_t>(K, n);
  idx.resize(static_cast<size_t>(n));
  for (int64_t c = 0; c < n; ++c) idx[c] = static_cast<int32_t>(c);
  if (m > 0 && m < n)
    std::nth_element(idx.begin(), idx.begin() + (m - 1), idx.end(), Beats{row});
  std::sort(idx.begin(), idx.begin() + m);
  for (int64_t i = 0; i < m; ++i) out[i] = idx[i];
  for (int64_t i = m; i < K; ++i) out[i] = -1;
  return 0;
}

}  // namespace

extern "C" {

// scores: host fp32, row r at scores + r*row_stride; lengths: host int32, one
// per row (rows b*next_n + j belong to batch element b, which does not change
// the selection); out_idx: host int32 [num_rows, K].  nthreads <= 0 means
// std::thread::hardware_concurrency().
int oracle_topk_ragged(const float* scores, int64_t row_stride, const int32_t* lengths,
                       int32_t num_rows, int32_t next_n, int32_t K, int32_t* out_idx,
                       int32_t nthreads) {
  if (num_rows < 0 || row_stride < 1 || K < 1 || next_n < 1) return -1;
  if (num_rows % next_n != 0) return -1;
  if (num_rows == 0) return 0;
  if (!scores || !lengths || !out_idx) return -1;
  int nt = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  if (nt < 1) nt = 1;
  if (nt > num_rows) nt = num_rows;
  std::atomic<int32_t> next_row{0};
  std::atomic<int> status{0};
  auto worker = [&]() {
    std::vector<int32_t> idx;
    for (;;) {
      const int32_t r = next_row.fetch_add(1);
      if (r >= num_rows) break;
      int64_t n = lengths[r];
      if (n < 0) n = 0;
      if (n > row_stride) n = row_stride;
      const int rc = one_row(scores + static_cast<int64_t>(r) * row_stride, n, K,
                             out_idx + static_cast<int64_t>(r) * K, idx);
      if (rc != 0) status.store(rc);
    }
  };
  if (nt == 1) {
    worker();
  } else {
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) pool.emplace_back(worker);
    for (auto& t : pool) t.join();
  }
  return status.load();
}

int oracle_abi_version(void) { return 1; }

}  // extern "C"
