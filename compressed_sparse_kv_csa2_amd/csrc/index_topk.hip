// csa2_index_topk and csa2_select_chain: the scan and its selections in the two launches of
// the filtered selection (fsel.hip) for rows whose candidates it can hold; longer rows take
// the separate scan (index_score.hip, scores written out) and top-k (topk.hip) launches
// inside the same call, with the same results.  csa2_replay_select: the causal score matrix
// of a chunk of queries (prefill.hip's contraction), then the same selections on it.
#include "csa2_internal.h"
#include "select_device.h"

namespace csa2 {

// Valid (non-negative) leading entries of each row of a -1 padded list.
__global__ __launch_bounds__(256) void k_count_valid(const int32_t* __restrict__ list, int k,
                                                     int32_t* __restrict__ n_out) {
  __shared__ uint32_t s_scan[32];
  const int b = blockIdx.x;
  uint32_t c = 0;
  for (int i = threadIdx.x; i < k; i += 256) c += list[(size_t)b * k + i] >= 0 ? 1u : 0u;
  uint32_t total;
  block_exclusive_scan(c, s_scan, &total);
  if (threadIdx.x == 0) n_out[b] = (int32_t)total;
}

namespace {

// Two-launch path of one selection: [scores f32 batch x n_cols][top-k workspace].
size_t two_step_bytes(int batch, int n_cols) {
  return align_up((size_t)batch * n_cols * 4, 256) + topk_ws_bytes(batch, n_cols);
}

hipError_t two_step(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                    const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand, int batch,
                    int n_cols, int k, int32_t* idx_out, float* score_out, char* p,
                    hipStream_t stream) {
  float* scores = reinterpret_cast<float*>(p);
  const TopkWs tw = topk_ws_carve(p + align_up((size_t)batch * n_cols * 4, 256), batch, n_cols);
  hipError_t e = launch_index_score(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols,
                                    scores, tw.hist1, stream);
  if (e != hipSuccess) return e;
  return launch_topk(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, true, tw, stream);
}

}  // namespace

// Every layout starts with the 256-byte status block (zero on the long-row path).
constexpr size_t kStatusBlock = 256;

// Rows the filtered selection may take hold room for either path (which one runs depends
// on k as well).
size_t index_topk_ws_bytes(int batch, int n_cols) {
  const size_t two = kStatusBlock + two_step_bytes(batch, n_cols);
  if (fsel_len_ok(n_cols)) return max(fsel_ws_bytes(batch, n_cols, false), two);
  return two;
}

hipError_t launch_index_topk(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                             const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                             int batch, int n_cols, int k, int32_t* idx_out, float* score_out,
                             void* ws, hipStream_t stream) {
  // short rows: one launch when few, else the scores written out and one selecting
  // workgroup per row (measured faster than the filtered selection's two launches there)
  if (fsmall_fits(batch, n_cols))
    return launch_fsmall(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols, k, idx_out,
                         score_out, ws, stream);
  if (fsel_fits(n_cols, k) && n_cols > kTopkSmallMax)
    return launch_fsel(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols, k, idx_out,
                       score_out, 0, nullptr, nullptr, 0, 0, nullptr, nullptr, false, ws, stream);
  return two_step(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols, k, idx_out,
                  score_out, static_cast<char*>(ws) + kStatusBlock, stream);
}

// Long rows: [status][two-step part][pool scores f32 batch x pool_k][pool sizes][Reindex
// part].
size_t select_chain_ws_bytes(int batch, int n_cols, int pool_k) {
  const size_t sep = kStatusBlock + two_step_bytes(batch, n_cols) + align_up((size_t)batch * pool_k * 4, 256) +
                     align_up((size_t)batch * 4, 256) + index_topk_ws_bytes(batch, pool_k);
  if (fsel_len_ok(n_cols)) return max(fsel_ws_bytes(batch, n_cols, true), sep);
  return sep;
}

hipError_t launch_select_chain(const uint16_t* q_full, const uint8_t* codes, const float* scale,
                               const int64_t* seq_base, const int32_t* n_valid, int batch,
                               int n_cols, int pool_k, int32_t* pool_out, float* pool_score_out,
                               int k, int32_t* own_out, const uint16_t* q_re, int n_re,
                               int32_t* re_out, float* re_score_out, void* ws,
                               hipStream_t stream) {
  if (fsel_fits(n_cols, pool_k))
    return launch_fsel(q_full, codes, scale, seq_base, n_valid, nullptr, batch, n_cols, pool_k,
                       pool_out, pool_score_out, k, own_out, q_re, n_re, k, re_out, re_score_out,
                       true, ws, stream);
  // rows too long for the filtered selection: the same selections one call at a time
  char* p = static_cast<char*>(ws) + kStatusBlock;
  char* after = p + two_step_bytes(batch, n_cols);
  float* pool_scores = pool_score_out ? pool_score_out : reinterpret_cast<float*>(after);
  char* after2 = after + align_up((size_t)batch * pool_k * 4, 256);
  int32_t* pool_n = reinterpret_cast<int32_t*>(after2);
  void* re_ws = after2 + align_up((size_t)batch * 4, 256);
  hipError_t e = two_step(q_full, codes, scale, seq_base, n_valid, nullptr, batch, n_cols, pool_k,
                          pool_out, pool_scores, p, stream);
  if (e != hipSuccess) return e;
  if (own_out == nullptr && n_re == 0) return hipSuccess;
  hipLaunchKernelGGL(k_count_valid, dim3(batch), dim3(256), 0, stream, pool_out, pool_k, pool_n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (own_out) {
    e = launch_topk(pool_scores, batch, pool_k, pool_n, pool_out, k, own_out, nullptr, false,
                    TopkWs{}, stream);
    if (e != hipSuccess) return e;
  }
  for (int r = 0; r < n_re; ++r) {
    e = launch_index_topk(q_re + (size_t)r * batch * kDIdx, codes, scale, seq_base, pool_n,
                          pool_out, batch, pool_k, k, re_out + (size_t)r * batch * k,
                          re_score_out ? re_score_out + (size_t)r * batch * k : nullptr, re_ws,
                          stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// csa2_replay_select: [selection part][score matrix f32][visible counts i32 T].  The
// selection part is the filtered selection's workspace (rows it takes; the matrix blocked)
// or, for longer rows, [status][top-k workspace][pool scores f32 T x pool_k][pool sizes i32
// T] (the matrix row-major, as csa2_topk reads it).
// A sequence with no entries runs the longer-row path on one column that no row sees.
static size_t replay_sel_bytes(int T, int n_entries, int pool_k) {
  if (fsel_fits(n_entries, pool_k)) return fsel_ws_bytes(T, n_entries, false);
  const int n_cols = max(n_entries, 1);
  return kStatusBlock + topk_ws_bytes(T, n_cols) + align_up((size_t)T * pool_k * 4, 256) +
         align_up((size_t)T * 4, 256);
}

// the matrix, blocked (whole blocks of 1,024 columns) or row-major
static size_t replay_scores_bytes(int T, int n_entries) {
  return align_up((size_t)T * align_up((size_t)max(n_entries, 1), 1024) * 4, 256);
}

size_t replay_select_ws_bytes(int T, int n_entries, int pool_k) {
  return replay_sel_bytes(T, n_entries, pool_k) + replay_scores_bytes(T, n_entries) +
         align_up((size_t)T * 4, 256);
}

hipError_t launch_replay_select(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                                int n_entries, int ratio, int64_t pos0, int T, int pool_k,
                                int32_t* pool_out, int32_t* pool_n_out, int k, int32_t* own_out,
                                void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + replay_sel_bytes(T, n_entries, pool_k));
  int32_t* vis = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(scores) + replay_scores_bytes(T, n_entries));
  const bool fits = n_entries > 0 && fsel_fits(n_entries, pool_k);
  if (fits) {
    hipError_t e = launch_causal_scores(q_idx, codes, scale, n_entries, ratio, pos0, T, true, scores, vis,
                                        pool_k, pool_n_out, stream);
    if (e != hipSuccess) return e;
    return launch_fsel(nullptr, nullptr, nullptr, nullptr, vis, nullptr, T, n_entries, pool_k, pool_out,
                       nullptr, k, own_out, nullptr, 0, 0, nullptr, nullptr, false, ws, stream, scores);
  }
  // longer rows (or no entries): a row-major matrix and csa2_topk's kernels
  const int n_cols = n_entries > 0 ? n_entries : 1;  // a row of nothing visible
  char* p = base + kStatusBlock;
  const TopkWs tw = topk_ws_carve(p, T, n_cols);
  float* pool_scores = reinterpret_cast<float*>(p + topk_ws_bytes(T, n_cols));
  int32_t* pool_n = pool_n_out ? pool_n_out
                               : reinterpret_cast<int32_t*>(reinterpret_cast<char*>(pool_scores) +
                                                            align_up((size_t)T * pool_k * 4, 256));
  hipError_t e = launch_causal_scores(q_idx, codes, scale, n_entries, ratio, pos0, T, false, scores, vis,
                                      pool_k, pool_n, stream);
  if (e == hipSuccess)
    e = launch_topk(scores, T, n_cols, vis, nullptr, pool_k, pool_out, pool_scores, false, tw, stream);
  if (e == hipSuccess && own_out)
    e = launch_topk(pool_scores, T, pool_k, pool_n, pool_out, k, own_out, nullptr, false, TopkWs{}, stream);
  return e;
}

}  // namespace csa2
