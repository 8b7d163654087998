// csa2_index_topk and csa2_select_chain: the scan and its selections in one launch of the
// filtered selection (fsel.hip) for rows up to its length limit; longer rows take the
// separate scan (index_score.hip, scores written out) and top-k (topk.hip) launches inside
// the same call, with the same results.
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
  if (fsel_fits(n_cols, k))
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

}  // namespace csa2
