// a1 Full scan and a3 Reindex re-score of FP4 indexer keys (the stream itself is
// scan_columns in scan_device.h).
//
// Scores are staged in LDS and written in one coalesced burst per workgroup at the end:
// stores inside the loop would sit in the same in-order counter as the prefetched loads
// and hold them up.  Optionally a 4096-bin histogram of the score keys' top 12 bits is
// accumulated (LDS, then one global add per non-empty bin) for the top-k that follows.
#include "csa2_internal.h"
#include "scan_device.h"

namespace csa2 {

constexpr int kScanMaxCols = 4096;  // columns per workgroup at most (scores staged in LDS)

template <bool CAND, bool HIST>
__global__ __launch_bounds__(kScanThreads) void k_index_score(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ cand, int n_cols,
    int cols_per_wg, float* __restrict__ scores, uint32_t* __restrict__ hist1) {
  __shared__ uint32_t s_hist[HIST ? kHist1Bins : 1];
  __shared__ __align__(16) float s_sc[kScanMaxCols];
  const int b = blockIdx.y;
  const int nv = min(n_valid[b], n_cols);
  const int64_t base = seq_base[b];
  const int32_t* cand_row = CAND ? cand + (size_t)b * n_cols : nullptr;
  float* out_row = scores + (size_t)b * n_cols;
  const int c0 = blockIdx.x * cols_per_wg;
  const int c1 = min(c0 + cols_per_wg, n_cols);

  if (nv <= 0) {  // nothing visible: every column of the range is -inf, no histogram
    for (int c = c0 + threadIdx.x; c < c1; c += kScanThreads) out_row[c] = -__builtin_inff();
    return;
  }
  scan_columns<CAND>(
      q_idx + (size_t)b * kDIdx, codes, scale, cand_row, base, nv, c0, c1,
      [&]() {
        if (HIST)
          for (int i = threadIdx.x; i < kHist1Bins; i += kScanThreads) s_hist[i] = 0u;
      },
      [&](int col, float score, bool valid) {
        s_sc[col - c0] = score;
        if (HIST && valid) {
          const uint32_t key = score_key(score);
          if (key != 0u) atomicAdd(&s_hist[key >> 20], 1u);
        }
      });

  // The scores leave in one coalesced burst: stores inside the loop would sit in the same
  // in-order counter as the prefetched loads and hold them up.
  __syncthreads();
  const int n = c1 - c0;
  for (int i = 4 * threadIdx.x; i < n; i += 4 * kScanThreads) {
    if (i + 3 < n && (reinterpret_cast<uintptr_t>(&out_row[c0 + i]) & 15) == 0) {
      *reinterpret_cast<float4*>(&out_row[c0 + i]) = *reinterpret_cast<const float4*>(&s_sc[i]);
    } else {
      for (int u = 0; u < 4 && i + u < n; ++u) out_row[c0 + i + u] = s_sc[i + u];
    }
  }
  if (HIST) {
    uint32_t* h = hist1 + (size_t)b * kHist1Bins;
    for (int i = threadIdx.x; i < kHist1Bins; i += kScanThreads) {
      uint32_t v = s_hist[i];
      if (v) atomic_add_agent(&h[i], v);
    }
  }
}

static int scan_cols_per_wg(int batch, int n_cols) {
  // aim for ~1024 workgroups on 256 CUs, 256..4096 columns each, a multiple of 256
  long long want = ((long long)n_cols * batch + 1023) / 1024;
  int c = (int)((want + 255) / 256 * 256);
  if (c < 256) c = 256;
  if (c > 4096) c = 4096;
  return c;
}

hipError_t launch_index_score(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                              const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                              int batch, int n_cols, float* scores, uint32_t* hist1,
                              hipStream_t stream) {
  const int cpw = scan_cols_per_wg(batch, n_cols);
  dim3 grid((n_cols + cpw - 1) / cpw, batch);
  dim3 block(kScanThreads);
  if (cand) {
    if (hist1)
      hipLaunchKernelGGL((k_index_score<true, true>), grid, block, 0, stream, q_idx, codes, scale,
                         seq_base, n_valid, cand, n_cols, cpw, scores, hist1);
    else
      hipLaunchKernelGGL((k_index_score<true, false>), grid, block, 0, stream, q_idx, codes, scale,
                         seq_base, n_valid, cand, n_cols, cpw, scores, hist1);
  } else {
    if (hist1)
      hipLaunchKernelGGL((k_index_score<false, true>), grid, block, 0, stream, q_idx, codes, scale,
                         seq_base, n_valid, cand, n_cols, cpw, scores, hist1);
    else
      hipLaunchKernelGGL((k_index_score<false, false>), grid, block, 0, stream, q_idx, codes, scale,
                         seq_base, n_valid, cand, n_cols, cpw, scores, hist1);
  }
  return hipGetLastError();
}

}  // namespace csa2
