// a1 Full scan and a3 Reindex re-score of FP4 indexer keys.
//
// score_c = scale_e * sum_d q_d * e2m1(code_ed), e = seq_base[b] + (cand ? cand[c] : c)
// (entry layout from "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", Q&A on
// the 890-byte count: 128 x 4 bit + a 4-byte scale; the dot-product score is this
// library's reading, the pages do not state the indexer's formula).
//
// HBM-bound stream: 68 bytes per entry.  Each wave reads 64 consecutive entries as four
// fully coalesced 1 KiB slabs (lane = 4 * entry + quarter, 16 bytes = 32 codes per lane).
// Codes become packed bf16 pairs with one v_cvt_scalef32_pk_bf16_fp4 each and meet the
// bf16 query in v_dot2_f32_bf16 (exact products, fp32 sums): about one VALU op per value,
// well under the VALU budget of streaming at full HBM rate.  The four quarter sums are
// combined with two lane swaps; lanes are then re-assigned so one 256-byte store writes
// the 64 scores.  Optionally a 4096-bin histogram of the score keys' top 12 bits is
// accumulated (LDS, then one global add per non-empty bin) for the top-k that follows.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kScanThreads = 256;

struct ScanSlab {
  uint4 w[4];  // 16 bytes of codes for each of the four 16-entry sub-slabs
};

template <bool CAND>
__device__ __forceinline__ int64_t scan_entry(int col, int nv, const int32_t* __restrict__ cand_row,
                                              int64_t base, bool& valid) {
  valid = col < nv;
  if (CAND) {
    int cj = valid ? cand_row[col] : -1;
    valid = valid && cj >= 0;
    return base + (int64_t)(valid ? cj : 0);
  }
  return base + (int64_t)(valid ? col : 0);
}

__device__ __forceinline__ float dot32(const uint4 w, const bf16x2 (&q)[16]) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<0>(w.x), q[0], a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<1>(w.x), q[1], a1, false);
  a2 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<2>(w.x), q[2], a2, false);
  a3 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<3>(w.x), q[3], a3, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<0>(w.y), q[4], a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<1>(w.y), q[5], a1, false);
  a2 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<2>(w.y), q[6], a2, false);
  a3 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<3>(w.y), q[7], a3, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<0>(w.z), q[8], a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<1>(w.z), q[9], a1, false);
  a2 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<2>(w.z), q[10], a2, false);
  a3 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<3>(w.z), q[11], a3, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<0>(w.w), q[12], a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<1>(w.w), q[13], a1, false);
  a2 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<2>(w.w), q[14], a2, false);
  a3 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<3>(w.w), q[15], a3, false);
  return (a0 + a1) + (a2 + a3);
}

template <bool CAND, bool HIST>
__global__ __launch_bounds__(kScanThreads) void k_index_score(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ cand, int n_cols,
    int cols_per_wg, float* __restrict__ scores, uint32_t* __restrict__ hist1) {
  __shared__ uint32_t s_hist[HIST ? kHist1Bins : 1];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int quarter = lane & 3;  // which 32 of the 128 values
  const int ent = lane >> 2;     // entry within a 16-entry sub-slab

  if (HIST) {
    for (int i = threadIdx.x; i < kHist1Bins; i += kScanThreads) s_hist[i] = 0u;
  }
  bf16x2 q[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + (size_t)b * kDIdx) + quarter * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = qp[i];
      q[4 * i + 0] = __builtin_bit_cast(bf16x2, v.x);
      q[4 * i + 1] = __builtin_bit_cast(bf16x2, v.y);
      q[4 * i + 2] = __builtin_bit_cast(bf16x2, v.z);
      q[4 * i + 3] = __builtin_bit_cast(bf16x2, v.w);
    }
  }
  const int nv = min(n_valid[b], n_cols);
  const int64_t base = seq_base[b];
  const int32_t* cand_row = CAND ? cand + (size_t)b * n_cols : nullptr;
  float* out_row = scores + (size_t)b * n_cols;
  const int c0 = blockIdx.x * cols_per_wg;
  const int c1 = min(c0 + cols_per_wg, n_cols);
  if (HIST) __syncthreads();

  // Load the 4 sub-slabs of the 64-column group starting at g.
  auto load_group = [&](int g, ScanSlab& s) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      bool valid;
      int64_t e = scan_entry<CAND>(g + it * 16 + ent, nv, cand_row, base, valid);
      s.w[it] = valid ? *reinterpret_cast<const uint4*>(codes + e * kIdxCodeBytes + quarter * 16)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  int g = c0 + wave * 64;
  ScanSlab cur;
  if (g < c1) load_group(g, cur);
  for (; g < c1; g += 4 * 64) {
    ScanSlab nxt;
    const int gn = g + 4 * 64;
    if (gn < c1) load_group(gn, nxt);  // keep the next group's loads in flight

    float s[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float v = dot32(cur.w[it], q);
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      s[it] = v;
    }
    // lane (4*ent + quarter) now owns column g + 16*quarter + ent
    float mine = quarter == 0 ? s[0] : quarter == 1 ? s[1] : quarter == 2 ? s[2] : s[3];
    const int col = g + 16 * quarter + ent;
    bool valid;
    int64_t e = scan_entry<CAND>(col, nv, cand_row, base, valid);
    float score = valid ? mine * scale[e] : -__builtin_inff();
    if (col < c1) out_row[col] = score;
    if (HIST && valid) atomicAdd(&s_hist[score_key(score) >> 20], 1u);
    cur = nxt;
  }

  if (HIST) {
    __syncthreads();
    uint32_t* h = hist1 + (size_t)b * kHist1Bins;
    for (int i = threadIdx.x; i < kHist1Bins; i += kScanThreads) {
      uint32_t v = s_hist[i];
      if (v) atomic_add_agent(&h[i], v);
    }
  }
}

static int scan_cols_per_wg(int batch, int n_cols) {
  // aim for >= ~1024 workgroups on 256 CUs, 256..4096 columns each, a multiple of 256
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
