// The FP4 indexer-key stream shared by the Full / Reindex scan (index_score.hip) and the
// fused scan + top-k (index_topk.hip).
//
// score_c = scale_e * sum_d q_d * e2m1(code_ed), e = seq_base[b] + (cand ? cand[c] : c)
// (entry layout from "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", Q&A on
// the 890-byte count: 128 x 4 bit + a 4-byte scale; the dot-product score is this
// library's reading, the pages do not state the indexer's formula).
//
// HBM-bound stream: 68 bytes per entry.  Each wave reads a group of 64 consecutive
// entries as four fully coalesced 1 KiB slabs (lane = 4 * entry + quarter, 16 bytes = 32
// codes per lane) plus the 256 bytes of their scales, all five loads issued together
// from addresses that are always in bounds (columns past the end are clamped and masked
// afterwards), and the next group's five loads are in flight while a group is computed.
// Codes become packed bf16 pairs with one v_cvt_scalef32_pk_bf16_fp4 each and meet the
// bf16 query in v_dot2_f32_bf16 (exact products, fp32 sums): about one VALU op per value,
// well under the VALU budget of streaming at full HBM rate.  The four quarter sums are
// combined with two lane swaps; lane (entry, quarter) then owns column 16*quarter + entry.
#pragma once
#include "csa2_device.h"

namespace csa2 {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / 64;

struct ScanGroup {
  uint4 w[4];   // 16 code bytes of entry 16*it + ent, it = 0..3
  float sc;     // scale of the lane's own column 16*quarter + ent
  int own_ok;   // the own column's candidate id is not a hole (Reindex)
};

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

// Issues the five loads of the group starting at column g.  Columns are clamped to
// nv - 1 (>= 0), and a hole in the candidate list reads entry 0 of the sequence, so every
// address is in bounds; the caller masks those columns.
template <bool CAND>
__device__ __forceinline__ ScanGroup load_group(const uint8_t* __restrict__ codes,
                                                const float* __restrict__ scale,
                                                const int32_t* __restrict__ cand_row, int64_t base,
                                                int g, int nv_m1, int ent, int quarter) {
  ScanGroup s;
  int64_t e[4];
  if (CAND) {
    int cj[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) cj[it] = cand_row[min(g + 16 * it + ent, nv_m1)];
    int own = cj[0];
#pragma unroll
    for (int it = 1; it < 4; ++it) own = quarter == it ? cj[it] : own;
    s.own_ok = own >= 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) e[it] = base + (cj[it] >= 0 ? cj[it] : 0);
    s.sc = scale[base + (own >= 0 ? own : 0)];
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it) e[it] = base + min(g + 16 * it + ent, nv_m1);
    s.own_ok = 1;
  }
#pragma unroll
  for (int it = 0; it < 4; ++it)
    s.w[it] = *reinterpret_cast<const uint4*>(codes + e[it] * kIdxCodeBytes + quarter * 16);
  if (!CAND) s.sc = scale[base + min(g + 16 * quarter + ent, nv_m1)];
  return s;
}

// Scores columns [c0, c1) of one sequence with a workgroup of THREADS threads (nv >= 1
// visible columns, c0 < c1).  `init()` runs once, by every thread, after the first loads are in
// flight, and is followed by a barrier (LDS set-up overlaps the first loads).  Then
// `sink(col, score, valid)` is called exactly once for every column of the range, by the
// lane that owns it; invalid columns (>= nv, or a candidate hole) come with score -inf.
template <bool CAND, int THREADS = kScanThreads, typename Init, typename Sink>
__device__ __forceinline__ void scan_columns(const uint16_t* __restrict__ q_row,
                                             const uint8_t* __restrict__ codes,
                                             const float* __restrict__ scale,
                                             const int32_t* __restrict__ cand_row, int64_t base,
                                             int nv, int c0, int c1, Init init, Sink sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int quarter = lane & 3;  // which 32 of the 128 values
  const int ent = lane >> 2;     // entry within a 16-entry sub-slab
  const int nv_m1 = nv - 1;

  // The query goes first: loads complete in order, so waiting for a group never waits
  // for a load issued after it.
  bf16x2 q[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q_row) + quarter * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = qp[i];
      q[4 * i + 0] = __builtin_bit_cast(bf16x2, v.x);
      q[4 * i + 1] = __builtin_bit_cast(bf16x2, v.y);
      q[4 * i + 2] = __builtin_bit_cast(bf16x2, v.z);
      q[4 * i + 3] = __builtin_bit_cast(bf16x2, v.w);
    }
  }

  // The wave's groups are g0, g0 + 256, ... < c1.  Two buffers alternate: while one group
  // is computed the other's loads are in flight.  Prefetches past the wave's last group
  // re-read the last group (cached), so every iteration issues the same loads.
  const int g0 = c0 + wave * 64;
  const int stride = THREADS;
  const int g_last = g0 < c1 ? g0 + (c1 - 1 - g0) / stride * stride : c0;
  ScanGroup A = load_group<CAND>(codes, scale, cand_row, base, min(g0, g_last), nv_m1, ent, quarter);
  ScanGroup B = load_group<CAND>(codes, scale, cand_row, base, min(g0 + stride, g_last), nv_m1, ent,
                                 quarter);
  init();
  __syncthreads();

  auto process = [&](const ScanGroup& cur, int g) {
    float s[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float v = dot32(cur.w[it], q);
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      s[it] = v;
    }
    // lane (4*ent + quarter) now owns column g + 16*quarter + ent
    const float mine = quarter == 0 ? s[0] : quarter == 1 ? s[1] : quarter == 2 ? s[2] : s[3];
    const int col = g + 16 * quarter + ent;
    const bool valid = col < nv && cur.own_ok;
    const float score = valid ? mine * cur.sc : -__builtin_inff();
    if (col < c1) sink(col, score, valid);
  };

  for (int g = g0; g < c1; g += 2 * stride) {
    process(A, g);
    A = load_group<CAND>(codes, scale, cand_row, base, min(g + 2 * stride, g_last), nv_m1, ent,
                         quarter);
    if (g + stride < c1) process(B, g + stride);
    B = load_group<CAND>(codes, scale, cand_row, base, min(g + 3 * stride, g_last), nv_m1, ent,
                         quarter);
  }
}

}  // namespace csa2
