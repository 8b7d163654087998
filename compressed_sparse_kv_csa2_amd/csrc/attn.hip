// a5 gather-dequant + a6 sparse attention over the selected main entries merged with the
// layer's own sliding window in ONE softmax (also the attention of the prefill chunk).
//
// out_h = sum_j p_hj v_j / sum_j p_hj,  p_hj = exp(z_hj - max), z_hj = (q_h . v_j) * scale,
// where each selected main entry and each window row v_j is both key and value
// ("从V4到V4.1 Flash：架构的激进进化", section on global KV sharing with per-layer
// sliding windows: the shared global entries and the layer's own window both feed the
// layer's attention; K = V and the single softmax are this library's reading).
// Main entry value e = e2m1(code_e) * e4m3(scale_{e/16}); window rows are raw E4M3
// ("DeepSeek V4.1 Flash 深度解析", part-4 entry on FP4 in the KV cache).
//
// Layout: one 64-lane wave per (row, head, split); lane l owns dims 8l..8l+7, so an entry
// is one coalesced 256-byte read of codes (+ its scale bytes) per wave.  A split walks
// its list positions (the k selected entries, then the window rows) in chunks of 32 and
// requests a whole chunk before using any of it, so a chunk costs one memory round trip.
// Decode uses many splits per row (each leaves max, sum, acc[512] in the workspace and
// the wave finishing a (row, head) last merges them by log-sum-exp, then returns its
// counter to zero); the prefill chunk has enough rows to use one split and writes its
// output directly.  fp32 throughout; exp2 with log2(e) folded into q.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kPart = 516;  // floats per partial: m, l, 2 pad, acc[512]

int attn_splits(int k) { return (k + kAttnSplit - 1) / kAttnSplit + kSwa / kAttnSplit; }

size_t attn_ws_bytes(int rows, int k) {
  const size_t parts = (size_t)rows * kHeads * attn_splits(k) * kPart * sizeof(float);
  const size_t counters = (size_t)rows * kHeads * sizeof(uint32_t);
  return align_up(parts, 256) + align_up(counters, 256);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

struct SoftmaxState {
  float m, l, acc[8];
};

// Adds one key/value row to the state.  Each lane holds 8 dims, unscaled, whose true
// values are v * vs; vs is the lane's own E4M3 group scale, so it scales the lane's
// partial dot before the cross-lane sum.
__device__ __forceinline__ void attend(SoftmaxState& st, const float (&qv)[8], const float (&v)[8],
                                       float vs) {
  float z = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) z = fmaf(qv[t], v[t], z);
  z = wave_sum(z * vs);
  const float m_new = fmaxf(st.m, z);
  const float alpha = exp2f(st.m - m_new);  // 0 on the first row (m = -inf)
  const float p = exp2f(z - m_new);
  st.l = st.l * alpha + p;
  const float pv = p * vs;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = fmaf(pv, v[t], st.acc[t] * alpha);
  st.m = m_new;
}

// MODE 0: decode row b (entries seq_base[b] + idx, window rows swa[b][0..swa_len[b])).
// MODE 1: prefill row t at position pos0 + t (entries idx from 0, window positions
//         max(0,p-127)..p, row r of `swa` holding position pos0 - 127 + r).
template <int MODE>
__global__ __launch_bounds__(64) void k_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_codes,
    const uint8_t* __restrict__ kv_scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa,
    const int32_t* __restrict__ swa_len, int64_t pos0, float qscale, float* __restrict__ out,
    float* __restrict__ part, uint32_t* __restrict__ done, int split_len, int n_splits) {
  __shared__ uint32_t s_flag;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;

  float qv[8];
  {
    const uint4 r = *reinterpret_cast<const uint4*>(q + ((size_t)b * kHeads + h) * kDKv + 8 * lane);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qv[2 * t] = bf16_bits_to_f32(w[t] & 0xffffu) * qscale;
      qv[2 * t + 1] = bf16_bits_to_f32(w[t] >> 16) * qscale;
    }
  }
  const int64_t base = MODE == 0 ? seq_base[b] : 0;
  const uint8_t* rows;
  int nrows;
  if (MODE == 0) {
    rows = swa + (size_t)b * kSwa * kDKv;
    nrows = swa_len[b];
  } else {
    const int64_t p = pos0 + b;
    const int64_t lo = p - (kSwa - 1) > 0 ? p - (kSwa - 1) : 0;
    rows = swa + (size_t)(lo - (pos0 - (kSwa - 1))) * kDKv;
    nrows = (int)(p - lo + 1);
  }
  const int32_t* irow = k > 0 ? idx + (size_t)b * k : nullptr;

  SoftmaxState st;
  st.m = -__builtin_inff();
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = 0.f;

  const int p_begin = split * split_len;
  const int p_end = min(p_begin + split_len, k + nrows);
  for (int c0 = p_begin; c0 < p_end; c0 += kAttnSplit) {
    // entry id (main) of position c0 + lane, or -1
    const int my_pos = c0 + lane;
    const int my_j = (lane < kAttnSplit && my_pos < k && my_pos < p_end) ? irow[my_pos] : -1;
    uint2 raw[kAttnSplit];
#pragma unroll
    for (int i = 0; i < kAttnSplit; ++i) {
      const int pos = c0 + i;
      raw[i] = make_uint2(0u, 0u);
      if (pos >= p_end) continue;
      if (pos < k) {
        const int j = __shfl(my_j, i);
        if (j >= 0) {
          const int64_t e = base + j;
          raw[i].x = *reinterpret_cast<const uint32_t*>(kv_codes + e * kKvCodeBytes + 4 * lane);
          raw[i].y = kv_scale[e * kKvScaleBytes + (lane >> 1)];
        }
      } else {
        raw[i] = *reinterpret_cast<const uint2*>(rows + (size_t)(pos - k) * kDKv + 8 * lane);
      }
    }
#pragma unroll
    for (int i = 0; i < kAttnSplit; ++i) {
      const int pos = c0 + i;
      if (pos >= p_end) break;
      if (pos < k) {
        if (__shfl(my_j, i) < 0) continue;
        const uint32_t w = raw[i].x;
        const f32x2 v0 = fp4x2<0>(w), v1 = fp4x2<1>(w), v2 = fp4x2<2>(w), v3 = fp4x2<3>(w);
        const float v[8] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
        attend(st, qv, v, e4m3_to_f32(raw[i].y));
      } else {
        const f32x2 a = fp8x2<false>(raw[i].x), c = fp8x2<true>(raw[i].x);
        const f32x2 d = fp8x2<false>(raw[i].y), e = fp8x2<true>(raw[i].y);
        const float v[8] = {a.x, a.y, c.x, c.y, d.x, d.y, e.x, e.y};
        attend(st, qv, v, 1.0f);
      }
    }
  }

  float4* O = reinterpret_cast<float4*>(out + ((size_t)b * kHeads + h) * kDKv + 8 * lane);
  if (n_splits == 1) {
    const float inv = st.l > 0.f ? 1.0f / st.l : 0.f;
    O[0] = make_float4(st.acc[0] * inv, st.acc[1] * inv, st.acc[2] * inv, st.acc[3] * inv);
    O[1] = make_float4(st.acc[4] * inv, st.acc[5] * inv, st.acc[6] * inv, st.acc[7] * inv);
    return;
  }

  float* P = part + (((size_t)b * kHeads + h) * n_splits + split) * kPart;
  if (lane == 0) {
    P[0] = st.m;
    P[1] = st.l;
  }
  reinterpret_cast<float4*>(P + 4)[2 * lane] = make_float4(st.acc[0], st.acc[1], st.acc[2], st.acc[3]);
  reinterpret_cast<float4*>(P + 4)[2 * lane + 1] =
      make_float4(st.acc[4], st.acc[5], st.acc[6], st.acc[7]);

  uint32_t* cnt = done + (size_t)b * kHeads + h;
  if (!arrive_last(cnt, (uint32_t)n_splits, &s_flag)) return;

  // ---- last split of (row, head): log-sum-exp merge of the partials
  const float* P0 = part + ((size_t)b * kHeads + h) * n_splits * kPart;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, P0[(size_t)s * kPart]);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < n_splits; ++s) {
      const float* Ps = P0 + (size_t)s * kPart;
      const float ms = Ps[0];
      if (ms == -__builtin_inff()) continue;
      const float wgt = exp2f(ms - M);
      L = fmaf(Ps[1], wgt, L);
      const float4 a = reinterpret_cast<const float4*>(Ps + 4)[2 * lane];
      const float4 c = reinterpret_cast<const float4*>(Ps + 4)[2 * lane + 1];
      o[0] = fmaf(a.x, wgt, o[0]);
      o[1] = fmaf(a.y, wgt, o[1]);
      o[2] = fmaf(a.z, wgt, o[2]);
      o[3] = fmaf(a.w, wgt, o[3]);
      o[4] = fmaf(c.x, wgt, o[4]);
      o[5] = fmaf(c.y, wgt, o[5]);
      o[6] = fmaf(c.z, wgt, o[6]);
      o[7] = fmaf(c.w, wgt, o[7]);
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] *= inv;
  }
  O[0] = make_float4(o[0], o[1], o[2], o[3]);
  O[1] = make_float4(o[4], o[5], o[6], o[7]);
  if (lane == 0) *cnt = 0u;
}

hipError_t launch_attn(int mode, const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       const int64_t* seq_base, const int32_t* idx, int k, const uint8_t* swa,
                       const int32_t* swa_len, int64_t pos0, float softmax_scale, int rows,
                       float* out, void* ws, hipStream_t stream) {
  const float qscale = softmax_scale * 1.4426950408889634f;  // log2(e)
  if (mode == 1) {
    const int len = k + kSwa;
    hipLaunchKernelGGL(k_attn<1>, dim3(1, kHeads, rows), dim3(64), 0, stream, q, kv_codes, kv_scale,
                       seq_base, idx, k, swa, swa_len, pos0, qscale, out, nullptr, nullptr, len, 1);
    return hipGetLastError();
  }
  const int n_splits = attn_splits(k);
  float* part = static_cast<float*>(ws);
  uint32_t* done = reinterpret_cast<uint32_t*>(
      static_cast<char*>(ws) + align_up((size_t)rows * kHeads * n_splits * kPart * sizeof(float), 256));
  hipLaunchKernelGGL(k_attn<0>, dim3(n_splits, kHeads, rows), dim3(64), 0, stream, q, kv_codes,
                     kv_scale, seq_base, idx, k, swa, swa_len, pos0, qscale, out, part, done,
                     kAttnSplit, n_splits);
  return hipGetLastError();
}

}  // namespace csa2
