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
// Every dequantised value is exact in bf16 (an E2M1 magnitude has at most 2 significant
// bits, an E4M3 scale at most 4, so the product has at most 6; window values have 4), so
// entries are staged in LDS as bf16 without rounding and q . v runs on v_dot2_f32_bf16
// (exact products, fp32 sums).  p . v accumulates in fp32.
//
// One 256-thread workgroup per (row, split).  A split walks its list positions (the k
// selected entries, then the window rows) in chunks of 32:
//   gather   thread (entry e, eighth) loads 32 code bytes + 4 scale bytes (or 64 window
//            bytes), dequantises 64 values and writes them to LDS;
//   q . v    thread (4 heads, 4 entries, dim slice) accumulates a 4x4 tile over 64 dims,
//            then the 8 slices are summed with 3 lane swaps;
//   softmax  16 lanes per head: running max / sum per head, rescale factor;
//   p . v    thread owns 2 dims of all 16 heads (32 fp32 accumulators).
// Decode uses several splits per row; each leaves (max, sum, acc[16][512]) in the
// workspace and k_attn_merge combines them by log-sum-exp.  The prefill chunk has many
// rows and runs one split per row, writing its output directly.  exp2 with log2(e)
// folded into the scale.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kChunk = 32;                      // list positions per chunk
constexpr int kRowWords = kDKv / 2 + 4;         // LDS row of 512 bf16 + 16 B pad, in u32
constexpr int kMaxSplits = 64;                  // splits per decode row
constexpr int kPart = 2 * kHeads + kHeads * kDKv;  // floats per split: m[16], l[16], acc

int attn_chunks(int k) { return (k + kSwa + kChunk - 1) / kChunk; }
int attn_splits(int k) { return min(attn_chunks(k), kMaxSplits); }

size_t attn_ws_bytes(int rows, int k) {
  return align_up((size_t)rows * attn_splits(k) * kPart * sizeof(float), 256);
}

// 8 E2M1 codes (one dword) times one scale -> 4 u32 of packed bf16 (exact).
__device__ __forceinline__ uint4 fp4x8_scaled_bf16(uint32_t w, float s) {
  const f32x2 a = fp4x2<0>(w), b = fp4x2<1>(w), c = fp4x2<2>(w), d = fp4x2<3>(w);
  auto pk = [](float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  };
  return make_uint4(pk(a.x * s, a.y * s), pk(b.x * s, b.y * s), pk(c.x * s, c.y * s),
                    pk(d.x * s, d.y * s));
}

// 4 E4M3 bytes -> 2 u32 of packed bf16 (exact).
__device__ __forceinline__ uint2 fp8x4_bf16(uint32_t w) {
  const f32x2 a = fp8x2<false>(w), b = fp8x2<true>(w);
  return make_uint2((__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xffff0000u),
                    (__float_as_uint(b.x) >> 16) | (__float_as_uint(b.y) & 0xffff0000u));
}

__device__ __forceinline__ float dot8(const uint4 a, const uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
  return acc;
}

// Raw bytes of one list position for one gather thread: 32 code bytes + 4 scale bytes of a
// main entry (kind 1) or 64 bytes of a window row (kind 2); kind 0 contributes nothing.
struct GatherRaw {
  uint4 w[4];
  uint32_t sc;
  int kind;
};

// Issues the loads of position pos for the thread's eighth `part` (no waiting here).
__device__ __forceinline__ GatherRaw gather_issue(int pos, int part, int k, int n_pos,
                                                  const int32_t* irow, int64_t base,
                                                  const uint8_t* kv_codes, const uint8_t* kv_scale,
                                                  const uint8_t* rows) {
  GatherRaw r;
  r.kind = 0;
  r.sc = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.w[i] = make_uint4(0u, 0u, 0u, 0u);
  if (pos < n_pos) {
    if (pos < k) {
      const int j = irow[pos];
      if (j >= 0) {
        const int64_t e = base + j;
        const uint4* cp = reinterpret_cast<const uint4*>(kv_codes + e * kKvCodeBytes + 32 * part);
        r.w[0] = cp[0];
        r.w[1] = cp[1];
        r.sc = *reinterpret_cast<const uint32_t*>(kv_scale + e * kKvScaleBytes + 4 * part);
        r.kind = 1;
      }
    } else {
      const uint4* rp = reinterpret_cast<const uint4*>(rows + (size_t)(pos - k) * kDKv + 64 * part);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.w[i] = rp[i];
      r.kind = 2;
    }
  }
  return r;
}

// Dequantises the raw bytes to 64 bf16 values and writes them to the LDS row slice.
__device__ __forceinline__ void gather_commit(const GatherRaw& r, uint32_t* dst) {
  uint4 o[8];
  if (r.kind == 1) {
    const float s0 = e4m3_to_f32(r.sc & 0xffu), s1 = e4m3_to_f32((r.sc >> 8) & 0xffu);
    const float s2 = e4m3_to_f32((r.sc >> 16) & 0xffu), s3 = e4m3_to_f32(r.sc >> 24);
    o[0] = fp4x8_scaled_bf16(r.w[0].x, s0);
    o[1] = fp4x8_scaled_bf16(r.w[0].y, s0);
    o[2] = fp4x8_scaled_bf16(r.w[0].z, s1);
    o[3] = fp4x8_scaled_bf16(r.w[0].w, s1);
    o[4] = fp4x8_scaled_bf16(r.w[1].x, s2);
    o[5] = fp4x8_scaled_bf16(r.w[1].y, s2);
    o[6] = fp4x8_scaled_bf16(r.w[1].z, s3);
    o[7] = fp4x8_scaled_bf16(r.w[1].w, s3);
  } else if (r.kind == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 a = fp8x4_bf16(r.w[i].x), bb = fp8x4_bf16(r.w[i].y);
      const uint2 cc = fp8x4_bf16(r.w[i].z), d = fp8x4_bf16(r.w[i].w);
      o[2 * i] = make_uint4(a.x, a.y, bb.x, bb.y);
      o[2 * i + 1] = make_uint4(cc.x, cc.y, d.x, d.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(dst + 4 * i) = o[i];
}

// MODE 0: decode row b (entries seq_base[b] + idx, window rows swa[b][0..swa_len[b])).
// MODE 1: prefill row t at position pos0 + t (entries idx from 0, window positions
//         max(0,p-127)..p, row r of `swa` holding position pos0 - 127 + r); one split.
template <int MODE>
__global__ __launch_bounds__(kAttnThreads) void k_attn_part(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_codes,
    const uint8_t* __restrict__ kv_scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa,
    const int32_t* __restrict__ swa_len, int64_t pos0, float qscale, float* __restrict__ out,
    float* __restrict__ part, int chunks_per_split, int n_splits) {
  __shared__ __align__(16) uint32_t s_q[kHeads * kRowWords];
  __shared__ __align__(16) uint32_t s_v[kChunk * kRowWords];
  __shared__ float s_z[kHeads][kChunk + 1];
  __shared__ __align__(16) float s_p[kChunk][kHeads];
  __shared__ float s_m[kHeads], s_l[kHeads], s_alpha[kHeads];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;

  // ---- issue the q row (16 x 512 bf16) and the first chunk's loads together
  uint4 qr[4];
  {
    const uint4* qg = reinterpret_cast<const uint4*>(q + (size_t)b * kHeads * kDKv);
#pragma unroll
    for (int i = 0; i < 4; ++i) qr[i] = qg[tid + i * kAttnThreads];  // 1024 uint4 = 16 rows x 64
  }
  const int64_t base = MODE == 0 ? seq_base[b] : 0;
  const uint8_t* rows;
  int nrows;
  if (MODE == 0) {
    rows = swa + (size_t)b * kSwa * kDKv;
    nrows = min(max(swa_len[b], 0), kSwa);
  } else {
    const int64_t p = pos0 + b;
    const int64_t lo = p - (kSwa - 1) > 0 ? p - (kSwa - 1) : 0;
    rows = swa + (size_t)(lo - (pos0 - (kSwa - 1))) * kDKv;
    nrows = (int)(p - lo + 1);
  }
  const int n_pos = k + nrows;
  const int32_t* irow = k > 0 ? idx + (size_t)b * k : nullptr;

  // thread roles
  const int g_e = tid >> 3, g_part = tid & 7;                 // gather: entry, eighth
  const int t_ds = tid & 7, t_jb = (tid >> 3) & 7, t_hb = tid >> 6;  // q . v tile
  const int s_h = tid >> 4, s_jj = tid & 15;                  // softmax: head, entry pair
  uint32_t* g_dst = &s_v[g_e * kRowWords + 32 * g_part];

  const int c_begin = split * chunks_per_split;
  const int c_end = min(c_begin + chunks_per_split, (n_pos + kChunk - 1) / kChunk);
  GatherRaw raw = gather_issue(c_begin * kChunk + g_e, g_part, k, n_pos, irow, base, kv_codes,
                               kv_scale, rows);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + i * kAttnThreads;
    *reinterpret_cast<uint4*>(&s_q[(v >> 6) * kRowWords + 4 * (v & 63)]) = qr[i];
  }
  if (tid < kHeads) {
    s_m[tid] = -__builtin_inff();
    s_l[tid] = 0.f;
  }
  float acc[kHeads][2];
#pragma unroll
  for (int h = 0; h < kHeads; ++h) acc[h][0] = acc[h][1] = 0.f;

  for (int c = c_begin; c < c_end; ++c) {
    const int p0 = c * kChunk;
    gather_commit(raw, g_dst);
    __syncthreads();
    if (c + 1 < c_end)  // next chunk's loads fly while this one is computed
      raw = gather_issue(p0 + kChunk + g_e, g_part, k, n_pos, irow, base, kv_codes, kv_scale, rows);

    // ---- z = q . v for 16 heads x 32 entries
    {
      float t[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) t[a][e] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w0 = 4 * t_ds + 32 * i;  // u32 offset of dims 8*t_ds + 64*i
        uint4 qv[4], vv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qv[a] = *reinterpret_cast<const uint4*>(&s_q[(4 * t_hb + a) * kRowWords + w0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = *reinterpret_cast<const uint4*>(&s_v[(4 * t_jb + e) * kRowWords + w0]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) t[a][e] = dot8(qv[a], vv[e], t[a][e]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = t[a][e];
          v += __shfl_xor(v, 1);
          v += __shfl_xor(v, 2);
          v += __shfl_xor(v, 4);
          t[a][e] = v;
        }
      if (t_ds == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * t_jb + e;
          const int pos = p0 + j;
          bool valid = pos < n_pos;
          if (valid && pos < k) valid = irow[pos] >= 0;
#pragma unroll
          for (int a = 0; a < 4; ++a) s_z[4 * t_hb + a][j] = valid ? t[a][e] * qscale : -__builtin_inff();
        }
      }
    }
    __syncthreads();

    // ---- online softmax update, 16 lanes per head
    {
      const float z0 = s_z[s_h][2 * s_jj], z1 = s_z[s_h][2 * s_jj + 1];
      float cm = fmaxf(z0, z1);
      cm = fmaxf(cm, __shfl_xor(cm, 1));
      cm = fmaxf(cm, __shfl_xor(cm, 2));
      cm = fmaxf(cm, __shfl_xor(cm, 4));
      cm = fmaxf(cm, __shfl_xor(cm, 8));
      const float m_old = s_m[s_h];
      const float m_new = fmaxf(m_old, cm);
      float p0v = 0.f, p1v = 0.f;
      if (m_new != -__builtin_inff()) {
        p0v = exp2f(z0 - m_new);
        p1v = exp2f(z1 - m_new);
      }
      float ps = p0v + p1v;
      ps += __shfl_xor(ps, 1);
      ps += __shfl_xor(ps, 2);
      ps += __shfl_xor(ps, 4);
      ps += __shfl_xor(ps, 8);
      s_p[2 * s_jj][s_h] = p0v;
      s_p[2 * s_jj + 1][s_h] = p1v;
      __syncthreads();  // every lane has read s_m before it changes
      if (s_jj == 0) {
        const float alpha = m_old == -__builtin_inff() ? 0.f : exp2f(m_old - m_new);
        s_alpha[s_h] = alpha;
        s_l[s_h] = s_l[s_h] * alpha + ps;
        s_m[s_h] = m_new;
      }
    }
    __syncthreads();

    // ---- acc = acc * alpha + p . v, thread owns dims 2*tid, 2*tid + 1
    {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        const float al = s_alpha[h];
        acc[h][0] *= al;
        acc[h][1] *= al;
      }
#pragma unroll 4
      for (int j = 0; j < kChunk; ++j) {
        const uint32_t w = s_v[j * kRowWords + tid];
        const float v0 = __uint_as_float(w << 16), v1 = __uint_as_float(w & 0xffff0000u);
        const float4* pp = reinterpret_cast<const float4*>(&s_p[j][0]);
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) {
          const float4 p4 = pp[h4];
          const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            acc[4 * h4 + u][0] = fmaf(pv[u], v0, acc[4 * h4 + u][0]);
            acc[4 * h4 + u][1] = fmaf(pv[u], v1, acc[4 * h4 + u][1]);
          }
        }
      }
    }
    __syncthreads();  // s_v / s_p are rewritten by the next chunk
  }

  __syncthreads();  // s_m / s_l final (also when this split had no positions)
  if (MODE == 1 || n_splits == 1) {
    float* O = out + (size_t)b * kHeads * kDKv;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      const float l = s_l[h];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      *reinterpret_cast<float2*>(&O[h * kDKv + 2 * tid]) = make_float2(acc[h][0] * inv, acc[h][1] * inv);
    }
    return;
  }
  float* P = part + ((size_t)b * n_splits + split) * kPart;
  if (tid < kHeads) {
    P[tid] = s_m[tid];
    P[kHeads + tid] = s_l[tid];
  }
#pragma unroll
  for (int h = 0; h < kHeads; ++h)
    *reinterpret_cast<float2*>(&P[2 * kHeads + h * kDKv + 2 * tid]) = make_float2(acc[h][0], acc[h][1]);
}

// Log-sum-exp merge of a decode row's splits for one head: 128 threads x 4 dims.  Each
// lane of every wave first takes one split's (max, sum), so the weights come from two wave
// reductions, then all splits' accumulators are read with independent loads.
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, int n_splits,
                                                    float* __restrict__ out) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_L;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const float* P0 = part + (size_t)b * n_splits * kPart;
  if (tid < 64) {
    const float ms = lane < n_splits ? P0[(size_t)lane * kPart + h] : -__builtin_inff();
    const float ls = lane < n_splits ? P0[(size_t)lane * kPart + kHeads + h] : 0.f;
    float M = ms;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = (ms == -__builtin_inff()) ? 0.f : exp2f(ms - M);
    float L = w * ls;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane < n_splits) s_w[lane] = w;
    if (lane == 0) s_L = L;
  }
  __syncthreads();
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* A = P0 + 2 * kHeads + h * kDKv + 4 * tid;
#pragma unroll 8
  for (int s = 0; s < n_splits; ++s) {
    const float w = s_w[s];
    const float4 a = *reinterpret_cast<const float4*>(A + (size_t)s * kPart);
    o.x = fmaf(a.x, w, o.x);
    o.y = fmaf(a.y, w, o.y);
    o.z = fmaf(a.z, w, o.z);
    o.w = fmaf(a.w, w, o.w);
  }
  const float L = s_L;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<float4*>(&out[((size_t)b * kHeads + h) * kDKv + 4 * tid]) =
      make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

hipError_t launch_attn(int mode, const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       const int64_t* seq_base, const int32_t* idx, int k, const uint8_t* swa,
                       const int32_t* swa_len, int64_t pos0, float softmax_scale, int rows,
                       float* out, void* ws, hipStream_t stream) {
  const float qscale = softmax_scale * 1.4426950408889634f;  // log2(e)
  const int chunks = attn_chunks(k);
  if (mode == 1) {
    hipLaunchKernelGGL(k_attn_part<1>, dim3(1, rows), dim3(kAttnThreads), 0, stream, q, kv_codes,
                       kv_scale, seq_base, idx, k, swa, swa_len, pos0, qscale, out, nullptr, chunks, 1);
    return hipGetLastError();
  }
  const int n_splits = attn_splits(k);
  const int cps = (chunks + n_splits - 1) / n_splits;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(k_attn_part<0>, dim3(n_splits, rows), dim3(kAttnThreads), 0, stream, q, kv_codes,
                     kv_scale, seq_base, idx, k, swa, swa_len, pos0, qscale, out, part, cps, n_splits);
  if (n_splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(kHeads, rows), dim3(128), 0, stream, part, n_splits, out);
  return hipGetLastError();
}

}  // namespace csa2
