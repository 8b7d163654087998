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
// All 16 heads share every entry, so per query the work is a dense [16 x 512] x [512 x n]
// contraction (about 114 flop per gathered byte) and runs on the matrix cores:
//   * every dequantised value is exact in bf16 (an E2M1 magnitude has at most 2 significant
//     bits, an E4M3 scale at most 4, so the product has at most 6; window values have 4),
//     so q . v on v_mfma_f32_16x16x32_bf16 has exact products and fp32 sums;
//   * p . v takes p as the sum of two bf16 halves (hi = p truncated, lo = bf16(p - hi)),
//     two MFMAs, relative error about 2^-16, fp32 sums.
// One 256-thread workgroup (4 waves) per (row, split) walks its list positions (the k
// selected entries, then the window rows) in chunks of 32:
//   gather   thread (wave w, lane l) loads dims 8l..8l+7 of positions 8w..8w+7 (4 code bytes
//            + 1 scale byte, or 8 window bytes each), dequantises them, and writes them to
//            LDS twice: row-major (position x dims, B operand of q . v) and, after an 8x8
//            register transpose, dims x positions (B operand of p . v).  Both layouts are
//            XOR-swizzled so that the 16-byte writes and the operand reads hit distinct banks;
//   q . v    wave w: entries 16(w&1)..+15 over half of the 512 dims (8 MFMAs); the two
//            halves are added in the softmax step;
//   softmax  16 lanes per head: running max and sum, rescale factor, p split into hi/lo;
//   p . v    wave w: 128 output dims (8 tiles of 16), 2 MFMAs each.
// Decode uses several splits per row; each leaves (max, sum, acc[16][512]) in the
// workspace and k_attn_merge combines them by log-sum-exp.  The prefill chunk has many
// rows and runs one split per row, writing its output directly.  exp2 with log2(e)
// folded into the scale.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kChunk = 32;                         // list positions per chunk
constexpr int kMaxSplits = 64;                     // splits per decode row
constexpr int kIdxWin = 1024;                      // list positions whose ids sit in LDS
constexpr int kPart = 2 * kHeads + kHeads * kDKv;  // floats per split: m[16], l[16], acc

typedef float f32x4v __attribute__((ext_vector_type(4)));

int attn_chunks(int k) { return (k + kSwa + kChunk - 1) / kChunk; }
int attn_splits(int k) { return min(attn_chunks(k), kMaxSplits); }

size_t attn_ws_bytes(int rows, int k) {
  return align_up((size_t)rows * attn_splits(k) * kPart * sizeof(float), 256);
}

// ---- LDS layouts (16-byte blocks)
// V row-major: 32 position rows x 64 blocks (8 dims each); block c of row p at c ^ (p & 15).
__device__ __forceinline__ int v_blk(int p, int c) { return p * 64 + (c ^ (p & 15)); }
// V transposed: 512 dim rows x 4 blocks (8 positions each).  Dim d lives in row
// R = (d & ~15) | ((d + (d >> 4)) & 15), block kb at kb ^ ((R >> 2) & 3).
__device__ __forceinline__ int vt_blk(int d, int kb) {
  const int R = (d & ~15) | ((d + (d >> 4)) & 15);
  return R * 4 + (kb ^ ((R >> 2) & 3));
}
// P (either half): 16 head rows x 4 blocks (8 positions each); block kb of head h at
// kb ^ ((h >> 2) & 3).
__device__ __forceinline__ int p_blk(int h, int kb) { return h * 4 + (kb ^ ((h >> 2) & 3)); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// 8 E2M1 codes (one dword) times one scale -> 8 bf16 (exact), element i from nibble i.
__device__ __forceinline__ uint4 fp4x8_scaled_bf16(uint32_t w, float s) {
  const f32x2 a = fp4x2<0>(w), b = fp4x2<1>(w), c = fp4x2<2>(w), d = fp4x2<3>(w);
  return make_uint4(pack_bf16(a.x * s, a.y * s), pack_bf16(b.x * s, b.y * s),
                    pack_bf16(c.x * s, c.y * s), pack_bf16(d.x * s, d.y * s));
}

// 8 E4M3 bytes -> 8 bf16 (exact).
__device__ __forceinline__ uint4 fp8x8_bf16(uint2 w) {
  const f32x2 a = fp8x2<false>(w.x), b = fp8x2<true>(w.x);
  const f32x2 c = fp8x2<false>(w.y), d = fp8x2<true>(w.y);
  return make_uint4(pack_bf16(a.x, a.y), pack_bf16(b.x, b.y), pack_bf16(c.x, c.y),
                    pack_bf16(d.x, d.y));
}

// Raw bytes of the thread's 8 positions: main bit pp set = main entry (x: 4 code bytes,
// y: the aligned scale dword holding the lane's scale byte); window bit = window row (x, y:
// 8 E4M3 bytes); neither = nothing (x, y read from a window row and ignored).
struct GatherRaw {
  uint2 r[8];
  uint32_t main_bits, win_bits;
};

// Issues the loads of positions p0 + 8w .. p0 + 8w + 7, dims 8l .. 8l + 7: exactly two dword
// loads per position whatever its kind (the source address is selected, not branched on), so
// the loads of later chunks stay in flight while an earlier chunk is used.  Entry ids come
// from the LDS window s_idx, which holds list positions idx_base onward.
__device__ __forceinline__ GatherRaw gather_issue(int p0, int w, int l, int k, int n_pos,
                                                  const int32_t* s_idx, int idx_base, int64_t base,
                                                  const uint8_t* kv_codes, const uint8_t* kv_scale,
                                                  const uint8_t* rows) {
  GatherRaw g;
  g.main_bits = 0u;
  g.win_bits = 0u;
  const uint8_t* pa[8];
  const uint8_t* pb[8];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    const int pos = p0 + 8 * w + pp;
    const int j = pos < k ? s_idx[pos - idx_base] : -1;
    const bool is_main = pos < k && j >= 0;
    const bool is_win = pos >= k && pos < n_pos;
    const int64_t e = base + (j > 0 ? j : 0);
    const uint8_t* wrow = rows + (size_t)(is_win ? pos - k : 0) * kDKv + 8 * l;
    pa[pp] = is_main ? kv_codes + e * kKvCodeBytes + 4 * l : wrow;
    pb[pp] = is_main ? kv_scale + e * kKvScaleBytes + ((l >> 1) & ~3) : wrow + 4;
    g.main_bits |= is_main ? 1u << pp : 0u;
    g.win_bits |= is_win ? 1u << pp : 0u;
  }
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    g.r[pp].x = *reinterpret_cast<const uint32_t*>(pa[pp]);
    g.r[pp].y = *reinterpret_cast<const uint32_t*>(pb[pp]);
  }
  return g;
}

// Dequantises the thread's 8 x 8 block and writes it to both LDS layouts.
__device__ __forceinline__ void gather_commit(const GatherRaw& g, int w, int l, uint4* s_v,
                                              uint4* s_vt) {
  uint4 v[8];
  const int sh = 8 * ((l >> 1) & 3);  // the lane's scale byte within its dword
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    if (g.main_bits & (1u << pp)) {
      v[pp] = fp4x8_scaled_bf16(g.r[pp].x, e4m3_to_f32((g.r[pp].y >> sh) & 0xffu));
    } else if (g.win_bits & (1u << pp)) {
      v[pp] = fp8x8_bf16(g.r[pp]);
    } else {
      v[pp] = make_uint4(0u, 0u, 0u, 0u);
    }
    s_v[v_blk(8 * w + pp, l)] = v[pp];
  }
  // 8x8 transpose of 16-bit elements: dims 8l+2i (low halves) and 8l+2i+1 (high halves),
  // each as positions 8w..8w+7
  const uint32_t lo_sel = 0x05040100u, hi_sel = 0x07060302u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wd[8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp)
      wd[pp] = i == 0 ? v[pp].x : i == 1 ? v[pp].y : i == 2 ? v[pp].z : v[pp].w;
    uint4 te, to;
    te.x = __builtin_amdgcn_perm(wd[1], wd[0], lo_sel);
    te.y = __builtin_amdgcn_perm(wd[3], wd[2], lo_sel);
    te.z = __builtin_amdgcn_perm(wd[5], wd[4], lo_sel);
    te.w = __builtin_amdgcn_perm(wd[7], wd[6], lo_sel);
    to.x = __builtin_amdgcn_perm(wd[1], wd[0], hi_sel);
    to.y = __builtin_amdgcn_perm(wd[3], wd[2], hi_sel);
    to.z = __builtin_amdgcn_perm(wd[5], wd[4], hi_sel);
    to.w = __builtin_amdgcn_perm(wd[7], wd[6], hi_sel);
    s_vt[vt_blk(8 * l + 2 * i, w)] = te;
    s_vt[vt_blk(8 * l + 2 * i + 1, w)] = to;
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

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
  __shared__ uint4 s_v[kChunk * 64];          // 32 KiB
  __shared__ uint4 s_vt[kDKv * 4];            // 32 KiB
  __shared__ uint4 s_p[2][kHeads * 4];        // 2 KiB: p hi, p lo
  __shared__ float s_s[2][kHeads][kChunk + 1];
  __shared__ float s_m[kHeads], s_l[kHeads], s_alpha[kHeads];
  __shared__ uint32_t s_valid[4];
  __shared__ int32_t s_idx[kIdxWin];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n16 = l & 15, g16 = l >> 4;

  // ---- q as A operands: head n16, dims 32*ks + 8*g16 .. +7 for this wave's 8 k-steps
  const int et = w & 1, kh = w >> 1;
  bf16x8 qa[8];
  {
    const uint16_t* qrow = q + ((size_t)b * kHeads + n16) * kDKv + 8 * g16;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qa[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + (8 * kh + kk) * 32));
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

  const int c_begin = split * chunks_per_split;
  const int c_end = min(c_begin + chunks_per_split, (n_pos + kChunk - 1) / kChunk);

  if (tid < kHeads) {
    s_m[tid] = -__builtin_inff();
    s_l[tid] = 0.f;
  }
  f32x4v acc[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) acc[tt] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const int s_h = tid >> 4, s_jj = tid & 15;  // softmax roles: head, position pair

  // Outer loop: windows of kIdxWin list positions whose entry ids are staged in LDS.
  // Inner loop: the window's chunks, each issuing exactly the same loads (the prefetch past
  // the window's last chunk re-reads that chunk), so the next two chunks stay in flight.
  for (int wc0 = c_begin; wc0 < c_end; wc0 += kIdxWin / kChunk) {
    const int wc1 = min(wc0 + kIdxWin / kChunk, c_end);
    const int idx_base = wc0 * kChunk;
    __syncthreads();  // the previous window's ids are no longer read
    for (int i = tid; i < kIdxWin; i += kAttnThreads)
      s_idx[i] = idx_base + i < k ? irow[idx_base + i] : -1;
    __syncthreads();
    GatherRaw raw_a = gather_issue(wc0 * kChunk, w, l, k, n_pos, s_idx, idx_base, base, kv_codes,
                                   kv_scale, rows);
    GatherRaw raw_b = gather_issue(min(wc0 + 1, wc1 - 1) * kChunk, w, l, k, n_pos, s_idx, idx_base,
                                   base, kv_codes, kv_scale, rows);
  for (int c = wc0; c < wc1; ++c) {
    gather_commit(raw_a, w, l, s_v, s_vt);
    if (l == 0) s_valid[w] = raw_a.main_bits | raw_a.win_bits;
    raw_a = raw_b;
    __syncthreads();
    raw_b = gather_issue(min(c + 2, wc1 - 1) * kChunk, w, l, k, n_pos, s_idx, idx_base, base,
                         kv_codes, kv_scale, rows);

    // ---- z partials: entries 16*et + n16, dims of k-steps 8*kh .. 8*kh + 7
    {
      f32x4v sacc = {0.f, 0.f, 0.f, 0.f};
      const int e = 16 * et + n16;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ks = 8 * kh + kk;
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], as_bf16x8(s_v[v_blk(e, 4 * ks + g16)]),
                                                        sacc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) s_s[kh][4 * g16 + j][e] = sacc[j];
    }
    __syncthreads();

    // ---- online softmax update, 16 lanes per head, 2 positions per lane
    {
      const int pa = 2 * s_jj, pb = pa + 1;
      const uint32_t vm = s_valid[pa >> 3];
      const bool va = (vm >> (pa & 7)) & 1u, vb = (vm >> (pb & 7)) & 1u;
      const float z0 = va ? (s_s[0][s_h][pa] + s_s[1][s_h][pa]) * qscale : -__builtin_inff();
      const float z1 = vb ? (s_s[0][s_h][pb] + s_s[1][s_h][pb]) * qscale : -__builtin_inff();
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
      // p = hi + lo: hi = p truncated to bf16, lo = bf16(p - hi)
      const uint32_t h0 = __float_as_uint(p0v) & 0xffff0000u, h1 = __float_as_uint(p1v) & 0xffff0000u;
      const float r0 = p0v - __uint_as_float(h0), r1 = p1v - __uint_as_float(h1);
      const uint32_t l0 = __builtin_bit_cast(uint16_t, (__bf16)r0);
      const uint32_t l1 = __builtin_bit_cast(uint16_t, (__bf16)r1);
      uint32_t* ph = reinterpret_cast<uint32_t*>(&s_p[0][p_blk(s_h, pa >> 3)]);
      uint32_t* pl = reinterpret_cast<uint32_t*>(&s_p[1][p_blk(s_h, pa >> 3)]);
      ph[(pa & 7) >> 1] = (h0 >> 16) | h1;
      pl[(pa & 7) >> 1] = l0 | (l1 << 16);
      __syncthreads();  // every lane has read s_m before it changes
      if (s_jj == 0) {
        const float alpha = m_old == -__builtin_inff() ? 0.f : exp2f(m_old - m_new);
        s_alpha[s_h] = alpha;
        s_l[s_h] = s_l[s_h] * alpha + ps;
        s_m[s_h] = m_new;
      }
    }
    __syncthreads();

    // ---- acc = acc * alpha + p . v for output dims (8w + tt)*16 + n16, heads 4*g16 + j
    {
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = s_alpha[4 * g16 + j];
      const bf16x8 a_hi = as_bf16x8(s_p[0][p_blk(n16, g16)]);
      const bf16x8 a_lo = as_bf16x8(s_p[1][p_blk(n16, g16)]);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][j] *= al[j];
        const bf16x8 bv = as_bf16x8(s_vt[vt_blk((8 * w + tt) * 16 + n16, g16)]);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bv, acc[tt], 0, 0, 0);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bv, acc[tt], 0, 0, 0);
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }
  }
  __syncthreads();  // s_m / s_l final (also when this split had no positions)

  if (MODE == 1 || n_splits == 1) {
    float* O = out + (size_t)b * kHeads * kDKv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * g16 + j;
      const float lsum = s_l[h];
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) O[h * kDKv + (8 * w + tt) * 16 + n16] = acc[tt][j] * inv;
    }
    return;
  }
  float* P = part + ((size_t)b * n_splits + split) * kPart;
  if (tid < kHeads) {
    P[tid] = s_m[tid];
    P[kHeads + tid] = s_l[tid];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      P[2 * kHeads + (4 * g16 + j) * kDKv + (8 * w + tt) * 16 + n16] = acc[tt][j];
}

// Log-sum-exp merge of a decode row's splits for one head: 128 threads x 4 dims.  Each
// lane of the first wave takes one split's (max, sum), so the weights come from two wave
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
    const float wgt = (ms == -__builtin_inff()) ? 0.f : exp2f(ms - M);
    float L = wgt * ls;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane < n_splits) s_w[lane] = wgt;
    if (lane == 0) s_L = L;
  }
  __syncthreads();
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* A = P0 + 2 * kHeads + h * kDKv + 4 * tid;
#pragma unroll 8
  for (int s = 0; s < n_splits; ++s) {
    const float wgt = s_w[s];
    const float4 a = *reinterpret_cast<const float4*>(A + (size_t)s * kPart);
    o.x = fmaf(a.x, wgt, o.x);
    o.y = fmaf(a.y, wgt, o.y);
    o.z = fmaf(a.z, wgt, o.z);
    o.w = fmaf(a.w, wgt, o.w);
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
