// KV write path: quantise new global-KV entries into the 68-byte indexer and 288-byte main
// formats, and write new sliding-window rows as E4M3 ("DeepSeek-V4.1 模型结构（0）：一张图
// 看懂 DeepSeek-V4.1-Flash", Q&A on how the 890-byte figure is derived: 128 x 4 bit + a
// 4-byte scale, 512 x 4 bit + 32 bytes of scale; "DeepSeek V4.1 Flash 深度解析", part-4
// entry on FP4 in the KV cache: the window stays FP8).  The encoders are this library's
// reading of those sizes:
//   indexer   scale = fl32(amax/6) over the 128 values (1 when below 2^-126),
//             code = E2M1(fl32(x/scale));
//   main      per 16 values scale = E4M3(fl32(amax/6)) (the zero code becomes 2^-9),
//             code = E2M1(fl32(x/scale));
//   E2M1      nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to the even code, saturating at 6,
//             sign bit = the value's sign bit; element 2i in the low nibble of byte i;
//   E4M3      nearest, ties to even, saturating at 448; window row of position p in ring
//             slot p mod 128.
// Per entry, lane l of a wave quantises main values 8l..8l+7 (half a scale group, the pair
// of lanes meets in one shuffle) and indexer values 2l, 2l+1 (the scale's maximum is a
// wave reduction), so every load and store of the wave is one contiguous run.  The
// indexer's divisions are IEEE divisions; the main entry's take the reciprocal path below,
// which gives the codes of the IEEE quotients.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kAppendWaves = 4;
constexpr int kAppendPerWave = 4;       // rows per wave

// E2M1 codes of two values (nibbles 0 and 1 of byte `sel` of the result, the rest of
// `old` kept): gfx950's converter with scale 1 rounds to nearest-even, saturates at 6 and
// keeps the sign bit, which is the E2M1 encoder stated at the top of this file (measured
// value for value against the definition, every tie included).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Quotients for the main entry without a division.  A bf16 value (8 significant bits)
// divided by an E4M3 scale (4 bits) either equals a value of at most 7 significant bits
// exactly or differs from every such value by at least 2^-9 of its size.  Every rounding
// boundary that matters here has at most 5 significant bits: the E2M1 midpoints 0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5, 5 and the E4M3 midpoints (for amax / 6 = amax * 2^-1 / 3,
// likewise at least 2^-10 away unless equal).  x * rcp(s) is within 3 ulps of x / s, so
// rounding it to the nearest multiple of 128 ulps (low 7 mantissa bits cleared) lands
// exactly on a boundary when the true quotient is one and on the same side of every
// boundary otherwise: the encoder then returns the code of the IEEE quotient.
__device__ __forceinline__ float snap128(float q) {
  return __uint_as_float((__float_as_uint(q) + 0x40u) & 0xffffff80u);
}

// E4M3 codes of two finite values in bytes 0 and 1: the converter rounds to nearest-even
// but turns magnitudes from 464 up into NaN, so values are clamped to +-448 first (which
// is where nearest-even with saturation sends them).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  typedef short v2i16 __attribute__((ext_vector_type(2)));
  const v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
      v2i16{0, 0}, __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f),
      __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f), 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

// Maximum over the wave without LDS: DPP within each row of 16 lanes, then the four rows'
// maxima read out of lanes 0, 16, 32, 48.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                      0xf, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0xb1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4e>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  v = dpp_max<0x140>(v);  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Value of a positive E4M3 code (0x01..0x7e): normal codes are the fp32 exponent and top
// mantissa bits shifted into place, subnormal codes are multiples of 2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return c >= 8u ? __uint_as_float((c << 20) + 0x3c000000u) : (float)c * 0x1p-9f;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Quantises the entry whose values lane holds: main values 8*lane .. +7 in xv, indexer
// values 2*lane, 2*lane + 1 in xi.
__device__ __forceinline__ void quantise_entry(const uint4 xv, const uint32_t xi, int lane, int64_t d,
                                               uint8_t* __restrict__ idx_codes,
                                               float* __restrict__ idx_scale,
                                               uint8_t* __restrict__ kv_codes,
                                               uint8_t* __restrict__ kv_scale) {
  // main entry: scale group lane / 2
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(w[j]);
    v[2 * j + 1] = bf16_hi(w[j]);
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j]));
  am = dpp_max<0xb1>(am);  // the lane pair sharing the scale group
  uint32_t sc = e4m3_pair(snap128(am * (1.0f / 6.0f)), 0.0f) & 0xffu;
  sc = sc == 0u ? 1u : sc;
  const float rs = __builtin_amdgcn_rcpf(e4m3_value(sc));
  uint32_t word = e2m1_pair<0>(0u, snap128(v[0] * rs), snap128(v[1] * rs));
  word = e2m1_pair<1>(word, snap128(v[2] * rs), snap128(v[3] * rs));
  word = e2m1_pair<2>(word, snap128(v[4] * rs), snap128(v[5] * rs));
  word = e2m1_pair<3>(word, snap128(v[6] * rs), snap128(v[7] * rs));
  reinterpret_cast<uint32_t*>(kv_codes + (size_t)d * (kDKv / 2))[lane] = word;
  if ((lane & 1) == 0) kv_scale[(size_t)d * (kDKv / 16) + (lane >> 1)] = (uint8_t)sc;

  // indexer entry: one scale for the whole entry
  const float x0 = bf16_lo(xi), x1 = bf16_hi(xi);
  const float ai = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  float scale = ai / 6.0f;
  scale = scale >= 0x1p-126f ? scale : 1.0f;
  // the fp32 scale has a full mantissa, so these quotients are IEEE divisions
  idx_codes[(size_t)d * (kDIdx / 2) + lane] = (uint8_t)e2m1_pair<0>(0u, x0 / scale, x1 / scale);
  if (lane == 0) idx_scale[d] = scale;
}

// A wave takes kAppendPerWave consecutive rows and issues every load (ids and values) before
// quantising the first, so each wave keeps about 5 KB of reads in flight.
__global__ __launch_bounds__(64 * kAppendWaves) void k_kv_append(
    const uint16_t* __restrict__ x_idx, const uint16_t* __restrict__ x_kv,
    const int64_t* __restrict__ dst, int n, int64_t capacity, uint8_t* __restrict__ idx_codes,
    float* __restrict__ idx_scale, uint8_t* __restrict__ kv_codes, uint8_t* __restrict__ kv_scale,
    int32_t* __restrict__ bad) {
  const int lane = threadIdx.x & 63;
  const int i0 = (blockIdx.x * kAppendWaves + (int)(threadIdx.x >> 6)) * kAppendPerWave;
  if (i0 >= n) return;  // wave-uniform
  uint4 xv[kAppendPerWave];
  uint32_t xi[kAppendPerWave];
  int64_t d[kAppendPerWave];
#pragma unroll
  for (int e = 0; e < kAppendPerWave; ++e) {
    const int i = min(i0 + e, n - 1);  // rows past n re-read the last row and are dropped
    d[e] = dst[i];
    xv[e] = reinterpret_cast<const uint4*>(x_kv + (size_t)i * kDKv)[lane];
    xi[e] = reinterpret_cast<const uint32_t*>(x_idx + (size_t)i * kDIdx)[lane];
  }
  int rejected = 0;
#pragma unroll
  for (int e = 0; e < kAppendPerWave; ++e) {
    if (i0 + e >= n) break;
    if (d[e] < 0 || d[e] >= capacity) {
      ++rejected;
      continue;
    }
    // the id is the same in every lane: take it as a scalar so the stores' bases are scalar
    const int64_t du = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(d[e] >> 32)) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane((int)d[e]));
    quantise_entry(xv[e], xi[e], lane, du, idx_codes, idx_scale, kv_codes, kv_scale);
  }
  if (rejected && lane == 0 && bad) atomicAdd(bad, rejected);
}

// One wave per sequence: lane l encodes values 8l..8l+7 of the new row.
__global__ __launch_bounds__(64 * kAppendWaves) void k_swa_append(const uint16_t* __restrict__ x,
                                                                  const int64_t* __restrict__ pos,
                                                                  int batch, uint8_t* __restrict__ swa) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kAppendWaves + (int)(threadIdx.x >> 6);
  if (b >= batch) return;
  const int64_t p = pos[b];
  if (p < 0) return;
  const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)b * kDKv)[lane];
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t lo = e4m3_pair(bf16_lo(w[0]), bf16_hi(w[0])) | (e4m3_pair(bf16_lo(w[1]), bf16_hi(w[1])) << 16);
  const uint32_t hi = e4m3_pair(bf16_lo(w[2]), bf16_hi(w[2])) | (e4m3_pair(bf16_lo(w[3]), bf16_hi(w[3])) << 16);
  uint8_t* row = swa + ((size_t)b * kSwa + (size_t)(p % kSwa)) * kDKv;
  reinterpret_cast<uint2*>(row)[lane] = make_uint2(lo, hi);
}

hipError_t launch_kv_append(const uint16_t* x_idx, const uint16_t* x_kv, const int64_t* dst, int n,
                            int64_t capacity, uint8_t* idx_codes, float* idx_scale, uint8_t* kv_codes,
                            uint8_t* kv_scale, int32_t* bad, hipStream_t stream) {
  constexpr int rows_per_wg = kAppendWaves * kAppendPerWave;
  if (n > 0)
    hipLaunchKernelGGL(k_kv_append, dim3((n + rows_per_wg - 1) / rows_per_wg), dim3(64 * kAppendWaves),
                       0, stream, x_idx, x_kv, dst, n, capacity, idx_codes, idx_scale, kv_codes,
                       kv_scale, bad);
  return hipGetLastError();
}

hipError_t launch_swa_append(const uint16_t* x, const int64_t* pos, int batch, uint8_t* swa,
                             hipStream_t stream) {
  if (batch > 0)
    hipLaunchKernelGGL(k_swa_append, dim3((batch + kAppendWaves - 1) / kAppendWaves),
                       dim3(64 * kAppendWaves), 0, stream, x, pos, batch, swa);
  return hipGetLastError();
}

}  // namespace csa2
