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
// contraction and runs on the matrix cores in fp16:
//   * every dequantised value is exact in fp16: an E2M1 magnitude has at most 2
//     significant bits and an E4M3 scale at most 4, so the product has at most 6 and lies
//     in [2^-10, 2688]; window values are E4M3 themselves.  gfx950 converts FP4 / FP8 to
//     fp16 pairs directly and the scale is one packed fp16 multiply per pair;
//   * q is scaled per head by a power of two so that its largest element lies in
//     [2^14, 2^15) and rounded to fp16 (exact unless an element is below 2^-28 of its
//     head's largest); the power of two is folded back into the softmax scale.  q . v on
//     v_mfma_f32_16x16x32_f16 then has exact products and fp32 sums;
//   * p . v takes p as the sum of two fp16 halves (hi = fp16(p), lo = fp16(p - hi)),
//     relative error about 2^-22, fp32 sums: one v_mfma_f32_16x16x32_f16 per output tile
//     whose K runs over the hi half at the segment's 16 positions, then the lo half at the
//     same positions (v's rows given twice).
// Work split: one 128-thread workgroup (2 waves) per (row, split) walks the split's
// 16-position segments of the row's list (the k selected entries, then the window rows);
// wave w owns dims 256 w .. 256 w + 255 of every segment:
//   gather   lane (position n, dim group g) loads dims 256 w + 64 g .. + 63 of position n
//            (32 code bytes + 4 scale bytes, or 64 window bytes); the next segment's
//            loads are issued as soon as this one's bytes are dequantised, into the same
//            registers, and a split's first segment before the query's prologue;
//   q . v    8 k-steps; k-step s of dim group g covers dims 256 w + 64 g + 8 s .. + 7, so
//            each lane dequantises exactly its own loaded bytes into the B operand; the two
//            waves' partial scores meet in LDS and are added in the same order by both;
//   softmax  per head over the segment's 16 positions, computed by both waves alike; the
//            running max moves only when a score exceeds it by more than 2^8, so one
//            ballot per segment usually shows that neither the segment's maximum (DPP row
//            reductions) nor a rescale of the accumulators is needed;
//   p . v    the dequantised half-segment is also written to the wave's LDS tile (positions
//            x dims, XOR-swizzled) and read back transposed with ds_read_b64_tr_b16 as the
//            B operand of 16 output tiles of 16 dims; p's hi and lo halves (each wave
//            writes its heads') go through LDS the same way.  Two workgroup barriers per
//            segment.
// A row with several splits leaves (max, sum, acc[16][512]) per split in the workspace and
// k_attn_merge combines them by log-sum-exp.  exp2 with log2(e) folded into
// the scale.
#include "csa2_device.h"
#include "csa2_internal.h"

#include <math.h>

namespace csa2 {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kAW = 2;                       // waves per workgroup, one per half of the dims
constexpr int kAThreads = 64 * kAW;
constexpr int kHalf = kDKv / kAW;            // dims per wave
constexpr int kHalfTiles = kHalf / 16;       // output tiles of 16 dims per wave
constexpr int kSeg = 16;                     // list positions per wave step
constexpr int kIdxStage = 1024;              // list positions whose entry ids sit in LDS
constexpr int kMaxSplits = 64;               // splits per decode row
constexpr int kSplitSlots = 1024;            // decode workgroups aimed for (4 per CU)
constexpr int kCuSplitMaxSegs = 5;           // longest split the one-per-CU rule may take
constexpr int kPart = 2 * kHeads + kHeads * kDKv;  // floats per split: m[16], l[16], acc
constexpr float kRescale = 8.0f;             // log2 headroom before the running max moves

int attn_segments(int k) { return (k + kSwa + kSeg - 1) / kSeg; }
int attn_splits(int k) { return min(attn_segments(k), kMaxSplits); }

// Decode segments per split.  Few rows: the fewest segments (at most kCuSplitMaxSegs) that
// put every row's splits on their own compute unit (measured at 640 positions per row: 1
// segment for 4 rows, 3 for 16, 5 for 32; the split rule below gave 2 and 3, and c3's 20
// attentions at 16 rows took 338 instead of 297 us).  Otherwise each extra segment in a
// split adds about one gather latency, while each split's partial (16 x 512 fp32) is
// written and read back once; the sum is smallest near sqrt(rows x segments / 200)
// segments per split (5 for 128 rows of 640 positions, i.e. 8 equal splits: 704 us for the
// replay's layers against 716 at 6, 706 at 7 and more at 9 and 13).
// Compute units of the current device (one split each for few rows); 256, an MI355X's
// count, when no device answers (workspace sizing on a host without one).
static int attn_cus() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
    return 256;
  return n_cu;
}

static int attn_segs_per_split(int rows, int k) {
  const int segs = attn_segments(k);
  const int n_cu = attn_cus();
  for (int s = 1; s <= min(kCuSplitMaxSegs, segs); ++s) {
    const int splits = (segs + s - 1) / s;
    if (splits <= kMaxSplits && (long long)rows * splits <= n_cu) return s;
  }
  int sps = max(1, (int)lround(sqrt((double)rows * segs / 200.0)));
  sps = max(sps, (int)(((long long)rows * segs + kSplitSlots - 1) / kSplitSlots));
  sps = max(sps, (segs + kMaxSplits - 1) / kMaxSplits);
  return min(sps, segs);
}

// Splits a row of k entries + its window is cut into for `rows` rows.
static int attn_used_splits(int rows, int k) {
  const int sps = attn_segs_per_split(rows, k);
  return (attn_segments(k) + sps - 1) / sps;
}

// Partials of the split rows; a launch whose rows are not split needs none.
size_t attn_ws_bytes(int rows, int k) {
  const int used = attn_used_splits(rows, k);
  return used > 1 ? align_up((size_t)rows * used * kPart * sizeof(float), 256) : 256;
}

// ---- LDS tiles
// V of one wave's half of a segment: 16 position rows x 32 blocks of 8 fp16 (512 B per
// row); block b of row r at b ^ vswz(r).  Conflict-free for the 16-byte row writes (16
// rows, one block) and for the transposed 8-byte reads (4 rows x 2 blocks per 16 lanes).
__device__ __forceinline__ int vswz(int r) { return ((r << 1) & 14) | ((r >> 3) & 1); }

__device__ __forceinline__ f16x4 tr_read(const f16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// DPP reductions over the 16 lanes of a row (xor 1, xor 2, half-row mirror, row mirror).
template <bool MAX>
__device__ __forceinline__ float row16(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false)));
  return v;
}

// Raw bytes of one lane's 64 dims of a position in a segment: main entry (m = 32 code
// bytes, sc = its 4 scale bytes), window row (w = 64 bytes), or nothing.  Every lane issues
// all seven loads whatever its kind (a lane of the other kind, or of nothing, reads the
// sequence's first entry or the first window row, which the segment's other lanes share):
// no branch, the addresses are one select and one shift-add each, and every lane's loads
// stay in flight.
struct Raw {
  uint4 m[2];
  uint4 w[4];
  uint32_t sc;
  int kind;  // 0 nothing, 1 main entry, 2 window row
};

__device__ __forceinline__ f16x8 deq_main(uint32_t w, f16 s) {
  const f16x2 ss = {s, s};
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ f16x8 deq_win(uint32_t w0, uint32_t w1) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// MODE 0: decode row b (entries seq_base[b] + idx, window rows swa[b][0..swa_len[b])).
// MODE 1: prefill row t at position pos0 + t (entries idx from 0, window positions
//         max(0,p-127)..p, row r of `swa` holding position pos0 - 127 + r); one split.
template <int MODE>
__global__ __launch_bounds__(kAThreads, 2) void k_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_codes,
    const uint8_t* __restrict__ kv_scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ idx, int k, const uint8_t* __restrict__ swa,
    const int32_t* __restrict__ swa_len, int64_t pos0, float qscale, float* __restrict__ out,
    float* __restrict__ part, int segs_per_split, int n_splits) {
  __shared__ __align__(16) f16 s_v[kAW][kSeg * kHalf];         // each wave's half of a segment
  __shared__ __align__(16) f16 s_p[2][kSeg * kHeads];          // p hi / lo, [position][head]
  __shared__ __align__(16) f32x4v s_z[kAW][64];                // partial scores per lane
  __shared__ __align__(16) float s_alpha[kHeads];              // this segment's rescale per head
  __shared__ __align__(16) float s_ml[2][kHeads];              // final max and sum per head
  __shared__ uint32_t s_mv[kAW];                               // a wave's heads moved their max
  __shared__ int32_t s_idx[kIdxStage];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // the row's base and window length first: the first gather's addresses need them, so
  // their latency overlaps the ids' and q's instead of following them
  const int64_t base = MODE == 0 ? seq_base[b] : 0;
  const int row_swa_len = MODE == 0 ? swa_len[b] : 0;
  const int n16 = lane & 15, g16 = lane >> 4;
  const int d0 = kHalf * w + 64 * g16;  // this lane's first dim in the q . v steps
  const int32_t* irow = k > 0 ? idx + (size_t)b * k : nullptr;
  const int seg_begin = split * segs_per_split;

  // this lane's position in the split's first segment and its entry id, loaded first: the
  // first gather depends on nothing else, so it is issued before q's prologue
  const int p_first = seg_begin * kSeg + n16;
  const int j_first = p_first < k ? irow[p_first] : -1;

  // the first stage's entry ids, loaded before q so that both latencies overlap
  constexpr int kIdPer = kIdxStage / kAThreads;
  int32_t ids[kIdPer];
  {
    const int n_first = min(min(segs_per_split, kIdxStage / kSeg) * kSeg, k - seg_begin * kSeg);
#pragma unroll
    for (int i = 0; i < kIdPer; ++i) {
      const int j = tid + i * kAThreads;
      ids[i] = j < n_first ? irow[seg_begin * kSeg + j] : -1;
    }
  }

  // ---- q as A operands (head n16, dims d0 + 8 s .. + 7 for k-step s), scaled per head by
  // a power of two into fp16's range
  const uint16_t* qrow = q + ((size_t)b * kHeads + n16) * kDKv;
  uint4 raw[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) raw[s] = reinterpret_cast<const uint4*>(qrow + d0)[s];

  const uint8_t* rows;
  int nrows;
  if (MODE == 0) {
    rows = swa + (size_t)b * kSwa * kDKv;
    nrows = min(max(row_swa_len, 0), kSwa);
  } else {
    const int64_t p = pos0 + b;
    const int64_t lo = p - (kSwa - 1) > 0 ? p - (kSwa - 1) : 0;
    rows = swa + (size_t)(lo - (pos0 - (kSwa - 1))) * kDKv;
    nrows = (int)(p - lo + 1);
  }
  const int n_pos = k + nrows;
  const int n_seg = (n_pos + kSeg - 1) / kSeg;
  const int seg_end = min(seg_begin + segs_per_split, n_seg);
  // this lane's bytes of entry 0 / window row 0: the gathers add the entry or row offset
  const uint8_t* code_base = kv_codes + base * kKvCodeBytes + d0 / 2;
  const uint8_t* scale_base = kv_scale + base * kKvScaleBytes + d0 / 16;
  const uint8_t* win_base = rows + d0;

  // Raw bytes of segment `seg` for this lane (entry id j if its position holds a main
  // entry); nothing at or past segment `stop`
  auto gather = [&](int seg, int j, int stop) {
    Raw r;
    const int p = seg * kSeg + n16;
    const int kind = (seg < stop && p < n_pos) ? (p < k ? (j >= 0 ? 1 : 0) : 2) : 0;
    r.kind = kind;
    const uint32_t jj = kind == 1 ? (uint32_t)j : 0u;
    const uint32_t pp = kind == 2 ? (uint32_t)(p - k) : 0u;
    const uint4* am = reinterpret_cast<const uint4*>(code_base + (uint64_t)jj * kKvCodeBytes);
    const uint4* aw = reinterpret_cast<const uint4*>(win_base + (uint64_t)pp * kDKv);
    r.m[0] = am[0];
    r.m[1] = am[1];
    r.sc = *reinterpret_cast<const uint32_t*>(scale_base + (uint64_t)jj * kKvScaleBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = aw[i];
    return r;
  };
  // the split's first segment is in flight through q's prologue and the ids' staging
  Raw r0 = gather(seg_begin, j_first, min(seg_begin + kIdxStage / kSeg, seg_end));
  __builtin_amdgcn_sched_barrier(0);  // issued before the prologue's first wait on q

  f16x8 qa[8];
  float qs[2];  // softmax scale of heads 8 w + 2 g16 + j (log2 units), with the head's power of two
  {
    float amax = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = word_of(raw[s], i);
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(u & 0xffffu)), fabsf(bf16_bits_to_f32(u >> 16))));
      }
    }
    // the head's largest element: over the four dim groups of this wave, then the waves
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (g16 == 0) s_z[w][n16][0] = amax;
    __syncthreads();
    amax = fmaxf(s_z[0][n16][0], s_z[1][n16][0]);
    int e = 0;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);  // amax = m * 2^ex, m in [0.5, 1)
      e = ex - 15;        // amax * 2^-e in [2^14, 2^15)
    }
    const float up = ldexpf(1.0f, -e);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      f16 v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = word_of(raw[s], i);
        v[2 * i] = (f16)(bf16_bits_to_f32(u & 0xffffu) * up);
        v[2 * i + 1] = (f16)(bf16_bits_to_f32(u >> 16) * up);
      }
      qa[s] = f16x8{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) qs[j] = qscale * ldexpf(1.0f, __shfl(e, 8 * w + 2 * g16 + j));
  }

  // running softmax state: wave w, lane (position n16, g16) runs heads 8 w + 2 g16 + j
  // (j = 0, 1): the running max (the same in the head's 16 lanes) and this lane's share of
  // the sum (its position's terms, added over the lanes at the end).  Accumulators of this
  // wave: acc[t] = tile t of its half, lane (dim 16 t + n16, heads 4 g16 + r)
  float m[2], lp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    m[j] = -__builtin_inff();
    lp[j] = 0.f;
  }
  f32x4v acc[kHalfTiles];
#pragma unroll
  for (int t = 0; t < kHalfTiles; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};

  f16* vt = s_v[w];
  // transposed-read coordinates of p . v: lane = 16 g + 4 mm + qq reads rows
  // 8 (g % 2) + mm and 8 (g % 2) + 4 + mm, columns 4 qq
  const int tr_row = 8 * (g16 & 1) + ((lane >> 2) & 3), tr_q = lane & 3;

  for (int stage0 = seg_begin; stage0 < seg_end; stage0 += kIdxStage / kSeg) {
    const int stage1 = min(stage0 + kIdxStage / kSeg, seg_end);
    const int idx_base = stage0 * kSeg;
    const int idx_n = min(stage1 * kSeg, k) - idx_base;  // ids this stage reads
    __syncthreads();  // the previous stage's ids are no longer read
    if (stage0 == seg_begin) {
#pragma unroll
      for (int i = 0; i < kIdPer; ++i) s_idx[tid + i * kAThreads] = ids[i];
    } else {
      for (int i = tid; i < idx_n; i += kAThreads) s_idx[i] = irow[idx_base + i];
    }
    __syncthreads();
    const int n_i = stage1 - stage0;

    // segment stage0 + i with its id from the stage's LDS copy (read whatever the kind)
    auto issue = [&](int i) {
      const int p = (stage0 + i) * kSeg + n16;
      return gather(stage0 + i, s_idx[min(max(p - idx_base, 0), kIdxStage - 1)], stage1);
    };

    auto compute = [&](Raw& r, int next) {
      // ---- dequantise this wave's half into B operands, stage it for p . v, and q . v.
      // The segment's kinds pick one of three straight-line paths (wave-uniform): main
      // entries (a lane with nothing dequantises with scale 0), window rows, or both.
      const bool any_win = __ballot(r.kind == 2) != 0ull;
      const bool any_main = __ballot(r.kind != 2) != 0ull;
      f16 sc[4];
      {
        const uint32_t scw = r.kind == 1 ? r.sc : 0u;
        const f16x2 s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scw, 1.0f, false);
        const f16x2 s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scw, 1.0f, true);
        sc[0] = s0.x; sc[1] = s0.y; sc[2] = s1.x; sc[3] = s1.y;
      }
      f32x4v z = {0.f, 0.f, 0.f, 0.f};
      f16* vrow = vt + n16 * kHalf;
      const int sw = vswz(n16);  // loop-invariant: the 8 write addresses stay in registers
      auto step = [&](int s, const f16x8& bv) {
        *reinterpret_cast<f16x8*>(vrow + 8 * ((8 * g16 + s) ^ sw)) = bv;
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[s], bv, z, 0, 0, 0);
      };
      if (!any_win) {
#pragma unroll
        for (int s = 0; s < 8; ++s) step(s, deq_main(word_of(r.m[s >> 2], s & 3), sc[s >> 1]));
      } else if (!any_main) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint4 v = r.w[s >> 1];
          step(s, (s & 1) ? deq_win(v.z, v.w) : deq_win(v.x, v.y));
        }
      } else {
        const bool win = r.kind == 2;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint4 v = r.w[s >> 1];
          const f16x8 bw = (s & 1) ? deq_win(v.z, v.w) : deq_win(v.x, v.y);
          const f16x8 bm = deq_main(word_of(r.m[s >> 2], s & 3), sc[s >> 1]);
          step(s, win ? bw : bm);
        }
      }
      // the raw bytes are dead: the next segment's loads go into the same registers and
      // stay in flight through the softmax and p . v (no second register set to copy from)
      const bool valid = r.kind != 0;
      if (next < n_i) r = issue(next);  // wave-uniform: nothing to load after the stage's last
      // ---- the two halves' scores, added in the same order in both waves
      s_z[w][lane] = z;
      __syncthreads();
      // ---- online softmax over the segment's positions for this wave's eight heads
      const int zl = 16 * (2 * w + (g16 >> 1)) + n16;  // tile lane holding heads 8w+2g16+j
      const float2 za = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(&s_z[0][zl]) + 2 * (g16 & 1));
      const float2 zb = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(&s_z[1][zl]) + 2 * (g16 & 1));
      const float zsum[2] = {za.x + zb.x, za.y + zb.y};
      float zs[2], alpha[2] = {1.0f, 1.0f};
      bool moved = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) zs[j] = valid ? zsum[j] * qs[j] : -__builtin_inff();
      // a head's running max moves only to a segment maximum above it by more than
      // kRescale, so one compare per lane tells whether any head of the wave needs its
      // segment maximum and rescale factor (the first segment, then rarely); otherwise
      // both stay as they are (factor 1), the same result as always reducing
      if (__ballot(zs[0] > m[0] + kRescale || zs[1] > m[1] + kRescale) != 0ull) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float cm = row16<true>(zs[j]);
          const float mu = cm > m[j] + kRescale ? cm : m[j];
          alpha[j] = mu == m[j] ? 1.0f : (m[j] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m[j] - mu));
          moved |= mu != m[j];
          m[j] = mu;
        }
      }
      float p[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        p[j] = zs[j] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(zs[j] - m[j]);
        lp[j] = lp[j] * alpha[j] + p[j];
      }
      // p = hi + lo in fp16, staged as [position][head]; each head's rescale and whether a
      // wave's maxima moved
      {
        const f16 h0 = (f16)p[0], h1 = (f16)p[1];
        const f16 o0 = (f16)(p[0] - (float)h0), o1 = (f16)(p[1] - (float)h1);
        const int at = n16 * kHeads + 8 * w + 2 * g16;
        *reinterpret_cast<f16x2*>(s_p[0] + at) = f16x2{h0, h1};
        *reinterpret_cast<f16x2*>(s_p[1] + at) = f16x2{o0, o1};
        if (n16 == 0) *reinterpret_cast<float2*>(s_alpha + 8 * w + 2 * g16) = float2{alpha[0], alpha[1]};
        const bool mv = __ballot(moved) != 0ull;
        if (lane == 0) s_mv[w] = mv ? 1u : 0u;
      }
      __syncthreads();
      if ((s_mv[0] | s_mv[1]) != 0u) {
        const f32x4v al = *reinterpret_cast<const f32x4v*>(s_alpha + 4 * g16);
#pragma unroll
        for (int t = 0; t < kHalfTiles; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[t][rr] *= al[rr];
      }
      // ---- acc += p . v over this wave's half: one v_mfma_f32_16x16x32_f16 per tile whose
      // K = 32 runs over p's hi half at the segment's 16 positions, then its lo half at the
      // same positions (lane groups 0, 1: hi, positions 0-7, 8-15; groups 2, 3: lo), with v's
      // rows given twice.  A = p (head, 8 positions), B = v (8 positions, dim), transposed
      // reads of rows tr_row and tr_row + 4.
      const f16* pb = s_p[g16 >> 1];
      const f16x4 pa = tr_read(pb + tr_row * kHeads + 4 * tr_q);
      const f16x4 pc = tr_read(pb + (tr_row + 4) * kHeads + 4 * tr_q);
      const f16x8 a8 = __builtin_shufflevector(pa, pc, 0, 1, 2, 3, 4, 5, 6, 7);
      const int tsw0 = vswz(tr_row), tsw1 = vswz(tr_row + 4);
      // tiles t and t + 8 share the swizzled block's low bits: loop-invariant bases,
      // immediate offsets
      const f16* vr0[8];
      const f16* vr1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        vr0[t] = vt + tr_row * kHalf + 8 * ((2 * t + (tr_q >> 1)) ^ tsw0) + 4 * (tr_q & 1);
        vr1[t] = vt + (tr_row + 4) * kHalf + 8 * ((2 * t + (tr_q >> 1)) ^ tsw1) + 4 * (tr_q & 1);
      }
#pragma unroll
      for (int t = 0; t < kHalfTiles; ++t) {
        const f16x4 b0 = tr_read(vr0[t & 7] + 128 * (t >> 3));
        const f16x4 b1 = tr_read(vr1[t & 7] + 128 * (t >> 3));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                        acc[t], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();  // the next segment rewrites this wave's tile
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // the next segment's loads are in flight while one is computed
    if (stage0 != seg_begin) r0 = issue(0);
    for (int i = 0; i < n_i; ++i) compute(r0, i + 1);
  }

  // ---- each head's max and sum (over its 16 lanes' shares), then out (one split) or this
  // split's (max, sum, acc)
  {
    const float lt0 = row16<false>(lp[0]), lt1 = row16<false>(lp[1]);
    if (n16 == 0) {
      *reinterpret_cast<float2*>(s_ml[0] + 8 * w + 2 * g16) = float2{m[0], m[1]};
      *reinterpret_cast<float2*>(s_ml[1] + 8 * w + 2 * g16) = float2{lt0, lt1};
    }
  }
  __syncthreads();
  if (n_splits == 1) {
    float* O = out + (size_t)b * kHeads * kDKv + kHalf * w;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g16 + r;
      const float lh = s_ml[1][h];
      const float inv = lh > 0.f ? 1.0f / lh : 0.f;
#pragma unroll
      for (int t = 0; t < kHalfTiles; ++t) O[h * kDKv + 16 * t + n16] = acc[t][r] * inv;
    }
    return;
  }
  // non-temporal stores: the merge launch reads the partials once, from another XCD as
  // often as not, and less is left in this XCD's L2 to write back at the kernel's end
  // (40-layer pass 723 -> 715 us)
  float* P = part + ((size_t)b * n_splits + split) * kPart;
  if (tid < kHeads) {
    __builtin_nontemporal_store(s_ml[0][tid], P + tid);
    __builtin_nontemporal_store(s_ml[1][tid], P + kHeads + tid);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kHalfTiles; ++t)
      __builtin_nontemporal_store(acc[t][r], P + 2 * kHeads + (4 * g16 + r) * kDKv + kHalf * w + 16 * t + n16);
}

// Log-sum-exp merge of a row's splits for one of QB equal blocks of one head's dims: 256
// threads; each sums 4 dims of the block over one group of splits (the groups interleave),
// with every load issued before the first is used, and the split groups meet in LDS.  The
// first wave turns each split's (max, sum) into its weight meanwhile (two wave
// reductions).  Quarters (8 split groups) up to kMergeManyRows rows, halves beyond
// (measured for 128 rows: 720 against 732 us for the replay's layers; whole heads 753).
constexpr int kMergeThreads = 256;
constexpr int kMergeManyRows = 32;  // rows above which a head's dims are merged in fewer blocks
template <int QB>
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge(const float* __restrict__ part,
                                                              int n_splits, float* __restrict__ out) {
  constexpr int kMergeQuarters = QB;                                      // blocks per head
  constexpr int kMergeDims = kDKv / kMergeQuarters;
  constexpr int kMergeLanes = kMergeDims / 4;                             // float4 lanes
  constexpr int kMergeGroups = kMergeThreads / kMergeLanes;               // split groups
  constexpr int kMergePer = (kMaxSplits + kMergeGroups - 1) / kMergeGroups;
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_L;
  __shared__ float4 s_o[kMergeGroups][kMergeLanes];
  const int h = blockIdx.x / kMergeQuarters, quarter = blockIdx.x % kMergeQuarters;
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int grp = tid / kMergeLanes, d = quarter * kMergeDims + 4 * (tid % kMergeLanes);
  const float* P0 = part + (size_t)b * n_splits * kPart;
  // each split's (max, sum) first: loads return in order, so the weights can be computed
  // while the accumulators are still on their way
  float ms = -__builtin_inff(), ls = 0.f;
  if (tid < 64 && lane < n_splits) {
    ms = P0[(size_t)lane * kPart + h];
    ls = P0[(size_t)lane * kPart + kHeads + h];
  }
  float4 a[kMergePer];
#pragma unroll
  for (int i = 0; i < kMergePer; ++i) {
    const int sp = grp + kMergeGroups * i;
    a[i] = sp < n_splits ? *reinterpret_cast<const float4*>(P0 + (size_t)sp * kPart + 2 * kHeads + h * kDKv + d)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid < 64) {
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
#pragma unroll
  for (int i = 0; i < kMergePer; ++i) {
    const int sp = grp + kMergeGroups * i;
    if (sp < n_splits) {
      const float wgt = s_w[sp];
      o.x = fmaf(a[i].x, wgt, o.x);
      o.y = fmaf(a[i].y, wgt, o.y);
      o.z = fmaf(a[i].z, wgt, o.z);
      o.w = fmaf(a[i].w, wgt, o.w);
    }
  }
  s_o[grp][tid % kMergeLanes] = o;
  __syncthreads();
  if (tid < kMergeLanes) {
    float4 t = s_o[0][tid];
#pragma unroll
    for (int g = 1; g < kMergeGroups; ++g) {
      const float4 u = s_o[g][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float L = s_L;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<float4*>(&out[((size_t)b * kHeads + h) * kDKv + d]) =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

hipError_t launch_attn(int mode, const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       const int64_t* seq_base, const int32_t* idx, int k, const uint8_t* swa,
                       const int32_t* swa_len, int64_t pos0, float softmax_scale, int rows,
                       float* out, void* ws, hipStream_t stream) {
  const float qscale = softmax_scale * 1.4426950408889634f;  // log2(e)
  const int segs = attn_segments(k);
  // rows are split over workgroups when they are few (decode batches, short prefill or
  // replay chunks); a prefill row's causal window may be shorter than 128, so its last
  // splits can be empty (they leave an empty partial)
  int sps = attn_segs_per_split(rows, k);
  int used = (segs + sps - 1) / sps;  // splits, each with at least one segment
  if (ws == nullptr) {                // no room for partials: one split per row
    sps = segs;
    used = 1;
  }
  float* part = static_cast<float*>(ws);
  if (mode == 1)
    hipLaunchKernelGGL(k_attn<1>, dim3(used, rows), dim3(kAThreads), 0, stream, q, kv_codes,
                       kv_scale, seq_base, idx, k, swa, swa_len, pos0, qscale, out, part, sps, used);
  else
    hipLaunchKernelGGL(k_attn<0>, dim3(used, rows), dim3(kAThreads), 0, stream, q, kv_codes,
                       kv_scale, seq_base, idx, k, swa, swa_len, pos0, qscale, out, part, sps, used);
  if (used > 1 && rows > kMergeManyRows)
    hipLaunchKernelGGL(k_attn_merge<2>, dim3(kHeads * 2, rows), dim3(kMergeThreads), 0, stream,
                       part, used, out);
  else if (used > 1)
    hipLaunchKernelGGL(k_attn_merge<4>, dim3(kHeads * 4, rows), dim3(kMergeThreads), 0, stream, part,
                       used, out);
  return hipGetLastError();
}

}  // namespace csa2
