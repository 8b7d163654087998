// a7 causal indexer contraction (BF16 MFMA) and a8 per-query top-k + attention for a
// prefill chunk: T consecutive query positions of one sequence, each scoring every
// entry it can see, taking its own top-k and attending over it plus its window
// ("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", content summary and the
// Q&A on prefill: prompt tokens run the encoder, whose Full layers score and select for
// every token; "从V4到V4.1 Flash：架构的激进进化", encoder section: one entry per two
// tokens).  Visibility is this library's reading: entry j is visible to position p once
// its last token (j+1)*ratio - 1 is at or before p.
//
// S[t][j] = scale_j * (q_t . e2m1(K_j)) is a dense T x N x 128 contraction on
// v_mfma_f32_32x32x16_bf16.  A workgroup owns 256 query rows (64 per wave, held as two
// sets of A operands that share every expanded B operand) and one split of 4,096 entries,
// which it streams through LDS in stages of 256 entries (raw 64 code bytes + fp32 scale
// each, double buffered, the next stage's loads in
// flight during the current stage's MFMAs, shared by the four waves).  Each wave expands
// its B operands from LDS to bf16 exactly (v_cvt_scalef32_pk_bf16_fp4); the 128 dims are
// permuted identically on both sides so each lane reads 32 contiguous code bytes.  The
// fp32 entry scale is applied to the fp32 accumulators.  The T x N score matrix is never
// stored:
//   pass 1 keeps, per row, the maximum of each group of 32 entries (a lane's column over
//          32 consecutive 32-entry tiles) as a 16-bit key prefix rounded down.  At least k
//          groups have maxima >= the k-th largest group maximum, so that value, theta_t,
//          is a rigorous lower bound on the row's k-th score;
//   pass 2 recomputes the contraction (taken transposed, see k_prefill_hits) and writes
//          the scores >= theta_t (typically several hundred per row) into the row's slots
//          for this split;
//   select resolves each row exactly in LDS (largest scores, ties to the lower entry) and
//          emits the chosen entries in ascending order.  A row whose candidates overflow a split's
//          slots (only possible with massive score ties) is resolved by recomputing its
//          scores in a streaming radix select; a row that sees at most k entries takes them
//          all.
// Stages past the causal frontier of a workgroup's rows are skipped.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "select_device.h"

namespace csa2 {

constexpr int kGemmThreads = 256;           // 4 waves x 64 query rows
constexpr int kSets = 2;                    // 32-row A operand sets per wave
constexpr int kWaveRows = 32 * kSets;
constexpr int kGemmRows = 4 * kWaveRows;
constexpr int kSplitEntries = 4096;         // entries per workgroup
constexpr int kStage = 256;                 // entries per LDS stage (8 tiles of 32)
constexpr int kStages = kSplitEntries / kStage;
constexpr int kRunStages = 4;               // group = one lane column over 32 tiles
constexpr int kGroupsPerSplit = kStages / kRunStages * 32;  // 128
constexpr int kSlots = 64;                  // candidate slots per (row, split): one per lane
static_assert(kSlots == 64, "select copies one split per wave, one slot per lane");
static_assert(kSplitEntries <= 4096, "queued hits hold the entry within its split in 12 bits");
constexpr int kCandLds = 4096;              // candidates a row may gather into LDS
constexpr int kSelThreads = 256;
static_assert(kSelThreads == 256, "the theta and select kernels give each of 256 bins a thread");
constexpr int kSelMaxSplits = 512;          // splits a row's fast path can gather (N <= 2M)
// Sampled threshold: pass 1 over every kSampleStride-th entry.  Used when kq = 3k/8 is at
// least kSampleMinQ and the first row sees at least kSampleMinGroupsPerQ * kq sample groups
// (each of 32 samples); with i.i.d. scores the candidates then number about 1.5 k per row
// (relative spread about 1 / sqrt(kq)), so fewer than k is a ~5 sigma event.
constexpr int kSampleStride = 4;
constexpr int kSampleMinQ = 128;
constexpr int kSampleMinGroupsPerQ = 4;

struct PrefillWs {
  uint16_t* gmax;               // [T][G] group maxima as key >> 16 (0 = empty group)
  float* theta;                 // [T]
  uint32_t* ccount;             // [T][n_splits] candidates found per split
  unsigned long long* cand;     // [T][n_splits][kSlots] (key << 32 | entry)
  void* attn;                   // attention partials (rows split over workgroups)
  int G, n_splits;              // G: row stride of gmax (groups of the full pass 1)
  int G_used;                   // groups the current pass 1 wrote per row (<= G)
};

static int prefill_splits(int n_entries) {
  return n_entries > 0 ? (n_entries + kSplitEntries - 1) / kSplitEntries : 1;
}

size_t prefill_ws_bytes(int T, int n_entries, int k) {
  const size_t S = (size_t)prefill_splits(n_entries);
  const size_t G = S * kGroupsPerSplit;
  size_t s = 0;
  s += align_up((size_t)T * G * 2, 256);
  s += align_up((size_t)T * 4, 256);
  s += align_up((size_t)T * S * 4, 256);
  s += align_up((size_t)T * S * kSlots * 8, 256);
  s += attn_ws_bytes(T, k);  // partials when the attention splits its rows (short chunks)
  return s;
}

static PrefillWs prefill_ws_carve(void* base, int T, int n_entries) {
  PrefillWs w;
  w.n_splits = prefill_splits(n_entries);
  w.G = w.n_splits * kGroupsPerSplit;
  w.G_used = w.G;
  char* p = static_cast<char*>(base);
  w.gmax = reinterpret_cast<uint16_t*>(p);
  p += align_up((size_t)T * w.G * 2, 256);
  w.theta = reinterpret_cast<float*>(p);
  p += align_up((size_t)T * 4, 256);
  w.ccount = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)T * w.n_splits * 4, 256);
  w.cand = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)T * w.n_splits * kSlots * 8, 256);
  w.attn = p;
  return w;
}

static int visible_host(int64_t pos, int ratio, int n_entries) {
  const int64_t v = (pos + 1) / ratio;
  return (int)(v < n_entries ? v : n_entries);
}

__device__ __forceinline__ int visible(int64_t pos, int ratio, int n_entries) {
  const int64_t v = (pos + 1) / ratio;
  return (int)(v < n_entries ? v : n_entries);
}

// Eight E2M1 codes (one dword) -> bf16x8 operand slice (exact).
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w) {
  const bf16x2 a = fp4x2_bf16<0>(w), b = fp4x2_bf16<1>(w), c = fp4x2_bf16<2>(w),
               d = fp4x2_bf16<3>(w);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// v_max_f32 without the quieting of signalling NaNs that fmaxf adds (scores are finite or -inf).
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// x of lane g of this lane's quad (a DPP operand of the instruction that uses it).
template <int G>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), G * 0x55, 0xf, 0xf, true));
}

// Largest of three products (canonical, finite): the compiler emits one v_max3_f32.
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// LDS stage: entry i's 64 code bytes as 4 blocks of 16 bytes, block b at b ^ ((i >> 2) & 3)
// so that 16 consecutive entries' reads of one block land in 16 distinct bank groups.
__device__ __forceinline__ int stage_blk(int i, int b) { return i * 4 + (b ^ ((i >> 2) & 3)); }

// The entry (within its tile of 32) at A row r: the inverse of e -> 8 ((e >> 2) & 3) +
// 4 (e >> 4) + (e & 3).
__device__ __forceinline__ int row_entry(int r) { return ((r >> 2) & 1) << 4 | (r >> 3) << 2 | (r & 3); }
// A raw buffer over n bytes: loads at offsets past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, int n_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n_bytes, 0x00020000);
}
// PASS 1: group maxima.
// Accumulator layout of v_mfma_f32_32x32x16_bf16: lane l holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  Operands: lane l holds row/column l % 32 and
// k-slice 8*(l/32)..+7; the dims behind k-step kk for half h are 64h + 8kk .. +7.
// A wave owns 64 rows as two sets of 32 (set s: rows 32s ..); each expanded B operand
// feeds one MFMA per set.
// STRIDE > 1: the contraction runs over every STRIDE-th entry (columns are sample indices,
// column c = entry STRIDE * c), for the sampled threshold.  A workgroup covers SPLIT
// columns (a multiple of one run of 1,024), SPLIT / 1,024 * 32 groups.
template <int STRIDE, int SPLIT>
__global__ __launch_bounds__(kGemmThreads, 2) void k_prefill_gmax(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, int n_entries, int ratio, int64_t pos0, int T, PrefillWs ws) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wg_row0 = blockIdx.x * kGemmRows;
  const int row0 = wg_row0 + wave * kWaveRows;
  static_assert(SPLIT % (kRunStages * kStage) == 0 && SPLIT <= kSplitEntries, "whole runs");
  constexpr int n_stages = SPLIT / kStage;
  constexpr int groups_per_split = n_stages / kRunStages * 32;
  const int split = blockIdx.y;
  const int n_cols = (n_entries + STRIDE - 1) / STRIDE;
  const int e_begin = split * SPLIT;  // columns
  const int e_end = min(e_begin + SPLIT, n_cols);
  const int rl = lane & 31, half = lane >> 5;
  // columns a row sees: the entries it sees, in columns
  auto vis_cols = [&](int64_t pos) { return (visible(pos, ratio, n_entries) + STRIDE - 1) / STRIDE; };

  // columns the wave's rows see: at most, and at least
  const int wave_nmax = row0 < T ? vis_cols(pos0 + min(row0 + kWaveRows - 1, T - 1)) : 0;
  const int wave_nmin = row0 < T ? vis_cols(pos0 + row0) : 0;

  // A operands: query row row0 + 32*s + rl, dims 64*half .. +63
  bf16x8 a[kSets][8];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    const int ar = min(row0 + 32 * s + rl, T - 1);
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + (size_t)ar * kDIdx + 64 * half);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) a[s][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
  }
  // row of accumulator r of set s within the wave
  auto wrow = [&](int s, int r) { return 32 * s + 8 * (r >> 2) + 4 * half + (r & 3); };
  // On a tile at the causal frontier, column col (entry STRIDE*col) is visible to wave row w
  // once the entry's last position (STRIDE*col+1)*ratio - 1 is at most pos0 + row0 + w, i.e.
  // once lim <= w - 4*half with lim the lane's offset below (clamped: far from the frontier
  // only its sign matters).
  // Rows past T need no mask: their maxima are never published.
  auto frontier_lim = [&](int col) {
    const int64_t d = ((int64_t)col * STRIDE + 1) * ratio - 1 - (pos0 + row0 + 4 * half);
    return col < n_cols ? (int)max(min(d, (int64_t)1 << 30), -((int64_t)1 << 30)) : (1 << 30);
  };
  auto wrow_h = [&](int s, int r) { return 32 * s + 8 * (r >> 2) + (r & 3); };  // wrow - 4*half

  // B operands straight from memory, two tiles ahead: lane (rl, half) takes code bytes
  // 32 half .. + 31 of column e0 + rl (entry STRIDE * column) and its scale.  Columns past
  // the end read as zeros (range-checked buffer loads); their maxima are never published.
  const __amdgpu_buffer_rsrc_t rs_code = buffer_over(codes, n_entries * kIdxCodeBytes);
  const __amdgpu_buffer_rsrc_t rs_scale = buffer_over(scale, n_entries * 4);
  // tiles of 32 columns that some row of the wave sees (wave-uniform)
  const int n_tiles = max(0, (min(e_end, wave_nmax) - e_begin + 31) / 32);
  struct TileIn {
    uint4 c0, c1;
    float sc;
  };
  auto load_tile = [&](int tt, TileIn& in) {
    const int ct = min(tt, n_tiles - 1);  // past the last tile: a repeat, never used
    const int e = (e_begin + ct * 32 + rl) * STRIDE;
    in.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_code, e * kIdxCodeBytes + 32 * half, 0, 0));
    in.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_code, e * kIdxCodeBytes + 32 * half + 16, 0, 0));
    in.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_scale, e * 4, 0, 0));
  };
  auto mfma_tile = [&](const TileIn& in, f32x16 (&acc)[kSets]) {
    const uint32_t cw[8] = {in.c0.x, in.c0.y, in.c0.z, in.c0.w, in.c1.x, in.c1.y, in.c1.z, in.c1.w};
#pragma unroll
    for (int s = 0; s < kSets; ++s) acc[s] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 bv = fp4x8_bf16(cw[kk]);
#pragma unroll
      for (int s = 0; s < kSets; ++s)
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][kk], bv, acc[s], 0, 0, 0);
    }
  };

  float rm[kSets][16];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) rm[s][r] = -__builtin_inff();
  // the running maxima take tile tt's scaled scores (masked at the causal frontier)
  auto take_max = [&](int tt, float sc, const f32x16 (&acc)[kSets]) {
    const int e0 = e_begin + tt * 32;
    if (e0 + 32 <= wave_nmin) {  // wave-uniform: every row sees the tile
#pragma unroll
      for (int s = 0; s < kSets; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) rm[s][r] = vmax(acc[s][r] * sc, rm[s][r]);
    } else {
      const int lim = frontier_lim(e0 + rl);
#pragma unroll
      for (int s = 0; s < kSets; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[s][r] * sc;
          rm[s][r] = lim <= wrow_h(s, r) ? vmax(v, rm[s][r]) : rm[s][r];
        }
    }
  };
  // group g of the split = lane column rl over the 32 tiles of run `run`
  auto publish = [&](int run) {
    const int g = split * groups_per_split + run * 32 + rl;
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = row0 + wrow(s, r);
        if (t < T) {
          const uint16_t key16 =
              rm[s][r] == -__builtin_inff() ? (uint16_t)0 : (uint16_t)(score_key(rm[s][r]) >> 16);
          ws.gmax[(size_t)t * ws.G + g] = key16;
        }
        rm[s][r] = -__builtin_inff();
      }
  };
  // Tiles in order, each one's loads issued two tiles ahead; a run's maxima are published
  // after its last tile.
  constexpr int kRuns = n_stages / kRunStages;
  int run_done = 0;
  if (n_tiles > 0) {
    TileIn in0, in1;
    load_tile(0, in0);
    load_tile(1, in1);
    int tt = 0;
    for (; tt + 1 < n_tiles; tt += 2) {
      {
        f32x16 acc[kSets];
        mfma_tile(in0, acc);
        const float sc = in0.sc;
        load_tile(tt + 2, in0);
        take_max(tt, sc, acc);  // tt is even: a run (32 tiles) ends only at an odd tile
      }
      __builtin_amdgcn_sched_barrier(0);  // one tile's accumulators live at a time
      {
        f32x16 acc[kSets];
        mfma_tile(in1, acc);
        const float sc = in1.sc;
        load_tile(tt + 3, in1);
        take_max(tt + 1, sc, acc);
        if ((tt + 2) % 32 == 0) publish(run_done++);
      }
    }
    if (tt < n_tiles) {
      f32x16 acc[kSets];
      mfma_tile(in0, acc);
      take_max(tt, in0.sc, acc);
    }
  }
  // the run holding the wave's last tile, and the runs past every row of the wave (empty)
  for (; run_done < kRuns; ++run_done) publish(run_done);
}

// PASS 2: the candidates.  The same contraction over every entry, taken transposed (the
// expanded keys as the A operand, entries x queries): lane l of a wave holds, for its
// query row0 + 32 s + l % 32, 16 scores of the tile.  The A operand is read straight from
// memory, each lane its 32 code bytes (lane l takes half l / 32 of the codes of A row
// l % 32), and A rows are assigned entries permuted (entry 16 h + 4 g + i at A row
// 8 g + 4 h + i), so that accumulator 4 g + i of lane half h = l / 32 is entry
// 16 h + 4 g + i: each lane holds 16 consecutive entries.  With no stage in LDS the waves
// run without barriers, and the LDS holds only the record queues.  Hits (scores >= the
// row's threshold) are rare, about one score in 200, so a lane only tests the largest of
// its 16 scores per tile; a lane that may hold a hit puts its 16 scores in the wave's LDS
// queue as one record (position from the ballot), and once 64 records are queued each lane
// sorts out one.  Slots of a (row, split) list come from
constexpr int kRecBatch = 64;               // records drained at once (one per lane)
constexpr int kRecQueue = 2 * kRecBatch;    // a batch + one tile's worth
// Queue layout: group g (scores 4 g .. 4 g + 3) of record j at s_rec[wave][g][j], so a
// record is written with one address and four offsets, and the lanes of one access touch
// consecutive 16-byte slots.
__global__ __launch_bounds__(kGemmThreads, 2) void k_prefill_hits(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, int n_entries, int ratio, int64_t pos0, int T, PrefillWs ws) {
  __shared__ uint32_t s_rcnt[kGemmRows];     // candidates of each of the workgroup's rows
  __shared__ float s_th[kGemmRows];          // each row's threshold (+inf past T)
  __shared__ int s_nv[kGemmRows];            // entries each row sees
  __shared__ float4 s_rec[4][4][kRecQueue];
  __shared__ uint32_t s_rtag[4][kRecQueue];  // record's row | its first entry's offset in the split << 8
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wg_row0 = blockIdx.x * kGemmRows;
  const int row0 = wg_row0 + wave * kWaveRows;
  const int split = blockIdx.y;
  const int e_begin = split * kSplitEntries;
  const int e_end = min(e_begin + kSplitEntries, n_entries);
  const int rl = lane & 31, half = lane >> 5;
  const int wave_nmax = row0 < T ? visible(pos0 + min(row0 + kWaveRows - 1, T - 1), ratio, n_entries) : 0;
  // tiles of 32 entries that some row of the wave sees (wave-uniform)
  const int n_tiles = max(0, (min(e_end, wave_nmax) - e_begin + 31) / 32);
  static_assert(kGemmThreads == kGemmRows, "one row of the workgroup per thread");
  {
    const int t = wg_row0 + tid;
    s_rcnt[tid] = 0u;
    s_th[tid] = t < T ? ws.theta[t] : __builtin_inff();
    s_nv[tid] = t < T ? visible(pos0 + t, ratio, n_entries) : 0;
  }
  // B operands: query row0 + 32 s + rl, dims 64*half .. +63, and its threshold
  bf16x8 qb[kSets][8];
  float th[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    const int t = row0 + 32 * s + rl;
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + (size_t)min(t, T - 1) * kDIdx + 64 * half);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[s][kk] = __builtin_bit_cast(bf16x8, qp[kk]);
    th[s] = t < T ? ws.theta[t] : __builtin_inff();
  }
  __syncthreads();

  float4* rq = &s_rec[wave][0][0];
  uint32_t* rt = s_rtag[wave];
  uint32_t qn = 0;  // queued records (wave-uniform)
  // Lane j takes record j of the first n: its hits (visible entries only) go to its row's
  // next slots.
  auto drain = [&](uint32_t n) {
    const uint32_t j = (uint32_t)lane;
    if (j < n) {
      const uint32_t tag = rt[j];
      const int lr = (int)(tag & 255u);        // row within the workgroup
      const int eb = e_begin + (int)(tag >> 8);  // entry of the record's score 0
      const float thr = s_th[lr];
      const int nvr = s_nv[lr];
      float v[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 x = rq[g * kRecQueue + j];
        v[4 * g] = x.x;
        v[4 * g + 1] = x.y;
        v[4 * g + 2] = x.z;
        v[4 * g + 3] = x.w;
      }
      uint32_t hm = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) hm |= (v[r] >= thr ? 1u : 0u) << r;
      const int nvis = nvr - eb;  // visible entries among the record's 16
      if (nvis < 16) hm &= nvis > 0 ? (1u << nvis) - 1u : 0u;
      if (hm != 0u) {
        uint32_t slot = atomicAdd(&s_rcnt[lr], (uint32_t)__popc(hm));
        unsigned long long* out = ws.cand + ((size_t)(wg_row0 + lr) * ws.n_splits + split) * kSlots;
        const float* recf = reinterpret_cast<const float*>(rq + j);
        while (hm != 0u) {
          const int r = __builtin_ctz(hm);
          hm &= hm - 1u;
          // score r, read back from the record (no register indexing)
          const float vr = recf[(r >> 2) * (4 * kRecQueue) + (r & 3)];
          if (slot < (uint32_t)kSlots)
            out[slot] = ((unsigned long long)score_key(vr) << 32) | (uint32_t)(eb + r);
          ++slot;
        }
      }
    }
  };

  // Tile loads, two tiles ahead: lane (rl, half) takes code bytes 32 half .. + 31 of A row
  // rl, and lane q of each quad the scales of entries 16 half + 4 q .. + 3 (the group whose
  // A rows its quad's lanes hold as accumulators 4 q .. 4 q + 3).  Entries past the end
  // read as zeros.
  const __amdgpu_buffer_rsrc_t rs_code = buffer_over(codes, n_entries * kIdxCodeBytes);
  const __amdgpu_buffer_rsrc_t rs_scale = buffer_over(scale, n_entries * 4);
  const int a_off = (e_begin + row_entry(rl)) * kIdxCodeBytes + 32 * half;
  const int s_off = (e_begin + 16 * half + 4 * (lane & 3)) * 4;
  struct TileIn {
    uint4 c0, c1;
    float sc[4];
  };
  auto load_tile = [&](int tt, TileIn& in) {
    const int ct = min(tt, n_tiles - 1);  // past the last tile: a repeat, never used
    in.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_code, a_off + ct * 32 * kIdxCodeBytes, 0, 0));
    in.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_code, a_off + ct * 32 * kIdxCodeBytes + 16, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      in.sc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_scale, s_off + (ct * 32 + i) * 4, 0, 0));
  };
  // Software pipelined: the MFMAs of a tile are issued together with the branch-free part
  // of the screening of the tile before it (scaling, row maxima, ballots), interleaved so
  // that one wave keeps the matrix and vector units busy at once; the record writes, which
  // branch, follow.
  auto mfma_tile = [&](const TileIn& in, f32x16 (&acc)[kSets]) {
    const uint32_t cw[8] = {in.c0.x, in.c0.y, in.c0.z, in.c0.w, in.c1.x, in.c1.y, in.c1.z, in.c1.w};
#pragma unroll
    for (int s = 0; s < kSets; ++s) acc[s] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 ka = fp4x8_bf16(cw[kk]);
#pragma unroll
      for (int s = 0; s < kSets; ++s)
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s][kk], acc[s], 0, 0, 0);
    }
  };
  // this lane's 16 entries of a tile: 16 half .. + 15; the scores are scaled in place, every
  // lane taking group g's scales from lane g of its quad
  auto screen_math = [&](const float (&sc)[4], f32x16 (&acc)[kSets], uint64_t (&m)[kSets], bool (&cand)[kSets]) {
    float ow[kSets][4];
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
      ow[s][0] = sc[0], ow[s][1] = sc[1], ow[s][2] = sc[2], ow[s][3] = sc[3];
      // a copy per set, so that each broadcast has one use and becomes the DPP operand of
      // its multiply
      if (s > 0) asm("" : "+v"(ow[s][0]), "+v"(ow[s][1]), "+v"(ow[s][2]), "+v"(ow[s][3]));
    }
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[s][i] *= quad_bcast<0>(ow[s][i]);
        acc[s][4 + i] *= quad_bcast<1>(ow[s][i]);
        acc[s][8 + i] *= quad_bcast<2>(ow[s][i]);
        acc[s][12 + i] *= quad_bcast<3>(ow[s][i]);
      }
      const f32x16& v = acc[s];
      const float m0 = vmax3(v[0], v[1], v[2]), m1 = vmax3(v[3], v[4], v[5]), m2 = vmax3(v[6], v[7], v[8]);
      const float m3 = vmax3(v[9], v[10], v[11]), m4 = vmax3(v[12], v[13], v[14]);
      const float mx = vmax3(vmax3(m0, m1, m2), vmax3(m3, m4, v[15]), m0);
      cand[s] = mx >= th[s];
      m[s] = __ballot(cand[s]);
    }
  };
  auto screen_emit = [&](int tt, const f32x16 (&acc)[kSets], const uint64_t (&m)[kSets],
                         const bool (&cand)[kSets]) {
    const uint32_t tag_e = (uint32_t)(tt * 32 + 16 * half) << 8;
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
      if (m[s] != 0ull) {  // wave-uniform
        if (cand[s]) {
          const uint32_t j = qn + __builtin_amdgcn_mbcnt_hi((uint32_t)(m[s] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m[s], 0u));
          float4* p = rq + j;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            p[g * kRecQueue] = make_float4(acc[s][4 * g], acc[s][4 * g + 1], acc[s][4 * g + 2], acc[s][4 * g + 3]);
          rt[j] = (uint32_t)(wave * kWaveRows + 32 * s + rl) | tag_e;
        }
        qn += (uint32_t)__popcll(m[s]);
        if (qn >= (uint32_t)kRecBatch) {
          drain((uint32_t)kRecBatch);
          // the rest (fewer than a batch) to the front, after every read of the batch (the
          // wave's LDS operations complete in order)
          const uint32_t rest = qn - (uint32_t)kRecBatch;
          const uint32_t j = (uint32_t)lane;
          if (j < rest) {
            float4 x[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) x[g] = rq[g * kRecQueue + kRecBatch + j];
            const uint32_t tg = rt[kRecBatch + j];
#pragma unroll
            for (int g = 0; g < 4; ++g) rq[g * kRecQueue + j] = x[g];
            rt[j] = tg;
          }
          qn = rest;
        }
      }
    }
  };
  // one tile's MFMAs (16) with the screening arithmetic of the tile before it: the first A
  // conversions, then an MFMA every few vector instructions
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
#pragma unroll
    for (int i = 0; i < 2 * 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
  };
  if (n_tiles > 0) {
    f32x16 a0[kSets], a1[kSets];
    uint64_t m[kSets];
    bool cand[kSets];
    TileIn in0, in1;
    float sc0[4], sc1[4];
    load_tile(0, in0);
    load_tile(1, in1);
    mfma_tile(in0, a0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc0[i] = in0.sc[i];
    load_tile(2, in0);
    int tt = 1;
    for (; tt + 1 < n_tiles; tt += 2) {
      mfma_tile(in1, a1);
      screen_math(sc0, a0, m, cand);
      interleave();
#pragma unroll
      for (int i = 0; i < 4; ++i) sc1[i] = in1.sc[i];
      load_tile(tt + 2, in1);
      screen_emit(tt - 1, a0, m, cand);
      mfma_tile(in0, a0);
      screen_math(sc1, a1, m, cand);
      interleave();
#pragma unroll
      for (int i = 0; i < 4; ++i) sc0[i] = in0.sc[i];
      load_tile(tt + 3, in0);
      screen_emit(tt, a1, m, cand);
    }
    if (tt < n_tiles) {
      mfma_tile(in1, a1);
      screen_math(sc0, a0, m, cand);
      screen_emit(tt - 1, a0, m, cand);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc1[i] = in1.sc[i];
      screen_math(sc1, a1, m, cand);
      screen_emit(tt, a1, m, cand);
    } else {
      screen_math(sc0, a0, m, cand);
      screen_emit(tt - 1, a0, m, cand);
    }
  }
  drain(qn);
  __syncthreads();
  if (wg_row0 + tid < T) ws.ccount[(size_t)(wg_row0 + tid) * ws.n_splits + split] = s_rcnt[tid];
}

// ---------------------------------------------------------------------------- helpers
__device__ void find_bin_wave(const uint32_t* h, int nbins, uint32_t need, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    out[0] = 0u;
    out[1] = 0u;
  }
  const int per = nbins / 64;
  const int hi = nbins - lane * per;
  uint32_t sum = 0;
  for (int i = 1; i <= per; ++i) sum += h[hi - i];
  uint32_t incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  const uint32_t excl = incl - sum;
  if (excl < need && need <= incl) {
    uint32_t acc = excl;
    for (int i = 1; i <= per; ++i) {
      uint32_t c = h[hi - i];
      if (acc + c >= need) {
        out[0] = (uint32_t)(hi - i);
        out[1] = acc;
        break;
      }
      acc += c;
    }
  }
}

__device__ uint32_t block_scan_excl(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < nwaves; ++w) {
      uint32_t t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[16] = run;
  }
  __syncthreads();
  const uint32_t r = scratch[wave] + incl - v;
  *total = scratch[16];
  __syncthreads();
  return r;
}

// theta_t: +inf for a row that takes all its (at most k) visible entries; otherwise the
// kq-th largest of the row's group maxima (G_used of them), or -inf when the row has fewer
// than kq non-empty groups.  With groups over every entry and kq = k this is a rigorous
// lower bound on the row's k-th score; over a sample it is an estimate, which the select
// checks (it needs at least k candidates).
__global__ __launch_bounds__(kSelThreads) void k_prefill_theta(int n_entries, int ratio,
                                                               int64_t pos0, int T, int k, int kq,
                                                               PrefillWs ws) {
  // 256 bins, each spread over 16 copies (copy = lane % 16) so that the many lanes whose
  // maxima share a bin do not serialise on one LDS word
  __shared__ uint32_t s_hist[256 * 16];
  __shared__ uint32_t s_bin[256];
  __shared__ uint32_t s_res[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n_t = visible(pos0 + t, ratio, n_entries);
  if (n_t <= k) {  // the select takes every visible entry: no candidates
    if (tid == 0) ws.theta[t] = __builtin_inff();
    return;
  }
  // the row's G = 128 * n_splits maxima as 16-byte chunks; up to kRegChunks per thread stay
  // in registers, a longer row is read again from memory at each level
  constexpr int kRegChunks = 4;
  const uint4* g4 = reinterpret_cast<const uint4*>(ws.gmax + (size_t)t * ws.G);
  const int nch = ws.G_used / 8;
  const bool cached = nch <= kRegChunks * kSelThreads;
  uint4 w[kRegChunks];
#pragma unroll
  for (int j = 0; j < kRegChunks; ++j) {
    const int c = tid + j * kSelThreads;
    w[j] = cached && c < nch ? g4[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  auto count = [&](const uint4& v, int shift, int level, uint32_t prefix) {
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t m = (x[h >> 1] >> (16 * (h & 1))) & 0xffffu;
      if (m != 0u && (level == 0 || (m >> 8) == prefix))
        atomicAdd(&s_hist[((m >> shift) & 255u) * 16 + (lane & 15)], 1u);
    }
  };
  uint32_t need = (uint32_t)kq, prefix = 0;
  for (int level = 0; level < 2; ++level) {
    const int shift = 8 - 8 * level;
#pragma unroll
    for (int j = 0; j < 4; ++j) reinterpret_cast<uint4*>(s_hist)[tid + j * kSelThreads] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (cached) {
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j) count(w[j], shift, level, prefix);
    } else {
      for (int c = tid; c < nch; c += kSelThreads) count(g4[c], shift, level, prefix);
    }
    __syncthreads();
    {
      const uint4* hp = reinterpret_cast<const uint4*>(s_hist + tid * 16);
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = hp[i];
        b += v.x + v.y + v.z + v.w;
      }
      s_bin[tid] = b;
    }
    __syncthreads();
    if (tid < 64) {
      find_bin_wave(s_bin, 256, need, s_res);
      if (level == 0) {  // non-empty groups: the histogram's total
        uint32_t tot = s_bin[4 * lane] + s_bin[4 * lane + 1] + s_bin[4 * lane + 2] + s_bin[4 * lane + 3];
        tot = wave_incl_scan(tot);
        if (lane == 63) s_res[2] = tot;
      }
    }
    __syncthreads();
    if (level == 0 && s_res[2] < (uint32_t)kq) {  // fewer than kq non-empty groups
      if (tid == 0) ws.theta[t] = -__builtin_inff();
      return;
    }
    need -= s_res[1];
    prefix = level == 0 ? s_res[0] : (prefix << 8) | s_res[0];
    __syncthreads();
  }
  if (tid == 0) ws.theta[t] = key_score(prefix << 16);
}

// The same threshold for rows of at most kThetaWaveMax group maxima (the sampled pass's
// 1,024 per row): one wave per row, 16 maxima per lane in registers.  The kq-th largest
// 16-bit key is found bit by bit from the top, as the largest value that at least kq
// maxima reach; each count is one ballot and popcount per register, so the wave needs no
// LDS, atomics or barriers.  Rows and special cases as in k_prefill_theta.
constexpr int kThetaWaveMax = 1024;
constexpr int kThetaRowsPerBlock = 4;
__global__ __launch_bounds__(64 * kThetaRowsPerBlock) void k_prefill_theta_wave(
    int n_entries, int ratio, int64_t pos0, int T, int k, int kq, PrefillWs ws) {
  const int t = blockIdx.x * kThetaRowsPerBlock + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // wave-uniform
  if (visible(pos0 + t, ratio, n_entries) <= k) {  // the select takes every visible entry
    if (lane == 0) ws.theta[t] = __builtin_inff();
    return;
  }
  const uint4* g4 = reinterpret_cast<const uint4*>(ws.gmax + (size_t)t * ws.G);
  const int nch = ws.G_used / 8;  // 16-byte chunks of 8 maxima, at most 128
  const uint4 c0 = lane < nch ? g4[lane] : make_uint4(0u, 0u, 0u, 0u);
  const uint4 c1 = lane + 64 < nch ? g4[lane + 64] : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  uint32_t v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = w[i] & 0xffffu;
    v[2 * i + 1] = w[i] >> 16;
  }
  auto count_ge = [&](uint32_t c) {  // maxima of the row >= c (c >= 1 leaves out empty groups)
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) n += (uint32_t)__popcll(__ballot(v[i] >= c));
    return n;
  };
  if (count_ge(1u) < (uint32_t)kq) {  // fewer than kq non-empty groups
    if (lane == 0) ws.theta[t] = -__builtin_inff();
    return;
  }
  uint32_t th = 0;
  for (int b = 15; b >= 0; --b) {
    const uint32_t c = th | (1u << b);
    if (count_ge(c) >= (uint32_t)kq) th = c;
  }
  if (lane == 0) ws.theta[t] = key_score(th << 16);
}

// Score of entry j for a query held as 64 bf16 pairs (fp32, same rounding class as the
// MFMA path: exact products, fp32 sums).
__device__ __forceinline__ float score_row(const bf16x2 (&qq)[64], const uint8_t* codes, const float* scale,
                                           int j) {
  const uint4* cp = reinterpret_cast<const uint4*>(codes + (size_t)j * kIdxCodeBytes);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = cp[i];
    const uint32_t ws_[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int base = 16 * i + 4 * d;
      a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<0>(ws_[d]), qq[base + 0], a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<1>(ws_[d]), qq[base + 1], a1, false);
      a0 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<2>(ws_[d]), qq[base + 2], a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_bf16<3>(ws_[d]), qq[base + 3], a1, false);
    }
  }
  return (a0 + a1) * scale[j];
}

// A row whose candidates cannot give its top k (a split's slots overflowed, or a sampled
// threshold let through fewer than k): the whole workgroup recomputes the row's scores in a
// streaming exact selection (8-bit radix levels over (key, ~entry)) and writes the chosen
// entries in ascending order.  hist: 256 bins; res: 4 words; scan: 32 words.
__device__ __forceinline__ void recompute_row(const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
                                           const float* __restrict__ scale, int t, int n_t, uint32_t k_eff, int k,
                                           int32_t* orow, uint32_t* hist, uint32_t* s_res, uint32_t* s_scan) {
  const int tid = threadIdx.x;
  bf16x2 qq[64];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + (size_t)t * kDIdx);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 v = qp[i];
      qq[4 * i + 0] = __builtin_bit_cast(bf16x2, v.x);
      qq[4 * i + 1] = __builtin_bit_cast(bf16x2, v.y);
      qq[4 * i + 2] = __builtin_bit_cast(bf16x2, v.z);
      qq[4 * i + 3] = __builtin_bit_cast(bf16x2, v.w);
    }
  }
  uint32_t need = k_eff;
  unsigned long long prefix = 0ull, pmask = 0ull;
  for (int level = 0; level < 8 && need > 0; ++level) {
    const int shift = 56 - 8 * level;
    hist[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < n_t; j += kSelThreads) {
      const unsigned long long comp =
          ((unsigned long long)score_key(score_row(qq, codes, scale, j)) << 32) | (uint32_t)~(uint32_t)j;
      if ((comp & pmask) == prefix) atomicAdd(&hist[(comp >> shift) & 255ull], 1u);
    }
    __syncthreads();
    if (tid < 64) find_bin_wave(hist, 256, need, s_res);
    __syncthreads();
    need -= s_res[1];
    prefix |= (unsigned long long)s_res[0] << shift;
    pmask |= 255ull << shift;
    __syncthreads();
  }
  // composites are unique: select comp >= prefix (all 64 bits resolved) in entry order
  uint32_t written = 0;
  for (int c0 = 0; c0 < n_t; c0 += kSelThreads) {
    const int j = c0 + tid;
    bool take = false;
    if (j < n_t) {
      const unsigned long long comp =
          ((unsigned long long)score_key(score_row(qq, codes, scale, j)) << 32) | (uint32_t)~(uint32_t)j;
      take = k_eff > 0 && comp >= prefix;
    }
    uint32_t tot;
    const uint32_t p = block_scan_excl(take ? 1u : 0u, s_scan, &tot);
    if (take && written + p < (uint32_t)k) orow[written + p] = j;
    written += tot;
  }
  for (int i = (int)written + tid; i < k; i += kSelThreads) orow[i] = -1;
}

// Exact per-row top-k from the candidate slots (or, on overflow, from recomputed scores),
// ascending entry ids, -1 padded.
__global__ __launch_bounds__(kSelThreads) void k_prefill_select(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, int n_entries, int ratio, int64_t pos0, int T, int k,
    int32_t* __restrict__ idx_out, PrefillWs ws) {
  __shared__ unsigned long long s_cand[kCandLds];
  __shared__ uint32_t s_hist[3][256];  // radix levels cycle through three histograms
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_total, s_over;
  __shared__ uint32_t s_co[kSelMaxSplits];   // split's first candidate | its count << 16
  __shared__ uint32_t s_sel[kSelMaxSplits];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_t = visible(pos0 + t, ratio, n_entries);
  int32_t* orow = idx_out + (size_t)t * k;
  const uint32_t k_eff = (uint32_t)min(k, n_t);

  if (n_t <= k) {  // every visible entry is selected
    for (int i = tid; i < k; i += kSelThreads) orow[i] = i < n_t ? i : -1;
    return;
  }

  // ---- gather the row's candidates from its split slots (wave 0 counts and offsets them,
  // then each wave copies whole splits, one slot per lane)
  const int S = ws.n_splits;
  const uint32_t* cc = ws.ccount + (size_t)t * S;
  if (tid < 64) {
    const int lane = tid;
    uint32_t carry = 0, over = S > kSelMaxSplits ? 1u : 0u;
    for (int s0 = 0; s0 < S && !over; s0 += 64) {
      const int s = s0 + lane;
      const uint32_t c = s < S ? cc[s] : 0u;
      over |= __ballot(c > (uint32_t)kSlots) != 0ull ? 1u : 0u;
      const uint32_t n = min(c, (uint32_t)kSlots);
      uint32_t incl = n;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      if (s < S) {
        s_co[s] = (carry + incl - n) | (n << 16);  // offsets < 512 * 64
      }
      carry += __shfl(incl, 63);
    }
    if (lane == 0) {
      s_total = carry;
      // too many candidates for LDS, or (a sampled threshold) too few to hold the top k:
      // the row is recomputed
      s_over = over | (carry > (uint32_t)kCandLds ? 1u : 0u) | (carry < k_eff ? 1u : 0u);
    }
  }
  __syncthreads();
  const uint32_t C = s_total;
  if (!s_over) {
    // ---- fast path: exact selection among the candidates
    {
      const int wave = tid >> 6, lane = tid & 63;
      constexpr int kBatch = 8;  // splits per wave with loads in flight together
      for (int s0 = wave; s0 < S; s0 += kBatch * (kSelThreads / 64)) {
        unsigned long long v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int s = s0 + j * (kSelThreads / 64);
          const bool have = s < S && lane < (int)(s_co[min(s, S - 1)] >> 16);
          v[j] = have ? ws.cand[((size_t)t * S + s) * kSlots + lane] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int s = s0 + j * (kSelThreads / 64);
          if (s < S && lane < (int)(s_co[s] >> 16)) s_cand[(s_co[s] & 0xffffu) + lane] = v[j];
        }
      }
    }
    s_hist[0][tid] = 0u;
    __syncthreads();
    // composite: key (32 bits) then ~entry (a lower entry ranks higher); 8 digits of 8 bits.
    // Radix levels find the threshold composite: the row takes every candidate >= prefix
    // (lower digits zero once a level's bin is taken whole).  Level L counts into histogram
    // L % 3 while clearing histogram (L + 1) % 3, and every wave finds the level's bin
    // itself, so a level costs one barrier.
    uint32_t need = k_eff;
    unsigned long long prefix = 0ull, pmask = 0ull;
    uint32_t remaining = C;
    const int lane = tid & 63;
    for (int level = 0; level < 8 && need > 0 && need < remaining; ++level) {
      const int shift = 56 - 8 * level;
      uint32_t* h = s_hist[level % 3];
      s_hist[(level + 1) % 3][tid] = 0u;
      for (uint32_t i = tid; i < C; i += kSelThreads) {
        const unsigned long long v = s_cand[i];
        const unsigned long long comp = (v & 0xffffffff00000000ull) | (uint32_t)~(uint32_t)v;
        if ((comp & pmask) == prefix) atomicAdd(&h[(comp >> shift) & 255ull], 1u);
      }
      __syncthreads();
      // the bin holding the need-th largest: lane l sums bins 255-4l .. 252-4l
      const uint4 hv = reinterpret_cast<const uint4*>(h)[63 - lane];  // bins 252-4l .. 255-4l
      const uint32_t c3 = hv.w, c2 = hv.z, c1 = hv.y, c0 = hv.x;
      const uint32_t sum = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
      const uint64_t hitm = __ballot(excl < need && need <= incl);
      const int src = __builtin_amdgcn_readfirstlane(max(__builtin_ffsll((long long)hitm) - 1, 0));
      uint32_t sel, above;
      {
        uint32_t a = excl, b = 252u - 4u * (uint32_t)lane + 3u, r = c3;
        if (a + c3 < need) { a += c3; b -= 1; r = c2;
          if (a + c2 < need) { a += c2; b -= 1; r = c1;
            if (a + c1 < need) { a += c1; b -= 1; r = c0; } } }
        sel = (uint32_t)__builtin_amdgcn_readlane((int)b, src);
        above = (uint32_t)__builtin_amdgcn_readlane((int)a, src);
        remaining = (uint32_t)__builtin_amdgcn_readlane((int)r, src);
      }
      need -= above;
      prefix |= (unsigned long long)sel << shift;
      pmask |= 255ull << shift;
    }
    // ---- the selected candidates in ascending entry order: splits hold ascending entry
    // ranges, so each wave places one split's selected slots after the selected entries of
    // the splits before it, each at its rank by entry within the split
    {
      const int wave = tid >> 6, lane = tid & 63;
      auto take = [&](int sp, uint32_t* e) {
        const uint32_t co = s_co[sp];
        const bool have = lane < (int)(co >> 16);
        const unsigned long long v = have ? s_cand[(co & 0xffffu) + lane] : 0ull;
        const unsigned long long comp = (v & 0xffffffff00000000ull) | (uint32_t)~(uint32_t)v;
        *e = (uint32_t)v;
        return have && comp >= prefix;
      };
      for (int sp = wave; sp < S; sp += kSelThreads / 64) {
        uint32_t e;
        const unsigned long long m = __ballot(take(sp, &e));
        if (lane == 0) s_sel[sp] = (uint32_t)__popcll(m);
      }
      __syncthreads();
      if (tid < 64) scan_counts_wave0_n<kSelMaxSplits / 64>(s_sel, S);
      __syncthreads();
      for (int sp = wave; sp < S; sp += kSelThreads / 64) {
        uint32_t e;
        const bool tk = take(sp, &e);
        const unsigned long long m = __ballot(tk);
        // the split's slots are normally in entry order already; otherwise each taken entry
        // is ranked among the taken lanes, bit by bit from the top of its 12-bit offset
        // (lanes that agree on the higher bits and have a 0 where this lane has a 1 are
        // below it), and moved to the lane of its rank so the stores go out in order
        const uint32_t prev = (uint32_t)__shfl_up((int)e, 1);
        const uint32_t nval = s_co[sp] >> 16;
        const bool sorted = __ballot(lane >= 1 && (uint32_t)lane < nval && prev >= e) == 0ull;
        if (sorted) {
          const uint32_t at = s_sel[sp] + lanes_below(m);
          if (tk && at < (uint32_t)k) orow[at] = (int32_t)e;
        } else {
          const uint32_t off = e - (uint32_t)(sp * kSplitEntries);
          uint32_t rank = 0;
          unsigned long long same = m;
#pragma unroll
          for (int b = 11; b >= 0; --b) {
            const bool one = (off >> b) & 1u;
            const unsigned long long ones = __ballot(one) & m;
            if (one) rank += (uint32_t)__popcll(same & ~ones);
            same &= one ? ones : ~ones;
          }
          const uint32_t cnt = (uint32_t)__popcll(m);
          const uint32_t dest = tk ? rank : cnt + lanes_below(~m);
          const uint32_t ev = (uint32_t)__builtin_amdgcn_ds_permute((int)(dest * 4u), (int)e);
          const uint32_t at = s_sel[sp] + (uint32_t)lane;
          if ((uint32_t)lane < cnt && at < (uint32_t)k) orow[at] = (int32_t)ev;
        }
      }
      for (int i = (int)k_eff + tid; i < k; i += kSelThreads) orow[i] = -1;
    }
    return;
  }

  recompute_row(q_idx, codes, scale, t, n_t, k_eff, k, orow, s_hist[0], s_res, s_scan);
}

// ---- rows of chunks with at most kRowSplits splits: one wave per row, its candidates in
// registers (slot `lane` of split u in key[u], ent[u]; key 0 = empty slot, a score's key
// is never 0), so that a row needs no workgroup barrier and every row of a 4,096-query
// chunk is resident at once.
constexpr int kRowSplits = 32;
constexpr int kSelRowsPerBlock = kSelThreads / 64;

__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, bool is_max) {
  // DPP row shifts, then row broadcasts; lane 63 ends with the result
  const int id = is_max ? 0 : -1;
  int x = (int)v;
  auto op = [&](int a, int b) { return is_max ? (int)max((unsigned)a, (unsigned)b) : (int)min((unsigned)a, (unsigned)b); };
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Bin of the need-th largest count of the wave's 256-bin histogram h (lane l holds bins
// 255 - 4 l .. 252 - 4 l); *above = elements in higher bins, *in_bin = the bin's count.
__device__ __forceinline__ uint32_t wave_find_bin(const uint32_t* h, uint32_t need, uint32_t* above,
                                                  uint32_t* in_bin) {
  const int lane = threadIdx.x & 63;
  const uint4 hv = reinterpret_cast<const uint4*>(h)[63 - lane];
  const uint32_t c3 = hv.w, c2 = hv.z, c1 = hv.y, c0 = hv.x;
  const uint32_t sum = c0 + c1 + c2 + c3;
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t excl = incl - sum;
  const uint64_t hitm = __ballot(excl < need && need <= incl);
  const int src = __builtin_amdgcn_readfirstlane(max(__builtin_ffsll((long long)hitm) - 1, 0));
  uint32_t a = excl, b = 252u - 4u * (uint32_t)lane + 3u, r = c3;
  if (a + c3 < need) { a += c3; b -= 1; r = c2;
    if (a + c2 < need) { a += c2; b -= 1; r = c1;
      if (a + c1 < need) { a += c1; b -= 1; r = c0; } } }
  *above = (uint32_t)__builtin_amdgcn_readlane((int)a, src);
  *in_bin = (uint32_t)__builtin_amdgcn_readlane((int)r, src);
  return (uint32_t)__builtin_amdgcn_readlane((int)b, src);
}

// One wave: row t's top k_eff (largest scores, ties to the lower entry) among its candidates,
// written in ascending entry order.  Radix levels of 8 bits over the key bits below those
// that every candidate shares, then, for keys equal to the threshold key, over the entry.
// Returns true when the candidates cannot give the top k (a split overflowed its slots, or
// fewer than k) or a split's slots are out of entry order: the row is then recomputed.
__device__ __forceinline__ bool select_row_wave(int t, uint32_t k_eff, int k, int32_t* orow,
                                                const PrefillWs& ws, uint32_t* h) {
  const int lane = threadIdx.x & 63;
  const int S = ws.n_splits;
  const uint32_t c = lane < S ? ws.ccount[(size_t)t * S + lane] : 0u;
  if (__ballot(c > (uint32_t)kSlots) != 0ull) return true;
  const uint32_t C = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(c), 63);
  if (C < k_eff) return true;
  uint32_t key[kRowSplits], ent[kRowSplits];
  const unsigned long long* cp = ws.cand + (size_t)t * S * kSlots + lane;
#pragma unroll
  for (int u = 0; u < kRowSplits; ++u) {
    const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)c, u);  // 0 for u >= S
    const unsigned long long v = (uint32_t)lane < n ? cp[(size_t)u * kSlots] : 0ull;
    key[u] = (uint32_t)(v >> 32);
    ent[u] = (uint32_t)v;
  }
  // take: key != 0 && (key > tkey || (key == tkey && ent <= tent))
  uint32_t tkey = 0u, tent = 0xffffffffu;
  uint32_t need = k_eff, remaining = C;
  if (need < remaining) {
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int u = 0; u < kRowSplits; ++u) {
      mx = max(mx, key[u]);
      mn = min(mn, key[u] != 0u ? key[u] : 0xffffffffu);
    }
    mn = wave_reduce_u32(mn, false);
    mx = wave_reduce_u32(mx, true);
    // key bits [lo, 32) are fixed (pfx = key >> lo); every candidate shares those above the
    // highest bit where the smallest and largest keys differ
    const uint32_t d = mn ^ mx;
    int lo = d != 0u ? 32 - __builtin_clz(d) : 0;
    uint32_t pfx = lo < 32 ? mn >> lo : 0u;
    bool first = true;
    while (need < remaining && lo > 0) {
      const int nlo = max(lo - 8, 0);
      const uint32_t dmask = (1u << (lo - nlo)) - 1u;
      reinterpret_cast<uint4*>(h)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < kRowSplits; ++u)
        if (key[u] != 0u && (first || (key[u] >> lo) == pfx)) atomicAdd(&h[(key[u] >> nlo) & dmask], 1u);
      uint32_t above, in_bin;
      const uint32_t sel = wave_find_bin(h, need, &above, &in_bin);
      need -= above;
      remaining = in_bin;
      pfx = (pfx << (lo - nlo)) | sel;
      lo = nlo;
      first = false;
    }
    if (need == remaining) {
      tkey = pfx << lo;  // every key with this prefix or above
    } else {
      // `remaining` candidates hold the threshold key pfx; the `need` of them with the lowest
      // entries: levels over the entry, digit 255 - (entry bits) so the largest bin is lowest
      tkey = pfx;
      uint32_t epfx = 0u;
      int elo = 32;
      while (need < remaining && elo > 0) {
        const int nlo = elo - 8;
        reinterpret_cast<uint4*>(h)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < kRowSplits; ++u)
          if (key[u] == tkey && (elo == 32 || (ent[u] >> elo) == epfx))
            atomicAdd(&h[255u - ((ent[u] >> nlo) & 255u)], 1u);
        uint32_t above, in_bin;
        const uint32_t sel = 255u - wave_find_bin(h, need, &above, &in_bin);
        need -= above;
        remaining = in_bin;
        epfx = (epfx << 8) | sel;
        elo = nlo;
      }
      // every entry whose prefix is at or below epfx
      tent = elo > 0 ? (epfx << elo) | ((1u << elo) - 1u) : epfx;
    }
  }
  // the chosen entries in ascending order: splits hold ascending entry ranges and a split's
  // slots are in entry order when the slot counter served its lanes in order (a split
  // found out of order hands the row back)
  uint32_t base = 0u;
#pragma unroll
  for (int u = 0; u < kRowSplits; ++u) {
    const bool tk = key[u] != 0u && (key[u] > tkey || (key[u] == tkey && ent[u] <= tent));
    const unsigned long long m = __ballot(tk);
    if (m != 0ull) {  // uniform
      const uint32_t e = ent[u];
      const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x138, 0xf, 0xf, false);  // wave_shr:1
      // the split's filled slots are lanes 0 .. its count - 1 (the non-zero keys)
      if (__ballot(lane >= 1 && key[u] != 0u && prev >= e) != 0ull) return true;
      const uint32_t at = base + lanes_below(m);
      if (tk && at < (uint32_t)k) orow[at] = (int32_t)e;
      base += (uint32_t)__popcll(m);
    }
  }
  for (int i = (int)k_eff + lane; i < k; i += 64) orow[i] = -1;
  return false;
}

// Grid: ceil(T / 4) workgroups of 4 waves, wave w selecting row 4 b + w; rows the waves
// hand back are recomputed by the whole workgroup afterwards.
__global__ __launch_bounds__(kSelThreads) void k_prefill_select_rows(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, int n_entries, int ratio, int64_t pos0, int T, int k,
    int32_t* __restrict__ idx_out, PrefillWs ws) {
  __shared__ uint4 s_wh[kSelRowsPerBlock][64];  // each wave's 256-bin histogram
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_redo[kSelRowsPerBlock];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kSelRowsPerBlock + wave;
  bool redo = false;
  if (t < T) {
    const int n_t = visible(pos0 + t, ratio, n_entries);
    int32_t* orow = idx_out + (size_t)t * k;
    if (n_t <= k) {  // every visible entry is selected
      for (int i = lane; i < k; i += 64) orow[i] = i < n_t ? i : -1;
    } else {
      redo = select_row_wave(t, (uint32_t)k, k, orow, ws, reinterpret_cast<uint32_t*>(s_wh[wave]));
    }
  }
  if (lane == 0) s_redo[wave] = redo ? 1u : 0u;
  __syncthreads();
  for (int w = 0; w < kSelRowsPerBlock; ++w) {
    if (s_redo[w] == 0u) continue;  // uniform
    const int tr = blockIdx.x * kSelRowsPerBlock + w;
    const int n_t = visible(pos0 + tr, ratio, n_entries);
    recompute_row(q_idx, codes, scale, tr, n_t, (uint32_t)min(k, n_t), k, idx_out + (size_t)tr * k, s_hist,
                  s_res, s_scan);
    __syncthreads();
  }
}

// ------------------------------------------------------------ causal score matrix
// The same contraction written out: S[t][j] = scale_j * (q_t . e2m1(K_j)) for the entries j
// that position pos0 + t sees, each row's visible count and, if asked, min(visible,
// pool_k).  For a replay chunk, whose queries each keep a pool far larger than the prefill
// slots hold: the keys are read once for all the queries and the selection runs on the
// matrix.  Layout: blocked, S[j / 1024][t][j % 1024] (each workgroup writes one contiguous
// block; columns a row does not see hold scores of no meaning), or row-major, S[t][j]
// (columns a row does not see are left unwritten).  A workgroup owns 128 query rows (a
// wave per 32) and one split of kScoreSplit entries streamed through LDS as in
// k_prefill_gmax.  The product is taken transposed, entries x queries (the expanded keys
// as the A operand), so that a lane's accumulators hold one query's scores for four runs
// of four consecutive entries: 16-byte stores.
constexpr int kScoreRows = 128;
constexpr int kScoreSplit = 1024;
static_assert(kScoreSplit == 1024, "a split is one block of the blocked layout");
template <bool BLOCKED>
__global__ __launch_bounds__(kGemmThreads, 2) void k_causal_scores(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, int n_entries, int ratio, int64_t pos0, int T,
    float* __restrict__ S, int32_t* __restrict__ n_vis, int pool_k, int32_t* __restrict__ pool_n) {
  __shared__ uint4 s_code[2][kStage * 4];
  __shared__ float4 s_sc[2][kStage / 4];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wg_row0 = blockIdx.x * kScoreRows;
  const int row0 = wg_row0 + wave * 32;
  const int rl = lane & 31, half = lane >> 5;
  if (blockIdx.y == 0 && tid < kScoreRows && wg_row0 + tid < T) {
    const int v = visible(pos0 + wg_row0 + tid, ratio, n_entries);
    n_vis[wg_row0 + tid] = v;
    if (pool_n) pool_n[wg_row0 + tid] = min(v, pool_k);
  }
  const int e_begin = blockIdx.y * kScoreSplit;
  const int e_end = min(e_begin + kScoreSplit, n_entries);
  const int wg_nmax = visible(pos0 + min(wg_row0 + kScoreRows - 1, T - 1), ratio, n_entries);
  const int wave_nmax = row0 < T ? visible(pos0 + min(row0 + 31, T - 1), ratio, n_entries) : 0;
  const int e_stop = min(e_end, wg_nmax);
  const int n_active = e_stop > e_begin ? (e_stop - e_begin + kStage - 1) / kStage : 0;
  if (n_active == 0) return;  // workgroup-uniform: before any barrier

  // B operand: the lane's query t = row0 + rl, dims 64*half + 8kk .. +7 (the k-slice of lane
  // half `half`, as the keys' A operand below)
  const int t = row0 + rl;
  bf16x8 qb[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q_idx + (size_t)min(t, T - 1) * kDIdx + 64 * half);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qb[kk] = __builtin_bit_cast(bf16x8, qp[kk]);
  }
  const int nv = t < T ? visible(pos0 + t, ratio, n_entries) : 0;
  float* srow = S + (BLOCKED ? ((size_t)blockIdx.y * (size_t)T + (size_t)min(t, T - 1)) * kScoreSplit - (size_t)e_begin
                             : (size_t)min(t, T - 1) * (size_t)n_entries);

  uint4 pc0 = make_uint4(0u, 0u, 0u, 0u), pc1 = pc0, pc2 = pc0, pc3 = pc0;
  float psc = 0.f;
  auto load_stage = [&](int st) {
    const int e = min(e_begin + st * kStage + tid, n_entries - 1);
    const uint4* cp = reinterpret_cast<const uint4*>(codes + (size_t)e * kIdxCodeBytes);
    pc0 = cp[0];
    pc1 = cp[1];
    pc2 = cp[2];
    pc3 = cp[3];
    psc = scale[e];
  };
  load_stage(0);
  for (int st = 0; st < n_active; ++st) {
    const int buf = st & 1;
    s_code[buf][stage_blk(tid, 0)] = pc0;
    s_code[buf][stage_blk(tid, 1)] = pc1;
    s_code[buf][stage_blk(tid, 2)] = pc2;
    s_code[buf][stage_blk(tid, 3)] = pc3;
    reinterpret_cast<float*>(s_sc[buf])[tid] = psc;
    __syncthreads();
    if (st + 1 < n_active) load_stage(st + 1);  // in flight during the MFMAs
    const int st_e0 = e_begin + st * kStage;
    for (int tt = 0; tt < kStage / 32; ++tt) {
      const int e0 = st_e0 + tt * 32;
      if (e0 >= wave_nmax) break;  // wave-uniform: the rest is beyond every row of the wave
      const int i = tt * 32 + rl;  // A operand: entry e0 + rl
      const uint4 c0 = s_code[buf][stage_blk(i, 2 * half)];
      const uint4 c1 = s_code[buf][stage_blk(i, 2 * half + 1)];
      const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp4x8_bf16(cw[kk]), qb[kk], acc, 0, 0, 0);
      // accumulator 4g + i: entry e0 + 8g + 4*half + i of query t
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sc = s_sc[buf][tt * 8 + 2 * g + half];
        const int col = e0 + 8 * g + 4 * half;
        f32x4 v;
        v[0] = acc[4 * g] * sc.x;
        v[1] = acc[4 * g + 1] * sc.y;
        v[2] = acc[4 * g + 2] * sc.z;
        v[3] = acc[4 * g + 3] * sc.w;
        if (BLOCKED) {
          if (t < T) *reinterpret_cast<f32x4*>(srow + col) = v;
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (col + x < nv) srow[col + x] = v[x];
        }
      }
    }
  }
}

hipError_t launch_causal_scores(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                                int n_entries, int ratio, int64_t pos0, int T, bool blocked,
                                float* scores, int32_t* n_vis, int pool_k, int32_t* pool_n,
                                hipStream_t stream) {
  // at least one split, so that the visible counts are written when nothing is visible
  const dim3 grid((unsigned)((T + kScoreRows - 1) / kScoreRows),
                  (unsigned)(n_entries > 0 ? (n_entries + kScoreSplit - 1) / kScoreSplit : 1));
  if (blocked)
    hipLaunchKernelGGL(k_causal_scores<true>, grid, dim3(kGemmThreads), 0, stream, q_idx, idx_codes,
                       idx_scale, n_entries, ratio, pos0, T, scores, n_vis, pool_k, pool_n);
  else
    hipLaunchKernelGGL(k_causal_scores<false>, grid, dim3(kGemmThreads), 0, stream, q_idx, idx_codes,
                       idx_scale, n_entries, ratio, pos0, T, scores, n_vis, pool_k, pool_n);
  return hipGetLastError();
}

hipError_t launch_prefill_select(const uint16_t* q_idx, const uint8_t* idx_codes,
                                 const float* idx_scale, int n_entries, int ratio, int64_t pos0,
                                 int T, int k, int32_t* idx_out, void* ws_base, hipStream_t stream) {
  PrefillWs ws = prefill_ws_carve(ws_base, T, n_entries);
  const int row_blocks = (T + kGemmRows - 1) / kGemmRows;
  // Threshold: from a 1-in-kSampleStride sample of the entries when every row sees enough of
  // them for the estimate to be sharp (the kq-th of ~n/128 sample group maxima, kq = 3k/8,
  // aims at about 1.5 k candidates per row), else the rigorous bound from every entry.
  const int kq = (3 * k + 7) / 8;
  const bool sampled = kq >= kSampleMinQ && n_entries > 0 &&
                       (int64_t)visible_host(pos0, ratio, n_entries) >= (int64_t)kSampleMinGroupsPerQ * kq * 32 * kSampleStride;
  if (sampled) {
    // a quarter of the columns: quarter-size splits keep the grid as wide as pass 2's
    constexpr int split = kSplitEntries / kSampleStride;
    const int n_cols = (n_entries + kSampleStride - 1) / kSampleStride;
    const int splits = (n_cols + split - 1) / split;
    ws.G_used = splits * (split / (kRunStages * kStage) * 32);
    hipLaunchKernelGGL((k_prefill_gmax<kSampleStride, split>), dim3(row_blocks, splits),
                       dim3(kGemmThreads), 0, stream, q_idx, idx_codes, idx_scale, n_entries, ratio,
                       pos0, T, ws);
  } else if (n_entries > 0) {
    hipLaunchKernelGGL((k_prefill_gmax<1, kSplitEntries>), dim3(row_blocks, ws.n_splits),
                       dim3(kGemmThreads), 0, stream, q_idx, idx_codes, idx_scale, n_entries, ratio,
                       pos0, T, ws);
  }
  if (ws.G_used <= kThetaWaveMax)
    hipLaunchKernelGGL(k_prefill_theta_wave, dim3((T + kThetaRowsPerBlock - 1) / kThetaRowsPerBlock),
                       dim3(64 * kThetaRowsPerBlock), 0, stream, n_entries, ratio, pos0, T, k,
                       sampled ? kq : k, ws);
  else
    hipLaunchKernelGGL(k_prefill_theta, dim3(T), dim3(kSelThreads), 0, stream, n_entries, ratio, pos0,
                       T, k, sampled ? kq : k, ws);
  if (n_entries > 0) {
    hipLaunchKernelGGL(k_prefill_hits, dim3(row_blocks, ws.n_splits),
                       dim3(kGemmThreads), 0, stream, q_idx, idx_codes, idx_scale, n_entries, ratio,
                       pos0, T, ws);
  }
  if (ws.n_splits <= kRowSplits)
    hipLaunchKernelGGL(k_prefill_select_rows, dim3((T + kSelRowsPerBlock - 1) / kSelRowsPerBlock),
                       dim3(kSelThreads), 0, stream, q_idx, idx_codes, idx_scale, n_entries, ratio, pos0,
                       T, k, idx_out, ws);
  else
    hipLaunchKernelGGL(k_prefill_select, dim3(T), dim3(kSelThreads), 0, stream, q_idx, idx_codes,
                       idx_scale, n_entries, ratio, pos0, T, k, idx_out, ws);
  return hipGetLastError();
}

hipError_t launch_prefill(const uint16_t* q_idx, const uint16_t* q, const uint8_t* idx_codes,
                          const float* idx_scale, const uint8_t* kv_codes, const uint8_t* kv_scale,
                          int n_entries, int ratio, int64_t pos0, int T, int k, const uint8_t* swa,
                          float softmax_scale, int32_t* idx_out, float* out, void* ws_base,
                          hipStream_t stream) {
  const hipError_t e = launch_prefill_select(q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, T, k,
                                             idx_out, ws_base, stream);
  if (e != hipSuccess) return e;
  const PrefillWs ws = prefill_ws_carve(ws_base, T, n_entries);
  return launch_attn(1, q, kv_codes, kv_scale, nullptr, idx_out, k, swa, nullptr, pos0, softmax_scale,
                     T, out, ws.attn, stream);
}

}  // namespace csa2
