// a2 top-k selection: the k largest scores of a row, ties to the lower column, written
// in ascending column order as entry ids (cand[c] or c), -1 padded.
//
// Used for the decoder pool (k = 16,384 of up to 2^20 columns) and for every top-512
// ("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", commentary on the four
// layer modes; "从V4到V4.1 Flash：架构的激进进化", decoder section on the hierarchical
// indexer).  The tie rule is this library's reading; the pages do not state one.
//
// Scores map to order-preserving u32 keys (key 0 marks an unusable column).  The
// selection is exact for the 64-bit composite (key << 32 | ~column), which is unique per
// column, so the k-th composite T is unique and the selected set is {column : comp >= T}.
// T is found digit by digit: a 12-bit level-1 histogram of the keys (bits 31..20; fused
// into the scan, or built here), an 11-bit level-2 histogram (bits 19..9) of the columns
// in the level-1 bin, then the few columns left in the level-2 bin are ranked directly;
// only massive ties fall back to radix passes over the remaining 41 composite bits.
//
// Short rows (<= 16,384 columns): k_topk_row, one 1024-thread workgroup per row, 16 keys
// per thread held in registers, every level in LDS, ballot compaction in column order.
//
// Long rows: four launches, none touching the scores more than once:
//   k_topk_bin      one workgroup per row: the level-1 bin b1 of the k-th key;
//   k_topk_filter   many workgroups per row (2,048 columns each): counts its columns above
//                   b1 and writes its columns inside b1 to its own candidate slots;
//   k_topk_resolve  one workgroup per row: level-2 histogram of the candidates, the exact
//                   k-th composite T, each chunk's output offset; it returns the level-1
//                   histogram to zero;
//   k_topk_compact  many workgroups per row: columns with comp >= T in column order at
//                   their chunk's offset (wave ballots, one LDS scan).
// No host round trip and no global atomics beyond the fused histogram.
#include "csa2_internal.h"
#include "select_device.h"

namespace csa2 {

constexpr int kBigThreads = 1024;
constexpr int kHistThreads = 256;
constexpr int kLongThreads = 256;                         // filter / compact (4 waves)
constexpr int kRowIters = kTopkSmallMax / kBigThreads;    // keys per thread in k_topk_row
constexpr int kTiedCap = 1024;                            // tied columns ranked in LDS

int topk_chunk_iters(int n_cols) { return n_cols <= (1 << 24) ? 8 : 32; }
int topk_n_chunks(int n_cols) {
  const int cc = kLongThreads * topk_chunk_iters(n_cols);
  return (n_cols + cc - 1) / cc;
}

size_t topk_ws_bytes(int batch, int n_cols) {
  const size_t chunks = (size_t)topk_n_chunks(n_cols);
  size_t s = 0;
  s += align_up((size_t)batch * kHist1Bins * 4, 256);
  s += align_up((size_t)batch * kRowInfo * 4, 256);
  s += align_up((size_t)batch * 8, 256);
  s += 3 * align_up((size_t)batch * chunks * 4, 256);
  s += 2 * align_up((size_t)batch * n_cols * 8, 256);
  return s;
}

TopkWs topk_ws_carve(void* base, int batch, int n_cols) {
  TopkWs w;
  char* p = static_cast<char*>(base);
  w.n_chunks = topk_n_chunks(n_cols);
  w.hist1 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist1Bins * 4, 256);
  w.counters = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kRowInfo * 4, 256);
  w.thr = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)batch * 8, 256);
  w.chunk_cnt = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * w.n_chunks * 4, 256);
  w.chunk_ccnt = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * w.n_chunks * 4, 256);
  w.chunk_off = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * w.n_chunks * 4, 256);
  w.list = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)batch * n_cols * 8, 256);
  w.tied = reinterpret_cast<unsigned long long*>(p);
  return w;
}

// ---------------------------------------------------------------------------- helpers
// Key of column col of a row, 0 when the column is not selectable.
__device__ __forceinline__ uint32_t col_key(const float* srow, const int32_t* crow, int nv, int col) {
  if (col >= nv) return 0u;
  if (crow && crow[col] < 0) return 0u;
  return score_key(srow[col]);
}

// Keys (0 = not selectable) and entry ids of the N columns col0 + i*step of a row.  Every
// load reads a column clamped to nv - 1, so all of them are issued back to back with no
// branch between them; out-of-range columns are masked afterwards.
template <int N>
__device__ __forceinline__ void load_keys(const float* srow, const int32_t* crow, int nv, int col0,
                                          int step, uint32_t (&key)[N], int32_t (&id)[N]) {
  const int lim = nv > 0 ? nv - 1 : 0;  // column 0 always exists (rows are never empty)
  float s[N];
  if (crow) {
#pragma unroll
    for (int i = 0; i < N; ++i) id[i] = crow[min(col0 + i * step, lim)];
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) id[i] = col0 + i * step;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) s[i] = srow[min(col0 + i * step, lim)];
#pragma unroll
  for (int i = 0; i < N; ++i)
    key[i] = (col0 + i * step < nv && id[i] >= 0) ? score_key(s[i]) : 0u;
}

__device__ __forceinline__ uint32_t digit2(uint32_t key) { return (key >> 9) & (kHist2Bins - 1); }

// Radix passes over the 41 composite bits below the 23 key bits fixed by the level-1 and
// level-2 bins: `visit(f)` calls f(composite) for every candidate still in play.  Returns
// the need-th largest composite.  Whole workgroup; s_h holds >= 512 bins.
template <typename Visit>
__device__ unsigned long long radix_tail(uint32_t b1, uint32_t b2, uint32_t need, uint32_t* s_h,
                                         uint32_t* s_res, Visit visit) {
  unsigned long long prefix = ((unsigned long long)((b1 << 11) | b2)) << 41;
  unsigned long long pmask = ~((1ull << 41) - 1ull);
  const int shifts[5] = {32, 24, 16, 8, 0};
  const int widths[5] = {9, 8, 8, 8, 8};
  for (int lvl = 0; lvl < 5; ++lvl) {
    const int shift = shifts[lvl], nb = 1 << widths[lvl];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) s_h[i] = 0u;
    __syncthreads();
    visit([&](unsigned long long c) {
      if ((c & pmask) == prefix) atomicAdd(&s_h[(c >> shift) & (unsigned long long)(nb - 1)], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) find_threshold_bin(s_h, nb, need, s_res);
    __syncthreads();
    need -= s_res[1];
    prefix |= (unsigned long long)s_res[0] << shift;
    pmask |= (unsigned long long)(nb - 1) << shift;
    __syncthreads();
  }
  return prefix;
}

// Rank of the tied composites in s_tied[0..nt): the one with exactly need-1 larger ones.
__device__ void rank_tied(const unsigned long long* s_tied, uint32_t nt, uint32_t need,
                          unsigned long long* s_T) {
  for (uint32_t i = threadIdx.x; i < nt; i += blockDim.x) {
    const unsigned long long c = s_tied[i];
    uint32_t r = 0;
    for (uint32_t j = 0; j < nt; ++j) r += s_tied[j] > c ? 1u : 0u;
    if (r == need - 1u) *s_T = c;
  }
}

// ---------------------------------------------------------------------------- short rows
// FUSED: the row's level-1 histogram is in hist1 (accumulated by the scan); it is returned
// to zero here.  Otherwise it is built in LDS.
template <bool FUSED>
__global__ __launch_bounds__(kBigThreads) void k_topk_row(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, uint32_t* __restrict__ hist1) {
  __shared__ uint32_t s_h[kHist1Bins];
  __shared__ unsigned long long s_tied[kTiedCap];
  __shared__ uint32_t s_cnt[kRowIters * 16];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_nt;
  __shared__ unsigned long long s_T;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = min(n_valid[b], n_cols);
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;
  uint32_t* h1 = FUSED ? hist1 + (size_t)b * kHist1Bins : nullptr;

  // ---- level-1 histogram: the fused one is loaded before the keys (loads complete in
  // order, so the histogram is not held up behind them); otherwise it is built in LDS
  uint32_t hv[kHist1Bins / kBigThreads];
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < kHist1Bins / kBigThreads; ++i) hv[i] = h1[tid + i * kBigThreads];
  }
  uint32_t key[kRowIters];
  int32_t id[kRowIters];
  load_keys<kRowIters>(srow, crow, nv, tid, kBigThreads, key, id);
  uint32_t my = 0;
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < kHist1Bins / kBigThreads; ++i) {
      s_h[tid + i * kBigThreads] = hv[i];
      my += hv[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kHist1Bins / kBigThreads; ++i) s_h[tid + i * kBigThreads] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kRowIters; ++it)
      if (key[it]) atomicAdd(&s_h[key[it] >> 20], 1u);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHist1Bins / kBigThreads; ++i) my += s_h[tid + i * kBigThreads];
  }
  if (tid == 0) {
    s_nt = 0u;
    s_T = 0ull;
  }
  uint32_t total;
  block_exclusive_scan(my, s_scan, &total);
  const uint32_t k_eff = min((uint32_t)k, total);

  if (k_eff < total) {
    find_bin_block<kHist1Bins / kBigThreads>(s_h, k_eff, s_scan, s_res);
    const uint32_t b1 = s_res[0];
    uint32_t need = k_eff - s_res[1];
    // ---- level 2 over the columns in bin b1
    for (int i = tid; i < kHist2Bins; i += kBigThreads) s_h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kRowIters; ++it)
      if (key[it] && (key[it] >> 20) == b1) atomicAdd(&s_h[digit2(key[it])], 1u);
    __syncthreads();
    find_bin_block<kHist2Bins / kBigThreads>(s_h, need, s_scan, s_res);
    const uint32_t b2 = s_res[0];
    need -= s_res[1];
    const uint32_t n_tied = s_h[b2];
    if (n_tied <= (uint32_t)kTiedCap) {
#pragma unroll
      for (int it = 0; it < kRowIters; ++it) {
        if (key[it] && (key[it] >> 20) == b1 && digit2(key[it]) == b2) {
          const uint32_t p = atomicAdd(&s_nt, 1u);
          if (p < (uint32_t)kTiedCap) s_tied[p] = composite(key[it], (uint32_t)(it * kBigThreads + tid));
        }
      }
      __syncthreads();
      rank_tied(s_tied, min(s_nt, (uint32_t)kTiedCap), need, &s_T);
    } else {
      __syncthreads();
      const unsigned long long T = radix_tail(b1, b2, need, s_h, s_res, [&](auto f) {
#pragma unroll
        for (int it = 0; it < kRowIters; ++it)
          if (key[it]) f(composite(key[it], (uint32_t)(it * kBigThreads + tid)));
      });
      if (tid == 0) s_T = T;
    }
    __syncthreads();
  }
  const unsigned long long T = s_T;  // 0 takes every selectable column

  // ---- compaction in column order: column = it*1024 + wave*64 + lane
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    const bool take = key[it] && composite(key[it], (uint32_t)(it * kBigThreads + tid)) >= T;
    const unsigned long long m = __ballot(take);
    if (lane == 0) s_cnt[it * 16 + wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  {
    const uint32_t v = tid < kRowIters * 16 ? s_cnt[tid] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(v, s_scan, &tot);
    if (tid < kRowIters * 16) s_cnt[tid] = ex;
  }
  __syncthreads();
  int32_t* orow = idx_out + (size_t)b * k;
  float* sout = score_out ? score_out + (size_t)b * k : nullptr;
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    const int col = it * kBigThreads + tid;
    const bool take = key[it] && composite(key[it], (uint32_t)col) >= T;
    const unsigned long long m = __ballot(take);
    if (take) {
      const uint32_t pos = s_cnt[it * 16 + wave] + lanes_below(m);
      if (pos < (uint32_t)k) {
        orow[pos] = id[it];
        if (sout) sout[pos] = key_score(key[it]);
      }
    }
  }
  for (int p = (int)k_eff + tid; p < k; p += kBigThreads) {
    orow[p] = -1;
    if (sout) sout[p] = -__builtin_inff();
  }
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < kHist1Bins / kBigThreads; ++i) h1[tid + i * kBigThreads] = 0u;
  }
}

// ---------------------------------------------------------------------------- long rows
__global__ __launch_bounds__(kHistThreads) void k_topk_hist(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, int cols_per_wg, uint32_t* __restrict__ hist1) {
  __shared__ uint32_t s_hist[kHist1Bins];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < kHist1Bins; i += kHistThreads) s_hist[i] = 0u;
  __syncthreads();
  const int nv = min(n_valid[b], n_cols);
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;
  const int c0 = blockIdx.x * cols_per_wg, c1 = min(c0 + cols_per_wg, nv);
  for (int c = c0 + threadIdx.x; c < c1; c += kHistThreads) {
    const uint32_t key = col_key(srow, crow, nv, c);
    if (key != 0u) atomicAdd(&s_hist[key >> 20], 1u);
  }
  __syncthreads();
  uint32_t* h = hist1 + (size_t)b * kHist1Bins;
  for (int i = threadIdx.x; i < kHist1Bins; i += kHistThreads) {
    uint32_t v = s_hist[i];
    if (v) atomic_add_agent(&h[i], v);
  }
}

// Per-row level-1 analysis (one 1024-thread workgroup per row): selectable columns, the
// effective k and, unless every column is taken, the bin b1 of the k-th key and the
// count above it, into the row's counters.
__global__ __launch_bounds__(kBigThreads) void k_topk_bin(int k, TopkWs ws) {
  __shared__ uint32_t s_h[kHist1Bins];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint32_t* h1 = ws.hist1 + (size_t)b * kHist1Bins;
  uint32_t my = 0;
#pragma unroll
  for (int i = 0; i < kHist1Bins / kBigThreads; ++i) {
    const uint32_t v = h1[tid + i * kBigThreads];
    s_h[tid + i * kBigThreads] = v;
    my += v;
  }
  uint32_t total;
  block_exclusive_scan(my, s_scan, &total);
  const uint32_t k_eff = min((uint32_t)k, total);
  if (k_eff < total) find_bin_block<kHist1Bins / kBigThreads>(s_h, k_eff, s_scan, s_res);
  if (tid == 0) {
    uint32_t* info = ws.counters + (size_t)b * kRowInfo;
    info[kInfoKeff] = k_eff;
    info[kInfoTotal] = total;
    info[kInfoBin1] = k_eff < total ? s_res[0] : 0u;
    info[kInfoAbove1] = k_eff < total ? s_res[1] : 0u;
  }
}

template <int ITERS>
__global__ __launch_bounds__(kLongThreads) void k_topk_filter(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, TopkWs ws) {
  __shared__ uint32_t s_cnt[ITERS * 4];
  __shared__ uint32_t s_scan[32];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;
  const int nv = min(n_valid[b], n_cols);
  const int c0 = chunk * kLongThreads * ITERS;
  const uint32_t* info = ws.counters + (size_t)b * kRowInfo;

  const bool all = info[kInfoKeff] == info[kInfoTotal];
  const uint32_t b1 = info[kInfoBin1];
  uint32_t key[ITERS];
  int32_t id[ITERS];
  load_keys<ITERS>(srow, crow, nv, c0 + tid, kLongThreads, key, id);

  uint32_t n_def = 0;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const uint32_t d1 = key[it] >> 20;
    n_def += (key[it] != 0u && (all || d1 > b1)) ? 1u : 0u;
    const unsigned long long m = __ballot(key[it] != 0u && !all && d1 == b1);
    if (lane == 0) s_cnt[it * 4 + wave] = (uint32_t)__popcll(m);
  }
  uint32_t defs;
  block_exclusive_scan(n_def, s_scan, &defs);  // barrier: s_cnt complete
  if (wave == 0) {
    const uint32_t nc = scan_counts_wave0(s_cnt, ITERS * 4);
    if (lane == 0) {
      ws.chunk_cnt[(size_t)b * ws.n_chunks + chunk] = defs;
      ws.chunk_ccnt[(size_t)b * ws.n_chunks + chunk] = nc;
    }
  }
  __syncthreads();
  unsigned long long* slots = ws.list + (size_t)b * n_cols + c0;  // this chunk's own slots
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const bool isc = key[it] != 0u && !all && (key[it] >> 20) == b1;
    const unsigned long long m = __ballot(isc);
    if (isc) {
      const uint32_t pos = s_cnt[it * 4 + wave] + lanes_below(m);
      slots[pos] = ((unsigned long long)key[it] << 32) | (uint32_t)(c0 + it * kLongThreads + tid);
    }
  }
}

// Loads candidates i0 .. i0+kCandBatch-1 of a chunk (n >= 1 of them) at once; indices past
// n re-read the last one.
constexpr int kCandBatch = 16;
__device__ __forceinline__ void load_batch(const unsigned long long* sl, uint32_t i0, uint32_t n,
                                           unsigned long long (&v)[kCandBatch]) {
#pragma unroll
  for (int u = 0; u < kCandBatch; ++u) v[u] = sl[min(i0 + (uint32_t)u, n - 1u)];
}

__global__ __launch_bounds__(kBigThreads) void k_topk_resolve(int n_cols, int chunk_cols, TopkWs ws) {
  __shared__ uint32_t s_h[kHist2Bins];
  __shared__ uint32_t s_chunk[kMaxChunks];
  __shared__ unsigned long long s_tied[kTiedCap];
  __shared__ unsigned long long s_T;
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[8];
  __shared__ uint32_t s_nt;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n_chunks = ws.n_chunks;
  uint32_t* h1 = ws.hist1 + (size_t)b * kHist1Bins;
  const uint32_t* info = ws.counters + (size_t)b * kRowInfo;
  const uint32_t* ccnt = ws.chunk_ccnt + (size_t)b * n_chunks;
  const unsigned long long* list = ws.list + (size_t)b * n_cols;
  const uint32_t k_eff = info[kInfoKeff], total = info[kInfoTotal];
  for (int i = tid; i < n_chunks; i += kBigThreads) s_chunk[i] = 0u;
  for (int i = tid; i < kHist2Bins; i += kBigThreads) s_h[i] = 0u;
  if (tid == 0) {
    s_nt = 0u;
    s_T = 0ull;
  }
  __syncthreads();

  if (k_eff < total) {
    const uint32_t b1 = info[kInfoBin1];
    const uint32_t need1 = k_eff - info[kInfoAbove1];
    // level-2 histogram of the candidates (each thread walks whole chunks)
    for (int ch = tid; ch < n_chunks; ch += kBigThreads) {
      const uint32_t n = min(ccnt[ch], (uint32_t)chunk_cols);
      const unsigned long long* sl = list + (size_t)ch * chunk_cols;
      for (uint32_t i0 = 0; i0 < n; i0 += kCandBatch) {
        unsigned long long v[kCandBatch];
        load_batch(sl, i0, n, v);
#pragma unroll
        for (int u = 0; u < kCandBatch; ++u)
          if (i0 + u < n) atomicAdd(&s_h[digit2((uint32_t)(v[u] >> 32))], 1u);
      }
    }
    __syncthreads();
    find_bin_block<kHist2Bins / kBigThreads>(s_h, need1, s_scan, s_res);
    const uint32_t b2 = s_res[0];
    const uint32_t need = need1 - s_res[1];
    const uint32_t n_tied = s_h[b2];
    const bool in_lds = n_tied <= (uint32_t)kTiedCap;
    unsigned long long* tied = ws.tied + (size_t)b * n_cols;
    for (int ch = tid; ch < n_chunks; ch += kBigThreads) {
      const uint32_t n = min(ccnt[ch], (uint32_t)chunk_cols);
      const unsigned long long* sl = list + (size_t)ch * chunk_cols;
      uint32_t above = 0;
      for (uint32_t i0 = 0; i0 < n; i0 += kCandBatch) {
        unsigned long long vb[kCandBatch];
        load_batch(sl, i0, n, vb);
#pragma unroll
        for (int u = 0; u < kCandBatch; ++u) {
          if (i0 + u >= n) continue;
          const unsigned long long v = vb[u];
          const uint32_t key = (uint32_t)(v >> 32), d2 = digit2(key);
          if (d2 > b2) {
            ++above;
          } else if (d2 == b2) {
            const uint32_t p = atomicAdd(&s_nt, 1u);
            const unsigned long long c = composite(key, (uint32_t)v);
            if (in_lds) {
              if (p < (uint32_t)kTiedCap) s_tied[p] = c;
            } else if (p < (uint32_t)n_cols) {
              tied[p] = c;
            }
          }
        }
      }
      s_chunk[ch] += above;  // chunk ch belongs to this thread here
    }
    __syncthreads();
    const uint32_t nt = min(s_nt, in_lds ? (uint32_t)kTiedCap : (uint32_t)n_cols);
    if (in_lds) {
      rank_tied(s_tied, nt, need, &s_T);
    } else {
      const unsigned long long T = radix_tail(b1, b2, need, s_h, s_res, [&](auto f) {
        for (uint32_t i = tid; i < nt; i += kBigThreads) f(tied[i]);
      });
      if (tid == 0) s_T = T;
    }
    __syncthreads();
    const unsigned long long T = s_T;
    for (uint32_t i = tid; i < nt; i += kBigThreads) {
      const unsigned long long c = in_lds ? s_tied[i] : tied[i];
      if (c >= T) atomicAdd(&s_chunk[(uint32_t)~(uint32_t)c / chunk_cols], 1u);
    }
  }
  __syncthreads();

  // output offset of every chunk: exclusive scan of (columns above b1) + (chosen candidates)
  const uint32_t* cc = ws.chunk_cnt + (size_t)b * n_chunks;
  const int per = (n_chunks + kBigThreads - 1) / kBigThreads;
  const int lo = min(tid * per, n_chunks), hi = min(lo + per, n_chunks);
  uint32_t mine = 0;
  for (int c = lo; c < hi; ++c) mine += cc[c] + s_chunk[c];
  uint32_t tot;
  uint32_t run = block_exclusive_scan(mine, s_scan, &tot);
  uint32_t* off = ws.chunk_off + (size_t)b * n_chunks;
  for (int c = lo; c < hi; ++c) {
    off[c] = run;
    run += cc[c] + s_chunk[c];
  }
  if (tid == 0) ws.thr[b] = k_eff < total ? s_T : 0ull;
  for (int i = tid; i < kHist1Bins; i += kBigThreads) h1[i] = 0u;  // ready for the next call
}

template <int ITERS>
__global__ __launch_bounds__(kLongThreads) void k_topk_compact(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, TopkWs ws) {
  __shared__ uint32_t s_cnt[ITERS * 4];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;
  const int nv = min(n_valid[b], n_cols);
  const int c0 = chunk * kLongThreads * ITERS;
  const unsigned long long T = ws.thr[b];
  const uint32_t k_eff = ws.counters[(size_t)b * kRowInfo + kInfoKeff];
  const uint32_t off = ws.chunk_off[(size_t)b * ws.n_chunks + chunk];

  uint32_t key[ITERS];
  int32_t id[ITERS];
  load_keys<ITERS>(srow, crow, nv, c0 + tid, kLongThreads, key, id);
  unsigned long long sel = 0ull;  // bit it: this thread's column of iteration it is taken
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const uint32_t col = (uint32_t)(c0 + it * kLongThreads + tid);
    const bool take = key[it] != 0u && composite(key[it], col) >= T;
    sel |= (unsigned long long)take << it;
    const unsigned long long m = __ballot(take);
    if (lane == 0) s_cnt[it * 4 + wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  if (wave == 0) scan_counts_wave0(s_cnt, ITERS * 4);
  __syncthreads();
  int32_t* orow = idx_out + (size_t)b * k;
  float* sout = score_out ? score_out + (size_t)b * k : nullptr;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const bool take = (sel >> it) & 1ull;
    const unsigned long long m = __ballot(take);
    if (take) {
      const uint32_t pos = off + s_cnt[it * 4 + wave] + lanes_below(m);
      if (pos < (uint32_t)k) {
        orow[pos] = id[it];
        if (sout) sout[pos] = key_score(key[it]);
      }
    }
  }
  for (int p = (int)k_eff + chunk * kLongThreads + tid; p < k; p += ws.n_chunks * kLongThreads) {
    orow[p] = -1;
    if (sout) sout[p] = -__builtin_inff();
  }
}

template <int ITERS>
static hipError_t launch_long(const float* scores, int batch, int n_cols, const int32_t* n_valid,
                              const int32_t* cand, int k, int32_t* idx_out, float* score_out,
                              const TopkWs& ws, hipStream_t stream) {
  const dim3 grid(ws.n_chunks, batch);
  hipLaunchKernelGGL(k_topk_bin, dim3(batch), dim3(kBigThreads), 0, stream, k, ws);
  hipLaunchKernelGGL(k_topk_filter<ITERS>, grid, dim3(kLongThreads), 0, stream, scores, n_cols,
                     n_valid, cand, ws);
  hipLaunchKernelGGL(k_topk_resolve, dim3(batch), dim3(kBigThreads), 0, stream, n_cols,
                     kLongThreads * ITERS, ws);
  hipLaunchKernelGGL(k_topk_compact<ITERS>, grid, dim3(kLongThreads), 0, stream, scores, n_cols,
                     n_valid, cand, k, idx_out, score_out, ws);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int batch, int n_cols, const int32_t* n_valid,
                       const int32_t* cand, int k, int32_t* idx_out, float* score_out,
                       bool hist_ready, const TopkWs& ws, hipStream_t stream) {
  if (n_cols <= kTopkSmallMax) {
    if (hist_ready)
      hipLaunchKernelGGL(k_topk_row<true>, dim3(batch), dim3(kBigThreads), 0, stream, scores, n_cols,
                         n_valid, cand, k, idx_out, score_out, ws.hist1);
    else
      hipLaunchKernelGGL(k_topk_row<false>, dim3(batch), dim3(kBigThreads), 0, stream, scores, n_cols,
                         n_valid, cand, k, idx_out, score_out, nullptr);
    return hipGetLastError();
  }
  if (!hist_ready) {
    const int cpw = 8192;
    hipLaunchKernelGGL(k_topk_hist, dim3((n_cols + cpw - 1) / cpw, batch), dim3(kHistThreads), 0,
                       stream, scores, n_cols, n_valid, cand, cpw, ws.hist1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (topk_chunk_iters(n_cols) == 8)
    return launch_long<8>(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, ws, stream);
  return launch_long<32>(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, ws, stream);
}

}  // namespace csa2
