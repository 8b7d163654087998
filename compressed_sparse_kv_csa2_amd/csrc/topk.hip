// a2 top-k selection: the k largest scores of a row, ties to the lower column, written
// in ascending column order as entry ids (cand[c] or c), -1 padded.
//
// Used for the decoder pool (k = 16,384 of up to 2^20 columns) and for every top-512
// ("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", commentary on the four
// layer modes; "从V4到V4.1 Flash：架构的激进进化", decoder section on the hierarchical
// indexer).  The tie rule is this library's reading; the pages do not state one.
//
// Scores map to order-preserving u32 keys.  The selection is exact for the 64-bit
// composite (key, ~column), which is unique per column, so the k-th element and
// therefore the selected set are unique.
//
// Short rows (<= 16,384 columns): one 1024-thread workgroup per row keeps all keys in
// LDS, finds the exact k-th key with four 8-bit radix passes, then compacts in column
// order, taking tied keys lowest column first.
//
// Long rows: a 12-bit histogram of the keys (fused into the scan, or k_topk_hist) names
// the bin holding the k-th key.  k_topk_filter then streams the scores once: columns
// above that bin become bits of a selection bitmap (one 64-bit ballot per wave), the
// few in it are appended to a candidate list with an 11-bit second-level histogram.
// The workgroup that finishes a row last resolves the candidates exactly (remaining
// key bits, then column bits) and compacts the bitmap into the ascending list, so the
// whole selection costs two launches and no host round trip.  It also returns the
// histograms and counters to zero for the next call.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int kBigThreads = 1024;
constexpr int kFilterCols = 16384;   // columns per filter workgroup (16 per thread)
constexpr int kHistThreads = 256;

size_t topk_ws_bytes(int batch, int n_cols) {
  const size_t words = ((size_t)n_cols + 63) / 64;
  size_t s = 0;
  s += align_up((size_t)batch * kHist1Bins * 4, 256);
  s += align_up((size_t)batch * kHist2Bins * 4, 256);
  s += align_up((size_t)batch * 4 * 4, 256);
  s += align_up((size_t)batch * words * 8, 256);
  s += 2 * align_up((size_t)batch * n_cols * 8, 256);
  return s;
}

TopkWs topk_ws_carve(void* base, int batch, int n_cols) {
  TopkWs w;
  char* p = static_cast<char*>(base);
  w.words = ((int64_t)n_cols + 63) / 64;
  w.hist1 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist1Bins * 4, 256);
  w.hist2 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist2Bins * 4, 256);
  w.counters = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * 4 * 4, 256);
  w.bitmap = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)batch * w.words * 8, 256);
  w.listA = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)batch * n_cols * 8, 256);
  w.listB = reinterpret_cast<unsigned long long*>(p);
  return w;
}

// ---------------------------------------------------------------------------- helpers
// Executed by ONE wave: finds the bin `sel` holding the need-th largest element of the
// histogram h[0..nbins) (nbins a multiple of 64, 1 <= need <= total) and the count of
// elements in bins above it.  Writes out[0] = sel, out[1] = above.
__device__ void find_threshold_bin(const uint32_t* h, int nbins, uint32_t need, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {  // defined result even if need exceeded the total (it never should)
    out[0] = 0u;
    out[1] = 0u;
  }
  const int per = nbins / 64;
  const int hi = nbins - lane * per;  // lane 0 owns the top bins
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

// Block-wide exclusive scan of one u32 per thread; returns the exclusive prefix and
// stores the block total in *total.  `scratch` holds >= 17 u32 of LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
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
  uint32_t r = scratch[wave] + incl - v;
  *total = scratch[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------- short rows
__global__ __launch_bounds__(kBigThreads) void k_topk_small(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  __shared__ uint32_t s_key[kTopkSmallMax];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[4];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nv = min(n_valid[b], n_cols);
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;

  uint32_t my_valid = 0;
  for (int c = tid; c < n_cols; c += kBigThreads) {
    bool v = c < nv && (!crow || crow[c] >= 0);
    s_key[c] = v ? score_key(srow[c]) : 0u;  // finite scores never map to key 0
    my_valid += v ? 1u : 0u;
  }
  uint32_t total_valid;
  block_exclusive_scan(my_valid, s_scan, &total_valid);  // also a barrier
  const uint32_t k_eff = min((uint32_t)k, total_valid);

  uint32_t T, need;  // select key > T, plus the `need` lowest columns with key == T
  if (k_eff == 0) {
    T = 0xffffffffu;
    need = 0;
  } else if (k_eff == total_valid) {
    T = 0u;
    need = 0;
  } else {
    uint32_t prefix = 0, pmask = 0;
    need = k_eff;
    for (int level = 0; level < 4; ++level) {
      const int shift = 24 - 8 * level;
      if (tid < 256) s_hist[tid] = 0u;
      __syncthreads();
      for (int c = tid; c < n_cols; c += kBigThreads) {
        uint32_t key = s_key[c];
        if ((key & pmask) == prefix && key != 0u) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) find_threshold_bin(s_hist, 256, need, s_res);
      __syncthreads();
      const uint32_t sel = s_res[0] & 255u, above = s_res[1];
      need -= above;
      prefix |= sel << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
  }

  const int per = (n_cols + kBigThreads - 1) / kBigThreads;
  const int lo = min(tid * per, n_cols), hi = min(lo + per, n_cols);
  uint32_t n_gt = 0, n_eq = 0;
  for (int c = lo; c < hi; ++c) {
    uint32_t key = s_key[c];
    n_gt += key > T ? 1u : 0u;
    n_eq += (key == T && need > 0) ? 1u : 0u;
  }
  uint32_t tmp;
  const uint32_t eq_before = block_exclusive_scan(n_eq, s_scan, &tmp);
  uint32_t take_eq = 0;
  if (need > eq_before) take_eq = min(n_eq, need - eq_before);
  uint32_t pos = block_exclusive_scan(n_gt + take_eq, s_scan, &tmp);
  uint32_t r = eq_before;
  int32_t* orow = idx_out + (size_t)b * k;
  float* srow_out = score_out ? score_out + (size_t)b * k : nullptr;
  for (int c = lo; c < hi; ++c) {
    uint32_t key = s_key[c];
    bool take = key > T;
    if (key == T && need > 0) {
      take = r < need;
      ++r;
    }
    if (take) {
      if (pos < (uint32_t)k) {
        orow[pos] = crow ? crow[c] : c;
        if (srow_out) srow_out[pos] = srow[c];
      }
      ++pos;
    }
  }
  for (int p = (int)k_eff + tid; p < k; p += kBigThreads) {
    orow[p] = -1;
    if (srow_out) srow_out[p] = -__builtin_inff();
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
    if (crow && crow[c] < 0) continue;
    atomicAdd(&s_hist[score_key(srow[c]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* h = hist1 + (size_t)b * kHist1Bins;
  for (int i = threadIdx.x; i < kHist1Bins; i += kHistThreads) {
    uint32_t v = s_hist[i];
    if (v) atomic_add_agent(&h[i], v);
  }
}

__device__ __forceinline__ void set_bit(unsigned long long* bm, uint32_t col) {
  atomic_or_agent(&bm[col >> 6], 1ull << (col & 63u));
}

__global__ __launch_bounds__(kBigThreads) void k_topk_filter(
    const float* __restrict__ scores, int n_cols, const int32_t* __restrict__ n_valid,
    const int32_t* __restrict__ cand, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, TopkWs ws, int n_chunks) {
  __shared__ uint32_t s_h[kHist1Bins];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[8];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* h1 = ws.hist1 + (size_t)b * kHist1Bins;
  uint32_t* h2 = ws.hist2 + (size_t)b * kHist2Bins;
  uint32_t* cnt = ws.counters + (size_t)b * 4;
  unsigned long long* bm = ws.bitmap + (size_t)b * ws.words;
  unsigned long long* listA = ws.listA + (size_t)b * n_cols;
  unsigned long long* listB = ws.listB + (size_t)b * n_cols;
  const float* srow = scores + (size_t)b * n_cols;
  const int32_t* crow = cand ? cand + (size_t)b * n_cols : nullptr;
  const int nv = min(n_valid[b], n_cols);

  // ---- level 1: the bin of the k-th key (every workgroup derives the same answer)
  uint32_t my = 0;
  for (int i = tid; i < kHist1Bins; i += kBigThreads) {
    uint32_t v = h1[i];
    s_h[i] = v;
    my += v;
  }
  uint32_t total;
  block_exclusive_scan(my, s_scan, &total);
  const uint32_t k_eff = min((uint32_t)k, total);
  const bool all = k_eff == total;
  uint32_t b1 = 0, need1 = 0;
  if (!all) {
    if (tid < 64) find_threshold_bin(s_h, kHist1Bins, k_eff, s_res);
    __syncthreads();
    b1 = s_res[0];
    need1 = k_eff - s_res[1];
  }

  // ---- stream this chunk's scores
  const int c0 = blockIdx.x * kFilterCols;
  for (int i = 0; i < kFilterCols / kBigThreads; ++i) {
    const int wcol = c0 + i * kBigThreads + wave * 64;
    if (wcol >= n_cols) break;
    const int col = wcol + lane;
    bool valid = col < nv && (!crow || crow[col] >= 0);
    uint32_t key = valid ? score_key(srow[col]) : 0u;
    uint32_t d1 = key >> 20;
    bool def = valid && (all || d1 > b1);
    bool isc = valid && !all && d1 == b1;
    unsigned long long mdef = __ballot(def);
    unsigned long long mc = __ballot(isc);
    if (lane == 0) bm[wcol >> 6] = mdef;
    if (mc) {
      uint32_t basepos = 0;
      if (lane == 0) basepos = atomic_add_agent(&cnt[0], (uint32_t)__popcll(mc));
      basepos = __shfl(basepos, 0);
      if (isc) {
        uint32_t r = (uint32_t)__popcll(mc & ((1ull << lane) - 1ull));
        listA[basepos + r] = ((unsigned long long)key << 32) | (uint32_t)col;
        atomic_add_agent(&h2[(key >> 9) & (kHist2Bins - 1)], 1u);
      }
    }
  }

  if (!arrive_last(&cnt[1], (uint32_t)n_chunks, &s_res[4])) return;

  // ---- last workgroup of row b: resolve the candidates exactly
  if (!all) {
    uint32_t C = ld_agent(&cnt[0]);
    uint32_t need = need1;
    for (int i = tid; i < kHist2Bins; i += kBigThreads) s_h[i] = ld_agent(&h2[i]);
    __syncthreads();
    if (tid < 64) find_threshold_bin(s_h, kHist2Bins, need, s_res);
    __syncthreads();
    const uint32_t b2 = s_res[0];
    need -= s_res[1];
    uint32_t C2 = s_h[b2];
    if (tid == 0) s_res[6] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < C; i += kBigThreads) {
      unsigned long long v = ld_agent(&listA[i]);
      uint32_t key = (uint32_t)(v >> 32);
      uint32_t d2 = (key >> 9) & (kHist2Bins - 1);
      if (d2 > b2) {
        set_bit(bm, (uint32_t)v);
      } else if (d2 == b2) {
        uint32_t p = atomicAdd(&s_res[6], 1u);
        listB[p] = v;
      }
    }
    __syncthreads();
    // remaining digits of the composite ((key & 511) << 32 | ~column): 9 key bits, then
    // four 8-bit digits of the inverted column (a lower column ranks higher)
    unsigned long long* cur = listB;
    unsigned long long* oth = listA;
    C = C2;
    for (int lvl = 0; lvl < 5 && need > 0; ++lvl) {
      if (C == need) break;
      const int nb = lvl == 0 ? 512 : 256;
      const int shift = lvl == 0 ? 32 : 24 - 8 * (lvl - 1);
      for (int i = tid; i < nb; i += kBigThreads) s_h[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < C; i += kBigThreads) {
        unsigned long long v = ld_agent(&cur[i]);
        unsigned long long comp = ((v >> 32) & 511ull) << 32 | (uint32_t)~(uint32_t)v;
        atomicAdd(&s_h[(comp >> shift) & (unsigned long long)(nb - 1)], 1u);
      }
      __syncthreads();
      if (tid < 64) find_threshold_bin(s_h, nb, need, s_res);
      if (tid == 0) s_res[6] = 0u;
      __syncthreads();
      const uint32_t sel = s_res[0];
      need -= s_res[1];
      const uint32_t newC = s_h[sel];
      for (uint32_t i = tid; i < C; i += kBigThreads) {
        unsigned long long v = ld_agent(&cur[i]);
        unsigned long long comp = ((v >> 32) & 511ull) << 32 | (uint32_t)~(uint32_t)v;
        uint32_t d = (uint32_t)((comp >> shift) & (unsigned long long)(nb - 1));
        if (d > sel) {
          set_bit(bm, (uint32_t)v);
        } else if (d == sel) {
          uint32_t p = atomicAdd(&s_res[6], 1u);
          oth[p] = v;
        }
      }
      __syncthreads();
      unsigned long long* t = cur;
      cur = oth;
      oth = t;
      C = newC;
    }
    if (need > 0) {  // C == need: take the rest
      for (uint32_t i = tid; i < C; i += kBigThreads) set_bit(bm, (uint32_t)ld_agent(&cur[i]));
    }
    __syncthreads();
  }

  // ---- compact the bitmap into the ascending list
  const int nw = (nv + 63) / 64;
  const int per = (nw + kBigThreads - 1) / kBigThreads;
  const int wlo = min(tid * per, nw), whi = min(wlo + per, nw);
  uint32_t mine = 0;
  for (int w = wlo; w < whi; ++w) mine += (uint32_t)__popcll(ld_agent(&bm[w]));
  uint32_t tot;
  uint32_t pos = block_exclusive_scan(mine, s_scan, &tot);
  int32_t* orow = idx_out + (size_t)b * k;
  float* sout = score_out ? score_out + (size_t)b * k : nullptr;
  for (int w = wlo; w < whi; ++w) {
    unsigned long long m = ld_agent(&bm[w]);
    while (m) {
      const int bit = __builtin_ctzll(m);
      m &= m - 1ull;
      const int col = w * 64 + bit;
      if (pos < (uint32_t)k) {
        orow[pos] = crow ? crow[col] : col;
        if (sout) sout[pos] = srow[col];
      }
      ++pos;
    }
  }
  for (int p = (int)tot + tid; p < k; p += kBigThreads) {
    orow[p] = -1;
    if (sout) sout[p] = -__builtin_inff();
  }
  // ---- return the workspace counters of this row to zero
  for (int i = tid; i < kHist1Bins; i += kBigThreads) h1[i] = 0u;
  for (int i = tid; i < kHist2Bins; i += kBigThreads) h2[i] = 0u;
  if (tid < 4) cnt[tid] = 0u;
}

hipError_t launch_topk(const float* scores, int batch, int n_cols, const int32_t* n_valid,
                       const int32_t* cand, int k, int32_t* idx_out, float* score_out,
                       bool hist_ready, const TopkWs& ws, hipStream_t stream) {
  if (!hist_ready && n_cols <= kTopkSmallMax) {
    hipLaunchKernelGGL(k_topk_small, dim3(batch), dim3(kBigThreads), 0, stream, scores, n_cols,
                       n_valid, cand, k, idx_out, score_out);
    return hipGetLastError();
  }
  if (!hist_ready) {
    const int cpw = 8192;
    hipLaunchKernelGGL(k_topk_hist, dim3((n_cols + cpw - 1) / cpw, batch), dim3(kHistThreads), 0,
                       stream, scores, n_cols, n_valid, cand, cpw, ws.hist1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_chunks = (n_cols + kFilterCols - 1) / kFilterCols;
  hipLaunchKernelGGL(k_topk_filter, dim3(n_chunks, batch), dim3(kBigThreads), 0, stream, scores,
                     n_cols, n_valid, cand, k, idx_out, score_out, ws, n_chunks);
  return hipGetLastError();
}

}  // namespace csa2
