// a1 + a2 (and a3 + a2): score the indexer keys and select the exact top-k without
// writing the scores; optionally followed by the selections a decoder layer chain makes
// inside that pool (the Full layer's own top-k by its scores, and the top-k of Reindex
// layers that re-score the pool with their own indexer queries).  "从V4到V4.1 Flash：架构
// 的激进进化", decoder section: the first layer's full scan yields a pool of about 16K
// positions that later layers search; "DeepSeek-V4.1 模型结构（0）：一张图看懂
// DeepSeek-V4.1-Flash", commentary on the four layer modes.
//
// Every selection returns what csa2_topk returns for the same scores: the k largest of a
// row, ties to the lower column, written in ascending column order as entry ids, -1
// padded.  Inside the pool, "column" means the pool position, which ascends with the
// entry id, so ties again go to the lowest entry.
//
// Design: a filtered scan, then a selection over the survivors.  The pool is 1.6 % of a
// 2^20-entry row, so the scan need not keep every key until the row's threshold is
// known: given a lower bound theta of the k-th key, each chunk of columns writes out only
// its keys >= theta (the candidates), and a second launch selects the exact top-k of each
// row among its candidates.
//   k_fscan, one persistent workgroup per compute unit:
//   * Work is a list of tasks claimed from one atomic counter: first each long row's
//     sample tasks (1,024 keys each: one column in 32, in groups of 64 spread evenly over
//     the row), then every row's chunks of 15 x 64 x 2 columns, row after row.  Chunks go
//     to whichever workgroup is free, so compute units that stream faster take more.
//   * theta of a row is an order statistic of its sample, chosen so that about
//     k + 4 sqrt(k) keys of the row are expected above it; the last sample task of the
//     row computes it.  Exactness never rests on it: when fewer than k keys of the row
//     turn out to be >= theta, or more than the selection holds, the selection scans the
//     row again keeping every key (slow, counted in the workspace).  Rows short enough
//     for the selection to hold whole use theta = 1 (every valid key).
//   * A workgroup is 15 streaming waves and one writer wave.  The streaming waves score a
//     chunk's columns into LDS with the next chunk's loads already in flight; meanwhile the
//     writer wave claims the next chunk and appends the previous chunk's keys >= theta
//     (in column order) to the row's candidate store, at a place it reserves with one
//     atomic add.  Stores never sit in a streaming wave's memory counter, so they never
//     hold up its loads.
//   * Only the writer of a chunk waits on other workgroups (for its row's theta), and the
//     sample tasks it waits for were claimed earlier by running workgroups that wait on
//     nothing: the launch needs no co-residency.
//   k_fselect, one workgroup per row:
//   * one round of coalesced loads brings the row's candidates (keys to LDS, columns to
//     registers) and each chunk's place in the store; the k-th composite (key, lower
//     column first) is found by narrowing 4,096-bin histograms over the range the keys
//     actually span until at most 64 remain, which are ranked directly.  A winner's output
//     position is the number of winners in the chunks before its own (column order) plus
//     those before it in its chunk's run, from a bitmap over the store.  The chained
//     selections run on the same candidates (own top-k) or on the pool's re-scores
//     (Reindex), which the writer computed as it stored each candidate.
// The launch boundary orders the candidate stores before the selection.  The selection
// returns the scan's counters to zero, so the workspace needs no clearing between calls.
#include "csa2_internal.h"
#include "scan_device.h"
#include "select_device.h"

// Timing hooks: compiled in only with CSA2_FS_TRACE (a measurement build); otherwise empty.
#ifdef CSA2_FS_TRACE
namespace csa2 {
__device__ unsigned long long g_fs_trace[1 << 20];
}
#define FS_TR(idx, val) (::csa2::g_fs_trace[(idx)] = (unsigned long long)(val))
#define FS_NOW() wall_clock64()
#else
#define FS_TR(idx, val) ((void)0)
#define FS_NOW() 0ull
#endif

namespace csa2 {
namespace {

constexpr int kT = 1024;                  // threads per workgroup
constexpr int kNW = kT / 64;              // waves
constexpr int kSW = 15;                   // streaming waves of the scan
constexpr int kMaxCand = 24576;           // candidates the selection holds (LDS + registers)
constexpr int kU = kMaxCand / kT;         // candidates per thread
constexpr int kPU = CSA2_MAX_K / kT;      // pool entries per thread
constexpr int kSampTask = 1024;           // sampled keys per sample task (16 waves x 64)
constexpr int kSampEvery = 32;            // one column in 32 is sampled
constexpr int kMaxSampTasks = 32;
constexpr int kSampRow = kSampTask * kMaxSampTasks;
constexpr int kMaxRows = 256;             // rows per launch
constexpr int kMaxRuns = 2048;            // chunks per row
constexpr int kBins = 4096;
constexpr int kG = 2;                     // groups of 64 columns per streaming wave and chunk
constexpr int kChunk = kSW * 64 * kG;     // 1,920 columns
constexpr int kCW = kChunk / 64;          // 64-column words of a chunk
constexpr int kRowWords = 16;             // per-row counters (64 bytes)
constexpr int kRwSamp = 0, kRwTheta = 1, kRwDone = 2, kRwShift = 3;
constexpr int kCtStatus = 0, kCtTask = 1, kCtSlow = 2;
constexpr uint32_t kSpin = 1u << 22;
constexpr int kChainRows = 16;            // rows per launch of a chained selection

__device__ __forceinline__ uint32_t ld_ag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_ag(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every vector memory operation this wave issued has completed; its
// agent-scope stores are then visible to every workgroup.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct FsArgs {
  const uint16_t* q;          // [batch][128] query of the scan
  const uint8_t* codes;
  const float* scale;
  const int64_t* seq_base;
  const int32_t* n_valid;
  const int32_t* cand;        // [batch][n_cols] (Reindex) or null
  int n_cols, runs;           // columns, chunks per row at most
  int row0, rows, batch;
  int k;
  int32_t* out;               // [batch][k]
  float* sout;                // [batch][k] or null
  int own_k;                  // 0: none
  int32_t* own_out;
  int n_re, re_k;
  const uint16_t* q_re;       // [n_re][batch][128]
  int32_t* re_out;            // [n_re][batch][re_k]
  float* re_sout;             // or null
  uint32_t* ctrl;             // status, task counter, slow rows
  uint32_t* roww;             // [rows][16]: sample tasks done, theta, picking workgroups done, shift
  uint32_t* samp;             // [rows][kSampRow]
  uint32_t* ccnt;             // [rows][runs] how many candidates each chunk has
  uint32_t* ckey;             // [rows][cap] candidate keys: chunk j's run (column order) at j * 1920
  uint32_t* ccol;             // [rows][cap] their columns
  uint32_t* rekey;            // [4][rows][cap] their Reindex re-scores (chain)
  uint32_t* pmap;             // [rows][16384] store index of each pool entry (chain, slow path)
  uint32_t* rhist;            // [rows][4096] candidates per bin of (key - theta) >> shift
  size_t cap;                 // per-row store: runs * 1920
};

// LDS the exact-threshold search and the ordered emission share.
struct Core {
  uint32_t hist[kBins];
  unsigned long long pub[64];
  uint32_t scan[32];
  uint32_t red[3 * kNW];
  uint32_t res[4];
  uint32_t misc[8];
};

// ------------------------------------------------------------------ workgroup reductions
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o));
  return v;
}

// Sum, max and min over the workgroup in one exchange.  Ends with a barrier.
__device__ __forceinline__ void block_smm(uint32_t& s, uint32_t& mx, uint32_t& mn, Core& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  s = wave_sum(s);
  mx = wave_max(mx);
  mn = wave_min(mn);
  if (lane == 0) {
    L.red[wave] = s;
    L.red[kNW + wave] = mx;
    L.red[2 * kNW + wave] = mn;
  }
  __syncthreads();
  uint32_t a = 0, b = 0, c = 0xffffffffu;
  for (int w = 0; w < kNW; ++w) {
    a += L.red[w];
    b = max(b, L.red[kNW + w]);
    c = min(c, L.red[2 * kNW + w]);
  }
  s = a;
  mx = b;
  mn = c;
  __syncthreads();
}

// Calls f(u, i) for the elements i < m this thread owns, i = threadIdx.x + kT * u: with
// U > 0 the loop is unrolled U times (u is a constant, so per-thread register arrays may
// be indexed by it, and U * kT >= m); with U = 0 it loops (u = 0).
template <int U, class F>
__device__ __forceinline__ void for_mine(int m, F f) {
  if constexpr (U > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (int)threadIdx.x + kT * u;
      if (i < m) f(u, i);
    }
  } else {
    for (int i = threadIdx.x; i < m; i += kT) f(0, i);
  }
}

// ------------------------------------------------------------------ the exact threshold
// Selected: key != 0 and (key > tkey or (key == tkey and x <= tx)).  tkey = 0 selects
// every non-zero key.
struct Thr {
  uint32_t tkey, tx, nsel, total;
};

__device__ __forceinline__ bool selected(const Thr& t, uint32_t key, uint32_t x) {
  return key != 0u && (key > t.tkey || (key == t.tkey && x <= t.tx));
}

// The need-th largest composite (key, then lower x first) among elements i < m with a
// non-zero key K(u, i) and unique tie index X(u, i), need = min(k, #non-zero).  The value
// range is narrowed with 4,096-bin histograms over the range actually present (keys
// first, then, for equal keys, ~x) until at most 64 elements remain in the chosen bin;
// those are ranked directly by wave 0.  Whole workgroup; ends with a barrier.
template <int U, class KF, class XF>
__device__ __forceinline__ Thr find_thr(KF K, XF X, int m, uint32_t k, Core& L, int tr = -1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int npass = 0;
  if (tr >= 0 && tid == 0) FS_TR(tr, FS_NOW() | ((unsigned long long)m << 44));
  uint32_t c = 0, mx = 0, mn = 0xffffffffu;
  for_mine<U>(m, [&](int u, int i) {
    const uint32_t v = K(u, i);
    if (v) {
      ++c;
      mx = max(mx, v);
      mn = min(mn, v);
    }
  });
  block_smm(c, mx, mn, L);
  Thr t;
  t.total = c;
  uint32_t need = min(k, c);
  t.nsel = need;
  t.tkey = 0u;
  t.tx = 0u;
  if (need == c) return t;  // every non-zero key (or none)

  uint32_t lo = mn, hi = mx, cnt_in = c, tkey = 0u;
  bool xphase = false;
  // member in the key phase: lo <= K <= hi; in the x phase: K == tkey and lo <= ~X <= hi
  while (cnt_in > 64u) {
    if (!xphase && lo == hi) {  // more than 64 equal keys: rank them by the tie index
      xphase = true;
      tkey = lo;
      uint32_t s2 = 0, xmx = 0, xmn = 0xffffffffu;
      for_mine<U>(m, [&](int u, int i) {
        if (K(u, i) == tkey) {
          const uint32_t v = ~X(u, i);
          ++s2;
          xmx = max(xmx, v);
          xmn = min(xmn, v);
        }
      });
      block_smm(s2, xmx, xmn, L);
      lo = xmn;
      hi = xmx;
      continue;
    }
    const uint32_t range = hi - lo;
    const int sh = range == 0u ? 0 : max(0, 32 - __clz((int)range) - 12);
    if (tr >= 0 && tid == 0 && npass < 8) FS_TR(tr + 1 + npass, FS_NOW() | ((unsigned long long)cnt_in << 44));
    ++npass;
    for (int i = tid; i < kBins; i += kT) L.hist[i] = 0u;
    __syncthreads();
    for_mine<U>(m, [&](int u, int i) {
      const uint32_t key = K(u, i);
      uint32_t v;
      bool mem;
      if (!xphase) {
        v = key;
        mem = key != 0u && key >= lo && key <= hi;
      } else {
        mem = key == tkey;
        v = mem ? ~X(u, i) : 0u;
        mem = mem && v >= lo && v <= hi;
      }
      if (mem) atomicAdd(&L.hist[(v - lo) >> sh], 1u);
    });
    __syncthreads();
    find_bin_block<kBins / kT>(L.hist, need, L.scan, L.res);  // ends with a barrier
    const uint32_t d = L.res[0];
    need -= L.res[1];
    cnt_in = L.hist[d];
    const uint32_t nlo = lo + (d << sh);
    hi = (uint32_t)min((unsigned long long)hi, (unsigned long long)nlo + (1ull << sh) - 1ull);
    lo = nlo;
    __syncthreads();  // L.hist and L.res are read before they are rewritten
  }
  // rank the <= 64 remaining members directly
  if (tr >= 0 && tid == 0) FS_TR(tr + 10, FS_NOW() | ((unsigned long long)npass << 44));
  if (tid == 0) L.misc[0] = 0u;
  __syncthreads();
  for_mine<U>(m, [&](int u, int i) {
    const uint32_t key = K(u, i);
    bool mem;
    uint32_t x = 0u;
    if (!xphase) {
      mem = key != 0u && key >= lo && key <= hi;
      if (mem) x = X(u, i);
    } else {
      mem = key == tkey;
      if (mem) {
        x = X(u, i);
        mem = ~x >= lo && ~x <= hi;
      }
    }
    if (mem) {
      const uint32_t slot = atomicAdd(&L.misc[0], 1u);
      if (slot < 64u) L.pub[slot] = ((unsigned long long)key << 32) | (uint32_t)~x;
    }
  });
  __syncthreads();
  if (wave == 0) {
    const uint32_t nt = min(L.misc[0], 64u);
    const unsigned long long cc = (uint32_t)lane < nt ? L.pub[lane] : 0ull;
    const uint32_t chi = (uint32_t)(cc >> 32), clo = (uint32_t)cc;
    uint32_t r = 0;
    for (uint32_t j = 0; j < nt; ++j) {
      const uint32_t ohi = __builtin_amdgcn_readlane(chi, j);
      const uint32_t olo = __builtin_amdgcn_readlane(clo, j);
      r += (ohi > chi || (ohi == chi && olo > clo)) ? 1u : 0u;
    }
    if ((uint32_t)lane < nt && r == need - 1u) {
      L.res[2] = chi;
      L.res[3] = ~clo;
    }
  }
  __syncthreads();
  t.tkey = L.res[2];
  t.tx = L.res[3];
  __syncthreads();
  return t;
}

// Calls emit(rank, i) for every element i < m with sel(i), rank = its position among them
// in index order.  Wave ballots, one scan of the per-(iteration, wave) counts per block
// of 64 iterations.  Whole workgroup; ends with a barrier.
template <class SelF, class EmitF>
__device__ __forceinline__ void emit_ordered(int m, SelF sel, EmitF emit, Core& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t carry = 0;
  for (int base = 0; base < m; base += 64 * kT) {
    const int iters = min(64, (m - base + kT - 1) / kT);
    unsigned long long bits = 0;
    for (int j = 0; j < iters; ++j) {
      const int i = base + j * kT + tid;
      const bool w = i < m && sel(i);
      bits |= (w ? 1ull : 0ull) << j;
      const unsigned long long msk = __ballot(w);
      if (lane == 0) L.hist[j * kNW + wave] = (uint32_t)__popcll(msk);
    }
    __syncthreads();
    if (wave == 0) {
      const int n = iters * kNW;  // <= 1024: 16 per lane
      uint32_t c[16];
      uint32_t part = 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        c[u] = 16 * lane + u < n ? L.hist[16 * lane + u] : 0u;
        part += c[u];
      }
      const uint32_t incl = wave_incl_scan(part);
      uint32_t run = carry + incl - part;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (16 * lane + u < n) L.hist[16 * lane + u] = run;
        run += c[u];
      }
      if (lane == 63) L.misc[1] = carry + incl;
    }
    __syncthreads();
    for (int j = 0; j < iters; ++j) {
      const bool w = (bits >> j) & 1ull;
      const unsigned long long msk = __ballot(w);
      if (w) emit(L.hist[j * kNW + wave] + lanes_below(msk), base + j * kT + tid);
    }
    carry = L.misc[1];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ shared helpers
// Sample tasks and chunk tasks of a row with n visible columns.
__device__ __forceinline__ int row_samples(int n) {
  return n > kMaxCand ? min(kMaxSampTasks, max(1, n / (kSampTask * kSampEvery))) : 0;
}
__device__ __forceinline__ int row_chunks(int n) { return max(1, (n + kChunk - 1) / kChunk); }

// Sample rank whose key serves as theta: about k * s / n sampled keys lie above the row's
// k-th key; four standard deviations and four keys more keep theta below it unless the
// sample is far from typical.  0: no useful threshold (theta = 1).
__device__ __forceinline__ uint32_t sample_rank(int k, int s, int n) {
  const float mu = (float)k * (float)s / (float)n;
  const float r = ceilf(mu + 4.0f * sqrtf(mu) + 4.0f);
  return r >= (float)s ? 0u : (uint32_t)r;
}

__device__ __forceinline__ void unpack_q(const uint4* qp, bf16x2 (&q)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = qp[i];
    q[4 * i + 0] = __builtin_bit_cast(bf16x2, v.x);
    q[4 * i + 1] = __builtin_bit_cast(bf16x2, v.y);
    q[4 * i + 2] = __builtin_bit_cast(bf16x2, v.z);
    q[4 * i + 3] = __builtin_bit_cast(bf16x2, v.w);
  }
}

__device__ __forceinline__ void load_q(const uint16_t* qrow, int quarter, bf16x2 (&q)[16]) {
  unpack_q(reinterpret_cast<const uint4*>(qrow) + quarter * 4, q);
}

// Score of the lane's own column of a group (lane = 4 * ent + quarter owns column
// g + 16 * quarter + ent): the scan's arithmetic (dot of each quarter, two lane swaps,
// times the entry scale).
__device__ __forceinline__ float group_score(const ScanGroup& s, const bf16x2 (&q)[16], int quarter) {
  float sc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float v = dot32(s.w[it], q);
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    sc[it] = v;
  }
  const float mine = quarter == 0 ? sc[0] : quarter == 1 ? sc[1] : quarter == 2 ? sc[2] : sc[3];
  return mine * s.sc;
}

// Largest j < n with pre[j] <= v (pre[0] = 0, ascending).
__device__ __forceinline__ int upper_index(const uint32_t* pre, int n, uint32_t v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ k_fscan
struct ScanLds {
  union {
    uint32_t key[kSampRow];               // a row's sample (theta), before any chunk
    struct {                              // per phase parity, per group of 64 columns:
      uint32_t skey[2][kCW][64];          //   its candidates' keys, in column order
      uint16_t soff[2][kCW][64];          //   their columns within the chunk
      uint32_t scnt[2][kCW];              //   how many
      uint32_t gpre[kCW + 1];             // writer: candidates before each group
    };
  };
  uint32_t spre[kMaxRows + 1];            // sample-task prefix per row
  uint32_t cpre[kMaxRows + 1];            // chunk-task prefix per row
  int64_t rbase[kMaxRows];                // seq_base of each row
  int32_t rn[kMaxRows];                   // visible columns of each row
  uint32_t rth[kMaxRows];                 // theta of each row, as the streaming waves read it
  uint32_t rsh[kMaxRows];                 // and its histogram shift
  uint32_t task[4];                       // the chunk task streamed in phase P, at P & 3
  unsigned long long claim;               // (phase << 32) | task, published by streaming wave 0
  __align__(16) uint16_t qre[kMaxReindex * kDIdx];
  Core c;
};

// Histogram shift of a row: candidate bins (key - theta) >> shift over [theta, top key of
// the sample], keys above it in the last bin.  kNoHist: rows without a sampled theta.
constexpr uint32_t kNoHist = 32u;

// One sample task: 16 waves score one group of 64 columns each (stratified over the row)
// into the row's sample; the last task of the row turns the sample into theta (and the
// bin width of the row's candidate histogram).
template <bool CAND>
__device__ __forceinline__ void sample_task(const FsArgs& a, ScanLds& L, int r, int si) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quarter = lane & 3, ent = lane >> 2;
  const int n = L.rn[r], ns = row_samples(n);
  const int b = a.row0 + r;
  const int g = si * kNW + wave;
  long long st = ((2LL * g + 1) * n) / (2LL * ns * kNW) - 32;
  st = st < 0 ? 0 : (st > n - 64 ? n - 64 : st);
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  bf16x2 q[16];
  load_q(a.q + (size_t)b * kDIdx, quarter, q);
  const ScanGroup s = load_group<CAND>(a.codes, a.scale, cand_row, L.rbase[r], (int)st, n - 1, ent, quarter);
  const float score = group_score(s, q, quarter);
  st_ag(&a.samp[(size_t)r * kSampRow + g * 64 + 16 * quarter + ent], s.own_ok ? score_key(score) : 0u);
  wait_vm();
  __syncthreads();
  if (tid == 0) FS_TR(blockIdx.x * 2048 + 2, FS_NOW());
  if (tid == 0)
    L.c.misc[2] = add_ag(&a.roww[r * kRowWords + kRwSamp], 1u) == (uint32_t)(ns - 1) ? 1u : 0u;
  __syncthreads();
  if (L.c.misc[2] == 0u) return;
  if (tid == 0) FS_TR(blockIdx.x * 2048 + 3, FS_NOW() | ((unsigned long long)(r + 1) << 52));
  // the last sample task of the row: theta = the sample key of rank sample_rank; every
  // load of the sample is issued before the first is stored
  const int m = ns * kSampTask;
  uint32_t top = 0u;
  {
    uint32_t v[kSampRow / kT];
#pragma unroll
    for (int u = 0; u < kSampRow / kT; ++u) {
      const int i = tid + kT * u;
      v[u] = i < m ? ld_ag(&a.samp[(size_t)r * kSampRow + i]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kSampRow / kT; ++u) {
      L.key[tid + kT * u] = v[u];
      top = max(top, v[u]);
    }
  }
  uint32_t dummy_s = 0, dummy_mn = 0xffffffffu;
  block_smm(dummy_s, top, dummy_mn, L.c);  // top: the largest sampled key
  if (tid == 0) FS_TR(blockIdx.x * 2048 + 4, FS_NOW());
  const uint32_t rk = sample_rank(a.k, m, n);
  uint32_t th = 1u;
  if (rk > 0u) {
    const Thr t = find_thr<0>([&](int, int i) { return L.key[i]; },
                              [&](int, int i) { return (uint32_t)i; }, m, rk, L.c, blockIdx.x * 2048 + 1500);
    th = (t.nsel == rk && t.tkey > 0u) ? t.tkey : 1u;
  }
  if (tid == 0) FS_TR(blockIdx.x * 2048 + 5, FS_NOW());
  if (tid == 0) {
    uint32_t sh = kNoHist;
    if (th > 1u) {
      const uint32_t range = top - th;
      sh = range == 0u ? 0u : (uint32_t)max(0, 32 - __clz((int)range) - 12);
    }
    st_ag(&a.roww[r * kRowWords + kRwShift], sh);
    wait_vm();  // the shift is visible before theta: whoever sees theta sees the shift
    st_ag(&a.roww[r * kRowWords + kRwTheta], th);
  }
  __syncthreads();
}

__device__ __forceinline__ void decode_task(const ScanLds& L, int rows, uint32_t n_samp,
                                            uint32_t n_tasks, uint32_t task, int& row, int& j) {
  row = -1;
  j = 0;
  if (task < n_tasks) {
    const uint32_t c = task - n_samp;
    row = upper_index(L.cpre, rows, c);
    j = (int)(c - L.cpre[row]);
  }
}

// The claim of phase P + 1, written by the writer in phase P; false if it never arrived
// (status bit 2; cannot happen while the writer runs).
__device__ __forceinline__ bool wait_claim(const FsArgs& a, const ScanLds& L, uint32_t phase,
                                           uint32_t& task) {
  unsigned long long cl;
  uint32_t spins = 0;
  while ((uint32_t)((cl = __hip_atomic_load(&L.claim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >> 32) !=
         phase + 1u) {
    if (++spins > kSpin) {
      if ((threadIdx.x & 63) == 0) atomicOr(&a.ctrl[kCtStatus], 2u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  task = (uint32_t)cl;
  return true;
}

// theta of row r and its histogram shift (sampled rows wait until the row's last sample
// task has set them; the shift is stored before theta).
__device__ __forceinline__ uint32_t row_theta(const FsArgs& a, const ScanLds& L, int r, uint32_t& sh) {
  sh = kNoHist;
  if (row_samples(L.rn[r]) == 0) return 1u;
  uint32_t th, spins = 0;
  while ((th = ld_ag(&a.roww[r * kRowWords + kRwTheta])) == 0u) {
    if (++spins > kSpin) {
      if ((threadIdx.x & 63) == 0) atomicOr(&a.ctrl[kCtStatus], 1u);
      return 1u;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  sh = ld_ag(&a.roww[r * kRowWords + kRwShift]);
  return th;
}

// The 15 streaming waves: score each chunk's columns and keep, per group of 64 columns,
// the keys >= theta in column order in the stage, issuing the next chunk's loads into each
// buffer as soon as it is processed.  Wave 0 claims chunks two phases ahead: the claim of
// phase P + 2 is issued in phase P just before that wave's loads of phase P + 1, so by
// the time it is read (after those loads' first buffer has been waited for) it has
// returned, and only loads precede it in the wave's memory counter.
template <bool CAND>
__device__ __forceinline__ void stream_loop(const FsArgs& a, ScanLds& L, uint32_t t,
                                            uint32_t n_samp, uint32_t n_tasks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int quarter = lane & 3, ent = lane >> 2;
  const int cg = 16 * quarter + ent;               // column of this lane inside a group
  const int src = 4 * (lane & 15) + (lane >> 4);   // lane owning column `lane` of a group
  int cur_row, cur_j;
  decode_task(L, a.rows, n_samp, n_tasks, t, cur_row, cur_j);
  ScanGroup buf[kG];
  int q_row = -1;
  uint32_t th = 1u;
  bf16x2 q[16];
  auto issue = [&](int u, int row, int j) {
    const int n = L.rn[row];
    if (n == 0) return;
    const int b = a.row0 + row;
    const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
    const int g = j * kChunk + (u * kSW + wave) * 64;
    buf[u] = load_group<CAND>(a.codes, a.scale, cand_row, L.rbase[row], min(g, n - 1), n - 1, ent,
                              quarter);
  };
  uint32_t nxt = 0xffffffffu;  // wave 0, lane 0: the claim in flight (the task after next)
  if (cur_row >= 0) {
    if (wave == 0 && lane == 0) nxt = add_ag(&a.ctrl[kCtTask], 1u);
    asm volatile("" ::: "memory");  // the claim is issued before the loads
#pragma unroll
    for (int u = 0; u < kG; ++u) issue(u, cur_row, cur_j);
  }
  uint32_t phase = 0;
  bool pending = false;  // the writer still has the last chunk to write
  while (cur_row >= 0 || pending) {
    int next_row = -1, next_j = 0;
    pending = cur_row >= 0;
    if (cur_row >= 0) {
      const int n = L.rn[cur_row];
      if (q_row != cur_row) {
        load_q(a.q + (size_t)(a.row0 + cur_row) * kDIdx, quarter, q);
        uint32_t sh;
        th = row_theta(a, L, cur_row, sh);
        if (wave == 0 && lane == 0) {
          L.rth[cur_row] = th;
          L.rsh[cur_row] = sh;
        }
        q_row = cur_row;
      }
      const int par = (int)(phase & 1u);
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int g = u * kSW + wave;                  // group index inside the chunk
        const int col = cur_j * kChunk + g * 64 + cg;
        bool cand = false;
        uint32_t key = 0u;
        if (n > 0) {
          const float score = group_score(buf[u], q, quarter);
          key = score_key(score);
          cand = col < n && buf[u].own_ok && key >= th;
        }
        // the candidates of this group in column order
        const bool by_col = __shfl(cand ? 1 : 0, src) != 0;
        const unsigned long long cmask = __ballot(by_col);
        if (cand) {
          const uint32_t rank = (uint32_t)__popcll(cmask & ((1ull << cg) - 1ull));
          L.skey[par][g][rank] = key;
          L.soff[par][g][rank] = (uint16_t)(g * 64 + cg);
        }
        if (lane == 0) L.scnt[par][g] = (uint32_t)__popcll(cmask);
        if (u == 0) {
          if (wave == 0 && lane == 0) FS_TR(blockIdx.x * 2048 + 600 + 3 * (int)min(phase, 99u), FS_NOW());
          uint32_t tn = 0xffffffffu;
          if (wave == 0) {
            if (lane == 0) {  // publish the next task, then claim the one after it
              L.task[(phase + 1u) & 3u] = nxt;
              __hip_atomic_store(&L.claim, ((unsigned long long)(phase + 1u) << 32) | nxt, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
              tn = nxt;
              nxt = nxt < n_tasks ? add_ag(&a.ctrl[kCtTask], 1u) : 0xffffffffu;
            }
            asm volatile("" ::: "memory");  // the claim is issued before the loads below
            tn = __builtin_amdgcn_readfirstlane(tn);
            decode_task(L, a.rows, n_samp, n_tasks, tn, next_row, next_j);
          } else if (wait_claim(a, L, phase, tn)) {
            decode_task(L, a.rows, n_samp, n_tasks, tn, next_row, next_j);
          }
          if (wave == 0 && lane == 0) FS_TR(blockIdx.x * 2048 + 601 + 3 * (int)min(phase, 99u), FS_NOW());
        }
        if (next_row >= 0) issue(u, next_row, next_j);  // this buffer is free again
      }
    }
    if (wave == 0 && lane == 0) FS_TR(blockIdx.x * 2048 + 602 + 3 * (int)min(phase, 99u), FS_NOW());
    ++phase;
    cur_row = next_row;
    cur_j = next_j;
    __syncthreads();
  }
}

// The writer wave: writes the candidates of the chunk streamed in the previous phase (the
// stage, in column order) to that chunk's own region of the row's store (chunk j at
// j * 1920: no reservation), its count, each candidate into the row's histogram and, when
// chained, its Reindex re-scores.  Nothing it issues returns a value, so its stores never
// hold up anything.
template <bool CAND>
__device__ __forceinline__ void writer_loop(const FsArgs& a, ScanLds& L, uint32_t t,
                                            uint32_t n_samp, uint32_t n_tasks) {
  const int lane = threadIdx.x & 63;
  const int quarter = lane & 3, ent = lane >> 2;
  int cur_row, cur_j;
  decode_task(L, a.rows, n_samp, n_tasks, t, cur_row, cur_j);
  int w_row = -1, w_j = 0, w_par = 0;   // chunk whose candidates wait in the stage w_par
  int re_row = -1;
  uint32_t phase = 0;
  while (cur_row >= 0 || w_row >= 0) {
    const int tb = blockIdx.x * 2048 + 16 + 5 * (int)min(phase, 99u);
    if (lane == 0) FS_TR(tb, FS_NOW() | ((unsigned long long)(w_row + 1) << 52));
    if (w_row >= 0) {
      const int b = a.row0 + w_row;
      // candidates of the chunk per group -> their places in the chunk's region
      const uint32_t cnt = lane < kCW ? L.scnt[w_par][lane] : 0u;
      const uint32_t incl = wave_incl_scan(cnt);
      const uint32_t n = __builtin_amdgcn_readlane(incl, 63);
      if (lane < kCW) L.gpre[lane] = incl - cnt;
      if (lane == 0) L.gpre[kCW] = n;
      const uint32_t th = L.rth[w_row], sh = L.rsh[w_row];
      const size_t rb = (size_t)w_row * a.cap + (size_t)w_j * kChunk;
      uint32_t* hist = a.rhist + (size_t)w_row * kBins;
      for (uint32_t e = lane; e < n; e += 64) {
        const int g = upper_index(L.gpre, kCW, e);
        const uint32_t key = L.skey[w_par][g][e - L.gpre[g]];
        const uint32_t off = L.soff[w_par][g][e - L.gpre[g]];
        a.ckey[rb + e] = key;
        a.ccol[rb + e] = (uint32_t)(w_j * kChunk) + off;
        if (sh != kNoHist) atomicAdd(&hist[min((key - th) >> sh, (uint32_t)(kBins - 1))], 1u);
      }
      if (lane == 0) {
        a.ccnt[(size_t)w_row * a.runs + w_j] = n;
        FS_TR(tb + 3, FS_NOW() | ((unsigned long long)n << 48));
      }
      if (!CAND && a.n_re > 0 && n > 0u) {
        // the Reindex layers' re-scores of this chunk's candidates (the scan's arithmetic)
        if (re_row != w_row) {
          for (int i = lane; i < a.n_re * (kDIdx / 8); i += 64) {
            const int l = i / (kDIdx / 8), part = i % (kDIdx / 8);
            reinterpret_cast<uint4*>(L.qre)[i] =
                reinterpret_cast<const uint4*>(a.q_re + ((size_t)l * a.batch + b) * kDIdx)[part];
          }
          re_row = w_row;
        }
        const int64_t sbase = L.rbase[w_row];
        for (uint32_t e0 = 0; e0 < n; e0 += 64) {
          uint4 w4[4];
          float sc4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t e = min(e0 + 16u * u + (uint32_t)ent, n - 1u);
            const int g = upper_index(L.gpre, kCW, e);
            const int64_t entry = sbase + (int64_t)(w_j * kChunk + L.soff[w_par][g][e - L.gpre[g]]);
            w4[u] = *reinterpret_cast<const uint4*>(a.codes + entry * kIdxCodeBytes + quarter * 16);
            sc4[u] = a.scale[entry];
          }
          for (int l = 0; l < a.n_re; ++l) {
            bf16x2 qr[16];
            unpack_q(reinterpret_cast<const uint4*>(L.qre + l * kDIdx) + quarter * 4, qr);
            uint32_t* rk = a.rekey + ((size_t)l * a.rows + w_row) * a.cap + (size_t)w_j * kChunk;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float v = dot32(w4[u], qr);
              v += __shfl_xor(v, 1);
              v += __shfl_xor(v, 2);
              const uint32_t e = e0 + 16u * u + (uint32_t)ent;
              if (quarter == 0 && e < n) rk[e] = score_key(v * sc4[u]);
            }
          }
        }
      }
    }
    if (lane == 0) FS_TR(tb + 4, FS_NOW());
    // the chunk streamed in this phase is written out in the next one
    w_row = cur_row;
    w_j = cur_j;
    w_par = (int)(phase & 1u);
    ++phase;
    __syncthreads();
    // the next phase's chunk: published by streaming wave 0 during the phase just ended
    if (cur_row >= 0) decode_task(L, a.rows, n_samp, n_tasks, L.task[phase & 3u], cur_row, cur_j);
  }
}

template <bool CAND>
__global__ __launch_bounds__(kT) void k_fscan(FsArgs a) {
  __shared__ ScanLds L;
  const int tid = threadIdx.x, wave = tid >> 6;
  if (tid == 0) FS_TR(blockIdx.x * 2048, FS_NOW());
  // per-row facts and the task layout: every row's sample tasks, then its chunks
  if (tid == 0) L.claim = add_ag(&a.ctrl[kCtTask], 1u);
  {
    uint32_t ns = 0, nc = 0;
    if (tid < a.rows) {
      const int b = a.row0 + tid;
      const int n = max(0, min(a.n_valid[b], a.n_cols));
      L.rn[tid] = n;
      L.rbase[tid] = a.seq_base[b];
      ns = (uint32_t)row_samples(n);
      nc = (uint32_t)row_chunks(n);
    }
    uint32_t tns, tnc;
    const uint32_t ps = block_exclusive_scan(ns, L.c.scan, &tns);
    const uint32_t pc = block_exclusive_scan(nc, L.c.scan, &tnc);
    if (tid < a.rows) {
      L.spre[tid] = ps;
      L.cpre[tid] = pc;
    }
    if (tid == 0) {
      L.spre[a.rows] = tns;
      L.cpre[a.rows] = tnc;
    }
  }
  __syncthreads();
  const uint32_t n_samp = L.spre[a.rows], n_tasks = n_samp + L.cpre[a.rows];
  uint32_t t = (uint32_t)L.claim;
  // sample tasks (whole workgroup, one at a time)
  while (t < n_samp) {
    const int r = upper_index(L.spre, a.rows, t);
    __syncthreads();
    if (tid == 0) L.claim = add_ag(&a.ctrl[kCtTask], 1u);
    sample_task<CAND>(a, L, r, (int)(t - L.spre[r]));
    __syncthreads();
    t = (uint32_t)L.claim;
  }
  if (tid == 0) FS_TR(blockIdx.x * 2048 + 1, FS_NOW());
  // chunk tasks: in phase P the streaming waves score chunk t_P into the stage P & 1
  // while the writer wave claims t_{P+1} (published in L.claim with tag P + 1) and writes
  // out the candidates of t_{P-1}; each kind of wave runs a loop of its own (keeping only
  // its own registers) and both meet at one barrier per phase.
  if (wave < kSW) stream_loop<CAND>(a, L, t, n_samp, n_tasks);
  else writer_loop<CAND>(a, L, t, n_samp, n_tasks);
}

// ------------------------------------------------------------------ k_fpick
// Grid: rows x S workgroups; workgroup (r, s) loads every candidate key of row r (in
// column order: chunk after chunk, each chunk's run in column order), finds the row's
// exact threshold (every workgroup of the row reaches the same one), marks the winners in
// a bitmap whose prefix gives each winner's output position, and writes the winners of
// its own slice of chunks.  The chained selections each go to one workgroup of the row.
struct PickLds {
  uint32_t key[kMaxCand];                 // slow path: scratch; Reindex: pool re-scores
  uint32_t off[kMaxRuns + 1];             // first candidate of each chunk (dense, col order)
  uint16_t blk[kMaxCand / 32];            // chunk of the first candidate of each 32-block
  uint32_t bm[kMaxCand / 32 + 1];         // winners, one bit per candidate
  uint32_t wp[kMaxCand / 32 + 1];         // winners before each bitmap word (and the total)
  uint32_t rbm[CSA2_MAX_K / 32 + 1];      // Reindex winners over pool positions
  uint32_t rwp[CSA2_MAX_K / 32 + 1];
  uint32_t pidx[64];                      // candidate index of each directly ranked key
  Core c;
};

// Chunk holding candidate i (i < the row's count).
__device__ __forceinline__ int chunk_of(const PickLds& L, uint32_t i) {
  int j = L.blk[i >> 5];
  while (L.off[j + 1] <= i) ++j;
  return j;
}

// Winners before index i of a bitmap with word prefix wp.
__device__ __forceinline__ uint32_t bits_before(const uint32_t* bm, const uint32_t* wp, uint32_t i) {
  const uint32_t w = i >> 5, b = i & 31u;
  return wp[w] + (uint32_t)__popc(bm[w] & ((1u << b) - 1u));
}
__device__ __forceinline__ bool bit_at(const uint32_t* bm, uint32_t i) { return (bm[i >> 5] >> (i & 31u)) & 1u; }

// wp[w] = set bits in bm[0 .. w) for the words covering m bits, and wp[words] = total.
// Whole workgroup; ends with a barrier.
__device__ __forceinline__ void bitmap_prefix(const uint32_t* bm, uint32_t* wp, int m, Core& C) {
  const int tid = threadIdx.x;
  const int words = (m + 31) / 32;  // <= 768
  const uint32_t c = tid < words ? (uint32_t)__popc(bm[tid]) : 0u;
  uint32_t tot;
  const uint32_t e = block_exclusive_scan(c, C.scan, &tot);
  if (tid < words) wp[tid] = e;
  if (tid == 0) wp[words] = tot;
  __syncthreads();
}

// Marks in L.bm the top-k of the m candidates (key kv[u] of candidate i = threadIdx.x +
// kT * u, ties to the lower index, i.e. the lower column).  With the row's histogram in
// L.c.hist (candidates per bin of (key - theta) >> sh, the last bin open-ended) the bin
// of the k-th key is read off it: keys above the bin win by ballot and the <= 64 keys in
// it are ranked directly.  Otherwise (no histogram, the last bin or a crowded one) the
// general search runs.  Returns the number selected.  Whole workgroup; ends with a barrier.
__device__ __forceinline__ uint32_t pick_marked(const uint32_t (&kv)[kU], int m, uint32_t k,
                                                uint32_t theta, uint32_t sh, PickLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t need = min(k, (uint32_t)m);
  if (sh != kNoHist && need < (uint32_t)m) {
    find_bin_block<kBins / kT>(L.c.hist, need, L.c.scan, L.c.res);  // ends with a barrier
    const uint32_t d = L.c.res[0], above = L.c.res[1], in_bin = L.c.hist[d];
    if (d < (uint32_t)(kBins - 1) && in_bin <= 64u) {
      const uint32_t lo = theta + (d << sh);
      const uint32_t hi = lo + ((1u << sh) - 1u);
      if (tid == 0) L.c.misc[0] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = tid + kT * u;
        const uint32_t key = i < m ? kv[u] : 0u;
        const unsigned long long msk = __ballot(key > hi);
        if (lane == 0) {
          L.bm[(kT * u + 64 * wave) >> 5] = (uint32_t)msk;
          L.bm[((kT * u + 64 * wave) >> 5) + 1] = (uint32_t)(msk >> 32);
        }
        if (key >= lo && key <= hi) {
          const uint32_t slot = atomicAdd(&L.c.misc[0], 1u);
          if (slot < 64u) {
            L.c.pub[slot] = ((unsigned long long)key << 32) | (uint32_t)~(uint32_t)i;
            L.pidx[slot] = (uint32_t)i;
          }
        }
      }
      if (tid == 0) L.bm[kMaxCand / 32] = 0u;
      __syncthreads();
      if (wave == 0) {  // the (need - above) best members of the bin win
        const uint32_t nt = min(L.c.misc[0], 64u);
        const unsigned long long cc = (uint32_t)lane < nt ? L.c.pub[lane] : 0ull;
        const uint32_t chi = (uint32_t)(cc >> 32), clo = (uint32_t)cc;
        uint32_t rk = 0;
        for (uint32_t j = 0; j < nt; ++j) {
          const uint32_t ohi = __builtin_amdgcn_readlane(chi, j);
          const uint32_t olo = __builtin_amdgcn_readlane(clo, j);
          rk += (ohi > chi || (ohi == chi && olo > clo)) ? 1u : 0u;
        }
        if ((uint32_t)lane < nt && rk < need - above) {
          const uint32_t i = L.pidx[lane];
          atomicOr(&L.bm[i >> 5], 1u << (i & 31));
        }
      }
      __syncthreads();
      return need;
    }
  }
  const Thr t = find_thr<kU>([&](int u, int) { return kv[u]; }, [&](int, int i) { return (uint32_t)i; },
                             m, k, L.c);
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = tid + kT * u;
    const unsigned long long msk = __ballot(i < m && selected(t, kv[u], (uint32_t)i));
    if (lane == 0) {
      L.bm[(kT * u + 64 * wave) >> 5] = (uint32_t)msk;
      L.bm[((kT * u + 64 * wave) >> 5) + 1] = (uint32_t)(msk >> 32);
    }
  }
  if (tid == 0) L.bm[kMaxCand / 32] = 0u;
  __syncthreads();
  return t.nsel;
}

// Entries p < n of `row` hold pool positions (written by this workgroup); replaces each by
// the pool entry at that position.  Every load of a step is issued before any is used.
__device__ __forceinline__ void deref_pool(int32_t* row, int n, const int32_t* pool) {
  wait_vm();
  __syncthreads();
  const int tid = threadIdx.x;
  uint32_t v[kPU];
#pragma unroll
  for (int u = 0; u < kPU; ++u) {
    const int p = tid + u * kT;
    v[u] = p < n ? ld_ag(reinterpret_cast<const uint32_t*>(row) + p) : 0u;
  }
#pragma unroll
  for (int u = 0; u < kPU; ++u)
    if (tid + u * kT < n) v[u] = ld_ag(reinterpret_cast<const uint32_t*>(pool) + v[u]);
#pragma unroll
  for (int u = 0; u < kPU; ++u)
    if (tid + u * kT < n) row[tid + u * kT] = (int32_t)v[u];
}

// Slow path of a row whose theta turned out too high or too low: this workgroup alone
// scores every column again and stores every key at store index = column (0 for a
// candidate hole), with the Reindex re-scores when chained.
template <bool CAND>
__device__ __forceinline__ void rescan_row(const FsArgs& a, int r, int n) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quarter = lane & 3, ent = lane >> 2;
  const int b = a.row0 + r;
  const int64_t base = a.seq_base[b];
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  uint32_t* ck = a.ckey + (size_t)r * a.cap;
  uint32_t* cc = a.ccol + (size_t)r * a.cap;
  bf16x2 q[16];
  load_q(a.q + (size_t)b * kDIdx, quarter, q);
  for (int g = wave * 64; g < n; g += kT) {
    const ScanGroup s = load_group<CAND>(a.codes, a.scale, cand_row, base, g, n - 1, ent, quarter);
    const float score = group_score(s, q, quarter);
    const int col = g + 16 * quarter + ent;
    if (col < n) {
      st_ag(&ck[col], s.own_ok ? score_key(score) : 0u);
      st_ag(&cc[col], (uint32_t)col);
    }
    for (int l = 0; l < a.n_re; ++l) {
      bf16x2 qr[16];
      load_q(a.q_re + ((size_t)l * a.batch + b) * kDIdx, quarter, qr);
      const float rs = group_score(s, qr, quarter);
      if (col < n) st_ag(&a.rekey[((size_t)l * a.rows + r) * a.cap + col], score_key(rs));
    }
  }
  wait_vm();
  __syncthreads();
}

// The slow path of a row (its theta was too high, or too many keys passed it): every key
// of the row again, the store then in column order (store index = column), and every
// selection of the row from global memory by this one workgroup.  Out of line, with the
// arguments by value, so the fast path keeps its registers.
template <bool CAND>
__device__ __noinline__ void slow_select(FsArgs a, PickLds* Lp, int r) {
  PickLds& L = *Lp;
  const int tid = threadIdx.x;
  const int b = a.row0 + r;
  const int n_row = max(0, min(a.n_valid[b], a.n_cols));
  const uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  int32_t* orow = a.out + (size_t)b * a.k;
  float* srow = a.sout ? a.sout + (size_t)b * a.k : nullptr;
  uint32_t* pm = a.n_re > 0 ? a.pmap + (size_t)r * CSA2_MAX_K : nullptr;
  rescan_row<CAND>(a, r, n_row);
  if (tid == 0) atomicAdd(&a.ctrl[kCtSlow], 1u);
  const int m = n_row;
  auto K = [&](int, int i) -> uint32_t { return ld_ag(&ck[i]); };
  auto X = [&](int, int i) -> uint32_t { return (uint32_t)i; };
  const Thr tp = find_thr<0>(K, X, m, (uint32_t)a.k, L.c);
  emit_ordered(
      m, [&](int i) { return selected(tp, ld_ag(&ck[i]), (uint32_t)i); },
      [&](uint32_t rank, int i) {
        orow[rank] = CAND ? cand_row[i] : i;
        if (srow) srow[rank] = key_score(ld_ag(&ck[i]));
        if (pm) st_ag(&pm[rank], (uint32_t)i);
      },
      L.c);
  for (int p = (int)tp.nsel + tid; p < a.k; p += kT) {
    orow[p] = -1;
    if (srow) srow[p] = -__builtin_inff();
  }
  if (a.own_k > 0) {
    const Thr to = find_thr<0>(K, X, m, (uint32_t)a.own_k, L.c);
    int32_t* own = a.own_out + (size_t)b * a.own_k;
    emit_ordered(
        m, [&](int i) { return selected(to, ld_ag(&ck[i]), (uint32_t)i); },
        [&](uint32_t rank, int i) { own[rank] = CAND ? cand_row[i] : i; }, L.c);
    for (int p = (int)to.nsel + tid; p < a.own_k; p += kT) own[p] = -1;
  }
  // Reindex layers: the top-re_k of the pool's re-scores by pool position
  const int P = (int)tp.nsel;
  if (a.n_re > 0) {
    const int32_t* pool = a.out + (size_t)b * a.k;
    wait_vm();
    __syncthreads();
    uint32_t sl[kPU];
#pragma unroll
    for (int u = 0; u < kPU; ++u) sl[u] = tid + u * kT < P ? ld_ag(&pm[tid + u * kT]) : 0u;
    for (int l = 0; l < a.n_re; ++l) {
      const uint32_t* rk = a.rekey + ((size_t)l * a.rows + r) * a.cap;
      uint32_t v[kPU];
#pragma unroll
      for (int u = 0; u < kPU; ++u) v[u] = tid + u * kT < P ? ld_ag(&rk[sl[u]]) : 0u;
#pragma unroll
      for (int u = 0; u < kPU; ++u)
        if (tid + u * kT < P) L.key[tid + u * kT] = v[u];
      __syncthreads();
      const Thr tr = find_thr<0>([&](int, int p) { return L.key[p]; },
                                 [&](int, int p) { return (uint32_t)p; }, P, (uint32_t)a.re_k, L.c);
      int32_t* orr = a.re_out + ((size_t)l * a.batch + b) * a.re_k;
      float* srr = a.re_sout ? a.re_sout + ((size_t)l * a.batch + b) * a.re_k : nullptr;
      emit_ordered(
          P, [&](int p) { return selected(tr, L.key[p], (uint32_t)p); },
          [&](uint32_t rank, int p) {
            st_ag(reinterpret_cast<uint32_t*>(orr) + rank, (uint32_t)p);
            if (srr) srr[rank] = key_score(L.key[p]);
          },
          L.c);
      deref_pool(orr, (int)tr.nsel, pool);
      for (int p = (int)tr.nsel + tid; p < a.re_k; p += kT) {
        orr[p] = -1;
        if (srr) srr[p] = -__builtin_inff();
      }
      __syncthreads();
    }
  }
}

// Reindex layer l of row r on the fast path: the top-re_k of the pool's re-scores (pool
// position = winner rank among the candidates; ties to the lower position), written as
// pool entries in pool order.  L.bm / L.wp mark the pool; gs[u] is candidate i's place in
// the store.
// Store slot of candidate i (chunk j's run starts at j * 1920).
__device__ __forceinline__ uint32_t slot_of(const PickLds& L, uint32_t i) {
  const int j = chunk_of(L, i);
  return (uint32_t)j * kChunk + (i - L.off[j]);
}

template <bool CAND>
__device__ __forceinline__ void pick_reindex(const FsArgs& a, PickLds& L, int r, int l, int m, uint32_t P) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = a.row0 + r;
  const uint32_t* rk = a.rekey + ((size_t)l * a.rows + r) * a.cap;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = tid + kT * u;
      v[u] = (i < m && bit_at(L.bm, (uint32_t)i)) ? rk[slot_of(L, (uint32_t)i)] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = tid + kT * u;
      if (i < m && bit_at(L.bm, (uint32_t)i)) L.key[bits_before(L.bm, L.wp, (uint32_t)i)] = v[u];
    }
  }
  __syncthreads();
  const Thr tr = find_thr<kPU>([&](int, int p) { return L.key[p]; }, [&](int, int p) { return (uint32_t)p; },
                               (int)P, (uint32_t)a.re_k, L.c, (1 << 20) - 131072 + (int)blockIdx.x * 16);
#pragma unroll
  for (int u = 0; u < kPU; ++u) {
    const int p = tid + kT * u;
    const unsigned long long msk = __ballot(p < (int)P && selected(tr, L.key[p], (uint32_t)p));
    if (lane == 0) {
      L.rbm[(kT * u + 64 * wave) >> 5] = (uint32_t)msk;
      L.rbm[((kT * u + 64 * wave) >> 5) + 1] = (uint32_t)(msk >> 32);
    }
  }
  if (tid == 0) L.rbm[CSA2_MAX_K / 32] = 0u;
  __syncthreads();
  bitmap_prefix(L.rbm, L.rwp, (int)P, L.c);
  int32_t* orr = a.re_out + ((size_t)l * a.batch + b) * a.re_k;
  float* srr = a.re_sout ? a.re_sout + ((size_t)l * a.batch + b) * a.re_k : nullptr;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  for (uint32_t i = tid; i < (uint32_t)m; i += kT) {  // few winners: one load each at most
    if (!bit_at(L.bm, i)) continue;
    const uint32_t p = bits_before(L.bm, L.wp, i);
    if (!bit_at(L.rbm, p)) continue;
    const uint32_t rank = bits_before(L.rbm, L.rwp, p);
    const uint32_t col = cc[slot_of(L, i)];
    orr[rank] = CAND ? cand_row[col] : (int32_t)col;
    if (srr) srr[rank] = key_score(L.key[p]);
  }
  for (int p = (int)tr.nsel + tid; p < a.re_k; p += kT) {
    orr[p] = -1;
    if (srr) srr[p] = -__builtin_inff();
  }
  __syncthreads();
}

// The Full layer's own top-own_k of the m candidates of row r (ties to the lower column), in
// column order.
template <bool CAND>
__device__ __forceinline__ void pick_own(const FsArgs& a, PickLds& L, int r, int m, uint32_t theta,
                                         uint32_t sh) {
  const int tid = threadIdx.x;
  const int b = a.row0 + r;
  const uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  const uint32_t* hist = a.rhist + (size_t)r * kBins;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  uint32_t kv[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = tid + kT * u;
    kv[u] = i < m ? ck[slot_of(L, (uint32_t)i)] : 0u;
  }
#pragma unroll
  for (int u = 0; u < kBins / kT; ++u) L.c.hist[tid + kT * u] = sh != kNoHist ? hist[tid + kT * u] : 0u;
  __syncthreads();
  const uint32_t n_own = pick_marked(kv, m, (uint32_t)a.own_k, theta, sh, L);
  bitmap_prefix(L.bm, L.wp, m, L.c);
  int32_t* own = a.own_out + (size_t)b * a.own_k;
  for (uint32_t i = tid; i < (uint32_t)m; i += kT) {
    if (!bit_at(L.bm, i)) continue;
    const uint32_t col = cc[slot_of(L, i)];
    own[bits_before(L.bm, L.wp, i)] = CAND ? cand_row[col] : (int32_t)col;
  }
  for (int p = (int)n_own + tid; p < a.own_k; p += kT) own[p] = -1;
}

// Grid: rows x (S + R): per row, S workgroups that each write a slice of the pool, then R
// workgroups with one chained selection each (Reindex layer 0 .. n_re - 1, then the Full
// layer's own top-k).
template <bool CAND>
__global__ __launch_bounds__(kT) void k_fpick(FsArgs a, int S) {
  __shared__ PickLds L;
  const int tid = threadIdx.x;
  const int R = a.n_re + (a.own_k > 0 ? 1 : 0);
  const int r = (int)blockIdx.x / (S + R), s = (int)blockIdx.x % (S + R);
  const int tb = (1 << 20) - 65536 + (int)blockIdx.x * 8;
  if (tid == 0) FS_TR(tb, FS_NOW());
  const int b = a.row0 + r;
  const int n_row = max(0, min(a.n_valid[b], a.n_cols));
  const int nch = row_chunks(n_row);
  const uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  int32_t* orow = a.out + (size_t)b * a.k;
  float* srow = a.sout ? a.sout + (size_t)b * a.k : nullptr;
  uint32_t* hist = a.rhist + (size_t)r * kBins;
  if (blockIdx.x == 0 && tid == 0) a.ctrl[kCtTask] = 0u;  // the scan that counted on it has ended
  // one round of loads: theta, the shift, the histogram and each chunk's count
  const bool sampled = row_samples(n_row) > 0;
  const uint32_t theta = sampled ? a.roww[r * kRowWords + kRwTheta] : 1u;
  const uint32_t sh = sampled ? a.roww[r * kRowWords + kRwShift] : kNoHist;
  uint32_t h[kBins / kT];
#pragma unroll
  for (int u = 0; u < kBins / kT; ++u) h[u] = sampled ? hist[tid + kT * u] : 0u;  // read again by the own-top-k workgroup
  const uint32_t c0 = 2 * tid < nch ? a.ccnt[(size_t)r * a.runs + 2 * tid] : 0u;
  const uint32_t c1 = 2 * tid + 1 < nch ? a.ccnt[(size_t)r * a.runs + 2 * tid + 1] : 0u;
#pragma unroll
  for (int u = 0; u < kBins / kT; ++u) L.c.hist[tid + kT * u] = h[u];
  uint32_t m_all;
  {
    const uint32_t e = block_exclusive_scan(c0 + c1, L.c.scan, &m_all);
    if (2 * tid < nch) L.off[2 * tid] = e;
    if (2 * tid + 1 < nch) L.off[2 * tid + 1] = e + c0;
    if (tid == 0) L.off[nch] = m_all;
  }
  __syncthreads();
  if (tid == 0) FS_TR(tb + 5, FS_NOW());
  const bool fast =
      m_all <= (uint32_t)kMaxCand && !(theta > 1u && m_all < (uint32_t)min(a.k, n_row));
  if (fast) {
    const int m = (int)m_all;
    for (int w = tid; w < (m + 31) / 32; w += kT) L.blk[w] = (uint16_t)upper_index(L.off, nch, 32u * w);
    __syncthreads();
    if (tid == 0) FS_TR(tb + 6, FS_NOW());
    // every candidate key of the row (candidate i = tid + kT * u), then the pool (or the only
    // selection) marked in L.bm
    uint32_t n_pool;
    {
      uint32_t kv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = tid + kT * u;
        kv[u] = i < m ? ck[slot_of(L, (uint32_t)i)] : 0u;
      }
      if (tid == 0) FS_TR(tb + 1, FS_NOW());
      n_pool = pick_marked(kv, m, (uint32_t)a.k, theta, sh, L);
    }
    bitmap_prefix(L.bm, L.wp, m, L.c);
    if (tid == 0) FS_TR(tb + 2, FS_NOW());
    if (s < S) {  // this workgroup's slice of chunks
      const int j0 = (int)((long long)s * nch / S), j1 = (int)((long long)(s + 1) * nch / S);
      const uint32_t i1 = L.off[j1];
      for (uint32_t i = L.off[j0] + tid; i < i1; i += kT) {
        if (!bit_at(L.bm, i)) continue;
        const uint32_t slot = slot_of(L, i);
        const uint32_t col = cc[slot];
        const uint32_t pos = bits_before(L.bm, L.wp, i);
        orow[pos] = CAND ? cand_row[col] : (int32_t)col;
        if (srow) srow[pos] = key_score(ck[slot]);
      }
      if (s == 0)
        for (int p = (int)n_pool + tid; p < a.k; p += kT) {
          orow[p] = -1;
          if (srow) srow[p] = -__builtin_inff();
        }
      if (tid == 0) FS_TR(tb + 3, FS_NOW());
    } else if (s - S < a.n_re) {
      pick_reindex<CAND>(a, L, r, s - S, m, n_pool);
    } else {
      pick_own<CAND>(a, L, r, m, theta, sh);
    }
  } else if (s == 0) {
    slow_select<CAND>(a, &L, r);
  }
  if (tid == 0) FS_TR(tb + 4, FS_NOW());
  // the last workgroup of the row returns the row's counters and histogram to zero (every
  // workgroup of the row has read them by then)
  wait_vm();
  __syncthreads();
  if (tid == 0) L.c.misc[4] = add_ag(&a.roww[r * kRowWords + kRwDone], 1u) == (uint32_t)(S + R - 1) ? 1u : 0u;
  __syncthreads();
  if (L.c.misc[4] != 0u) {
    if (sampled)
      for (int i = tid; i < kBins; i += kT) hist[i] = 0u;
    if (tid < kRowWords) a.roww[r * kRowWords + tid] = 0u;
  }
}

// ---------------------------------------------------------------------------- host side
constexpr int kMaxDevices = 64;

// Scan workgroups resident per device at once: the persistent grid's size (correctness
// does not depend on it).  Immutable device properties, cached once per device.
int fs_capacity() {
  static int cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (cache[dev] > 0) return cache[dev];
  int per_cu_a = 0, per_cu_b = 0, n_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_a, reinterpret_cast<const void*>(k_fscan<false>),
                                                   kT, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_b, reinterpret_cast<const void*>(k_fscan<true>),
                                                   kT, 0) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cache[dev] = max(1, min(per_cu_a, per_cu_b)) * n_cu;
  return cache[dev];
}

struct FsShape {
  int runs, rows_ws;
  size_t cap;
};

FsShape fs_shape(int batch, int n_cols, bool chain) {
  FsShape s;
  s.runs = (n_cols + kChunk - 1) / kChunk;
  s.cap = (size_t)s.runs * kChunk;
  s.rows_ws = min(batch, chain ? kChainRows : kMaxRows);
  return s;
}

struct FsParts {
  uint32_t *ctrl, *roww, *samp, *ccnt, *ckey, *ccol, *rekey, *pmap, *rhist;
  size_t bytes;
};

// Workspace: [ctrl 256 B][per row 64 B][samples][histograms][chunk counts][candidate keys][their
// columns] and, for a chain, [their Reindex re-scores][pool -> store index].
FsParts fs_carve(char* p, const FsShape& s, bool chain) {
  FsParts f{};
  size_t off = 0;
  auto take = [&](size_t n) {
    uint32_t* q = p ? reinterpret_cast<uint32_t*>(p + off) : nullptr;
    off += align_up(n, 256);
    return q;
  };
  const size_t R = (size_t)s.rows_ws;
  f.ctrl = take(256);
  f.roww = take(R * kRowWords * 4);
  f.samp = take(R * kSampRow * 4);
  f.rhist = take(R * kBins * 4);
  f.ccnt = take(R * s.runs * 4);
  f.ckey = take(R * s.cap * 4);
  f.ccol = take(R * s.cap * 4);
  if (chain) {
    f.rekey = take((size_t)kMaxReindex * R * s.cap * 4);
    f.pmap = take(R * CSA2_MAX_K * 4);
  }
  f.bytes = off;
  return f;
}

}  // namespace

#ifdef CSA2_FS_TRACE
extern "C" int csa2_fs_trace_copy(void* host, size_t n) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_fs_trace), n * 8) == hipSuccess ? 0 : -1;
}
extern "C" int csa2_fs_trace_zero() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_fs_trace)) != hipSuccess) return -1;
  return hipMemset(p, 0, sizeof(unsigned long long) << 20) == hipSuccess ? 0 : -1;
}
#endif

bool fsel_fits(int n_cols) { return n_cols >= 1 && n_cols <= kMaxRuns * kChunk; }

size_t fsel_ws_bytes(int batch, int n_cols, bool chain) {
  return fs_carve(nullptr, fs_shape(batch, n_cols, chain), chain).bytes;
}

hipError_t launch_fsel(const uint16_t* q, const uint8_t* codes, const float* scale,
                       const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                       int batch, int n_cols, int k, int32_t* out, float* sout, int own_k,
                       int32_t* own_out, const uint16_t* q_re, int n_re, int re_k,
                       int32_t* re_out, float* re_sout, bool chain_ws, void* ws,
                       hipStream_t stream) {
  const FsShape s = fs_shape(batch, n_cols, chain_ws);
  const FsParts f = fs_carve(static_cast<char*>(ws), s, chain_ws);
  const int cap_wg = fs_capacity();
  if (cap_wg <= 0) return hipErrorInvalidDevice;
  FsArgs a{};
  a.q = q;
  a.codes = codes;
  a.scale = scale;
  a.seq_base = seq_base;
  a.n_valid = n_valid;
  a.cand = cand;
  a.n_cols = n_cols;
  a.runs = s.runs;
  a.batch = batch;
  a.k = k;
  a.out = out;
  a.sout = sout;
  a.own_k = own_out ? own_k : 0;
  a.own_out = own_out;
  a.n_re = n_re;
  a.re_k = re_k;
  a.q_re = q_re;
  a.re_out = re_out;
  a.re_sout = re_sout;
  a.ctrl = f.ctrl;
  a.roww = f.roww;
  a.samp = f.samp;
  a.ccnt = f.ccnt;
  a.ckey = f.ckey;
  a.ccol = f.ccol;
  a.rekey = f.rekey;
  a.pmap = f.pmap;
  a.rhist = f.rhist;
  a.cap = s.cap;
  for (int r0 = 0; r0 < batch; r0 += s.rows_ws) {
    a.row0 = r0;
    a.rows = min(s.rows_ws, batch - r0);
    const long long tasks = (long long)a.rows * (s.runs + kMaxSampTasks);
    const int grid = (int)min((long long)cap_wg, tasks);
    // picking workgroups per row: about one per compute unit in all, at most one per chunk
    const int S = max(1, min(s.runs, cap_wg / a.rows));
    const int R = a.n_re + (a.own_k > 0 ? 1 : 0);
    if (cand) {
      hipLaunchKernelGGL(k_fscan<true>, dim3(grid), dim3(kT), 0, stream, a);
      hipLaunchKernelGGL(k_fpick<true>, dim3(a.rows * (S + R)), dim3(kT), 0, stream, a, S);
    } else {
      hipLaunchKernelGGL(k_fscan<false>, dim3(grid), dim3(kT), 0, stream, a);
      hipLaunchKernelGGL(k_fpick<false>, dim3(a.rows * (S + R)), dim3(kT), 0, stream, a, S);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
