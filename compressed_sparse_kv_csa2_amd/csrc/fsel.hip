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
// Design: a segmented scan, then a selection over the survivors.  The pool is 1.6 % of a
// 2^20-entry row, so the scan need not keep every key until the row's threshold is known:
// each segment of a row keeps only as many of its best keys as the row's top-k can
// plausibly hold there, and a second launch selects the exact top-k among them.
//   k_fseg, one workgroup per (row, segment of `seg` columns; seg a power of two in
//   [1024, 16384], the longest that still gives every compute unit a workgroup):
//   * scores its columns into LDS (the Full scan's arithmetic), counting the valid ones
//     and their largest key;
//   * keeps every key at or above the lower edge of the 4,096-value bin holding its
//     seg_keep-th key (bins over the 2^24 key values below the largest, then over the rest
//     when that window holds too few): whole bins, so equal keys stay together and every
//     key left out is below every key kept;
//   * writes the kept keys and columns in column order to its own run of the row's store
//     (ranks from wave ballots, no atomics), and their count, flagged when keys were left
//     out; when chained, the kept entries' Reindex re-scores follow.
//   k_fpick, rows x (S + R) workgroups, S slices of the output and R chained selections:
//   * every workgroup loads the row's segment counts, their prefix (the dense index of the
//     candidates in column order), each candidate's store slot, then all of its keys;
//   * the k-th composite (key, lower column first) comes from a histogram of the 2^24 key
//     values below the largest and one of the exact values in the bin that holds it (the
//     general digit-by-digit search when the window does not hold it); one ballot pass
//     marks the winners in a bitmap whose prefix is each winner's output position;
//   * exactness: a flagged segment whose kept keys all won may have left a winner out;
//     then (or when the candidates exceed what the selection holds) the row is scored
//     again keeping every key (slow, counted in the workspace's status block);
//   * slices write their share of the output; a chained selection (own top-k, or a
//     Reindex layer's top-k over the pool's re-scores, in pool order) runs in one
//     workgroup of its own.
// The launch boundary orders the candidate stores before the selection, and no workgroup
// waits on another.  The last workgroup of a row returns its counter to zero, so the
// workspace needs no clearing between calls.
#include <cmath>

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
constexpr int kSeg = 16384;               // columns per scan segment at most (keys in LDS)
constexpr int kSegMin = 1024;             // and at least
constexpr int kSegU = kSeg / kT;          // segment keys per thread
constexpr int kMaxCand = 24576;           // candidates the selection holds (LDS + registers)
constexpr int kU = kMaxCand / kT;         // candidates per thread
constexpr int kPU = CSA2_MAX_K / kT;      // pool entries per thread
constexpr int kMaxRows = 256;             // rows per launch
constexpr int kMaxRuns = 2048;            // segments per row
constexpr int kBins = 4096;
constexpr int kRowWords = 16;             // per-row counters (64 bytes)
constexpr int kRwDone = 0;
constexpr int kCtStatus = 0, kCtSlow = 2;
constexpr uint32_t kTrunc = 0x80000000u;  // segment count flag: the segment kept only its top keys
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
// A value every lane of the wave holds alike, moved to a scalar register.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

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
  const float* smat;          // scores already computed (see smat_at) or null
  int smat_rows;              // rows of the score matrix
  int n_cols, runs;           // columns, segments per row at most
  int seg;                    // columns per segment (a power of two in [1024, 16384])
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
  uint32_t* ctrl;             // status, -, rows re-scanned
  uint32_t* roww;             // [rows][16]: picking workgroups done
  uint32_t* ccnt;             // [rows][runs] candidates of each segment (| kTrunc when truncated)
  uint32_t* ckey;             // [rows][cap] candidate keys: segment j's run (column order) at j * seg
  uint32_t* ccol;             // [rows][cap] their columns
  uint32_t* rekey;            // [4][rows][cap] their Reindex re-scores (chain)
  uint32_t* pmap;             // [rows][16384] store index of each pool entry (chain, slow path)
  size_t cap;                 // per-row store: runs * seg
};

// LDS the exact-threshold search and the ordered emission share.
struct Core {
  uint32_t hist[kBins + 64];  // + one overflow bin per lane (never read)
  unsigned long long pub[64];
  uint32_t scan[32];
  uint32_t red[3 * kNW];
  uint32_t res[4];
  uint32_t misc[8];
};

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
#pragma unroll 4
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

// Bin of the need-th largest element of h[0 .. 4 kT) (thread t owns the 4 bins just below
// 4 (kT - t); one block scan orders them from the top).  With clamp, need becomes
// min(need, total) first.  res[0] = bin, res[1] = elements in higher bins, res[2] = total,
// res[3] = need (after the clamp).  Ends with a barrier.
__device__ __forceinline__ void find_bin4(const uint32_t* h, uint32_t need, bool clamp, Core& C) {
  const int tid = threadIdx.x;
  const int top = 4 * (kT - tid);
  uint32_t c[4];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = h[top - 1 - i];
    sum += c[i];
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(sum, C.scan, &total);
  if (clamp) need = min(need, total);
  if (tid == 0) {
    C.res[0] = 0u;
    C.res[1] = 0u;
    C.res[2] = total;
    C.res[3] = need;
  }
  __syncthreads();
  if (need > 0u && excl < need && need <= excl + sum) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (acc + c[i] >= need) {
        C.res[0] = (uint32_t)(top - 1 - i);
        C.res[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
}

// Largest of v over a wave (DPP row shifts and broadcasts; lane 63 ends with it).
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  int x = (int)v;
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = (int)max((unsigned)x, (unsigned)__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Sum and largest of (s, mx) over the workgroup.  Ends with a barrier.
__device__ __forceinline__ void block_sum_max(uint32_t& s, uint32_t& mx, Core& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(s), 63);
  const uint32_t wm = wave_max_dpp(mx);
  if (lane == 0) {
    L.red[wave] = ws;
    L.red[kNW + wave] = wm;
  }
  __syncthreads();
  uint32_t a = 0u, b = 0u;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    a += L.red[w];
    b = max(b, L.red[kNW + w]);
  }
  s = uni(a);
  mx = uni(b);
  __syncthreads();
}

// The need-th largest composite (key, then lower x first) among elements i < m with a
// non-zero key K(u, i) and unique tie index X(u, i), need = min(k, #non-zero).  One sweep
// finds the count and the largest key; then 4,096-bin histograms of windows [lo, hi]: the
// first holds the 2^24 key values up to the largest, so a top-k's threshold bin usually
// holds a few keys; a window with fewer than need members hands them all over as above the
// threshold and the next window is everything below it; otherwise the next window is the
// threshold's bin, until at most 64 members remain and wave 0 ranks them directly.  More
// than 64 equal keys are ranked by ~x the same way.  Whole workgroup; ends with a barrier.
template <int U, class KF, class XF>
__device__ __forceinline__ Thr find_thr_any(KF K, XF X, int m, uint32_t k, Core& L, int tr = -1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Thr t;
  t.tkey = 0u;
  t.tx = 0u;
  if (tr >= 0 && tid == 0) FS_TR(tr, FS_NOW());
  uint32_t c = 0, mx = 0;
  for_mine<U>(m, [&](int u, int i) {
    const uint32_t v = K(u, i);
    if (v) {
      ++c;
      mx = max(mx, v);
    }
  });
  block_sum_max(c, mx, L);
  t.total = c;
  uint32_t need = min(k, c);
  t.nsel = need;
  if (need == c) return t;  // every non-zero key (or none)
  uint32_t hi = mx, lo = mx >= (1u << 24) ? mx - ((1u << 24) - 1u) : 1u, tkey = 0u;
  bool xphase = false;
  uint32_t cnt_in = 0xffffffffu;
  auto member = [&](int u, int i, uint32_t& v) -> bool {
    const uint32_t key = K(u, i);
    if (!xphase) {
      v = key;
      return key != 0u && key >= lo && key <= hi;
    }
    if (key != tkey) return false;
    v = ~X(u, i);
    return v >= lo && v <= hi;
  };
  for (int pass = 0; pass < 12; ++pass) {
    if (!xphase && lo == hi && cnt_in > 64u) {  // more than 64 equal keys: rank them by ~x
      xphase = true;
      tkey = lo;
      lo = 0u;
      hi = 0xffffffffu;
    }
    const uint32_t range = hi - lo;
    const int sh = range == 0u ? 0 : max(0, 32 - __clz((int)range) - 12);
    for (int i = tid; i < kBins; i += kT) L.hist[i] = 0u;
    __syncthreads();
    for_mine<U>(m, [&](int u, int i) {
      uint32_t v;
      if (member(u, i, v)) atomicAdd(&L.hist[(v - lo) >> sh], 1u);
    });
    __syncthreads();
    find_bin4(L.hist, need, false, L);  // ends with a barrier
    const uint32_t in_window = uni(L.res[2]);
    if (tr >= 0 && tid == 0 && pass < 8) FS_TR(tr + 1 + pass, FS_NOW() | ((unsigned long long)in_window << 44));
    if (in_window < need) {  // the threshold lies below this window
      need -= in_window;
      hi = lo - 1u;
      lo = xphase ? 0u : 1u;
      cnt_in = 0xffffffffu;
      __syncthreads();
      continue;
    }
    const uint32_t d = uni(L.res[0]);
    need -= uni(L.res[1]);
    cnt_in = uni(L.hist[d]);
    const uint32_t nlo = lo + (d << sh);
    hi = (uint32_t)min((unsigned long long)hi, (unsigned long long)nlo + (1ull << sh) - 1ull);
    lo = nlo;
    __syncthreads();  // L.hist and L.res are read before they are rewritten
    if (cnt_in <= 64u) break;
  }
  // rank the <= 64 remaining members directly
  if (tid == 0) L.misc[0] = 0u;
  __syncthreads();
  for_mine<U>(m, [&](int u, int i) {
    uint32_t v;
    if (member(u, i, v)) {
      const uint32_t slot = atomicAdd(&L.misc[0], 1u);
      if (slot < 64u) L.pub[slot] = ((unsigned long long)K(u, i) << 32) | (uint32_t)~X(u, i);
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
  t.tkey = uni(L.res[2]);
  t.tx = uni(L.res[3]);
  if (tr >= 0 && tid == 0) FS_TR(tr + 10, FS_NOW());
  __syncthreads();
  return t;
}

// Register form of the same search for U > 0: each thread's U keys (element i = tid + kT * u)
// are read once into registers, and every sweep is straight-line code over them.  K must
// return 0 for i >= m.
template <int U, class KF, class XF>
__device__ __forceinline__ Thr find_thr(KF K, XF X, int m, uint32_t k, Core& L, int tr = -1) {
  if constexpr (U == 0) {
    return find_thr_any<0>(K, X, m, k, L, tr);
  } else {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    Thr t;
    t.tkey = 0u;
    t.tx = 0u;
    if (tr >= 0 && tid == 0) FS_TR(tr, FS_NOW());
    uint32_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kk[u] = K(u, tid + kT * u);
    uint32_t c = 0, mx = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      c += kk[u] != 0u ? 1u : 0u;
      mx = max(mx, kk[u]);
    }
    block_sum_max(c, mx, L);
    t.total = c;
    uint32_t need = min(k, c);
    t.nsel = need;
    if (need == c) return t;  // every non-zero key (or none)
    uint32_t hi = mx, lo = mx >= (1u << 24) ? mx - ((1u << 24) - 1u) : 1u, tkey = 0u;
    bool xphase = false;
    uint32_t cnt_in = 0xffffffffu;
    for (int pass = 0; pass < 12; ++pass) {
      if (!xphase && lo == hi && cnt_in > 64u) {  // more than 64 equal keys: rank them by ~x
        xphase = true;
        tkey = lo;
        lo = 0u;
        hi = 0xffffffffu;
      }
      const uint32_t range = hi - lo;
      const int sh = range == 0u ? 0 : max(0, 32 - __clz((int)range) - 12);
#pragma unroll
      for (int i = 0; i < kBins / kT; ++i) L.hist[tid + kT * i] = 0u;
      __syncthreads();
      if (!xphase) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t v = kk[u];
          if (v != 0u && v >= lo && v <= hi) atomicAdd(&L.hist[(v - lo) >> sh], 1u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t v = ~X(u, tid + kT * u);
          if (kk[u] == tkey && v >= lo && v <= hi) atomicAdd(&L.hist[(v - lo) >> sh], 1u);
        }
      }
      __syncthreads();
      find_bin4(L.hist, need, false, L);  // ends with a barrier
      const uint32_t in_window = L.res[2];
      if (tr >= 0 && tid == 0 && pass < 8) FS_TR(tr + 1 + pass, FS_NOW() | ((unsigned long long)in_window << 44));
      if (in_window < need) {  // the threshold lies below this window
        need -= in_window;
        hi = lo - 1u;
        lo = xphase ? 0u : 1u;
        cnt_in = 0xffffffffu;
        __syncthreads();
        continue;
      }
      const uint32_t d = uni(L.res[0]);
      need -= uni(L.res[1]);
      cnt_in = uni(L.hist[d]);
      const uint32_t nlo = lo + (d << sh);
      hi = (uint32_t)min((unsigned long long)hi, (unsigned long long)nlo + (1ull << sh) - 1ull);
      lo = nlo;
      __syncthreads();  // L.hist and L.res are read before they are rewritten
      if (cnt_in <= 64u) break;
    }
    // rank the <= 64 remaining members directly
    if (tid == 0) L.misc[0] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t key = kk[u];
      const uint32_t x = X(u, tid + kT * u);
      const uint32_t v = xphase ? ~x : key;
      const bool mem = (xphase ? key == tkey : key != 0u) && v >= lo && v <= hi;
      if (mem) {
        const uint32_t slot = atomicAdd(&L.misc[0], 1u);
        if (slot < 64u) L.pub[slot] = ((unsigned long long)key << 32) | (uint32_t)~x;
      }
    }
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
    t.tkey = uni(L.res[2]);
    t.tx = uni(L.res[3]);
    if (tr >= 0 && tid == 0) FS_TR(tr + 10, FS_NOW());
    __syncthreads();
    return t;
  }
}

// The same threshold for the common case, from registers, with the count c of non-zero
// keys and the largest key mx given: one 4,096-bin histogram of the 2^24 key values up to
// mx (bins of 4,096 values), one of the exact values inside the threshold's bin, done.  The
// general search runs instead when the threshold lies below that window, or when keys
// equal to the threshold key must be split by the tie index.  kk[u] = 0 for i >= m.
// DENSE: nearly every key lies in the first window (the pool's candidates), so its histogram
// pass takes no branch per key (a key below the window wraps to a huge bin and lands in
// the lane's overflow bin); otherwise keys outside a window skip it.
template <int U, bool DENSE = false, class XF>
__device__ __forceinline__ Thr find_thr_lean(const uint32_t (&kk)[U], XF X, int m, uint32_t k, uint32_t c,
                                             uint32_t mx, Core& L) {
  const int tid = threadIdx.x;
  Thr t;
  t.total = c;
  t.nsel = min(k, c);
  t.tkey = 0u;
  t.tx = 0xffffffffu;
  if (t.nsel == c) return t;  // every non-zero key (or none)
  uint32_t need = t.nsel;
  const uint32_t lo = mx >= (1u << 24) ? mx - ((1u << 24) - 1u) : 1u;
#pragma unroll
  for (int i = 0; i < kBins / kT; ++i) L.hist[tid + kT * i] = 0u;
  __syncthreads();
  if (DENSE) {
    const uint32_t ovf = kBins + (threadIdx.x & 63u);
#pragma unroll
    for (int u = 0; u < U; ++u) atomicAdd(&L.hist[min((kk[u] - lo) >> 12, ovf)], 1u);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t v = kk[u];
      if (v >= lo) atomicAdd(&L.hist[(v - lo) >> 12], 1u);
    }
  }
  __syncthreads();
  find_bin4(L.hist, need, false, L);  // ends with a barrier
  bool general = uni(L.res[2]) < need;  // the threshold lies below the window
  uint32_t tkey = 0u;
  if (!general) {
    const uint32_t lo2 = lo + (uni(L.res[0]) << 12);
    need -= uni(L.res[1]);
    __syncthreads();  // L.res is read before it is rewritten
#pragma unroll
    for (int i = 0; i < kBins / kT; ++i) L.hist[tid + kT * i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t e = kk[u] - lo2;  // few keys fall in the threshold's bin
      if (e < 4096u) atomicAdd(&L.hist[e], 1u);
    }
    __syncthreads();
    find_bin4(L.hist, need, false, L);
    const uint32_t d = uni(L.res[0]);
    tkey = lo2 + d;
    need -= uni(L.res[1]);
    general = need != uni(L.hist[d]);  // equal keys to split by the tie index
    __syncthreads();
  }
  if (general) return find_thr<U>([&](int u, int) { return kk[u]; }, X, m, k, L);
  t.tkey = tkey;  // every key == tkey is taken (tx = all)
  return t;
}

// Calls emit(rank, u, i) for every element i = threadIdx.x + kT * u (u < U, i < m) whose
// bit u of `mine` is set, rank = its position among them in index order (U * kT <= 64 kT);
// returns how many there are.  Ballots, one scan of the per-(u, wave) counts by wave 0.
// Whole workgroup; ends with a barrier.
template <int U, class EmitF>
__device__ __forceinline__ uint32_t emit_reg(uint32_t mine, EmitF emit, Core& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(U * kNW <= 1024, "counts fit the scan");
  uint32_t below[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned long long msk = __ballot((mine >> u) & 1u);
    below[u] = lanes_below(msk);
    if (lane == 0) L.hist[u * kNW + wave] = (uint32_t)__popcll(msk);
  }
  __syncthreads();
  if (wave == 0) {  // U * kNW counts in (u, wave) order = index order
    constexpr int PER = (U * kNW + 63) / 64;
    uint32_t c[PER];
    uint32_t part = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      c[q] = PER * lane + q < U * kNW ? L.hist[PER * lane + q] : 0u;
      part += c[q];
    }
    const uint32_t incl = wave_incl_scan(part);
    uint32_t run = incl - part;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (PER * lane + q < U * kNW) L.hist[PER * lane + q] = run;
      run += c[q];
    }
    if (lane == 63) L.misc[5] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u)
    if ((mine >> u) & 1u) emit(L.hist[u * kNW + wave] + below[u], u, tid + kT * u);
  const uint32_t total = uni(L.misc[5]);
  __syncthreads();
  return total;
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
// Segments of a row with n visible columns (one, possibly empty, for n = 0).
__device__ __forceinline__ int row_segs(int n, int seg) { return max(1, (n + seg - 1) / seg); }

// Keys a segment of len columns keeps, of a row of n visible columns whose top-k is
// wanted: every key when the row is short enough for the selection to hold it whole;
// otherwise about e = k len / n of the row's top-k are expected in the segment, and six
// standard deviations and four more keep every one of them unless the row is far from
// typical (the selection detects that case and scans the row again).
__device__ __forceinline__ uint32_t seg_keep(int k, int len, int n) {
  if (n <= kMaxCand) return (uint32_t)len;
  const float e = (float)k * (float)len / (float)n;
  return (uint32_t)ceilf(e + 6.0f * sqrtf(e) + 4.0f);
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

// ------------------------------------------------------------------ k_fseg
struct SegLds {
  uint32_t key[kSeg];                     // the segment's keys (0 = not selectable)
  uint16_t pick[kSeg];                    // local columns of the kept keys, in column order
  __align__(16) uint16_t qre[kMaxReindex * kDIdx];
  Core c;
};

// The segment's cut: the lower edge of the 4,096-value bin (of the 2^24 key values up to the
// largest, mx) that holds its keep-th largest key, so that every key >= cut (at least keep
// of them, all of them when fewer than keep are non-zero) is kept.  Keeping whole bins keeps
// equal keys together: what is left out is below everything kept.  Whole workgroup; ends
// with a barrier.
template <int U>
__device__ __forceinline__ uint32_t seg_cut(const uint32_t (&kv)[U], uint32_t keep, uint32_t cnt, uint32_t mx,
                                            Core& L) {
  const int tid = threadIdx.x;
  if (keep >= cnt) return 1u;  // every non-zero key
  const uint32_t lo = mx >= (1u << 24) ? mx - ((1u << 24) - 1u) : 1u;
#pragma unroll
  for (int i = 0; i < kBins / kT; ++i) L.hist[tid + kT * i] = 0u;
  __syncthreads();
  // most of a segment's keys lie below the window: they skip the histogram
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t v = kv[u];
    if (v >= lo) atomicAdd(&L.hist[(v - lo) >> 12], 1u);
  }
  __syncthreads();
  find_bin4(L.hist, keep, false, L);  // ends with a barrier
  uint32_t cut = lo + (uni(L.res[0]) << 12);
  const uint32_t in_window = uni(L.res[2]);
  __syncthreads();
  if (in_window < keep && lo > 1u) {  // the cut lies below the window: bins over [1, lo)
    const uint32_t range = lo - 2u;
    const int sh = range == 0u ? 0 : max(0, 32 - __clz((int)range) - 12);
#pragma unroll
    for (int i = 0; i < kBins / kT; ++i) L.hist[tid + kT * i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t v = kv[u];
      if (v != 0u && v < lo) atomicAdd(&L.hist[(v - 1u) >> sh], 1u);
    }
    __syncthreads();
    find_bin4(L.hist, keep - in_window, false, L);
    cut = 1u + (uni(L.res[0]) << sh);
    __syncthreads();
  }
  return cut;
}

// Grid: rows x runs.  Workgroup (r, j) scores columns [16384 j, 16384 (j + 1)) of row r into
// LDS, keeps every key at or above its cut (at least seg_keep of them), and writes them in
// column order to segment j's run of the row's store, with their count (flagged when keys were
// left out) and, when chained, their Reindex re-scores (the scan's arithmetic).
template <bool CAND>
__global__ __launch_bounds__(kT) void k_fseg(FsArgs a) {
  __shared__ SegLds L;
  const int tid = threadIdx.x, quarter = tid & 3;
  const int r = (int)blockIdx.x / a.runs, j = (int)blockIdx.x % a.runs;
  const int b = a.row0 + r;
  const int n = max(0, min(a.n_valid[b], a.n_cols));
  if (j >= row_segs(n, a.seg)) return;
  const int c0 = j * a.seg, len = max(0, min(n - c0, a.seg));
  const int64_t base = a.seq_base[b];
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  if (tid == 0) FS_TR(blockIdx.x * 8, FS_NOW());
  uint32_t cnt = 0u, mx = 0u;  // this thread's valid columns and their largest key
  if (len > 0)
    scan_columns<CAND, kT>(a.q + (size_t)b * kDIdx, a.codes, a.scale, cand_row, base, n, c0, c0 + len,
                           [] {},
                           [&](int col, float score, bool valid) {
                             const uint32_t key = valid ? score_key(score) : 0u;
                             L.key[col - c0] = key;
                             cnt += valid ? 1u : 0u;
                             mx = max(mx, key);
                           });
  block_sum_max(cnt, mx, L.c);  // ends with a barrier
  if (tid == 0) FS_TR(blockIdx.x * 8 + 1, FS_NOW());
  // keys of column c0 + tid + kT u, u < 16, in registers
  uint32_t kv[kSegU];
#pragma unroll
  for (int u = 0; u < kSegU; ++u) kv[u] = tid + kT * u < len ? L.key[tid + kT * u] : 0u;
  const uint32_t cut = seg_cut(kv, seg_keep(a.k, len, n), cnt, mx, L.c);
  if (tid == 0) FS_TR(blockIdx.x * 8 + 2, FS_NOW());
  const size_t rb = (size_t)r * a.cap + (size_t)j * a.seg;
  uint32_t mine = 0u;
#pragma unroll
  for (int u = 0; u < kSegU; ++u) mine |= (kv[u] != 0u && kv[u] >= cut ? 1u : 0u) << u;
  const uint32_t kept = emit_reg<kSegU>(
      mine,
      [&](uint32_t rank, int u, int i) {
        a.ckey[rb + rank] = kv[u];
        a.ccol[rb + rank] = (uint32_t)(c0 + i);
        L.pick[rank] = (uint16_t)i;
      },
      L.c);
  if (tid == 0) a.ccnt[(size_t)r * a.runs + j] = kept | (kept < cnt ? kTrunc : 0u);
  if (tid == 0) FS_TR(blockIdx.x * 8 + 3, FS_NOW());
  if (!CAND && a.n_re > 0 && kept > 0u) {
    // the Reindex layers' re-scores of the kept entries: 4 lanes (quarters) per entry
    for (int i = tid; i < a.n_re * (kDIdx / 8); i += kT) {
      const int l = i / (kDIdx / 8), part = i % (kDIdx / 8);
      reinterpret_cast<uint4*>(L.qre)[i] =
          reinterpret_cast<const uint4*>(a.q_re + ((size_t)l * a.batch + b) * kDIdx)[part];
    }
    __syncthreads();
    const uint32_t m = kept;
    for (uint32_t p0 = 0; p0 < m; p0 += kT / 4) {
      const uint32_t p = p0 + (uint32_t)(tid >> 2);
      const uint32_t pc = min(p, m - 1u);
      const int64_t entry = base + (int64_t)(c0 + L.pick[pc]);
      const uint4 w = *reinterpret_cast<const uint4*>(a.codes + entry * kIdxCodeBytes + quarter * 16);
      const float sc = a.scale[entry];
      for (int l = 0; l < a.n_re; ++l) {
        bf16x2 qr[16];
        unpack_q(reinterpret_cast<const uint4*>(L.qre + l * kDIdx) + quarter * 4, qr);
        float v = dot32(w, qr);
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if (quarter == 0 && p < m) a.rekey[(size_t)l * a.rows * a.cap + rb + p] = score_key(v * sc);
      }
    }
  }
  if (tid == 0) FS_TR(blockIdx.x * 8 + 4, FS_NOW());
}

// Score-matrix variant (a chunk of queries scored by one contraction): column c of row b is
// at smat_at(a, b, c), in blocks of 1,024 columns that each hold every row.  The keys go
// straight to registers and only the cut needs LDS, so two workgroups share a compute unit
// and one's loads overlap the other's cut.
__device__ __forceinline__ size_t smat_at(const FsArgs& a, int b, int c) {
  return ((size_t)(c >> 10) * (size_t)a.smat_rows + (size_t)b) * 1024u + (size_t)(c & 1023);
}

__global__ __launch_bounds__(kT) void k_fseg_mat(FsArgs a) {
  __shared__ Core L;
  const int tid = threadIdx.x;
  const int r = (int)blockIdx.x / a.runs, j = (int)blockIdx.x % a.runs;
  const int b = a.row0 + r;
  const int n = max(0, min(a.n_valid[b], a.n_cols));
  if (j >= row_segs(n, a.seg)) return;
  const int c0 = j * a.seg, len = max(0, min(n - c0, a.seg));
  float v[kSegU];
#pragma unroll
  for (int u = 0; u < kSegU; ++u)
    v[u] = tid + kT * u < len ? __builtin_nontemporal_load(a.smat + smat_at(a, b, c0 + tid + kT * u)) : 0.f;
  uint32_t kv[kSegU], cnt = 0u, mx = 0u;  // every column < n is valid
#pragma unroll
  for (int u = 0; u < kSegU; ++u) {
    const bool in = tid + kT * u < len;
    kv[u] = in ? score_key(v[u]) : 0u;
    cnt += in ? 1u : 0u;
    mx = max(mx, kv[u]);
  }
  block_sum_max(cnt, mx, L);  // ends with a barrier
  const uint32_t cut = seg_cut(kv, seg_keep(a.k, len, n), cnt, mx, L);
  const size_t rb = (size_t)r * a.cap + (size_t)j * a.seg;
  uint32_t mine = 0u;
#pragma unroll
  for (int u = 0; u < kSegU; ++u) mine |= (kv[u] != 0u && kv[u] >= cut ? 1u : 0u) << u;
  const uint32_t kept = emit_reg<kSegU>(
      mine,
      [&](uint32_t rank, int u, int i) {
        a.ckey[rb + rank] = kv[u];
        a.ccol[rb + rank] = (uint32_t)(c0 + i);
      },
      L);
  if (tid == 0) a.ccnt[(size_t)r * a.runs + j] = kept | (kept < cnt ? kTrunc : 0u);
}

// ------------------------------------------------------------------ k_fpick
// Grid: rows x S workgroups; workgroup (r, s) loads every candidate key of row r (in
// column order: chunk after chunk, each chunk's run in column order), finds the row's
// exact threshold (every workgroup of the row reaches the same one), marks the winners in
// a bitmap whose prefix gives each winner's output position, and writes the winners of
// its own slice of chunks.  The chained selections each go to one workgroup of the row.
struct PickLds {
  uint32_t key[kMaxCand];                 // each candidate's store slot; Reindex: pool re-scores
  uint32_t off[kMaxRuns + 1];             // first candidate of each chunk (dense, col order)
  uint16_t blk[kMaxCand / 32];            // chunk of the first candidate of each 32-block
  uint32_t bm[kMaxCand / 32 + 1];         // winners, one bit per candidate
  uint32_t wp[kMaxCand / 32 + 1];         // winners before each bitmap word (and the total)
  uint32_t rbm[kMaxCand / 32 + 1];        // Reindex winners over the candidates
  uint32_t rwp[kMaxCand / 32 + 1];
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

// bm bits of candidates i = threadIdx.x + kT * u (u < U): bit i set where sel(u) holds.  The
// wave's ballot for u covers words 32 u + 2 wave and 32 u + 2 wave + 1; the U ballots go
// into one register (lane 2 u + h keeps word half h of ballot u) and out in one store.
template <int U, class SelF>
__device__ __forceinline__ void mark_bits(uint32_t* bm, SelF sel) {
  static_assert(2 * U <= 64, "one word per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t val = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned long long m = __ballot(sel(u));
    val = lane == 2 * u ? (uint32_t)m : val;
    val = lane == 2 * u + 1 ? (uint32_t)(m >> 32) : val;
  }
  if (lane < 2 * U) bm[32 * (lane >> 1) + 2 * wave + (lane & 1)] = val;
}

// bm bits of the keys kv[u] (candidate i = threadIdx.x + kT * u, zero at and past m) that
// threshold t selects.  When t takes every key equal to its key (no split by index), the
// test is one compare.
template <int U>
__device__ __forceinline__ void mark_selected(uint32_t* bm, const Thr& t, const uint32_t (&kv)[U], int m) {
  const int tid = threadIdx.x;
  if (t.tx == 0xffffffffu) {
    const uint32_t lo = max(t.tkey, 1u);  // a zero key is never selected
    mark_bits<U>(bm, [&](int u) { return kv[u] >= lo; });
  } else {
    mark_bits<U>(bm, [&](int u) {
      const int i = tid + kT * u;
      return (i < m) & selected(t, kv[u], (uint32_t)i);
    });
  }
}

// Marks in L.bm the top-k of the m candidates (key kv[u] of candidate i = threadIdx.x +
// kT * u, ties to the lower index, i.e. the lower column).  Returns the number selected and
// the threshold.  Whole workgroup; ends with a barrier.
__device__ __forceinline__ Thr pick_marked(const uint32_t (&kv)[kU], int m, uint32_t k, PickLds& L,
                                          int tr = -1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c = 0u, mx = 0u;  // every candidate key is non-zero: the count is m
#pragma unroll
  for (int u = 0; u < kU; ++u) mx = max(mx, kv[u]);
  block_sum_max(c, mx, L.c);
  const Thr t = find_thr_lean<kU, true>(kv, [&](int, int i) { return (uint32_t)i; }, m, k, (uint32_t)m, mx, L.c);
  mark_selected<kU>(L.bm, t, kv, m);
  if (tid == 0) L.bm[kMaxCand / 32] = 0u;
  __syncthreads();
  return t;
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

// Slow path of a row whose segments left out a key of its top-k (or whose candidates
// exceed what the selection holds): this workgroup alone scores every column again and stores every key at store index = column (0 for a
// candidate hole), with the Reindex re-scores when chained.
template <bool CAND>
__device__ __forceinline__ void rescan_row(const FsArgs& a, int r, int n) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int quarter = lane & 3, ent = lane >> 2;
  const int b = a.row0 + r;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  uint32_t* ck = a.ckey + (size_t)r * a.cap;
  uint32_t* cc = a.ccol + (size_t)r * a.cap;
  if (a.smat) {  // the scores are given
    for (int col = tid; col < n; col += kT) {
      st_ag(&ck[col], score_key(a.smat[smat_at(a, b, col)]));
      st_ag(&cc[col], (uint32_t)col);
    }
    wait_vm();
    __syncthreads();
    return;
  }
  const int64_t base = a.seq_base[b];
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

// The slow path of a row (a segment left out one of its top-k, or too many candidates):
// every key of the row again, the store then in column order (store index = column), and every
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

// Index of the set bit of rank r (from 0) of a bitmap whose word prefix wp has words + 1
// entries (r < wp[words]).
__device__ __forceinline__ uint32_t nth_bit(const uint32_t* bm, const uint32_t* wp, int words, uint32_t r) {
  const int w = upper_index(wp, words, r);
  uint32_t x = bm[w];
  for (uint32_t q = r - wp[w]; q > 0u; --q) x &= x - 1u;  // drop the lower set bits
  return (uint32_t)w * 32u + (uint32_t)__builtin_ctz(x);
}

// Store slot of candidate i (segment j's run starts at j * seg).
__device__ __forceinline__ uint32_t slot_of(const PickLds& L, uint32_t i, int seg) {
  const int j = chunk_of(L, i);
  return (uint32_t)j * (uint32_t)seg + (i - L.off[j]);
}

// Reindex layer l of row r on the fast path: the top-re_k of the pool's re-scores (ties to
// the lower pool position), written as pool entries in pool order.  The pool's winners in
// candidate order are in pool order, so the selection runs over the candidates with every
// non-winner's re-score taken as 0 (not selectable).  L.key holds each candidate's re-score.
template <bool CAND>
__device__ __forceinline__ void pick_reindex(const FsArgs& a, PickLds& L, int r, int l, int m, uint32_t P) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int trb = (1 << 20) - 262144 + (int)blockIdx.x * 16;
  if (tid == 0) FS_TR(trb + 4, FS_NOW());
  const int b = a.row0 + r;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  // every bitmap word is written (no bit at or past m), so the reads need no bounds test
  uint32_t kk[kU], c = 0u, mx = 0u;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = tid + kT * u;
    const uint32_t w = L.bm[i >> 5], key = L.key[i];
    kk[u] = (w >> (i & 31)) & 1u ? key : 0u;
    c += kk[u] != 0u ? 1u : 0u;
    mx = max(mx, kk[u]);
  }
  block_sum_max(c, mx, L.c);
  if (tid == 0) FS_TR(trb, FS_NOW());
  const Thr tr = find_thr_lean<kU>(kk, [&](int, int i) { return (uint32_t)i; }, m, (uint32_t)a.re_k, c, mx, L.c);
  if (tid == 0) FS_TR(trb + 1, FS_NOW());
  mark_selected<kU>(L.rbm, tr, kk, m);
  if (tid == 0) L.rbm[kMaxCand / 32] = 0u;
  __syncthreads();
  bitmap_prefix(L.rbm, L.rwp, m, L.c);
  int32_t* orr = a.re_out + ((size_t)l * a.batch + b) * a.re_k;
  float* srr = a.re_sout ? a.re_sout + ((size_t)l * a.batch + b) * a.re_k : nullptr;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  if (tid == 0) FS_TR(trb + 2, FS_NOW());
  // a thread per output rank: its candidate index, its column
  for (uint32_t q = tid; q < tr.nsel; q += kT) {
    const uint32_t i = nth_bit(L.rbm, L.rwp, (m + 31) / 32, q);
    const uint32_t col = cc[slot_of(L, i, a.seg)];
    orr[q] = CAND ? cand_row[col] : (int32_t)col;
    if (srr) srr[q] = key_score(L.key[i]);
  }
  for (int p = (int)tr.nsel + tid; p < a.re_k; p += kT) {
    orr[p] = -1;
    if (srr) srr[p] = -__builtin_inff();
  }
  if (tid == 0) FS_TR(trb + 3, FS_NOW());
  __syncthreads();
}

// The Full layer's own top-own_k of the m candidates of row r (ties to the lower column), in
// column order.
template <bool CAND>
__device__ __forceinline__ void pick_own(const FsArgs& a, PickLds& L, int r, int m) {
  const int tid = threadIdx.x;
  const int b = a.row0 + r;
  const uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  uint32_t kv[kU];  // L.key holds each candidate's store slot
#pragma unroll
  for (int u = 0; u < kU; ++u) kv[u] = tid + kT * u < m ? L.key[tid + kT * u] : 0u;
#pragma unroll
  for (int u = 0; u < kU; ++u) kv[u] = tid + kT * u < m ? ck[kv[u]] : 0u;
  const uint32_t n_own = pick_marked(kv, m, (uint32_t)a.own_k, L).nsel;
  bitmap_prefix(L.bm, L.wp, m, L.c);
  int32_t* own = a.own_out + (size_t)b * a.own_k;
  for (uint32_t q = tid; q < n_own; q += kT) {  // a thread per output rank
    const uint32_t col = cc[slot_of(L, nth_bit(L.bm, L.wp, (m + 31) / 32, q), a.seg)];
    own[q] = CAND ? cand_row[col] : (int32_t)col;
  }
  for (int p = (int)n_own + tid; p < a.own_k; p += kT) own[p] = -1;
}

// Grid: rows x (S + R): per row, S workgroups that each write a slice of the pool, then R
// workgroups with one chained selection each (Reindex layer 0 .. n_re - 1, then the Full
// layer's own top-k).  The candidates are exact when no segment that left keys out had all
// of its kept keys selected (then its best left-out key is below the threshold); otherwise,
// or when they exceed what the selection holds, the row takes the slow path.
template <bool CAND>
__global__ __launch_bounds__(kT) void k_fpick(FsArgs a, int S) {
  __shared__ PickLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.n_re + (a.own_k > 0 ? 1 : 0);
  const int r = (int)blockIdx.x / (S + R), s = (int)blockIdx.x % (S + R);
  const int tb = (1 << 20) - 65536 + (int)blockIdx.x * 8;
  if (tid == 0) FS_TR(tb, FS_NOW());
  const int b = a.row0 + r;
  const int n_row = max(0, min(a.n_valid[b], a.n_cols));
  const int nsg = row_segs(n_row, a.seg);
  const uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const uint32_t* cc = a.ccol + (size_t)r * a.cap;
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  int32_t* orow = a.out + (size_t)b * a.k;
  float* srow = a.sout ? a.sout + (size_t)b * a.k : nullptr;
  // each segment's count (thread t: segments 2t, 2t + 1), their prefix = dense offsets
  const uint32_t r0 = 2 * tid < nsg ? a.ccnt[(size_t)r * a.runs + 2 * tid] : 0u;
  const uint32_t r1 = 2 * tid + 1 < nsg ? a.ccnt[(size_t)r * a.runs + 2 * tid + 1] : 0u;
  const uint32_t c0 = r0 & ~kTrunc, c1 = r1 & ~kTrunc;
  uint32_t m_all;
  {
    const uint32_t e = block_exclusive_scan(c0 + c1, L.c.scan, &m_all);
    m_all = uni(m_all);
    if (2 * tid < nsg) L.off[2 * tid] = e;
    if (2 * tid + 1 < nsg) L.off[2 * tid + 1] = e + c0;
    if (tid == 0) L.off[nsg] = m_all;
  }
  __syncthreads();
  if (tid == 0) FS_TR(tb + 5, FS_NOW());
  bool fast = m_all <= (uint32_t)kMaxCand;
  if (fast) {
    const int m = (int)m_all;
    for (int w = tid; w < (m + 31) / 32; w += kT) L.blk[w] = (uint16_t)upper_index(L.off, nsg, 32u * w);
    // each candidate's store slot (a wave per segment)
    for (int j = wave; j < nsg; j += kNW) {
      const uint32_t o = L.off[j], c = L.off[j + 1] - o;
      for (uint32_t e = lane; e < c; e += 64) L.key[o + e] = (uint32_t)j * (uint32_t)a.seg + e;
    }
    __syncthreads();
    if (tid == 0) FS_TR(tb + 6, FS_NOW());
    // every candidate key of the row (candidate i = tid + kT * u, all loads in flight at
    // once), then the pool (or the only selection) marked in L.bm
    uint32_t n_pool;
    {
      uint32_t kv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = tid + kT * u;
        kv[u] = i < m ? L.key[i] : 0u;
      }
      if (s >= S && s - S < a.n_re) {
        // a Reindex workgroup loads its layer's re-scores with the keys, into L.key (each
        // candidate's slot is read before it is overwritten: same thread, same index)
        const uint32_t* rk = a.rekey + ((size_t)(s - S) * a.rows + r) * a.cap;
        uint32_t rv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const bool in = tid + kT * u < m;
          rv[u] = in ? rk[kv[u]] : 0u;
          kv[u] = in ? ck[kv[u]] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (tid + kT * u < m) L.key[tid + kT * u] = rv[u];
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) kv[u] = tid + kT * u < m ? ck[kv[u]] : 0u;
      }
      if (tid == 0) FS_TR(tb + 1, FS_NOW());
      n_pool = pick_marked(kv, m, (uint32_t)a.k, L, (1 << 20) - 131072 + (int)blockIdx.x * 16).nsel;
    }
    bitmap_prefix(L.bm, L.wp, m, L.c);
    // a truncated segment whose kept keys all won may have left out a winner
    bool bad = false;
    if (2 * tid < nsg && (r0 & kTrunc) &&
        bits_before(L.bm, L.wp, L.off[2 * tid + 1]) - bits_before(L.bm, L.wp, L.off[2 * tid]) == c0)
      bad = true;
    if (2 * tid + 1 < nsg && (r1 & kTrunc) &&
        bits_before(L.bm, L.wp, L.off[2 * tid + 2]) - bits_before(L.bm, L.wp, L.off[2 * tid + 1]) == c1)
      bad = true;
    fast = !__syncthreads_or(bad);
    if (tid == 0) FS_TR(tb + 2, FS_NOW());
    if (fast) {
      if (s < S && (long long)m <= 2LL * kT * S) {
        // this workgroup's slice of the candidates (at most two per thread): each winner's
        // output position from the bitmap's prefix
        const uint32_t i0 = (uint32_t)((long long)s * m / S), i1 = (uint32_t)((long long)(s + 1) * m / S);
        for (uint32_t i = i0 + tid; i < i1; i += kT) {
          if (!bit_at(L.bm, i)) continue;
          const uint32_t slot = slot_of(L, i, a.seg);
          const uint32_t col = cc[slot];
          const uint32_t pos = bits_before(L.bm, L.wp, i);
          orow[pos] = CAND ? cand_row[col] : (int32_t)col;
          if (srow) srow[pos] = key_score(ck[slot]);
        }
      } else if (s < S && n_pool <= (uint32_t)kT * (uint32_t)S) {
        // this workgroup's slice of the output, one rank per thread: its winner by bitmap rank
        const uint32_t q0 = (uint32_t)((long long)s * n_pool / S), q1 = (uint32_t)((long long)(s + 1) * n_pool / S);
        const uint32_t q = q0 + (uint32_t)tid;
        if (q < q1) {
          const uint32_t slot = slot_of(L, nth_bit(L.bm, L.wp, (m + 31) / 32, q), a.seg);
          const uint32_t col = cc[slot];
          orow[q] = CAND ? cand_row[col] : (int32_t)col;
          if (srow) srow[q] = key_score(ck[slot]);
        }
      } else if (s < S) {
        // few slices for many winners: this workgroup's candidates in blocks of eight per
        // thread (candidate i = tid + kT u), each block's slots first, then all of its loads
        // in flight, then each winner written at its bitmap position
        const uint32_t i0 = (uint32_t)((long long)s * m / S), i1 = (uint32_t)((long long)(s + 1) * m / S);
        constexpr int kB = 8;
        static_assert(kU % kB == 0, "whole blocks");
        for (int u0 = 0; u0 < kU; u0 += kB) {
          if (kT * u0 >= (int)i1) break;  // uniform: the rest is past the slice
          uint32_t sl[kB], col[kB];
#pragma unroll
          for (int v = 0; v < kB; ++v) {
            const uint32_t i = (uint32_t)(tid + kT * (u0 + v));
            sl[v] = i >= i0 && i < i1 && bit_at(L.bm, i) ? slot_of(L, i, a.seg) : ~0u;
          }
#pragma unroll
          for (int v = 0; v < kB; ++v) col[v] = sl[v] != ~0u ? cc[sl[v]] : 0u;
#pragma unroll
          for (int v = 0; v < kB; ++v)
            if (sl[v] != ~0u) {
              const uint32_t pos = bits_before(L.bm, L.wp, (uint32_t)(tid + kT * (u0 + v)));
              orow[pos] = CAND ? cand_row[col[v]] : (int32_t)col[v];
              if (srow) srow[pos] = key_score(ck[sl[v]]);
            }
        }
      }
      if (s < S) {
        if (s == 0)
          for (int p = (int)n_pool + tid; p < a.k; p += kT) {
            orow[p] = -1;
            if (srow) srow[p] = -__builtin_inff();
          }
        if (tid == 0) FS_TR(tb + 3, FS_NOW());
      } else if (s - S < a.n_re) {
        pick_reindex<CAND>(a, L, r, s - S, m, n_pool);
      } else {
        pick_own<CAND>(a, L, r, m);
      }
    }
  }
  if (!fast && s == 0) slow_select<CAND>(a, &L, r);
  if (tid == 0) FS_TR(tb + 4, FS_NOW());
  // the last workgroup of the row returns the row's counter to zero
  wait_vm();
  __syncthreads();
  if (tid == 0) L.c.misc[4] = add_ag(&a.roww[r * kRowWords + kRwDone], 1u) == (uint32_t)(S + R - 1) ? 1u : 0u;
  __syncthreads();
  if (L.c.misc[4] != 0u && tid < kRowWords) a.roww[r * kRowWords + tid] = 0u;
}

// ------------------------------------------------------------------ k_fsmall
// Rows of at most kSmallCols columns (a Reindex layer's pool), in one launch.  Workgroup
// (r, p) scores columns [1024 p, 1024 (p + 1)) of row r into the row's key array (0 for an
// invalid column); the workgroup that finishes its row last (an agent-scope counter: no
// workgroup waits for another) then takes the row's top-k from the keys, marks the winners
// in a bitmap and writes each at its bitmap position, so the list comes out in column
// order.  The counter is returned to zero by that workgroup.
constexpr int kSmallCols = 16384;
constexpr int kSmallU = kSmallCols / kT;
struct SmallLds {
  uint32_t bm[kSmallCols / 32 + 1];
  uint32_t wp[kSmallCols / 32 + 1];
  Core c;
};

template <bool CAND>
__global__ __launch_bounds__(kT) void k_fsmall(FsArgs a) {
  __shared__ SmallLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.runs;  // workgroups per row
  const int r = (int)blockIdx.x / P, p = (int)blockIdx.x % P;
  const int b = a.row0 + r;
  const int n = max(0, min(a.n_valid[b], a.n_cols));
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  uint32_t* ck = a.ckey + (size_t)r * a.cap;
  const int c0 = p * kT;
  const int tb = (1 << 20) - 200000 + (int)blockIdx.x * 8;
  if (tid == 0) FS_TR(tb, FS_NOW());
  {
    // one group of 64 columns per wave, no prefetch: the memory counter that the wait
    // below drains holds only this group's loads and stores
    const int quarter = lane & 3, ent = lane >> 2;
    const int g = c0 + wave * 64;
    if (g < n) {
      bf16x2 q[16];
      load_q(a.q + (size_t)b * kDIdx, quarter, q);
      const ScanGroup sg = load_group<CAND>(a.codes, a.scale, cand_row, a.seq_base[b], g, n - 1, ent, quarter);
      const float score = group_score(sg, q, quarter);
      const int col = g + 16 * quarter + ent;
      if (col < n) st_ag(&ck[col], sg.own_ok ? score_key(score) : 0u);
    }
  }
  // The keys are agent-scope stores, complete (at the device's coherence point) once this
  // wave's memory counter drains, before the row's counter moves; the last workgroup reads
  // them with agent-scope loads.  No cache-wide fence is needed.
  wait_vm();
  __syncthreads();
  if (tid == 0) FS_TR(tb + 1, FS_NOW());
  if (tid == 0) L.c.misc[4] = add_ag(&a.roww[r * kRowWords + kRwDone], 1u) == (uint32_t)(P - 1) ? 1u : 0u;
  __syncthreads();
  if (tid == 0) FS_TR(tb + 2, FS_NOW());
  if (L.c.misc[4] == 0u) return;  // workgroup-uniform
  // the row's last workgroup: every key of the row is written
  if (tid == 0) st_ag(&a.roww[r * kRowWords + kRwDone], 0u);
  uint32_t kv[kSmallU], c = 0u, mx = 0u;
  int32_t cid[kSmallU];  // entry id of each column, loaded with the keys
#pragma unroll
  for (int u = 0; u < kSmallU; ++u) {
    const int i = tid + kT * u;
    kv[u] = i < n ? ld_ag(&ck[i]) : 0u;
    cid[u] = CAND ? (i < n ? cand_row[i] : -1) : i;
  }
#pragma unroll
  for (int u = 0; u < kSmallU; ++u) {
    c += kv[u] != 0u ? 1u : 0u;
    mx = max(mx, kv[u]);
  }
  block_sum_max(c, mx, L.c);
  if (tid == 0) FS_TR(tb + 3, FS_NOW());
  const Thr t = find_thr_lean<kSmallU>(kv, [&](int, int i) { return (uint32_t)i; }, n, (uint32_t)a.k, c, mx, L.c);
  if (tid == 0) FS_TR(tb + 4, FS_NOW());
  mark_selected<kSmallU>(L.bm, t, kv, n);
  if (tid == 0) L.bm[kSmallCols / 32] = 0u;
  __syncthreads();
  bitmap_prefix(L.bm, L.wp, n, L.c);
  if (tid == 0) FS_TR(tb + 5, FS_NOW());
  int32_t* orow = a.out + (size_t)b * a.k;
  float* srow = a.sout ? a.sout + (size_t)b * a.k : nullptr;
#pragma unroll
  for (int u = 0; u < kSmallU; ++u) {
    const int i = tid + kT * u;
    if (i < n && bit_at(L.bm, (uint32_t)i)) {
      const uint32_t pos = bits_before(L.bm, L.wp, (uint32_t)i);
      orow[pos] = cid[u];
      if (srow) srow[pos] = key_score(kv[u]);
    }
  }
  for (int q = (int)t.nsel + tid; q < a.k; q += kT) {
    orow[q] = -1;
    if (srow) srow[q] = -__builtin_inff();
  }
  if (tid == 0) FS_TR(tb + 6, FS_NOW());
}

// ---------------------------------------------------------------------------- host side
// Compute units of the current device (the picking grid's size aims at one workgroup
// each; correctness does not depend on it).
int fs_capacity() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n_cu;
}

struct FsShape {
  int runs, rows_ws;
  size_t cap;
};

// Workspace shape covering every segment length a launch may choose: the store holds
// n_cols rounded up to the longest segment, the counts one per shortest segment.
FsShape fs_shape(int batch, int n_cols, bool chain) {
  FsShape s;
  s.runs = (n_cols + kSegMin - 1) / kSegMin;
  s.cap = (size_t)((n_cols + kSeg - 1) / kSeg) * kSeg;
  s.rows_ws = min(batch, chain ? kChainRows : kMaxRows);
  return s;
}

// The kept keys of a row of n_cols columns cut into segs segments fit the selection: every
// key when the row is short enough, else at most k + 6 sqrt(k segs) + 5 segs (the sum of
// seg_keep over its segments) plus 2 per segment for the keys sharing the cut's bin.
bool fs_capacity_ok(int n_cols, int k, int segs) {
  if (n_cols <= kMaxCand) return true;
  return (double)k + 6.0 * std::sqrt((double)k * segs) + 7.0 * segs <= (double)kMaxCand;
}

// Segment length of a launch of `rows` rows: the longest that still gives every compute
// unit a workgroup (shorter segments, more workgroups), within the selection's capacity
// and at most kMaxRuns segments per row; 0 when none fits.
int fs_seg(int rows, int n_cols, int k, int n_cu) {
  int best = 0;
  for (int seg = kSeg; seg >= kSegMin; seg /= 2) {
    const int segs = (n_cols + seg - 1) / seg;
    if (segs > kMaxRuns || !fs_capacity_ok(n_cols, k, segs)) break;
    best = seg;
    if ((long long)rows * segs >= n_cu) break;
  }
  return best;
}

struct FsParts {
  uint32_t *ctrl, *roww, *ccnt, *ckey, *ccol, *rekey, *pmap;
  size_t bytes;
};

// Workspace: [ctrl 256 B][per row 64 B][segment counts][candidate keys][their columns] and,
// for a chain, [their Reindex re-scores][pool -> store index].
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

// Rows up to n_cols long whose top-k the filtered selection takes (with its longest
// segments, the fewest kept keys).
bool fsel_fits(int n_cols, int k) {
  return n_cols >= 1 && n_cols <= kMaxRuns * kSeg && fs_capacity_ok(n_cols, k, (n_cols + kSeg - 1) / kSeg);
}

bool fsel_len_ok(int n_cols) { return n_cols >= 1 && n_cols <= kMaxRuns * kSeg; }

size_t fsel_ws_bytes(int batch, int n_cols, bool chain) {
  return fs_carve(nullptr, fs_shape(batch, n_cols, chain), chain).bytes;
}

hipError_t launch_fsel(const uint16_t* q, const uint8_t* codes, const float* scale,
                       const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                       int batch, int n_cols, int k, int32_t* out, float* sout, int own_k,
                       int32_t* own_out, const uint16_t* q_re, int n_re, int re_k,
                       int32_t* re_out, float* re_sout, bool chain_ws, void* ws,
                       hipStream_t stream, const float* smat) {
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
  a.smat = smat;
  a.smat_rows = batch;
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
  a.ccnt = f.ccnt;
  a.ckey = f.ckey;
  a.ccol = f.ccol;
  a.rekey = f.rekey;
  a.pmap = f.pmap;
  a.cap = s.cap;
  for (int r0 = 0; r0 < batch; r0 += s.rows_ws) {
    a.row0 = r0;
    a.rows = min(s.rows_ws, batch - r0);
    a.seg = fs_seg(a.rows, n_cols, k, cap_wg);
    if (a.seg == 0) return hipErrorInvalidValue;  // excluded by fsel_fits
    a.runs = (n_cols + a.seg - 1) / a.seg;
    a.cap = (size_t)a.runs * a.seg;
    // picking workgroups per row: about one per compute unit in all, none with fewer than
    // 128 of the k winners to write
    const int R = a.n_re + (a.own_k > 0 ? 1 : 0);
    const int S = max(1, min(cap_wg / a.rows - R, (k + 127) / 128));
    const dim3 g_seg((unsigned)(a.rows * a.runs)), g_pick((unsigned)(a.rows * (S + R)));
    if (cand) {
      hipLaunchKernelGGL(k_fseg<true>, g_seg, dim3(kT), 0, stream, a);
      hipLaunchKernelGGL(k_fpick<true>, g_pick, dim3(kT), 0, stream, a, S);
    } else if (smat) {
      hipLaunchKernelGGL(k_fseg_mat, g_seg, dim3(kT), 0, stream, a);
      hipLaunchKernelGGL(k_fpick<false>, g_pick, dim3(kT), 0, stream, a, S);
    } else {
      hipLaunchKernelGGL(k_fseg<false>, g_seg, dim3(kT), 0, stream, a);
      hipLaunchKernelGGL(k_fpick<false>, g_pick, dim3(kT), 0, stream, a, S);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Short rows, and few enough of them that their workgroups run in about one wave of the
// device (with more rows the serial selection of each row's last workgroup costs more than
// the two-launch selection).
bool fsmall_fits(int batch, int n_cols) {
  return n_cols >= 1 && n_cols <= kSmallCols &&
         (long long)batch * ((n_cols + kT - 1) / kT) <= 2LL * max(fs_capacity(), 1);
}

// Uses the filtered selection's workspace (its key store and row counters).
hipError_t launch_fsmall(const uint16_t* q, const uint8_t* codes, const float* scale,
                         const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                         int batch, int n_cols, int k, int32_t* out, float* sout, void* ws,
                         hipStream_t stream) {
  const FsShape s = fs_shape(batch, n_cols, false);
  const FsParts f = fs_carve(static_cast<char*>(ws), s, false);
  FsArgs a{};
  a.q = q;
  a.codes = codes;
  a.scale = scale;
  a.seq_base = seq_base;
  a.n_valid = n_valid;
  a.cand = cand;
  a.n_cols = n_cols;
  a.runs = (n_cols + kT - 1) / kT;
  a.batch = batch;
  a.k = k;
  a.out = out;
  a.sout = sout;
  a.ctrl = f.ctrl;
  a.roww = f.roww;
  a.ckey = f.ckey;
  a.cap = s.cap;
  for (int r0 = 0; r0 < batch; r0 += s.rows_ws) {
    a.row0 = r0;
    a.rows = min(s.rows_ws, batch - r0);
    const dim3 grid((unsigned)(a.rows * a.runs));
    if (cand)
      hipLaunchKernelGGL(k_fsmall<true>, grid, dim3(kT), 0, stream, a);
    else
      hipLaunchKernelGGL(k_fsmall<false>, grid, dim3(kT), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
