// a1 + a2 (and a3 + a2): score the indexer keys and select the top-k in one launch,
// without writing the scores to memory; optionally followed, in the same launch, by the
// selections a decoder layer chain makes inside that pool: the Full layer's own top-k by
// its scores, and the top-k of Reindex layers that re-score the pool with their own
// indexer queries ("从V4到V4.1 Flash：架构的激进进化", decoder section: the first layer's
// full scan yields a pool of about 16K positions that later layers search; "DeepSeek-V4.1
// 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", commentary on the four layer modes).
//
// Every selection returns what csa2_topk returns for the same scores: the k largest of a
// row, ties to the lower column, written in ascending column order as entry ids, -1
// padded.  Inside the pool, "column" means the pool position, which ascends with the
// entry id, so ties again go to the lowest entry.
//
// Every 1,024-thread workgroup scores up to 16,384 columns of one row with the stream of
// scan_device.h (16 waves: as many loads in flight per CU as the stand-alone scan) and
// keeps their order-preserving u32 keys in LDS (key 0 = not selectable).  A selection
// over keys held by the row's workgroups (64 for a 2^20-column row) finds the exact k-th
// composite (key << 32 | ~position, unique) digit by digit, meeting at row barriers:
//   1. level 1, key bits 31..20: each workgroup's LDS histogram is added to the row's.
//      If the bin b1 of the k-th key holds at most 1,024 keys, go to 3 with that bin;
//   2. level 2, bits 19..9, over the keys in b1: the bin (b1, b2);
//   3. each workgroup publishes how many of its keys lie above the bin and the composites
//      of its keys inside it.  Every workgroup ranks the published composites itself:
//      that fixes the k-th composite T, which tied keys are taken, and each workgroup's
//      output offset (the sum of the selections of the workgroups before it).
// When a workgroup has more keys in the bin than it may publish (massive ties), the row
// goes one level deeper instead: a level-3 histogram (bits 8..0) fixes the threshold key,
// then (#keys above it, #keys equal to it) of every workgroup fix each workgroup's share
// of the equal keys (the lowest positions win) and its offset.
// Each workgroup then writes its selected entries in position order with wave ballots.
// For the chained selections each workgroup keeps the pool entries it selected (their
// keys and columns, in LDS); the Full layer's own top-k reuses those keys, a Reindex layer
// first gathers and re-scores those entries with its query (the same arithmetic as the
// scan, so the same scores as csa2_index_score).  Workgroup 0 of the row returns every
// histogram to zero once all workgroups have read it, and the last workgroup to leave
// resets the row's barrier counters: the workspace is ready for the next call without a
// clearing launch.
//
// Everything one workgroup tells another goes through agent-scope atomics: read-modify-
// writes whose returned values are waited for before the workgroup arrives at the next
// barrier (so they have been performed), and atomic loads after the barrier.  Plain data
// never crosses workgroups inside the launch, so the barriers need no cache write-back or
// invalidation (measured on MI355X: a 64-workgroup barrier costs about 1.5 us this way and
// about 4-16 us with agent-scope fences).
//
// The barriers need every workgroup of the launch resident at once.  The host sizes each
// launch to the device's capacity (one workgroup per CU), which an otherwise idle device
// dispatches at once.  Each wait is bounded: after 2^20 polls (about a second) it gives
// up and sets a sticky status word in the workspace, so every wave exits even when the
// device is shared and that assumption fails (the call's result is then undefined).
//
// Speculative fine window (the scan's selection on rows of at least 64K columns): the scan
// also counts key bits 31..16 for the 16 level-1 bins around the bin b1 of the previous
// call on this row (a hint kept in the workspace; successive decode steps see similar
// score distributions).  When the new b1 falls in that window, its fine counts are
// complete and the sub-bin of the k-th key usually holds few enough keys to publish at
// once, which saves the level-2 round; otherwise level 2 runs.  The result never depends
// on the hint, only the time does.
//
// Workspace: [status: 256 B][per row 32 u32, 256-aligned: barrier arrivals, departures,
// fine-window hint][batch x kMaxSel selection blocks of kSelBytes: h1 u32[4096] |
// h2 u32[2048] | h3 u32[512] | per-workgroup counts u32[256] | published composites
// u64[2048]][batch x fine counts u32[4096 x 16]].
#include "csa2_internal.h"
#include "scan_device.h"
#include "select_device.h"

namespace csa2 {

constexpr int kFuseThreads = 1024;                        // 16 waves
constexpr int kFuseWaves = kFuseThreads / 64;
constexpr int kFuseKeysPerThread = 16;
constexpr int kFuseMaxCols = kFuseThreads * kFuseKeysPerThread;  // 16,384 keys in LDS
constexpr int kPubMax = 1024;                             // published composites ranked in LDS
constexpr uint32_t kSpinLimit = 1u << 20;

constexpr size_t kSelH2 = kHist1Bins * 4;
constexpr size_t kSelH3 = kSelH2 + kHist2Bins * 4;
constexpr size_t kSelCnt = kSelH3 + kHist3Bins * 4;
constexpr size_t kSelPub = kSelCnt + kFuseMaxWg * 4;
constexpr size_t kSelBytes = kSelPub + kPubSlots * 8;
constexpr int kFineSub = 16;           // sub-bins (key bits 19..16) per level-1 bin
constexpr int kFineWin = 16;           // level-1 bins of the scan's fine window
constexpr uint32_t kFineMinRow = 65536;  // rows this long count the window
constexpr size_t kFineBytes = (size_t)kHist1Bins * kFineSub * 4;  // per row

static_assert(kFuseThreads * 4 == kHist1Bins, "level-1 bins: 4 per thread");
static_assert(kFuseThreads * 2 == kHist2Bins, "level-2 bins: 2 per thread");
static_assert(kHist3Bins == 8 * 64, "level-3 bins: 8 per lane of one wave");
static_assert(kFuseMaxWg <= kFuseThreads, "per-workgroup counts: one per thread");
static_assert(kPubSlots == 2 * kFuseThreads, "published slots: two per thread");
static_assert(kSelBytes % 256 == 0, "selection blocks stay 256-byte aligned");

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ uint32_t xchg_agent(T* p, T v) {
  return (uint32_t)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barriers of the workgroups of one row.  sync(pending): `pending` combines the values
// returned by this thread's atomics since the previous barrier; using it makes the thread
// wait until they have been performed before its workgroup arrives.
struct RowSync {
  uint32_t* arrivals;
  uint32_t* status;
  uint32_t nw;     // workgroups in the row
  uint32_t done;   // barriers passed (the same in every workgroup of the row)

  __device__ void sync(uint32_t pending) {
    asm volatile("" ::"v"(pending));
    __syncthreads();
    ++done;
    if (threadIdx.x == 0) {
      const uint32_t target = done * nw;
      add_agent(arrivals, 1u);
      uint32_t spins = 0;
      while (ld_agent(arrivals) < target) {
        if (++spins == kSpinLimit) {
          st_agent(status, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }
};

// LDS scratch of a selection.
struct SelLds {
  uint32_t* h;                 // [4096] histograms
  uint32_t* cnt;               // [16 x 16] per-(iteration, wave) counts
  unsigned long long* pub;     // [2 x kPubMax] staged / gathered composites
  uint32_t* selt;              // [kFuseMaxWg] per-workgroup counts
  uint32_t* scan;              // [32] block-scan scratch
  uint32_t* res;               // [4]
  uint32_t* misc;              // [4]
  unsigned long long* T;       // [1]
  uint32_t* bits;              // [512] selection bitmap over the local index
  uint32_t* bits2;             // [512] keys inside the threshold bin
};

// One selection's global arrays for this row.
struct SelWs {
  uint32_t* h1;
  uint32_t* h2;
  uint32_t* h3;
  uint32_t* cnt;               // [kFuseMaxWg]
  unsigned long long* pub;     // [kPubSlots]: workgroup w owns [w * cap, (w + 1) * cap)
  uint32_t* fine;              // [4096][16] counts inside the scan's window (stage 0)
  uint32_t* hint;              // [1] b1 + 1 of the previous call (0: none)
  uint32_t* above;             // [1] keys above the scan's window (stage 0)
};

__device__ __forceinline__ SelWs sel_ws(char* sel_base, int row, int sel, char* fine_base,
                                        uint32_t* sync) {
  char* p = sel_base + ((size_t)row * kMaxSel + sel) * kSelBytes;
  return SelWs{reinterpret_cast<uint32_t*>(p), reinterpret_cast<uint32_t*>(p + kSelH2),
               reinterpret_cast<uint32_t*>(p + kSelH3), reinterpret_cast<uint32_t*>(p + kSelCnt),
               reinterpret_cast<unsigned long long*>(p + kSelPub),
               reinterpret_cast<uint32_t*>(fine_base + (size_t)row * kFineBytes),
               sync + (size_t)row * kSyncStride + 2, sync + (size_t)row * kSyncStride + 3};
}

// Adds the non-empty bins of an LDS histogram of N * 1,024 bins (N = 1: 512 bins) to a
// global one; returns the combined values the atomics returned (for RowSync::sync).  The
// atomics are issued back to back and their returns only combined at the end.
template <int N>
__device__ __forceinline__ uint32_t flush_hist(const uint32_t* s_h, int nbins, uint32_t* g) {
  uint32_t r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int bin = threadIdx.x + i * kFuseThreads;
    const uint32_t v = bin < nbins ? s_h[bin] : 0u;
    r[i] = 0u;
    if (v) r[i] = add_agent(&g[bin], v);
  }
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) pending |= r[i];
  return pending;
}

// LDS histogram, over `nbins` bins of (key >> shift) & (nbins - 1), of the non-zero keys
// with key >> (shift + dbits) == pre (dbits = log2 nbins; pre = 0 with shift + dbits = 32
// takes every key).  Whole workgroup; ends with a barrier.
__device__ __forceinline__ void local_hist(const uint32_t* keys, int n_local, uint32_t pre,
                                           int shift, int nbins, int dbits, uint32_t* s_h) {
  for (int i = threadIdx.x; i < nbins; i += kFuseThreads) s_h[i] = 0u;
  __syncthreads();
  const int top = shift + dbits;
  for (int i = threadIdx.x; i < n_local; i += kFuseThreads) {
    const uint32_t key = keys[i];
    if (key != 0u && (top >= 32 || (key >> top) == pre))
      atomicAdd(&s_h[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
  }
  __syncthreads();
}

// Searches an LDS histogram h[0..PER * 1024) for the bin holding the k-th largest element,
// from the top.  Returns the total count; when 1 <= k <= total, out[0] = the bin and
// out[1] = the elements in higher bins.  Whole workgroup; ends with a barrier.
template <int PER>
__device__ uint32_t hist_select(const uint32_t* h, uint32_t k, uint32_t* s_scan, uint32_t* out) {
  const int top = PER * (kFuseThreads - (int)threadIdx.x);
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[top - 1 - i];
    sum += c[i];
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(sum, s_scan, &total);  // ends with a barrier
  if (excl < k && k <= excl + sum) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= k) {
        out[0] = (uint32_t)(top - 1 - i);
        out[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  return total;
}

// One pass of wave ballots over the 16,384 LDS keys (wave w covers local indices
// [1024 w, 1024 w + 1024); keys past the row's end are 0): L.bits marks key > top and,
// when `inside`, L.bits2 marks lo <= key <= top (1 <= lo).  Every key is loaded before
// the first ballot, and lane 0 writes each wave's words four iterations at a time.
// Whole workgroup; ends with a barrier.
__device__ __forceinline__ void mark_pass(const uint32_t* keys, uint32_t lo, uint32_t top,
                                          bool inside, const SelLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t* kw = keys + wave * (kFuseMaxCols / kFuseWaves);
  uint32_t kv[kFuseKeysPerThread];
#pragma unroll
  for (int j = 0; j < kFuseKeysPerThread; ++j) kv[j] = kw[j * 64 + lane];
  uint4* ba = reinterpret_cast<uint4*>(L.bits) + wave * (kFuseKeysPerThread / 2);
  uint4* bi = reinterpret_cast<uint4*>(L.bits2) + wave * (kFuseKeysPerThread / 2);
#pragma unroll
  for (int g = 0; g < kFuseKeysPerThread / 4; ++g) {
    uint32_t wa[8], wi[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t key = kv[4 * g + u];
      const unsigned long long ma = __ballot(key > top);
      const unsigned long long mi = __ballot(inside && key - lo <= top - lo);
      wa[2 * u] = (uint32_t)ma;
      wa[2 * u + 1] = (uint32_t)(ma >> 32);
      wi[2 * u] = (uint32_t)mi;
      wi[2 * u + 1] = (uint32_t)(mi >> 32);
    }
    if (lane == 0) {
      ba[2 * g] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
      ba[2 * g + 1] = make_uint4(wa[4], wa[5], wa[6], wa[7]);
      bi[2 * g] = make_uint4(wi[0], wi[1], wi[2], wi[3]);
      bi[2 * g + 1] = make_uint4(wi[4], wi[5], wi[6], wi[7]);
    }
  }
  __syncthreads();
}

// Publishes this workgroup's count of keys above the bin (key >> shift > pre; every
// non-zero key when `all`) and the composites of its keys inside it (key >> shift == pre,
// at most `cap` of them; the count says how many there were).  The keys above the bin are
// also marked in L.bits (local index i -> bit i; every word below n_local is written).
// One pass of wave ballots marks both sets; the composites are then compacted in position
// order from the second bitmap.  Returns the combined values of the atomics (for
// RowSync::sync).
__device__ __forceinline__ uint32_t publish(const uint32_t* keys, int n_local, uint32_t pos0,
                                            uint32_t pre, int shift, bool all, int cap,
                                            uint32_t* cnt_slot, unsigned long long* pub,
                                            const SelLds& L) {
  const int tid = threadIdx.x;
  // above: key > top; inside: lo <= key <= top (key 0 is never either)
  const uint32_t lo = all ? 1u : max(pre << shift, 1u);
  const uint32_t top = all ? 0u : (pre << shift) + ((1u << shift) - 1u);
  mark_pass(keys, lo, top, !all, L);
  // thread t owns local indices [16t, 16t + 16)
  const uint32_t wa = L.bits[tid >> 1], wi = L.bits2[tid >> 1];
  uint32_t ma = (tid & 1) ? (wa >> 16) : (wa & 0xffffu);
  uint32_t mi = (tid & 1) ? (wi >> 16) : (wi & 0xffffu);
  uint32_t tot;
  uint32_t slot = block_exclusive_scan(((uint32_t)__popc(ma) << 16) | (uint32_t)__popc(mi), L.scan,
                                       &tot) & 0xffffu;
  const uint32_t n_pub = tot & 0xffffu, total_above = tot >> 16;
  while (mi) {
    const uint32_t i = 16u * tid + (uint32_t)__builtin_ctz(mi);
    mi &= mi - 1u;
    if (slot < (uint32_t)cap) L.pub[slot] = composite(keys[i], pos0 + i);
    ++slot;
  }
  __syncthreads();
  uint32_t pending = 0;
  if (tid < (int)min(n_pub, (uint32_t)cap)) pending |= xchg_agent(&pub[tid], L.pub[tid]);
  if (tid == kFuseThreads - 1)
    pending |= xchg_agent(cnt_slot, (total_above << 16) | min(n_pub, 0xffffu));
  return pending;
}

// The need-th largest (1 <= need <= nt) of the nt unique composites in L.pub[0..nt), whose
// keys agree above bit `shift`; stored in *L.T (*L.T must be ~0 before).  Few composites:
// wave 0 ranks them directly; otherwise one 256-bin radix pass over the 8 key bits below
// `shift` and the few composites left in the chosen digit are ranked directly.  Whole
// workgroup; the caller's barrier publishes *L.T.  Uses L.pub[kPubMax..2 kPubMax) and L.h.
__device__ __forceinline__ void rank_composites(const SelLds& L, uint32_t nt, uint32_t need,
                                                int shift) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (nt <= 64u) {
    if (wave == 0) {
      const unsigned long long c = (uint32_t)lane < nt ? L.pub[lane] : 0ull;
      const uint32_t chi = (uint32_t)(c >> 32), clo = (uint32_t)c;
      uint32_t r = 0;
      for (uint32_t j = 0; j < nt; ++j) {
        const uint32_t ohi = __builtin_amdgcn_readlane(chi, j);
        const uint32_t olo = __builtin_amdgcn_readlane(clo, j);
        r += (ohi > chi || (ohi == chi && olo > clo)) ? 1u : 0u;
      }
      if ((uint32_t)lane < nt && r == need - 1u) *L.T = c;
    }
    return;
  }
  const int dsh = shift - 8;
  if (tid < 256) L.h[tid] = 0u;
  if (tid == 0) L.misc[0] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < nt; i += kFuseThreads)
    atomicAdd(&L.h[(uint32_t)(L.pub[i] >> (32 + dsh)) & 255u], 1u);
  __syncthreads();
  if (wave == 0) find_threshold_bin(L.h, 256, need, L.res);
  __syncthreads();
  const uint32_t da = L.res[0], need_b = need - L.res[1];
  for (uint32_t i = tid; i < nt; i += kFuseThreads) {
    const unsigned long long c = L.pub[i];
    if (((uint32_t)(c >> (32 + dsh)) & 255u) == da) L.pub[kPubMax + atomicAdd(&L.misc[0], 1u)] = c;
  }
  __syncthreads();
  const uint32_t nb = L.misc[0];
  const unsigned long long* cb = L.pub + kPubMax;
  for (uint32_t i = tid; i < nb; i += kFuseThreads) {
    const unsigned long long c = cb[i];
    uint32_t r = 0;
    uint32_t j = 0;
    for (; j + 8 <= nb; j += 8) {  // eight loads in flight per step
      unsigned long long x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = cb[j + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += x[u] > c ? 1u : 0u;
    }
    for (; j < nb; ++j) r += cb[j] > c ? 1u : 0u;
    if (r == need_b - 1u) *L.T = c;
  }
}

struct SelResult {
  uint32_t sel;     // entries this workgroup selected
  uint32_t offset;  // output position of its first one
  uint32_t total;   // entries the row selected
};

// One selection over keys[0..n_local) of every workgroup of the row (LDS; local index i =
// j * 1024 + thread, at position pos0 + i; key 0 = not selectable).  h1_ready: L.h already
// holds this workgroup's level-1 histogram.  Writes orow[0..k) (id_of(i), ascending
// positions, -1 padded) and srow (scores, -inf padded) if given; calls on_sel(rank, i) for
// the workgroup's selected entries in position order.  Whole workgroup, every workgroup of
// the row; ends with a barrier.
template <typename IdOf, typename OnSel>
__device__ __forceinline__ SelResult row_select(const uint32_t* keys, int n_local, uint32_t pos0, int k,
                                bool h1_ready, bool keep_hint, uint32_t fine_lo,
                                uint32_t pending_in,
                                const SelWs& g, RowSync& rs, const SelLds& L,
                                int wg, int nwg, int32_t* orow, float* srow, IdOf id_of,
                                OnSel on_sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int iters = (n_local + kFuseThreads - 1) / kFuseThreads;
  const int cap = min(kPubSlots / nwg, kPubMax);
  const bool fine_on = fine_lo != 0xffffffffu;  // the scan counted the fine window
  uint32_t pending = pending_in;

  // ---- level 1: every workgroup's histogram into the row's, then the bin of the k-th key
  if (!h1_ready) local_hist(keys, n_local, 0u, 20, kHist1Bins, 12, L.h);
  pending |= flush_hist<4>(L.h, kHist1Bins, g.h1);
  rs.sync(pending);
  pending = 0;
  uint32_t k_eff = (uint32_t)k;
  bool all = false;           // the same in every workgroup of the row
  uint32_t pre = 0, need = 0;  // need: keys still to take at or below the bin
  uint32_t b1 = 0, need1 = 0;
  int shift = 20;
  bool pub_now = true;  // publish now (always when every key is taken)
  bool fast = false;    // the k-th key's fine sub-bin came from the scan's window
  if (fine_on) {
    // the window's 256 fine counts (index (bin - fine_lo) * 16 + sub-bin) and the keys
    // above it: when the k-th key falls inside and its sub-bin is small enough, level 1
    // and its histogram are skipped
    if (tid < kFineWin * kFineSub) L.h[tid] = ld_agent(&g.fine[(fine_lo << 4) + tid]);
    if (tid == kFineWin * kFineSub) L.misc[2] = ld_agent(g.above);
    __syncthreads();
    if (wave == 0) {
      const uint32_t above = L.misc[2];
      const int hi = kFineWin * kFineSub - 4 * lane;  // lane 0 owns the top counts
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = L.h[hi - 1 - j];
        sum += c4[j];
      }
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t win = __builtin_amdgcn_readlane(incl, 63);
      const bool hit = above < (uint32_t)k && (uint32_t)k - above <= win;
      uint32_t idx = 0u, before = 0u;  // the sub-bin and the keys above it (absolute)
      if (hit) {
        const uint32_t want = (uint32_t)k - above;
        uint32_t acc = incl - sum;
        bool mine = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!mine && acc < want && want <= acc + c4[j]) {
            mine = true;
            idx = (uint32_t)(hi - 1 - j);
            before = above + acc;
          }
          acc += c4[j];
        }
        const unsigned long long owner = __ballot(mine);
        const int ol = (int)__builtin_ctzll(owner);
        idx = __builtin_amdgcn_readlane(idx, ol);
        before = __builtin_amdgcn_readlane(before, ol);
        // keys above the sub-bin's level-1 bin (for the massive-tie rule)
        const uint32_t bin_top = ((idx >> 4) + 1u) << 4;
        uint32_t part = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) part += (uint32_t)(hi - 1 - j) >= bin_top ? c4[j] : 0u;
        const uint32_t above_bin = above + __builtin_amdgcn_readlane(wave_incl_scan(part), 63);
        if (lane == 0) {
          L.res[0] = idx;
          L.res[1] = before;
          L.res[2] = L.h[idx];
          L.res[3] = above_bin;
        }
      }
      if (lane == 0) L.misc[1] = hit ? 1u : 0u;
    }
    __syncthreads();
    if (L.misc[1] != 0u && L.res[2] <= (uint32_t)kPubMax) {
      fast = true;
      b1 = fine_lo + (L.res[0] >> 4);
      need1 = (uint32_t)k - L.res[3];
      pre = (b1 << 4) | (L.res[0] & 15u);
      need = (uint32_t)k - L.res[1];
      shift = 16;
      if (keep_hint && wg == 0 && tid == 0) st_agent(g.hint, b1 + 1u);  // for the next call
    }
    __syncthreads();  // L.h, L.res and L.misc are read before they are rewritten
  }
  if (!fast) {
#pragma unroll
    for (int i = 0; i < 4; ++i) L.h[tid + i * kFuseThreads] = ld_agent(&g.h1[tid + i * kFuseThreads]);
    __syncthreads();
    const uint32_t total = hist_select<4>(L.h, (uint32_t)k, L.scan, L.res);
    k_eff = min((uint32_t)k, total);
    all = k_eff == total;
    if (!all) {
      b1 = pre = L.res[0];
      need1 = need = k_eff - L.res[1];
      pub_now = L.h[pre] <= (uint32_t)kPubMax;
      if (keep_hint && wg == 0 && tid == 0) st_agent(g.hint, b1 + 1u);  // for the next call
      if (!pub_now && fine_on && b1 - fine_lo < (uint32_t)kFineWin) {
        // the fine counts of b1 are complete: the sub-bin of the need-th key
        __syncthreads();
        if (tid < kFineSub) L.h[tid] = ld_agent(&g.fine[(b1 << 4) + tid]);
        __syncthreads();
        if (wave == 0) {
          const uint32_t c = lane < kFineSub ? L.h[kFineSub - 1 - lane] : 0u;  // from the top
          const uint32_t incl = wave_incl_scan(c);
          if (lane < kFineSub && incl - c < need && need <= incl) {
            L.res[0] = (uint32_t)(kFineSub - 1 - lane);
            L.res[1] = incl - c;
            L.res[2] = c;
          }
        }
        __syncthreads();
        if (L.res[2] <= (uint32_t)kPubMax) {
          pre = (b1 << 4) | L.res[0];
          need -= L.res[1];
          shift = 16;
          pub_now = true;
        }
      }
    }
  }
  __syncthreads();  // L.h and L.res are read before they are rewritten
  if (pub_now) {
    pending |= publish(keys, n_local, pos0, pre, shift, all, cap, g.cnt + wg, g.pub + wg * cap, L);
  } else {
    local_hist(keys, n_local, pre, 9, kHist2Bins, 11, L.h);
    pending |= flush_hist<2>(L.h, kHist2Bins, g.h2);
  }
  rs.sync(pending);
  pending = 0;
  if (wg == 0) {
    for (int i = tid; i < kHist1Bins; i += kFuseThreads) st_agent(&g.h1[i], 0u);
    if (fine_on && tid < kFineWin * kFineSub) st_agent(&g.fine[(fine_lo << 4) + tid], 0u);
    if (fine_on && tid == kFineWin * kFineSub) st_agent(g.above, 0u);
  }

  // ---- level 2 (when b1 held too many keys): the bin (b1, b2), then publish
  if (!pub_now) {
    L.h[tid] = ld_agent(&g.h2[tid]);
    L.h[tid + kFuseThreads] = ld_agent(&g.h2[tid + kFuseThreads]);
    __syncthreads();
    hist_select<2>(L.h, need, L.scan, L.res);
    pre = (pre << 11) | L.res[0];
    need -= L.res[1];
    shift = 9;
    pending |= publish(keys, n_local, pos0, pre, shift, false, cap, g.cnt + wg, g.pub + wg * cap, L);
    rs.sync(pending);
    pending = 0;
    if (wg == 0)
      for (int i = tid; i < kHist2Bins; i += kFuseThreads) st_agent(&g.h2[i], 0u);
  }

  // ---- the published composites: every workgroup ranks them itself
  const uint32_t cv = tid < nwg ? ld_agent(&g.cnt[tid]) : 0u;
  const int s0 = tid, s1 = tid + kFuseThreads;
  const int v0 = s0 / cap, v1 = s1 / cap;
  const unsigned long long t0 = v0 < nwg ? ld_agent(&g.pub[s0]) : 0ull;
  const unsigned long long t1 = v1 < nwg ? ld_agent(&g.pub[s1]) : 0ull;
  const uint32_t npub_v = cv & 0xffffu;
  if (tid < nwg) L.selt[tid] = npub_v;
  uint32_t pub_total;
  block_exclusive_scan(npub_v, L.scan, &pub_total);  // barrier: L.selt complete
  const bool overflow =
      (__syncthreads_or(tid < nwg && npub_v > (uint32_t)cap) != 0) || pub_total > (uint32_t)kPubMax;

  // selected: key > tkey, or key == tkey at a position <= cut (when has_cut)
  uint32_t tkey = 0u, cut = 0u;
  bool has_cut = false;
  uint32_t offset;
  if (!overflow) {
    const bool ok0 = v0 < nwg && (uint32_t)(s0 - v0 * cap) < L.selt[v0];
    const bool ok1 = v1 < nwg && (uint32_t)(s1 - v1 * cap) < L.selt[v1];
    uint32_t nt;
    const uint32_t p = block_exclusive_scan((ok0 ? 1u : 0u) + (ok1 ? 1u : 0u), L.scan, &nt);
    if (ok0) L.pub[p] = t0;
    if (ok1) L.pub[p + (ok0 ? 1u : 0u)] = t1;
    if (tid < nwg) L.selt[tid] = 0u;
    if (tid == 0) *L.T = ~0ull;
    __syncthreads();
    if (!all) rank_composites(L, nt, need, shift);
    __syncthreads();
    if (!all) {
      const unsigned long long T = *L.T;
      tkey = (uint32_t)(T >> 32);
      cut = ~(uint32_t)T;
      has_cut = true;
      if (ok0 && t0 >= T) {
        atomicAdd(&L.selt[v0], 1u);
        if (v0 == wg) {  // this workgroup's own tied key is taken
          const uint32_t i = ~(uint32_t)t0 - pos0;
          atomicOr(&L.bits[i >> 5], 1u << (i & 31));
        }
      }
      if (ok1 && t1 >= T) {
        atomicAdd(&L.selt[v1], 1u);
        if (v1 == wg) {
          const uint32_t i = ~(uint32_t)t1 - pos0;
          atomicOr(&L.bits[i >> 5], 1u << (i & 31));
        }
      }
    }
    __syncthreads();
    const uint32_t sel_v = tid < nwg ? (cv >> 16) + L.selt[tid] : 0u;
    block_exclusive_scan(tid < wg ? sel_v : 0u, L.scan, &offset);
  } else {
    // massive ties: the threshold key from a level-3 histogram (after level 2, if the
    // keys were published at level 1), then each workgroup's share of the equal keys
    if (shift != 9) {  // published from b1 or its fine sub-bin: level 2 from b1
      pre = b1;
      need = need1;
      local_hist(keys, n_local, pre, 9, kHist2Bins, 11, L.h);
      pending |= flush_hist<2>(L.h, kHist2Bins, g.h2);
      rs.sync(pending);
      pending = 0;
      L.h[tid] = ld_agent(&g.h2[tid]);
      L.h[tid + kFuseThreads] = ld_agent(&g.h2[tid + kFuseThreads]);
      __syncthreads();
      hist_select<2>(L.h, need, L.scan, L.res);
      pre = (pre << 11) | L.res[0];
      need -= L.res[1];
    }
    local_hist(keys, n_local, pre, 0, kHist3Bins, 9, L.h);
    pending |= flush_hist<1>(L.h, kHist3Bins, g.h3);
    rs.sync(pending);
    pending = 0;
    if (wg == 0)
      for (int i = tid; i < kHist2Bins; i += kFuseThreads) st_agent(&g.h2[i], 0u);
    if (tid < kHist3Bins) L.h[tid] = ld_agent(&g.h3[tid]);
    __syncthreads();
    if (wave == 0) find_threshold_bin(L.h, kHist3Bins, need, L.res);
    __syncthreads();
    tkey = (pre << 9) | L.res[0];
    const uint32_t need_eq = need - L.res[1];  // keys equal to tkey still to take, >= 1
    uint32_t n_gt = 0, n_eq = 0;
    for (int i = tid; i < n_local; i += kFuseThreads) {
      const uint32_t key = keys[i];
      n_gt += key > tkey ? 1u : 0u;
      n_eq += key == tkey ? 1u : 0u;
    }
    uint32_t packed;  // both counts are <= 16,384
    block_exclusive_scan((n_gt << 16) | n_eq, L.scan, &packed);
    if (tid == 0) pending |= xchg_agent(g.cnt + wg, packed);
    rs.sync(pending);
    pending = 0;
    if (wg == 0 && tid < kHist3Bins) st_agent(&g.h3[tid], 0u);
    // the equal keys go to the lowest positions: workgroup by workgroup, then locally
    const uint32_t cw = tid < nwg ? ld_agent(&g.cnt[tid]) : 0u;
    const uint32_t eq_v = cw & 0xffffu;
    uint32_t unused;
    const uint32_t eq_before = block_exclusive_scan(eq_v, L.scan, &unused);
    const uint32_t take_v = min(eq_v, need_eq > eq_before ? need_eq - eq_before : 0u);
    if (tid == wg) L.misc[2] = take_v;
    block_exclusive_scan(tid < wg ? (cw >> 16) + take_v : 0u, L.scan, &offset);  // barrier
    const uint32_t take = L.misc[2];
    if (take > 0u) {  // position of this workgroup's take-th equal key
      for (int j = 0; j < iters; ++j) {
        const int i = j * kFuseThreads + tid;
        const unsigned long long m = __ballot(i < n_local && keys[i] == tkey);
        if (lane == 0) L.cnt[j * kFuseWaves + wave] = (uint32_t)__popcll(m);
      }
      __syncthreads();
      if (wave == 0) scan_counts_wave0_n<4>(L.cnt, iters * kFuseWaves);
      __syncthreads();
      for (int j = 0; j < iters; ++j) {
        const int i = j * kFuseThreads + tid;
        const bool eq = i < n_local && keys[i] == tkey;
        const unsigned long long m = __ballot(eq);
        if (eq && L.cnt[j * kFuseWaves + wave] + lanes_below(m) == take - 1u)
          L.misc[3] = pos0 + (uint32_t)i;
      }
      __syncthreads();
      cut = L.misc[3];
      has_cut = true;
    }
  }

  // ---- the selected entries in position order
  int32_t* const out_ids = orow;
  if (!overflow) {
    // from the bitmap: thread t owns local indices [16t, 16t + 16)
    const int i0 = 16 * tid;
    const uint32_t w = L.bits[tid >> 1];
    uint32_t m = (tid & 1) ? (w >> 16) : (w & 0xffffu);
    if (i0 >= n_local) m = 0u;
    else if (i0 + 16 > n_local) m &= (1u << (n_local - i0)) - 1u;
    uint32_t n_sel;
    uint32_t rank = block_exclusive_scan((uint32_t)__popc(m), L.scan, &n_sel);
    if (tid == 0) L.misc[1] = n_sel;
    while (m) {
      const int i = i0 + __builtin_ctz(m);
      m &= m - 1u;
      const uint32_t pos = offset + rank;
      if (pos < (uint32_t)k) {
        out_ids[pos] = id_of(i);
        if (srow) srow[pos] = key_score(keys[i]);
      }
      on_sel(rank, i);
      ++rank;
    }
  } else {
    uint32_t selbits = 0;
    for (int j = 0; j < iters; ++j) {
      const int i = j * kFuseThreads + tid;
      const uint32_t key = i < n_local ? keys[i] : 0u;
      const bool take =
          key != 0u && (key > tkey || (key == tkey && has_cut && pos0 + (uint32_t)i <= cut));
      selbits |= (take ? 1u : 0u) << j;
      const unsigned long long m = __ballot(take);
      if (lane == 0) L.cnt[j * kFuseWaves + wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t n = scan_counts_wave0_n<4>(L.cnt, iters * kFuseWaves);
      if (lane == 0) L.misc[1] = n;
    }
    __syncthreads();
    for (int j = 0; j < iters; ++j) {
      const bool take = (selbits >> j) & 1u;
      const unsigned long long m = __ballot(take);
      if (take) {
        const int i = j * kFuseThreads + tid;
        const uint32_t rank = L.cnt[j * kFuseWaves + wave] + lanes_below(m);
        const uint32_t pos = offset + rank;
        if (pos < (uint32_t)k) {
          out_ids[pos] = id_of(i);
          if (srow) srow[pos] = key_score(keys[i]);
        }
        on_sel(rank, i);
      }
    }
  }
  for (int p = (int)k_eff + wg * kFuseThreads + tid; p < k; p += nwg * kFuseThreads) {
    orow[p] = -1;
    if (srow) srow[p] = -__builtin_inff();
  }
  const SelResult r{L.misc[1], offset, k_eff};
  __syncthreads();
  return r;
}

// Top-k of keys[0..n) (LDS; key 0 = not selectable; position = index) by one workgroup,
// with the rule of the row selections: the k largest, ties to the lower position, written
// in position order as id_of(i) into orow[0..k), -1 padded; scores into srow if given.
// L.h holds the keys' level-1 histogram on entry.  The level-1 bin (or the level-2 bin
// when it holds too many) is ranked from its composites, gathered in the same pass that
// marks the keys above it in a bitmap; massive ties take level 3 and the lowest positions
// among the equal keys.
template <typename IdOf>
__device__ __forceinline__ void wg_select(const uint32_t* keys, int n, int k, const SelLds& L,
                                          int32_t* orow, float* srow, IdOf id_of) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int iters = (n + kFuseThreads - 1) / kFuseThreads;
  const uint32_t total = hist_select<4>(L.h, (uint32_t)k, L.scan, L.res);
  const uint32_t k_eff = min((uint32_t)k, total);
  // selected: key > tkey, or key == tkey at index <= cut (when has_cut); marked in L.bits
  uint32_t tkey = 0u, cut = 0u;
  bool has_cut = false, marked = false;
  if (k_eff < total) {
    uint32_t pre = L.res[0], need = k_eff - L.res[1];
    int shift = 20;
    bool small = L.h[pre] <= (uint32_t)kPubMax;
    __syncthreads();
    if (!small) {
      local_hist(keys, n, pre, 9, kHist2Bins, 11, L.h);
      hist_select<2>(L.h, need, L.scan, L.res);
      const uint32_t b2 = L.res[0];
      need -= L.res[1];
      small = L.h[b2] <= (uint32_t)kPubMax;
      pre = (pre << 11) | b2;
      shift = 9;
      __syncthreads();
    }
    if (small) {
      // one pass of ballots: the keys above the bin into L.bits, the bin's keys into
      // L.bits2; then the bin's composites are compacted into L.pub
      if (tid == 0) *L.T = ~0ull;
      mark_pass(keys, max(pre << shift, 1u), (pre << shift) + ((1u << shift) - 1u), true, L);
      const uint32_t wi = L.bits2[tid >> 1];
      uint32_t mi = (tid & 1) ? (wi >> 16) : (wi & 0xffffu);
      uint32_t nt;
      uint32_t slot = block_exclusive_scan((uint32_t)__popc(mi), L.scan, &nt);
      while (mi) {
        const uint32_t i = 16u * tid + (uint32_t)__builtin_ctz(mi);
        mi &= mi - 1u;
        L.pub[slot++] = composite(keys[i], i);
      }
      __syncthreads();
      rank_composites(L, nt, need, shift);
      __syncthreads();
      const unsigned long long T = *L.T;
      for (uint32_t t = tid; t < nt; t += kFuseThreads) {
        const unsigned long long c = L.pub[t];
        if (c >= T) {
          const uint32_t i = ~(uint32_t)c;
          atomicOr(&L.bits[i >> 5], 1u << (i & 31));
        }
      }
      marked = true;
    } else {
      local_hist(keys, n, pre, 0, kHist3Bins, 9, L.h);
      if (wave == 0) find_threshold_bin(L.h, kHist3Bins, need, L.res);
      __syncthreads();
      tkey = (pre << 9) | L.res[0];
      const uint32_t need_eq = need - L.res[1];
      for (int j = 0; j < iters; ++j) {
        const int i = j * kFuseThreads + tid;
        const unsigned long long m = __ballot(i < n && keys[i] == tkey);
        if (lane == 0) L.cnt[j * kFuseWaves + wave] = (uint32_t)__popcll(m);
      }
      __syncthreads();
      if (wave == 0) scan_counts_wave0_n<4>(L.cnt, iters * kFuseWaves);
      __syncthreads();
      for (int j = 0; j < iters; ++j) {
        const int i = j * kFuseThreads + tid;
        const bool eq = i < n && keys[i] == tkey;
        const unsigned long long m = __ballot(eq);
        if (eq && L.cnt[j * kFuseWaves + wave] + lanes_below(m) == need_eq - 1u) L.misc[3] = (uint32_t)i;
      }
      __syncthreads();
      cut = L.misc[3];
      has_cut = true;
    }
  }
  if (!marked) {  // every selectable key, or the massive-tie rule: mark by wave ballots
    for (int j = 0; j < iters; ++j) {
      const int i = j * kFuseThreads + tid;
      const uint32_t key = i < n ? keys[i] : 0u;
      const bool take = key != 0u && (key > tkey || (key == tkey && has_cut && (uint32_t)i <= cut));
      const unsigned long long m = __ballot(take);
      if (lane == 0) {
        L.bits[(j * kFuseThreads + wave * 64) >> 5] = (uint32_t)m;
        L.bits[((j * kFuseThreads + wave * 64) >> 5) + 1] = (uint32_t)(m >> 32);
      }
    }
  }
  __syncthreads();
  // one scan over the bitmap gives every output position
  const int i0 = 16 * tid;
  const uint32_t w = L.bits[tid >> 1];
  uint32_t m = (tid & 1) ? (w >> 16) : (w & 0xffffu);
  if (i0 >= n) m = 0u;
  else if (i0 + 16 > n) m &= (1u << (n - i0)) - 1u;
  uint32_t n_sel;
  uint32_t rank = block_exclusive_scan((uint32_t)__popc(m), L.scan, &n_sel);
  while (m) {
    const int i = i0 + __builtin_ctz(m);
    m &= m - 1u;
    if (rank < (uint32_t)k) {
      orow[rank] = id_of(i);
      if (srow) srow[rank] = key_score(keys[i]);
    }
    ++rank;
  }
  for (int p = (int)k_eff + tid; p < k; p += kFuseThreads) {
    orow[p] = -1;
    if (srow) srow[p] = -__builtin_inff();
  }
  __syncthreads();
}

struct ChainArgs {
  const uint16_t* q_idx;     // [batch][128] query of the scan
  const uint8_t* codes;
  const float* scale;
  const int64_t* seq_base;
  const int32_t* n_valid;
  const int32_t* cand;       // candidate map of the scan (CAND)
  int n_cols, cols_per_wg, row0;
  int k;                     // the scan's selection (the pool)
  int32_t* idx_out;          // [batch][k]
  float* score_out;          // [batch][k] or null
  int own_k;                 // top-own_k of the pool by the scan's scores (0: none)
  int32_t* own_out;          // [batch][own_k]
  int n_re;                  // Reindex layers re-scoring the pool (0..kMaxReindex)
  int re_k;
  const uint16_t* q_re;      // [n_re][batch][128]
  int32_t* re_out;           // [n_re][batch][re_k]
  float* re_score_out;       // [n_re][batch][re_k] or null
  int batch;
  uint32_t* status;
  uint32_t* sync;
  char* sel_base;
  char* fine_base;
  uint32_t* pool_base;       // [batch][kMaxSel][16384]: pool ids, then each layer's keys
};

template <bool CAND>
__global__ __launch_bounds__(kFuseThreads) void k_index_topk(ChainArgs a) {
  __shared__ uint32_t s_key[kFuseMaxCols];
  __shared__ uint32_t s_h[kHist1Bins];
  __shared__ uint16_t s_plist[CAND ? 1 : kFuseMaxCols];  // columns of this workgroup's pool
  __shared__ unsigned long long s_pub[2 * kPubMax];
  __shared__ uint32_t s_cnt[kFuseKeysPerThread * kFuseWaves];
  __shared__ uint32_t s_selt[kFuseMaxWg];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_misc[4];
  __shared__ unsigned long long s_T;
  __shared__ __align__(16) uint32_t s_bits[kFuseMaxCols / 32];
  __shared__ __align__(16) uint32_t s_bits2[kFuseMaxCols / 32];
  __shared__ uint32_t s_fine[kFineWin * kFineSub];
  __shared__ __align__(16) uint16_t s_qre[CAND ? 1 : kMaxReindex * kDIdx];  // Reindex queries
  const int b = a.row0 + (int)blockIdx.y, wg = blockIdx.x, nwg = gridDim.x;
  const int tid = threadIdx.x;
  const int nv = min(a.n_valid[b], a.n_cols);
  const int c0 = wg * a.cols_per_wg, c1 = min(c0 + a.cols_per_wg, a.n_cols);
  const int32_t* cand_row = CAND ? a.cand + (size_t)b * a.n_cols : nullptr;
  const int64_t base = a.seq_base[b];
  RowSync rs{a.sync + (size_t)b * kSyncStride, a.status, (uint32_t)nwg, 0u};
  SelLds L;
  L.h = s_h;
  L.cnt = s_cnt;
  L.pub = s_pub;
  L.selt = s_selt;
  L.scan = s_scan;
  L.res = s_res;
  L.misc = s_misc;
  L.T = &s_T;
  L.bits = s_bits;
  L.bits2 = s_bits2;

  // ---- score the columns [c0, c1): keys into LDS, level-1 histogram in LDS, and the fine
  // counts of the window around the previous call's level-1 bin (long rows)
  uint32_t fine_lo = 0xffffffffu;
  const bool long_row = (uint32_t)nv >= kFineMinRow;
  if (long_row) {
    const uint32_t h = ld_agent(sel_ws(a.sel_base, b, 0, a.fine_base, a.sync).hint);
    if (h != 0u) fine_lo = min(h - 1u >= 8u ? h - 9u : 0u, (uint32_t)(kHist1Bins - kFineWin));
  }
  const bool fine_on = fine_lo != 0xffffffffu;
  if (!CAND && tid < a.n_re * (kDIdx / 8)) {  // read long before the re-scores use them
    const int rl = tid / (kDIdx / 8), part = tid % (kDIdx / 8);
    reinterpret_cast<uint4*>(s_qre)[tid] =
        reinterpret_cast<const uint4*>(a.q_re + ((size_t)rl * a.batch + b) * kDIdx)[part];
  }
  uint32_t n_above_win = 0;  // this thread's keys above the window
  for (int i = tid; i < kFuseMaxCols; i += kFuseThreads) s_key[i] = 0u;
  if (nv > 0) {
    scan_columns<CAND, kFuseThreads>(
        a.q_idx + (size_t)b * kDIdx, a.codes, a.scale, cand_row, base, nv, c0, c1,
        [&]() {
          for (int i = tid; i < kHist1Bins; i += kFuseThreads) s_h[i] = 0u;
          if (tid < kFineWin * kFineSub) s_fine[tid] = 0u;
          if (tid == 0) s_misc[3] = 0u;
        },
        [&](int col, float score, bool valid) {
          const uint32_t key = valid ? score_key(score) : 0u;
          s_key[col - c0] = key;
          if (key != 0u) {
            atomicAdd(&s_h[key >> 20], 1u);
            const uint32_t cw = (key >> 20) - fine_lo;
            if (fine_on && cw < (uint32_t)kFineWin)
              atomicAdd(&s_fine[(cw << 4) | ((key >> 16) & 15u)], 1u);
            n_above_win += (fine_on && (key >> 20) >= fine_lo + kFineWin) ? 1u : 0u;
          }
        });
    if (fine_on) {
      const uint32_t wsum = wave_incl_scan(n_above_win);
      if ((tid & 63) == 63 && wsum) atomicAdd(&s_misc[3], wsum);
    }
    __syncthreads();
  }
  uint32_t fine_pending = 0;
  if (fine_on && nv > 0 && tid <= kFineWin * kFineSub) {
    const SelWs g0 = sel_ws(a.sel_base, b, 0, a.fine_base, a.sync);
    const uint32_t v = tid < kFineWin * kFineSub ? s_fine[tid] : s_misc[3];
    if (v) fine_pending = add_agent(tid < kFineWin * kFineSub ? &g0.fine[(fine_lo << 4) + tid] : g0.above, v);
  }

  // ---- the scan's selection (the pool when chained)
  const bool chain = !CAND && (a.own_k > 0 || a.n_re > 0);
  const SelResult pool = row_select(
      s_key, c1 - c0, (uint32_t)c0, a.k, nv > 0, long_row, fine_lo, fine_pending,
      sel_ws(a.sel_base, b, 0, a.fine_base, a.sync), rs, L, wg, nwg,
      a.idx_out + (size_t)b * a.k, a.score_out ? a.score_out + (size_t)b * a.k : nullptr,
      [&](int i) { return CAND ? cand_row[c0 + i] : c0 + i; },
      [&](uint32_t rank, int i) {
        if (chain) s_plist[rank] = (uint16_t)i;
      });

  if (chain) {
    // Every workgroup writes its pool entries' ids and, for every layer, their keys (the
    // Full layer's own keys, or the Reindex layer's re-scores) at their pool positions;
    // after one barrier, workgroup L selects layer L's top-k from the whole pool in LDS.
    const int n_pool = (int)pool.sel;
    const int own = a.own_k > 0 ? 1 : 0;
    const int n_layers = own + a.n_re;
    uint32_t* parr = a.pool_base + (size_t)b * kMaxSel * kFuseMaxCols;
    uint32_t pending = 0;
    {
      uint32_t r[kFuseKeysPerThread];
#pragma unroll
      for (int j = 0; j < kFuseKeysPerThread; ++j) {
        const int i = j * kFuseThreads + tid;
        r[j] = i < n_pool ? xchg_agent(&parr[pool.offset + i], (uint32_t)(c0 + s_plist[i])) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kFuseKeysPerThread; ++j) pending |= r[j];
    }
    const int lane = tid & 63, wave = tid >> 6, quarter = lane & 3, ent = lane >> 2;
    for (int lyr = 0; lyr < n_layers; ++lyr) {
      // this layer's keys of the pool entries: written at their pool positions and
      // counted into the layer's level-1 histogram (the selector's first step)
      uint32_t* pk = parr + (size_t)(1 + lyr) * kFuseMaxCols + pool.offset;
      for (int i = tid; i < kHist1Bins; i += kFuseThreads) s_h[i] = 0u;
      __syncthreads();
      if (own && lyr == 0) {
        uint32_t r[kFuseKeysPerThread];
#pragma unroll
        for (int j = 0; j < kFuseKeysPerThread; ++j) {
          const int i = j * kFuseThreads + tid;
          r[j] = 0u;
          if (i < n_pool) {
            const uint32_t key = s_key[s_plist[i]];
            r[j] = xchg_agent(&pk[i], key);
            atomicAdd(&s_h[key >> 20], 1u);
          }
        }
#pragma unroll
        for (int j = 0; j < kFuseKeysPerThread; ++j) pending |= r[j];
      } else {
        // re-score with the Reindex layer's query (the scan's arithmetic)
        const int rl = lyr - own;
        bf16x2 q[16];
        {
          const uint4* qp = reinterpret_cast<const uint4*>(s_qre + rl * kDIdx) + quarter * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = qp[i];
            q[4 * i + 0] = __builtin_bit_cast(bf16x2, v.x);
            q[4 * i + 1] = __builtin_bit_cast(bf16x2, v.y);
            q[4 * i + 2] = __builtin_bit_cast(bf16x2, v.z);
            q[4 * i + 3] = __builtin_bit_cast(bf16x2, v.w);
          }
        }
        constexpr int kU = 4;  // groups of 16 entries per wave in flight
        for (int g0 = wave * 16 * kU; g0 < n_pool; g0 += kFuseWaves * 16 * kU) {
          uint4 w[kU];
          float sc[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int i = min(g0 + u * 16 + ent, n_pool - 1);
            const int64_t e = base + c0 + s_plist[i];
            w[u] = *reinterpret_cast<const uint4*>(a.codes + e * kIdxCodeBytes + quarter * 16);
            sc[u] = a.scale[e];
          }
          uint32_t rr[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            float v = dot32(w[u], q);
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            const int i = g0 + u * 16 + ent;
            rr[u] = 0u;
            if (quarter == 0 && i < n_pool) {
              const uint32_t key = score_key(v * sc[u]);
              rr[u] = xchg_agent(&pk[i], key);
              atomicAdd(&s_h[key >> 20], 1u);
            }
          }
#pragma unroll
          for (int u = 0; u < kU; ++u) pending |= rr[u];
        }
      }
      __syncthreads();
      pending |= flush_hist<4>(s_h, kHist1Bins, sel_ws(a.sel_base, b, 1 + lyr, a.fine_base, a.sync).h1);
    }
    rs.sync(pending);
    for (int lyr = wg; lyr < n_layers; lyr += nwg) {
      const uint32_t* pk = parr + (size_t)(1 + lyr) * kFuseMaxCols;
      uint32_t* gh = sel_ws(a.sel_base, b, 1 + lyr, a.fine_base, a.sync).h1;
      const int n_all = (int)pool.total;
      uint32_t kk[kFuseKeysPerThread];
#pragma unroll
      for (int j = 0; j < kFuseKeysPerThread; ++j) {
        const int i = j * kFuseThreads + tid;
        kk[j] = i < n_all ? ld_agent(&pk[i]) : 0u;
      }
      uint32_t hh[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) hh[u] = ld_agent(&gh[tid + u * kFuseThreads]);
#pragma unroll
      for (int j = 0; j < kFuseKeysPerThread; ++j) s_key[j * kFuseThreads + tid] = kk[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s_h[tid + u * kFuseThreads] = hh[u];
        st_agent(&gh[tid + u * kFuseThreads], 0u);  // ready for the next call
      }
      __syncthreads();
      const bool is_own = own && lyr == 0;
      const int kl = is_own ? a.own_k : a.re_k;
      int32_t* orow = is_own ? a.own_out + (size_t)b * a.own_k
                             : a.re_out + ((size_t)(lyr - own) * a.batch + b) * a.re_k;
      float* srow = is_own || !a.re_score_out
                        ? nullptr
                        : a.re_score_out + ((size_t)(lyr - own) * a.batch + b) * a.re_k;
      wg_select(s_key, n_all, kl, L, orow, srow,
                [&](int i) { return (int32_t)ld_agent(&parr[i]); });
    }
  }

  // ---- the last workgroup of the row to leave resets the row's barrier counters
  if (tid == 0) {
    const uint32_t old = add_agent(rs.arrivals + 1, 1u);
    if (old == rs.nw - 1u) {
      st_agent(rs.arrivals, 0u);
      st_agent(rs.arrivals + 1, 0u);
    }
  }
}

// Valid (non-negative) leading entries of each row of a -1 padded list.
__global__ __launch_bounds__(256) void k_count_valid(const int32_t* __restrict__ list, int k,
                                                     int32_t* __restrict__ n_out) {
  __shared__ uint32_t s_scan[32];
  const int b = blockIdx.x;
  uint32_t c = 0;
  for (int i = threadIdx.x; i < k; i += 256) c += list[(size_t)b * k + i] >= 0 ? 1u : 0u;
  uint32_t total;
  block_exclusive_scan(c, s_scan, &total);
  if (threadIdx.x == 0) n_out[b] = (int32_t)total;
}

// ---------------------------------------------------------------------------- host side
namespace {

constexpr int kMaxDevices = 64;
int g_capacity[kMaxDevices];  // co-resident workgroups of k_index_topk per device (0: unknown)

int fused_capacity() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (g_capacity[dev] > 0) return g_capacity[dev];
  int per_cu_a = 0, per_cu_b = 0, n_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu_a, reinterpret_cast<const void*>(k_index_topk<false>), kFuseThreads, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu_b, reinterpret_cast<const void*>(k_index_topk<true>), kFuseThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  g_capacity[dev] = min(min(per_cu_a, per_cu_b) * n_cu, kFuseMaxWg);
  return g_capacity[dev];
}

// Columns per workgroup: a multiple of 1,024 up to 16,384, spreading the whole batch over
// the device's capacity where it can.
int fused_cols_per_wg(int batch, int n_cols, int capacity) {
  const long long want = ((long long)n_cols * batch + capacity - 1) / capacity;
  long long c = (want + kFuseThreads - 1) / kFuseThreads * kFuseThreads;
  if (c < kFuseThreads) c = kFuseThreads;
  if (c > kFuseMaxCols) c = kFuseMaxCols;
  return (int)c;
}

// The single-launch kernel applies when one row's workgroups fit the device at once.
bool fused_fits(int batch, int n_cols, int capacity, int* cpw_out, int* nwg_out) {
  if (capacity <= 0) return false;
  const int cpw = fused_cols_per_wg(batch, n_cols, capacity);
  const long long nwg = ((long long)n_cols + cpw - 1) / cpw;
  if (nwg > capacity) return false;
  *cpw_out = cpw;
  *nwg_out = (int)nwg;
  return true;
}

size_t fuse_part_bytes(int batch) {
  return 256 + align_up((size_t)batch * kSyncStride * 4, 256) + (size_t)batch * kMaxSel * kSelBytes +
         (size_t)batch * kFineBytes + (size_t)batch * kMaxSel * kFuseMaxCols * 4;
}

struct FuseParts {
  uint32_t* status;
  uint32_t* sync;
  char* sel_base;
  char* fine_base;
  uint32_t* pool_base;
};

FuseParts fuse_carve(void* base, int batch) {
  char* p = static_cast<char*>(base);
  FuseParts f;
  f.status = reinterpret_cast<uint32_t*>(p);
  f.sync = reinterpret_cast<uint32_t*>(p + 256);
  f.sel_base = p + 256 + align_up((size_t)batch * kSyncStride * 4, 256);
  f.fine_base = f.sel_base + (size_t)batch * kMaxSel * kSelBytes;
  f.pool_base = reinterpret_cast<uint32_t*>(f.fine_base + (size_t)batch * kFineBytes);
  return f;
}

// Two-launch path of one selection: [scores f32 batch x n_cols][top-k workspace].
size_t two_step_bytes(int batch, int n_cols) {
  return align_up((size_t)batch * n_cols * 4, 256) + topk_ws_bytes(batch, n_cols);
}

hipError_t two_step(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                    const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand, int batch,
                    int n_cols, int k, int32_t* idx_out, float* score_out, char* p,
                    hipStream_t stream) {
  float* scores = reinterpret_cast<float*>(p);
  const TopkWs tw = topk_ws_carve(p + align_up((size_t)batch * n_cols * 4, 256), batch, n_cols);
  hipError_t e = launch_index_score(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols,
                                    scores, tw.hist1, stream);
  if (e != hipSuccess) return e;
  return launch_topk(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, true, tw, stream);
}

hipError_t launch_fused(ChainArgs a, int batch, int nwg, int capacity, bool cand,
                        hipStream_t stream) {
  const int rows_per_launch = max(1, capacity / nwg);
  for (int r0 = 0; r0 < batch; r0 += rows_per_launch) {
    a.row0 = r0;
    const int rows = min(rows_per_launch, batch - r0);
    if (cand)
      hipLaunchKernelGGL(k_index_topk<true>, dim3(nwg, rows), dim3(kFuseThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(k_index_topk<false>, dim3(nwg, rows), dim3(kFuseThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

ChainArgs base_args(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                    const int64_t* seq_base, const int32_t* n_valid, int batch, int n_cols, int cpw,
                    void* ws_base) {
  const FuseParts f = fuse_carve(ws_base, batch);
  ChainArgs a{};
  a.q_idx = q_idx;
  a.codes = codes;
  a.scale = scale;
  a.seq_base = seq_base;
  a.n_valid = n_valid;
  a.n_cols = n_cols;
  a.cols_per_wg = cpw;
  a.batch = batch;
  a.status = f.status;
  a.sync = f.sync;
  a.sel_base = f.sel_base;
  a.fine_base = f.fine_base;
  a.pool_base = f.pool_base;
  return a;
}

}  // namespace

size_t index_topk_ws_bytes(int batch, int n_cols) {
  int cpw = 0, nwg = 0;
  const size_t fuse = fuse_part_bytes(batch);
  if (fused_fits(batch, n_cols, fused_capacity(), &cpw, &nwg)) return fuse;
  return fuse + two_step_bytes(batch, n_cols);
}

hipError_t launch_index_topk(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                             const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                             int batch, int n_cols, int k, int32_t* idx_out, float* score_out,
                             void* ws_base, hipStream_t stream) {
  const int capacity = fused_capacity();
  int cpw = 0, nwg = 0;
  if (!fused_fits(batch, n_cols, capacity, &cpw, &nwg))
    return two_step(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols, k, idx_out,
                    score_out, static_cast<char*>(ws_base) + fuse_part_bytes(batch), stream);
  ChainArgs a = base_args(q_idx, codes, scale, seq_base, n_valid, batch, n_cols, cpw, ws_base);
  a.cand = cand;
  a.k = k;
  a.idx_out = idx_out;
  a.score_out = score_out;
  return launch_fused(a, batch, nwg, capacity, cand != nullptr, stream);
}

// Two-launch layout: [fuse part][two-step part][pool scores f32 batch x pool_k][pool sizes].
size_t select_chain_ws_bytes(int batch, int n_cols, int pool_k) {
  int cpw = 0, nwg = 0;
  const size_t fuse = fuse_part_bytes(batch);
  if (fused_fits(batch, n_cols, fused_capacity(), &cpw, &nwg)) return fuse;
  return fuse + two_step_bytes(batch, n_cols) + align_up((size_t)batch * pool_k * 4, 256) +
         align_up((size_t)batch * 4, 256);
}

hipError_t launch_select_chain(const uint16_t* q_full, const uint8_t* codes, const float* scale,
                               const int64_t* seq_base, const int32_t* n_valid, int batch,
                               int n_cols, int pool_k, int32_t* pool_out, float* pool_score_out,
                               int k, int32_t* own_out, const uint16_t* q_re, int n_re,
                               int32_t* re_out, float* re_score_out, void* ws_base,
                               hipStream_t stream) {
  const int capacity = fused_capacity();
  int cpw = 0, nwg = 0;
  if (fused_fits(batch, n_cols, capacity, &cpw, &nwg)) {
    ChainArgs a = base_args(q_full, codes, scale, seq_base, n_valid, batch, n_cols, cpw, ws_base);
    a.k = pool_k;
    a.idx_out = pool_out;
    a.score_out = pool_score_out;
    a.own_k = own_out ? k : 0;
    a.own_out = own_out;
    a.n_re = n_re;
    a.re_k = k;
    a.q_re = q_re;
    a.re_out = re_out;
    a.re_score_out = re_score_out;
    return launch_fused(a, batch, nwg, capacity, false, stream);
  }
  // rows too long for one resident grid: the same selections one call at a time (the
  // pool selections use the fused kernel with the still-clean fuse part of the workspace)
  char* p = static_cast<char*>(ws_base) + fuse_part_bytes(batch);
  char* after = p + two_step_bytes(batch, n_cols);
  float* pool_scores =
      pool_score_out ? pool_score_out : reinterpret_cast<float*>(after);
  int32_t* pool_n = reinterpret_cast<int32_t*>(after + align_up((size_t)batch * pool_k * 4, 256));
  hipError_t e = two_step(q_full, codes, scale, seq_base, n_valid, nullptr, batch, n_cols, pool_k,
                          pool_out, pool_scores, p, stream);
  if (e != hipSuccess) return e;
  if (own_out == nullptr && n_re == 0) return hipSuccess;
  hipLaunchKernelGGL(k_count_valid, dim3(batch), dim3(256), 0, stream, pool_out, pool_k, pool_n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (own_out) {
    e = launch_topk(pool_scores, batch, pool_k, pool_n, pool_out, k, own_out, nullptr, false,
                    TopkWs{}, stream);
    if (e != hipSuccess) return e;
  }
  for (int r = 0; r < n_re; ++r) {
    e = launch_index_topk(q_re + (size_t)r * batch * kDIdx, codes, scale, seq_base, pool_n,
                          pool_out, batch, pool_k, k, re_out + (size_t)r * batch * k,
                          re_score_out ? re_score_out + (size_t)r * batch * k : nullptr, ws_base,
                          stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
