// a1 + a2 (and a3 + a2): score the indexer keys and select the top-k in one launch,
// without writing the scores to memory.
//
// Same result as k_index_score followed by the top-k of topk.hip: the k largest scores of
// a row, ties to the lower column, written in ascending column order as entry ids
// (cand[c] or c), -1 padded ("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash",
// commentary on the four layer modes; "从V4到V4.1 Flash：架构的激进进化", decoder section on
// the pool of about 16K positions that later layers search).
//
// Every 1,024-thread workgroup scores up to 16,384 columns of one row with the stream of
// scan_device.h (16 waves: as many loads in flight per CU as the stand-alone scan) and
// keeps their order-preserving u32 keys in LDS (key 0 = not selectable).  The row's
// workgroups (64 for a 2^20-column row) then find the exact k-th composite
// (key << 32 | ~column, unique per column) digit by digit, meeting at row barriers:
//   1. level 1, key bits 31..20: each workgroup's LDS histogram is added to the row's;
//   2. level 2, bits 19..9, over the keys in the level-1 bin b1;
//   3. each workgroup publishes how many of its keys lie above the level-2 bin (b1, b2)
//      and the composites of its keys inside it (a handful per row).  Every workgroup then
//      ranks those few composites itself: that fixes the k-th composite T, which of the
//      row's tied keys are taken, and every workgroup's output offset.
// Only when some workgroup holds more than 4 keys of the level-2 bin (massive ties) do
// the workgroups take two more barriers: a level-3 histogram (bits 8..0) fixes the
// threshold key, then (#keys above it, #keys equal to it) of every workgroup fix each
// workgroup's share of the equal keys (the lowest columns win) and its offset.
// Each workgroup then compacts its selected columns in column order with wave ballots.
// The histograms are returned to zero by workgroup 0 of the row once every workgroup has
// read them, and the last workgroup to leave resets the row's barrier counters, so the
// workspace is ready for the next call without a separate clearing launch.
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
#include "csa2_internal.h"
#include "scan_device.h"
#include "select_device.h"

namespace csa2 {

constexpr int kFuseThreads = 1024;                        // 16 waves
constexpr int kFuseWaves = kFuseThreads / 64;
constexpr int kFuseKeysPerThread = 16;
constexpr int kFuseMaxCols = kFuseThreads * kFuseKeysPerThread;  // 16,384 keys in LDS
constexpr uint32_t kSpinLimit = 1u << 20;

static_assert(kFuseThreads * 4 == kHist1Bins, "level-1 bins: 4 per thread");
static_assert(kFuseThreads * 2 == kHist2Bins, "level-2 bins: 2 per thread");
static_assert(kHist3Bins == 8 * 64, "level-3 bins: 8 per lane of one wave");
static_assert(kFuseMaxWg <= kFuseThreads, "offsets: one workgroup per thread");

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of the workgroups of one row: returns once the row's arrival counter has reached
// `target` (= barriers passed so far x workgroups per row).  `pending` combines the values
// returned by this thread's atomics since the previous barrier: using it makes the thread
// wait until they have been performed before its workgroup arrives.
__device__ void row_sync(uint32_t* arrivals, uint32_t target, uint32_t* status,
                         uint32_t pending) {
  asm volatile("" ::"v"(pending));
  __syncthreads();
  if (threadIdx.x == 0) {
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

// Adds the non-empty bins of an LDS histogram of N * 1,024 bins (N = 1: 512 bins) to a
// global one; returns the combined values the atomics returned (for row_sync).  The
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

// Searches an LDS histogram h[0..PER * 1024) for the bin holding the k-th largest element,
// from the top.  Returns the total count; when 1 <= k <= total, out[0] = the bin and out[1] = the
// elements in higher bins.  Whole workgroup; ends with a barrier.
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

template <bool CAND>
__global__ __launch_bounds__(kFuseThreads) void k_index_topk(
    const uint16_t* __restrict__ q_idx, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, const int64_t* __restrict__ seq_base,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ cand, int n_cols,
    int cols_per_wg, int row0, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, FuseWs ws) {
  __shared__ uint32_t s_h[kHist1Bins];
  __shared__ uint32_t s_key[kFuseMaxCols];
  __shared__ uint32_t s_cnt[kFuseKeysPerThread * kFuseWaves];
  __shared__ unsigned long long s_tied[kFuseMaxWg * kTiedPerWg];
  __shared__ uint32_t s_selt[kFuseMaxWg];
  __shared__ uint32_t s_scan[32];
  __shared__ uint32_t s_res[4];
  __shared__ uint32_t s_misc[4];
  __shared__ unsigned long long s_T;
  const int b = row0 + (int)blockIdx.y, wg = blockIdx.x, nwg = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = min(n_valid[b], n_cols);
  const int c0 = wg * cols_per_wg, c1 = min(c0 + cols_per_wg, n_cols);
  const int iters = cols_per_wg / kFuseThreads;  // key i = j * 1024 + tid, j < iters
  const int32_t* cand_row = CAND ? cand + (size_t)b * n_cols : nullptr;
  uint32_t* arrivals = ws.sync + (size_t)b * kSyncStride;
  uint32_t* g1 = ws.hist1 + (size_t)b * kHist1Bins;
  uint32_t* g2 = ws.hist2 + (size_t)b * kHist2Bins;
  uint32_t* g3 = ws.hist3 + (size_t)b * kHist3Bins;
  uint32_t* cnt = ws.wgcnt + (size_t)b * kFuseMaxWg;
  unsigned long long* tied = ws.tied + (size_t)b * kFuseMaxWg * kTiedPerWg;
  const uint32_t nw = (uint32_t)nwg;
  uint32_t pending = 0;

  // ---- score the columns [c0, c1): keys into LDS, level-1 histogram into the row's
  for (int i = tid; i < kFuseMaxCols; i += kFuseThreads) s_key[i] = 0u;
  if (nv > 0) {
    scan_columns<CAND, kFuseThreads>(
        q_idx + (size_t)b * kDIdx, codes, scale, cand_row, seq_base[b], nv, c0, c1,
        [&]() {
          for (int i = tid; i < kHist1Bins; i += kFuseThreads) s_h[i] = 0u;
        },
        [&](int col, float score, bool valid) {
          const uint32_t key = valid ? score_key(score) : 0u;
          s_key[col - c0] = key;
          if (key != 0u) atomicAdd(&s_h[key >> 20], 1u);
        });
    __syncthreads();
    pending |= flush_hist<4>(s_h, kHist1Bins, g1);
  }
  row_sync(arrivals, nw, ws.status, pending);
  pending = 0;

  // ---- level 1: the bin b1 of the k-th key (or every selectable column)
#pragma unroll
  for (int i = 0; i < 4; ++i) s_h[tid + i * kFuseThreads] = ld_agent(&g1[tid + i * kFuseThreads]);
  __syncthreads();
  const uint32_t total = hist_select<4>(s_h, (uint32_t)k, s_scan, s_res);
  const uint32_t k_eff = min((uint32_t)k, total);
  const bool all = k_eff == total;  // the same in every workgroup of the row
  uint32_t b1 = 0, need = 0;        // need: keys still to take at or below the prefix
  if (!all) {
    b1 = s_res[0];
    need = k_eff - s_res[1];
    __syncthreads();
    for (int i = tid; i < kHist2Bins; i += kFuseThreads) s_h[i] = 0u;
    __syncthreads();
    for (int j = 0; j < iters; ++j) {
      const uint32_t key = s_key[j * kFuseThreads + tid];
      if (key != 0u && (key >> 20) == b1) atomicAdd(&s_h[(key >> 9) & (kHist2Bins - 1)], 1u);
    }
    __syncthreads();
    pending |= flush_hist<2>(s_h, kHist2Bins, g2);
  }
  row_sync(arrivals, 2u * nw, ws.status, pending);
  pending = 0;

  // ---- level 2: the bin (b1, b2); publish the keys above it and the composites inside it
  if (wg == 0)
    for (int i = tid; i < kHist1Bins; i += kFuseThreads) st_agent(&g1[i], 0u);
  uint32_t pre = 0;  // key >> 9 of the level-2 bin
  if (!all) {
    s_h[tid] = ld_agent(&g2[tid]);
    s_h[tid + kFuseThreads] = ld_agent(&g2[tid + kFuseThreads]);
    __syncthreads();
    hist_select<2>(s_h, need, s_scan, s_res);
    pre = (b1 << 11) | s_res[0];
    need -= s_res[1];
  }
  {
    if (tid == 0) s_misc[0] = 0u;
    __syncthreads();
    uint32_t n_above = 0;
    for (int j = 0; j < iters; ++j) {
      const uint32_t key = s_key[j * kFuseThreads + tid];
      if (key == 0u) continue;
      if (all || (key >> 9) > pre) {
        ++n_above;
      } else if ((key >> 9) == pre) {  // staged in LDS, published below
        const uint32_t slot = atomicAdd(&s_misc[0], 1u);
        if (slot < (uint32_t)kTiedPerWg)
          s_tied[slot] = composite(key, (uint32_t)(c0 + j * kFuseThreads + tid));
      }
    }
    uint32_t above_total;
    block_exclusive_scan(n_above, s_scan, &above_total);  // barrier: s_misc[0], s_tied ready
    // one round trip: the tied composites and the counts leave together
    const uint32_t n_tied = s_misc[0];
    if (tid < (int)min(n_tied, (uint32_t)kTiedPerWg))
      pending |= (uint32_t)__hip_atomic_exchange(&tied[wg * kTiedPerWg + tid], s_tied[tid],
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == kTiedPerWg)
      pending |= __hip_atomic_exchange(&cnt[wg], (above_total << 16) | min(n_tied, 0xffffu),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  row_sync(arrivals, 3u * nw, ws.status, pending);
  pending = 0;

  // ---- the k-th composite T from the published tied keys; this workgroup's offset
  if (wg == 0)
    for (int i = tid; i < kHist2Bins; i += kFuseThreads) st_agent(&g2[i], 0u);
  const uint32_t cv = tid < nwg ? ld_agent(&cnt[tid]) : 0u;
  const unsigned long long tv =
      tid < nwg * kTiedPerWg
          ? __hip_atomic_load(&tied[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
          : 0ull;
  const uint32_t n_tied_v = cv & 0xffffu;  // of workgroup v = tid
  if (tid < nwg) s_selt[tid] = n_tied_v;
  // massive ties: some workgroup could not publish all of its tied keys
  const bool slow = __syncthreads_or(n_tied_v > (uint32_t)kTiedPerWg) != 0;
  // selected: key > tkey, or key == tkey and column <= col_cut (-1: no equal key)
  uint32_t tkey = 0u;
  int col_cut = -1;
  uint32_t offset;
  if (!slow) {
    const int v = tid / kTiedPerWg;
    const bool valid = v < nwg && (uint32_t)(tid % kTiedPerWg) < s_selt[v];
    uint32_t nt;
    const uint32_t pos = block_exclusive_scan(valid ? 1u : 0u, s_scan, &nt);  // barrier
    if (valid) s_tied[pos] = tv;
    if (tid < nwg) s_selt[tid] = 0u;
    if (tid == 0) s_T = ~0ull;
    __syncthreads();
    if (!all && valid) {
      uint32_t r = 0;  // composites are unique: exactly one has rank need - 1
      for (uint32_t i = 0; i < nt; ++i) r += s_tied[i] > tv ? 1u : 0u;
      if (r == need - 1u) s_T = tv;
    }
    __syncthreads();
    if (!all) {
      const unsigned long long T = s_T;
      tkey = (uint32_t)(T >> 32);
      col_cut = (int)~(uint32_t)T;
      if (valid && tv >= T) atomicAdd(&s_selt[v], 1u);
    }
    __syncthreads();
    const uint32_t sel_v = tid < nwg ? (cv >> 16) + s_selt[tid] : 0u;
    block_exclusive_scan(tid < wg ? sel_v : 0u, s_scan, &offset);
  } else {
    // level 3 over the keys of the level-2 bin: the threshold key
    for (int i = tid; i < kHist3Bins; i += kFuseThreads) s_h[i] = 0u;
    __syncthreads();
    for (int j = 0; j < iters; ++j) {
      const uint32_t key = s_key[j * kFuseThreads + tid];
      if (key != 0u && (key >> 9) == pre) atomicAdd(&s_h[key & (kHist3Bins - 1)], 1u);
    }
    __syncthreads();
    pending |= flush_hist<1>(s_h, kHist3Bins, g3);
    row_sync(arrivals, 4u * nw, ws.status, pending);
    pending = 0;
    if (tid < kHist3Bins) s_h[tid] = ld_agent(&g3[tid]);
    __syncthreads();
    if (wave == 0) find_threshold_bin(s_h, kHist3Bins, need, s_res);
    __syncthreads();
    tkey = (pre << 9) | s_res[0];
    const uint32_t need_eq = need - s_res[1];  // keys equal to tkey still to take, >= 1
    uint32_t n_gt = 0, n_eq = 0;
    for (int j = 0; j < iters; ++j) {
      const uint32_t key = s_key[j * kFuseThreads + tid];
      n_gt += key > tkey ? 1u : 0u;
      n_eq += key == tkey ? 1u : 0u;
    }
    uint32_t packed;  // both counts are <= 16,384
    block_exclusive_scan((n_gt << 16) | n_eq, s_scan, &packed);
    if (tid == 0)
      pending |= __hip_atomic_exchange(&cnt[wg], packed, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    row_sync(arrivals, 5u * nw, ws.status, pending);
    pending = 0;
    if (wg == 0 && tid < kHist3Bins) st_agent(&g3[tid], 0u);
    // the equal keys go to the lowest columns: workgroup by workgroup, then by column
    const uint32_t cw = tid < nwg ? ld_agent(&cnt[tid]) : 0u;
    const uint32_t eq_v = cw & 0xffffu;
    uint32_t unused;
    const uint32_t eq_before = block_exclusive_scan(eq_v, s_scan, &unused);
    const uint32_t take_v = min(eq_v, need_eq > eq_before ? need_eq - eq_before : 0u);
    if (tid == wg) s_misc[2] = take_v;
    if (tid == 0) s_misc[3] = 0xffffffffu;
    block_exclusive_scan(tid < wg ? (cw >> 16) + take_v : 0u, s_scan, &offset);  // barrier
    const uint32_t take = s_misc[2];
    if (take > 0u) {  // column of this workgroup's take-th equal key, in column order
      for (int j = 0; j < iters; ++j) {
        const unsigned long long m = __ballot(s_key[j * kFuseThreads + tid] == tkey);
        if (lane == 0) s_cnt[j * kFuseWaves + wave] = (uint32_t)__popcll(m);
      }
      __syncthreads();
      if (wave == 0) scan_counts_wave0_n<4>(s_cnt, iters * kFuseWaves);
      __syncthreads();
      for (int j = 0; j < iters; ++j) {
        const bool eq = s_key[j * kFuseThreads + tid] == tkey;
        const unsigned long long m = __ballot(eq);
        if (eq && s_cnt[j * kFuseWaves + wave] + lanes_below(m) == take - 1u)
          s_misc[3] = (uint32_t)(c0 + j * kFuseThreads + tid);
      }
      __syncthreads();
      col_cut = (int)s_misc[3];
    }
  }

  // ---- compaction in column order of the selected columns
  uint32_t selbits = 0;
  for (int j = 0; j < iters; ++j) {
    const uint32_t key = s_key[j * kFuseThreads + tid];
    const int col = c0 + j * kFuseThreads + tid;
    const bool take = key > tkey || (key == tkey && key != 0u && col <= col_cut);
    selbits |= (take ? 1u : 0u) << j;
    const unsigned long long m = __ballot(take);
    if (lane == 0) s_cnt[j * kFuseWaves + wave] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  if (wave == 0) scan_counts_wave0_n<4>(s_cnt, iters * kFuseWaves);
  __syncthreads();
  int32_t* orow = idx_out + (size_t)b * k;
  float* srow = score_out ? score_out + (size_t)b * k : nullptr;
  for (int j = 0; j < iters; ++j) {
    const bool take = (selbits >> j) & 1u;
    const unsigned long long m = __ballot(take);
    if (take) {
      const uint32_t pos = offset + s_cnt[j * kFuseWaves + wave] + lanes_below(m);
      const int col = c0 + j * kFuseThreads + tid;
      if (pos < (uint32_t)k) {
        orow[pos] = CAND ? cand_row[col] : col;
        if (srow) srow[pos] = key_score(s_key[j * kFuseThreads + tid]);
      }
    }
  }
  for (int p = (int)k_eff + wg * kFuseThreads + tid; p < k; p += nwg * kFuseThreads) {
    orow[p] = -1;
    if (srow) srow[p] = -__builtin_inff();
  }

  // ---- the last workgroup of the row to leave resets the row's barrier counters
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = add_agent(arrivals + 1, 1u);
    if (old == nw - 1u) {
      st_agent(arrivals, 0u);
      st_agent(arrivals + 1, 0u);
    }
  }
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
  g_capacity[dev] = min(per_cu_a, per_cu_b) * n_cu;
  return g_capacity[dev];
}

// Columns per workgroup: a multiple of 1,024 up to 16,384, spreading the whole batch over
// the device's capacity (one workgroup per CU) where it can.
int fused_cols_per_wg(int batch, int n_cols, int capacity) {
  const long long want = ((long long)n_cols * batch + capacity - 1) / capacity;
  long long c = (want + kFuseThreads - 1) / kFuseThreads * kFuseThreads;
  if (c < kFuseThreads) c = kFuseThreads;
  if (c > kFuseMaxCols) c = kFuseMaxCols;
  return (int)c;
}

// The fused launch applies when one row's workgroups fit the device at once.
bool fused_fits(int n_cols, int capacity, int* cpw_out, int* nwg_out, int batch) {
  if (capacity <= 0) return false;
  const int cpw = fused_cols_per_wg(batch, n_cols, capacity);
  const long long nwg = ((long long)n_cols + cpw - 1) / cpw;
  if (nwg > kFuseMaxWg || nwg > capacity) return false;
  *cpw_out = cpw;
  *nwg_out = (int)nwg;
  return true;
}

size_t fuse_part_bytes(int batch) {
  size_t s = 256;  // status
  s += align_up((size_t)batch * kHist1Bins * 4, 256);
  s += align_up((size_t)batch * kHist2Bins * 4, 256);
  s += align_up((size_t)batch * kHist3Bins * 4, 256);
  s += align_up((size_t)batch * kSyncStride * 4, 256);
  s += align_up((size_t)batch * kFuseMaxWg * 4, 256);
  s += align_up((size_t)batch * kFuseMaxWg * kTiedPerWg * 8, 256);
  return s;
}

FuseWs fuse_carve(void* base, int batch) {
  FuseWs w;
  char* p = static_cast<char*>(base);
  w.status = reinterpret_cast<uint32_t*>(p);
  p += 256;
  w.hist1 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist1Bins * 4, 256);
  w.hist2 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist2Bins * 4, 256);
  w.hist3 = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kHist3Bins * 4, 256);
  w.sync = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kSyncStride * 4, 256);
  w.wgcnt = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kFuseMaxWg * 4, 256);
  w.tied = reinterpret_cast<unsigned long long*>(p);
  return w;
}

}  // namespace

// Fused layout: [FuseWs part].  Otherwise (a row too long for one resident grid):
// [FuseWs part][scores f32 batch x n_cols][top-k workspace] for the two-launch path.
size_t index_topk_ws_bytes(int batch, int n_cols) {
  int cpw = 0, nwg = 0;
  const size_t fuse = fuse_part_bytes(batch);
  if (fused_fits(n_cols, fused_capacity(), &cpw, &nwg, batch)) return fuse;
  return fuse + align_up((size_t)batch * n_cols * 4, 256) + topk_ws_bytes(batch, n_cols);
}

hipError_t launch_index_topk(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                             const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                             int batch, int n_cols, int k, int32_t* idx_out, float* score_out,
                             void* ws_base, hipStream_t stream) {
  const int capacity = fused_capacity();
  int cpw = 0, nwg = 0;
  if (!fused_fits(n_cols, capacity, &cpw, &nwg, batch)) {
    char* p = static_cast<char*>(ws_base) + fuse_part_bytes(batch);
    float* scores = reinterpret_cast<float*>(p);
    p += align_up((size_t)batch * n_cols * 4, 256);
    const TopkWs tw = topk_ws_carve(p, batch, n_cols);
    hipError_t e = launch_index_score(q_idx, codes, scale, seq_base, n_valid, cand, batch, n_cols,
                                      scores, tw.hist1, stream);
    if (e != hipSuccess) return e;
    return launch_topk(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, true, tw, stream);
  }
  FuseWs ws = fuse_carve(ws_base, batch);
  const int rows_per_launch = max(1, capacity / nwg);
  for (int r0 = 0; r0 < batch; r0 += rows_per_launch) {
    const int rows = min(rows_per_launch, batch - r0);
    if (cand)
      hipLaunchKernelGGL(k_index_topk<true>, dim3(nwg, rows), dim3(kFuseThreads), 0, stream, q_idx,
                         codes, scale, seq_base, n_valid, cand, n_cols, cpw, r0, k, idx_out,
                         score_out, ws);
    else
      hipLaunchKernelGGL(k_index_topk<false>, dim3(nwg, rows), dim3(kFuseThreads), 0, stream, q_idx,
                         codes, scale, seq_base, n_valid, cand, n_cols, cpw, r0, k, idx_out,
                         score_out, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
