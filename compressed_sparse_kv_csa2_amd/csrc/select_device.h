// Workgroup-level building blocks of the radix selections (topk.hip, index_topk.hip):
// block scans, histogram threshold search, ballot ranks.
#pragma once
#include "csa2_device.h"

namespace csa2 {

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8 within
// each row of 16 lanes, then row_bcast:15 (rows 1 and 3 add the last lane of the row
// before) and row_bcast:31 (rows 2 and 3 add lane 31).  Lanes outside a shift's row, or
// rows masked off, add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return (uint32_t)x;
}


// Executed by ONE wave: finds the bin holding the need-th largest element of h[0..nbins)
// (nbins a multiple of 64, 1 <= need <= total).  out[0] = bin, out[1] = elements above.
inline __device__ void find_threshold_bin(const uint32_t* h, int nbins, uint32_t need, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {  // defined result even if need exceeded the total (it never should)
    out[0] = 0u;
    out[1] = 0u;
  }
  const int per = nbins / 64;
  const int hi = nbins - lane * per;  // lane 0 owns the top bins
  uint32_t sum = 0;
  for (int i = 1; i <= per; ++i) sum += h[hi - i];
  const uint32_t incl = wave_incl_scan(sum);
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
// stores the block total in *total.  `scratch` holds >= 16 u32 of LDS.  Each wave scans the
// per-wave totals itself (one LDS read per lane, then DPP), so no wave walks the others'
// totals one by one.  Two barriers; ends with one (scratch is free again).
inline __device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  const uint32_t wincl = wave_incl_scan(lane < nwaves ? scratch[lane] : 0u);
  const int src = __builtin_amdgcn_readfirstlane(wave > 0 ? wave - 1 : 0);
  const uint32_t before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)wincl, src) : 0u;
  *total = (uint32_t)__builtin_amdgcn_readlane((int)wincl, 63);
  __syncthreads();
  return before + incl - v;
}

// Block-wide search of a histogram h[0..PER * blockDim.x) in LDS for the bin holding the
// need-th largest element (1 <= need <= total): thread t owns the PER bins just below bin
// PER*(blockDim - t), and one block scan orders them from the top.  out[0] = bin,
// out[1] = elements in higher bins.  Ends with a barrier.
template <int PER>
__device__ void find_bin_block(const uint32_t* h, uint32_t need, uint32_t* s_scan, uint32_t* out) {
  const int top = PER * (int)(blockDim.x - threadIdx.x);
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[top - 1 - i];
    sum += c[i];
  }
  if (threadIdx.x == 0) {  // defined result even if need exceeded the total (it never should)
    out[0] = 0u;
    out[1] = 0u;
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(sum, s_scan, &total);
  if (excl < need && need <= excl + sum) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= need) {
        out[0] = (uint32_t)(top - 1 - i);
        out[1] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ unsigned long long composite(uint32_t key, uint32_t col) {
  return ((unsigned long long)key << 32) | (uint32_t)~col;
}

__device__ __forceinline__ uint32_t lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive scan, in place, of the n <= 64 * PER per-(iteration, wave) counts in s_cnt, by
// wave 0; returns the total to every lane of wave 0.
template <int PER>
__device__ uint32_t scan_counts_wave0_n(uint32_t* s_cnt, int n) {
  const int lane = threadIdx.x & 63;
  uint32_t c[PER];
  uint32_t part = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = PER * lane + i < n ? s_cnt[PER * lane + i] : 0u;
    part += c[i];
  }
  const uint32_t incl = wave_incl_scan(part);
  uint32_t run = incl - part;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (PER * lane + i < n) s_cnt[PER * lane + i] = run;
    run += c[i];
  }
  return __shfl(incl, 63);
}

inline __device__ uint32_t scan_counts_wave0(uint32_t* s_cnt, int n) {
  return scan_counts_wave0_n<2>(s_cnt, n);
}

}  // namespace csa2
