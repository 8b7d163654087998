// Host-side launchers shared between the C-ABI front end (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// ---- top-k workspace layout (bytes), per call of `batch` rows of `n_cols` ----
constexpr int kHist1Bins = 4096;   // level-1 digit: key bits 31..20
constexpr int kHist2Bins = 2048;   // level-2 digit: key bits 19..9
constexpr int kTopkSmallMax = 16384;  // rows this long or shorter are selected in LDS

struct TopkWs {
  uint32_t* hist1;         // [batch][4096]
  uint32_t* hist2;         // [batch][2048]
  uint32_t* counters;      // [batch][4]: candidate count, arrivals
  unsigned long long* bitmap;  // [batch][words]
  unsigned long long* listA;   // [batch][n_cols]  (key << 32 | column)
  unsigned long long* listB;   // [batch][n_cols]
  int64_t words;
};

size_t topk_ws_bytes(int batch, int n_cols);
TopkWs topk_ws_carve(void* base, int batch, int n_cols);

hipError_t launch_index_score(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                              const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                              int batch, int n_cols, float* scores, uint32_t* hist1,
                              hipStream_t stream);

hipError_t launch_topk(const float* scores, int batch, int n_cols, const int32_t* n_valid,
                       const int32_t* cand, int k, int32_t* idx_out, float* score_out,
                       bool hist_ready, const TopkWs& ws, hipStream_t stream);

// ---- attention ----
constexpr int kAttnSplit = 32;  // list positions per wave
int attn_splits(int k);          // main splits + window splits
size_t attn_ws_bytes(int rows, int k);

// mode 0: decode (row b uses seq_base[b], swa + b*128 rows, swa_len[b])
// mode 1: prefill (row t at position pos0+t, entries from 0, window rows from swa)
hipError_t launch_attn(int mode, const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       const int64_t* seq_base, const int32_t* idx, int k, const uint8_t* swa,
                       const int32_t* swa_len, int64_t pos0, float softmax_scale, int rows,
                       float* out, void* ws, hipStream_t stream);

// ---- prefill ----
size_t prefill_ws_bytes(int T, int n_entries, int k);
hipError_t launch_prefill(const uint16_t* q_idx, const uint16_t* q, const uint8_t* idx_codes,
                          const float* idx_scale, const uint8_t* kv_codes, const uint8_t* kv_scale,
                          int n_entries, int ratio, int64_t pos0, int T, int k, const uint8_t* swa,
                          float softmax_scale, int32_t* idx_out, float* out, void* ws,
                          hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace csa2
