// Host-side launchers shared between the C-ABI front end (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include "csa2.h"
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// ---- top-k workspace layout (bytes), per call of `batch` rows of `n_cols` ----
constexpr int kHist1Bins = 4096;   // level-1 digit: key bits 31..20
constexpr int kHist2Bins = 2048;   // level-2 digit: key bits 19..9
constexpr int kTopkSmallMax = 16384;  // rows this long or shorter are selected in LDS

constexpr int kRowInfo = 8;           // per-row counters of the long-row top-k
constexpr int kInfoCand = 0, kInfoKeff = 1, kInfoTotal = 2, kInfoBin1 = 3, kInfoAbove1 = 4;
constexpr int kMaxChunks = 8192;      // column chunks per row of the long-row path
constexpr int kTopkMaxCols = 1 << 26; // longest row csa2_topk accepts

struct TopkWs {
  uint32_t* hist1;               // [batch][4096] level-1 histogram (fused into the scan)
  uint32_t* counters;            // [batch][kRowInfo], indices kInfo*
  unsigned long long* thr;       // [batch] k-th composite (key << 32 | ~column)
  uint32_t* chunk_cnt;           // [batch][n_chunks] columns above the level-1 bin
  uint32_t* chunk_ccnt;          // [batch][n_chunks] candidates (columns in the bin)
  uint32_t* chunk_off;           // [batch][n_chunks] output offset of each chunk
  unsigned long long* list;      // [batch][n_cols] candidates (key << 32 | column), each
                                 // chunk in its own slots starting at its first column
  unsigned long long* tied;      // [batch][n_cols] tied candidates when too many for LDS
  int n_chunks;
};

// ---- scan + top-k in one launch (fsel.hip) and its dispatch (index_topk.hip) ----
constexpr int kMaxReindex = CSA2_MAX_REINDEX;  // Reindex layers one chained call re-scores

// Rows the single-launch filtered selection handles (longer rows: index_score + topk).
bool fsel_fits(int n_cols, int k);
bool fsel_len_ok(int n_cols);
size_t fsel_ws_bytes(int batch, int n_cols, bool chain);
// Rows of at most 16,384 columns, few of them: scan and top-k in one launch (the row's last
// workgroup selects), in the filtered selection's workspace.
bool fsmall_fits(int batch, int n_cols);
hipError_t launch_fsmall(const uint16_t* q, const uint8_t* codes, const float* scale,
                         const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                         int batch, int n_cols, int k, int32_t* out, float* sout, void* ws,
                         hipStream_t stream);
hipError_t launch_fsel(const uint16_t* q, const uint8_t* codes, const float* scale,
                       const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                       int batch, int n_cols, int k, int32_t* out, float* sout, int own_k,
                       int32_t* own_out, const uint16_t* q_re, int n_re, int re_k,
                       int32_t* re_out, float* re_sout, bool chain_ws, void* ws,
                       hipStream_t stream, const float* smat = nullptr);

size_t index_topk_ws_bytes(int batch, int n_cols);
hipError_t launch_index_topk(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                             const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                             int batch, int n_cols, int k, int32_t* idx_out, float* score_out,
                             void* ws, hipStream_t stream);
size_t select_chain_ws_bytes(int batch, int n_cols, int pool_k);
hipError_t launch_select_chain(const uint16_t* q_full, const uint8_t* codes, const float* scale,
                               const int64_t* seq_base, const int32_t* n_valid, int batch,
                               int n_cols, int pool_k, int32_t* pool_out, float* pool_score_out,
                               int k, int32_t* own_out, const uint16_t* q_re, int n_re,
                               int32_t* re_out, float* re_score_out, void* ws, hipStream_t stream);

size_t replay_select_ws_bytes(int T, int n_entries, int pool_k);
hipError_t launch_replay_select(const uint16_t* q_idx, const uint8_t* codes, const float* scale,
                                int n_entries, int ratio, int64_t pos0, int T, int pool_k,
                                int32_t* pool_out, int32_t* pool_n_out, int k, int32_t* own_out,
                                void* ws, hipStream_t stream);

int topk_chunk_iters(int n_cols);
int topk_n_chunks(int n_cols);
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
int attn_segments(int k);        // 16-position segments of k entries + a full window
int attn_splits(int k);          // decode splits per row
size_t attn_ws_bytes(int rows, int k);

// mode 0: decode (row b uses seq_base[b], swa + b*128 rows, swa_len[b])
// mode 1: prefill (row t at position pos0+t, entries from 0, window rows from swa)
hipError_t launch_attn(int mode, const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       const int64_t* seq_base, const int32_t* idx, int k, const uint8_t* swa,
                       const int32_t* swa_len, int64_t pos0, float softmax_scale, int rows,
                       float* out, void* ws, hipStream_t stream);

// ---- prefill ----
size_t prefill_ws_bytes(int T, int n_entries, int k);
// S[t][j] for the entries j that position pos0 + t sees (blocked: at (j / 1024 * T + t) *
// 1024 + j % 1024, T * round_up(n_entries, 1024) floats; else row-major), each row's visible
// count and, when pool_n is given, min(visible, pool_k)
hipError_t launch_causal_scores(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                                int n_entries, int ratio, int64_t pos0, int T, bool blocked,
                                float* scores, int32_t* n_vis, int pool_k, int32_t* pool_n,
                                hipStream_t stream);
hipError_t launch_prefill_select(const uint16_t* q_idx, const uint8_t* idx_codes,
                                 const float* idx_scale, int n_entries, int ratio, int64_t pos0,
                                 int T, int k, int32_t* idx_out, void* ws, hipStream_t stream);
hipError_t launch_prefill(const uint16_t* q_idx, const uint16_t* q, const uint8_t* idx_codes,
                          const float* idx_scale, const uint8_t* kv_codes, const uint8_t* kv_scale,
                          int n_entries, int ratio, int64_t pos0, int T, int k, const uint8_t* swa,
                          float softmax_scale, int32_t* idx_out, float* out, void* ws,
                          hipStream_t stream);

// ---- KV write path (append.hip) ----
hipError_t launch_kv_append(const uint16_t* x_idx, const uint16_t* x_kv, const int64_t* dst, int n,
                            int64_t capacity, uint8_t* idx_codes, float* idx_scale, uint8_t* kv_codes,
                            uint8_t* kv_scale, int32_t* bad, hipStream_t stream);
hipError_t launch_swa_append(const uint16_t* x, const int64_t* pos, int batch, uint8_t* swa,
                             hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace csa2
