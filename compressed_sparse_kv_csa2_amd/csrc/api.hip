// C-ABI front end: argument validation on the host, workspace carving, launches.
// Declarations and their contracts are in include/csa2.h.
#include "csa2.h"
#include "csa2_internal.h"

#include <stdint.h>

#include <atomic>

using namespace csa2;

// Split partials of csa2_sparse_attn_decode_noalloc: a file-scope device array, so that
// entry point allocates nothing.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes this name to a kernel (on the host it is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress returns for
// the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Device address of `scratch` on the current device, looked up on that device's first call
// and kept per device; null when the lookup fails.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];

void* scratch_addr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch_addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_ALIGNMENT: return "misaligned pointer";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_UNSUPPORTED: return "unsupported shape";
    case CSA2_ERR_HIP: return "HIP runtime error";
    case CSA2_ERR_SCRATCH: return "shape needs more than the library's static scratch holds";
    default: return "unknown status";
  }
}

int csa2_version(void) { return 100; }

int csa2_index_score(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                     const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                     int32_t batch, int32_t n_cols, float* scores, void* topk_ws,
                     size_t topk_ws_size, void* stream) {
  if (!q_idx || !idx_codes || !idx_scale || !seq_base || !n_valid || !scores) return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || n_cols < 1) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(idx_codes, 16) || !aligned(idx_scale, 4) ||
      !aligned(seq_base, 8) || !aligned(n_valid, 4) || !aligned(scores, 4) ||
      (cand && !aligned(cand, 4)))
    return CSA2_ERR_ALIGNMENT;
  uint32_t* hist1 = nullptr;
  if (topk_ws) {
    if (n_cols > kTopkMaxCols) return CSA2_ERR_UNSUPPORTED;
    if (topk_ws_size < topk_ws_bytes(batch, n_cols)) return CSA2_ERR_WORKSPACE;
    if (!aligned(topk_ws, 256)) return CSA2_ERR_ALIGNMENT;
    hist1 = topk_ws_carve(topk_ws, batch, n_cols).hist1;
  }
  return from_hip(launch_index_score(q_idx, idx_codes, idx_scale, seq_base, n_valid, cand, batch,
                                     n_cols, scores, hist1, static_cast<hipStream_t>(stream)));
}

size_t csa2_topk_workspace_size(int32_t batch, int32_t n_cols, int32_t k) {
  (void)k;
  if (batch < 1 || n_cols < 1 || n_cols > kTopkMaxCols) return 0;
  return topk_ws_bytes(batch, n_cols);
}

int csa2_topk(const float* scores, int32_t batch, int32_t n_cols, const int32_t* n_valid,
              const int32_t* cand, int32_t k, int32_t* idx_out, float* score_out, uint32_t flags,
              void* workspace, size_t ws_bytes, void* stream) {
  if (!scores || !n_valid || !idx_out) return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || n_cols < 1 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_INVALID_ARG;
  if (flags & ~CSA2_TOPK_HIST_FUSED) return CSA2_ERR_INVALID_ARG;
  if (n_cols > kTopkMaxCols) return CSA2_ERR_UNSUPPORTED;
  if (!aligned(scores, 4) || !aligned(n_valid, 4) || !aligned(idx_out, 4) ||
      (score_out && !aligned(score_out, 4)) || (cand && !aligned(cand, 4)))
    return CSA2_ERR_ALIGNMENT;
  const bool fused = (flags & CSA2_TOPK_HIST_FUSED) != 0;
  const bool needs_ws = fused || n_cols > kTopkSmallMax;
  TopkWs ws{};
  if (needs_ws) {
    if (!workspace || ws_bytes < topk_ws_bytes(batch, n_cols)) return CSA2_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
    ws = topk_ws_carve(workspace, batch, n_cols);
  }
  return from_hip(launch_topk(scores, batch, n_cols, n_valid, cand, k, idx_out, score_out, fused, ws,
                              static_cast<hipStream_t>(stream)));
}

size_t csa2_index_topk_workspace_size(int32_t batch, int32_t n_cols, int32_t k) {
  (void)k;
  if (batch < 1 || n_cols < 1 || n_cols > kTopkMaxCols) return 0;
  return index_topk_ws_bytes(batch, n_cols);
}

int csa2_index_topk(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                    const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                    int32_t batch, int32_t n_cols, int32_t k, int32_t* idx_out, float* score_out,
                    void* workspace, size_t ws_bytes, void* stream) {
  if (!q_idx || !idx_codes || !idx_scale || !seq_base || !n_valid || !idx_out)
    return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || n_cols < 1 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_INVALID_ARG;
  if (n_cols > kTopkMaxCols) return CSA2_ERR_UNSUPPORTED;
  if (!aligned(q_idx, 16) || !aligned(idx_codes, 16) || !aligned(idx_scale, 4) ||
      !aligned(seq_base, 8) || !aligned(n_valid, 4) || !aligned(idx_out, 4) ||
      (score_out && !aligned(score_out, 4)) || (cand && !aligned(cand, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < index_topk_ws_bytes(batch, n_cols)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_index_topk(q_idx, idx_codes, idx_scale, seq_base, n_valid, cand, batch,
                                    n_cols, k, idx_out, score_out, workspace,
                                    static_cast<hipStream_t>(stream)));
}

size_t csa2_select_chain_workspace_size(int32_t batch, int32_t n_cols, int32_t pool_k) {
  if (batch < 1 || n_cols < 1 || n_cols > kTopkMaxCols || pool_k < 1 || pool_k > CSA2_MAX_K)
    return 0;
  return select_chain_ws_bytes(batch, n_cols, pool_k);
}

int csa2_select_chain(const uint16_t* q_full, const uint8_t* idx_codes, const float* idx_scale,
                      const int64_t* seq_base, const int32_t* n_valid, int32_t batch,
                      int32_t n_cols, int32_t pool_k, int32_t* pool_out, float* pool_score_out,
                      int32_t k, int32_t* own_out, const uint16_t* q_re, int32_t n_re,
                      int32_t* re_out, float* re_score_out, void* workspace, size_t ws_bytes,
                      void* stream) {
  if (!q_full || !idx_codes || !idx_scale || !seq_base || !n_valid || !pool_out)
    return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || n_cols < 1 || pool_k < 1 || pool_k > CSA2_MAX_K || k < 1 || k > CSA2_MAX_K)
    return CSA2_ERR_INVALID_ARG;
  if (n_re < 0 || n_re > CSA2_MAX_REINDEX || (n_re > 0 && (!q_re || !re_out)))
    return CSA2_ERR_INVALID_ARG;
  if (n_cols > kTopkMaxCols) return CSA2_ERR_UNSUPPORTED;
  if (!aligned(q_full, 16) || !aligned(idx_codes, 16) || !aligned(idx_scale, 4) ||
      !aligned(seq_base, 8) || !aligned(n_valid, 4) || !aligned(pool_out, 4) ||
      (pool_score_out && !aligned(pool_score_out, 4)) || (own_out && !aligned(own_out, 4)) ||
      (q_re && !aligned(q_re, 16)) || (re_out && !aligned(re_out, 4)) ||
      (re_score_out && !aligned(re_score_out, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < select_chain_ws_bytes(batch, n_cols, pool_k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_select_chain(q_full, idx_codes, idx_scale, seq_base, n_valid, batch,
                                      n_cols, pool_k, pool_out, pool_score_out, k, own_out, q_re,
                                      n_re > 0 ? n_re : 0, re_out, re_score_out, workspace,
                                      static_cast<hipStream_t>(stream)));
}

size_t csa2_replay_select_workspace_size(int32_t T, int32_t n_entries, int32_t pool_k) {
  if (T < 1 || n_entries < 0 || n_entries > kTopkMaxCols || pool_k < 1 || pool_k > CSA2_MAX_K) return 0;
  return replay_select_ws_bytes(T, n_entries, pool_k);
}

int csa2_replay_select(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                       int32_t n_entries, int32_t ratio, int64_t pos0, int32_t T, int32_t pool_k,
                       int32_t* pool_out, int32_t* pool_n_out, int32_t k, int32_t* own_out,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (!q_idx || !pool_out) return CSA2_ERR_INVALID_ARG;
  if (n_entries > 0 && (!idx_codes || !idx_scale)) return CSA2_ERR_INVALID_ARG;
  if (T < 1 || n_entries < 0 || ratio < 1 || pos0 < 0 || pool_k < 1 || pool_k > CSA2_MAX_K)
    return CSA2_ERR_INVALID_ARG;
  if (own_out && (k < 1 || k > CSA2_MAX_K)) return CSA2_ERR_INVALID_ARG;
  if (n_entries > kTopkMaxCols) return CSA2_ERR_UNSUPPORTED;
  if (!aligned(q_idx, 16) || (idx_codes && !aligned(idx_codes, 16)) ||
      (idx_scale && !aligned(idx_scale, 4)) || !aligned(pool_out, 4) ||
      (pool_n_out && !aligned(pool_n_out, 4)) || (own_out && !aligned(own_out, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < replay_select_ws_bytes(T, n_entries, pool_k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_replay_select(q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, T, pool_k,
                                       pool_out, pool_n_out, own_out ? k : 0, own_out, workspace,
                                       static_cast<hipStream_t>(stream)));
}

int csa2_workspace_status(const void* workspace, uint32_t* out, void* stream) {
  if (!workspace || !out) return CSA2_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  uint32_t w[3] = {0, 0, 0};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(w, workspace, sizeof(w), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  out[0] = w[0];
  out[1] = w[2];
  return CSA2_OK;
}

size_t csa2_attn_workspace_size(int32_t batch, int32_t k) {
  if (batch < 1 || k < 0) return 0;
  return attn_ws_bytes(batch, k);
}

int csa2_sparse_attn_decode(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                            const int64_t* seq_base, const int32_t* idx, int32_t k, const uint8_t* swa,
                            const int32_t* swa_len, float softmax_scale, int32_t batch, float* out,
                            void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !kv_codes || !kv_scale || !seq_base || !swa || !swa_len || !out) return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || k < 0 || k > CSA2_MAX_K || (k > 0 && !idx)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_codes, 16) || !aligned(kv_scale, 4) || !aligned(swa, 16) ||
      !aligned(seq_base, 8) || !aligned(swa_len, 4) || !aligned(out, 16) ||
      (idx && !aligned(idx, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < attn_ws_bytes(batch, k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_attn(0, q, kv_codes, kv_scale, seq_base, idx, k, swa, swa_len, 0,
                              softmax_scale, batch, out, workspace, static_cast<hipStream_t>(stream)));
}

size_t csa2_attn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int csa2_sparse_attn_decode_noalloc(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                                    const int64_t* seq_base, const int32_t* idx, int32_t k,
                                    const uint8_t* swa, const int32_t* swa_len, float softmax_scale,
                                    int32_t batch, float* out, void* stream) {
  if (!q || !kv_codes || !kv_scale || !seq_base || !swa || !swa_len || !out) return CSA2_ERR_INVALID_ARG;
  if (batch < 1 || k < 0 || k > CSA2_MAX_K || (k > 0 && !idx)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_codes, 16) || !aligned(kv_scale, 4) || !aligned(swa, 16) ||
      !aligned(seq_base, 8) || !aligned(swa_len, 4) || !aligned(out, 16) ||
      (idx && !aligned(idx, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (attn_ws_bytes(batch, k) > kNoAllocScratchBytes) return CSA2_ERR_SCRATCH;
  void* ws = scratch_addr();
  if (ws == nullptr) return CSA2_ERR_HIP;
  return from_hip(launch_attn(0, q, kv_codes, kv_scale, seq_base, idx, k, swa, swa_len, 0,
                              softmax_scale, batch, out, ws, static_cast<hipStream_t>(stream)));
}

size_t csa2_prefill_workspace_size(int32_t T, int32_t n_entries, int32_t k) {
  if (T < 1 || n_entries < 0 || k < 1) return 0;
  return prefill_ws_bytes(T, n_entries, k);
}

int csa2_prefill_chunk(const uint16_t* q_idx, const uint16_t* q, const uint8_t* idx_codes,
                       const float* idx_scale, const uint8_t* kv_codes, const uint8_t* kv_scale,
                       int32_t n_entries, int32_t ratio, int64_t pos0, int32_t T, int32_t k,
                       const uint8_t* swa, float softmax_scale, int32_t* idx_out, float* out,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (!q_idx || !q || !swa || !idx_out || !out) return CSA2_ERR_INVALID_ARG;
  if (n_entries > 0 && (!idx_codes || !idx_scale || !kv_codes || !kv_scale)) return CSA2_ERR_INVALID_ARG;
  if (T < 1 || n_entries < 0 || ratio < 1 || pos0 < 0 || k < 1 || k > CSA2_MAX_K)
    return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(q, 16) || !aligned(swa, 16) || !aligned(idx_out, 4) ||
      !aligned(out, 16) || (idx_codes && !aligned(idx_codes, 16)) ||
      (idx_scale && !aligned(idx_scale, 4)) || (kv_codes && !aligned(kv_codes, 16)) ||
      (kv_scale && !aligned(kv_scale, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < prefill_ws_bytes(T, n_entries, k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_prefill(q_idx, q, idx_codes, idx_scale, kv_codes, kv_scale, n_entries, ratio,
                                 pos0, T, k, swa, softmax_scale, idx_out, out, workspace,
                                 static_cast<hipStream_t>(stream)));
}

int csa2_prefill_select(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                        int32_t n_entries, int32_t ratio, int64_t pos0, int32_t T, int32_t k,
                        int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!q_idx || !idx_out) return CSA2_ERR_INVALID_ARG;
  if (n_entries > 0 && (!idx_codes || !idx_scale)) return CSA2_ERR_INVALID_ARG;
  if (T < 1 || n_entries < 0 || ratio < 1 || pos0 < 0 || k < 1 || k > CSA2_MAX_K)
    return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(idx_out, 4) || (idx_codes && !aligned(idx_codes, 16)) ||
      (idx_scale && !aligned(idx_scale, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < prefill_ws_bytes(T, n_entries, k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_prefill_select(q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, T, k,
                                        idx_out, workspace, static_cast<hipStream_t>(stream)));
}

int csa2_sparse_attn_prefill(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                             const int32_t* idx, int32_t k, const uint8_t* swa, int64_t pos0,
                             int32_t T, float softmax_scale, float* out, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (!q || !swa || !out || !kv_codes || !kv_scale) return CSA2_ERR_INVALID_ARG;
  if (T < 1 || k < 0 || k > CSA2_MAX_K || pos0 < 0 || (k > 0 && !idx)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(swa, 16) || !aligned(out, 16) || !aligned(kv_codes, 16) ||
      !aligned(kv_scale, 4) || (idx && !aligned(idx, 4)))
    return CSA2_ERR_ALIGNMENT;
  if (!workspace || ws_bytes < attn_ws_bytes(T, k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_attn(1, q, kv_codes, kv_scale, nullptr, k > 0 ? idx : nullptr, k, swa,
                              nullptr, pos0, softmax_scale, T, out, workspace,
                              static_cast<hipStream_t>(stream)));
}

int csa2_kv_append(const uint16_t* x_idx, const uint16_t* x_kv, const int64_t* dst, int32_t n,
                   uint8_t* idx_codes, float* idx_scale, uint8_t* kv_codes, uint8_t* kv_scale,
                   int64_t capacity, int32_t* bad, void* stream) {
  if (n < 0 || capacity < 1) return CSA2_ERR_INVALID_ARG;
  if (n == 0) return CSA2_OK;
  if (!x_idx || !x_kv || !dst || !idx_codes || !idx_scale || !kv_codes || !kv_scale)
    return CSA2_ERR_INVALID_ARG;
  if (!aligned(x_idx, 16) || !aligned(x_kv, 16) || !aligned(dst, 8) || !aligned(idx_codes, 16) ||
      !aligned(idx_scale, 4) || !aligned(kv_codes, 16) || (bad && !aligned(bad, 4)))
    return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_kv_append(x_idx, x_kv, dst, n, capacity, idx_codes, idx_scale, kv_codes,
                                   kv_scale, bad, static_cast<hipStream_t>(stream)));
}

int csa2_swa_append(const uint16_t* x, const int64_t* pos, int32_t batch, uint8_t* swa,
                    void* stream) {
  if (batch < 0) return CSA2_ERR_INVALID_ARG;
  if (batch == 0) return CSA2_OK;
  if (!x || !pos || !swa) return CSA2_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(pos, 8) || !aligned(swa, 16)) return CSA2_ERR_ALIGNMENT;
  return from_hip(launch_swa_append(x, pos, batch, swa, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
