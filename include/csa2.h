/*
 * csa2.h -- C ABI of the CSA2 compressed-sparse-attention hot path for MI355X (gfx950).
 *
 * The library computes one CSA2 attention step over an FP4 global KV cache:
 *   1. index score  -- every visible 68-byte indexer key (128 x E2M1 + fp32 scale) is
 *                      scored against a 128-d bf16 indexer query (Full mode), or only the
 *                      entries of a candidate pool are (Reindex mode);
 *   2. top-k        -- the k best entries, ties to the lower entry index, listed ascending;
 *   3. attention    -- the selected 288-byte main entries (512 x E2M1 + 32 E4M3 scales) are
 *                      gathered, dequantised and attended by 16 query heads, merged in one
 *                      softmax with the layer's own 128-row E4M3 sliding window;
 *   4. prefill      -- a chunk of queries, each scoring its causally visible keys (a BF16
 *                      MFMA contraction), taking its own top-k and attending;
 *   5. write path   -- new entries quantised into the two formats, new window rows into
 *                      their E4M3 rings (csa2_kv_append, csa2_swa_append).
 * Compositions (a decoder's layer chain in one call, a prefill or replay chunk's attention
 * over lists made elsewhere) are entry points of their own below.
 *
 * Pages this interface follows (cited by title and section):
 *   [STRUCT] "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash" (xhh.club):
 *            Q&A on how the 890-byte global KV figure is derived (entry sizes 288 B and
 *            68 B); commentary on the four layer modes (Full / Reindex / Reuse, top-512).
 *   [DEEP]   "DeepSeek V4.1 Flash 深度解析" (daiw.net): part-1 entry on CSA2 (cross-layer
 *            sharing, hierarchical candidate pool in the decoder); part-4 entry on FP4 in
 *            the KV cache (main KV 4-bit in its own format, sliding window FP8).
 *   [V4TO41] "从V4到V4.1 Flash：架构的激进进化" (prism.simon-ai.net): section on the CSA2
 *            architecture (three modes); section on global KV sharing with per-layer sliding
 *            windows; decoder section (a first full scan builds a pool of about 16K
 *            positions, later layers search their top-512 inside it).
 * Where the pages are silent the readings are: score = fp32 scale x (query . E2M1 codes);
 * ties to the lowest entry index; every entry and window row is both key and value; one
 * softmax over their union with the caller's scale (1/sqrt(512)); causal visibility of an
 * entry once its last token is at or before the query position.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless stated; the caller owns every buffer.  The
 *    library allocates nothing and is re-entrant, except that calls sharing one workspace
 *    must not overlap in time.  Its only global state is the static scratch array of
 *    csa2_sparse_attn_decode_noalloc and that array's per-device address.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *    asynchronous; kernel faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host BEFORE anything is enqueued; on error nothing is
 *    launched and a negative status is returned (csa2_status_string names it).
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).  Code planes must be
 *    16-byte aligned; fp32/int planes 4-byte aligned (int64 8-byte).
 *  - Workspaces: size them with the *_workspace_size query, zero-fill them ONCE before
 *    first use (e.g. hipMemset or torch.zeros); every call returns the counters it uses to
 *    zero before it completes, so a workspace can be reused call after call without
 *    clearing -- by calls of the shape it was last zero-filled for (the same batch and
 *    sizes given to the size query): the layout of its counters depends on that shape,
 *    so a call of another shape needs the workspace zero-filled again first.  Reusing a
 *    workspace across calls on different streams needs the caller's ordering.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_D_IDX 128      /* indexer key / query width */
#define CSA2_D_KV 512       /* main KV width */
#define CSA2_HEADS 16       /* query heads; one shared KV head */
#define CSA2_SWA 128        /* sliding-window rows per layer and sequence */
#define CSA2_MAX_K 16384    /* largest k accepted by csa2_topk / csa2_prefill_chunk */
#define CSA2_MAX_REINDEX 4  /* Reindex layers one csa2_select_chain call serves */

enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = -1, /* null pointer, negative or out-of-range size */
  CSA2_ERR_ALIGNMENT = -2,   /* a plane is not aligned as stated above */
  CSA2_ERR_WORKSPACE = -3,   /* workspace pointer missing or smaller than the query says */
  CSA2_ERR_UNSUPPORTED = -4, /* a shape the kernels do not handle */
  CSA2_ERR_HIP = -5,         /* a HIP launch or runtime call failed */
  CSA2_ERR_SCRATCH = -6      /* the shape needs more than the static scratch holds */
};

/* flags for csa2_topk */
#define CSA2_TOPK_HIST_FUSED 1u /* csa2_index_score already accumulated the level-1
                                   radix histogram of `scores` into this workspace */

/* Static description of a status code. */
const char* csa2_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int csa2_version(void);

/*
 * csa2_index_score -- a1 Full scan / a3 Reindex re-score.
 *   [V4TO41] CSA2 architecture section (Full runs the sparse indexer over its keys;
 *   Reindex picks again with its own indexer query); [STRUCT] Q&A on the 890-byte count
 *   (68-byte indexer entry = 128 x 4 bit + 4-byte scale).
 *
 *   q_idx      bf16 [batch][128]              indexer query of each sequence
 *   idx_codes  u8   [n_total][64]             E2M1 codes, element 2i in the low nibble
 *   idx_scale  f32  [n_total]                 per-entry scale
 *   seq_base   i64  [batch]                   entry number of column 0 of sequence b
 *   n_valid    i32  [batch]                   visible columns of sequence b (<= n_cols)
 *   cand       i32  [batch][n_cols] or NULL   Reindex: column c scores entry
 *                                             seq_base[b] + cand[b][c]; cand < 0 is a hole.
 *                                             NULL (Full): column c scores seq_base[b] + c.
 *   scores     f32  [batch][n_cols]  (out)    score_c = scale * sum_d q_d * e2m1(code_cd);
 *                                             -inf for holes and columns >= n_valid[b].
 *   topk_ws / topk_ws_bytes  optional: a csa2_topk workspace sized for (batch, n_cols, k);
 *              when given, the level-1 radix histogram of the scores is accumulated into
 *              it and the next csa2_topk call on these scores must pass
 *              CSA2_TOPK_HIST_FUSED.  NULL: no histogram.
 * Errors: INVALID_ARG (null planes, batch < 1, n_cols < 1), ALIGNMENT, WORKSPACE.
 */
int csa2_index_score(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                     const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                     int32_t batch, int32_t n_cols, float* scores,
                     void* topk_ws, size_t topk_ws_bytes, void* stream);

/* Bytes of workspace csa2_topk needs for this shape. */
size_t csa2_topk_workspace_size(int32_t batch, int32_t n_cols, int32_t k);

/*
 * csa2_topk -- a2 top-k selection (pool of 16,384 and top-512 alike).
 *   [STRUCT] commentary on the four layer modes (Reindex re-picks a top-512 inside the
 *   pool); [V4TO41] decoder section (first layer's full scan yields a pool of about 16K
 *   positions, later layers search their top-512 in it).
 *
 *   scores     f32 [batch][n_cols]            finite scores; columns >= n_valid[b] ignored
 *   n_valid    i32 [batch]                    device
 *   cand       i32 [batch][n_cols] or NULL    column -> entry id map; a column whose
 *                                             cand < 0 is ignored.  Must be ascending in
 *                                             the entry id over its valid columns (a pool
 *                                             from a previous call is) so ties by column
 *                                             are ties by entry id.
 *   k          1..16384
 *   idx_out    i32 [batch][k]  (out)          the k best columns (score descending, ties to
 *                                             the lower column), written ASCENDING as entry
 *                                             ids (cand[b][c] or c); -1 padded when fewer
 *                                             than k columns are valid.
 *   score_out  f32 [batch][k] or NULL (out)   score of each listed entry, -inf for padding
 *   flags      CSA2_TOPK_HIST_FUSED or 0
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE.
 */
int csa2_topk(const float* scores, int32_t batch, int32_t n_cols, const int32_t* n_valid,
              const int32_t* cand, int32_t k, int32_t* idx_out, float* score_out,
              uint32_t flags, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace csa2_index_topk needs for this shape on the current device. */
size_t csa2_index_topk_workspace_size(int32_t batch, int32_t n_cols, int32_t k);

/*
 * csa2_index_topk -- a1 + a2 (Full) or a3 + a2 (Reindex) in one call: scores the columns
 * exactly as csa2_index_score does and selects the top-k exactly as csa2_topk does on
 * those scores (same rule, same output), without writing the scores to memory.
 *   [V4TO41] CSA2 architecture section (Full runs the sparse indexer over its keys and
 *   keeps the best entries; Reindex re-picks with its own indexer query) and decoder
 *   section (pool of about 16K positions); [STRUCT] commentary on the four layer modes.
 *
 *   q_idx, idx_codes, idx_scale, seq_base, n_valid, cand   as for csa2_index_score
 *                                             (cand ascending in the entry id over its
 *                                             valid columns, as for csa2_topk)
 *   k          1..16384
 *   idx_out    i32 [batch][k]  (out)          as for csa2_topk
 *   score_out  f32 [batch][k] or NULL (out)   as for csa2_topk
 *   workspace  device, 256-byte aligned, csa2_index_topk_workspace_size bytes, zero-filled
 *              before its first use; each call leaves it ready for the next call of the
 *              same shape.  It starts with a status block (csa2_workspace_status).  Calls
 *              sharing one workspace must not run concurrently.
 * Two launches when the selection can hold the row's candidates: one workgroup per
 * segment of the row keeps the segment's best keys (enough of them for every key of the
 * row's top-k unless the row is far from typical), then each row's exact top-k is taken
 * among them.  No workgroup waits on another, so no co-residency is needed.  A row whose
 * segments left out a key of its top-k is detected and scored again by one workgroup
 * (slower, counted in the status block); the result never depends on the cut.  Rows
 * where k + 6 sqrt(k s) + 7 s > 24,576 for s segments of 16,384 columns (a pool of 16,384
 * beyond 1,556,480 columns) run csa2_index_score's and csa2_topk's kernels.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE, UNSUPPORTED (n_cols > 2^26), HIP.
 */
int csa2_index_topk(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                    const int64_t* seq_base, const int32_t* n_valid, const int32_t* cand,
                    int32_t batch, int32_t n_cols, int32_t k, int32_t* idx_out, float* score_out,
                    void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace csa2_select_chain needs for this shape on the current device. */
size_t csa2_select_chain_workspace_size(int32_t batch, int32_t n_cols, int32_t pool_k);

/*
 * csa2_select_chain -- the selections of a decoder layer chain in one call: the Full
 * layer's scan and pool (a1 + a2), its own top-k inside the pool, and the top-k of up to
 * four Reindex layers that re-score the pool with their own indexer queries (a3 + a2).
 *   [V4TO41] decoder section (the first layer's full scan yields a pool of about 16K
 *   positions that later layers search for their top-512); [STRUCT] commentary on the
 *   four layer modes (Reindex re-picks inside the pool).
 *
 *   q_full, idx_codes, idx_scale, seq_base, n_valid, batch, n_cols   as csa2_index_topk
 *   pool_k         1..16384: pool size
 *   pool_out       i32 [batch][pool_k] (out)  = csa2_index_topk(q_full, k = pool_k)
 *   pool_score_out f32 [batch][pool_k] or NULL (out), its scores
 *   k              1..16384: top-k of the layers below
 *   own_out        i32 [batch][k] or NULL (out) = csa2_topk(pool scores, cand = pool, k):
 *                  the Full layer's own top-k, inside its pool
 *   q_re           bf16 [n_re][batch][128]     Reindex queries (NULL when n_re = 0)
 *   n_re           0..4
 *   re_out         i32 [n_re][batch][k] (out)  = csa2_index_topk(q_re[r], cand = pool,
 *                  n_valid = pool entries, k) for each layer r
 *   re_score_out   f32 [n_re][batch][k] or NULL (out), their scores
 *   workspace      as csa2_index_topk (zero-filled before first use, left ready; starts
 *                  with the status block)
 * Outputs are bit-identical to the separate calls named above.  Rows that csa2_index_topk
 * runs as two launches do so here too: the segments compute the Reindex re-scores of the
 * keys they keep as they write them, and each chained selection takes one workgroup of
 * the second launch.  Other rows run the separate calls.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE, UNSUPPORTED (n_cols > 2^26), HIP.
 */
int csa2_select_chain(const uint16_t* q_full, const uint8_t* idx_codes, const float* idx_scale,
                      const int64_t* seq_base, const int32_t* n_valid, int32_t batch,
                      int32_t n_cols, int32_t pool_k, int32_t* pool_out, float* pool_score_out,
                      int32_t k, int32_t* own_out, const uint16_t* q_re, int32_t n_re,
                      int32_t* re_out, float* re_score_out, void* workspace, size_t ws_bytes,
                      void* stream);

/* Bytes of workspace csa2_replay_select needs for this shape. */
size_t csa2_replay_select_workspace_size(int32_t T, int32_t n_entries, int32_t pool_k);

/*
 * csa2_replay_select -- the Full layer's selections for T consecutive query positions of
 * one sequence (the decoder's bounded replay): per query, the pool of its pool_k best
 * visible entries and its own top-k inside that pool, by the rule csa2_select_chain
 * applies to one decode query.
 *   [STRUCT] content summary and Q&A on prefill (on eviction or restore the decoder replays
 *   only its last 128 tokens); [V4TO41] decoder section (a full scan yields a pool of about
 *   16K positions, later layers pick their top-512 inside it) and the section on the
 *   bounded window replay.
 *
 *   q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, T   as csa2_prefill_chunk (query t
 *              at position pos0 + t sees entries j < min(n_entries, (pos0 + t + 1) / ratio))
 *   pool_k     1..16384
 *   pool_out   i32 [T][pool_k] (out)   the query's pool_k best visible entries (ties to the
 *              lower entry), ascending entry ids, -1 padded
 *   pool_n_out i32 [T] or NULL (out)   valid entries of each pool, min(visible, pool_k): the
 *              n_valid of a Reindex call on the pool
 *   k          1..16384, read only when own_out is given
 *   own_out    i32 [T][k] or NULL (out) the k best entries of each pool by the same scores,
 *              ascending entry ids, -1 padded
 *   workspace  device, 256-byte aligned, csa2_replay_select_workspace_size bytes (it holds
 *              the T x n_entries score matrix), zero-filled before its first use; each call
 *              leaves it ready.  It starts with the status block (csa2_workspace_status).
 *              Calls sharing one workspace must not run concurrently.
 * The scores come from csa2_prefill_chunk's MFMA contraction, which reads the keys once for
 * all T queries, written out as a score matrix that the filtered selection of
 * csa2_index_topk then selects from (csa2_topk's kernels for rows beyond its capacity).
 * They are the same products as csa2_index_score's summed in another order, so a list can
 * differ from a decode call's only where the last bits of fp32 rounding decide a tie.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE, UNSUPPORTED (n_entries > 2^26), HIP.
 */
int csa2_replay_select(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                       int32_t n_entries, int32_t ratio, int64_t pos0, int32_t T, int32_t pool_k,
                       int32_t* pool_out, int32_t* pool_n_out, int32_t k, int32_t* own_out,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * csa2_workspace_status -- reads the status block at the start of a csa2_index_topk,
 * csa2_select_chain or csa2_replay_select workspace.  Enqueues a 12-byte copy on `stream` and synchronizes the
 * stream, so it reports on every call enqueued there before it.
 *   out  host u32 [2] (out):
 *     out[0]  error bits, reserved: always 0 (no kernel of these calls waits on another
 *             workgroup, so none can give up waiting).
 *     out[1]  rows selected by the slow path since the workspace was zero-filled: a
 *             segment left out a key of the row's top-k, or the row's candidates exceeded
 *             what the selection holds; each such row was scored again and selected
 *             exactly.
 * Errors: INVALID_ARG (null pointers), ALIGNMENT (workspace not 256-byte aligned), HIP.
 */
int csa2_workspace_status(const void* workspace, uint32_t* out, void* stream);

/* Bytes of workspace csa2_sparse_attn_decode needs for this shape. */
size_t csa2_attn_workspace_size(int32_t batch, int32_t k);

/*
 * csa2_sparse_attn_decode -- a5 gather-dequant + a6 attention (also a4 Reuse: pass the
 * source layer's index list unchanged; k = 0 gives a window-only layer).
 *   [V4TO41] CSA2 architecture section (Reuse attends over the earlier layer's selected
 *   entries without an indexer); section on global KV sharing with per-layer windows;
 *   [STRUCT] Q&A on the 890-byte count (288-byte main entry = 512 x 4 bit + 32 B scale);
 *   [DEEP] part-4 entry on FP4 in the KV cache (window stays FP8).
 *
 *   q          bf16 [batch][16][512]
 *   kv_codes   u8   [n_total][256]   E2M1, element 2i in the low nibble
 *   kv_scale   u8   [n_total][32]    E4M3, scale g covers values 16g..16g+15
 *   seq_base   i64  [batch]
 *   idx        i32  [batch][k] or NULL when k == 0; entry seq_base[b] + idx; -1 = skip
 *   swa        u8   [batch][128][512] E4M3 window rows; rows 0..swa_len[b]-1 are used
 *   swa_len    i32  [batch]          0..128
 *   out        f32  [batch][16][512] (out) softmax over (selected entries U window rows),
 *              z = (q_h . v) * softmax_scale, out_h = sum p v; zero when nothing attends.
 * Errors: INVALID_ARG (k < 0 or > 16384, null planes), ALIGNMENT, WORKSPACE.
 */
int csa2_sparse_attn_decode(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                            const int64_t* seq_base, const int32_t* idx, int32_t k,
                            const uint8_t* swa, const int32_t* swa_len, float softmax_scale,
                            int32_t batch, float* out, void* workspace, size_t ws_bytes,
                            void* stream);

/*
 * csa2_sparse_attn_decode_noalloc -- csa2_sparse_attn_decode for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and results.
 * The split partials live in a static device array of csa2_attn_noalloc_max_bytes()
 * (16 MiB) that the library holds on each GPU it runs on until the process ends; its
 * device address is looked up on each device's first call (hipGetSymbolAddress) and kept.
 * The call allocates and frees nothing.  Every call on one GPU shares that GPU's array,
 * so calls that overlap in time on one GPU (different streams or threads) race; nothing
 * in the array needs to start at zero (each split writes its partial before the merge
 * reads it).
 * Errors: as csa2_sparse_attn_decode, and SCRATCH when csa2_attn_workspace_size(batch, k)
 * exceeds csa2_attn_noalloc_max_bytes(); HIP if the address lookup fails.
 */
int csa2_sparse_attn_decode_noalloc(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                                    const int64_t* seq_base, const int32_t* idx, int32_t k,
                                    const uint8_t* swa, const int32_t* swa_len, float softmax_scale,
                                    int32_t batch, float* out, void* stream);

/* Bytes of the static scratch csa2_sparse_attn_decode_noalloc uses (16 MiB). */
size_t csa2_attn_noalloc_max_bytes(void);

/* Bytes of workspace csa2_prefill_chunk needs for this shape. */
size_t csa2_prefill_workspace_size(int32_t T, int32_t n_entries, int32_t k);

/*
 * csa2_prefill_chunk -- a7 causal indexer contraction (BF16 MFMA) + a8 per-query top-k
 * and attention, for T consecutive query positions of one sequence.
 *   [STRUCT] content summary and Q&A on prefill (prompt tokens run the encoder, whose
 *   Full layers score and select per token); [V4TO41] encoder section (1:2 token
 *   compression: one entry per two tokens) and section on the sliding window.
 *
 *   q_idx      bf16 [T][128]        indexer queries, query t at position pos0 + t
 *   q          bf16 [T][16][512]
 *   idx_codes, idx_scale, kv_codes, kv_scale   entries 0..n_entries-1 of the sequence
 *   ratio      tokens per entry (>= 1); entry j is visible to position p when
 *              (j+1)*ratio - 1 <= p, i.e. j < (p+1)/ratio
 *   pos0       position of query 0 (>= 0)
 *   k          1..16384 entries per query
 *   swa        u8 [T+127][512]      E4M3 window rows; row r holds position pos0-127+r.
 *              Query t attends rows for positions max(0,p-127)..p.  Rows for negative
 *              positions are never read.
 *   idx_out    i32 [T][k] (out)     ascending entry ids, -1 padded
 *   out        f32 [T][16][512] (out)
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE.
 */
int csa2_prefill_chunk(const uint16_t* q_idx, const uint16_t* q, const uint8_t* idx_codes,
                       const float* idx_scale, const uint8_t* kv_codes,
                       const uint8_t* kv_scale, int32_t n_entries, int32_t ratio, int64_t pos0,
                       int32_t T, int32_t k, const uint8_t* swa, float softmax_scale,
                       int32_t* idx_out, float* out, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * csa2_prefill_select -- a7 and the per-query top-k of csa2_prefill_chunk without the
 * attention: idx_out is exactly what csa2_prefill_chunk writes for the same arguments.  For
 * a layer group whose Full layer selects once and whose Reuse layers attend over the same
 * lists (csa2_sparse_attn_prefill per layer).
 *   [STRUCT] content summary and Q&A on prefill; [V4TO41] CSA2 architecture (Reuse).
 *   Arguments as csa2_prefill_chunk; the workspace is csa2_prefill_workspace_size(T,
 *   n_entries, k) bytes, 256-byte aligned, no zero-filling needed.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE.
 */
int csa2_prefill_select(const uint16_t* q_idx, const uint8_t* idx_codes, const float* idx_scale,
                        int32_t n_entries, int32_t ratio, int64_t pos0, int32_t T, int32_t k,
                        int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_prefill -- a5 + a6 for T consecutive query positions of one sequence,
 * each over its own list and its own causal window: the attention half of
 * csa2_prefill_chunk, for lists made elsewhere (a Reuse layer of a prefill or replay chunk
 * attends over the list of the layer it reuses).
 *   [V4TO41] CSA2 architecture (Reuse attends over an earlier layer's selection) and
 *   section on global KV sharing with per-layer windows; [STRUCT] Q&A on prefill.
 *   q          bf16 [T][16][512]     query t at position pos0 + t
 *   kv_codes, kv_scale               entries of the sequence from 0 (as csa2_prefill_chunk)
 *   idx        i32 [T][k] or NULL when k == 0; entry ids, -1 = skip
 *   swa        u8 [T+127][512]       E4M3 window rows; row r holds position pos0-127+r;
 *              query t attends the rows for positions max(0,p-127)..p
 *   out        f32 [T][16][512] (out)
 *   workspace  device, 256-byte aligned, csa2_attn_workspace_size(T, k) bytes (partials when
 *              few rows are split over workgroups); no zero-filling needed
 * Errors: INVALID_ARG (T < 1, k < 0 or > 16384, pos0 < 0, null pointers), ALIGNMENT,
 * WORKSPACE.
 */
int csa2_sparse_attn_prefill(const uint16_t* q, const uint8_t* kv_codes, const uint8_t* kv_scale,
                             const int32_t* idx, int32_t k, const uint8_t* swa, int64_t pos0,
                             int32_t T, float softmax_scale, float* out, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * csa2_kv_append -- the write path in front of the hot path: quantise n new global-KV
 * entries into entry ids dst[i] of the four planes.
 *   [STRUCT] Q&A on the 890-byte count (indexer entry = 128 x 4 bit + 4-byte scale = 68 B,
 *   main entry = 512 x 4 bit + 32 B of scale = 288 B); [DEEP] part-4 entry on FP4 in the KV
 *   cache (main KV and indexer in different 4-bit formats).  Encoders (this library's
 *   reading; csa2_index_score and csa2_sparse_attn_decode decode exactly these):
 *     indexer  scale = fp32(amax/6) over the 128 values (1 if below 2^-126),
 *              code_d = E2M1(fp32(x_d / scale));
 *     main     per 16 values scale = E4M3(fp32(amax/6)) (code 0 becomes 1, i.e. 2^-9),
 *              code_d = E2M1(fp32(x_d / scale));
 *     E2M1 / E4M3  nearest, ties to even, saturating (6 / 448); the sign bit is the
 *              value's; element 2i in the low nibble.  Inputs must be finite.
 *
 *   x_idx      bf16 [n][128]      new indexer vectors
 *   x_kv       bf16 [n][512]      new main vectors
 *   dst        i64  [n]           entry id of each row; ids must be distinct.  A row whose
 *                                 id is outside [0, capacity) is not written.
 *   idx_codes  u8 [capacity][64], idx_scale f32 [capacity], kv_codes u8 [capacity][256],
 *   kv_scale   u8 [capacity][32]  (in/out) the planes; only rows dst[i] are written
 *   bad        i32 [1] or NULL    (in/out) if given, the number of rows not written
 *                                 (dst out of range) is added to *bad
 * n = 0 launches nothing.  Errors: INVALID_ARG (n < 0, capacity < 1, null planes),
 * ALIGNMENT (x_idx, x_kv, kv_codes, idx_codes 16 B; idx_scale, bad 4 B; dst 8 B).
 */
int csa2_kv_append(const uint16_t* x_idx, const uint16_t* x_kv, const int64_t* dst, int32_t n,
                   uint8_t* idx_codes, float* idx_scale, uint8_t* kv_codes, uint8_t* kv_scale,
                   int64_t capacity, int32_t* bad, void* stream);

/*
 * csa2_swa_append -- write one new window row per sequence as E4M3 into its ring:
 * swa[b][pos[b] mod 128] = E4M3(x[b]) (nearest, ties to even, saturating at 448).
 *   [DEEP] part-4 entry on FP4 in the KV cache (the sliding window stays FP8); [V4TO41]
 *   section on global KV sharing with per-layer windows (128 tokens per layer).
 *   x      bf16 [batch][512]
 *   pos    i64  [batch]   position of the new token; a sequence with pos < 0 is skipped
 *   swa    u8   [batch][128][512] (in/out) the layer's rings; csa2_sparse_attn_decode
 *          attends rows 0..swa_len-1 with swa_len = min(pos + 1, 128)
 * Errors: INVALID_ARG (batch < 0, null pointers), ALIGNMENT (x, swa 16 B; pos 8 B).
 */
int csa2_swa_append(const uint16_t* x, const int64_t* pos, int32_t batch, uint8_t* swa,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H_ */
