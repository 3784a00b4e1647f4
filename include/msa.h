/*
 * msa.h - MiniMax Sparse Attention (MSA) hot path on AMD Instinct MI355X (gfx950).
 *
 * MSA splits the KV cache into 128-token blocks, scores every block with a light
 * indexer for each query tile or GQA query group, keeps the top-k blocks and runs
 * exact softmax attention over those blocks only. Pages this follows:
 *   [dd]   daily.dev, "MiniMax M3: 1M-token multimodal reasoning model now available
 *          with NVIDIA and vLLM support", sections "Summary", "What makes M3
 *          different" and "Serving options" (128-token KV blocks, top blocks per
 *          query, prefill/decode kernels for sparse GQA, KV-block-major prefill).
 *   [feat] models.inteligile.com, "MiniMax-M3" feature page, table "Checked in its
 *          code", rows "Indexer-selected sparse attention (DeepSeek Sparse
 *          Attention)", "Grouped-query attention" and "Learnable attention sink";
 *          method list "Two-phase forward", "LSE fusion", "Exp-free TopK kernel".
 *   [vllm] 24-ai.news, "MiniMax M3 in vLLM: Day-0-Unterstuetzung ...", section
 *          "Warum ist ein Million-Token-Kontext eine Serving-Herausforderung?"
 *          (each query or GQA query group scores all blocks with light indexer
 *          kernels; KV-block-major layout).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the name starts with h_ (host memory).
 *     Arrays are dense, row-major, with the shapes given below, 16-byte aligned.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronizes; each call only enqueues kernels on `stream` (a hipStream_t,
 *     NULL for the default stream) and returns.
 *   - Arguments are validated on the host before anything is enqueued. On an
 *     error nothing is enqueued and no output is written; msa_last_error() then
 *     describes the problem (thread-local string). Launch failures are reported
 *     as MSA_ERR_HIP. Device-side values (seq_lens, block_table, ids) are not
 *     checked: out-of-range entries are undefined behaviour.
 *   - Calls are re-entrant and thread-safe.
 *   - Debugging aid: with the environment variable MSA_LOG set to a non-zero
 *     value, every kernel launch prints its kernel, grid, block and dynamic LDS
 *     bytes to stderr, and every refused call its status and reason (read at
 *     every call; off by default).
 *
 * Data layout (block-major paged caches, [dd] "Serving options", [vllm]):
 *   k_cache            [num_phys_blocks][H_kv][128][D]     (dtype), token-major
 *   v_cache            [num_phys_blocks][H_kv][D][128]     (dtype), d-major: each
 *                      block of values is stored transposed, so that the P.V
 *                      contraction over a block's keys reads contiguous rows
 *   k_idx_cache        [num_phys_blocks][H_i][128][D_i]    (dtype), token-major
 *   block_table        int32 [num_seqs][max_blocks_per_seq], logical -> physical
 *   seq_lens           int32 [num_seqs], tokens in the cache INCLUDING the new
 *                      queries (their K/V/k_idx are inserted before these calls)
 *   Token s of sequence r lives in physical block block_table[r][s / 128], row
 *   s % 128. Byte offsets are 64-bit.
 *
 * FP8 caches (geom->cache_format == MSA_CACHE_FP8_E4M3; [dd] "What's coming" lists
 * FP8 KV-cache paths, the format is this library's): the three caches hold one
 * byte per element, an OCP E4M3 code (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite 448, S.1111.111 = NaN), same shapes as above.
 * Every 32 consecutive channels of one token's head vector share a scale 2^e,
 * stored as the byte e + 127 (OCP E8M0); the element's value is code * 2^e.
 *   k_scale            uint8 [num_phys_blocks][H_kv][128][D/32]
 *   v_scale            uint8 [num_phys_blocks][H_kv][D/32][128]  (token fastest,
 *                      like the d-major V codes)
 *   k_idx_scale        uint8 [num_phys_blocks][H_i][128][D_i/32]
 * A writer picks e as the smallest integer with max|x| / 2^e <= 448 over the 32
 * channels and stores the nearest code of x / 2^e (ties to even), as
 * msa_qk_norm_rope_insert does. Scales never span tokens, so inserting a token
 * touches only that token's bytes.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_BLOCK_SIZE 128

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,          /* null pointer, bad size or inconsistent shape */
  MSA_ERR_UNSUPPORTED = 2,          /* valid but not built: dtype, D, D_i, block size */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,  /* a workspace smaller than required */
  MSA_ERR_HIP = 4                   /* a HIP launch failed */
} msa_status_t;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype_t;

typedef enum {
  MSA_CACHE_PLAIN = 0,      /* caches in geom->dtype */
  MSA_CACHE_FP8_E4M3 = 1    /* E4M3 codes + a power-of-two scale per 32 channels */
} msa_cache_format_t;

/* Head geometry ([feat] "Grouped-query attention": 64 query heads share 4 KV heads;
 * query head i reads KV head i / (num_q_heads / num_kv_heads)).
 *   num_q_heads % num_kv_heads == 0, (num_q_heads / num_kv_heads) <= 16 for bf16
 *   head_dim in {64, 128}; idx_head_dim in {32, 64}
 *   num_sel_groups is num_kv_heads (group g sums indexer heads
 *     [g*H_s, (g+1)*H_s), H_s = num_idx_heads / num_sel_groups, and selects the
 *     blocks of KV head g) or 1 (the sum over all indexer heads selects for every
 *     KV head); num_idx_heads % num_sel_groups == 0, H_s in {1, 2, 4, 8},
 *     H_s * idx_head_dim <= 512
 *   block_size must be 128.
 *   dtype applies to q, q_idx, out and (cache_format PLAIN) the three caches.
 *   cache_format MSA_CACHE_FP8_E4M3 needs dtype MSA_BF16; it is read by every
 *     indexer and attention call and written by msa_qk_norm_rope_insert. */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_idx_heads;
  int32_t idx_head_dim;
  int32_t num_sel_groups;
  int32_t block_size;
  int32_t dtype;                    /* msa_dtype_t */
  int32_t cache_format;             /* msa_cache_format_t */
} msa_geom_t;

/* The three caches are written only by msa_qk_norm_rope_insert; every other
 * call reads them. */
typedef struct {
  void *k_cache;
  void *v_cache;
  void *k_idx_cache;
  int64_t num_phys_blocks;
  const int32_t *block_table;       /* [num_seqs][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  const int32_t *seq_lens;          /* [num_seqs] */
  int32_t num_seqs;
  uint8_t *k_scale;                 /* FP8 caches only (else ignored), see above */
  uint8_t *v_scale;
  uint8_t *k_idx_scale;
} msa_cache_t;

/* One prefill unit: the new queries of request r whose positions fall in the
 * 128-token block tau (its diagonal block). Rows [row0, row0 + num_rows) of q and
 * q_idx, positions [pos0, pos0 + num_rows). Built by msa_prefill_plan. */
typedef struct {
  int32_t r, tau, row0, num_rows, pos0;
} msa_unit_t;

/* A (chunked) prefill batch. Request r's q_lens[r] new queries are the last
 * q_lens[r] tokens of its cache, stored in q/q_idx after those of requests
 * 0..r-1 (total_q rows in all). units is the DEVICE copy of the plan. */
typedef struct {
  const msa_unit_t *units;          /* [total_units], device */
  int32_t total_units;
  int32_t total_q;
} msa_batch_t;

/* Host-side plan of a prefill batch: splits each request's new queries at
 * 128-position boundaries ([dd]: 128-token blocks; the first unit of a chunk that
 * starts mid-block is partial). With h_units == NULL only *h_num_units is set.
 * Otherwise up to `capacity` units are written in request order, tiles ascending.
 * Needs 0 <= h_q_lens[r] <= h_seq_lens[r], and at most 2^31 - 1 units and query
 * rows in all (row offsets are int32); else MSA_ERR_INVALID_ARG. Pure host code. */
msa_status_t msa_prefill_plan(const int32_t *h_seq_lens, const int32_t *h_q_lens,
                              int32_t num_seqs, msa_unit_t *h_units, int32_t capacity,
                              int32_t *h_num_units);

/* Debugging aids for the device-side values the calls trust (out-of-range
 * entries are undefined behaviour there): pure host code over HOST copies, to be
 * run on a batch that misbehaves. Each returns MSA_OK, or MSA_ERR_INVALID_ARG with
 * msa_last_error() naming the first violation.
 * msa_validate_block_table: for every sequence r, seq_lens[r] >= 1 fits in
 *   max_blocks_per_seq blocks of 128 and the entries of its blocks, block_table[r]
 *   [0 .. ceil(seq_lens[r] / 128) - 1], are physical blocks in [0, num_phys_blocks).
 * msa_validate_ids: every list of ids [num_rows][num_sel_groups][topk] (the
 *   selection's output, or a caller's own) holds distinct entries in
 *   [0, max_blocks_per_seq) before its first -1. */
msa_status_t msa_validate_block_table(const int32_t *h_block_table, const int32_t *h_seq_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_phys_blocks);
msa_status_t msa_validate_ids(const int32_t *h_ids, int32_t num_rows, int32_t num_sel_groups,
                              int32_t topk, int32_t max_blocks_per_seq);

/* Step 1, indexer block scores ([feat] row "Indexer-selected sparse attention":
 * a lightning indexer scores keys per head and pools them into blocks; [vllm]:
 * each query or GQA query group scores every available block).
 *   q_idx   prefill: [batch->total_q][H_i][D_i]; decode (batch == NULL):
 *           [num_seqs][H_i][D_i], the one new query of sequence r at position
 *           seq_lens[r] - 1.
 *   scores  fp32 [U][num_sel_groups][max_blocks_per_seq], U = total_units
 *           (prefill) or num_seqs (decode). For unit u with diagonal block tau
 *           and group g:
 *             b <  tau : max over the unit's queries t and block b's 128 keys s of
 *                        sum_{h in g} q_idx[t,h,:] . k_idx[s,h,:] (fp32 accumulate)
 *             b == tau : +inf (the diagonal block is always kept)
 *             b >  tau : -inf (causal: future blocks are never kept)
 * Prefill runs on bf16 MFMA for bf16 inputs; decode streams k_idx once.
 * A prefill batch with no units enqueues nothing (q_idx and scores may be NULL). */
msa_status_t msa_index_scores(const msa_geom_t *geom, const msa_cache_t *cache,
                              const msa_batch_t *batch, const void *q_idx,
                              float *scores, void *stream);

/* Step 2, block top-k ([feat]: topk = min(topk_blocks, num_key_blocks), -inf
 * selections become -1; [feat] method "Exp-free TopK kernel": raw scores are
 * ranked, no softmax). Generic over rows:
 *   scores fp32 [num_rows][row_len]; ids int32 [num_rows][topk].
 * Per row, the K = min(topk, #entries > -inf) entries of highest score are kept,
 * equal scores ordered by lower index; their indices are written in ascending
 * order and the remaining topk - K slots are set to -1. NaN scores are undefined.
 * Requires 1 <= topk, 1 <= row_len; num_rows == 0 enqueues nothing. */
msa_status_t msa_select_topk_blocks(const float *scores, int32_t num_rows,
                                    int32_t row_len, int32_t topk, int32_t *ids,
                                    void *stream);

/* Step 3, sparse prefill attention ([dd] "Serving options": prefill kernel for
 * sparse GQA; [feat] rows "Grouped-query attention", "Learnable attention sink":
 * plain softmax, no sink, no output gate).
 *   q    [total_q][H_q][D];  ids int32 [total_units][num_sel_groups][topk]
 *   out  [total_q][H_q][D] (dtype, rounded to nearest even);
 *   lse  fp32 [total_q][H_q] natural-log logsumexp of the logits, or NULL.
 * Query t of unit u, head i (KV head j = i / G, selection group g = j or 0)
 * attends to every key s of the blocks ids[u][g][*] with s <= pos(t):
 *   out = softmax(softmax_scale * q . k) . v  (fp32 softmax).
 * ids rows: distinct block ids, ended by the first -1 (entries after it are
 * ignored); step 2's output (ascending, the unit's diagonal block last) is the
 * fast case. Every listed block is masked by position, so any order and any
 * subset give the result above: a listed id after the unit's diagonal block tau
 * holds only future keys and is not read; ids must lie in [0,
 * max_blocks_per_seq) (out-of-range values are undefined behaviour). A query row
 * with no visible key (its list holds no block up to its own position) gets
 * out = 0 and lse = -inf.
 * softmax_scale must be finite; <= 0 selects 1/sqrt(D). bf16 runs on MFMA with
 * fp32 accumulation; probabilities are rounded to bf16 for the P.V product. A
 * batch with no units enqueues nothing (q, ids and out may be NULL). */
msa_status_t msa_sparse_attn_prefill(const msa_geom_t *geom, const msa_cache_t *cache,
                                     const msa_batch_t *batch, const void *q,
                                     const int32_t *ids, int32_t topk,
                                     float softmax_scale, void *out, float *lse,
                                     void *stream);

/* Bytes of device workspace msa_sparse_attn_prefill_staged needs for a batch of
 * total_units units: 0 unless the caches are FP8; for FP8 a slot map over
 * cache->num_phys_blocks x H_kv and room for H_kv * min(num_phys_blocks,
 * total_units * topk) bf16 copies of a block's K and V rows (64 KiB each at
 * D = 128). Returns 0 for invalid arguments. */
size_t msa_prefill_workspace_size(const msa_geom_t *geom, const msa_cache_t *cache,
                                  int32_t total_units, int32_t topk);

/* Step 3 as msa_sparse_attn_prefill (same arguments, rows, masking and result),
 * with a workspace. On FP8 caches ([dd] "What's coming": FP8 KV-cache paths) every
 * (physical block, KV head) that some unit keeps is converted once, exactly, to
 * bf16 in the workspace, and the bf16 attention reads those copies: the same
 * result up to the order of fp32 sums, without converting a block again in every
 * work-group that reads it. Other caches need no workspace (size 0; workspace may
 * be NULL) and run as msa_sparse_attn_prefill.
 *   workspace >= msa_prefill_workspace_size(geom, cache, batch->total_units, topk)
 *   bytes, device, 256-byte aligned, owned by the caller; its contents are
 *   rebuilt by every call (nothing needs clearing), and calls that share one
 *   workspace must be ordered on a stream.
 *   MSA_ERR_WORKSPACE_TOO_SMALL when workspace_bytes is below that size (nothing
 *   is enqueued). Block-table entries must lie in [0, num_phys_blocks). */
msa_status_t msa_sparse_attn_prefill_staged(const msa_geom_t *geom, const msa_cache_t *cache,
                                            const msa_batch_t *batch, const void *q,
                                            const int32_t *ids, int32_t topk,
                                            float softmax_scale, void *workspace,
                                            size_t workspace_bytes, void *out, float *lse,
                                            void *stream);

/* Bytes of device workspace msa_sparse_attn_decode needs. num_splits <= 0 picks
 * the library's own split count for this shape (the same one the decode call
 * picks for num_splits <= 0). For msa_sparse_attn_decode_per_token pass the
 * number of token rows, num_seqs * tokens_per_seq, as num_seqs. */
size_t msa_decode_workspace_size(const msa_geom_t *geom, int32_t num_seqs,
                                 int32_t topk, int32_t num_splits);

/* Steps 3+4 for decode, split-KV with a log-sum-exp combine ([dd] "Serving
 * options": decode kernel for sparse GQA; [feat] methods "Two-phase forward" and
 * "LSE fusion").
 *   q   [num_seqs][H_q][D], the new query of sequence r at position seq_lens[r]-1
 *   ids int32 [num_seqs][num_sel_groups][topk], rows as for the prefill call
 *       (distinct ids, ended by -1; keys after the query are masked by position,
 *       later blocks are not read; a query with no visible key gets out = 0 and
 *       lse = -inf)
 *   workspace >= msa_decode_workspace_size(...) bytes, device, 256-byte aligned
 *   out [num_seqs][H_q][D] (dtype); lse fp32 [num_seqs][H_q] or NULL.
 * The selected slots are split into num_splits parts (<= 0: automatic), each
 * part is attended separately and the parts are merged by their logsumexp; the
 * result equals one softmax over all selected keys up to fp32 rounding.
 * softmax_scale must be finite; <= 0 selects 1/sqrt(D). */
msa_status_t msa_sparse_attn_decode(const msa_geom_t *geom, const msa_cache_t *cache,
                                    const void *q, const int32_t *ids, int32_t topk,
                                    float softmax_scale, int32_t num_splits,
                                    void *workspace, size_t workspace_bytes, void *out,
                                    float *lse, void *stream);

/* Bytes of the static scratch that msa_sparse_attn_decode_static uses, per GPU. */
#define MSA_STATIC_SCRATCH_BYTES (16u * 1024u * 1024u)

/* msa_sparse_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as msa_sparse_attn_decode without the workspace: the
 * split partials go to a scratch array of MSA_STATIC_SCRATCH_BYTES that the
 * library keeps in static device memory, one copy on each GPU it runs on, held
 * until the process ends (its address is looked up once per device, on the
 * first call there, with hipGetSymbolAddress: make that first call outside any
 * graph capture). The call allocates and frees nothing.
 *   MSA_ERR_WORKSPACE_TOO_SMALL when msa_decode_workspace_size(geom, num_seqs,
 *   topk, num_splits) exceeds MSA_STATIC_SCRATCH_BYTES (nothing is enqueued).
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * partials in it; each call writes every entry it reads, so nothing needs to
 * start at zero. Calls that overlap in time on one GPU (streams with no order
 * between them) race on the array and give undefined results; calls ordered on
 * one stream are safe. */
msa_status_t msa_sparse_attn_decode_static(const msa_geom_t *geom, const msa_cache_t *cache,
                                           const void *q, const int32_t *ids, int32_t topk,
                                           float softmax_scale, int32_t num_splits, void *out,
                                           float *lse, void *stream);

/* Per-query-token selection for T new tokens per sequence (multi-token decode:
 * speculative verification, multi-token prediction). [feat] row "Indexer-selected
 * sparse attention": the model selects per query token ([B, H_idx, S_q, topk]).
 * Sequence r has T = tokens_per_seq (1 <= T <= 8, T * num_sel_groups <= 128) new
 * tokens at positions seq_lens[r] - T + i, stored as rows r * T + i; each token
 * row is its own unit: it scores the blocks with its own indexer query, keeps its
 * own diagonal block (position / 128) and top-k, and attends causally. T = 1 is
 * the decode path of msa_index_scores / msa_sparse_attn_decode.
 *   msa_index_scores_per_token:  q_idx [num_seqs * T][H_i][D_i]
 *       -> scores fp32 [num_seqs * T][num_sel_groups][max_blocks_per_seq]
 *   msa_select_topk_blocks over those rows -> ids [num_seqs * T][num_sel_groups][topk]
 *   msa_sparse_attn_decode_per_token:  q [num_seqs * T][H_q][D], ids as above
 *       -> out [num_seqs * T][H_q][D], lse fp32 [num_seqs * T][H_q] or NULL;
 *       workspace >= msa_decode_workspace_size(geom, num_seqs * T, topk, num_splits).
 * Requires seq_lens[r] >= T (device values are not checked). */
msa_status_t msa_index_scores_per_token(const msa_geom_t *geom, const msa_cache_t *cache,
                                        int32_t tokens_per_seq, const void *q_idx,
                                        float *scores, void *stream);
msa_status_t msa_sparse_attn_decode_per_token(const msa_geom_t *geom, const msa_cache_t *cache,
                                              int32_t tokens_per_seq, const void *q,
                                              const int32_t *ids, int32_t topk,
                                              float softmax_scale, int32_t num_splits,
                                              void *workspace, size_t workspace_bytes,
                                              void *out, float *lse, void *stream);

/* Per-query-token selection in prefill ([feat] row "Indexer-selected sparse
 * attention": the model selects per query token, [B, H_idx, S_q, topk]). Every
 * new token of a planned prefill batch is its own selection unit: row t (of
 * unit u, position p = u.pos0 + t - u.row0, diagonal block p / 128) scores the
 * blocks with its own indexer query, keeps its own top-k and attends causally
 * over its own blocks. A batch of T new tokens per sequence gives the same rows
 * as msa_index_scores_per_token.
 *   msa_index_scores_prefill_tokens: q_idx [total_q][H_i][D_i] ->
 *       scores fp32 [total_q][num_sel_groups][max_blocks_per_seq]; for row t
 *       and group g, block b < p/128 scores the max over its 128 keys s of
 *       sum_{h in g} q_idx[t,h,:] . k_idx[s,h,:]; b == p/128 is +inf, later -inf.
 *   msa_select_topk_blocks over those rows -> ids [total_q][num_sel_groups][topk]
 *   msa_sparse_attn_prefill_tokens: q [total_q][H_q][D], ids as above (rows as
 *       for msa_sparse_attn_prefill: distinct ids, ended by the first -1,
 *       masked by position) -> out [total_q][H_q][D], lse fp32 [total_q][H_q] or
 *       NULL. Every 32 rows of a unit are attended together over the union
 *       of their lists, each row over its own blocks only. workspace (device,
 *       256-byte aligned) of msa_prefill_tokens_workspace_size(geom, total_units,
 *       total_q, topk) bytes holds the unions (0 bytes for fp32: workspace may
 *       be NULL). max_blocks_per_seq <= 131072.
 * softmax_scale as for msa_sparse_attn_prefill. A batch with no units enqueues
 * nothing. */
msa_status_t msa_index_scores_prefill_tokens(const msa_geom_t *geom, const msa_cache_t *cache,
                                             const msa_batch_t *batch, const void *q_idx,
                                             float *scores, void *stream);
size_t msa_prefill_tokens_workspace_size(const msa_geom_t *geom, int32_t total_units,
                                         int32_t total_q, int32_t topk);
msa_status_t msa_sparse_attn_prefill_tokens(const msa_geom_t *geom, const msa_cache_t *cache,
                                            const msa_batch_t *batch, const void *q,
                                            const int32_t *ids, int32_t topk,
                                            float softmax_scale, void *workspace,
                                            size_t workspace_bytes, void *out, float *lse,
                                            void *stream);

/* Step 0, the new tokens before step 1: per-head RMSNorm of queries and keys,
 * partial rotary embedding, and the insert of K, V and the indexer keys into the
 * caches ([feat] table "Checked in its code", rows "QK normalization" and
 * "Partial RoPE" (partial_rotary_factor 0.5, rotary_dim 64); [dd] "Serving
 * options": fused QK-norm + RoPE + KV insert). For a new token at position p and
 * a head vector x (D channels), with R = rotary_dim:
 *   n[c] = x[c] / sqrt(mean(x^2) + eps) * w[c]        (w = q_norm_w or k_norm_w)
 *   c < R/2, a = p * rope_theta^(-2c/R):
 *     y[c] = n[c] cos a - n[c+R/2] sin a;  y[c+R/2] = n[c+R/2] cos a + n[c] sin a
 *   c >= R: y[c] = n[c]
 * Angles are formed in fp64; the rest runs in fp32 and is rounded to dtype
 * (nearest even) once.
 *   batch    prefill: the planned batch (msa_prefill_plan), token t of unit u is
 *            row u.row0 + t at position u.pos0 + t; NULL: decode, the one new
 *            token of sequence r is row r at position seq_lens[r] - 1
 *   q        [rows][H_q][D]        -> q_out [rows][H_q][D] (may equal q: in place)
 *   k        [rows][H_kv][D]       -> k_cache rows, normalized and rotated
 *   v        [rows][H_kv][D]       -> v_cache (d-major blocks), unchanged bits
 *   k_idx    [rows][H_i][D_i]      -> k_idx_cache rows, unchanged bits
 *   q_norm_w, k_norm_w  [D] (dtype), shared by all heads
 *   eps >= 0, rope_theta > 0, rotary_dim 0 (no rotation) or a power of two with
 *   16 <= rotary_dim <= D (bf16; 8 <= rotary_dim for fp32).
 * rows = batch->total_q or num_seqs. A new token at position p of request r goes
 * to physical block block_table[r][p / 128], row p % 128; nothing else in the
 * caches is written, and q_idx is not an input (the indexer query is used as
 * given). Non-finite results (eps == 0 with an all-zero head) are undefined.
 * A prefill batch with no units enqueues nothing. */
msa_status_t msa_qk_norm_rope_insert(const msa_geom_t *geom, const msa_cache_t *cache,
                                     const msa_batch_t *batch, const void *q, const void *k,
                                     const void *v, const void *k_idx, const void *q_norm_w,
                                     const void *k_norm_w, float eps, float rope_theta,
                                     int32_t rotary_dim, void *q_out, void *stream);

const char *msa_status_string(msa_status_t status);
const char *msa_last_error(void);
int32_t msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
