// C-ABI entry points of libmsa: host-side validation, then kernel launches.
// Every check here runs before anything is enqueued; see msa.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "msa.h"
#include "msa_launch.h"

namespace msa {

bool log_enabled() {
  const char *v = std::getenv("MSA_LOG");
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

void log_launch(const char *kernel, dim3 grid, dim3 block, size_t lds) {
  std::fprintf(stderr, "msa: launch %s grid (%u, %u, %u) block (%u, %u, %u) lds %zu\n", kernel,
               grid.x, grid.y, grid.z, block.x, block.y, block.z, lds);
}

}  // namespace msa

namespace {

thread_local std::string g_last_error;

msa_status_t fail(msa_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (msa::log_enabled()) std::fprintf(stderr, "msa: refused (status %d): %s\n", st, buf);
  return st;
}

msa_status_t ok() {
  g_last_error.clear();
  return MSA_OK;
}

msa_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// Geometry checks shared by every call. Fills `out` on success.
msa_status_t check_geom(const msa_geom_t *g, msa::Geom *out) {
  MSA_REQUIRE(g != nullptr, MSA_ERR_INVALID_ARG, "geom is NULL");
  MSA_REQUIRE(g->num_q_heads > 0 && g->num_kv_heads > 0 && g->head_dim > 0 &&
                  g->num_idx_heads > 0 && g->idx_head_dim > 0 && g->num_sel_groups > 0,
              MSA_ERR_INVALID_ARG, "geometry sizes must be positive");
  MSA_REQUIRE(g->num_q_heads % g->num_kv_heads == 0, MSA_ERR_INVALID_ARG,
              "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", g->num_q_heads,
              g->num_kv_heads);
  MSA_REQUIRE(g->num_sel_groups == 1 || g->num_sel_groups == g->num_kv_heads,
              MSA_ERR_INVALID_ARG, "num_sel_groups (%d) must be 1 or num_kv_heads (%d)",
              g->num_sel_groups, g->num_kv_heads);
  MSA_REQUIRE(g->num_idx_heads % g->num_sel_groups == 0, MSA_ERR_INVALID_ARG,
              "num_idx_heads (%d) is not a multiple of num_sel_groups (%d)",
              g->num_idx_heads, g->num_sel_groups);
  MSA_REQUIRE(g->block_size == MSA_BLOCK_SIZE, MSA_ERR_UNSUPPORTED,
              "block_size %d unsupported (only 128)", g->block_size);
  MSA_REQUIRE(g->dtype == MSA_F32 || g->dtype == MSA_BF16, MSA_ERR_UNSUPPORTED,
              "dtype %d unsupported", g->dtype);
  MSA_REQUIRE(g->head_dim == 64 || g->head_dim == 128, MSA_ERR_UNSUPPORTED,
              "head_dim %d unsupported (64 or 128)", g->head_dim);
  MSA_REQUIRE(g->idx_head_dim == 32 || g->idx_head_dim == 64, MSA_ERR_UNSUPPORTED,
              "idx_head_dim %d unsupported (32 or 64)", g->idx_head_dim);
  const int hs = g->num_idx_heads / g->num_sel_groups;
  MSA_REQUIRE(hs == 1 || hs == 2 || hs == 4 || hs == 8, MSA_ERR_UNSUPPORTED,
              "indexer heads per selection group (%d) must be 1, 2, 4 or 8", hs);
  MSA_REQUIRE(hs * g->idx_head_dim <= 512, MSA_ERR_UNSUPPORTED,
              "indexer group width %d exceeds 512", hs * g->idx_head_dim);
  MSA_REQUIRE(g->num_sel_groups <= 16, MSA_ERR_UNSUPPORTED, "more than 16 selection groups");
  MSA_REQUIRE(g->dtype != MSA_BF16 || g->num_q_heads / g->num_kv_heads <= 16,
              MSA_ERR_UNSUPPORTED, "bf16 needs at most 16 query heads per KV head");
  MSA_REQUIRE(g->cache_format == MSA_CACHE_PLAIN || g->cache_format == MSA_CACHE_FP8_E4M3,
              MSA_ERR_UNSUPPORTED, "cache_format %d unsupported", g->cache_format);
  MSA_REQUIRE(g->cache_format != MSA_CACHE_FP8_E4M3 || g->dtype == MSA_BF16,
              MSA_ERR_UNSUPPORTED, "FP8 caches need dtype bf16");
  out->Hq = g->num_q_heads;
  out->Hkv = g->num_kv_heads;
  out->D = g->head_dim;
  out->Hi = g->num_idx_heads;
  out->Di = g->idx_head_dim;
  out->nsel = g->num_sel_groups;
  out->bf16 = g->dtype == MSA_BF16;
  out->fp8 = g->cache_format == MSA_CACHE_FP8_E4M3;
  return ok();
}

msa_status_t check_cache(const msa_cache_t *c, bool need_kv, bool need_kidx, bool fp8) {
  MSA_REQUIRE(c != nullptr, MSA_ERR_INVALID_ARG, "cache is NULL");
  MSA_REQUIRE(!need_kv || (c->k_cache != nullptr && c->v_cache != nullptr),
              MSA_ERR_INVALID_ARG, "k_cache / v_cache is NULL");
  MSA_REQUIRE(!need_kidx || c->k_idx_cache != nullptr, MSA_ERR_INVALID_ARG,
              "k_idx_cache is NULL");
  MSA_REQUIRE(!fp8 || !need_kv || (c->k_scale != nullptr && c->v_scale != nullptr),
              MSA_ERR_INVALID_ARG, "FP8 caches: k_scale / v_scale is NULL");
  MSA_REQUIRE(!fp8 || !need_kidx || c->k_idx_scale != nullptr, MSA_ERR_INVALID_ARG,
              "FP8 caches: k_idx_scale is NULL");
  MSA_REQUIRE(c->block_table != nullptr && c->seq_lens != nullptr, MSA_ERR_INVALID_ARG,
              "block_table / seq_lens is NULL");
  MSA_REQUIRE(c->num_phys_blocks > 0 && c->max_blocks_per_seq > 0 && c->num_seqs > 0,
              MSA_ERR_INVALID_ARG, "cache sizes must be positive");
  return ok();
}

msa_status_t check_batch(const msa_batch_t *b) {
  MSA_REQUIRE(b != nullptr, MSA_ERR_INVALID_ARG, "batch is NULL");
  MSA_REQUIRE(b->total_units >= 0 && b->total_q >= 0, MSA_ERR_INVALID_ARG,
              "batch sizes must be non-negative");
  MSA_REQUIRE(b->total_units == 0 || b->units != nullptr, MSA_ERR_INVALID_ARG,
              "batch units is NULL");
  return ok();
}

float resolve_scale(float s, int D) { return s > 0.f ? s : 1.0f / std::sqrt(float(D)); }


// Bit-level NaN test: the library is built with -fno-honor-nans, under which
// `x != x` may be folded away.
bool is_nan_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof(u));
  return (u & 0x7fffffffu) > 0x7f800000u;
}

// Neither NaN nor +-inf, by the bits (see is_nan_bits).
bool finite_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof(u));
  return (u & 0x7f800000u) != 0x7f800000u;
}

constexpr int kMaxTokensPerSeq = 8;

msa_status_t check_tokens(int T, const msa::Geom &g) {
  MSA_REQUIRE(T >= 1 && T <= kMaxTokensPerSeq, MSA_ERR_UNSUPPORTED,
              "tokens_per_seq %d unsupported (1 .. %d)", T, kMaxTokensPerSeq);
  MSA_REQUIRE(T * g.nsel <= 128, MSA_ERR_UNSUPPORTED,
              "tokens_per_seq * num_sel_groups (%d) exceeds 128", T * g.nsel);
  return MSA_OK;
}

// Decode indexer for T tokens per sequence (validated arguments).
msa_status_t index_decode(const msa_geom_t *geom, const msa_cache_t *cache, int T,
                          const void *q_idx, float *scores, void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, false, true, g.fp8)) != MSA_OK) return st;
  if ((st = check_tokens(T, g)) != MSA_OK) return st;
  MSA_REQUIRE(q_idx != nullptr && scores != nullptr, MSA_ERR_INVALID_ARG,
              "q_idx / scores is NULL");
  return hip_status(msa::launch_index_decode(g, *cache, T, q_idx, scores,
                                             static_cast<hipStream_t>(stream)),
                    "index_decode");
}

// Split-KV decode attention for T tokens per sequence.
// With static_scratch the split partials go to the library's static array instead
// of the caller's workspace.
msa_status_t attn_decode(const msa_geom_t *geom, const msa_cache_t *cache, int T, const void *q,
                         const int32_t *ids, int32_t topk, float softmax_scale,
                         int32_t num_splits, void *workspace, size_t workspace_bytes,
                         bool static_scratch, void *out, float *lse, void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, true, false, g.fp8)) != MSA_OK) return st;
  if ((st = check_tokens(T, g)) != MSA_OK) return st;
  MSA_REQUIRE(q != nullptr && ids != nullptr && out != nullptr, MSA_ERR_INVALID_ARG,
              "q / ids / out is NULL");
  MSA_REQUIRE(topk >= 1, MSA_ERR_INVALID_ARG, "topk must be positive");
  MSA_REQUIRE(finite_bits(softmax_scale), MSA_ERR_INVALID_ARG,
              "softmax_scale must be finite (<= 0 selects 1/sqrt(head_dim))");
  const int rows = cache->num_seqs * T;
  const int s = num_splits > 0 ? (num_splits < topk ? num_splits : topk)
                               : msa::decode_auto_splits(g, rows, topk);
  if (g.bf16 && static_scratch) {
    const size_t need = msa::decode_workspace_bytes(g, rows, s);
    MSA_REQUIRE(need <= MSA_STATIC_SCRATCH_BYTES, MSA_ERR_WORKSPACE_TOO_SMALL,
                "static scratch: %zu bytes needed, the limit is %zu (fewer sequences or "
                "splits, or msa_sparse_attn_decode with a workspace)",
                need, static_cast<size_t>(MSA_STATIC_SCRATCH_BYTES));
    hipError_t e = msa::static_decode_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, "static scratch address");
  } else if (g.bf16) {
    const size_t need = msa::decode_workspace_bytes(g, rows, s);
    MSA_REQUIRE(workspace != nullptr, MSA_ERR_INVALID_ARG, "workspace is NULL");
    MSA_REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 256 == 0, MSA_ERR_INVALID_ARG,
                "workspace must be 256-byte aligned");
    MSA_REQUIRE(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace %zu bytes < %zu needed", workspace_bytes, need);
  }
  return hip_status(msa::launch_attn_decode(g, *cache, T, q, ids, topk,
                                            resolve_scale(softmax_scale, g.D), s, workspace,
                                            out, lse, static_cast<hipStream_t>(stream)),
                    "sparse_attn_decode");
}

}  // namespace

extern "C" {

msa_status_t msa_prefill_plan(const int32_t *h_seq_lens, const int32_t *h_q_lens,
                              int32_t num_seqs, msa_unit_t *h_units, int32_t capacity,
                              int32_t *h_num_units) {
  MSA_REQUIRE(h_seq_lens != nullptr && h_q_lens != nullptr && h_num_units != nullptr,
              MSA_ERR_INVALID_ARG, "plan: NULL argument");
  MSA_REQUIRE(num_seqs > 0, MSA_ERR_INVALID_ARG, "plan: num_seqs must be positive");
  int64_t count = 0, total_q = 0;
  for (int r = 0; r < num_seqs; ++r) {
    const int L = h_seq_lens[r], n = h_q_lens[r];
    MSA_REQUIRE(L > 0 && n >= 0 && n <= L, MSA_ERR_INVALID_ARG,
                "plan: request %d has seq_len %d and q_len %d", r, L, n);
    if (n > 0) count += (L - 1) / MSA_BLOCK_SIZE - (L - n) / MSA_BLOCK_SIZE + 1;
    total_q += n;
  }
  MSA_REQUIRE(count <= 2147483647, MSA_ERR_INVALID_ARG, "plan: too many units");
  // unit rows are int32 offsets into the batch's query rows
  MSA_REQUIRE(total_q <= 2147483647, MSA_ERR_INVALID_ARG,
              "plan: %lld query rows in all, more than an int32 row index holds",
              static_cast<long long>(total_q));
  if (h_units != nullptr) {
    MSA_REQUIRE(capacity >= count, MSA_ERR_INVALID_ARG,
                "plan: capacity %d < %lld units", capacity, static_cast<long long>(count));
    int64_t u = 0, row = 0;
    for (int r = 0; r < num_seqs; ++r) {
      const int L = h_seq_lens[r], n = h_q_lens[r], first = L - n;
      for (int p = first; p < L;) {
        const int tau = p / MSA_BLOCK_SIZE;
        const int end = (tau + 1) * MSA_BLOCK_SIZE < L ? (tau + 1) * MSA_BLOCK_SIZE : L;
        h_units[u++] = msa_unit_t{r, tau, static_cast<int32_t>(row + (p - first)), end - p, p};
        p = end;
      }
      row += n;
    }
  }
  *h_num_units = static_cast<int32_t>(count);
  return ok();
}

msa_status_t msa_validate_block_table(const int32_t *h_block_table, const int32_t *h_seq_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_phys_blocks) {
  MSA_REQUIRE(h_block_table != nullptr && h_seq_lens != nullptr, MSA_ERR_INVALID_ARG,
              "validate: NULL argument");
  MSA_REQUIRE(num_seqs > 0 && max_blocks_per_seq > 0 && num_phys_blocks > 0,
              MSA_ERR_INVALID_ARG, "validate: sizes must be positive");
  for (int r = 0; r < num_seqs; ++r) {
    const int L = h_seq_lens[r];
    MSA_REQUIRE(L > 0 && (static_cast<int64_t>(L) + MSA_BLOCK_SIZE - 1) / MSA_BLOCK_SIZE <=
                             max_blocks_per_seq,
                MSA_ERR_INVALID_ARG, "validate: sequence %d has %d tokens, more than %d blocks",
                r, L, max_blocks_per_seq);
    const int nb = (L + MSA_BLOCK_SIZE - 1) / MSA_BLOCK_SIZE;
    const int32_t *row = h_block_table + static_cast<size_t>(r) * max_blocks_per_seq;
    for (int b = 0; b < nb; ++b)
      MSA_REQUIRE(row[b] >= 0 && row[b] < num_phys_blocks, MSA_ERR_INVALID_ARG,
                  "validate: block_table[%d][%d] = %d is not a physical block (0 .. %lld)", r, b,
                  row[b], static_cast<long long>(num_phys_blocks - 1));
  }
  return ok();
}

msa_status_t msa_validate_ids(const int32_t *h_ids, int32_t num_rows, int32_t num_sel_groups,
                              int32_t topk, int32_t max_blocks_per_seq) {
  MSA_REQUIRE(h_ids != nullptr || num_rows == 0, MSA_ERR_INVALID_ARG, "validate: ids is NULL");
  MSA_REQUIRE(num_rows >= 0 && num_sel_groups > 0 && topk > 0 && max_blocks_per_seq > 0,
              MSA_ERR_INVALID_ARG, "validate: bad sizes");
  std::vector<int32_t> seen;
  for (int64_t l = 0; l < static_cast<int64_t>(num_rows) * num_sel_groups; ++l) {
    const int32_t *row = h_ids + l * topk;
    seen.clear();
    for (int i = 0; i < topk && row[i] != -1; ++i) {
      MSA_REQUIRE(row[i] >= 0 && row[i] < max_blocks_per_seq, MSA_ERR_INVALID_ARG,
                  "validate: row %lld group %lld entry %d is %d, outside 0 .. %d (end a list "
                  "with -1)", static_cast<long long>(l / num_sel_groups),
                  static_cast<long long>(l % num_sel_groups), i, row[i],
                  max_blocks_per_seq - 1);
      seen.push_back(row[i]);
    }
    std::sort(seen.begin(), seen.end());
    MSA_REQUIRE(std::adjacent_find(seen.begin(), seen.end()) == seen.end(), MSA_ERR_INVALID_ARG,
                "validate: row %lld group %lld lists a block twice",
                static_cast<long long>(l / num_sel_groups),
                static_cast<long long>(l % num_sel_groups));
  }
  return ok();
}

msa_status_t msa_index_scores(const msa_geom_t *geom, const msa_cache_t *cache,
                              const msa_batch_t *batch, const void *q_idx, float *scores,
                              void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, false, true, g.fp8)) != MSA_OK) return st;
  if (batch != nullptr) {
    if ((st = check_batch(batch)) != MSA_OK) return st;
    if (batch->total_units == 0) return ok();   // nothing to score
  }
  if (batch == nullptr) return index_decode(geom, cache, 1, q_idx, scores, stream);
  MSA_REQUIRE(q_idx != nullptr && scores != nullptr, MSA_ERR_INVALID_ARG,
              "q_idx / scores is NULL");
  return hip_status(msa::launch_index_prefill(g, *cache, *batch, q_idx, scores,
                                              static_cast<hipStream_t>(stream)),
                    "index_prefill");
}

msa_status_t msa_select_topk_blocks(const float *scores, int32_t num_rows, int32_t row_len,
                                    int32_t topk, int32_t *ids, void *stream) {
  MSA_REQUIRE(num_rows >= 0, MSA_ERR_INVALID_ARG, "num_rows must be non-negative");
  MSA_REQUIRE(row_len >= 1, MSA_ERR_INVALID_ARG, "row_len must be positive");
  MSA_REQUIRE(topk >= 1, MSA_ERR_INVALID_ARG, "topk must be positive");
  if (num_rows == 0) return ok();
  MSA_REQUIRE(scores != nullptr && ids != nullptr, MSA_ERR_INVALID_ARG, "scores / ids is NULL");
  return hip_status(msa::launch_topk(scores, num_rows, row_len, topk, ids,
                                     static_cast<hipStream_t>(stream)),
                    "select_topk_blocks");
}

namespace {

msa_status_t attn_prefill(const msa_geom_t *geom, const msa_cache_t *cache,
                          const msa_batch_t *batch, const void *q, const int32_t *ids,
                          int32_t topk, float softmax_scale, bool staged, void *workspace,
                          size_t workspace_bytes, void *out, float *lse, void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, true, false, g.fp8)) != MSA_OK) return st;
  if ((st = check_batch(batch)) != MSA_OK) return st;
  MSA_REQUIRE(topk >= 1, MSA_ERR_INVALID_ARG, "topk must be positive");
  if (batch->total_units == 0) return ok();     // no queries
  MSA_REQUIRE(q != nullptr && ids != nullptr && out != nullptr, MSA_ERR_INVALID_ARG,
              "q / ids / out is NULL");
  MSA_REQUIRE(finite_bits(softmax_scale), MSA_ERR_INVALID_ARG,
              "softmax_scale must be finite (<= 0 selects 1/sqrt(head_dim))");
  void *stage = nullptr;
  if (staged) {
    const size_t need = msa::prefill_stage_bytes(g, cache->num_phys_blocks, batch->total_units,
                                                 topk);
    if (need > 0) {
      MSA_REQUIRE(workspace != nullptr, MSA_ERR_INVALID_ARG, "workspace is NULL");
      MSA_REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 256 == 0, MSA_ERR_INVALID_ARG,
                  "workspace must be 256-byte aligned");
      MSA_REQUIRE(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
                  "workspace %zu bytes < %zu needed", workspace_bytes, need);
      stage = workspace;
    }
  }
  return hip_status(msa::launch_attn_prefill(g, *cache, *batch, q, ids, topk,
                                             resolve_scale(softmax_scale, g.D), stage, out, lse,
                                             static_cast<hipStream_t>(stream)),
                    staged ? "sparse_attn_prefill_staged" : "sparse_attn_prefill");
}

}  // namespace

msa_status_t msa_sparse_attn_prefill(const msa_geom_t *geom, const msa_cache_t *cache,
                                     const msa_batch_t *batch, const void *q,
                                     const int32_t *ids, int32_t topk, float softmax_scale,
                                     void *out, float *lse, void *stream) {
  return attn_prefill(geom, cache, batch, q, ids, topk, softmax_scale, false, nullptr, 0, out,
                      lse, stream);
}

size_t msa_prefill_workspace_size(const msa_geom_t *geom, const msa_cache_t *cache,
                                  int32_t total_units, int32_t topk) {
  msa::Geom g;
  if (check_geom(geom, &g) != MSA_OK || cache == nullptr || total_units < 0 || topk <= 0)
    return 0;
  return msa::prefill_stage_bytes(g, cache->num_phys_blocks, total_units, topk);
}

msa_status_t msa_sparse_attn_prefill_staged(const msa_geom_t *geom, const msa_cache_t *cache,
                                            const msa_batch_t *batch, const void *q,
                                            const int32_t *ids, int32_t topk,
                                            float softmax_scale, void *workspace,
                                            size_t workspace_bytes, void *out, float *lse,
                                            void *stream) {
  return attn_prefill(geom, cache, batch, q, ids, topk, softmax_scale, true, workspace,
                      workspace_bytes, out, lse, stream);
}

msa_status_t msa_index_scores_prefill_tokens(const msa_geom_t *geom, const msa_cache_t *cache,
                                             const msa_batch_t *batch, const void *q_idx,
                                             float *scores, void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, false, true, g.fp8)) != MSA_OK) return st;
  if ((st = check_batch(batch)) != MSA_OK) return st;
  if (batch->total_units == 0) return ok();
  MSA_REQUIRE(q_idx != nullptr && scores != nullptr, MSA_ERR_INVALID_ARG,
              "q_idx / scores is NULL");
  return hip_status(msa::launch_index_prefill_tokens(g, *cache, *batch, q_idx, scores,
                                                     static_cast<hipStream_t>(stream)),
                    "index_scores_prefill_tokens");
}

size_t msa_prefill_tokens_workspace_size(const msa_geom_t *geom, int32_t total_units,
                                         int32_t total_q, int32_t topk) {
  msa::Geom g;
  if (check_geom(geom, &g) != MSA_OK || total_units < 0 || total_q < 0 || topk <= 0) return 0;
  return msa::tokens_workspace_bytes(g, total_units, total_q, topk);
}

msa_status_t msa_sparse_attn_prefill_tokens(const msa_geom_t *geom, const msa_cache_t *cache,
                                            const msa_batch_t *batch, const void *q,
                                            const int32_t *ids, int32_t topk,
                                            float softmax_scale, void *workspace,
                                            size_t workspace_bytes, void *out, float *lse,
                                            void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, true, false, g.fp8)) != MSA_OK) return st;
  if ((st = check_batch(batch)) != MSA_OK) return st;
  MSA_REQUIRE(topk >= 1, MSA_ERR_INVALID_ARG, "topk must be positive");
  if (batch->total_units == 0) return ok();
  MSA_REQUIRE(q != nullptr && ids != nullptr && out != nullptr, MSA_ERR_INVALID_ARG,
              "q / ids / out is NULL");
  MSA_REQUIRE(finite_bits(softmax_scale), MSA_ERR_INVALID_ARG,
              "softmax_scale must be finite (<= 0 selects 1/sqrt(head_dim))");
  MSA_REQUIRE(cache->max_blocks_per_seq <= msa::kMaxTokenBlocks, MSA_ERR_UNSUPPORTED,
              "per-token prefill attention takes at most %d blocks per sequence",
              msa::kMaxTokenBlocks);
  const size_t need = msa::tokens_workspace_bytes(g, batch->total_units, batch->total_q, topk);
  if (need > 0) {
    MSA_REQUIRE(workspace != nullptr, MSA_ERR_INVALID_ARG, "workspace is NULL");
    MSA_REQUIRE(reinterpret_cast<uintptr_t>(workspace) % 256 == 0, MSA_ERR_INVALID_ARG,
                "workspace must be 256-byte aligned");
    MSA_REQUIRE(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace %zu bytes < %zu needed", workspace_bytes, need);
  }
  return hip_status(msa::launch_attn_prefill_tokens(g, *cache, *batch, q, ids, topk,
                                                    resolve_scale(softmax_scale, g.D),
                                                    workspace, out, lse,
                                                    static_cast<hipStream_t>(stream)),
                    "sparse_attn_prefill_tokens");
}

size_t msa_decode_workspace_size(const msa_geom_t *geom, int32_t num_seqs, int32_t topk,
                                 int32_t num_splits) {
  msa::Geom g;
  if (check_geom(geom, &g) != MSA_OK || num_seqs <= 0 || topk <= 0) return 0;
  const int s = num_splits > 0 ? (num_splits < topk ? num_splits : topk)
                               : msa::decode_auto_splits(g, num_seqs, topk);
  return msa::decode_workspace_bytes(g, num_seqs, s);
}

msa_status_t msa_sparse_attn_decode(const msa_geom_t *geom, const msa_cache_t *cache,
                                    const void *q, const int32_t *ids, int32_t topk,
                                    float softmax_scale, int32_t num_splits,
                                    void *workspace, size_t workspace_bytes, void *out,
                                    float *lse, void *stream) {
  return attn_decode(geom, cache, 1, q, ids, topk, softmax_scale, num_splits, workspace,
                     workspace_bytes, false, out, lse, stream);
}

msa_status_t msa_sparse_attn_decode_static(const msa_geom_t *geom, const msa_cache_t *cache,
                                           const void *q, const int32_t *ids, int32_t topk,
                                           float softmax_scale, int32_t num_splits, void *out,
                                           float *lse, void *stream) {
  return attn_decode(geom, cache, 1, q, ids, topk, softmax_scale, num_splits, nullptr, 0, true,
                     out, lse, stream);
}

msa_status_t msa_index_scores_per_token(const msa_geom_t *geom, const msa_cache_t *cache,
                                        int32_t tokens_per_seq, const void *q_idx,
                                        float *scores, void *stream) {
  return index_decode(geom, cache, tokens_per_seq, q_idx, scores, stream);
}

msa_status_t msa_sparse_attn_decode_per_token(const msa_geom_t *geom, const msa_cache_t *cache,
                                              int32_t tokens_per_seq, const void *q,
                                              const int32_t *ids, int32_t topk,
                                              float softmax_scale, int32_t num_splits,
                                              void *workspace, size_t workspace_bytes,
                                              void *out, float *lse, void *stream) {
  return attn_decode(geom, cache, tokens_per_seq, q, ids, topk, softmax_scale, num_splits,
                     workspace, workspace_bytes, false, out, lse, stream);
}

const char *msa_status_string(msa_status_t status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char *msa_last_error(void) { return g_last_error.c_str(); }

int32_t msa_version(void) { return 2; }

msa_status_t msa_qk_norm_rope_insert(const msa_geom_t *geom, const msa_cache_t *cache,
                                     const msa_batch_t *batch, const void *q, const void *k,
                                     const void *v, const void *k_idx, const void *q_norm_w,
                                     const void *k_norm_w, float eps, float rope_theta,
                                     int32_t rotary_dim, void *q_out, void *stream) {
  msa::Geom g;
  msa_status_t st = check_geom(geom, &g);
  if (st != MSA_OK) return st;
  if ((st = check_cache(cache, true, true, g.fp8)) != MSA_OK) return st;
  if (batch != nullptr) {
    if ((st = check_batch(batch)) != MSA_OK) return st;
    if (batch->total_units == 0) return ok();
  }
  MSA_REQUIRE(q != nullptr && k != nullptr && v != nullptr && k_idx != nullptr &&
                  q_out != nullptr,
              MSA_ERR_INVALID_ARG, "q / k / v / k_idx / q_out is NULL");
  MSA_REQUIRE(q_norm_w != nullptr && k_norm_w != nullptr, MSA_ERR_INVALID_ARG,
              "q_norm_w / k_norm_w is NULL");
  MSA_REQUIRE(!is_nan_bits(eps) && eps >= 0.f && std::isfinite(eps), MSA_ERR_INVALID_ARG,
              "eps must be finite and >= 0");
  MSA_REQUIRE(!is_nan_bits(rope_theta) && rope_theta > 0.f && std::isfinite(rope_theta),
              MSA_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  const int min_rd = g.bf16 ? 16 : 8;   // two 16-byte lane chunks
  MSA_REQUIRE(rotary_dim == 0 || (rotary_dim >= min_rd && rotary_dim <= g.D &&
                                  (rotary_dim & (rotary_dim - 1)) == 0),
              MSA_ERR_UNSUPPORTED,
              "rotary_dim %d unsupported (0, or a power of two in [%d, head_dim])", rotary_dim,
              min_rd);
  return hip_status(msa::launch_qk_norm_rope_insert(g, *cache, batch, q, k, v, k_idx, q_norm_w,
                                                    k_norm_w, eps, rope_theta, rotary_dim,
                                                    q_out, static_cast<hipStream_t>(stream)),
                    "qk_norm_rope_insert");
}

}  // extern "C"
