// Internal launchers of the MSA kernels. The C-ABI entry points in msa_api.hip
// validate their arguments and then call these; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Debugging aid: with MSA_LOG set to a non-zero value in the environment, every
// kernel launch prints its kernel, grid, block and dynamic LDS bytes to stderr,
// and every refused call its reason. Off by default; the variable is read at every
// launch, so a process can switch it on and off.
bool log_enabled();
void log_launch(const char *kernel, dim3 grid, dim3 block, size_t lds);
#define MSA_LOG_LAUNCH(kernel, grid, block, lds)                                      \
  do {                                                                               \
    if (::msa::log_enabled()) ::msa::log_launch(kernel, dim3(grid), dim3(block), lds); \
  } while (0)

struct Geom {
  int Hq, Hkv, D, Hi, Di, nsel;
  bool bf16;
  bool fp8;   // FP8 E4M3 caches with power-of-two scales per 32 channels
  int G() const { return Hq / Hkv; }
  int Hs() const { return Hi / nsel; }
};

// Decode with T new tokens per sequence (T = 1: one), each selecting its own blocks.
hipError_t launch_index_decode(const Geom &g, const msa_cache_t &c, int T, const void *q_idx,
                               float *scores, hipStream_t st);
hipError_t launch_index_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                const void *q_idx, float *scores, hipStream_t st);
// Per-query-token scores of a prefill batch: scores [total_q][n_sel][max_blocks].
hipError_t launch_index_prefill_tokens(const Geom &g, const msa_cache_t &c,
                                       const msa_batch_t &b, const void *q_idx, float *scores,
                                       hipStream_t st);
hipError_t launch_topk(const float *scores, int rows, int row_len, int topk, int32_t *ids,
                       hipStream_t st);
// stage_ws (FP8 caches; NULL: convert in the attention kernel) holds
// prefill_stage_bytes: bf16 copies of the kept blocks, converted once each.
hipError_t launch_attn_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                               const void *q, const int32_t *ids, int topk, float scale,
                               void *stage_ws, void *out, float *lse, hipStream_t st);
size_t prefill_stage_bytes(const Geom &g, int64_t num_phys, int total_units, int topk);
// Per-query-token prefill attention: ids [total_q][n_sel][topk]; workspace of
// tokens_workspace_bytes (bf16: per (unit, group) the union of its rows' lists and
// the row masks; fp32 needs none).
size_t tokens_workspace_bytes(const Geom &g, int total_units, int total_q, int topk);
hipError_t launch_attn_prefill_tokens(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                      const void *q, const int32_t *ids, int topk, float scale,
                                      void *workspace, void *out, float *lse, hipStream_t st);
// Largest block table width the per-token prefill attention takes (its union bitmap
// lives in LDS).
constexpr int kMaxTokenBlocks = 131072;
// Split count used when the caller passes num_splits <= 0.
int decode_auto_splits(const Geom &g, int num_seqs, int topk);
size_t decode_workspace_bytes(const Geom &g, int num_seqs, int num_splits);
hipError_t launch_attn_decode(const Geom &g, const msa_cache_t &c, int T, const void *q,
                              const int32_t *ids, int topk, float scale, int num_splits,
                              void *workspace, void *out, float *lse, hipStream_t st);
// Device address of this GPU's static scratch (MSA_STATIC_SCRATCH_BYTES), the
// workspace of msa_sparse_attn_decode_static; resolved on the first call per device.
hipError_t static_decode_scratch(void **ptr);

hipError_t launch_qk_norm_rope_insert(const Geom &g, const msa_cache_t &c, const msa_batch_t *b,
                                      const void *q, const void *k, const void *v,
                                      const void *k_idx, const void *q_norm_w,
                                      const void *k_norm_w, float eps, float theta, int rd,
                                      void *q_out, hipStream_t st);

}  // namespace msa
