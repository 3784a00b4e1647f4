// Internal launchers of the MSA kernels. The C-ABI entry points in msa_api.hip
// validate their arguments and then call these; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

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
hipError_t launch_topk(const float *scores, int rows, int row_len, int topk, int32_t *ids,
                       hipStream_t st);
hipError_t launch_attn_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                               const void *q, const int32_t *ids, int topk, float scale,
                               void *out, float *lse, hipStream_t st);
// Split count used when the caller passes num_splits <= 0.
int decode_auto_splits(const Geom &g, int num_seqs, int topk);
size_t decode_workspace_bytes(const Geom &g, int num_seqs, int num_splits);
hipError_t launch_attn_decode(const Geom &g, const msa_cache_t &c, int T, const void *q,
                              const int32_t *ids, int topk, float scale, int num_splits,
                              void *workspace, void *out, float *lse, hipStream_t st);

hipError_t launch_qk_norm_rope_insert(const Geom &g, const msa_cache_t &c, const msa_batch_t *b,
                                      const void *q, const void *k, const void *v,
                                      const void *k_idx, const void *q_norm_w,
                                      const void *k_norm_w, float eps, float theta, int rd,
                                      void *q_out, hipStream_t st);

}  // namespace msa
