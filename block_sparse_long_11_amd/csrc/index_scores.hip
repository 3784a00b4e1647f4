// Indexer block scores (step 1 of MSA).
//
// [feat] models.inteligile.com "MiniMax-M3", table "Checked in its code", row
// "Indexer-selected sparse attention": a lightning indexer scores keys per head
// and pools the scores into blocks. [vllm] 24-ai.news "MiniMax M3 in vLLM",
// section "Warum ist ein Million-Token-Kontext eine Serving-Herausforderung?":
// each query or GQA query group scores all available blocks with light indexer
// kernels.
//
// Score of block b < tau for unit u and selection group g:
//   max over the unit's queries t and the block's keys s of
//   sum_{h in g} q_idx[t,h,:] . k_idx[s,h,:]
// b == tau (the diagonal block) is +inf, b > tau is -inf.
//
// Decode (one query per unit) is a single streaming pass over every indexer key
// of every sequence: HBM-bound, so each work-group reads one whole 128-token
// block (all indexer heads, contiguous in the block-major cache) with 16-byte
// coalesced loads and reduces with cross-lane shuffles. Prefill (128 queries per
// unit) is a dense 128 x 128 x (H_s * D_i) contraction per (tile, block) and runs
// on bf16 MFMA with a max-pool epilogue.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

// ---------------------------------------------------------------------------
// decode: one work-group of 256 threads per (sequence, logical block)
// ---------------------------------------------------------------------------

template <bool BF16, int DI, int HS>
__global__ __launch_bounds__(256) void index_decode_kernel(
    const void *__restrict__ q_idx, const void *__restrict__ k_idx,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    int max_blocks, int nsel, float *__restrict__ scores) {
  constexpr int EPV = BF16 ? 8 : 4;      // elements per 16-byte load
  constexpr int LPR = DI / EPV;          // lanes covering one token row of one head
  constexpr int ROWS = 256 / LPR;        // token rows per pass
  constexpr int PASSES = kBlk / ROWS;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ float red[4][16];

  const int Hi = nsel * HS;
  const int r = blockIdx.x / max_blocks;
  const int b = blockIdx.x - r * max_blocks;
  const int L = seq_lens[r];
  const int tau = (L - 1) / kBlk;
  float *out = scores + static_cast<size_t>(r) * nsel * max_blocks + b;
  if (b >= tau) {
    if (threadIdx.x < nsel) out[static_cast<size_t>(threadIdx.x) * max_blocks] =
        (b == tau) ? pos_inf() : neg_inf();
    return;
  }
  const int64_t phys = block_table[static_cast<size_t>(r) * max_blocks + b];
  const int t = threadIdx.x;
  const int piece = t % LPR;
  const int row = t / LPR;
  const char *kblk = static_cast<const char *>(k_idx) +
                     static_cast<size_t>(phys) * Hi * kBlk * DI * ESZ;
  const char *qrow = static_cast<const char *>(q_idx) + static_cast<size_t>(r) * Hi * DI * ESZ;
  const int wave = t / kWave, lane = t % kWave;

  for (int g = 0; g < nsel; ++g) {
    uint4 qv[HS];
#pragma unroll
    for (int hh = 0; hh < HS; ++hh)
      qv[hh] = *reinterpret_cast<const uint4 *>(qrow + ((g * HS + hh) * DI + piece * EPV) * ESZ);
    uint4 kv[PASSES][HS];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int hh = 0; hh < HS; ++hh)
        kv[p][hh] = load_stream16(
            kblk + ((static_cast<size_t>(g * HS + hh) * kBlk + p * ROWS + row) * DI +
                    piece * EPV) * ESZ);
    float m = neg_inf();
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int hh = 0; hh < HS; ++hh) {
        if constexpr (BF16) {
          acc = dot2_bf16(qv[hh].x, kv[p][hh].x, acc);
          acc = dot2_bf16(qv[hh].y, kv[p][hh].y, acc);
          acc = dot2_bf16(qv[hh].z, kv[p][hh].z, acc);
          acc = dot2_bf16(qv[hh].w, kv[p][hh].w, acc);
        } else {
          acc = fmaf(__uint_as_float(qv[hh].x), __uint_as_float(kv[p][hh].x), acc);
          acc = fmaf(__uint_as_float(qv[hh].y), __uint_as_float(kv[p][hh].y), acc);
          acc = fmaf(__uint_as_float(qv[hh].z), __uint_as_float(kv[p][hh].z), acc);
          acc = fmaf(__uint_as_float(qv[hh].w), __uint_as_float(kv[p][hh].w), acc);
        }
      }
      acc = group_sum<LPR>(acc);   // full dot product of token row p*ROWS+row
      m = fmaxf(m, acc);
    }
    m = group_max<kWave>(m);
    if (lane == 0) red[wave][g] = m;
  }
  __syncthreads();
  if (t < nsel)
    out[static_cast<size_t>(t) * max_blocks] =
        fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
}

// ---------------------------------------------------------------------------
// prefill, bf16: MFMA 32x32x16, one work-group per (unit, group, block chunk)
// ---------------------------------------------------------------------------
//
// Each of the 4 waves holds 32 query rows of the tile as the A operand
// (lane l: row l%32, 8 consecutive group-dim elements at (l/32)*8 of each
// 16-wide k step) and streams the indexer keys of the block as the B operand
// (lane l: key l%32, the same 8 elements), 4 tiles of 32 keys per block.
// The accumulator element (lane l, register i) is query row
// (i/4)*8 + (l/32)*4 + i%4 and key l%32; rows past the unit's last query are
// masked before the max.

constexpr int kChunk = 16;   // blocks per work-group

template <int DI, int HS>
__global__ __launch_bounds__(256) void index_prefill_bf16_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ block_table, const msa_unit_t *__restrict__ units,
    int max_blocks, int nsel, float *__restrict__ scores) {
  constexpr int GD = HS * DI;          // group dim
  constexpr int KS = GD / 16;          // k steps
  __shared__ float red[4][kChunk];

  const int u = blockIdx.x, g = blockIdx.z;
  const msa_unit_t un = units[u];
  const int Hi = nsel * HS;
  const int b0 = blockIdx.y * kChunk;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  float *out = scores + (static_cast<size_t>(u) * nsel + g) * max_blocks;
  if (b0 >= un.tau) {
    for (int i = t; i < kChunk && b0 + i < max_blocks; i += 256)
      out[b0 + i] = (b0 + i == un.tau) ? pos_inf() : neg_inf();
    return;
  }
  const int nblk = min(kChunk, un.tau - b0);

  // A operand: this wave's 32 query rows (clamped; masked rows are ignored)
  const int qr = wave * 32 + (lane % 32);
  const int qrow = un.row0 + min(qr, un.num_rows - 1);
  bf16x8 a[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int kk = ks * 16 + (lane / 32) * 8;
    const int h = g * HS + kk / DI, d = kk % DI;
    a[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(
        q_idx + (static_cast<size_t>(qrow) * Hi + h) * DI + d));
  }
  // rows of the accumulator held by this lane that are real queries
  bool rv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    rv[i] = (wave * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4)) < un.num_rows;

  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  for (int bi = 0; bi < nblk; ++bi) {
    const int64_t phys = bt[b0 + bi];
    const uint16_t *kb = k_idx + static_cast<size_t>(phys) * Hi * kBlk * DI;
    float m = neg_inf();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int key = nt * 32 + (lane % 32);
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kk = ks * 16 + (lane / 32) * 8;
        const int h = g * HS + kk / DI, d = kk % DI;
        const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4 *>(
            kb + (static_cast<size_t>(h) * kBlk + key) * DI + d));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) m = rv[i] ? fmaxf(m, acc[i]) : m;
    }
    m = group_max<kWave>(m);
    if (lane == 0) red[wave][bi] = m;
  }
  __syncthreads();
  if (t < nblk)
    out[b0 + t] = fmaxf(fmaxf(red[0][t], red[1][t]), fmaxf(red[2][t], red[3][t]));
  else if (t < kChunk && b0 + t < max_blocks)   // the diagonal and the future blocks
    out[b0 + t] = (b0 + t == un.tau) ? pos_inf() : neg_inf();
}

// ---------------------------------------------------------------------------
// prefill, fp32: plain FMA, one work-group of 128 threads per (unit, group, block)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(128) void index_prefill_f32_kernel(
    const float *__restrict__ q_idx, const float *__restrict__ k_idx,
    const int32_t *__restrict__ block_table, const msa_unit_t *__restrict__ units,
    int max_blocks, int nsel, int Hi, int Di, float *__restrict__ scores) {
  __shared__ float red[2];
  const int u = blockIdx.x, g = blockIdx.z, b = blockIdx.y;
  const msa_unit_t un = units[u];
  const int Hs = Hi / nsel;
  float *out = scores + (static_cast<size_t>(u) * nsel + g) * max_blocks;
  if (b >= un.tau) {
    if (threadIdx.x == 0) out[b] = (b == un.tau) ? pos_inf() : neg_inf();
    return;
  }
  const int s = threadIdx.x;   // key of the block
  const int64_t phys = block_table[static_cast<size_t>(un.r) * max_blocks + b];
  float m = neg_inf();
  for (int t = 0; t < un.num_rows; ++t) {
    float acc = 0.f;
    for (int hh = 0; hh < Hs; ++hh) {
      const int h = g * Hs + hh;
      const float *qv = q_idx + (static_cast<size_t>(un.row0 + t) * Hi + h) * Di;
      const float *kv = k_idx + ((static_cast<size_t>(phys) * Hi + h) * kBlk + s) * Di;
      for (int d = 0; d < Di; ++d) acc = fmaf(qv[d], kv[d], acc);
    }
    m = fmaxf(m, acc);
  }
  m = group_max<kWave>(m);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[b] = fmaxf(red[0], red[1]);
}

template <bool BF16, int DI>
hipError_t dispatch_decode_hs(const Geom &g, const msa_cache_t &c, const void *q_idx,
                              float *scores, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(c.num_seqs) * c.max_blocks_per_seq);
  switch (g.Hs()) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    index_decode_kernel<BF16, DI, HS><<<grid, 256, 0, st>>>(                             \
        q_idx, c.k_idx_cache, c.block_table, c.seq_lens, c.max_blocks_per_seq, g.nsel,   \
        scores);                                                                         \
    break;
    MSA_CASE(1) MSA_CASE(2) MSA_CASE(4) MSA_CASE(8)
#undef MSA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DI>
hipError_t dispatch_prefill_bf16(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                 const void *q_idx, float *scores, hipStream_t st) {
  const dim3 grid(b.total_units, (c.max_blocks_per_seq + kChunk - 1) / kChunk, g.nsel);
  const uint16_t *q = static_cast<const uint16_t *>(q_idx);
  const uint16_t *k = static_cast<const uint16_t *>(c.k_idx_cache);
  switch (g.Hs()) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    if (HS * DI > 512) return hipErrorInvalidValue;                                      \
    index_prefill_bf16_kernel<DI, HS><<<grid, 256, 0, st>>>(                             \
        q, k, c.block_table, b.units, c.max_blocks_per_seq, g.nsel, scores);             \
    break;
    MSA_CASE(1) MSA_CASE(2) MSA_CASE(4) MSA_CASE(8)
#undef MSA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_decode(const Geom &g, const msa_cache_t &c, const void *q_idx,
                               float *scores, hipStream_t st) {
  if (g.bf16) {
    return g.Di == 64 ? dispatch_decode_hs<true, 64>(g, c, q_idx, scores, st)
                      : dispatch_decode_hs<true, 32>(g, c, q_idx, scores, st);
  }
  return g.Di == 64 ? dispatch_decode_hs<false, 64>(g, c, q_idx, scores, st)
                    : dispatch_decode_hs<false, 32>(g, c, q_idx, scores, st);
}

hipError_t launch_index_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                const void *q_idx, float *scores, hipStream_t st) {
  if (b.total_units == 0) return hipSuccess;
  if (g.bf16) {
    return g.Di == 64 ? dispatch_prefill_bf16<64>(g, c, b, q_idx, scores, st)
                      : dispatch_prefill_bf16<32>(g, c, b, q_idx, scores, st);
  }
  const dim3 grid(b.total_units, c.max_blocks_per_seq, g.nsel);
  index_prefill_f32_kernel<<<grid, 128, 0, st>>>(
      static_cast<const float *>(q_idx), static_cast<const float *>(c.k_idx_cache),
      c.block_table, b.units, c.max_blocks_per_seq, g.nsel, g.Hi, g.Di, scores);
  return hipGetLastError();
}

}  // namespace msa
