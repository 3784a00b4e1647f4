// Sparse prefill attention (step 3 of MSA, prefill).
//
// [dd] daily.dev "MiniMax M3 ...", section "Serving options": prefill kernels for
// sparse GQA. [feat] models.inteligile.com "MiniMax-M3", table "Checked in its
// code": rows "Grouped-query attention" (query head i reads KV head i / G) and
// "Learnable attention sink" (plain softmax in fp32, no sink, no output gate);
// method list "FlashAttention" (online softmax) and "query concatenation" (the
// queries that share a KV block are stacked against it).
//
// Query t of unit u (positions pos0 .. pos0+num_rows-1, diagonal block tau),
// head i, attends to every key s of the kept blocks of its group with
// s <= pos(t). Only the diagonal block needs the causal test: every other kept
// block lies entirely before the unit's first query.
//
// bf16 path (MFMA 32x32x16, fp32 accumulate). A work-group of 8 waves owns
// (unit, KV head j, 2 query heads): 2 heads x 128 token rows = 256 query rows, one
// wave per (head, 32 rows). For each kept block the group stages K as [key][d]
// and V transposed as [d][key] in LDS, then every wave computes
//   S^T = K . Q^T           (A = K from LDS, B = its Q rows held in registers)
//   O^T += V^T . P^T        (A = V^T from LDS, B = P taken straight from S^T)
// Computing the transposed products keeps each query in one lane pair, so the
// online-softmax row statistics need a single cross-lane exchange, and lets the
// probabilities feed the second product without an LDS round trip. For that the
// accumulator's key order inside each 16-key group (lane half a, register
// 8h+jj holds key 16h + 8(jj/4) + 4a + jj%4) is mirrored by storing V^T with
// keys 4-7 and 8-11 of every 16-key group swapped.
//
// fp32 path: plain FMA, one thread per (query, head); for small exact checks.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPrefThreads = 512;

// Position of key k (0..127) in the swapped order used for V^T rows.
__device__ __forceinline__ int vt_pos(int k) {
  const int grp = (k >> 2) & 3;                    // 4-key group inside 16
  const int sw = (grp == 1) ? 2 : (grp == 2) ? 1 : grp;
  return (k & ~15) | (sw << 2) | (k & 3);
}

template <int D>
__global__ __launch_bounds__(kPrefThreads) void attn_prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, float scale_log2,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int KS = D / 16;        // k steps of S^T = K Q^T
  constexpr int DT = D / 32;        // d tiles of O^T
  constexpr int KROW = D + 8;       // padded LDS row (elements) of K
  constexpr int VROW = kBlk + 8;    // padded LDS row (elements) of V^T
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlk * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VROW];

  const int G = Hq / Hkv;
  const int pairs = (G + 1) / 2;
  const int u = blockIdx.x;
  const int j = blockIdx.y / pairs, hp = blockIdx.y % pairs;
  const msa_unit_t un = units[u];
  const int g = (nsel == Hkv) ? j : 0;
  const int32_t *sel = ids + (static_cast<size_t>(u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int hl = 2 * hp + wave / 4;                // head inside the group
  const int slab = wave % 4;                       // 32-row slab of the tile
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + (lane % 32);
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  // B operand of S^T: this lane's query row, 8 d at (l/32)*8 of each k step
  bf16x8 qb[KS];
  {
    const uint16_t *qp = q + (static_cast<size_t>(qrow) * Hq + head) * D + (lane / 32) * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(qp + ks * 16));
  }

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -1e30f;   // running max (log2 domain); finite so alpha is never NaN
  float l_run = 0.f;      // this lane's share of the row sum

  for (int slot = 0; slot < topk; ++slot) {
    const int b = sel[slot];
    if (b < 0) break;                              // ids ascending, -1 at the tail
    const int64_t phys = bt[b];
    const size_t head_off = (static_cast<size_t>(phys) * Hkv + j) * kBlk * D;
    __syncthreads();                               // previous block fully consumed
    // stage K: [key][d], 16-byte chunks
    for (int c = t; c < kBlk * D / 8; c += kPrefThreads) {
      const int key = c / (D / 8), dc = c % (D / 8);
      *reinterpret_cast<uint4 *>(&Ks[key * KROW + dc * 8]) =
          *reinterpret_cast<const uint4 *>(kc + head_off + key * D + dc * 8);
    }
    // stage V^T: a thread takes 4 consecutive keys x 8 d and writes 8 rows of 4 keys
    for (int c = t; c < (kBlk / 4) * (D / 8); c += kPrefThreads) {
      const int ka = c % (kBlk / 4), dc = c / (kBlk / 4);
      uint4 vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vv[i] = *reinterpret_cast<const uint4 *>(vc + head_off + (ka * 4 + i) * D + dc * 8);
      const int p = vt_pos(ka * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e / 2, sh = (e % 2) * 16;
        auto pick = [&](const uint4 &x) -> uint32_t {
          const uint32_t word = (w == 0) ? x.x : (w == 1) ? x.y : (w == 2) ? x.z : x.w;
          return (word >> sh) & 0xffffu;
        };
        uint2 pk;
        pk.x = pick(vv[0]) | (pick(vv[1]) << 16);
        pk.y = pick(vv[2]) | (pick(vv[3]) << 16);
        *reinterpret_cast<uint2 *>(&Vt[(dc * 8 + e) * VROW + p]) = pk;
      }
    }
    __syncthreads();
    if (!active) continue;

    // S^T tiles: 4 x (32 keys x 32 queries)
    f32x16 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x16{};
      const uint16_t *kr = &Ks[(kt * 32 + lane % 32) * KROW + (lane / 32) * 8];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4 *>(kr + ks * 16));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s[kt], 0, 0, 0);
      }
    }
    // scale, causal mask on the diagonal block, row max
    const bool diag = (b == un.tau);
    float mx = -1e30f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
        float x = s[kt][i] * scale_log2;
        if (diag && b * kBlk + key > qpos) x = neg_inf();
        s[kt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[8];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          const float p0 = exp2f(s[kt][8 * h + jj] - m_new);
          const float p1 = exp2f(s[kt][8 * h + jj + 1] - m_new);
          psum += p0 + p1;
          w[jj / 2] = pack_bf16x2(p0, p1);
        }
        pb[kt * 2 + h] = as_bf16x8(uint4{w[0], w[1], w[2], w[3]});
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] *= alpha;
      const uint16_t *vr = &Vt[(dt * 32 + lane % 32) * VROW + (lane / 32) * 8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4 *>(vr + ks * 16));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], o[dt], 0, 0, 0);
      }
    }
  }
  if (!active || !row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.f / l_tot;
  uint16_t *op = out + (static_cast<size_t>(qrow) * Hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = dt * 32 + i4 * 8 + (lane / 32) * 4;
      uint2 pk;
      pk.x = pack_bf16x2(o[dt][i4 * 4 + 0] * inv, o[dt][i4 * 4 + 1] * inv);
      pk.y = pack_bf16x2(o[dt][i4 * 4 + 2] * inv, o[dt][i4 * 4 + 3] * inv);
      *reinterpret_cast<uint2 *>(op + d) = pk;
    }
  if (lse != nullptr && lane < 32)
    lse[static_cast<size_t>(qrow) * Hq + head] = (m_run + log2f(l_tot)) * kLn2;
}

}  // namespace

// fp32 attention, shared by prefill (units from the plan) and decode (one query
// per sequence at position seq_len - 1). One thread per (query row, head).
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, float scale, float *__restrict__ out,
    float *__restrict__ lse) {
  const int u = blockIdx.x, head = blockIdx.y;
  msa_unit_t un;
  if (units != nullptr) {
    un = units[u];
  } else {
    const int L = seq_lens[u];
    un = msa_unit_t{u, (L - 1) / kBlk, u, 1, L - 1};
  }
  const int t = threadIdx.x;
  if (t >= un.num_rows) return;
  const int G = Hq / Hkv, j = head / G;
  const int g = (nsel == Hkv) ? j : 0;
  const int32_t *sel = ids + (static_cast<size_t>(u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  const int qrow = un.row0 + t, qpos = un.pos0 + t;
  float qv[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = q[(static_cast<size_t>(qrow) * Hq + head) * D + d];
    acc[d] = 0.f;
  }
  float m = neg_inf(), l = 0.f;
  for (int slot = 0; slot < topk; ++slot) {
    const int b = sel[slot];
    if (b < 0) break;
    const int64_t phys = bt[b];
    const float *kb = kc + (static_cast<size_t>(phys) * Hkv + j) * kBlk * D;
    const float *vb = vc + (static_cast<size_t>(phys) * Hkv + j) * kBlk * D;
    for (int key = 0; key < kBlk; ++key) {
      if (b * kBlk + key > qpos) break;
      float x = 0.f;
      for (int d = 0; d < D; ++d) x = fmaf(qv[d], kb[key * D + d], x);
      x *= scale;
      const float m_new = fmaxf(m, x);
      const float alpha = expf(m - m_new);
      const float p = expf(x - m_new);
      l = l * alpha + p;
      for (int d = 0; d < D; ++d) acc[d] = acc[d] * alpha + p * vb[key * D + d];
      m = m_new;
    }
  }
  float *op = out + (static_cast<size_t>(qrow) * Hq + head) * D;
  for (int d = 0; d < D; ++d) op[d] = acc[d] / l;
  if (lse != nullptr) lse[static_cast<size_t>(qrow) * Hq + head] = m + logf(l);
}

hipError_t launch_attn_f32(const Geom &g, const msa_cache_t &c, const msa_unit_t *units,
                           int num_units, const void *q, const int32_t *ids, int topk,
                           float scale, void *out, float *lse, hipStream_t st) {
  const dim3 grid(num_units, g.Hq);
  const float *qf = static_cast<const float *>(q);
  const float *kf = static_cast<const float *>(c.k_cache);
  const float *vf = static_cast<const float *>(c.v_cache);
  if (g.D == 64)
    attn_f32_kernel<64><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                              ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                              g.nsel, scale, static_cast<float *>(out), lse);
  else
    attn_f32_kernel<128><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                               ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                               g.nsel, scale, static_cast<float *>(out), lse);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                               const void *q, const int32_t *ids, int topk, float scale,
                               void *out, float *lse, hipStream_t st) {
  if (b.total_units == 0) return hipSuccess;
  if (!g.bf16)
    return launch_attn_f32(g, c, b.units, b.total_units, q, ids, topk, scale, out, lse, st);
  const int pairs = (g.G() + 1) / 2;
  const dim3 grid(b.total_units, g.Hkv * pairs);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const uint16_t *kb = static_cast<const uint16_t *>(c.k_cache);
  const uint16_t *vb = static_cast<const uint16_t *>(c.v_cache);
  uint16_t *ob = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  if (g.D == 64)
    attn_prefill_bf16_kernel<64><<<grid, kPrefThreads, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, sl2, ob, lse);
  else
    attn_prefill_bf16_kernel<128><<<grid, kPrefThreads, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, sl2, ob, lse);
  return hipGetLastError();
}

}  // namespace msa
