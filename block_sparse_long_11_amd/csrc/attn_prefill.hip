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
// bf16 path (MFMA 32x32x16, fp32 accumulate). A work-group of 8 waves (two per
// SIMD, so one wave's softmax arithmetic overlaps the other's MFMAs) owns (unit,
// KV head j, 2 query heads): 128 token rows x 2 heads, one wave per (head, 32
// tokens). Per kept block the group stages K ([key][d]) and V ([d][key], the
// cache's d-major blocks) in LDS by direct global->LDS loads, 16-byte chunks
// XOR-swizzled by row, into one of two buffers while the other is being read.
// Per 32-key tile each wave computes
//   S^T = K . Q^T           (A = K rows from LDS, B = Q held in registers)
//   O^T += V^T . P^T        (A = V^T rows from LDS, B = P from S^T's registers)
// The S^T row m of a tile is fed key (m with bits 2 and 3 swapped): then lane
// half a, register 8h+jj holds key 16h + 8a + jj, which is exactly the k-index
// the P^T operand needs, so V^T is read in natural key order.
// Online softmax in log2 units with a lazy reference maximum: O and the row sum
// are rescaled only when a row's maximum grows by more than 8 (probabilities
// stay <= 2^8); the result is exact after the final division by the row sum.
//
// fp32 path: plain FMA, one thread per (query, head); for small exact checks.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// 8 waves of 32 query rows (two per SIMD): measured faster on MI355X than 4 waves
// (one per SIMD), with or without two 32-row tiles per wave.
constexpr int kPrefWaves = 8;
constexpr float kSlack = 8.f;

// S^T tile row m (0..31) -> key inside the 32-key tile: swap bits 2 and 3.
__device__ __forceinline__ int srow_key(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, bf16x2));
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vtc, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int num_uj, int pairs, float c,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int KS = D / 16;              // 16-wide d steps of S^T
  constexpr int DT = D / 32;              // 32-row d tiles of O^T
  constexpr int CH = D / 8;               // 16-byte chunks per K row
  constexpr int NT = NW * kWave;          // threads
  constexpr int HPW = NW / 4;             // query heads per work-group
  constexpr int KCH = kBlk * CH / NT;
  constexpr int VCH = D * 16 / NT;
  // Two LDS buffers per operand, filled by direct global->LDS loads while the
  // other one is being read. K: chunk c of row r at c ^ kswz(r), keyed on the
  // lane that reads row r; V^T: chunk c of row d at c ^ (d % 16).
  auto kswz = [](int r) { return srow_key(r % 32) % CH; };
  __shared__ u32x4 Ks0[kBlk * CH], Ks1[kBlk * CH];
  __shared__ u32x4 Vs0[D * 16], Vs1[D * 16];

  // XCD-aware order: the `pairs` work-groups of one (unit, KV head) get ids that
  // are equal mod 8 (same XCD, same L2) and adjacent in that XCD's dispatch order;
  // (unit, KV head) pairs are taken from the last unit down (most blocks first).
  const int id = blockIdx.x;
  const int uj_rev = 8 * (id / (8 * pairs)) + id % 8;
  const int hp = (id / 8) % pairs;
  if (uj_rev >= num_uj) return;
  const int uj = num_uj - 1 - uj_rev;
  const int u = uj / Hkv, j = uj % Hkv;
  const msa_unit_t un = units[u];
  const int G = Hq / Hkv;
  const int g = (nsel == Hkv) ? j : 0;
  const int32_t *sel = ids + (static_cast<size_t>(u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int a = lane / 32, n = lane % 32;
  const int hl = HPW * hp + wave / 4;     // head inside the group
  const int slab = wave % 4;              // 32-token slab of the tile
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + n;
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  bf16x8 qf[KS];
  {
    const uint16_t *pq = q + (static_cast<size_t>(qrow) * Hq + head) * D + a * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(pq + ks * 16));
  }

  // Enqueue the direct loads of block b into (Kd, Vd). Instruction i of wave w
  // fills LDS chunks (NW i + w) * 64 + lane; each lane fetches the global chunk
  // that the swizzle places there.
  auto issue = [&](int b, u32x4 *Kd, u32x4 *Vd) __attribute__((always_inline)) {
    const size_t off = (static_cast<size_t>(bt[b]) * Hkv + j) * kBlk * D;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int base = (NW * i + wave) * 64;
      const int p = base + lane, r = p / CH, ch = (p % CH) ^ kswz(r);
      __builtin_amdgcn_global_load_lds(
          kc + off + r * D + ch * 8,
          (__attribute__((address_space(3))) void *)(Kd + base), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int base = (NW * i + wave) * 64;
      const int p = base + lane, r = p / 16, ch = (p % 16) ^ (r % 16);
      __builtin_amdgcn_global_load_lds(
          vtc + off + r * kBlk + ch * 8,
          (__attribute__((address_space(3))) void *)(Vd + base), 16, 0, 0);
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_ref = neg_inf();                // reference maximum, log2 units
  float l_run = 0.f;                      // this lane's share of the row sum

  // Per 32-key tile: the 8 K fragments and the 8 V^T fragments are read from LDS
  // into registers first (batched reads, one wait), then S^T = K Q^T, the online
  // softmax and O^T += V^T P^T.
  // MASK is true only for the diagonal block: it gets its own copy of the code so
  // that the other blocks carry no masking work.
  auto compute = [&](auto mask_tag, int b, const u32x4 *Kb, const u32x4 *Vb)
                     __attribute__((always_inline)) {
    constexpr bool diag = decltype(mask_tag)::value;
    const int lim = qpos - b * kBlk;      // keys with offset > lim are masked
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int krow = kt * 32 + srow_key(n);
      const int sw = kswz(krow);          // = n % CH: 8 consecutive lanes hit 8 chunks
      bf16x8 kf[KS], vf[2 * DT];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = __builtin_bit_cast(bf16x8, Kb[krow * CH + ((2 * ks + a) ^ sw)]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int d = dt * 32 + n, ch = 4 * kt + 2 * h + a;
          vf[2 * dt + h] = __builtin_bit_cast(bf16x8, Vb[d * 16 + (ch ^ (d % 16))]);
        }
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
      if constexpr (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt * 32 + 16 * (i / 8) + 8 * a + (i % 8);
          if (key > lim) s[i] = neg_inf();
        }
      }
      float x = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) x = fmaxf(fmaxf(x, s[i]), s[i + 1]);
      x = fmaxf(x, s[15]);
      {   // max with the other half of the wave (same query column)
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                          __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * c;
      }
      const bool need = x > m_ref + kSlack;
      if (__any(need)) {
        const float nm = need ? x : m_ref;
        const float al = __builtin_amdgcn_exp2f(m_ref - nm);
        m_ref = nm;
        l_run *= al;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= al;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + jj], c, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + jj + 1], c, -m_ref));
          w[jj / 2] = cvt_pk_bf16(p0, p1);
          l_run += p0 + p1;
        }
        pf[h] = as_bf16x8(uint4{w[0], w[1], w[2], w[3]});
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * dt + h], pf[h], o[dt], 0, 0, 0);
    }
  };

  // The diagonal block (the last kept id) is attended first, from buffer 0, with
  // the causal mask; the other kept blocks then alternate between the buffers.
  // At the top of each step only that block's loads are outstanding; after the
  // barrier every wave has finished with the other buffer, which then receives
  // the next block. The softmax is order-independent, so the order is free.
  int nk = 0;
  while (nk < topk && sel[nk] >= 0) ++nk;
  const std::true_type masked{};
  const std::false_type plain{};
  issue(sel[nk - 1], Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0)
  __syncthreads();
  if (nk > 1) issue(sel[0], Ks1, Vs1);
  if (active) compute(masked, sel[nk - 1], Ks0, Vs0);
  for (int slot = 0; slot + 1 < nk;) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (slot + 2 < nk) issue(sel[slot + 1], Ks0, Vs0);
    if (active) compute(plain, sel[slot], Ks1, Vs1);
    if (++slot + 1 >= nk) break;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (slot + 2 < nk) issue(sel[slot + 1], Ks1, Vs1);
    if (active) compute(plain, sel[slot], Ks0, Vs0);
    ++slot;
  }
  if (!active) return;
  float sum;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!row_ok) return;
  const float inv = 1.f / sum;
  uint16_t *op = out + (static_cast<size_t>(qrow) * Hq + head) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = dt * 32 + i4 * 8 + a * 4;
      uint2 w;
      w.x = cvt_pk_bf16(o[dt][i4 * 4 + 0] * inv, o[dt][i4 * 4 + 1] * inv);
      w.y = cvt_pk_bf16(o[dt][i4 * 4 + 2] * inv, o[dt][i4 * 4 + 3] * inv);
      *reinterpret_cast<uint2 *>(op + d) = w;
    }
  if (lse != nullptr && a == 0)
    lse[static_cast<size_t>(qrow) * Hq + head] = (m_ref + __builtin_log2f(sum)) * kLn2;
}

}  // namespace

// fp32 attention, shared by prefill (units from the plan) and decode (one query
// per sequence at position seq_len - 1). One thread per (query row, head).
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vtc,
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
    const float *vb = vtc + (static_cast<size_t>(phys) * Hkv + j) * D * kBlk;
    for (int key = 0; key < kBlk; ++key) {
      if (b * kBlk + key > qpos) break;
      float x = 0.f;
      for (int d = 0; d < D; ++d) x = fmaf(qv[d], kb[key * D + d], x);
      x *= scale;
      const float m_new = fmaxf(m, x);
      const float alpha = expf(m - m_new);
      const float p = expf(x - m_new);
      l = l * alpha + p;
      for (int d = 0; d < D; ++d) acc[d] = acc[d] * alpha + p * vb[d * kBlk + key];
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
  constexpr int NW = kPrefWaves;
  const int pairs = (g.G() + NW / 4 - 1) / (NW / 4);   // work-groups per (unit, KV head)
  const int num_uj = b.total_units * g.Hkv;
  const int groups8 = (num_uj + 7) / 8;
  const dim3 grid(groups8 * 8 * pairs);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const uint16_t *kb = static_cast<const uint16_t *>(c.k_cache);
  const uint16_t *vb = static_cast<const uint16_t *>(c.v_cache);
  uint16_t *ob = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  if (g.D == 64)
    attn_prefill_bf16_kernel<64, NW><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, ob, lse);
  else
    attn_prefill_bf16_kernel<128, NW><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, ob, lse);
  return hipGetLastError();
}

}  // namespace msa
