// Split-KV sparse decode attention and its log-sum-exp combine (steps 3 and 4 of
// MSA, decode).
//
// [dd] daily.dev "MiniMax M3 ...", section "Serving options": decode kernels for
// sparse GQA. [feat] models.inteligile.com "MiniMax-M3", method list "Two-phase
// forward" and "LSE fusion": the kept blocks are attended in independent parts
// whose partial results are merged through their logsumexp; "query
// concatenation": the G query heads that share a KV head are stacked against
// each KV block. Row "Grouped-query attention": query head i reads KV head i / G.
//
// A sequence may bring T new tokens, each with its own kept blocks (multi-token
// decode, per-token selection): token row x = r T + i of sequence r sits at
// seq_len - T + i, and everything below is per token row (T = 1: one per sequence).
//
// Phase 1: one work-group (4 waves) per (token row, KV head j, split). Its G <= 16
// query heads form the N = 16 columns of MFMA 16x16x32 bf16 products; each wave
// takes 32 keys of every kept block of the split and reads its operands straight
// from HBM with 16-byte loads (K rows token-major, V rows d-major):
//   S^T = K . Q^T    (A = 16 K rows per tile, B = the stacked queries in registers)
//   O^T += V^T . P^T (A = V^T rows, B = probabilities from S^T's registers)
// Tile tt's A row m is fed key 8(m/4) + 4tt + m%4 of the wave's 32, so that lane l
// ends up holding keys 8(l/16) .. 8(l/16)+7: the k-indices it supplies to the
// P^T operand, in natural order, matching one contiguous 16-byte V^T read.
// The waves' partial (max, sum, O) are merged in LDS and written normalised, with
// their natural-log lse, to the workspace.
// Phase 2: per (sequence, query head) the parts are merged:
//   lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) o_s.
//
// FP8 caches (E4M3 codes, a power-of-two scale per 32 channels of a token's head
// row): a K operand row of 8 channels lies in one scale block, so its 8 codes
// become bf16 with the scale applied in the conversion (exact: every E4M3 value
// times a power of two is a bf16 value). The 8 keys of a V^T operand row each
// carry their own scale, so the scale moves to the other operand: for the
// 32-channel block c the probabilities are multiplied by 2^e(c, key) before
// their bf16 rounding (exact, a power of two commutes with the rounding) and the
// V codes convert unscaled.
#include <mutex>

#include "msa_device.h"
#include "msa_launch.h"

// Scratch of msa_sparse_attn_decode_static: the split partials (o_part, lse_part)
// of the decode attention, for callers that cannot allocate. Each GPU the library
// runs on holds its own copy until the process ends. In host code this name is a
// stand-in, not a device address: kernels and copies take the address resolved by
// static_decode_scratch() below.
static __device__ __align__(256) unsigned char scratch[MSA_STATIC_SCRATCH_BYTES];

namespace msa {

hipError_t launch_attn_f32(const Geom &g, const msa_cache_t &c, const msa_unit_t *units,
                           int num_units, int T, const void *q, const int32_t *ids, int topk,
                           float scale, void *out, float *lse, hipStream_t st,
                           bool per_token = false);

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDecThreads = 256;
constexpr float kSlack = 8.f;

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, bf16x2));
}

// 8 E4M3 codes (two words) as a bf16x8 MFMA operand, each times `scale`
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 w, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, true);
  return as_bf16x8(uint4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                         __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)});
}

__device__ __forceinline__ float scale_of(uint32_t byte) {
  return ldexpf(1.0f, static_cast<int>(byte) - 127);
}

template <int D, bool FP8>
__global__ __launch_bounds__(kDecThreads) void attn_decode_bf16_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kc_,
    const void *__restrict__ vtc_, const uint8_t *__restrict__ ksc,
    const uint8_t *__restrict__ vsc, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int T, int num_splits, int per_split, float c,
    float *__restrict__ o_part, float *__restrict__ lse_part) {
  constexpr int KS = D / 32;   // k steps of S^T (one FP8 scale block each)
  constexpr int DT = D / 16;   // d tiles of O^T
  constexpr int NC = D / 32;   // FP8 scale blocks per head row
  const uint16_t *kc = static_cast<const uint16_t *>(kc_);
  const uint16_t *vtc = static_cast<const uint16_t *>(vtc_);
  const uint8_t *kc8 = static_cast<const uint8_t *>(kc_);
  const uint8_t *vtc8 = static_cast<const uint8_t *>(vtc_);
  __shared__ float Ow[4][16][D + 1];
  __shared__ float Mw[4][16], Lw[4][16];

  const int x = blockIdx.x / Hkv, j = blockIdx.x % Hkv, sp = blockIdx.y;   // token row x
  const int r = x / T;                                                       // its sequence
  const int G = Hq / Hkv;
  const int g = (nsel == Hkv) ? j : 0;
  const int32_t *sel = ids + (static_cast<size_t>(x) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(r) * max_blocks;
  const int qpos = seq_lens[r] - T + x % T;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  // the kept list ends at its first -1: nk ids, found by a ballot per 64 slots
  int nk = topk;
  for (int c0 = 0; c0 < topk; c0 += kWave) {
    const uint64_t pad = __ballot(c0 + lane < topk && sel[c0 + lane] < 0);
    if (pad != 0) {
      nk = c0 + static_cast<int>(__builtin_ctzll(pad));
      break;
    }
  }
  const int slot0 = sp * per_split, slot1 = min(nk, slot0 + per_split);

  const int n = lane % 16;               // stacked query head (column)
  const int q4 = lane / 16;              // lane quarter: 8 d (or 8 keys) per k step

  bf16x8 qb[KS];
  {
    const bool live = n < G;
    const uint16_t *qp =
        q + (static_cast<size_t>(x) * Hq + j * G + (live ? n : 0)) * D + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = *reinterpret_cast<const uint4 *>(qp + ks * 32);
      if (!live) v = uint4{0, 0, 0, 0};
      qb[ks] = as_bf16x8(v);
    }
  }
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
  float m_ref = neg_inf(), l_run = 0.f;
  bool any = false;

  for (int slot = slot0; slot < slot1; ++slot) {
    const int b = sel[slot];
    if (b > qpos / kBlk) continue;       // only future keys: not read
    any = true;
    const int64_t phys = bt[b];
    const size_t off = (static_cast<size_t>(phys) * Hkv + j) * kBlk * D;
    // bf16: the block's V^T operands are requested with its K rows, ahead of the
    // softmax that decides nothing about them (one memory round trip per block;
    // measured slower for FP8 caches, which load V after the softmax)
    uint4 vraw[FP8 ? 1 : DT];
    if constexpr (!FP8) {
      const uint16_t *vr = vtc + off + n * kBlk + wave * 32 + q4 * 8;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vraw[dt] = *reinterpret_cast<const uint4 *>(vr + dt * 16 * kBlk);
    }
    // S^T: 2 tiles of 16 keys x 16 heads over this wave's 32 keys
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{};
      const int key = wave * 32 + 8 * (n / 4) + 4 * tt + (n % 4);
      if constexpr (FP8) {
        const uint8_t *kr = kc8 + off + key * D + q4 * 8;
        const uint8_t *sr = ksc + (off / 32) + key * NC;      // the key's scale bytes
        uint32_t sb[NC];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sb[ks] = sr[ks];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = fp8x8_to_bf16(*reinterpret_cast<const uint2 *>(kr + ks * 32),
                                         scale_of(sb[ks]));
          s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], s[tt], 0, 0, 0);
        }
      } else {
        const uint16_t *kr = kc + off + key * D + q4 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4 *>(kr + ks * 32));
          s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], s[tt], 0, 0, 0);
        }
      }
    }
    // register i of tile tt holds key wave*32 + 8*q4 + 4*tt + i
    const int lim = qpos - b * kBlk - (wave * 32 + 8 * q4);
    float mx = neg_inf();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * tt + i > lim) s[tt][i] = neg_inf();
        mx = fmaxf(mx, s[tt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
    const bool need = mx > m_ref + kSlack;
    if (__any(need)) {
      const float nm = need ? mx : m_ref;
      const float al = __builtin_amdgcn_exp2f(m_ref - nm);
      m_ref = nm;
      l_run *= al;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= al;
    }
    float p[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tt * 4 + i] = (m_ref == neg_inf()) ? 0.f
                        : __builtin_amdgcn_exp2f(fmaf(s[tt][i], c, -m_ref));
        l_run += p[tt * 4 + i];
      }
    if constexpr (FP8) {
      // scales of this lane's 8 keys in each 32-channel block: v_scale[c][key]
      const uint8_t *sr = vsc + (off / 32) + wave * 32 + q4 * 8;
      uint2 sw[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) sw[c] = *reinterpret_cast<const uint2 *>(sr + c * kBlk);
      const uint8_t *vr = vtc8 + off + n * kBlk + wave * 32 + q4 * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float ps[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w = i < 4 ? sw[c].x : sw[c].y;
          ps[i] = ldexpf(p[i], static_cast<int>((w >> (8 * (i % 4))) & 0xffu) - 127);
        }
        const bf16x8 pb = as_bf16x8(uint4{cvt_pk_bf16(ps[0], ps[1]), cvt_pk_bf16(ps[2], ps[3]),
                                          cvt_pk_bf16(ps[4], ps[5]), cvt_pk_bf16(ps[6], ps[7])});
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {                // the two 16-row tiles of block c
          const int dt = 2 * c + dd;
          const bf16x8 a =
              fp8x8_to_bf16(*reinterpret_cast<const uint2 *>(vr + dt * 16 * kBlk), 1.0f);
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[dt], 0, 0, 0);
        }
      }
    } else {
      const bf16x8 pb = as_bf16x8(uint4{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]),
                                        cvt_pk_bf16(p[4], p[5]), cvt_pk_bf16(p[6], p[7])});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vraw[dt]), pb, o[dt], 0, 0, 0);
    }
  }

  // merge the 4 waves: per column n the waves hold (m, partial l, O^T)
  float l_w = l_run + __shfl_xor(l_run, 16, kWave);
  l_w += __shfl_xor(l_w, 32, kWave);
  if (lane < 16) {
    Mw[wave][n] = m_ref;
    Lw[wave][n] = l_w;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) Ow[wave][n][dt * 16 + q4 * 4 + i] = o[dt][i];
  __syncthreads();
  const size_t part0 = static_cast<size_t>(x) * Hq * num_splits;
  for (int e = t; e < G * D; e += kDecThreads) {
    const int hn = e / D, d = e % D;
    const size_t pi = part0 + static_cast<size_t>(j * G + hn) * num_splits + sp;
    if (!any) {
      o_part[pi * D + d] = 0.f;
      if (d == 0) lse_part[pi] = neg_inf();
      continue;
    }
    const float M = fmaxf(fmaxf(Mw[0][hn], Mw[1][hn]), fmaxf(Mw[2][hn], Mw[3][hn]));
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (Mw[w][hn] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(Mw[w][hn] - M);
      L += Lw[w][hn] * f;
      acc += Ow[w][hn][d] * f;
    }
    o_part[pi * D + d] = acc / L;
    if (d == 0) lse_part[pi] = (M + __builtin_log2f(L)) * kLn2;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void combine_kernel(const float *__restrict__ o_part,
                                                    const float *__restrict__ lse_part,
                                                    int num_splits, void *__restrict__ out,
                                                    float *__restrict__ lse) {
  const size_t row = blockIdx.x;   // sequence * Hq + head
  const int d = threadIdx.x;
  const float *lp = lse_part + row * num_splits;
  const float *op = o_part + row * num_splits * D + d;
  float M = neg_inf();
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, lp[s]);
  // An empty part has lse -inf and o 0, so it adds exp(-inf) * 0 = 0: no branch,
  // and eight parts' loads are issued before they are used. M is finite whenever
  // some part saw a key (the part holding the diagonal block sees the query's own).
  float L = 0.f, acc = 0.f;
  int s = 0;
  for (; s + 8 <= num_splits; s += 8) {
    float lv[8], ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      lv[u] = lp[s + u];
      ov[u] = op[static_cast<size_t>(s + u) * D];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = __expf(lv[u] - M);
      L += w;
      acc += w * ov[u];
    }
  }
  for (; s < num_splits; ++s) {
    const float w = __expf(lp[s] - M);
    L += w;
    acc += w * op[static_cast<size_t>(s) * D];
  }
  // no part saw a key (an id list without any block up to the query's own):
  // out = 0 and lse = -inf
  const bool seen = M != neg_inf();
  const float v = seen ? acc / L : 0.f;
  if constexpr (BF16)
    static_cast<uint16_t *>(out)[row * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  else
    static_cast<float *>(out)[row * D + d] = v;
  if (lse != nullptr && d == 0) lse[row] = seen ? M + __logf(L) : neg_inf();
}

}  // namespace

// About 512 work-groups (two per CU): more parts cost more in the combine than
// they win in latency (measured over 32-256 units: 1M decode 16 parts 28 us
// against 64 parts 37 us, 128k batch of 64 2 parts 109 us against 8 parts 121 us).
int decode_auto_splits(const Geom &g, int num_seqs, int topk) {
  const int units = num_seqs * g.Hkv;
  int s = (512 + units - 1) / units;
  s = s < 1 ? 1 : (s > topk ? topk : s);
  const int per = (topk + s - 1) / s;
  return (topk + per - 1) / per;
}

size_t decode_workspace_bytes(const Geom &g, int num_seqs, int num_splits) {
  const size_t parts = static_cast<size_t>(num_seqs) * g.Hq * num_splits;
  const size_t o_bytes = (parts * g.D * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return o_bytes + ((parts * sizeof(float) + 255) & ~static_cast<size_t>(255));
}

// Device address of the current GPU's copy of `scratch`, resolved once per device
// (with that device current) and kept.
hipError_t static_decode_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode(const Geom &g, const msa_cache_t &c, int T, const void *q,
                              const int32_t *ids, int topk, float scale, int num_splits,
                              void *workspace, void *out, float *lse, hipStream_t st) {
  if (c.num_seqs == 0) return hipSuccess;
  const int rows = c.num_seqs * T;        // token rows
  if (!g.bf16)
    return launch_attn_f32(g, c, nullptr, rows, T, q, ids, topk, scale, out, lse, st);
  const int per = (topk + num_splits - 1) / num_splits;
  const size_t parts = static_cast<size_t>(rows) * g.Hq * num_splits;
  float *o_part = static_cast<float *>(workspace);
  float *lse_part = reinterpret_cast<float *>(
      static_cast<char *>(workspace) +
      ((parts * g.D * sizeof(float) + 255) & ~static_cast<size_t>(255)));
  const dim3 grid(rows * g.Hkv, num_splits);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const float sl2 = scale * kLog2e;
#define MSA_DEC(DD, F8)                                                                    \
  attn_decode_bf16_kernel<DD, F8><<<grid, kDecThreads, 0, st>>>(                           \
      qb, c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.block_table, c.seq_lens, ids,     \
      topk, c.max_blocks_per_seq, g.Hq, g.Hkv, g.nsel, T, num_splits, per, sl2, o_part,    \
      lse_part)
  MSA_LOG_LAUNCH(g.fp8 ? "attn_decode_bf16_kernel (FP8 caches)" : "attn_decode_bf16_kernel", grid,
                 kDecThreads, 0);
  MSA_LOG_LAUNCH("combine_kernel", rows * g.Hq, g.D, 0);
  if (g.D == 64) {
    if (g.fp8) MSA_DEC(64, true); else MSA_DEC(64, false);
    combine_kernel<64, true><<<rows * g.Hq, 64, 0, st>>>(o_part, lse_part, num_splits, out,
                                                          lse);
  } else {
    if (g.fp8) MSA_DEC(128, true); else MSA_DEC(128, false);
    combine_kernel<128, true><<<rows * g.Hq, 128, 0, st>>>(o_part, lse_part, num_splits,
                                                            out, lse);
  }
#undef MSA_DEC
  return hipGetLastError();
}

}  // namespace msa
