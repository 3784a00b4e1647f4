// New tokens, before the indexer and attention steps: per-head RMSNorm of the
// queries and keys, partial rotary embedding, and the insert of K, V and the
// indexer keys into the block-major caches.
//
// What is computed (models.inteligile.com "MiniMax-M3" feature page, table
// "Checked in its code", rows "QK normalization" and "Partial RoPE"; daily.dev
// "MiniMax M3: 1M-token multimodal reasoning model ...", section "Serving
// options", which names the fused QK-norm + RoPE + KV insert step). For a token
// at position p and a head vector x of D channels:
//   n[c]  = x[c] / sqrt(mean_c'(x[c']^2) + eps) * w[c]            (w shared by heads)
//   for c < R/2 (R = rotary_dim), a = p * theta^(-2c/R):
//     y[c]       = n[c] cos a - n[c + R/2] sin a
//     y[c + R/2] = n[c + R/2] cos a + n[c] sin a
//   y[c] = n[c] for c >= R.
// Queries become q_out; keys go to k_cache; V and the indexer keys are copied
// unchanged into v_cache (transposed per block) and k_idx_cache.
//
// One work-group per (unit, KV head j) in prefill, per (sequence, j) in decode.
// A unit's tokens share one 128-token block, so the group owns the rows
// [rbase, rbase + n) of that physical block for KV head j (and for the indexer
// heads j, j + H_kv, ...), and the query heads [j*G, (j+1)*G) of its rows: no
// two groups touch the same bytes.
//
//   1. V rows are staged in LDS and written as d-major rows of the V block
//      (16-byte stores along the token axis when the segment is 8-aligned), and
//      the indexer keys are copied row by row.
//   2. The cos/sin table of the unit's positions is built in fp64 in LDS: per
//      channel pair one sincos at the first position of a segment, then exact
//      rotations by the per-step angle (fp64 keeps p * theta^(-2c/R) accurate at
//      positions near 2^20, where an fp32 angle would be off by ~0.06 rad).
//   3. Query and key rows stream through: D/EPL lanes per head row, each lane
//      holding 16 bytes (EPL channels). The sum of squares is reduced across the
//      row's lanes with DPP; the rotation partner of channel c (c + R/2 or
//      c - R/2) sits R/(2*EPL) lanes away, a power of two, so it is fetched with
//      one xor lane shuffle per channel. Four rows per lane are in flight at once.
// Everything is HBM streaming: each input byte is read once and each output byte
// written once.
//
// FP8 caches: K, V and the indexer keys are stored as E4M3 codes with one
// power-of-two scale 2^e per 32 channels of a token's head row (e the smallest
// with max|x| / 2^e <= 448, stored as e + 127; codes round x / 2^e to nearest
// even). Four lanes (8 channels each) share a 32-channel block: they take its
// maximum with DPP, and each converts its channels with v_cvt_pk_fp8_f32. V's
// scales, one per (token, block), are found from the staged tile before the
// transposed codes are written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // head rows per lane in flight

struct InsertArgs {
  const msa_unit_t *units;   // NULL: decode, one token per sequence
  const int32_t *seq_lens;
  const int32_t *block_table;
  int mbps;                  // max blocks per sequence
  const char *q, *k, *v, *kidx, *qw, *kw;
  char *q_out, *kc, *vc, *ic;
  uint8_t *ks, *vs, *is;     // FP8 caches: scale bytes of K, V, indexer keys
  int Hq, Hkv, Hi, Di, rd;
  float eps, theta;
};

template <bool BF>
__device__ __forceinline__ void unpack16(const uint4 &v, float *x) {
  if constexpr (BF) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
}

template <bool BF>
__device__ __forceinline__ uint4 pack16(const float *x) {
  if constexpr (BF) {
    return uint4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
  } else {
    return uint4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                 __float_as_uint(x[3])};
  }
}

// EPL raw elements of SZ bytes (16 bytes in all), moved without conversion.
template <int SZ, int EPL>
struct Bits {
  using E = typename std::conditional<SZ == 2, uint16_t, uint32_t>::type;
  E e[EPL];
};

// Exponent of the power-of-two scale of a 32-channel block whose largest
// magnitude is amax: the smallest e with amax / 2^e <= 448 (448 = 0.875 * 2^9, the
// largest E4M3 value), clamped to the scale byte's range [-127, 127].
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.f) return -127;
  int k;
  const float fr = frexpf(amax, &k);   // amax = fr * 2^k, fr in [0.5, 1)
  const int e = k - 9 + (fr > 0.875f ? 1 : 0);
  return min(max(e, -127), 127);
}

// E4M3 codes (nearest, ties to even) of four values within [-448, 448], byte i
// holding the i-th value.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Codes of 8 channels scaled by 2^-e.
__device__ __forceinline__ uint2 fp8x8(const float *x, int e) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = ldexpf(x[i], -e);
  return uint2{fp8x4(y[0], y[1], y[2], y[3]), fp8x4(y[4], y[5], y[6], y[7])};
}

__device__ __forceinline__ float absmax8(const float *x) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

__device__ __forceinline__ uint4 ld16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(char *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

template <bool BF, int D, bool FP8>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_insert_kernel(InsertArgs a) {
  static_assert(!FP8 || BF, "FP8 caches come with bf16 inputs");
  constexpr int SZ = BF ? 2 : 4;      // bytes per element
  constexpr int EPL = 16 / SZ;        // elements per lane (16 bytes)
  constexpr int LPH = D / EPL;        // lanes per head row
  constexpr int NI = kThreads / LPH;  // head rows per pass
  constexpr int RB = D * SZ;          // bytes per head row
  static_assert(LPH >= 8 && LPH <= 32, "lanes per head row");

  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int j = blockIdx.y;

  int r, row0, n, pos0;
  if (a.units != nullptr) {
    const msa_unit_t u = a.units[blockIdx.x];
    r = u.r;
    row0 = u.row0;
    n = u.num_rows;
    pos0 = u.pos0;
  } else {
    r = blockIdx.x;
    row0 = r;
    n = 1;
    pos0 = a.seq_lens[r] - 1;
  }
  if (pos0 < 0) return;
  const int rbase = pos0 % kBlk;
  n = min(n, kBlk - rbase);           // a unit never crosses its block
  if (n <= 0) return;
  const int64_t phys = a.block_table[static_cast<int64_t>(r) * a.mbps + pos0 / kBlk];

  // ---- 1. V (staged, written d-major) and indexer keys (copied) ----------
  {
    const char *vsrc = a.v + (static_cast<int64_t>(row0) * a.Hkv + j) * RB;
    const int64_t vrow = static_cast<int64_t>(a.Hkv) * RB;   // bytes between tokens
    constexpr int CPR = RB / 16;
    for (int c = tid; c < n * CPR; c += kThreads) {
      const int t = c / CPR, ch = c - t * CPR;
      *reinterpret_cast<uint4 *>(lds + t * RB + ch * 16) = ld16(vsrc + t * vrow + ch * 16);
    }

    const int nh = (a.Hi - j + a.Hkv - 1) / a.Hkv;           // indexer heads j, j+H_kv, ...
    const int IB = a.Di * SZ, CPI = IB / 16;
    if constexpr (FP8) {
      // (token, head, 32-channel block) per group of 4 lanes, 8 channels a lane
      const int NCI = a.Di / 32;
      const int items = n * nh * NCI;
      const int q4 = tid % 4, grp4 = tid / 4;
      for (int base = 0; base < items; base += kThreads / 4) {
        const int it = base + grp4;
        const bool ok = it < items;
        const int itc = ok ? it : items - 1;
        const int cb = itc % NCI, rest = itc / NCI;
        const int m = rest % nh, t = rest / nh;
        const int h = j + m * a.Hkv;
        float x[8];
        unpack16<true>(ld16(a.kidx + (static_cast<int64_t>(row0 + t) * a.Hi + h) * IB +
                            cb * 64 + q4 * 16), x);
        const int ex = mx_exponent(group_max<4>(absmax8(x)));
        const uint2 w = fp8x8(x, ex);
        if (ok) {
          const int64_t rowb = (phys * a.Hi + h) * kBlk + rbase + t;   // cache row
          *reinterpret_cast<uint2 *>(a.ic + rowb * a.Di + cb * 32 + q4 * 8) = w;
          if (q4 == 0) a.is[rowb * NCI + cb] = static_cast<uint8_t>(ex + 127);
        }
      }
    } else {
      for (int c = tid; c < n * nh * CPI; c += kThreads) {
        const int ch = c % CPI, rest = c / CPI;
        const int m = rest % nh, t = rest / nh;
        const int h = j + m * a.Hkv;
        const uint4 x =
            ld16(a.kidx + (static_cast<int64_t>(row0 + t) * a.Hi + h) * IB + ch * 16);
        st16(a.ic + ((phys * a.Hi + h) * kBlk + rbase + t) * IB + ch * 16, x);
      }
    }
    __syncthreads();

    if constexpr (FP8) {
      constexpr int NC = D / 32;
      int *es = reinterpret_cast<int *>(lds + n * RB);         // exponents [n][NC]
      uint8_t *vsd = a.vs + (phys * a.Hkv + j) * NC * kBlk;   // scales [NC][128]
      const int q4 = tid % 4, grp4 = tid / 4;
      for (int base = 0; base < n * NC; base += kThreads / 4) {
        const int it = base + grp4;
        const bool ok = it < n * NC;
        const int itc = ok ? it : n * NC - 1;
        const int t = itc / NC, cb = itc % NC;
        float x[8];
        unpack16<true>(*reinterpret_cast<const uint4 *>(lds + t * RB + cb * 64 + q4 * 16), x);
        const int ex = mx_exponent(group_max<4>(absmax8(x)));
        if (ok && q4 == 0) {
          es[t * NC + cb] = ex;
          vsd[cb * kBlk + rbase + t] = static_cast<uint8_t>(ex + 127);
        }
      }
      __syncthreads();
      uint8_t *vdst8 = reinterpret_cast<uint8_t *>(a.vc) + (phys * a.Hkv + j) * D * kBlk;
      auto val = [&](int t, int d) {
        return ldexpf(bf16_to_f32(*reinterpret_cast<const uint16_t *>(lds + t * RB + d * 2)),
                      -es[t * NC + d / 32]);
      };
      if (rbase % 16 == 0 && n % 16 == 0) {
        // lane -> (channel d, 16 consecutive tokens): 16-byte stores along a d-row
        for (int c = tid; c < D * (n / 16); c += kThreads) {
          const int d = c % D, t0 = (c / D) * 16;
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = fp8x4(val(t0 + 4 * i, d), val(t0 + 4 * i + 1, d), val(t0 + 4 * i + 2, d),
                         val(t0 + 4 * i + 3, d));
          st16(reinterpret_cast<char *>(vdst8 + d * kBlk + rbase + t0),
               uint4{w[0], w[1], w[2], w[3]});
        }
      } else {
        for (int c = tid; c < D * n; c += kThreads) {
          const int t = c % n, d = c / n;
          vdst8[d * kBlk + rbase + t] = static_cast<uint8_t>(fp8x4(val(t, d), 0.f, 0.f, 0.f));
        }
      }
    } else {
      char *vdst = a.vc + (phys * a.Hkv + j) * static_cast<int64_t>(D) * kBlk * SZ;
      if (rbase % EPL == 0 && n % EPL == 0) {
        // lane -> (channel d, EPL consecutive tokens): 16-byte stores along a d-row
        for (int c = tid; c < D * (n / EPL); c += kThreads) {
          const int d = c % D, tc = c / D;
          Bits<SZ, EPL> x;
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            x.e[e] = *reinterpret_cast<const typename Bits<SZ, EPL>::E *>(
                lds + (tc * EPL + e) * RB + d * SZ);
          st16(vdst + (static_cast<int64_t>(d) * kBlk + rbase + tc * EPL) * SZ,
               __builtin_bit_cast(uint4, x));
        }
      } else {
        for (int c = tid; c < D * n; c += kThreads) {
          const int t = c % n, d = c / n;
          using E = typename Bits<SZ, EPL>::E;
          *reinterpret_cast<E *>(vdst + (static_cast<int64_t>(d) * kBlk + rbase + t) * SZ) =
              *reinterpret_cast<const E *>(lds + t * RB + d * SZ);
        }
      }
    }
    __syncthreads();   // the LDS tile is reused below
  }

  // ---- 2. cos/sin table [n][R/2] of the unit's positions -----------------
  const int half = a.rd >> 1;
  float2 *tab = reinterpret_cast<float2 *>(lds);
  if (half > 0) {
    const int segs = kThreads / half;                  // half divides 256
    const int len = (n + segs - 1) / segs;
    const int i = tid % half, t0 = (tid / half) * len;
    if (t0 < n) {
      const double inv = pow(static_cast<double>(a.theta), -2.0 * i / a.rd);
      double s, c, ds, dc;
      sincos(static_cast<double>(pos0 + t0) * inv, &s, &c);
      sincos(inv, &ds, &dc);
      const int t1 = min(n, t0 + len);
      for (int t = t0; t < t1; ++t) {
        tab[t * half + i] = make_float2(static_cast<float>(c), static_cast<float>(s));
        const double c2 = c * dc - s * ds;
        s = s * dc + c * ds;
        c = c2;
      }
    }
  }
  __syncthreads();

  // ---- 3. query and key rows: RMSNorm, rotation, store -------------------
  const int lane = tid % LPH, grp = tid / LPH;
  const int c0 = lane * EPL;                           // first channel of this lane
  const bool rot = c0 < a.rd;
  const bool lower = c0 < half;
  const int i0 = lower ? c0 : c0 - half;               // angle index of channel c0
  const int xo = half > 0 ? half / EPL : 0;            // lane distance to the partner
  const float sgn = lower ? -1.f : 1.f;

  float wq[EPL], wk[EPL];
  unpack16<BF>(ld16(a.qw + c0 * SZ), wq);
  unpack16<BF>(ld16(a.kw + c0 * SZ), wk);

  const int G = a.Hq / a.Hkv;
  const int per_tok = G + 1;                           // G query heads, then the key
  const int items = n * per_tok;
  const float inv_d = 1.0f / D;

  for (int base = 0; base < items; base += NI * kUnroll) {
    uint4 raw[kUnroll];
    char *dst[kUnroll];
    int tt[kUnroll];
    bool isk[kUnroll], ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = base + u * NI + grp;
      ok[u] = it < items;
      const int itc = ok[u] ? it : items - 1;
      const int t = itc / per_tok, hh = itc - t * per_tok;
      tt[u] = t;
      isk[u] = hh == G;
      const int64_t row = row0 + t;
      const char *src;
      if (isk[u]) {
        src = a.k + (row * a.Hkv + j) * RB;
        dst[u] = a.kc + ((phys * a.Hkv + j) * kBlk + rbase + t) * RB;
      } else {
        const int64_t off = (row * a.Hq + j * G + hh) * RB;
        src = a.q + off;
        dst[u] = a.q_out + off;
      }
      raw[u] = ld16(src + c0 * SZ);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float x[EPL];
      unpack16<BF>(raw[u], x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
      ss = group_sum<LPH>(ss);
      const float rn = 1.0f / sqrtf(ss * inv_d + a.eps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = x[e] * rn * (isk[u] ? wk[e] : wq[e]);
      if (half > 0) {
        const float2 *cs = tab + tt[u] * half + i0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float p = __shfl_xor(x[e], xo);
          if (rot) {
            const float2 w = cs[e];
            x[e] = fmaf(sgn * p, w.y, x[e] * w.x);
          }
        }
      }
      if constexpr (FP8) {
        // keys: codes and a scale per 32 channels (4 lanes); queries stay bf16
        const int ex = mx_exponent(group_max<4>(absmax8(x)));
        if (ok[u] && isk[u]) {
          const int64_t rowk = (phys * a.Hkv + j) * kBlk + rbase + tt[u];   // cache row
          *reinterpret_cast<uint2 *>(a.kc + rowk * D + c0) = fp8x8(x, ex);
          if (lane % 4 == 0) a.ks[rowk * (D / 32) + c0 / 32] = static_cast<uint8_t>(ex + 127);
        } else if (ok[u]) {
          st16(dst[u] + c0 * SZ, pack16<BF>(x));
        }
      } else {
        if (ok[u]) st16(dst[u] + c0 * SZ, pack16<BF>(x));
      }
    }
  }
}

template <bool BF, int D, bool FP8 = false>
hipError_t launch_one(const InsertArgs &a, dim3 grid, size_t lds, hipStream_t st) {
  MSA_LOG_LAUNCH(FP8 ? "qk_norm_rope_insert_kernel (FP8 caches)" : "qk_norm_rope_insert_kernel", grid,
                 kThreads, lds);
  hipLaunchKernelGGL((qk_norm_rope_insert_kernel<BF, D, FP8>), grid, dim3(kThreads), lds, st,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope_insert(const Geom &g, const msa_cache_t &c, const msa_batch_t *b,
                                      const void *q, const void *k, const void *v,
                                      const void *k_idx, const void *q_norm_w,
                                      const void *k_norm_w, float eps, float theta, int rd,
                                      void *q_out, hipStream_t st) {
  InsertArgs a;
  a.units = b != nullptr ? b->units : nullptr;
  a.seq_lens = c.seq_lens;
  a.block_table = c.block_table;
  a.mbps = c.max_blocks_per_seq;
  a.q = static_cast<const char *>(q);
  a.k = static_cast<const char *>(k);
  a.v = static_cast<const char *>(v);
  a.kidx = static_cast<const char *>(k_idx);
  a.qw = static_cast<const char *>(q_norm_w);
  a.kw = static_cast<const char *>(k_norm_w);
  a.q_out = static_cast<char *>(q_out);
  a.kc = static_cast<char *>(c.k_cache);
  a.vc = static_cast<char *>(c.v_cache);
  a.ic = static_cast<char *>(c.k_idx_cache);
  a.ks = c.k_scale;
  a.vs = c.v_scale;
  a.is = c.k_idx_scale;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.Hi = g.Hi;
  a.Di = g.Di;
  a.rd = rd;
  a.eps = eps;
  a.theta = theta;

  const int rows = b != nullptr ? kBlk : 1;            // tokens per work-group at most
  const int sz = g.bf16 ? 2 : 4;
  // the V tile (+ FP8 block exponents) in phase 1, the cos/sin table after it
  const size_t lds = std::max<size_t>(size_t(rows) * (rd / 2) * sizeof(float2),
                                      size_t(rows) * g.D * sz +
                                          (g.fp8 ? size_t(rows) * (g.D / 32) * sizeof(int) : 0));
  const dim3 grid(b != nullptr ? b->total_units : c.num_seqs, g.Hkv);
  if (g.fp8)
    return g.D == 64 ? launch_one<true, 64, true>(a, grid, lds, st)
                     : launch_one<true, 128, true>(a, grid, lds, st);
  if (g.bf16)
    return g.D == 64 ? launch_one<true, 64>(a, grid, lds, st)
                     : launch_one<true, 128>(a, grid, lds, st);
  return g.D == 64 ? launch_one<false, 64>(a, grid, lds, st)
                   : launch_one<false, 128>(a, grid, lds, st);
}

}  // namespace msa
