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
#include <algorithm>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

// ---------------------------------------------------------------------------
// decode: one work-group of 256 threads per (sequence, logical block)
// ---------------------------------------------------------------------------
//
// A sequence may bring T new tokens (multi-token decode with per-token
// selection): token i sits at seq_len - T + i, is score row (r T + i), and the
// block's keys, streamed once, are scored against each token's query in turn.
// Block b is the diagonal of token i when b == (seq_len - T + i) / 128 (+inf),
// after it when larger (-inf).

constexpr int kMaxOutRows = 128;   // T * n_sel per sequence at most

// 16-byte LDS chunks taken by the decode schedule's prefix sums (num_seqs + 1 ints
// when the schedule is compacted); a kernel's own dynamic LDS follows them
__host__ __device__ inline int decode_pfx_chunks(int num_seqs, bool compact) {
  return compact ? ((num_seqs + 1) * 4 + 15) / 16 : 0;
}

// Writes the +inf / -inf entries of token rows whose diagonal is at or before b;
// returns whether some token of the sequence needs block b scored.
__device__ __forceinline__ bool decode_edges(float *out, int b, int L, int T, int nsel,
                                             int max_blocks) {
  if (b < (L - 1) / kBlk) return true;       // before the last token's diagonal
  for (int e = threadIdx.x; e < T * nsel; e += blockDim.x) {
    const int tau = (L - T + e / nsel) / kBlk;
    out[static_cast<size_t>(e) * max_blocks] = (b == tau) ? pos_inf() : neg_inf();
  }
  return false;
}

// Final per-token scores of block b from the waves' maxima (red[w][i n_sel + g]).
template <int NWAVE>
__device__ __forceinline__ void decode_finish(float *out, const float (*red)[kMaxOutRows],
                                              int b, int L, int T, int nsel, int max_blocks) {
  for (int e = threadIdx.x; e < T * nsel; e += blockDim.x) {
    const int tau = (L - T + e / nsel) / kBlk;
    float m = red[0][e];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) m = fmaxf(m, red[w][e]);
    out[static_cast<size_t>(e) * max_blocks] = b < tau ? m : (b == tau ? pos_inf() : neg_inf());
  }
}

// Work schedule of the decode indexers, for ragged batches (sequences of mixed
// lengths, block tables wider than most sequences). With `compact`, each
// work-group first builds in LDS (pfx, num_seqs + 1 ints) the prefix sum of the
// blocks every sequence needs scored (those before its last token's diagonal,
// (seq_len - 1) / 128) and works on that compacted list of (sequence, block)
// items (sequence by binary search), so a batch costs what its real blocks cost;
// the +inf / -inf entries at and after each sequence's last diagonal are written
// by a loop strided over all threads of the grid. Without `compact` (more
// sequences than the LDS prefix sum holds) the items are all (sequence, block)
// pairs and the empty ones only write their entries.
//
// Items are handed out by guided self-scheduling: the grid is four times the
// work-groups that fit on the device at once; the first quarter (dispatched
// first, all resident) take three quarters of the items in equal contiguous
// chunks, and the other work-groups take small chunks of the rest, dispatched in
// block-id order as slots free up, so that CUs that run slower end up with less
// work. `score(r, b, L, out)` scores one block (its own barriers included) and is
// called uniformly by the whole work-group.
__device__ __forceinline__ void guided_chunk(int64_t n, int64_t &it0, int64_t &it1) {
  const int64_t G = gridDim.x, w = blockIdx.x;
  if (G == 1) {
    it0 = 0;
    it1 = n;
    return;
  }
  const int64_t R = G >= 4 ? G / 4 : 1;   // G - R >= 1
  const int64_t c1 = (3 * n / 4) / R;
  if (w < R) {
    it0 = w * c1;
    it1 = it0 + c1;
    return;
  }
  const int64_t rest = n - c1 * R, c2 = (rest + (G - R) - 1) / (G - R);
  it0 = c1 * R + (w - R) * c2;
  it1 = it0 + c2 < n ? it0 + c2 : n;
}

template <typename Score>
__device__ __forceinline__ void decode_schedule(const int32_t *__restrict__ seq_lens,
                                                int num_seqs, int max_blocks, int T, int nsel,
                                                float *scores, bool compact, int *pfx,
                                                Score score) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const size_t row_stride = static_cast<size_t>(T) * nsel * max_blocks;   // per sequence
  if (!compact) {
    int64_t it0, it1;
    guided_chunk(static_cast<int64_t>(num_seqs) * max_blocks, it0, it1);
    for (int64_t it = it0; it < it1; ++it) {
      const int r = static_cast<int>(it / max_blocks);
      const int b = static_cast<int>(it - static_cast<int64_t>(r) * max_blocks);
      const int L = seq_lens[r];
      float *out = scores + r * row_stride + b;
      if (decode_edges(out, b, L, T, nsel, max_blocks)) score(r, b, L, out);
    }
    return;
  }
  __shared__ int wsum[4];
  int carry = 0;
  for (int base = 0; base < num_seqs; base += 256) {
    const int r = base + t;
    int x = r < num_seqs ? max((seq_lens[r] - 1) / kBlk, 0) : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {   // inclusive scan inside the wave
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) wsum[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (r < num_seqs) pfx[r + 1] = before + x;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (t == 0) pfx[0] = 0;
  __syncthreads();
  const int64_t total = static_cast<int64_t>(num_seqs) * max_blocks;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + t; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(e / max_blocks);
    const int b = static_cast<int>(e - static_cast<int64_t>(r) * max_blocks);
    const int L = seq_lens[r];
    if (b < (L - 1) / kBlk) continue;          // scored below
    float *out = scores + r * row_stride + b;
    for (int k = 0; k < T * nsel; ++k) {
      const int tau = (L - T + k / nsel) / kBlk;
      out[static_cast<size_t>(k) * max_blocks] = (b == tau) ? pos_inf() : neg_inf();
    }
  }
  int64_t it0, it1;
  guided_chunk(pfx[num_seqs], it0, it1);
  for (int it = static_cast<int>(it0); it < it1; ++it) {
    int lo = 0, hi = num_seqs;                 // pfx[lo] <= it < pfx[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (pfx[mid] <= it) lo = mid; else hi = mid;
    }
    score(lo, it - pfx[lo], seq_lens[lo], scores + lo * row_stride + (it - pfx[lo]));
  }
}

template <bool BF16, int DI, int HS>
__global__ __launch_bounds__(256) void index_decode_kernel(
    const void *__restrict__ q_idx, const void *__restrict__ k_idx,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    int num_seqs, int max_blocks, int nsel, int T, bool compact, float *__restrict__ scores) {
  constexpr int EPV = BF16 ? 8 : 4;      // elements per 16-byte load
  constexpr int LPR = DI / EPV;          // lanes covering one token row of one head
  constexpr int ROWS = 256 / LPR;        // token rows per pass
  constexpr int PASSES = kBlk / ROWS;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ float red[4][kMaxOutRows];
  extern __shared__ int pfx[];
  const int Hi = nsel * HS;

  decode_schedule(seq_lens, num_seqs, max_blocks, T, nsel, scores, compact, pfx,
                  [&](int r, int b, int L, float *out) __attribute__((always_inline)) {
  const int64_t phys = block_table[static_cast<size_t>(r) * max_blocks + b];
  const int t = threadIdx.x;
  const int piece = t % LPR;
  const int row = t / LPR;
  const char *kblk = static_cast<const char *>(k_idx) +
                     static_cast<size_t>(phys) * Hi * kBlk * DI * ESZ;
  const int wave = t / kWave, lane = t % kWave;

  for (int g = 0; g < nsel; ++g) {
    uint4 kv[PASSES][HS];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int hh = 0; hh < HS; ++hh)
        kv[p][hh] = load_stream16(
            kblk + ((static_cast<size_t>(g * HS + hh) * kBlk + p * ROWS + row) * DI +
                    piece * EPV) * ESZ);
    for (int i = 0; i < T; ++i) {
      const char *qrow =
          static_cast<const char *>(q_idx) + static_cast<size_t>(r * T + i) * Hi * DI * ESZ;
      uint4 qv[HS];
#pragma unroll
      for (int hh = 0; hh < HS; ++hh)
        qv[hh] =
            *reinterpret_cast<const uint4 *>(qrow + ((g * HS + hh) * DI + piece * EPV) * ESZ);
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
      if (lane == 0) red[wave][i * nsel + g] = m;
    }
  }
  __syncthreads();
  decode_finish<4>(out, red, b, L, T, nsel, max_blocks);
  __syncthreads();   // red is refilled by the next block
  });
}

// ---------------------------------------------------------------------------
// decode over FP8 indexer keys (E4M3 codes, one power-of-two scale per 32
// channels of a token's head row): same work-group layout as above, a token row
// of one head is D_i bytes of codes, 16 per lane. The codes become bf16 exactly
// (every E4M3 value is a bf16 value) and meet the bf16 query in
// v_dot2c_f32_bf16; a lane's 16 channels lie in one scale block, so its partial
// dot product is multiplied by that block's 2^e (exact) before the lanes of the
// row are summed. The result is the dot product with the decoded keys up to the
// order of the fp32 sums. A block's bytes: codes H_i*128*D_i plus scales
// H_i*128*D_i/32, about half of the bf16 block.
// ---------------------------------------------------------------------------

template <int DI, int HS>
__global__ __launch_bounds__(256) void index_decode_fp8_kernel(
    const uint16_t *__restrict__ q_idx, const uint8_t *__restrict__ k_idx,
    const uint8_t *__restrict__ k_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, int num_seqs, int max_blocks, int nsel, int T,
    bool compact, float *__restrict__ scores) {
  constexpr int LPR = DI / 16;           // lanes per token row of one head
  constexpr int ROWS = 256 / LPR;        // token rows per pass
  constexpr int PASSES = kBlk / ROWS;
  constexpr int SPR = DI / 32;           // scale bytes per token row
  __shared__ float red[4][kMaxOutRows];
  extern __shared__ int pfx[];           // prefix sums (compact), then the block's scales
  const int Hi = nsel * HS;
  uint4 *sc_lds = reinterpret_cast<uint4 *>(pfx) + decode_pfx_chunks(num_seqs, compact);
  const int nsc16 = Hi * kBlk * SPR / 16;   // 16-byte chunks of one block's scale bytes

  decode_schedule(seq_lens, num_seqs, max_blocks, T, nsel, scores, compact, pfx,
                  [&](int r, int b, int L, float *out) __attribute__((always_inline)) {
  const int64_t phys = block_table[static_cast<size_t>(r) * max_blocks + b];
  const int t = threadIdx.x;
  const int piece = t % LPR;
  const int row = t / LPR;
  const int chunk = piece / 2;           // 32-channel scale block of this lane
  const uint8_t *kblk = k_idx + static_cast<size_t>(phys) * Hi * kBlk * DI;
  const uint8_t *sblk = k_scale + static_cast<size_t>(phys) * Hi * kBlk * SPR;
  const int wave = t / kWave, lane = t % kWave;
  // The block's scale bytes (contiguous, Hi * 128 * D_i / 32) are read in one
  // coalesced pass of non-temporal 16-byte loads, like the codes, and staged in
  // LDS. (Read as cached single bytes they made the kernel 40% slower whenever
  // the caches held other data: 0.90 ms against 0.65 ms on the 1M decode after
  // a 1 GiB write.)
  uint4 sv{};
  if (t < nsc16) sv = load_stream16(sblk + 16 * t);
  for (int i = t + 256; i < nsc16; i += 256)   // only when a block has more than 4 KiB of scales
    sc_lds[i] = load_stream16(sblk + 16 * i);
  const uint8_t *sl = reinterpret_cast<const uint8_t *>(sc_lds);

  for (int g = 0; g < nsel; ++g) {
    uint4 kv[PASSES][HS];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int hh = 0; hh < HS; ++hh) {
        const size_t tok = static_cast<size_t>(g * HS + hh) * kBlk + p * ROWS + row;
        kv[p][hh] = load_stream16(kblk + tok * DI + piece * 16);
      }
    if (g == 0) {
      if (t < nsc16) sc_lds[t] = sv;
      __syncthreads();
    }
    uint32_t sc[PASSES][HS];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int hh = 0; hh < HS; ++hh)
        sc[p][hh] = sl[((g * HS + hh) * kBlk + p * ROWS + row) * SPR + chunk];
    for (int ti = 0; ti < T; ++ti) {
      const uint16_t *qrow = q_idx + static_cast<size_t>(r * T + ti) * Hi * DI;
      uint32_t qw[HS][8];                // this lane's 16 query channels, bf16 pairs
#pragma unroll
      for (int hh = 0; hh < HS; ++hh) {
        const uint16_t *qp = qrow + (g * HS + hh) * DI + piece * 16;
        const uint4 a = *reinterpret_cast<const uint4 *>(qp);
        const uint4 c = *reinterpret_cast<const uint4 *>(qp + 8);
        qw[hh][0] = a.x; qw[hh][1] = a.y; qw[hh][2] = a.z; qw[hh][3] = a.w;
        qw[hh][4] = c.x; qw[hh][5] = c.y; qw[hh][6] = c.z; qw[hh][7] = c.w;
      }
      float m = neg_inf();
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        float acc = 0.f;
#pragma unroll
        for (int hh = 0; hh < HS; ++hh) {
          const uint32_t w[4] = {kv[p][hh].x, kv[p][hh].y, kv[p][hh].z, kv[p][hh].w};
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
            const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
            part = dot2_bf16(qw[hh][2 * i], __builtin_bit_cast(uint32_t, lo), part);
            part = dot2_bf16(qw[hh][2 * i + 1], __builtin_bit_cast(uint32_t, hi), part);
          }
          acc = fmaf(part, ldexpf(1.0f, static_cast<int>(sc[p][hh]) - 127), acc);
        }
        acc = group_sum<LPR>(acc);   // full group score of token row p*ROWS+row
        m = fmaxf(m, acc);
      }
      m = group_max<kWave>(m);
      if (lane == 0) red[wave][ti * nsel + g] = m;
    }
  }
  __syncthreads();
  decode_finish<4>(out, red, b, L, T, nsel, max_blocks);
  __syncthreads();   // red is refilled by the next block
  });
}

// ---------------------------------------------------------------------------
// work order of the prefill indexers
// ---------------------------------------------------------------------------
//
// [feat] method list "Pre-scheduled tile chunking"; [blog] shaam.blog "Serving AI
// agents at scale", section "What makes MiniMax M3 different": KV outer, each key
// block read once. An item is (x, block chunk y, selection group z), x a tile
// pair (group width <= 128) or a tile (wider groups). Work-group ids are dealt
// to the 8 XCDs round-robin (id % 8), each XCD with its own L2. Every XCD owns a
// fixed set of (z, y) combos: with Z dividing 8, one group and every (8 / Z)-th
// chunk, taken in boustrophedon order (class c, then 8/Z - 1 - c, ...) so that
// the causal work, heavier in early chunks, evens out between XCDs; with Z a
// multiple of 8, Z / 8 groups and every chunk. An XCD runs its items in x-blocks
// of XB: for each x-block, each of its combos in turn, and inside a combo the XB
// consecutive x. The work-groups resident on one XCD then read one key chunk
// (fetched into that L2 once for the whole x-block) and, combo after combo, the
// same query rows. Items past the end (x >= X, y >= Y) do nothing.
struct ItemOrder {
  int X;      // x items
  int Y;      // block chunks
  int Z;      // selection groups
  int XB;     // x per x-block
  int CPX;    // combos per XCD

  static ItemOrder make(int X, int Y, int Z, int XB) {
    int cpx;
    if (8 % Z == 0) cpx = (Y + 8 / Z - 1) / (8 / Z);
    else if (Z % 8 == 0) cpx = (Z / 8) * Y;
    else cpx = (Y * Z + 7) / 8;
    return ItemOrder{X, Y, Z, XB, cpx};
  }
  int64_t grid() const {
    return int64_t{8} * ((X + XB - 1) / XB) * XB * CPX;
  }
  __device__ __forceinline__ bool item(int L, int &x, int &y, int &z) const {
    const int xcd = L % 8, k = L / 8;
    const int xi = k % XB, cc = (k / XB) % CPX, xb = k / (XB * CPX);
    x = xb * XB + xi;
    if (8 % Z == 0) {
      const int nc = 8 / Z, cls = xcd / Z;
      z = xcd % Z;
      y = cc * nc + ((cc & 1) ? nc - 1 - cls : cls);
    } else if (Z % 8 == 0) {
      z = (cc / Y) * 8 + xcd;
      y = cc % Y;
    } else {
      const int c = cc * 8 + ((cc & 1) ? 7 - xcd : xcd);
      y = c / Z;
      z = c % Z;
    }
    return x < X && y < Y && z < Z;
  }
};

// ---------------------------------------------------------------------------
// prefill, bf16, group width 256 or 512 (one selection group over all indexer
// heads): MFMA 32x32x16 on LDS-staged keys, 32 or 64 keys at a time
// ---------------------------------------------------------------------------
//
// A work-group of 8 waves (two per SIMD) scores two adjacent query tiles of one
// request (units 2x and 2x + 1 of the plan; a pair split by a request boundary
// runs as two passes of one tile) against a chunk of kChunkW candidate blocks,
// in the XCD-aware order of ItemOrder. Wave w holds 32 query rows of tile w / 4
// over the whole group width in registers (the A operand). The keys go through
// LDS a stage at a time: 32 or 64 keys of a block over all GD channels (32 KiB of
// bf16 keys at 512 channels), double-buffered by direct global->LDS loads with
// 16-byte chunks XOR-swizzled by key. Every wave contracts each 32-key tile of a
// stage over the whole width into two accumulators (even and odd k steps, so
// consecutive MFMAs do not depend on each other), adds them and max-pools. One
// accumulator pair per wave (32 registers) leaves room for two waves per SIMD
// next to the 128 registers of query rows, and one staged tile
// serves all 256 query rows. Rows past a unit's end repeat its last row.
//
// FP8 indexer keys: a staged key row is GD codes (16 per chunk) plus the tile's
// scale bytes; the group channels are contracted in the order
// (ks / 2) * 32 + (lane / 32) * 16 + (ks % 2) * 8 (the query operand uses the same
// order), so one 16-byte read gives a lane two k steps in one 32-channel scale
// block, converted with that block's power of two.

constexpr int kChunkW = 16;   // blocks per work-group
constexpr int kWideThreads = 512;

template <int DI, int HS, bool FP8, bool PT>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void index_prefill_wide_kernel(
    const uint16_t *__restrict__ q_idx, const void *__restrict__ k_idx_,
    const uint8_t *__restrict__ k_scale, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, int num_units, int max_blocks, int nsel,
    ItemOrder order, float *__restrict__ scores) {
  constexpr int GD = HS * DI;          // group width
  constexpr int KS = GD / 16;          // k steps of the whole group
  constexpr int CHG = FP8 ? GD / 16 : GD / 8;   // 16-byte chunks per staged key row
  constexpr int CPH = FP8 ? DI / 16 : DI / 8;   // 16-byte chunks per head row
  constexpr int NS = DI / 32;          // FP8 scale bytes per key and head
  // keys per stage: 64 (two 32-key tiles, half the barriers) where the staging
  // addresses fit beside the query rows; 32 for bf16 keys 512 channels wide
  constexpr int TK = (FP8 || GD <= 256) ? 64 : 32;
  constexpr int SPB = kBlk / TK;       // stages per block
  constexpr int NWV = kWideThreads / kWave;
  constexpr int NLD = TK * CHG / kWideThreads;  // direct loads per thread per stage
  constexpr int SCH = FP8 ? HS * TK * NS / 16 : 1;   // 16-byte chunks of a stage's scales
  static_assert(GD == 256 || GD == 512, "group width 256 or 512");
  static_assert(TK * CHG % kWideThreads == 0, "staging split");
  static_assert(!FP8 || SCH <= kWave, "one wave stages the scales");
  __shared__ u32x4 Kb[2][TK * CHG];
  __shared__ u32x4 Ks[2][SCH];
  __shared__ float red[NWV][kChunkW];
  const uint16_t *k_idx = static_cast<const uint16_t *>(k_idx_);
  const uint8_t *k_idx8 = static_cast<const uint8_t *>(k_idx_);
  // chunk c of key row r sits at c ^ (r % 16): the 16 rows one LDS pass reads at
  // the same chunk land on 16 distinct 16-byte bank positions
  auto swz = [](int key) { return key % 16; };

  int x, y, g;                          // item: tile pair x, block chunk y, group g
  if (!order.item(static_cast<int>(blockIdx.x), x, y, g)) return;
  const int u_first = 2 * x;
  if (u_first >= num_units) return;
  const bool paired =
      u_first + 1 < num_units && units[u_first + 1].r == units[u_first].r;
  const int npass = (!paired && u_first + 1 < num_units) ? 2 : 1;
  const int Hi = nsel * HS;
  const int b0 = y * kChunkW;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  for (int pass = 0; pass < npass; ++pass) {
  if (pass > 0) __syncthreads();        // the previous pass is done with LDS
  const int u0 = u_first + pass;
  const int ntile = paired ? 2 : 1;
  const msa_unit_t un0 = units[u0];
  const int tau_max = units[u0 + ntile - 1].tau;

  // +inf / -inf entries of the tiles inside this chunk (per token: of every row)
  if constexpr (PT) {
    for (int e = t; e < ntile * kBlk * kChunkW; e += kWideThreads) {
      const int tt = e / (kBlk * kChunkW), i = (e / kChunkW) % kBlk, b = b0 + e % kChunkW;
      const msa_unit_t ut = units[u0 + tt];
      if (i < ut.num_rows && b >= ut.tau && b < max_blocks)
        scores[(static_cast<size_t>(ut.row0 + i) * nsel + g) * max_blocks + b] =
            (b == ut.tau) ? pos_inf() : neg_inf();
    }
  } else {
    for (int e = t; e < ntile * kChunkW; e += kWideThreads) {
      const int tt = e / kChunkW, b = b0 + e % kChunkW;
      const int tau = units[u0 + tt].tau;
      if (b >= tau && b < max_blocks)
        scores[(static_cast<size_t>(u0 + tt) * nsel + g) * max_blocks + b] =
            (b == tau) ? pos_inf() : neg_inf();
    }
  }
  if (b0 >= tau_max) continue;
  const int nblk = min(kChunkW, tau_max - b0);

  // this wave's 32 query rows over the whole group width
  const int tt = wave / 4;
  const bool tile_live = tt < ntile;
  const msa_unit_t mine = units[u0 + (tile_live ? tt : 0)];
  const bool wave_live = tile_live && (wave % 4) * 32 < mine.num_rows;
  const int qrow = mine.row0 + min((wave % 4) * 32 + lane % 32, mine.num_rows - 1);
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int kk = FP8 ? (ks / 2) * 32 + (lane / 32) * 16 + (ks % 2) * 8
                       : ks * 16 + (lane / 32) * 8;
    const int h = g * HS + kk / DI, d = kk % DI;
    qf[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(
        q_idx + (static_cast<size_t>(qrow) * Hi + h) * DI + d));
  }

  const int32_t *bt = block_table + static_cast<size_t>(un0.r) * max_blocks;
  // stage st = block st / SPB, keys (st % SPB) * TK .., into buffer st % 2
  auto issue = [&](int st) __attribute__((always_inline)) {
    const size_t phys = static_cast<size_t>(bt[b0 + st / SPB]);
    const int key0 = (st % SPB) * TK;
    u32x4 *dst = Kb[st % 2];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int base = (NWV * i + wave) * 64;
      const int p = base + lane, key = p / CHG, c = (p % CHG) ^ swz(key);
      const int h = g * HS + c / CPH;
      const void *src;
      if constexpr (FP8)
        src = k_idx8 + ((phys * Hi + h) * kBlk + key0 + key) * DI + (c % CPH) * 16;
      else
        src = k_idx + ((phys * Hi + h) * kBlk + key0 + key) * DI + (c % CPH) * 8;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void *)(dst + base), 16, 0, 0);
    }
    if constexpr (FP8) {
      // scales of the tile: head hh's 32 keys x NS bytes are contiguous
      if (wave == 0 && lane < SCH) {
        const int hh = lane / (TK * NS / 16), off = (lane % (TK * NS / 16)) * 16;
        __builtin_amdgcn_global_load_lds(
            k_scale + ((phys * Hi + g * HS + hh) * kBlk + key0) * NS + off,
            (__attribute__((address_space(3))) void *)Ks[st % 2], 16, 0, 0);
      }
    }
  };

  const int nst = SPB * nblk;
  float m = neg_inf();                  // tile pooling: this lane's running maximum
  float mt = neg_inf();                 // per token: this lane's query over the block
  issue(0);
  for (int st = 0; st < nst; ++st) {
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this stage's keys landed
    __syncthreads();
    if (st + 1 < nst) issue(st + 1);
    const int bi = st / SPB, b = b0 + bi;
    const u32x4 *src = Kb[st % 2];
    const uint8_t *sb = reinterpret_cast<const uint8_t *>(Ks[st % 2]);
#pragma unroll
    for (int kt = 0; kt < TK / 32; ++kt) {
    const int key = kt * 32 + lane % 32;
    if (wave_live && b < mine.tau) {
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
      auto mma = [&](f32x16 &acc, const bf16x8 &kf, int ks) __attribute__((always_inline)) {
        if constexpr (PT)   // keys x queries: a lane holds one query and 16 keys
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, acc, 0, 0, 0);
      };
      if constexpr (FP8) {
#pragma unroll
        for (int k2 = 0; k2 < KS / 2; ++k2) {
          const u32x4 w = src[key * CHG + ((2 * k2 + lane / 32) ^ swz(key))];
          const int hh = (k2 * 32) / DI, sub = (k2 * 32 % DI) / 32;
          const float sc = ldexpf(1.0f, static_cast<int>(sb[(hh * TK + key) * NS + sub]) - 127);
          uint32_t o[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[2 * i] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, false));
            o[2 * i + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, true));
          }
          mma(acc0, as_bf16x8(uint4{o[0], o[1], o[2], o[3]}), 2 * k2);
          mma(acc1, as_bf16x8(uint4{o[4], o[5], o[6], o[7]}), 2 * k2 + 1);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
          mma(acc0, __builtin_bit_cast(bf16x8, src[key * CHG + ((2 * ks + lane / 32) ^ swz(key))]),
              ks);
          mma(acc1,
              __builtin_bit_cast(bf16x8, src[key * CHG + ((2 * ks + 2 + lane / 32) ^ swz(key))]),
              ks + 1);
        }
      }
      float v = neg_inf();
#pragma unroll
      for (int i = 0; i < 16; ++i) v = fmaxf(v, acc0[i] + acc1[i]);
      if constexpr (PT) mt = fmaxf(mt, v); else m = fmaxf(m, v);
    }
    }
    if (st % SPB == SPB - 1) {          // the block is complete
      if constexpr (PT) {
        // the two lane halves hold the same query's other 16 keys of each tile
        if (wave_live && b < mine.tau) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                           __float_as_uint(mt), false, false);
          const float sv = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          const int rit = (wave % 4) * 32 + lane;
          if (lane < 32 && rit < mine.num_rows)
            scores[(static_cast<size_t>(mine.row0 + rit) * nsel + g) * max_blocks + b] = sv;
        }
        mt = neg_inf();
      } else {
        const float mm = group_max<kWave>(m);
        if (lane == 0) red[wave][bi] = mm;
        m = neg_inf();
      }
    }
  }
  if constexpr (!PT) {
    __syncthreads();
    // tile tt owns blocks b < tau_tt: the maximum over its four waves
    for (int e = t; e < ntile * nblk; e += kWideThreads) {
      const int tile = e / nblk, bi = e % nblk, b = b0 + bi;
      if (b >= units[u0 + tile].tau) continue;
      scores[(static_cast<size_t>(u0 + tile) * nsel + g) * max_blocks + b] =
          fmaxf(fmaxf(red[4 * tile][bi], red[4 * tile + 1][bi]),
                fmaxf(red[4 * tile + 2][bi], red[4 * tile + 3][bi]));
    }
  }
  }   // pass
}

// ---------------------------------------------------------------------------
// prefill, bf16, group width <= 128: MFMA 32x32x16 on LDS-staged keys
// ---------------------------------------------------------------------------
//
// A work-group handles two adjacent query tiles of one request (units 2x and
// 2x + 1 of the plan, 128 query rows each; a pair split by a request boundary
// is done as two passes of one tile) and one selection group, over a chunk of
// kChunk2 candidate blocks, in the XCD-aware order of ItemOrder. Each block's group keys (128
// keys x GD, the group's indexer heads side by side) are staged in LDS by direct
// global->LDS loads, 16-byte chunks XOR-swizzled by key, double-buffered so the
// next block is in flight while this one is scored; one staged block serves every
// query row of the group. Wave w owns 64 rows (two 32-row MFMA tiles) of tile
// w/2: every key fragment read from LDS feeds two MFMAs. A = query rows in
// registers, B = key rows from LDS. Per 32-key sub-tile, row set a's MFMA chain
// runs while row set b's accumulator of the previous sub-tile is max-pooled, then
// b's chain while a's is pooled; the next sub-tile's fragments are read (and, for
// FP8 keys, converted) meanwhile. Rows past a unit's end repeat its last row, so they never change a
// maximum.
//
// FP8 indexer keys: the staged rows are the group's E4M3 codes (GD bytes a key,
// swizzled in 16-byte chunks by key / (16 / chunks per row) so a 16-lane read
// pass covers distinct banks), and the blocks' scale bytes are staged beside
// them. The contraction takes the group channels in the order
// (ks / 2) * 32 + (lane / 32) * 16 + (ks % 2) * 8 for k step ks and lane half
// lane / 32 (the query operand uses the same order), so one 16-byte LDS read
// gives a lane its codes for two k steps, all in one 32-channel scale block; they
// become bf16 with that block's power of two applied in the conversion (exact).

constexpr int kChunk2 = 32;   // blocks per work-group (16: 1-3% slower, 64: slower on the 32k prefill)
// Query tiles per work-group: two (256 query rows, 4 waves, two work-groups per CU).
constexpr int kTiles = 2;
constexpr int kIdxThreads = kTiles * 2 * kWave;
// x-block sizes of ItemOrder: 32 tile pairs (their query rows of one group, 2 MiB
// at 128 channels, and the current 1 MiB key chunk fit one XCD's 4 MB L2); 4 tile
// pairs for the wide kernel (512 channels: 1 MiB of query rows beside 2 MiB key
// chunks; 8 measured 3-5% slower, 2 and 1 far slower)
constexpr int kPairBlock = 32;
constexpr int kWidePairBlock = 4;

template <int DI, int HS, bool FP8, bool PT>
__global__ __launch_bounds__(kIdxThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void index_prefill_bf16_kernel(
    const uint16_t *__restrict__ q_idx, const void *__restrict__ k_idx_,
    const uint8_t *__restrict__ k_scale, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, int num_units, int max_blocks, int nsel,
    ItemOrder order, float *__restrict__ scores) {
  constexpr int GD = HS * DI;            // group width
  constexpr int KS = GD / 16;            // k steps
  constexpr int CHG = FP8 ? GD / 16 : GD / 8;   // 16-byte chunks per staged key row
  constexpr int CPH = FP8 ? DI / 16 : DI / 8;   // chunks per head
  constexpr int NW = kIdxThreads / kWave;
  constexpr int NLD = (kBlk * CHG + kIdxThreads - 1) / kIdxThreads;
  constexpr int NS = DI / 32;            // FP8 scale bytes per key and head
  constexpr int SCH = FP8 ? HS * kBlk * NS / 16 : 1;   // 16-byte chunks of a block's scales
  static_assert(GD <= 128, "group width");
  static_assert(!FP8 || SCH <= kWave, "one wave stages the scales");
  __shared__ u32x4 Kb0[kBlk * CHG], Kb1[kBlk * CHG];
  __shared__ u32x4 Ks0[SCH], Ks1[SCH];
  __shared__ float red[NW][kChunk2];
  // per token: the scores of up to kFlushB blocks of the tile pair's rows, written
  // out as runs of a score row instead of one scattered float per row and block
  // (row stride kFlushB + 1, odd, so 64 consecutive rows hit 64 distinct banks)
  constexpr int kFlushB = 8, kPStride = kFlushB + 1;
  __shared__ float pts[PT ? kTiles * kBlk * kPStride : 1];
  static_assert(kTiles * kBlk == kIdxThreads, "one thread per staged row");
  const uint16_t *k_idx = static_cast<const uint16_t *>(k_idx_);
  const uint8_t *k_idx8 = static_cast<const uint8_t *>(k_idx_);
  // FP8 row swizzle: keys sharing a 256-byte bank row get distinct chunk slots
  auto swz = [](int key) { return FP8 ? (key / (16 / CHG)) % CHG : key % CHG; };

  // item: tile pair x (units 2x and 2x + 1), block chunk y, selection group g
  int x, y, g;
  if (!order.item(static_cast<int>(blockIdx.x), x, y, g)) return;
  const int u_first = 2 * x;
  if (u_first >= num_units) return;
  // units of one request go together; a pair split by a request boundary is two
  // passes of one tile each
  const bool paired =
      u_first + 1 < num_units && units[u_first + 1].r == units[u_first].r;
  const int npass = (!paired && u_first + 1 < num_units) ? 2 : 1;
  const int Hi = nsel * HS;
  const int b0 = y * kChunk2;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  for (int pass = 0; pass < npass; ++pass) {
  if (pass > 0) __syncthreads();          // the previous pass is done with LDS
  const int u0 = u_first + pass;
  const int ntile = paired ? kTiles : 1;
  const msa_unit_t un0 = units[u0];
  const int tau_max = units[u0 + ntile - 1].tau;

  // the +inf / -inf entries of every tile inside this chunk (per token: of every
  // row of the tile; consecutive threads take consecutive blocks of one row)
  if constexpr (PT) {
    for (int e = t; e < ntile * kBlk * kChunk2; e += kIdxThreads) {
      const int tt = e / (kBlk * kChunk2), i = (e / kChunk2) % kBlk, b = b0 + e % kChunk2;
      const msa_unit_t ut = units[u0 + tt];
      if (i < ut.num_rows && b >= ut.tau && b < max_blocks)
        scores[(static_cast<size_t>(ut.row0 + i) * nsel + g) * max_blocks + b] =
            (b == ut.tau) ? pos_inf() : neg_inf();
    }
  } else {
    for (int e = t; e < ntile * kChunk2; e += kIdxThreads) {
      const int tt = e / kChunk2, b = b0 + e % kChunk2;
      const int tau = units[u0 + tt].tau;
      if (b >= tau && b < max_blocks)
        scores[(static_cast<size_t>(u0 + tt) * nsel + g) * max_blocks + b] =
            (b == tau) ? pos_inf() : neg_inf();
    }
  }
  if (b0 >= tau_max) continue;
  const int nblk = min(kChunk2, tau_max - b0);

  // this wave's tile and its two 32-row MFMA tiles
  const int tt = wave / 2;
  const bool tile_live = tt < ntile;
  const msa_unit_t mine = units[u0 + (tile_live ? tt : 0)];
  const bool wave_live = tile_live && (wave % 2) * 64 < mine.num_rows;
  bf16x8 qa[KS], qb[KS];
  {
    const int r0 = (wave % 2) * 64 + (lane % 32), r1 = r0 + 32;
    const int q0 = mine.row0 + min(r0, mine.num_rows - 1);
    const int q1 = mine.row0 + min(r1, mine.num_rows - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int kk = FP8 ? (ks / 2) * 32 + (lane / 32) * 16 + (ks % 2) * 8
                         : ks * 16 + (lane / 32) * 8;
      const int h = g * HS + kk / DI, d = kk % DI;
      qa[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(
          q_idx + (static_cast<size_t>(q0) * Hi + h) * DI + d));
      qb[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(
          q_idx + (static_cast<size_t>(q1) * Hi + h) * DI + d));
    }
  }

  const int32_t *bt = block_table + static_cast<size_t>(un0.r) * max_blocks;
  auto issue = [&](int b, u32x4 *dst, u32x4 *sdst) __attribute__((always_inline)) {
    const size_t phys = static_cast<size_t>(bt[b]);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int base = (NW * i + wave) * 64;
      if (base < kBlk * CHG) {
        const int p = base + lane, key = p / CHG, c = (p % CHG) ^ swz(key);
        const int h = g * HS + c / CPH;
        const void *src;
        if constexpr (FP8)
          src = k_idx8 + ((phys * Hi + h) * kBlk + key) * DI + (c % CPH) * 16;
        else
          src = k_idx + ((phys * Hi + h) * kBlk + key) * DI + (c % CPH) * 8;
        __builtin_amdgcn_global_load_lds(
            src, (__attribute__((address_space(3))) void *)(dst + base), 16, 0, 0);
      }
    }
    if constexpr (FP8) {
      // the group's scale bytes: head hh's [128][NS] bytes are contiguous
      if (wave == 0 && lane < SCH) {
        const int hh = lane / (kBlk * NS / 16), off = (lane % (kBlk * NS / 16)) * 16;
        __builtin_amdgcn_global_load_lds(
            k_scale + (phys * Hi + g * HS + hh) * kBlk * NS + off,
            (__attribute__((address_space(3))) void *)sdst, 16, 0, 0);
      }
    }
  };
  auto score = [&](int bi, const u32x4 *src, const u32x4 *ssrc) __attribute__((always_inline)) {
    const int b = b0 + bi;
    float m = neg_inf();
    float ma = neg_inf(), mb = neg_inf();   // per token: this lane's query of each row set
    if (wave_live && b < mine.tau) {
      bf16x8 kf[2][KS];
      f32x16 acc0, acc1;
      auto rd = [&](int nt, bf16x8 *dst) __attribute__((always_inline)) {
        const int key = nt * 32 + lane % 32;
        if constexpr (FP8) {
          const uint8_t *sb = reinterpret_cast<const uint8_t *>(ssrc);
#pragma unroll
          for (int k2 = 0; k2 < KS / 2; ++k2) {
            const u32x4 w = src[key * CHG + ((2 * k2 + lane / 32) ^ swz(key))];
            const int hh = (k2 * 32) / DI, sub = (k2 * 32 % DI) / 32;
            const float sc =
                ldexpf(1.0f, static_cast<int>(sb[(hh * kBlk + key) * NS + sub]) - 127);
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              o[2 * i] = __builtin_bit_cast(
                  uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, false));
              o[2 * i + 1] = __builtin_bit_cast(
                  uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, true));
            }
            dst[2 * k2] = as_bf16x8(uint4{o[0], o[1], o[2], o[3]});
            dst[2 * k2 + 1] = as_bf16x8(uint4{o[4], o[5], o[6], o[7]});
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            dst[ks] = __builtin_bit_cast(bf16x8,
                                         src[key * CHG + ((2 * ks + lane / 32) ^ swz(key))]);
        }
      };
      // one chain of three-input maxima (8 per accumulator): the pairwise form,
      // max(m, max(a, b)), compiled to 12 instructions
      auto pool = [&](float &mm, const f32x16 &v) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) mm = fmaxf(fmaxf(mm, v[i]), v[i + 1]);
      };
      rd(0, kf[0]);
      // row set a's chain while row set b's previous sub-tile is pooled, then row
      // set b's chain while a's is pooled, so the wave does not wait for a
      // sub-tile's results before the next sub-tile's MFMAs: beside each MFMA one
      // max3 (bf16 keys), or three VALU instructions of the pooling and of the next
      // fragments' FP8 conversions
      auto chain = [&](f32x16 &acc, const bf16x8 *q, int cb) __attribute__((always_inline)) {
        acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (PT)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cb][ks], q[ks], acc, 0, 0, 0);
          else
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[ks], kf[cb][ks], acc, 0, 0, 0);
        }
      };
      float &pa = PT ? ma : m, &pb = PT ? mb : m;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int cb = nt & 1;
        if (nt < 3) rd(nt + 1, kf[cb ^ 1]);
        constexpr int NV = FP8 ? 3 : 1;   // VALU instructions beside each MFMA
        chain(acc0, qa, cb);
        if (nt > 0) pool(pb, acc1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
        }
        chain(acc1, qb, cb);
        pool(pa, acc0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
        }
      }
      pool(pb, acc1);
    }
    if constexpr (PT) {
      // lanes 0..31 take the other half's keys of row set a, lanes 32..63 those of
      // row set b: lane l then holds the block score of tile row 64 (wave % 2) + l
      if (wave_live && b < mine.tau) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ma), __float_as_uint(mb),
                                                         false, false);
        const float v = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const int rit = (wave % 2) * 64 + lane;
        if (rit < mine.num_rows) pts[(tt * kBlk + rit) * kPStride + bi % kFlushB] = v;
      }
      // every kFlushB blocks (and after the last): each thread writes one row's
      // staged scores, the blocks before that row's diagonal, as one run
      if (bi % kFlushB == kFlushB - 1 || bi == nblk - 1) {
        __syncthreads();
        const int fb = bi - bi % kFlushB, cnt = bi % kFlushB + 1;
        const int tt2 = t / kBlk, i = t % kBlk;
        if (tt2 < ntile) {
          const msa_unit_t ut = units[u0 + tt2];
          if (i < ut.num_rows) {
            float *dst = scores + (static_cast<size_t>(ut.row0 + i) * nsel + g) * max_blocks +
                         b0 + fb;
            const float *srcp = pts + t * kPStride;
            const int nv = min(cnt, ut.tau - b0 - fb);
            if (nv == kFlushB && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
              *reinterpret_cast<float4 *>(dst) = make_float4(srcp[0], srcp[1], srcp[2], srcp[3]);
              *reinterpret_cast<float4 *>(dst + 4) =
                  make_float4(srcp[4], srcp[5], srcp[6], srcp[7]);
            } else {
              for (int k = 0; k < nv; ++k) dst[k] = srcp[k];
            }
          }
        }
      }
    } else {
      m = group_max<kWave>(m);
      if (lane == 0) red[wave][bi] = m;
    }
  };

  issue(b0, Kb0, Ks0);
  for (int bi = 0;;) {
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this block's keys landed
    __syncthreads();
    if (bi + 1 < nblk) issue(b0 + bi + 1, Kb1, Ks1);
    score(bi, Kb0, Ks0);
    if (++bi >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (bi + 1 < nblk) issue(b0 + bi + 1, Kb0, Ks0);
    score(bi, Kb1, Ks1);
    if (++bi >= nblk) break;
  }
  if constexpr (!PT) {                    // per-token scores are already stored
    __syncthreads();
    // finished rows: tile t owns blocks b < tau_t
    for (int e = t; e < ntile * nblk; e += kIdxThreads) {
      const int tile = e / nblk, bi = e % nblk, b = b0 + bi;
      if (b >= units[u0 + tile].tau) continue;
      scores[(static_cast<size_t>(u0 + tile) * nsel + g) * max_blocks + b] =
          fmaxf(red[2 * tile][bi], red[2 * tile + 1][bi]);
    }
  }
  }   // pass
}

// ---------------------------------------------------------------------------
// prefill, fp32: plain FMA, one work-group of 128 threads per (unit, group, block)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(128) void index_prefill_f32_kernel(
    const float *__restrict__ q_idx, const float *__restrict__ k_idx,
    const int32_t *__restrict__ block_table, const msa_unit_t *__restrict__ units,
    int max_blocks, int nsel, int Hi, int Di, bool per_token, float *__restrict__ scores) {
  __shared__ float red[2];
  const int u = blockIdx.x, g = blockIdx.z, b = blockIdx.y;
  const msa_unit_t un = units[u];
  const int Hs = Hi / nsel;
  float *out = scores + (static_cast<size_t>(u) * nsel + g) * max_blocks;
  if (per_token) {
    // one row per query token: max over the block's keys only
    auto row_out = [&](int t) {
      return scores + (static_cast<size_t>(un.row0 + t) * nsel + g) * max_blocks;
    };
    if (b >= un.tau) {
      for (int t = threadIdx.x; t < un.num_rows; t += 128)
        row_out(t)[b] = (b == un.tau) ? pos_inf() : neg_inf();
      return;
    }
    const int s = threadIdx.x;
    const int64_t phys = block_table[static_cast<size_t>(un.r) * max_blocks + b];
    for (int t = 0; t < un.num_rows; ++t) {
      float acc = 0.f;
      for (int hh = 0; hh < Hs; ++hh) {
        const int h = g * Hs + hh;
        const float *qv = q_idx + (static_cast<size_t>(un.row0 + t) * Hi + h) * Di;
        const float *kv = k_idx + ((static_cast<size_t>(phys) * Hi + h) * kBlk + s) * Di;
        for (int d = 0; d < Di; ++d) acc = fmaf(qv[d], kv[d], acc);
      }
      acc = group_max<kWave>(acc);
      if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = acc;
      __syncthreads();
      if (threadIdx.x == 0) row_out(t)[b] = fmaxf(red[0], red[1]);
      __syncthreads();
    }
    return;
  }
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

// Grid of the decode indexers: four times the work-groups resident at once (CUs x
// work-groups per CU for this kernel and LDS size), never more than there are
// (sequence, block) pairs; the compacted schedule when the per-sequence prefix
// sum fits in LDS.
constexpr int kMaxCompactSeqs = 16384;

struct DecodeLaunch {
  dim3 grid;
  size_t lds;
  bool compact;
};

// extra_lds: bytes of dynamic LDS the kernel needs after the prefix sums
template <typename Kernel>
DecodeLaunch decode_launch(const msa_cache_t &c, Kernel kernel, size_t extra_lds = 0) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const bool compact = c.num_seqs <= kMaxCompactSeqs;
  const size_t lds =
      static_cast<size_t>(decode_pfx_chunks(c.num_seqs, compact)) * 16 + extra_lds;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int64_t pairs = static_cast<int64_t>(c.num_seqs) * c.max_blocks_per_seq;
  const int64_t groups = std::min<int64_t>(pairs, static_cast<int64_t>(cus) * per_cu * 4);
  return DecodeLaunch{dim3(static_cast<unsigned>(std::max<int64_t>(groups, 1))), lds, compact};
}

template <bool BF16, int DI>
hipError_t dispatch_decode_hs(const Geom &g, const msa_cache_t &c, int T, const void *q_idx,
                              float *scores, hipStream_t st) {
  switch (g.Hs()) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    {                                                                                    \
    const DecodeLaunch dl = decode_launch(c, index_decode_kernel<BF16, DI, HS>);        \
    MSA_LOG_LAUNCH("index_decode_kernel", dl.grid, 256, dl.lds);                          \
    index_decode_kernel<BF16, DI, HS><<<dl.grid, 256, dl.lds, st>>>(                     \
        q_idx, c.k_idx_cache, c.block_table, c.seq_lens, c.num_seqs,                     \
        c.max_blocks_per_seq, g.nsel, T, dl.compact, scores);                            \
    }                                                                                    \
    break;
    MSA_CASE(1) MSA_CASE(2) MSA_CASE(4) MSA_CASE(8)
#undef MSA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DI>
hipError_t dispatch_decode_fp8(const Geom &g, const msa_cache_t &c, int T, const void *q_idx,
                               float *scores, hipStream_t st) {
  const uint16_t *q = static_cast<const uint16_t *>(q_idx);
  const uint8_t *k = static_cast<const uint8_t *>(c.k_idx_cache);
  switch (g.Hs()) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    {                                                                                    \
    const DecodeLaunch dl = decode_launch(c, index_decode_fp8_kernel<DI, HS>,           \
                                          static_cast<size_t>(g.Hi) * kBlk * (DI / 32)); \
    MSA_LOG_LAUNCH("index_decode_fp8_kernel", dl.grid, 256, dl.lds);                      \
    index_decode_fp8_kernel<DI, HS><<<dl.grid, 256, dl.lds, st>>>(                       \
        q, k, c.k_idx_scale, c.block_table, c.seq_lens, c.num_seqs, c.max_blocks_per_seq, \
        g.nsel, T, dl.compact, scores);                                                  \
    }                                                                                    \
    break;
    MSA_CASE(1) MSA_CASE(2) MSA_CASE(4) MSA_CASE(8)
#undef MSA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DI, bool FP8, bool PT>
hipError_t dispatch_prefill_bf16(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                 const void *q_idx, float *scores, hipStream_t st) {
  const uint16_t *q = static_cast<const uint16_t *>(q_idx);
  const int hs = g.Hs();
  if (hs * DI <= 128) {
    const ItemOrder ord = ItemOrder::make((b.total_units + 1) / 2,
                                          (c.max_blocks_per_seq + kChunk2 - 1) / kChunk2,
                                          g.nsel, kPairBlock);
    if (ord.grid() > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(ord.grid()));
    MSA_LOG_LAUNCH(PT ? "index_prefill_bf16_kernel (per token)" : "index_prefill_bf16_kernel", grid,
                   kIdxThreads, 0);
    switch (hs) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    if constexpr (HS * DI <= 128)                                                        \
      index_prefill_bf16_kernel<DI, HS, FP8, PT><<<grid, kIdxThreads, 0, st>>>(          \
          q, c.k_idx_cache, c.k_idx_scale, c.block_table, b.units, b.total_units,        \
          c.max_blocks_per_seq, g.nsel, ord, scores);                                    \
    break;
      MSA_CASE(1) MSA_CASE(2) MSA_CASE(4)
#undef MSA_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const ItemOrder ord = ItemOrder::make((b.total_units + 1) / 2,
                                        (c.max_blocks_per_seq + kChunkW - 1) / kChunkW, g.nsel,
                                        kWidePairBlock);
  if (ord.grid() > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(ord.grid()));
  MSA_LOG_LAUNCH(PT ? "index_prefill_wide_kernel (per token)" : "index_prefill_wide_kernel", grid,
                 kWideThreads, 0);
  switch (hs) {
#define MSA_CASE(HS)                                                                     \
  case HS:                                                                               \
    if constexpr (HS * DI == 256 || HS * DI == 512)                                      \
      index_prefill_wide_kernel<DI, HS, FP8, PT><<<grid, kWideThreads, 0, st>>>(         \
          q, c.k_idx_cache, c.k_idx_scale, c.block_table, b.units, b.total_units,        \
          c.max_blocks_per_seq, g.nsel, ord, scores);                                    \
    else                                                                                 \
      return hipErrorInvalidValue;                                                       \
    break;
    MSA_CASE(4) MSA_CASE(8)
#undef MSA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_decode(const Geom &g, const msa_cache_t &c, int T, const void *q_idx,
                               float *scores, hipStream_t st) {
  if (g.fp8) {
    return g.Di == 64 ? dispatch_decode_fp8<64>(g, c, T, q_idx, scores, st)
                      : dispatch_decode_fp8<32>(g, c, T, q_idx, scores, st);
  }
  if (g.bf16) {
    return g.Di == 64 ? dispatch_decode_hs<true, 64>(g, c, T, q_idx, scores, st)
                      : dispatch_decode_hs<true, 32>(g, c, T, q_idx, scores, st);
  }
  return g.Di == 64 ? dispatch_decode_hs<false, 64>(g, c, T, q_idx, scores, st)
                    : dispatch_decode_hs<false, 32>(g, c, T, q_idx, scores, st);
}

template <bool PT>
hipError_t launch_prefill_scores(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                 const void *q_idx, float *scores, hipStream_t st) {
  if (b.total_units == 0) return hipSuccess;
  if (g.fp8) {
    return g.Di == 64 ? dispatch_prefill_bf16<64, true, PT>(g, c, b, q_idx, scores, st)
                      : dispatch_prefill_bf16<32, true, PT>(g, c, b, q_idx, scores, st);
  }
  if (g.bf16) {
    return g.Di == 64 ? dispatch_prefill_bf16<64, false, PT>(g, c, b, q_idx, scores, st)
                      : dispatch_prefill_bf16<32, false, PT>(g, c, b, q_idx, scores, st);
  }
  const dim3 grid(b.total_units, c.max_blocks_per_seq, g.nsel);
  MSA_LOG_LAUNCH("index_prefill_f32_kernel", grid, 128, 0);
  index_prefill_f32_kernel<<<grid, 128, 0, st>>>(
      static_cast<const float *>(q_idx), static_cast<const float *>(c.k_idx_cache),
      c.block_table, b.units, c.max_blocks_per_seq, g.nsel, g.Hi, g.Di, PT, scores);
  return hipGetLastError();
}

hipError_t launch_index_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                const void *q_idx, float *scores, hipStream_t st) {
  return launch_prefill_scores<false>(g, c, b, q_idx, scores, st);
}

hipError_t launch_index_prefill_tokens(const Geom &g, const msa_cache_t &c,
                                       const msa_batch_t &b, const void *q_idx, float *scores,
                                       hipStream_t st) {
  return launch_prefill_scores<true>(g, c, b, q_idx, scores, st);
}

}  // namespace msa
