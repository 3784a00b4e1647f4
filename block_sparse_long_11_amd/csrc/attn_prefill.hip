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
// bf16 path (MFMA 32x32x16, fp32 accumulate). A work-group of 8 waves owns (unit,
// KV head j, 2 query heads): 128 token rows x 2 heads, one wave per (head, 32
// tokens); waves w and w + 4 share a SIMD. Per 32-key tile each wave computes
//   S^T = K . Q^T           (A = K rows from LDS, B = Q held in registers)
//   O^T += V^T . P^T        (A = V^T rows from LDS, B = P from S^T's registers)
// The S^T row m of a tile is fed key (m with bits 2 and 3 swapped): then lane
// half a, register 8h+jj holds key 16h + 8a + jj, which is exactly the k-index
// the P^T operand needs, so V^T is read in natural key order.
//
// Ping-pong: every tile T is split into an MFMA phase M(T) (S^T of tile T and
// O^T += V^T P^T of tile T-1) and a softmax phase S(T) (mask, row maximum,
// exponentials, P, and the LDS reads of the operands of M(T+1)). Phases end at
// work-group barriers, and waves 4..7 run one phase behind waves 0..3, so on
// every SIMD one wave issues MFMAs while the other does the softmax.
//
// K/V staging: half-blocks of 64 keys (K as [key][d], V as the cache's d-major
// [d][key]) go through a ring of 4 LDS slots by direct global->LDS loads,
// 16-byte chunks XOR-swizzled by row. Half-block h+3 is requested in S(2h+1),
// after the last read of the slot it overwrites (half-block h-1, read up to
// S(2h-1) by the trailing waves); every wave waits for its loads of half-block
// h+1 at the end of S(2h), two barriers before the first read of it in S(2h+1).
//
// Online softmax in log2 units with a lazy reference maximum: O and the row sum
// are rescaled only when a row's maximum grows by more than 8 (probabilities
// stay <= 2^8); the result is exact after the final division by the row sum.
//
// FP8 caches (E4M3 codes, a power-of-two scale per 32 channels of a token's head
// row): attn_prefill_fp8_kernel keeps the work-group layout, the LDS layout and
// swizzles, the operand reads and the softmax of the bf16 kernel, but fills the
// LDS tiles itself: each thread loads 16 codes of one K row (one scale) and 16
// keys of one V^T row (16 scales) of a half-block, converts them to bf16 (exact:
// E4M3 times a power of two is a bf16 value) and writes them; the next
// half-block's codes are in flight while the current one is attended. Phases are
// not ping-ponged (the staged registers leave no room for it).
//
// fp32 path: plain FMA, one thread per (query, head); for small exact checks.
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
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

// Work-group barrier between phases. It does not wait for outstanding memory
// operations (the direct loads are waited for explicitly), and neither the
// compiler's memory-operation order nor its instruction schedule crosses it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(n) (n < 16), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// Direct global->LDS load of 16 bytes per lane: lane i reads gbase + voff (its
// own offset) and writes LDS byte address lds + 16 i. Issued as one instruction
// so that the compiler does not add waits of its own before later LDS reads;
// completion is waited for explicitly (wait_vm) before a barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(uint32_t lds, const void *gbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int V>
using ic = std::integral_constant<int, V>;

template <int D>
__global__ __launch_bounds__(kPrefWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vtc, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int num_uj, int pairs, float c,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int NW = kPrefWaves;
  constexpr int KS = D / 16;              // 16-wide d steps of S^T
  constexpr int DT = D / 32;              // 32-row d tiles of O^T
  constexpr int CH = D / 8;               // 16-byte chunks per K row
  constexpr int NT = NW * kWave;          // threads
  constexpr int HB = kBlk / 2;            // keys per half-block
  constexpr int VC = HB / 8;              // 16-byte chunks per V^T row of a half-block
  constexpr int KCH = HB * CH / NT;       // direct loads per wave per half-block: K
  constexpr int VCH = D * VC / NT;        //   and V^T
  constexpr int LPH = KCH + VCH;
  constexpr int KSLOT = HB * CH * 16;     // bytes of one ring slot: K
  constexpr int VSLOT = D * VC * 16;      //   and V^T
  constexpr int VBASE = 4 * KSLOT;        // V^T slots follow the 4 K slots
  static_assert(HB * CH % NT == 0 && D * VC % NT == 0, "staging split");
  static_assert(4 * KSLOT <= 65536 && 4 * VSLOT <= 65536, "ds offsets");
  // Ring of 4 half-block slots. K: chunk c of row r at c ^ (srow_key(r % 32) % CH),
  // keyed on the lane that reads row r; V^T (rows of 8 chunks): chunk c of row d at
  // c ^ ((d / 2) % 8), so that the 16 lanes of one LDS pass (16 rows, two per
  // 256-byte bank line) hit 16 distinct bank groups.
  __shared__ u32x4 smem[4 * (HB * CH + D * VC)];
  const char *lds = reinterpret_cast<const char *>(smem);
  const uint32_t lds_addr = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)smem));

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

  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int a = lane / 32, n = lane % 32;
  const int grp = wave / 4;               // 0 leads, 1 trails by one phase
  const int hl = 2 * hp + grp;            // head inside the group
  const int slab = wave % 4;              // 32-token slab of the tile
  // Waves past the group's heads or the unit's rows compute on clamped (valid)
  // rows like the others and store nothing.
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + n;
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  // Kept blocks, attended in the order: diagonal block (the last kept id) first,
  // then the others in id order. Lane p of phys holds the physical block of
  // position 64 * phys_chunk + p.
  int nk = 0;
  while (nk < topk && sel[nk] >= 0) ++nk;
  if (nk == 0) return;                    // nothing kept (never produced by the selection)
  const int diag_b = sel[nk - 1];
  const int NH = 2 * nk;                  // half-blocks
  int phys_chunk = -1, phys = 0;
  auto phys_at = [&](int p) __attribute__((always_inline)) {
    if ((p >> 6) != phys_chunk) {
      phys_chunk = p >> 6;
      const int pl = 64 * phys_chunk + lane;
      phys = pl < nk ? bt[sel[pl == 0 ? nk - 1 : pl - 1]] : 0;
      wait_vm<0>();   // completes here, so no wait is needed where phys is read
    }
    return __builtin_amdgcn_readlane(phys, p & 63);
  };

  bf16x8 qf[KS];
  {
    const uint16_t *pq = q + (static_cast<size_t>(qrow) * Hq + head) * D + a * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(pq + ks * 16));
  }

  // Direct loads: instruction i of wave w fills the slot's chunks
  // (NW i + w) * 64 + lane; each lane fetches the global chunk that the swizzle
  // places there (byte offsets from the half-block's first K row / V^T column).
  uint32_t kgo[KCH], vgo[VCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int p = (NW * i + wave) * 64 + lane, rr = p / CH;
    kgo[i] = (rr * D + ((p % CH) ^ (srow_key(rr % 32) % CH)) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int p = (NW * i + wave) * 64 + lane, rr = p / VC;
    vgo[i] = (rr * kBlk + ((p % VC) ^ ((rr >> 1) % VC)) * 8) * 2;
  }
  auto issue = [&](int hb, auto r) __attribute__((always_inline)) {
    constexpr int R = decltype(r)::value % 4;
    const size_t off = (static_cast<size_t>(phys_at(hb >> 1)) * Hkv + j) * kBlk * D;
    const uint16_t *kg = kc + off + (hb & 1) * HB * D;
    const uint16_t *vg = vtc + off + (hb & 1) * HB;
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      load_lds16(lds_addr + R * KSLOT + (NW * i + wave) * 1024, kg, kgo[i]);
#pragma unroll
    for (int i = 0; i < VCH; ++i)
      load_lds16(lds_addr + VBASE + R * VSLOT + (NW * i + wave) * 1024, vg, vgo[i]);
  };

  // Per-lane LDS byte offsets of the operand fragments inside a slot: K fragment
  // ks of tile row srow_key(n), and V^T fragment (tile kt2 of the half-block,
  // 16-key half h) of row n of each 32-row d tile.
  int koff[KS], voff[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (srow_key(n) * CH + ((2 * ks + a) ^ (n % CH))) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = VBASE + (n * VC + ((2 * i + a) ^ ((n >> 1) % VC))) * 16;

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  f32x16 s = f32x16{};
  bf16x8 kf[KS], vf[2 * DT], pf[2];
  float m_ref = neg_inf();                // reference maximum, log2 units
  float l_run = 0.f;                      // this lane's share of the row sum

  auto read_k = [&](auto r, int kt2) __attribute__((always_inline)) {
    constexpr int R = decltype(r)::value % 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8 *>(lds + koff[ks] + R * KSLOT + kt2 * 32 * CH * 16);
  };
  auto read_v = [&](auto r, int kt2) __attribute__((always_inline)) {
    constexpr int R = decltype(r)::value % 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        vf[2 * dt + h] = *reinterpret_cast<const bf16x8 *>(lds + voff[2 * kt2 + h] + R * VSLOT +
                                                           dt * 32 * VC * 16);
  };

  // M phase: S^T = K Q^T of the current tile and O^T += V^T P^T of the previous
  // one, interleaved so that neither accumulation chain waits on itself.
  auto mphase = [&](auto pv_tag, auto qk_tag) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
    if constexpr (QK) s = f32x16{};
    constexpr int NI = KS > 2 * DT ? KS : 2 * DT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (QK)
        if (i < KS) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], s, 0, 0, 0);
      if constexpr (PV)
        if (i < 2 * DT)
          o[i / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[i % 2], o[i / 2], 0, 0, 0);
    }
  };

  // Softmax of tile kt (0..3) of a block; masked for the diagonal block.
  auto softmax = [&](auto mask_tag, int kt) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      const int lim = qpos - diag_b * kBlk - kt * 32;   // tile keys with offset > lim are masked
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i / 8) + 8 * a + (i % 8) > lim) s[i] = neg_inf();
    }
    float x = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) x = fmaxf(fmaxf(x, s[i]), s[i + 1]);
    x = fmaxf(x, s[15]);
    {   // max with the other half of the wave (same query column)
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
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
  };

  // Tiles 4 bp .. 4 bp + 3 of block position bp, whose half-blocks sit in ring
  // slots R0 and R0 + 1; the next block's are R0 + 2 and R0 + 3.
  auto block_step = [&](auto mask_tag, auto r0, int bp) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int R0 = decltype(r0)::value;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int T = 4 * bp + kt;
      if (MASK && kt == 0)
        mphase(std::false_type{}, std::true_type{});     // first tile: no previous P
      else
        mphase(std::true_type{}, std::true_type{});
      phase_barrier();
      if (kt == 0) read_k(ic<R0>{}, 1);
      else if (kt == 1) read_k(ic<R0 + 1>{}, 0);
      else if (kt == 2) read_k(ic<R0 + 1>{}, 1);
      else if (T + 1 < 4 * nk) read_k(ic<R0 + 2>{}, 0);
      if (kt < 2) read_v(ic<R0>{}, kt);
      else read_v(ic<R0 + 1>{}, kt - 2);
      softmax(mask_tag, kt);
      if (kt == 1) {
        if (2 * bp + 3 < NH) issue(2 * bp + 3, ic<R0 + 3>{});
      } else if (kt == 3) {
        if (2 * bp + 4 < NH) issue(2 * bp + 4, ic<R0 + 4>{});
      } else {
        const int hb = 2 * bp + kt / 2 + 1;   // first read in S(T + 1)
        if (hb < NH) {
          if (hb + 1 < NH) wait_vm<LPH>();    // half-block hb + 1 may stay in flight
          else wait_vm<0>();
        }
      }
      phase_barrier();
    }
  };

  // Prologue: half-blocks 0..2 requested, 0 waited for, K of tile 0 read.
  issue(0, ic<0>{});
  issue(1, ic<1>{});
  if (NH > 2) {
    issue(2, ic<2>{});
    wait_vm<2 * LPH>();
  } else {
    wait_vm<LPH>();
  }
  phase_barrier();
  read_k(ic<0>{}, 0);
  if (grp == 1) phase_barrier();

  block_step(std::true_type{}, ic<0>{}, 0);
  for (int bp = 1; bp < nk; bp += 2) {
    block_step(std::false_type{}, ic<2>{}, bp);
    if (bp + 1 >= nk) break;
    block_step(std::false_type{}, ic<0>{}, bp + 1);
  }
  mphase(std::true_type{}, std::false_type{});          // O^T += V^T P^T of the last tile
  if (grp == 0) phase_barrier();

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

// FP8 K/V: same tiles as attn_prefill_bf16_kernel, staged through registers.
template <int D>
__global__ __launch_bounds__(kPrefWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_fp8_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kc8,
    const uint8_t *__restrict__ vtc8, const uint8_t *__restrict__ ksc,
    const uint8_t *__restrict__ vsc, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int num_uj, int pairs, float c,
    uint16_t *__restrict__ out, float *__restrict__ lse) {
  constexpr int NW = kPrefWaves;
  constexpr int NT = NW * kWave;          // threads
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CH = D / 8;               // 16-byte bf16 chunks per K row
  constexpr int HB = kBlk / 2;            // keys per half-block
  constexpr int VC = HB / 8;              // 16-byte bf16 chunks per V^T row of a half-block
  constexpr int KSLOT = HB * CH * 16;
  constexpr int VSLOT = D * VC * 16;
  constexpr int VBASE = 2 * KSLOT;        // two K slots, then two V^T slots
  constexpr int UK = HB * D / 16;         // 16-code staging units of a half-block: K
  constexpr int UV = D * HB / 16;         //   and V^T
  constexpr int NS = D / 32;              // scale bytes per K row
  static_assert(UK <= NT && UV <= NT, "one staging unit per thread");
  __shared__ u32x4 smem[2 * (HB * CH + D * VC)];
  char *lds = reinterpret_cast<char *>(smem);

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

  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int a = lane / 32, n = lane % 32;
  const int hl = 2 * hp + wave / 4;
  const int slab = wave % 4;
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + n;
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  int nk = 0;
  while (nk < topk && sel[nk] >= 0) ++nk;
  if (nk == 0) return;
  const int diag_b = sel[nk - 1];
  const int NH = 2 * nk;                  // half-blocks, the diagonal block's first
  auto phys_of = [&](int p) { return bt[sel[p == 0 ? nk - 1 : p - 1]]; };

  bf16x8 qf[KS];
  {
    const uint16_t *pq = q + (static_cast<size_t>(qrow) * Hq + head) * D + a * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4 *>(pq + ks * 16));
  }

  // staging: K unit t = (row t / (D/16), 16 channels t % (D/16)); V^T unit t =
  // (d-row t / (HB/16), 16 keys t % (HB/16))
  const int k_row = t / (D / 16), k_m = t % (D / 16);
  const int v_row = t / (HB / 16), v_m = t % (HB / 16);
  uint4 kcode = {}, vcode = {}, vscale = {};
  uint32_t kscale = 0;
  auto load = [&](int hb) __attribute__((always_inline)) {
    const size_t blk = static_cast<size_t>(phys_of(hb >> 1)) * Hkv + j;   // (phys, j)
    const int key0 = (hb & 1) * HB;
    if (t < UK) {
      const size_t row = blk * kBlk + key0 + k_row;
      kcode = *reinterpret_cast<const uint4 *>(kc8 + row * D + k_m * 16);
      kscale = ksc[row * NS + k_m / 2];
    }
    if (t < UV) {
      vcode = *reinterpret_cast<const uint4 *>(vtc8 + (blk * D + v_row) * kBlk + key0 + v_m * 16);
      vscale = *reinterpret_cast<const uint4 *>(vsc + (blk * NS + v_row / 32) * kBlk + key0 +
                                                v_m * 16);
    }
  };
  auto store = [&](int slot) __attribute__((always_inline)) {
    if (t < UK) {
      const float sc = ldexpf(1.0f, static_cast<int>(kscale) - 127);
      const uint32_t w[4] = {kcode.x, kcode.y, kcode.z, kcode.w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, false));
        o[2 * i + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], sc, true));
      }
      const int sw = srow_key(k_row % 32) % CH;
      char *base = lds + slot * KSLOT + k_row * CH * 16;
      *reinterpret_cast<uint4 *>(base + ((2 * k_m) ^ sw) * 16) = uint4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<uint4 *>(base + ((2 * k_m + 1) ^ sw) * 16) = uint4{o[4], o[5], o[6], o[7]};
    }
    if (t < UV) {
      const uint32_t w[4] = {vcode.x, vcode.y, vcode.z, vcode.w};
      const uint32_t e[4] = {vscale.x, vscale.y, vscale.z, vscale.w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
        const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
        auto ex = [&](int b) { return static_cast<int>((e[i] >> (8 * b)) & 0xffu) - 127; };
        o[2 * i] = cvt_pk_bf16(ldexpf(lo.x, ex(0)), ldexpf(lo.y, ex(1)));
        o[2 * i + 1] = cvt_pk_bf16(ldexpf(hi.x, ex(2)), ldexpf(hi.y, ex(3)));
      }
      const int sw = (v_row >> 1) % VC;
      char *base = lds + VBASE + slot * VSLOT + v_row * VC * 16;
      *reinterpret_cast<uint4 *>(base + ((2 * v_m) ^ sw) * 16) = uint4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<uint4 *>(base + ((2 * v_m + 1) ^ sw) * 16) = uint4{o[4], o[5], o[6], o[7]};
    }
  };

  int koff[KS], voff[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = (srow_key(n) * CH + ((2 * ks + a) ^ (n % CH))) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = VBASE + (n * VC + ((2 * i + a) ^ ((n >> 1) % VC))) * 16;

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_ref = neg_inf(), l_run = 0.f;

  load(0);
  for (int hb = 0; hb < NH; ++hb) {
    const int slot = hb & 1;
    store(slot);
    __syncthreads();
    if (hb + 1 < NH) load(hb + 1);
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      bf16x8 kf[KS], vf[2 * DT], pf[2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8 *>(lds + koff[ks] + slot * KSLOT +
                                                   kt2 * 32 * CH * 16);
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
      if (hb < 2) {   // the diagonal block: keys past the query are masked
        const int lim = qpos - diag_b * kBlk - (hb * 2 + kt2) * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i / 8) + 8 * a + (i % 8) > lim) s[i] = neg_inf();
      }
      float x = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) x = fmaxf(x, s[i]);
      {
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                          false, false);
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
          vf[2 * dt + h] = *reinterpret_cast<const bf16x8 *>(
              lds + voff[2 * kt2 + h] + slot * VSLOT + dt * 32 * VC * 16);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i)
        o[i / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[i % 2], o[i / 2], 0, 0, 0);
    }
    __syncthreads();   // every wave is done with this slot before it is refilled
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

// fp32 attention, shared by prefill (units from the plan) and decode (T query rows
// per sequence, row r T + i at position seq_len - T + i). One thread per (query
// row, head).
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vtc,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const msa_unit_t *__restrict__ units, int T, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, float scale, float *__restrict__ out,
    float *__restrict__ lse) {
  const int u = blockIdx.x, head = blockIdx.y;
  msa_unit_t un;
  if (units != nullptr) {
    un = units[u];
  } else {
    const int r = u / T, p = seq_lens[r] - T + u % T;
    un = msa_unit_t{r, p / kBlk, u, 1, p};
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
                           int num_units, int T, const void *q, const int32_t *ids, int topk,
                           float scale, void *out, float *lse, hipStream_t st) {
  const dim3 grid(num_units, g.Hq);
  const float *qf = static_cast<const float *>(q);
  const float *kf = static_cast<const float *>(c.k_cache);
  const float *vf = static_cast<const float *>(c.v_cache);
  if (g.D == 64)
    attn_f32_kernel<64><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                              T, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                              g.nsel, scale, static_cast<float *>(out), lse);
  else
    attn_f32_kernel<128><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                               T, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                               g.nsel, scale, static_cast<float *>(out), lse);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                               const void *q, const int32_t *ids, int topk, float scale,
                               void *out, float *lse, hipStream_t st) {
  if (b.total_units == 0) return hipSuccess;
  if (!g.bf16)
    return launch_attn_f32(g, c, b.units, b.total_units, 1, q, ids, topk, scale, out, lse, st);
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
  if (g.fp8) {
    const uint8_t *k8 = static_cast<const uint8_t *>(c.k_cache);
    const uint8_t *v8 = static_cast<const uint8_t *>(c.v_cache);
    if (g.D == 64)
      attn_prefill_fp8_kernel<64><<<grid, NW * 64, 0, st>>>(
          qb, k8, v8, c.k_scale, c.v_scale, c.block_table, b.units, ids, topk,
          c.max_blocks_per_seq, g.Hq, g.Hkv, g.nsel, num_uj, pairs, sl2, ob, lse);
    else
      attn_prefill_fp8_kernel<128><<<grid, NW * 64, 0, st>>>(
          qb, k8, v8, c.k_scale, c.v_scale, c.block_table, b.units, ids, topk,
          c.max_blocks_per_seq, g.Hq, g.Hkv, g.nsel, num_uj, pairs, sl2, ob, lse);
    return hipGetLastError();
  }
  if (g.D == 64)
    attn_prefill_bf16_kernel<64><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, ob, lse);
  else
    attn_prefill_bf16_kernel<128><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, ob, lse);
  return hipGetLastError();
}

}  // namespace msa
