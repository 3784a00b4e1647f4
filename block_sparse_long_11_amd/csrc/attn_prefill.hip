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
// s <= pos(t). The causal test runs on every kept block that reaches the unit's
// first query (id >= tau): for the selection's own output that is the diagonal
// block alone, attended first, so the steady state has no masking work. A kept
// id past tau holds only future keys: it is not read (the diagonal's physical
// block stands in, fully masked). A row that sees no key at all (an id list
// without any block up to its diagonal) gets out = 0 and lse = -inf.
//
// bf16 path (MFMA 32x32x16, fp32 accumulate). A work-group of 8 waves owns (unit,
// KV head j, 2 query heads): 128 token rows x 2 heads, one wave per (head, 32
// tokens); waves w and w + 4 share a SIMD. With per-token selection it owns 32
// rows x 8 heads instead (the same query rows per K/V tile), and reads the union
// of those 32 rows' kept blocks. Per 32-key tile each wave computes
//   S^T = K . Q^T           (A = K rows from LDS, B = Q held in registers)
//   O^T += V^T . P^T        (A = V^T rows from LDS, B = P from S^T's registers)
// The S^T row m of a tile is fed key (m with bits 2 and 3 swapped): then lane
// half a, register 8h+jj holds key 16h + 8a + jj, which is exactly the k-index
// the P^T operand needs, so V^T is read in natural key order.
//
// Ping-pong: every tile T is split into an MFMA phase M(T) and a softmax phase
// S(T). M(T) accumulates S^T of tile T and, for tile T-1, forms the probabilities
// (against the reference maximum S(T-1) left), packs P, adds the row sum and
// accumulates O^T += V^T P^T, each score MFMA followed by a pair of exponentials
// so that the VALU work fills the matrix core's cycles, and (for a tile no mask
// touches) takes tile T's row maximum behind its P.V MFMAs. S(T) masks tile T (and
// then takes its row maximum), rescales O and the row sum when needed, and reads
// the operands of M(T+1) from LDS: it is kept short, since the softmax phase is
// the one that both waves of a SIMD end up waiting for at the barrier. Scores of
// even and odd tiles alternate between two accumulators, so tile T's scores wait
// in place for M(T+1). Phases end at
// work-group barriers, and waves 4..7 run one phase behind waves 0..3, so on
// every SIMD one wave is in an MFMA phase while the other is in a softmax phase.
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
#include <algorithm>
#include <type_traits>

#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPrefWaves = 8;
constexpr float kSlack = 8.f;

// Initial reference maximum (log2 units): finite and far below any logit, so a
// tile whose keys are all masked for a row before it has seen a visible key adds
// exp2(-inf) = 0 instead of NaN.
constexpr float kMaxFloor = -1e30f;

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

}  // namespace

// Per-query-token prefill (each token row keeps its own blocks): for every (unit,
// group, 32-row slab s of the unit's rows) the union of the slab's rows' kept ids,
// ascending, and for each union entry a 32-bit row mask (bit n: row 32 s + n
// keeps the block). The list of slab s starts at base(): inside the extent of its
// rows' own id lists, which bound the union's size.
struct TokenUnion {
  const int32_t *count;     // [U][n_sel][4] union sizes
  const int32_t *ids;       // union ids
  const uint32_t *masks;    // [entry]
  __device__ __forceinline__ size_t base(const msa_unit_t &un, int nsel, int g, int topk,
                                         int slab) const {
    return (static_cast<size_t>(un.row0) * nsel + static_cast<size_t>(g) * un.num_rows +
            static_cast<size_t>(32 * slab)) * topk;
  }
};

namespace {

// Output of one query row and head from O^T (lane half a holds d = 32 dt + 8 i4 +
// 4 a .. +3), the row sum and the reference maximum. A row without any visible
// key (sum 0) gets out = 0 and lse = -inf.
template <int D>
__device__ __forceinline__ void store_row(uint16_t *__restrict__ out, float *__restrict__ lse,
                                          int qrow, int Hq, int head, int a, const f32x16 *o,
                                          float sum, float m_ref) {
  constexpr int DT = D / 32;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
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
    lse[static_cast<size_t>(qrow) * Hq + head] =
        sum > 0.f ? (m_ref + __builtin_log2f(sum)) * kLn2 : neg_inf();
}

template <int D, bool PT>
__global__ __launch_bounds__(kPrefWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vtc, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ remap, const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int num_uj, int pairs, float c,
    TokenUnion tu, uint16_t *__restrict__ out, float *__restrict__ lse) {
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

  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int a = lane / 32, n = lane % 32;
  const int grp = wave / 4;               // 0 leads, 1 trails by one phase
  // Work-group hp of (unit, KV head j) takes 2 heads x the tile's 4 slabs of 32
  // rows (wave w: head 2 hp + w / 4, slab w % 4); per token, 8 heads x one slab
  // (slab hp % 4, heads 8 (hp / 4) + 2 (w % 4) + w / 4), so that its waves read
  // the union of that slab's lists alone
  const int slab = PT ? hp % 4 : wave % 4;
  const int hl = PT ? 8 * (hp / 4) + 2 * (wave % 4) + grp : 2 * hp + grp;
  // per token: the union of the slab's rows' lists (ascending) and its row masks
  const size_t ubase = PT ? tu.base(un, nsel, g, topk, slab) : 0;
  const int32_t *sel = PT ? tu.ids + ubase : ids + (static_cast<size_t>(u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  // Waves past the group's heads or the unit's rows compute on clamped (valid)
  // rows like the others and store nothing.
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + n;
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  // Kept blocks, attended in the order: the last kept id (the diagonal block, for
  // the selection's ascending output) first, then the others in list order. Lane
  // p of phys holds the K/V block of position 64 * phys_chunk + p: the cache's
  // (physical block, KV head j) index, or with remap (bf16 copies of FP8 blocks)
  // the copy's slot; lane p of logical holds its logical id; bit p of late marks
  // the positions whose block reaches the unit's first query (id >= tau) and so
  // takes the causal test.
  int nk = 0;
  if constexpr (PT)
    nk = tu.count[(static_cast<size_t>(u) * nsel + g) * 4 + slab];
  else
    while (nk < topk && sel[nk] >= 0) ++nk;
  if (nk == 0) {                          // nothing kept: no visible key
    if (active && row_ok) {
      f32x16 z[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) z[dt] = f32x16{};
      store_row<D>(out, lse, qrow, Hq, head, a, z, 0.f, 0.f);
    }
    return;
  }
  const int first_b = sel[nk - 1];
  const int NH = 2 * nk;                  // half-blocks
  int phys_chunk = -1, phys = 0;
  auto phys_at = [&](int p) __attribute__((always_inline)) {
    if ((p >> 6) != phys_chunk) {
      phys_chunk = p >> 6;
      const int pl = 64 * phys_chunk + lane;
      phys = 0;
      if (pl < nk) {
        const uint32_t bh = static_cast<uint32_t>(bt[min(sel[pl == 0 ? nk - 1 : pl - 1], un.tau)]) *
                                static_cast<uint32_t>(Hkv) + static_cast<uint32_t>(j);
        phys = remap != nullptr ? max(remap[bh], 0) : static_cast<int>(bh);
      }
      wait_vm<0>();   // completes here, so no wait is needed where phys is read
    }
    return __builtin_amdgcn_readlane(phys, p & 63);
  };
  // Same positions, for the causal test: lane p of logical holds the id, bit p
  // of late is set when that block reaches the unit's first query (id >= tau).
  // Loaded up front for the first 64 positions, so the loop reloads only past 64.
  // Per token, lane p of keepw also holds the row-mask word of this wave's 32
  // rows for that position (bit n: row 32 slab + n keeps the block).
  int late_chunk = -1, logical = 0;
  uint64_t late = 0;
  uint32_t keepw = 0;
  auto late_at = [&](int p) __attribute__((always_inline)) {
    if ((p >> 6) != late_chunk) {
      late_chunk = p >> 6;
      const int pl = 64 * late_chunk + lane;
      const int ix = pl == 0 ? nk - 1 : pl - 1;
      logical = pl < nk ? sel[ix] : 0;
      if constexpr (PT) keepw = pl < nk ? tu.masks[ubase + ix] : 0u;
      late = __ballot(pl < nk && logical >= un.tau);
    }
    return ((late >> (p & 63)) & 1) != 0;
  };
  late_at(0);

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
    const size_t off = static_cast<size_t>(static_cast<uint32_t>(phys_at(hb >> 1))) * kBlk * D;
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
  // S^T of the even and the odd tiles: a tile's scores stay in place from its M
  // phase, through its softmax phase, to the next M phase, which forms its
  // probabilities while it accumulates the next tile's scores in the other half
  f32x16 sc[2] = {f32x16{}, f32x16{}};
  bf16x8 kf[KS], vf[2 * DT], pf[2];
  float m_ref = kMaxFloor;                // reference maximum, log2 units
  float l_run = 0.f;                      // this lane's share of the row sum
  float xm = 0.f;                         // the tile maximum an M phase formed
  float thr = kMaxFloor + kSlack;         // m_ref + kSlack, kept with m_ref
  float msub = 0.f;                       // per token: +inf when this lane's row does not
                                          // keep the block of the tile in its softmax phase

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

  // M phase: S^T = K Q^T of the current tile into sc[P], and for the previous tile
  // (scores in sc[1 - P], its softmax phase done) the probabilities against the
  // reference maximum that phase left, their row sum and O^T += V^T P^T. The
  // score MFMAs do not wait for the probabilities, so the exponentials run while
  // the matrix core is busy with them. With MX (a tile no mask will touch) the
  // phase also takes the new tile's row maximum, behind the P.V MFMAs, so that
  // the softmax phase, the one both waves of a SIMD wait for, does not.
  auto mphase = [&](auto pv_tag, auto qk_tag, auto par, auto mx_tag) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
    constexpr bool MX = decltype(mx_tag)::value && QK;
    constexpr int P = decltype(par)::value;
    if constexpr (QK) {
      sc[P] = f32x16{};
#pragma unroll
      for (int i = 0; i < KS; ++i)
        sc[P] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], sc[P], 0, 0, 0);
    }
    if constexpr (PV) {
      const float mr = PT ? m_ref + msub : m_ref;   // a row without the block: exp2(-inf) = 0
      float ls = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 8; jj += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[1 - P][8 * h + jj], c, -mr));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[1 - P][8 * h + jj + 1], c, -mr));
          w[jj / 2] = cvt_pk_bf16(p0, p1);
          ls += p0 + p1;
        }
        pf[h] = as_bf16x8(uint4{w[0], w[1], w[2], w[3]});
      }
      l_run += ls;
      asm volatile("" : "+v"(l_run));   // summed here, not where the next phase uses it
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i)
        o[i / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[i % 2], o[i / 2], 0, 0, 0);
    }
    if constexpr (MX) {
      const f32x16 &s = sc[P];
      float x = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) x = fmaxf(fmaxf(x, s[i]), s[i + 1]);
      x = fmaxf(x, s[15]);
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
      xm = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * c;
      asm volatile("" : "+v"(xm));          // finished here, not in the softmax phase
    }
    if constexpr (PV && QK) {
      // issue order: each score MFMA followed by VALU work of the probabilities (fma,
      // exp), each P.V MFMA by the rest of it, the packing, the sums and the row
      // maximum, so that the VALU work fills the matrix core's cycles instead of
      // following them. At head_dim 128, 3 VALU instructions beside each score MFMA
      // and 5 beside each P.V MFMA measured best (4 and 4: 0.8-1.4% slower; 2-6 and
      // 6-3 slower still)
      constexpr int kSV = KS == 8 ? 3 : 32 / KS;
      constexpr int kPV = KS == 8 ? 5 : (24 + (MX ? 12 : 0)) / (2 * DT);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kSV, 0);
      }
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kPV, 0);
      }
    }
  };

  // Softmax phase of tile kt (0..3) of the block at position bp, scores in sc[P]:
  // the causal mask (the first block always, MASK; any other one only when it
  // reaches the unit's first query), the tile's row maximum (taken here only for a
  // masked tile; the M phase took it for the others) and, when it grew by more than
  // the slack, the rescale of O and the row sum.
  auto softmax = [&](auto mask_tag, auto par, int kt, int bp) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int P = decltype(par)::value;
    f32x16 &s = sc[P];
    bool do_mask = MASK;
    if constexpr (!MASK || PT) {
      const bool lt = late_at(bp);
      if constexpr (!MASK) do_mask = lt;
    }
    if (do_mask) {
      const int b = MASK ? first_b : __builtin_amdgcn_readlane(logical, bp & 63);
      const int lim = qpos - b * kBlk - kt * 32;   // tile keys with offset > lim are masked
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i / 8) + 8 * a + (i % 8) > lim) s[i] = neg_inf();
    }
    float x;
    if (!MASK && !do_mask) {
      x = xm;                               // formed in the tile's M phase
    } else {
      x = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) x = fmaxf(fmaxf(x, s[i]), s[i + 1]);
      x = fmaxf(x, s[15]);
      {   // max with the other half of the wave (same query column)
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                          false, false);
        x = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * c;
      }
    }
    // per token: a row that does not keep this block sees none of its keys (its
    // maximum ignores the tile, its probabilities are exp2(-inf) = 0)
    if constexpr (PT) {
      const bool keep = ((__builtin_amdgcn_readlane(keepw, bp & 63) >> n) & 1u) != 0;
      x = keep ? x : neg_inf();
      msub = keep ? 0.f : pos_inf();
    }
    const bool need = x > thr;
    if (__any(need)) {
      const float nm = need ? x : m_ref;
      const float al = __builtin_amdgcn_exp2f(m_ref - nm);
      m_ref = nm;
      thr = m_ref + kSlack;
      l_run *= al;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= al;
    }
  };

  // Tiles 4 bp .. 4 bp + 3 of block position bp, whose half-blocks sit in ring
  // slots R0 and R0 + 1; the next block's are R0 + 2 and R0 + 3. Tile kt's scores
  // use sc[kt % 2] (four tiles a block keep the parity of every block's tiles).
  auto block_step = [&](auto mask_tag, auto r0, int bp) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int R0 = decltype(r0)::value;
    auto tile = [&](auto ktc) __attribute__((always_inline)) {
      constexpr int kt = decltype(ktc)::value;
      constexpr int P = kt % 2;
      const int T = 4 * bp + kt;
      // the tile maximum in the M phase for the blocks with no static mask
      using MXT = std::integral_constant<bool, !MASK>;
      if (MASK && kt == 0)
        mphase(std::false_type{}, std::true_type{}, ic<P>{}, MXT{});   // no previous P
      else
        mphase(std::true_type{}, std::true_type{}, ic<P>{}, MXT{});
      phase_barrier();
      if constexpr (kt == 0) read_k(ic<R0>{}, 1);
      else if constexpr (kt == 1) read_k(ic<R0 + 1>{}, 0);
      else if constexpr (kt == 2) read_k(ic<R0 + 1>{}, 1);
      else if (T + 1 < 4 * nk) read_k(ic<R0 + 2>{}, 0);
      if constexpr (kt < 2) read_v(ic<R0>{}, kt);
      else read_v(ic<R0 + 1>{}, kt - 2);
      softmax(mask_tag, ic<P>{}, kt, bp);
      if constexpr (kt == 1) {
        if (2 * bp + 3 < NH) issue(2 * bp + 3, ic<R0 + 3>{});
      } else if constexpr (kt == 3) {
        if (2 * bp + 4 < NH) issue(2 * bp + 4, ic<R0 + 4>{});
      } else {
        const int hb = 2 * bp + kt / 2 + 1;   // first read in S(T + 1)
        if (hb < NH) {
          if (hb + 1 < NH) wait_vm<LPH>();    // half-block hb + 1 may stay in flight
          else wait_vm<0>();
        }
      }
      phase_barrier();
    };
    tile(ic<0>{});
    tile(ic<1>{});
    tile(ic<2>{});
    tile(ic<3>{});
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
  // probabilities and O^T += V^T P^T of the last tile (odd: its scores are in sc[1])
  mphase(std::true_type{}, std::false_type{}, ic<0>{}, std::false_type{});
  if (grp == 0) phase_barrier();

  if (!active) return;
  float sum;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (!row_ok) return;
  store_row<D>(out, lse, qrow, Hq, head, a, o, sum, m_ref);
}

// FP8 K/V: same tiles as attn_prefill_bf16_kernel, staged through registers.
template <int D, bool PT>
__global__ __launch_bounds__(kPrefWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_fp8_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kc8,
    const uint8_t *__restrict__ vtc8, const uint8_t *__restrict__ ksc,
    const uint8_t *__restrict__ vsc, const int32_t *__restrict__ block_table,
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk,
    int max_blocks, int Hq, int Hkv, int nsel, int num_uj, int pairs, float c,
    TokenUnion tu, uint16_t *__restrict__ out, float *__restrict__ lse) {
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

  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int a = lane / 32, n = lane % 32;
  // heads and slabs of the waves as in the bf16 kernel
  const int slab = PT ? hp % 4 : wave % 4;
  const int hl = PT ? 8 * (hp / 4) + 2 * (wave % 4) + wave / 4 : 2 * hp + wave / 4;
  const size_t ubase = PT ? tu.base(un, nsel, g, topk, slab) : 0;
  const int32_t *sel = PT ? tu.ids + ubase : ids + (static_cast<size_t>(u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  const bool active = hl < G && slab * 32 < un.num_rows;
  const int head = j * G + min(hl, G - 1);
  const int row_in_tile = slab * 32 + n;
  const bool row_ok = row_in_tile < un.num_rows;
  const int qrow = un.row0 + min(row_in_tile, un.num_rows - 1);
  const int qpos = row_ok ? un.pos0 + row_in_tile : 0x7fffffff;

  int nk = 0;
  if constexpr (PT)
    nk = tu.count[(static_cast<size_t>(u) * nsel + g) * 4 + slab];
  else
    while (nk < topk && sel[nk] >= 0) ++nk;
  if (nk == 0) {                          // nothing kept: no visible key
    if (active && row_ok) {
      f32x16 z[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) z[dt] = f32x16{};
      store_row<D>(out, lse, qrow, Hq, head, a, z, 0.f, 0.f);
    }
    return;
  }
  const int NH = 2 * nk;                  // half-blocks, the last kept id's first
  // logical id at position p (the last kept id first); a block past tau holds
  // only future keys and is read from the diagonal's physical block, masked
  auto ix_of = [&](int p) { return p == 0 ? nk - 1 : p - 1; };
  auto id_of = [&](int p) { return sel[ix_of(p)]; };
  auto phys_of = [&](int p) { return bt[min(id_of(p), un.tau)]; };

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
  float m_ref = kMaxFloor, l_run = 0.f;

  load(0);
  for (int hb = 0; hb < NH; ++hb) {
    const int slot = hb & 1;
    store(slot);
    __syncthreads();
    if (hb + 1 < NH) load(hb + 1);
    // the causal test, for a block that reaches the unit's first query
    const int blk_id = id_of(hb >> 1);
    const bool late = blk_id >= un.tau;
    // per token: whether this lane's row keeps the block
    bool keep = true;
    if constexpr (PT) keep = ((tu.masks[ubase + ix_of(hb >> 1)] >> n) & 1u) != 0;
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
      if (late) {     // keys past the query are masked
        const int lim = qpos - blk_id * kBlk - ((hb & 1) * 2 + kt2) * 32;
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
      x = keep ? x : neg_inf();
      const float mr_add = keep ? 0.f : pos_inf();
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
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + jj], c, -(m_ref + mr_add)));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * h + jj + 1], c, -(m_ref + mr_add)));
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
  store_row<D>(out, lse, qrow, Hq, head, a, o, sum, m_ref);
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
    int max_blocks, int Hq, int Hkv, int nsel, float scale, bool per_token,
    float *__restrict__ out, float *__restrict__ lse) {
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
  const int qrow = un.row0 + t, qpos = un.pos0 + t;
  // per token, every query row has its own list
  const int32_t *sel = ids + (static_cast<size_t>(per_token ? qrow : u) * nsel + g) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  float qv[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = q[(static_cast<size_t>(qrow) * Hq + head) * D + d];
    acc[d] = 0.f;
  }
  float m = neg_inf(), l = 0.f;
  for (int slot = 0; slot < topk; ++slot) {
    const int b = sel[slot];
    if (b < 0) break;
    if (b > qpos / kBlk) continue;       // only future keys
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
  // a row without any visible key gets out = 0 and lse = -inf
  float *op = out + (static_cast<size_t>(qrow) * Hq + head) * D;
  for (int d = 0; d < D; ++d) op[d] = l > 0.f ? acc[d] / l : 0.f;
  if (lse != nullptr) lse[static_cast<size_t>(qrow) * Hq + head] = l > 0.f ? m + logf(l) : neg_inf();
}

hipError_t launch_attn_f32(const Geom &g, const msa_cache_t &c, const msa_unit_t *units,
                           int num_units, int T, const void *q, const int32_t *ids, int topk,
                           float scale, void *out, float *lse, hipStream_t st,
                           bool per_token) {
  const dim3 grid(num_units, g.Hq);
  const float *qf = static_cast<const float *>(q);
  const float *kf = static_cast<const float *>(c.k_cache);
  const float *vf = static_cast<const float *>(c.v_cache);
  MSA_LOG_LAUNCH("attn_f32_kernel", grid, 128, 0);
  if (g.D == 64)
    attn_f32_kernel<64><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                              T, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                              g.nsel, scale, per_token, static_cast<float *>(out),
                                              lse);
  else
    attn_f32_kernel<128><<<grid, 128, 0, st>>>(qf, kf, vf, c.block_table, c.seq_lens, units,
                                               T, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
                                               g.nsel, scale, per_token, static_cast<float *>(out),
                                               lse);
  return hipGetLastError();
}

// Union of the kept lists of one (unit, group, 32-row slab) for the per-token
// prefill: one work-group per triple. Each row's list ends at its first -1; ids
// outside [0, tau] hold no key visible to the unit's rows and are left out. The
// ids set bits of an LDS bitmap over [0, tau]; an exclusive scan of the words'
// popcounts gives every block its rank, so the union comes out ascending; each
// kept (row, id) then ORs the row's bit into the mask word of its block's entry
// (zeroed first).
constexpr int kUnionThreads = 256;
constexpr int kUnionLdsMasks = 2048;      // most row-mask words a union keeps in LDS

__global__ __launch_bounds__(kUnionThreads) void token_union_kernel(
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk, int nsel,
    TokenUnion tu, int32_t *__restrict__ count, int32_t *__restrict__ uids,
    uint32_t *__restrict__ masks, int mcap) {
  // [W] bitmap, [W] exclusive prefix, then mcap entries' row masks
  extern __shared__ uint32_t bits[];
  __shared__ int nkr[32];                 // each row's list length
  __shared__ int wsum[kUnionThreads / kWave];
  const int u = blockIdx.x, g = blockIdx.y, slab = blockIdx.z, t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const msa_unit_t un = units[u];
  const int n = min(32, un.num_rows - 32 * slab), tau = un.tau;   // rows of the slab
  const size_t ci = (static_cast<size_t>(u) * nsel + g) * 4 + slab;
  if (n <= 0) {                           // a slab past the unit's rows
    if (t == 0) count[ci] = 0;
    return;
  }
  const int W = tau / 32 + 1;             // words covering blocks [0, tau]
  uint32_t *pre = bits + W;
  const size_t base = tu.base(un, nsel, g, topk, slab);
  auto row_ids = [&](int i) {
    return ids + (static_cast<size_t>(un.row0 + 32 * slab + i) * nsel + g) * topk;
  };
  for (int w = t; w < W; w += kUnionThreads) bits[w] = 0u;
  // each row's list length: the position of its first -1 (topk if none), from
  // independent loads rather than a walk along the row
  if (t < n) nkr[t] = topk;
  __syncthreads();
  for (int e = t; e < n * topk; e += kUnionThreads) {
    const int i = e / topk, k = e % topk;
    if (row_ids(i)[k] < 0) atomicMin(&nkr[i], k);
  }
  __syncthreads();
  for (int e = t; e < n * topk; e += kUnionThreads) {
    const int i = e / topk, k = e % topk;
    if (k >= nkr[i]) continue;
    const int b = row_ids(i)[k];
    if (b >= 0 && b <= tau) atomicOr(&bits[b / 32], 1u << (b % 32));
  }
  __syncthreads();
  // exclusive scan of popcounts: thread t owns words [t * per, (t + 1) * per)
  const int per = (W + kUnionThreads - 1) / kUnionThreads;
  const int w0 = min(W, t * per), w1 = min(W, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(bits[w]);
  int x = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  int before = x - local;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int total = 0;
  for (int w = 0; w < kUnionThreads / kWave; ++w) total += wsum[w];
  for (int w = w0; w < w1; ++w) {
    pre[w] = before;
    uint32_t m = bits[w];
    while (m != 0u) {
      const int bit = __ffs(m) - 1;
      uids[base + before++] = w * 32 + bit;
      m &= m - 1u;
    }
  }
  // the row masks are ORed together in LDS when the union fits there (then
  // written out whole), else in place with global atomics
  uint32_t *lm = pre + W;
  const bool in_lds = total <= mcap;
  if (in_lds) {
    for (int e = t; e < total; e += kUnionThreads) lm[e] = 0u;
  } else {
    for (int e = t; e < total; e += kUnionThreads) masks[base + e] = 0u;
  }
  if (t == 0) count[ci] = total;
  if (!in_lds) __threadfence();           // the zeros reach L2 before the ORs below
  __syncthreads();
  for (int e = t; e < n * topk; e += kUnionThreads) {
    const int i = e / topk, k = e % topk;
    if (k >= nkr[i]) continue;
    const int b = row_ids(i)[k];
    if (b < 0 || b > tau) continue;
    const int pos = pre[b / 32] + __popc(bits[b / 32] & ((1u << (b % 32)) - 1u));
    if (in_lds)
      atomicOr(&lm[pos], 1u << i);
    else
      atomicOr(&masks[base + pos], 1u << i);
  }
  if (in_lds) {
    __syncthreads();
    for (int e = t; e < total; e += kUnionThreads) masks[base + e] = lm[e];
  }
}

// FP8 caches, staged: every (physical block, KV head) that a unit keeps is
// converted once into bf16 copies laid out like the bf16 caches' blocks (K as
// [128][D], V^T as [D][128]), and the bf16 kernel attends the copies. The
// conversion is exact (an E4M3 code times a power of two is a bf16 value), so the
// result equals attending the FP8 blocks directly up to the order of the fp32
// sums; each block is converted once instead of once per work-group that reads it.
// Two layouts, both of H_kv * min(num_phys, units * topk) copies:
//   direct (num_phys <= units * topk): copy (block, head) sits where the cache
//     holds it; the lists set a flag per kept pair, and the conversion takes the
//     flagged pairs and clears their flags (a flag left set, e.g. by a workspace's
//     first contents, only costs a conversion that nothing reads);
//   claimed (larger caches): the slot map is reset, the first list entry to reach
//     a pair claims the next slot for it, and the attention looks slots up.
struct Stage {
  int32_t *count;       // claimed: slots in use
  int32_t *slot_of;     // [num_phys * Hkv]: claimed: slot of (block, head), -1 when not
                        // kept; direct: nonzero when kept
  int32_t *src;         // claimed: [S] (block, head) of each slot
  uint16_t *k;          // [S][128][D]
  uint16_t *vt;         // [S][D][128]
  int64_t S;            // copies
  bool direct;
};

namespace {

constexpr int kStageThreads = 256;

size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t stage_slots(const Geom &g, int64_t num_phys, int total_units, int topk) {
  return static_cast<int64_t>(g.Hkv) *
         std::min<int64_t>(num_phys, static_cast<int64_t>(total_units) * topk);
}

Stage stage_layout(const Geom &g, int64_t num_phys, int total_units, int topk, char *ws) {
  Stage st{};
  st.S = stage_slots(g, num_phys, total_units, topk);
  st.direct = num_phys <= static_cast<int64_t>(total_units) * topk;
  const size_t map = al256(static_cast<size_t>(num_phys) * g.Hkv * 4);
  const size_t src = al256(static_cast<size_t>(st.S) * 4);
  const size_t blk = static_cast<size_t>(st.S) * kBlk * g.D * 2;
  st.count = reinterpret_cast<int32_t *>(ws);
  st.slot_of = reinterpret_cast<int32_t *>(ws + 256);
  st.src = reinterpret_cast<int32_t *>(ws + 256 + map);
  st.k = reinterpret_cast<uint16_t *>(ws + 256 + map + src);
  st.vt = reinterpret_cast<uint16_t *>(ws + 256 + map + src + blk);
  return st;
}

__global__ __launch_bounds__(kStageThreads) void stage_reset_kernel(Stage st, int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * kStageThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStageThreads + threadIdx.x; i < n;
       i += step)
    st.slot_of[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *st.count = 0;
}

// One wave per (unit, selection group) list, a lane per id, 64 at a time. Lists
// end at their first negative id; an id past the diagonal is read from the
// diagonal's block, as the attention kernel reads it. Direct: every kept pair's
// flag is set. Claimed: a lane that finds its pair unclaimed claims it, and the
// wave's claims take consecutive slots from one atomic add.
template <bool DIRECT>
__global__ __launch_bounds__(kStageThreads) void stage_mark_kernel(
    const msa_unit_t *__restrict__ units, const int32_t *__restrict__ ids, int topk, int nsel,
    int Hkv, const int32_t *__restrict__ block_table, int max_blocks, int64_t num_phys,
    int rows, Stage st) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (kStageThreads / kWave) + threadIdx.x / kWave;
  if (e >= rows) return;                  // uniform over the wave
  const int u = e / nsel, g = e % nsel;
  const msa_unit_t un = units[u];
  const int32_t *row = ids + static_cast<size_t>(e) * topk;
  const int32_t *bt = block_table + static_cast<size_t>(un.r) * max_blocks;
  const int heads = Hkv / nsel;          // the KV heads that read group g's list
  for (int c0 = 0; c0 < topk; c0 += kWave) {
    const int i = c0 + lane;
    const int id = i < topk ? row[i] : -1;
    const uint64_t neg = __ballot(id < 0);
    const int end = neg != 0 ? __builtin_ctzll(neg) : kWave;   // first ended lane
    bool live = lane < end;
    int pb = 0;
    if (live) {
      pb = bt[min(id, un.tau)];
      live = pb >= 0 && pb < num_phys;
    }
    for (int h = 0; h < heads; ++h) {
      const uint32_t bh = static_cast<uint32_t>(pb) * static_cast<uint32_t>(Hkv) +
                          static_cast<uint32_t>(heads == 1 ? g : h);
      if constexpr (DIRECT) {
        if (live) st.slot_of[bh] = 1;
        continue;
      }
      const bool claim = live && atomicCAS(&st.slot_of[bh], -1, -2) == -1;
      const uint64_t cm = __ballot(claim);
      if (cm == 0) continue;
      const int first = __builtin_ctzll(cm);
      int base = 0;
      if (lane == first) base = atomicAdd(st.count, __popcll(cm));
      base = __builtin_amdgcn_readlane(base, first);
      const int slot = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                  static_cast<uint32_t>(cm >> 32),
                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cm), 0u)));
      if (claim && slot < st.S) {
        st.src[slot] = static_cast<int32_t>(bh);
        st.slot_of[bh] = slot;
      }
    }
    if (end < kWave) break;
  }
}

// One work-group per copy: K rows in 16-code chunks of one key (one scale each)
// and V^T rows in 16-key chunks of one channel (a scale per key). Direct: work-
// group b converts pair b if its flag is set and then clears the flag; claimed:
// work-group s converts the pair that claimed slot s.
template <int D, bool DIRECT>
__global__ __launch_bounds__(kStageThreads) void stage_convert_kernel(
    const uint8_t *__restrict__ k8, const uint8_t *__restrict__ v8,
    const uint8_t *__restrict__ ksc, const uint8_t *__restrict__ vsc, Stage st) {
  constexpr int NS = D / 32;              // scale bytes per K row / V^T rows per scale row
  const int slot = blockIdx.x;
  size_t bh;
  if constexpr (DIRECT) {
    const bool kept = st.slot_of[slot] != 0;
    __syncthreads();                      // every thread has read the flag before it is cleared
    if (!kept) return;
    bh = static_cast<size_t>(slot);
  } else {
    if (slot >= min(static_cast<int64_t>(*st.count), st.S)) return;
    bh = static_cast<uint32_t>(st.src[slot]);
  }
  const uint8_t *kb = k8 + bh * kBlk * D;
  const uint8_t *ks = ksc + bh * kBlk * NS;
  uint16_t *ko = st.k + static_cast<size_t>(slot) * kBlk * D;
  constexpr int IT = kBlk * D / 16 / kStageThreads;   // 16-code chunks per thread, K and V^T
  static_assert(IT * kStageThreads * 16 == kBlk * D, "chunks per thread");
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = it * kStageThreads + threadIdx.x;
    const int key = c / (D / 16), m = c % (D / 16);
    const uint4 w = *reinterpret_cast<const uint4 *>(kb + static_cast<size_t>(key) * D + m * 16);
    const float sc = ldexpf(1.0f, static_cast<int>(ks[key * NS + m / 2]) - 127);
    const uint32_t wi[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_bit_cast(uint32_t,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wi[i], sc, false));
      o[2 * i + 1] = __builtin_bit_cast(uint32_t,
                                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wi[i], sc, true));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(ko + static_cast<size_t>(key) * D + m * 16);
    dst[0] = uint4{o[0], o[1], o[2], o[3]};
    dst[1] = uint4{o[4], o[5], o[6], o[7]};
  }
  const uint8_t *vb = v8 + bh * D * kBlk;
  const uint8_t *vs = vsc + bh * NS * kBlk;
  uint16_t *vo = st.vt + static_cast<size_t>(slot) * D * kBlk;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = it * kStageThreads + threadIdx.x;
    const int d = c / (kBlk / 16), m = c % (kBlk / 16);
    const uint4 w = *reinterpret_cast<const uint4 *>(vb + static_cast<size_t>(d) * kBlk + m * 16);
    const uint4 e = *reinterpret_cast<const uint4 *>(vs + static_cast<size_t>(d / 32) * kBlk +
                                                     m * 16);
    const uint32_t wi[4] = {w.x, w.y, w.z, w.w};
    const uint32_t ei[4] = {e.x, e.y, e.z, e.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wi[i], false);
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wi[i], true);
      auto ex = [&](int b) { return static_cast<int>((ei[i] >> (8 * b)) & 0xffu) - 127; };
      o[2 * i] = cvt_pk_bf16(ldexpf(lo.x, ex(0)), ldexpf(lo.y, ex(1)));
      o[2 * i + 1] = cvt_pk_bf16(ldexpf(hi.x, ex(2)), ldexpf(hi.y, ex(3)));
    }
    uint4 *dst = reinterpret_cast<uint4 *>(vo + static_cast<size_t>(d) * kBlk + m * 16);
    dst[0] = uint4{o[0], o[1], o[2], o[3]};
    dst[1] = uint4{o[4], o[5], o[6], o[7]};
  }
  if constexpr (DIRECT)
    if (threadIdx.x == 0) st.slot_of[slot] = 0;
}

template <int D>
void stage_kept_blocks(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                       const int32_t *ids, int topk, const Stage &sg, hipStream_t st) {
  const int rows = b.total_units * g.nsel;
  constexpr int kMarkRows = kStageThreads / kWave;   // one wave per list
  const int mark_groups = (rows + kMarkRows - 1) / kMarkRows;
  const uint8_t *k8 = static_cast<const uint8_t *>(c.k_cache);
  const uint8_t *v8 = static_cast<const uint8_t *>(c.v_cache);
  const dim3 cgrid(static_cast<unsigned>(sg.S));
  if (sg.direct) {
    MSA_LOG_LAUNCH("stage_mark_kernel (in place)", mark_groups, kStageThreads, 0);
    MSA_LOG_LAUNCH("stage_convert_kernel (in place)", cgrid, kStageThreads, 0);
    stage_mark_kernel<true><<<mark_groups, kStageThreads, 0, st>>>(
        b.units, ids, topk, g.nsel, g.Hkv, c.block_table, c.max_blocks_per_seq,
        c.num_phys_blocks, rows, sg);
    stage_convert_kernel<D, true><<<cgrid, kStageThreads, 0, st>>>(k8, v8, c.k_scale, c.v_scale,
                                                                  sg);
    return;
  }
  const int64_t n = c.num_phys_blocks * g.Hkv;
  const int reset_groups = static_cast<int>(std::min<int64_t>((n + kStageThreads - 1) /
                                                              kStageThreads, 1024));
  MSA_LOG_LAUNCH("stage_reset_kernel", reset_groups, kStageThreads, 0);
  MSA_LOG_LAUNCH("stage_mark_kernel (claimed slots)", mark_groups, kStageThreads, 0);
  MSA_LOG_LAUNCH("stage_convert_kernel (claimed slots)", cgrid, kStageThreads, 0);
  stage_reset_kernel<<<reset_groups, kStageThreads, 0, st>>>(sg, n);
  stage_mark_kernel<false><<<mark_groups, kStageThreads, 0, st>>>(
      b.units, ids, topk, g.nsel, g.Hkv, c.block_table, c.max_blocks_per_seq, c.num_phys_blocks,
      rows, sg);
  stage_convert_kernel<D, false><<<cgrid, kStageThreads, 0, st>>>(k8, v8, c.k_scale, c.v_scale,
                                                                 sg);
}

}  // namespace

size_t prefill_stage_bytes(const Geom &g, int64_t num_phys, int total_units, int topk) {
  if (!g.fp8 || total_units <= 0 || topk <= 0 || num_phys <= 0) return 0;
  const int64_t S = stage_slots(g, num_phys, total_units, topk);
  return 256 + al256(static_cast<size_t>(num_phys) * g.Hkv * 4) + al256(static_cast<size_t>(S) * 4) +
         2 * static_cast<size_t>(S) * kBlk * g.D * 2;
}

size_t tokens_workspace_bytes(const Geom &g, int total_units, int total_q, int topk) {
  if (!g.bf16) return 0;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t entries = static_cast<size_t>(total_q) * g.nsel * topk;
  return al(static_cast<size_t>(total_units) * g.nsel * 16) + al(entries * 4) + al(entries * 4);
}

template <bool PT>
hipError_t launch_prefill_attention(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                    const void *q, const int32_t *ids, int topk, float scale,
                                    void *workspace, void *stage_ws, void *out, float *lse,
                                    hipStream_t st);

hipError_t launch_attn_prefill(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                               const void *q, const int32_t *ids, int topk, float scale,
                               void *stage_ws, void *out, float *lse, hipStream_t st) {
  return launch_prefill_attention<false>(g, c, b, q, ids, topk, scale, nullptr, stage_ws, out,
                                         lse, st);
}

hipError_t launch_attn_prefill_tokens(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                      const void *q, const int32_t *ids, int topk, float scale,
                                      void *workspace, void *out, float *lse, hipStream_t st) {
  return launch_prefill_attention<true>(g, c, b, q, ids, topk, scale, workspace, nullptr, out,
                                        lse, st);
}

template <bool PT>
hipError_t launch_prefill_attention(const Geom &g, const msa_cache_t &c, const msa_batch_t &b,
                                    const void *q, const int32_t *ids, int topk, float scale,
                                    void *workspace, void *stage_ws, void *out, float *lse,
                                    hipStream_t st) {
  if (b.total_units == 0) return hipSuccess;
  if (!g.bf16)
    return launch_attn_f32(g, c, b.units, b.total_units, 1, q, ids, topk, scale, out, lse, st,
                           PT);
  TokenUnion tu{nullptr, nullptr, nullptr};
  if constexpr (PT) {
    auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const size_t entries = static_cast<size_t>(b.total_q) * g.nsel * topk;
    char *ws = static_cast<char *>(workspace);
    int32_t *cnt = reinterpret_cast<int32_t *>(ws);
    int32_t *uids = reinterpret_cast<int32_t *>(ws + al(static_cast<size_t>(b.total_units) *
                                                         g.nsel * 16));
    uint32_t *msk = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(uids) +
                                                 al(entries * 4));
    tu = TokenUnion{cnt, uids, msk};
    const int W = c.max_blocks_per_seq / 32 + 1;   // bitmap words for any tau of the table
    // LDS row masks for unions of up to mcap blocks (a slab's union holds at most
    // W * 32 ids, and at most 32 rows times topk), when there are at most 2048
    const int64_t most = std::min<int64_t>(int64_t(W) * 32, int64_t(32) * topk);
    const int mcap = most <= kUnionLdsMasks ? static_cast<int>(most) : 0;
    const size_t lds = (2 * size_t(W) + size_t(mcap)) * sizeof(uint32_t);
    const dim3 ugrid(b.total_units, g.nsel, 4);
    MSA_LOG_LAUNCH("token_union_kernel", ugrid, kUnionThreads, lds);
    token_union_kernel<<<ugrid, kUnionThreads, lds, st>>>(b.units, ids, topk, g.nsel, tu, cnt,
                                                          uids, msk, mcap);
  }
  constexpr int NW = kPrefWaves;
  // work-groups per (unit, KV head): of 2 heads each, per token of 8 heads x 4 slabs
  const int pairs = PT ? 4 * ((g.G() + 7) / 8) : (g.G() + NW / 4 - 1) / (NW / 4);
  const int num_uj = b.total_units * g.Hkv;
  const int groups8 = (num_uj + 7) / 8;
  const dim3 grid(groups8 * 8 * pairs);
  const uint16_t *qb = static_cast<const uint16_t *>(q);
  const uint16_t *kb = static_cast<const uint16_t *>(c.k_cache);
  const uint16_t *vb = static_cast<const uint16_t *>(c.v_cache);
  uint16_t *ob = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  const int32_t *remap = nullptr;
  if (g.fp8 && stage_ws != nullptr && !PT) {   // kept blocks to bf16 once, then the bf16 kernel
    const Stage sg = stage_layout(g, c.num_phys_blocks, b.total_units, topk,
                                  static_cast<char *>(stage_ws));
    if (g.D == 64)
      stage_kept_blocks<64>(g, c, b, ids, topk, sg, st);
    else
      stage_kept_blocks<128>(g, c, b, ids, topk, sg, st);
    kb = sg.k;
    vb = sg.vt;
    remap = sg.direct ? nullptr : sg.slot_of;   // direct copies sit where the cache's blocks do
  } else if (g.fp8) {
    const uint8_t *k8 = static_cast<const uint8_t *>(c.k_cache);
    const uint8_t *v8 = static_cast<const uint8_t *>(c.v_cache);
    MSA_LOG_LAUNCH(PT ? "attn_prefill_fp8_kernel (per token)" : "attn_prefill_fp8_kernel", grid,
                   NW * 64, 0);
    if (g.D == 64)
      attn_prefill_fp8_kernel<64, PT><<<grid, NW * 64, 0, st>>>(
          qb, k8, v8, c.k_scale, c.v_scale, c.block_table, b.units, ids, topk,
          c.max_blocks_per_seq, g.Hq, g.Hkv, g.nsel, num_uj, pairs, sl2, tu, ob, lse);
    else
      attn_prefill_fp8_kernel<128, PT><<<grid, NW * 64, 0, st>>>(
          qb, k8, v8, c.k_scale, c.v_scale, c.block_table, b.units, ids, topk,
          c.max_blocks_per_seq, g.Hq, g.Hkv, g.nsel, num_uj, pairs, sl2, tu, ob, lse);
    return hipGetLastError();
  }
  MSA_LOG_LAUNCH(PT ? "attn_prefill_bf16_kernel (per token)" : "attn_prefill_bf16_kernel", grid,
                 NW * 64, 0);
  if (g.D == 64)
    attn_prefill_bf16_kernel<64, PT><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, remap, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, tu, ob, lse);
  else
    attn_prefill_bf16_kernel<128, PT><<<grid, NW * 64, 0, st>>>(
        qb, kb, vb, c.block_table, remap, b.units, ids, topk, c.max_blocks_per_seq, g.Hq, g.Hkv,
        g.nsel, num_uj, pairs, sl2, tu, ob, lse);
  return hipGetLastError();
}

}  // namespace msa
