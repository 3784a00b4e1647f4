// Block top-k selection (step 2 of MSA).
//
// [feat] models.inteligile.com "MiniMax-M3", table "Checked in its code", row
// "Indexer-selected sparse attention": topk = min(topk_blocks, num_key_blocks) and
// selections whose score is -inf become -1. Method list "Exp-free TopK kernel":
// raw scores are ranked directly, no softmax.
//
// Rows of up to 512 entries: one wave per row (topk_rows_wave_kernel). Longer rows:
// one work-group per row. Scores are mapped to order-preserving uint32 keys and
// the K-th largest key is found exactly by a 4-pass radix select (8 bits per
// pass, LDS histograms with integer atomics, so the result does not depend on
// thread timing). The kept entries (key above the threshold, plus the lowest
// indices among those equal to it) are then written in ascending index order by
// two block-wide prefix scans. Entries equal to -inf are never kept.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {
namespace {

constexpr int kTopkThreads = 512;

// -0.0 and +0.0 are the same score (ties go to the lower index), so both map to
// the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = (f == 0.f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t kNegInfKey = 0x007fffffu;   // order_key(-inf)

// Exclusive prefix sum over the work-group; also returns the total.
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    const int s = tmp[w];
    base += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const float *__restrict__ scores, int row_len, int topk, int32_t *__restrict__ ids) {
  __shared__ int hist[256];
  __shared__ int sfx[256];
  __shared__ int tmp[kTopkThreads / kWave];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;

  const int t = threadIdx.x;
  const float *row = scores + static_cast<size_t>(blockIdx.x) * row_len;
  int32_t *out = ids + static_cast<size_t>(blockIdx.x) * topk;

  // number of kept entries K = min(topk, #(score > -inf))
  int nvalid = 0;
  for (int i = t; i < row_len; i += kTopkThreads) nvalid += order_key(row[i]) > kNegInfKey;
  int total;
  (void)block_exclusive_scan(nvalid, tmp, total);
  const int K = min(topk, total);

  uint32_t prefix = 0, mask = 0;
  int remaining = K;   // how many still to take at or below the current prefix
  if (K > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (t < 256) hist[t] = 0;
      __syncthreads();
      for (int i = t; i < row_len; i += kTopkThreads) {
        const uint32_t k = order_key(row[i]);
        if (k > kNegInfKey && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      // suffix sums: sfx[d] = #entries in bins >= d
      if (t < 256) sfx[t] = hist[t];
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        int v = 0;
        if (t < 256 && t + o < 256) v = sfx[t + o];
        __syncthreads();
        if (t < 256) sfx[t] += v;
        __syncthreads();
      }
      if (t < 256) {
        const int above = (t < 255) ? sfx[t + 1] : 0;
        if (above < remaining && remaining <= sfx[t]) {
          s_prefix = prefix | (static_cast<uint32_t>(t) << shift);
          s_remaining = remaining - above;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      mask |= 255u << shift;
      __syncthreads();
    }
  }
  // prefix is now the exact key of the K-th largest entry; `remaining` entries
  // equal to it are taken, lowest index first.
  const uint32_t thr = prefix;
  const int chunk = (row_len + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(row_len, t * chunk), i1 = min(row_len, i0 + chunk);
  int n_eq = 0;
  if (K > 0)
    for (int i = i0; i < i1; ++i) n_eq += order_key(row[i]) == thr;
  const int eq_before = block_exclusive_scan(n_eq, tmp, total);
  int n_sel = 0;
  if (K > 0) {
    int e = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = order_key(row[i]);
      if (k > thr) ++n_sel;
      else if (k == thr) { n_sel += e < remaining; ++e; }
    }
  }
  int pos = block_exclusive_scan(n_sel, tmp, total);
  if (K > 0) {
    int e = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = order_key(row[i]);
      bool take = false;
      if (k > thr) take = true;
      else if (k == thr) { take = e < remaining; ++e; }
      if (take) out[pos++] = i;
    }
  }
  for (int i = K + t; i < topk; i += kTopkThreads) out[i] = -1;
}

// Rows of at most 512 * KPT entries: the same selection with the row's keys held
// in registers (thread t owns the KPT consecutive entries from t * KPT, so the
// ascending output order needs no reshuffle) and three barriers per radix pass:
// the 256-bin suffix sums are wave-level scans joined through the four wave
// totals, and two histogram buffers alternate so that clearing the next one
// needs no barrier of its own.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_reg_kernel(
    const float *__restrict__ scores, int row_len, int topk, int32_t *__restrict__ ids) {
  __shared__ int hist[2][256];
  __shared__ int wtot[4];
  __shared__ int tmp[kTopkThreads / kWave];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const float *row = scores + static_cast<size_t>(blockIdx.x) * row_len;
  int32_t *out = ids + static_cast<size_t>(blockIdx.x) * topk;
  const int i0 = t * KPT;

  uint32_t key[KPT];
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    key[j] = (i0 + j < row_len) ? order_key(row[i0 + j]) : 0u;   // 0: below every score
    nvalid += key[j] > kNegInfKey;
  }
  if (t < 256) {
    hist[0][t] = 0;
    hist[1][t] = 0;
  }
  int total;
  (void)block_exclusive_scan(nvalid, tmp, total);   // its barriers also order the clears
  const int K = min(topk, total);

  uint32_t prefix = 0, mask = 0;
  int remaining = K;
  if (K > 0) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass, cur = pass & 1;
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (key[j] > kNegInfKey && (key[j] & mask) == prefix)
          atomicAdd(&hist[cur][(key[j] >> shift) & 255u], 1);
      if (t < 256) hist[cur ^ 1][t] = 0;        // for the next pass; unused in this one
      __syncthreads();
      int h = 0, sfx = 0;
      if (t < 256) {
        h = hist[cur][t];
        sfx = h;                                // inclusive suffix sum inside the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int v = __shfl_down(sfx, o, kWave);
          if (lane + o < kWave) sfx += v;
        }
        if (lane == 0) wtot[wave] = sfx;
      }
      __syncthreads();
      if (t < 256) {
        for (int w = wave + 1; w < 4; ++w) sfx += wtot[w];   // bins of the higher waves
        const int above = sfx - h;
        if (above < remaining && remaining <= sfx) {
          s_prefix = prefix | (static_cast<uint32_t>(t) << shift);
          s_remaining = remaining - above;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      mask |= 255u << shift;
    }
  }
  // prefix is the exact key of the K-th largest entry; `remaining` entries equal
  // to it are taken, lowest index first.
  const uint32_t thr = prefix;
  int n_eq = 0;
  if (K > 0)
#pragma unroll
    for (int j = 0; j < KPT; ++j) n_eq += key[j] == thr;
  const int eq_before = block_exclusive_scan(n_eq, tmp, total);
  int n_sel = 0;
  if (K > 0) {
    int e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (key[j] > thr) ++n_sel;
      else if (key[j] == thr) { n_sel += e < remaining; ++e; }
    }
  }
  int pos = block_exclusive_scan(n_sel, tmp, total);
  if (K > 0) {
    int e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      bool take = false;
      if (key[j] > thr) take = true;
      else if (key[j] == thr) { take = e < remaining; ++e; }
      if (take) out[pos++] = i0 + j;
    }
  }
  for (int i = K + t; i < topk; i += kTopkThreads) out[i] = -1;
}

// Rows of at most 64 * E entries: one wave per row, four rows per work-group, no
// LDS and no barriers. Lane l holds the E consecutive entries from l * E. The
// threshold is built bit by bit from the top: the largest with at least K keys at
// or above it (the K-th largest key), each count being the popcounts of one ballot
// per register; the search stops early once exactly K keys are at or above it,
// which then separates the K largest from the rest. Entries above it are kept,
// and of those equal to it the lowest indices, counted with v_mbcnt (set bits of
// lower lanes); the same counts give every kept entry its output slot, so the ids
// come out ascending.
template <int E>
__global__ __launch_bounds__(256) void topk_rows_wave_kernel(const float *__restrict__ scores,
                                                             int rows, int row_len, int topk,
                                                             int32_t *__restrict__ ids) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + static_cast<int>(threadIdx.x) / kWave;
  if (row >= rows) return;                     // the whole wave
  const float *rp = scores + static_cast<size_t>(row) * row_len;
  int32_t *out = ids + static_cast<size_t>(row) * topk;
  const int i0 = lane * E;
  auto below = [](uint64_t m) {                // set bits of m in lanes below this one
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
  };
  uint32_t key[E];
#pragma unroll
  for (int j = 0; j < E; ++j)
    key[j] = (i0 + j < row_len) ? order_key(rp[i0 + j]) : 0u;   // 0: below every score
  int total = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) total += __popcll(__ballot(key[j] > kNegInfKey));
  const int K = min(topk, total);
  if (K > 0) {
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) c += __popcll(__ballot(key[j] >= cand));
      if (c >= K) {
        thr = cand;
        if (c == K) break;                     // the same for every lane
      }
    }
    // thr is the key of the K-th largest entry (every one of the K largest is
    // above -inf), or a threshold with exactly the K largest at or above it;
    // `remaining` entries equal to it are taken, lowest index first
    int n_gt = 0, eq_before = 0;
    uint64_t eq[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      n_gt += __popcll(__ballot(key[j] > thr));
      eq[j] = __ballot(key[j] == thr);
      eq_before += below(eq[j]);
    }
    const int remaining = K - n_gt;
    bool take[E];
    int e = eq_before;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      take[j] = key[j] > thr || (key[j] == thr && e < remaining);
      e += key[j] == thr;
    }
    int pos = 0;                               // kept entries of lower lanes
#pragma unroll
    for (int j = 0; j < E; ++j) pos += below(__ballot(take[j]));
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (take[j]) out[pos++] = i0 + j;
  }
  for (int i = K + lane; i < topk; i += kWave) out[i] = -1;
}

}  // namespace

hipError_t launch_topk(const float *scores, int rows, int row_len, int topk, int32_t *ids,
                       hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int per_lane = (row_len + kWave - 1) / kWave;
#define MSA_TOPK_WAVE(E)                                                              \
  if (per_lane <= E) {                                                                \
    MSA_LOG_LAUNCH("topk_rows_wave_kernel", (rows + 3) / 4, 256, 0);                   \
    topk_rows_wave_kernel<E><<<(rows + 3) / 4, 256, 0, st>>>(scores, rows, row_len, topk, \
                                                             ids);                    \
    return hipGetLastError();                                                         \
  }
  MSA_TOPK_WAVE(1) MSA_TOPK_WAVE(2) MSA_TOPK_WAVE(4) MSA_TOPK_WAVE(8)
#undef MSA_TOPK_WAVE
  const int per = (row_len + kTopkThreads - 1) / kTopkThreads;   // entries per thread
#define MSA_TOPK(KPT)                                                                 \
  if (per <= KPT) {                                                                   \
    MSA_LOG_LAUNCH("topk_rows_reg_kernel", rows, kTopkThreads, 0);                     \
    topk_rows_reg_kernel<KPT><<<rows, kTopkThreads, 0, st>>>(scores, row_len, topk, ids); \
    return hipGetLastError();                                                         \
  }
  MSA_TOPK(1) MSA_TOPK(2) MSA_TOPK(4) MSA_TOPK(8) MSA_TOPK(16) MSA_TOPK(32)
#undef MSA_TOPK
  MSA_LOG_LAUNCH("topk_rows_kernel", rows, kTopkThreads, 0);
  topk_rows_kernel<<<rows, kTopkThreads, 0, st>>>(scores, row_len, topk, ids);
  return hipGetLastError();
}

}  // namespace msa
