// Peak-rate probes of gfx950 (see include/msa_probe.h): the practical ceilings of
// a streaming HBM read, of a plain device copy and of dense bf16 MFMA issue (on small constant operands
// and on random full-mantissa operands), and the co-execution of MFMA and fp32
// VALU work of two waves on one SIMD, measured on the same GPU as the kernels
// they bound.
#include <hip/hip_runtime.h>

#include "msa_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;   // 16-byte loads per thread per round

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ buf,
                                                               size_t n16,
                                                               uint32_t *__restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * kInFlight;
  uint32_t acc = 0;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kInFlight + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      const size_t e = base + static_cast<size_t>(i) * kThreads;
      v[i] = e < n16 ? __builtin_nontemporal_load(buf + e) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  // one word per work-group: the xor of its threads' words
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kThreads; ++i) r ^= red[i];
    sink[blockIdx.x] = r;
  }
}

// Device copy: 16-byte loads, 8 in flight per thread, then 16-byte stores of the
// same chunks, grid-stride (no non-temporal hints: a plain copy's own rate).
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4 *__restrict__ src,
                                                        u32x4 *__restrict__ dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * kInFlight;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kInFlight + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      const size_t e = base + static_cast<size_t>(i) * kThreads;
      if (e < n16) v[i] = src[e];
    }
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      const size_t e = base + static_cast<size_t>(i) * kThreads;
      if (e < n16) dst[e] = v[i];
    }
  }
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float *__restrict__ sink) {
  // operands from the thread id: values in registers, no memory in the loop
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * static_cast<float>((t + i) % 7));
    b[i] = static_cast<__bf16>(0.001f * static_cast<float>((t * 3 + i) % 5));
  }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  if (t % 64 == 0) sink[blockIdx.x * (kThreads / 64) + t / 64] = s;
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Operands uniform in (-1.7, 1.7), every bf16 mantissa bit in use: 8 pairs per lane.
__device__ __forceinline__ void random_operands(bf16x8 *a, bf16x8 *b, uint32_t seed) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t h = mix32(seed * 131u + static_cast<uint32_t>(i * 17 + k));
      a[i][k] = static_cast<__bf16>((static_cast<float>(h & 0xffffu) / 32768.f - 1.f) * 1.7f);
      b[i][k] = static_cast<__bf16>((static_cast<float>(h >> 16) / 32768.f - 1.f) * 1.7f);
    }
}

__global__ __launch_bounds__(kThreads) void mfma_random_kernel(int iters,
                                                               float *__restrict__ sink) {
  bf16x8 a[8], b[8];
  random_operands(a, b, blockIdx.x * kThreads + threadIdx.x);
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[k][i];
  if (threadIdx.x % 64 == 0) sink[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = s;
}

// Work-groups of 8 waves with 128 KiB of LDS (one per CU, two waves per SIMD: waves
// w and w + 4 share one). Waves 0-3 run rounds of 16 random-operand MFMAs (one
// chain of 8 interleaved with four chains of 2, as in an attention tile); waves
// 4-7 run rounds of a softmax tile's fp32 work on 16 values (max3 tree, 16 x (fma,
// exp2, add), 8 bf16 packs). mode bit 0 runs the MFMA waves, bit 1 the VALU waves.
constexpr int kCoThreads = 512;

__global__ __launch_bounds__(kCoThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_valu_kernel(int iters, int mode, float *__restrict__ sink) {
  __shared__ float hold[32768];           // 128 KiB: one work-group per CU
  hold[threadIdx.x] = static_cast<float>(threadIdx.x);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
  float r = 0.f;
  if (wave < 4 && (mode & 1)) {
    bf16x8 a[8], b[8];
    random_operands(a, b, blockIdx.x * kCoThreads + threadIdx.x);
    f32x16 s = f32x16{}, o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], s, 0, 0, 0);
        o[i / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[i], a[(i + 3) & 7], o[i / 2], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) r += s[i] + o[0][i] + o[1][i] + o[2][i] + o[3][i];
  }
  if (wave >= 4 && (mode & 2)) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = hold[(threadIdx.x + i) % kCoThreads] * 1e-3f;
    float m = 0.f;
    uint32_t packed = 0;
    for (int it = 0; it < iters; ++it) {
      const float x0 = fmaxf(fmaxf(v[0], v[1]), v[2]), x1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
      const float x2 = fmaxf(fmaxf(v[6], v[7]), v[8]), x3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
      const float x4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
      const float x = fmaxf(fmaxf(fmaxf(x0, x1), x2), fmaxf(fmaxf(x3, x4), v[15]));
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(v[i], 0.1f, -m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(v[i + 1], 0.1f, -m));
        l += p0 + p1;
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        packed ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{p0, p1}, b2));
        v[i] = fmaf(p0, 1e-3f, v[i]);
        v[i + 1] = fmaf(p1, 1e-3f, v[i + 1]);
      }
      m = fmaf(x, 1e-6f, l * 1e-6f);
    }
    r += m + static_cast<float>(packed & 1u);
  }
  if (threadIdx.x % 64 == 0) sink[blockIdx.x * 8 + wave] = r;
}

}  // namespace

extern "C" {

int msa_probe_stream_read(const void *buf, size_t bytes, int groups, uint32_t *sink,
                          void *stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 32768 != 0 || groups < 1 ||
      groups > 65536 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return -1;
  stream_read_kernel<<<groups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return static_cast<int>(hipGetLastError());
}

int msa_probe_copy(const void *src, void *dst, size_t bytes, int groups, void *stream) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (src == nullptr || dst == nullptr || bytes == 0 || bytes % 16 != 0 || groups < 1 ||
      groups > 65536 || s % 16 != 0 || d % 16 != 0 || (s < d + bytes && d < s + bytes))
    return -1;
  copy_kernel<<<groups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16);
  return static_cast<int>(hipGetLastError());
}

int msa_probe_mfma_bf16(int groups, int iters, float *sink, void *stream) {
  if (sink == nullptr || groups < 1 || groups > 65536 || iters < 1) return -1;
  mfma_kernel<<<groups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return static_cast<int>(hipGetLastError());
}

int msa_probe_mfma_bf16_random(int groups, int iters, float *sink, void *stream) {
  if (sink == nullptr || groups < 1 || groups > 65536 || iters < 1) return -1;
  mfma_random_kernel<<<groups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return static_cast<int>(hipGetLastError());
}

int msa_probe_mfma_valu(int groups, int iters, int mode, float *sink, void *stream) {
  if (sink == nullptr || groups < 1 || groups > 32768 || iters < 1 || mode < 1 || mode > 3)
    return -1;
  mfma_valu_kernel<<<groups, kCoThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, mode,
                                                                               sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
