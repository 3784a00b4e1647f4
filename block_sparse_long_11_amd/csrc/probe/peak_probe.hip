// Peak-rate probes of gfx950 (see include/msa_probe.h): the practical ceilings of
// a streaming HBM read and of dense bf16 MFMA issue, measured on the same GPU as
// the kernels they bound.
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

int msa_probe_mfma_bf16(int groups, int iters, float *sink, void *stream) {
  if (sink == nullptr || groups < 1 || groups > 65536 || iters < 1) return -1;
  mfma_kernel<<<groups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
