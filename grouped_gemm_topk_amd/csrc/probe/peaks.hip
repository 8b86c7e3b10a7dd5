// Achievable-peak probes for the roofline denominators (measurement only; not
// part of libmoe's hot path and built into a library of its own).
//
//  moe_probe_mfma_loop:  every wave keeps NACC independent 32x32x16 bf16
//                        accumulators busy for `iters` rounds with no memory
//                        traffic; flops = grid * 4 waves * iters * NACC * 32768.
//  moe_probe_hbm_read:   a grid-stride streaming read of `bytes` (16 B per lane
//                        per load, eight loads in flight per lane, non-temporal
//                        so the stream does not settle in the caches); one
//                        32-bit fold per thread is written so nothing is elided.
//
// Both return 0 or the hipError_t of the launch.  Pointers are device pointers;
// `out` must hold grid * 256 elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAcc = 16;

__global__ void __launch_bounds__(256) mfma_loop_kernel(float* __restrict__ out, int iters) {
  f32x16 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((threadIdx.x & 7) * 0.125f);
    b[i] = (__bf16)(i * 0.0625f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kUnroll = 8;

__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                       unsigned* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256 * kUnroll;
  unsigned acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; base < n16; base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int moe_probe_mfma_loop(float* out, int grid, int iters, void* stream) {
  if (!out || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

extern "C" int moe_probe_mfma_flops_per_wave_iter(void) { return kAcc * 32 * 32 * 16 * 2; }

extern "C" int moe_probe_hbm_read(const void* src, int64_t bytes, unsigned* out, int grid, void* stream) {
  if (!src || !out || grid <= 0 || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, out);
  return (int)hipGetLastError();
}
