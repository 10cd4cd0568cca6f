// Measurement probes for the benchmark (librba_probe.so): the dense bf16
// MFMA rate and the HBM bandwidth of a plain copy that the chip sustains.
// The entry points and their contracts are declared in rba_probe.h.
#include "rba_probe.h"

#include <hip/hip_runtime.h>

#include "rba.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 4 independent accumulator chains per wave; with 2 workgroups of 4 waves
// per compute unit every SIMD holds two such waves.
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.01f * (float)(((lane * 8 + i) % 13) - 6));
    b[i] = (__bf16)(0.01f * (float)(((lane * 5 + 3 * i) % 11) - 5));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Four 16-byte vectors per thread per sweep, all loads issued before the
// stores, so each wave keeps 4 KiB of reads in flight.
__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n4) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  for (; i + 256 * (U - 1) < n4; i += stride) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + 256 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + 256 * u);
  }
  for (int u = 0; u < U; ++u)
    if (i + 256 * u < n4) dst[i + 256 * u] = src[i + 256 * u];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int rba_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, double* flops_per_launch, void* stream) {
  if (workgroups < 1 || iters < 1 || !out || !flops_per_launch || !aligned16(out)) return RBA_ERR_INVALID;
  *flops_per_launch = (double)workgroups * 4 * iters * 4 * 32768.0;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

int rba_probe_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || workgroups < 1 || !aligned16(src) || !aligned16(dst))
    return RBA_ERR_INVALID;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return RBA_ERR_INVALID;
  hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? RBA_OK : RBA_ERR_HIP;
}

}  // extern "C"
