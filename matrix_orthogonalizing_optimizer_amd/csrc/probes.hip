// Measurement aids (muon_probe_mfma, muon_probe_copy in libmuon.h): the two
// ceilings a benchmark reports its kernels against, measured on the device
// it runs on.  Neither is part of the optimizer step.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "gemm.hpp"
#include "libmuon.h"

namespace muon {
namespace {

constexpr int kChains = 8;  // independent accumulators per wave

// Register-only bf16 MFMA loop: each wave runs iters rounds of kChains
// independent v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 = 32768 FLOP each);
// a chain's next MFMA is issued kChains MFMAs after its previous one, which
// covers the instruction's latency.  One float per workgroup reaches sink,
// so the work is not elided.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void probe_mfma_kernel(int32_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int q = 0; q < kChains; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < kChains; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kChains; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  s = wave_sum(s);
  __shared__ float part[4];
  if (lane == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

// Streaming copy, 16 bytes per lane per access, non-temporal on both sides:
// each workgroup moves one contiguous block of 256 x kUnroll 16-byte words
// (word u * 256 + thread of the block), all loads before the stores.
constexpr int kUnroll = 4;
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x;
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (base + u * 256 < n16) v[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (base + u * 256 < n16) __builtin_nontemporal_store(v[u], dst + base + u * 256);
}

// The same streaming copy with the GEMMs' load path: global -> LDS with
// buffer_load_dwordx4 ... lds at the default cache policy (each lane's 16
// bytes land at the wave's LDS base + 16 * lane), then LDS -> global with
// ordinary 16-byte stores.  Calibrates the memory counters for the loads the
// Newton-Schulz GEMMs issue.
__global__ __launch_bounds__(256) void probe_copy_lds_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                             int64_t n16) {
  __shared__ u32x4 buf[256 * kUnroll];
  const int64_t base = (int64_t)blockIdx.x * 256 * kUnroll;
  const int64_t left = n16 - base;
  const int64_t here = left < 256 * kUnroll ? left : 256 * kUnroll;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + base, (uint32_t)(here * 16));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    copy16_to_lds(r, &buf[u * 256 + wave * 64], (uint32_t)((u * 256 + wave * 64 + lane) * 16));
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (u * 256 + (int)threadIdx.x < here) dst[base + u * 256 + threadIdx.x] = buf[u * 256 + threadIdx.x];
}

}  // namespace
}  // namespace muon

extern "C" {

muon_status muon_probe_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream) {
  if (workgroups <= 0 || iters <= 0 || !sink || !flops) return MUON_E_ARG;
  *flops = (double)workgroups * 4.0 * (double)iters * muon::kChains * 32768.0;
  hipLaunchKernelGGL(muon::probe_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_E_HIP;
}

muon_status muon_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)src & 15) != 0 ||
      ((uintptr_t)dst & 15) != 0)
    return MUON_E_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (n16 + 256 * muon::kUnroll - 1) / (256 * muon::kUnroll);
  if (blocks > 0x7fffffff) return MUON_E_ARG;
  const unsigned grid = (unsigned)blocks;
  hipLaunchKernelGGL(muon::probe_copy_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const muon::u32x4*>(src), reinterpret_cast<muon::u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_E_HIP;
}

muon_status muon_probe_copy_lds(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || (bytes & 15) != 0 || ((uintptr_t)src & 15) != 0 ||
      ((uintptr_t)dst & 15) != 0)
    return MUON_E_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (n16 + 256 * muon::kUnroll - 1) / (256 * muon::kUnroll);
  if (blocks > 0x7fffffff) return MUON_E_ARG;
  hipLaunchKernelGGL(muon::probe_copy_lds_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const muon::u32x4*>(src),
                     reinterpret_cast<muon::u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_E_HIP;
}

}  // extern "C"
