// Launchers of the elementwise kernels and the GEMM dtype dispatch.
#include <cstring>

#include "elementwise.hpp"
#include "launch.hpp"

namespace muon {

hipError_t launch_gemm(int tile, int ti, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s) {
  if (a.totalTiles <= 0) return hipSuccess;
  switch (ti) {
    case DT_BF16: return launch_gemm_bf16(tile, to, sym, epi, trans, a, s);
    case DT_F16: return launch_gemm_f16(tile, to, sym, epi, trans, a, s);
    case DT_F32: return launch_gemm_f32(tile, to, sym, epi, trans, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_momentum(int gdtype, int xdtype, bool tall, const MomArgs& a, int64_t blocks,
                           hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const dim3 g((unsigned)blocks), b(256);
  if (tall) {
    // the working layout is the parameter's own: row-contiguous tiles
    if (a.D == nullptr) return hipErrorInvalidValue;
    if (gdtype == DT_BF16 && xdtype == DT_BF16) hipLaunchKernelGGL((momentum_rows_kernel<bf16, bf16>), g, b, 0, s, a);
    else if (gdtype == DT_F32 && xdtype == DT_F32) hipLaunchKernelGGL((momentum_rows_kernel<float, float>), g, b, 0, s, a);
    else if (gdtype == DT_BF16 && xdtype == DT_F32) hipLaunchKernelGGL((momentum_rows_kernel<bf16, float>), g, b, 0, s, a);
    else if (gdtype == DT_F32 && xdtype == DT_BF16) hipLaunchKernelGGL((momentum_rows_kernel<float, bf16>), g, b, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (gdtype == DT_BF16 && xdtype == DT_BF16) hipLaunchKernelGGL((momentum_kernel<bf16, bf16>), g, b, 0, s, a);
  else if (gdtype == DT_F32 && xdtype == DT_F32) hipLaunchKernelGGL((momentum_kernel<float, float>), g, b, 0, s, a);
  else if (gdtype == DT_BF16 && xdtype == DT_F32) hipLaunchKernelGGL((momentum_kernel<bf16, float>), g, b, 0, s, a);
  else if (gdtype == DT_F32 && xdtype == DT_BF16) hipLaunchKernelGGL((momentum_kernel<float, bf16>), g, b, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const float* partials, int32_t per_unit, float4* aux, int32_t units,
                                hipStream_t s) {
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(units), dim3(256), 0, s, partials, per_unit, aux);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void upload_kernel(const BlobArgs a) {
  for (uint32_t i = threadIdx.x; i < a.nwords; i += 256) a.dst[i] = a.words[i];
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes % 4 != 0 || reinterpret_cast<uintptr_t>(dst) % 4 != 0) return hipErrorInvalidValue;
  const size_t words = bytes / 4;
  BlobArgs a;
  for (size_t w0 = 0; w0 < words; w0 += BLOB_WORDS) {
    const size_t nw = words - w0 < (size_t)BLOB_WORDS ? words - w0 : (size_t)BLOB_WORDS;
    a.dst = static_cast<uint32_t*>(dst) + w0;
    a.nwords = (uint32_t)nw;
    a.pad = 0;
    std::memcpy(a.words, static_cast<const uint32_t*>(src) + w0, nw * 4);
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_adamw(const AdamArgs& a0, int64_t total_blocks, hipStream_t s) {
  const int64_t kMaxGrid = (int64_t)1 << 22;
  AdamArgs a = a0;
  for (int64_t b0 = 0; b0 < total_blocks; b0 += kMaxGrid) {
    const int64_t nb = total_blocks - b0 < kMaxGrid ? total_blocks - b0 : kMaxGrid;
    a.block_base = b0;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)nb), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace muon
