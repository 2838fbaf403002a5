// Host-side launchers of the libmuon kernels (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_args.hpp"

namespace muon {

// GEMM launch for input dtype ti / output dtype to (DT_*), tile edge 128 or
// 256, symmetric-output flag, epilogue kind and operand layout (trans: both
// operands K-major, element (i, k) at p[k * ld + i]).  Returns
// hipErrorInvalidValue for a combination that is not instantiated.
hipError_t launch_gemm(int tile, int ti, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16(int tile, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f16(int tile, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f32(int tile, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s);

hipError_t launch_momentum(int gdtype, int xdtype, bool tall, const MomArgs& a, int64_t blocks,
                           hipStream_t s);
hipError_t launch_norm_finalize(const float* partials, int32_t per_unit, float4* aux, int32_t units,
                                hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, int64_t total_blocks, hipStream_t s);
// Writes `bytes` (a multiple of 4) from host memory src to device memory dst
// (4-byte aligned) through the arguments of ceil(bytes / 3 KiB) small kernel
// launches on s; src may be reused as soon as the call returns.
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace muon
