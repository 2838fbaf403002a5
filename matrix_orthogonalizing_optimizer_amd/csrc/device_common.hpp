// Device-side types and helpers shared by the libmuon kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The same address as a global-memory pointer.  Accesses through a generic
// pointer the compiler cannot trace to a kernel argument (say, one read from
// a descriptor table) compile to FLAT instructions, which also count in
// lgkmcnt: an LDS wait after them then waits for those global stores to
// complete too (the fused update's epilogue did, once per strip: 1-3.5%
// of that kernel).
template <typename T> __device__ __forceinline__ __attribute__((address_space(1))) T* as_global(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// Storage dtype codes used on the device side.
enum : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Per-unit device descriptor (one independent matrix of a Muon parameter).
// Pointers address the unit's origin inside the caller's tensors.
struct __attribute__((aligned(16))) UnitDesc {
  const void* g;   // gradient (param dtype), rows x cols, leading dim ld
  float* mom;      // momentum (fp32) or nullptr (plain orthogonalization)
  void* w;         // parameter (param dtype), updated in place
  float* o;        // optional fp32 copy of the orthogonalized update
  int64_t ld;      // leading dimension of g / mom / w / o (elements)
  float scale;     // rms_scale * sqrt(scale_dim)
  int32_t pad0;
};
static_assert(sizeof(UnitDesc) == 48, "UnitDesc layout");

// One AdamW parameter of the grouped elementwise launch.
struct __attribute__((aligned(16))) AdamDesc {
  void* w;
  const void* g;
  float* m;
  float* v;
  int64_t numel;
  int64_t block0;  // first block of this parameter in the launch
  int32_t dtype;   // DT_F32 or DT_BF16
  int32_t vec_ok;  // all four pointers 16-byte aligned
  int64_t pad;
};
static_assert(sizeof(AdamDesc) == 64, "AdamDesc layout");

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ uint16_t bits16(bf16 x) { return __builtin_bit_cast(uint16_t, x); }
__device__ __forceinline__ uint16_t bits16(f16 x) { return __builtin_bit_cast(uint16_t, x); }

// Two floats -> two 16-bit values of T in one 32-bit word (a in the low
// half), one v_cvt_pk_{bf16,f16}_f32, rounding to nearest even as the
// element-wise conversion does.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (__is_same(T, bf16)) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
}

// Deterministic wave64 sum (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Deterministic sum over a 256-thread block; result valid in every thread.
__device__ __forceinline__ float block_sum_256(float v, float* red /* >= 4 floats LDS */) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

}  // namespace muon
