// Instantiations of the grouped MFMA GEMM with bf16 operands.
#include "gemm.hpp"
#include "launch.hpp"

namespace muon {

namespace {
// 256 x 256 products with row-major operands run 8 waves (two per SIMD, 128 x 64
// outputs each): 1-3% faster than 4 waves of 128 x 128 on the update, the fused
// update and the polynomial product.
template <int T, typename TO, bool SYM, int EPI, bool TRANS = false, int NW = (T == 256 && !TRANS ? 8 : 4)>
hipError_t go(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<T, T, bf16, TO, SYM, EPI, TRANS, NW>), dim3(a.totalTiles), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// The K-major product (A = Y^T Y, K = n, the unit's long side) runs 8 waves
// up to K = 8192 and one wave per SIMD above: 8 waves measured 7.7% faster
// at K = 2048, 2.5% at K = 4096, and 1.1-1.7% slower at K = 14336.
constexpr int KMAJOR_8W_MAX_K = 8192;

template <int T, typename TO>
hipError_t go_kmajor(const GemmArgs& a, hipStream_t s) {
  if constexpr (T == 256) {
    if (a.K <= KMAJOR_8W_MAX_K) return go<T, TO, true, EPI_SCALE, true, 8>(a, s);
  }
  return go<T, TO, true, EPI_SCALE, true, 4>(a, s);
}

template <int T>
hipError_t dispatch(int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s) {
  if (!trans && sym && epi == EPI_SCALE && to == DT_BF16) return go<T, bf16, true, EPI_SCALE>(a, s);
  if (!trans && sym && epi == EPI_SCALE && to == DT_F16) return go<T, f16, true, EPI_SCALE>(a, s);
  if (!trans && sym && epi == EPI_POLY && to == DT_BF16) return go<T, bf16, true, EPI_POLY>(a, s);
  if (!trans && !sym && epi == EPI_SCALE && to == DT_BF16) return go<T, bf16, false, EPI_SCALE>(a, s);
  if (!trans && !sym && epi == EPI_FINAL && to == DT_BF16) return go<T, bf16, false, EPI_FINAL>(a, s);
  if (!trans && !sym && epi == EPI_FINAL && to == DT_F32) return go<T, float, false, EPI_FINAL>(a, s);
  // K-major operands (A = Y^T Y from the transposed copy)
  if (trans && sym && epi == EPI_SCALE && to == DT_BF16) return go_kmajor<T, bf16>(a, s);
  if (trans && sym && epi == EPI_SCALE && to == DT_F16) return go_kmajor<T, f16>(a, s);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_gemm_bf16(int tile, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s) {
  return tile == 256 ? dispatch<256>(to, sym, epi, trans, a, s) : dispatch<128>(to, sym, epi, trans, a, s);
}

}  // namespace muon
