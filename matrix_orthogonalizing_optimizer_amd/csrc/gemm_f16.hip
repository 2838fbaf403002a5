// Instantiations of the grouped MFMA GEMM with f16 operands.
#include "gemm.hpp"
#include "launch.hpp"

namespace muon {

namespace {
// 256 x 256 products (all row-major here) run 8 waves, two per SIMD, as the
// bf16 ones do
template <int T, typename TO, bool SYM, int EPI, bool TRANS = false, int NW = (T == 256 && !TRANS ? 8 : 4)>
hipError_t go(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<T, T, f16, TO, SYM, EPI, TRANS, NW>), dim3(a.totalTiles), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int T>
hipError_t dispatch(int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s) {
  if (!trans && sym && epi == EPI_SCALE && to == DT_F16) return go<T, f16, true, EPI_SCALE>(a, s);
  if (!trans && sym && epi == EPI_SCALE && to == DT_BF16) return go<T, bf16, true, EPI_SCALE>(a, s);
  if (!trans && sym && epi == EPI_POLY && to == DT_F16) return go<T, f16, true, EPI_POLY>(a, s);
  if (!trans && sym && epi == EPI_POLY && to == DT_BF16) return go<T, bf16, true, EPI_POLY>(a, s);
  if (!trans && !sym && epi == EPI_SCALE && to == DT_F16) return go<T, f16, false, EPI_SCALE>(a, s);
  if (!trans && !sym && epi == EPI_SCALE && to == DT_BF16) return go<T, bf16, false, EPI_SCALE>(a, s);
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_gemm_f16(int tile, int to, bool sym, int epi, bool trans, const GemmArgs& a, hipStream_t s) {
  return tile == 256 ? dispatch<256>(to, sym, epi, trans, a, s) : dispatch<128>(to, sym, epi, trans, a, s);
}

}  // namespace muon
