// Argument blocks of the libmuon kernels (shared by launchers and kernels).
#pragma once

#include "device_common.hpp"

namespace muon {

// Epilogues: C = alpha L R^T (SCALE); C = alpha L R^T + beta E + gamma I
// (POLY); the fused parameter update (FINAL).
enum : int32_t { EPI_SCALE = 0, EPI_POLY = 1, EPI_FINAL = 2 };
enum : int32_t { SEL_ONE = 0, SEL_INV_S = 1, SEL_INV_S2 = 2 };
enum : int32_t { FINAL_UPDATE = 0, FINAL_STORE = 1 };

struct GemmArgs {
  const void* L;   // M x K, K contiguous
  const void* R;   // N x K, K contiguous
  const void* E;   // epilogue addend (EPI_POLY), same layout as C
  void* C;         // direct output (M x N), or null; EPI_FINAL writes the parameters (TO = their dtype)
  void* C2;        // mirror output (N x M, the transpose), or null; C for a symmetric product
  int64_t ldl, ldr, lde, ldc, ldc2;
  int64_t sL, sR, sE, sC, sC2;  // per-unit strides in elements
  int32_t M, N, K;         // logical per-unit sizes
  int32_t units, tilesM, tilesN, tilesPerUnit, totalTiles;
  float alpha, beta, gamma;
  int32_t alphaSel;        // SEL_*: alpha is multiplied by aux[u].y or aux[u].z
  const float4* aux;       // per unit {s^2, 1/s, 1/s^2, 0}
  const UnitDesc* desc;    // EPI_FINAL: per-unit parameter pointers
  float lr, wd;            // EPI_FINAL
  int32_t finalMode;       // FINAL_UPDATE or FINAL_STORE
  int32_t wvec;            // EPI_FINAL: parameter / update_out rows are 16-byte aligned, ld % 8 == 0
};

// Momentum kernel (see elementwise.hpp).
struct MomArgs {
  const UnitDesc* desc;
  void* D;         // U in the parameter's own layout (rows x cols), or null
  void* T;         // U transposed (cols x rows), or null
  int64_t ldd, ldt;  // leading dimensions (multiples of 8)
  int64_t sD, sT;    // per-unit element strides
  float* partials; // one per workgroup
  int32_t rows, cols;      // unit shape in parameter layout
  int32_t tilesR, tilesC, tilesPerUnit;
  float mu;
  int32_t nesterov;
  int32_t vec_ok;  // every unit's g/mom rows are 16-byte aligned and cols % 8 == 0
};

// AdamW kernel (see elementwise.hpp).
struct AdamArgs {
  const AdamDesc* desc;
  int64_t block_base;  // first global block of this launch
  int32_t nparams;
  float one_minus_b1, one_minus_b2, eps, keep, step;
};

// Host table -> device memory through kernel arguments: one launch carries
// up to BLOB_WORDS 32-bit words of a descriptor table, so no host staging
// buffer, no host-to-device copy and no wait on the host are involved.
constexpr int BLOB_WORDS = 768;  // 3 KiB of payload per launch
struct BlobArgs {
  uint32_t* dst;
  uint32_t nwords;
  uint32_t pad;
  uint32_t words[BLOB_WORDS];
};

}  // namespace muon
