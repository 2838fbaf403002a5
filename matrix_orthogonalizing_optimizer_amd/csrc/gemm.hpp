// Grouped MFMA GEMM for the Newton-Schulz contractions on gfx950.
//
// One launch computes, for every unit u of a bucket chunk,
//     C_u = epilogue( L_u . op(R_u) )
// where L_u is M x K row-major (K contiguous) and op(R_u) is either R_u^T
// with R_u stored N x K (K contiguous, "RT") or R_u stored K x N (N
// contiguous, "RN").  The Newton-Schulz step of "Muon Optimizer and the
// Distributed Implementation" (section "Newton-Schulz Iteration"),
//     A = X X^T,   B = b A + c A A,   X' = a X + B X,
// maps onto it as: A and B are symmetric products (RT with R = L, only the
// upper-triangle tiles computed and mirror-written), X' is an RN product.
//
// Tiling (CDNA4, wave64): a 256-thread workgroup owns a BM x BN output tile,
// 2 x 2 waves each own (BM/2) x (BN/2) built from 32x32 MFMA tiles
// (v_mfma_f32_32x32x16_{bf16,f16}; fp32 uses four v_mfma_f32_32x32x2_f32 per
// 16-byte fragment).  K advances by 128 bytes per stage; operands are staged
// global -> registers -> LDS with double-buffered LDS and an XOR swizzle over
// 16-byte chunks so that fragment reads and stores are bank-conflict free.
// RN operands are transposed in registers (8x8 16-bit or 4x4 32-bit blocks)
// on their way to LDS, so every fragment read is a 16-byte ds_read along K.
//
// Bounds: rows are checked exactly; along the contiguous dimension a 16-byte
// chunk is loaded when its first element is in range.  This relies on every
// operand having a leading dimension that is a multiple of 8 elements with
// zero padding, which the workspace layout guarantees.
#pragma once

#include "kernel_args.hpp"

namespace muon {

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mfma<f16> {
  static constexpr int EPC = 8;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int EPC = 4;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    // bit-cast the whole vector: a bit-cast of one vector-element lvalue
    // was lowered to element 0 for every e
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
  }
};

// Swizzled 16-byte slot of (row, chunk) in an LDS tile with 8 chunks per row.
__device__ __forceinline__ int lds_slot(int row, int chunk) {
  return row * 8 + (chunk ^ (row & 7) ^ ((row >> 3) & 7));
}

// 8x8 transpose of 16-bit elements: in[r] holds row r (8 elements in 4
// words); out[c] receives column c.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1, sh = (c & 1) * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = (in[2 * j][w] >> sh) & 0xffffu;
      uint32_t hi = (in[2 * j + 1][w] >> sh) & 0xffffu;
      out[c][j] = lo | (hi << 16);
    }
  }
}

// Upper-triangle tile t (row-major over bi <= bj) of a T x T tile grid.
__device__ __forceinline__ void upper_tile(int t, int T, int& bi, int& bj) {
  int i = 0;
  while (t >= T - i) {
    t -= T - i;
    ++i;
  }
  bi = i;
  bj = i + t;
}

template <int BM, int BN, typename TI, typename TO, bool RN, bool SYM, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const GemmArgs a) {
  constexpr int EPC = Mfma<TI>::EPC;
  constexpr int BK = 8 * EPC;            // K elements per stage (128 bytes per row)
  constexpr int WTM = BM / 64;           // 32x32 tiles per wave along M
  constexpr int WTN = BN / 64;           // ... along N
  constexpr int NLA = BM * 8 / 256;      // 16-byte chunks of L per thread per stage
  constexpr int NLB = BN * 8 / 256;      // chunks of R (RT layout)
  constexpr int NBLK = (BN / EPC) * 8;   // EPC x EPC blocks of R (RN layout) per stage
  constexpr int NBT = (NBLK + 255) / 256;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(!SYM || BM == BN, "symmetric output needs square tiles");

  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- workgroup -> (unit, tile): XCD-contiguous ranges of logical tiles
  int logical;
  {
    const int b = blockIdx.x, tot = a.totalTiles;
    const int xcd = b & 7, loc = b >> 3, q = tot >> 3, r = tot & 7;
    logical = xcd * q + (xcd < r ? xcd : r) + loc;
  }
  const int unit = logical / a.tilesPerUnit;
  const int tt = logical - unit * a.tilesPerUnit;
  int bi, bj;
  if constexpr (SYM) {
    upper_tile(tt, a.tilesM, bi, bj);
  } else {
    constexpr int GROUP = 4;
    const int per_group = GROUP * a.tilesN;
    const int g = tt / per_group;
    const int first = g * GROUP;
    const int gm = min(a.tilesM - first, GROUP);
    const int w = tt - g * per_group;
    bi = first + w % gm;
    bj = w / gm;
  }
  const int row0 = bi * BM, col0 = bj * BN;

  const TI* __restrict__ Lp = reinterpret_cast<const TI*>(a.L) + (int64_t)unit * a.sL;
  const TI* __restrict__ Rp = reinterpret_cast<const TI*>(a.R) + (int64_t)unit * a.sR;

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 ra[NLA];
  u32x4 rb[RN ? NBT * EPC : NLB];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      const int id = i * 256 + tid;
      const int r = id >> 3, c = id & 7;
      const int gr = row0 + r, gk = k0 + c * EPC;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < a.M && gk < a.K) v = *reinterpret_cast<const u32x4*>(Lp + (int64_t)gr * a.ldl + gk);
      ra[i] = v;
    }
    if constexpr (!RN) {
#pragma unroll
      for (int i = 0; i < NLB; ++i) {
        const int id = i * 256 + tid;
        const int r = id >> 3, c = id & 7;
        const int gr = col0 + r, gk = k0 + c * EPC;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gr < a.N && gk < a.K) v = *reinterpret_cast<const u32x4*>(Rp + (int64_t)gr * a.ldr + gk);
        rb[i] = v;
      }
    } else {
      constexpr int NG = BN / EPC;  // column groups per stage
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
        const int blk = bt * 256 + tid;
        const int ng = blk % NG, kg = blk / NG;
        const int gn = col0 + ng * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int gk = k0 + kg * EPC + e;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (blk < NBLK && gk < a.K && gn < a.N)
            v = *reinterpret_cast<const u32x4*>(Rp + (int64_t)gk * a.ldr + gn);
          rb[bt * EPC + e] = v;
        }
      }
    }
  };

  auto store_stage = [&](int buf) {
    u32x4* sL = lds[buf];
    u32x4* sR = lds[buf] + BM * 8;
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      const int id = i * 256 + tid;
      sL[lds_slot(id >> 3, id & 7)] = ra[i];
    }
    if constexpr (!RN) {
#pragma unroll
      for (int i = 0; i < NLB; ++i) {
        const int id = i * 256 + tid;
        sR[lds_slot(id >> 3, id & 7)] = rb[i];
      }
    } else {
      constexpr int NG = BN / EPC;
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
        const int blk = bt * 256 + tid;
        if (blk < NBLK) {
          const int ng = blk % NG, kg = blk / NG;
          if constexpr (EPC == 8) {
            u32x4 in[8], out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) in[e] = rb[bt * 8 + e];
            transpose8x8_b16(in, out);
#pragma unroll
            for (int c = 0; c < 8; ++c) sR[lds_slot(ng * 8 + c, kg)] = out[c];
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              u32x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = rb[bt * 4 + e][c];
              sR[lds_slot(ng * 4 + c, kg)] = o;
            }
          }
        }
      }
    }
  };

  const int half = lane >> 5;
  const int l32 = lane & 31;
  auto compute_stage = [&](int buf) {
    const u32x4* sL = lds[buf];
    const u32x4* sR = lds[buf] + BM * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 fa[WTM], fb[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) fa[i] = sL[lds_slot(wm * (BM / 2) + i * 32 + l32, 2 * s + half)];
#pragma unroll
      for (int j = 0; j < WTN; ++j) fb[j] = sR[lds_slot(wn * (BN / 2) + j * 32 + l32, 2 * s + half)];
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) Mfma<TI>::run(acc[i][j], fa[i], fb[j]);
    }
  };

  const int nk = (a.K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_stage((kt + 1) * BK);
    compute_stage(kt & 1);
    if (more) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue
  float alpha = a.alpha;
  float4 ax = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.aux) ax = a.aux[unit];
  if (a.alphaSel == SEL_INV_S) alpha *= ax.y;
  else if (a.alphaSel == SEL_INV_S2) alpha *= ax.z;

  const TI* __restrict__ Ep = reinterpret_cast<const TI*>(a.E) + (int64_t)unit * a.sE;
  TO* __restrict__ Cp = reinterpret_cast<TO*>(a.C) + (int64_t)unit * a.sC;

  UnitDesc d;
  float keep = 1.f, step = 0.f;
  if constexpr (EPI == EPI_FINAL) {
    d = a.desc[unit];
    keep = 1.f - a.lr * a.wd;
    step = a.lr * d.scale;
  }

#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int gj = col0 + wn * (BN / 2) + j * 32 + l32;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int gi0 = row0 + wm * (BM / 2) + i * 32 + g4 * 8 + half * 4;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gi = gi0 + r;
          float x = acc[i][j][g4 * 4 + r];
          if constexpr (EPI == EPI_SCALE) {
            x = alpha * x;
          } else if constexpr (EPI == EPI_POLY) {
            float e = 0.f;
            if (gi < a.M && gj < a.ldc) e = to_f32(Ep[(int64_t)gi * a.lde + gj]);
            x = alpha * x + a.beta * e + (gi == gj ? a.gamma : 0.f);
          } else {
            float e = 0.f;
            if (a.beta != 0.f && gi < a.M && gj < a.N) e = to_f32(Ep[(int64_t)gi * a.lde + gj]);
            x = alpha * (a.beta * e + x);
          }
          v[r] = x;
        }
        if constexpr (EPI == EPI_FINAL) {
          if (gj < a.N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int gi = gi0 + r;
              if (gi < a.M) {
                const int64_t off = a.tall ? (int64_t)gj * d.ld + gi : (int64_t)gi * d.ld + gj;
                if (a.finalMode == FINAL_UPDATE) {
                  if (a.wdtype == DT_BF16) {
                    bf16* w = reinterpret_cast<bf16*>(d.w) + off;
                    *w = from_f32<bf16>(to_f32(*w) * keep - step * v[r]);
                  } else {
                    float* w = reinterpret_cast<float*>(d.w) + off;
                    *w = *w * keep - step * v[r];
                  }
                  if (d.o) d.o[off] = v[r];
                } else {
                  if (a.wdtype == DT_BF16) reinterpret_cast<bf16*>(d.w)[off] = from_f32<bf16>(v[r]);
                  else reinterpret_cast<float*>(d.w)[off] = v[r];
                }
              }
            }
          }
        } else if (SYM && bi == bj) {
          // diagonal tile of a symmetric product: the upper triangle is
          // stored and mirrored, so the result is exactly symmetric even
          // when L . R^T is symmetric only up to rounding
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int gi = gi0 + r;
            if (gi <= gj && gi < a.M && gj < a.ldc) {
              const TO val = from_f32<TO>(v[r]);
              Cp[(int64_t)gi * a.ldc + gj] = val;
              if (gi < gj && gj < a.M) Cp[(int64_t)gj * a.ldc + gi] = val;
            }
          }
        } else {
          // direct tile
          if (gj < a.ldc) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (gi0 + r < a.M) Cp[(int64_t)(gi0 + r) * a.ldc + gj] = from_f32<TO>(v[r]);
          }
          // mirror tile of a symmetric product: 4 consecutive columns of row gj
          if constexpr (SYM) {
            if (gj < a.M && gi0 < a.ldc) {
              TO* dst = Cp + (int64_t)gj * a.ldc + gi0;
              if constexpr (sizeof(TO) == 2) {
                u32x2 p;
                p[0] = (uint32_t)bits16(from_f32<TO>(v[0])) | ((uint32_t)bits16(from_f32<TO>(v[1])) << 16);
                p[1] = (uint32_t)bits16(from_f32<TO>(v[2])) | ((uint32_t)bits16(from_f32<TO>(v[3])) << 16);
                *reinterpret_cast<u32x2*>(dst) = p;
              } else {
                *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace muon
