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
// Bounds: operands are read with buffer loads over exactly the unit's
// matrix; a chunk whose row is out of range, or whose first k is past K,
// gets an out-of-range offset and reads as zero.  Along the contiguous
// dimension a 16-byte chunk is read when its first element is in range,
// which relies on leading dimensions that are multiples of 8 with zero
// padding (the workspace layout guarantees it).  Every operand matrix must
// be smaller than 2^31 bytes (checked by the planner).
//
// Epilogue: each wave stages its accumulators in LDS one 32-row strip at a
// time and writes them back with 16-byte row-contiguous accesses (direct
// pass) and, for symmetric products and tall-parameter updates, with the
// strip transposed (mirror pass).
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

// Buffer resource over [p, p + bytes): loads at offsets >= bytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

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

// 8 consecutive elements of type T at p (16-byte aligned for 16-bit T,
// 32 bytes for fp32) <-> 8 floats.
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  }
}

template <typename T> __device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)bits16(from_f32<T>(v[2 * j])) | ((uint32_t)bits16(from_f32<T>(v[2 * j + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = w;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// Fused parameter update of 8 consecutive parameter elements (one row of the
// parameter block, columns c..c+7, n_valid of them in range):
// W <- W (1 - lr wd) - lr scale O; optionally O is also stored in fp32.
template <typename TW>
__device__ __forceinline__ void final_row8(TW* w, float* o, const float (&v)[8], int n_valid, bool vec,
                                           float keep, float step, bool store_only) {
  if (vec && n_valid == 8) {
    float x[8];
    if (!store_only) {
      load8(w, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * keep - step * v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = v[e];
    }
    store8(w, x);
    if (o) store8(o, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < n_valid) {
        const float x = store_only ? v[e] : to_f32(w[e]) * keep - step * v[e];
        w[e] = from_f32<TW>(x);
        if (o) o[e] = v[e];
      }
    }
  }
}

template <int BM, int BN, typename TI, typename TO, bool RN, bool SYM, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const GemmArgs a) {
  constexpr int EPC = Mfma<TI>::EPC;
  constexpr int ES = (int)sizeof(TI);
  constexpr int BK = 8 * EPC;            // K elements per stage (128 bytes per row)
  constexpr int WTM = BM / 64;           // 32x32 tiles per wave along M
  constexpr int WTN = BN / 64;           // ... along N
  constexpr int WN = BN / 2;             // wave sub-tile width
  constexpr int NLA = BM * 8 / 256;      // 16-byte chunks of L per thread per stage
  constexpr int NLB = BN * 8 / 256;      // chunks of R (RT layout)
  constexpr int NG = BN / EPC;           // column groups of an RN stage
  constexpr int NBLK = NG * 8;           // EPC x EPC blocks of an RN stage
  constexpr int NBT = (NBLK + 255) / 256;
  constexpr int SROW = WN + 8;           // epilogue strip row stride (floats)
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(!SYM || BM == BN, "symmetric output needs square tiles");
  static_assert(4 * 32 * SROW * 4 <= 2 * (BM + BN) * 8 * 16, "epilogue staging fits in LDS");

  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;

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

  const TI* Lp = reinterpret_cast<const TI*>(a.L) + (int64_t)unit * a.sL;
  const TI* Rp = reinterpret_cast<const TI*>(a.R) + (int64_t)unit * a.sR;
  const __amdgpu_buffer_rsrc_t rL = make_rsrc(Lp, (uint32_t)((int64_t)a.M * a.ldl * ES));
  const __amdgpu_buffer_rsrc_t rR = make_rsrc(Rp, (uint32_t)((int64_t)(RN ? a.K : a.N) * a.ldr * ES));

  // per-thread byte offsets of the stage-0 chunks; a chunk whose row is out
  // of range (or, in the tail stage, whose first k is) reads as zero
  uint32_t offL[NLA];
  int kcL[NLA];  // k of the chunk within a stage
  bool rowokL[NLA];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int id = i * 256 + tid;
    const int r = id >> 3, c = id & 7;
    rowokL[i] = row0 + r < a.M;
    offL[i] = rowokL[i] ? (uint32_t)(((int64_t)(row0 + r) * a.ldl + c * EPC) * ES) : 0u;
    kcL[i] = c * EPC;
  }
  uint32_t offR[RN ? NBT : NLB];
  int kcR[RN ? NBT : NLB];
  bool okR[RN ? NBT : NLB];
  if constexpr (!RN) {
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
      const int id = i * 256 + tid;
      const int r = id >> 3, c = id & 7;
      okR[i] = col0 + r < a.N;
      offR[i] = okR[i] ? (uint32_t)(((int64_t)(col0 + r) * a.ldr + c * EPC) * ES) : 0u;
      kcR[i] = c * EPC;
    }
  } else {
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt) {
      const int blk = bt * 256 + tid;
      const int ng = blk % NG, kg = blk / NG;
      okR[bt] = blk < NBLK && col0 + ng * EPC < a.N;
      offR[bt] = okR[bt] ? (uint32_t)(((int64_t)(kg * EPC) * a.ldr + col0 + ng * EPC) * ES) : 0u;
      kcR[bt] = kg * EPC;
    }
  }

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
    const bool tail = k0 + BK > a.K;
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
      const bool ok = rowokL[i] && (!tail || k0 + kcL[i] < a.K);
      ra[i] = bload(rL, ok ? offL[i] + (uint32_t)(k0 * ES) : OOB);
    }
    if constexpr (!RN) {
#pragma unroll
      for (int i = 0; i < NLB; ++i) {
        const bool ok = okR[i] && (!tail || k0 + kcR[i] < a.K);
        rb[i] = bload(rR, ok ? offR[i] + (uint32_t)(k0 * ES) : OOB);
      }
    } else {
      const uint32_t kstep = (uint32_t)((int64_t)k0 * a.ldr * ES);
      const uint32_t rowb = (uint32_t)(a.ldr * ES);
#pragma unroll
      for (int bt = 0; bt < NBT; ++bt) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const bool ok = okR[bt] && (!tail || k0 + kcR[bt] + e < a.K);
          rb[bt * EPC + e] = bload(rR, ok ? offR[bt] + kstep + (uint32_t)e * rowb : OOB);
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

  auto compute_stage = [&](int buf) {
    const u32x4* sL = lds[buf];
    const u32x4* sR = lds[buf] + BM * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 fa[WTM], fb[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) fa[i] = sL[lds_slot(wm * (BM / 2) + i * 32 + l32, 2 * s + half)];
#pragma unroll
      for (int j = 0; j < WTN; ++j) fb[j] = sR[lds_slot(wn * WN + j * 32 + l32, 2 * s + half)];
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

  // ---------------------------------------------------------------- epilogue
  float alpha = a.alpha;
  if (a.alphaSel != SEL_ONE) {
    const float4 ax = a.aux[unit];
    alpha *= a.alphaSel == SEL_INV_S ? ax.y : ax.z;
  }
  const TI* Ep = reinterpret_cast<const TI*>(a.E) + (int64_t)unit * a.sE;
  TO* Cp = reinterpret_cast<TO*>(a.C) + (int64_t)unit * a.sC;

  float keep = 1.f, step = 0.f;
  UnitDesc d;
  if constexpr (EPI == EPI_FINAL) {
    d = a.desc[unit];
    keep = 1.f - a.lr * a.wd;
    step = a.lr * d.scale;
  }
  const bool diag = SYM && bi == bj;
  const bool mirror = (SYM) || (EPI == EPI_FINAL && a.tall);
  float* strip = reinterpret_cast<float*>(&lds[0][0]) + wid * (32 * SROW);

#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    // accumulators of MFMA row-tile i -> strip[32][WN]
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          strip[(g4 * 8 + half * 4 + r) * SROW + j * 32 + l32] = acc[i][j][g4 * 4 + r];
    __syncthreads();
    const int gr0 = row0 + wm * (BM / 2) + i * 32;  // global row of strip row 0
    const int gc0 = col0 + wn * WN;                 // global column of strip column 0

    // direct pass: strip row r, columns c8..c8+7
    if (!(EPI == EPI_FINAL && a.tall)) {
#pragma unroll 2
      for (int t = 0; t < 32 * WN / 8 / 64; ++t) {
        const int q = t * 64 + lane;
        const int r = q / (WN / 8), c8 = (q % (WN / 8)) * 8;
        const int gi = gr0 + r, gj = gc0 + c8;
        if (gi >= a.M) continue;
        float v[8];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(strip + r * SROW + c8);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(strip + r * SROW + c8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[e + 4] = hi[e]; }
        if constexpr (EPI == EPI_FINAL) {
          if (gj >= a.N) continue;
          float e8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (a.beta != 0.f) load8(Ep + (int64_t)gi * a.lde + gj, e8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = alpha * (a.beta * e8[e] + v[e]);
          const int64_t off = (int64_t)gi * d.ld + gj;
          const int nv = min(8, a.N - gj);
          float* o = d.o ? d.o + off : nullptr;
          if (a.wdtype == DT_BF16)
            final_row8(reinterpret_cast<bf16*>(d.w) + off, o, v, nv, a.wvec != 0, keep, step,
                       a.finalMode == FINAL_STORE);
          else
            final_row8(reinterpret_cast<float*>(d.w) + off, o, v, nv, a.wvec != 0, keep, step,
                       a.finalMode == FINAL_STORE);
        } else {
          if (gj >= a.ldc) continue;
          if constexpr (EPI == EPI_SCALE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= alpha;
          } else if constexpr (EPI == EPI_POLY) {
            float e8[8];
            load8(Ep + (int64_t)gi * a.lde + gj, e8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = alpha * v[e] + a.beta * e8[e] + (gi == gj + e ? a.gamma : 0.f);
          } else {
            float e8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (a.beta != 0.f) load8(Ep + (int64_t)gi * a.lde + gj, e8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = alpha * (a.beta * e8[e] + v[e]);
          }
          TO* dst = Cp + (int64_t)gi * a.ldc + gj;
          if (!diag || gi <= gj) {
            store8(dst, v);
          } else if (gi < gj + 8) {
            // diagonal tile: only the upper triangle (gi <= column) is stored
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gi <= gj + e) dst[e] = from_f32<TO>(v[e]);
          }
        }
      }
    }

    // mirror pass: strip column jj, rows c8..c8+7 -> output row gc0 + jj
    if (mirror) {
      // recompute the epilogue values for the transposed positions: the
      // symmetric epilogues are symmetric, so the value of (gi, gj) is the
      // value stored at (gj, gi)
#pragma unroll 2
      for (int t = 0; t < 32 * WN / 8 / 64; ++t) {
        const int q = t * 64 + lane;
        const int jj = q % WN, c8 = (q / WN) * 8;
        const int gj = gc0 + jj;       // output row
        const int gi = gr0 + c8;       // first output column
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = strip[(c8 + e) * SROW + jj];
        if constexpr (EPI == EPI_FINAL) {
          // tall unit: parameter row gj (< n), columns gi.. (< m)
          if (gj >= a.N || gi >= a.M) continue;
          float e8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (a.beta != 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              e8[e] = (gi + e < a.M) ? to_f32(Ep[(int64_t)(gi + e) * a.lde + gj]) : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = alpha * (a.beta * e8[e] + v[e]);
          const int64_t off = (int64_t)gj * d.ld + gi;
          const int nv = min(8, a.M - gi);
          float* o = d.o ? d.o + off : nullptr;
          if (a.wdtype == DT_BF16)
            final_row8(reinterpret_cast<bf16*>(d.w) + off, o, v, nv, a.wvec != 0, keep, step,
                       a.finalMode == FINAL_STORE);
          else
            final_row8(reinterpret_cast<float*>(d.w) + off, o, v, nv, a.wvec != 0, keep, step,
                       a.finalMode == FINAL_STORE);
        } else if constexpr (SYM) {
          if (gj >= a.M || gi >= a.ldc) continue;
          if (diag && gi + 7 >= gj) {
            // diagonal tile: lower-triangle positions (column < row) only
            bool any = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) any |= gi + e < gj;
            if (!any) continue;
          }
          if constexpr (EPI == EPI_SCALE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= alpha;
          } else if constexpr (EPI == EPI_POLY) {
            // E symmetric: E[gi + e][gj] = E[gj][gi + e]
            float e8[8];
            load8(Ep + (int64_t)gj * a.lde + gi, e8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = alpha * v[e] + a.beta * e8[e];
          } else {
            float e8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (a.beta != 0.f) load8(Ep + (int64_t)gj * a.lde + gi, e8);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = alpha * (a.beta * e8[e] + v[e]);
          }
          TO* dst = Cp + (int64_t)gj * a.ldc + gi;
          if (!diag || gi + 7 < gj) {
            store8(dst, v);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gi + e < gj) dst[e] = from_f32<TO>(v[e]);
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace muon
