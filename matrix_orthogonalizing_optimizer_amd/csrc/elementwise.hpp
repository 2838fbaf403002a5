// HBM-bound kernels of the Muon step: fused momentum + Frobenius partial
// sums (writing the Newton-Schulz input in its working layout), the
// deterministic per-unit norm finalization, and the AdamW fallback.
#pragma once

#include "consts.hpp"
#include "kernel_args.hpp"

namespace muon {

// ---------------------------------------------------------------------------
// K-M: momentum / Nesterov + sum of squares.
// [Blog] "Formulation of Muon Optimizer": M_t = mu M_{t-1} + G_t;
// "Variation of Muon Optimizer": Nesterov orthogonalizes mu M_t + G_t.
// One workgroup handles a 64 x 256 tile of one unit (parameter layout) and
// writes U as is (D, leading dimension ldd) and/or transposed through LDS
// (T, leading dimension ldt), whichever is set, pad columns zero.  The tile's
// 64 rows make each transposed row one 128-byte line of 16-bit values; its
// 256 columns make each row's loads 512 bytes of G and 1 KB of M (measured
// on the 4096 x 14336 wide bucket: 5.15 TB/s against 4.58 with 64 x 128
// tiles and 4.81 with 128 x 128; the square and 1024 x 4096 buckets within
// noise of either).
// Each workgroup writes one partial sum of U^2 (fp32, fixed order).
// ---------------------------------------------------------------------------

// 8 elements of T from p, 16-byte aligned (32 for fp32)
template <typename T> __device__ __forceinline__ void ld8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x4*>(p)));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
  } else {
    const f32x4 lo = __builtin_nontemporal_load(as_global(reinterpret_cast<const f32x4*>(p)));
    const f32x4 hi = __builtin_nontemporal_load(as_global(reinterpret_cast<const f32x4*>(p + 4)));
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[e + 4] = hi[e]; }
  }
}

// streaming stores: the data is not read again by this kernel
template <typename T> __device__ __forceinline__ void st8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)bits16(from_f32<T>(v[2 * j])) | ((uint32_t)bits16(from_f32<T>(v[2 * j + 1])) << 16);
    __builtin_nontemporal_store(w, as_global(reinterpret_cast<u32x4*>(p)));
  } else {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, as_global(reinterpret_cast<f32x4*>(p)));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, as_global(reinterpret_cast<f32x4*>(p + 4)));
  }
}

// 4 consecutive elements of T at p (8-byte aligned for 16-bit T, 16 for fp32)
// <-> 4 floats, streaming.
template <typename T> __device__ __forceinline__ void ld4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x2*>(p)));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
  } else {
    const f32x4 x = __builtin_nontemporal_load(as_global(reinterpret_cast<const f32x4*>(p)));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
}

template <typename T> __device__ __forceinline__ void st4(T* p, const float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[j] = (uint32_t)bits16(from_f32<T>(v[2 * j])) | ((uint32_t)bits16(from_f32<T>(v[2 * j + 1])) << 16);
    __builtin_nontemporal_store(w, as_global(reinterpret_cast<u32x2*>(p)));
  } else {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, as_global(reinterpret_cast<f32x4*>(p)));
  }
}

template <typename TG, typename TX>
__global__ __launch_bounds__(256) void momentum_kernel(const MomArgs a) {
  constexpr int CGS = KM_TC / 8;    // 8-column groups per tile row
  constexpr int RPP = 256 / CGS;    // rows per pass of the workgroup
  constexpr int NH = KM_TR / RPP;   // passes (rows per thread)
  constexpr int CPT = KM_TR / 8;    // 8-element chunks per transposed row
  constexpr int NJ = KM_TC * CPT / 256;  // transposed chunks per thread
  static_assert(KM_TR % 64 == 0 && KM_TC % 64 == 0 && 256 % CGS == 0 && KM_TR % RPP == 0 &&
                (KM_TC * CPT) % 256 == 0, "tile shape");
  __shared__ float tile[KM_TR][KM_TC + 1];
  __shared__ float red[4];
  const int unit = blockIdx.x / a.tilesPerUnit;
  const int t = blockIdx.x - unit * a.tilesPerUnit;
  const int tr = t / a.tilesC, tc = t - tr * a.tilesC;
  const int r0 = tr * KM_TR, c0 = tc * KM_TC;
  const UnitDesc d = a.desc[unit];
  const TG* __restrict__ G = reinterpret_cast<const TG*>(d.g);
  float* __restrict__ M = d.mom;
  TX* __restrict__ X = a.D ? reinterpret_cast<TX*>(a.D) + (int64_t)unit * a.sD : nullptr;
  TX* __restrict__ XT = a.T ? reinterpret_cast<TX*>(a.T) + (int64_t)unit * a.sT : nullptr;

  const int tid = threadIdx.x;
  const int cg = tid % CGS;  // 8-column group
  const int rr = tid / CGS;  // rows rr + RPP h
  const int c = c0 + cg * 8;
  const bool cin = c < a.cols;
  const bool full = a.vec_ok && c + 8 <= a.cols;

  // loads of all rows first
  float g[NH][8], m[NH][8];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int r = r0 + rr + RPP * h;
#pragma unroll
    for (int e = 0; e < 8; ++e) { g[h][e] = 0.f; m[h][e] = 0.f; }
    if (r < a.rows && cin) {
      const int64_t off = (int64_t)r * d.ld + c;
      if (full) {
        ld8(G + off, g[h]);
        if (M) ld8(M + off, m[h]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (c + e < a.cols) {
            g[h][e] = to_f32(G[off + e]);
            if (M) m[h][e] = M[off + e];
          }
        }
      }
    }
  }

  float ss = 0.f;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int lr = rr + RPP * h;
    const int r = r0 + lr;
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (M) {
        const float mn = fmaf(a.mu, m[h][e], g[h][e]);
        m[h][e] = mn;
        u[e] = a.nesterov ? fmaf(a.mu, mn, g[h][e]) : mn;
      } else {
        u[e] = g[h][e];
      }
      ss = fmaf(u[e], u[e], ss);
    }
    if (r < a.rows && cin) {
      const int64_t off = (int64_t)r * d.ld + c;
      if (M) {
        if (full) {
          st8(M + off, m[h]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < a.cols) M[off + e] = m[h][e];
        }
      }
      // own layout: row r, columns c..c+8 (columns past cols are zero padding)
      if (X) st8(X + (int64_t)r * a.ldd + c, u);
    }
    if (XT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[lr][cg * 8 + e] = u[e];
    }
  }
  __syncthreads();
  // transposed layout: row c0 + cc, columns r0 .. r0 + KM_TR: KM_TC rows x CPT
  // chunks of 8 (consecutive lanes write consecutive chunks of one row)
#pragma unroll
  for (int j = 0; j < NJ && XT; ++j) {
    const int q = tid + 256 * j;
    const int cc = q / CPT, rq = q % CPT;
    const int gc = c0 + cc, gr = r0 + rq * 8;
    if (gc < a.cols && gr < a.rows) {
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = tile[rq * 8 + e][cc];
      st8(XT + (int64_t)gc * a.ldt + gr, u);
    }
  }
  const float s = block_sum_256(ss, red);
  if (tid == 0) a.partials[blockIdx.x] = s;
}

// The same for a tall unit, whose parameter block already has the working
// layout (U is written as is): row-contiguous KMR_TR x 512 tiles (4 x 512:
// one row per wave), each wave covering 512 consecutive columns of a row (1
// KB of a 16-bit G, 2 KB of M), so that a workgroup's accesses fall in few
// DRAM pages (14336 x 4096 units: 8.14 ms per 64-unit bucket against
// 8.50-8.73 with 8 x 512 tiles and 8.37 with 16 x 512).  A lane takes
// 4-element pieces (columns 4 l .. 4 l + 3 and 256 further on), so every
// load and store instruction of a wave covers one contiguous range, as in
// the AdamW kernel.  One partial sum of U^2 per workgroup.
template <typename TG, typename TX>
__global__ __launch_bounds__(256) void momentum_rows_kernel(const MomArgs a) {
  constexpr int NHR = KMR_TR / 4;   // rows per thread (4 waves, one row each per pass)
  constexpr int NP = KMR_TC / 256;  // 4-element pieces per lane and row
  static_assert(KMR_TR % 4 == 0 && KMR_TC % 256 == 0, "tile shape");
  __shared__ float red[4];
  const int unit = blockIdx.x / a.tilesPerUnit;
  const int t = blockIdx.x - unit * a.tilesPerUnit;
  const int tr = t / a.tilesC, tc = t - tr * a.tilesC;
  const UnitDesc d = a.desc[unit];
  const TG* __restrict__ G = reinterpret_cast<const TG*>(d.g);
  float* __restrict__ M = d.mom;
  TX* __restrict__ X = reinterpret_cast<TX*>(a.D) + (int64_t)unit * a.sD;

  const int tid = threadIdx.x;
  float g[NHR][NP][4], m[NHR][NP][4];
#pragma unroll
  for (int h = 0; h < NHR; ++h) {
    const int r = tr * KMR_TR + (tid >> 6) + 4 * h;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int c = tc * KMR_TC + p * 256 + (tid & 63) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) { g[h][p][e] = 0.f; m[h][p][e] = 0.f; }
      if (r < a.rows && c < a.cols) {
        const int64_t off = (int64_t)r * d.ld + c;
        if (a.vec_ok && c + 4 <= a.cols) {
          ld4(G + off, g[h][p]);
          if (M) ld4(M + off, m[h][p]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (c + e < a.cols) {
              g[h][p][e] = to_f32(G[off + e]);
              if (M) m[h][p][e] = M[off + e];
            }
          }
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int h = 0; h < NHR; ++h) {
    const int r = tr * KMR_TR + (tid >> 6) + 4 * h;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int c = tc * KMR_TC + p * 256 + (tid & 63) * 4;
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (M) {
          const float mn = fmaf(a.mu, m[h][p][e], g[h][p][e]);
          m[h][p][e] = mn;
          u[e] = a.nesterov ? fmaf(a.mu, mn, g[h][p][e]) : mn;
        } else {
          u[e] = g[h][p][e];
        }
        ss = fmaf(u[e], u[e], ss);
      }
      if (r < a.rows && c < a.cols && M) {
        const int64_t off = (int64_t)r * d.ld + c;
        if (a.vec_ok && c + 4 <= a.cols) {
          st4(M + off, m[h][p]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.cols) M[off + e] = m[h][p][e];
        }
      }
      // the working copy's zero padding up to ldd (a multiple of 8) is
      // written here too: u is zero past cols
      if (r < a.rows && c < a.ldd) st4(X + (int64_t)r * a.ldd + c, u);
    }
  }
  const float s = block_sum_256(ss, red);
  if (tid == 0) a.partials[blockIdx.x] = s;
}

// Per-unit norm: sums the unit's partials in a fixed order and stores
// {s^2, 1/s, 1/s^2, 0}.  A zero unit gets 1/s = 0 so its update is zero
// ("Newton-Schulz Iteration": G <- G / ||G||_F; the page prints no epsilon).
__global__ __launch_bounds__(256) void norm_finalize_kernel(const float* __restrict__ partials,
                                                            int32_t per_unit, float4* __restrict__ aux) {
  __shared__ float red[4];
  const int unit = blockIdx.x;
  const float* p = partials + (int64_t)unit * per_unit;
  float s = 0.f;
  for (int i = threadIdx.x; i < per_unit; i += 256) s += p[i];
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) {
    float inv = 0.f, inv2 = 0.f;
    if (s > 0.f) {
      inv = 1.0f / sqrtf(s);
      inv2 = 1.0f / s;
    }
    aux[unit] = make_float4(s, inv, inv2, 0.f);
  }
}

// ---------------------------------------------------------------------------
// K-W: the AdamW backup of the [Moonlight] code, one grouped launch over all
// AdamW parameters: m <- m + (1-b1)(g-m); v <- v + (1-b2)(g^2-v);
// W <- W (1 - lr wd) - step * m / (eps + sqrt(v)), step = lr sqrt(1-b2^t)/(1-b1^t).
// ---------------------------------------------------------------------------

__device__ __forceinline__ void adam_elem(float& w, float g, float& m, float& v, const AdamArgs& a) {
  m = fmaf(a.one_minus_b1, g - m, m);
  v = fmaf(a.one_minus_b2, g * g - v, v);
  w = w * a.keep - a.step * (m / (a.eps + sqrtf(v)));
}

// A workgroup's ADAM_EPB elements in pieces of 4 per lane: lane l of a pass
// takes elements 4 l .. 4 l + 3 of its wave's 256, so every load and store
// instruction of a wave covers one contiguous range (512 bytes of a 16-bit
// tensor, 1 KB of an fp32 one).  With 8 elements per lane the fp32 moments
// took two 16-byte pieces 32 bytes apart per lane, each instruction touching
// twice the cache lines: 6% slower (5.26 against 5.58 TB/s on the
// Llama-3-8B-shaped AdamW set).
template <typename TW>
__device__ __forceinline__ void adamw_tile(const AdamDesc& d, int64_t base, const AdamArgs& a) {
  constexpr int NCH = ADAM_EPB / (256 * 4);  // 4-element pieces per thread
  TW* __restrict__ W = reinterpret_cast<TW*>(d.w);
  const TW* __restrict__ G = reinterpret_cast<const TW*>(d.g);
  int64_t i0[NCH];
  bool vec[NCH];
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    i0[it] = base + (int64_t)(it * 256 + threadIdx.x) * 4;
    vec[it] = d.vec_ok && i0[it] + 4 <= d.numel;
  }
  // every load of the tile is issued before the first use
  float w[NCH][4], g[NCH][4], m[NCH][4], v[NCH][4];
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    if (vec[it]) {
      ld4(W + i0[it], w[it]);
      ld4(G + i0[it], g[it]);
      ld4(d.m + i0[it], m[it]);
      ld4(d.v + i0[it], v[it]);
    }
  }
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    if (vec[it]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) adam_elem(w[it][e], g[it][e], m[it][e], v[it][e], a);
      st4(W + i0[it], w[it]);
      st4(d.m + i0[it], m[it]);
      st4(d.v + i0[it], v[it]);
    } else {
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0[it] + e;
        if (i >= d.numel) break;
        float wi = to_f32(W[i]), gi = to_f32(G[i]), mi = d.m[i], vi = d.v[i];
        adam_elem(wi, gi, mi, vi, a);
        d.m[i] = mi;
        d.v[i] = vi;
        W[i] = from_f32<TW>(wi);
      }
    }
  }
}

__global__ __launch_bounds__(256) void adamw_kernel(const AdamArgs a) {
  // find the parameter owning this workgroup (binary search over block0)
  int lo = 0, hi = a.nparams - 1;
  const int64_t b = a.block_base + blockIdx.x;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.desc[mid].block0 <= b) lo = mid;
    else hi = mid - 1;
  }
  const AdamDesc d = a.desc[lo];
  const int64_t base = (b - d.block0) * ADAM_EPB;
  if (d.dtype == DT_BF16) adamw_tile<bf16>(d, base, a);
  else adamw_tile<float>(d, base, a);
}

}  // namespace muon
