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
// One workgroup handles a 32 x 128 tile of one unit (parameter layout).  The
// unit is written to the workspace X0 as a row-major m x n matrix with
// leading dimension ldx (zero padded): as is for a wide unit, transposed
// through LDS for a tall one, so every later GEMM sees a wide operand.
// Each workgroup writes one partial sum of U^2 (fp32, fixed order).
// ---------------------------------------------------------------------------

template <typename TG, typename TX>
__global__ __launch_bounds__(256) void momentum_kernel(const MomArgs a) {
  __shared__ float tile[KM_TR][KM_TC + 1];
  __shared__ float red[4];
  const int unit = blockIdx.x / a.tilesPerUnit;
  const int t = blockIdx.x - unit * a.tilesPerUnit;
  const int tr = t / a.tilesC, tc = t - tr * a.tilesC;
  const int r0 = tr * KM_TR, c0 = tc * KM_TC;
  const UnitDesc d = a.desc[unit];
  const TG* __restrict__ G = reinterpret_cast<const TG*>(d.g);
  float* __restrict__ M = d.mom;
  TX* __restrict__ X = reinterpret_cast<TX*>(a.D) + (int64_t)unit * a.sD;
  TX* __restrict__ XT = reinterpret_cast<TX*>(a.T) + (int64_t)unit * a.sT;

  const int tid = threadIdx.x;
  const int cg = tid & 15;   // 8-column group
  const int rr = tid >> 4;   // 0..15
  float ss = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int lr = rr + 16 * h;
    const int r = r0 + lr;
    const int c = c0 + cg * 8;
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = 0.f;
    if (r < a.rows && c < a.cols) {
      const int64_t off = (int64_t)r * d.ld + c;
      float g[8], m[8];
      const bool full = a.vec_ok && (c + 8 <= a.cols);
      if (full) {
        if constexpr (sizeof(TG) == 2) {
          u32x4 raw = *reinterpret_cast<const u32x4*>(G + off);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            g[e] = to_f32(__builtin_bit_cast(TG, (uint16_t)(raw[e >> 1] >> ((e & 1) * 16))));
        } else {
          f32x4 g0 = *reinterpret_cast<const f32x4*>(G + off);
          f32x4 g1 = *reinterpret_cast<const f32x4*>(G + off + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { g[e] = g0[e]; g[e + 4] = g1[e]; }
        }
        if (M) {
          f32x4 m0 = *reinterpret_cast<const f32x4*>(M + off);
          f32x4 m1 = *reinterpret_cast<const f32x4*>(M + off + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { m[e] = m0[e]; m[e + 4] = m1[e]; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool in = c + e < a.cols;
          g[e] = in ? to_f32(G[off + e]) : 0.f;
          m[e] = (in && M) ? M[off + e] : 0.f;
        }
      }
      if (M) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float mn = fmaf(a.mu, m[e], g[e]);
          m[e] = mn;
          u[e] = a.nesterov ? fmaf(a.mu, mn, g[e]) : mn;
        }
        if (full) {
          *reinterpret_cast<f32x4*>(M + off) = f32x4{m[0], m[1], m[2], m[3]};
          *reinterpret_cast<f32x4*>(M + off + 4) = f32x4{m[4], m[5], m[6], m[7]};
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < a.cols) M[off + e] = m[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = g[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(u[e], u[e], ss);
    }
    // own layout: row r, columns c..c+8 (columns past cols are zero padding)
    if (r < a.rows && c < a.cols) {
      TX* dst = X + (int64_t)r * a.ldd + c;
      if constexpr (sizeof(TX) == 2) {
        u32x4 p;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p[j] = (uint32_t)bits16(from_f32<TX>(u[2 * j])) |
                 ((uint32_t)bits16(from_f32<TX>(u[2 * j + 1])) << 16);
        *reinterpret_cast<u32x4*>(dst) = p;
      } else {
        *reinterpret_cast<f32x4*>(dst) = f32x4{u[0], u[1], u[2], u[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{u[4], u[5], u[6], u[7]};
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[lr][cg * 8 + e] = u[e];
  }
  {
    __syncthreads();
    // transposed layout: row (c0 + c), columns r0 .. r0+32: 128 rows x 4 chunks of 8
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j;
      const int c = q >> 2, rq = q & 3;
      const int gc = c0 + c, gr = r0 + rq * 8;
      if (gc < a.cols && gr < a.rows) {
        TX* dst = XT + (int64_t)gc * a.ldt + gr;
        float u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = tile[rq * 8 + e][c];
        if constexpr (sizeof(TX) == 2) {
          u32x4 p;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            p[k] = (uint32_t)bits16(from_f32<TX>(u[2 * k])) |
                   ((uint32_t)bits16(from_f32<TX>(u[2 * k + 1])) << 16);
          *reinterpret_cast<u32x4*>(dst) = p;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{u[0], u[1], u[2], u[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{u[4], u[5], u[6], u[7]};
        }
      }
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
  for (int it = 0; it < ADAM_EPB / (256 * 8); ++it) {
    const int64_t i0 = base + (int64_t)(it * 256 + threadIdx.x) * 8;
    if (i0 >= d.numel) break;
    if (d.vec_ok && i0 + 8 <= d.numel) {
      float w[8], g[8], m[8], v[8];
      f32x4 m0 = *reinterpret_cast<const f32x4*>(d.m + i0), m1 = *reinterpret_cast<const f32x4*>(d.m + i0 + 4);
      f32x4 v0 = *reinterpret_cast<const f32x4*>(d.v + i0), v1 = *reinterpret_cast<const f32x4*>(d.v + i0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { m[e] = m0[e]; m[e + 4] = m1[e]; v[e] = v0[e]; v[e + 4] = v1[e]; }
      if (d.dtype == DT_BF16) {
        u32x4 wr = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(d.w) + i0);
        u32x4 gr = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(d.g) + i0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w[e] = to_f32(__builtin_bit_cast(bf16, (uint16_t)(wr[e >> 1] >> ((e & 1) * 16))));
          g[e] = to_f32(__builtin_bit_cast(bf16, (uint16_t)(gr[e >> 1] >> ((e & 1) * 16))));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) adam_elem(w[e], g[e], m[e], v[e], a);
        u32x4 wo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wo[j] = (uint32_t)bits16(from_f32<bf16>(w[2 * j])) | ((uint32_t)bits16(from_f32<bf16>(w[2 * j + 1])) << 16);
        *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(d.w) + i0) = wo;
      } else {
        const float* wp = reinterpret_cast<const float*>(d.w) + i0;
        const float* gp = reinterpret_cast<const float*>(d.g) + i0;
        f32x4 w0 = *reinterpret_cast<const f32x4*>(wp), w1 = *reinterpret_cast<const f32x4*>(wp + 4);
        f32x4 g0 = *reinterpret_cast<const f32x4*>(gp), g1 = *reinterpret_cast<const f32x4*>(gp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { w[e] = w0[e]; w[e + 4] = w1[e]; g[e] = g0[e]; g[e + 4] = g1[e]; }
#pragma unroll
        for (int e = 0; e < 8; ++e) adam_elem(w[e], g[e], m[e], v[e], a);
        float* wq = reinterpret_cast<float*>(d.w) + i0;
        *reinterpret_cast<f32x4*>(wq) = f32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<f32x4*>(wq + 4) = f32x4{w[4], w[5], w[6], w[7]};
      }
      *reinterpret_cast<f32x4*>(d.m + i0) = f32x4{m[0], m[1], m[2], m[3]};
      *reinterpret_cast<f32x4*>(d.m + i0 + 4) = f32x4{m[4], m[5], m[6], m[7]};
      *reinterpret_cast<f32x4*>(d.v + i0) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(d.v + i0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
      for (int e = 0; e < 8; ++e) {
        const int64_t i = i0 + e;
        if (i >= d.numel) break;
        float w, g;
        if (d.dtype == DT_BF16) {
          w = to_f32(reinterpret_cast<const bf16*>(d.w)[i]);
          g = to_f32(reinterpret_cast<const bf16*>(d.g)[i]);
        } else {
          w = reinterpret_cast<const float*>(d.w)[i];
          g = reinterpret_cast<const float*>(d.g)[i];
        }
        float m = d.m[i], v = d.v[i];
        adam_elem(w, g, m, v, a);
        d.m[i] = m;
        d.v[i] = v;
        if (d.dtype == DT_BF16) reinterpret_cast<bf16*>(d.w)[i] = from_f32<bf16>(w);
        else reinterpret_cast<float*>(d.w)[i] = w;
      }
    }
  }
}

}  // namespace muon
