// C ABI of libmuon: validation, workspace layout and the launch sequence of
// one Muon optimizer step.
//
// Per bucket chunk (units of one shape), standard method ("Muon Optimizer and
// the Distributed Implementation", sections "Formulation of Muon Optimizer"
// and "Newton-Schulz Iteration"):
//   K-M    M <- mu M + G;  U = G + mu M (Nesterov) or M;  Y0 = U^T of the wide
//          orientation (a tall parameter block already has that layout)
//          and partial sums of U^2  [momentum_kernel: wide; momentum_rows_kernel: tall]
//   norm   s^2 per unit, 1/s, 1/s^2                      [norm_finalize_kernel]
//   k = 0..steps-1 with (a_k, b_k, c_k):
//     A = X X^T            (k = 0: times 1/s^2, folding X0 = U / s)
//     P = a I + b A + c A A (symmetric: upper tiles, mirror-written)
//     X' = P X = a X + (b A + c A^2) X   (k = 0: times 1/s), computed as
//                          Y' = Y P^T on the transposed copy; the last step
//                          is computed in the parameter's layout (O^T = Y P^T
//                          for a tall unit, O = P Y^T for a wide one) and its
//                          epilogue applies W <- W (1 - lr wd) - lr scale O
// Gram method (DeepSpeed page: iterate on the square Gram matrix R = X X^T):
//   R = 2^e X0 X0^T / s^2 (power-of-two scaled, fp16 for a bf16 bucket);
//   P_k = a I + b R + c R^2;  Q <- P_k Q;  R <- P_k R P_k;  O = Q X0 / s.
//   Restarted chain (an extension): after ceil(steps / 2) steps X_r = Q X0 / s,
//   R = 2^e X_r X_r^T, Q = I; the remaining steps continue; O = Q X_r.
//   All of R_k, P_k, Q are polynomials in R_0: symmetric and commuting, so
//   every m x m product is computed as a symmetric one (upper tiles).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "consts.hpp"
#include "launch.hpp"
#include "libmuon.h"
#include "plan.hpp"
#include "timing.hpp"

using namespace muon;

namespace {

constexpr float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};

struct ChainParams {
  float mu;
  int32_t nesterov;
  int32_t steps;
  const float* coeffs;  // steps x 3
  float lr, wd;
  int32_t final_mode;
  int32_t vec_ok;
  int32_t has_mom;
  int32_t wvec;  // parameter / update_out rows 16-byte aligned (fused update epilogue)
};

int dt_dev(int32_t muon_dtype) { return muon_dtype == MUON_F32 ? DT_F32 : DT_BF16; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

GemmArgs gemm_args(int tile, int32_t cnt, int M, int N, int K, bool sym) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.M = M;
  g.N = N;
  g.K = K;
  g.units = cnt;
  g.tilesM = (int32_t)ceil_div(M, tile);
  g.tilesN = (int32_t)ceil_div(N, tile);
  g.tilesPerUnit = sym ? g.tilesM * (g.tilesM + 1) / 2 : g.tilesM * g.tilesN;
  g.totalTiles = g.tilesPerUnit * cnt;
  g.alpha = 1.f;
  return g;
}

#define HIP_TRY(x)                          \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return MUON_E_HIP; \
  } while (0)

// Momentum + norm for one chunk, then the Newton-Schulz chain and the fused
// update (or a plain store of O for ns_orthogonalize).  Every unit is kept
// as Y = X^T (n x m, the wide orientation transposed): the symmetric product
// A = X X^T = Y^T Y reads Y K-major, the update Y' = Y P^T reads it row-major,
// so one copy serves both.
muon_status run_chunk(const PlanBucket& b, const UnitDesc* d_desc, float4* d_aux, float* d_part,
                      char* data, int32_t cnt, const ChainParams& cp, hipStream_t st) {
  const int cdt = dt_dev(b.cdtype);
  const int pdt = dt_dev(b.pdtype);
  const int es = elem_size(b.cdtype);
  const int64_t m = b.m, n = b.n;
  const int64_t sy = n * b.mp, ss = m * b.mp;
  char* Y0 = data + b.off[0];

  // K-M: a tall unit's parameter block has the layout of Y (written as is), a
  // wide unit's is X (written transposed)
  MomArgs ma;
  std::memset(&ma, 0, sizeof(ma));
  ma.desc = d_desc;
  if (b.tall) {
    ma.D = Y0; ma.ldd = b.mp; ma.sD = sy;
  } else {
    ma.T = Y0; ma.ldt = b.mp; ma.sT = sy;
  }
  ma.partials = d_part;
  ma.rows = (int32_t)(b.tall ? n : m);
  ma.cols = (int32_t)(b.tall ? m : n);
  ma.tilesR = (int32_t)ceil_div(ma.rows, b.tall ? KMR_TR : KM_TR);
  ma.tilesC = (int32_t)ceil_div(ma.cols, b.tall ? KMR_TC : KM_TC);
  ma.tilesPerUnit = b.km_tiles;
  ma.mu = cp.mu;
  ma.nesterov = cp.nesterov;
  ma.vec_ok = cp.vec_ok;
  const double elems = (double)cnt * (double)m * (double)n;
  const double units = (double)cnt;
  const double mm_n = units * 2.0 * (double)m * (double)m * (double)n;  // 2 m^2 n per unit
  const double mmm = units * 2.0 * (double)m * (double)m * (double)m;   // 2 m^3 per unit
  const double pes = b.pdtype == MUON_F32 ? 4.0 : 2.0;
  const double km_bytes = elems * (pes + (cp.has_mom ? 8.0 : 0.0) + (double)es);
  HIP_TRY(timed(F_MOMENTUM, 0.0, km_bytes, st, [&] {
    return launch_momentum(pdt, cdt, b.tall != 0, ma, (int64_t)cnt * b.km_tiles, st);
  }));
  HIP_TRY(timed(F_NORM, 0.0, 0.0, st, [&] { return launch_norm_finalize(d_part, b.km_tiles, d_aux, cnt, st); }));

  const int T = b.tile;
  // The last product, fused with the parameter update, computed in the
  // parameter block's own layout so that the epilogue writes whole rows: a
  // tall unit's block has Y's layout, O^T = Y P^T (L = Y, R = P); a wide
  // unit's has X's, O = P X = P Y^T (L = P, R = Y).  Yop: the n x m operand
  // (Y), Pop: the m x m one (P, or Q for the Gram chain).
  auto final_gemm = [&](const void* Yop, const void* Pop) {
    GemmArgs g;
    if (b.tall) {
      g = gemm_args(T, cnt, (int)n, (int)m, (int)m, false);
      g.L = Yop; g.ldl = b.mp; g.sL = sy;
      g.R = Pop; g.ldr = b.mp; g.sR = ss;
    } else {
      g = gemm_args(T, cnt, (int)m, (int)n, (int)m, false);
      g.L = Pop; g.ldl = b.mp; g.sL = ss;
      g.R = Yop; g.ldr = b.mp; g.sR = sy;
    }
    g.desc = d_desc;
    g.lr = cp.lr;
    g.wd = cp.wd;
    g.finalMode = cp.final_mode;
    g.wvec = cp.wvec;
    return g;
  };
  // symmetric product L . R^T of m x m output into C (both triangles)
  auto sym_args = [&](const void* L, int64_t ldl, int64_t sL, const void* R, int64_t ldr, int64_t sR,
                      int K, void* C) {
    GemmArgs g = gemm_args(T, cnt, (int)m, (int)m, K, true);
    g.L = L; g.ldl = ldl; g.sL = sL;
    g.R = R; g.ldr = ldr; g.sR = sR;
    g.C = C; g.ldc = b.mp; g.sC = ss;
    g.C2 = C; g.ldc2 = b.mp; g.sC2 = ss;
    return g;
  };

  if (b.method == MUON_NS_STANDARD) {
    char* Y[2] = {Y0, data + b.off[1]};
    char* A = data + b.off[2];
    char* B = data + b.off[3];
    for (int k = 0; k < cp.steps; ++k) {
      const float ca = cp.coeffs[3 * k], cb = cp.coeffs[3 * k + 1], cc = cp.coeffs[3 * k + 2];
      // A = X X^T = Y^T Y  (k = 0: U U^T / s^2), Y read K-major
      GemmArgs g = sym_args(Y[k & 1], b.mp, sy, Y[k & 1], b.mp, sy, (int)n, A);
      g.alphaSel = k == 0 ? SEL_INV_S2 : SEL_ONE;
      g.aux = d_aux;
      HIP_TRY(timed(F_SYRK, mm_n, 0.0, st,
                    [&] { return launch_gemm(T, cdt, cdt, true, EPI_SCALE, true, g, st); }));
      // P = a I + b A + c A A^T  (a X + (b A + c A^2) X = P X: the a X term
      // rides on P's diagonal, so the update reads no addend)
      g = sym_args(A, b.mp, ss, A, b.mp, ss, (int)m, B);
      g.E = A; g.lde = b.mp; g.sE = ss;
      g.alpha = cc; g.beta = cb; g.gamma = ca;
      HIP_TRY(timed(F_POLY, mmm, 0.0, st,
                    [&] { return launch_gemm(T, cdt, cdt, true, EPI_POLY, false, g, st); }));
      // Y' = Y P^T  (k = 0: (P U)^T / s); the last one fused with the update
      if (k + 1 < cp.steps) {
        g = gemm_args(T, cnt, (int)n, (int)m, (int)m, false);
        g.L = Y[k & 1]; g.ldl = b.mp; g.sL = sy;
        g.R = B; g.ldr = b.mp; g.sR = ss;
        g.C = Y[(k + 1) & 1]; g.ldc = b.mp; g.sC = sy;
      } else {
        g = final_gemm(Y[k & 1], B);
      }
      g.alpha = 1.f; g.beta = 0.f;
      g.alphaSel = k == 0 ? SEL_INV_S : SEL_ONE;
      g.aux = d_aux;
      if (k + 1 < cp.steps) {
        HIP_TRY(timed(F_UPDATE, mm_n, 0.0, st,
                      [&] { return launch_gemm(T, cdt, cdt, false, EPI_SCALE, false, g, st); }));
      } else {
        HIP_TRY(timed(F_FINAL, mm_n, elems * 2.0 * pes, st,
                      [&] { return launch_gemm(T, cdt, pdt, false, EPI_FINAL, false, g, st); }));
      }
    }
    return MUON_OK;
  }

  // Gram chain: m x m work in fp16 (bf16 bucket) or fp32, R scaled by 2^e.
  // Z = Q^T is kept: Z' = Z P (P symmetric); the last product stores Q = Z'^T.
  const int sdt = cdt == DT_F32 ? DT_F32 : DT_F16;
  const int qdt_last = cdt == DT_F32 ? DT_F32 : DT_BF16;  // Q feeds the final GEMM with Y0
  float rs = 1.f;
  if (sdt == DT_F16) {
    int e = 0;
    while ((int64_t(1) << e) < m && e < 15) ++e;
    rs = std::ldexp(1.f, e);
  }
  char* R = data + b.off[1];
  char* Tm = data + b.off[2];
  char* PZ[3] = {data + b.off[3], data + b.off[4], data + b.off[5]};
  // Restarted chain: after `ra` steps X_r = Q X_0 is formed and the chain
  // starts again from it (R = 2^e X_r X_r^T, Q = I); the final product then
  // takes X_r.  Yb / bsel: the iterate the current chain started from and
  // the scale that turns it into X (1 / s for U).
  const int ra = restart_after(b.method, cp.steps);
  char* Yb = Y0;
  int bsel = SEL_INV_S;
  GemmArgs g = sym_args(Y0, b.mp, sy, Y0, b.mp, sy, (int)n, R);
  g.alpha = rs; g.alphaSel = SEL_INV_S2; g.aux = d_aux;
  HIP_TRY(timed(F_GRAM_R0, mm_n, 0.0, st,
                [&] { return launch_gemm(T, cdt, sdt, true, EPI_SCALE, true, g, st); }));
  int z = -1;  // buffer holding Z (after the last step: Q); -1: Q = I
  for (int k = 0; k < cp.steps; ++k) {
    const bool last = k + 1 == cp.steps;
    const bool restart = !last && ra > 0 && k + 1 == ra;
    // Q feeds a product with the 16-bit iterate after the last step and at a restart
    const int qdt = (last || restart) ? qdt_last : sdt;
    const float ca = cp.coeffs[3 * k], cb = cp.coeffs[3 * k + 1], cc = cp.coeffs[3 * k + 2];
    int p = 0;
    while (p == z) ++p;
    // P = a I + (b / rs) R + (c / rs^2) R R^T
    g = sym_args(R, b.mp, ss, R, b.mp, ss, (int)m, PZ[p]);
    g.E = R; g.lde = b.mp; g.sE = ss;
    g.alpha = cc / (rs * rs); g.beta = cb / rs; g.gamma = ca;
    HIP_TRY(timed(F_GRAM_P, mmm, 0.0, st, [&] {
      return launch_gemm(T, sdt, z < 0 ? qdt : sdt, true, EPI_POLY, false, g, st);
    }));
    if (z < 0) {
      z = p;  // Z_0 = P_0^T = P_0
    } else {
      int zn = 0;
      while (zn == z || zn == p) ++zn;
      // Z' = Z P.  Every R_k, P_k and their products are polynomials in R_0,
      // so they commute and are symmetric: Z = Q, and Z P is computed as a
      // symmetric product (upper tiles + mirror); the last one is Q itself
      g = sym_args(PZ[z], b.mp, ss, PZ[p], b.mp, ss, (int)m, PZ[zn]);
      HIP_TRY(timed(F_GRAM_Q, mmm, 0.0, st,
                    [&] { return launch_gemm(T, sdt, qdt, true, EPI_SCALE, false, g, st); }));
      z = zn;
    }
    if (restart) {
      // X_r = Q X_b, as Y_r = Y_b Q^T (Q symmetric): the standard method's update product
      char* Yr = data + b.off[6];
      g = gemm_args(T, cnt, (int)n, (int)m, (int)m, false);
      g.L = Yb; g.ldl = b.mp; g.sL = sy;
      g.R = PZ[z]; g.ldr = b.mp; g.sR = ss;
      g.C = Yr; g.ldc = b.mp; g.sC = sy;
      g.alpha = 1.f; g.beta = 0.f;
      g.alphaSel = bsel; g.aux = d_aux;
      HIP_TRY(timed(F_UPDATE, mm_n, 0.0, st,
                    [&] { return launch_gemm(T, cdt, cdt, false, EPI_SCALE, false, g, st); }));
      // R = 2^e X_r X_r^T = 2^e Y_r^T Y_r (Y_r read K-major)
      g = sym_args(Yr, b.mp, sy, Yr, b.mp, sy, (int)n, R);
      g.alpha = rs; g.alphaSel = SEL_ONE; g.aux = d_aux;
      HIP_TRY(timed(F_GRAM_R0, mm_n, 0.0, st,
                    [&] { return launch_gemm(T, cdt, sdt, true, EPI_SCALE, true, g, st); }));
      Yb = Yr;
      bsel = SEL_ONE;
      z = -1;
    } else if (!last) {
      // Tm = P R  (R symmetric: its rows serve as R^T; P and R commute, so
      // Tm is symmetric too: upper tiles + mirror)
      g = sym_args(PZ[p], b.mp, ss, R, b.mp, ss, (int)m, Tm);
      HIP_TRY(timed(F_GRAM_T, mmm, 0.0, st,
                    [&] { return launch_gemm(T, sdt, sdt, true, EPI_SCALE, false, g, st); }));
      // R = Tm P  (P symmetric; the result is symmetric: upper tiles + mirror)
      g = sym_args(Tm, b.mp, ss, PZ[p], b.mp, ss, (int)m, R);
      HIP_TRY(timed(F_GRAM_R, mmm, 0.0, st,
                    [&] { return launch_gemm(T, sdt, sdt, true, EPI_SCALE, false, g, st); }));
    }
  }
  // O = Q X0 / s (O^T = Y0 Q^T / s for a tall unit; after a restart Q X_r),
  // fused with the update
  g = final_gemm(Yb, PZ[z]);
  g.beta = 0.f;
  g.alphaSel = bsel;
  g.aux = d_aux;
  HIP_TRY(timed(F_FINAL, mm_n, elems * 2.0 * pes, st,
                [&] { return launch_gemm(T, cdt, pdt, false, EPI_FINAL, false, g, st); }));
  return MUON_OK;
}

bool finite(float x) { return std::isfinite(x); }

// Update scale of one unit (muon_scale_mode); u.rows x u.cols is the unit in
// parameter layout, u.scale_dim the resolved D.
double unit_scale(const muon_hparams& hp, const PlanUnit& u) {
  const double gamma = hp.extra_scale == 0.f ? 1.0 : (double)hp.extra_scale;
  switch (hp.scale_mode) {
    case MUON_SCALE_SPECTRAL: return gamma * std::sqrt((double)u.rows / (double)u.cols);
    case MUON_SCALE_UNIT_RMS: return gamma * std::sqrt((double)u.scale_dim);
    default: return gamma * (double)hp.rms_scale * std::sqrt((double)u.scale_dim);
  }
}

// Per-step (a, b, c), held by value (no heap use on the paths that must not
// allocate).
struct CoeffTable {
  float v[3 * MAX_NS_STEPS];
  const float* data() const { return v; }
};

muon_status coeff_table(int32_t steps, const float* coeffs, CoeffTable& out) {
  if (steps < 1 || steps > MAX_NS_STEPS) return MUON_E_ARG;
  for (int k = 0; k < steps; ++k)
    for (int j = 0; j < 3; ++j) {
      const float v = coeffs ? coeffs[3 * k + j] : kQuintic[j];
      if (!finite(v)) return MUON_E_ARG;
      out.v[3 * k + j] = v;
    }
  return MUON_OK;
}

char* align_base(void* p) {
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  return reinterpret_cast<char*>((u + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int32_t muon_version(void) { return 101; }

muon_status muon_ns_coefficients(int32_t kind, int32_t steps, float* out, size_t cap) {
  if (!out || steps < 1 || steps > MAX_NS_STEPS) return MUON_E_ARG;
  if (kind != MUON_COEFF_QUINTIC && kind != MUON_COEFF_HYBRID) return MUON_E_ARG;
  if (kind == MUON_COEFF_HYBRID && steps < 2) return MUON_E_ARG;
  if (cap < (size_t)steps * 3) return MUON_E_CAPACITY;
  const float refined[3] = {1.875f, -1.25f, 0.375f};
  for (int32_t k = 0; k < steps; ++k) {
    const float* c = (kind == MUON_COEFF_HYBRID && k >= steps - 2) ? refined : kQuintic;
    for (int j = 0; j < 3; ++j) out[3 * k + j] = c[j];
  }
  return MUON_OK;
}

const char* muon_status_string(int32_t s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_E_ARG: return "invalid argument";
    case MUON_E_SHAPE: return "invalid shape";
    case MUON_E_DTYPE: return "invalid dtype";
    case MUON_E_METHOD: return "invalid ns_method";
    case MUON_E_WORKSPACE: return "workspace missing or too small";
    case MUON_E_HIP: return "HIP runtime error";
    case MUON_E_PLAN: return "plan and call disagree";
    case MUON_E_CAPACITY: return "output array too small";
  }
  return "unknown status";
}

muon_status muon_plan_create(const muon_param_shape* table, int32_t n, const muon_plan_options* opts,
                             muon_plan** out) {
  if (!out) return MUON_E_ARG;
  *out = nullptr;
  muon_plan* p = new (std::nothrow) muon_plan;
  if (!p) return MUON_E_ARG;
  const muon_status st = build_plan(table, n, opts, p->impl);
  if (st != MUON_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MUON_OK;
}

void muon_plan_destroy(muon_plan* plan) { delete plan; }

muon_status muon_plan_workspace_bytes(const muon_plan* plan, size_t* bytes) {
  if (!plan || !bytes) return MUON_E_ARG;
  *bytes = plan->impl.lay.total;
  return MUON_OK;
}

muon_status muon_plan_buckets(const muon_plan* plan, int32_t* out, size_t cap, size_t* len) {
  if (!plan || !len) return MUON_E_ARG;
  const auto& B = plan->impl.buckets;
  const size_t need = B.size() * 8;
  *len = need;
  if (cap < need) return out || cap ? MUON_E_CAPACITY : MUON_OK;
  if (!out && need) return MUON_E_ARG;
  for (size_t i = 0; i < B.size(); ++i) {
    const int32_t v[8] = {B[i].m, B[i].n, B[i].tall, B[i].pdtype, B[i].cdtype, B[i].method,
                          B[i].first, B[i].count};
    std::memcpy(out + 8 * i, v, sizeof(v));
  }
  return MUON_OK;
}

muon_status muon_plan_units(const muon_plan* plan, int64_t* out, size_t cap, size_t* len) {
  if (!plan || !len) return MUON_E_ARG;
  const auto& U = plan->impl.units;
  const size_t need = U.size() * 6;
  *len = need;
  if (cap < need) return out || cap ? MUON_E_CAPACITY : MUON_OK;
  if (!out && need) return MUON_E_ARG;
  for (size_t i = 0; i < U.size(); ++i) {
    const int64_t v[6] = {U[i].param, U[i].row0, U[i].rows, U[i].cols, U[i].tall, U[i].scale_dim};
    std::memcpy(out + 6 * i, v, sizeof(v));
  }
  return MUON_OK;
}

muon_status muon_step(const muon_plan* plan, const muon_param_ptrs* ptrs, int32_t n,
                      const muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !hp) return MUON_E_ARG;
  const PlanImpl& P = plan->impl;
  if (n != (int32_t)P.table.size()) return MUON_E_PLAN;
  if (n > 0 && !ptrs) return MUON_E_ARG;
  CoeffTable coeffs;
  muon_status st = coeff_table(hp->ns_steps, hp->coeffs, coeffs);
  if (st != MUON_OK) return st;
  if (!finite(hp->lr) || !finite(hp->momentum) || !finite(hp->weight_decay) || !finite(hp->rms_scale))
    return MUON_E_ARG;
  if (!finite(hp->extra_scale) || hp->extra_scale < 0.f) return MUON_E_ARG;
  if (hp->scale_mode != MUON_SCALE_MOONLIGHT && hp->scale_mode != MUON_SCALE_SPECTRAL &&
      hp->scale_mode != MUON_SCALE_UNIT_RMS)
    return MUON_E_ARG;
  if (!P.adam.empty()) {
    if (!finite(hp->adam_lr) || !finite(hp->adam_beta1) || !finite(hp->adam_beta2) ||
        !finite(hp->adam_eps) || !finite(hp->adam_weight_decay) || hp->adam_step < 1)
      return MUON_E_ARG;
    if (hp->adam_beta1 >= 1.f || hp->adam_beta2 >= 1.f) return MUON_E_ARG;
  }
  // pointer checks
  for (int32_t p = 0; p < n; ++p) {
    const muon_param_shape& s = P.table[p];
    if (s.rows == 0 || s.cols == 0) continue;
    const muon_param_ptrs& q = ptrs[p];
    const size_t es = s.dtype == MUON_F32 ? 4 : 2;
    if (!q.param || !q.grad || !aligned(q.param, es) || !aligned(q.grad, es)) return MUON_E_ARG;
    if (s.kind == MUON_KIND_MUON) {
      if (!q.momentum || !aligned(q.momentum, 4)) return MUON_E_ARG;
      if (q.update_out && !aligned(q.update_out, 4)) return MUON_E_ARG;
    } else {
      if (!q.exp_avg || !q.exp_avg_sq || !aligned(q.exp_avg, 4) || !aligned(q.exp_avg_sq, 4))
        return MUON_E_ARG;
    }
  }
  if (P.lay.total > 0 && (!workspace || workspace_bytes < P.lay.total)) return MUON_E_WORKSPACE;
  if (P.lay.total == 0) return MUON_OK;
  hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
  char* ws = align_base(workspace);

  // per-unit descriptors, uploaded once per step
  std::vector<UnitDesc> hd(P.units.size());
  for (size_t i = 0; i < P.units.size(); ++i) {
    const PlanUnit& u = P.units[i];
    const muon_param_shape& s = P.table[u.param];
    const muon_param_ptrs& q = ptrs[u.param];
    const size_t es = s.dtype == MUON_F32 ? 4 : 2;
    const int64_t off = u.row0 * s.cols;
    UnitDesc d;
    std::memset(&d, 0, sizeof(d));
    d.g = static_cast<const char*>(q.grad) + off * es;
    d.mom = q.momentum + off;
    d.w = static_cast<char*>(q.param) + off * es;
    d.o = q.update_out ? q.update_out + off : nullptr;
    d.ld = s.cols;
    d.scale = (float)unit_scale(*hp, u);
    hd[i] = d;
  }
  std::vector<AdamDesc> ad;
  int64_t adam_blocks = 0;
  double adam_bytes = 0.0;
  for (int32_t p : P.adam) {
    const muon_param_shape& s = P.table[p];
    const int64_t numel = s.rows * s.cols;
    if (numel == 0) continue;
    const muon_param_ptrs& q = ptrs[p];
    AdamDesc d;
    std::memset(&d, 0, sizeof(d));
    d.w = q.param;
    d.g = q.grad;
    d.m = q.exp_avg;
    d.v = q.exp_avg_sq;
    d.numel = numel;
    d.block0 = adam_blocks;
    d.dtype = dt_dev(s.dtype);
    d.vec_ok = aligned(q.param, 16) && aligned(q.grad, 16) && aligned(q.exp_avg, 16) &&
               aligned(q.exp_avg_sq, 16);
    adam_blocks += ceil_div(numel, ADAM_EPB);
    adam_bytes += (double)numel * (s.dtype == MUON_F32 ? 28.0 : 22.0);
    ad.push_back(d);
  }
  UnitDesc* d_desc = reinterpret_cast<UnitDesc*>(ws + P.lay.off_desc);
  AdamDesc* d_adesc = reinterpret_cast<AdamDesc*>(ws + P.lay.off_adesc);
  // descriptor tables travel in kernel arguments: no host staging, no copy
  // from pageable memory, nothing the host waits for
  if (!hd.empty()) HIP_TRY(launch_upload(d_desc, hd.data(), hd.size() * sizeof(UnitDesc), st_));
  if (!ad.empty()) HIP_TRY(launch_upload(d_adesc, ad.data(), ad.size() * sizeof(AdamDesc), st_));

  ChainParams cp;
  cp.mu = hp->momentum;
  cp.nesterov = hp->nesterov ? 1 : 0;
  cp.steps = hp->ns_steps;
  cp.coeffs = coeffs.data();
  cp.lr = hp->lr;
  cp.wd = hp->weight_decay;
  cp.final_mode = FINAL_UPDATE;
  cp.has_mom = 1;
  float4* d_aux = reinterpret_cast<float4*>(ws + P.lay.off_aux);
  float* d_part = reinterpret_cast<float*>(ws + P.lay.off_part);
  char* data = ws + P.lay.off_data;
  for (const PlanBucket& b : P.buckets) {
    for (int32_t s0 = 0; s0 < b.count; s0 += b.chunk) {
      const int32_t cnt = std::min(b.chunk, b.count - s0);
      bool vec = true, wv = true;
      for (int32_t i = 0; i < cnt; ++i) {
        const UnitDesc& d = hd[(size_t)b.first + s0 + i];
        vec = vec && aligned(d.g, 16) && aligned(d.mom, 16) && (d.ld % 8 == 0);
        wv = wv && aligned(d.w, 16) && (!d.o || aligned(d.o, 16)) && (d.ld % 8 == 0);
      }
      cp.vec_ok = vec ? 1 : 0;
      cp.wvec = wv ? 1 : 0;
      st = run_chunk(b, d_desc + b.first + s0, d_aux, d_part, data, cnt, cp, st_);
      if (st != MUON_OK) return st;
    }
  }
  if (adam_blocks > 0) {
    AdamArgs aa;
    std::memset(&aa, 0, sizeof(aa));
    aa.desc = d_adesc;
    aa.nparams = (int32_t)ad.size();
    aa.one_minus_b1 = 1.f - hp->adam_beta1;
    aa.one_minus_b2 = 1.f - hp->adam_beta2;
    aa.eps = hp->adam_eps;
    aa.keep = 1.f - hp->adam_lr * hp->adam_weight_decay;
    const double t = (double)hp->adam_step;
    const double bc1 = 1.0 - std::pow((double)hp->adam_beta1, t);
    const double bc2 = 1.0 - std::pow((double)hp->adam_beta2, t);
    aa.step = (float)((double)hp->adam_lr * std::sqrt(bc2) / bc1);
    HIP_TRY(timed(F_ADAMW, 0.0, adam_bytes, st_, [&] { return launch_adamw(aa, adam_blocks, st_); }));
  }
  return MUON_OK;
}

static void ns_layout(const PlanBucket& b, size_t& off_aux, size_t& off_part, size_t& off_data,
                      size_t& total) {
  auto al = [](size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; };
  off_aux = al(sizeof(UnitDesc));
  off_part = off_aux + al(16);
  off_data = off_part + al((size_t)b.km_tiles * 4);
  total = off_data + b.data_bytes + WS_ALIGN;
}

static muon_status ns_bucket(int64_t rows, int64_t cols, int32_t dtype, int32_t method, PlanBucket& b) {
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_E_DTYPE;
  if (!valid_method(method)) return MUON_E_METHOD;
  if (rows < 0 || cols < 0 || rows > ((int64_t)1 << 30) || cols > ((int64_t)1 << 30)) return MUON_E_SHAPE;
  std::memset(&b, 0, sizeof(b));
  b.m = (int32_t)std::min(rows, cols);
  b.n = (int32_t)std::max(rows, cols);
  b.tall = rows > cols ? 1 : 0;
  b.pdtype = dtype;
  b.method = resolve_method(method, dtype, b.m, b.n);
  b.cdtype = resolve_cdtype(dtype, b.method, b.m, b.n);
  b.first = 0;
  b.count = 1;
  bucket_derive(b, ~size_t(0));
  if (!bucket_addressable(b)) return MUON_E_SHAPE;
  return MUON_OK;
}

muon_status ns_orthogonalize_workspace_bytes(int64_t rows, int64_t cols, int32_t dtype, int32_t method,
                                             size_t* bytes) {
  if (!bytes) return MUON_E_ARG;
  PlanBucket b;
  const muon_status st = ns_bucket(rows, cols, dtype, method, b);
  if (st != MUON_OK) return st;
  if (rows == 0 || cols == 0) {
    *bytes = 0;
    return MUON_OK;
  }
  size_t a, p, d, t;
  ns_layout(b, a, p, d, t);
  *bytes = t;
  return MUON_OK;
}

muon_status ns_orthogonalize(void* X, int64_t rows, int64_t cols, int64_t ld, int32_t dtype, int32_t steps,
                             const float* coeffs, int32_t method, void* workspace, size_t workspace_bytes,
                             void* stream) {
  PlanBucket b;
  muon_status st = ns_bucket(rows, cols, dtype, method, b);
  if (st != MUON_OK) return st;
  CoeffTable cf;
  st = coeff_table(steps, coeffs, cf);
  if (st != MUON_OK) return st;
  if (ld < cols) return MUON_E_SHAPE;
  if (rows == 0 || cols == 0) return MUON_OK;
  const size_t es = dtype == MUON_F32 ? 4 : 2;
  if (!X || !aligned(X, es)) return MUON_E_ARG;
  size_t off_aux, off_part, off_data, total;
  ns_layout(b, off_aux, off_part, off_data, total);
  if (!workspace || workspace_bytes < total) return MUON_E_WORKSPACE;
  hipStream_t st_ = reinterpret_cast<hipStream_t>(stream);
  char* ws = align_base(workspace);
  UnitDesc d;
  std::memset(&d, 0, sizeof(d));
  d.g = X;
  d.mom = nullptr;
  d.w = X;
  d.o = nullptr;
  d.ld = ld;
  d.scale = 0.f;
  HIP_TRY(launch_upload(ws, &d, sizeof(d), st_));
  ChainParams cp;
  cp.mu = 0.f;
  cp.nesterov = 0;
  cp.steps = steps;
  cp.coeffs = cf.data();
  cp.lr = 0.f;
  cp.wd = 0.f;
  cp.final_mode = FINAL_STORE;
  cp.has_mom = 0;
  cp.vec_ok = aligned(X, 16) && (ld % 8 == 0);
  cp.wvec = cp.vec_ok;
  return run_chunk(b, reinterpret_cast<UnitDesc*>(ws), reinterpret_cast<float4*>(ws + off_aux),
                   reinterpret_cast<float*>(ws + off_part), ws + off_data, 1, cp, st_);
}

}  // extern "C"
