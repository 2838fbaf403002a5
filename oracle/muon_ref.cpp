// Plain fp64 C++ reference of the Muon optimizer step.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
// call this file's library: only the test suite, the package's smoke check
// and the benchmark's CPU-baseline leg use it.  It shares no code with the
// HIP library (no kernels, headers, helpers or constants) and no code with
// the numpy reference next to it; the three meet only through the seeded
// input generators.
//
// Every step is written from the pages, in their order and notation, in
// double precision, single source, no BLAS.  Matrix products are plain
// triple loops whose sums run over k in increasing order; the only
// concession to speed is that independent output rows are shared among
// std::threads, which changes no arithmetic.
//
// Sources (web pages; cited by title and section):
//   [Blog]      "Muon Optimizer and the Distributed Implementation" —
//               "Formulation of Muon Optimizer", "Sign of a Matrix",
//               "Newton-Schulz Iteration", "Variation of Muon Optimizer"
//   [Moonlight] the Kimi/Moonlight summary page — "权重衰减机制",
//               "参数更新尺度调整:一致的更新 RMS", "代码" (the printed Muon class)
//   [DeepSpeed] "DeepSpeed 集成 Muon 优化器实战…" — NS_METHODS and the Gram
//               variant
//   [MindSpeed] the MindSpeed "Muon 优化器" document — QKV split
//
// Build: g++ -O2 -std=c++17 -fPIC -shared -pthread (no fast-math: the
// summation order of every dot product is the one written here).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

int g_threads = 0;  // 0: std::thread::hardware_concurrency()

int thread_count() {
  int t = g_threads > 0 ? g_threads : (int)std::thread::hardware_concurrency();
  return t > 0 ? t : 1;
}

// Runs body(i) for i in [0, n) on the worker threads, rows split in
// contiguous ranges.
template <typename F> void parallel_rows(int64_t n, F body) {
  const int64_t nt = std::min<int64_t>(thread_count(), std::max<int64_t>(n, 1));
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (n + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t lo = t * per, hi = std::min(n, lo + per);
    if (lo >= hi) break;
    pool.emplace_back([=] {
      for (int64_t i = lo; i < hi; ++i) body(i);
    });
  }
  for (auto& th : pool) th.join();
}

using Mat = std::vector<double>;  // row-major

// C (M x N) = A (M x K) * B (K x N): C[i][j] = sum_k A[i][k] B[k][j], k ascending.
Mat matmul(const Mat& A, const Mat& B, int64_t M, int64_t K, int64_t N) {
  Mat C((size_t)(M * N), 0.0);
  parallel_rows(M, [&](int64_t i) {
    double* c = &C[(size_t)(i * N)];
    for (int64_t k = 0; k < K; ++k) {
      const double a = A[(size_t)(i * K + k)];
      const double* b = &B[(size_t)(k * N)];
      for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
    }
  });
  return C;
}

Mat transpose(const Mat& A, int64_t M, int64_t N) {
  Mat T((size_t)(M * N));
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) T[(size_t)(j * M + i)] = A[(size_t)(i * N + j)];
  return T;
}

Mat identity(int64_t m) {
  Mat I((size_t)(m * m), 0.0);
  for (int64_t i = 0; i < m; ++i) I[(size_t)(i * m + i)] = 1.0;
  return I;
}

// [Blog] "Newton-Schulz Iteration": X <- a X + (b A + c A A) X with A = X X^T,
// one (a, b, c) per step; X is m x n with m <= n, already normalized.
Mat ns_standard(Mat X, int64_t m, int64_t n, const double* coeffs, int steps) {
  for (int k = 0; k < steps; ++k) {
    const double a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
    const Mat Xt = transpose(X, m, n);
    const Mat A = matmul(X, Xt, m, n, m);
    const Mat AA = matmul(A, A, m, m, m);
    Mat B((size_t)(m * m));
    for (size_t e = 0; e < B.size(); ++e) B[e] = b * A[e] + c * AA[e];
    const Mat BX = matmul(B, X, m, m, n);
    for (size_t e = 0; e < X.size(); ++e) X[e] = a * X[e] + BX[e];
  }
  return X;
}

// [DeepSpeed] Gram variant: iterate on the square R = X X^T.  The page states
// only that; the reading taken is the exact rewrite of the standard step:
// P_k = a I + b R_k + c R_k R_k, X_{k+1} = P_k X_k, so R_{k+1} = P_k R_k P_k
// and the result is Q X_0 with Q = P_{N-1} ... P_0.  restart > 0: after that
// many steps the chain restarts once (an extension; the pages have none):
// X_r = Q X_0 is formed, R = X_r X_r^T recomputed and Q reset to I.
Mat ns_gram(const Mat& X0, int64_t m, int64_t n, const double* coeffs, int steps, int restart) {
  Mat X = X0;
  Mat R = matmul(X, transpose(X, m, n), m, n, m);
  Mat Q = identity(m);
  for (int k = 0; k < steps; ++k) {
    const double a = coeffs[3 * k], b = coeffs[3 * k + 1], c = coeffs[3 * k + 2];
    const Mat RR = matmul(R, R, m, m, m);
    Mat P((size_t)(m * m));
    for (int64_t i = 0; i < m; ++i)
      for (int64_t j = 0; j < m; ++j) {
        const size_t e = (size_t)(i * m + j);
        P[e] = (i == j ? a : 0.0) + b * R[e] + c * RR[e];
      }
    Q = matmul(P, Q, m, m, m);
    if (k + 1 == steps) break;
    if (restart > 0 && k + 1 == restart) {
      X = matmul(Q, X, m, m, n);
      R = matmul(X, transpose(X, m, n), m, n, m);
      Q = identity(m);
    } else {
      R = matmul(matmul(P, R, m, m, m), P, m, m, m);
    }
  }
  return matmul(Q, X, m, m, n);
}

const double kQuintic[3] = {3.4445, -4.7750, 2.0315};  // [Blog] "Newton-Schulz Iteration"

}  // namespace

extern "C" {

// Worker threads of the matrix products (0 = all hardware threads).
void ref_set_threads(int32_t n) { g_threads = n; }
int32_t ref_threads(void) { return thread_count(); }

// [Blog] "Formulation of Muon Optimizer": M <- mu M + G; the matrix to
// orthogonalize is G + mu M (Nesterov; "Variation of Muon Optimizer" and the
// [Moonlight] code) or M.  M updated in place, U written.
void ref_momentum(double* M, const double* G, int64_t count, double mu, int32_t nesterov, double* U) {
  for (int64_t i = 0; i < count; ++i) {
    M[i] = mu * M[i] + G[i];
    U[i] = nesterov ? G[i] + mu * M[i] : M[i];
  }
}

// NewtonSchulz(G) of one rows x cols matrix into O (same shape).  A tall G
// is processed as its transpose ([Blog] "Sign of a Matrix": msign(G) =
// (G G^T)^{-1/2} G = G (G^T G)^{-1/2}), G is divided by its Frobenius norm
// ("Newton-Schulz Iteration"; a zero matrix gives O = 0), then `steps`
// iterations with coeffs (steps x 3, or null for the quintic every step).
// method 0 = standard, 1 = Gram, 3 = Gram restarted after ceil(steps / 2)
// steps (steps >= 2).  Returns 0, or -1 for bad arguments.
int32_t ref_orthogonalize(const double* G, int64_t rows, int64_t cols, int32_t steps, const double* coeffs,
                          int32_t method, double* O) {
  if (rows < 0 || cols < 0 || steps < 0 || (method != 0 && method != 1 && method != 3)) return -1;
  const size_t cnt = (size_t)(rows * cols);
  if (cnt == 0) return 0;
  std::vector<double> sched((size_t)steps * 3);
  for (int k = 0; k < steps; ++k)
    for (int j = 0; j < 3; ++j) sched[(size_t)(3 * k + j)] = coeffs ? coeffs[3 * k + j] : kQuintic[j];
  const bool tall = rows > cols;
  const int64_t m = tall ? cols : rows, n = tall ? rows : cols;
  Mat X(G, G + cnt);
  if (tall) X = transpose(X, rows, cols);
  double ss = 0.0;
  for (size_t e = 0; e < cnt; ++e) ss += X[e] * X[e];
  const double s = std::sqrt(ss);
  if (s == 0.0) {
    std::memset(O, 0, cnt * sizeof(double));
    return 0;
  }
  for (size_t e = 0; e < cnt; ++e) X[e] /= s;
  const int restart = method == 3 && steps >= 2 ? (steps + 1) / 2 : 0;
  X = method == 0 ? ns_standard(X, m, n, sched.data(), steps) : ns_gram(X, m, n, sched.data(), steps, restart);
  if (tall) X = transpose(X, m, n);
  std::memcpy(O, X.data(), cnt * sizeof(double));
  return 0;
}

// Scale of the orthogonalized update of a rows x cols unit (d_out x d_in),
// D = scale_dim if > 0 else max(rows, cols) (the reading for split blocks is
// the block's own shape):
//   mode 0: rms_scale sqrt(D)      [Moonlight] "参数更新尺度调整" (0.2)
//   mode 1: sqrt(d_out / d_in)     [Blog] "Variation of Muon Optimizer" (muP)
//   mode 2: sqrt(D)                [Blog] DeepSeek-V4 listing, "Rescale update RMS"
// times gamma (the listing's update rescaling factor).  Returns -1 for an
// unknown mode.
double ref_muon_scale_mode(int64_t rows, int64_t cols, int64_t scale_dim, double rms_scale, int32_t mode,
                           double gamma) {
  const int64_t d = scale_dim > 0 ? scale_dim : std::max(rows, cols);
  switch (mode) {
    case 0: return gamma * rms_scale * std::sqrt((double)d);
    case 1: return gamma * std::sqrt((double)rows / (double)cols);
    case 2: return gamma * std::sqrt((double)d);
  }
  return -1.0;
}

double ref_muon_scale(int64_t rows, int64_t cols, int64_t scale_dim, double rms_scale) {
  return ref_muon_scale_mode(rows, cols, scale_dim, rms_scale, 0, 1.0);
}

// [Blog] DeepSeek-V4 listing: ten Newton-Schulz steps, eight with the quintic
// and two with an improved Newton iteration (coefficients not printed; read
// as the odd quintic with p(1) = 1, p'(1) = p''(1) = 0: (15/8, -5/4, 3/8)).
// kind 0: quintic every step; kind 1: that hybrid, steps >= 2.  Writes
// steps x 3 doubles; returns 0 or -1.
int32_t ref_coefficients(int32_t kind, int32_t steps, double* out) {
  if (steps < 1 || (kind != 0 && kind != 1) || (kind == 1 && steps < 2)) return -1;
  const double refined[3] = {15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0};
  for (int32_t k = 0; k < steps; ++k)
    for (int j = 0; j < 3; ++j) out[3 * k + j] = (kind == 1 && k >= steps - 2) ? refined[j] : kQuintic[j];
  return 0;
}

// [Moonlight] "权重衰减机制" / "代码": W <- W (1 - lr wd) - lr scale O.
void ref_weight_update(double* W, const double* O, int64_t count, double lr, double wd, double scale) {
  for (int64_t i = 0; i < count; ++i) W[i] = W[i] * (1.0 - lr * wd) - (lr * scale) * O[i];
}

// The AdamW fallback for the parameters Muon does not take ([Moonlight]
// "代码": the optimizer's AdamW backup), step t >= 1:
//   m_t = b1 m + (1 - b1) g,  v_t = b2 v + (1 - b2) g^2,
//   W_t = W (1 - lr wd) - lr sqrt(1 - b2^t) / (1 - b1^t) * m_t / (eps + sqrt(v_t))
// (the bias corrections scale the step, so eps meets the uncorrected sqrt(v_t)).
void ref_adamw(double* W, const double* g, double* m, double* v, int64_t count, int64_t t, double lr,
               double b1, double b2, double eps, double wd) {
  const double step = lr * std::sqrt(1.0 - std::pow(b2, (double)t)) / (1.0 - std::pow(b1, (double)t));
  for (int64_t i = 0; i < count; ++i) {
    m[i] = b1 * m[i] + (1.0 - b1) * g[i];
    v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
    W[i] = W[i] * (1.0 - lr * wd) - step * (m[i] / (eps + std::sqrt(v[i])));
  }
}

// Shape table -> units -> buckets, by brute force.  table: n rows of 6
// int64 (kind, dtype, rows, cols, split_rows, scale_dim).  A Muon parameter
// becomes one unit, or one per row block of split_rows ([MindSpeed] QKV
// split); units with equal (m, n, tall, param dtype, compute dtype, method)
// share a bucket, buckets numbered by first appearance, units in table
// order.  units_out: 6 int64 per unit (param, row0, rows, cols, tall,
// scale_dim resolved), in bucket order; buckets_out: 8 int32 per bucket
// (m, n, tall, pdtype, cdtype, method, first, count).  Returns the unit
// count (or -1 when a capacity is exceeded); *nbuckets gets the bucket count.
int64_t ref_plan(const int64_t* table, int32_t n, int32_t method, int32_t ns_dtype, int64_t* units_out,
                 int64_t units_cap, int32_t* buckets_out, int32_t buckets_cap, int32_t* nbuckets) {
  struct U { int64_t p, r0, rows, cols, tall, sd; };
  std::vector<U> order;
  for (int32_t p = 0; p < n; ++p) {
    const int64_t* t = table + 6 * p;
    if (t[0] != 0 || t[2] == 0 || t[3] == 0) continue;
    const int64_t h = t[4] > 0 ? t[4] : t[2];
    for (int64_t r = 0; r < t[2]; r += h)
      order.push_back({p, r, h, t[3], h > t[3] ? 1 : 0, t[5] > 0 ? t[5] : std::max(h, t[3])});
  }
  std::vector<std::vector<int64_t>> keys, members;
  for (size_t i = 0; i < order.size(); ++i) {
    const U& u = order[i];
    const int64_t pdt = table[6 * u.p + 1];
    const int64_t m = std::min(u.rows, u.cols), nn = std::max(u.rows, u.cols);
    // Gram's fp16 chain is within the bf16 tolerance only for m >= 512 and
    // n >= 3m: method 2 picks Gram there (where it also does less work).
    // An explicit Gram request outside it runs its chain in fp32 when the
    // requested compute dtype is bf16 (code 1 -> 0), and runs the standard
    // method when it is fp32 (the fp32 chain there is above the fp32
    // tolerance).  The restarted chain (3) stays 3 for a bf16 compute dtype
    // when m >= 256 and is taken as a Gram request (1) otherwise.
    const bool fp16_ok = m >= 512 && nn >= 3 * m;
    int64_t cdt = ns_dtype < 0 ? pdt : ns_dtype;
    int64_t meth = method;
    if (method == 3 && (cdt == 0 || m < 256)) meth = 1;
    if (method == 2) meth = fp16_ok ? 1 : 0;
    else if (meth == 1 && cdt == 0 && !fp16_ok) meth = 0;
    if (meth == 1 && cdt == 1 && !fp16_ok) cdt = 0;
    const std::vector<int64_t> key = {m, nn, u.tall, pdt, cdt, meth};
    size_t b = 0;
    while (b < keys.size() && keys[b] != key) ++b;
    if (b == keys.size()) {
      keys.push_back(key);
      members.emplace_back();
    }
    members[b].push_back((int64_t)i);
  }
  if ((int64_t)order.size() > units_cap || (int64_t)keys.size() > buckets_cap) return -1;
  int64_t w = 0;
  for (size_t b = 0; b < keys.size(); ++b) {
    int32_t* o = buckets_out + 8 * b;
    for (int j = 0; j < 6; ++j) o[j] = (int32_t)keys[b][(size_t)j];
    o[6] = (int32_t)w;
    o[7] = (int32_t)members[b].size();
    for (int64_t i : members[b]) {
      const U& u = order[(size_t)i];
      const int64_t v[6] = {u.p, u.r0, u.rows, u.cols, u.tall, u.sd};
      std::memcpy(units_out + 6 * w, v, sizeof(v));
      ++w;
    }
  }
  *nbuckets = (int32_t)keys.size();
  return w;
}

}  // extern "C"
