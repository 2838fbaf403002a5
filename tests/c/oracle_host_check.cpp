// Host driver of the C++ fp64 reference (oracle/muon_ref.cpp) for builds
// under the address, undefined-behaviour and thread sanitizers.
//   oracle_host_check plan   reads shape tables from stdin in the format of
//                            plan_host_check and prints their units and
//                            buckets (ref_plan).
//   oracle_host_check math T runs every reference routine with T worker
//                            threads on seeded inputs of awkward shapes and
//                            prints one line per call; exit status 1 when an
//                            output is not finite.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

extern "C" {
void ref_set_threads(int32_t n);
void ref_momentum(double* M, const double* G, int64_t count, double mu, int32_t nesterov, double* U);
int32_t ref_orthogonalize(const double* G, int64_t rows, int64_t cols, int32_t steps, const double* coeffs,
                          int32_t method, double* O);
double ref_muon_scale_mode(int64_t rows, int64_t cols, int64_t scale_dim, double rms_scale, int32_t mode,
                           double gamma);
int32_t ref_coefficients(int32_t kind, int32_t steps, double* out);
void ref_weight_update(double* W, const double* O, int64_t count, double lr, double wd, double scale);
void ref_adamw(double* W, const double* g, double* m, double* v, int64_t count, int64_t t, double lr, double b1,
               double b2, double eps, double wd);
int64_t ref_plan(const int64_t* table, int32_t n, int32_t method, int32_t ns_dtype, int64_t* units_out,
                 int64_t units_cap, int32_t* buckets_out, int32_t buckets_cap, int32_t* nbuckets);
}

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
double uniform_pm1() {  // xorshift64*, mapped to [-1, 1)
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  const uint64_t r = g_state * 0x2545f4914f6cdd1dull;
  return (double)(r >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
std::vector<double> fill(size_t n) {
  std::vector<double> v(n);
  for (double& x : v) x = uniform_pm1();
  return v;
}
bool finite(const std::vector<double>& v) {
  for (double x : v)
    if (!std::isfinite(x)) return false;
  return true;
}

int run_plan() {
  int n, method, ns_dtype;
  while (std::scanf("%d %d %d", &n, &method, &ns_dtype) == 3) {
    std::vector<int64_t> t((size_t)(n > 0 ? n : 0) * 6);
    for (auto& x : t) {
      long long v;
      if (std::scanf("%lld", &v) != 1) return 2;
      x = v;
    }
    int64_t cap = 0;
    for (int p = 0; p < n; ++p) {
      const int64_t* r = &t[(size_t)p * 6];
      if (r[0] == 0 && r[2] > 0 && r[3] > 0) cap += r[4] > 0 ? r[2] / r[4] : 1;
    }
    std::vector<int64_t> units((size_t)(cap > 0 ? cap : 1) * 6);
    std::vector<int32_t> buckets((size_t)(cap > 0 ? cap : 1) * 8);
    int32_t nb = 0;
    const int64_t nu = ref_plan(t.empty() ? nullptr : t.data(), n, method, ns_dtype, units.data(), cap,
                                buckets.data(), (int32_t)(cap > 0 ? cap : 1), &nb);
    std::printf("status %d\n", nu < 0 ? -1 : 0);
    for (int64_t i = 0; i < nu; ++i) {
      const int64_t* u = &units[(size_t)i * 6];
      std::printf("unit %lld %lld %lld %lld %lld %lld\n", (long long)u[0], (long long)u[1], (long long)u[2],
                  (long long)u[3], (long long)u[4], (long long)u[5]);
    }
    for (int32_t b = 0; nu >= 0 && b < nb; ++b) {
      const int32_t* o = &buckets[(size_t)b * 8];
      std::printf("bucket %d %d %d %d %d %d %d %d\n", o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]);
    }
    std::printf("end\n");
  }
  return 0;
}

int run_math(int threads) {
  ref_set_threads(threads);
  int bad = 0;
  const int64_t shapes[][2] = {{1, 1}, {1, 9}, {9, 1}, {2, 3}, {3, 2}, {17, 9}, {9, 17}, {33, 70}, {70, 33}, {64, 64},
                               {0, 5}, {5, 0}};
  for (const auto& s : shapes) {
    const int64_t r = s[0], c = s[1];
    const size_t cnt = (size_t)(r * c);
    for (int method : {0, 1, 3}) {
      for (int steps = 0; steps <= 6; steps += 3) {
        const std::vector<double> G = fill(cnt);
        std::vector<double> coeffs = fill((size_t)steps * 3 + 1);
        for (double& x : coeffs) x *= 0.5;
        std::vector<double> O(cnt + 1, 0.0);
        const int32_t rc1 = ref_orthogonalize(G.data(), r, c, steps, nullptr, method, O.data());
        const bool ok1 = rc1 == 0 && finite(O);
        const int32_t rc2 = ref_orthogonalize(G.data(), r, c, steps, steps ? coeffs.data() : nullptr, method, O.data());
        const bool ok2 = rc2 == 0 && finite(O);
        std::printf("orthogonalize %lld %lld method %d steps %d: %s\n", (long long)r, (long long)c, method, steps,
                    ok1 && ok2 ? "ok" : "bad");
        bad += !(ok1 && ok2);
      }
    }
    std::vector<double> zero(cnt), O(cnt + 1, 1.0);
    const bool okz = ref_orthogonalize(zero.data(), r, c, 5, nullptr, 0, O.data()) == 0 && finite(O);
    bad += !okz;
  }
  if (ref_orthogonalize(nullptr, -1, 3, 5, nullptr, 0, nullptr) != -1) ++bad;
  if (ref_orthogonalize(nullptr, 3, 3, 5, nullptr, 7, nullptr) != -1) ++bad;

  for (int steps = 1; steps <= 64; ++steps) {
    std::vector<double> c((size_t)steps * 3);
    bad += ref_coefficients(0, steps, c.data()) != 0 || !finite(c);
    if (steps >= 2) bad += ref_coefficients(1, steps, c.data()) != 0 || !finite(c);
  }
  bad += ref_coefficients(1, 1, nullptr) != -1;
  bad += ref_coefficients(2, 5, nullptr) != -1;

  for (int mode = 0; mode < 3; ++mode) bad += !std::isfinite(ref_muon_scale_mode(3, 7, mode == 2 ? 11 : 0, 0.2, mode, 1.5));
  bad += ref_muon_scale_mode(3, 7, 0, 0.2, 3, 1.0) != -1.0;

  for (int64_t count : {0, 1, 7, 1001}) {
    std::vector<double> M = fill((size_t)count), G = fill((size_t)count), U((size_t)count);
    ref_momentum(M.data(), G.data(), count, 0.95, 1, U.data());
    ref_momentum(M.data(), G.data(), count, 0.95, 0, U.data());
    std::vector<double> W = fill((size_t)count);
    ref_weight_update(W.data(), U.data(), count, 0.02, 0.1, 0.2);
    std::vector<double> m((size_t)count, 0.0), v((size_t)count, 0.0);
    for (int64_t t = 1; t <= 3; ++t) ref_adamw(W.data(), G.data(), m.data(), v.data(), count, t, 3e-4, 0.9, 0.95, 1e-8, 0.1);
    const bool ok = finite(M) && finite(U) && finite(W) && finite(m) && finite(v);
    std::printf("elementwise %lld: %s\n", (long long)count, ok ? "ok" : "bad");
    bad += !ok;
  }
  std::printf("math %s\n", bad ? "bad" : "ok");
  return bad ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "plan") == 0) return run_plan();
  if (argc >= 3 && std::strcmp(argv[1], "math") == 0) return run_math(std::atoi(argv[2]));
  std::fprintf(stderr, "usage: oracle_host_check plan | math THREADS\n");
  return 2;
}
