// Host driver of the library's planner (csrc/plan.cpp, no HIP) for builds
// under the address and undefined-behaviour sanitizers.  Reads shape tables
// from stdin, each as a line "n method ns_dtype" followed by n rows of
// "kind dtype rows cols split_rows scale_dim", and prints for each its
// status, its units and buckets (the lines the reference planner prints too)
// and the chunk and workspace layout figures ("derived" lines).
#include <cstdio>
#include <vector>

#include "plan.hpp"

int main() {
  int n, method, ns_dtype;
  while (std::scanf("%d %d %d", &n, &method, &ns_dtype) == 3) {
    std::vector<muon_param_shape> t((size_t)(n > 0 ? n : 0));
    for (auto& s : t) {
      long long v[6];
      if (std::scanf("%lld %lld %lld %lld %lld %lld", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5]) != 6) return 2;
      s.kind = (int32_t)v[0];
      s.dtype = (int32_t)v[1];
      s.rows = v[2];
      s.cols = v[3];
      s.split_rows = v[4];
      s.scale_dim = v[5];
    }
    muon::PlanImpl P;
    const muon_plan_options o{method, ns_dtype};
    const muon_status st = muon::build_plan(t.empty() ? nullptr : t.data(), n, &o, P);
    std::printf("status %d\n", (int)st);
    if (st == MUON_OK) {
      for (const muon::PlanUnit& u : P.units)
        std::printf("unit %d %lld %lld %lld %d %lld\n", u.param, (long long)u.row0, (long long)u.rows,
                    (long long)u.cols, u.tall, (long long)u.scale_dim);
      for (const muon::PlanBucket& b : P.buckets) {
        std::printf("bucket %d %d %d %d %d %d %d %d\n", b.m, b.n, b.tall, b.pdtype, b.cdtype, b.method, b.first,
                    b.count);
        std::printf("derived %d %d %lld %d %zu\n", b.chunk, b.tile, (long long)b.mp, b.km_tiles, b.data_bytes);
      }
      for (int32_t a : P.adam) std::printf("adam %d\n", a);
      std::printf("derived layout %zu %zu %zu %zu %zu %zu\n", P.lay.off_desc, P.lay.off_adesc, P.lay.off_aux,
                  P.lay.off_part, P.lay.off_data, P.lay.total);
    }
    std::printf("end\n");
  }
  return 0;
}
