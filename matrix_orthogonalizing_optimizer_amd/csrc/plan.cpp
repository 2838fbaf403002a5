// Host-only planner of libmuon (no HIP calls).
//
// A Muon parameter becomes one unit, or one unit per row block when
// split_rows > 0 (the MindSpeed "Muon 优化器" document splits a fused QKV
// weight into its Q/K/V sub-matrices and orthogonalizes each; the DeepSpeed
// page names per-attention-head "Muon Split").  Units of equal
// (m, n, tall, param dtype, compute dtype, method) share a bucket, numbered
// by first appearance, and are processed together by grouped launches.
#include "plan.hpp"

#include <algorithm>
#include <cmath>

#include "consts.hpp"

namespace muon {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int32_t elem_size(int32_t cdtype) { return cdtype == MUON_F32 ? 4 : 2; }

static size_t align_ws(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

// The Gram chain in fp16 (R scaled by a power of two) stays within the bf16
// tolerance on the workload gradients only for m >= 512 and n >= 3m: closer
// to square, or smaller, the normalized noise spectrum reaches down to where
// the quintic amplifies the chain's rounding (emulated: 5.3e-2 at 512 x 860,
// 5.8e-2 at 768 x 768, 3.5e-2 at 256 x 512; at most 1.25e-2 inside the
// region).  MUON_NS_AUTO picks Gram exactly there (where it also does less
// work than the standard method, n/m > 5/3).  An explicit Gram request
// outside the region is served in a precision that meets the tolerance: a
// 16-bit compute dtype runs the Gram chain in fp32 (~1e-4, far inside the
// bf16 tolerance); an fp32 one runs the standard iteration, since the fp32
// Gram chain loses ~50x against it there (1.1-1.8e-4 measured on 768 x 768,
// 512 x 860 and 96 x 300, above the fp32 tolerance of 1e-4).
bool gram_fp16_ok(int64_t m, int64_t n) { return m >= 512 && n >= 3 * m; }

// The restarted chain (MUON_NS_GRAM_RESTART) serves the 16-bit compute dtype
// for m >= 256: one restart after ceil(steps / 2) steps keeps the fp16 chain
// within the bf16 tolerance there (emulated at most 0.92e-2 from 256 x 256
// to 2048 x 2048, ranks 8 and 64; the emulation matched the kernels to a few
// percent where both were measured).  Below, rank-64 gradients reach
// 1.2-2.7e-2 (128 x 128 to 160 x 160), too close to 2e-2 or past it, so
// such a unit is resolved as a plain Gram request (the fp32 chain), as is
// any fp32 request.
constexpr int64_t kRestartMinM = 256;

int32_t resolve_method(int32_t method, int32_t cdtype, int64_t m, int64_t n) {
  if (method == MUON_NS_AUTO) return gram_fp16_ok(m, n) ? MUON_NS_GRAM : MUON_NS_STANDARD;
  if (method == MUON_NS_GRAM_RESTART && (cdtype == MUON_F32 || m < kRestartMinM)) method = MUON_NS_GRAM;
  if (method == MUON_NS_GRAM && cdtype == MUON_F32 && !gram_fp16_ok(m, n)) return MUON_NS_STANDARD;
  return method;
}

bool valid_method(int32_t method) {
  return method == MUON_NS_STANDARD || method == MUON_NS_GRAM || method == MUON_NS_AUTO ||
         method == MUON_NS_GRAM_RESTART;
}

int32_t restart_after(int32_t method, int32_t steps) {
  return method == MUON_NS_GRAM_RESTART && steps >= 2 ? (steps + 1) / 2 : 0;
}

int32_t resolve_cdtype(int32_t cdtype, int32_t method, int64_t m, int64_t n) {
  if (method == MUON_NS_GRAM && cdtype == MUON_BF16 && !gram_fp16_ok(m, n)) return MUON_F32;
  return cdtype;
}

bool bucket_addressable(const PlanBucket& b) {
  // every GEMM operand of one unit is addressed with 32-bit byte offsets
  const uint64_t es = (uint64_t)elem_size(b.cdtype);
  return (uint64_t)b.n * (uint64_t)b.mp * es < (uint64_t(1) << 31);
}

// Per unit: Y = X^T (n x mp), the transposed copy of the unit kept through the
// iteration (the symmetric products read it K-major); standard method: Y0,
// Y1, A, P; Gram: Y0, R, T and three P / Z buffers (m x mp each, fp16 for a
// bf16 bucket); the restarted chain also Yr, the restart's iterate (n x mp).
size_t per_unit_data_bytes(const PlanBucket& b) {
  const size_t es = (size_t)elem_size(b.cdtype);
  const size_t yb = (size_t)b.n * (size_t)b.mp * es;
  const size_t sb = (size_t)b.m * (size_t)b.mp * es;
  if (b.method == MUON_NS_GRAM) return yb + 5 * sb;
  if (b.method == MUON_NS_GRAM_RESTART) return 2 * yb + 5 * sb;
  return 2 * yb + 2 * sb;
}

void bucket_derive(PlanBucket& b, size_t chunk_cap_bytes) {
  b.mp = round_up(b.m, 8);
  b.tile = b.m <= 192 ? 128 : 256;
  // momentum kernel tiles over the unit in parameter layout
  const int64_t prow = b.tall ? b.n : b.m, pcol = b.tall ? b.m : b.n;
  const int64_t ktr = b.tall ? KMR_TR : KM_TR, ktc = b.tall ? KMR_TC : KM_TC;
  b.km_tiles = (int32_t)(((prow + ktr - 1) / ktr) * ((pcol + ktc - 1) / ktc));
  const size_t per = per_unit_data_bytes(b);
  int64_t chunk = (int64_t)(chunk_cap_bytes / std::max<size_t>(per, 1));
  chunk = std::max<int64_t>(1, std::min<int64_t>(chunk, b.count));
  b.chunk = (int32_t)chunk;
  const size_t es = (size_t)elem_size(b.cdtype);
  const size_t yb = align_ws((size_t)chunk * b.n * b.mp * es);
  const size_t sb = align_ws((size_t)chunk * b.m * b.mp * es);
  size_t o = 0;
  for (int i = 0; i < 8; ++i) b.off[i] = 0;
  b.off[0] = o; o += yb;
  if (b.method == MUON_NS_GRAM || b.method == MUON_NS_GRAM_RESTART) {
    for (int i = 1; i < 6; ++i) { b.off[i] = o; o += sb; }
    if (b.method == MUON_NS_GRAM_RESTART) { b.off[6] = o; o += yb; }
  } else {
    b.off[1] = o; o += yb;
    b.off[2] = o; o += sb;
    b.off[3] = o; o += sb;
  }
  b.data_bytes = o;
}

muon_status build_plan(const muon_param_shape* table, int32_t n, const muon_plan_options* opts,
                       PlanImpl& P) {
  if (n < 0 || (n > 0 && !table)) return MUON_E_ARG;
  muon_plan_options o{MUON_NS_STANDARD, -1};
  if (opts) o = *opts;
  if (!valid_method(o.ns_method)) return MUON_E_METHOD;
  if (o.ns_dtype != -1 && o.ns_dtype != MUON_F32 && o.ns_dtype != MUON_BF16) return MUON_E_DTYPE;
  P.table.assign(table, table + n);
  P.opts = o;
  const int64_t kMaxDim = (int64_t)1 << 30;

  std::vector<PlanUnit> order;  // table order
  for (int32_t p = 0; p < n; ++p) {
    const muon_param_shape& s = table[p];
    if (s.kind != MUON_KIND_MUON && s.kind != MUON_KIND_ADAMW) return MUON_E_ARG;
    if (s.dtype != MUON_F32 && s.dtype != MUON_BF16) return MUON_E_DTYPE;
    if (s.rows < 0 || s.cols < 0 || s.split_rows < 0 || s.scale_dim < 0) return MUON_E_SHAPE;
    if (s.rows > kMaxDim || s.cols > kMaxDim) return MUON_E_SHAPE;
    if (s.kind == MUON_KIND_ADAMW) {
      if (s.split_rows != 0) return MUON_E_SHAPE;
      P.adam.push_back(p);
      continue;
    }
    if (s.split_rows > 0 && s.rows % s.split_rows != 0) return MUON_E_SHAPE;
    if (s.rows == 0 || s.cols == 0) continue;
    const int64_t h = s.split_rows > 0 ? s.split_rows : s.rows;
    for (int64_t r = 0; r < s.rows; r += h) {
      PlanUnit u;
      u.param = p;
      u.row0 = r;
      u.rows = h;
      u.cols = s.cols;
      u.tall = h > s.cols ? 1 : 0;
      u.scale_dim = s.scale_dim > 0 ? s.scale_dim : std::max(h, s.cols);
      order.push_back(u);
    }
  }

  // buckets by first appearance
  std::vector<std::vector<int32_t>> members;
  for (size_t i = 0; i < order.size(); ++i) {
    const PlanUnit& u = order[i];
    const int32_t m = (int32_t)std::min(u.rows, u.cols), nn = (int32_t)std::max(u.rows, u.cols);
    const int32_t pdt = P.table[u.param].dtype;
    const int32_t req = o.ns_dtype < 0 ? pdt : o.ns_dtype;
    const int32_t meth = resolve_method(o.ns_method, req, m, nn);
    const int32_t cdt = resolve_cdtype(req, meth, m, nn);
    size_t bi = 0;
    for (; bi < P.buckets.size(); ++bi) {
      const PlanBucket& b = P.buckets[bi];
      if (b.m == m && b.n == nn && b.tall == u.tall && b.pdtype == pdt && b.cdtype == cdt && b.method == meth)
        break;
    }
    if (bi == P.buckets.size()) {
      PlanBucket b{};
      b.m = m;
      b.n = nn;
      b.tall = u.tall;
      b.pdtype = pdt;
      b.cdtype = cdt;
      b.method = meth;
      P.buckets.push_back(b);
      members.emplace_back();
    }
    members[bi].push_back((int32_t)i);
  }
  P.units.clear();
  for (size_t bi = 0; bi < P.buckets.size(); ++bi) {
    PlanBucket& b = P.buckets[bi];
    b.first = (int32_t)P.units.size();
    b.count = (int32_t)members[bi].size();
    for (int32_t i : members[bi]) P.units.push_back(order[i]);
    bucket_derive(b, CHUNK_CAP_BYTES);
    if (!bucket_addressable(b)) return MUON_E_SHAPE;
    P.max_chunk = std::max(P.max_chunk, b.chunk);
    P.max_partials = std::max<int64_t>(P.max_partials, (int64_t)b.chunk * b.km_tiles);
    P.max_data = std::max(P.max_data, b.data_bytes);
  }

  Layout& L = P.lay;
  size_t off = 0;
  L.off_desc = off;
  off = align_ws(off + P.units.size() * 48);
  L.off_adesc = off;
  off = align_ws(off + P.adam.size() * 64);
  L.off_aux = off;
  off = align_ws(off + (size_t)P.max_chunk * 16);
  L.off_part = off;
  off = align_ws(off + (size_t)P.max_partials * 4);
  L.off_data = off;
  off += P.max_data;
  L.total = off == 0 ? 0 : off + WS_ALIGN;  // slack to align the caller's base
  return MUON_OK;
}

}  // namespace muon
