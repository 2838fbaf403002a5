// Host-only planner: shape table -> units -> buckets -> workspace layout.
// No HIP calls; usable without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "libmuon.h"

namespace muon {

struct PlanUnit {
  int32_t param;
  int64_t row0, rows, cols;  // block of the parameter (parameter layout)
  int32_t tall;              // rows > cols: processed as the transpose
  int64_t scale_dim;         // resolved: max(rows, cols) unless overridden
};

// A bucket is processed chunk by chunk; every chunk of `chunk` units shares
// one workspace data region laid out as below (offsets from the data base).
struct PlanBucket {
  int32_t m, n, tall, pdtype, cdtype, method;
  int32_t first, count;  // range in the bucket-ordered unit list
  int32_t chunk;         // units per chunk
  int32_t tile;          // GEMM tile edge (128 or 256)
  int64_t mp;            // leading dimension of every workspace matrix (round_up(m, 8))
  int32_t km_tiles;      // momentum-kernel workgroups per unit
  size_t off[8];         // data sub-buffers: standard Y0 Y1 A B; gram Y0 R T PZ0 PZ1 PZ2 (Yr)
  size_t data_bytes;     // per chunk
};

struct Layout {
  size_t off_desc = 0, off_adesc = 0, off_aux = 0, off_part = 0, off_data = 0, total = 0;
};

struct PlanImpl {
  std::vector<muon_param_shape> table;
  muon_plan_options opts{};
  std::vector<PlanUnit> units;  // bucket order
  std::vector<PlanBucket> buckets;
  std::vector<int32_t> adam;    // table indices of AdamW parameters
  int32_t max_chunk = 0;
  int64_t max_partials = 0;
  size_t max_data = 0;
  Layout lay;
};

// Sizes shared by the planner and ns_orthogonalize.
int64_t round_up(int64_t x, int64_t m);
int32_t elem_size(int32_t cdtype);
void bucket_derive(PlanBucket& b, size_t chunk_cap_bytes);
bool bucket_addressable(const PlanBucket& b);  // one unit's n x m operand < 2^31 bytes
bool gram_fp16_ok(int64_t m, int64_t n);  // the fp16 Gram chain meets the bf16 tolerance
// the method a unit runs (AUTO -> standard or Gram; an fp32 Gram request
// outside gram_fp16_ok -> standard), cdtype the requested compute dtype
int32_t resolve_method(int32_t method, int32_t cdtype, int64_t m, int64_t n);
// the compute dtype it runs in (a bf16 Gram unit outside gram_fp16_ok -> fp32)
int32_t resolve_cdtype(int32_t cdtype, int32_t method, int64_t m, int64_t n);
bool valid_method(int32_t method);  // a muon_ns_method value
// steps after which the restarted Gram chain restarts (0: no restart)
int32_t restart_after(int32_t method, int32_t steps);
size_t per_unit_data_bytes(const PlanBucket& b);

muon_status build_plan(const muon_param_shape* table, int32_t n, const muon_plan_options* opts,
                       PlanImpl& out);

constexpr size_t WS_ALIGN = 256;
// data bytes per chunk: large enough that a bucket of Llama-3-8B-sized
// units runs as one chunk (fewer launches, and the symmetric products' last
// partial round of 256 tiles is paid once per bucket)
constexpr size_t CHUNK_CAP_BYTES = size_t(24) << 30;
constexpr int32_t MAX_NS_STEPS = 64;

}  // namespace muon

struct muon_plan {
  muon::PlanImpl impl;
};
