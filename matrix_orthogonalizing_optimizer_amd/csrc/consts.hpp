// Tiling constants shared by the host planner and the kernels.
#pragma once

namespace muon {
constexpr int KM_TR = 64;       // momentum kernel tile rows (parameter layout)
constexpr int KM_TC = 256;      // momentum kernel tile columns
constexpr int KMR_TR = 4;       // momentum kernel tile rows, tall units (row-contiguous tiles)
constexpr int KMR_TC = 512;     // momentum kernel tile columns, tall units
constexpr int ADAM_EPB = 4096;  // AdamW elements per workgroup
}  // namespace muon
