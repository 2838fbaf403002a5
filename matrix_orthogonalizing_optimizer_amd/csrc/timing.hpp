// Optional per-launch HIP-event timing of the library's kernels (for the
// benchmark's live per-kernel figures).  Off by default; no cost when off.
#pragma once

#include <hip/hip_runtime.h>

namespace muon {

enum Family : int {
  F_MOMENTUM = 0,
  F_NORM,
  F_SYRK,      // A = X X^T (standard)
  F_POLY,      // P = a I + b A + c A A
  F_UPDATE,    // X' = P X (= a X + B X)
  F_FINAL,     // last X' = P X fused with the parameter update
  F_GRAM_R0,   // R = X0 X0^T (Gram)
  F_GRAM_P,    // P = a I + b R + c R R
  F_GRAM_Q,    // Q <- P Q
  F_GRAM_T,    // T = P R
  F_GRAM_R,    // R <- T P
  F_ADAMW,
  F_COUNT
};

bool timing_on();
hipEvent_t timing_event();  // from a reusable pool
void timing_record(int fam, hipEvent_t e0, hipEvent_t e1, double flops, double bytes);

template <class F>
hipError_t timed(int fam, double flops, double bytes, hipStream_t s, F&& launch) {
  if (!timing_on()) return launch();
  hipEvent_t e0 = timing_event(), e1 = timing_event();
  if (!e0 || !e1) return launch();
  hipError_t r = hipEventRecord(e0, s);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(e1, s);
  if (r != hipSuccess) return r;
  timing_record(fam, e0, e1, flops, bytes);
  return hipSuccess;
}

}  // namespace muon
