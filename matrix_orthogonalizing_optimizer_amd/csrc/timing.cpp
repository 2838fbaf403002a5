// Per-launch HIP-event timing (see timing.hpp and muon_timing_* in libmuon.h).
#include "timing.hpp"

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "libmuon.h"

namespace muon {

namespace {

const char* kNames[F_COUNT] = {"momentum_norm", "norm_finalize", "ns_gram_A", "ns_poly_P",
                               "ns_update_PX", "ns_final_update", "gram_r0", "gram_p",
                               "gram_q", "gram_t", "gram_r", "adamw"};

struct Rec {
  int fam;
  hipEvent_t e0, e1;
  double flops, bytes;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

}  // namespace

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

hipEvent_t timing_event() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence when the event completes, so recording
  // it does not write back and invalidate the caches between the kernels it
  // brackets (the default fence cost ~0.2 ms per momentum launch and slowed
  // the work that followed)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

void timing_record(int fam, hipEvent_t e0, hipEvent_t e1, double flops, double bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{fam, e0, e1, flops, bytes});
}

}  // namespace muon

using namespace muon;

extern "C" {

muon_status muon_timing_enable(int32_t enable) {
  g_on.store(enable != 0);
  return MUON_OK;
}

muon_status muon_timing_collect(muon_kernel_timing* out, int32_t cap, int32_t* n) {
  if (!n || cap < 0 || (cap > 0 && !out)) return MUON_E_ARG;
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_recs);
  }
  muon_kernel_timing acc[F_COUNT];
  std::memset(acc, 0, sizeof(acc));
  muon_status st = MUON_OK;
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
      st = MUON_E_HIP;
    acc[r.fam].launches += 1;
    acc[r.fam].total_ms += ms;
    acc[r.fam].flops += r.flops;
    acc[r.fam].bytes += r.bytes;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Rec& r : recs) {
      g_pool.push_back(r.e0);
      g_pool.push_back(r.e1);
    }
  }
  int32_t k = 0;
  for (int f = 0; f < F_COUNT; ++f) {
    if (acc[f].launches == 0) continue;
    if (k < cap) {
      out[k] = acc[f];
      std::strncpy(out[k].name, kNames[f], sizeof(out[k].name) - 1);
      out[k].name[sizeof(out[k].name) - 1] = 0;
    }
    ++k;
  }
  *n = k;
  return st;
}

}  // extern "C"
