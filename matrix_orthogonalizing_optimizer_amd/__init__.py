"""libmuon for AMD Instinct MI355X: the Muon optimizer step as hand-written
HIP kernels behind a C ABI (include/libmuon.h), with a thin ctypes binding
of the same names."""
from ._lib import (EXPORTED, MUON_BF16, MUON_F32, MUON_KIND_ADAMW, MUON_KIND_MUON,  # noqa: F401
                   MUON_NS_GRAM, MUON_NS_STANDARD, MuonError, Plan, lib, make_hparams,
                   muon_plan_buckets, muon_plan_create, muon_plan_units, muon_plan_workspace_bytes,
                   muon_status_string, muon_step, muon_timing_collect, muon_timing_enable,
                   muon_version, ns_orthogonalize, ns_orthogonalize_workspace_bytes)
