"""libmuon for AMD Instinct MI355X: the Muon optimizer step as hand-written
HIP kernels behind a C ABI (include/libmuon.h), with a thin ctypes binding
of the same names."""
from ._lib import (EXPORTED, MUON_BF16, MUON_COEFF_HYBRID, MUON_COEFF_QUINTIC,  # noqa: F401
                   MUON_F32, MUON_KIND_ADAMW, MUON_KIND_MUON, MUON_NS_AUTO, MUON_NS_GRAM, MUON_NS_GRAM_RESTART,
                   MUON_NS_STANDARD,
                   MUON_SCALE_MOONLIGHT, MUON_SCALE_SPECTRAL, MUON_SCALE_UNIT_RMS, MuonError, Plan,
                   lib, make_hparams, muon_ns_coefficients, muon_probe_copy, muon_probe_copy_lds, muon_probe_mfma,
                   muon_plan_buckets, muon_plan_create, muon_plan_units, muon_plan_workspace_bytes,
                   muon_status_string, muon_step, muon_timing_collect, muon_timing_enable,
                   muon_version, ns_orthogonalize, ns_orthogonalize_noalloc,
                   ns_orthogonalize_workspace_bytes)
