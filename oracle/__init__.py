"""fp64 CPU reference of the Muon optimizer step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the product path.
"""
from .muon_ref import *  # noqa: F401,F403
from .muon_ref import (QUINTIC, DEFAULT_STEPS, RMS_SCALE, OracleHparams, OracleUnit,  # noqa: F401
                       momentum_update, frobenius_normalize, ns_standard, ns_gram,
                       orthogonalize, quintic_scalar, muon_scale, weight_update,
                       adamw_update, plan_units, plan_buckets, muon_step, coeff_schedule,
                       hybrid_schedule, REFINED)
