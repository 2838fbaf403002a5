"""ns_orthogonalize_noalloc (the entry point that allocates nothing; its
scratch memory is a device array inside the library) called through the
C ABI, against ns_orthogonalize with a caller workspace on the same inputs:
two calls in a row, the second with a smaller matrix, must both match.  The
two entry points run the same kernels, so the results are compared bit for
bit (stricter than the 2e-2 / 1e-4 bars, which they also meet against the
reference).  Sizes above the array are rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import cref
from tests.gpu_util import dev, f64, rel
from workloads import gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu


def _noalloc(X, steps=5, method=0):
    """Direct C-ABI call (no binding helper in between)."""
    L = mo.lib()
    rows, cols = X.shape
    dt = 0 if X.dtype == torch.float32 else 1
    st = L.ns_orthogonalize_noalloc(ctypes.c_void_p(X.data_ptr()), rows, cols, X.stride(0), dt, steps,
                                    None, method, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_point(dtype):
    d = dev()
    for shape, method in (((1024, 3000), 0), ((300, 700), 0), ((2048, 512), 1), ((768, 1536), 3)):
        print(f"ns_orthogonalize_noalloc {shape} {dtype} method {method}", flush=True)
        G = gen.lowrank_gradient(*shape, 8, shape[0] + shape[1], "cpu", torch.float64).to(dtype)
        a = G.to(d).contiguous()
        b = G.to(d).contiguous()
        mo.ns_orthogonalize(a, method=method)
        assert _noalloc(b, method=method) == 0
        torch.cuda.synchronize()
        assert torch.equal(a, b), shape
        tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
        if shape[0] * shape[1] <= 300 * 700:
            assert rel(f64(b), cref.orthogonalize(f64(G))) <= tol


def test_noalloc_rejects_what_does_not_fit():
    d = dev()
    X = torch.zeros(4096, 4096, dtype=torch.bfloat16, device=d)
    assert mo.ns_orthogonalize_workspace_bytes(4096, 4096, 1) > mo._lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(X) == -5  # MUON_E_WORKSPACE, nothing launched
    small = torch.zeros(0, 16, dtype=torch.bfloat16, device=d)
    assert _noalloc(small) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(X).item() == 0
