"""GPU parity of ns_orthogonalize (the Newton-Schulz chain alone) against
the plain C++ fp64 reference (oracle/muon_ref.cpp), plus the bit-exact
symmetries of the HIP path.

Tolerances (relative Frobenius error against the reference): 2e-2 on the
bf16 path, 1e-4 on the fp32 path.  Inputs are the workload generator's
low-rank gradients (geometric spectrum 1..1e-3, 1e-3 noise), or
well-conditioned matrices for the shapes below 64 on a side, rounded once to
the storage dtype; the reference receives exactly those values."""
import numpy as np
import pytest
import torch

from oracle import cref
from tests.gpu_util import BLOCK_TOL_BF16, block_rel_max, dev, f64, rel
from workloads import gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _input(rows, cols, dtype, seed, rank=8):
    g = gen.lowrank_gradient(rows, cols, rank, seed, "cpu", torch.float64)
    return g.to(dtype)


def _run(G, method=0, steps=5, coeffs=None):
    X = G.to(dev()).contiguous()
    mo.ns_orthogonalize(X, steps=steps, coeffs=coeffs, method=method)
    torch.cuda.synchronize()
    return X


# several tiles plus ragged tails, tall and wide, the workload unit shapes
SHAPES = [(256, 512), (512, 256), (300, 700), (700, 300), (129, 1000), (768, 768), (128, 2048),
          (1408, 2048), (2048, 1408)]
# tiny and degenerate shapes (one 128 x 128 tile, mostly padding)
TINY = [(37, 50), (50, 37), (1, 64), (64, 1), (8, 8), (1, 1), (3, 200), (63, 63), (64, 200)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_standard_matches_oracle(shape, dtype):
    print(f"ns standard {shape} {dtype}", flush=True)
    G = _input(*shape, dtype, seed=shape[0] * 7919 + shape[1])
    O = f64(_run(G))
    ref = cref.orthogonalize(f64(G))
    assert rel(O, ref) <= TOL[dtype], rel(O, ref)
    if dtype == torch.bfloat16:
        assert block_rel_max(O, ref) <= BLOCK_TOL_BF16


@pytest.mark.parametrize("shape", [(384, 8192), (8200, 384)])
def test_kmajor_wave_count_threshold(shape):
    """A = X X^T is read K-major with K = n, the long side: two waves per
    SIMD up to K = 8192, one above.  Both sides of the threshold, tall and
    wide, bf16."""
    print(f"ns standard K-major threshold {shape}", flush=True)
    G = _input(*shape, torch.bfloat16, seed=shape[0] * 7919 + shape[1])
    O = f64(_run(G))
    ref = cref.orthogonalize(f64(G))
    assert rel(O, ref) <= TOL[torch.bfloat16], rel(O, ref)
    assert block_rel_max(O, ref) <= BLOCK_TOL_BF16


@pytest.mark.parametrize("shape", TINY)
def test_standard_tiny_fp32(shape):
    print(f"ns standard tiny fp32 {shape}", flush=True)
    G = _input(*shape, torch.float32, seed=shape[0] * 7919 + shape[1])
    O = f64(_run(G))
    ref = cref.orthogonalize(f64(G))
    assert rel(O, ref) <= 1e-4, rel(O, ref)


@pytest.mark.parametrize("shape", TINY)
def test_standard_tiny_bf16_well_conditioned(shape):
    """The bf16 path on shapes below 64 on a side, two Newton-Schulz steps
    (every kernel of the chain, both working copies of the iteration).  The
    workload generator is not used here: at these sizes it leaves normalized
    singular values below ~1.6e-3, where the quintic amplifies any rounding
    by up to a^5 ~ 485.  Singular values uniform in [0.3, 1] avoid that, but
    with normalized values near 1/sqrt(m) three or more steps pass through
    the band where the map expands errors, and a rounding emulation of bf16
    storage gives 1.3-3e-2 after five steps on some of these shapes: a
    property of the iteration in 16-bit arithmetic, not of the tiles.  After
    two steps the emulation stays below 1.3e-2."""
    print(f"ns standard tiny bf16 {shape}", flush=True)
    G = gen.conditioned_matrix(*shape, 0.3, 1.0, seed=shape[0] * 131 + shape[1]).to(torch.bfloat16)
    O = f64(_run(G, steps=2))
    ref = cref.orthogonalize(f64(G), steps=2)
    assert rel(O, ref) <= 2e-2, rel(O, ref)


# Gram variant.  Inside m >= 512, n >= 3m the chain runs in fp16 (R scaled by
# a power of two); every other Gram shape computes in fp32, so an explicit
# request for the Gram variant is held to the same tolerance everywhere.
GRAM_SHAPES = [(512, 1792), (1792, 512), (1024, 3584), (1000, 3500),       # fp16 chain
               (256, 1024), (300, 1100), (768, 768), (512, 860), (96, 300)]  # fp32
GRAM_WIDE_FP16 = [(768, 3072), (3072, 768)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", GRAM_SHAPES + GRAM_WIDE_FP16)
def test_gram_matches_oracle(shape, dtype):
    print(f"ns gram {shape} {dtype}", flush=True)
    for rank in (8, 64):
        G = _input(*shape, dtype, seed=shape[0] * 31 + shape[1] + rank, rank=rank)
        O = f64(_run(G, method=1))
        ref = cref.orthogonalize(f64(G), method="standard")
        assert rel(O, ref) <= TOL[dtype], (rank, rel(O, ref))


# Restarted Gram chain (an extension): fp16 for every 16-bit unit with
# m >= 256, small, square and ragged ones included, where the plain fp16
# chain misses the tolerance (emulated 1.9-17e-2); m < 256 takes the fp32
# Gram chain (255 x 300, 129 x 1000, 96 x 300, 64 x 200).  bf16 against the
# reference's restarted chain (equal to the standard result in fp64), with
# the per-block bound.
RESTART_SHAPES = [(256, 512), (512, 256), (256, 256), (300, 1100), (384, 384), (768, 768), (512, 860),
                  (1024, 1024), (1408, 2048), (768, 3072), (3072, 768),
                  (255, 300), (129, 1000), (96, 300), (64, 200)]


@pytest.mark.parametrize("shape", RESTART_SHAPES)
def test_gram_restart_matches_oracle(shape):
    print(f"ns gram restart {shape}", flush=True)
    for rank in (8, 64):
        G = _input(*shape, torch.bfloat16, seed=shape[0] * 37 + shape[1] + rank, rank=rank)
        O = f64(_run(G, method=mo.MUON_NS_GRAM_RESTART))
        ref = cref.orthogonalize(f64(G), method="gram_restart")
        e, eb = rel(O, ref), block_rel_max(O, ref)
        print(f"  rank {rank}: rel {e:.3e} block {eb:.3e}", flush=True)
        assert e <= TOL[torch.bfloat16] and eb <= BLOCK_TOL_BF16, (rank, e, eb)


@pytest.mark.parametrize("steps", [2, 3, 10])
def test_gram_restart_step_counts(steps):
    """The restart sits after ceil(steps / 2) steps: 2, 3 and 10 steps
    (the ten-step hybrid schedule) against the reference."""
    print(f"ns gram restart steps={steps}", flush=True)
    coeffs = mo.muon_ns_coefficients(mo.MUON_COEFF_HYBRID, steps) if steps == 10 else None
    G = _input(384, 1000, torch.bfloat16, seed=steps + 5)
    O = f64(_run(G, method=mo.MUON_NS_GRAM_RESTART, steps=steps, coeffs=coeffs))
    ref = cref.orthogonalize(f64(G), steps=steps, coeffs=coeffs, method="gram_restart")
    assert rel(O, ref) <= TOL[torch.bfloat16], rel(O, ref)


@pytest.mark.parametrize("shape", [(256, 1024), (768, 3072)])
def test_gram_restart_fp32_resolves_as_gram(shape):
    print(f"ns gram restart fp32 {shape}", flush=True)
    G = _input(*shape, torch.float32, seed=shape[0] + 1)
    O = f64(_run(G, method=mo.MUON_NS_GRAM_RESTART))
    ref = cref.orthogonalize(f64(G), method="standard")
    assert rel(O, ref) <= TOL[torch.float32], rel(O, ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_coefficient_schedule_and_steps(dtype):
    G = _input(200, 330, dtype, seed=5)
    sched = [(3.4445, -4.7750, 2.0315)] * 3 + [(1.5, -0.5, 0.0)] * 3
    O = f64(_run(G, steps=6, coeffs=sched))
    ref = cref.orthogonalize(f64(G), steps=6, coeffs=sched)
    assert rel(O, ref) <= TOL[dtype]
    O1 = f64(_run(G, steps=1))
    assert rel(O1, cref.orthogonalize(f64(G), steps=1)) <= TOL[dtype]


def test_zero_transpose_and_scaling_bit_exact():
    d = dev()
    Z = torch.zeros(64, 96, dtype=torch.bfloat16, device=d)
    mo.ns_orthogonalize(Z)
    assert torch.count_nonzero(Z).item() == 0
    G = _input(300, 700, torch.bfloat16, seed=11)
    a = _run(G)
    c = _run(G.t().contiguous())
    # implicit transposition of a tall matrix: the identical chain runs
    assert torch.equal(c, a.t())
    # power-of-two scaling leaves the result unchanged
    assert torch.equal(_run(G * 4), a)


def test_run_to_run_deterministic():
    G = _input(1000, 1500, torch.bfloat16, seed=13)
    a = _run(G)
    b = _run(G)
    assert torch.equal(a, b)


def test_strided_rows_in_place():
    d = dev()
    G = _input(96, 160, torch.float32, seed=17)
    big = torch.zeros(96, 200, dtype=torch.float32, device=d)
    big[:, :160] = G.to(d)
    view = big[:, :160]
    mo.ns_orthogonalize(view)
    torch.cuda.synchronize()
    assert rel(f64(view), cref.orthogonalize(f64(G))) <= 1e-4
    assert torch.count_nonzero(big[:, 160:]).item() == 0


def _ulp_bf16(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


@pytest.mark.parametrize("shape", [(300, 700), (256, 512), (1024, 1024)])
def test_sign_symmetry(shape):
    """NS(-G) = -NS(G).  With -G every product of the chain sees negated
    operands only in the update products (A = X X^T and P are identical).
    fp32 path: bit-exact after five steps (the fp32 matrix instruction
    accumulates sign-symmetrically).  bf16 path: after one step (one product
    of each kind) at most 1e-4 of the elements differ, each by at most one
    bf16 ulp of its value: the bf16 matrix instruction's accumulation is not
    sign-symmetric bit for bit (measured: 0 of 210000 and 131072, 8 of
    1048576 elements).  After five steps those single-ulp differences have
    been carried through four more steps like any rounding: the bound is
    1e-2 relative (measured 0.5-4.8e-3)."""
    print(f"ns sign symmetry {shape}", flush=True)
    G32 = _input(*shape, torch.float32, seed=11)
    assert torch.equal(_run(-G32), -_run(G32))
    G = G32.to(torch.bfloat16)
    a, b = f64(_run(G, steps=1)), f64(_run(-G, steps=1))
    diff = np.abs(a + b)
    assert np.count_nonzero(diff) <= 1e-4 * a.size, np.count_nonzero(diff)
    assert np.all(diff <= _ulp_bf16(a))
    a, b = f64(_run(G)), f64(_run(-G))
    assert rel(b, -a) <= 1e-2, rel(b, -a)


def _random_cases():
    """Seeded random shapes and methods: bf16 with min side >= 128 (the
    workload generator's inputs; smaller sides are covered above with
    well-conditioned inputs), fp32 from 1 to 700 on a side."""
    r = np.random.default_rng(20261203)
    cases = []
    for i in range(12):
        if i < 8:
            a, b = (int(round(float(np.exp(r.uniform(np.log(128), np.log(1100)))))) for _ in range(2))
            dtype = torch.bfloat16
        else:
            a, b = int(r.integers(1, 701)), int(r.integers(1, 701))
            dtype = torch.float32
        cases.append(((a, b), int(r.choice([0, 1, 3])), dtype))
    return cases


@pytest.mark.parametrize("shape,method,dtype", _random_cases())
def test_random_shapes_and_methods(shape, method, dtype):
    """Random ragged shapes (tall and wide) through every method, against the
    C++ reference's standard result (all methods agree with it in fp64)."""
    print(f"ns random {shape} method {method} {dtype}", flush=True)
    G = _input(*shape, dtype, seed=shape[0] * 7 + shape[1] + method)
    O = f64(_run(G, method=method))
    ref = cref.orthogonalize(f64(G), method="standard")
    e = rel(O, ref)
    assert e <= TOL[dtype], e
    if dtype == torch.bfloat16:
        assert block_rel_max(O, ref) <= BLOCK_TOL_BF16
