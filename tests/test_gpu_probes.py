"""GPU checks of the measurement aids the benchmark reports its kernels
against: both streaming copies (plain, and through the GEMMs' global -> LDS loads)
move every byte (a ragged length included) and
the register-only MFMA loop completes with the FLOP count the header states,
writing a finite value per workgroup."""
import pytest
import torch

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu


def test_probe_copy_moves_every_byte():
    print("muon_probe_copy 1 MiB + 48 B", flush=True)
    nbytes = (1 << 20) + 48
    g = torch.Generator(device="cuda:0").manual_seed(5)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda:0")
    mo.muon_probe_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0  # nothing past the end


def test_probe_mfma_runs():
    print("muon_probe_mfma 8 workgroups x 16 rounds", flush=True)
    sink = torch.full((8,), float("nan"), dtype=torch.float32, device="cuda:0")
    flops = mo.muon_probe_mfma(8, 16, sink)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 16 * 8 * 32768
    assert bool(torch.isfinite(sink).all())


def test_probe_copy_lds_moves_every_byte():
    print("muon_probe_copy_lds 1 MiB + 48 B", flush=True)
    nbytes = (1 << 20) + 48
    g = torch.Generator(device="cuda:0").manual_seed(6)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda:0")
    mo.muon_probe_copy_lds(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0  # nothing past the end
