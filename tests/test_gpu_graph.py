"""The library's calls only enqueue work (no allocation, no host wait, no
memset nodes), so they can be captured into a HIP graph.  A captured
muon_step and a captured ns_orthogonalize_noalloc are replayed three times,
with the state reset eagerly and the device synchronized between replays;
every replay must equal the eager call bit for bit."""
import pytest
import torch

from tests.gpu_util import StepRunner, dev, hp_from
from workloads import configs, gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("method", [0, 3])
def test_muon_step_graph_replays_match_eager(method):
    """Standard method, and the restarted Gram chain (its restart is host
    orchestration of the same kernels)."""
    print(f"muon_step under graph capture, method {method}", flush=True)
    d = dev()
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 1536, 512, 0, 0), (0, 1, 768, 768, 256, 0),
             (0, 0, 300, 701, 0, 0), (1, 1, 1, 1001, 0, 0), (1, 1, 64, 256, 0, 0)]
    wl = configs.Workload("graph", table, [f"p{i}" for i in range(len(table))], rank=8, hp=configs._hp())
    P0, M0, EA0, ES0 = gen.make_state(wl, "cpu")
    G = [g.to(d) for g in gen.make_grads(wl, 0, "cpu")]
    to = lambda xs: [None if x is None else x.to(d) for x in xs]
    run = StepRunner(table, method=method, device=d)
    hp = hp_from(wl.hp)
    # eager
    P, M, EA, ES = to(P0), to(M0), to(EA0), to(ES0)
    run.step(P, G, M, EA, ES, hp)
    torch.cuda.synchronize()
    eager = [x.clone() for x in P + M + EA + ES if x is not None]
    # captured on torch's capture stream
    Ps, Ms, EAs, ESs = to(P0), to(M0), to(EA0), to(ES0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step(Ps, G, Ms, EAs, ESs, hp)
    state = [x for x in Ps + Ms + EAs + ESs if x is not None]
    init = [x for x in to(P0) + to(M0) + to(EA0) + to(ES0) if x is not None]
    for replay in range(3):
        for s, i in zip(state, init):
            s.copy_(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s, e in zip(state, eager):
            assert torch.equal(s, e), replay


def test_noalloc_graph_replays_match_eager():
    print("ns_orthogonalize_noalloc under graph capture", flush=True)
    d = dev()
    G0 = gen.lowrank_gradient(1024, 3000, 8, 5, "cpu", torch.float64).to(torch.bfloat16).to(d)
    a = G0.clone()
    mo.ns_orthogonalize_noalloc(a)   # eager (also takes the scratch array's address)
    torch.cuda.synchronize()
    X = G0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mo.ns_orthogonalize_noalloc(X)
    for replay in range(3):
        X.copy_(G0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(X, a), replay
