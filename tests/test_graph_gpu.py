"""The MuonH step inside a captured HIP graph.

The step allocates nothing, synchronises nothing and records no memset
(its tail-balancing counters and its non-finite status word are cleared by
a kernel), so a caller can capture it. The graph is replayed several times, with eager work and
synchronisations between the replays, and every replay must leave W and M
bit for bit where the same number of eager steps leaves them (the kernels
are deterministic, and each replay runs the same launches on the same
buffers).
"""
from __future__ import annotations

import sys

import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shapes", [
    # small: fixed tile deal
    [(256, 512), (512, 256), (300, 200)],
    # 192 small matrices: every GEMM launch uses the run-time tail claims
    [(512, 512)] * 96 + [(768, 512)] * 96,
])
def test_step_replays_in_a_hip_graph(shapes):
    need_gpu()
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    W0 = [torch.from_numpy(workloads.host_custom(s, 0.02, (71, i))).to(dev) for i, s in enumerate(shapes)]
    G = [torch.from_numpy(workloads.host_custom(s, 0.01, (72, i))).to(dev) for i, s in enumerate(shapes)]
    lr, beta, k, replays = 0.02, 0.95, 5, 4

    # eager: 1 + replays steps, state kept after each
    opt_e = mh.MuonH(shapes)
    W_e = [w.clone() for w in W0]
    M_e = [torch.zeros_like(w) for w in W0]
    opt_e.init(W_e)
    states = []
    for _ in range(1 + replays):
        opt_e.step(W_e, G, M_e, lr, beta, k)
        torch.cuda.synchronize()
        states.append(([w.clone() for w in W_e], [m.clone() for m in M_e]))

    # graph: one eager step (builds the pointer tables), then capture one step
    opt_g = mh.MuonH(shapes)
    W_g = [w.clone() for w in W0]
    M_g = [torch.zeros_like(w) for w in W0]
    opt_g.init(W_g)
    opt_g.step(W_g, G, M_g, lr, beta, k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        opt_g.step(W_g, G, M_g, lr, beta, k)
    torch.cuda.synchronize()
    for r in range(replays):
        graph.replay()
        torch.cuda.synchronize()
        # eager work between replays (its own launches and a reduction)
        scratch = torch.randn(1 << 20, device=dev)
        float(scratch.sum())
        torch.cuda.synchronize()
        W_ref, M_ref = states[1 + r]
        for i in range(len(shapes)):
            assert torch.equal(W_g[i], W_ref[i]), f"replay {r}: W of matrix {i}"
            assert torch.equal(M_g[i], M_ref[i]), f"replay {r}: M of matrix {i}"
        say(f"[graph] replay {r} equals eager step {2 + r}")
    # the status word is cleared by a kernel inside the graph: finite replays report 0
    assert opt_g.status() == 0
