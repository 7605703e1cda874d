"""Robustness of the GPU path, checked bit for bit against itself:

* a workspace full of stale bytes (every byte 0xFF, which reads as NaN in
  bf16 and fp32) gives exactly the results of a zeroed one: the step never
  reads workspace memory it has not written in the same call (padding,
  norm partials, tail counters and the status word included);
* checkpoint and resume: a run restored from (W, M) and the radius R
  (set_radius, the canonical state: the digest page "Puro-2B trains for
  $6.9K, attention sinks hit 99%, LoopArena tops at 24.69%", section "The
  load-bearing tricks aren't in the abstract", fixes each matrix's norm at
  its value at initialization) into a new plan, workspace and freshly
  allocated tensors continues bit for bit like the run that never stopped.
"""
from __future__ import annotations

import pytest

import workloads
from parity_bar import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHAPES = [(300, 200), (200, 300), (257, 129), (64, 1), (512, 512), (129, 2052)]


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(shapes, key, steps, gdt=torch.float32):
    dev = torch.device("cuda")
    W = [torch.from_numpy(workloads.host_custom(s, 0.02, (key, 0, i))).to(dev)
         for i, s in enumerate(shapes)]
    G = [[torch.from_numpy(workloads.host_custom(s, 0.01, (key, st + 1, i))).to(dev).to(gdt)
          for i, s in enumerate(shapes)] for st in range(steps)]
    return W, G


@pytest.mark.parametrize("prec", ["bf16", "split_bf16", "fp32"])
@pytest.mark.parametrize("k", [0, 5])
def test_stale_workspace_gives_the_same_bits(prec, k):
    need_gpu()
    import orthogonalized_updates_amd as mh
    W0, G = _inputs(SHAPES, 80, 2)
    runs = []
    for fill in (0x00, 0xFF):
        opt = mh.MuonH(SHAPES, precision=prec)
        opt.workspace.fill_(fill)
        W = [w.clone() for w in W0]
        M = [torch.zeros(s, device="cuda") for s in SHAPES]
        opt.init(W)
        for st in range(2):
            opt.step(W, G[st], M, 0.02, 0.95, k)
        torch.cuda.synchronize()
        assert opt.status() == 0
        say(f"[stale workspace {prec} k={k}] fill 0x{fill:02x} done")
        runs.append(([w.cpu() for w in W], [m.cpu() for m in M],
                     [opt.read_update(i).cpu() for i in range(len(SHAPES))]))
    for name, a, b in zip(("W", "M", "O"), runs[0], runs[1]):
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"{name}[{i}] depends on the workspace's old contents"


def test_stale_workspace_muon_wd():
    need_gpu()
    import orthogonalized_updates_amd as mh
    W0, G = _inputs(SHAPES, 81, 2)
    runs = []
    for fill in (0x00, 0xFF):
        opt = mh.MuonH(SHAPES)
        opt.workspace.fill_(fill)
        W = [w.clone() for w in W0]
        M = [torch.zeros(s, device="cuda") for s in SHAPES]
        for st in range(2):
            opt.step_muon_wd(W, G[st], M, 0.02, 0.95, 0.1, 5)
        torch.cuda.synchronize()
        runs.append([w.cpu() for w in W] + [m.cpu() for m in M])
    for x, y in zip(*runs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("prec,mdt", [("bf16", "fp32"), ("bf16", "bf16"), ("fp32", "fp32")])
def test_checkpoint_resume_continues_bit_for_bit(prec, mdt):
    need_gpu()
    import orthogonalized_updates_amd as mh
    mtype = torch.bfloat16 if mdt == "bf16" else torch.float32
    steps, cut = 4, 2
    W0, G = _inputs(SHAPES, 82, steps)

    # the run that never stops
    opt = mh.MuonH(SHAPES, precision=prec, mom_dtype=mdt)
    W = [w.clone() for w in W0]
    M = [torch.zeros(s, dtype=mtype, device="cuda") for s in SHAPES]
    opt.init(W)
    for st in range(steps):
        opt.step(W, G[st], M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    ref = ([w.cpu() for w in W], [m.cpu() for m in M])

    # stop after `cut` steps, keep (W, M, R) on the host
    opt_a = mh.MuonH(SHAPES, precision=prec, mom_dtype=mdt)
    W = [w.clone() for w in W0]
    M = [torch.zeros(s, dtype=mtype, device="cuda") for s in SHAPES]
    R = opt_a.init(W)
    for st in range(cut):
        opt_a.step(W, G[st], M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    ckpt = {"W": [w.cpu().clone() for w in W], "M": [m.cpu().clone() for m in M],
            "R": R.cpu().clone()}
    del opt_a, W, M, R
    torch.cuda.empty_cache()

    # resume: new plan and workspace, new tensors, radius restored (not re-measured)
    opt_b = mh.MuonH(SHAPES, precision=prec, mom_dtype=mdt)
    W = [t.to("cuda") for t in ckpt["W"]]
    M = [t.to("cuda") for t in ckpt["M"]]
    opt_b.set_radius(ckpt["R"])
    for st in range(cut, steps):
        opt_b.step(W, G[st], M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        assert torch.equal(W[i].cpu(), ref[0][i]), f"W[{i}] after resume"
        assert torch.equal(M[i].cpu(), ref[1][i]), f"M[{i}] after resume"
