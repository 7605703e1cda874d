"""The non-finite report of a step (muonh_step_status).

Non-finite inputs are not errors: they propagate into the matrix they are
in, and the step records whether a momentum norm ||M|| or a trial update
norm ||W - lr*O|| was NaN or infinite. The record is cleared at the start
of every step. A non-finite matrix must not leak into the other matrices
of the same batched launches: those come out bit for bit as in a step
without it.
"""
from __future__ import annotations

import sys

import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(256, 512), (512, 256), (300, 200), (512, 512)]


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _state(prec, seed=80):
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    opt = mh.MuonH(SHAPES, precision=prec)
    W = [torch.from_numpy(workloads.host_custom(s, 0.02, (seed, i))).to(dev) for i, s in enumerate(SHAPES)]
    G = [torch.from_numpy(workloads.host_custom(s, 0.01, (seed + 1, i))).to(dev) for i, s in enumerate(SHAPES)]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in SHAPES]
    R = opt.init(W)
    return opt, W, G, M, R


def test_init_clears_the_record():
    need_gpu()
    import orthogonalized_updates_amd as mh
    opt = mh.MuonH(SHAPES)
    opt.workspace.fill_(255)  # a workspace full of stale bytes
    W = [torch.from_numpy(workloads.host_custom(s, 0.02, (80, i))).cuda() for i, s in enumerate(SHAPES)]
    opt.init(W)
    assert opt.status() == 0
    say("[status] init clears the record")


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_finite_step_reports_nothing(prec):
    need_gpu()
    opt, W, G, M, _ = _state(prec)
    opt.step(W, G, M, 0.02, 0.95, 5)
    assert opt.status() == 0
    say(f"[status] {prec}: finite step -> 0")


@pytest.mark.parametrize("prec,k", [("bf16", 5), ("fp32", 5), ("bf16", 0)])
def test_nan_gradient_sets_both_bits_and_stays_in_its_matrix(prec, k):
    import orthogonalized_updates_amd as mh
    need_gpu()
    opt, W, G, M, _ = _state(prec)
    ref_opt, W_ref, G_ref, M_ref, _ = _state(prec)
    G[1][7, 3] = float("nan")
    opt.step(W, G, M, 0.02, 0.95, k)
    ref_opt.step(W_ref, G_ref, M_ref, 0.02, 0.95, k)
    st = opt.status()
    assert st == mh.MUONH_NONFINITE_MOMENTUM | mh.MUONH_NONFINITE_UPDATE
    assert ref_opt.status() == 0
    assert torch.isnan(W[1]).all()
    for i in (0, 2, 3):
        assert torch.equal(W[i], W_ref[i]), f"matrix {i} changed by the NaN in matrix 1"
        assert torch.equal(M[i], M_ref[i])
    say(f"[status] {prec} k={k}: NaN gradient -> {st}, other matrices bit-exact")


def test_infinite_weight_sets_the_update_bit_only():
    import orthogonalized_updates_amd as mh
    need_gpu()
    opt, W, G, M, _ = _state("bf16")
    W[2][0, 0] = float("inf")  # after init: R stays finite, the trial update is not
    opt.step(W, G, M, 0.02, 0.95, 5)
    st = opt.status()
    assert st == mh.MUONH_NONFINITE_UPDATE
    assert torch.isfinite(M[2]).all()
    say(f"[status] infinite weight -> {st}")


def test_record_is_cleared_by_the_next_step():
    need_gpu()
    opt, W, G, M, _ = _state("bf16")
    G[0][0, 0] = float("inf")
    opt.step(W, G, M, 0.02, 0.95, 5)
    assert opt.status() != 0
    # same plan and workspace, fresh finite tensors
    _, W2, G2, M2, _ = _state("bf16", seed=90)
    opt.init(W2)
    opt.step(W2, G2, M2, 0.02, 0.95, 5)
    assert opt.status() == 0
    say("[status] record cleared by the next step")


def test_muon_wd_sets_the_momentum_bit_only():
    import orthogonalized_updates_amd as mh
    need_gpu()
    opt, W, G, M, _ = _state("bf16")
    G[3][100, 100] = float("nan")
    opt.step_muon_wd(W, G, M, 0.02, 0.95, 0.1, 5)
    st = opt.status()
    assert st == mh.MUONH_NONFINITE_MOMENTUM
    say(f"[status] muon_wd NaN gradient -> {st}")
