"""Host-side argument checks of the Python binding that need device
tensors: W, G and M must be disjoint (the step updates W and M in place and
reads G; the library's muonh_check_disjoint finds the overlap and the
binding names the caller's tensors), and a rejected call enqueues nothing."""
from __future__ import annotations

import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_overlapping_state_is_rejected_before_any_work():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    shapes = [(256, 512), (300, 200)]
    opt = mh.MuonH(shapes)
    W = [torch.from_numpy(workloads.host_custom(s, 0.02, (95, i))).to(dev) for i, s in enumerate(shapes)]
    G = [torch.from_numpy(workloads.host_custom(s, 0.01, (96, i))).to(dev) for i, s in enumerate(shapes)]
    M = [torch.zeros(s, device=dev) for s in shapes]
    opt.init(W)
    W0 = [w.clone() for w in W]
    with pytest.raises(ValueError, match="overlap"):
        opt.step(W, W, M, 0.02, 0.95, 5)  # G is W
    big = torch.zeros(256 * 512 + 300 * 200 + 8, device=dev)
    M_shared = [big[:256 * 512].view(256, 512), big[256 * 512 - 8:256 * 512 - 8 + 300 * 200].view(300, 200)]
    with pytest.raises(mh.MuonHAliasError, match=r"moms\[[01]\] overlaps moms\[[01]\]"):
        opt.step(W, G, M_shared, 0.02, 0.95, 5)
    with pytest.raises(ValueError, match="overlap"):
        opt.step_muon_wd(W, G, [W[0], M[1]], 0.02, 0.95, 0.1, 5)
    torch.cuda.synchronize()
    for w, w0 in zip(W, W0):
        assert torch.equal(w, w0)  # nothing ran
    opt.step(W, G, M, 0.02, 0.95, 5)  # disjoint tensors are accepted
    torch.cuda.synchronize()
    assert opt.status() == 0
