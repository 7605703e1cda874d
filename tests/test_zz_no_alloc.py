"""muonh_step_noalloc, the step for callers that cannot allocate device
memory, against muonh_step with a caller workspace.

Both run the same kernels on the same inputs, so W and M must come out equal
bit for bit. The entry point is called through the C ABI (the binding's
pointer arrays, R and stream) two times in a row with different plans, the
second one smaller: the fixed per-GPU array keeps the first call's contents,
and the second must not depend on them.
"""
from __future__ import annotations

import pytest

import workloads
from parity_bar import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# first call: plans close to the array's size (82.5 MiB of bf16 operands,
# 118.8 MiB of fp32 ones); second call: a smaller plan
BIG = {"bf16": [(2048, 2048), (2048, 2048), (1000, 3000), (129, 2052)],
       "fp32": [(2048, 2048), (700, 3000), (129, 2052)]}
SMALL = [(300, 200), (200, 300), (64, 96)]


def _noalloc(mh, opt, W, G, M, lr, beta, k):
    lib = mh.get_lib()
    return lib.muonh_step_noalloc(opt.plan.handle, opt._ptr_array("W", W), opt._ptr_array("G", G),
                                  opt._ptr_array("M", M), opt._R_plan.data_ptr(), lr, beta, k,
                                  opt._stream())


def _compare(shapes, prec, key, steps=2):
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    opt = mh.MuonH(shapes, precision=prec)
    assert opt.plan.workspace_bytes <= mh.MUONH_NOALLOC_WORKSPACE_BYTES
    W0 = [torch.from_numpy(workloads.host_custom(s, 0.02, (key, 0, i))).to(dev)
          for i, s in enumerate(shapes)]
    W_a = [w.clone() for w in W0]
    W_b = [w.clone() for w in W0]
    M_a = [torch.zeros(s, device=dev) for s in shapes]
    M_b = [torch.zeros(s, device=dev) for s in shapes]
    opt.init(W_a)
    for st in range(steps):
        G = [torch.from_numpy(workloads.host_custom(s, 0.01, (key, st + 1, i))).to(dev)
             for i, s in enumerate(shapes)]
        opt.step(W_a, G, M_a, 0.02, 0.95, 5)
        mh.check(_noalloc(mh, opt, W_b, G, M_b, 0.02, 0.95, 5))
        torch.cuda.synchronize()
        say(f"[noalloc {prec} {len(shapes)} matrices] step {st}")
    for i in range(len(shapes)):
        assert torch.equal(W_a[i], W_b[i]), f"W[{i}]"
        assert torch.equal(M_a[i], M_b[i]), f"M[{i}]"


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_noalloc_step_matches_the_workspace_step(prec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _compare(BIG[prec], prec, 110)   # first call: close to the array's size
    _compare(SMALL, prec, 111)       # second call: smaller, on the first call's leftovers
