"""GPU parity of the bf16 gradient / momentum storage (plan flags
MUONH_GRAD_BF16, MUONH_MOM_BF16) against the fp64 oracle.

Teacher-forced per step, as tests/test_parity_gpu.py, with the oracle's
bf16-state reading (oracle/bf16_state_oracle.py): a bf16 gradient is taken
as given; a bf16 momentum is the exact beta*M + G rounded once to bf16.
The kernel rounds the same exact value once, so
  * a bf16 momentum must equal the oracle's bit for bit (every element);
  * an fp32 momentum (with a bf16 gradient) within 1e-6 relative;
  * O, W and the sphere to the bars of tests/parity_bar.py (O: 2e-2 bf16,
    5e-4 split, 1e-5 fp32, whole matrix and every 256 x 256 tile of 4096
    entries or more, the oracle-order floor only for the listed tiny
    shapes; W: 2e-6 of the oracle's projection of the GPU's own O and the
    first-order bound of the full step; | ||W||/R - 1 | <= 1e-5).
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from parity_bar import assert_muon_wd, assert_muonh, muon_wd_errors, muonh_errors, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PRECS = ["fp32", "bf16", "split_bf16"]
COMBOS = [("bf16", "fp32"), ("fp32", "bf16"), ("bf16", "bf16")]
RAGGED = [(1, 1), (3, 5), (5, 3), (1, 64), (64, 1), (300, 200), (257, 129), (130, 700),
          (300, 200), (511, 513)]


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def host(t):
    """Exact host values of a device tensor (bf16 widens exactly to fp32)."""
    return t.float().cpu().numpy()


def dev_tensor(a, dtype, offset=0):
    """Device tensor of `a` in `dtype`; offset > 0 makes it a view `offset`
    elements into a larger buffer (not aligned for the vector path)."""
    shape = a.shape
    base = torch.zeros(a.size + offset, dtype=dtype, device="cuda")
    t = base[offset:].view(shape)
    t.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype))
    t._keep = base
    return t


def check_state_step(opt, W, M, G_vals, W_pre, M_pre, R, lr, beta, k, prec, mdt, indices, label,
                     wd=None):
    """The GPU step just taken against the oracle for matrices `indices`
    (MuonH, or Muon with decoupled decay when wd is given)."""
    bf_m = mdt == "bf16"
    for i in indices:
        o_gpu = opt.read_update(i).cpu().numpy()
        w_gpu = W[i].cpu().numpy()
        m_gpu = host(M[i])
        if wd is None:
            err = muonh_errors(o_gpu, w_gpu, m_gpu, G_vals[i], W_pre[i], M_pre[i], float(R[i]), lr,
                               beta, k, prec, mom_bf16=bf_m)
            assert_muonh(err, f"{label} mat {i}")
        else:
            err = muon_wd_errors(o_gpu, w_gpu, m_gpu, G_vals[i], W_pre[i], M_pre[i], lr, beta, wd, k,
                                 prec, mom_bf16=bf_m)
            assert_muon_wd(err, f"{label} mat {i}")


def run_state(shapes, *, steps, k, prec, gdt, mdt, wid, offset=0, wd=None, label=""):
    need_gpu()
    import orthogonalized_updates_amd as mh
    wl = workloads.Workload(wid=wid, name=label, shapes=tuple(shapes), steps=steps, ns_iters=(k,))
    opt = mh.MuonH(shapes, precision=prec, grad_dtype=gdt, mom_dtype=mdt)
    W = [dev_tensor(workloads.host_weight(wl, i), torch.float32, offset) for i in range(len(shapes))]
    M = [dev_tensor(np.zeros(s, np.float32), tdtype(mdt), offset) for s in shapes]
    say(f"[{label}] init")
    R = opt.init(W).cpu().numpy() if wd is None else None
    idx = list(range(len(shapes)))
    for step in range(steps):
        G = [dev_tensor(workloads.host_grad(wl, i, step), tdtype(gdt), offset)
             for i in range(len(shapes))]
        G_vals = {i: host(G[i]) for i in idx}
        W_pre = {i: W[i].cpu().numpy() for i in idx}
        M_pre = {i: host(M[i]) for i in idx}
        say(f"[{label}] step {step}")
        if wd is None:
            opt.step(W, G, M, wl.lr, wl.beta, k)
        else:
            opt.step_muon_wd(W, G, M, wl.lr, wl.beta, wd, k)
        torch.cuda.synchronize()
        check_state_step(opt, W, M, G_vals, W_pre, M_pre, R, wl.lr, wl.beta, k, prec, mdt, idx,
                         f"{label} step {step}", wd=wd)


@pytest.mark.parametrize("gdt,mdt", COMBOS)
@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("k", [0, 5])
def test_state_ragged_groups(gdt, mdt, prec, k):
    run_state(RAGGED, steps=3, k=k, prec=prec, gdt=gdt, mdt=mdt, wid=90,
              label=f"state G={gdt} M={mdt} {prec} k={k}")


@pytest.mark.parametrize("gdt,mdt", COMBOS)
@pytest.mark.parametrize("prec,k", [("bf16", 5), ("fp32", 5), ("bf16", 0)])
def test_state_misaligned_pointers(gdt, mdt, prec, k):
    # one element into each buffer: 2-byte (bf16) or 4-byte (fp32) offsets,
    # so every tensor takes the scalar path; bf16 operands with K >= 1 run
    # the fused momentum + cast, fp32 operands and K = 0 the streaming
    # momentum kernel
    run_state([(37, 52), (52, 37), (64, 128)], steps=2, k=k, prec=prec, gdt=gdt, mdt=mdt,
              wid=91, offset=1, label=f"state misaligned G={gdt} M={mdt} {prec} k={k}")


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_state_muon_wd(prec):
    run_state(RAGGED, steps=3, k=5, prec=prec, gdt="bf16", mdt="bf16", wid=92, wd=0.1,
              label=f"state muon-wd {prec}")


def test_state_momentum_norm_extremes():
    # bf16 momentum with norms that take the deferred-normalisation fallback
    # (1e-15, 1e15) and two ordinary ones; the stored bf16 M feeds it
    need_gpu()
    import orthogonalized_updates_amd as mh
    shapes = [(96, 160), (160, 96), (128, 128), (200, 120)]
    gscale = [1e-15, 1e15, 1e-6, 1.0]
    opt = mh.MuonH(shapes, grad_dtype="bf16", mom_dtype="bf16")
    W = [dev_tensor(workloads.host_custom(s, 0.02, (93, 0, i)), torch.float32) for i, s in enumerate(shapes)]
    M = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    R = opt.init(W).cpu().numpy()
    for st in range(2):
        G = [dev_tensor(workloads.host_custom(s, 0.01, (93, st + 1, i)) * gscale[i], torch.bfloat16)
             for i, s in enumerate(shapes)]
        idx = list(range(len(shapes)))
        G_vals = {i: host(G[i]) for i in idx}
        W_pre = {i: W[i].cpu().numpy() for i in idx}
        M_pre = {i: host(M[i]) for i in idx}
        say(f"[state norm extremes] step {st}")
        opt.step(W, G, M, 0.02, 0.95, 5)
        torch.cuda.synchronize()
        check_state_step(opt, W, M, G_vals, W_pre, M_pre, R, 0.02, 0.95, 5, "bf16", "bf16", idx,
                         f"state norm extremes step {st}")


def test_state_bitwise_determinism():
    need_gpu()
    import orthogonalized_updates_amd as mh
    shapes = [(300, 200), (200, 300), (256, 512)]
    outs = []
    for rep in range(2):
        opt = mh.MuonH(shapes, grad_dtype="bf16", mom_dtype="bf16")
        W = [dev_tensor(workloads.host_custom(s, 0.02, (94, 0, i)), torch.float32) for i, s in enumerate(shapes)]
        M = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        opt.init(W)
        for st in range(3):
            G = [dev_tensor(workloads.host_custom(s, 0.01, (94, st + 1, i)), torch.bfloat16)
                 for i, s in enumerate(shapes)]
            opt.step(W, G, M, 0.02, 0.95, 5)
        torch.cuda.synchronize()
        outs.append([w.cpu().numpy() for w in W] + [host(m) for m in M])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_state_qwen3_2b_full_size_sampled():
    # the benchmark's launch configuration with bf16 gradients and momentum:
    # two steps, layers 0 and 27 checked
    need_gpu()
    import orthogonalized_updates_amd as mh
    torch.cuda.empty_cache()
    wl = workloads.WORKLOADS["qwen3_2b"]
    dev = torch.device("cuda")
    opt = mh.MuonH(wl.shapes, grad_dtype="bf16", mom_dtype="bf16")
    say(f"[state qwen3_2b] generating {wl.n_matrices} matrices on the device")
    W = [workloads.device_weight_(wl, i, torch.empty(s, device=dev)) for i, s in enumerate(wl.shapes)]
    M = [torch.zeros(s, dtype=torch.bfloat16, device=dev) for s in wl.shapes]
    G32 = torch.empty(max(r * c for r, c in wl.shapes), device=dev)
    G = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in wl.shapes]
    R = opt.init(W).cpu().numpy()
    sample = list(range(0, 7)) + list(range(27 * 7, 28 * 7))
    for step in range(2):
        for i, (r, c) in enumerate(wl.shapes):
            g = G32[: r * c].view(r, c)
            workloads.device_grad_(wl, i, step, g)
            G[i].copy_(g)
        G_vals = {i: host(G[i]) for i in sample}
        W_pre = {i: W[i].cpu().numpy() for i in sample}
        M_pre = {i: host(M[i]) for i in sample}
        say(f"[state qwen3_2b] step {step}")
        opt.step(W, G, M, wl.lr, wl.beta, 5)
        torch.cuda.synchronize()
        check_state_step(opt, W, M, G_vals, W_pre, M_pre, R, wl.lr, wl.beta, 5, "bf16", "bf16",
                         sample, f"state qwen3_2b step {step}")
        norms = torch.stack([torch.linalg.vector_norm(w.double()) for w in W]).cpu().numpy()
        assert np.max(np.abs(norms / R - 1.0)) <= 1e-5
