"""GPU parity: the HIP MuonH step (through the C ABI) against the fp64 oracle.

Parity is teacher-forced per step: before each GPU step the pre-step fp32
(W, M) are copied to the host, the oracle runs the same step from them with
the same G, and the GPU's results after the step are compared:
  * update O      : relative Frobenius error <= 2e-2 (bf16 MFMA Newton-Schulz),
                    <= 5e-4 (split-bf16 operands) and <= 1e-5 (fp32 mode).
                    Where storage rounding alone already costs more (tiny
                    matrices with a few singular values: the emulated floor
                    of tests/bf16_floor.py), a bf16 or split result must
                    instead be within 1.3x of that floor. The split bound:
                    a hi + lo pair carries ~16 significant bits against
                    bf16's 8, so its floor is ~2^-8 of bf16's (~2e-2 at 8
                    iterations -> ~8e-5; emulated 2e-5..6e-5), with margin;
  * momentum M    : relative Frobenius error <= 1e-6 (fp32 fma vs fp64);
  * weights W     : within 2e-6 (relative Frobenius) of the oracle's projection
                    of the GPU's own O (this isolates the elementwise phases
                    from the Newton-Schulz rounding), and within the first-order
                    bound of the oracle's full step: W = R W'/||W'|| with
                    W' = W - lr O moves by at most R lr ||dO|| / ||W'|| when O
                    moves by dO, so ||dW||/R <= 1.5 lr ||dO|| / ||W'|| + 1e-6;
  * sphere        : | ||W||_F / R - 1 | <= 1e-5 for every matrix.
The tolerances for O and the sphere are the ones the method's specification
states; the others follow from fp32 rounding of a fused multiply-add per
element (M) and of the two-level fp32/fp64 norm (W).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

from bf16_floor import floor as bf16_floor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL_O = {"bf16": 2e-2, "split_bf16": 5e-4, "fp32": 1e-5}
PRECS = ["fp32", "bf16", "split_bf16"]


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_opt(shapes, prec):
    import orthogonalized_updates_amd as mh
    return mh.MuonH(shapes, precision=prec)


def check_step(opt, W, M, G, W_pre, M_pre, R_gpu, lr, beta, k, prec, indices, label):
    """Compare the GPU step just taken with the oracle, for matrices `indices`."""
    worst = {"O": 0.0, "M": 0.0, "Wproj": 0.0, "Wfull": 0.0, "sphere": 0.0}
    for i in indices:
        o_gpu = opt.read_update(i).cpu().numpy()
        w_gpu = W[i].cpu().numpy()
        m_gpu = M[i].cpu().numpy()
        g = G[i].cpu().numpy() if hasattr(G[i], "cpu") else G[i]
        r = float(R_gpu[i])
        w_o, m_o, o_o = oracle.muonh_step(W_pre[i], g, M_pre[i], r, lr, beta, k)
        e_o = rel(o_gpu, o_o)
        e_m = rel(m_gpu, m_o)
        e_wp = rel(w_gpu, oracle.hyperball_project(W_pre[i], o_gpu, r, lr))
        e_wf = rel(w_gpu, w_o)
        trial = np.linalg.norm(W_pre[i].astype(np.float64) - lr * o_o)
        bound_wf = 1.5 * lr * np.linalg.norm(o_gpu - o_o) / max(trial, 1e-30) + 1e-6
        e_s = abs(np.linalg.norm(w_gpu.astype(np.float64)) / r - 1.0) if r > 0 else 0.0
        for key, v in (("O", e_o), ("M", e_m), ("Wproj", e_wp), ("Wfull", e_wf), ("sphere", e_s)):
            worst[key] = max(worst[key], v)
        tol_o = TOL_O[prec]
        if prec != "fp32" and e_o > tol_o:
            fl = bf16_floor(oracle.momentum_update(M_pre[i], g, beta), k, o_o, prec)
            tol_o = max(tol_o, 1.3 * fl)
            say(f"{label} mat {i}: O err {e_o:.3e} above {TOL_O[prec]:.0e}; {prec} floor {fl:.3e}")
        assert e_o <= tol_o, f"{label} mat {i}: O rel err {e_o:.3e} > {tol_o:.3e}"
        assert e_m <= 1e-6, f"{label} mat {i}: M rel err {e_m:.3e}"
        assert e_wp <= 2e-6, f"{label} mat {i}: W vs projection of GPU O {e_wp:.3e}"
        assert e_wf <= bound_wf, f"{label} mat {i}: W vs oracle step {e_wf:.3e} > {bound_wf:.3e}"
        assert e_s <= 1e-5, f"{label} mat {i}: ||W||/R - 1 = {e_s:.3e}"
    return worst


def run_host_workload(shapes, *, steps, k, prec, lr=0.02, beta=0.95, wid=50, w_std=0.02,
                      g_std=0.01, heavy_tail=False, check_every=1, indices=None, label=""):
    """Seeded host inputs, GPU steps, oracle comparison every `check_every` steps."""
    need_gpu()
    wl = workloads.Workload(wid=wid, name=label, shapes=tuple(shapes), steps=steps, ns_iters=(k,),
                            lr=lr, beta=beta, w_std=w_std, g_std=g_std, heavy_tail=heavy_tail)
    dev = torch.device("cuda")
    opt = make_opt(shapes, prec)
    W = [torch.from_numpy(workloads.host_weight(wl, i)).to(dev) for i in range(len(shapes))]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    say(f"[{label}] init {len(shapes)} matrices {prec} k={k}")
    R = opt.init(W)
    torch.cuda.synchronize()
    R_host = R.cpu().numpy()
    for i in range(len(shapes)):
        r_o = oracle.init_radius(W[i].cpu().numpy())
        assert abs(R_host[i] - r_o) <= 1e-6 * max(r_o, 1e-30), f"R[{i}] {R_host[i]} vs {r_o}"
    idx = list(range(len(shapes))) if indices is None else indices
    worst_all = {}
    for step in range(steps):
        G_host = [workloads.host_grad(wl, i, step) for i in range(len(shapes))]
        G = [torch.from_numpy(g).to(dev) for g in G_host]
        check = (step % check_every == 0) or step == steps - 1
        if check:
            W_pre = {i: W[i].cpu().numpy() for i in idx}
            M_pre = {i: M[i].cpu().numpy() for i in idx}
        say(f"[{label}] step {step}")
        opt.step(W, G, M, lr, beta, k)
        torch.cuda.synchronize()
        if check:
            worst = check_step(opt, W, M, G_host, W_pre, M_pre, R_host, lr, beta, k, prec, idx,
                               f"{label} step {step}")
            for key, v in worst.items():
                worst_all[key] = max(worst_all.get(key, 0.0), v)
        # the sphere invariant on every matrix, every step
        for i in range(len(shapes)):
            if R_host[i] > 0:
                n = float(torch.linalg.vector_norm(W[i].double()))
                assert abs(n / R_host[i] - 1.0) <= 1e-5
    say(f"[{label}] worst errors: " + ", ".join(f"{k_}={v:.2e}" for k_, v in worst_all.items()))
    return worst_all


# ---------------------------------------------------------------------------
# Small workload (one 128x256 matrix, 10 steps) and ragged multi-group sets
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prec", PRECS)
def test_single_128x256(prec):
    wl = workloads.WORKLOADS["single_128x256"]
    run_host_workload(wl.shapes, steps=wl.steps, k=5, prec=prec, wid=wl.wid,
                      label=f"single_128x256 {prec}")


RAGGED = [(1, 1), (3, 5), (5, 3), (1, 64), (64, 1), (300, 200), (257, 129), (130, 700),
          (300, 200), (511, 513)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("k", [0, 1, 5])
def test_ragged_groups(prec, k):
    run_host_workload(RAGGED, steps=3, k=k, prec=prec, wid=51, label=f"ragged k={k} {prec}")


# 40 distinct shapes: more shape groups than one launch descriptor holds
# (16), so every phase runs as several grouped launches, and the finalize
# kernels see matrix ranges that are not the whole plan.
MANY = [(8 + 7 * i, 300 - 6 * i) for i in range(40)]


@pytest.mark.parametrize("prec,k", [("bf16", 5), ("split_bf16", 5), ("fp32", 5), ("bf16", 0)])
def test_more_shape_groups_than_one_launch_holds(prec, k):
    assert len(set(MANY)) == 40
    run_host_workload(MANY, steps=2, k=k, prec=prec, wid=57, label=f"40 groups {prec} k={k}")


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_maximum_dimension(prec):
    # the largest dimension a plan accepts (65536) on both sides: the Gram of
    # the short side runs over K = 65536 (2048 ring stages), the tall matrix
    # takes the transposed path
    import orthogonalized_updates_amd as mh
    need_gpu()
    mh.get_lib()
    top = 65536
    run_host_workload([(top, 256), (256, top)], steps=1, k=5, prec=prec, wid=58,
                      label=f"max dim {prec}")


@pytest.mark.parametrize("prec", ["bf16", "split_bf16"])
def test_eight_iterations(prec):
    run_host_workload([(384, 640), (640, 384)], steps=2, k=8, prec=prec, wid=52,
                      label=f"k8 {prec}")


def test_heavy_tailed_grads():
    run_host_workload([(512, 1536), (1536, 512)] * 3, steps=3, k=5, prec="bf16", wid=53,
                      heavy_tail=True, label="heavy-tail")


@pytest.mark.parametrize("prec", PRECS)
def test_single_2048(prec):
    wl = workloads.WORKLOADS["single_2048"]
    steps = wl.steps if prec == "bf16" else 3
    run_host_workload(wl.shapes, steps=steps, k=5, prec=prec, wid=wl.wid, check_every=4,
                      label=f"single_2048 {prec}")


# ---------------------------------------------------------------------------
# Degenerate cases
# ---------------------------------------------------------------------------

def _setup(shapes, prec="bf16", w=None):
    need_gpu()
    dev = torch.device("cuda")
    opt = make_opt(shapes, prec)
    if w is None:
        W = [torch.from_numpy(workloads.host_custom(s, 0.02, (60, i))).to(dev) for i, s in enumerate(shapes)]
    else:
        W = [t.to(dev) for t in w]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    return opt, W, M


def test_zero_weights_stay_zero():
    shapes = [(64, 96)]
    opt, W, M = _setup(shapes, w=[torch.zeros(64, 96)])
    R = opt.init(W)
    G = [torch.from_numpy(workloads.host_custom((64, 96), 0.01, (61, 0))).cuda()]
    opt.step(W, G, M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert float(R[0]) == 0.0
    # R = 0: W' = -lr*O is nonzero, and the projection scales it by R/||W'|| = 0
    assert torch.count_nonzero(W[0]) == 0


def test_zero_gradient_zero_momentum_keeps_w():
    shapes = [(200, 120), (120, 200)]
    opt, W, M = _setup(shapes)
    opt.init(W)
    W0 = [w.clone() for w in W]
    G = [torch.zeros(s, device="cuda") for s in shapes]
    opt.step(W, G, M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.count_nonzero(M[i]) == 0
        assert torch.count_nonzero(opt.read_update(i)) == 0
        # W is rescaled by R/||W|| = 1 up to float rounding of the norm
        assert float((W[i] - W0[i]).abs().max()) <= 4e-7 * float(W0[i].abs().max())


# storage rounding of X0 alone: fp32 ~6e-8, split ~2^-17, bf16 ~2^-9 (relative)
TOL_X0 = {"fp32": 1e-6, "split_bf16": 2e-5, "bf16": 4e-3}


@pytest.mark.parametrize("prec", PRECS)
def test_zero_iterations_is_normalised_momentum(prec):
    shapes = [(96, 160), (160, 96)]
    opt, W, M = _setup(shapes, prec)
    opt.init(W)
    G = [torch.from_numpy(workloads.host_custom(s, 0.01, (62, i))).cuda() for i, s in enumerate(shapes)]
    opt.step(W, G, M, 0.02, 0.0, 0)
    torch.cuda.synchronize()
    for i in range(2):
        m = M[i].cpu().numpy().astype(np.float64)
        expected = m / (np.linalg.norm(m) + 1e-7)
        assert rel(opt.read_update(i).cpu().numpy(), expected) <= TOL_X0[prec]
        np.testing.assert_array_equal(M[i].cpu().numpy(), G[i].cpu().numpy())  # beta = 0


def test_zero_lr_keeps_w():
    shapes = [(128, 128)]
    opt, W, M = _setup(shapes)
    opt.init(W)
    W0 = W[0].clone()
    G = [torch.from_numpy(workloads.host_custom((128, 128), 0.01, (63, 0))).cuda()]
    opt.step(W, G, M, 0.0, 0.9, 5)
    torch.cuda.synchronize()
    assert float((W[0] - W0).abs().max()) <= 4e-7 * float(W0.abs().max())


def test_misaligned_pointers_take_the_scalar_path():
    need_gpu()
    shapes = [(33, 47), (47, 33)]
    dev = torch.device("cuda")
    bufs = {}

    def view(name, i, s, fill):
        b = torch.zeros(s[0] * s[1] + 1, dtype=torch.float32, device=dev)
        v = b[1:].view(s)  # 4-byte offset: not 16-byte aligned
        v.copy_(fill)
        bufs[(name, i)] = b
        return v

    W = [view("W", i, s, torch.from_numpy(workloads.host_custom(s, 0.02, (64, i)))) for i, s in enumerate(shapes)]
    M = [view("M", i, s, torch.zeros(s)) for i, s in enumerate(shapes)]
    G_host = [workloads.host_custom(s, 0.01, (65, i)) for i, s in enumerate(shapes)]
    G = [view("G", i, s, torch.from_numpy(g)) for i, (s, g) in enumerate(zip(shapes, G_host))]
    assert all(t.data_ptr() % 16 for t in W + M + G)
    opt = make_opt(shapes, "fp32")
    R = opt.init(W).cpu().numpy()
    W_pre = {i: W[i].cpu().numpy() for i in range(2)}
    M_pre = {i: M[i].cpu().numpy() for i in range(2)}
    opt.step(W, G, M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    check_step(opt, W, M, G_host, W_pre, M_pre, R, 0.02, 0.95, 5, "fp32", [0, 1], "misaligned")


# ---------------------------------------------------------------------------
# Determinism, batch invariance, orientation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prec", ["bf16", "split_bf16"])
def test_bitwise_determinism_and_batch_invariance(prec):
    need_gpu()
    shapes = [(256, 512), (512, 256), (256, 512), (100, 300)]
    dev = torch.device("cuda")
    W_init = [torch.from_numpy(workloads.host_custom(s, 0.02, (66, i))) for i, s in enumerate(shapes)]
    G_host = [torch.from_numpy(workloads.host_custom(s, 0.01, (67, i))) for i, s in enumerate(shapes)]

    def run(sel):
        opt = make_opt([shapes[i] for i in sel], prec)
        W = [W_init[i].to(dev) for i in sel]
        M = [torch.zeros(shapes[i], device=dev) for i in sel]
        G = [G_host[i].to(dev) for i in sel]
        opt.init(W)
        for _ in range(2):
            opt.step(W, G, M, 0.02, 0.95, 5)
        torch.cuda.synchronize()
        return [w.cpu() for w in W], [opt.read_update(j).cpu() for j in range(len(sel))]

    w_a, o_a = run([0, 1, 2, 3])
    w_b, o_b = run([0, 1, 2, 3])
    for x, y in zip(w_a + o_a, w_b + o_b):
        assert torch.equal(x, y)
    w_c, o_c = run([2])   # matrix 2 alone equals matrix 2 inside the batch
    assert torch.equal(w_c[0], w_a[2]) and torch.equal(o_c[0], o_a[2])


def test_tail_balanced_launches_compute_every_tile():
    # 192 small matrices: every GEMM launch has two or more rounds of tiles,
    # so the last positions of each XCD's tile list are claimed at run time.
    # Each matrix must come out bit for bit as it does alone (a launch of a
    # few tiles, fixed deal), over two steps (both counter sets in use).
    need_gpu()
    shapes = [(512, 512)] * 96 + [(768, 512)] * 96
    dev = torch.device("cuda")
    W_init = [torch.from_numpy(workloads.host_custom(s, 0.02, (68, i))) for i, s in enumerate(shapes)]
    G_host = [torch.from_numpy(workloads.host_custom(s, 0.01, (69, i))) for i, s in enumerate(shapes)]

    def run(sel):
        opt = make_opt([shapes[i] for i in sel], "bf16")
        W = [W_init[i].to(dev) for i in sel]
        M = [torch.zeros(shapes[i], device=dev) for i in sel]
        G = [G_host[i].to(dev) for i in sel]
        opt.init(W)
        for _ in range(2):
            opt.step(W, G, M, 0.02, 0.95, 5)
        torch.cuda.synchronize()
        return [w.cpu() for w in W], [opt.read_update(j).cpu() for j in range(len(sel))]

    w_all, o_all = run(list(range(len(shapes))))
    say("[tail balance] batch done")
    for i in range(len(shapes)):
        w_1, o_1 = run([i])
        assert torch.equal(w_1[0], w_all[i]) and torch.equal(o_1[0], o_all[i]), f"matrix {i}"


# the tall matrix runs on the transposed layout: equal up to summation order
TOL_TALL = {"fp32": (1e-6, 1e-6), "split_bf16": (1e-4, 1e-5), "bf16": (1e-2, 1e-3)}


@pytest.mark.parametrize("prec", PRECS)
def test_tall_matrix_equals_transposed_wide(prec):
    need_gpu()
    dev = torch.device("cuda")
    m = workloads.host_custom((192, 448), 0.01, (68, 0))
    w = workloads.host_custom((192, 448), 0.02, (68, 1))
    opt = make_opt([(192, 448), (448, 192)], prec)
    W = [torch.from_numpy(w).to(dev), torch.from_numpy(np.ascontiguousarray(w.T)).to(dev)]
    M = [torch.zeros((192, 448), device=dev), torch.zeros((448, 192), device=dev)]
    G = [torch.from_numpy(m).to(dev), torch.from_numpy(np.ascontiguousarray(m.T)).to(dev)]
    opt.init(W)
    opt.step(W, G, M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    o_wide = opt.read_update(0).cpu().numpy()
    o_tall = opt.read_update(1).cpu().numpy()
    tol_o, tol_w = TOL_TALL[prec]
    assert rel(o_tall, o_wide.T) <= tol_o
    assert rel(W[1].cpu().numpy(), W[0].cpu().numpy().T) <= tol_w


def test_caller_stream_is_used():
    # the same steps on a second stream (default priority) and on the default
    # stream give identical bits; the second stream's work is ordered only by
    # that stream, so a launch on the wrong stream would race with the copies
    need_gpu()
    import orthogonalized_updates_amd as mh
    shapes = [(300, 200), (200, 300), (512, 512)]
    outs = []
    for use_side in (False, True):
        side = torch.cuda.Stream()
        ctx = torch.cuda.stream(side) if use_side else torch.cuda.stream(torch.cuda.current_stream())
        with ctx:
            opt = make_opt(shapes, "bf16")
            W = [torch.from_numpy(workloads.host_custom(s, 0.02, (75, 0, i))).to("cuda") for i, s in enumerate(shapes)]
            M = [torch.zeros(s, device="cuda") for s in shapes]
            opt.init(W)
            for st in range(3):
                G = [torch.from_numpy(workloads.host_custom(s, 0.01, (75, st + 1, i))).to("cuda")
                     for i, s in enumerate(shapes)]
                opt.step(W, G, M, 0.02, 0.95, 5)
            ad = mh.AdamW([1000, 4099])
            P = [torch.from_numpy(workloads.host_custom((n,), 0.02, (75, 9, n))).to("cuda") for n in (1000, 4099)]
            Z = [[torch.zeros(n, device="cuda") for n in (1000, 4099)] for _ in range(2)]
            Gd = [torch.from_numpy(workloads.host_custom((n,), 0.01, (75, 10, n))).to("cuda") for n in (1000, 4099)]
            ad.step(P, Gd, Z[0], Z[1], lr=1e-3, step=1)
            res = [w.cpu().numpy() for w in W] + [m.cpu().numpy() for m in M] + [p.cpu().numpy() for p in P]
        torch.cuda.synchronize()
        outs.append(res)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Full-size workloads in the benchmark's launch configuration, sampled
# ---------------------------------------------------------------------------

def run_device_workload(name, *, steps, k, sample, label, prec="bf16"):
    need_gpu()
    torch.cuda.empty_cache()
    wl = workloads.WORKLOADS[name]
    dev = torch.device("cuda")
    opt = make_opt(wl.shapes, prec)
    say(f"[{label}] generating {wl.n_matrices} matrices ({wl.n_params} params) on the device")
    W = [workloads.device_weight_(wl, i, torch.empty(s, device=dev)) for i, s in enumerate(wl.shapes)]
    M = [torch.zeros(s, device=dev) for s in wl.shapes]
    G = [torch.empty(s, device=dev) for s in wl.shapes]
    R = opt.init(W)
    torch.cuda.synchronize()
    R_host = R.cpu().numpy()
    for i in sample:
        r_o = oracle.init_radius(W[i].cpu().numpy())
        assert abs(R_host[i] - r_o) <= 1e-6 * r_o
    for step in range(steps):
        for i, s in enumerate(wl.shapes):
            workloads.device_grad_(wl, i, step, G[i])
        W_pre = {i: W[i].cpu().numpy() for i in sample}
        M_pre = {i: M[i].cpu().numpy() for i in sample}
        G_host = {i: G[i].cpu().numpy() for i in sample}
        say(f"[{label}] step {step}")
        opt.step(W, G, M, wl.lr, wl.beta, k)
        torch.cuda.synchronize()
        worst = check_step(opt, W, M, G_host, W_pre, M_pre, R_host, wl.lr, wl.beta, k, prec,
                           sample, f"{label} step {step}")
        say(f"[{label}] step {step} worst: " + ", ".join(f"{a}={b:.2e}" for a, b in worst.items()))
        norms = torch.stack([torch.linalg.vector_norm(w.double()) for w in W]).cpu().numpy()
        assert np.max(np.abs(norms / R_host - 1.0)) <= 1e-5


def test_qwen3_2b_full_size_sampled():
    # layers 0 and 27: q, k, v, o, gate, up, down
    sample = list(range(0, 7)) + list(range(27 * 7, 28 * 7))
    run_device_workload("qwen3_2b", steps=2, k=5, sample=sample, label="qwen3_2b")


def test_long_run_stays_on_the_sphere():
    # 60 consecutive steps on the full 2B-shaped set with fresh gradients:
    # every matrix keeps its radius (projection error does not accumulate),
    # W and M stay finite, and the last step still matches the oracle on
    # sampled matrices
    need_gpu()
    torch.cuda.empty_cache()
    wl = workloads.WORKLOADS["qwen3_2b"]
    dev = torch.device("cuda")
    opt = make_opt(wl.shapes, "bf16")
    W = [workloads.device_weight_(wl, i, torch.empty(s, device=dev)) for i, s in enumerate(wl.shapes)]
    M = [torch.zeros(s, device=dev) for s in wl.shapes]
    G = [torch.empty(s, device=dev) for s in wl.shapes]
    R_host = opt.init(W).cpu().numpy()
    sample = [0, 6, 100, 195]
    steps = 60
    for step in range(steps):
        for i in range(len(wl.shapes)):
            workloads.device_grad_(wl, i, 1000 + step, G[i])
        if step == steps - 1:
            W_pre = {i: W[i].cpu().numpy() for i in sample}
            M_pre = {i: M[i].cpu().numpy() for i in sample}
            G_host = {i: G[i].cpu().numpy() for i in sample}
        opt.step(W, G, M, wl.lr, wl.beta, 5)
        if step % 20 == 0:
            say(f"[long run] step {step}")
    torch.cuda.synchronize()
    norms = torch.stack([torch.linalg.vector_norm(w.double()) for w in W]).cpu().numpy()
    assert np.max(np.abs(norms / R_host - 1.0)) <= 1e-5
    assert all(bool(torch.isfinite(w).all()) and bool(torch.isfinite(m).all()) for w, m in zip(W, M))
    check_step(opt, W, M, G_host, W_pre, M_pre, R_host, wl.lr, wl.beta, 5, "bf16", sample,
               "long run, last step")


def test_occupancy_full_size_sampled():
    run_device_workload("occupancy_512x1536", steps=2, k=5, sample=[0, 1, 255, 256, 300, 511],
                        label="occupancy")


@pytest.mark.parametrize("k,prec", [(5, "bf16"), (8, "split_bf16")])
def test_large_full_size_sampled(k, prec):
    # 64 matrices of 4096x14336 (32 wide, 32 tall); one step, checked on one
    # matrix of each orientation. At 8 iterations bf16 storage alone costs
    # ~2.5e-2 on these (above the 2e-2 bound), so that count runs with
    # split-bf16 operands.
    run_device_workload("large_4096x14336", steps=1, k=k, sample=[0, 63], prec=prec,
                        label=f"large k={k} {prec}")


# ---------------------------------------------------------------------------
# muonh_step against muonh_step_timed (the same schedule plus phase events):
# the results must agree bit for bit, step after step, on a set with several
# shape groups of both orientations.
# ---------------------------------------------------------------------------

def test_step_and_timed_step_agree_bitwise():
    need_gpu()
    dev = torch.device("cuda")
    shapes = [(1024, 3072)] * 12 + [(3072, 1024)] * 12 + [(2048, 2048)] * 8 + [(256, 1024)] * 8
    k = 5
    W0 = [workloads.device_normal_(torch.empty(s, device=dev), 0.02, 70, i, 0, 0)
          for i, s in enumerate(shapes)]
    Gs = [[workloads.device_normal_(torch.empty(s, device=dev), 0.01, 70, i, st, 1)
           for i, s in enumerate(shapes)] for st in range(3)]
    runs = []
    for timed in (False, True):
        opt = make_opt(shapes, "bf16")
        W = [w.clone() for w in W0]
        M = [torch.zeros(s, device=dev) for s in shapes]
        opt.init(W)
        for st in range(3):
            say(f"[step vs timed] timed={timed} step {st}")
            if timed:
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(3 * k + 3)]
                for e in evs:
                    e.record()
                opt.step_timed(W, Gs[st], M, 0.02, 0.95, k, evs)
            else:
                opt.step(W, Gs[st], M, 0.02, 0.95, k)
        torch.cuda.synchronize()
        runs.append(([w.cpu() for w in W], [m.cpu() for m in M],
                     [opt.read_update(i).cpu() for i in range(len(shapes))]))
    for name, a, b in zip(("W", "M", "O"), runs[0], runs[1]):
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"{name}[{i}] differs between step and step_timed"


# ---------------------------------------------------------------------------
# Deferred normalisation of X0 (bf16 and split operands): momentum norms far
# outside [2^-40, 2^40] take the fallback that writes X0 normalised; a norm
# of 1e-6 stays on the deferred path, where eps = 1e-7 still moves X0 by ~8 %.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prec", ["bf16", "split_bf16"])
def test_momentum_norm_extremes(prec):
    need_gpu()
    dev = torch.device("cuda")
    shapes = [(96, 160), (160, 96), (128, 128), (200, 120)]
    gscale = [1e-15, 1e15, 1e-6, 1.0]  # ||M|| ~ 1.2 * scale after the first step
    opt, W, M = _setup(shapes, prec)
    R = opt.init(W).cpu().numpy()
    for st in range(2):
        G_host = [(workloads.host_custom(sh, 0.01, (72, st, i)) * gscale[i]).astype(np.float32)
                  for i, sh in enumerate(shapes)]
        G = [torch.from_numpy(g).to(dev) for g in G_host]
        W_pre = {i: W[i].cpu().numpy() for i in range(len(shapes))}
        M_pre = {i: M[i].cpu().numpy() for i in range(len(shapes))}
        say(f"[norm extremes {prec}] step {st}")
        opt.step(W, G, M, 0.02, 0.95, 5)
        torch.cuda.synchronize()
        check_step(opt, W, M, G_host, W_pre, M_pre, R, 0.02, 0.95, 5, prec,
                   list(range(len(shapes))), f"norm extremes {prec} step {st}")


# ---------------------------------------------------------------------------
# Muon with decoupled weight decay (muonh_step_muon_wd): same momentum and
# Newton-Schulz, then W <- (1 - lr*wd) W - lr O. O and M as for MuonH. W is
# checked against the oracle's update applied to the GPU's own O, and against
# the oracle's full step within lr*||dO||. The two terms can cancel (a small
# matrix whose decayed W nearly equals lr*O), so the fp32 part of both bounds
# is relative to the terms, not to the result: per element the GPU rounds
# (1 - lr*wd)*w once and the fused multiply-add once, i.e. a few ulps of
# |w| + lr*|o|; 1e-6 * (||W|| + lr*||O||) allows about 16.
# ---------------------------------------------------------------------------

def check_muon_step(opt, W, M, G, W_pre, M_pre, lr, beta, wd, k, prec, indices, label):
    for i in indices:
        o_gpu = opt.read_update(i).cpu().numpy()
        w_gpu = W[i].cpu().numpy()
        m_gpu = M[i].cpu().numpy()
        g = G[i].cpu().numpy() if hasattr(G[i], "cpu") else G[i]
        w_o, m_o, o_o = oracle.muon_wd_step(W_pre[i], g, M_pre[i], lr, beta, wd, k)
        e_o = rel(o_gpu, o_o)
        tol_o = TOL_O[prec]
        if prec != "fp32" and e_o > tol_o:
            fl = bf16_floor(oracle.momentum_update(M_pre[i], g, beta), k, o_o, prec)
            tol_o = max(tol_o, 1.3 * fl)
        assert e_o <= tol_o, f"{label} mat {i}: O rel err {e_o:.3e} > {tol_o:.3e}"
        assert rel(m_gpu, m_o) <= 1e-6, f"{label} mat {i}: M"
        w_pre = W_pre[i].astype(np.float64)
        w_own = (1.0 - lr * wd) * w_pre - lr * o_gpu
        fp32 = 1e-6 * (np.linalg.norm(w_pre) + lr * np.linalg.norm(o_gpu))
        d_own = np.linalg.norm(w_gpu - w_own)
        assert d_own <= fp32, f"{label} mat {i}: W vs decayed update of GPU O: {d_own:.3e} > {fp32:.3e}"
        d_full = np.linalg.norm(w_gpu - w_o)
        bound = 1.5 * lr * np.linalg.norm(o_gpu - o_o) + fp32
        assert d_full <= bound, f"{label} mat {i}: W vs oracle step: {d_full:.3e} > {bound:.3e}"


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("k", [0, 5])
def test_muon_wd_ragged_groups(prec, k):
    need_gpu()
    dev = torch.device("cuda")
    wl = workloads.Workload(wid=73, name="muon", shapes=tuple(RAGGED), steps=3, ns_iters=(k,),
                            lr=0.02, beta=0.95, w_std=0.02, g_std=0.01, heavy_tail=False)
    opt = make_opt(RAGGED, prec)
    W = [torch.from_numpy(workloads.host_weight(wl, i)).to(dev) for i in range(len(RAGGED))]
    M = [torch.zeros(s, device=dev) for s in RAGGED]
    idx = list(range(len(RAGGED)))
    for st in range(3):
        G_host = [workloads.host_grad(wl, i, st) for i in idx]
        G = [torch.from_numpy(g).to(dev) for g in G_host]
        W_pre = {i: W[i].cpu().numpy() for i in idx}
        M_pre = {i: M[i].cpu().numpy() for i in idx}
        say(f"[muon-wd {prec} k={k}] step {st}")
        opt.step_muon_wd(W, G, M, 0.02, 0.95, 0.1, k)
        torch.cuda.synchronize()
        check_muon_step(opt, W, M, G_host, W_pre, M_pre, 0.02, 0.95, 0.1, k, prec, idx,
                        f"muon-wd {prec} k={k} step {st}")


def test_muon_wd_decay_only():
    need_gpu()
    shapes = [(64, 96), (96, 64)]
    opt, W, M = _setup(shapes)
    W0 = [w.cpu().numpy().astype(np.float64) for w in W]
    G = [torch.zeros(s, device="cuda") for s in shapes]
    opt.step_muon_wd(W, G, M, 0.02, 0.9, 0.1, 5)
    torch.cuda.synchronize()
    for i in range(2):
        assert rel(W[i].cpu().numpy(), (1 - 0.02 * 0.1) * W0[i]) <= 1e-7
        assert torch.count_nonzero(opt.read_update(i)) == 0


def test_muon_wd_full_size_sampled_after_a_muonh_step():
    # one plan and workspace shared by both entry points
    need_gpu()
    torch.cuda.empty_cache()
    wl = workloads.WORKLOADS["qwen3_2b"]
    dev = torch.device("cuda")
    opt = make_opt(wl.shapes, "bf16")
    W = [workloads.device_weight_(wl, i, torch.empty(s, device=dev)) for i, s in enumerate(wl.shapes)]
    M = [torch.zeros(s, device=dev) for s in wl.shapes]
    G = [torch.empty(s, device=dev) for s in wl.shapes]
    opt.init(W)
    for i, s in enumerate(wl.shapes):
        workloads.device_grad_(wl, i, 0, G[i])
    say("[muon-wd qwen3_2b] muonh step")
    opt.step(W, G, M, wl.lr, wl.beta, 5)
    for i, s in enumerate(wl.shapes):
        workloads.device_grad_(wl, i, 1, G[i])
    sample = list(range(0, 7)) + list(range(27 * 7, 28 * 7)) + [100, 150]
    W_pre = {i: W[i].cpu().numpy() for i in sample}
    M_pre = {i: M[i].cpu().numpy() for i in sample}
    G_host = {i: G[i].cpu().numpy() for i in sample}
    say("[muon-wd qwen3_2b] muon-wd step")
    opt.step_muon_wd(W, G, M, wl.lr, wl.beta, 0.1, 5)
    torch.cuda.synchronize()
    check_muon_step(opt, W, M, G_host, W_pre, M_pre, wl.lr, wl.beta, 0.1, 5, "bf16", sample,
                    "muon-wd qwen3_2b")
