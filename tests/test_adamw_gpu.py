"""GPU parity of the AdamW step (muonh_adamw_step) against the fp64 oracle.

Teacher-forced per step: the oracle takes the GPU's pre-step fp32 p, m, v and
the same g. The kernel computes in fp32 with the step constants from fp64, so
each result is within a few ulps of its terms: per element,
  |dm| <= 4e-7 (beta1 |m0| + (1 - beta1) |g|)
  |dv| <= 5e-7 (beta2 v0 + (1 - beta2) g^2)
  |dp| <= 3e-7 (|p0| + |p1|) + 2e-6 lr |m_hat / (sqrt(v_hat) + eps)|
          + (lr / (1 - beta1^t)) |dm|max / (sqrt(v_hat) + eps)
(u = 2^-24 = 6e-8; the adaptive ratio goes through about ten fp32 roundings).
The last term carries the absolute error of the new m into p: where
beta1 m0 and (1 - beta1) g nearly cancel, m is small and its rounding error
is large relative to it, so a bound relative to the ratio alone is too tight.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(p_gpu, m_gpu, v_gpu, p0, g, m0, v0, step, label, hp=HP):
    p0, g, m0, v0 = (np.asarray(x, dtype=np.float64) for x in (p0, g, m0, v0))
    p1, m1, v1 = oracle.adamw_step(p0, g, m0, v0, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                   hp["weight_decay"], step)
    b1, b2 = hp["beta1"], hp["beta2"]
    tm = 4e-7 * (b1 * np.abs(m0) + (1 - b1) * np.abs(g)) + 1e-38
    tv = 5e-7 * (b2 * v0 + (1 - b2) * g * g) + 1e-38
    ratio = (m1 / (1 - b1 ** step)) / (np.sqrt(v1 / (1 - b2 ** step)) + hp["eps"])
    den = np.sqrt(v1 / (1 - b2 ** step)) + hp["eps"]
    tp = (3e-7 * (np.abs(p0) + np.abs(p1)) + 2e-6 * hp["lr"] * np.abs(ratio)
          + hp["lr"] / (1 - b1 ** step) * tm / den + 1e-38)
    for name, got, exp, tol in (("m", m_gpu, m1, tm), ("v", v_gpu, v1, tv), ("p", p_gpu, p1, tp)):
        err = np.abs(np.asarray(got, dtype=np.float64) - exp)
        bad = np.flatnonzero(err > tol)
        assert bad.size == 0, (f"{label}: {name} off at {bad.size} elements, first {bad[0]}: "
                               f"{err.flat[bad[0]]:.3e} > {tol.flat[bad[0]]:.3e}")


def run(sizes, steps, key, offset=0, label=""):
    """Seeded host tensors (optionally views at a float offset, so not
    16-byte aligned), `steps` GPU steps, each checked against the oracle."""
    need_gpu()
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    keep = []

    def dev_tensor(a):
        base = torch.zeros(a.size + offset, dtype=torch.float32, device=dev)
        t = base[offset:]
        t.copy_(torch.from_numpy(a.astype(np.float32)))
        keep.append(base)
        return t

    P = [dev_tensor(workloads.host_custom((n,), 0.02, (key, 0, i))) for i, n in enumerate(sizes)]
    M = [dev_tensor(np.zeros(n, np.float32)) for n in sizes]
    V = [dev_tensor(np.zeros(n, np.float32)) for n in sizes]
    opt = mh.AdamW(sizes, device=dev)
    for st in range(1, steps + 1):
        G_h = [workloads.host_custom((n,), 0.01, (key, st, i)) for i, n in enumerate(sizes)]
        G = [dev_tensor(g) for g in G_h]
        pre = [(P[i].cpu().numpy(), M[i].cpu().numpy(), V[i].cpu().numpy()) for i in range(len(sizes))]
        say(f"[adamw {label}] step {st}")
        opt.step(P, G, M, V, step=st, **HP)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            check(P[i].cpu().numpy(), M[i].cpu().numpy(), V[i].cpu().numpy(), pre[i][0], G_h[i],
                  pre[i][1], pre[i][2], st, f"{label} step {st} tensor {i}")


RAGGED = [0, 1, 3, 4, 7, 4096, 4097, 65536, 100003]


def test_adamw_ragged_sizes():
    run(RAGGED, 3, 80, label="ragged")


def test_adamw_misaligned_tensors_take_the_scalar_path():
    run([5, 4096, 10001], 2, 81, offset=1, label="misaligned")


def test_adamw_more_tensors_than_one_launch_holds():
    rng = np.random.default_rng(82)
    run([int(x) for x in rng.integers(1, 5000, size=150)], 2, 82, label="150 tensors")


def test_adamw_decay_only():
    need_gpu()
    import orthogonalized_updates_amd as mh
    dev = torch.device("cuda")
    p = torch.from_numpy(workloads.host_custom((9000,), 0.02, (83, 0, 0))).to(dev)
    p0 = p.cpu().numpy().astype(np.float64)
    z = [torch.zeros(9000, device=dev) for _ in range(3)]
    mh.AdamW([9000], device=dev).step([p], [z[0]], [z[1]], [z[2]], step=4, **HP)
    torch.cuda.synchronize()
    exp = p0 * (1 - HP["lr"] * HP["weight_decay"])
    assert np.max(np.abs(p.cpu().numpy() - exp) / np.maximum(np.abs(exp), 1e-30)) <= 1.2e-7
    assert not torch.any(z[1]) and not torch.any(z[2])


def test_adamw_full_size_embedding_sampled():
    # the largest tensor of the non-matrix parameter set, one step, 4 slices
    need_gpu()
    import orthogonalized_updates_amd as mh
    torch.cuda.empty_cache()
    dev = torch.device("cuda")
    n = workloads.ADAMW_SETS["qwen3_2b_rest"][0]
    p = workloads.device_normal_(torch.empty(n, device=dev), 0.02, 84, 0, 0, 0)
    g = workloads.device_normal_(torch.empty(n, device=dev), 0.01, 84, 0, 1, 1)
    m = workloads.device_normal_(torch.empty(n, device=dev), 0.001, 84, 0, 1, 2)
    v = workloads.device_normal_(torch.empty(n, device=dev), 1e-4, 84, 0, 1, 3).square_()
    sl = [slice(0, 4096), slice(n // 3, n // 3 + 4097), slice(n // 2, n // 2 + 513), slice(n - 1000, n)]
    pre = [(p[s].cpu().numpy(), g[s].cpu().numpy(), m[s].cpu().numpy(), v[s].cpu().numpy()) for s in sl]
    say("[adamw full size] step 7")
    mh.AdamW([n], device=dev).step([p], [g], [m], [v], step=7, **HP)
    torch.cuda.synchronize()
    for s, (p0, g0, m0, v0) in zip(sl, pre):
        check(p[s].cpu().numpy(), m[s].cpu().numpy(), v[s].cpu().numpy(), p0, g0, m0, v0, 7,
              f"full size slice {s.start}")
