"""Host logic of bench.py (no GPU): the algorithmic work it divides by, the
committed-traffic lookup, the one-GPU guard and the CPU-baseline legs."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_ns_flops_of_the_2b_set():
    wl = workloads.WORKLOADS["qwen3_2b"]
    f = bench.ns_flops(wl.shapes, 5)
    # per iteration: Gram s^2 l, polynomial s^3, apply 2 s^2 l, summed over
    # 56 x 2048^2, 56 x 512x2048, 84 x 2048x6144 (after transposition)
    gram = 56 * 2048 ** 3 + 56 * 512 ** 2 * 2048 + 84 * 2048 ** 2 * 6144
    poly = 56 * 2048 ** 3 + 56 * 512 ** 3 + 84 * 2048 ** 3
    assert f["gram"] == gram and f["poly"] == poly and f["apply"] == 2 * gram
    assert f["apply"] == pytest.approx(5.3515e12, rel=1e-4)
    # 5 iterations of 3 s^2 l + s^3: the per-step total of this set
    assert 5 * sum(f.values()) == pytest.approx(4.620e13, rel=1e-3)


def test_ns_flops_transposes_tall_matrices():
    assert bench.ns_flops([(6144, 2048)], 1) == bench.ns_flops([(2048, 6144)], 1)


@pytest.mark.parametrize("ns_bytes,fused,variant,g,m,pre,post", [
    (2, True, "muonh", 4, 4, 14, 16),      # default: momentum + cast fused, bf16 operands
    (2, True, "muon_wd", 4, 4, 14, 10),    # one decayed-update pass after NS
    (2, True, "muonh", 2, 2, 8, 16),       # bf16 gradient and momentum
    (2, True, "muonh", 4, 2, 10, 16),      # bf16 momentum only
    (4, True, "muonh", 4, 4, 16, 20),      # split operands: 4 bytes per element
    (4, False, "muonh", 4, 4, 24, 20),     # fp32 operands: the cast re-reads M, writes X and X^T
])
def test_elementwise_bytes(ns_bytes, fused, variant, g, m, pre, post):
    assert bench.elementwise_bytes(1, ns_bytes, fused, variant, g, m) == (pre, post)


def test_committed_traffic_lookup(tmp_path, monkeypatch):
    import hashlib
    (tmp_path / "profiles").mkdir()
    src_dir = tmp_path / "orthogonalized_updates_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "k.hip").write_text("// header\nkernel source\n\n")
    sha = hashlib.sha256(b"kernel source").hexdigest()[:16]
    assert bench.code_sha16(str(src_dir / "k.hip")) == sha
    rec = {"kernel": "k_x", "source": "k.hip", "source_sha256_16": sha, "traffic_bytes_per_launch": 1234}
    (tmp_path / "profiles" / "s.md").write_text("# summary\n\n```\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_traffic("k_x", "s.md", "k.hip") == 1234
    assert bench.committed_traffic("k_y", "s.md", "k.hip") is None        # other kernel
    assert bench.committed_traffic("k_x", "missing.md", "k.hip") is None  # no summary
    # comments and blank lines are not code: the counters stay valid
    (src_dir / "k.hip").write_text("// reworded header\n\nkernel source  // note\n")
    assert bench.committed_traffic("k_x", "s.md", "k.hip") == 1234
    (src_dir / "k.hip").write_text("kernel source, changed\n")
    assert bench.committed_traffic("k_x", "s.md", "k.hip") is None        # stale counters


def test_committed_summaries_name_their_source_hash():
    # every machine-readable traffic line in profiles/ carries the fields the lookup reads
    pdir = os.path.join(ROOT, "profiles")
    lines = []
    for name in os.listdir(pdir):
        for line in open(os.path.join(pdir, name)):
            if line.startswith("{") and "traffic_bytes_per_launch" in line:
                lines.append(json.loads(line))
    assert lines
    for rec in lines:
        assert {"kernel", "source", "source_sha256_16", "traffic_bytes_per_launch"} <= set(rec)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _bench_sample(wl, k, spoil_tile=False):
    """Host arrays shaped like bench.py's sample: pre-step inputs of one matrix
    per shape, and 'GPU' results made from the oracle's own, rounded to fp32
    (optionally with one 256x256 tile of O negated)."""
    import numpy as np

    import oracle
    out = {}
    for _, idx in wl.shape_groups():
        i = idx[0]
        w = workloads.host_weight(wl, i)
        g = workloads.host_grad(wl, i, 0)
        m = np.zeros_like(w)
        r = oracle.init_radius(w)
        w1, m1, o1 = oracle.muonh_step(w, g, m, r, wl.lr, wl.beta, k)
        o = o1.astype(np.float32)
        if spoil_tile:
            o[:256, :256] *= -1
        out[i] = {"w_pre": w, "m_pre": m, "g": g, "r": r, "o": o, "w": w1.astype(np.float32),
                  "m": m1.astype(np.float32)}
    return out


def test_cpu_baselines_report_the_oracle():
    wl = workloads.WORKLOADS["single_128x256"]
    r = bench.cpu_baseline(wl, 5, 0.05, _bench_sample(wl, 5))
    assert r["kind"] == "oracle" and r["unit"] == "params/s" and r["value"] > 0 and r["cores"] >= 1
    assert r["parity"]["ok"] and r["parity"]["matrices"][0]["o_rel_err"] < 1e-6
    bad = bench.cpu_baseline(wl, 5, 0.05, _bench_sample(wl, 5, spoil_tile=True))
    assert not bad["parity"]["ok"]
    assert bad["parity"]["matrices"][0]["o_worst_tile_rel_err"] > 1.0
    a = bench.adamw_cpu_baseline(1000, 0.05)
    assert a["kind"] == "oracle" and a["value"] > 0 and a["cores"] == 1


def test_clock_sampler_without_a_gpu_reports_why():
    with bench.ClockSampler(period_s=0.001) as c:
        pass
    rec = c.summary()
    assert rec["source"].startswith("amdsmi") and (rec["mhz_mean"] is not None or rec["note"])
    pw = c.power_summary()
    assert {"cap_w", "w_mean", "ppt_limit_share", "window_s"} <= set(pw)
    assert pw["ppt_limit_share"] is not None or pw["note"]
    assert bench.runtime_versions()["rocm"]
