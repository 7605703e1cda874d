#!/usr/bin/env python3
"""MuonH optimizer-step benchmark on one MI355X.

A step is one full MuonH step over the whole matrix set: momentum, the
normalised bf16 cast, 5 Newton-Schulz iterations (Gram, polynomial, apply) on
bf16 MFMA with fp32 accumulation, the trial update and the projection onto
each matrix's init-norm sphere. Inputs are synthetic and seeded (workloads.py)
and already resident in HBM when the timed region starts.

Prints ONE JSON line: params updated per second for the whole set, step time,
the roofline of the dominant kernel (from HIP events recorded inside the
timed steps), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host.

With --variant muon_wd the same plan runs the Muon baseline (decoupled
weight decay instead of the projection); with --variant adamw the step is
one AdamW update of the parameters outside the matrix group (the embedding
and norm vectors of the same 2B-shaped model), an HBM-bound elementwise
launch.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--workload qwen3_2b]
                       [--variant muonh|muon_wd|adamw]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "MuonH step time & params updated/s (2B-shaped set); NS TFLOP/s % MFMA peak"
METRIC_MUON_WD = ("Muon + decoupled weight decay (the baseline) step time & params updated/s "
                  "(2B-shaped set); NS TFLOP/s % MFMA peak")
METRIC_ADAMW = ("AdamW step time & params updated/s (non-matrix parameters of the 2B-shaped "
                "model); HBM GB/s % peak")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


POWER_SETTLE_S = 1.2


def ns_flops(shapes, k):
    """Algorithmic Newton-Schulz flops per launch of each phase (one iteration).

    Per matrix with short side s and long side l: the Gram X X^T is symmetric,
    s^2 l; the polynomial's A A is symmetric, s^3; the apply B X is 2 s^2 l.
    """
    gram = poly = apply = 0.0
    for r, c in shapes:
        s, l = min(r, c), max(r, c)
        gram += float(s) * s * l
        poly += float(s) ** 3
        apply += 2.0 * s * s * l
    return {"gram": gram, "poly": poly, "apply": apply}


def elementwise_bytes(n_params, ns_bytes, fused, variant="muonh", g_bytes=4, m_bytes=4):
    """Algorithmic HBM bytes of the streaming phases, per step.

    before Newton-Schulz: momentum reads G, M and writes M (g + 2m B/param:
      12 with fp32 G and M, 6 with both in bf16) and X0 is written once
      (ns_bytes); with bf16 or split operands and at least one iteration the
      two happen in one pass (fused), otherwise the cast reads M again and,
      in fp32 mode, writes X and X^T: g + 2m + m + 2*ns_bytes B/param;
    after: the trial-norm pass reads W and O (4 + ns_bytes), the projection
      reads W and O and writes W (8 + ns_bytes); the Muon baseline's decayed
      update is one pass that reads W and O and writes W (8 + ns_bytes).
    """
    mom = g_bytes + 2 * m_bytes
    pre = n_params * (mom + ns_bytes if fused else mom + m_bytes + 2 * ns_bytes)
    if variant == "muon_wd":
        post = n_params * (8 + ns_bytes)
    else:
        post = n_params * (4 + ns_bytes + 8 + ns_bytes)
    return pre, post


def cpu_baseline(wl, k, budget_s, sample, variant="muonh", weight_decay=0.1, mom_bf16=False,
                 prec="bf16"):
    """The fp64 oracle on the host, timed on one matrix of each distinct
    shape and extrapolated by count to the whole set (matrices are
    independent), on the very inputs of one more GPU step taken after the
    timed ones: `sample` maps a matrix index to its host arrays (pre-step W,
    M, G and R, and the GPU's O, W, M after that step). Each oracle result is
    also compared with the GPU's (the parity bar of the tests: O within 2e-2
    with bf16 operands, on the whole matrix and on every 256 x 256 tile of
    4096 or more entries). With mom_bf16 the oracle keeps the momentum in
    bf16 (one rounding of the exact value)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    groups = wl.shape_groups()
    per_shape_budget = budget_s / max(len(groups), 1)
    total = 0.0
    used = 0.0
    parts = []
    checks = []
    for (r, c), idx in groups:
        i = idx[0]
        x = sample[i]
        runs = 0
        t0 = time.perf_counter()
        while True:
            if variant == "muon_wd":
                w_o, m_o, o_o = oracle.muon_wd_step(x["w_pre"], x["g"], x["m_pre"], wl.lr, wl.beta,
                                                    weight_decay, k, mom_bf16=mom_bf16)
            else:
                w_o, m_o, o_o = oracle.muonh_step(x["w_pre"], x["g"], x["m_pre"], x["r"], wl.lr,
                                                  wl.beta, k, mom_bf16=mom_bf16)
            runs += 1
            el = time.perf_counter() - t0
            if el >= per_shape_budget or runs >= 5:
                break
        t = el / runs
        used += el
        total += t * len(idx)
        parts.append(f"{r}x{c}: {t:.3f} s x {len(idx)}")
        checks.append(parity_numbers(i, (r, c), x, o_o, m_o, w_o, mom_bf16))
    out = {
        "value": wl.n_params / total,
        "unit": "params/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": ("one fp64 oracle step (momentum, Newton-Schulz k=%d, %s) of one matrix "
                   "per distinct shape, on the inputs of a GPU step taken after the timed ones, "
                   "timed over %.1f s and extrapolated by matrix count to the full set (%s); "
                   "est. %.1f s per full step"
                   % (k, "decayed update" if variant == "muon_wd" else "projection", used,
                      "; ".join(parts), total)),
        "host_cpu": host_cpu(),
    }
    tol = {"bf16": 2e-2, "split_bf16": 5e-4, "fp32": 1e-5}[prec]
    out["parity"] = {"matrices": checks, "o_bar": tol,
                     "ok": all(cm["o_rel_err"] <= tol and cm["o_worst_tile_rel_err"] <= tol
                               for cm in checks)}
    return out


def parity_numbers(i, shape, x, o_o, m_o, w_o, mom_bf16):
    """The GPU's results of one matrix against the oracle's on the same inputs."""
    import numpy as np

    def rel(a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        nb = np.linalg.norm(b)
        return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))
    worst_tile = 0.0
    for r0 in range(0, o_o.shape[0], 256):
        for c0 in range(0, o_o.shape[1], 256):
            t = o_o[r0:r0 + 256, c0:c0 + 256]
            if t.size >= 4096:
                worst_tile = max(worst_tile, rel(x["o"][r0:r0 + 256, c0:c0 + 256], t))
    rec = {"index": int(i), "shape": list(shape), "o_rel_err": rel(x["o"], o_o),
           "o_worst_tile_rel_err": worst_tile, "w_rel_err": rel(x["w"], w_o)}
    if mom_bf16:
        rec["m_bits_differing"] = int(np.count_nonzero(np.asarray(x["m"], np.float64) != m_o))
    else:
        rec["m_rel_err"] = rel(x["m"], m_o)
    return rec


class ClockSampler:
    """Samples the GPU's graphics clock and socket power (amdsmi) on a host
    thread while steps run, after dropping the first `settle_s` seconds, and
    reads the firmware's power-limit residency counters at the start and end
    of the sampled window. Reports the clock's mean, min and max in MHz, the
    mean of the power samples in W against the power cap, and the share of
    the firmware's accumulation ticks spent at the package power limit, or
    why it could not. The firmware refreshes all of these about once a
    second, so the window has to span a few seconds."""

    def __init__(self, period_s=0.002, power_every=25, settle_s=0.0):
        import threading
        self.period = period_s
        self.power_every = power_every
        self.settle = settle_s
        self.samples = []
        self.power = []
        self.error = None
        self.cap_w = None
        self.m0 = self.m1 = None
        self.t0 = self.t1 = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # pragma: no cover - depends on the machine
            self.error = f"amdsmi unavailable: {e}"[:160]
            return
        try:
            cap = amdsmi.amdsmi_get_power_cap_info(self._h)["power_cap"]
            self.cap_w = round(cap / 1e6, 1) if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:  # pragma: no cover
            self.cap_w = None

    def _read(self):
        info = self._smi.amdsmi_get_clock_info(self._h, self._smi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def _read_power(self):
        try:
            w = self._smi.amdsmi_get_power_info(self._h)["current_socket_power"]
            return float(w) if isinstance(w, (int, float)) else None
        except Exception:  # pragma: no cover
            return None

    def _metrics(self):
        try:
            m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
            return {k: m.get(k) for k in ("accumulation_counter", "ppt_residency_acc",
                                          "socket_thm_residency_acc")}
        except Exception:  # pragma: no cover
            return None

    def _run(self):
        n = 0
        start = time.perf_counter()
        while not self._stop.is_set() and time.perf_counter() - start < self.settle:
            self._stop.wait(self.period)
        if self._stop.is_set():
            return
        self.m0 = self._metrics()
        self.t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # pragma: no cover
                self.error = f"clock read failed: {e}"[:160]
                return
            if n % self.power_every == 0:
                w = self._read_power()
                if w is not None:
                    self.power.append(w)
            n += 1
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
            if self.t0 is not None:
                self.t1 = time.perf_counter()
                self.m1 = self._metrics()
        try:
            if self.error is None:
                self._smi.amdsmi_shut_down()
        except Exception:  # pragma: no cover
            pass
        return False

    def power_summary(self):
        out = {"source": "amdsmi current socket power, sampled on a host thread",
               "cap_w": self.cap_w, "w_mean": None, "w_max": None, "samples": len(self.power),
               "ppt_limit_share": None}
        if self.power:
            out["w_mean"] = round(sum(self.power) / len(self.power), 1)
            out["w_max"] = max(self.power)
        try:
            dacc = self.m1["accumulation_counter"] - self.m0["accumulation_counter"]
            dppt = self.m1["ppt_residency_acc"] - self.m0["ppt_residency_acc"]
            if dacc > 0:
                out["ppt_limit_share"] = round(dppt / dacc, 3)
                out["ppt_ticks"] = int(dacc)
            else:
                out["note"] = "the firmware's residency counters did not advance in the timed region"
        except Exception:
            out["note"] = "power-limit residency counters unavailable"
        out["window_s"] = round(self.t1 - self.t0, 3) if self.t0 and self.t1 else None
        return out

    def summary(self):
        if not self.samples:
            return {"source": "amdsmi gfx clock", "mhz_mean": None,
                    "note": self.error or "no samples"}
        v = self.samples
        return {"source": "amdsmi gfx clock, sampled on a host thread",
                "samples": len(v), "mhz_mean": round(sum(v) / len(v), 1),
                "mhz_min": min(v), "mhz_max": max(v)}


def runtime_versions():
    """ROCm release of the installation and the HIP runtime torch uses."""
    rocm = None
    for path in ("/opt/rocm/.info/version",):
        try:
            with open(path) as f:
                rocm = f.read().strip()
        except OSError:
            pass
    try:
        import torch
        hip = torch.version.hip
        name = torch.cuda.get_device_name(0) if torch.cuda.is_available() else None
    except Exception:  # pragma: no cover
        hip, name = None, None
    return {"rocm": rocm, "hip_runtime": hip, "device": name}


def host_cpu() -> str:
    """CPU model from /proc/cpuinfo and the logical CPU count of the host."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def code_sha16(path: str) -> str:
    """First 16 hex digits of the SHA-256 of a source file's code: each line
    with any // comment cut off and trailing blanks stripped, blank lines
    dropped, so that comment edits do not count as changes."""
    import hashlib
    lines = []
    for line in open(path, encoding="utf-8"):
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def committed_traffic(kernel_name: str, summary: str, source: str = "ns_gemm.hip"):
    """HBM bytes per launch of `kernel_name` from the committed rocprofv3
    counter summary profiles/`summary` (FETCH_SIZE + WRITE_SIZE, each scaled
    by its factor on a plain copy of known size), or None when there is no
    such summary or the kernel's source code has changed since the counters
    were taken (the summary records code_sha16 of the source)."""
    path = os.path.join(ROOT, "profiles", summary)
    src = os.path.join(ROOT, "orthogonalized_updates_amd", "csrc", source)
    try:
        sha = code_sha16(src)
        for line in open(path):
            line = line.strip()
            if line.startswith("{") and '"traffic_bytes_per_launch"' in line:
                rec = json.loads(line)
                if rec.get("kernel") == kernel_name and rec.get("source_sha256_16") == sha:
                    return int(rec["traffic_bytes_per_launch"])
    except (OSError, ValueError):
        return None
    return None


def calibrate_copy() -> int:
    """A plain device copy of known size: each launch reads and writes 1 GiB.

    Run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, its counters give the
    factor between the counters and true HBM bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 3}), flush=True)
    return 0


ADAMW_WID = 5          # seed id of the AdamW parameter sets
ADAMW_HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
ADAMW_BYTES_PER_ELEM = 28   # reads p, g, m, v and writes p, m, v (fp32)


def adamw_cpu_baseline(n_params, budget_s):
    """The fp64 oracle AdamW step on a 2^22-element slice of synthetic
    embedding-like data, repeated for about `budget_s` seconds; the rate
    per element holds for the whole set (every element is independent)."""
    import numpy as np

    import oracle
    n = 1 << 22
    p = workloads.host_normal((n,), 0.02, ADAMW_WID, 0, 0, workloads.KIND_W0).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    grads = [workloads.host_normal((n,), 0.01, ADAMW_WID, 0, s, workloads.KIND_G)
             for s in (1, 2)]
    runs, el = 0, 0.0
    while el < budget_s and runs < 10000:
        t1 = time.perf_counter()
        p, m, v = oracle.adamw_step(p, grads[runs % 2], m, v, step=runs + 1, **ADAMW_HP)
        el += time.perf_counter() - t1
        runs += 1
    return {
        "value": n * runs / el,
        "unit": "params/s",
        "cores": 1,
        "kind": "oracle",
        "sample": ("%d fp64 oracle AdamW steps over a %d-element slice (two gradients "
                   "alternating), %.1f s; numpy elementwise, one thread; est. %.2f s per full "
                   "%d-element step" % (runs, n, el, n_params * el / (n * runs), n_params)),
        "host_cpu": host_cpu(),
    }


def bench_adamw(args, mh, torch) -> int:
    """AdamW over a non-matrix parameter set: one grouped launch per step."""
    sizes = workloads.ADAMW_SETS[args.adamw_set]
    n = int(sum(sizes))
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    opt = mh.AdamW(sizes, device=dev)
    print(f"[bench] adamw {args.adamw_set}: {len(sizes)} tensors, {n} params",
          file=sys.stderr, flush=True)
    P = [workloads.device_normal_(torch.empty(k, device=dev), 0.02, ADAMW_WID, i, 0,
                                  workloads.KIND_W0) for i, k in enumerate(sizes)]
    M = [torch.zeros(k, device=dev) for k in sizes]
    V = [torch.zeros(k, device=dev) for k in sizes]
    pool = max(1, min(args.warmup + args.steps, int(96e9 // (4 * n))))
    G = [[workloads.device_normal_(torch.empty(k, device=dev), 0.01, ADAMW_WID, i, p + 1,
                                   workloads.KIND_G) for i, k in enumerate(sizes)]
         for p in range(pool)]
    torch.cuda.synchronize(dev)
    for w in range(args.warmup):
        opt.step(P, G[w % pool], M, V, step=w + 1, **ADAMW_HP)
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps), gradient pool {pool}", file=sys.stderr,
          flush=True)
    events = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in evs:
            e.record()
        events.append(evs)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(args.steps):
        st = args.warmup + s + 1
        events[s][0].record()
        opt.step(P, G[(st - 1) % pool], M, V, step=st, **ADAMW_HP)
        events[s][1].record()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    launches_per_step = -(-len(sizes) // mh.ADAMW_MAX_TENSORS_PER_LAUNCH)
    kern_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    avg_launch_ms = kern_ms / launches_per_step
    bytes_per_launch = ADAMW_BYTES_PER_ELEM * n / launches_per_step
    gbs = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC_ADAMW,
        "value": n * args.steps / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.adamw_set}: token embedding and norm vectors of the "
                               f"28-layer Qwen3-style 2B model",
                   "tensors": len(sizes), "params": n, "update": "adamw", **ADAMW_HP},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": committed_traffic("k_adamw",
                                                  f"adamw_step_{args.adamw_set}_hbm_counters.md",
                                                  "adamw.hip"),
                     "kernel": "k_adamw", "avg_launch_ms": round(avg_launch_ms, 4),
                     "algorithmic_bytes_per_launch": bytes_per_launch},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = adamw_cpu_baseline(n, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_2b", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--ns-iters", type=int, default=None)
    ap.add_argument("--precision", default="bf16", choices=["bf16", "split_bf16", "fp32"],
                    help="Newton-Schulz operands: bf16 (default), split_bf16 (hi + lo bf16 "
                         "pairs, 3 MFMAs per product) or fp32 (debug mode)")
    ap.add_argument("--ns-fp32", action="store_true", help="same as --precision fp32")
    ap.add_argument("--variant", default="muonh", choices=["muonh", "muon_wd", "adamw"],
                    help="muonh (default): the MuonH step; muon_wd: the Muon baseline with "
                         "decoupled weight decay on the same plan; adamw: AdamW over the "
                         "non-matrix parameter set (--adamw-set)")
    ap.add_argument("--adamw-set", default="qwen3_2b_rest", choices=sorted(workloads.ADAMW_SETS))
    ap.add_argument("--grad-dtype", default="fp32", choices=["fp32", "bf16"],
                    help="storage of the gradients G (default fp32)")
    ap.add_argument("--mom-dtype", default="fp32", choices=["fp32", "bf16"],
                    help="storage of the momentum M (default fp32)")
    ap.add_argument("--weight-decay", type=float, default=0.1,
                    help="weight decay of the muon_wd variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-window", type=float, default=3.5,
                    help="seconds of untimed steps after the timed ones over which the clock, "
                         "power and power-limit residency are read (0: none)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.ns_fp32:
        args.precision = "fp32"
    if args.calibrate_copy:
        return calibrate_copy()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this MuonH build runs on one GPU only (no collectives); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2

    import torch

    import orthogonalized_updates_amd as mh
    if not mh.LIB_PATH.exists():
        import __graft_entry__
        __graft_entry__.build()
    if args.variant == "adamw":
        return bench_adamw(args, mh, torch)

    wl = workloads.WORKLOADS[args.workload]
    k = args.ns_iters if args.ns_iters is not None else wl.ns_iters[0]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    opt = mh.MuonH(wl.shapes, precision=args.precision, grad_dtype=args.grad_dtype,
                   mom_dtype=args.mom_dtype, device=dev)
    gdt = torch.bfloat16 if args.grad_dtype == "bf16" else torch.float32
    mdt = torch.bfloat16 if args.mom_dtype == "bf16" else torch.float32
    g_bytes, m_bytes = (2 if args.grad_dtype == "bf16" else 4), (2 if args.mom_dtype == "bf16" else 4)

    print(f"[bench] {wl.name}: {wl.n_matrices} matrices, {wl.n_params} params, k={k}, "
          f"workspace {opt.plan.workspace_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)
    W = [workloads.device_weight_(wl, i, torch.empty(s, device=dev)) for i, s in enumerate(wl.shapes)]
    M = [torch.zeros(s, dtype=mdt, device=dev) for s in wl.shapes]
    # Distinct gradients per step (pool bounded to ~96 GB), generated before
    # timing (in fp32, then converted when G is stored in bf16).
    per_set = g_bytes * wl.n_params
    pool = max(1, min(args.warmup + args.steps, int(96e9 // per_set)))
    G = []
    for p in range(pool):
        G.append([workloads.device_grad_(wl, i, p, torch.empty(s, device=dev)).to(gdt)
                  for i, s in enumerate(wl.shapes)])
    opt.init(W)
    torch.cuda.synchronize(dev)

    for w in range(args.warmup):
        if args.variant == "muon_wd":
            opt.step_muon_wd(W, G[w % pool], M, wl.lr, wl.beta, args.weight_decay, k)
        else:
            opt.step(W, G[w % pool], M, wl.lr, wl.beta, k)
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps), gradient pool {pool}", file=sys.stderr,
          flush=True)

    n_ev = 3 * k + 3
    events = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for e in evs:
            e.record()  # creates the HIP event
        events.append(evs)
    torch.cuda.synchronize(dev)

    t0 = time.perf_counter()
    for s in range(args.steps):
        if args.variant == "muon_wd":
            opt.step_muon_wd(W, G[(args.warmup + s) % pool], M, wl.lr, wl.beta,
                             args.weight_decay, k, events=events[s])
        else:
            opt.step_timed(W, G[(args.warmup + s) % pool], M, wl.lr, wl.beta, k, events[s])
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / args.steps

    # After the timed steps: every matrix still on its sphere (MuonH)
    sphere = None
    if args.variant == "muonh":
        norms = torch.stack([torch.linalg.vector_norm(w.double()) for w in W])
        sphere = float((norms / opt.R.double() - 1.0).abs().max())

    # Clock and power under this load. The firmware refreshes amdsmi's
    # readings about once a second, which the timed steps (under a second by
    # default) do not span, so they are read over untimed steps of the same
    # work run after them, dropping the first POWER_SETTLE_S seconds.
    n_pw = 0
    if args.power_window > 0:
        n_pw = max(1, int(math.ceil(args.power_window / max(elapsed / args.steps, 1e-4))))
    with ClockSampler(settle_s=min(POWER_SETTLE_S, 0.4 * args.power_window)) as clock:
        for s in range(n_pw):
            if args.variant == "muon_wd":
                opt.step_muon_wd(W, G[s % pool], M, wl.lr, wl.beta, args.weight_decay, k)
            else:
                opt.step(W, G[s % pool], M, wl.lr, wl.beta, k)
        torch.cuda.synchronize(dev)

    # Phase durations from the events recorded inside the timed steps.
    pre = post = 0.0
    phase = {"gram": 0.0, "poly": 0.0, "apply": 0.0}
    for evs in events:
        pre += evs[0].elapsed_time(evs[1])
        for it in range(k):
            phase["gram"] += evs[1 + 3 * it].elapsed_time(evs[2 + 3 * it])
            phase["poly"] += evs[2 + 3 * it].elapsed_time(evs[3 + 3 * it])
            phase["apply"] += evs[3 + 3 * it].elapsed_time(evs[4 + 3 * it])
        post += evs[n_ev - 2].elapsed_time(evs[n_ev - 1])
    nst = args.steps
    launches = nst * k
    flops = ns_flops(wl.shapes, k)
    ns_ms = sum(phase.values()) / nst
    ns_tflops = (sum(flops.values()) * k) / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
    fp32 = args.precision == "fp32"
    peak_mfma = PEAK_FP32_MFMA_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    ns_bytes = 2 if args.precision == "bf16" else 4
    pre_b, post_b = elementwise_bytes(wl.n_params, ns_bytes, fused=not fp32 and k >= 1,
                                      variant=args.variant, g_bytes=g_bytes, m_bytes=m_bytes)
    pre_ms, post_ms = pre / nst, post / nst
    dom = max(phase, key=lambda p: phase[p]) if k > 0 else None

    # bf16 operands run the 16x16x32 kernel, split bf16 the 32x32x16 one
    kname = "k_ns_gemm_m16" if args.precision == "bf16" else "k_ns_gemm_bf16"
    if fp32:
        kname = "k_ns_gemm<fp32>"
    kernel_names = {p: f"{kname}<{p.capitalize()}>" for p in ("gram", "poly", "apply")}
    if dom is not None:
        avg_ms = phase[dom] / launches
        achieved = flops[dom] / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": round(achieved / peak_mfma, 4),
                    "traffic": (committed_traffic(kernel_names[dom],
                                                  f"muonh_step_{wl.name}_hbm_counters.md")
                                if args.precision == "bf16" else None),
                    "kernel": kernel_names[dom], "avg_launch_ms": round(avg_ms, 4),
                    "algorithmic_flop_per_launch": flops[dom]}
    else:
        gbs = (pre_b + post_b) / ((pre_ms + post_ms) * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}

    result = {
        "metric": METRIC_MUON_WD if args.variant == "muon_wd" else METRIC,
        "value": wl.n_params * nst / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": nst,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.notes}", "matrices": wl.n_matrices,
                   "params": wl.n_params, "ns_iters": k, "lr": wl.lr, "beta": wl.beta,
                   "master_weights": "fp32", "ns_operands": args.precision,
                   "grad_dtype": args.grad_dtype, "mom_dtype": args.mom_dtype,
                   "update": ("muon_wd (weight_decay=%g)" % args.weight_decay
                              if args.variant == "muon_wd" else "muonh")},
        "roofline": roofline,
        "phases": {
            "ns_ms": round(ns_ms, 4),
            "ns_tflops_algorithmic": round(ns_tflops, 2),
            "ns_frac_of_peak": round(ns_tflops / peak_mfma, 4),
            "gram_ms": round(phase["gram"] / nst, 4), "poly_ms": round(phase["poly"] / nst, 4),
            "apply_ms": round(phase["apply"] / nst, 4),
            "pre_ns_ms": round(pre_ms, 4), "post_ns_ms": round(post_ms, 4),
            "pre_ns_gbs": round(pre_b / (pre_ms * 1e-3) / 1e9, 1) if pre_ms > 0 else None,
            "post_ns_gbs": round(post_b / (post_ms * 1e-3) / 1e9, 1) if post_ms > 0 else None,
            "elementwise_frac_of_hbm": round((pre_b + post_b) / ((pre_ms + post_ms) * 1e-3) / 1e9
                                             / PEAK_HBM_GBS, 4),
        },
        "cpu_baseline": None,
    }
    result["selfcheck"] = {"sphere_max_abs_dev": sphere, "sphere_bar": 1e-5,
                           "matrices": wl.n_matrices}
    result["env"] = {**runtime_versions(), "gfx_clock": clock.summary(),
                     "power": clock.power_summary(),
                     "clock_power_window": f"{n_pw} untimed steps after the timed ones; samples "
                                           f"after the first {min(POWER_SETTLE_S, 0.4 * args.power_window):.1f} s"}
    if not args.no_cpu_baseline:
        # one more GPU step, untimed, whose inputs and results the oracle
        # leg takes for one matrix of each distinct shape
        idx = [ids[0] for _, ids in wl.shape_groups()]
        gs = G[(args.warmup + args.steps) % pool]
        sample = {i: {"w_pre": W[i].cpu().numpy(), "m_pre": M[i].float().cpu().numpy(),
                      "g": gs[i].float().cpu().numpy(), "r": float(opt.R[i])} for i in idx}
        if args.variant == "muon_wd":
            opt.step_muon_wd(W, gs, M, wl.lr, wl.beta, args.weight_decay, k)
        else:
            opt.step(W, gs, M, wl.lr, wl.beta, k)
        torch.cuda.synchronize(dev)
        for i in idx:
            sample[i].update({"o": opt.read_update(i).cpu().numpy(), "w": W[i].cpu().numpy(),
                              "m": M[i].float().cpu().numpy()})
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, k, args.cpu_budget, sample, args.variant,
                                              args.weight_decay, args.mom_dtype == "bf16",
                                              args.precision)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
