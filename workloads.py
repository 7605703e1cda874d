"""Seeded synthetic workloads for the MuonH optimizer step.

This module holds the workload table (matrix shapes, counts, step counts and
input distributions) and the seeded random generators that both the oracle
side (tests, CPU baseline) and the HIP side (tests, bench) draw their inputs
from. It contains none of the optimizer's arithmetic: it only produces weights
and gradients.

The pages describe a Qwen3-configured 2B model trained with MuonH on its
matrix weights (Puro model card, sections "Quickstart" and "Training"), but
publish neither layer shapes nor any optimizer workload. The shapes below are
Qwen3-style stand-ins for that model's per-layer projections; no dataset or
checkpoint is involved anywhere.

Every tensor is keyed by (workload id, matrix index, step, kind) so that any
single matrix can be regenerated on its own:
  kind 0 = initial weights W0, kind 1 = gradient normal draw,
  kind 2 = heavy-tail Bernoulli mask of the gradient.

Host generation uses numpy's PCG64; device generation (for workloads too big to
generate on the host every step) uses torch's seeded device generator. The two
streams are different random numbers with the same distribution; a test that
compares the GPU path with the oracle always hands both sides the very same
arrays.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

SEED_ROOT = 2026

KIND_W0 = 0
KIND_G = 1
KIND_G_MASK = 2


@dataclass(frozen=True)
class Workload:
    """One synthetic optimizer workload: a list of matrix shapes plus the run."""

    wid: int                      # numeric id, part of every seed key
    name: str
    shapes: Tuple[Tuple[int, int], ...]   # one (rows, cols) per matrix, step order
    steps: int
    ns_iters: Tuple[int, ...]     # Newton-Schulz iteration counts exercised
    lr: float = 0.02
    beta: float = 0.95
    w_std: float = 0.02           # W0 ~ N(0, w_std^2)
    g_std: float = 0.01           # G ~ N(0, g_std^2)   (variance 1e-4)
    heavy_tail: bool = False      # G *= (1 + 10 * Bernoulli(0.01))
    notes: str = ""

    @property
    def n_matrices(self) -> int:
        return len(self.shapes)

    @property
    def n_params(self) -> int:
        return int(sum(r * c for r, c in self.shapes))

    def shape_groups(self) -> List[Tuple[Tuple[int, int], List[int]]]:
        """Distinct shapes in order of first appearance, with matrix indices."""
        groups: dict = {}
        for i, s in enumerate(self.shapes):
            groups.setdefault(s, []).append(i)
        return list(groups.items())


def _qwen3_2b_shapes(layers: int = 28) -> Tuple[Tuple[int, int], ...]:
    # Per layer: q, o (2048x2048); k, v (512x2048); gate, up (6144x2048);
    # down (2048x6144). Embeddings are not matrix-group parameters here.
    per_layer = [(2048, 2048), (512, 2048), (512, 2048), (2048, 2048),
                 (6144, 2048), (6144, 2048), (2048, 6144)]
    return tuple(s for _ in range(layers) for s in per_layer)


WORKLOADS = {
    "single_128x256": Workload(
        wid=0, name="single_128x256", shapes=((128, 256),), steps=10,
        ns_iters=(5,), notes="one small matrix; the oracle finishes in well under a second"),
    "single_2048": Workload(
        wid=1, name="single_2048", shapes=((2048, 2048),), steps=20,
        ns_iters=(5,), notes="one attention q/o-projection-shaped matrix"),
    "qwen3_2b": Workload(
        wid=2, name="qwen3_2b", shapes=_qwen3_2b_shapes(), steps=10,
        ns_iters=(5,), notes="28-layer Qwen3-style 2B matrix set, 196 matrices"),
    "occupancy_512x1536": Workload(
        wid=3, name="occupancy_512x1536",
        shapes=tuple([(512, 1536)] * 256 + [(1536, 512)] * 256), steps=10,
        ns_iters=(5,), heavy_tail=True,
        notes="256 wide plus 256 tall matrices (auto-transpose), heavy-tailed gradients"),
    "large_4096x14336": Workload(
        wid=4, name="large_4096x14336",
        shapes=tuple([(4096, 14336)] * 32 + [(14336, 4096)] * 32), steps=5,
        ns_iters=(5, 8), w_std=0.01,
        notes="64 large matrices, MFMA saturation"),
}


def _qwen3_2b_rest() -> tuple:
    """Element counts of the parameters outside the MuonH matrix group of a
    Qwen3-style 2B model, for the AdamW step: a tied token embedding of
    151,936 x 2048, then per layer two RMSNorm scales of 2048 and the q/k
    norms of 128, then the final norm. The pages name a Qwen3 configuration
    but print no vocabulary or norm layout; these sizes stand in for it."""
    sizes = [151936 * 2048]
    for _ in range(28):
        sizes += [2048, 2048, 128, 128]
    sizes.append(2048)
    return tuple(sizes)


# AdamW parameter sets: flat tensor sizes (elements).
ADAMW_SETS = {"qwen3_2b_rest": _qwen3_2b_rest()}


def seed_key(wid: int, mat: int, step: int, kind: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_ROOT, int(wid), int(mat), int(step), int(kind)])


def host_normal(shape: Sequence[int], std: float, wid: int, mat: int, step: int,
                kind: int) -> np.ndarray:
    """fp32 N(0, std^2) array from numpy PCG64 keyed by (wid, mat, step, kind)."""
    rng = np.random.Generator(np.random.PCG64(seed_key(wid, mat, step, kind)))
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    x *= np.float32(std)
    return x


def host_weight(w: Workload, mat: int) -> np.ndarray:
    r, c = w.shapes[mat]
    return host_normal((r, c), w.w_std, w.wid, mat, 0, KIND_W0)


def host_grad(w: Workload, mat: int, step: int) -> np.ndarray:
    r, c = w.shapes[mat]
    g = host_normal((r, c), w.g_std, w.wid, mat, step, KIND_G)
    if w.heavy_tail:
        rng = np.random.Generator(np.random.PCG64(seed_key(w.wid, mat, step, KIND_G_MASK)))
        mask = rng.random((r, c), dtype=np.float32) < np.float32(0.01)
        g *= (np.float32(1.0) + np.float32(10.0) * mask.astype(np.float32))
    return g


def host_custom(shape: Sequence[int], std: float, key: Sequence[int]) -> np.ndarray:
    """fp32 normal array for ad-hoc test cases, keyed by an arbitrary int tuple."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 99, *key])))
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    x *= np.float32(std)
    return x


def _device_seed(wid: int, mat: int, step: int, kind: int) -> int:
    return int(seed_key(wid, mat, step, kind).generate_state(1, dtype=np.uint64)[0] >> 1)


def device_normal_(out, std: float, wid: int, mat: int, step: int, kind: int):
    """Fill a torch device tensor in place with N(0, std^2) from a keyed seed."""
    import torch
    g = torch.Generator(device=out.device)
    g.manual_seed(_device_seed(wid, mat, step, kind))
    out.normal_(0.0, std, generator=g)
    return out


def device_weight_(w: Workload, mat: int, out):
    return device_normal_(out, w.w_std, w.wid, mat, 0, KIND_W0)


def device_grad_(w: Workload, mat: int, step: int, out):
    import torch
    device_normal_(out, w.g_std, w.wid, mat, step, KIND_G)
    if w.heavy_tail:
        g = torch.Generator(device=out.device)
        g.manual_seed(_device_seed(w.wid, mat, step, KIND_G_MASK))
        mask = torch.rand(out.shape, device=out.device, generator=g) < 0.01
        out.mul_(1.0 + 10.0 * mask.to(out.dtype))
    return out
