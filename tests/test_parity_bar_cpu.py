"""The test tooling's memoised oracle step (tests/parity_bar.py) against the
oracle's own one-call step: equal bit for bit, a repeated momentum served
from the memo, a changed one recomputed, and the memo held to its size cap."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import parity_bar


@pytest.fixture
def memo_everything(monkeypatch):
    monkeypatch.setattr(parity_bar, "NS_MEMO_MIN_ENTRIES", 0)
    monkeypatch.setattr(parity_bar, "_ns_memo", type(parity_bar._ns_memo)())
    return parity_bar


def inputs(shape, seed, bf16=False):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(shape).astype(np.float32) * 0.02
    g = rng.standard_normal(shape).astype(np.float32) * 0.01
    m = rng.standard_normal(shape).astype(np.float32) * 0.01
    if bf16:
        # values a bf16 momentum and gradient can hold (low 16 bits clear)
        g = (g.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        m = (m.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return w, g, m, float(np.linalg.norm(w.astype(np.float64)))


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32)])
@pytest.mark.parametrize("mom_bf16", [False, True])
def test_memoised_step_equals_oracle_step(memo_everything, shape, mom_bf16):
    w, g, m, r = inputs(shape, 7, bf16=mom_bf16)
    ref = oracle.muonh_step(w, g, m, r, 0.02, 0.95, 5, mom_bf16=mom_bf16)
    for _ in range(2):  # the second call is served from the memo
        got = memo_everything.oracle_muonh_step(w, g, m, r, 0.02, 0.95, 5, mom_bf16=mom_bf16)
        for a, b in zip(got, ref):
            assert a.shape == b.shape and np.array_equal(a, b)
    assert len(memo_everything._ns_memo) == 1


def test_memo_keys_on_momentum_bytes_and_iterations(memo_everything):
    w, g, m, r = inputs((16, 48), 3)
    m_new = oracle.momentum_update(m, g, 0.9)
    o5 = memo_everything.oracle_newton_schulz(m_new, 5)
    assert memo_everything.oracle_newton_schulz(m_new.copy(), 5) is o5
    assert not o5.flags.writeable
    o8 = memo_everything.oracle_newton_schulz(m_new, 8)
    assert np.array_equal(o8, oracle.newton_schulz(m_new, 8)) and not np.array_equal(o8, o5)
    m2 = m_new.copy()
    m2[3, 7] = np.nextafter(m2[3, 7], np.inf)  # one ulp in one entry
    o2 = memo_everything.oracle_newton_schulz(m2, 5)
    assert o2 is not o5 and np.array_equal(o2, oracle.newton_schulz(m2, 5))
    assert len(memo_everything._ns_memo) == 3


def test_memo_stays_under_its_byte_cap(memo_everything, monkeypatch):
    shape = (16, 32)
    one = 16 * 32 * 8
    monkeypatch.setattr(memo_everything, "NS_MEMO_MAX_BYTES", 3 * one)
    keep = []
    for seed in range(6):
        w, g, m, r = inputs(shape, 100 + seed)
        keep.append(oracle.momentum_update(m, g, 0.95))
        memo_everything.oracle_newton_schulz(keep[-1], 5)
    assert len(memo_everything._ns_memo) == 3
    assert sum(v.nbytes for v in memo_everything._ns_memo.values()) <= 3 * one
    # the newest entries are the ones kept
    o_last = memo_everything.oracle_newton_schulz(keep[-1], 5)
    assert len(memo_everything._ns_memo) == 3 and np.array_equal(o_last, oracle.newton_schulz(keep[-1], 5))


def test_small_matrices_are_not_memoised():
    w, g, m, r = inputs((8, 8), 1)
    before = len(parity_bar._ns_memo)
    parity_bar.oracle_muonh_step(w, g, m, r, 0.02, 0.95, 5)
    assert len(parity_bar._ns_memo) == before
