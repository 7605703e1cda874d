"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and its plan and validation logic behaves as documented.
No call here reaches a HIP runtime function (every case is rejected, or is a
host-only plan query, before any device work is enqueued)."""
from __future__ import annotations

import ctypes
import re

import pytest

import orthogonalized_updates_amd as mh


def header_functions():
    text = mh.HEADER_PATH.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(muonh_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("muonh_plan_create", "muonh_plan_destroy", "muonh_workspace_bytes", "muonh_init",
              "muonh_step", "muonh_step_timed", "muonh_step_muon_wd", "muonh_step_muon_wd_timed",
              "muonh_read_update", "muonh_step_status", "muonh_last_error",
              "muonh_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(mh.LIB_PATH))
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, f"symbols declared in muonh.h but not exported: {missing}"


def test_abi_version():
    assert mh.lib.muonh_abi_version() == 3


def _create(groups, flags=0):
    arr = (mh.GroupDesc * max(len(groups), 1))(*[mh.GroupDesc(*g) for g in groups])
    h = ctypes.c_void_p()
    st = mh.lib.muonh_plan_create(ctypes.byref(h), arr, len(groups), flags)
    return st, h


@pytest.mark.parametrize("groups,flags,code", [
    ([], 0, mh.MUONH_EINVAL),                      # no groups (empty input)
    ([(4, 4, 1)], 0x10, mh.MUONH_EINVAL),          # unknown flag
    ([(4, 4, 1)], mh.MUONH_NS_FP32 | mh.MUONH_NS_SPLIT_BF16, mh.MUONH_EINVAL),  # two precisions
    ([(0, 4, 1)], 0, mh.MUONH_ESHAPE),             # zero rows
    ([(4, -1, 1)], 0, mh.MUONH_ESHAPE),            # negative cols
    ([(4, 4, 0)], 0, mh.MUONH_ESHAPE),             # empty group
    ([(65537, 4, 1)], 0, mh.MUONH_ESHAPE),         # beyond the max dimension
    ([(65536, 65536, 2048)], 0, mh.MUONH_ESHAPE),  # 2^31 cast tiles: past 32-bit block indices
])
def test_plan_create_rejects(groups, flags, code):
    st, h = _create(groups, flags)
    assert st == code
    assert h.value is None
    assert mh.lib.muonh_last_error().decode()


def test_plan_create_null_arguments():
    assert mh.lib.muonh_plan_create(None, None, 1, 0) == mh.MUONH_EINVAL
    h = ctypes.c_void_p()
    assert mh.lib.muonh_plan_create(ctypes.byref(h), None, 1, 0) == mh.MUONH_EINVAL


def test_plan_counts_and_workspace_growth():
    p = mh.Plan([(2048, 2048, 56), (512, 2048, 56), (6144, 2048, 56), (2048, 6144, 28)])
    assert p.num_matrices == 196
    assert p.num_params == 1_350_565_888
    # bf16 operands: two X buffers (s x l), A and B (s x s) per matrix, padded to 256
    ws = p.workspace_bytes
    ns = 56 * 2 * (2 * 2048 * 2048 + 2 * 2048 * 2048) + 56 * 2 * (2 * 512 * 2048 + 2 * 512 * 512) \
        + 84 * 2 * (2 * 2048 * 6144 + 2 * 2048 * 2048)
    assert ns <= ws <= ns + 196 * (256 * 8 + 16) + 4096
    shapes = [(2048, 2048, 56), (512, 2048, 56), (6144, 2048, 56), (2048, 6144, 28)]
    # fp32 debug: X, two X^T copies, A and B, 4 bytes each
    p32 = mh.Plan(shapes, ns_fp32=True)
    ns32 = 56 * 4 * (3 * 2048 * 2048 + 2 * 2048 * 2048) + 56 * 4 * (3 * 512 * 2048 + 2 * 512 * 512) \
        + 84 * 4 * (3 * 2048 * 6144 + 2 * 2048 * 2048)
    assert ns32 <= p32.workspace_bytes <= ns32 + 196 * (256 * 8 + 16) + 4096
    # split bf16: a hi and a lo value per element, so twice the operand bytes
    psp = mh.Plan(shapes, precision="split_bf16")
    assert 2 * ns <= psp.workspace_bytes <= 2 * ns + 196 * (256 * 8 + 16) + 4096
    assert psp.precision == "split_bf16" and p32.precision == "fp32" and p.precision == "bf16"


def test_binding_rejects_unknown_precision():
    with pytest.raises(ValueError):
        mh.Plan([(4, 4, 1)], precision="fp16")
    with pytest.raises(ValueError):
        mh.Plan([(4, 4, 1)], ns_fp32=True, precision="split_bf16")


@pytest.mark.parametrize("flags", [mh.MUONH_GRAD_BF16, mh.MUONH_MOM_BF16,
                                   mh.MUONH_GRAD_BF16 | mh.MUONH_MOM_BF16 | mh.MUONH_NS_SPLIT_BF16,
                                   mh.MUONH_MOM_BF16 | mh.MUONH_NS_FP32])
def test_plan_accepts_state_storage_flags(flags):
    st, h = _create([(4, 4, 1)], flags)
    assert st == mh.MUONH_OK and h.value
    # the storage of G and M does not change the workspace
    ref = mh.Plan([(4, 4, 1)], precision="fp32" if flags & mh.MUONH_NS_FP32 else
                  "split_bf16" if flags & mh.MUONH_NS_SPLIT_BF16 else "bf16")
    assert mh.lib.muonh_workspace_bytes(h) == ref.workspace_bytes
    mh.lib.muonh_plan_destroy(h)


def test_binding_rejects_unknown_state_dtype():
    with pytest.raises(ValueError):
        mh.Plan([(4, 4, 1)], grad_dtype="fp16")
    with pytest.raises(ValueError):
        mh.Plan([(4, 4, 1)], mom_dtype="float32")
    p = mh.Plan([(4, 4, 1)], grad_dtype="bf16", mom_dtype="bf16")
    assert (p.grad_dtype, p.mom_dtype) == ("bf16", "bf16")


def test_plan_padding_of_ragged_shapes():
    p = mh.Plan([(1, 1, 1)])
    # one 256x256 block per operand buffer (2 X, A, B) in bf16
    assert 4 * 256 * 256 * 2 <= p.workspace_bytes <= 4 * 256 * 256 * 2 + 256 * 8 + 4096
    assert p.num_params == 1


class _FakeDev:
    """Non-null addresses that the library must never dereference: every call
    below fails argument validation first."""
    ptr = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    misaligned = ctypes.c_void_p(0x100010)


@pytest.mark.parametrize("lr,beta,iters,code", [
    (float("nan"), 0.95, 5, mh.MUONH_EINVAL),
    (-0.1, 0.95, 5, mh.MUONH_EINVAL),
    (float("inf"), 0.95, 5, mh.MUONH_EINVAL),
    (0.02, 1.0, 5, mh.MUONH_EINVAL),
    (0.02, -0.5, 5, mh.MUONH_EINVAL),
    (0.02, float("nan"), 5, mh.MUONH_EINVAL),
    (0.02, 0.95, -1, mh.MUONH_EINVAL),
    (0.02, 0.95, 33, mh.MUONH_EINVAL),
])
def test_step_rejects_bad_scalars(lr, beta, iters, code):
    p = mh.Plan([(8, 8, 1)])
    f = _FakeDev
    st = mh.lib.muonh_step(p.handle, f.ptr, f.ptr, f.ptr, f.ptr, lr, beta, iters, f.ws,
                           p.workspace_bytes, None)
    assert st == code


@pytest.mark.parametrize("wd,lr,code", [
    (-0.1, 0.02, mh.MUONH_EINVAL),
    (float("nan"), 0.02, mh.MUONH_EINVAL),
    (float("inf"), 0.02, mh.MUONH_EINVAL),
    (0.1, float("nan"), mh.MUONH_EINVAL),
])
def test_muon_wd_step_rejects_bad_scalars(wd, lr, code):
    p = mh.Plan([(8, 8, 1)])
    f = _FakeDev
    st = mh.lib.muonh_step_muon_wd(p.handle, f.ptr, f.ptr, f.ptr, lr, 0.95, wd, 5, f.ws,
                                   p.workspace_bytes, None)
    assert st == code
    assert "weight_decay" in mh.lib.muonh_last_error().decode() or lr != lr


def test_muon_wd_step_rejects_null_arrays_and_events():
    p = mh.Plan([(8, 8, 1)])
    f = _FakeDev
    n = p.workspace_bytes
    assert mh.lib.muonh_step_muon_wd(None, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 0.1, 5, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step_muon_wd(p.handle, f.ptr, None, f.ptr, 0.02, 0.9, 0.1, 5, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step_muon_wd(p.handle, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 0.1, 5, f.ws, n - 1, None) == mh.MUONH_EWORKSPACE
    assert mh.lib.muonh_step_muon_wd_timed(p.handle, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 0.1, 5, f.ws, n, None,
                                           None, 18) == mh.MUONH_EINVAL
    ev = (ctypes.c_void_p * 4)(*([0x1000] * 4))
    assert mh.lib.muonh_step_muon_wd_timed(p.handle, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 0.1, 5, f.ws, n, None,
                                           ev, 4) == mh.MUONH_EINVAL  # needs 3*5+3 events


def test_step_rejects_null_and_workspace_problems():
    p = mh.Plan([(8, 8, 1)])
    f = _FakeDev
    n = p.workspace_bytes
    assert mh.lib.muonh_step(None, f.ptr, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 5, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step(p.handle, None, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 5, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step(p.handle, f.ptr, f.ptr, f.ptr, None, 0.02, 0.9, 5, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step(p.handle, f.ptr, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 5, None, n, None) == mh.MUONH_EWORKSPACE
    assert mh.lib.muonh_step(p.handle, f.ptr, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 5, f.misaligned, n, None) == mh.MUONH_EWORKSPACE
    assert mh.lib.muonh_step(p.handle, f.ptr, f.ptr, f.ptr, f.ptr, 0.02, 0.9, 5, f.ws, n - 1, None) == mh.MUONH_EWORKSPACE
    assert "needs" in mh.lib.muonh_last_error().decode()


def test_init_and_read_update_validation():
    p = mh.Plan([(8, 8, 2)])
    f = _FakeDev
    n = p.workspace_bytes
    assert mh.lib.muonh_init(p.handle, None, f.ptr, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_init(p.handle, f.ptr, None, f.ws, n, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_init(p.handle, f.ptr, f.ptr, f.ws, 0, None) == mh.MUONH_EWORKSPACE
    assert mh.lib.muonh_read_update(p.handle, 2, f.ptr, f.ws, n, None) == mh.MUONH_ESHAPE
    assert mh.lib.muonh_read_update(p.handle, -1, f.ptr, f.ws, n, None) == mh.MUONH_ESHAPE
    assert mh.lib.muonh_read_update(p.handle, 0, None, f.ws, n, None) == mh.MUONH_EINVAL


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert mh.lib.muonh_status_string(code)
    assert mh.lib.muonh_status_string(7) == b"unknown status"


# ----------------------------------------------------------------------------
# muonh_adamw_step argument validation (nothing is dereferenced)
# ----------------------------------------------------------------------------

def _adamw_call(n=1, sizes=(8,), lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, step=1, arrays=True):
    f = _FakeDev
    sz = (ctypes.c_int64 * max(len(sizes), 1))(*sizes) if sizes is not None else None
    a = f.ptr if arrays else None
    return mh.lib.muonh_adamw_step(n, ctypes.cast(sz, ctypes.c_void_p) if sz is not None else None,
                                   a, a, a, a, lr, b1, b2, eps, wd, step, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), mh.MUONH_EINVAL),
    (dict(sizes=None), mh.MUONH_EINVAL),
    (dict(arrays=False), mh.MUONH_EINVAL),
    (dict(lr=float("nan")), mh.MUONH_EINVAL),
    (dict(lr=-1e-3), mh.MUONH_EINVAL),
    (dict(b1=1.0), mh.MUONH_EINVAL),
    (dict(b2=-0.1), mh.MUONH_EINVAL),
    (dict(eps=float("nan")), mh.MUONH_EINVAL),
    (dict(eps=-1.0), mh.MUONH_EINVAL),
    (dict(wd=float("inf")), mh.MUONH_EINVAL),
    (dict(step=0), mh.MUONH_EINVAL),
    (dict(sizes=(-5,)), mh.MUONH_ESHAPE),
    (dict(sizes=((1 << 40) + 1,)), mh.MUONH_ESHAPE),
])
def test_adamw_rejects_bad_arguments(kw, code):
    assert _adamw_call(**kw) == code
    assert mh.lib.muonh_last_error().decode()


def test_adamw_zero_tensors_is_a_no_op():
    assert mh.lib.muonh_adamw_step(0, None, None, None, None, None, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1,
                                   None) == mh.MUONH_OK


def test_step_status_rejects_before_any_device_work():
    # NULL flags, NULL plan and a workspace that is too small: all host checks
    p = mh.Plan([(256, 256, 1)])
    flags = ctypes.c_uint32(7)
    assert mh.lib.muonh_step_status(p.handle, None, 0, None, None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step_status(None, None, 0, None, ctypes.byref(flags)) == mh.MUONH_EINVAL
    st = mh.lib.muonh_step_status(p.handle, ctypes.c_void_p(256), 16, None, ctypes.byref(flags))
    assert st == mh.MUONH_EWORKSPACE
    assert flags.value == 7  # untouched on error
    assert mh.lib.muonh_last_error().decode()


def _disjoint(plan, W, G, M):
    arrs = [(ctypes.c_void_p * len(x))(*x) for x in (W, G, M)]
    return mh.lib.muonh_check_disjoint(plan.handle, *arrs)


def test_check_disjoint_host_only():
    # fake device addresses: the check only compares byte ranges, nothing is
    # dereferenced. Plan order: two 4x8 fp32 matrices, then one 3x5.
    p = mh.Plan([(4, 8, 2), (3, 5, 1)])
    n = [4 * 8 * 4, 4 * 8 * 4, 3 * 5 * 4]   # fp32 bytes per matrix
    base = 1 << 20

    def packed(start):
        out, at = [], start
        for b in n:
            out.append(at)
            at += b
        return out
    W, G, M = packed(base), packed(2 * base), packed(3 * base)
    assert _disjoint(p, W, G, M) == mh.MUONH_OK          # adjacent, touching only
    assert _disjoint(p, W, W, M) == mh.MUONH_EALIAS      # G is W
    assert "overlaps" in mh.lib.muonh_last_error().decode()
    M2 = list(M)
    M2[1] = M[0] + 64                                    # two momenta share bytes
    assert _disjoint(p, W, G, M2) == mh.MUONH_EALIAS
    msg = mh.lib.muonh_last_error().decode()
    assert "M[1]" in msg and "M[0]" in msg
    W2 = list(W)
    W2[2] = G[0] + n[0] - 4                              # last 4 bytes of G[0]
    assert _disjoint(p, W2, G, M) == mh.MUONH_EALIAS
    W3 = list(W)
    W3[2] = G[0] - n[2]                                  # ends exactly where G[0] starts
    assert _disjoint(p, W3, G, M) == mh.MUONH_OK
    # containment: a small span inside a large one that is not its neighbour
    big = mh.Plan([(64, 64, 1), (1, 4, 2)])
    Wb = [base, 2 * base, 3 * base]
    Gb = [base + 1024, 4 * base, 5 * base]               # G[0] starts inside W[0]
    Mb = [6 * base, 7 * base, 8 * base]
    assert _disjoint(big, Wb, Gb, Mb) == mh.MUONH_EALIAS
    assert mh.lib.muonh_check_disjoint(None, None, None, None) == mh.MUONH_EINVAL


def test_check_disjoint_bf16_state_sizes():
    # with bf16 G and M a matrix spans 2 bytes per entry, so spans that
    # would overlap in fp32 are disjoint
    p = mh.Plan([(4, 8, 2)], grad_dtype="bf16", mom_dtype="bf16")
    W = [1 << 20, (1 << 20) + 128]
    G = [2 << 20, (2 << 20) + 64]
    M = [3 << 20, (3 << 20) + 64]
    assert _disjoint(p, W, G, M) == mh.MUONH_OK
    p32 = mh.Plan([(4, 8, 2)])
    assert _disjoint(p32, W, G, M) == mh.MUONH_EALIAS


def test_noalloc_rejects_plans_beyond_its_array():
    # the size check runs before any HIP call: fake, never dereferenced
    # pointers are enough
    big = mh.Plan([(4096, 14336, 1)])
    assert big.workspace_bytes > mh.MUONH_NOALLOC_WORKSPACE_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = mh.lib.muonh_step_noalloc(big.handle, fake, fake, fake, fake, 0.02, 0.95, 5, None)
    assert st == mh.MUONH_EWORKSPACE
    assert "MUONH_NOALLOC_WORKSPACE_BYTES" in mh.lib.muonh_last_error().decode()
    # argument errors are reported first, as for muonh_step
    assert mh.lib.muonh_step_noalloc(big.handle, None, fake, fake, fake, 0.02, 0.95, 5,
                                     None) == mh.MUONH_EINVAL
    assert mh.lib.muonh_step_noalloc(big.handle, fake, fake, fake, fake, 0.02, 1.5, 5,
                                     None) == mh.MUONH_EINVAL
