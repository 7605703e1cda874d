"""MI355X (gfx950) MuonH optimizer step: Python binding of libmuonh.so.

The binding only marshals arguments: it groups matrices by shape, builds the
device arrays of device pointers the C ABI takes (include/muonh.h), allocates
the workspace with torch and passes torch's current HIP stream. Every step of
the optimizer runs in the library's HIP kernels. There is no fallback: if the
library is missing, the first call into it raises ImportError.

MuonH (digest page "Puro-2B trains for $6.9K, attention sinks hit 99%,
LoopArena tops at 24.69%", section "The load-bearing tricks aren't in the
abstract"; model card "Puro", section "Training"): momentum, Newton-Schulz
orthogonalization, then projection of every weight matrix back onto the
sphere of its initial Frobenius norm, with no weight decay.

MuonH(shapes, precision=..., grad_dtype=..., mom_dtype=...) runs the step
(step, step_timed) and, on the same plan, the Muon baseline with decoupled
weight decay (step_muon_wd); AdamW(numels) updates the parameters outside
the matrix group. Gradients and momenta may be float32 or bfloat16 tensors
(grad_dtype / mom_dtype); weights are float32.
"""
from __future__ import annotations

import ctypes
import re
from collections import OrderedDict
from pathlib import Path
from typing import Dict, List, Optional, Sequence, Tuple

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libmuonh.so"
HEADER_PATH = _PKG.parent / "include" / "muonh.h"

MUONH_OK = 0
MUONH_EINVAL = -1
MUONH_ESHAPE = -2
MUONH_EWORKSPACE = -3
MUONH_EHIP = -4
MUONH_ENOMEM = -5
MUONH_EALIAS = -6
MUONH_NS_FP32 = 1
MUONH_NS_SPLIT_BF16 = 2
MUONH_GRAD_BF16 = 4
MUONH_MOM_BF16 = 8
MUONH_NONFINITE_MOMENTUM = 1
MUONH_NONFINITE_UPDATE = 2
# Bytes of muonh_step_noalloc's fixed per-GPU workspace (include/muonh.h).
MUONH_NOALLOC_WORKSPACE_BYTES = 128 << 20

# Newton-Schulz operand precision -> plan flag
PRECISIONS = {"bf16": 0, "split_bf16": MUONH_NS_SPLIT_BF16, "fp32": MUONH_NS_FP32}
# Storage dtype of the gradient / momentum -> whether it takes the bf16 flag
STATE_DTYPES = ("fp32", "bf16")

# Tensors per grouped AdamW launch (the library splits larger lists).
ADAMW_MAX_TENSORS_PER_LAUNCH = 128

NS_COEFFS = (3.4445, -4.7750, 2.0315)


class MuonHError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"muonh error {status}: {message}")
        self.status = status


class MuonHAliasError(MuonHError, ValueError):
    """MUONH_EALIAS: two of the W, G, M tensors overlap in memory."""

    def __init__(self, message: str):
        super().__init__(MUONH_EALIAS, message)


# Device pointer arrays kept per pointer tuple (a least-recently-used cache):
# a training loop that cycles through a few gradient buffers uploads each
# array once.
PTR_CACHE_ENTRIES = 64


class GroupDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("count", ctypes.c_int32)]


def _load_library() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m orthogonalized_updates_amd.build` "
            "(the MuonH step has no non-HIP implementation)")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_float)
    sig = {
        "muonh_abi_version": (i32, []),
        "muonh_plan_create": (ctypes.c_int, [ctypes.POINTER(vp), ctypes.POINTER(GroupDesc), i32,
                                             ctypes.c_uint32]),
        "muonh_plan_destroy": (None, [vp]),
        "muonh_plan_num_matrices": (i64, [vp]),
        "muonh_plan_num_params": (i64, [vp]),
        "muonh_workspace_bytes": (sz, [vp]),
        "muonh_init": (ctypes.c_int, [vp, vp, vp, vp, sz, vp]),
        "muonh_step": (ctypes.c_int, [vp, vp, vp, vp, vp, f32, f32, i32, vp, sz, vp]),
        "muonh_step_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, f32, f32, i32, vp]),
        "muonh_step_timed": (ctypes.c_int, [vp, vp, vp, vp, vp, f32, f32, i32, vp, sz, vp,
                                            ctypes.POINTER(vp), i32]),
        "muonh_step_muon_wd": (ctypes.c_int, [vp, vp, vp, vp, f32, f32, f32, i32, vp, sz, vp]),
        "muonh_step_muon_wd_timed": (ctypes.c_int, [vp, vp, vp, vp, f32, f32, f32, i32, vp, sz,
                                                    vp, ctypes.POINTER(vp), i32]),
        "muonh_read_update": (ctypes.c_int, [vp, i64, vp, vp, sz, vp]),
        "muonh_adamw_step": (ctypes.c_int, [i32, vp, vp, vp, vp, vp, f32, f32, f32, f32, f32,
                                            i32, vp]),
        "muonh_step_status": (ctypes.c_int, [vp, vp, sz, vp, ctypes.POINTER(ctypes.c_uint32)]),
        "muonh_check_disjoint": (ctypes.c_int, [vp, vp, vp, vp]),
        "muonh_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "muonh_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB: Optional[ctypes.CDLL] = None


def get_lib() -> ctypes.CDLL:
    """The loaded libmuonh.so (loaded on first use; ImportError if not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load_library()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return get_lib()
    raise AttributeError(name)


def check(status: int) -> None:
    if status != MUONH_OK:
        lib = get_lib()
        raise MuonHError(status, lib.muonh_last_error().decode(errors="replace")
                         or lib.muonh_status_string(status).decode())


def _precision(precision: str, ns_fp32: bool) -> str:
    if ns_fp32:
        if precision not in ("bf16", "fp32"):
            raise ValueError("ns_fp32=True conflicts with precision=%r" % (precision,))
        precision = "fp32"
    if precision not in PRECISIONS:
        raise ValueError("precision must be one of %s, got %r" % (sorted(PRECISIONS), precision))
    return precision


class Plan:
    """Owns a muonh_plan for shape groups [(rows, cols, count), ...].

    precision: Newton-Schulz operand precision, "bf16" (default),
    "split_bf16" (hi + lo bf16 pairs, three bf16 products each) or "fp32";
    ns_fp32=True is the same as precision="fp32". grad_dtype / mom_dtype:
    storage of G and M, "fp32" (default) or "bf16".
    """

    def __init__(self, groups: Sequence[Tuple[int, int, int]], ns_fp32: bool = False,
                 precision: str = "bf16", grad_dtype: str = "fp32", mom_dtype: str = "fp32"):
        precision = _precision(precision, ns_fp32)
        for name, v in (("grad_dtype", grad_dtype), ("mom_dtype", mom_dtype)):
            if v not in STATE_DTYPES:
                raise ValueError(f"{name} must be one of {STATE_DTYPES}, got {v!r}")
        flags = (PRECISIONS[precision] | (MUONH_GRAD_BF16 if grad_dtype == "bf16" else 0)
                 | (MUONH_MOM_BF16 if mom_dtype == "bf16" else 0))
        arr = (GroupDesc * len(groups))(*[GroupDesc(int(r), int(c), int(n)) for r, c, n in groups])
        handle = ctypes.c_void_p()
        check(get_lib().muonh_plan_create(ctypes.byref(handle), arr, len(groups), flags))
        self.handle = handle
        self.groups = [tuple(int(v) for v in g) for g in groups]
        self.precision = precision
        self.ns_fp32 = precision == "fp32"
        self.grad_dtype = grad_dtype
        self.mom_dtype = mom_dtype

    @property
    def num_matrices(self) -> int:
        return int(get_lib().muonh_plan_num_matrices(self.handle))

    @property
    def num_params(self) -> int:
        return int(get_lib().muonh_plan_num_params(self.handle))

    @property
    def workspace_bytes(self) -> int:
        return int(get_lib().muonh_workspace_bytes(self.handle))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.muonh_plan_destroy(h)
            self.handle = None


class _PtrArrays:
    """Device arrays of device pointers, one per pointer tuple, kept in a
    least-recently-used cache of PTR_CACHE_ENTRIES. A new array is copied
    from pinned host memory without blocking (the copy is ordered on the
    current stream before the launch that reads it; torch keeps the pinned
    buffer until the copy is done), so changing pointers never waits for
    the GPU. Each use records the current stream on the array, so that an
    array evicted while a launch on another stream still reads it is not
    reused before that launch completes."""

    def __init__(self, torch, device):
        self.torch = torch
        self.device = device
        self.cache: "OrderedDict" = OrderedDict()

    def get(self, ptrs: Tuple[int, ...]) -> int:
        torch = self.torch
        arr = self.cache.get(ptrs)
        if arr is None:
            host = torch.tensor(ptrs, dtype=torch.int64).pin_memory()
            arr = host.to(self.device, non_blocking=True)
            self.cache[ptrs] = arr
            if len(self.cache) > PTR_CACHE_ENTRIES:
                self.cache.popitem(last=False)
        else:
            self.cache.move_to_end(ptrs)
        arr.record_stream(torch.cuda.current_stream(self.device))
        return int(arr.data_ptr())


class MuonH:
    """MuonH over a list of fp32 weight matrices on one GPU.

    shapes: (rows, cols) of each matrix, in the caller's order. Matrices are
    grouped by shape internally; every method takes and returns lists in the
    caller's order. grad_dtype / mom_dtype ("fp32" or "bf16"): the torch
    dtype the gradients / momenta must have (float32 or bfloat16).
    """

    def __init__(self, shapes: Sequence[Tuple[int, int]], *, ns_fp32: bool = False,
                 precision: str = "bf16", grad_dtype: str = "fp32", mom_dtype: str = "fp32",
                 device=None):
        import torch
        get_lib()
        self.torch = torch
        self.shapes = [(int(r), int(c)) for r, c in shapes]
        if not self.shapes:
            raise ValueError("MuonH needs at least one matrix")
        dev = torch.device(device if device is not None else "cuda")
        if dev.type != "cuda":
            raise ValueError("MuonH runs on a ROCm GPU device only")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        buckets: Dict[Tuple[int, int], List[int]] = {}
        for i, s in enumerate(self.shapes):
            buckets.setdefault(s, []).append(i)
        self.plan_order: List[int] = [i for idx in buckets.values() for i in idx]
        self.plan_index = {caller: p for p, caller in enumerate(self.plan_order)}
        self.plan = Plan([(r, c, len(idx)) for (r, c), idx in buckets.items()], ns_fp32=ns_fp32,
                         precision=precision, grad_dtype=grad_dtype, mom_dtype=mom_dtype)
        tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}
        self._dtypes = {"weights": torch.float32, "grads": tdt[grad_dtype],
                        "moms": tdt[mom_dtype]}
        nbytes = max(self.plan.workspace_bytes, 256)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        if self.workspace.data_ptr() % 256:
            raise MuonHError(MUONH_EWORKSPACE, "torch returned a workspace that is not 256-aligned")
        self.R = torch.zeros(len(self.shapes), dtype=torch.float32, device=self.device)
        self._ptrs = _PtrArrays(torch, self.device)
        self._disjoint_ok: "OrderedDict" = OrderedDict()  # (W, G, M) pointer tuples checked

    # -- marshalling ------------------------------------------------------
    def _check(self, tensors, name: str):
        torch = self.torch
        if len(tensors) != len(self.shapes):
            raise ValueError(f"{name}: expected {len(self.shapes)} tensors, got {len(tensors)}")
        dt = self._dtypes[name]
        for i, t in enumerate(tensors):
            if not isinstance(t, torch.Tensor) or t.dtype != dt:
                raise TypeError(f"{name}[{i}] must be a {dt} torch tensor")
            if t.device != self.device:
                raise ValueError(f"{name}[{i}] is on {t.device}, expected {self.device}")
            if tuple(t.shape) != self.shapes[i] or not t.is_contiguous():
                raise ValueError(f"{name}[{i}] must be a contiguous {self.shapes[i]} tensor")

    def _check_state(self, weights, grads, moms):
        """Types and shapes of W, G and M, and that no two of their tensors
        overlap in memory (the step updates W and M in place and reads G).
        The library checks the byte ranges on the host
        (muonh_check_disjoint), once per combination of pointers; an overlap
        raises MuonHAliasError (a ValueError) naming the caller's tensors."""
        self._check(weights, "weights")
        self._check(grads, "grads")
        self._check(moms, "moms")
        ptrs = [tuple(int(ts[c].data_ptr()) for c in self.plan_order)
                for ts in (weights, grads, moms)]
        key = tuple(ptrs)
        if key in self._disjoint_ok:
            self._disjoint_ok.move_to_end(key)
            return
        arrs = [(ctypes.c_void_p * len(p))(*p) for p in ptrs]
        st = get_lib().muonh_check_disjoint(self.plan.handle, *arrs)
        if st == MUONH_EALIAS:
            raise MuonHAliasError(self._caller_names(get_lib().muonh_last_error().decode()))
        check(st)
        self._disjoint_ok[key] = True
        if len(self._disjoint_ok) > PTR_CACHE_ENTRIES:
            self._disjoint_ok.popitem(last=False)

    def _caller_names(self, msg: str) -> str:
        """The library names matrices by plan index ("G[3] overlaps W[3]");
        translate to the caller's lists and indices."""
        names = {"W": "weights", "G": "grads", "M": "moms"}

        def repl(m):
            return f"{names[m.group(1)]}[{self.plan_order[int(m.group(2))]}]"
        return re.sub(r"\b([WGM])\[(\d+)\]", repl, msg) + "; W, G and M must be disjoint"

    def _ptr_array(self, name: str, tensors) -> int:
        return self._ptrs.get(tuple(int(tensors[c].data_ptr()) for c in self.plan_order))

    def _stream(self) -> int:
        return int(self.torch.cuda.current_stream(self.device).cuda_stream)

    # -- API ----------------------------------------------------------------
    def init(self, weights) -> "object":
        """R[i] = ||W0[i]||_F (device float32, caller order)."""
        self._check(weights, "weights")
        r_plan = self.torch.empty_like(self.R)
        check(get_lib().muonh_init(self.plan.handle, self._ptr_array("W", weights), r_plan.data_ptr(),
                             self.workspace.data_ptr(), self.workspace.numel(), self._stream()))
        inv = self.torch.tensor(self.plan_order, dtype=self.torch.int64, device=self.device)
        self.R = self.torch.empty_like(r_plan).index_copy_(0, inv, r_plan)
        self._R_plan = r_plan
        return self.R

    def set_radius(self, radius) -> None:
        """Restore R (caller order), e.g. from a checkpoint."""
        r = radius.to(device=self.device, dtype=self.torch.float32).contiguous()
        if r.numel() != len(self.shapes):
            raise ValueError("radius must have one entry per matrix")
        self.R = r
        inv = self.torch.tensor(self.plan_order, dtype=self.torch.int64, device=self.device)
        self._R_plan = r.index_select(0, inv)

    def step(self, weights, grads, moms, lr: float, beta: float = 0.95, ns_iters: int = 5) -> None:
        """One MuonH step: moms and weights are updated in place."""
        self._check_state(weights, grads, moms)
        if not hasattr(self, "_R_plan"):
            raise RuntimeError("call init() (or set_radius()) before step()")
        check(get_lib().muonh_step(self.plan.handle, self._ptr_array("W", weights),
                             self._ptr_array("G", grads), self._ptr_array("M", moms),
                             self._R_plan.data_ptr(), float(lr), float(beta), int(ns_iters),
                             self.workspace.data_ptr(), self.workspace.numel(), self._stream()))

    def step_noalloc(self, weights, grads, moms, lr: float, beta: float = 0.95,
                     ns_iters: int = 5) -> None:
        """step() without this object's workspace (muonh_step_noalloc): the
        library's fixed per-GPU array of MUONH_NOALLOC_WORKSPACE_BYTES serves
        instead, for plans that fit it. read_update() and status() do not
        see such a step. The pointer arrays are still device tensors of this
        object (uploaded once per pointer combination)."""
        self._check_state(weights, grads, moms)
        if not hasattr(self, "_R_plan"):
            raise RuntimeError("call init() (or set_radius()) before step_noalloc()")
        check(get_lib().muonh_step_noalloc(self.plan.handle, self._ptr_array("W", weights),
                                           self._ptr_array("G", grads),
                                           self._ptr_array("M", moms), self._R_plan.data_ptr(),
                                           float(lr), float(beta), int(ns_iters),
                                           self._stream()))

    def step_timed(self, weights, grads, moms, lr: float, beta: float, ns_iters: int,
                   events) -> None:
        """step() plus hipEventRecord of `events` (torch.cuda.Event list of
        length 3*ns_iters+3, already recorded once) at the phase boundaries."""
        self._check_state(weights, grads, moms)
        if not hasattr(self, "_R_plan"):
            raise RuntimeError("call init() (or set_radius()) before step_timed()")
        arr = (ctypes.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
        check(get_lib().muonh_step_timed(self.plan.handle, self._ptr_array("W", weights),
                                   self._ptr_array("G", grads), self._ptr_array("M", moms),
                                   self._R_plan.data_ptr(), float(lr), float(beta), int(ns_iters),
                                   self.workspace.data_ptr(), self.workspace.numel(),
                                   self._stream(), arr, len(events)))

    def step_muon_wd(self, weights, grads, moms, lr: float, beta: float = 0.95,
                     weight_decay: float = 0.1, ns_iters: int = 5, events=None) -> None:
        """The baseline MuonH is measured against: Muon with decoupled weight
        decay, W <- (1 - lr*wd) W - lr O (no projection, no radius). With
        `events` (as for step_timed), records the phase boundaries."""
        self._check_state(weights, grads, moms)
        args = [self.plan.handle, self._ptr_array("W", weights), self._ptr_array("G", grads),
                self._ptr_array("M", moms), float(lr), float(beta), float(weight_decay),
                int(ns_iters), self.workspace.data_ptr(), self.workspace.numel(), self._stream()]
        if events is None:
            check(get_lib().muonh_step_muon_wd(*args))
        else:
            arr = (ctypes.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
            check(get_lib().muonh_step_muon_wd_timed(*args, arr, len(events)))

    def read_update(self, index: int):
        """The update O of matrix `index` from the last step (fp32, rows x cols)."""
        r, c = self.shapes[index]
        out = self.torch.empty((r, c), dtype=self.torch.float32, device=self.device)
        check(get_lib().muonh_read_update(self.plan.handle, self.plan_index[index], out.data_ptr(),
                                    self.workspace.data_ptr(), self.workspace.numel(),
                                    self._stream()))
        return out

    def status(self) -> int:
        """Non-finite bits of the last step (MUONH_NONFINITE_MOMENTUM: a
        momentum norm was NaN or infinite; MUONH_NONFINITE_UPDATE: a trial
        update norm was). Waits for the current stream."""
        flags = ctypes.c_uint32(0)
        check(get_lib().muonh_step_status(self.plan.handle, self.workspace.data_ptr(),
                                          self.workspace.numel(), self._stream(),
                                          ctypes.byref(flags)))
        return int(flags.value)


__all__ = ["MuonH", "Plan", "MuonHError", "GroupDesc", "get_lib", "check", "LIB_PATH", "HEADER_PATH",
           "NS_COEFFS", "MUONH_OK", "MUONH_EINVAL", "MUONH_ESHAPE", "MUONH_EWORKSPACE",
           "MUONH_EHIP", "MUONH_ENOMEM", "MUONH_EALIAS", "MuonHAliasError", "MUONH_NS_FP32", "MUONH_NS_SPLIT_BF16", "MUONH_GRAD_BF16",
           "MUONH_MOM_BF16", "MUONH_NONFINITE_MOMENTUM", "MUONH_NONFINITE_UPDATE",
           "MUONH_NOALLOC_WORKSPACE_BYTES", "AdamW",
           "PTR_CACHE_ENTRIES"]


class AdamW:
    """AdamW over a list of fp32 tensors on one GPU: the parameters outside
    the MuonH group (model card page "Puro", section "Training": AdamW with
    weight decay 0.1). Any shapes; tensors are treated as flat arrays and
    updated in place by the library's grouped HIP launch (muonh_adamw_step).
    """

    def __init__(self, numels: Sequence[int], *, device=None):
        import torch
        get_lib()
        self.torch = torch
        self.numels = [int(n) for n in numels]
        if any(n < 0 for n in self.numels):
            raise ValueError("numels must be >= 0")
        dev = torch.device(device if device is not None else "cuda")
        if dev.type != "cuda":
            raise ValueError("AdamW runs on a ROCm GPU device only")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self._sizes = (ctypes.c_int64 * max(len(self.numels), 1))(*self.numels)
        self._ptrs = _PtrArrays(torch, self.device)

    def _check(self, tensors, name: str):
        torch = self.torch
        if len(tensors) != len(self.numels):
            raise ValueError(f"{name}: expected {len(self.numels)} tensors, got {len(tensors)}")
        for i, t in enumerate(tensors):
            if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
                raise TypeError(f"{name}[{i}] must be a float32 torch tensor")
            if t.device != self.device:
                raise ValueError(f"{name}[{i}] is on {t.device}, expected {self.device}")
            if t.numel() != self.numels[i] or not t.is_contiguous():
                raise ValueError(f"{name}[{i}] must be contiguous with {self.numels[i]} elements")

    def _ptr_array(self, name: str, tensors) -> int:
        return self._ptrs.get(tuple(int(t.data_ptr()) for t in tensors))

    def step(self, params, grads, exp_avg, exp_avg_sq, lr: float, beta1: float = 0.9,
             beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.1,
             step: int = 1) -> None:
        """One AdamW step (1-based `step`); params, exp_avg, exp_avg_sq in place."""
        for ts, nm in ((params, "params"), (grads, "grads"), (exp_avg, "exp_avg"),
                       (exp_avg_sq, "exp_avg_sq")):
            self._check(ts, nm)
        if not self.numels:
            return
        stream = int(self.torch.cuda.current_stream(self.device).cuda_stream)
        check(get_lib().muonh_adamw_step(
            len(self.numels), ctypes.cast(self._sizes, ctypes.c_void_p),
            self._ptr_array("P", params), self._ptr_array("G", grads),
            self._ptr_array("M", exp_avg), self._ptr_array("V", exp_avg_sq),
            float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step),
            stream))
