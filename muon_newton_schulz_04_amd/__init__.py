"""Python binding of the MI355X Muon Newton-Schulz library.

Argument marshalling only: every step of the update runs in the HIP kernels
of ``lib/libmuon_mi355x.so`` (built by ``build.py``); torch supplies device
memory and streams. The names mirror the C ABI in ``include/muon.h``.
There is no CPU fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "LIB_PATH", "MuonError", "MuonMatrix", "MuonConfig", "MuonBufferInfo",
    "KERNEL_NAMES", "load_library", "muon_abi_version", "muon_status_str",
    "muon_workspace_bytes", "muon_plan_create", "muon_plan_step", "muon_plan_destroy",
    "muon_step", "muon_orthogonalize", "muon_schedule_query", "muon_plan_set_timing",
    "muon_plan_kernel_times", "muon_plan_buffer_info", "MuonPlan", "make_config",
    "muon_plan_set_chained", "muon_plan_set_chain_timeout", "muon_plan_chain_state",
    "muon_plan_chain_times",
    "MuonWeight", "MuonApply", "muon_plan_set_weights", "muon_plan_step_apply",
    "muon_plan_step_noalloc", "MUON_SCRATCH_BYTES",
    "MuonAdamTensor", "MuonAdamConfig", "AdamPlan", "muon_adam_plan_create",
    "muon_adam_plan_step", "muon_adam_plan_destroy", "muon_adam_work_items",
    "MUON_F32", "MUON_BF16", "MUON_PRECISION_DEFAULT",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmuon_mi355x.so")
MUON_F32, MUON_BF16 = 0, 1
KERNEL_NAMES = ["momentum", "normalize", "gram", "poly", "update"]
STATUS = ["MUON_OK", "MUON_E_INVALID", "MUON_E_DTYPE", "MUON_E_SHAPE", "MUON_E_ALIGN",
          "MUON_E_WORKSPACE", "MUON_E_DEVICE", "MUON_E_LAUNCH", "MUON_E_ALLOC", "MUON_E_SCRATCH"]
MUON_SCRATCH_BYTES = 128 << 20


class MuonError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS[code] if 0 <= code < len(STATUS) else code} "
                         f"({muon_status_str(code)})")


class MuonMatrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class MuonConfig(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("steps", ctypes.c_int32), ("momentum", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("eps", ctypes.c_float),
                ("precision", ctypes.c_int32)]


class MuonWeight(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("lr_mul", ctypes.c_float), ("wd_mul", ctypes.c_float)]


class MuonApply(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("wd", ctypes.c_float)]


class MuonAdamTensor(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("lr_mul", ctypes.c_float), ("wd_mul", ctypes.c_float)]


class MuonAdamConfig(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("wd", ctypes.c_float), ("step", ctypes.c_int32)]


class MuonBufferInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("m", "n", "mp", "np", "x_lo", "x_op0", "x_op1", "gram", "poly", "x0_scale")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads the HIP library (once). Raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"Muon HIP library not built: {path} missing "
                          "(run python -m muon_newton_schulz_04_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "muon_abi_version": (i32, []),
        "muon_status_str": (ctypes.c_char_p, [i32]),
        "muon_workspace_bytes": (i32, [P(MuonMatrix), i32, i32, P(sz)]),
        "muon_plan_create": (i32, [P(MuonMatrix), i32, i32, P(vp)]),
        "muon_plan_step": (i32, [vp, P(MuonConfig), vp, sz, vp]),
        "muon_plan_step_noalloc": (i32, [vp, P(MuonConfig), vp]),
        "muon_plan_destroy": (None, [vp]),
        "muon_step": (i32, [P(MuonMatrix), i32, i32, P(MuonConfig), vp, sz, vp]),
        "muon_orthogonalize": (i32, [P(MuonMatrix), i32, i32, P(MuonConfig), vp, sz, vp]),
        "muon_schedule_query": (i32, [P(MuonMatrix), i32, i32, i32, P(i32), i64, P(i64)]),
        "muon_plan_set_timing": (i32, [vp, i32]),
        "muon_plan_kernel_times": (i32, [vp, P(ctypes.c_double), P(i64)]),
        "muon_plan_chain_times": (i32, [vp, P(ctypes.c_double), P(i64)]),
        "muon_plan_buffer_info": (i32, [vp, i32, P(MuonBufferInfo)]),
        "muon_plan_set_chained": (i32, [vp, i32]),
        "muon_plan_set_chain_timeout": (i32, [vp, i64]),
        "muon_plan_chain_state": (i32, [vp, P(i32), P(i32)]),
        "muon_plan_set_weights": (i32, [vp, P(MuonWeight), i32]),
        "muon_plan_step_apply": (i32, [vp, P(MuonConfig), P(MuonApply), vp, sz, vp]),
        "muon_adam_plan_create": (i32, [P(MuonAdamTensor), i32, i32, P(vp)]),
        "muon_adam_plan_step": (i32, [vp, P(MuonAdamConfig), vp]),
        "muon_adam_plan_destroy": (None, [vp]),
        "muon_adam_work_items": (i32, [P(MuonAdamTensor), i32, i32, P(i64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        raise MuonError(code, where)


def muon_abi_version() -> int:
    return load_library().muon_abi_version()


def muon_status_str(code: int) -> str:
    return load_library().muon_status_str(int(code)).decode()


# ------------------------------------------------------------ marshalling

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("matrices must be 2-D")
    rows, cols = t.shape
    if rows and cols > 1 and t.stride(1) != 1:
        raise ValueError("matrices must be row-major with unit column stride")
    return t.stride(0) if rows > 1 else cols


def _matrices(grads, momenta, outs):
    """muon_matrix array (and dtype code) from lists of torch tensors."""
    n = len(grads)
    if len(outs) != n or (momenta is not None and len(momenta) != n):
        raise ValueError("grads, momenta and outs must have the same length")
    arr = (MuonMatrix * max(n, 1))()
    dt = None
    for i in range(n):
        g, o = grads[i], outs[i]
        m = None if momenta is None else momenta[i]
        for t in (g, o) + (() if m is None else (m,)):
            d = _dtype_code(t)
            if dt is None:
                dt = d
            elif d != dt:
                raise TypeError("all tensors of a call must share one dtype")
            if t.shape != g.shape:
                raise ValueError("grad, momentum and out must have the same shape")
        ld = _ld(g)
        if _ld(o) != ld or (m is not None and _ld(m) != ld):
            raise ValueError("grad, momentum and out must share one row stride")
        arr[i] = MuonMatrix(g.shape[0], g.shape[1], ld, _ptr(g), _ptr(m), _ptr(o))
    return arr, n, (MUON_BF16 if dt is None else dt)


def _shape_matrices(shapes: Sequence, dtype: int):
    """muon_matrix array for shape-only host queries: distinct, aligned,
    never dereferenced placeholder addresses."""
    n = len(shapes)
    arr = (MuonMatrix * max(n, 1))()
    es = 4 if dtype == MUON_F32 else 2
    base = 1 << 44
    for i, (r, c) in enumerate(shapes):
        span = ((r * c * es) + 4095) // 4096 * 4096 + 4096
        arr[i] = MuonMatrix(r, c, c, base, base + span, base + 2 * span)
        base += 3 * span
    return arr, n


MUON_PRECISION_DEFAULT = 0


def make_config(a: float, b: float, c: float, steps: int, momentum: float = 0.0,
                nesterov: bool = False, eps: float = 1e-7,
                precision: int = MUON_PRECISION_DEFAULT) -> MuonConfig:
    return MuonConfig(a, b, c, int(steps), momentum, 1 if nesterov else 0, eps, int(precision))


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, device, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return workspace


# ---------------------------------------------------------------- entry points

def muon_workspace_bytes(mats, dtype: Optional[int] = None) -> int:
    """Workspace bytes for a list of gradient tensors, or of (rows, cols)
    shapes with ``dtype`` (MUON_BF16 / MUON_F32)."""
    lib = load_library()
    if len(mats) and isinstance(mats[0], (tuple, list)):
        arr, n = _shape_matrices(mats, dtype if dtype is not None else MUON_BF16)
        dt = dtype if dtype is not None else MUON_BF16
    else:
        arr, n, dt = _matrices(mats, None, mats)
    out = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, n, dt, ctypes.byref(out)), "muon_workspace_bytes")
    return out.value


def muon_schedule_query(shapes: Sequence, dtype: int, kind: int) -> np.ndarray:
    """Host-only: the (items, 4) int32 schedule of kernel ``kind``."""
    lib = load_library()
    arr, n = _shape_matrices(shapes, dtype)
    cnt = ctypes.c_int64(0)
    _check(lib.muon_schedule_query(arr, n, dtype, kind, None, 0, ctypes.byref(cnt)),
           "muon_schedule_query")
    buf = np.zeros((max(cnt.value, 1), 4), dtype=np.int32)
    _check(lib.muon_schedule_query(arr, n, dtype, kind,
                                   buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   cnt.value, ctypes.byref(cnt)), "muon_schedule_query")
    return buf[: cnt.value]


class MuonPlan:
    """A plan over fixed tensors (their pointers are baked into the plan)."""

    def __init__(self, grads, momenta, outs):
        lib = load_library()
        self._keep = (list(grads), None if momenta is None else list(momenta), list(outs))
        arr, n, dt = _matrices(grads, momenta, outs)
        self.dtype = dt
        self.n = n
        self.device = grads[0].device if n else None
        h = ctypes.c_void_p(None)
        _check(lib.muon_plan_create(arr, n, dt, ctypes.byref(h)), "muon_plan_create")
        self.handle = h
        ws = ctypes.c_size_t(0)
        _check(lib.muon_workspace_bytes(arr, n, dt, ctypes.byref(ws)), "muon_workspace_bytes")
        self.workspace_bytes = ws.value

    def step(self, cfg: MuonConfig, workspace=None, stream=None):
        ws = _workspace(self.workspace_bytes, self.device, workspace)
        _check(load_library().muon_plan_step(self.handle, ctypes.byref(cfg), ws.data_ptr(),
                                             ws.numel(), _stream_handle(stream)),
               "muon_plan_step")
        return ws

    def step_noalloc(self, cfg: MuonConfig, stream=None):
        """muon_plan_step_noalloc: the same step with the library's fixed
        device scratch array as workspace (no allocation)."""
        _check(load_library().muon_plan_step_noalloc(self.handle, ctypes.byref(cfg),
                                                     _stream_handle(stream)),
               "muon_plan_step_noalloc")

    def set_weights(self, weights, lr_mul=None, wd_mul=None):
        """Attaches one weight tensor per matrix (same shape and dtype as its
        grad, row-major); lr_mul / wd_mul: per-matrix multipliers (default 1)."""
        n = self.n
        if len(weights) != n:
            raise ValueError("one weight per matrix")
        lr_mul = [1.0] * n if lr_mul is None else list(lr_mul)
        wd_mul = [1.0] * n if wd_mul is None else list(wd_mul)
        arr = (MuonWeight * max(n, 1))()
        grads = self._keep[0]
        for i, w in enumerate(weights):
            if w is None:
                arr[i] = MuonWeight(None, 0, lr_mul[i], wd_mul[i])
                continue
            if w.shape != grads[i].shape or _dtype_code(w) != self.dtype:
                raise ValueError("weight must match its grad's shape and dtype")
            arr[i] = MuonWeight(_ptr(w), _ld(w), float(lr_mul[i]), float(wd_mul[i]))
        _check(load_library().muon_plan_set_weights(self.handle, arr, n), "muon_plan_set_weights")
        self._weights = list(weights)

    def step_apply(self, cfg: MuonConfig, lr: float, wd: float, workspace=None, stream=None):
        """One Muon update whose last step writes W <- W (1 - lr wd wd_mul) - lr lr_mul X
        into the attached weights (``out`` is not written)."""
        ws = _workspace(self.workspace_bytes, self.device, workspace)
        ap = MuonApply(float(lr), float(wd))
        _check(load_library().muon_plan_step_apply(self.handle, ctypes.byref(cfg), ctypes.byref(ap),
                                                   ws.data_ptr(), ws.numel(),
                                                   _stream_handle(stream)),
               "muon_plan_step_apply")
        return ws

    def set_timing(self, mode):
        """0 / False: off; 1 / True: each kernel over the whole set in its own
        timed launch; 2: the step's own launches timed as they run."""
        _check(load_library().muon_plan_set_timing(self.handle, int(mode)), "muon_plan_set_timing")

    def chain_times(self):
        """(total ms, launches) of the chained launches timed with mode 2
        since the last read."""
        ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(load_library().muon_plan_chain_times(self.handle, ctypes.byref(ms), ctypes.byref(n)),
               "muon_plan_chain_times")
        return ms.value, n.value

    def kernel_times(self):
        """{kernel name: (total ms, launches)} since timing was enabled / last read."""
        ms = (ctypes.c_double * 5)()
        n = (ctypes.c_int64 * 5)()
        _check(load_library().muon_plan_kernel_times(self.handle, ms, n), "muon_plan_kernel_times")
        return {KERNEL_NAMES[k]: (ms[k], n[k]) for k in range(5)}

    def set_chained(self, on: bool):
        """Use the chained launch where the plan has one (default) or the separate launches."""
        _check(load_library().muon_plan_set_chained(self.handle, 1 if on else 0),
               "muon_plan_set_chained")

    def set_chain_timeout(self, microseconds: int):
        """Bound of one wait of the chained launch (default 2 s)."""
        _check(load_library().muon_plan_set_chain_timeout(self.handle, int(microseconds)),
               "muon_plan_set_chain_timeout")

    def chain_state(self):
        """(chained, error): whether steps use the chained launch, and the plan's error
        word since the last query (0: none; waits for the device, clears the word)."""
        c, e = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(load_library().muon_plan_chain_state(self.handle, ctypes.byref(c), ctypes.byref(e)),
               "muon_plan_chain_state")
        return int(c.value), int(e.value)

    def buffer_info(self, idx: int) -> dict:
        info = MuonBufferInfo()
        _check(load_library().muon_plan_buffer_info(self.handle, idx, ctypes.byref(info)),
               "muon_plan_buffer_info")
        return {f: getattr(info, f) for f, _ in MuonBufferInfo._fields_}

    def destroy(self):
        if self.handle:
            load_library().muon_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def muon_plan_create(grads, momenta, outs) -> MuonPlan:
    return MuonPlan(grads, momenta, outs)


def muon_plan_step(plan: MuonPlan, cfg: MuonConfig, workspace=None, stream=None):
    return plan.step(cfg, workspace, stream)


def muon_plan_destroy(plan: MuonPlan):
    plan.destroy()


def muon_plan_set_weights(plan: MuonPlan, weights, lr_mul=None, wd_mul=None):
    plan.set_weights(weights, lr_mul, wd_mul)


def muon_plan_step_apply(plan: MuonPlan, cfg: MuonConfig, lr: float, wd: float, workspace=None,
                         stream=None):
    return plan.step_apply(cfg, lr, wd, workspace, stream)


def muon_plan_step_noalloc(plan: MuonPlan, cfg: MuonConfig, stream=None):
    return plan.step_noalloc(cfg, stream)


def muon_plan_set_timing(plan: MuonPlan, mode):
    plan.set_timing(mode)


def muon_plan_chain_times(plan: MuonPlan):
    return plan.chain_times()


def muon_plan_kernel_times(plan: MuonPlan):
    return plan.kernel_times()


def muon_plan_set_chained(plan: MuonPlan, on: bool):
    plan.set_chained(on)


def muon_plan_set_chain_timeout(plan: MuonPlan, microseconds: int):
    plan.set_chain_timeout(microseconds)


def muon_plan_chain_state(plan: MuonPlan):
    return plan.chain_state()


def muon_plan_buffer_info(plan: MuonPlan, idx: int) -> dict:
    return plan.buffer_info(idx)


def muon_step(grads: List, momenta: Optional[List], outs: List, cfg: MuonConfig,
              workspace=None, stream=None):
    """One Muon update of every matrix (plan cached by the library)."""
    lib = load_library()
    arr, n, dt = _matrices(grads, momenta, outs)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, n, dt, ctypes.byref(ws_bytes)), "muon_workspace_bytes")
    ws = _workspace(ws_bytes.value, grads[0].device if n else "cuda", workspace)
    _check(lib.muon_step(arr, n, dt, ctypes.byref(cfg), ws.data_ptr(), ws.numel(),
                         _stream_handle(stream)), "muon_step")
    return ws


def muon_orthogonalize(grads: List, outs: List, cfg: MuonConfig, workspace=None, stream=None):
    """Normalise + Newton-Schulz only (no momentum state)."""
    lib = load_library()
    arr, n, dt = _matrices(grads, None, outs)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.muon_workspace_bytes(arr, n, dt, ctypes.byref(ws_bytes)), "muon_workspace_bytes")
    ws = _workspace(ws_bytes.value, grads[0].device if n else "cuda", workspace)
    _check(lib.muon_orthogonalize(arr, n, dt, ctypes.byref(cfg), ws.data_ptr(), ws.numel(),
                                  _stream_handle(stream)), "muon_orthogonalize")
    return ws


# ------------------------------------------------------------------ Adam branch

def _adam_tensors(params, grads, exp_avgs, exp_avg_sqs, lr_mul=None, wd_mul=None):
    """muon_adam_tensor array (and dtype code) from lists of torch tensors
    (each contiguous; moments float32)."""
    import torch
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads and the two moment lists must have the same length")
    lr_mul = [1.0] * n if lr_mul is None else list(lr_mul)
    wd_mul = [1.0] * n if wd_mul is None else list(wd_mul)
    arr = (MuonAdamTensor * max(n, 1))()
    dt = None
    for i in range(n):
        p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        for t in (p, g, m, v):
            if not t.is_contiguous():
                raise ValueError("Adam tensors must be contiguous")
            if t.numel() != p.numel():
                raise ValueError("param, grad and moments must have the same element count")
        if m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError("Adam moments are float32")
        d = _dtype_code(p)
        if _dtype_code(g) != d:
            raise TypeError("param and grad must share one dtype")
        if dt is None:
            dt = d
        elif d != dt:
            raise TypeError("all parameters of a call must share one dtype")
        arr[i] = MuonAdamTensor(p.numel(), _ptr(p), _ptr(g), _ptr(m), _ptr(v),
                                float(lr_mul[i]), float(wd_mul[i]))
    return arr, n, (MUON_BF16 if dt is None else dt)


def muon_adam_work_items(params, grads, exp_avgs, exp_avg_sqs) -> int:
    arr, n, dt = _adam_tensors(params, grads, exp_avgs, exp_avg_sqs)
    out = ctypes.c_int64(0)
    _check(load_library().muon_adam_work_items(arr, n, dt, ctypes.byref(out)), "muon_adam_work_items")
    return out.value


class AdamPlan:
    """Adam over a fixed list of tensors (pointers baked into the plan)."""

    def __init__(self, params, grads, exp_avgs, exp_avg_sqs, lr_mul=None, wd_mul=None):
        lib = load_library()
        self._keep = (list(params), list(grads), list(exp_avgs), list(exp_avg_sqs))
        arr, n, dt = _adam_tensors(params, grads, exp_avgs, exp_avg_sqs, lr_mul, wd_mul)
        self.dtype = dt
        h = ctypes.c_void_p(None)
        _check(lib.muon_adam_plan_create(arr, n, dt, ctypes.byref(h)), "muon_adam_plan_create")
        self.handle = h

    def step(self, lr: float, beta1: float, beta2: float, eps: float, wd: float, step: int,
             stream=None):
        cfg = MuonAdamConfig(float(lr), float(beta1), float(beta2), float(eps), float(wd), int(step))
        _check(load_library().muon_adam_plan_step(self.handle, ctypes.byref(cfg),
                                                  _stream_handle(stream)), "muon_adam_plan_step")

    def destroy(self):
        if self.handle:
            load_library().muon_adam_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def muon_adam_plan_create(params, grads, exp_avgs, exp_avg_sqs, lr_mul=None, wd_mul=None):
    return AdamPlan(params, grads, exp_avgs, exp_avg_sqs, lr_mul, wd_mul)


def muon_adam_plan_step(plan: AdamPlan, lr, beta1, beta2, eps, wd, step, stream=None):
    plan.step(lr, beta1, beta2, eps, wd, step, stream)


def muon_adam_plan_destroy(plan: AdamPlan):
    plan.destroy()
