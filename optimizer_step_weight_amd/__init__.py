"""Python binding of libforge.so, the fused weight-gradient + optimizer step for MI355X.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  Tensors are PyTorch device tensors (PyTorch provides device memory and the
stream); they are passed to the C ABI as raw pointers and sizes.  If the library is not
built, or was built from other sources than the ones beside it, every call raises: there is
no fallback path.  Tensors must be CUDA tensors on the current device; scale tensors must be
fp32 with the element count their tensor's format names (the library cannot see allocation
sizes, so a short buffer would be read out of bounds).

Entry points (same names as the C ABI in include/forge.h, without the ``forge_`` prefix):
    wgrad_step, dgrad, linear_backward_step, wgrad_gemm, optimizer_step,
    step_scalars, device_check, version, build_id, status_string, last_error
"""
from __future__ import annotations

import ctypes
import os
from typing import Any, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libforge.so")

OPT = {"adamw": 0, "nadam": 1, "radam": 2, "lion": 3, "rmsprop": 4, "adagrad": 5, "sgd": 6, "sgd_momentum": 7}
F32, BF16, FP8_E4M3, I8_B64, U8_B64, I8DYN_B64, U8DYN_B64 = 0, 1, 2, 3, 4, 5, 6
STATUS = {0: "FORGE_OK", 1: "FORGE_ERR_ARG", 2: "FORGE_ERR_SHAPE", 3: "FORGE_ERR_DTYPE", 4: "FORGE_ERR_LAYOUT",
          5: "FORGE_ERR_ALIAS", 6: "FORGE_ERR_DEVICE", 7: "FORGE_ERR_LAUNCH"}
SCALARS = ("decay", "l2", "c1", "c2", "c3", "b1", "omb1", "b2", "omb2", "eps", "lr", "rectified")


class ForgeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64), ("scale", ctypes.c_void_p)]


class Hyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("wd_mode", ctypes.c_int32),
                ("momentum", ctypes.c_float), ("alpha", ctypes.c_float), ("momentum_decay", ctypes.c_float)]


class StepOpts(ctypes.Structure):
    _fields_ = [("w_preround_out", ctypes.c_void_p), ("sr_enable", ctypes.c_int32)]


_P = ctypes.POINTER
_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(or python -m optimizer_step_weight_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        T, H, O = _P(Tensor), _P(Hyper), _P(StepOpts)
        st, i32, i64, u64, vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        L.forge_wgrad_step.argtypes = [T, T, T, T, T, H, i32, i64, u64, O, vp]
        L.forge_dgrad.argtypes = [T, T, T, vp]
        L.forge_linear_backward_step.argtypes = [T, T, T, T, T, T, H, i32, i64, u64, O, vp]
        L.forge_linear_backward_step_fused.argtypes = [T, T, T, T, T, T, H, i32, i64, u64, O, vp, i64, vp]
        L.forge_linear_backward_step_fused_noalloc.argtypes = [T, T, T, T, T, T, H, i32, i64, u64, O, vp]
        L.forge_backward_workspace_bytes.argtypes = [i64]
        L.forge_backward_workspace_bytes.restype = i64
        L.forge_wgrad_gemm.argtypes = [T, T, T, vp]
        L.forge_optimizer_step.argtypes = [T, T, T, T, H, i32, i64, u64, O, vp]
        L.forge_step_scalars.argtypes = [i32, H, i64, _P(ctypes.c_float), i32]
        L.forge_status_string.argtypes = [st]
        L.forge_status_string.restype = ctypes.c_char_p
        L.forge_last_error.restype = ctypes.c_char_p
        L.forge_version.restype = i32
        L.forge_build_id.restype = ctypes.c_char_p
        L.forge_clock_sample.argtypes = [ctypes.c_double, vp, vp]
        L.forge_clock_sample.restype = st
        L.forge_realtime_hz.restype = ctypes.c_double
        L.forge_device_check.argtypes = [i32]
        for f in ("forge_wgrad_step", "forge_dgrad", "forge_linear_backward_step", "forge_linear_backward_step_fused",
                  "forge_linear_backward_step_fused_noalloc", "forge_wgrad_gemm", "forge_optimizer_step",
                  "forge_step_scalars", "forge_device_check"):
            getattr(L, f).restype = st
        from . import _build
        built, want = L.forge_build_id().decode(), _build.source_hash()
        if built != want:
            raise ImportError(f"{LIB_PATH} was built from other sources (build id {built}, sources {want}); "
                              "rebuild it with __graft_entry__.build()")
        _lib_handle = L
    return _lib_handle


def _check(status: int):
    if status != 0:
        raise ForgeError(status, _lib().forge_last_error().decode())


def _dtype_code(t, dyn: bool = False) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    if t.dtype == torch.int8:
        return I8DYN_B64 if dyn else I8_B64
    if t.dtype == torch.uint8:
        return U8DYN_B64 if dyn else U8_B64
    raise TypeError(f"unsupported dtype {t.dtype}")


def _on_device(t, what: str):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor (got a {t.device} tensor)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def _scale_count(code: int, rows: int, cols: int) -> Optional[int]:
    """Element count of the scale buffer a format needs (None: the format has no scale)."""
    if code == FP8_E4M3:
        return 1
    if code in (I8_B64, U8_B64, I8DYN_B64, U8DYN_B64):
        return rows * cols // 64
    return None


def _tensor(t, scale=None, dyn: bool = False) -> Optional[Tensor]:
    import torch
    if t is None:
        return None
    if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise ValueError("tensors must be 2-D with unit column stride")
    code = _dtype_code(t, dyn)
    want = _scale_count(code, t.shape[0], t.shape[1])
    if scale is not None:
        if want is None:
            raise ValueError(f"a {t.dtype} tensor takes no scale")
        if scale.dtype != torch.float32 or not scale.is_contiguous() or scale.numel() != want:
            raise ValueError(f"the scale of a {t.dtype} [{t.shape[0]}, {t.shape[1]}] tensor must be a contiguous "
                             f"float32 tensor of {want} elements (got {scale.dtype}, {scale.numel()})")
        _on_device(scale, "scale")
    _on_device(t, "tensor")
    return Tensor(t.data_ptr(), code, t.shape[0], t.shape[1], t.stride(0) if t.numel() > 0 else t.shape[1],
                  None if scale is None else scale.data_ptr())


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _hyper(h: Any) -> Hyper:
    get = (lambda k, d: h.get(k, d)) if isinstance(h, dict) else (lambda k, d: getattr(h, k, d))
    return Hyper(get("lr", 1e-3), get("beta1", 0.9), get("beta2", 0.999), get("eps", 1e-8),
                 get("weight_decay", 0.0), int(get("wd_mode", 0)), get("momentum", 0.9), get("alpha", 0.99),
                 get("momentum_decay", 0.004))


def _opt(opt) -> int:
    return OPT[opt] if isinstance(opt, str) else int(opt)


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _opts(w_preround_out, sr, W):
    if w_preround_out is None and sr:
        return None
    if w_preround_out is not None:
        import torch
        _on_device(w_preround_out, "w_preround_out")
        if (w_preround_out.dtype != torch.float32 or not w_preround_out.is_contiguous()
                or w_preround_out.numel() != W.numel()):
            raise ValueError("w_preround_out must be a contiguous float32 tensor with one element per weight")
    return StepOpts(None if w_preround_out is None else w_preround_out.data_ptr(), 1 if sr else 0)


def _dyn(state_map: str) -> bool:
    if state_map not in ("linear", "dynamic"):
        raise ValueError(f"state_map must be 'linear' or 'dynamic' (got {state_map!r})")
    return state_map == "dynamic"


def wgrad_step(X, dY, W, m=None, v=None, *, opt="adamw", hyper=None, step: int, seed: int,
               x_scale=None, dy_scale=None, m_scale=None, v_scale=None, w_preround_out=None, sr=True,
               state_map="linear", stream=None):
    """Fused step: W, m, v updated in place from g = dY^T X (forge_wgrad_step).  8-bit moments
    (int8 m, uint8 v with block scales) use the linear absmax map, or the dynamic map with
    state_map="dynamic"."""
    o = _opts(w_preround_out, sr, W)
    dyn = _dyn(state_map)
    _check(_lib().forge_wgrad_step(_ref(_tensor(X, x_scale)), _ref(_tensor(dY, dy_scale)), _ref(_tensor(W)),
                                   _ref(_tensor(m, m_scale, dyn)), _ref(_tensor(v, v_scale, dyn)),
                                   ctypes.byref(_hyper(hyper)), _opt(opt), int(step), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                   _ref(o), _stream(stream)))


def dgrad(dY, W, dX, *, stream=None):
    """dX = dY W with the weight as it is now (forge_dgrad)."""
    _check(_lib().forge_dgrad(_ref(_tensor(dY)), _ref(_tensor(W)), _ref(_tensor(dX)), _stream(stream)))


def linear_backward_step(X, dY, W, dX, m=None, v=None, *, opt="adamw", hyper=None, step: int, seed: int,
                         m_scale=None, v_scale=None, w_preround_out=None, sr=True, state_map="linear", stream=None):
    """dgrad then the fused step, in that order (forge_linear_backward_step)."""
    o = _opts(w_preround_out, sr, W)
    dyn = _dyn(state_map)
    _check(_lib().forge_linear_backward_step(
        _ref(_tensor(X)), _ref(_tensor(dY)), _ref(_tensor(W)), _ref(_tensor(dX)), _ref(_tensor(m, m_scale, dyn)),
        _ref(_tensor(v, v_scale, dyn)), ctypes.byref(_hyper(hyper)), _opt(opt), int(step),
        int(seed) & 0xFFFFFFFFFFFFFFFF, _ref(o), _stream(stream)))


def backward_workspace_bytes(K: int) -> int:
    """Workspace bytes linear_backward_step_fused needs for a weight of K columns."""
    return int(_lib().forge_backward_workspace_bytes(int(K)))


def linear_backward_step_fused(X, dY, W, dX, m=None, v=None, *, opt="adamw", hyper=None, step: int, seed: int,
                               m_scale=None, v_scale=None, w_preround_out=None, sr=True, state_map="linear",
                               workspace=None, stream=None):
    """dgrad and the fused step in one launch (forge_linear_backward_step_fused).  `workspace` is a
    device tensor of at least backward_workspace_bytes(K) bytes; one is allocated when it is None.
    Returns the workspace (its int32 word 1 is nonzero if a wait hit its bound)."""
    import torch
    o = _opts(w_preround_out, sr, W)
    dyn = _dyn(state_map)
    if workspace is None:
        workspace = torch.empty(backward_workspace_bytes(W.shape[1]) // 4, dtype=torch.int32, device=W.device)
    _on_device(workspace, "workspace")
    _check(_lib().forge_linear_backward_step_fused(
        _ref(_tensor(X)), _ref(_tensor(dY)), _ref(_tensor(W)), _ref(_tensor(dX)), _ref(_tensor(m, m_scale, dyn)),
        _ref(_tensor(v, v_scale, dyn)), ctypes.byref(_hyper(hyper)), _opt(opt), int(step),
        int(seed) & 0xFFFFFFFFFFFFFFFF, _ref(o), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return workspace


def linear_backward_step_fused_noalloc(X, dY, W, dX, m=None, v=None, *, opt="adamw", hyper=None, step: int,
                                       seed: int, m_scale=None, v_scale=None, w_preround_out=None, sr=True,
                                       state_map="linear", stream=None):
    """linear_backward_step_fused with the library's own counters: allocates nothing
    (forge_linear_backward_step_fused_noalloc).  Calls on one device must not overlap."""
    o = _opts(w_preround_out, sr, W)
    dyn = _dyn(state_map)
    _check(_lib().forge_linear_backward_step_fused_noalloc(
        _ref(_tensor(X)), _ref(_tensor(dY)), _ref(_tensor(W)), _ref(_tensor(dX)), _ref(_tensor(m, m_scale, dyn)),
        _ref(_tensor(v, v_scale, dyn)), ctypes.byref(_hyper(hyper)), _opt(opt), int(step),
        int(seed) & 0xFFFFFFFFFFFFFFFF, _ref(o), _stream(stream)))


def wgrad_gemm(X, dY, dW, *, x_scale=None, dy_scale=None, stream=None):
    """Unfused phase 1: dW = dY^T X written to the fp32 buffer dW (forge_wgrad_gemm)."""
    _check(_lib().forge_wgrad_gemm(_ref(_tensor(X, x_scale)), _ref(_tensor(dY, dy_scale)), _ref(_tensor(dW)),
                                   _stream(stream)))


def optimizer_step(dW, W, m=None, v=None, *, opt="adamw", hyper=None, step: int, seed: int, m_scale=None,
                   v_scale=None, w_preround_out=None, sr=True, state_map="linear", stream=None):
    """Unfused phase 2: the rule applied to a materialised gradient (forge_optimizer_step)."""
    o = _opts(w_preround_out, sr, W)
    dyn = _dyn(state_map)
    _check(_lib().forge_optimizer_step(_ref(_tensor(dW)), _ref(_tensor(W)), _ref(_tensor(m, m_scale, dyn)),
                                       _ref(_tensor(v, v_scale, dyn)), ctypes.byref(_hyper(hyper)), _opt(opt),
                                       int(step), int(seed) & 0xFFFFFFFFFFFFFFFF, _ref(o), _stream(stream)))


def step_scalars(opt, hyper, step: int) -> dict:
    """Per-step scalars the kernels receive (host only)."""
    out = (ctypes.c_float * len(SCALARS))()
    _check(_lib().forge_step_scalars(_opt(opt), ctypes.byref(_hyper(hyper)), int(step), out, len(SCALARS)))
    return dict(zip(SCALARS, list(out)))


def device_check(device: int = 0) -> None:
    _check(_lib().forge_device_check(int(device)))


def version() -> int:
    return int(_lib().forge_version())


def build_id() -> str:
    return _lib().forge_build_id().decode()


def clock_sample(seconds: float, out, *, stream=None) -> None:
    """Measurement helper (include/forge_measure.h): one wave on `stream` writes the shader-clock
    cycles and real-time ticks of a `seconds`-long interval to `out` (2 x int64, device)."""
    _on_device(out, "out")
    if out.numel() < 2 or out.element_size() != 8 or not out.is_contiguous():
        raise ValueError("out must be a contiguous 64-bit tensor of at least 2 elements")
    _check(_lib().forge_clock_sample(float(seconds), out.data_ptr(), _stream(stream)))


def realtime_hz() -> float:
    return float(_lib().forge_realtime_hz())


def status_string(status: int) -> str:
    return _lib().forge_status_string(int(status)).decode()


def last_error() -> str:
    return _lib().forge_last_error().decode()


# the C ABI names
forge_wgrad_step = wgrad_step
forge_dgrad = dgrad
forge_linear_backward_step = linear_backward_step
forge_wgrad_gemm = wgrad_gemm
forge_optimizer_step = optimizer_step
forge_step_scalars = step_scalars
forge_device_check = device_check
forge_version = version
forge_build_id = build_id
forge_status_string = status_string
forge_last_error = last_error
