"""ctypes binding of libforge.so; argument marshalling only.

Each Python function has the name of the C entry point it calls and takes
torch tensors: bf16 X / dY, float32 W and optimizer state, all contiguous on
the current HIP device. Sizes are read off the tensors; the library validates
everything else and its status code is raised as ForgeError.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(PKG, "libforge.so")

FORGE_TILE_DEFAULT = 0
FORGE_TILE_256x128 = 1
FORGE_TILE_128x128 = 2
FORGE_TILE_256x256 = 3
FORGE_TILE_PERSISTENT = 4

FORGE_F32 = 0
FORGE_BF16 = 1
FORGE_FP8_E4M3 = 2
FORGE_FP8_E5M2 = 3

STATUS = {
    0: "FORGE_OK", 1: "FORGE_ERR_NULL", 2: "FORGE_ERR_SHAPE", 3: "FORGE_ERR_ALIGN",
    4: "FORGE_ERR_ALIAS", 5: "FORGE_ERR_HPARAM", 6: "FORGE_ERR_CLIP_NOT_FUSABLE",
    7: "FORGE_ERR_TILE", 8: "FORGE_ERR_DEVICE", 9: "FORGE_ERR_LAUNCH", 10: "FORGE_ERR_DTYPE",
}

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class AdamWParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", _i64),
                ("max_grad_norm", ctypes.c_double)]


class SgdmParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("max_grad_norm", ctypes.c_double)]


class ForgeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        self.name = STATUS.get(self.status, str(status))
        super().__init__(f"{where}: {self.name} ({forge_status_string(self.status)})")


_LIB = None


def library() -> ctypes.CDLL:
    """The loaded libforge.so. Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m weight_gradient_gemm_amd.build` (needs hipcc)")
        lib = ctypes.CDLL(library_path)
        lib.forge_wgrad_adamw.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                          ctypes.POINTER(AdamWParams), _i32, _vp]
        lib.forge_wgrad_sgdm.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                         ctypes.POINTER(SgdmParams), _i32, _vp]
        lib.forge_wgrad.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]
        lib.forge_adamw.argtypes = [_vp, _vp, _vp, _vp, _i64, ctypes.POINTER(AdamWParams), _vp]
        lib.forge_sgdm.argtypes = [_vp, _vp, _vp, _i64, ctypes.POINTER(SgdmParams), _vp]
        lib.forge_grouped_wgrad_adamw.argtypes = [_vp, _vp, ctypes.POINTER(_i64), _i32, _vp, _vp,
                                                  _vp, _i64, _i64, ctypes.POINTER(AdamWParams),
                                                  _i32, _vp]
        lib.forge_wgrad_bf16.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]
        lib.forge_wgrad_adamw_bf16state.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                                    ctypes.POINTER(AdamWParams), _i32, _vp]
        lib.forge_adamw_mixed.argtypes = [_vp, _i32, _vp, _vp, _vp, _i32, _i64,
                                          ctypes.POINTER(AdamWParams), _vp]
        lib.forge_dgrad.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp]
        lib.forge_linear_backward_adamw.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64,
                                                    _i64, _i64, ctypes.POINTER(AdamWParams),
                                                    _i32, _vp]
        lib.forge_linear_backward_sgdm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64,
                                                   _i64, ctypes.POINTER(SgdmParams), _i32, _vp]
        lib.forge_dgrad_bf16w.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _i32, _vp]
        lib.forge_linear_backward_adamw_bf16w.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64,
            ctypes.POINTER(AdamWParams), _i32, _vp]
        lib.forge_linear_backward_sgdm_bf16w.argtypes = [
            _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, ctypes.POINTER(SgdmParams),
            _i32, _vp]
        lib.forge_grouped_wgrad_sgdm.argtypes = [_vp, _vp, ctypes.POINTER(_i64), _i32, _vp, _vp,
                                                 _i64, _i64, ctypes.POINTER(SgdmParams), _i32,
                                                 _vp]
        lib.forge_wgrad_adamw_bf16w.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                                ctypes.POINTER(AdamWParams), _i32, _vp]
        lib.forge_wgrad_sgdm_bf16w.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                               ctypes.POINTER(SgdmParams), _i32, _vp]
        _d = ctypes.c_double
        lib.forge_wgrad_fp8.argtypes = [_vp, _i32, _d, _vp, _i32, _d, _vp, _i64, _i64, _i64,
                                        _i32, _vp]
        lib.forge_wgrad_adamw_fp8.argtypes = [_vp, _i32, _d, _vp, _i32, _d, _vp, _vp, _vp, _i64,
                                              _i64, _i64, ctypes.POINTER(AdamWParams), _i32, _vp]
        lib.forge_status_string.argtypes = [_i32]
        lib.forge_status_string.restype = ctypes.c_char_p
        for name in ("forge_wgrad_adamw", "forge_wgrad_sgdm", "forge_wgrad", "forge_adamw",
                     "forge_sgdm", "forge_grouped_wgrad_adamw", "forge_wgrad_bf16",
                     "forge_wgrad_adamw_bf16state", "forge_adamw_mixed", "forge_dgrad",
                     "forge_linear_backward_adamw", "forge_linear_backward_sgdm",
                     "forge_wgrad_fp8", "forge_wgrad_adamw_fp8", "forge_dgrad_bf16w",
                     "forge_linear_backward_adamw_bf16w", "forge_linear_backward_sgdm_bf16w",
                     "forge_wgrad_adamw_bf16w", "forge_wgrad_sgdm_bf16w",
                     "forge_grouped_wgrad_sgdm"):
            getattr(lib, name).restype = _i32
        _LIB = lib
    return _LIB


def forge_status_string(status: int) -> str:
    """The library's text for a status code (unknown codes get a generic text)."""
    return library().forge_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise ForgeError(status, where)


# --------------------------------------------------------------------------
# tensor marshalling
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() or None


def _want(t, dtype, name):
    if t is None:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        # the library launches on the current device; another device's memory would fault
        raise ValueError(f"{name} is on {t.device} but the current device is cuda:{cur} "
                         "(select it with torch.cuda.device)")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {stream.device} but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(stream.cuda_stream)


def _shape2(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm):
    return AdamWParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                       int(step), float(max_grad_norm))


def _state_like(W, others, d_out, d_in, lead=(), dtype=None):
    """Shape (and dtype: float32 unless given) of W and the state tensors."""
    want = (*lead, d_out, d_in)
    for name, t in (("W", W), *others):
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
        _want(t, (dtype or {}).get(name, _torch().float32), name)


def _xdy(X, dY):
    torch = _torch()
    _want(X, torch.bfloat16, "X")
    _want(dY, torch.bfloat16, "dY")
    T, d_in = _shape2(X, "X")
    T2, d_out = _shape2(dY, "dY")
    if T2 != T:
        raise ValueError(f"X has {T} token rows, dY has {T2}")
    return T, d_in, d_out


def _dtype_code(t, name):
    torch = _torch()
    if t.dtype == torch.float32:
        return FORGE_F32
    if t.dtype == torch.bfloat16:
        return FORGE_BF16
    raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")


# --------------------------------------------------------------------------
# entry points (names as in include/forge.h)
# --------------------------------------------------------------------------
def forge_wgrad_adamw(X, dY, W, m, v, *, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.01, max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT,
                      stream=None) -> None:
    """W, m, v <- AdamW(W, m, v, g = dY^T X), in place, g never stored."""
    torch = _torch()
    _want(X, torch.bfloat16, "X")
    _want(dY, torch.bfloat16, "dY")
    T, d_in = _shape2(X, "X")
    T2, d_out = _shape2(dY, "dY")
    if T2 != T:
        raise ValueError(f"X has {T} token rows, dY has {T2}")
    _state_like(W, (("m", m), ("v", v)), d_out, d_in)
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_wgrad_adamw(_ptr(X), _ptr(dY), _ptr(W), _ptr(m), _ptr(v), T, d_in,
                                       d_out, ctypes.byref(p), int(tile), _stream(stream)),
           "forge_wgrad_adamw")


def forge_wgrad_sgdm(X, dY, W, mom, *, lr=1e-3, momentum=0.9, weight_decay=0.0,
                     max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """W, mom <- SGD-momentum(W, mom, g = dY^T X), in place, g never stored."""
    torch = _torch()
    _want(X, torch.bfloat16, "X")
    _want(dY, torch.bfloat16, "dY")
    T, d_in = _shape2(X, "X")
    T2, d_out = _shape2(dY, "dY")
    if T2 != T:
        raise ValueError(f"X has {T} token rows, dY has {T2}")
    _state_like(W, (("mom", mom),), d_out, d_in)
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_wgrad_sgdm(_ptr(X), _ptr(dY), _ptr(W), _ptr(mom), T, d_in, d_out,
                                      ctypes.byref(p), int(tile), _stream(stream)),
           "forge_wgrad_sgdm")


def forge_wgrad(X, dY, grad, *, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """grad <- dY^T X in float32 (the unfused comparison path)."""
    torch = _torch()
    _want(X, torch.bfloat16, "X")
    _want(dY, torch.bfloat16, "dY")
    T, d_in = _shape2(X, "X")
    T2, d_out = _shape2(dY, "dY")
    if T2 != T:
        raise ValueError(f"X has {T} token rows, dY has {T2}")
    _state_like(grad, (), d_out, d_in)
    _check(library().forge_wgrad(_ptr(X), _ptr(dY), _ptr(grad), T, d_in, d_out, int(tile),
                                 _stream(stream)), "forge_wgrad")


def forge_adamw(grad, W, m, v, *, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                weight_decay=0.01, max_grad_norm=0.0, stream=None) -> None:
    """Elementwise AdamW from a stored float32 gradient (unfused path)."""
    torch = _torch()
    for name, t in (("grad", grad), ("W", W), ("m", m), ("v", v)):
        _want(t, torch.float32, name)
        if t.numel() != grad.numel():
            raise ValueError(f"{name} has {t.numel()} elements, grad has {grad.numel()}")
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_adamw(_ptr(grad), _ptr(W), _ptr(m), _ptr(v), grad.numel(),
                                 ctypes.byref(p), _stream(stream)), "forge_adamw")


def forge_sgdm(grad, W, mom, *, lr=1e-3, momentum=0.9, weight_decay=0.0, max_grad_norm=0.0,
               stream=None) -> None:
    """Elementwise SGD-momentum from a stored float32 gradient (unfused path)."""
    torch = _torch()
    for name, t in (("grad", grad), ("W", W), ("mom", mom)):
        _want(t, torch.float32, name)
        if t.numel() != grad.numel():
            raise ValueError(f"{name} has {t.numel()} elements, grad has {grad.numel()}")
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_sgdm(_ptr(grad), _ptr(W), _ptr(mom), grad.numel(), ctypes.byref(p),
                                _stream(stream)), "forge_sgdm")


def _grouped_args(X_perm, dY_perm, offsets, W, others):
    """Routed rows and host offsets; W and the state [E, d_out, d_in] float32."""
    torch = _torch()
    _want(X_perm, torch.bfloat16, "X_perm")
    _want(dY_perm, torch.bfloat16, "dY_perm")
    R, d_in = _shape2(X_perm, "X_perm")
    R2, d_out = _shape2(dY_perm, "dY_perm")
    if R2 != R:
        raise ValueError(f"X_perm has {R} rows, dY_perm has {R2}")
    offs = [int(x) for x in offsets]
    E = len(offs) - 1
    if E < 1:
        raise ValueError("offsets must hold E+1 >= 2 entries")
    if offs[-1] != R:
        raise ValueError(f"offsets[E] = {offs[-1]} but X_perm has {R} rows")
    _state_like(W, others, d_out, d_in, lead=(E,))
    return (_i64 * (E + 1))(*offs), E, d_in, d_out


def forge_grouped_wgrad_adamw(X_perm, dY_perm, offsets, W, m, v, *, step, lr=1e-3, beta1=0.9,
                              beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
                              tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """AdamW on E routed experts; expert e contracts rows offsets[e]:offsets[e+1].

    ``offsets`` is a host sequence of E+1 ints. Experts with no rows still
    take the step (zero gradient)."""
    arr, E, d_in, d_out = _grouped_args(X_perm, dY_perm, offsets, W, (("m", m), ("v", v)))
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_grouped_wgrad_adamw(_ptr(X_perm), _ptr(dY_perm), arr, E, _ptr(W),
                                               _ptr(m), _ptr(v), d_in, d_out, ctypes.byref(p),
                                               int(tile), _stream(stream)),
           "forge_grouped_wgrad_adamw")


def forge_grouped_wgrad_sgdm(X_perm, dY_perm, offsets, W, mom, *, lr=1e-3, momentum=0.9,
                             weight_decay=0.0, max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT,
                             stream=None) -> None:
    """SGD-momentum on E routed experts; experts with no rows still take the
    step (zero gradient, so only the coupled decay and the momentum move them)."""
    arr, E, d_in, d_out = _grouped_args(X_perm, dY_perm, offsets, W, (("mom", mom),))
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_grouped_wgrad_sgdm(_ptr(X_perm), _ptr(dY_perm), arr, E, _ptr(W),
                                              _ptr(mom), d_in, d_out, ctypes.byref(p), int(tile),
                                              _stream(stream)),
           "forge_grouped_wgrad_sgdm")


# --------------------------------------------------------------------------
# precision variants
# --------------------------------------------------------------------------
def forge_wgrad_bf16(X, dY, grad, *, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """grad (bfloat16) <- dY^T X rounded to bf16 from the float32 accumulator."""
    torch = _torch()
    T, d_in, d_out = _xdy(X, dY)
    _state_like(grad, (), d_out, d_in, dtype={"W": torch.bfloat16})
    _check(library().forge_wgrad_bf16(_ptr(X), _ptr(dY), _ptr(grad), T, d_in, d_out, int(tile),
                                      _stream(stream)), "forge_wgrad_bf16")


def forge_wgrad_adamw_bf16state(X, dY, W, m, v, *, step, lr=1e-3, beta1=0.9, beta2=0.999,
                                eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
                                tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """Fused AdamW with m, v in bfloat16 (W float32), in place."""
    torch = _torch()
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("m", m), ("v", v)), d_out, d_in,
                dtype={"m": torch.bfloat16, "v": torch.bfloat16})
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_wgrad_adamw_bf16state(_ptr(X), _ptr(dY), _ptr(W), _ptr(m), _ptr(v), T,
                                                 d_in, d_out, ctypes.byref(p), int(tile),
                                                 _stream(stream)),
           "forge_wgrad_adamw_bf16state")


def forge_adamw_mixed(grad, W, m, v, *, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.01, max_grad_norm=0.0, stream=None) -> None:
    """Elementwise AdamW; grad and the state (m, v, one dtype) float32 or bfloat16."""
    torch = _torch()
    _want(W, torch.float32, "W")
    gd = _dtype_code(grad, "grad")
    sd = _dtype_code(m, "m")
    if v.dtype != m.dtype:
        raise TypeError(f"m and v must share a dtype, got {m.dtype} and {v.dtype}")
    for name, t in (("grad", grad), ("m", m), ("v", v)):
        _want(t, t.dtype, name)
    for name, t in (("W", W), ("m", m), ("v", v)):
        if t.numel() != grad.numel():
            raise ValueError(f"{name} has {t.numel()} elements, grad has {grad.numel()}")
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_adamw_mixed(_ptr(grad), gd, _ptr(W), _ptr(m), _ptr(v), sd,
                                       grad.numel(), ctypes.byref(p), _stream(stream)),
           "forge_adamw_mixed")


def _dx_args(dY, W, dX, w_name="W"):
    """Shapes of the input-gradient contraction: dY [T, d_out] bf16, W
    [d_out, d_in] float32 (Wb: bf16), dX [T, d_in] float32 or bf16."""
    torch = _torch()
    _want(dY, torch.bfloat16, "dY")
    _want(W, torch.bfloat16 if w_name == "Wb" else torch.float32, w_name)
    T, d_out = _shape2(dY, "dY")
    d_out2, d_in = _shape2(W, w_name)
    if d_out2 != d_out:
        raise ValueError(f"{w_name} has {d_out2} rows, dY has {d_out} columns")
    if tuple(dX.shape) != (T, d_in):
        raise ValueError(f"dX must have shape {(T, d_in)}, got {tuple(dX.shape)}")
    code = _dtype_code(dX, "dX")
    _want(dX, dX.dtype, "dX")
    return T, d_in, d_out, code


def forge_dgrad(dY, W, dX, *, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """dX <- dY W_b (W_b: W rounded to bf16), float32 accumulation, stored in dX's dtype."""
    T, d_in, d_out, code = _dx_args(dY, W, dX)
    _check(library().forge_dgrad(_ptr(dY), _ptr(W), _ptr(dX), code, T, d_in, d_out, int(tile),
                                 _stream(stream)), "forge_dgrad")


def forge_linear_backward_adamw(X, dY, W, m, v, dX, *, step, lr=1e-3, beta1=0.9, beta2=0.999,
                                eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
                                tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """dX <- dY W_b from the weight on entry, then the fused AdamW step on W, m, v."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("m", m), ("v", v)), d_out, d_in)
    _, _, _, code = _dx_args(dY, W, dX)
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_linear_backward_adamw(_ptr(X), _ptr(dY), _ptr(W), _ptr(m), _ptr(v),
                                                 _ptr(dX), code, T, d_in, d_out, ctypes.byref(p),
                                                 int(tile), _stream(stream)),
           "forge_linear_backward_adamw")


def forge_linear_backward_sgdm(X, dY, W, mom, dX, *, lr=1e-3, momentum=0.9, weight_decay=0.0,
                               max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """dX <- dY W_b from the weight on entry, then the fused SGD-momentum step."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("mom", mom),), d_out, d_in)
    _, _, _, code = _dx_args(dY, W, dX)
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_linear_backward_sgdm(_ptr(X), _ptr(dY), _ptr(W), _ptr(mom), _ptr(dX),
                                                code, T, d_in, d_out, ctypes.byref(p), int(tile),
                                                _stream(stream)),
           "forge_linear_backward_sgdm")


def forge_dgrad_bf16w(dY, Wb, dX, *, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """dX <- dY Wb from a bf16 copy Wb of the weight, float32 accumulation."""
    T, d_in, d_out, code = _dx_args(dY, Wb, dX, "Wb")
    _check(library().forge_dgrad_bf16w(_ptr(dY), _ptr(Wb), _ptr(dX), code, T, d_in, d_out,
                                       int(tile), _stream(stream)), "forge_dgrad_bf16w")


def forge_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, *, step, lr=1e-3, beta1=0.9,
                                      beta2=0.999, eps=1e-8, weight_decay=0.01,
                                      max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT,
                                      stream=None) -> None:
    """dX <- dY Wb from the bf16 copy on entry, then the fused AdamW step on W,
    m, v, which also stores bf16(W) into Wb."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("m", m), ("v", v)), d_out, d_in)
    _, _, _, code = _dx_args(dY, Wb, dX, "Wb")
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_linear_backward_adamw_bf16w(
        _ptr(X), _ptr(dY), _ptr(W), _ptr(m), _ptr(v), _ptr(Wb), _ptr(dX), code, T, d_in, d_out,
        ctypes.byref(p), int(tile), _stream(stream)), "forge_linear_backward_adamw_bf16w")


def forge_linear_backward_sgdm_bf16w(X, dY, W, mom, Wb, dX, *, lr=1e-3, momentum=0.9,
                                     weight_decay=0.0, max_grad_norm=0.0,
                                     tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """dX <- dY Wb from the bf16 copy on entry, then the fused SGD-momentum
    step, which also stores bf16(W) into Wb."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("mom", mom),), d_out, d_in)
    _, _, _, code = _dx_args(dY, Wb, dX, "Wb")
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_linear_backward_sgdm_bf16w(
        _ptr(X), _ptr(dY), _ptr(W), _ptr(mom), _ptr(Wb), _ptr(dX), code, T, d_in, d_out,
        ctypes.byref(p), int(tile), _stream(stream)), "forge_linear_backward_sgdm_bf16w")


def _wb_like(Wb, d_out, d_in):
    torch = _torch()
    _want(Wb, torch.bfloat16, "Wb")
    if tuple(Wb.shape) != (d_out, d_in):
        raise ValueError(f"Wb must have shape {(d_out, d_in)}, got {tuple(Wb.shape)}")


def forge_wgrad_adamw_bf16w(X, dY, W, m, v, Wb, *, step, lr=1e-3, beta1=0.9, beta2=0.999,
                            eps=1e-8, weight_decay=0.01, max_grad_norm=0.0,
                            tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """The fused AdamW step of forge_wgrad_adamw, also storing bf16(W) into Wb."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("m", m), ("v", v)), d_out, d_in)
    _wb_like(Wb, d_out, d_in)
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_wgrad_adamw_bf16w(_ptr(X), _ptr(dY), _ptr(W), _ptr(m), _ptr(v),
                                             _ptr(Wb), T, d_in, d_out, ctypes.byref(p), int(tile),
                                             _stream(stream)), "forge_wgrad_adamw_bf16w")


def forge_wgrad_sgdm_bf16w(X, dY, W, mom, Wb, *, lr=1e-3, momentum=0.9, weight_decay=0.0,
                           max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """The fused SGD-momentum step of forge_wgrad_sgdm, also storing bf16(W) into Wb."""
    T, d_in, d_out = _xdy(X, dY)
    _state_like(W, (("mom", mom),), d_out, d_in)
    _wb_like(Wb, d_out, d_in)
    p = SgdmParams(float(lr), float(momentum), float(weight_decay), float(max_grad_norm))
    _check(library().forge_wgrad_sgdm_bf16w(_ptr(X), _ptr(dY), _ptr(W), _ptr(mom), _ptr(Wb), T,
                                            d_in, d_out, ctypes.byref(p), int(tile),
                                            _stream(stream)), "forge_wgrad_sgdm_bf16w")


_FP8 = {"e4m3": FORGE_FP8_E4M3, "e5m2": FORGE_FP8_E5M2}


def _fp8_args(X8, x_fmt, dY8, dy_fmt):
    """fp8 operands are uint8 tensors of codes; formats by name ("e4m3", "e5m2")."""
    torch = _torch()
    _want(X8, torch.uint8, "X8")
    _want(dY8, torch.uint8, "dY8")
    T, d_in = _shape2(X8, "X8")
    T2, d_out = _shape2(dY8, "dY8")
    if T2 != T:
        raise ValueError(f"X8 has {T} token rows, dY8 has {T2}")
    try:
        return T, d_in, d_out, _FP8[x_fmt], _FP8[dy_fmt]
    except KeyError as e:
        raise ValueError(f"fp8 format must be one of {sorted(_FP8)}, got {e}") from None


def forge_wgrad_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, grad, *,
                    tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """grad (float32) <- x_scale dy_scale dY8^T X8 from fp8 codes."""
    T, d_in, d_out, xf, yf = _fp8_args(X8, x_fmt, dY8, dy_fmt)
    _state_like(grad, (), d_out, d_in)
    _check(library().forge_wgrad_fp8(_ptr(X8), xf, float(x_scale), _ptr(dY8), yf,
                                     float(dy_scale), _ptr(grad), T, d_in, d_out, int(tile),
                                     _stream(stream)), "forge_wgrad_fp8")


def forge_wgrad_adamw_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, W, m, v, *, step, lr=1e-3,
                          beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                          max_grad_norm=0.0, tile=FORGE_TILE_DEFAULT, stream=None) -> None:
    """Fused weight gradient from fp8 inputs + AdamW on W, m, v in place."""
    T, d_in, d_out, xf, yf = _fp8_args(X8, x_fmt, dY8, dy_fmt)
    _state_like(W, (("m", m), ("v", v)), d_out, d_in)
    p = _adamw(step, lr, beta1, beta2, eps, weight_decay, max_grad_norm)
    _check(library().forge_wgrad_adamw_fp8(_ptr(X8), xf, float(x_scale), _ptr(dY8), yf,
                                           float(dy_scale), _ptr(W), _ptr(m), _ptr(v), T, d_in,
                                           d_out, ctypes.byref(p), int(tile), _stream(stream)),
           "forge_wgrad_adamw_fp8")
