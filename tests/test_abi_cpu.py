"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments with the documented status codes before
touching any buffer. Fake, never-dereferenced pointers are used throughout;
the one case that passes validation is only run where no GPU is visible.
"""
import ctypes
import os
import re
import subprocess

import pytest

from weight_gradient_gemm_amd import _lib

NULL = None
A = 0x100000          # fake, 16-byte aligned "device" addresses far apart
B = 0x200000000
C = 0x400000000
D = 0x600000000
X_ADDR = 0x800000000
Y_ADDR = 0xA00000000
WB_ADDR = 0xC00000000


@pytest.fixture(scope="module")
def lib():
    return _lib.library()


def declared_symbols(root):
    with open(os.path.join(root, "include", "forge.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"FORGE_API\s+[\w\s\*]*?\b(forge_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib, root):
    names = declared_symbols(root)
    assert names == sorted(["forge_adamw", "forge_adamw_mixed", "forge_dgrad",
                            "forge_dgrad_bf16w", "forge_grouped_wgrad_adamw", "forge_grouped_wgrad_sgdm",
                            "forge_linear_backward_adamw", "forge_linear_backward_adamw_bf16w",
                            "forge_linear_backward_sgdm", "forge_linear_backward_sgdm_bf16w",
                            "forge_sgdm", "forge_status_string",
                            "forge_wgrad", "forge_wgrad_adamw", "forge_wgrad_adamw_bf16state",
                            "forge_wgrad_adamw_bf16w", "forge_wgrad_adamw_fp8", "forge_wgrad_bf16", "forge_wgrad_fp8",
                            "forge_wgrad_sgdm", "forge_wgrad_sgdm_bf16w"])
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (forge_\w+)", out))
    assert set(names) <= exported


def test_status_strings(lib):
    for s in range(-1, 12):
        txt = _lib.forge_status_string(s)
        assert isinstance(txt, str) and txt
    assert "clipping" in _lib.forge_status_string(6)
    assert "element type" in _lib.forge_status_string(10)


def adam(**kw):
    base = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1,
                max_grad_norm=0.0)
    base.update(kw)
    return _lib.AdamWParams(base["lr"], base["beta1"], base["beta2"], base["eps"],
                            base["weight_decay"], base["step"], base["max_grad_norm"])


def sgd(**kw):
    base = dict(lr=1e-3, momentum=0.9, weight_decay=0.0, max_grad_norm=0.0)
    base.update(kw)
    return _lib.SgdmParams(base["lr"], base["momentum"], base["weight_decay"],
                           base["max_grad_norm"])


def call_adamw(lib, X=X_ADDR, dY=Y_ADDR, W=A, m=B, v=C, T=64, d_in=64, d_out=32, p=None,
               tile=0):
    p = adam() if p is None else p
    return lib.forge_wgrad_adamw(X, dY, W, m, v, T, d_in, d_out, ctypes.byref(p), tile, None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=NULL), 1), (dict(m=NULL), 1), (dict(v=NULL), 1), (dict(X=NULL), 1), (dict(dY=NULL), 1),
    (dict(T=-1), 2), (dict(d_in=-8), 2), (dict(d_out=-8), 2), (dict(T=1 << 31), 2),
    (dict(d_in=(1 << 22) + 8), 2), (dict(d_out=(1 << 22) + 8), 2),
    (dict(d_in=12), 3), (dict(d_out=20), 3), (dict(W=A + 4), 3), (dict(X=X_ADDR + 2), 3),
    (dict(dY=Y_ADDR + 8), 3),
    (dict(m=A), 4), (dict(v=A + 64), 4), (dict(W=X_ADDR), 4), (dict(m=Y_ADDR - 16), 4),
    (dict(p=adam(max_grad_norm=1.0)), 6), (dict(p=adam(max_grad_norm=float("inf"))), 6),
    (dict(p=adam(max_grad_norm=-1.0)), 5), (dict(p=adam(max_grad_norm=float("nan"))), 5),
    (dict(p=adam(beta1=1.0)), 5), (dict(p=adam(beta2=-0.1)), 5), (dict(p=adam(lr=-1e-3)), 5),
    (dict(p=adam(eps=float("nan"))), 5), (dict(p=adam(step=0)), 5),
    (dict(p=adam(weight_decay=float("inf"))), 5),
    (dict(tile=5), 7), (dict(tile=-1), 7),
])
def test_wgrad_adamw_rejects(lib, kw, status):
    assert call_adamw(lib, **kw) == status


def test_clip_request_beats_other_hparam_errors(lib):
    # fail closed on clipping even when another hyperparameter is also off
    assert call_adamw(lib, p=adam(max_grad_norm=0.5, beta1=2.0)) == 6


def test_empty_outputs_are_noops(lib):
    # nothing to update: OK without a device (no launch, nothing touched)
    assert call_adamw(lib, d_in=0) == 0
    assert call_adamw(lib, d_out=0, W=NULL, m=NULL, v=NULL) == 0
    assert lib.forge_adamw(A, B, C, D, 0, ctypes.byref(adam()), None) == 0


def test_no_gpu_means_device_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: valid fake pointers would launch a kernel")
    assert call_adamw(lib) == 8
    assert call_adamw(lib, T=0, X=NULL, dY=NULL) == 8
    p = sgd()
    assert lib.forge_wgrad_sgdm(X_ADDR, Y_ADDR, A, B, 64, 64, 32, ctypes.byref(p), 0, None) == 8
    assert lib.forge_wgrad(X_ADDR, Y_ADDR, A, 64, 64, 32, 0, None) == 8
    assert lib.forge_adamw(A, B, C, D, 100, ctypes.byref(adam()), None) == 8
    assert lib.forge_sgdm(A, B, C, 100, ctypes.byref(sgd()), None) == 8
    offs = (ctypes.c_int64 * 3)(0, 10, 10)
    assert lib.forge_grouped_wgrad_adamw(X_ADDR, Y_ADDR, offs, 2, A, B, C, 64, 32,
                                         ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_grouped_wgrad_sgdm(X_ADDR, Y_ADDR, offs, 2, A, B, 64, 32,
                                        ctypes.byref(sgd()), 0, None) == 8
    assert lib.forge_wgrad_bf16(X_ADDR, Y_ADDR, A, 64, 64, 32, 0, None) == 8
    assert lib.forge_wgrad_adamw_bf16state(X_ADDR, Y_ADDR, A, B, C, 64, 64, 32,
                                           ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_adamw_mixed(A, 1, B, C, D, 1, 100, ctypes.byref(adam()), None) == 8
    assert lib.forge_dgrad(Y_ADDR, A, B, 1, 64, 64, 32, 0, None) == 8
    assert lib.forge_wgrad_fp8(X_ADDR, 2, 1.0, Y_ADDR, 3, 1.0, A, 64, 64, 32, 0, None) == 8
    assert lib.forge_wgrad_adamw_fp8(X_ADDR, 2, 1.0, Y_ADDR, 3, 1.0, A, B, C, 64, 64, 32,
                                     ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_linear_backward_adamw(X_ADDR, Y_ADDR, A, B, C, D, 1, 64, 64, 32,
                                           ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_linear_backward_sgdm(X_ADDR, Y_ADDR, A, B, D, 0, 64, 64, 32,
                                          ctypes.byref(sgd()), 0, None) == 8
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, B, 1, 64, 64, 32, 0, None) == 8
    assert lib.forge_linear_backward_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, WB_ADDR, D, 1, 64, 64,
                                                 32, ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_linear_backward_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, D, 0, 64, 64, 32,
                                                ctypes.byref(sgd()), 0, None) == 8
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, WB_ADDR, 64, 64, 32,
                                       ctypes.byref(adam()), 0, None) == 8
    assert lib.forge_wgrad_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, 64, 64, 32,
                                      ctypes.byref(sgd()), 0, None) == 8


def test_sgdm_and_unfused_reject(lib):
    p = sgd(momentum=1.0)
    assert lib.forge_wgrad_sgdm(X_ADDR, Y_ADDR, A, B, 64, 64, 32, ctypes.byref(p), 0, None) == 5
    p = sgd(max_grad_norm=2.0)
    assert lib.forge_wgrad_sgdm(X_ADDR, Y_ADDR, A, B, 64, 64, 32, ctypes.byref(p), 0, None) == 6
    assert lib.forge_wgrad_sgdm(X_ADDR, Y_ADDR, A, A, 64, 64, 32, ctypes.byref(sgd()), 0,
                                None) == 4
    assert lib.forge_wgrad(X_ADDR, Y_ADDR, NULL, 64, 64, 32, 0, None) == 1
    assert lib.forge_wgrad(X_ADDR, Y_ADDR, X_ADDR + 64, 64, 64, 32, 0, None) == 4
    assert lib.forge_adamw(A, B, C, D, -1, ctypes.byref(adam()), None) == 2
    assert lib.forge_adamw(A, A, C, D, 100, ctypes.byref(adam()), None) == 4
    assert lib.forge_adamw(A + 4, B, C, D, 100, ctypes.byref(adam()), None) == 3
    assert lib.forge_adamw(A, B, C, D, 100, None, None) == 1
    assert lib.forge_sgdm(A, B, NULL, 100, ctypes.byref(sgd()), None) == 1


def test_precision_variants_reject(lib):
    F32, BF16 = _lib.FORGE_F32, _lib.FORGE_BF16
    n = 128
    # bf16 buffers are 2 bytes per element: m at A + 2n does not overlap a bf16 grad at A
    assert lib.forge_adamw_mixed(A, BF16, B, A + 2 * n, C, BF16, n, ctypes.byref(adam()),
                                 None) != 4
    # ... but does overlap a float32 grad at A
    assert lib.forge_adamw_mixed(A, F32, B, A + 2 * n, C, BF16, n, ctypes.byref(adam()),
                                 None) == 4
    assert lib.forge_adamw_mixed(A, 7, B, C, D, F32, n, ctypes.byref(adam()), None) == 10
    assert lib.forge_adamw_mixed(A, F32, B, C, D, -1, n, ctypes.byref(adam()), None) == 10
    assert lib.forge_adamw_mixed(A, BF16, B, C, D, BF16, n, ctypes.byref(adam(max_grad_norm=1.0)),
                                 None) == 6
    assert lib.forge_adamw_mixed(A, BF16, B, C + 8, D, BF16, n, ctypes.byref(adam()), None) == 3
    # bf16 gradient: [32, 64] bf16 is 4 KiB, so an X 4 KiB after it does not overlap
    assert lib.forge_wgrad_bf16(X_ADDR, Y_ADDR, X_ADDR - 4096, 64, 64, 32, 0, None) != 4
    assert lib.forge_wgrad_bf16(X_ADDR, Y_ADDR, X_ADDR - 2048, 64, 64, 32, 0, None) == 4
    assert lib.forge_wgrad_bf16(X_ADDR, Y_ADDR, NULL, 64, 64, 32, 0, None) == 1
    assert lib.forge_wgrad_bf16(X_ADDR, Y_ADDR, A, 64, 64, 32, 9, None) == 7
    p = adam()
    assert lib.forge_wgrad_adamw_bf16state(X_ADDR, Y_ADDR, A, B, B + 2 * 64 * 32, 64, 64, 32,
                                           ctypes.byref(p), 0, None) != 4
    assert lib.forge_wgrad_adamw_bf16state(X_ADDR, Y_ADDR, A, B, B + 2 * 64 * 32 - 16, 64, 64,
                                           32, ctypes.byref(p), 0, None) == 4
    p = adam(max_grad_norm=3.0)
    assert lib.forge_wgrad_adamw_bf16state(X_ADDR, Y_ADDR, A, B, C, 64, 64, 32, ctypes.byref(p),
                                           0, None) == 6


def test_dgrad_and_linear_backward_reject(lib):
    F32, BF16 = _lib.FORGE_F32, _lib.FORGE_BF16
    T, d_in, d_out = 64, 64, 32
    # dgrad: dY [T, d_out] bf16 at Y_ADDR, W [d_out, d_in] f32 at A, dX [T, d_in] at B
    assert lib.forge_dgrad(Y_ADDR, A, B, 5, T, d_in, d_out, 0, None) == 10
    assert lib.forge_dgrad(Y_ADDR, A, NULL, F32, T, d_in, d_out, 0, None) == 1
    assert lib.forge_dgrad(NULL, A, B, F32, T, d_in, d_out, 0, None) == 1
    assert lib.forge_dgrad(Y_ADDR, A, B, F32, -1, d_in, d_out, 0, None) == 2
    assert lib.forge_dgrad(Y_ADDR, A, B, F32, T, 60, d_out, 0, None) == 3
    assert lib.forge_dgrad(Y_ADDR, A, B + 4, F32, T, d_in, d_out, 0, None) == 3
    # dX overlapping W (8 KiB of float32) or dY (4 KiB of bf16)
    assert lib.forge_dgrad(Y_ADDR, A, A + 8192 - 16, BF16, T, d_in, d_out, 0, None) == 4
    assert lib.forge_dgrad(Y_ADDR, A, A + 8192, BF16, T, d_in, d_out, 0, None) != 4
    assert lib.forge_dgrad(Y_ADDR, A, Y_ADDR + 4096 - 16, F32, T, d_in, d_out, 0, None) == 4
    assert lib.forge_dgrad(Y_ADDR, A, B, F32, T, d_in, d_out, 9, None) == 7
    # nothing to write: no device needed
    assert lib.forge_dgrad(Y_ADDR, A, NULL, F32, 0, d_in, d_out, 0, None) == 0
    assert lib.forge_dgrad(Y_ADDR, A, NULL, F32, T, 0, d_out, 0, None) == 0

    def lb(dX=D, dt=BF16, X=X_ADDR, p=None, tile=0, m=B, v=C):
        p = adam() if p is None else p
        return lib.forge_linear_backward_adamw(X, Y_ADDR, A, m, v, dX, dt, T, d_in, d_out,
                                               ctypes.byref(p), tile, None)

    assert lb(dt=3) == 10
    assert lb(dX=NULL) == 1
    assert lb(p=adam(max_grad_norm=1.0)) == 6
    assert lb(tile=11) == 7
    assert lb(m=A) == 4                       # state overlaps W (wgrad checks first)
    assert lb(dX=B + 16) == 4                 # dX overlaps m
    assert lb(dX=X_ADDR + 16) == 4            # dX overlaps X
    assert lb(dX=A + 64) == 4                 # dX overlaps W
    assert lib.forge_linear_backward_sgdm(X_ADDR, Y_ADDR, A, B, B + 32, F32, T, d_in, d_out,
                                          ctypes.byref(sgd()), 0, None) == 4
    assert lib.forge_linear_backward_sgdm(X_ADDR, Y_ADDR, A, B, D, F32, T, d_in, d_out,
                                          ctypes.byref(sgd(momentum=2.0)), 0, None) == 5


def test_bf16_weight_copy_calls_reject(lib):
    F32, BF16 = _lib.FORGE_F32, _lib.FORGE_BF16
    T, d_in, d_out = 64, 64, 32
    # dgrad from Wb [d_out, d_in] bf16 (4 KiB) at WB_ADDR into dX at B
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, B, 5, T, d_in, d_out, 0, None) == 10
    assert lib.forge_dgrad_bf16w(Y_ADDR, NULL, B, F32, T, d_in, d_out, 0, None) == 1
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR + 8, B, F32, T, d_in, d_out, 0, None) == 3
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, WB_ADDR + 4096 - 16, F32, T, d_in, d_out, 0,
                                 None) == 4
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, WB_ADDR + 4096, BF16, T, d_in, d_out, 0,
                                 None) != 4
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, B, F32, T, d_in, d_out, 9, None) == 7
    assert lib.forge_dgrad_bf16w(Y_ADDR, WB_ADDR, NULL, F32, 0, d_in, d_out, 0, None) == 0

    def lb(Wb=WB_ADDR, dX=D, dt=BF16, p=None, m=B, tile=0):
        p = adam() if p is None else p
        return lib.forge_linear_backward_adamw_bf16w(X_ADDR, Y_ADDR, A, m, C, Wb, dX, dt, T,
                                                     d_in, d_out, ctypes.byref(p), tile, None)

    assert lb(Wb=NULL) == 1
    assert lb(dX=NULL) == 1
    assert lb(dt=2) == 10
    assert lb(Wb=WB_ADDR + 2) == 3
    assert lb(Wb=A + 8192 - 16) == 4          # the copy overlaps W (8 KiB of float32)
    assert lb(Wb=B + 16) == 4                 # the copy overlaps m
    assert lb(Wb=X_ADDR + 16) == 4            # the copy overlaps X
    assert lb(dX=WB_ADDR + 16) == 4           # dX overlaps the copy it reads
    assert lb(dX=A + 64) == 4                 # dX overlaps W, which the step writes
    assert lb(dX=C + 64) == 4                 # dX overlaps v
    assert lb(p=adam(max_grad_norm=1.0)) == 6
    assert lb(p=adam(beta2=1.5)) == 5
    assert lb(tile=11) == 7
    assert lib.forge_linear_backward_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, A + 16, D, F32, T, d_in,
                                                d_out, ctypes.byref(sgd()), 0, None) == 4
    assert lib.forge_linear_backward_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, D, F32, T, d_in,
                                                d_out, ctypes.byref(sgd(momentum=2.0)), 0,
                                                None) == 5
    # nothing to write: no device needed
    assert lib.forge_linear_backward_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, D, F32, T, 0,
                                                d_out, ctypes.byref(sgd()), 0, None) == 0
    # the fused steps alone
    p = adam()
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, NULL, T, d_in, d_out,
                                       ctypes.byref(p), 0, None) == 1
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, WB_ADDR + 8, T, d_in, d_out,
                                       ctypes.byref(p), 0, None) == 3
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, C + 16, T, d_in, d_out,
                                       ctypes.byref(p), 0, None) == 4
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, WB_ADDR, T, d_in, d_out,
                                       ctypes.byref(adam(max_grad_norm=2.0)), 0, None) == 6
    assert lib.forge_wgrad_adamw_bf16w(X_ADDR, Y_ADDR, A, B, C, WB_ADDR, T, d_in, d_out,
                                       ctypes.byref(p), 8, None) == 7
    assert lib.forge_wgrad_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, Y_ADDR + 32, T, d_in, d_out,
                                      ctypes.byref(sgd()), 0, None) == 4
    assert lib.forge_wgrad_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, T, d_in, d_out,
                                      ctypes.byref(sgd(lr=-1.0)), 0, None) == 5
    assert lib.forge_wgrad_sgdm_bf16w(X_ADDR, Y_ADDR, A, B, WB_ADDR, T, 0, d_out,
                                      ctypes.byref(sgd()), 0, None) == 0


def test_fp8_rejects(lib):
    E4, E5 = _lib.FORGE_FP8_E4M3, _lib.FORGE_FP8_E5M2

    def g(xf=E4, sx=1.0, yf=E5, sy=1.0, grad=A, T=64, d_in=64, d_out=32, X=X_ADDR, tile=0):
        return lib.forge_wgrad_fp8(X, xf, sx, Y_ADDR, yf, sy, grad, T, d_in, d_out, tile, None)

    assert g(xf=_lib.FORGE_BF16) == 10
    assert g(yf=7) == 10
    assert g(sx=0.0) == 5
    assert g(sy=-1.0) == 5
    assert g(sx=float("nan")) == 5
    assert g(sx=1e-30, sy=1e-30) == 5        # the product is not a normal float32
    assert g(sx=1e30, sy=1e30) == 5          # the product overflows float32
    assert g(d_in=72) == 3                   # fp8 rows need multiples of 16
    assert g(d_out=40) == 3
    assert g(grad=NULL) == 1
    assert g(tile=9) == 7
    # X8 is 1 byte per element: a gradient 64*64 bytes after X does not overlap it
    assert g(grad=X_ADDR + 64 * 64) != 4
    assert g(grad=X_ADDR + 64 * 64 - 16) == 4
    assert lib.forge_wgrad_adamw_fp8(X_ADDR, E4, 1.0, Y_ADDR, E5, 1.0, A, B, C, 64, 64, 32,
                                     ctypes.byref(adam(max_grad_norm=1.0)), 0, None) == 6
    assert lib.forge_wgrad_adamw_fp8(X_ADDR, E4, 1.0, Y_ADDR, E5, 1.0, A, A, C, 64, 64, 32,
                                     ctypes.byref(adam()), 0, None) == 4
    assert lib.forge_wgrad_adamw_fp8(X_ADDR, E4, 1.0, Y_ADDR, E5, 1.0, A, B, C, 64, 64, 32,
                                     None, 0, None) == 1


def test_grouped_rejects(lib):
    def call(offs, E=None, W=A, m=B, v=C, d_in=64, d_out=32, p=None):
        E = len(offs) - 1 if E is None else E
        arr = (ctypes.c_int64 * len(offs))(*offs)
        p = adam() if p is None else p
        return lib.forge_grouped_wgrad_adamw(X_ADDR, Y_ADDR, arr, E, W, m, v, d_in, d_out,
                                             ctypes.byref(p), 0, None)

    assert lib.forge_grouped_wgrad_adamw(X_ADDR, Y_ADDR, None, 2, A, B, C, 64, 32,
                                         ctypes.byref(adam()), 0, None) == 1
    assert call([0], E=0) == 2
    assert call([0] * 258, E=257) == 2
    assert call([1, 4, 9]) == 2                  # offsets[0] != 0
    assert call([0, 9, 4]) == 2                  # decreasing
    assert call([0, 4, 9], d_in=36) == 3
    assert call([0, 4, 9], m=A + 64 * 32 * 4) == 4   # m overlaps expert 1 of W
    assert call([0, 4, 9], p=adam(max_grad_norm=1.0)) == 6


def test_grouped_sgdm_rejects(lib):
    def call(offs, W=A, mom=B, d_in=64, d_out=32, p=None, tile=0):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        p = sgd() if p is None else p
        return lib.forge_grouped_wgrad_sgdm(X_ADDR, Y_ADDR, arr, len(offs) - 1, W, mom, d_in,
                                            d_out, ctypes.byref(p), tile, None)

    assert lib.forge_grouped_wgrad_sgdm(X_ADDR, Y_ADDR, None, 2, A, B, 64, 32,
                                        ctypes.byref(sgd()), 0, None) == 1
    assert call([0, 4, 9], mom=NULL) == 1
    assert call([0, 9, 4]) == 2
    assert call([0, 4, 9], d_out=36) == 3
    assert call([0, 4, 9], mom=A + 64 * 32 * 4) == 4     # mom overlaps expert 1 of W
    assert call([0, 4, 9], p=sgd(max_grad_norm=0.5)) == 6
    assert call([0, 4, 9], p=sgd(momentum=1.0)) == 5
    assert call([0, 4, 9], tile=9) == 7
    assert call([0, 4, 9], d_in=0) == 0                   # nothing to update


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "library_path", str(tmp_path / "libforge.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.library()


def test_kernel_sources_have_no_atomics_or_split_k(root):
    # no atomics anywhere in the device code (order of accumulation is fixed)
    csrc = os.path.join(root, "weight_gradient_gemm_amd", "csrc")
    for fn in os.listdir(csrc):
        with open(os.path.join(csrc, fn)) as f:
            text = f.read()
        code = re.sub(r"//.*", "", text)
        assert not re.search(r"atomic(Add|Max|Min|CAS|Exch|_)", code, re.I) or fn == "forge.hip", fn
        assert not re.search(r"split_?k", code, re.I), fn
    with open(os.path.join(csrc, "wgrad_kernels.hpp")) as f:
        kern = re.sub(r"//.*", "", f.read())
    assert "atomic" not in kern.lower()
