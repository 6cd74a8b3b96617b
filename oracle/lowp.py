"""Oracle for 8-bit floating-point (fp8) inputs to the weight gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FORGE assessment, "Math verified, not asserted", P6: the paper's own int8 and
fp8 rows are 4x and 44x worse than its baseline. The fp8 variant of the
contraction takes X and dY as fp8 codes with one float scale per tensor:

    g[o, i] = s_x s_dy sum_t dY8[t, o] X8[t, i]

(X8, dY8 the decoded fp8 values), rounded once to float32, then the ordinary
float32 optimizer step. The two fp8 encodings are the OCP ones:
  E4M3: sign, 4 exponent bits (bias 7), 3 fraction bits; exponent 0 holds
        subnormals 2^-6 f/8; no infinities; S.1111.111 is NaN; largest 448.
  E5M2: sign, 5 exponent bits (bias 15), 2 fraction bits; exponent 0 holds
        subnormals 2^-14 f/4; exponent 31 holds inf (f = 0) and NaN.
Products of fp8 values are exact in float64, as are the sums here.
"""
from __future__ import annotations

import numpy as np

from .floor import U32

E4M3 = "e4m3"
E5M2 = "e5m2"
_LAYOUT = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}   # exponent bits, fraction bits, bias


def fp8_to_f64(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Decode fp8 codes (uint8) of the given format to float64, exactly."""
    eb, fb, bias = _LAYOUT[fmt]
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> fb) & ((1 << eb) - 1)
    f = b & ((1 << fb) - 1)
    normal = sign * (1.0 + f / float(1 << fb)) * np.exp2(e.astype(np.float64) - bias)
    sub = sign * (f / float(1 << fb)) * 2.0 ** (1 - bias)
    out = np.where(e == 0, sub, normal)
    top = (1 << eb) - 1
    if fmt == E4M3:
        out = np.where((e == top) & (f == (1 << fb) - 1), np.nan, out)
    else:
        out = np.where((e == top) & (f == 0), sign * np.inf, out)
        out = np.where((e == top) & (f != 0), np.nan, out)
    return out


def wgrad_fp8_f64(X8: np.ndarray, x_fmt: str, x_scale: float, dY8: np.ndarray, dy_fmt: str,
                  dy_scale: float) -> np.ndarray:
    """s_x s_dy dY8^T X8 in float64 ([d_out, d_in], not rounded)."""
    X = fp8_to_f64(X8, x_fmt)
    dY = fp8_to_f64(dY8, dy_fmt)
    if X.shape[0] != dY.shape[0]:
        raise ValueError("X and dY must have the same number of token rows")
    return (float(x_scale) * float(dy_scale)) * (dY.T @ X)


def wgrad_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale) -> np.ndarray:
    """wgrad_fp8_f64 rounded once to float32."""
    return wgrad_fp8_f64(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale).astype(np.float32)


def wgrad_fp8_rows(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    return wgrad_fp8(X8, x_fmt, x_scale, np.ascontiguousarray(dY8[:, rows]), dy_fmt, dy_scale)


def acc_floor_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, rows=None,
                  exact_max: bool = True) -> np.ndarray:
    """Floor of the scaled fp8 sum: the weight-gradient floor 4 u sqrt(T)
    sqrt(sum_t (dY X)^2) on the decoded values, times |s_x s_dy|, plus one
    rounding of the scale product applied to the sum, plus the fp8 dot-product
    loss (mfma_fp8_floor)."""
    X = fp8_to_f64(X8, x_fmt)
    dY = fp8_to_f64(dY8 if rows is None else np.ascontiguousarray(dY8[:, rows]), dy_fmt)
    T = X.shape[0]
    s = abs(float(x_scale) * float(dy_scale))
    tau = 4.0 * U32 * np.sqrt(max(T, 1)) * np.sqrt((dY * dY).T @ (X * X)) * s
    return (tau + 2.0 * U32 * np.abs((dY.T @ X) * s)
            + mfma_fp8_floor(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, rows, exact_max))


# The fp8 matrix instruction's dot product is not exact. Measured on gfx950
# with controlled sums (one 64-token instruction): the products of each run of
# 8 consecutive tokens are aligned to the largest of them, and each product is
# truncated toward zero to a multiple of 2^(E - 13), E the exponent of that
# largest product (1 + 2^-13 survives; 1 + 2^-14, 1 - 2^-14 and 1 + 1.5 2^-14
# come out as 1; eight products of 2^-14 on their own are exact); the run sums
# and the float32 accumulator then add without further loss. The pages fix no
# precision for this path, so its tolerance is taken from that arithmetic:
# each product loses at most min(|p_t|, 2^(E - FP8_DOT_BITS + 1)) (twice the
# measured step), with the opposite sign to the product, and these losses add
# like the float32 rounding errors of the accumulation floor: as a random walk,
# four times the root sum of squares.
FP8_DOT_BITS = 13
FP8_RUN = 8


def mfma_fp8_floor(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, rows=None,
                   exact_max: bool = True) -> np.ndarray:
    """Bound of the fp8 dot-product loss (the weight's [d_out, d_in] layout,
    or the given rows of it). exact_max: each element's own largest product
    per run (O(T d_out d_in)); otherwise the run's largest |X| and |dY| bound
    it and each product of the run counts a full step (cheaper, looser)."""
    # (P, the run's products, exists only on the exact path)
    X = np.abs(fp8_to_f64(X8, x_fmt))
    dY = np.abs(fp8_to_f64(dY8 if rows is None else np.ascontiguousarray(dY8[:, rows]), dy_fmt))
    T = X.shape[0]
    sq = np.zeros((dY.shape[1], X.shape[1]))
    for r0 in range(0, T, FP8_RUN):
        xr, dr = X[r0:r0 + FP8_RUN], dY[r0:r0 + FP8_RUN]
        if exact_max:
            P = dr[:, :, None] * xr[:, None, :]
            top = P.max(axis=0)
        else:
            top = np.outer(dr.max(axis=0), xr.max(axis=0))
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(top > 0, top, 1.0)))
        step = np.where(top > 0, np.exp2(e - FP8_DOT_BITS + 1), 0.0)
        if exact_max:
            sq += (np.minimum(P, step) ** 2).sum(axis=0)
        else:
            sq += xr.shape[0] * step * step
    return 4.0 * np.sqrt(sq) * abs(float(x_scale) * float(dy_scale))


def study(d_in: int = 256, d_out: int = 256, T: int = 1024, steps: int = 8, seed: int = 31,
          x_fmt: str = E4M3, dy_fmt: str = E5M2, lr: float = 1e-3, beta1: float = 0.9,
          beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01) -> dict:
    """fp8 inputs against bf16 inputs (P6's fp8 row vs its baseline).

    The same float32 draws (X, dY ~ N(0, 1)) are encoded as bf16 (baseline)
    and as fp8 with power-of-two per-tensor scales; each run takes the
    oracle's float32 AdamW steps on its own gradients. Reference: the exact
    gradient of the float32 draws and float64 AdamW. Reported: normwise
    relative errors of the step-1 gradient and of the total parameter change,
    and their fp8 / bf16 ratios. The page gives the ratio (44x) but not its
    setup or measure; this is our reading.
    """
    from synth import bf16_bits_from_f32, fp8_inputs, normal_f32   # seeded inputs only
    from .precision_study import normwise
    from .ref import adamw_step, adamw_step_f64, wgrad

    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
    W0 = normal_f32(seed, (d_out, d_in), 0.02)
    Wb, mb, vb = W0.copy(), np.zeros_like(W0), np.zeros_like(W0)
    W8, m8, v8 = W0.copy(), np.zeros_like(W0), np.zeros_like(W0)
    Wr, mr, vr = W0.astype(np.float64), np.zeros(W0.shape), np.zeros(W0.shape)
    g_err = {}
    for t in range(1, steps + 1):
        X = normal_f32(seed + 2 * t, (T, d_in))
        dY = normal_f32(seed + 2 * t + 1, (T, d_out))
        g_ref = dY.astype(np.float64).T @ X.astype(np.float64)
        g_b = wgrad(bf16_bits_from_f32(X), bf16_bits_from_f32(dY))
        X8, sx, dY8, sdy = fp8_inputs(X, dY, x_fmt, dy_fmt)
        g_8 = wgrad_fp8(X8, x_fmt, sx, dY8, dy_fmt, sdy)
        if t == 1:
            g_err = {"bf16": normwise(g_b, g_ref), "fp8": normwise(g_8, g_ref)}
        Wb, mb, vb = adamw_step(Wb, mb, vb, g_b, t, **hp)
        W8, m8, v8 = adamw_step(W8, m8, v8, g_8, t, **hp)
        Wr, mr, vr = adamw_step_f64(Wr, mr, vr, g_ref, t, **hp)
    dref = Wr - W0.astype(np.float64)
    err = {"bf16": normwise(Wb.astype(np.float64) - W0, dref),
           "fp8": normwise(W8.astype(np.float64) - W0, dref)}
    return {"grad_error": g_err, "update_error": err,
            "ratio_grad": g_err["fp8"] / g_err["bf16"], "ratio_update": err["fp8"] / err["bf16"],
            "setup": dict(d_in=d_in, d_out=d_out, T=T, steps=steps, seed=seed, x_fmt=x_fmt,
                          dy_fmt=dy_fmt, **hp)}


if __name__ == "__main__":   # pragma: no cover - prints the numbers quoted in the design notes
    for fx, fy in ((E4M3, E5M2), (E4M3, E4M3), (E5M2, E5M2)):
        r = study(x_fmt=fx, dy_fmt=fy)
        print(f"X {fx} dY {fy}: gradient error bf16 {r['grad_error']['bf16']:.3e} fp8 "
              f"{r['grad_error']['fp8']:.3e} ratio {r['ratio_grad']:.1f}x; update error bf16 "
              f"{r['update_error']['bf16']:.3e} fp8 {r['update_error']['fp8']:.3e} ratio "
              f"{r['ratio_update']:.1f}x")
