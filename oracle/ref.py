"""Plain CPU definition of the weight gradient and the optimizer steps.

TEST INFRASTRUCTURE ONLY (see the package docstring). numpy; float64 for the
contraction, float32 for the optimizer step, each float32 operation rounded
as numpy rounds it. No tiling, no fusion, no reordering.

Page cited throughout: "docs(audit): FORGE assessment + residency-aware
epilogue-fusion track" (Tessera PR 565), hereafter "the FORGE assessment".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


class ClipNotFusable(ValueError):
    """Raised for any global-norm clipping request.

    The FORGE assessment, "Math verified, not asserted", P2: exact global-norm
    clipping cannot be fused into the epilogue (the clipped first moment
    differs from the unclipped one by a term in the previous moment, which
    needs the whole gradient's norm first), so a clip request must fail closed.
    """


def _check_clip(max_grad_norm) -> None:
    if max_grad_norm is None:
        return
    x = float(max_grad_norm)
    if x != x or x < 0.0:
        raise ValueError("max_grad_norm must be 0 (no clipping) or positive")
    if x > 0.0:
        raise ClipNotFusable("global-norm clipping cannot be fused into the weight-gradient "
                             "epilogue; run clipping unfused or disable it")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# the contraction
# --------------------------------------------------------------------------
def wgrad(X_bits: np.ndarray, dY_bits: np.ndarray) -> np.ndarray:
    """Weight gradient in the weight's [d_out, d_in] layout, float32.

    The FORGE assessment, "What's already in tree and easy to miss": the weight
    gradient is the matmul of the forward input and the output gradient with
    the input transposed, reduced over every token; "K kept whole" means one
    complete reduction per element. Here g[o, i] = sum_t dY[t, o] * X[t, i],
    summed in float64 (each bf16 x bf16 product is exact in float64) and
    rounded once to float32, round-to-nearest-even.
    """
    X = bf16_bits_to_f64(X_bits)
    dY = bf16_bits_to_f64(dY_bits)
    if X.shape[0] != dY.shape[0]:
        raise ValueError("X and dY must have the same number of token rows")
    return (dY.T @ X).astype(F32)


def wgrad_rows(X_bits: np.ndarray, dY_bits: np.ndarray, rows) -> np.ndarray:
    """Rows ``rows`` (output features o) of :func:`wgrad`, computed directly."""
    rows = np.asarray(rows, dtype=np.int64)
    X = bf16_bits_to_f64(X_bits)
    dY = bf16_bits_to_f64(np.ascontiguousarray(dY_bits[:, rows]))
    return (dY.T @ X).astype(F32)


def dgrad_f64(dY_bits: np.ndarray, W) -> np.ndarray:
    """The input gradient dX = dY W of the same linear layer, in float64, not
    rounded: dX[t, i] = sum_o dY[t, o] * W_b[o, i], with W_b the weight
    rounded to bf16 (the operand precision of the layer's bf16 matmuls; W is
    the float32 master weight).

    FORGE assessment, "Math verified, not asserted", P1: the update happens in
    place, so dX must be formed from the weight as it was before the step (the
    in-place dX-before-update hazard). Each bf16 x bf16 product is exact in
    float64.
    """
    Wb = bf16_round(np.asarray(W, dtype=F32)).astype(np.float64)
    dY = bf16_bits_to_f64(dY_bits)
    if dY.shape[1] != Wb.shape[0]:
        raise ValueError("dY has d_out columns, W has d_out rows")
    return dY @ Wb


def dgrad(dY_bits: np.ndarray, W) -> np.ndarray:
    """dgrad_f64 rounded once to float32 (round to nearest, ties to even)."""
    return dgrad_f64(dY_bits, W).astype(F32)


def grouped_wgrad(X_perm_bits: np.ndarray, dY_perm_bits: np.ndarray, offsets,
                  rows=None) -> list:
    """Per-expert gradients: expert e contracts routed rows offsets[e]..offsets[e+1).

    An expert with no rows has an exactly zero gradient. ``rows`` optionally
    restricts every expert's output to those output features.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    out = []
    d_in = X_perm_bits.shape[1]
    d_out = dY_perm_bits.shape[1]
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        n_o = d_out if rows is None else len(rows)
        if b == a:
            out.append(np.zeros((n_o, d_in), dtype=F32))
        elif rows is None:
            out.append(wgrad(X_perm_bits[a:b], dY_perm_bits[a:b]))
        else:
            out.append(wgrad_rows(X_perm_bits[a:b], dY_perm_bits[a:b], rows))
    return out


# --------------------------------------------------------------------------
# AdamW (decoupled weight decay), float32
# --------------------------------------------------------------------------
def adamw_moments(m, v, g, beta1: float, beta2: float):
    """First and second moments after one step, float32.

    m_t = beta1 m_{t-1} + (1 - beta1) g_t ;  v_t = beta2 v_{t-1} + (1 - beta2) g_t^2
    """
    m = np.asarray(m, dtype=F32)
    v = np.asarray(v, dtype=F32)
    g = np.asarray(g, dtype=F32)
    m_new = F32(beta1) * m + F32(1.0 - beta1) * g
    v_new = F32(beta2) * v + F32(1.0 - beta2) * (g * g)
    return m_new, v_new


def adamw_param(W, m_new, v_new, step: int, lr: float, beta1: float, beta2: float,
                eps: float, weight_decay: float):
    """Parameter update of AdamW from the new moments, float32.

    Bias-corrected moments m_hat = m_t / (1 - beta1^t), v_hat = v_t / (1 - beta2^t)
    (the corrections formed in float64, then rounded to float32), and the
    decoupled decay applied to the previous weight, scaled by the step size:
        W_t = W_{t-1} - lr * ( m_hat / (sqrt(v_hat) + eps) + weight_decay * W_{t-1} )
    """
    if step < 1:
        raise ValueError("step is 1-based")
    W = np.asarray(W, dtype=F32)
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    m_hat = np.asarray(m_new, dtype=F32) / F32(bc1)
    v_hat = np.asarray(v_new, dtype=F32) / F32(bc2)
    upd = m_hat / (np.sqrt(v_hat) + F32(eps)) + F32(weight_decay) * W
    return W - F32(lr) * upd


def adamw_step(W, m, v, g, step: int, lr: float = 1e-3, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01,
               max_grad_norm: float = 0.0):
    """One unfused AdamW step. Returns new (W, m, v); inputs are not modified.

    The FORGE assessment, introduction: the optimizer consumes the tile's
    float32 gradient; "Claim hygiene on the source": AdamW is one of the two
    released optimizers. The page gives no formula: this is the decoupled
    weight-decay form with bias correction and eps added to sqrt(v_hat).
    """
    _check_clip(max_grad_norm)
    m_new, v_new = adamw_moments(m, v, g, beta1, beta2)
    W_new = adamw_param(W, m_new, v_new, step, lr, beta1, beta2, eps, weight_decay)
    return W_new, m_new, v_new


# --------------------------------------------------------------------------
# Precision variants (FORGE assessment, "What's already in tree and easy to
# miss": the existing lowering truncates the float32 accumulator to bf16;
# "Math verified, not asserted", P6: float32 vs bf16 gradient and state)
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), as float32.

    bf16 keeps the top 16 bits of the float32 pattern; rounding adds half of
    the dropped part, plus one if the kept part is odd, before truncating.
    The exponent range is float32's, so the same bit arithmetic rounds
    subnormals and overflows to infinity correctly. NaN stays NaN (quiet).
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=F32))
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(F32).copy()
    nan = np.isnan(a)
    out[nan] = a[nan]
    return out


def adamw_step_mixed(W, m, v, g, step: int, grad_bf16: bool, state_bf16: bool,
                     lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.01):
    """One AdamW step with a bf16-rounded gradient and/or bf16 moments.

    grad_bf16: the gradient is rounded to bf16 before the step (the unfused
    path that stores a bf16 gradient). state_bf16: m, v hold bf16 values; the
    step computes the new float32 moments, updates W from them, and stores
    them rounded to bf16. Otherwise the float32 step of adamw_step.
    """
    g = bf16_round(g) if grad_bf16 else np.asarray(g, dtype=F32)
    m_new, v_new = adamw_moments(m, v, g, beta1, beta2)
    W_new = adamw_param(W, m_new, v_new, step, lr, beta1, beta2, eps, weight_decay)
    if state_bf16:
        m_new, v_new = bf16_round(m_new), bf16_round(v_new)
    return W_new, m_new, v_new


def wgrad_f64(X_bits: np.ndarray, dY_bits: np.ndarray) -> np.ndarray:
    """The weight gradient in float64, not rounded (precision reference)."""
    return bf16_bits_to_f64(dY_bits).T @ bf16_bits_to_f64(X_bits)


def adamw_step_f64(W, m, v, g, step: int, lr: float = 1e-3, beta1: float = 0.9,
                   beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01):
    """AdamW in float64 throughout (the reference the precision variants are
    measured against); same formula as adamw_step."""
    W = np.asarray(W, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    return W - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * W), m, v


# --------------------------------------------------------------------------
# SGD with momentum, float32
# --------------------------------------------------------------------------
def sgdm_step(W, b, g, lr: float = 1e-3, momentum: float = 0.9, weight_decay: float = 0.0,
              max_grad_norm: float = 0.0):
    """One unfused SGD-momentum step. Returns new (W, b).

    The FORGE assessment, "Claim hygiene on the source": SGD is the other
    released optimizer. Coupled weight decay, no dampening, no Nesterov:
        d_t = g_t + weight_decay * W_{t-1};  b_t = momentum * b_{t-1} + d_t;
        W_t = W_{t-1} - lr * b_t              (b_0 = 0)
    """
    _check_clip(max_grad_norm)
    W = np.asarray(W, dtype=F32)
    b = np.asarray(b, dtype=F32)
    g = np.asarray(g, dtype=F32)
    d = g + F32(weight_decay) * W
    b_new = F32(momentum) * b + d
    return W - F32(lr) * b_new, b_new


# --------------------------------------------------------------------------
# routed experts
# --------------------------------------------------------------------------
def grouped_adamw_step(W, m, v, grads, step: int, **hp):
    """AdamW on every expert, including experts that received no tokens.

    The FORGE assessment, "Math verified, not asserted", P5: an expert that
    gets no tokens runs no contraction, yet its moments must still decay (a
    zero gradient step); skipping it is the error the page quantifies. So every
    expert takes the same step t with g_e = 0 when it is empty.
    """
    W_out, m_out, v_out = [], [], []
    for e in range(len(grads)):
        a, b_, c = adamw_step(W[e], m[e], v[e], grads[e], step, **hp)
        W_out.append(a)
        m_out.append(b_)
        v_out.append(c)
    return np.stack(W_out), np.stack(m_out), np.stack(v_out)


def grouped_sgdm_step(W, b, grads, **hp):
    """SGD-momentum on every expert, including experts that received no
    tokens (P5 as for AdamW): with g_e = 0 the coupled decay still moves the
    buffer (b' = momentum b + weight_decay W) and so the weight."""
    W_out, b_out = [], []
    for e in range(len(grads)):
        w_new, b_new = sgdm_step(W[e], b[e], grads[e], **hp)
        W_out.append(w_new)
        b_out.append(b_new)
    return np.stack(W_out), np.stack(b_out)
