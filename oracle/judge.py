"""Two separate judgments of a GPU result: accuracy against the oracle, and
bitwise invariance between GPU runs. They are never mixed: a tolerance never
enters an invariance check, and bitwise equality is never asked of the GPU
against the oracle (the page "WS1 C4 (#270) Landing Plan — Gradient-invariance
harness & adapters", section 2, keeps accuracy and cross-config invariance
apart, the latter with zero tolerance).

TEST INFRASTRUCTURE ONLY.

Accuracy bar (per element, every step):
  * moments m, v (SGD: momentum buffer b):
        |x_gpu - x_ref| <= 1e-4 |x_ref| + x_err      (x_err from StateFloor)
  * AdamW per-step weight delta dW = W_t - W_{t-1}, each path on its own
    trajectory, evaluated in float64:
        |dW_gpu - dW_ref| <= 1e-3 lr + lr D
    D bounds how far the update u = m_hat / (sqrt(v_hat) + eps) can move when
    every past gradient g_s moves within its floor tau_s. To first order,
        D1 = 2 * sum_s |du/dg_s| tau_s,
        du/dg_s = du/dm (1 - beta1) beta1^(t-s) + du/dv 2 (1 - beta2) beta2^(t-s) g_s
    (the factor 2 covers second-order terms). Where the expansion is not
    valid - a moment's floor is nonzero and at least half the moment, so a
    sign or a square root near zero can move - D takes the cap 2 C_t, where C_t bounds
    |u| over all gradient histories from zero state (C_1 = 1; at step 1 this
    is exactly the elements with |g_ref| <= tau/2-ish, whose sign a correct
    float32 sum does not fix; at later steps the elements whose history sits
    at the floor, where correct orders differ by O(lr) just the same). D is
    also capped there elsewhere. Elements with D > 1e-3 are counted
    ("ambiguous"); parity tests bound their share (ambiguous_budget).
  * SGD-momentum weight delta: dW = -lr b, so the floor of b carries over:
        |dW_gpu - dW_ref| <= 1e-3 lr + lr (b_err + 1e-6 |b_ref|)
  * epilogue consistency (AdamW): the oracle's float32 parameter update
    applied to the GPU's own W_{t-1}, m_t, v_t must land within 1e-3 lr of the
    GPU's W_t, on every element.

Precision variants (bf16 gradient and/or bf16 moments; judge_adamw_mixed):
each step is judged from the same state on both sides (the GPU's previous
W, m, v), so the only input difference is the float32 accumulation floor tau.
  * bf16 gradient: rounding is monotone, so the GPU's rounded gradient lies
    between the roundings of g_ref - tau and g_ref + tau; the floor becomes
    the distance from the oracle's rounded gradient to the farther of the two.
  * moments: the float32 bar above plus the rounding of the two terms of the
    recurrence, 4 u (beta |x_prev| + (1 - beta) |y|) with u = 2^-24 (y = g or
    g^2), which a fused multiply-add and a separate product and sum may
    disagree by where the terms cancel;
  * bf16 moments: the GPU's stored moment must be one of the bf16 roundings
    of that float32 interval, i.e. it lies between the roundings of the
    interval's ends.
  * the weight delta is judged as above (W is computed from the unrounded
    new moments on both sides); the epilogue consistency check needs the
    GPU's unrounded moments and applies only with float32 state.

Input gradient dX = dY W_b (judge_dgrad): float32 output within the
accumulation floor of the exact sum; bf16 output between the bf16 roundings
of the exact sum minus and plus that floor.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .floor import U32, StateFloor, dgrad_floor
from .ref import adamw_param, adamw_step_mixed, bf16_round, dgrad_f64

REL_STATE = 1e-4
ABS_DW = 1e-3


@dataclass
class Report:
    passed: bool
    checks: dict = field(default_factory=dict)

    def __str__(self) -> str:
        parts = [f"{k}: {v}" for k, v in self.checks.items()]
        return ("PASS " if self.passed else "FAIL ") + "; ".join(parts)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _check(name, err, bound, checks):
    bad = int(np.count_nonzero(~(err <= bound)))
    checks[name] = {"fails": bad, "max_err": float(np.max(err)) if err.size else 0.0,
                    "max_ratio": float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0}
    return bad == 0


def normwise(a, ref) -> float:
    a, ref = _f64(a), _f64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a - ref))


def update_bound(t: int, beta1: float, beta2: float) -> float:
    """C_t: the largest |m_hat / sqrt(v_hat)| over all gradient histories of
    length t from zero state (Cauchy-Schwarz over the moment weights)."""
    bc1, bc2 = 1.0 - beta1 ** t, 1.0 - beta2 ** t
    tot = 0.0
    for k in range(t):                       # k = t - s steps back
        w = (1.0 - beta1) * beta1 ** k / bc1
        w2 = (1.0 - beta2) * beta2 ** k / bc2
        if w2 > 0:
            tot += w * w / w2
    return float(np.sqrt(tot)) if beta2 > 0 else 1.0


def update_floor(step, m_ref, v_ref, floor, beta1, beta2, eps, zero_start=True):
    """D: bound on |u_gpu - u_ref| from the gradient floors (see module doc)."""
    bc1, bc2 = 1.0 - beta1 ** step, 1.0 - beta2 ** step
    m = _f64(m_ref)
    v = np.maximum(_f64(v_ref), 0.0)
    s = np.sqrt(v / bc2)
    den = s + eps
    du_dm = 1.0 / (bc1 * den)
    with np.errstate(divide="ignore", invalid="ignore"):
        du_dv = np.where(s > 0, -(m / bc1) / (den * den) / (2.0 * s * bc2), 0.0)
    d1 = np.zeros_like(m)
    t = len(floor.g_hist)
    for k in range(t):                       # gradient of step k + 1
        back = t - 1 - k
        a = (1.0 - beta1) * beta1 ** back
        b = 2.0 * (1.0 - beta2) * beta2 ** back
        d1 += np.abs(du_dm * a + du_dv * b * floor.g_hist[k]) * floor.tau_hist[k]
    d = 2.0 * d1
    cap = 2.0 * update_bound(step, beta1, beta2) if zero_start else np.inf
    # (a moment with a zero floor is exact, e.g. a zero gradient from zero state)
    invalid = (((floor.m_err >= 0.5 * np.abs(m)) & (floor.m_err > 0))
               | ((floor.v_err >= 0.5 * v) & (floor.v_err > 0)))
    d = np.where(invalid, cap, np.minimum(d, cap))
    return d


def judge_adamw(step, W_prev_gpu, W_gpu, m_gpu, v_gpu, W_prev_ref, W_ref, m_ref, v_ref,
                g_ref, tau, floor, lr, beta1, beta2, eps, weight_decay,
                zero_start=True, ambiguous_budget=None, ambiguous_min=8) -> Report:
    """ambiguous_budget: if given, the step also fails when more than
    max(ambiguous_min, ambiguous_budget x elements) elements take the widened
    weight-delta bar (the set is the oracle's alone, so the budget bounds
    where a regression could hide)."""
    checks = {}
    ok = True
    ok &= _check("m", np.abs(_f64(m_gpu) - _f64(m_ref)),
                 REL_STATE * np.abs(_f64(m_ref)) + floor.m_err, checks)
    ok &= _check("v", np.abs(_f64(v_gpu) - _f64(v_ref)),
                 REL_STATE * np.abs(_f64(v_ref)) + floor.v_err, checks)
    d_gpu = _f64(W_gpu) - _f64(W_prev_gpu)
    d_ref = _f64(W_ref) - _f64(W_prev_ref)
    D = update_floor(step, m_ref, v_ref, floor, beta1, beta2, eps, zero_start)
    checks["ambiguous"] = int(np.count_nonzero(D > ABS_DW))
    if ambiguous_budget is not None:
        limit = max(int(ambiguous_min), int(ambiguous_budget * D.size))
        checks["ambiguous_limit"] = limit
        ok &= checks["ambiguous"] <= limit
    ok &= _check("dW", np.abs(d_gpu - d_ref), ABS_DW * lr + lr * D, checks)
    W_cons = adamw_param(W_prev_gpu, m_gpu, v_gpu, step, lr, beta1, beta2, eps, weight_decay)
    ok &= _check("epilogue", np.abs(_f64(W_gpu) - _f64(W_cons)),
                 np.full(d_gpu.shape, ABS_DW * lr), checks)
    checks["normwise_m"] = normwise(m_gpu, m_ref)
    checks["normwise_dW"] = normwise(d_gpu, d_ref)
    return Report(bool(ok), checks)


def judge_sgdm(W_prev_gpu, W_gpu, b_gpu, W_prev_ref, W_ref, b_ref, floor, lr) -> Report:
    checks = {}
    ok = True
    b_err = floor.m_err
    ok &= _check("b", np.abs(_f64(b_gpu) - _f64(b_ref)),
                 REL_STATE * np.abs(_f64(b_ref)) + b_err, checks)
    d_gpu = _f64(W_gpu) - _f64(W_prev_gpu)
    d_ref = _f64(W_ref) - _f64(W_prev_ref)
    bound = ABS_DW * lr + lr * (b_err + 1e-6 * np.abs(_f64(b_ref)))
    ok &= _check("dW", np.abs(d_gpu - d_ref), bound, checks)
    checks["normwise_b"] = normwise(b_gpu, b_ref)
    return Report(bool(ok), checks)


def bitwise_equal(a, b) -> bool:
    """Invariance judgment: identical float32 bit patterns, element by element."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and bool(np.array_equal(a.view(np.uint32), b.view(np.uint32)))


def _f32_toward(x64, direction):
    """Float32 values next to x64 on the given side (-1 below, +1 above)."""
    x64 = np.asarray(x64, dtype=np.float64)
    y = x64.astype(np.float32)
    if direction < 0:
        return np.where(y.astype(np.float64) > x64, np.nextafter(y, np.float32(-np.inf)), y)
    return np.where(y.astype(np.float64) < x64, np.nextafter(y, np.float32(np.inf)), y)


def bf16_bracket(lo64, hi64):
    """Smallest and largest bf16 rounding of any float32 in [lo64, hi64]."""
    return bf16_round(_f32_toward(lo64, -1)), bf16_round(_f32_toward(hi64, +1))


def _check_bracket(name, x, lo, hi, checks):
    x, lo, hi = _f64(x), _f64(lo), _f64(hi)
    bad = ~((x >= lo) & (x <= hi))
    checks[name] = {"fails": int(np.count_nonzero(bad)),
                    "max_err": float(np.max(np.maximum(lo - x, x - hi))) if x.size else 0.0}
    return not bad.any()


def judge_adamw_mixed(step, W_prev, m_prev, v_prev, W_gpu, m_gpu, v_gpu, g_ref, tau,
                      grad_bf16, state_bf16, lr, beta1, beta2, eps, weight_decay) -> Report:
    """One AdamW step of a precision variant, both sides from (W_prev, m_prev,
    v_prev); m, v arrays as float32 (bf16 values when state_bf16)."""
    checks = {}
    ok = True
    g_ref = _f64(g_ref)
    tau = _f64(tau)
    if grad_bf16:
        g_use = _f64(bf16_round(g_ref.astype(np.float32)))
        g_lo, g_hi = bf16_bracket(g_ref - tau, g_ref + tau)
        tau = np.maximum(_f64(g_hi) - g_use, g_use - _f64(g_lo))
    else:
        g_use = g_ref
    W_ref, m32, v32 = adamw_step_mixed(W_prev, m_prev, v_prev, g_ref.astype(np.float32), step,
                                       grad_bf16, False, lr, beta1, beta2, eps, weight_decay)
    floor = StateFloor(np.shape(m32), "adamw", beta1, beta2)
    floor.update(tau, g_use)
    # float32 evaluation of beta x_prev + (1 - beta) y in any order (fused or
    # not): at most a few roundings of the two terms, which matters where they
    # cancel and the relative bar alone is too tight
    arith_m = 4 * U32 * (beta1 * np.abs(_f64(m_prev)) + (1 - beta1) * np.abs(g_use))
    arith_v = 4 * U32 * (beta2 * np.abs(_f64(v_prev)) + (1 - beta2) * g_use * g_use)
    for name, x_gpu, x_ref, err in (("m", m_gpu, m32, floor.m_err + arith_m),
                                    ("v", v_gpu, v32, floor.v_err + arith_v)):
        allow = REL_STATE * np.abs(_f64(x_ref)) + err
        if state_bf16:
            lo, hi = bf16_bracket(_f64(x_ref) - allow, _f64(x_ref) + allow)
            ok &= _check_bracket(name, x_gpu, lo, hi, checks)
            checks[name + "_rounded_equal"] = float(np.mean(
                _f64(x_gpu) == _f64(bf16_round(np.asarray(x_ref, np.float32)))))
        else:
            ok &= _check(name, np.abs(_f64(x_gpu) - _f64(x_ref)), allow, checks)
    d_gpu = _f64(W_gpu) - _f64(W_prev)
    d_ref = _f64(W_ref) - _f64(W_prev)
    D = update_floor(step, m32, v32, floor, beta1, beta2, eps, zero_start=False)
    checks["ambiguous"] = int(np.count_nonzero(D > ABS_DW))
    ok &= _check("dW", np.abs(d_gpu - d_ref), ABS_DW * lr + lr * D, checks)
    if not state_bf16:
        W_cons = adamw_param(W_prev, m_gpu, v_gpu, step, lr, beta1, beta2, eps, weight_decay)
        ok &= _check("epilogue", np.abs(_f64(W_gpu) - _f64(W_cons)),
                     np.full(d_gpu.shape, ABS_DW * lr), checks)
    checks["normwise_dW"] = normwise(d_gpu, d_ref)
    return Report(bool(ok), checks)


def judge_dgrad(dX_gpu, dY_bits, W_before, bf16_out: bool, rows=None) -> Report:
    """dX (float32, or bf16 widened to float32) against the exact dY W_b,
    W_b the bf16 rounding of the weight before the step; `rows`: the token
    rows dX_gpu holds (all if None)."""
    dY_bits = np.asarray(dY_bits)
    if rows is not None:
        dY_bits = dY_bits[np.asarray(rows, dtype=np.int64)]
    ref = dgrad_f64(dY_bits, W_before)
    tau = dgrad_floor(dY_bits, W_before)
    checks = {}
    if bf16_out:
        lo, hi = bf16_bracket(ref - tau, ref + tau)
        ok = _check_bracket("dX", dX_gpu, lo, hi, checks)
        checks["dX_rounded_equal"] = float(np.mean(
            _f64(dX_gpu) == _f64(bf16_round(ref.astype(np.float32)))))
    else:
        # the float32 rounding of the exact sum is within half an ulp of it
        ulp = np.abs(ref) * 2.0 ** -24
        ok = _check("dX", np.abs(_f64(dX_gpu) - ref), tau + ulp, checks)
    checks["normwise"] = normwise(dX_gpu, ref)
    return Report(bool(ok), checks)
