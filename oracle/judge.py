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
        |dW_gpu - dW_ref| <= 1e-3 lr
    except at step 1 where |g_ref| <= tau (the sign of g is not determined
    by a correct float32 sum there); those elements get 2 lr + 1e-3 lr and
    are counted.
  * SGD-momentum weight delta: dW = -lr b, so the floor of b carries over:
        |dW_gpu - dW_ref| <= 1e-3 lr + lr (b_err + 1e-6 |b_ref|)
  * epilogue consistency (AdamW): the oracle's float32 parameter update
    applied to the GPU's own W_{t-1}, m_t, v_t must land within 1e-3 lr of the
    GPU's W_t, on every element.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .ref import adamw_param

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


def judge_adamw(step, W_prev_gpu, W_gpu, m_gpu, v_gpu, W_prev_ref, W_ref, m_ref, v_ref,
                g_ref, tau, floor, lr, beta1, beta2, eps, weight_decay) -> Report:
    checks = {}
    ok = True
    ok &= _check("m", np.abs(_f64(m_gpu) - _f64(m_ref)),
                 REL_STATE * np.abs(_f64(m_ref)) + floor.m_err, checks)
    ok &= _check("v", np.abs(_f64(v_gpu) - _f64(v_ref)),
                 REL_STATE * np.abs(_f64(v_ref)) + floor.v_err, checks)
    d_gpu = _f64(W_gpu) - _f64(W_prev_gpu)
    d_ref = _f64(W_ref) - _f64(W_prev_ref)
    bound = np.full(d_gpu.shape, ABS_DW * lr)
    if step == 1:
        s1 = np.abs(_f64(g_ref)) <= _f64(tau)
        bound[s1] = 2.0 * lr + ABS_DW * lr
        checks["S1"] = int(np.count_nonzero(s1))
    ok &= _check("dW", np.abs(d_gpu - d_ref), bound, checks)
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
