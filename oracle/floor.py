"""Accumulation floor: how far a correct float32-accumulated gradient may sit
from the oracle's correctly rounded one, and how that gap carries into the
optimizer state.

TEST INFRASTRUCTURE ONLY. Any summation order of T float32 additions is a
correct weight gradient; the page fixes none. With unit roundoff u = 2^-24 and
s[o, i] = sqrt(sum_t (dY[t, o] X[t, i])^2), a random-walk estimate of the
error of a float32 running sum is u sqrt(T) s; the floor takes four times it:

    tau[o, i] = 4 * 2^-24 * sqrt(T) * s[o, i]

and carries it through the moment recurrences
    m_err_t = beta1 m_err_{t-1} + (1 - beta1) tau_t
    v_err_t = beta2 v_err_{t-1} + (1 - beta2) (2 |g_t| tau_t + tau_t^2)
(SGD-momentum: b_err_t = momentum b_err_{t-1} + tau_t).
"""
from __future__ import annotations

import numpy as np

from .ref import bf16_bits_to_f64

U32 = 2.0 ** -24


def acc_floor(X_bits: np.ndarray, dY_bits: np.ndarray) -> np.ndarray:
    """tau in the weight's [d_out, d_in] layout (float64)."""
    X = bf16_bits_to_f64(X_bits)
    dY = bf16_bits_to_f64(dY_bits)
    T = X.shape[0]
    s2 = (dY * dY).T @ (X * X)
    return 4.0 * U32 * np.sqrt(max(T, 1)) * np.sqrt(s2)


def dgrad_floor(dY_bits: np.ndarray, W) -> np.ndarray:
    """tau of the input gradient dX = dY W_b (a float32 sum over the d_out
    outputs), in dX's [T, d_in] layout (float64)."""
    from .ref import bf16_round
    Wb = bf16_round(np.asarray(W, dtype=np.float32)).astype(np.float64)
    dY = bf16_bits_to_f64(dY_bits)
    K = Wb.shape[0]
    s2 = (dY * dY) @ (Wb * Wb)
    return 4.0 * U32 * np.sqrt(max(K, 1)) * np.sqrt(s2)


def acc_floor_rows(X_bits: np.ndarray, dY_bits: np.ndarray, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    return acc_floor(X_bits, np.ascontiguousarray(dY_bits[:, rows]))


class StateFloor:
    """Propagated floors for the optimizer state of one tensor (or a sample).

    Also keeps each element's gradient and floor history (float32), from which
    the AdamW judgment forms the first-order sensitivity of the update to
    every past gradient."""

    def __init__(self, shape, kind: str = "adamw", beta1: float = 0.9, beta2: float = 0.999,
                 momentum: float = 0.9):
        self.kind = kind
        self.beta1, self.beta2, self.momentum = beta1, beta2, momentum
        self.m_err = np.zeros(shape, dtype=np.float64)
        self.v_err = np.zeros(shape, dtype=np.float64)
        self.g_hist: list = []
        self.tau_hist: list = []

    def update(self, tau: np.ndarray, g_ref: np.ndarray, arith=None) -> None:
        """One step's floors. arith: the rounding floor of the step's own
        float32 state arithmetic (sgdm_arith_floor), carried on like tau."""
        tau = np.asarray(tau, dtype=np.float64)
        self.g_hist.append(np.asarray(g_ref, dtype=np.float32))
        self.tau_hist.append(tau.astype(np.float32))
        if self.kind == "adamw":
            g = np.abs(np.asarray(g_ref, dtype=np.float64))
            self.m_err = self.beta1 * self.m_err + (1.0 - self.beta1) * tau
            self.v_err = self.beta2 * self.v_err + (1.0 - self.beta2) * (2.0 * g * tau + tau * tau)
        elif self.kind == "sgdm":
            self.m_err = self.momentum * self.m_err + tau
        else:
            raise ValueError(self.kind)
        if arith is not None:
            self.m_err = self.m_err + np.asarray(arith, dtype=np.float64)


def sgdm_arith_floor(b_prev, g, W_prev, momentum: float, weight_decay: float) -> np.ndarray:
    """Rounding floor of one float32 momentum update b = momentum b + (g + wd W)
    itself: whatever the order or fusion of its multiply-adds, each of at most
    three roundings is within u of a term no larger than momentum |b| + |g| +
    wd |W|; 4 u times that sum bounds them (the moment floor of the mixed
    AdamW judgment has the same form). It matters where the terms cancel,
    e.g. a routed expert with no tokens whose decay and momentum history
    nearly balance."""
    return 4.0 * U32 * (momentum * np.abs(np.asarray(b_prev, dtype=np.float64))
                        + np.abs(np.asarray(g, dtype=np.float64))
                        + weight_decay * np.abs(np.asarray(W_prev, dtype=np.float64)))
