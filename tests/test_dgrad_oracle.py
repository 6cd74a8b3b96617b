"""Pins of the oracle's input gradient dX = dY W_b and of its judgment (page
"docs(audit): FORGE assessment + residency-aware epilogue-fusion track",
section "Math verified, not asserted", P1: the in-place dX-before-update
hazard).

Exact rational brute force on tiny shapes, a hand-worked example that fixes
the orientation, the bf16 rounding of the weight operand, the accumulation
floor against real float32 sums, and planted mistakes the judgment must
reject (dX from the updated weight, a transposed weight, the float32 weight
used without rounding).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import judge
from synth import normal_bf16, normal_f32
from tests.test_oracle_pins import bf16_fraction
from tests.test_precision_oracle import _nearest_bf16_bruteforce

F32 = np.float32


def _bf16_bits_of_rounded(W):
    """bf16 bit patterns of W rounded to nearest (brute-force neighbour choice)."""
    return (_nearest_bf16_bruteforce(np.asarray(W, F32)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("T,d_in,d_out", [(1, 3, 2), (4, 5, 8), (6, 8, 7)])
def test_dgrad_exact_bruteforce(T, d_in, d_out):
    dYb = normal_bf16(400 + T, (T, d_out))
    W = normal_f32(401 + T, (d_out, d_in), 0.5)
    Wq = _bf16_bits_of_rounded(W)
    got = oracle.dgrad_f64(dYb, W)
    for t in range(T):
        for i in range(d_in):
            q = sum((bf16_fraction(dYb[t, o]) * bf16_fraction(Wq[o, i]) for o in range(d_out)),
                    Fraction(0))
            assert got[t, i] == float(q)
    assert got.shape == (T, d_in)


def test_dgrad_orientation_hand_worked():
    # dY = [[1, 2]] (one token, d_out = 2), W = [[1, 0, 3], [0, 1, 0]]:
    # dX[0, i] = 1 W[0, i] + 2 W[1, i] = [1, 2, 3]
    one, two = 0x3F80, 0x4000
    dYb = np.array([[one, two]], dtype=np.uint16)
    W = np.array([[1, 0, 3], [0, 1, 0]], F32)
    assert np.array_equal(oracle.dgrad(dYb, W), np.array([[1, 2, 3]], F32))


def test_dgrad_rounds_the_weight_to_bf16():
    # W = 1 + 2^-10 is not a bf16 value; the operand is 1
    dYb = np.array([[0x3F80]], dtype=np.uint16)
    W = np.array([[1 + 2 ** -10]], F32)
    assert oracle.dgrad(dYb, W)[0, 0] == 1.0


def _fp32_rowsums(dYb, W, chunk):
    """A float32 sum over d_out in ascending chunks (a GPU-like order)."""
    dY = oracle.bf16_bits_to_f64(dYb).astype(F32)
    Wb = oracle.bf16_round(W)
    acc = np.zeros((dY.shape[0], W.shape[1]), F32)
    for k0 in range(0, W.shape[0], chunk):
        acc = (acc + (dY[:, k0:k0 + chunk].astype(np.float64)
                      @ Wb[k0:k0 + chunk].astype(np.float64)).astype(F32)).astype(F32)
    return acc


@pytest.mark.parametrize("chunk", [1, 16])
def test_dgrad_floor_bounds_fp32_accumulation(chunk):
    dYb = normal_bf16(410, (48, 2048), 1e-2)
    W = normal_f32(411, (2048, 40), 0.02)
    got = _fp32_rowsums(dYb, W, chunk)
    err = np.abs(got.astype(np.float64) - oracle.dgrad_f64(dYb, W))
    tau = oracle.dgrad_floor(dYb, W)
    assert np.all(err <= tau)
    assert np.max(err / tau) > 0.05        # at most 20x the largest real error (0.10-0.39 here)
    # a bf16-rounded dX misses the floor by far more than that margin
    ref = oracle.dgrad_f64(dYb, W)
    err_bf16 = np.abs(oracle.bf16_round(ref.astype(F32)).astype(np.float64) - ref)
    assert np.mean(err_bf16 > 20 * tau) > 0.5


@pytest.mark.parametrize("bf16_out", [False, True])
def test_dgrad_judge_accepts_fp32_orders_and_rejects_mistakes(bf16_out):
    dYb = normal_bf16(420, (64, 1024))
    W = normal_f32(421, (1024, 96), 0.02)

    def out(x):
        return oracle.bf16_round(x) if bf16_out else x

    for chunk in (1, 16, 64):
        rep = judge.judge_dgrad(out(_fp32_rowsums(dYb, W, chunk)), dYb, W, bf16_out)
        assert rep.passed, str(rep)
    # dX formed from the weight after an AdamW step (the in-place hazard)
    z = np.zeros_like(W)
    W_after, _, _ = oracle.adamw_step(W, z, z, normal_f32(422, W.shape), 1)
    assert not judge.judge_dgrad(out(_fp32_rowsums(dYb, W_after, 16)), dYb, W, bf16_out).passed
    # the float32 weight used as the operand, without the bf16 rounding
    dY = oracle.bf16_bits_to_f64(dYb)
    unrounded = (dY @ W.astype(np.float64)).astype(F32)
    assert not judge.judge_dgrad(out(unrounded), dYb, W, bf16_out).passed
    # a transposed weight (square case)
    Wsq = normal_f32(423, (96, 96), 0.02)
    dYsq = normal_bf16(424, (64, 96))
    wrong = (oracle.bf16_bits_to_f64(dYsq) @ oracle.bf16_round(Wsq).T.astype(np.float64))
    assert not judge.judge_dgrad(out(wrong.astype(F32)), dYsq, Wsq, bf16_out).passed


def test_dgrad_judge_rows():
    dYb = normal_bf16(430, (40, 256))
    W = normal_f32(431, (256, 24), 0.02)
    full = _fp32_rowsums(dYb, W, 16)
    rows = [0, 7, 39]
    assert judge.judge_dgrad(full[rows], dYb, W, False, rows=rows).passed
