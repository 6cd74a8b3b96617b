"""Pins of the oracle's precision variants: bf16 rounding, AdamW with a bf16
gradient or bf16 moments, the float64 reference step, and the P6 study
(page "docs(audit): FORGE assessment + residency-aware epilogue-fusion track",
sections "What's already in tree and easy to miss" and "Math verified, not
asserted", P6).

The rounding is checked against hand-picked bit patterns (ties, subnormals,
overflow), against a brute-force nearest-neighbour choice and against
torch's float-to-bfloat16 conversion; the optimizer variants against steps
worked by hand in exact arithmetic.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import judge, precision_study
from synth import normal_bf16, normal_f32
from tests.test_oracle_pins import bf16_fraction, fraction_to_f32

F32 = np.float32


def f32_from_bits(u):
    return np.array(u, dtype=np.uint32).view(F32)


def bits32(a):
    return np.ascontiguousarray(a, dtype=F32).view(np.uint32)


@pytest.mark.parametrize("x_bits,expect_bits", [
    (0x3F808000, 0x3F800000),   # 1 + 2^-8: tie, kept part even -> down
    (0x3F818000, 0x3F820000),   # 1 + 3*2^-8: tie, kept part odd -> up
    (0x3F808001, 0x3F810000),   # just above the tie -> up
    (0x3F807FFF, 0x3F800000),   # just below the tie -> down
    (0xBF818000, 0xBF820000),   # sign does not change the rule
    (0x7F7F0000, 0x7F7F0000),   # largest finite bf16 is kept
    (0x7F7FFFFF, 0x7F800000),   # past the largest bf16 + half a step -> inf
    (0x7F7F7FFF, 0x7F7F0000),   # below the half step -> largest finite
    (0x00018000, 0x00020000),   # subnormal tie, odd -> up
    (0x00008000, 0x00000000),   # subnormal tie, even -> zero
    (0x00008001, 0x00010000),   # smallest bf16 subnormal
    (0x80000000, 0x80000000),   # -0 keeps its sign
    (0x7F800000, 0x7F800000),   # inf
])
def test_bf16_round_bit_patterns(x_bits, expect_bits):
    got = oracle.bf16_round(f32_from_bits([x_bits]))
    assert int(bits32(got)[0]) == expect_bits


def test_bf16_round_nan_stays_nan():
    got = oracle.bf16_round(np.array([np.nan, -np.nan], F32))
    assert np.all(np.isnan(got))


def _nearest_bf16_bruteforce(x: np.ndarray) -> np.ndarray:
    """Pick between the two bf16 values around x by distance (float64 holds
    both differences exactly); ties go to the even 7-bit fraction, and the
    step past the largest finite value is 2^128 (rounds to infinity)."""
    u = bits32(x).astype(np.int64)
    lo_bits = u & 0xFFFF0000                      # toward zero
    hi_bits = lo_bits + 0x10000                   # next bf16 away from zero
    lo = lo_bits.astype(np.uint32).view(F32).astype(np.float64)
    hi = hi_bits.astype(np.uint32).view(F32).astype(np.float64)
    # past the largest finite bf16 the next step is 2^128, which encodes as inf
    hi = np.where(np.isinf(hi), np.copysign(2.0 ** 128, hi), hi)
    ax = x.astype(np.float64)
    dlo, dhi = np.abs(ax - lo), np.abs(hi - ax)
    lo_even = ((lo_bits >> 16) & 1) == 0
    pick_lo = (dlo < dhi) | ((dlo == dhi) & lo_even)
    return np.where(pick_lo, lo_bits, hi_bits).astype(np.uint32)


def test_bf16_round_matches_bruteforce_over_all_exponents():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]         # finite only
    u[:256] = (u[:256] & 0xFFFF0000) | 0x8000     # exact ties
    x = u.view(F32)
    got = bits32(oracle.bf16_round(x))
    assert np.array_equal(got, _nearest_bf16_bruteforce(x))


def test_bf16_round_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]
    x = u.view(F32)
    t = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bits32(oracle.bf16_round(x)), bits32(t))


def test_mixed_adamw_hand_worked_bf16_state():
    # beta1 = 1/2, beta2 = 3/4, lr = 1/10, eps = 0, weight_decay = 0, W0 = 2,
    # g1 = 1 + 2^-6 + 2^-7 (a bf16 value), g2 = 0. Worked by hand:
    #   t=1: m = g/2 = 0.51171875 (bf16 exact), v = g^2/4 = 0.2618560791015625,
    #        stored v = 0.26171875 (nearest bf16); W from the unrounded moments:
    #        m_hat / sqrt(v_hat) = g / |g| = 1, so W1 = 2 - 1/10 = 1.9
    #   t=2: from the stored state: m = 0.255859375, v = 0.1962890625,
    #        m_hat = m / (3/4), v_hat = v / (7/16), W2 = 1.9 - m_hat / sqrt(v_hat) / 10
    hp = dict(lr=0.1, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.0)
    g = F32(1 + 2 ** -6 + 2 ** -7)
    W, m, v = np.array([2.0], F32), np.zeros(1, F32), np.zeros(1, F32)
    W, m, v = oracle.adamw_step_mixed(W, m, v, np.array([g]), 1, False, True, **hp)
    assert W[0] == F32(1.9) and m[0] == 0.51171875 and v[0] == 0.26171875
    W, m, v = oracle.adamw_step_mixed(W, m, v, np.zeros(1, F32), 2, False, True, **hp)
    assert m[0] == 0.255859375 and v[0] == 0.1962890625
    expect = 1.9 - (0.255859375 / 0.75) / math.sqrt(0.1962890625 / 0.4375) / 10
    assert abs(float(W[0]) - expect) <= 2.5e-7


def test_mixed_adamw_hand_worked_bf16_gradient():
    # g = 1 + 2^-8 + 2^-20 rounds to 1 + 2^-7 before the step; with
    # beta1 = 1/2, beta2 = 3/4 the moments are g_r/2 and g_r^2/4 exactly
    hp = dict(lr=0.1, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.5)
    g = np.array([1 + 2 ** -8 + 2 ** -20], F32)
    gr = 1 + 2 ** -7
    W, m, v = oracle.adamw_step_mixed(np.array([2.0], F32), np.zeros(1, F32), np.zeros(1, F32),
                                      g, 1, True, False, **hp)
    assert m[0] == gr / 2 and v[0] == F32(gr * gr / 4)
    assert W[0] == F32(2 - (1 + 0.5 * 2) / 10)
    # the float32 path keeps the unrounded gradient
    _, m32, _ = oracle.adamw_step_mixed(np.array([2.0], F32), np.zeros(1, F32), np.zeros(1, F32),
                                        g, 1, False, False, **hp)
    assert m32[0] == F32(g[0] / 2)


def test_f64_step_hand_worked():
    # the hand-worked steps of the float32 pin, now to float64 accuracy
    hp = dict(lr=0.1, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.5)
    expect = [9 / 5, 171 / 100, 171 / 100 - ((4 / 7) / math.sqrt(208 / 37) + 171 / 200) / 10]
    W, m, v = np.array([2.0]), np.zeros(1), np.zeros(1)
    for t, g in enumerate([4.0, -2.0, 1.0], start=1):
        W, m, v = oracle.adamw_step_f64(W, m, v, np.array([g]), t, **hp)
        assert W.dtype == np.float64
        assert abs(W[0] - expect[t - 1]) <= 1e-15 * abs(expect[t - 1]), t


def test_f64_step_sign_descent_limit():
    g = normal_f32(62, (4096,)).astype(np.float64)
    W0 = normal_f32(63, g.shape).astype(np.float64)
    z = np.zeros_like(W0)
    W1, _, _ = oracle.adamw_step_f64(W0, z, z, g, 1, lr=1e-3, beta1=0.0, beta2=0.0, eps=0.0,
                                     weight_decay=0.0)
    assert np.all(np.abs(W1 - (W0 - 1e-3 * np.sign(g))) <= 1e-18 + 1e-16 * np.abs(W0))


@pytest.mark.parametrize("T,d_in,d_out", [(1, 3, 2), (7, 5, 4), (16, 8, 8)])
def test_wgrad_f64_exact(T, d_in, d_out):
    # products of bf16 values are exact in float64; these small sums are too
    Xb = normal_bf16(90 + T, (T, d_in))
    dYb = normal_bf16(91 + T, (T, d_out))
    got = oracle.wgrad_f64(Xb, dYb)
    for o in range(d_out):
        for i in range(d_in):
            q = sum((bf16_fraction(dYb[t, o]) * bf16_fraction(Xb[t, i]) for t in range(T)),
                    Fraction(0))
            assert got[o, i] == float(q)
    # and its float32 rounding is the oracle's gradient
    assert np.array_equal(bits32(oracle.wgrad(Xb, dYb)),
                          bits32(np.array([[fraction_to_f32(Fraction(x)) for x in r]
                                           for r in got], F32)))


def test_p6_study_benefit_orders():
    """The float32 gradient is worth orders of magnitude with float32 state
    and about nothing with bf16 state (P6 gives ~900x and ~1x)."""
    res = precision_study.run()
    b = res["benefit"]
    assert b["fp32_state"]["dW"] > 300, b
    assert 0.7 < b["bf16_state"]["dW"] < 2.0, b
    for name in ("bf16_state", "bf16_both"):
        _, m, v = res["runs"][name]
        assert precision_study.bf16_state_is_representable(m)
        assert precision_study.bf16_state_is_representable(v)
    for name in ("fp32", "bf16_grad"):
        _, m, _ = res["runs"][name]
        assert not precision_study.bf16_state_is_representable(m)
    # every variant stays near the float64 run: bf16 costs ~2^-9, not more
    assert max(e["dW"] for e in res["errors"].values()) < 1e-2


# --------------------------------------------------------------------------
# the mixed-precision judgment: accepts any correct float32 accumulation order,
# rejects plausible mistakes (planted here, in CPU stand-ins)
# --------------------------------------------------------------------------
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _truncate_bf16(x):
    return (bits32(x) & np.uint32(0xFFFF0000)).view(F32)


def _standin_step(W, m, v, g, t, grad_bf16, state_bf16, planted):
    """A 'GPU' step written from CPU pieces, with an optional planted mistake."""
    if planted == "w_from_rounded_state":
        g = oracle.bf16_round(g) if grad_bf16 else g
        m1, v1 = oracle.adamw_moments(m, v, g, HP["beta1"], HP["beta2"])
        m1, v1 = oracle.bf16_round(m1), oracle.bf16_round(v1)
        return oracle.adamw_param(W, m1, v1, t, **HP), m1, v1
    if planted == "truncated_state":
        W1, m1, v1 = oracle.adamw_step_mixed(W, m, v, g, t, grad_bf16, False, **HP)
        return W1, _truncate_bf16(m1), _truncate_bf16(v1)
    if planted == "gradient_not_rounded":
        return oracle.adamw_step_mixed(W, m, v, g, t, False, state_bf16, **HP)
    return oracle.adamw_step_mixed(W, m, v, g, t, grad_bf16, state_bf16, **HP)


def _judge_mixed_run(grad_bf16, state_bf16, chunk=16, planted=None, steps=3):
    from tests.test_oracle_pins import _fp32_sums
    d_in, d_out, T = 32, 24, 1024
    W = normal_f32(220, (d_out, d_in), 0.02)
    m, v = np.zeros_like(W), np.zeros_like(W)
    reps = []
    for t in range(1, steps + 1):
        Xb = normal_bf16(230 + t, (T, d_in))
        dYb = normal_bf16(240 + t, (T, d_out))
        g = _fp32_sums(Xb, dYb, chunk)
        W1, m1, v1 = _standin_step(W, m, v, g, t, grad_bf16, state_bf16, planted)
        reps.append(judge.judge_adamw_mixed(t, W, m, v, W1, m1, v1, oracle.wgrad(Xb, dYb),
                                            oracle.acc_floor(Xb, dYb), grad_bf16, state_bf16,
                                            **HP))
        W, m, v = W1, m1, v1
    return reps


@pytest.mark.parametrize("grad_bf16,state_bf16", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("chunk", [1, 64])
def test_mixed_judge_accepts_fp32_accumulation_orders(grad_bf16, state_bf16, chunk):
    for r in _judge_mixed_run(grad_bf16, state_bf16, chunk):
        assert r.passed, str(r)


@pytest.mark.parametrize("grad_bf16,state_bf16,planted", [
    (False, True, "w_from_rounded_state"),
    (True, True, "w_from_rounded_state"),
    (False, True, "truncated_state"),
    (True, False, "gradient_not_rounded"),
    (True, True, "gradient_not_rounded"),
])
def test_mixed_judge_rejects_planted_mistakes(grad_bf16, state_bf16, planted):
    assert not all(r.passed for r in _judge_mixed_run(grad_bf16, state_bf16, planted=planted))


def test_bf16_bracket_contains_both_roundings():
    g = normal_f32(250, (4096,))
    tau = np.abs(g).astype(np.float64) * 2.0 ** -10
    lo, hi = judge.bf16_bracket(g - tau, g + tau)
    assert np.all(lo <= oracle.bf16_round(g)) and np.all(oracle.bf16_round(g) <= hi)
    assert np.any(lo < hi)
    lo0, hi0 = judge.bf16_bracket(g.astype(np.float64), g.astype(np.float64))
    assert np.array_equal(bits32(lo0), bits32(oracle.bf16_round(g)))
    assert np.array_equal(bits32(hi0), bits32(lo0))


@pytest.mark.parametrize("state_bf16", [False, True])
def test_mixed_judge_accepts_fused_multiply_add_moments(state_bf16):
    """Exact gradient (floor 0): moments formed with one rounding of
    beta m + ((1 - beta) g), as a fused multiply-add does, still pass where
    the two terms cancel."""
    n = 1 << 16
    W = normal_f32(260, (n,), 0.02)
    m = normal_f32(261, (n,), 0.1)
    v = np.abs(normal_f32(262, (n,), 1e-2))
    g = normal_f32(263, (n,))
    g[:64] = (-F32(HP["beta1"]) * m[:64] / F32(1 - HP["beta1"])).astype(F32)   # cancellation
    if state_bf16:
        m, v = oracle.bf16_round(m), oracle.bf16_round(v)
    b1, c1 = F32(HP["beta1"]), F32(1 - HP["beta1"])
    b2, c2 = F32(HP["beta2"]), F32(1 - HP["beta2"])
    m1 = (b1.astype(np.float64) * m + (c1 * g).astype(np.float64)).astype(F32)
    v1 = (b2.astype(np.float64) * v + (c2 * (g * g)).astype(np.float64)).astype(F32)
    W1 = oracle.adamw_param(W, m1, v1, 5, **HP)
    if state_bf16:
        m1, v1 = oracle.bf16_round(m1), oracle.bf16_round(v1)
    rep = judge.judge_adamw_mixed(5, W, m, v, W1, m1, v1, g, np.zeros(n), False, state_bf16, **HP)
    assert rep.passed, str(rep)
