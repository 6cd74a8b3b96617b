"""Pins of the CPU oracle against things other than itself: exact rational
arithmetic, closed forms of the optimizer recurrences, and invariants stated
on the page "docs(audit): FORGE assessment + residency-aware epilogue-fusion
track" (section "Math verified, not asserted").

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
transposed operand, a wrong index, a misplaced eps or bias correction) fails.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import judge
from synth import bf16_bits_from_f32, normal_bf16, normal_f32

F32 = np.float32
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


# --------------------------------------------------------------------------
# exact helpers written from the number formats' definitions
# --------------------------------------------------------------------------
def bf16_fraction(b: int) -> Fraction:
    """bfloat16: sign bit 15, 8 exponent bits (bias 127), 7 fraction bits."""
    b = int(b)
    sign = -1 if (b >> 15) & 1 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    val = Fraction(128 + f, 128)
    return sign * (val * (Fraction(1 << (e - 127)) if e >= 127 else Fraction(1, 1 << (127 - e))))


def fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to float32, to nearest, ties to even."""
    if q == 0:
        return F32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)

    def p2(k):
        return Fraction(1 << k) if k >= 0 else Fraction(1, 1 << -k)

    e = a.numerator.bit_length() - a.denominator.bit_length()
    while p2(e) > a:
        e -= 1
    while p2(e + 1) <= a:
        e += 1
    quantum = max(e, -126) - 23
    scaled = a / p2(quantum)
    n = scaled.numerator // scaled.denominator
    r = scaled - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return F32(sign * float(n * p2(quantum)))


def exact_wgrad(Xb, dYb):
    T, d_in = Xb.shape
    d_out = dYb.shape[1]
    Xq = [[bf16_fraction(Xb[t, i]) for i in range(d_in)] for t in range(T)]
    Dq = [[bf16_fraction(dYb[t, o]) for o in range(d_out)] for t in range(T)]
    out = np.zeros((d_out, d_in), dtype=F32)
    for o in range(d_out):
        for i in range(d_in):
            out[o, i] = fraction_to_f32(sum((Dq[t][o] * Xq[t][i] for t in range(T)), Fraction(0)))
    return out


def bits(a):
    return np.ascontiguousarray(a, dtype=F32).view(np.uint32)


def test_helpers_against_known_values():
    assert bf16_fraction(0x3F80) == 1
    assert bf16_fraction(0xC040) == -3
    assert bf16_fraction(0x3E80) == Fraction(1, 4)
    assert fraction_to_f32(Fraction(1, 3)) == F32(1.0) / F32(3.0)
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: goes to the even one, 1
    assert fraction_to_f32(1 + Fraction(1, 1 << 24)) == F32(1.0)
    assert fraction_to_f32(1 + Fraction(3, 1 << 24)) == F32(1.0) + F32(2.0 ** -22)


# --------------------------------------------------------------------------
# the contraction
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,d_in,d_out", [(8, 4, 4), (8, 5, 3), (13, 3, 6)])
def test_wgrad_bruteforce_exact(T, d_in, d_out):
    Xb = normal_bf16(11 + T, (T, d_in))
    dYb = normal_bf16(17 + T, (T, d_out))
    g = oracle.wgrad(Xb, dYb)
    assert g.shape == (d_out, d_in) and g.dtype == np.float32
    assert np.array_equal(bits(g), bits(exact_wgrad(Xb, dYb)))


def test_wgrad_bruteforce_cancellation():
    # rows of very different magnitude and exact cancellation
    T, d_in, d_out = 8, 4, 3
    x = normal_f32(5, (T, d_in))
    y = normal_f32(6, (T, d_out))
    x[::2] *= 2.0 ** 12
    y[1::3] *= 2.0 ** -9
    Xb, dYb = bf16_bits_from_f32(x), bf16_bits_from_f32(y)
    Xb = np.concatenate([Xb, Xb])
    dYb = np.concatenate([dYb, dYb ^ np.uint16(0x8000)])    # second half negates the first
    g = oracle.wgrad(Xb, dYb)
    assert np.array_equal(bits(g), bits(exact_wgrad(Xb, dYb)))
    assert np.all(g == 0)


def test_wgrad_rows_and_power_of_two_scaling():
    Xb = normal_bf16(21, (64, 24))
    dYb = normal_bf16(22, (64, 16))
    g = oracle.wgrad(Xb, dYb)
    rows = [0, 5, 15]
    assert np.array_equal(bits(oracle.wgrad_rows(Xb, dYb, rows)), bits(g[rows]))
    # scaling dY by 2^3 adds 3 to every bf16 exponent and scales g exactly
    dY8 = (dYb.astype(np.uint32) + (3 << 7)).astype(np.uint16)
    assert np.array_equal(bits(oracle.wgrad(Xb, dY8)), bits(g * F32(8.0)))


def test_grouped_wgrad_slices_and_empty_experts():
    Xb = normal_bf16(31, (11, 4))
    dYb = normal_bf16(32, (11, 3))
    offsets = [0, 3, 3, 11, 11]          # experts 1 and 3 receive nothing
    gs = oracle.grouped_wgrad(Xb, dYb, offsets)
    assert len(gs) == 4
    assert np.array_equal(bits(gs[0]), bits(exact_wgrad(Xb[0:3], dYb[0:3])))
    assert np.array_equal(bits(gs[2]), bits(exact_wgrad(Xb[3:11], dYb[3:11])))
    for e in (1, 3):
        assert gs[e].shape == (3, 4) and np.all(bits(gs[e]) == 0)


# --------------------------------------------------------------------------
# AdamW
# --------------------------------------------------------------------------
def _ulp(x):
    return np.spacing(np.abs(np.asarray(x, dtype=F32))).astype(np.float64)


def _adamw_probe_grad(n=4096, seed=41):
    g = normal_f32(seed, (n,))
    g[:64] *= F32(1e-8)                  # around eps: placement of eps matters here
    g[64:128] *= F32(1e-5)
    g[128:192] *= F32(1e3)
    return g


def test_adamw_step1_closed_form():
    g = _adamw_probe_grad()
    W0 = normal_f32(42, g.shape, 0.02)
    z = np.zeros_like(W0)
    W1, m1, v1 = oracle.adamw_step(W0, z, z, g, 1, **HP)
    g64, W64 = g.astype(np.float64), W0.astype(np.float64)
    assert np.all(np.abs(m1 - 0.1 * g64) <= 2 * _ulp(m1))
    assert np.all(np.abs(v1 - 0.001 * g64 * g64) <= 4 * _ulp(v1))
    expect = -HP["lr"] * g64 / (np.abs(g64) + HP["eps"]) - HP["lr"] * HP["weight_decay"] * W64
    got = W1.astype(np.float64) - W64
    assert np.all(np.abs(got - expect) <= 2 * _ulp(W1) + 1e-6 * HP["lr"])


def test_adamw_constant_gradient_every_step():
    # with g_t = c the bias-corrected moments are exactly c and c^2 at every t
    c = _adamw_probe_grad(1024, 43)
    W = normal_f32(44, c.shape, 0.02)
    m = np.zeros_like(W)
    v = np.zeros_like(W)
    hp = dict(HP, weight_decay=0.0)
    for t in range(1, 8):
        Wn, m, v = oracle.adamw_step(W, m, v, c, t, **hp)
        c64 = c.astype(np.float64)
        expect = -hp["lr"] * c64 / (np.abs(c64) + hp["eps"])
        got = Wn.astype(np.float64) - W.astype(np.float64)
        assert np.all(np.abs(got - expect) <= 2 * _ulp(Wn) + 1e-5 * hp["lr"]), t
        W = Wn


def test_adamw_moments_match_geometric_sums():
    gs = [normal_f32(50 + s, (2048,)) for s in range(6)]
    m = np.zeros(2048, F32)
    v = np.zeros(2048, F32)
    for t, g in enumerate(gs, start=1):
        m, v = oracle.adamw_moments(m, v, g, 0.9, 0.999)
        em = sum(0.1 * 0.9 ** (t - s) * gs[s - 1].astype(np.float64) for s in range(1, t + 1))
        ev = sum(0.001 * 0.999 ** (t - s) * gs[s - 1].astype(np.float64) ** 2 for s in range(1, t + 1))
        scale_m = sum(0.1 * 0.9 ** (t - s) * np.abs(gs[s - 1].astype(np.float64)) for s in range(1, t + 1))
        assert np.all(np.abs(m - em) <= 1e-6 * scale_m + 1e-30)
        assert np.all(np.abs(v - ev) <= 1e-6 * ev + 1e-30)


def test_adamw_hand_worked_steps():
    # beta1 = 1/2, beta2 = 3/4, lr = 1/10, eps = 0, weight_decay = 1/2, W0 = 2,
    # gradients 4, -2, 1 (worked by hand in exact arithmetic):
    #   t=1: m=2, v=4, m_hat=4, v_hat=16, W1 = 2 - (4/4 + 1)/10          = 9/5
    #   t=2: m=0, v=4, v_hat=64/7,      W2 = 9/5 - (0 + 9/10)/10          = 171/100
    #   t=3: m=1/2, v=13/4, m_hat=4/7, v_hat=208/37,
    #        W3 = 171/100 - (4/7 / sqrt(208/37) + 171/200)/10
    hp = dict(lr=0.1, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.5)
    W, m, v = np.array([2.0], F32), np.zeros(1, F32), np.zeros(1, F32)
    expect = [9 / 5, 171 / 100, 171 / 100 - ((4 / 7) / math.sqrt(208 / 37) + 171 / 200) / 10]
    exp_m = [2.0, 0.0, 0.5]
    exp_v = [4.0, 4.0, 3.25]
    for t, g in enumerate([4.0, -2.0, 1.0], start=1):
        W, m, v = oracle.adamw_step(W, m, v, np.array([g], F32), t, **hp)
        assert m[0] == exp_m[t - 1] and v[0] == exp_v[t - 1]
        assert abs(float(W[0]) - expect[t - 1]) <= 4e-7 * abs(expect[t - 1]), (t, W[0])


def test_adamw_sign_descent_limit():
    # beta1 = beta2 = weight_decay = 0, eps = 0: the step is -lr * sign(g)
    g = normal_f32(60, (4096,))
    W0 = normal_f32(61, g.shape)
    z = np.zeros_like(W0)
    W1, _, _ = oracle.adamw_step(W0, z, z, g, 1, lr=1e-3, beta1=0.0, beta2=0.0, eps=0.0,
                                 weight_decay=0.0)
    expect = W0.astype(np.float64) - 1e-3 * np.sign(g)
    assert np.all(np.abs(W1 - expect) <= _ulp(W1))


def test_adamw_zero_gradient_is_a_decay_step():
    # the routed-expert rule: no tokens means g = 0, and the state still moves
    W0 = normal_f32(70, (4096,), 0.02)
    m0 = normal_f32(71, W0.shape, 0.1)
    v0 = np.abs(normal_f32(72, W0.shape, 0.01))
    g = np.zeros_like(W0)
    t = 4
    W1, m1, v1 = oracle.adamw_step(W0, m0, v0, g, t, **HP)
    assert np.array_equal(bits(m1), bits(F32(0.9) * m0))
    assert np.array_equal(bits(v1), bits(F32(0.999) * v0))
    mh = 0.9 * m0.astype(np.float64) / (1 - 0.9 ** t)
    vh = 0.999 * v0.astype(np.float64) / (1 - 0.999 ** t)
    expect = W0 - 1e-3 * (mh / (np.sqrt(vh) + 1e-8) + 0.01 * W0.astype(np.float64))
    assert np.all(np.abs(W1 - expect) <= 2 * _ulp(W1) + 1e-6 * 1e-3)
    # from zero state only the decoupled decay acts
    z = np.zeros_like(W0)
    W1z, m1z, v1z = oracle.adamw_step(W0, z, z, g, 1, **HP)
    assert np.all(m1z == 0) and np.all(v1z == 0)
    assert np.all(np.abs(W1z - W0.astype(np.float64) * (1 - 1e-5)) <= _ulp(W1z))


def test_clip_identity_and_fail_closed():
    # m_t(c g) - c m_t(g) = (1 - c) beta1 m_{t-1}: a clipped first moment needs m_{t-1}
    m_prev = normal_f32(80, (2048,))
    g = normal_f32(81, m_prev.shape)
    z = np.zeros_like(g)
    for c in (0.25, 0.5, 0.9):
        mc, _ = oracle.adamw_moments(m_prev, z, F32(c) * g, 0.9, 0.999)
        m1, _ = oracle.adamw_moments(m_prev, z, g, 0.9, 0.999)
        lhs = mc.astype(np.float64) - c * m1.astype(np.float64)
        rhs = (1 - c) * 0.9 * m_prev.astype(np.float64)
        assert np.all(np.abs(lhs - rhs) <= 1e-6 * (np.abs(m_prev) + np.abs(g)))
    W = normal_f32(82, g.shape)
    W_copy = W.copy()
    with pytest.raises(oracle.ClipNotFusable):
        oracle.adamw_step(W, z, z, g, 1, max_grad_norm=1.0)
    with pytest.raises(oracle.ClipNotFusable):
        oracle.sgdm_step(W, z, g, max_grad_norm=float("inf"))
    with pytest.raises(ValueError):
        oracle.adamw_step(W, z, z, g, 1, max_grad_norm=-1.0)
    assert np.array_equal(W, W_copy)


# --------------------------------------------------------------------------
# SGD-momentum
# --------------------------------------------------------------------------
def test_sgdm_reduces_to_plain_sgd():
    g = normal_f32(90, (4096,))
    W0 = normal_f32(91, g.shape)
    W1, b1 = oracle.sgdm_step(W0, np.zeros_like(W0), g, lr=1e-3, momentum=0.0, weight_decay=0.0)
    assert np.array_equal(bits(b1), bits(g))
    assert np.all(np.abs(W1 - (W0.astype(np.float64) - 1e-3 * g)) <= _ulp(W1))


def test_sgdm_closed_forms():
    c = normal_f32(92, (2048,))
    W0 = normal_f32(93, c.shape)
    W, b = W0.copy(), np.zeros_like(W0)
    total = np.zeros(c.shape)
    for t in range(1, 6):
        W, b = oracle.sgdm_step(W, b, c, lr=1e-3, momentum=0.9, weight_decay=0.0)
        coef = (1 - 0.9 ** t) / (1 - 0.9)
        assert np.all(np.abs(b - coef * c.astype(np.float64)) <= 1e-6 * coef * np.abs(c))
        total += coef * c.astype(np.float64)
        mag = np.abs(W0.astype(np.float64)) + 1e-3 * np.abs(total)
        assert np.all(np.abs(W - (W0.astype(np.float64) - 1e-3 * total)) <= 2 * t * _ulp(mag))
    # coupled decay enters the buffer: b_1 = g + wd W_0
    W1, b1 = oracle.sgdm_step(W0, np.zeros_like(W0), c, lr=1e-3, momentum=0.9, weight_decay=0.01)
    assert np.all(np.abs(b1 - (c + 0.01 * W0.astype(np.float64))) <= _ulp(b1) + _ulp(0.01 * W0))


# --------------------------------------------------------------------------
# routed experts
# --------------------------------------------------------------------------
def test_grouped_step_decays_empty_experts():
    E, d_out, d_in = 3, 4, 8
    W = normal_f32(100, (E, d_out, d_in), 0.02)
    m = normal_f32(101, W.shape, 0.1)
    v = np.abs(normal_f32(102, W.shape, 0.01))
    Xb = normal_bf16(103, (6, d_in))
    dYb = normal_bf16(104, (6, d_out))
    grads = oracle.grouped_wgrad(Xb, dYb, [0, 6, 6, 6])
    W1, m1, v1 = oracle.grouped_adamw_step(W, m, v, grads, 2, **HP)
    for e in (1, 2):
        assert np.array_equal(bits(m1[e]), bits(F32(0.9) * m[e]))
        assert not np.array_equal(bits(W1[e]), bits(W[e]))
    Wd, md, vd = oracle.adamw_step(W[0], m[0], v[0], oracle.wgrad(Xb, dYb), 2, **HP)
    assert np.array_equal(bits(W1[0]), bits(Wd)) and np.array_equal(bits(v1[0]), bits(vd))


def test_grouped_sgdm_moves_empty_experts_by_decay_only():
    """SGD-momentum on routed experts (P5): an empty expert with no momentum
    history and no decay stays put exactly; with decay it shrinks toward zero
    (every element keeps its sign and loses magnitude), and with a momentum
    history it keeps moving along it; a non-empty expert is the dense step on
    its own rows."""
    E, d_out, d_in = 3, 4, 8
    W = normal_f32(110, (E, d_out, d_in), 0.02)
    Xb = normal_bf16(113, (6, d_in))
    dYb = normal_bf16(114, (6, d_out))
    grads = oracle.grouped_wgrad(Xb, dYb, [0, 6, 6, 6])
    zero = np.zeros_like(W)
    W1, b1 = oracle.grouped_sgdm_step(W, zero, grads, lr=1e-3, momentum=0.9, weight_decay=0.0)
    for e in (1, 2):
        assert np.array_equal(bits(W1[e]), bits(W[e])) and not np.any(b1[e])
    W2, b2 = oracle.grouped_sgdm_step(W, zero, grads, lr=1e-2, momentum=0.9, weight_decay=0.5)
    for e in (1, 2):
        assert np.all(np.sign(W2[e]) == np.sign(W[e]))
        assert np.all(np.abs(W2[e]) < np.abs(W[e]))
    hist = normal_f32(115, W.shape, 1e-3)
    W3, _ = oracle.grouped_sgdm_step(W, hist, grads, lr=1e-3, momentum=0.9, weight_decay=0.0)
    for e in (1, 2):
        assert np.all(np.sign(W[e] - W3[e]) == np.sign(hist[e]))
    Wd, bd = oracle.sgdm_step(W[0], zero[0], oracle.wgrad(Xb, dYb), lr=1e-2, momentum=0.9,
                              weight_decay=0.5)
    assert np.array_equal(bits(W2[0]), bits(Wd)) and np.array_equal(bits(b2[0]), bits(bd))


def test_sgdm_judge_arithmetic_floor():
    """With an exact gradient (tau = 0) the SGD-momentum judgment accepts a
    buffer formed with fused multiply-adds where momentum b and wd W cancel,
    and still rejects a wrong momentum and a dropped decay term."""
    n = 1 << 16
    W = normal_f32(120, (n,), 0.02)
    b = normal_f32(121, (n,), 1e-3)
    g = np.zeros(n, dtype=F32)
    hp = dict(lr=1e-3, momentum=0.9, weight_decay=0.01)
    b[:256] = (-F32(0.01) * W[:256] / F32(0.9)).astype(F32)        # near cancellation
    W_ref, b_ref = oracle.sgdm_step(W, b, g, **hp)
    # one rounding of momentum b + wd W, as a fused multiply-add gives
    b_fma = (0.9 * b.astype(np.float64) + (F32(0.01) * W).astype(np.float64)).astype(F32)
    W_fma = (W - F32(1e-3) * b_fma).astype(F32)

    def run(b_gpu, W_gpu, arith=True):
        fl = oracle.StateFloor((n,), "sgdm", momentum=0.9)
        fl.update(np.zeros(n), g, oracle.sgdm_arith_floor(b, g, W, 0.9, 0.01) if arith else None)
        return judge.judge_sgdm(W, W_gpu, b_gpu, W, W_ref, b_ref, fl, 1e-3)

    assert not np.array_equal(bits(b_fma), bits(b_ref))           # the two roundings differ
    assert not run(b_fma, W_fma, arith=False).passed               # so the floor is needed
    assert run(b_fma, W_fma).passed
    W_bad, b_bad = oracle.sgdm_step(W, b, g, lr=1e-3, momentum=0.89, weight_decay=0.01)
    assert not run(b_bad, W_bad).passed
    W_bad, b_bad = oracle.sgdm_step(W, b, g, lr=1e-3, momentum=0.9, weight_decay=0.0)
    assert not run(b_bad, W_bad).passed


# --------------------------------------------------------------------------
# accumulation floor and the judge
# --------------------------------------------------------------------------
def _fp32_sums(Xb, dYb, chunk):
    """float32 running sums of exact products, in chunks of ``chunk`` tokens."""
    X = oracle.bf16_bits_to_f64(Xb)
    dY = oracle.bf16_bits_to_f64(dYb)
    acc = np.zeros((dY.shape[1], X.shape[1]), dtype=F32)
    for t0 in range(0, X.shape[0], chunk):
        part = (dY[t0:t0 + chunk].T @ X[t0:t0 + chunk]).astype(F32)
        acc = (acc + part).astype(F32)
    return acc


@pytest.mark.parametrize("chunk", [1, 16])
def test_floor_bounds_fp32_accumulation(chunk):
    Xb = normal_bf16(110, (2048, 32))
    dYb = normal_bf16(111, (2048, 24), 1e-2)
    g_ref = oracle.wgrad(Xb, dYb)
    tau = oracle.acc_floor(Xb, dYb)
    g32 = _fp32_sums(Xb, dYb, chunk)
    err = np.abs(g32.astype(np.float64) - g_ref)
    assert np.all(err <= tau)
    assert np.max(err / tau) > 0.05        # at most 20x the largest real error (0.12-0.21 here)
    assert np.allclose(oracle.acc_floor_rows(Xb, dYb, [3, 7]), tau[[3, 7]], rtol=1e-12, atol=0)


def test_floor_tightness_guards_the_bf16_rejection():
    """Why the floor must be tight: the bf16-rounded gradient (the rounding the
    fusion deletes; FORGE assessment, "What's already in tree and easy to
    miss") misses the floor by up to ~760x. A floor up to 20x too loose (all
    the tightness pin above allows) still rejects it; one 1000x too loose
    would accept every element."""
    Xb = normal_bf16(110, (2048, 32))
    dYb = normal_bf16(111, (2048, 24), 1e-2)
    g_ref = oracle.wgrad(Xb, dYb)
    tau = oracle.acc_floor(Xb, dYb)
    err_bf16 = np.abs(oracle.bf16_round(g_ref).astype(np.float64) - g_ref)
    for k in (1, 10, 20):
        assert np.mean(err_bf16 > k * tau) > 0.5
    assert np.all(err_bf16 <= 1000 * tau)


def _run_judged(g_gpu_fn, steps=3, planted=None):
    """Run the oracle next to a 'GPU' stand-in built from CPU pieces; return reports."""
    d_in, d_out, T = 32, 24, 1024
    W = normal_f32(120, (d_out, d_in), 0.02)
    Wg, mg, vg = W.copy(), np.zeros_like(W), np.zeros_like(W)
    Wr, mr, vr = W.copy(), np.zeros_like(W), np.zeros_like(W)
    fl = oracle.StateFloor(W.shape)
    reports = []
    for t in range(1, steps + 1):
        Xb = normal_bf16(130 + t, (T, d_in))
        dYb = normal_bf16(140 + t, (T, d_out))
        g_ref = oracle.wgrad(Xb, dYb)
        tau = oracle.acc_floor(Xb, dYb)
        fl.update(tau, g_ref)
        Wr_new, mr, vr = oracle.adamw_step(Wr, mr, vr, g_ref, t, **HP)
        g = g_gpu_fn(Xb, dYb)
        hp = dict(HP)
        if planted == "no_bias_correction":
            hp = dict(HP)
            m_new, v_new = oracle.adamw_moments(mg, vg, g, 0.9, 0.999)
            Wg_new = Wg - F32(1e-3) * (m_new / (np.sqrt(v_new) + F32(1e-8)) + F32(0.01) * Wg)
            mg_new, vg_new = m_new, v_new
        else:
            Wg_new, mg_new, vg_new = oracle.adamw_step(Wg, mg, vg, g, t, **hp)
        reports.append(judge.judge_adamw(t, Wg, Wg_new, mg_new, vg_new, Wr, Wr_new, mr, vr,
                                         g_ref, tau, fl, **HP))
        Wg, mg, vg, Wr = Wg_new, mg_new, vg_new, Wr_new
    return reports


def test_judge_accepts_fp32_accumulation_orders():
    for chunk in (1, 16, 64):
        for r in _run_judged(lambda X, D: _fp32_sums(X, D, chunk)):
            assert r.passed, str(r)


def test_judge_rejects_planted_mistakes():
    def bf16_grad(X, D):
        g = oracle.wgrad(X, D)
        return (bf16_bits_from_f32(g).astype(np.uint32) << 16).view(F32)

    assert not all(r.passed for r in _run_judged(bf16_grad))
    assert not all(r.passed for r in _run_judged(oracle.wgrad, planted="no_bias_correction"))

    def dropped_token(X, D):
        return oracle.wgrad(X[1:], D[1:])

    assert not all(r.passed for r in _run_judged(dropped_token))


def test_judge_sparse_softmax_gradients_over_steps():
    """Sparse softmax-gradient rows (LM-head-like): most gradient elements have a
    short history near the accumulation floor. Correct float32 accumulation in
    any order passes every step; a 2e-3 lr error on a well-determined element
    does not."""
    from synth import lmhead_dy
    T, d_in, V = 256, 32, 4096
    W = normal_f32(160, (V, d_in), 0.02)
    hp = dict(HP)
    for chunk in (1, 16):
        Wg, mg, vg = W.copy(), np.zeros_like(W), np.zeros_like(W)
        Wr, mr, vr = W.copy(), np.zeros_like(W), np.zeros_like(W)
        fl = oracle.StateFloor(W.shape)
        for t in range(1, 6):
            Xb = normal_bf16(170 + t, (T, d_in))
            dYb = lmhead_dy(180 + t, T, V, support=32)
            g_ref = oracle.wgrad(Xb, dYb)
            tau = oracle.acc_floor(Xb, dYb)
            fl.update(tau, g_ref)
            Wr_new, mr, vr = oracle.adamw_step(Wr, mr, vr, g_ref, t, **hp)
            Wg_new, mg, vg = oracle.adamw_step(Wg, mg, vg, _fp32_sums(Xb, dYb, chunk), t, **hp)
            rep = judge.judge_adamw(t, Wg, Wg_new, mg, vg, Wr, Wr_new, mr, vr, g_ref, tau, fl, **hp)
            assert rep.passed, (chunk, t, str(rep))
            # plant an error of 2e-3 lr on the best-determined element
            k = np.unravel_index(np.argmax(np.abs(g_ref) / (tau + 1e-30)), g_ref.shape)
            bad = Wg_new.copy()
            bad[k] += np.float32(2e-3 * hp["lr"])
            rep_bad = judge.judge_adamw(t, Wg, bad, mg, vg, Wr, Wr_new, mr, vr, g_ref, tau, fl, **hp)
            assert not rep_bad.passed
            Wg, Wr = Wg_new, Wr_new


def test_strict_bar_fails_a_correct_fp32_order_at_every_step():
    """Premise of the widened weight-delta bar (judge.update_floor): where a
    weight's gradient history sits at the accumulation floor, correct float32
    orders disagree on the gradient's sign or zero, the AdamW update (close to
    sign(g) from zero state) differs by O(lr), and no bar of 1e-3 lr can hold,
    at step 1 and at every later step alike. A softmax-gradient column
    (LM-head-like): a vocabulary entry with probability ~1 in one row
    (dY = 1), a probability 2^-24 in the next and the label of a third row
    with probability 0 (dY = -1), against X = 1. The exact sum is 2^-24; the
    sequential float32 order rounds 1 + 2^-24 to 1 and ends at 0."""
    T, d_in, V = 3, 8, 8
    Xb = bf16_bits_from_f32(np.ones((T, d_in), F32))
    dY = normal_f32(190, (T, V), 1e-2)
    dY[:, 0] = [1.0, 2.0 ** -24, -1.0]
    dYb = bf16_bits_from_f32(dY)
    g_ref = oracle.wgrad(Xb, dYb)
    g_seq = _fp32_sums(Xb, dYb, 1)
    tau = oracle.acc_floor(Xb, dYb)
    assert np.all(g_ref[0] == F32(2.0 ** -24)) and np.all(g_seq[0] == 0)
    assert np.all(np.abs(g_seq.astype(np.float64) - g_ref) <= tau)   # a correct order
    W = normal_f32(191, (V, d_in), 0.02)
    Wg, mg, vg = W.copy(), np.zeros_like(W), np.zeros_like(W)
    Wr, mr, vr = W.copy(), np.zeros_like(W), np.zeros_like(W)
    fl = oracle.StateFloor(W.shape)
    for t in range(1, 4):
        fl.update(tau, g_ref)
        Wr_new, mr, vr = oracle.adamw_step(Wr, mr, vr, g_ref, t, **HP)
        Wg_new, mg, vg = oracle.adamw_step(Wg, mg, vg, g_seq, t, **HP)
        dd = np.abs((Wg_new.astype(np.float64) - Wg) - (Wr_new.astype(np.float64) - Wr))
        assert np.all(dd[0] > 0.5 * HP["lr"]) and np.all(dd[1:] <= 1e-3 * HP["lr"]), t
        rep = judge.judge_adamw(t, Wg, Wg_new, mg, vg, Wr, Wr_new, mr, vr, g_ref, tau, fl, **HP)
        assert rep.passed and rep.checks["ambiguous"] >= d_in, (t, str(rep))
        Wg, Wr = Wg_new, Wr_new


def test_ambiguous_budget():
    """The judge can cap how many elements take the widened weight-delta bar:
    the sign-ambiguous row above is 8 of 64 elements."""
    T, d_in, V = 3, 8, 8
    Xb = bf16_bits_from_f32(np.ones((T, d_in), F32))
    dY = normal_f32(190, (T, V), 1e-2)
    dY[:, 0] = [1.0, 2.0 ** -24, -1.0]
    dYb = bf16_bits_from_f32(dY)
    g_ref, tau = oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb)
    W = normal_f32(191, (V, d_in), 0.02)
    z = np.zeros_like(W)
    fl = oracle.StateFloor(W.shape)
    fl.update(tau, g_ref)
    Wr, mr, vr = oracle.adamw_step(W, z, z, g_ref, 1, **HP)
    args = (1, W, Wr, mr, vr, W, Wr, mr, vr, g_ref, tau, fl)
    assert judge.judge_adamw(*args, **HP, ambiguous_budget=8 / 64).passed
    rep = judge.judge_adamw(*args, **HP, ambiguous_budget=0.0, ambiguous_min=7)
    assert not rep.passed and rep.checks["ambiguous"] == 8


def test_update_bound_closed_forms():
    # one step from zero state: |m_hat / sqrt(v_hat)| = |g| / |g| = 1
    assert judge.update_bound(1, 0.9, 0.999) == pytest.approx(1.0)
    # equal betas: m_hat^2 <= v_hat by Jensen, so the bound is 1 at every step
    for t in (2, 7, 50):
        assert judge.update_bound(t, 0.9, 0.9) == pytest.approx(1.0)


def test_bitwise_judgment():
    a = normal_f32(150, (64,))
    b = a.copy()
    assert judge.bitwise_equal(a, b)
    b[7] = np.nextafter(b[7], F32(np.inf))
    assert not judge.bitwise_equal(a, b)
    assert not judge.bitwise_equal(np.zeros(1, F32), -np.zeros(1, F32))
