"""GPU parity of the input gradient dX = dY W_b and of the linear-backward
calls that order it before the fused optimizer step (page "docs(audit): FORGE
assessment + residency-aware epilogue-fusion track", section "Math verified,
not asserted", P1: the in-place dX-before-update hazard).

Accuracy against the oracle's exact dY W_b (oracle.judge.judge_dgrad), every
tiling bitwise equal, and the combined call bitwise equal to the two calls in
the safe order. The bf16-copy calls (dX from a bf16 copy of W that the fused
step refreshes) are held to the same bar, and the refreshed copy must be the
oracle's nearest-even bf16 rounding of the updated W, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import judge
from synth import DenseCase
from tests._gpu import (AdamWParity, SgdmParity, adamw_hp, bf16_dev, bits_equal, f32_dev, host,
                        host_f32, log, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wg():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_gradient_gemm_amd as wg
    wg.library()
    return wg


def _sync():
    torch_mod().cuda.synchronize()


# K = d_out tails: 200 = 6 stages + 8, 392 = 12 stages + 8, 8 = one partial stage
CASES = [DenseCase("ragged_77x264x200", T=77, d_in=264, d_out=200, seed_base=60000),
         DenseCase("tiles_300x520x392", T=300, d_in=520, d_out=392, seed_base=61000),
         DenseCase("k8_130x136x8", T=130, d_in=136, d_out=8, seed_base=62000)]


def _dx(dtype, T, d_in):
    torch = torch_mod()
    return torch.full((T, d_in), float("nan"), device="cuda", dtype=dtype)


@pytest.mark.parametrize("bf16_out", [False, True])
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_dgrad_against_oracle(wg, case, tile, bf16_out):
    torch = torch_mod()
    _, dYb = synth.dense_inputs(case, 1)
    W0, _, _ = synth.dense_state(case)
    log(f"[{case.name}] dgrad tile {tile} bf16_out={bf16_out}")
    dX = _dx(torch.bfloat16 if bf16_out else torch.float32, case.T, case.d_in)
    wg.forge_dgrad(bf16_dev(dYb), f32_dev(W0), dX, tile=tile)
    _sync()
    rep = judge.judge_dgrad(host_f32(dX), dYb, W0, bf16_out)
    log(f"  {rep}")
    assert rep.passed, str(rep)


@pytest.mark.parametrize("bf16_out", [False, True])
def test_dgrad_bitwise_across_tilings(wg, bf16_out):
    torch = torch_mod()
    case = CASES[1]
    _, dYb = synth.dense_inputs(case, 2)
    W0, _, _ = synth.dense_state(case)
    dY, W = bf16_dev(dYb), f32_dev(W0)
    outs = []
    for tile in (1, 2, 3, 0, 1):
        dX = _dx(torch.bfloat16 if bf16_out else torch.float32, case.T, case.d_in)
        wg.forge_dgrad(dY, W, dX, tile=tile)
        _sync()
        outs.append(host_f32(dX))
    assert all(bits_equal(o, outs[0]) for o in outs[1:])


def test_dgrad_zero_outputs_writes_zeros(wg):
    torch = torch_mod()
    dY = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    for dtype in (torch.float32, torch.bfloat16):
        dX = _dx(dtype, 40, 64)
        wg.forge_dgrad(dY, W, dX)
        _sync()
        got = host_f32(dX)
        assert np.all(got == 0) and not np.any(np.signbit(got))


@pytest.mark.parametrize("bf16_out", [False, True])
def test_linear_backward_adamw(wg, bf16_out):
    """Three steps: dX from the weight before each step, W/m/v as the fused
    step, and the whole bitwise the two calls in the safe order."""
    torch = torch_mod()
    case = CASES[0]
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    W2, m2, v2 = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    par = AdamWParity(W0, m0, v0, hp)
    dt = torch.bfloat16 if bf16_out else torch.float32
    for t in (1, 2, 3):
        Xb, dYb = synth.dense_inputs(case, t)
        X, dY = bf16_dev(Xb), bf16_dev(dYb)
        log(f"[{case.name}] linear backward adamw step {t} bf16_out={bf16_out}")
        W_prev = host(W)
        dX = _dx(dt, case.T, case.d_in)
        wg.forge_linear_backward_adamw(X, dY, W, m, v, dX, step=t, **hp)
        # the same two steps issued separately, in the safe order
        dX2 = _dx(dt, case.T, case.d_in)
        wg.forge_dgrad(dY, W2, dX2)
        wg.forge_wgrad_adamw(X, dY, W2, m2, v2, step=t, **hp)
        # and the hazard: dX formed after the update
        dX_late = _dx(dt, case.T, case.d_in)
        wg.forge_dgrad(dY, W2, dX_late)
        _sync()
        rep = judge.judge_dgrad(host_f32(dX), dYb, W_prev, bf16_out)
        log(f"  dX {rep}")
        assert rep.passed, str(rep)
        rep = par.step(t, oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W),
                       host(m), host(v))
        log(f"  W {rep}")
        assert rep.passed, str(rep)
        assert bits_equal(host_f32(dX), host_f32(dX2))
        assert bits_equal(host(W), host(W2)) and bits_equal(host(m), host(m2))
        assert not judge.judge_dgrad(host_f32(dX_late), dYb, W_prev, bf16_out).passed


def test_linear_backward_sgdm(wg):
    torch = torch_mod()
    case = CASES[1]
    hp = dict(lr=case.lr, momentum=case.momentum, weight_decay=0.01)
    W0, _, _ = synth.dense_state(case)
    W, b = f32_dev(W0), f32_dev(np.zeros_like(W0))
    par = SgdmParity(W0, np.zeros_like(W0), hp)
    for t in (1, 2):
        Xb, dYb = synth.dense_inputs(case, t)
        log(f"[{case.name}] linear backward sgdm step {t}")
        W_prev = host(W)
        dX = _dx(torch.float32, case.T, case.d_in)
        wg.forge_linear_backward_sgdm(bf16_dev(Xb), bf16_dev(dYb), W, b, dX, **hp)
        _sync()
        rep = judge.judge_dgrad(host(dX), dYb, W_prev, False)
        assert rep.passed, str(rep)
        rep = par.step(oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W), host(b))
        assert rep.passed, str(rep)


def test_linear_backward_zero_tokens(wg):
    """No tokens: dX is empty and the fused step is a decay step."""
    torch = torch_mod()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(630, (32, 64), 0.02)
    m0 = synth.normal_f32(631, W0.shape, 0.1)
    v0 = np.abs(synth.normal_f32(632, W0.shape, 0.01))
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wg.forge_linear_backward_adamw(X, dY, W, m, v, dX, step=2, **hp)
    _sync()
    assert bits_equal(host(m), np.float32(0.9) * m0)


def _wb_dev(W):
    """The caller's bf16 copy of a float32 weight, rounded once (the seeded
    input encoder, nearest even)."""
    return bf16_dev(synth.bf16_bits_from_f32(np.ascontiguousarray(W, dtype=np.float32)))


def _copy_is_rounded(Wb, W) -> bool:
    return bits_equal(host_f32(Wb), oracle.bf16_round(host(W)))


@pytest.mark.parametrize("bf16_out", [False, True])
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_dgrad_bf16w_against_oracle(wg, case, tile, bf16_out):
    torch = torch_mod()
    _, dYb = synth.dense_inputs(case, 3)
    W0, _, _ = synth.dense_state(case)
    log(f"[{case.name}] dgrad from the bf16 copy, tile {tile} bf16_out={bf16_out}")
    dt = torch.bfloat16 if bf16_out else torch.float32
    dY = bf16_dev(dYb)
    dX = _dx(dt, case.T, case.d_in)
    wg.forge_dgrad_bf16w(dY, _wb_dev(W0), dX, tile=tile)
    dX32 = _dx(dt, case.T, case.d_in)
    wg.forge_dgrad(dY, f32_dev(W0), dX32, tile=tile)
    _sync()
    rep = judge.judge_dgrad(host_f32(dX), dYb, W0, bf16_out)
    log(f"  {rep}")
    assert rep.passed, str(rep)
    assert bits_equal(host_f32(dX), host_f32(dX32))


@pytest.mark.parametrize("tile", [0, 3, 4])
@pytest.mark.parametrize("case", CASES[:2], ids=lambda c: c.name)
def test_linear_backward_adamw_bf16w(wg, case, tile):
    """Three steps from one initial rounding of W: dX from the copy, the fused
    step judged against the oracle, the copy refreshed to bf16(W'), and all of
    it bitwise the float32-weight call."""
    torch = torch_mod()
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    W, m, v, Wb = f32_dev(W0), f32_dev(m0), f32_dev(v0), _wb_dev(W0)
    W2, m2, v2 = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    par = AdamWParity(W0, m0, v0, hp)
    for t in (1, 2, 3):
        Xb, dYb = synth.dense_inputs(case, 10 + t)
        X, dY = bf16_dev(Xb), bf16_dev(dYb)
        log(f"[{case.name}] linear backward adamw from the bf16 copy, tile {tile}, step {t}")
        W_prev = host(W)
        dX = _dx(torch.bfloat16, case.T, case.d_in)
        wg.forge_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, step=t, tile=tile, **hp)
        dX2 = _dx(torch.bfloat16, case.T, case.d_in)
        wg.forge_linear_backward_adamw(X, dY, W2, m2, v2, dX2, step=t, tile=tile, **hp)
        _sync()
        rep = judge.judge_dgrad(host_f32(dX), dYb, W_prev, True)
        log(f"  dX {rep}")
        assert rep.passed, str(rep)
        rep = par.step(t, oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W),
                       host(m), host(v))
        log(f"  W {rep}")
        assert rep.passed, str(rep)
        assert _copy_is_rounded(Wb, W)
        assert bits_equal(host_f32(dX), host_f32(dX2))
        assert bits_equal(host(W), host(W2)) and bits_equal(host(m), host(m2))
        assert bits_equal(host(v), host(v2))


def test_linear_backward_sgdm_bf16w(wg):
    torch = torch_mod()
    case = CASES[1]
    hp = dict(lr=case.lr, momentum=case.momentum, weight_decay=0.01)
    W0, _, _ = synth.dense_state(case)
    W, b, Wb = f32_dev(W0), f32_dev(np.zeros_like(W0)), _wb_dev(W0)
    par = SgdmParity(W0, np.zeros_like(W0), hp)
    for t in (1, 2):
        Xb, dYb = synth.dense_inputs(case, 20 + t)
        log(f"[{case.name}] linear backward sgdm from the bf16 copy, step {t}")
        W_prev = host(W)
        dX = _dx(torch.float32, case.T, case.d_in)
        wg.forge_linear_backward_sgdm_bf16w(bf16_dev(Xb), bf16_dev(dYb), W, b, Wb, dX, **hp)
        _sync()
        rep = judge.judge_dgrad(host(dX), dYb, W_prev, False)
        assert rep.passed, str(rep)
        rep = par.step(oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W), host(b))
        assert rep.passed, str(rep)
        assert _copy_is_rounded(Wb, W)


def test_linear_backward_bf16w_zero_tokens(wg):
    """No tokens: dX is empty, the fused step decays W and still refreshes the
    copy."""
    torch = torch_mod()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(640, (40, 64), 0.02)
    m0 = synth.normal_f32(641, W0.shape, 0.1)
    v0 = np.abs(synth.normal_f32(642, W0.shape, 0.01))
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    Wb = torch.zeros((40, 64), dtype=torch.bfloat16, device="cuda")
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 40), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wg.forge_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, step=2, **hp)
    _sync()
    assert bits_equal(host(m), np.float32(0.9) * m0)
    assert _copy_is_rounded(Wb, W)
    assert not bits_equal(host(W), W0)


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_fused_steps_refresh_the_bf16_copy(wg, tile):
    """The fused steps alone with the copy refresh: W and the state judged
    against the oracle and bitwise those of the plain fused calls; the copy
    the oracle's bf16 rounding of the new W."""
    case = CASES[0]
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    W, m, v, Wb = f32_dev(W0), f32_dev(m0), f32_dev(v0), _wb_dev(np.zeros_like(W0))
    W2, m2, v2 = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    par = AdamWParity(W0, m0, v0, hp)
    for t in (1, 2):
        Xb, dYb = synth.dense_inputs(case, 30 + t)
        X, dY = bf16_dev(Xb), bf16_dev(dYb)
        log(f"[{case.name}] fused AdamW refreshing the bf16 copy, tile {tile}, step {t}")
        W_prev = host(W)
        wg.forge_wgrad_adamw_bf16w(X, dY, W, m, v, Wb, step=t, tile=tile, **hp)
        wg.forge_wgrad_adamw(X, dY, W2, m2, v2, step=t, tile=tile, **hp)
        _sync()
        rep = par.step(t, oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W),
                       host(m), host(v))
        assert rep.passed, str(rep)
        assert _copy_is_rounded(Wb, W)
        assert bits_equal(host(W), host(W2)) and bits_equal(host(m), host(m2))
        assert bits_equal(host(v), host(v2))
    hs = dict(lr=case.lr, momentum=case.momentum, weight_decay=0.01)
    W, b, Wb = f32_dev(W0), f32_dev(np.zeros_like(W0)), _wb_dev(np.zeros_like(W0))
    W2, b2 = f32_dev(W0), f32_dev(np.zeros_like(W0))
    spar = SgdmParity(W0, np.zeros_like(W0), hs)
    Xb, dYb = synth.dense_inputs(case, 40)
    log(f"[{case.name}] fused SGD-momentum refreshing the bf16 copy, tile {tile}")
    wg.forge_wgrad_sgdm_bf16w(bf16_dev(Xb), bf16_dev(dYb), W, b, Wb, tile=tile, **hs)
    wg.forge_wgrad_sgdm(bf16_dev(Xb), bf16_dev(dYb), W2, b2, tile=tile, **hs)
    _sync()
    rep = spar.step(oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W0, host(W), host(b))
    assert rep.passed, str(rep)
    assert _copy_is_rounded(Wb, W)
    assert bits_equal(host(W), host(W2)) and bits_equal(host(b), host(b2))
