"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element on the same seeded inputs, plus the GPU-side bitwise invariants.

Accuracy (tolerance, vs the oracle) and invariance (bitwise, GPU vs GPU) are
judged separately; see oracle/judge.py for the bars.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import DenseCase
from tests._gpu import (AdamWParity, SgdmParity, adamw_hp, bf16_dev, bits_equal, f32_dev, host,
                        log, run_dense_adamw, run_dense_sgdm, torch_mod)

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


RAGGED = DenseCase("ragged_77x264x200", T=77, d_in=264, d_out=200, seed_base=50000, steps=3)


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_ragged_dense_adamw(wg, tile):
    run_dense_adamw(wg, RAGGED, RAGGED.steps, tile=tile)


# 18 x 17 tiles of 256x256 (both edges ragged; the last column's second half
# tile lies wholly past d_out): enough tiles that the persistent schedule runs
# both phases, whole tiles and half tiles on every XCD. T = 45: one stage and
# a 13-token tail.
PERSIST = DenseCase("persistent_45x4360x4104", T=45, d_in=4360, d_out=4104, seed_base=55000,
                    steps=2)


def test_persistent_schedule_adamw(wg):
    run_dense_adamw(wg, PERSIST, PERSIST.steps, tile=4)


# Several tiles per compute unit (9 x 17 = 153 tiles of 256x256) and a long
# mainloop: T = 2000 is 62 stages of 32 tokens and a 16-token tail.
LONG = DenseCase("long_2000x2056x4104", T=2000, d_in=2056, d_out=4104, seed_base=57000, steps=2)


def test_long_mainloop_adamw(wg):
    run_dense_adamw(wg, LONG, LONG.steps, tile=4)


def test_long_mainloop_sgdm(wg):
    run_dense_sgdm(wg, LONG, 2, tile=4, weight_decay=0.01)


def test_long_mainloop_gradient_bitwise_equals_grid_tiles(wg):
    torch = torch_mod()
    Xb, dYb = synth.dense_inputs(LONG, 1)
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    out = {}
    for tile in (4, 3, 1):
        log(f"[{LONG.name}] gradient, tile {tile}")
        g = torch.full((LONG.d_out, LONG.d_in), float("nan"), device="cuda")
        wg.forge_wgrad(X, dY, g, tile=tile)
        _sync()
        out[tile] = host(g)
    assert bits_equal(out[4], out[3]) and bits_equal(out[4], out[1])


def test_persistent_gradient_bitwise_equals_grid_tiles(wg):
    torch = torch_mod()
    Xb, dYb = synth.dense_inputs(PERSIST, 1)
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    out = {}
    for tile in (4, 3, 1):
        g = torch.full((PERSIST.d_out, PERSIST.d_in), float("nan"), device="cuda")
        wg.forge_wgrad(X, dY, g, tile=tile)
        _sync()
        out[tile] = host(g)
    assert all(bits_equal(out[4], out[t]) for t in (3, 1))
    rows = np.array([0, 1, 255, 256, 2047, 4095, 4096, 4103])
    err = np.abs(out[4][rows].astype(np.float64) - oracle.wgrad_rows(Xb, dYb, rows))
    assert np.all(err <= oracle.acc_floor_rows(Xb, dYb, rows))


@pytest.mark.parametrize("tile", [3, 4])
def test_eps_zero_exact_root(wg, tile):
    case = DenseCase("eps0_77x264x200", T=77, d_in=264, d_out=200, seed_base=56000, steps=3,
                     eps=0.0)
    run_dense_adamw(wg, case, case.steps, tile=tile)


def test_config0_tiny_dense_adamw(wg):
    case = synth.dense_case(0)
    run_dense_adamw(wg, case, case.steps)


def test_many_tiles_single_token_and_tail(wg):
    # T = 1 and T = 33: one partial MFMA chunk, and one full stage plus a 1-token tail
    for T in (1, 33):
        case = DenseCase(f"tail_T{T}", T=T, d_in=520, d_out=136, seed_base=51000 + T, steps=2)
        run_dense_adamw(wg, case, case.steps, tile=1)


def _state(case):
    W0, m0, v0 = synth.dense_state(case)
    return f32_dev(W0), f32_dev(m0), f32_dev(v0)


def test_bitwise_tilings_unfused_and_repeat(wg):
    """One gradient, four GPU routes, one bit pattern: tile 256x128, tile
    128x128, the unfused pair (stored fp32 gradient + elementwise AdamW), and a
    repeat of the first (FORGE assessment, P1)."""
    torch = torch_mod()
    case = DenseCase("bitwise_300x520x392", T=300, d_in=520, d_out=392, seed_base=52000)
    hp = adamw_hp(case)
    results = []
    for route in ("tile1", "tile2", "tile3", "tile4", "unfused", "tile1_again"):
        W, m, v = _state(case)
        for t in (1, 2):
            Xb, dYb = synth.dense_inputs(case, t)
            X, dY = bf16_dev(Xb), bf16_dev(dYb)
            if route == "unfused":
                g = torch.empty_like(W)
                wg.forge_wgrad(X, dY, g, tile=1)
                wg.forge_adamw(g, W, m, v, step=t, **hp)
            else:
                tile = {"tile2": 2, "tile3": 3, "tile4": 4}.get(route, 1)
                wg.forge_wgrad_adamw(X, dY, W, m, v, step=t, tile=tile, **hp)
        _sync()
        results.append((route, host(W), host(m), host(v)))
    base = results[0]
    for route, W, m, v in results[1:]:
        assert bits_equal(W, base[1]) and bits_equal(m, base[2]) and bits_equal(v, base[3]), route


def test_unfused_gradient_against_oracle(wg):
    torch = torch_mod()
    case = DenseCase("grad_300x520x392", T=300, d_in=520, d_out=392, seed_base=53000)
    Xb, dYb = synth.dense_inputs(case, 1)
    for tile in (1, 2, 3, 4):
        g = torch.full((case.d_out, case.d_in), float("nan"), device="cuda")
        wg.forge_wgrad(bf16_dev(Xb), bf16_dev(dYb), g, tile=tile)
        _sync()
        err = np.abs(host(g).astype(np.float64) - oracle.wgrad(Xb, dYb))
        assert np.all(err <= oracle.acc_floor(Xb, dYb)), tile


def test_zero_tokens_is_a_decay_step(wg):
    torch = torch_mod()
    case = DenseCase("decay_0x64x32", T=0, d_in=64, d_out=32, seed_base=54000)
    W0 = synth.normal_f32(1, (32, 64), 0.02)
    m0 = synth.normal_f32(2, (32, 64), 0.1)
    v0 = np.abs(synth.normal_f32(3, (32, 64), 0.01))
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    empty_y = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    wg.forge_wgrad_adamw(empty, empty_y, W, m, v, step=3, **adamw_hp(case))
    _sync()
    assert bits_equal(host(m), np.float32(0.9) * m0)
    assert bits_equal(host(v), np.float32(0.999) * v0)
    Wr, _, _ = oracle.adamw_step(W0, m0, v0, np.zeros_like(W0), 3, **adamw_hp(case))
    assert np.all(np.abs(host(W).astype(np.float64) - Wr) <= 1e-3 * case.lr)


def test_clip_request_fails_closed(wg):
    case = RAGGED
    W, m, v = _state(case)
    W_before = host(W)
    Xb, dYb = synth.dense_inputs(case, 1)
    with pytest.raises(wg.ForgeError) as ei:
        wg.forge_wgrad_adamw(bf16_dev(Xb), bf16_dev(dYb), W, m, v, step=1, max_grad_norm=1.0)
    assert ei.value.status == 6
    _sync()
    assert bits_equal(host(W), W_before) and not host(m).any()


@pytest.mark.parametrize("tile,wd", [(1, 0.0), (2, 0.01), (4, 0.01)])
def test_ragged_dense_sgdm(wg, tile, wd):
    run_dense_sgdm(wg, RAGGED, 3, tile=tile, weight_decay=wd)


def test_sgdm_fused_equals_unfused(wg):
    torch = torch_mod()
    case = DenseCase("sgdm_bitwise_200x264x136", T=200, d_in=264, d_out=136, seed_base=55000)
    out = []
    for route in ("fused", "unfused"):
        W0, _, _ = synth.dense_state(case)
        W, b = f32_dev(W0), torch.zeros_like(f32_dev(W0))
        for t in (1, 2):
            Xb, dYb = synth.dense_inputs(case, t)
            if route == "fused":
                wg.forge_wgrad_sgdm(bf16_dev(Xb), bf16_dev(dYb), W, b, weight_decay=0.01)
            else:
                g = torch.empty_like(W)
                wg.forge_wgrad(bf16_dev(Xb), bf16_dev(dYb), g)
                wg.forge_sgdm(g, W, b, weight_decay=0.01)
        _sync()
        out.append((host(W), host(b)))
    assert bits_equal(out[0][0], out[1][0]) and bits_equal(out[0][1], out[1][1])


# --------------------------------------------------------------------------
# grouped (routed experts)
# --------------------------------------------------------------------------
def run_grouped(wg, X_perm_b, dY_perm_b, offsets, W, m, v, t, hp, tile=0):
    wg.forge_grouped_wgrad_adamw(bf16_dev(X_perm_b), bf16_dev(dY_perm_b), offsets, W, m, v,
                                 step=t, tile=tile, **hp)


@pytest.mark.parametrize("tile", [1, 3])
def test_grouped_small_with_empty_experts(wg, tile):
    E, d_in, d_out = 4, 136, 264
    offsets = [0, 37, 37, 100, 117]           # expert 1 empty, ragged counts
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(60, (E, d_out, d_in), 0.02)
    m0 = synth.normal_f32(61, W0.shape, 0.01)    # warm state so the empty expert's decay shows
    v0 = np.abs(synth.normal_f32(62, W0.shape, 1e-3))
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    pars = [AdamWParity(W0[e], m0[e], v0[e], hp) for e in range(E)]
    for t in (1, 2):
        log(f"[grouped small] step {t}")
        Xb = synth.normal_bf16(63 + t, (offsets[-1], d_in))
        dYb = synth.normal_bf16(73 + t, (offsets[-1], d_out))
        W_prev = host(W)
        run_grouped(wg, Xb, dYb, offsets, W, m, v, t, hp, tile=tile)
        _sync()
        Wg, mg, vg = host(W), host(m), host(v)
        grads = oracle.grouped_wgrad(Xb, dYb, offsets)
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            tau = oracle.acc_floor(Xb[a:b], dYb[a:b]) if b > a else np.zeros((d_out, d_in))
            rep = pars[e].step(t, grads[e], tau, W_prev[e], Wg[e], mg[e], vg[e])
            assert rep.passed, f"expert {e} step {t}: {rep}"
        assert not bits_equal(Wg[1], W_prev[1])   # the empty expert still moved


def test_grouped_most_experts(wg):
    """FORGE_MAX_EXPERTS (256) experts in one call, a fifth of them empty and
    the rest with 1 to 12 rows, on a small layer: the whole expert table goes
    to the kernel by value; every expert judged against the oracle over two
    steps from a warm state, and two tilings bitwise equal."""
    E, d_in, d_out = 256, 24, 16
    rng = np.random.default_rng(88)
    counts = rng.integers(1, 13, size=E)
    counts[rng.random(E) < 0.2] = 0
    offsets = [0] + [int(x) for x in np.cumsum(counts)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(89, (E, d_out, d_in), 0.02)
    m0 = synth.normal_f32(90, W0.shape, 0.01)
    v0 = np.abs(synth.normal_f32(91, W0.shape, 1e-3))
    states = {tl: [f32_dev(W0), f32_dev(m0), f32_dev(v0)] for tl in (1, 3)}
    pars = [AdamWParity(W0[e], m0[e], v0[e], hp) for e in range(E)]
    for t in (1, 2):
        log(f"[grouped E={E}] step {t}, {offsets[-1]} rows")
        Xb = synth.normal_bf16(92 + t, (offsets[-1], d_in))
        dYb = synth.normal_bf16(94 + t, (offsets[-1], d_out))
        W_prev = host(states[3][0])
        for tl, (W, m, v) in states.items():
            run_grouped(wg, Xb, dYb, offsets, W, m, v, t, hp, tile=tl)
        _sync()
        Wg, mg, vg = (host(a) for a in states[3])
        assert all(bits_equal(host(a), b) for a, b in zip(states[1], (Wg, mg, vg)))
        grads = oracle.grouped_wgrad(Xb, dYb, offsets)
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            tau = oracle.acc_floor(Xb[a:b], dYb[a:b]) if b > a else np.zeros((d_out, d_in))
            rep = pars[e].step(t, grads[e], tau, W_prev[e], Wg[e], mg[e], vg[e])
            assert rep.passed, f"expert {e} step {t}: {rep}"


@pytest.mark.parametrize("tile", [0, 4])
def test_grouped_single_expert(wg, tile):
    """A grouped call with one expert on a shape of 256 full 256x256 tiles
    (where the dense default would pick a persistent schedule): every tile id
    launches, the result matches the oracle's grouped step and is bitwise the
    256x256 grid launch."""
    d_in = d_out = 4096
    offsets = [0, 61]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(85, (1, d_out, d_in), 0.02)
    m0, v0 = np.zeros_like(W0), np.zeros_like(W0)
    Xb = synth.normal_bf16(86, (offsets[-1], d_in))
    dYb = synth.normal_bf16(87, (offsets[-1], d_out))
    out = {}
    for tl in (tile, 3):
        log(f"[grouped E=1] tile {tl}")
        W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
        run_grouped(wg, Xb, dYb, offsets, W, m, v, 1, hp, tile=tl)
        _sync()
        out[tl] = (host(W), host(m), host(v))
    par = AdamWParity(W0[0], m0[0], v0[0], hp)
    g = oracle.grouped_wgrad(Xb, dYb, offsets)[0]
    rep = par.step(1, g, oracle.acc_floor(Xb, dYb), W0[0], out[tile][0][0], out[tile][1][0],
                   out[tile][2][0])
    assert rep.passed, str(rep)
    assert all(bits_equal(a, b) for a, b in zip(out[tile], out[3]))


def test_grouped_sgdm_with_empty_experts(wg):
    """SGD-momentum on routed experts: each expert judged against the oracle's
    step on its own rows; the empty expert moves by its decay and momentum;
    each expert bitwise the dense call on its rows."""
    torch = torch_mod()
    E, d_in, d_out = 4, 136, 264
    offsets = [0, 37, 37, 100, 117]           # expert 1 empty, ragged counts
    hp = dict(lr=1e-3, momentum=0.9, weight_decay=0.01)
    W0 = synth.normal_f32(90, (E, d_out, d_in), 0.02)
    b0 = synth.normal_f32(91, W0.shape, 1e-3)    # a momentum history
    for tile in (1, 2, 3):
        W, b = f32_dev(W0), f32_dev(b0)
        pars = [SgdmParity(W0[e], b0[e], hp) for e in range(E)]
        for t in (1, 2):
            log(f"[grouped sgdm] tile {tile} step {t}")
            Xb = synth.normal_bf16(93 + t, (offsets[-1], d_in))
            dYb = synth.normal_bf16(97 + t, (offsets[-1], d_out))
            W_prev, b_prev = host(W), host(b)
            wg.forge_grouped_wgrad_sgdm(bf16_dev(Xb), bf16_dev(dYb), offsets, W, b, tile=tile,
                                        **hp)
            _sync()
            Wg, bg = host(W), host(b)
            grads = oracle.grouped_wgrad(Xb, dYb, offsets)
            for e in range(E):
                a, c = offsets[e], offsets[e + 1]
                tau = oracle.acc_floor(Xb[a:c], dYb[a:c]) if c > a else np.zeros((d_out, d_in))
                rep = pars[e].step(grads[e], tau, W_prev[e], Wg[e], bg[e])
                assert rep.passed, f"expert {e} step {t}: {rep}"
                Wd, bd = f32_dev(W_prev[e]), f32_dev(b_prev[e])
                Xe = bf16_dev(Xb[a:c]) if c > a else torch.empty((0, d_in), dtype=torch.bfloat16,
                                                                  device="cuda")
                dYe = bf16_dev(dYb[a:c]) if c > a else torch.empty((0, d_out),
                                                                    dtype=torch.bfloat16,
                                                                    device="cuda")
                wg.forge_wgrad_sgdm(Xe, dYe, Wd, bd, tile=1, **hp)
                _sync()
                assert bits_equal(Wg[e], host(Wd)) and bits_equal(bg[e], host(bd)), (tile, e)
            assert not bits_equal(Wg[1], W_prev[1])     # the empty expert still moved


def test_grouped_expert_equals_dense_call(wg):
    """Expert e of a grouped call is bitwise the dense call on its rows."""
    E, d_in, d_out = 3, 264, 136
    offsets = [0, 50, 50, 83]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(80, (E, d_out, d_in), 0.02)
    Xb = synth.normal_bf16(81, (offsets[-1], d_in))
    dYb = synth.normal_bf16(82, (offsets[-1], d_out))
    for tile in (1, 2, 3):
        W, m, v = f32_dev(W0), f32_dev(np.zeros_like(W0)), f32_dev(np.zeros_like(W0))
        run_grouped(wg, Xb, dYb, offsets, W, m, v, 1, hp, tile=tile)
        _sync()
        Wg, mg = host(W), host(m)
        torch = torch_mod()
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            Wd, md, vd = f32_dev(W0[e]), f32_dev(np.zeros_like(W0[e])), f32_dev(np.zeros_like(W0[e]))
            if b > a:
                wg.forge_wgrad_adamw(bf16_dev(Xb[a:b]), bf16_dev(dYb[a:b]), Wd, md, vd, step=1,
                                     tile=1, **hp)
            else:
                wg.forge_wgrad_adamw(torch.empty((0, d_in), dtype=torch.bfloat16, device="cuda"),
                                     torch.empty((0, d_out), dtype=torch.bfloat16, device="cuda"),
                                     Wd, md, vd, step=1, tile=1, **hp)
            _sync()
            assert bits_equal(Wg[e], host(Wd)) and bits_equal(mg[e], host(md)), (tile, e)
