"""GPU parity of the fp8-input weight gradient (page "docs(audit): FORGE
assessment + residency-aware epilogue-fusion track", section "Math verified,
not asserted", P6: the paper's fp8 row).

The fp8 kernels against the oracle's exact scaled contraction within the
float32 accumulation floor plus the measured loss of the fp8 dot product
(oracle.lowp.mfma_fp8_floor), every tiling bitwise equal, the fused AdamW step
judged like the bf16 one and bitwise equal to the unfused pair, subnormal
codes, and the fp8-vs-bf16 accuracy study on the GPU.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import lowp
from synth import DenseCase
from tests._gpu import (AdamWParity, adamw_hp, bf16_dev, bits_equal, f32_dev, host, log,
                        torch_mod)

pytestmark = pytest.mark.gpu

FMTS = [("e4m3", "e5m2"), ("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e5m2", "e4m3")]
# fp8 rows need d_in, d_out multiples of 16; T tails of 13 and 44 tokens in 64-token stages
RAGGED = DenseCase("fp8_ragged_77x272x208", T=77, d_in=272, d_out=208, seed_base=70000, steps=3)
MANY = DenseCase("fp8_tiles_300x528x400", T=300, d_in=528, d_out=400, seed_base=71000, steps=2)
PERSIST = DenseCase("fp8_persistent_45x4368x4112", T=45, d_in=4368, d_out=4112,
                    seed_base=72000, steps=2)


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


def u8_dev(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def _inputs(case, step, fx, fy):
    X8, sx, dY8, sdy = synth.dense_inputs_fp8(case, step, fx, fy)
    return X8, sx, dY8, sdy


def _grad(wg, X8, fx, sx, dY8, fy, sdy, d_in, d_out, tile):
    torch = torch_mod()
    g = torch.full((d_out, d_in), float("nan"), device="cuda")
    wg.forge_wgrad_fp8(u8_dev(X8), fx, sx, u8_dev(dY8), fy, sdy, g, tile=tile)
    _sync()
    return host(g)


@pytest.mark.parametrize("fx,fy", FMTS)
@pytest.mark.parametrize("tile", [1, 2, 3, 4])
@pytest.mark.parametrize("case", [RAGGED, MANY], ids=lambda c: c.name)
def test_wgrad_fp8_against_oracle(wg, case, tile, fx, fy):
    X8, sx, dY8, sdy = _inputs(case, 1, fx, fy)
    log(f"[{case.name}] fp8 {fx} x {fy} tile {tile}")
    g = _grad(wg, X8, fx, sx, dY8, fy, sdy, case.d_in, case.d_out, tile)
    err = np.abs(g.astype(np.float64) - lowp.wgrad_fp8_f64(X8, fx, sx, dY8, fy, sdy))
    tau = lowp.acc_floor_fp8(X8, fx, sx, dY8, fy, sdy)
    log(f"  max err / floor {np.max(err / tau):.3f}")
    assert np.all(err <= tau)


def test_wgrad_fp8_non_power_of_two_scales(wg):
    X8, sx, dY8, sdy = _inputs(MANY, 2, "e4m3", "e5m2")
    sx, sdy = sx * 0.37, sdy * 1.9
    g = _grad(wg, X8, "e4m3", sx, dY8, "e5m2", sdy, MANY.d_in, MANY.d_out, 0)
    err = np.abs(g.astype(np.float64) - lowp.wgrad_fp8_f64(X8, "e4m3", sx, dY8, "e5m2", sdy))
    assert np.all(err <= lowp.acc_floor_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy))


def test_wgrad_fp8_subnormal_codes(wg):
    """Every code of both formats, subnormals included (NaN and inf codes
    excepted), against the exact oracle."""
    rng = np.random.default_rng(7)
    T, d_in, d_out = 96, 64, 48
    X8 = rng.integers(0, 256, (T, d_in), dtype=np.uint8)
    dY8 = rng.integers(0, 256, (T, d_out), dtype=np.uint8)
    X8[(X8 & 0x7F) == 0x7F] = 0x01                          # e4m3 NaN -> smallest subnormal
    dY8[(dY8 & 0x7C) == 0x7C] = 0x02                        # e5m2 inf/NaN -> a subnormal
    X8[:8] = rng.integers(0, 8, (8, d_in)) | (rng.integers(0, 2, (8, d_in)) << 7)   # subnormals
    dY8[:8] = rng.integers(0, 4, (8, d_out)) | (rng.integers(0, 2, (8, d_out)) << 7)
    g = _grad(wg, X8, "e4m3", 1.0, dY8, "e5m2", 1.0, d_in, d_out, 1)
    err = np.abs(g.astype(np.float64) - lowp.wgrad_fp8_f64(X8, "e4m3", 1.0, dY8, "e5m2", 1.0))
    assert np.all(err <= lowp.acc_floor_fp8(X8, "e4m3", 1.0, dY8, "e5m2", 1.0))
    # rows of subnormals alone: no flush to zero
    Xs, Ys = X8[:8].copy(), dY8[:8].copy()
    g_sub = _grad(wg, Xs, "e4m3", 1.0, Ys, "e5m2", 1.0, d_in, d_out, 1)
    ref_sub = lowp.wgrad_fp8_f64(Xs, "e4m3", 1.0, Ys, "e5m2", 1.0)
    assert np.all(np.abs(g_sub - ref_sub) <= lowp.acc_floor_fp8(Xs, "e4m3", 1.0, Ys, "e5m2", 1.0))
    assert np.count_nonzero(g_sub) >= 0.5 * np.count_nonzero(ref_sub) > 0


def test_wgrad_fp8_bitwise_across_tilings(wg):
    X8, sx, dY8, sdy = _inputs(PERSIST, 1, "e4m3", "e5m2")
    outs = [_grad(wg, X8, "e4m3", sx, dY8, "e5m2", sdy, PERSIST.d_in, PERSIST.d_out, t)
            for t in (4, 3, 1, 2, 4)]
    assert all(bits_equal(o, outs[0]) for o in outs[1:])
    rows = np.array([0, 255, 256, 4111])
    err = np.abs(outs[0][rows].astype(np.float64)
                 - lowp.wgrad_fp8_f64(X8, "e4m3", sx, np.ascontiguousarray(dY8[:, rows]), "e5m2",
                                      sdy))
    assert np.all(err <= lowp.acc_floor_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy, rows=rows))


@pytest.mark.parametrize("tile", [1, 4])
def test_fused_adamw_fp8(wg, tile):
    case = RAGGED
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    par = AdamWParity(W0, m0, v0, hp)
    for t in range(1, case.steps + 1):
        X8, sx, dY8, sdy = _inputs(case, t, "e4m3", "e5m2")
        log(f"[{case.name}] fp8 adamw step {t} tile {tile}")
        W_prev = host(W)
        wg.forge_wgrad_adamw_fp8(u8_dev(X8), "e4m3", sx, u8_dev(dY8), "e5m2", sdy, W, m, v,
                                 step=t, tile=tile, **hp)
        _sync()
        rep = par.step(t, lowp.wgrad_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy),
                       lowp.acc_floor_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy), W_prev, host(W),
                       host(m), host(v))
        log(f"  {rep}")
        assert rep.passed, f"step {t}: {rep}"


def test_fused_adamw_fp8_equals_unfused(wg):
    torch = torch_mod()
    case = MANY
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    out = []
    for route in ("fused", "unfused"):
        W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
        for t in (1, 2):
            X8, sx, dY8, sdy = _inputs(case, t, "e4m3", "e5m2")
            if route == "fused":
                wg.forge_wgrad_adamw_fp8(u8_dev(X8), "e4m3", sx, u8_dev(dY8), "e5m2", sdy, W, m,
                                         v, step=t, **hp)
            else:
                g = torch.empty_like(W)
                wg.forge_wgrad_fp8(u8_dev(X8), "e4m3", sx, u8_dev(dY8), "e5m2", sdy, g)
                wg.forge_adamw(g, W, m, v, step=t, **hp)
        _sync()
        out.append((host(W), host(m), host(v)))
    assert all(bits_equal(a, b) for a, b in zip(out[0], out[1]))


def test_fp8_vs_bf16_study_on_gpu(wg):
    """The paper's fp8 row on the GPU: gradient and update errors of fp8 and
    bf16 inputs (same float32 draws) against a float64 run."""
    torch = torch_mod()
    d_in = d_out = 512
    T, steps, seed = 4096, 6, 41
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(seed, (d_out, d_in), 0.02)
    Wb, mb, vb = f32_dev(W0), torch.zeros(W0.shape, device="cuda"), torch.zeros(W0.shape,
                                                                                 device="cuda")
    W8, m8, v8 = f32_dev(W0), torch.zeros_like(mb), torch.zeros_like(mb)
    Wr, mr, vr = W0.astype(np.float64), np.zeros(W0.shape), np.zeros(W0.shape)
    g_err = None
    for t in range(1, steps + 1):
        X = synth.normal_f32(seed + 2 * t, (T, d_in))
        dY = synth.normal_f32(seed + 2 * t + 1, (T, d_out))
        g_ref = dY.astype(np.float64).T @ X.astype(np.float64)
        Xb, dYb = synth.bf16_bits_from_f32(X), synth.bf16_bits_from_f32(dY)
        X8, sx, dY8, sdy = synth.fp8_inputs(X, dY)
        if t == 1:
            gb = torch.empty(W0.shape, device="cuda")
            wg.forge_wgrad(bf16_dev(Xb), bf16_dev(dYb), gb)
            g8 = torch.empty(W0.shape, device="cuda")
            wg.forge_wgrad_fp8(u8_dev(X8), "e4m3", sx, u8_dev(dY8), "e5m2", sdy, g8)
            _sync()
            g_err = (lowp_norm(host(gb), g_ref), lowp_norm(host(g8), g_ref))
        wg.forge_wgrad_adamw(bf16_dev(Xb), bf16_dev(dYb), Wb, mb, vb, step=t, **hp)
        wg.forge_wgrad_adamw_fp8(u8_dev(X8), "e4m3", sx, u8_dev(dY8), "e5m2", sdy, W8, m8, v8,
                                 step=t, **hp)
        Wr, mr, vr = oracle.adamw_step_f64(Wr, mr, vr, g_ref, t, **hp)
    _sync()
    dref = Wr - W0
    u_err = (lowp_norm(host(Wb).astype(np.float64) - W0, dref),
             lowp_norm(host(W8).astype(np.float64) - W0, dref))
    log(f"[fp8 study] gradient error bf16 {g_err[0]:.3e} fp8 {g_err[1]:.3e} "
        f"ratio {g_err[1] / g_err[0]:.1f}x; update error bf16 {u_err[0]:.3e} fp8 {u_err[1]:.3e} "
        f"ratio {u_err[1] / u_err[0]:.1f}x")
    assert 10 < g_err[1] / g_err[0] < 100
    assert u_err[1] > u_err[0]


def lowp_norm(a, ref):
    from oracle.precision_study import normwise
    return normwise(a, ref)
