"""A seeded sweep of ragged shapes through the main calls, each judged against
the oracle: T from 1 to 600 tokens, d_in and d_out any multiple of 8 (of 16
for fp8) up to 640, a tile id drawn at random. The fixed cases elsewhere pick
their tails by hand; this sweep walks residues of every tile and stage size
(256, 128, 64, 32, 16, 8) that they do not.

Per shape: one fused AdamW step (W, m, v judged element by element against
the oracle's step on its exact gradient), one fused SGD-momentum step with
weight decay (judged the same way), the input gradient from the float32
weight (judged) and from its bf16 copy (bitwise the same); on the same shapes
rounded up to multiples of 16, the fp8-input gradient (judged against the
exact fp8 sum, and against the model of the fp8 instruction with the float32
floor alone). A second sweep draws routed-expert calls: 1 to 12 experts with
random row counts (some empty) on random layers, every expert judged.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import judge, lowp
from synth import DenseCase
from tests._gpu import (AdamWParity, SgdmParity, adamw_hp, bf16_dev, bits_equal, f32_dev, host,
                        host_f32, log, torch_mod)

pytestmark = pytest.mark.gpu


def _shapes(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        T = int(rng.integers(1, 601))
        d_in = 8 * int(rng.integers(1, 81))
        d_out = 8 * int(rng.integers(1, 81))
        tile = int(rng.integers(0, 5))
        out.append((DenseCase(f"sweep{k}_{T}x{d_in}x{d_out}", T=T, d_in=d_in, d_out=d_out,
                              seed_base=80000 + 100 * k, steps=1), tile))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def wg():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_gradient_gemm_amd as wg
    wg.library()
    return wg


@pytest.mark.parametrize("case,tile", SHAPES, ids=[f"{c.name}_t{t}" for c, t in SHAPES])
def test_sweep_fused_adamw_and_dgrad(wg, case, tile):
    torch = torch_mod()
    hp = adamw_hp(case)
    Xb, dYb = synth.dense_inputs(case, 1)
    W0, m0, v0 = synth.dense_state(case)
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    log(f"[{case.name}] input gradient (float32 weight and bf16 copy)")
    dX = torch.full((case.T, case.d_in), float("nan"), device="cuda", dtype=torch.bfloat16)
    dXc = torch.full_like(dX, float("nan"))
    wg.forge_dgrad(dY, f32_dev(W0), dX, tile=tile)
    wg.forge_dgrad_bf16w(dY, bf16_dev(synth.bf16_bits_from_f32(W0)), dXc, tile=tile)
    torch.cuda.synchronize()
    rep = judge.judge_dgrad(host_f32(dX), dYb, W0, True)
    assert rep.passed, str(rep)
    assert bits_equal(host_f32(dX), host_f32(dXc))

    log(f"[{case.name}] fused AdamW step, tile {tile}")
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    wg.forge_wgrad_adamw(X, dY, W, m, v, step=1, tile=tile, **hp)
    torch.cuda.synchronize()
    par = AdamWParity(W0, m0, v0, hp)
    g_ref, tau = oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb)
    rep = par.step(1, g_ref, tau, W0, host(W), host(m), host(v))
    assert rep.passed, str(rep)

    log(f"[{case.name}] fused SGD-momentum step, tile {tile}")
    hs = dict(lr=case.lr, momentum=case.momentum, weight_decay=0.01)
    b0 = synth.normal_f32(case.seed_base + 7, W0.shape, 1e-3)      # a momentum history
    W, b = f32_dev(W0), f32_dev(b0)
    wg.forge_wgrad_sgdm(X, dY, W, b, tile=tile, **hs)
    torch.cuda.synchronize()
    spar = SgdmParity(W0, b0, hs)
    rep = spar.step(g_ref, tau, W0, host(W), host(b))
    assert rep.passed, str(rep)


def _up16(d):
    return d + (d % 16)


# The same shapes with d_in and d_out rounded up to multiples of 16.
FP8_SHAPES = [(DenseCase(f"fp8_{c.name}", T=c.T, d_in=_up16(c.d_in), d_out=_up16(c.d_out),
                         seed_base=c.seed_base + 50, steps=1), t) for c, t in SHAPES]


@pytest.mark.parametrize("case,tile", FP8_SHAPES, ids=[f"{c.name}_t{t}" for c, t in FP8_SHAPES])
def test_sweep_fp8_gradient(wg, case, tile):
    torch = torch_mod()
    X8, sx, dY8, sdy = synth.dense_inputs_fp8(case, 1)
    log(f"[{case.name}] fp8 gradient, tile {tile}")
    g = torch.full((case.d_out, case.d_in), float("nan"), device="cuda")
    wg.forge_wgrad_fp8(torch.from_numpy(X8).to("cuda"), "e4m3", sx,
                       torch.from_numpy(dY8).to("cuda"), "e5m2", sdy, g, tile=tile)
    torch.cuda.synchronize()
    ref = lowp.wgrad_fp8_f64(X8, "e4m3", sx, dY8, "e5m2", sdy)
    err = np.abs(host(g).astype(np.float64) - ref)
    tau = lowp.acc_floor_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy)
    assert np.all(err <= tau), f"max err / floor {np.max(err / tau):.3f}"
    model = lowp.mfma_fp8_dot(X8, "e4m3", dY8, "e5m2") * float(np.float32(sx * sdy))
    inner = lowp.acc_floor_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy, dot_loss=False)
    err_m = np.abs(host(g).astype(np.float64) - model)
    assert np.all(err_m <= inner), f"model: max err / fp32 floor {np.max(err_m / inner):.3f}"


def _grouped_cases(n=16, seed=4048):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        E = int(rng.integers(1, 13))
        counts = rng.integers(0, 200, size=E)
        counts[rng.random(E) < 0.25] = 0
        d_in = 8 * int(rng.integers(1, 49))
        d_out = 8 * int(rng.integers(1, 49))
        tile = int(rng.choice([0, 1, 2, 3]))
        out.append((k, [0] + [int(x) for x in np.cumsum(counts)], d_in, d_out, tile))
    return out


GROUPED = _grouped_cases()


@pytest.mark.parametrize("k,offsets,d_in,d_out,tile", GROUPED,
                         ids=[f"g{k}_E{len(o) - 1}_R{o[-1]}_{di}x{do}_t{t}"
                              for k, o, di, do, t in GROUPED])
def test_sweep_grouped_adamw(wg, k, offsets, d_in, d_out, tile):
    E = len(offsets) - 1
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    W0 = synth.normal_f32(90000 + 10 * k, (E, d_out, d_in), 0.02)
    m0 = synth.normal_f32(90001 + 10 * k, W0.shape, 0.01)
    v0 = np.abs(synth.normal_f32(90002 + 10 * k, W0.shape, 1e-3))
    Xb = synth.normal_bf16(90003 + 10 * k, (offsets[-1], d_in))
    dYb = synth.normal_bf16(90004 + 10 * k, (offsets[-1], d_out))
    log(f"[grouped sweep {k}] E {E}, rows {offsets[-1]}, {d_in}x{d_out}, tile {tile}")
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    wg.forge_grouped_wgrad_adamw(bf16_dev(Xb), bf16_dev(dYb), offsets, W, m, v, step=3,
                                 tile=tile, **hp)
    torch_mod().cuda.synchronize()
    Wg, mg, vg = host(W), host(m), host(v)
    grads = oracle.grouped_wgrad(Xb, dYb, offsets)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        tau = oracle.acc_floor(Xb[a:b], dYb[a:b]) if b > a else np.zeros((d_out, d_in))
        par = AdamWParity(W0[e], m0[e], v0[e], hp)
        rep = par.step(3, grads[e], tau, W0[e], Wg[e], mg[e], vg[e])
        assert rep.passed, f"expert {e}: {rep}"
