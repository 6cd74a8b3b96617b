"""Edge cases of the fused step on the GPU.

- A run split in two with the state taken to the host and back in between (a
  checkpoint and a resume) is bitwise the same as the run in one piece: the
  step depends only on W, m, v, the inputs and the step number (FORGE
  assessment, "Math verified, not asserted", P1: exact and repeatable).
- The smallest shapes the ABI accepts (d_in and d_out multiples of 8, one to
  a few tokens), on every tile id, against the oracle: every tile is a tail in
  both directions and the token loop has a single partial stage.
- The largest d_in and the largest d_out the ABI accepts (2^22), each with the
  other dimension at its smallest, a ragged token count and every element
  judged: the largest stage rows and state rows the 32-bit buffer windows
  hold, and 16384 tiles along one axis; and 2^22 + 17 tokens on a small layer.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import DenseCase
from oracle import judge
from tests._gpu import (AdamWParity, SgdmParity, adamw_hp, bf16_dev, bits_equal, f32_dev, host,
                        host_f32, log, run_dense_adamw, torch_mod)

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


@pytest.mark.parametrize("tile", [0, 4])
def test_split_run_equals_whole_run(wg, tile):
    case = DenseCase("split_300x520x392", T=300, d_in=520, d_out=392, seed_base=66000, steps=10)
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    batches = [tuple(bf16_dev(a) for a in synth.dense_inputs(case, t)) for t in range(1, 11)]
    log(f"[{case.name}] 10 AdamW steps in one run and as 5 + 5 with a host round trip, tile {tile}")
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    for t, (X, dY) in enumerate(batches, 1):
        wg.forge_wgrad_adamw(X, dY, W, m, v, step=t, tile=tile, **hp)
    W2, m2, v2 = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    for t, (X, dY) in enumerate(batches[:5], 1):
        wg.forge_wgrad_adamw(X, dY, W2, m2, v2, step=t, tile=tile, **hp)
    _sync()
    saved = [host(W2), host(m2), host(v2)]                 # checkpoint
    del W2, m2, v2
    W2, m2, v2 = (f32_dev(a) for a in saved)               # resume in fresh buffers
    for t, (X, dY) in enumerate(batches[5:], 6):
        wg.forge_wgrad_adamw(X, dY, W2, m2, v2, step=t, tile=tile, **hp)
    _sync()
    assert bits_equal(host(W), host(W2))
    assert bits_equal(host(m), host(m2)) and bits_equal(host(v), host(v2))


@pytest.mark.parametrize("T,d_in,d_out", [(1, 8, 8), (4, 8, 8), (8, 16, 8), (17, 8, 24)])
@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_smallest_shapes(wg, T, d_in, d_out, tile):
    torch = torch_mod()
    case = DenseCase(f"tiny_{T}x{d_in}x{d_out}", T=T, d_in=d_in, d_out=d_out,
                     seed_base=67000 + 100 * T + d_in + d_out, steps=2)
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    par = AdamWParity(W0, m0, v0, hp)
    for t in (1, 2):
        Xb, dYb = synth.dense_inputs(case, t)
        log(f"[{case.name}] AdamW step {t}, tile {tile}")
        W_prev = host(W)
        wg.forge_wgrad_adamw(bf16_dev(Xb), bf16_dev(dYb), W, m, v, step=t, tile=tile, **hp)
        _sync()
        rep = par.step(t, oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W_prev, host(W),
                       host(m), host(v))
        assert rep.passed, str(rep)
    hs = dict(lr=case.lr, momentum=case.momentum, weight_decay=0.01)
    Xb, dYb = synth.dense_inputs(case, 3)
    W, b = f32_dev(W0), f32_dev(np.zeros_like(W0))
    spar = SgdmParity(W0, np.zeros_like(W0), hs)
    wg.forge_wgrad_sgdm(bf16_dev(Xb), bf16_dev(dYb), W, b, tile=tile, **hs)
    _sync()
    rep = spar.step(oracle.wgrad(Xb, dYb), oracle.acc_floor(Xb, dYb), W0, host(W), host(b))
    assert rep.passed, str(rep)
    g = torch.full((d_out, d_in), float("nan"), device="cuda")
    wg.forge_wgrad(bf16_dev(Xb), bf16_dev(dYb), g, tile=tile)
    _sync()
    err = np.abs(host(g).astype(np.float64) - oracle.wgrad_f64(Xb, dYb))
    assert np.all(err <= oracle.acc_floor(Xb, dYb))


MAX_DIM = 1 << 22                                     # the ABI's largest d_in and d_out


@pytest.mark.parametrize("d_in,d_out", [(MAX_DIM, 8), (8, MAX_DIM)], ids=["max_d_in", "max_d_out"])
@pytest.mark.parametrize("tile", [0, 3])
def test_largest_dims(wg, d_in, d_out, tile):
    torch = torch_mod()
    case = DenseCase(f"maxdim_33x{d_in}x{d_out}", T=33, d_in=d_in, d_out=d_out,
                     seed_base=68000 + (d_in > d_out), steps=2)
    W, _, _ = run_dense_adamw(wg, case, 2, tile=tile)
    # the input gradient from the updated weight (K = d_out up to 2^22)
    Xb, dYb = synth.dense_inputs(case, 3)
    W_host = host(W)
    dX = torch.full((case.T, d_in), float("nan"), device="cuda", dtype=torch.bfloat16)
    log(f"[{case.name}] dX, tile {tile}")
    wg.forge_dgrad(bf16_dev(dYb), W, dX, tile=0 if tile == 0 else 3)
    _sync()
    rep = judge.judge_dgrad(host_f32(dX), dYb, W_host, True)
    assert rep.passed, str(rep)


@pytest.mark.parametrize("tile", [0, 3])
def test_many_tokens(wg, tile):
    """2^22 + 17 tokens (131073 stages of one tile, the last one partial) on a
    small layer: the stage counters and running pointers over a long token
    loop, every element judged. No budget on widened weight-delta bars: the
    float32 floor grows like sqrt(T) against a random gradient (here ~5e-4 of
    it), so at step 2 a correct float32 order can move an ordinary element's
    update by ~1e-3 lr, and a fifth of these 128 weights are ambiguous."""
    case = DenseCase("manytok_4194321x16x8", T=(1 << 22) + 17, d_in=16, d_out=8,
                     seed_base=68100, steps=2)
    run_dense_adamw(wg, case, 2, tile=tile, ambiguous_budget=None)


def test_tensor_on_another_device_is_refused(wg, monkeypatch):
    """The binding refuses tensors and streams that are not on the current
    device (the launch would touch another GPU's memory) before calling the
    library; on the right device the same call runs."""
    torch = torch_mod()
    X = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((16, 32), dtype=torch.bfloat16, device="cuda")
    W, m, v = (torch.zeros((32, 64), device="cuda") for _ in range(3))
    real = torch.cuda.current_device()
    monkeypatch.setattr(torch.cuda, "current_device", lambda: real + 1)
    with pytest.raises(ValueError, match="current device"):
        wg.forge_wgrad_adamw(X, dY, W, m, v, step=1)
    s = torch.cuda.Stream()                         # a stream of the real device
    with pytest.raises(ValueError, match="current device"):
        wg._lib._stream(s)
    monkeypatch.undo()
    wg.forge_wgrad_adamw(X, dY, W, m, v, step=1, stream=s)
    s.synchronize()
    wg.forge_wgrad_adamw(X, dY, W, m, v, step=2)
    _sync()
    assert not np.any(host(m)) and bits_equal(host(W), np.zeros((32, 64), np.float32))

