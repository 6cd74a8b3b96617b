"""The library's calls captured in a HIP graph and replayed.

Every call is a plain stream-ordered kernel launch with its arguments passed
by value (no allocation, no memset, no host synchronisation), so a captured
sequence of optimizer steps must replay to the same bits as the eager calls.
Each test captures several steps, then replays the graph three times from a
freshly copied initial state, with eager work of the program between the
replays, and checks every replay bitwise against the eager run.
"""
import pytest

import synth
from synth import DenseCase, GroupedCase
from tests._gpu import adamw_hp, bf16_dev, bits_equal, f32_dev, host, host_f32, log, torch_mod

pytestmark = pytest.mark.gpu

CASE = DenseCase("graph_300x520x392", T=300, d_in=520, d_out=392, seed_base=64000)
STEPS = (1, 2, 3)


@pytest.fixture(scope="module")
def wg():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_gradient_gemm_amd as wg
    wg.library()
    return wg


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    torch = torch_mod()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, live, initial, expected, between):
    """Replay g three times, each from the initial values, and compare the
    live tensors with the expected ones bit for bit."""
    torch = torch_mod()
    for r in range(3):
        for t, t0 in zip(live, initial):
            t.copy_(t0)
        between()
        torch.cuda.synchronize()
        log(f"  replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(live, expected):
            assert bits_equal(host_f32(t), e), f"replay {r}"


@pytest.mark.parametrize("tile", [0, 3, 4])
def test_fused_adamw_steps_replay(wg, tile):
    torch = torch_mod()
    hp = adamw_hp(CASE)
    W0, m0, v0 = synth.dense_state(CASE)
    batches = [tuple(bf16_dev(a) for a in synth.dense_inputs(CASE, t)) for t in STEPS]
    log(f"[{CASE.name}] graph of {len(STEPS)} fused AdamW steps, tile {tile}")
    We, me, ve = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    for t, (X, dY) in zip(STEPS, batches):
        wg.forge_wgrad_adamw(X, dY, We, me, ve, step=t, tile=tile, **hp)
    torch.cuda.synchronize()
    expected = [host(We), host(me), host(ve)]

    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    initial = [f32_dev(W0), f32_dev(m0), f32_dev(v0)]

    def steps():
        for t, (X, dY) in zip(STEPS, batches):
            wg.forge_wgrad_adamw(X, dY, W, m, v, step=t, tile=tile, **hp)

    g = _capture(steps)
    grad = torch.empty_like(W)
    _replay_and_check(g, [W, m, v], initial, expected,
                      lambda: wg.forge_wgrad(batches[0][0], batches[0][1], grad))


def test_linear_backward_bf16w_replay(wg):
    """dX from the bf16 copy, then the fused step that refreshes it: three
    steps in one graph (two kernels per step)."""
    torch = torch_mod()
    hp = adamw_hp(CASE)
    W0, m0, v0 = synth.dense_state(CASE)
    Wb0 = synth.bf16_bits_from_f32(W0)
    batches = [tuple(bf16_dev(a) for a in synth.dense_inputs(CASE, t)) for t in STEPS]
    log(f"[{CASE.name}] graph of {len(STEPS)} linear-backward steps from the bf16 copy")

    def run(W, m, v, Wb, dXs):
        for t, (X, dY), dX in zip(STEPS, batches, dXs):
            wg.forge_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, step=t, **hp)

    def fresh_dx():
        return [torch.full((CASE.T, CASE.d_in), float("nan"), device="cuda",
                           dtype=torch.bfloat16) for _ in STEPS]

    We, me, ve, Wbe, dXe = f32_dev(W0), f32_dev(m0), f32_dev(v0), bf16_dev(Wb0), fresh_dx()
    run(We, me, ve, Wbe, dXe)
    torch.cuda.synchronize()
    expected = [host(We), host(me), host(ve), host_f32(Wbe)] + [host_f32(d) for d in dXe]

    W, m, v, Wb, dXs = f32_dev(W0), f32_dev(m0), f32_dev(v0), bf16_dev(Wb0), fresh_dx()
    initial = [f32_dev(W0), f32_dev(m0), f32_dev(v0), bf16_dev(Wb0)] + fresh_dx()
    g = _capture(lambda: run(W, m, v, Wb, dXs))
    scratch = torch.empty((CASE.T, CASE.d_in), device="cuda", dtype=torch.float32)
    _replay_and_check(g, [W, m, v, Wb] + dXs, initial, expected,
                      lambda: wg.forge_dgrad(batches[1][1], W, scratch))


def test_grouped_adamw_replay(wg):
    """Routed experts (one empty) in a graph: the host offsets are captured by
    value in the launch."""
    torch = torch_mod()
    case = GroupedCase("graph_grouped", E=8, T=200, top_k=2, d_in=264, d_out=136,
                       seed_base=65000)
    hp = adamw_hp(case)
    W0, m0, v0 = synth.grouped_state(case)
    Xb, dYb, offsets = synth.grouped_inputs(case, 1)
    offs = [int(o) for o in offsets]
    assert any(offs[e + 1] == offs[e] for e in range(case.E))      # an empty expert
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    log(f"[{case.name}] graph of 2 grouped AdamW steps")
    We, me, ve = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    for t in (1, 2):
        wg.forge_grouped_wgrad_adamw(X, dY, offs, We, me, ve, step=t, **hp)
    torch.cuda.synchronize()
    expected = [host(We), host(me), host(ve)]

    W, m, v = f32_dev(W0), f32_dev(m0), f32_dev(v0)
    initial = [f32_dev(W0), f32_dev(m0), f32_dev(v0)]

    def steps():
        for t in (1, 2):
            wg.forge_grouped_wgrad_adamw(X, dY, offs, W, m, v, step=t, **hp)

    g = _capture(steps)
    _replay_and_check(g, [W, m, v], initial, expected, lambda: None)


# fp8 inputs need d_in and d_out multiples of 16
CASE16 = DenseCase("graph_300x528x400", T=300, d_in=528, d_out=400, seed_base=66000)


@pytest.mark.parametrize("kind", ["sgdm", "bf16_state", "fp8_adamw"])
def test_other_fused_steps_replay(wg, kind):
    """The other fused epilogues in a graph: SGD-momentum, AdamW with bf16
    moments, and AdamW from fp8 inputs (three steps each)."""
    torch = torch_mod()
    case = CASE16
    hp = adamw_hp(case)
    W0, m0, v0 = synth.dense_state(case)
    if kind == "fp8_adamw":
        batches = []
        for t in STEPS:
            X8, sx, dY8, sdy = synth.dense_inputs_fp8(case, t)
            batches.append((torch.from_numpy(X8).to("cuda"), sx, torch.from_numpy(dY8).to("cuda"),
                            sdy))
    else:
        batches = [tuple(bf16_dev(a) for a in synth.dense_inputs(case, t)) for t in STEPS]
    sdt = torch.bfloat16 if kind == "bf16_state" else torch.float32
    log(f"[{case.name}] graph of {len(STEPS)} steps: {kind}")

    def state():
        W = f32_dev(W0)
        m = torch.zeros(W.shape, device="cuda", dtype=sdt)
        v = torch.zeros(W.shape, device="cuda", dtype=sdt)
        return [W, m, v]

    def run(W, m, v):
        for t, b in zip(STEPS, batches):
            if kind == "sgdm":
                wg.forge_wgrad_sgdm(b[0], b[1], W, m, lr=hp["lr"], momentum=0.9,
                                    weight_decay=hp["weight_decay"])
            elif kind == "bf16_state":
                wg.forge_wgrad_adamw_bf16state(b[0], b[1], W, m, v, step=t, **hp)
            else:
                wg.forge_wgrad_adamw_fp8(b[0], "e4m3", b[1], b[2], "e5m2", b[3], W, m, v,
                                         step=t, **hp)

    eager = state()
    run(*eager)
    torch.cuda.synchronize()
    expected = [host_f32(t) for t in eager]
    live = state()
    initial = state()
    g = _capture(lambda: run(*live))
    _replay_and_check(g, live, initial, expected, lambda: run(*state()))
