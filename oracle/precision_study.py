"""CPU study: what the float32 gradient buys, with float32 and with bf16 state.

TEST INFRASTRUCTURE ONLY (runs the oracle's own arithmetic; nothing on the
product path imports it).

FORGE assessment, "Math verified, not asserted", P6: keeping the weight
gradient in the float32 accumulator instead of rounding it to bf16 (the
rounding the existing lowering performs, section "What's already in tree and
easy to miss") is worth about 900x in accuracy when the optimizer state is
float32, and about 1x when the state itself is bf16. The page gives neither
the setup nor the error measure. Reading taken here: the error of a short
AdamW run against a float64 run on the same inputs, measured on the total
parameter change W_K - W_0 (normwise relative), and the benefit is the ratio
of the bf16-gradient error to the float32-gradient error at equal state
precision.

Variants (gradient precision, state precision):
  fp32        float32 gradient, float32 m, v
  bf16_grad   bf16 gradient,    float32 m, v
  bf16_state  float32 gradient, bf16 m, v
  bf16_both   bf16 gradient,    bf16 m, v
The float32 gradient here is the correctly rounded one (oracle.wgrad); a GPU
run replaces it with its float32 accumulation, whose error is larger.
"""
from __future__ import annotations

import numpy as np

from .ref import adamw_step_f64, adamw_step_mixed, bf16_round, wgrad, wgrad_f64

VARIANTS = {"fp32": (False, False), "bf16_grad": (True, False),
            "bf16_state": (False, True), "bf16_both": (True, True)}


def normwise(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def errors(W0, runs: dict, ref) -> dict:
    """Normwise relative errors of each run's (W, m, v) against ref's; the
    parameter change is taken from W0."""
    W0 = np.asarray(W0, dtype=np.float64)
    Wr, mr, vr = ref
    out = {}
    for name, (W, m, v) in runs.items():
        out[name] = {"dW": normwise(np.asarray(W, np.float64) - W0, np.asarray(Wr) - W0),
                     "m": normwise(m, mr), "v": normwise(v, vr)}
    return out


def benefits(err: dict) -> dict:
    """bf16-gradient error over float32-gradient error, per state precision."""
    return {"fp32_state": {k: err["bf16_grad"][k] / err["fp32"][k] for k in ("dW", "m", "v")},
            "bf16_state": {k: err["bf16_both"][k] / err["bf16_state"][k] for k in ("dW", "m", "v")}}


def reference_run(W0, inputs, hp: dict):
    """The float64 run: exact gradient, float64 AdamW. inputs: per-step
    (X_bits, dY_bits)."""
    W = np.asarray(W0, dtype=np.float64)
    m = np.zeros_like(W)
    v = np.zeros_like(W)
    for t, (Xb, dYb) in enumerate(inputs, start=1):
        W, m, v = adamw_step_f64(W, m, v, wgrad_f64(Xb, dYb), t, **hp)
    return W, m, v


def run(d_in: int = 256, d_out: int = 256, T: int = 1024, steps: int = 8, seed: int = 11,
        lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
        weight_decay: float = 0.01) -> dict:
    """The four variants and the float64 reference on one seeded input stream
    (X, dY ~ N(0, 1) in bf16, W0 ~ N(0, 0.02^2), zero initial state)."""
    from synth import normal_bf16, normal_f32   # seeded inputs only

    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)
    W0 = normal_f32(seed, (d_out, d_in), 0.02)
    inputs = [(normal_bf16(seed + 2 * t, (T, d_in)), normal_bf16(seed + 2 * t + 1, (T, d_out)))
              for t in range(1, steps + 1)]
    runs = {}
    for name, (gb, sb) in VARIANTS.items():
        W = W0.copy()
        m = np.zeros_like(W0)
        v = np.zeros_like(W0)
        for t, (Xb, dYb) in enumerate(inputs, start=1):
            W, m, v = adamw_step_mixed(W, m, v, wgrad(Xb, dYb), t, gb, sb, **hp)
        runs[name] = (W, m, v)
    ref = reference_run(W0, inputs, hp)
    err = errors(W0, runs, ref)
    return {"errors": err, "benefit": benefits(err), "runs": runs, "reference": ref,
            "setup": dict(d_in=d_in, d_out=d_out, T=T, steps=steps, seed=seed, **hp)}


def bf16_state_is_representable(m) -> bool:
    """Every value of a bf16 state buffer is a bf16 value."""
    m = np.asarray(m, dtype=np.float32)
    return bool(np.array_equal(bf16_round(m).view(np.uint32), m.view(np.uint32)))


if __name__ == "__main__":   # pragma: no cover - prints the table quoted in the design notes
    res = run()
    print("setup:", res["setup"])
    for name, e in res["errors"].items():
        print(f"{name:11s} dW {e['dW']:.3e}  m {e['m']:.3e}  v {e['v']:.3e}")
    for k, b in res["benefit"].items():
        print(f"benefit with {k}: dW {b['dW']:.1f}x  m {b['m']:.1f}x  v {b['v']:.1f}x")
