"""CPU study: global-norm clipping around a gradient spike.

TEST INFRASTRUCTURE ONLY (a host-side study on the oracle's own AdamW
arithmetic; nothing on the product path imports it).

FORGE assessment, "Math verified, not asserted", P2: exact global-norm
clipping scales the whole gradient by min(1, c / ||g||) before any moment is
updated, so a per-tile epilogue cannot apply it (the clipped first moment
differs from the unclipped one by a term in the previous moment). The page
then states that the two approximations one might fuse instead both fail:
clipping the update after the optimizer, and clipping with the previous
step's norm, each leave sqrt(v) inflated after a gradient spike exactly as
much as no clipping at all (3.18x ten steps after the spike, setup not given).

This study runs the four variants side by side on the same gradient stream:
  exact       g_t <- g_t min(1, c / ||g_t||), then AdamW
  none        AdamW on g_t
  clip_update AdamW on g_t, then the parameter change scaled to norm <= u_max
  delayed     g_t <- g_t min(1, c / ||g_{t-1}||), then AdamW
The gradient stream is N(0, 1) per element, steady state (a long warm-up so
the bias corrections are ~1), then one step multiplied by `spike`. Reported:
sqrt of the mean bias-corrected second moment, and the mean of its square
root, each as a ratio to the exact-clipping run, `after` steps past the
spike. The AdamW arithmetic is the oracle's float32 step (oracle.ref).
"""
from __future__ import annotations

import numpy as np

from .ref import F32, adamw_moments, adamw_param

VARIANTS = ("exact", "none", "clip_update", "delayed")


def _norm(x) -> float:
    return float(np.sqrt(np.sum(np.asarray(x, dtype=np.float64) ** 2)))


def run(P: int = 4096, warm: int = 3000, spike: float = 100.0, after: int = 10,
        clip_factor: float = 1.0, seed: int = 7, lr: float = 1e-3, beta1: float = 0.9,
        beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0) -> dict:
    """Run the four variants; returns per-variant trajectories and ratios.

    c = clip_factor * sqrt(P), the expected norm of an N(0, 1) gradient, so
    exact clipping leaves ordinary steps alone and scales the spike back to an
    ordinary norm. u_max (clip_update) is the largest parameter-change norm
    seen during the warm-up, so only the spike step's change is clipped.
    """
    rng = np.random.default_rng(seed)
    steps = warm + 1 + after
    grads = rng.standard_normal((steps, P)).astype(F32)
    grads[warm] *= F32(spike)                      # step warm + 1 (1-based) is the spike
    c = clip_factor * np.sqrt(P)
    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay)

    # u_max from the unclipped warm-up (identical in every variant up to the spike)
    W = np.zeros(P, F32); m = np.zeros(P, F32); v = np.zeros(P, F32)
    u_max = 0.0
    for t in range(1, warm + 1):
        m, v = adamw_moments(m, v, grads[t - 1], beta1, beta2)
        W_new = adamw_param(W, m, v, t, lr, beta1, beta2, eps, weight_decay)
        u_max = max(u_max, _norm(W_new.astype(np.float64) - W))
        W = W_new

    out = {}
    for name in VARIANTS:
        W = np.zeros(P, F32); m = np.zeros(P, F32); v = np.zeros(P, F32)
        prev_norm = None
        rms, mean_sqrt = [], []
        for t in range(1, steps + 1):
            g = grads[t - 1]
            if name == "exact":
                g = g * F32(min(1.0, c / _norm(g)))
            elif name == "delayed" and prev_norm is not None:
                g = g * F32(min(1.0, c / prev_norm))
            prev_norm = _norm(grads[t - 1])
            m, v = adamw_moments(m, v, g, beta1, beta2)
            W_new = adamw_param(W, m, v, t, **hp)
            if name == "clip_update":
                d = W_new.astype(np.float64) - W
                dn = _norm(d)
                if dn > u_max:
                    W_new = (W + d * (u_max / dn)).astype(F32)
            W = W_new
            v_hat = v.astype(np.float64) / (1.0 - beta2 ** t)
            rms.append(float(np.sqrt(np.mean(v_hat))))
            mean_sqrt.append(float(np.mean(np.sqrt(v_hat))))
        out[name] = {"v": v, "m": m, "W": W, "rms_sqrt_v": rms, "mean_sqrt_v": mean_sqrt}

    k = warm + after                               # index of `after` steps past the spike
    ratios = {name: {"rms_sqrt_v": out[name]["rms_sqrt_v"][k] / out["exact"]["rms_sqrt_v"][k],
                     "mean_sqrt_v": out[name]["mean_sqrt_v"][k] / out["exact"]["mean_sqrt_v"][k]}
              for name in VARIANTS}
    return {"runs": out, "ratios": ratios, "clip_norm": c, "update_norm_max": u_max,
            "setup": dict(P=P, warm=warm, spike=spike, after=after, clip_factor=clip_factor,
                          seed=seed, **hp)}


if __name__ == "__main__":   # pragma: no cover - prints the table quoted in the design notes
    res = run()
    print("setup:", res["setup"])
    for name, r in res["ratios"].items():
        print(f"{name:12s} sqrt(mean v_hat) ratio {r['rms_sqrt_v']:.3f}   "
              f"mean sqrt(v_hat) ratio {r['mean_sqrt_v']:.3f}")
