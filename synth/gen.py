"""Seeded synthetic workloads for the fused weight-gradient + optimizer path.

Every array is a pure function of an integer seed and a shape. Nothing here
computes any part of the method: the functions draw random numbers, encode
them as bfloat16 bit patterns, and lay out routing tables.

Seed convention (one per config ``k``):
  * inputs of optimizer step ``s`` (1-based): ``1000*k + s``
  * weight initialisation:                   ``1000*k + 999``
  * routing of the grouped (MoE) workload:    ``1000*k + 998``

Large arrays are drawn in fixed chunks of ``CHUNK`` elements, chunk ``c`` from
``SeedSequence(seed, spawn_key=(c,))``, so the values do not depend on how many
threads fill them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 20


# --------------------------------------------------------------------------
# primitive draws and encodings
# --------------------------------------------------------------------------
def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) in float32: a float32 standard normal times float32(std)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    s32 = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(c,))))
        seg = out[lo:hi]
        rng.standard_normal(hi - lo, dtype=np.float32, out=seg)
        if std != 1.0:
            np.multiply(seg, s32, out=seg)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns (uint16).

    Round to nearest, ties to even (what ``torch.Tensor.to(torch.bfloat16)``
    does). Results that would be bfloat16 subnormals are flushed to a signed
    zero, so no device denormal mode can change a product. Inputs are finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    b = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    sub = (b & np.uint16(0x7F80)) == 0
    b[sub] &= np.uint16(0x8000)
    return b


def normal_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    return bf16_bits_from_f32(normal_f32(seed, shape, std))


# fp8 (OCP) encodings: exponent bits, fraction bits, bias, largest finite code
FP8_FORMATS = {"e4m3": (4, 3, 7, 0x7E), "e5m2": (5, 2, 15, 0x7B)}


def _fp8_positive_values(fmt: str) -> np.ndarray:
    """Values of the non-negative finite codes 0 .. largest, in code order."""
    eb, fb, bias, top = FP8_FORMATS[fmt]
    c = np.arange(top + 1)
    e, f = c >> fb, c & ((1 << fb) - 1)
    return np.where(e == 0, f / (1 << fb) * 2.0 ** (1 - bias),
                    (1 + f / (1 << fb)) * np.exp2(e - float(bias)))


def fp8_bits_from_f32(a: np.ndarray, fmt: str) -> np.ndarray:
    """Encode float32 values as fp8 codes (uint8): nearest value, ties to the
    even code, magnitudes past the largest finite value saturate to it."""
    vals = _fp8_positive_values(fmt)
    x = np.asarray(a, dtype=np.float64)
    mag = np.minimum(np.abs(x), vals[-1])
    hi = np.clip(np.searchsorted(vals, mag), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = mag - vals[lo], vals[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code[mag == 0] = 0
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def fp8_scale(a: np.ndarray, fmt: str) -> float:
    """Power-of-two per-tensor scale s with max |a| / s within the format."""
    amax = float(np.max(np.abs(a))) if np.size(a) else 0.0
    if amax == 0.0:
        return 1.0
    return float(2.0 ** np.ceil(np.log2(amax / _fp8_positive_values(fmt)[-1])))


def fp8_inputs(X: np.ndarray, dY: np.ndarray, x_fmt: str = "e4m3", dy_fmt: str = "e5m2"):
    """(X8, s_x, dY8, s_dy): per-tensor power-of-two scaling, then fp8 codes."""
    sx, sdy = fp8_scale(X, x_fmt), fp8_scale(dY, dy_fmt)
    return (fp8_bits_from_f32(np.asarray(X, np.float32) / np.float32(sx), x_fmt), sx,
            fp8_bits_from_f32(np.asarray(dY, np.float32) / np.float32(sdy), dy_fmt), sdy)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DenseCase:
    """One dense layer: X [T, d_in], dY [T, d_out], W/m/v [d_out, d_in]."""
    name: str
    T: int
    d_in: int
    d_out: int
    seed_base: int
    x_std: float = 1.0
    dy_std: float = 1.0
    w_std: float = 0.02
    steps: int = 3
    dy_kind: str = "normal"          # "normal" | "softmax_grad"
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    momentum: float = 0.9

    def input_seed(self, step: int) -> int:
        return self.seed_base + step

    @property
    def w_seed(self) -> int:
        return self.seed_base + 999

    @property
    def flops(self) -> int:
        return 2 * self.T * self.d_in * self.d_out


@dataclass(frozen=True)
class GroupedCase:
    """Routed experts: E experts, each W_e [d_out, d_in]; X [T, d_in] tokens,
    each routed to ``top_k`` distinct experts."""
    name: str
    E: int
    T: int
    top_k: int
    d_in: int
    d_out: int
    seed_base: int
    n_empty: int = 2                 # experts that receive no tokens
    zipf_s: float = 1.1
    x_std: float = 1.0
    dy_std: float = 1.0
    w_std: float = 0.02
    steps: int = 3
    warm_start: bool = False         # step 1 routes to all experts
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    extra: dict = field(default_factory=dict, compare=False)

    def input_seed(self, step: int) -> int:
        return self.seed_base + step

    @property
    def w_seed(self) -> int:
        return self.seed_base + 999

    @property
    def route_seed(self) -> int:
        return self.seed_base + 998


CONFIGS = {
    0: DenseCase("tiny_dense_512x256x256", T=512, d_in=256, d_out=256, seed_base=0, steps=3),
    1: DenseCase("llama3_8b_mlp_down_T8192", T=8192, d_in=14336, d_out=4096, seed_base=1000,
                 dy_std=1e-2, steps=10),
    2: DenseCase("llama3_8b_qkv_gqa_T16384", T=16384, d_in=4096, d_out=6144, seed_base=2000,
                 steps=3),
    3: DenseCase("lm_head_128256_T4096", T=4096, d_in=4096, d_out=128256, seed_base=3000,
                 dy_kind="softmax_grad", steps=5),
    4: GroupedCase("moe_8x14336x4096_T16384_top2", E=8, T=16384, top_k=2, d_in=4096,
                   d_out=14336, seed_base=4000, steps=3),
}


def dense_case(k: int) -> DenseCase:
    c = CONFIGS[k]
    assert isinstance(c, DenseCase)
    return c


def grouped_case(k: int = 4) -> GroupedCase:
    c = CONFIGS[k]
    assert isinstance(c, GroupedCase)
    return c


# --------------------------------------------------------------------------
# dense inputs
# --------------------------------------------------------------------------
LMHEAD_SUPPORT = 256
LMHEAD_ALPHA = 0.1
LMHEAD_FLOOR = 1e-30


def lmhead_dy(seed: int, T: int, V: int, support: int = LMHEAD_SUPPORT,
              alpha: float = LMHEAD_ALPHA) -> np.ndarray:
    """Softmax-gradient-like rows for an LM head, as bfloat16 bits [T, V].

    Row t: a label y_t ~ U[0, V); a probability vector p that is Dirichlet(alpha)
    on a random support of ``support`` distinct vocabulary ids and zero
    elsewhere (probabilities below 1e-30 are set to 0); dY[t, j] = p_j for
    j != y_t and dY[t, y_t] = p_{y_t} - 1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    support = min(support, V)
    labels = rng.integers(0, V, size=T)
    out = np.zeros((T, V), dtype=np.uint16)
    for t in range(T):
        ids = rng.choice(V, size=support, replace=False, shuffle=False)
        w = rng.gamma(alpha, size=support)
        tot = w.sum()
        p = w / tot if tot > 0 else np.full(support, 1.0 / support)
        p[p < LMHEAD_FLOOR] = 0.0
        hit = np.nonzero(ids == labels[t])[0]
        if hit.size:
            p[hit[0]] -= 1.0
        else:
            ids = np.append(ids, labels[t])
            p = np.append(p, -1.0)
        out[t, ids] = bf16_bits_from_f32(p.astype(np.float32))
    return out


def dense_inputs(case: DenseCase, step: int):
    """(X bits [T, d_in], dY bits [T, d_out]) for optimizer step ``step`` (>=1)."""
    seed = case.input_seed(step)
    X = normal_bf16(seed * 2, (case.T, case.d_in), case.x_std)
    if case.dy_kind == "softmax_grad":
        dY = lmhead_dy(seed * 2 + 1, case.T, case.d_out)
    else:
        dY = normal_bf16(seed * 2 + 1, (case.T, case.d_out), case.dy_std)
    return X, dY


def dense_inputs_f32(case: DenseCase, step: int):
    """The float32 draws behind dense_inputs (before the bf16 encoding)."""
    seed = case.input_seed(step)
    X = normal_f32(seed * 2, (case.T, case.d_in), case.x_std)
    dY = normal_f32(seed * 2 + 1, (case.T, case.d_out), case.dy_std)
    return X, dY


def dense_inputs_fp8(case: DenseCase, step: int, x_fmt: str = "e4m3", dy_fmt: str = "e5m2"):
    """(X8, s_x, dY8, s_dy) from the same float32 draws as dense_inputs."""
    return fp8_inputs(*dense_inputs_f32(case, step), x_fmt, dy_fmt)


def dense_state(case: DenseCase):
    """(W, m, v) float32 [d_out, d_in]; W ~ N(0, w_std^2), m = v = 0."""
    W = normal_f32(case.w_seed, (case.d_out, case.d_in), case.w_std)
    z = np.zeros_like(W)
    return W, z, z.copy()


# --------------------------------------------------------------------------
# routed (grouped) inputs
# --------------------------------------------------------------------------
def moe_loads(n_active: int, total: int, s: float = 1.1) -> np.ndarray:
    """Zipf(s) loads over ranks 1..n_active, scaled to ``total`` rows by the
    largest-remainder rule (ties go to the lower rank)."""
    w = np.arange(1, n_active + 1, dtype=np.float64) ** (-s)
    q = w / w.sum() * total
    base = np.floor(q).astype(np.int64)
    rem = total - int(base.sum())
    order = sorted(range(n_active), key=lambda r: (-(q[r] - base[r]), r))
    for r in order[:rem]:
        base[r] += 1
    return base


def moe_routing(case: GroupedCase, step: int = 1):
    """Routing table for one step.

    Returns (offsets [E+1] int64, rows [sum loads] int64): expert e owns
    routed rows offsets[e]..offsets[e+1]-1 and routed row j comes from token
    rows[j]. Each token is routed to ``top_k`` distinct experts.
    """
    E, T, k = case.E, case.T, case.top_k
    rng = np.random.Generator(np.random.PCG64(case.route_seed))
    expert_of_rank = rng.permutation(E)
    token_perm = rng.permutation(T)
    n_active = E if (case.warm_start and step == 1) else E - case.n_empty
    loads_rank = moe_loads(n_active, k * T, case.zipf_s)
    if loads_rank.max() > T:
        raise ValueError("an expert would receive a token twice")
    loads = np.zeros(E, dtype=np.int64)
    for r in range(n_active):
        loads[expert_of_rank[r]] = loads_rank[r]
    # expert-major slot list laid over the tokens: slot j -> token_perm[j mod T]
    slot_start = np.concatenate([[0], np.cumsum(loads_rank)])
    offsets = np.concatenate([[0], np.cumsum(loads)]).astype(np.int64)
    rows = np.empty(int(offsets[-1]), dtype=np.int64)
    for r in range(n_active):
        e = expert_of_rank[r]
        j = np.arange(slot_start[r], slot_start[r + 1])
        rows[offsets[e]:offsets[e + 1]] = token_perm[j % T]
    return offsets, rows


def grouped_inputs(case: GroupedCase, step: int):
    """(X_perm bits [R, d_in], dY_perm bits [R, d_out], offsets [E+1]) for a step.

    X [T, d_in] is drawn per token and gathered into expert-major order; dY is
    drawn per routed row.
    """
    offsets, rows = moe_routing(case, step)
    seed = case.input_seed(step)
    X = normal_bf16(seed * 2, (case.T, case.d_in), case.x_std)
    X_perm = np.ascontiguousarray(X[rows])
    dY_perm = normal_bf16(seed * 2 + 1, (int(offsets[-1]), case.d_out), case.dy_std)
    return X_perm, dY_perm, offsets


def grouped_state(case: GroupedCase):
    """(W, m, v) float32 [E, d_out, d_in]; W ~ N(0, w_std^2), m = v = 0."""
    W = normal_f32(case.w_seed, (case.E, case.d_out, case.d_in), case.w_std)
    z = np.zeros_like(W)
    return W, z, z.copy()
