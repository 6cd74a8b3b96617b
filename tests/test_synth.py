"""The seeded generators: determinism, encodings, and the workload recipes."""
import numpy as np
import torch

import synth
from synth import gen


def test_same_seed_same_bytes_and_chunk_independence():
    a = synth.normal_f32(7, (3, gen.CHUNK // 2 + 5))
    b = synth.normal_f32(7, (3, gen.CHUNK // 2 + 5))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = synth.normal_f32(8, a.shape)
    assert not np.array_equal(a, c)
    # the first chunk does not depend on the total size
    d = synth.normal_f32(7, (1000,))
    assert np.array_equal(a.reshape(-1)[:1000].view(np.uint32), d.view(np.uint32))


def test_bf16_encoding_matches_torch_rne():
    x = synth.normal_f32(9, (100000,))
    x[:1000] *= np.float32(1e-3)
    x[1000:2000] *= np.float32(1e30)
    got = synth.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # subnormal results are flushed to signed zero
    tiny = np.array([1e-39, -1e-39, 3e-41], dtype=np.float32)
    assert list(synth.bf16_bits_from_f32(tiny)) == [0, 0x8000, 0]


def test_dense_config_shapes_and_scales():
    c0 = synth.dense_case(0)
    X, dY = synth.dense_inputs(c0, 1)
    assert X.shape == (512, 256) and dY.shape == (512, 256) and X.dtype == np.uint16
    W, m, v = synth.dense_state(c0)
    assert W.shape == (256, 256) and W.dtype == np.float32
    assert abs(float(W.std()) - 0.02) < 1e-3 and not m.any() and not v.any()
    X2, _ = synth.dense_inputs(c0, 2)
    assert not np.array_equal(X, X2)
    c1 = synth.dense_case(1)
    assert (c1.T, c1.d_in, c1.d_out, c1.dy_std, c1.steps) == (8192, 14336, 4096, 1e-2, 10)


def test_moe_loads_and_routing():
    case = synth.grouped_case(4)
    loads = synth.moe_loads(6, 2 * case.T, case.zipf_s)
    assert list(loads) == [14294, 6668, 4269, 3111, 2434, 1992]
    offsets, rows = synth.moe_routing(case, 1)
    counts = np.diff(offsets)
    assert offsets[0] == 0 and offsets[-1] == 2 * case.T
    assert sorted(counts.tolist(), reverse=True) == [14294, 6668, 4269, 3111, 2434, 1992, 0, 0]
    # every token goes to exactly top_k distinct experts
    per_token = np.zeros(case.T, dtype=np.int64)
    for e in range(case.E):
        toks = rows[offsets[e]:offsets[e + 1]]
        assert len(np.unique(toks)) == len(toks)
        per_token[toks] += 1
    assert np.all(per_token == 2)
    warm = gen.GroupedCase(**{**case.__dict__, "warm_start": True})
    o1, _ = synth.moe_routing(warm, 1)
    o2, _ = synth.moe_routing(warm, 2)
    assert np.all(np.diff(o1) > 0) and np.count_nonzero(np.diff(o2) == 0) == 2


def test_lmhead_rows_are_softmax_gradients():
    dY = synth.lmhead_dy(5, 16, 4096, support=64)
    vals = (dY.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.count_nonzero(vals < 0, axis=1) == 1)
    assert np.all(vals.min(axis=1) <= -0.0) and np.all(vals.min(axis=1) >= -1.0)
    assert np.all(np.abs(vals.sum(axis=1)) < 2e-2)       # p sums to 1, minus the label
    assert np.all(np.count_nonzero(vals, axis=1) <= 65)
