"""Seeded input generator: bf16 rounding, determinism, distributions, routes (CPU)."""
import numpy as np
import pytest
import torch

import datagen as dg


def test_rne_tie_cases_on_raw_bits():
    # 1.00390625 (0x3F808000) is a tie between 0x3F80 and 0x3F81 -> even 0x3F80
    # 0x3F818000 is a tie between 0x3F81 and 0x3F82 -> even 0x3F82
    bits = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0xBF808000, 0xBF818000,
                     0x00000000, 0x80000000, 0x7F7F8000], dtype=np.uint32)
    out = dg.rne_bf16(bits.view(np.float32))
    assert out.tolist() == [0x3F80, 0x3F82, 0x3F80, 0x3F81, 0xBF80, 0xBF82, 0x0000, 0x8000, 0x7F80]


def test_rne_matches_torch_library_rounding():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(20_000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(20_000) * 1e30).astype(np.float32),
        rng.integers(0, 2**32, 50_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    a = a[np.isfinite(a)]
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dg.rne_bf16(a), ref)


def test_bf16_decode_roundtrip_exact():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = dg.bf16_to_f32(bits)
    fin = np.isfinite(f)
    assert np.array_equal(dg.rne_bf16(f[fin]), bits[fin])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[fin], ref[fin])


def test_determinism_and_independence():
    w = dg.workload("decode1")
    a = dg.make_inputs(w, seed=0)
    b = dg.make_inputs(w, seed=0)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = dg.make_inputs(w, seed=1)
    assert not np.array_equal(a["W1"], c["W1"])
    # weights do not depend on the token count; x does
    d = dg.make_inputs(dg.workload("decode16"), seed=0)
    for k in ("W1", "W2", "b1", "b2"):
        assert np.array_equal(a[k], d[k]), k
    assert a["x"].shape == (1, 4096) and d["x"].shape == (16, 4096)
    assert not np.array_equal(a["W1"], a["W2"])


def test_distributions():
    w = dg.workload("geglu768")
    t = dg.make_inputs(w, seed=0)
    x = dg.bf16_to_f32(t["x"]).astype(np.float64)
    assert t["x"].shape == (8192, 768) and t["Wg"].shape == (3072, 768) and t["Wd"].shape == (768, 3072)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    for k, bound in (("Wg", w.w1_bound), ("Wu", w.w1_bound), ("Wd", w.w2_bound)):
        v = dg.bf16_to_f32(t[k]).astype(np.float64)
        assert np.abs(v).max() <= bound * (1 + 2 ** -8)
        assert abs(v.std() - bound / np.sqrt(3)) < 0.01 * bound
    tiny = dg.make_inputs(dg.workload("tiny"), seed=0)
    assert set(tiny) == {"x", "W1", "b1", "W2", "b2"}
    assert tiny["W1"].shape == (64, 32) and tiny["W2"].shape == (32, 64)
    assert np.abs(dg.bf16_to_f32(tiny["b2"])).max() <= 0.125 * (1 + 2 ** -8)


def test_routes():
    ids, gw = dg.make_routes(4096, 8, 2, seed=0)
    assert ids.dtype == np.int32 and gw.dtype == np.float32 and ids.shape == gw.shape == (4096, 2)
    assert ids.min() >= 0 and ids.max() < 8
    assert np.all(ids[:, 0] != ids[:, 1])                       # distinct experts per token
    assert np.allclose(gw.sum(1), 1.0, atol=1e-6) and gw.min() > 0
    counts = np.bincount(ids.ravel(), minlength=8)
    assert counts.sum() == 8192 and np.all(np.abs(counts - 1024) < 6 * 27.7)
    i2, g2 = dg.make_routes(4096, 8, 2, seed=0)
    assert np.array_equal(ids, i2) and np.array_equal(gw, g2)
    with pytest.raises(ValueError):
        dg.make_routes(4, 2, 3)
