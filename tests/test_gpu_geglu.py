"""fmlp_geglu on the GPU against the fp64 oracle: the 8192-token 768/3072
workload in full, the 8192/28672 FFN at 1 and 16 tokens in full and at 4096
tokens on sampled rows, random ragged shapes on both paths, and special cases."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bf16_ulp, bits_of, f64_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _run(x, Wg, Wu, Wd, path="auto", ws=None):
    with F.force_path(path):
        y = F.fmlp_geglu(x, Wg, Wu, Wd, workspace=ws)
    torch.cuda.synchronize()
    return y


SHAPES = [
    # (M, D, H)
    (1, 8, 8), (1, 64, 64), (2, 136, 264), (7, 512, 1000), (16, 256, 512), (16, 1024, 2048),
    (17, 64, 128), (33, 96, 200), (64, 128, 64), (129, 256, 384), (300, 520, 1048), (777, 768, 3072),
]


@pytest.mark.parametrize("M,D,H", SHAPES)
def test_geglu_random(M, D, H):
    rng = np.random.default_rng(M * 131 + D * 7 + H)
    x = rand_bf16(rng, (M, D))
    Wg = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wu = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wd = rand_bf16(rng, (D, H), H ** -0.5, "uniform")
    ref = oracle.geglu(f64_of_bits(x), f64_of_bits(Wg), f64_of_bits(Wu), f64_of_bits(Wd))
    d = [to_dev(a) for a in (x, Wg, Wu, Wd)]
    for p in (["auto", "gemm", "decode"] if M <= 16 else ["auto"]):
        print(f"case geglu M={M} D={D} H={H} path={p}", flush=True)
        assert_parity(_run(*d, path=p), ref, f"geglu {M}x{D}x{H} {p}")


def test_geglu_persistent_multi_tile_ragged():
    """Gate+up on 256x256 tiles, 9 x 33 = 297 of them (more than 256 CUs),
    with tails in tokens (2100 = 8*256 + 52), hidden (4104) and dim (264)."""
    rng = np.random.default_rng(2100)
    M, D, H = 2100, 264, 4104
    x = rand_bf16(rng, (M, D))
    Wg = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wu = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wd = rand_bf16(rng, (D, H), H ** -0.5, "uniform")
    print(f"case geglu persistent M={M} D={D} H={H}", flush=True)
    y = _run(*(to_dev(a) for a in (x, Wg, Wu, Wd)))
    ref = oracle.geglu(f64_of_bits(x), f64_of_bits(Wg), f64_of_bits(Wu), f64_of_bits(Wd))
    assert_parity(y, ref, f"geglu {M}x{D}x{H}")


def test_geglu768_full():
    w = datagen.workload("geglu768")
    t = datagen.make_inputs(w, seed=0)
    print(f"case {w.name} full", flush=True)
    y = _run(*(to_dev(t[k]) for k in ("x", "Wg", "Wu", "Wd")))
    ref = oracle.geglu(*(f64_of_bits(t[k]) for k in ("x", "Wg", "Wu", "Wd")))
    assert_parity(y, ref, w.name)


class _LargeWeights(dict):
    """The 8192/28672 weights as bits, on the device, and (once) in fp64."""

    def f64(self):
        if "_f64" not in self:
            self["_f64"] = tuple(f64_of_bits(self["bits"][k]) for k in ("Wg", "Wu", "Wd"))
        return self["_f64"]


@pytest.fixture(scope="module")
def large_weights():
    w = datagen.workload("large1")
    t = datagen.make_inputs(w, seed=0)
    lw = _LargeWeights(bits=t)
    return t, {k: to_dev(t[k]) for k in ("Wg", "Wu", "Wd")}, lw


@pytest.mark.slow
@pytest.mark.parametrize("T", [1, 16])
def test_large_decode_full(large_weights, T):
    t, dw, lw = large_weights
    w = datagen.workload(f"large{T}")
    x = datagen.make_inputs(w, seed=0, with_weights=False)["x"]
    ws = F.workspace_for(DEV, F.fmlp_geglu_workspace_size(T, w.K, w.H))
    print(f"case {w.name} full", flush=True)
    y = _run(to_dev(x), dw["Wg"], dw["Wu"], dw["Wd"], ws=ws)
    ref = oracle.geglu(f64_of_bits(x), *lw.f64())
    assert_parity(y, ref, w.name)
    assert F.barrier_timeouts(ws) == 0


def prefill_sample_rows(T: int, tile: int = 256, frag: int = 16) -> np.ndarray:
    """One row from every 16-row fragment group of every 256-row tile of T
    rows, its offset inside the group cycling through all 16 positions (so
    every fragment row of the MFMA layout and every m-tile is compared), plus
    the first and last rows."""
    groups = np.arange((T + frag - 1) // frag)
    rows = groups * frag + (groups * 5 + (groups // (tile // frag))) % frag
    rows = np.concatenate([[0, T - 1], rows[rows < T]])
    return np.unique(rows)


@pytest.mark.slow
def test_large_prefill_sampled_rows(large_weights):
    """T = 4096 through the tiled path, compared on 256 rows (one in every
    16-row fragment group of every 256-row m-tile) over all 8192 columns;
    rows are independent, so the oracle on a row sample is the oracle of those
    rows.  The rest of y must be finite."""
    t, dw, lw = large_weights
    w = datagen.workload("large4096")
    x = datagen.make_inputs(w, seed=0, with_weights=False)["x"]
    print(f"case {w.name} (sampled rows)", flush=True)
    y = _run(to_dev(x), dw["Wg"], dw["Wu"], dw["Wd"])
    rows = prefill_sample_rows(w.M)
    assert len(rows) >= 256
    assert len(np.unique(rows // 256)) == w.M // 256 and len(np.unique(rows % 16)) == 16
    ref = oracle.geglu(f64_of_bits(x[rows]), *lw.f64())
    assert_parity(y[torch.from_numpy(rows).to(DEV)], ref, f"{w.name} {len(rows)} rows")
    assert np.isfinite(f64_of(y)).all()


@pytest.mark.parametrize("M,path", [(4, "decode"), (16, "gemm"), (200, "gemm")])
def test_geglu_special_cases(M, path):
    rng = np.random.default_rng(M)
    D = H = 64
    x = rand_bf16(rng, (M, D))
    I = datagen.rne_bf16(np.eye(H, D, dtype=np.float32))
    Z = np.zeros((H, D), np.uint16)
    W = rand_bf16(rng, (H, D), 0.125, "uniform")
    Wd = rand_bf16(rng, (D, H), 0.125, "uniform")
    print(f"case geglu special M={M} path={path}", flush=True)
    # Wg = Wu = Wd = I -> y = bf16(bf16(gelu_tanh(x) * x))
    y = f64_of(_run(to_dev(x), to_dev(I), to_dev(I), to_dev(I), path))
    xf = f64_of_bits(x)
    want = oracle.gelu_tanh(xf) * xf
    assert np.all(np.abs(y - want) <= 2 * bf16_ulp(want) + 1e-30)
    # Wu = 0 -> y = 0; Wd = 0 -> y = 0
    assert not np.any(f64_of(_run(to_dev(x), to_dev(W), to_dev(Z), to_dev(Wd), path)))
    assert not np.any(f64_of(_run(to_dev(x), to_dev(W), to_dev(W), to_dev(np.zeros((D, H), np.uint16)), path)))
    # gate and up are not interchangeable
    Wu = rand_bf16(rng, (H, D), 0.125, "uniform")
    a = f64_of(_run(to_dev(x), to_dev(W), to_dev(Wu), to_dev(Wd), path))
    b = f64_of(_run(to_dev(x), to_dev(Wu), to_dev(W), to_dev(Wd), path))
    assert np.max(np.abs(a - b)) > 1e-3
    ref = oracle.geglu(xf, f64_of_bits(W), f64_of_bits(Wu), f64_of_bits(Wd))
    assert np.max(np.abs(a - ref)) <= 1e-2 * np.max(np.abs(ref)) + 1e-3


def test_geglu_determinism():
    rng = np.random.default_rng(9)
    for M in (3, 500):
        d = [to_dev(rand_bf16(rng, s, 0.05, "uniform")) for s in ((M, 1024), (2048, 1024), (2048, 1024), (1024, 2048))]
        print(f"case geglu determinism M={M}", flush=True)
        a = bits_of(_run(*d))
        b = bits_of(_run(*d))
        assert np.array_equal(a, b)
