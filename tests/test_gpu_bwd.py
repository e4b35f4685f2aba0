"""The backward pass on the GPU against the fp64 oracle (oracle.linear_bwd,
oracle.glu_bwd): every gradient element by element at the parity bar, on
random shapes with ragged token counts (not multiples of 8 or of a tile),
several tiles, every activation, with and without a bias; the 768/3072 GeGLU
workload in full; the 8192/28672 GeGLU at 4096 tokens on sampled gradient
entries (dx rows; dWg, dWu rows and dWd columns of sampled hidden units);
zero tokens; determinism.

ReLU's derivative jumps at 0: where a pre-activation lies within the fp32
recomputation's error of 0 the two sides could take different branches.  The
Linear cases therefore zero dy wherever the oracle's |z| < 1e-3 (dz is then 0
whatever branch is taken); the ReLU-gated block gives every gate a constant
+-1 through a unit input feature, so that every |g| stays clear of 0
(checked)"""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bits_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu

ACTS = ["none", "gelu_erf", "gelu_tanh", "relu", "silu"]
KINK_MARGIN = 1e-3


def _clear_of_kink(z):
    return float(np.min(np.abs(z))) > KINK_MARGIN


def _linear_case(seed, M, K, N, act, bias):
    rng = np.random.default_rng(seed)
    x = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.3, "uniform") if bias else None
    dy = rand_bf16(rng, (M, N))
    if act == "relu":
        z = f64_of_bits(x) @ f64_of_bits(W).T + (0 if b is None else f64_of_bits(b))
        dy = np.where(np.abs(z) < KINK_MARGIN, np.uint16(0), dy).astype(np.uint16)
    return x, W, b, dy


@pytest.mark.parametrize("M,K,N", [(1, 64, 32), (5, 72, 40), (37, 256, 200), (129, 320, 264),
                                   (300, 520, 1048), (1000, 768, 1536)])
@pytest.mark.parametrize("act", ACTS)
def test_linear_bwd_random(M, K, N, act):
    bias = (M + K) % 2 == 1 or act == "gelu_erf"
    x, W, b, dy = _linear_case(M + K + N, M, K, N, act, bias)
    print(f"case linear_bwd M={M} K={K} N={N} act={act} bias={bias}", flush=True)
    dx, dW, db = F.fmlp_linear_bwd(to_dev(x), to_dev(W), None if b is None else to_dev(b), act, to_dev(dy))
    torch.cuda.synchronize()
    rx, rW, rb = oracle.linear_bwd(f64_of_bits(x), f64_of_bits(W), None if b is None else f64_of_bits(b), act,
                                   f64_of_bits(dy))
    assert_parity(dx, rx, f"dx {M}x{K}x{N} {act}")
    assert_parity(dW, rW, f"dW {M}x{K}x{N} {act}")
    if bias:
        assert_parity(db, rb, f"db {M}x{K}x{N} {act}")


def _glu_case(seed, M, D, H, act):
    for attempt in range(20):
        rng = np.random.default_rng(seed * 1000 + attempt)
        x = rand_bf16(rng, (M, D))
        Wg = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
        if act != "relu":
            break
        # gate h = +-1 * x[:, 0] + (the rest, |.| < 1 in practice): x[:, 0] = 1
        x[:, 0] = datagen.rne_bf16(np.ones(M, np.float32))
        Wg[:, 0] = datagen.rne_bf16(rng.choice([-1.0, 1.0], size=H).astype(np.float32))
        Wg[:, 1:] = rand_bf16(rng, (H, D - 1), 0.2 * D ** -0.5, "uniform")   # the rest: std ~0.12
        if _clear_of_kink(f64_of_bits(x) @ f64_of_bits(Wg).T):
            break
    else:
        pytest.fail("no ReLU input clear of the kink")
    Wu = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wd = rand_bf16(rng, (D, H), H ** -0.5, "uniform")
    dy = rand_bf16(rng, (M, D))
    return x, Wg, Wu, Wd, dy


@pytest.mark.parametrize("M,D,H", [(1, 64, 64), (7, 96, 200), (40, 256, 520), (257, 320, 1024),
                                   (600, 512, 1536)])
@pytest.mark.parametrize("act", ACTS)
def test_glu_bwd_random(M, D, H, act):
    x, Wg, Wu, Wd, dy = _glu_case(M + D + H, M, D, H, act)
    print(f"case glu_bwd M={M} D={D} H={H} act={act}", flush=True)
    got = F.fmlp_glu_bwd(*(to_dev(a) for a in (x, Wg, Wu, Wd)), act, to_dev(dy))
    torch.cuda.synchronize()
    ref = oracle.glu_bwd(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)), act, f64_of_bits(dy))
    for g, r, n in zip(got, ref, ("dx", "dWg", "dWu", "dWd")):
        assert_parity(g, r, f"{n} {M}x{D}x{H} {act}")


def test_glu_bwd_geglu768_full():
    """The 8192-token 768/3072 GeGLU workload's backward, every gradient in full
    (its weight gradients run split over the tokens in 7 parts of 18 or 19
    stages)."""
    w = datagen.workload("geglu768")
    t = datagen.make_inputs(w, seed=0)
    dy = datagen.normal_bf16(datagen.rng_for(0, w.family, "dy"), (w.M, w.N))
    print(f"case {w.name} backward, full", flush=True)
    got = F.fmlp_glu_bwd(*(to_dev(t[k]) for k in ("x", "Wg", "Wu", "Wd")), "gelu_tanh", to_dev(dy))
    torch.cuda.synchronize()
    ref = oracle.glu_bwd(*(f64_of_bits(t[k]) for k in ("x", "Wg", "Wu", "Wd")), "gelu_tanh", f64_of_bits(dy))
    for g, r, n in zip(got, ref, ("dx", "dWg", "dWu", "dWd")):
        assert_parity(g, r, f"{w.name} {n}")


def bwd_sample(T, H, tile=256):
    """Token rows: one per 16-row fragment group of every 256-row m-tile (as in
    the forward's sample); hidden units: the first and last of every 128-wide
    output tile of the gate+up GEMM plus every 64th unit."""
    groups = np.arange(T // 16)
    rows = np.unique(np.concatenate([[0, T - 1], groups * 16 + (groups * 5) % 16]))
    hid = np.unique(np.concatenate([np.arange(0, H, 128), np.arange(127, H, 128), np.arange(0, H, 64)]))
    return rows, hid


@pytest.mark.slow
def test_glu_bwd_large_sampled():
    """The 8192/28672 GeGLU at 4096 tokens: dx on 257 token rows over all 8192
    columns; dWg and dWu rows and dWd columns of 672 hidden units (all 8192
    entries each), every one a sum over all 4096 tokens."""
    w = datagen.workload("large4096")
    t = datagen.make_inputs(w, seed=0)
    dy = datagen.normal_bf16(datagen.rng_for(0, w.family, "dy4096"), (w.M, w.N))
    print(f"case {w.name} backward (sampled gradient entries)", flush=True)
    dev = [to_dev(t[k]) for k in ("x", "Wg", "Wu", "Wd")]
    ws = torch.empty(F.lib().fmlp_glu_bwd_workspace_size(w.M, w.K, w.H), dtype=torch.uint8, device=DEV)
    dx, dWg, dWu, dWd = F.fmlp_glu_bwd(*dev, "gelu_tanh", to_dev(dy), workspace=ws)
    torch.cuda.synchronize()
    del ws
    rows, hid = bwd_sample(w.M, w.H)
    ref = oracle.glu_bwd_sampled(*(f64_of_bits(t[k]) for k in ("x", "Wg", "Wu", "Wd")), "gelu_tanh",
                                 f64_of_bits(dy), rows, hid)
    r_t, h_t = torch.from_numpy(rows).to(DEV), torch.from_numpy(hid).to(DEV)
    assert_parity(dx[r_t], ref[0], f"{w.name} dx rows")
    assert_parity(dWg[h_t], ref[1], f"{w.name} dWg rows")
    assert_parity(dWu[h_t], ref[2], f"{w.name} dWu rows")
    assert_parity(dWd[:, h_t], ref[3], f"{w.name} dWd columns")
    for g in (dx, dWg, dWu, dWd):
        assert torch.isfinite(g.float()).all()


def test_glu_bwd_kmajor_ragged_sampled():
    """A shape whose backward GEMMs all read their row-contracted operands
    k-major (256x256 tiles fill the chip): dm over Wd's rows, dx over [Wg; Wu]
    with the weights switching at row H, and the three weight gradients over
    the tokens (split in 3 parts).  Ragged everywhere: 8200 tokens (a partial
    last 64-row stage), and widths that are not multiples of a tile.  Sampled
    as the large workload's backward: token rows of dx over all columns, whole
    rows of dWg, dWu and whole columns of dWd."""
    M, D, H = 8200, 2056, 2112
    x, Wg, Wu, Wd, dy = _glu_case(29, M, D, H, "gelu_tanh")
    print(f"case glu_bwd k-major M={M} D={D} H={H}", flush=True)
    dx, dWg, dWu, dWd = F.fmlp_glu_bwd(*(to_dev(a) for a in (x, Wg, Wu, Wd)), "gelu_tanh", to_dev(dy))
    torch.cuda.synchronize()
    rows, hid = bwd_sample(M, H)
    ref = oracle.glu_bwd_sampled(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)), "gelu_tanh", f64_of_bits(dy), rows, hid)
    r_t, h_t = torch.from_numpy(rows).to(DEV), torch.from_numpy(hid).to(DEV)
    assert_parity(dx[r_t], ref[0], "k-major dx rows")
    assert_parity(dWg[h_t], ref[1], "k-major dWg rows")
    assert_parity(dWu[h_t], ref[2], "k-major dWu rows")
    assert_parity(dWd[:, h_t], ref[3], "k-major dWd columns")


@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_bwd_kmajor_ragged(with_bias):
    """The linear backward with dx over W's rows read k-major (256x256 tiles
    fill the chip) and dW over the tokens read k-major (dz and x as they lie);
    ragged token count and widths.  Without a bias, dz is not transposed at all."""
    M, K, N = 8200, 2056, 520
    rng = np.random.default_rng(31 + with_bias)
    x, W = rand_bf16(rng, (M, K)), rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.3, "uniform") if with_bias else None
    dy = rand_bf16(rng, (M, N))
    print(f"case linear_bwd k-major M={M} K={K} N={N} bias={with_bias}", flush=True)
    dx, dW, db = F.fmlp_linear_bwd(to_dev(x), to_dev(W), to_dev(b) if with_bias else None, "gelu_tanh", to_dev(dy))
    torch.cuda.synchronize()
    rdx, rdW, rdb = oracle.linear_bwd(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b) if with_bias else None,
                                      "gelu_tanh", f64_of_bits(dy))
    assert_parity(dx, rdx, "k-major linear dx")
    assert_parity(dW, rdW, "k-major linear dW")
    if with_bias:
        assert_parity(db, rdb, "k-major linear db")


def test_bwd_zero_tokens_gives_zero_weight_gradients():
    K, N = 64, 48
    W = to_dev(rand_bf16(np.random.default_rng(0), (N, K), 0.1, "uniform"))
    b = torch.ones(N, dtype=torch.bfloat16, device=DEV)
    x = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    dy = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    dW = torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV)
    db = torch.full((N,), 7.0, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    print("case bwd zero tokens", flush=True)
    F.fmlp_linear_bwd(x, W, b, "gelu_erf", dy, out=(dx, dW, db))
    dWg = torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV)
    dWu = torch.full((N, K), 7.0, dtype=torch.bfloat16, device=DEV)
    dWd = torch.full((K, N), 7.0, dtype=torch.bfloat16, device=DEV)
    F.fmlp_glu_bwd(x, W, W, W.t().contiguous(), "silu", x, out=(dx, dWg, dWu, dWd))
    torch.cuda.synchronize()
    for g in (dW, db, dWg, dWu, dWd):
        assert not torch.any(g != 0)


def test_bwd_determinism():
    x, Wg, Wu, Wd, dy = _glu_case(5, 333, 256, 768, "gelu_tanh")
    d = [to_dev(a) for a in (x, Wg, Wu, Wd)]
    print("case bwd determinism", flush=True)
    a = [bits_of(g) for g in F.fmlp_glu_bwd(*d, "gelu_tanh", to_dev(dy))]
    b = [bits_of(g) for g in F.fmlp_glu_bwd(*d, "gelu_tanh", to_dev(dy))]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _wgrad_split(R, T, C):
    """The token split the library takes for a weight gradient (R x C over T
    padded tokens): mirrors its documented rule, to know which cases run split."""
    tiles = (-(-R // 256)) * (-(-C // 256))
    if tiles >= 256:
        return 1
    return max(1, min(256 // tiles, 8, (-(-T // 64)) // 8))


@pytest.mark.parametrize("M,K,N,act,parts", [(8190, 264, 520, "gelu_tanh", 8), (2043, 1024, 1032, "silu", 4),
                                             (5000, 712, 600, "relu", 8), (1000, 264, 2056, "gelu_erf", 2)])
def test_linear_bwd_token_split(M, K, N, act, parts):
    """Weight gradients split over the tokens (fp32 parts summed in part
    order): 4 and 8 parts, parts of unequal length (79 stages of 64 tokens in
    8 parts, with a token tail), ragged token counts, and bitwise equal on a
    second call."""
    assert _wgrad_split(N, -(-M // 8) * 8, K) == parts
    x, W, b, dy = _linear_case(M * 3 + K, M, K, N, act, True)
    print(f"case linear_bwd token split M={M} K={K} N={N} act={act} parts={parts}", flush=True)
    d = [to_dev(a) for a in (x, W, b, dy)]
    dx, dW, db = F.fmlp_linear_bwd(d[0], d[1], d[2], act, d[3])
    dW2 = F.fmlp_linear_bwd(d[0], d[1], d[2], act, d[3])[1]
    torch.cuda.synchronize()
    rx, rW, rb = oracle.linear_bwd(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), act, f64_of_bits(dy))
    assert_parity(dx, rx, f"dx {M}x{K}x{N} {act}")
    assert_parity(dW, rW, f"dW {M}x{K}x{N} {act} ({parts} parts)")
    assert_parity(db, rb, f"db {M}x{K}x{N} {act}")
    assert np.array_equal(bits_of(dW), bits_of(dW2))


def test_glu_bwd_token_split():
    M, D, H = 4096, 256, 640
    assert _wgrad_split(H, M, D) == 8 and _wgrad_split(D, M, H) == 8
    x, Wg, Wu, Wd, dy = _glu_case(17, M, D, H, "gelu_tanh")
    print(f"case glu_bwd token split M={M} D={D} H={H}", flush=True)
    got = F.fmlp_glu_bwd(*(to_dev(a) for a in (x, Wg, Wu, Wd)), "gelu_tanh", to_dev(dy))
    torch.cuda.synchronize()
    ref = oracle.glu_bwd(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)), "gelu_tanh", f64_of_bits(dy))
    for g, r, n in zip(got, ref, ("dx", "dWg", "dWu", "dWd")):
        assert_parity(g, r, f"{n} {M}x{D}x{H} (8 parts)")
