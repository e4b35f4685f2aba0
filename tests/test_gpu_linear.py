"""fmlp_linear on the GPU against the fp64 oracle: random shapes spanning
several tiles and ragged tails on both the decode (M <= 16) and the tiled
GEMM path, and pins the tolerance cannot see: the GELU variant, bf16
round-to-nearest-even, and the bias."""
import numpy as np
import pytest
import torch

import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import (DEV, assert_parity, bf16_ulp, bits_of, f64_of, f64_of_bits, rand_bf16,
                      to_dev)

pytestmark = pytest.mark.gpu

SHAPES = [
    # (M, K, N)
    (1, 8, 8), (1, 4096, 64), (2, 40, 24), (5, 136, 264), (16, 520, 136), (16, 64, 8),
    (17, 64, 8), (33, 200, 72), (100, 64, 128), (128, 128, 128), (255, 520, 136),
    (300, 72, 264), (513, 1000, 392), (1024, 32, 64), (2048, 768, 3072),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("act", ["none", "gelu_erf", "gelu_tanh"])
def test_linear_random(M, K, N, act):
    rng = np.random.default_rng(M * 1000003 + K * 101 + N)
    x = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.5, "uniform")
    for bias in (None, b):
        print(f"case linear M={M} K={K} N={N} act={act} bias={bias is not None}", flush=True)
        y = F.fmlp_linear(to_dev(x), to_dev(W), None if bias is None else to_dev(bias), act)
        torch.cuda.synchronize()
        ref = oracle.linear(f64_of_bits(x), f64_of_bits(W), None if bias is None else f64_of_bits(bias), act)
        assert_parity(y, ref, f"linear {M}x{K}x{N} {act}")


@pytest.mark.parametrize("M,K,N", [
    (4100, 328, 4104),   # 256x256 tiles: 17 x 17 = 289 > 256 CUs, so some blocks run two
    (8200, 136, 1000),   # 128x128 tiles: 65 x 8 = 520 > 512 block slots
    (8000, 200, 768),    # 128x192 tiles: 63 x 4 = 252, one round; tails in M and K
])
@pytest.mark.parametrize("act", ["gelu_erf", "gelu_tanh"])
def test_linear_persistent_multi_tile_ragged(M, K, N, act):
    """More tiles than the persistent grid holds, with a tail in M, N and K:
    blocks carry the load stream and the epilogue across tile boundaries."""
    rng = np.random.default_rng(M + K + N)
    x = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.5, "uniform")
    print(f"case linear persistent M={M} K={K} N={N} act={act}", flush=True)
    y = F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), act)
    torch.cuda.synchronize()
    ref = oracle.linear(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), act)
    assert_parity(y, ref, f"linear {M}x{K}x{N} {act}")


@pytest.mark.parametrize("M,K,N", [
    (1, 256, 12328),     # one-stage tiles, three or four per block (ragged last tile)
    (16, 512, 12288),    # one-stage tiles, three per block, sixteen tokens
    (3, 1024, 8192),     # two-stage tiles, two per block
])
def test_decode_short_tiles_at_stream_end(M, K, N):
    """Tiles of one or two stages at the end of a block's stream, where steps
    have no barrier of their own: each tile's partial sums must not be
    overwritten by the next tile's before the control wave has reduced them."""
    rng = np.random.default_rng(M + K + N)
    x = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.5, "uniform")
    print(f"case linear decode short tiles M={M} K={K} N={N}", flush=True)
    with F.force_path("decode"):
        for _ in range(3):
            y = F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), "gelu_erf")
    torch.cuda.synchronize()
    ref = oracle.linear(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), "gelu_erf")
    assert_parity(y, ref, f"linear decode {M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 16, 40, 300])
def test_gelu_variant_pin(M):
    """Identity W, no bias, x in [-4, -2.5]: here the two GELU forms differ by
    7-59 bf16 ulps, so the kernel must match its own variant to 1 ulp."""
    K = N = 128
    vals = np.linspace(-4.0, -2.5, M * K).reshape(M, K).astype(np.float32)
    import datagen
    x = datagen.rne_bf16(vals)
    I = datagen.rne_bf16(np.eye(N, K, dtype=np.float32))
    xf = f64_of_bits(x)
    for act, other in (("gelu_erf", "gelu_tanh"), ("gelu_tanh", "gelu_erf")):
        print(f"case gelu pin M={M} act={act}", flush=True)
        y = f64_of(F.fmlp_linear(to_dev(x), to_dev(I), None, act))
        want = oracle.activation(xf, act)
        wrong = oracle.activation(xf, other)
        ulp = bf16_ulp(want)
        assert np.max(np.abs(y - want) / ulp) <= 1.0
        # the pin has teeth: the other variant is many ulps away somewhere
        assert np.max(np.abs(wrong - want) / ulp) > 5.0


@pytest.mark.parametrize("M", [1, 16, 64])
def test_rne_pin(M):
    """Identity W + a bias that lands exactly between two bf16 numbers: round
    to nearest even, bitwise (truncation or round-half-up would differ)."""
    import datagen
    K = N = 64
    # x = 1.0078125 (0x3F81) + 2^-8 -> tie between 0x3F81 and 0x3F82 -> 0x3F82
    # x = 1.0       (0x3F80) + 2^-8 -> tie between 0x3F80 and 0x3F81 -> 0x3F80
    # x = -1.0078125 + (-2^-8) -> 0xBF82 ; 1.0 + 2^-7 -> exact 0x3F81
    xs = np.array([1.0078125, 1.0, -1.0078125, 1.0], np.float32)
    bs = np.array([2 ** -8, 2 ** -8, -(2 ** -8), 2 ** -7], np.float32)
    want = [0x3F82, 0x3F80, 0xBF82, 0x3F81]
    x = np.zeros((M, K), np.float32)
    b = np.zeros(N, np.float32)
    for j in range(4):
        x[:, j] = xs[j]
        b[j] = bs[j]
    I = np.eye(N, K, dtype=np.float32)
    print(f"case rne pin M={M}", flush=True)
    y = bits_of(F.fmlp_linear(to_dev(datagen.rne_bf16(x)), to_dev(datagen.rne_bf16(I)),
                              to_dev(datagen.rne_bf16(b)), "none"))
    for j in range(4):
        assert np.all(y[:, j] == want[j]), (j, hex(int(y[0, j])))


@pytest.mark.parametrize("M", [1, 16, 200])
@pytest.mark.parametrize("act", ["none", "gelu_erf", "gelu_tanh"])
def test_bias_pin(M, act):
    """W = 0 -> y = bf16(act(b)) exactly (within the final rounding)."""
    import datagen
    rng = np.random.default_rng(M)
    K, N = 64, 136
    x = rand_bf16(rng, (M, K))
    W = np.zeros((N, K), np.uint16)
    b = rand_bf16(rng, (N,), 3.0, "uniform")
    print(f"case bias pin M={M} act={act}", flush=True)
    y = bits_of(F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), act))
    want = datagen.rne_bf16(oracle.activation(f64_of_bits(b), act).astype(np.float32))
    # fp32 epilogue vs fp64 oracle: allow one bf16 ulp
    diff = np.abs(f64_of_bits(y) - f64_of_bits(np.broadcast_to(want, (M, N))))
    assert np.all(diff <= bf16_ulp(f64_of_bits(want))[None, :])


def test_large_bias_tight():
    """Large biases at a tight bar (4 bf16 ulps of max|ref|): a dropped or
    misplaced bias cannot hide inside the loose parity tolerance."""
    rng = np.random.default_rng(3)
    for M in (8, 96):
        K, N = 256, 264
        x = rand_bf16(rng, (M, K))
        W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
        b = rand_bf16(rng, (N,), 8.0, "uniform")
        print(f"case large bias M={M}", flush=True)
        y = f64_of(F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), "gelu_erf"))
        ref = oracle.linear(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), "gelu_erf")
        assert np.max(np.abs(y - ref)) <= 4 * bf16_ulp(np.max(np.abs(ref)))


def test_determinism_bitwise():
    rng = np.random.default_rng(11)
    for M in (7, 333):
        x = to_dev(rand_bf16(rng, (M, 1024)))
        W = to_dev(rand_bf16(rng, (520, 1024), 1 / 32, "uniform"))
        print(f"case determinism M={M}", flush=True)
        a = bits_of(F.fmlp_linear(x, W, None, "gelu_tanh"))
        b = bits_of(F.fmlp_linear(x, W, None, "gelu_tanh"))
        assert np.array_equal(a, b)


def test_leading_dims_flattened():
    """[batch, seq, dim] inputs are flattened to batch*seq rows."""
    rng = np.random.default_rng(5)
    x = rand_bf16(rng, (4, 8, 64))
    W = rand_bf16(rng, (32, 64), 1 / 8, "uniform")
    y = F.fmlp_linear(to_dev(x), to_dev(W))
    assert tuple(y.shape) == (4, 8, 32)
    ref = oracle.linear(f64_of_bits(x).reshape(32, 64), f64_of_bits(W))
    assert_parity(y.reshape(32, 32), ref, "flattened")


def test_errors_raise():
    x = torch.zeros(4, 30, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(8, 30, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(F.FmlpError, match="K=30"):
        F.fmlp_linear(x, W)
