"""FP8 (E4M3) weights on the decode path, on the GPU against the fp64 oracle:
one layer, the two-layer MLP and the gated block at 1..16 tokens, ragged
inner sizes (multiples of 16 that are not multiples of 64), several row
tiles and a partial last tile, every activation, and the special codes
(subnormals, signed zeros, the largest finite value).  At one token with a
hidden size up to 4096 the two layers run in one launch (h exchanged as
epoch-tagged words); that form is checked bitwise against the two-launch
form and across back-to-back calls."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, f64_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _codes(rng, rows, cols, bound):
    q, s = datagen.e4m3_weights(rng, rows, cols, bound)
    return q, s, torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)


@pytest.mark.parametrize("M,K,N", [(1, 16, 16), (1, 4096, 4096), (16, 4096, 4096), (3, 1040, 200),
                                   (7, 528, 24), (16, 8192, 48), (2, 28672, 32),
                                   # activations too wide to stage, several tokens, a partial last tile
                                   (16, 8192, 8200), (9, 8208, 8216)])
@pytest.mark.parametrize("act", ["none", "gelu_erf", "silu"])
def test_linear_w8(M, K, N, act):
    rng = np.random.default_rng(M * 131 + K + N)
    x = rand_bf16(rng, (M, K))
    q, s, qd, sd = _codes(rng, N, K, K ** -0.5)
    b = rand_bf16(rng, (N,), 0.5, "uniform")
    for bias in (None, b):
        print(f"case linear_w8 M={M} K={K} N={N} act={act} bias={bias is not None}", flush=True)
        y = F.fmlp_linear_w8(to_dev(x), qd, sd, None if bias is None else to_dev(bias), act)
        torch.cuda.synchronize()
        ref = oracle.linear_w8(f64_of_bits(x), q, s, None if bias is None else f64_of_bits(bias), act)
        assert_parity(y, ref, f"linear_w8 {M}x{K}x{N} {act}")


@pytest.mark.parametrize("M,K,H,N", [(1, 4096, 4096, 4096), (16, 4096, 4096, 4096), (5, 1040, 336, 272),
                                     (1, 1040, 336, 272), (1, 8192, 16, 4096), (1, 16, 4096, 16)])
def test_mlp2_w8(M, K, H, N):
    rng = np.random.default_rng(M + K + H + N)
    x = rand_bf16(rng, (M, K))
    q1, s1, q1d, s1d = _codes(rng, H, K, 1 / 64)
    q2, s2, q2d, s2d = _codes(rng, N, H, 1 / 64)
    b1 = rand_bf16(rng, (H,), 1 / 64, "uniform")
    b2 = rand_bf16(rng, (N,), 1 / 64, "uniform")
    print(f"case mlp2_w8 M={M} K={K} H={H} N={N}", flush=True)
    y = F.fmlp_mlp2_w8(to_dev(x), q1d, s1d, to_dev(b1), q2d, s2d, to_dev(b2), "gelu_erf")
    torch.cuda.synchronize()
    ref = oracle.mlp2_w8(f64_of_bits(x), q1, s1, f64_of_bits(b1), q2, s2, f64_of_bits(b2), "gelu_erf")
    assert_parity(y, ref, f"mlp2_w8 {M}x{K}x{H}x{N}")


# the full-size shapes once, with the GeGLU gate; the others with both gates
_GLU_W8_CASES = [(M, 8192, 28672, "gelu_tanh") for M in (1, 16)] + [
    (M, D, H, act) for (M, D, H) in [(4, 1040, 2064), (16, 768, 3072), (16, 4096, 1040), (9, 4096, 2048),
                                     (1, 768, 3072), (1, 4096, 1040)] for act in ("gelu_tanh", "silu")]


@pytest.mark.parametrize("M,D,H,gate_act", _GLU_W8_CASES)
def test_glu_w8(M, D, H, gate_act):
    rng = np.random.default_rng(M * 3 + D + H)
    x = rand_bf16(rng, (M, D))
    qg, sg, qgd, sgd = _codes(rng, H, D, D ** -0.5)
    qu, su, qud, sud = _codes(rng, H, D, D ** -0.5)
    qdn, sdn, qdd, sdd = _codes(rng, D, H, H ** -0.5)
    print(f"case glu_w8 M={M} D={D} H={H} {gate_act}", flush=True)
    y = F.fmlp_glu_w8(to_dev(x), qgd, sgd, qud, sud, qdd, sdd, gate_act)
    torch.cuda.synchronize()
    if H * D > 2 ** 26:
        # full size: the oracle on a sample of output columns (every token)
        cols = np.sort(rng.choice(D, size=48, replace=False))
        Wg, Wu = oracle.dequant_w8(qg, sg), oracle.dequant_w8(qu, su)
        xf = f64_of_bits(x)
        m = oracle.activation(xf @ Wg.T, gate_act) * (xf @ Wu.T)
        ref = m @ oracle.dequant_w8(qdn[cols], sdn[cols]).T
        assert_parity(y[:, cols], ref, f"glu_w8 {M}x{D}x{H} sampled")
    else:
        ref = oracle.glu_w8(f64_of_bits(x), qg, sg, qu, su, qdn, sdn, gate_act)
        assert_parity(y, ref, f"glu_w8 {M}x{D}x{H} {gate_act}")


def test_w8_special_codes():
    """Every finite code in every column position, subnormals and signed zeros
    included: identity-like x picks single weights, so y[m, n] = s[n] * e4m3(q[n, m])
    exactly (one product, no sum).  A zero code of either sign gives a zero
    (the fp32 sum starts at +0, so the sign of a zero product is not kept)."""
    K = N = 256
    M = 16
    q = (np.arange(N * K, dtype=np.int64).reshape(N, K) * 7 % 256).astype(np.uint8)
    q = np.where((q & 0x7F) == 0x7F, q ^ 1, q).astype(np.uint8)
    s = np.ones(N, dtype=np.float32)
    x = np.zeros((M, K), dtype=np.uint16)
    for m in range(M):
        x[m, 17 * m] = 0x3F80   # 1.0 at k = 17 m
    print("case w8 special codes", flush=True)
    y = f64_of(F.fmlp_linear_w8(to_dev(x), torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)))
    want = oracle.e4m3_decode(q[:, 17 * np.arange(M)]).T      # [M, N]
    assert np.array_equal(y, want)


def test_w8_float8_dtype_and_errors():
    rng = np.random.default_rng(5)
    x = rand_bf16(rng, (2, 64))
    q, s, qd, sd = _codes(rng, 32, 64, 0.125)
    y0 = F.fmlp_linear_w8(to_dev(x), qd, sd)
    y1 = F.fmlp_linear_w8(to_dev(x), qd.view(torch.float8_e4m3fn), sd)
    assert torch.equal(y0, y1)
    with pytest.raises(F.FmlpError, match="M <= 16"):
        F.fmlp_linear_w8(to_dev(rand_bf16(rng, (17, 64))), qd, sd)
    with pytest.raises(F.FmlpError, match="multiple of 16"):
        F.fmlp_linear_w8(to_dev(rand_bf16(rng, (2, 24))), torch.zeros(32, 24, dtype=torch.uint8, device=DEV), sd)
    empty = F.fmlp_linear_w8(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), qd, sd)
    assert empty.shape == (0, 32)


# (form, K, H, N): rows of at most 4096 codes with one layer-1 tile per block
# take the two-role kernel (a gated layer 1 of one or two load batches, blocks
# without a layer-2 tile, blocks with several); K = 8192 takes the one-role kernel
_ONE_LAUNCH_CASES = [("mlp2", 4096, 4096, 4096), ("glu", 4096, 4096, 4096), ("mlp2", 1040, 336, 272),
                     ("glu", 768, 3072, 768), ("glu", 2112, 1040, 2112), ("mlp2", 1040, 64, 272),
                     ("mlp2", 8192, 1024, 1040), ("glu", 8192, 2048, 8192)]


@pytest.mark.parametrize("form,K,H,N", _ONE_LAUNCH_CASES)
def test_w8_one_launch_equals_two_launches(form, K, H, N):
    """At one token the one-launch form computes exactly what the two launches
    do (same per-tile order, h rounded to bf16 once): bitwise equal, over 20
    back-to-back calls that alternate two inputs on one workspace, with no
    barrier wait given up and the decode generation moving once per call."""
    rng = np.random.default_rng(77 + K + H + N)
    xs = [to_dev(rand_bf16(rng, (1, K))) for _ in range(2)]
    if form == "mlp2":
        q1, s1, q1d, s1d = _codes(rng, H, K, 1 / 64)
        q2, s2, q2d, s2d = _codes(rng, N, H, 1 / 64)
        b1, b2 = to_dev(rand_bf16(rng, (H,), 1 / 64, "uniform")), to_dev(rand_bf16(rng, (N,), 1 / 64, "uniform"))
        ws = F.workspace_for(DEV, int(F.lib().fmlp_w8_workspace_size(1, H)))
        call = lambda x, out: F.fmlp_mlp2_w8(x, q1d, s1d, b1, q2d, s2d, b2, "gelu_erf", out=out)  # noqa: E731
    else:
        qg, sg, qgd, sgd = _codes(rng, H, K, K ** -0.5)
        qu, su, qud, sud = _codes(rng, H, K, K ** -0.5)
        qdn, sdn, qdd, sdd = _codes(rng, K, H, H ** -0.5)
        ws = F.workspace_for(DEV, int(F.lib().fmlp_w8_workspace_size(1, H)))
        call = lambda x, out: F.fmlp_glu_w8(x, qgd, sgd, qud, sud, qdd, sdd, "silu", out=out)  # noqa: E731
    print(f"case fp8 {form} K={K} H={H} N={N} one launch vs two launches", flush=True)
    with F.force_path("gemm"):
        want = [call(x, None) for x in xs]
    torch.cuda.synchronize()
    gen0, tmo0 = F.decode_generation(ws), F.barrier_timeouts(ws)
    outs = [torch.empty(1, N, dtype=torch.bfloat16, device=DEV) for _ in range(20)]
    for i in range(20):
        call(xs[i % 2], outs[i])
    torch.cuda.synchronize()
    for i in range(20):
        assert torch.equal(outs[i].view(torch.int16), want[i % 2].view(torch.int16)), f"call {i}"
    assert F.decode_generation(ws) == (gen0 + 20) & 0xFFFFFFFF
    assert F.barrier_timeouts(ws) == tmo0
