"""ReLU and SiLU epilogues and the gated block with a chosen gate activation
(SwiGLU, ReGLU, exact-GELU GeGLU, bilinear) on the GPU against the fp64
oracle: every path (decode, small fused, tiled GEMM, grouped MoE), activation
pins on identity weights, and equality with the GeGLU entry points when the
gate activation is the tanh GELU."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bf16_ulp, bits_of, f64_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu

NEW_ACTS = ["relu", "silu"]
GATE_ACTS = ["silu", "relu", "gelu_erf", "none"]


@pytest.mark.parametrize("M,K,N", [(1, 520, 136), (16, 4096, 64), (3, 1024, 8192), (300, 72, 264),
                                   (2048, 768, 3072), (4100, 328, 4104)])
@pytest.mark.parametrize("act", NEW_ACTS)
def test_linear_new_acts(M, K, N, act):
    rng = np.random.default_rng(M * 7 + K + N)
    x = rand_bf16(rng, (M, K))
    W = rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.5, "uniform")
    for bias in (None, b):
        print(f"case linear M={M} K={K} N={N} act={act} bias={bias is not None}", flush=True)
        y = F.fmlp_linear(to_dev(x), to_dev(W), None if bias is None else to_dev(bias), act)
        torch.cuda.synchronize()
        ref = oracle.linear(f64_of_bits(x), f64_of_bits(W), None if bias is None else f64_of_bits(bias), act)
        assert_parity(y, ref, f"linear {M}x{K}x{N} {act}")


@pytest.mark.parametrize("M", [1, 16, 300])
def test_new_act_pins(M):
    """Identity W, no bias, x across [-8, 8]: the kernel matches the oracle's
    activation to 1 bf16 ulp, where the other activations are many ulps away."""
    K = N = 128
    vals = np.linspace(-8.0, 8.0, M * K).reshape(M, K).astype(np.float32)
    x = datagen.rne_bf16(vals)
    I = datagen.rne_bf16(np.eye(N, K, dtype=np.float32))
    xf = f64_of_bits(x)
    for act in NEW_ACTS:
        print(f"case act pin M={M} act={act}", flush=True)
        y = f64_of(F.fmlp_linear(to_dev(x), to_dev(I), None, act))
        want = oracle.activation(xf, act)
        ulp = bf16_ulp(want)
        assert np.max(np.abs(y - want) / ulp) <= 1.0, act
        for other in ("gelu_erf", "gelu_tanh", "relu", "silu"):
            if other != act:
                assert np.max(np.abs(oracle.activation(xf, other) - want) / ulp) > 5.0, (act, other)


@pytest.mark.parametrize("M,K,H,N,path", [(1, 4096, 1024, 4096, "decode"), (16, 512, 256, 1024, "decode"),
                                          (64, 32, 64, 32, "small"), (300, 768, 1024, 392, "gemm")])
@pytest.mark.parametrize("act", NEW_ACTS)
def test_mlp2_new_acts(M, K, H, N, path, act):
    rng = np.random.default_rng(M + K + H + N)
    t = {"x": rand_bf16(rng, (M, K)),
         "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"), "b1": rand_bf16(rng, (H,), 0.2, "uniform"),
         "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"), "b2": rand_bf16(rng, (N,), 0.2, "uniform")}
    d = {k: to_dev(v) for k, v in t.items()}
    print(f"case mlp2 {act} M={M} K={K} H={H} N={N} path={path}", flush=True)
    with F.force_path(path):
        y = F.fmlp_mlp2(d["x"], d["W1"], d["b1"], d["W2"], d["b2"], act)
    torch.cuda.synchronize()
    ref = oracle.mlp2(*(f64_of_bits(t[k]) for k in ("x", "W1", "b1", "W2", "b2")), act)
    assert_parity(y, ref, f"mlp2 {act} {M}x{K}x{H}x{N} {path}")


def _glu_inputs(rng, M, D, H):
    return (rand_bf16(rng, (M, D)), rand_bf16(rng, (H, D), D ** -0.5, "uniform"),
            rand_bf16(rng, (H, D), D ** -0.5, "uniform"), rand_bf16(rng, (D, H), H ** -0.5, "uniform"))


@pytest.mark.parametrize("M,D,H", [(1, 256, 512), (16, 1024, 2048), (1, 4096, 4096), (300, 520, 1048),
                                   (777, 768, 3072), (2100, 264, 4104)])
@pytest.mark.parametrize("gate_act", GATE_ACTS)
def test_glu_gate_acts(M, D, H, gate_act):
    rng = np.random.default_rng(M * 3 + D + H)
    x, Wg, Wu, Wd = _glu_inputs(rng, M, D, H)
    ref = oracle.glu(f64_of_bits(x), f64_of_bits(Wg), f64_of_bits(Wu), f64_of_bits(Wd), gate_act)
    d = [to_dev(a) for a in (x, Wg, Wu, Wd)]
    for p in (["decode", "gemm"] if M <= 16 else ["auto"]):
        print(f"case glu {gate_act} M={M} D={D} H={H} path={p}", flush=True)
        with F.force_path(p):
            y = F.fmlp_glu(*d, gate_act=gate_act)
        torch.cuda.synchronize()
        assert_parity(y, ref, f"glu {gate_act} {M}x{D}x{H} {p}")


@pytest.mark.parametrize("M,path", [(1, "decode"), (16, "decode"), (300, "gemm")])
def test_glu_tanh_is_geglu_bitwise(M, path):
    rng = np.random.default_rng(5 + M)
    d = [to_dev(a) for a in _glu_inputs(rng, M, 512, 1024)]
    print(f"case glu(gelu_tanh) == geglu M={M} path={path}", flush=True)
    with F.force_path(path):
        a = bits_of(F.fmlp_glu(*d, gate_act="gelu_tanh"))
        b = bits_of(F.fmlp_geglu(*d))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


def test_swiglu768_full():
    """The 8192-token 768/3072 gated block with a SiLU gate, in full."""
    w = datagen.workload("geglu768")
    t = datagen.make_inputs(w, seed=0)
    print("case swiglu768 full", flush=True)
    y = F.fmlp_glu(*(to_dev(t[k]) for k in ("x", "Wg", "Wu", "Wd")), gate_act="silu")
    torch.cuda.synchronize()
    ref = oracle.glu(*(f64_of_bits(t[k]) for k in ("x", "Wg", "Wu", "Wd")), "silu")
    assert_parity(y, ref, "swiglu 8192x768x3072")


@pytest.mark.parametrize("T,D,H,E,k", [(5, 64, 128, 4, 2), (300, 256, 512, 8, 2), (1000, 128, 256, 16, 2)])
def test_moe_glu_silu(T, D, H, E, k):
    rng = np.random.default_rng(T + D + H + E + k)
    x = rand_bf16(rng, (T, D))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    gw = rng.random((T, k)).astype(np.float32)
    Wg = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wu = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wd = np.stack([rand_bf16(rng, (D, H), H ** -0.5, "uniform") for _ in range(E)])
    dv = [to_dev(x), to_dev(ids, torch.int32), to_dev(gw, torch.float32), to_dev(Wg), to_dev(Wu), to_dev(Wd)]
    print(f"case moe swiglu T={T} D={D} H={H} E={E} k={k}", flush=True)
    y = F.fmlp_moe_glu(*dv, gate_act="silu")
    torch.cuda.synchronize()
    ref = oracle.moe_glu(f64_of_bits(x), ids, gw.astype(np.float64),
                         lambda e: (f64_of_bits(Wg[e]), f64_of_bits(Wu[e]), f64_of_bits(Wd[e])), "silu")
    assert_parity(y, ref, f"moe swiglu {T}x{D}x{H} E{E}")
    # the tanh-GELU gate through the generic entry equals the GeGLU entry bitwise
    a = bits_of(F.fmlp_moe_glu(*dv, gate_act="gelu_tanh"))
    b = bits_of(F.fmlp_moe_geglu(*dv))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
