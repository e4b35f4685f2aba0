"""The decode kernel (1-16 tokens) and the small MLP for every activation, against
the fp64 oracle (oracle.linear, oracle.mlp2, oracle.glu): one layer, the
two-layer MLP and the gated block in one launch, at 1, 3 and 16 tokens (the
kernel's three activation-row classes).  The one-token two-layer shapes have
at least as many first-layer tiles as blocks, so their hidden values go
through the word-tagged exchange; the others through the flag exchange.  The
activation is compiled into each kernel, so every (form, class, activation)
here is a kernel of its own."""
import numpy as np
import pytest
import torch

import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import assert_parity, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu

ACTS = ["none", "gelu_erf", "gelu_tanh", "relu", "silu"]
TOKENS = [1, 3, 16]


@pytest.mark.parametrize("M", TOKENS)
@pytest.mark.parametrize("act", ACTS)
def test_decode_linear_acts(act, M):
    rng = np.random.default_rng(M * 7 + ACTS.index(act))
    K, N = 512, 520
    x, W = rand_bf16(rng, (M, K)), rand_bf16(rng, (N, K), K ** -0.5, "uniform")
    b = rand_bf16(rng, (N,), 0.3, "uniform")
    print(f"case decode linear {act} M={M}", flush=True)
    with F.force_path("decode"):
        y = F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), act)
    torch.cuda.synchronize()
    assert_parity(y, oracle.linear(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), act), f"linear {act} M={M}")


@pytest.mark.parametrize("M", TOKENS)
@pytest.mark.parametrize("act", ACTS)
def test_decode_mlp2_acts(act, M):
    rng = np.random.default_rng(M * 11 + ACTS.index(act))
    K, H, N = 256, 4096, 264   # 256 first-layer tiles
    t = {"x": rand_bf16(rng, (M, K)), "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"),
         "b1": rand_bf16(rng, (H,), 0.3, "uniform"), "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"),
         "b2": rand_bf16(rng, (N,), 0.3, "uniform")}
    print(f"case decode mlp2 {act} M={M}", flush=True)
    d = {k: to_dev(v) for k, v in t.items()}
    with F.force_path("decode"):
        y = F.fmlp_mlp2(d["x"], d["W1"], d["b1"], d["W2"], d["b2"], act)
    torch.cuda.synchronize()
    ref = oracle.mlp2(*(f64_of_bits(t[k]) for k in ("x", "W1", "b1", "W2", "b2")), act)
    assert_parity(y, ref, f"mlp2 {act} M={M}")


@pytest.mark.parametrize("M", TOKENS)
@pytest.mark.parametrize("act", ACTS)
def test_decode_glu_acts(act, M):
    rng = np.random.default_rng(M * 13 + ACTS.index(act))
    D, H = 256, 4096
    x = rand_bf16(rng, (M, D))
    Wg, Wu = rand_bf16(rng, (H, D), D ** -0.5, "uniform"), rand_bf16(rng, (H, D), D ** -0.5, "uniform")
    Wd = rand_bf16(rng, (D, H), H ** -0.5, "uniform")
    print(f"case decode glu {act} M={M}", flush=True)
    with F.force_path("decode"):
        y = F.fmlp_glu(*(to_dev(a) for a in (x, Wg, Wu, Wd)), act)
    torch.cuda.synchronize()
    assert_parity(y, oracle.glu(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)), act), f"glu {act} M={M}")


@pytest.mark.parametrize("act", ACTS)
def test_small_mlp2_acts(act):
    """The single-launch small MLP (K, H, N <= 128), also one kernel per
    activation, with a ragged last block of token rows."""
    rng = np.random.default_rng(17 + ACTS.index(act))
    M, K, H, N = 100, 32, 72, 40
    t = {"x": rand_bf16(rng, (M, K)), "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"),
         "b1": rand_bf16(rng, (H,), 0.3, "uniform"), "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"),
         "b2": rand_bf16(rng, (N,), 0.3, "uniform")}
    print(f"case small mlp2 {act}", flush=True)
    d = {k: to_dev(v) for k, v in t.items()}
    with F.force_path("small"):
        y = F.fmlp_mlp2(d["x"], d["W1"], d["b1"], d["W2"], d["b2"], act)
    torch.cuda.synchronize()
    ref = oracle.mlp2(*(f64_of_bits(t[k]) for k in ("x", "W1", "b1", "W2", "b2")), act)
    assert_parity(y, ref, f"small mlp2 {act}")
