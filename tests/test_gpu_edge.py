"""Degenerate inputs on the GPU through the C ABI: zero tokens on every call
(a no-op that leaves the output untouched), one token and one expert, inner
dimensions at the smallest legal size (8), and output rows that are exactly a
tile edge."""
import numpy as np
import pytest
import torch

import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def test_zero_tokens_is_a_noop():
    rng = np.random.default_rng(1)
    W = to_dev(rand_bf16(rng, (64, 32), 0.2, "uniform"))
    W2 = to_dev(rand_bf16(rng, (32, 64), 0.2, "uniform"))
    x = torch.empty(0, 32, dtype=torch.bfloat16, device=DEV)
    print("case zero tokens", flush=True)
    assert F.fmlp_linear(x, W, None, "silu").shape == (0, 64)
    assert F.fmlp_mlp2(x, W, None, W2, None, "gelu_erf").shape == (0, 32)
    Wg = to_dev(rand_bf16(rng, (64, 32), 0.2, "uniform"))
    Wd = to_dev(rand_bf16(rng, (32, 64), 0.2, "uniform"))
    assert F.fmlp_glu(x, Wg, Wg, Wd, gate_act="relu").shape == (0, 32)
    ids = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    gw = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    We = to_dev(np.stack([rand_bf16(rng, (64, 32), 0.2, "uniform")] * 2))
    Wde = to_dev(np.stack([rand_bf16(rng, (32, 64), 0.2, "uniform")] * 2))
    assert F.fmlp_moe_geglu(x, ids, gw, We, We, Wde).shape == (0, 32)
    Wr = to_dev(rand_bf16(rng, (4, 32), 0.2, "uniform"))
    r_ids, r_gw = F.fmlp_moe_route(x, Wr, 2)
    torch.cuda.synchronize()
    assert r_ids.shape == (0, 2) and r_gw.shape == (0, 2)


@pytest.mark.parametrize("M", [1, 5, 16, 17, 256, 257])
def test_smallest_inner_dims(M):
    """K = N = 8 (one 16-byte row): every path's masks of a mostly empty tile."""
    rng = np.random.default_rng(M)
    x = rand_bf16(rng, (M, 8))
    W = rand_bf16(rng, (8, 8), 0.3, "uniform")
    b = rand_bf16(rng, (8,), 0.3, "uniform")
    print(f"case smallest inner dims M={M}", flush=True)
    for act in ("gelu_tanh", "relu"):
        y = F.fmlp_linear(to_dev(x), to_dev(W), to_dev(b), act)
        torch.cuda.synchronize()
        assert_parity(y, oracle.linear(f64_of_bits(x), f64_of_bits(W), f64_of_bits(b), act), f"linear 8x8 M={M}")
    W2 = rand_bf16(rng, (8, 8), 0.3, "uniform")
    y = F.fmlp_glu(to_dev(x), to_dev(W), to_dev(W2), to_dev(W2), gate_act="silu")
    torch.cuda.synchronize()
    assert_parity(y, oracle.glu(*(f64_of_bits(a) for a in (x, W, W2, W2)), "silu"), f"glu 8 M={M}")


def test_one_token_one_expert():
    rng = np.random.default_rng(9)
    D, H = 64, 128
    x = rand_bf16(rng, (1, D))
    Wg = rand_bf16(rng, (1, H, D), D ** -0.5, "uniform")
    Wu = rand_bf16(rng, (1, H, D), D ** -0.5, "uniform")
    Wd = rand_bf16(rng, (1, D, H), H ** -0.5, "uniform")
    ids = np.zeros((1, 1), dtype=np.int32)
    gw = np.ones((1, 1), dtype=np.float32)
    print("case one token one expert", flush=True)
    y = F.fmlp_moe_glu(to_dev(x), to_dev(ids, torch.int32), to_dev(gw, torch.float32), to_dev(Wg), to_dev(Wu),
                       to_dev(Wd), gate_act="gelu_tanh")
    torch.cuda.synchronize()
    ref = oracle.geglu(f64_of_bits(x), f64_of_bits(Wg[0]), f64_of_bits(Wu[0]), f64_of_bits(Wd[0]))
    assert_parity(y, ref, "moe one token one expert")
