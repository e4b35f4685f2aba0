"""fmlp_moe_route on the GPU: router logits against the fp64 oracle, the
integer top-k ids exactly against the oracle's decision taken on the kernel's
own fp32 logits, the gate weights against the softmax of those logits, ties,
determinism, the 4096-token 8-expert workload in full, and routing straight
into the gated MoE."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import assert_parity, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _check(x, Wr, k, what):
    d = F.fmlp_moe_route(to_dev(x), to_dev(Wr), k, with_logits=True)
    torch.cuda.synchronize()
    ids, gw, lg = (a.cpu().numpy() for a in d)
    ref_ids, ref_gw, ref_lg = oracle.moe_router(f64_of_bits(x), f64_of_bits(Wr), k)
    # logits: fp32 accumulation against fp64, the parity bound and a tighter one
    assert_parity(d[2], ref_lg, f"{what} logits")
    assert np.max(np.abs(lg - ref_lg)) <= 1e-4 * max(np.max(np.abs(ref_lg)), 1e-3), what
    # ids: the same decision taken on the kernel's own fp32 logits, exactly
    own_ids, own_gw = oracle.route_topk(lg.astype(np.float64), k)
    assert np.array_equal(ids, own_ids), what
    assert np.max(np.abs(gw - own_gw)) <= 2e-6, what
    np.testing.assert_allclose(gw.sum(axis=1), 1.0, rtol=0, atol=2e-6)
    # against the fp64 decision: equal wherever the k-th and (k+1)-th logits are
    # not within the fp32 error of each other (there either choice is correct)
    E = Wr.shape[0]
    if k < E:
        s = np.sort(ref_lg, axis=1)[:, ::-1]
        clear = (s[:, k - 1] - s[:, k]) > 1e-4 * max(np.max(np.abs(ref_lg)), 1e-3)
        assert np.array_equal(ids[clear], ref_ids[clear]), what
        assert np.max(np.abs(gw[clear] - ref_gw[clear]), initial=0.0) <= 1e-4, what
    return ids, gw


@pytest.mark.parametrize("T,D,E,k", [
    (1, 64, 2, 1), (5, 128, 8, 2), (37, 520, 8, 2), (300, 4096, 8, 2), (1000, 256, 13, 3),
    (257, 1024, 16, 4), (130, 512, 32, 8), (99, 384, 64, 8), (64, 96, 1, 1), (77, 64, 64, 1),
    # up to 16 experts on the matrix cores (k tails: D not a multiple of 32);
    # past 16 with the router weights past 64 KB: read through the caches
    (33, 8192, 8, 2), (200, 4104, 16, 2), (17, 40, 16, 8), (70, 1536, 32, 3), (50, 2048, 64, 4),
    # more 16-token tiles than CUs (the 8-step load batches, two blocks per CU),
    # the last at the workload's width with twice its tokens
    (4200, 264, 8, 2), (5000, 4104, 16, 3), (8192, 4096, 8, 2),
])
def test_router_random(T, D, E, k):
    rng = np.random.default_rng(T + D + E + k)
    x = rand_bf16(rng, (T, D))
    Wr = rand_bf16(rng, (E, D), D ** -0.5, "uniform")
    print(f"case router T={T} D={D} E={E} k={k}", flush=True)
    _check(x, Wr, k, f"router {T}x{D} E{E} k{k}")


def test_router_ties_go_to_lower_id():
    """Experts with identical router rows have bitwise equal logits (the same
    products summed in the same order): the lower id must come first."""
    rng = np.random.default_rng(3)
    T, D = 100, 256
    x = rand_bf16(rng, (T, D))
    w = rand_bf16(rng, (3, D), D ** -0.5, "uniform")
    Wr = np.stack([w[0], w[1], w[0], w[2], w[1], w[0]])   # experts 0,2,5 equal; 1,4 equal
    print("case router ties", flush=True)
    ids, gw = _check(x, Wr, 6, "router ties")
    for r in ids.tolist():
        pos = {e: i for i, e in enumerate(r)}
        assert pos[0] < pos[2] < pos[5] and pos[1] < pos[4]
    # equal logits give equal gate weights
    g = dict(zip(ids[0].tolist(), gw[0].tolist()))
    assert g[0] == g[2] == g[5] and g[1] == g[4]


def test_router_workload_full_and_deterministic():
    w = datagen.workload("router")
    x = datagen.make_inputs(datagen.workload("moe"), seed=0, with_weights=False)["x"]
    Wr = datagen.router_weights(w, seed=0)
    print("case router workload 4096x4096 E8 top2", flush=True)
    ids, gw = _check(x, Wr, w.top_k, "router workload")
    d = F.fmlp_moe_route(to_dev(x), to_dev(Wr), w.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(d[0].cpu().numpy(), ids)
    assert np.array_equal(d[1].cpu().numpy(), gw)
    # every expert gets tokens: the routing is not degenerate at this init
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert counts.min() > 0.05 * ids.size / w.E, counts


def test_route_then_moe():
    """Routes computed on the device feed the gated MoE directly."""
    rng = np.random.default_rng(11)
    T, D, H, E, k = 300, 256, 512, 8, 2
    x = rand_bf16(rng, (T, D))
    Wr = rand_bf16(rng, (E, D), D ** -0.5, "uniform")
    Wg = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wu = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wd = np.stack([rand_bf16(rng, (D, H), H ** -0.5, "uniform") for _ in range(E)])
    xd = to_dev(x)
    print("case route then moe", flush=True)
    ids, gw = F.fmlp_moe_route(xd, to_dev(Wr), k)
    y = F.fmlp_moe_glu(xd, ids, gw, to_dev(Wg), to_dev(Wu), to_dev(Wd), gate_act="silu")
    torch.cuda.synchronize()
    ref = oracle.moe_glu(f64_of_bits(x), ids.cpu().numpy(), gw.cpu().numpy().astype(np.float64),
                         lambda e: (f64_of_bits(Wg[e]), f64_of_bits(Wu[e]), f64_of_bits(Wd[e])), "silu")
    assert_parity(y, ref, "route then moe")
