"""fmlp_moe_geglu on the GPU against the fp64 oracle: small random routings
(ragged and empty experts, duplicate ids, top_k 1..3), reductions to the dense
GeGLU, invalid-id accounting, and the 8-expert 4096-token workload on sampled
tokens."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bits_of, f64_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _experts(rng, E, D, H):
    Wg = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wu = np.stack([rand_bf16(rng, (H, D), D ** -0.5, "uniform") for _ in range(E)])
    Wd = np.stack([rand_bf16(rng, (D, H), H ** -0.5, "uniform") for _ in range(E)])
    return Wg, Wu, Wd


def _oracle(x, ids, gw, Wg, Wu, Wd):
    return oracle.moe_geglu(f64_of_bits(x), ids, gw.astype(np.float64),
                            lambda e: (f64_of_bits(Wg[e]), f64_of_bits(Wu[e]), f64_of_bits(Wd[e])))


def _run(x, ids, gw, Wg, Wu, Wd, ws=None):
    y = F.fmlp_moe_geglu(to_dev(x), to_dev(ids, torch.int32), to_dev(gw, torch.float32),
                         to_dev(Wg), to_dev(Wu), to_dev(Wd), workspace=ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,D,H,E,k", [
    (1, 64, 64, 2, 1), (5, 64, 128, 4, 2), (37, 128, 96, 4, 2), (300, 256, 512, 8, 2),
    (129, 64, 200, 3, 3), (1000, 128, 256, 16, 2), (64, 96, 64, 1, 1),
    (300, 256, 4096, 4, 2), (700, 128, 4160, 8, 2),   # down projection split over K (K tail in the second)
])
def test_moe_random(T, D, H, E, k):
    rng = np.random.default_rng(T * 17 + D + H + E + k)
    x = rand_bf16(rng, (T, D))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    gw = rng.random((T, k)).astype(np.float32)
    Wg, Wu, Wd = _experts(rng, E, D, H)
    print(f"case moe T={T} D={D} H={H} E={E} k={k}", flush=True)
    assert_parity(_run(x, ids, gw, Wg, Wu, Wd), _oracle(x, ids, gw, Wg, Wu, Wd), f"moe {T}x{D}x{H} E{E} k{k}")


def test_moe_skewed_and_empty_experts():
    rng = np.random.default_rng(1)
    T, D, H, E, k = 700, 128, 256, 8, 2
    x = rand_bf16(rng, (T, D))
    ids = np.where(rng.random((T, k)) < 0.9, 5, 2).astype(np.int32)   # experts 5 and 2 only
    ids[:3] = [[0, 7], [7, 7], [0, 0]]                                # duplicates
    gw = rng.random((T, k)).astype(np.float32)
    Wg, Wu, Wd = _experts(rng, E, D, H)
    print("case moe skewed/empty experts", flush=True)
    assert_parity(_run(x, ids, gw, Wg, Wu, Wd), _oracle(x, ids, gw, Wg, Wu, Wd), "moe skewed")


def test_moe_top1_equals_dense_geglu():
    rng = np.random.default_rng(2)
    T, D, H, E = 250, 256, 512, 4
    x = rand_bf16(rng, (T, D))
    Wg, Wu, Wd = _experts(rng, E, D, H)
    dense = F.fmlp_geglu(to_dev(x), to_dev(Wg[3]), to_dev(Wu[3]), to_dev(Wd[3]))
    ids = np.full((T, 1), 3, np.int32)
    gw = np.ones((T, 1), np.float32)
    print("case moe top1 == dense", flush=True)
    y = _run(x, ids, gw, Wg, Wu, Wd)
    # same m rounding; y differs only by the fp32 -> bf16 round of the combine
    assert np.max(np.abs(f64_of(y) - f64_of(dense))) <= 1e-2 * np.max(np.abs(f64_of(dense))) + 1e-3


def test_moe_invalid_ids_counted_and_skipped():
    rng = np.random.default_rng(3)
    T, D, H, E, k = 50, 64, 64, 4, 2
    x = rand_bf16(rng, (T, D))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[4, 1] = 9
    ids[10, 0] = -1
    gw = rng.random((T, k)).astype(np.float32)
    Wg, Wu, Wd = _experts(rng, E, D, H)
    ws = F.workspace_for(DEV, F.fmlp_moe_workspace_size(T, D, H, E, k))
    print("case moe invalid ids", flush=True)
    y = _run(x, ids, gw, Wg, Wu, Wd, ws)
    assert F.moe_invalid_ids(ws) == 2
    ok_ids = ids.copy()
    gw0 = gw.copy()
    bad = (ids < 0) | (ids >= E)
    ok_ids[bad] = 0
    gw0[bad] = 0.0          # an invalid pair contributes nothing
    assert_parity(y, _oracle(x, ok_ids, gw0, Wg, Wu, Wd), "moe invalid ids")


def test_moe_many_pairs_and_partial_expert_batch():
    """More (token, slot) pairs than the routing kernel keeps in registers per
    thread (the rest are re-read), an expert count that is not a multiple of
    the routing batch, and invalid ids in both the register and re-read runs."""
    rng = np.random.default_rng(6)
    T, D, H, E, k = 5000, 64, 64, 6, 2
    x = rand_bf16(rng, (T, D))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[0, 0] = -1          # first pair of the first run
    ids[2503, 1] = E        # deep in a run (position 19 of 20)
    ids[4999, 1] = 77       # the last pair
    gw = rng.random((T, k)).astype(np.float32)
    Wg, Wu, Wd = _experts(rng, E, D, H)
    ws = F.workspace_for(DEV, F.fmlp_moe_workspace_size(T, D, H, E, k))
    print("case moe many pairs", flush=True)
    y = _run(x, ids, gw, Wg, Wu, Wd, ws)
    assert F.moe_invalid_ids(ws) == 3
    ok_ids = ids.copy()
    gw0 = gw.copy()
    bad = (ids < 0) | (ids >= E)
    ok_ids[bad] = 0
    gw0[bad] = 0.0
    assert_parity(y, _oracle(x, ok_ids, gw0, Wg, Wu, Wd), "moe many pairs")


def _route_tables(ws, T, E, k):
    """The route tables in an fmlp_moe_geglu workspace, at the offsets the
    library lays them out: after the 8 KB header, tok_of, scale_of and pos_of
    ([T*k] each), then group_off and tile_off ([E+1] each), every array
    starting on a 256-byte boundary."""
    P = T * k
    ru = lambda n: -(-n // 256) * 256
    o = 8192
    out = {}
    for name, n, dt in (("tok_of", P, torch.int32), ("scale_of", P, torch.float32), ("pos_of", P, torch.int32),
                        ("group_off", E + 1, torch.int32), ("tile_off", E + 1, torch.int32)):
        out[name] = ws[o:o + 4 * n].view(dt).cpu().numpy()
        o += ru(4 * n)
    return out


@pytest.mark.parametrize("T,E,k,case", [
    (1, 1, 1, "random"), (257, 64, 3, "random"), (700, 8, 2, "skewed"), (5000, 6, 2, "invalid"),
    (3000, 1000, 8, "random"), (4096, 8, 2, "workload"), (2048, 3, 1, "one expert"),
    (600, 1024, 2, "random"),   # the most experts a call takes
    (65536, 16, 4, "random"),   # 512 blocks of pairs: the scan reads many batches of block counts
])
def test_moe_route_tables_exact(T, E, k, case):
    """The bucketing itself, exactly: every valid (token, slot) pair p = t*k + j
    sits in its expert's segment in pair order (a stable sort by expert), with
    its token and gate weight; pos_of maps each pair to its row (-1 if its id
    is invalid); group_off and tile_off are the prefix sums of the expert
    sizes and of their 256-row tile counts.  Blocks of the routing kernels
    hold 512 pairs, so these cases span one to 512 of them, partial last ones
    and up to 1024 experts."""
    rng = np.random.default_rng(T + E + k)
    if case == "workload":
        ids, gw = datagen.make_routes(T, E, k, seed=0)
    else:
        ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        gw = rng.random((T, k)).astype(np.float32)
    if case == "skewed":
        ids = np.where(rng.random((T, k)) < 0.9, 5, 2).astype(np.int32)
        ids[:3] = [[0, 7], [7, 7], [0, 0]]
    if case == "invalid":
        ids[0, 0], ids[2503, 1], ids[4999, 1], ids[1000, 0] = -1, E, 77, -5
    if case == "one expert":
        ids[:] = 1
    D = H = 64
    Wg, Wu, Wd = (np.zeros((E, H, D), np.uint16), np.zeros((E, H, D), np.uint16), np.zeros((E, D, H), np.uint16))
    ws = F.workspace_for(DEV, F.fmlp_moe_workspace_size(T, D, H, E, k))
    x = rand_bf16(rng, (T, D))
    print(f"case moe route tables T={T} E={E} k={k} {case}", flush=True)
    _run(x, ids, gw, Wg, Wu, Wd, ws)
    got = _route_tables(ws, T, E, k)
    flat, wflat = ids.reshape(-1), gw.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    vp = np.nonzero(valid)[0]
    order = vp[np.argsort(flat[vp], kind="stable")]
    n = len(order)
    assert F.moe_invalid_ids(ws) == len(flat) - n
    assert np.array_equal(got["tok_of"][:n], (order // k).astype(np.int32))
    assert np.array_equal(got["scale_of"][:n].view(np.int32), wflat[order].view(np.int32))
    pos = np.full(len(flat), -1, np.int32)
    pos[order] = np.arange(n, dtype=np.int32)
    assert np.array_equal(got["pos_of"], pos)
    counts = np.bincount(flat[vp], minlength=E)
    assert np.array_equal(got["group_off"], np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    tiles = -(-counts // 256)
    assert np.array_equal(got["tile_off"], np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32))


def test_moe_determinism():
    rng = np.random.default_rng(4)
    T, D, H, E, k = 513, 256, 384, 8, 2
    x = rand_bf16(rng, (T, D))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    gw = rng.random((T, k)).astype(np.float32)
    Wg, Wu, Wd = _experts(rng, E, D, H)
    print("case moe determinism", flush=True)
    assert np.array_equal(bits_of(_run(x, ids, gw, Wg, Wu, Wd)), bits_of(_run(x, ids, gw, Wg, Wu, Wd)))


def moe_sample_tokens(ids: np.ndarray, E: int, n_min: int = 512, tile: int = 256, seed: int = 0) -> np.ndarray:
    """Tokens whose routed rows sit at the edges of every expert's segment and
    of every 256-row tile in it (positions 0, 255, 256, ..., last of the
    segment: tail tiles included), topped up with random tokens to at least
    n_min.  Pairs are bucketed per expert stably in pair order (t * top_k + j)."""
    T, k = ids.shape
    pick = set()
    flat = ids.reshape(-1)
    for e in range(E):
        seg = np.nonzero(flat == e)[0] // k       # tokens of expert e's rows, in segment order
        if len(seg) == 0:
            continue
        edges = {0, len(seg) - 1}
        for b in range(0, len(seg), tile):
            edges.update({b, min(b + tile - 1, len(seg) - 1)})
        pick.update(int(seg[i]) for i in edges)
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, dtype=np.int64))
    extra = rng.choice(rest, size=max(0, n_min - len(pick)), replace=False)
    return np.unique(np.concatenate([np.fromiter(pick, dtype=np.int64), extra]))


@pytest.mark.slow
def test_moe_workload_sampled_tokens():
    """The 8 x (4096/14336) top-2 workload at 4096 tokens, compared on at least
    512 tokens (tokens are independent) that include the first and last routed
    row of every expert segment and of every 256-row tile in it, so tail tiles
    and both K halves of the down projection are compared."""
    w = datagen.workload("moe")
    x = datagen.make_inputs(w, seed=0, with_weights=False)["x"]
    ids, gw = datagen.make_routes(w.M, w.E, w.top_k, seed=0)
    experts = [datagen.expert_weights(w, e, seed=0) for e in range(w.E)]
    Wg = torch.stack([to_dev(e[0]) for e in experts])
    Wu = torch.stack([to_dev(e[1]) for e in experts])
    Wd = torch.stack([to_dev(e[2]) for e in experts])
    print(f"case {w.name} (sampled tokens)", flush=True)
    ws = F.workspace_for(DEV, F.fmlp_moe_workspace_size(w.M, w.K, w.H, w.E, w.top_k))
    y = F.fmlp_moe_geglu(to_dev(x), to_dev(ids, torch.int32), to_dev(gw, torch.float32), Wg, Wu, Wd,
                         workspace=ws)
    torch.cuda.synchronize()
    assert F.moe_invalid_ids(ws) == 0
    toks = moe_sample_tokens(ids, w.E)
    assert len(toks) >= 512
    ref = oracle.moe_geglu(f64_of_bits(x[toks]), ids[toks], gw[toks].astype(np.float64),
                           lambda e: tuple(f64_of_bits(a) for a in experts[e]))
    assert_parity(y[torch.from_numpy(toks).to(DEV)], ref, f"{w.name} {len(toks)} tokens")
    assert np.isfinite(f64_of(y)).all()
