"""Pins that tie the fp64 oracle to something other than itself.

Each ``check_*`` takes the oracle module ``o`` and raises AssertionError when the
oracle disagrees with:
  * brute force: pure-Python loops on tiny shapes, using libm's math.erf /
    math.tanh (not the oracle's scipy/numpy path);
  * library routines the pages name: ``F.gelu(..., approximate="tanh")`` and the
    exact ``F.gelu`` (torch, float64, CPU);
  * closed forms and identities (Phi(1), gelu(x) - gelu(-x) = x, ...);
  * the page's printed strides-and-views example (tests/golden/transpose_view.json);
  * invariants (fusion does not change the math; MoE linearity / permutation).

The same checks are run against planted mistakes in test_oracle_mutants.py to
show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# brute force (pure Python, libm)
# ---------------------------------------------------------------------------
def _bf_act(z: float, act: str) -> float:
    if act == "none":
        return z
    if act == "gelu_erf":
        return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
    if act == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * z * (1.0 + math.tanh(c * (z + 0.044715 * z ** 3)))
    if act == "relu":
        return z if z > 0.0 else 0.0
    if act == "silu":
        return z / (1.0 + math.exp(-z)) if z > -700.0 else 0.0
    raise ValueError(act)


def bf_linear(x, W, b, act):
    M, K = len(x), len(x[0])
    N = len(W)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[m][k]) * float(W[n][k])
            if b is not None:
                s += float(b[n])
            y[m][n] = _bf_act(s, act)
    return y


def bf_geglu(x, Wg, Wu, Wd, gate_act="gelu_tanh"):
    g = bf_linear(x, Wg, None, "none")
    u = bf_linear(x, Wu, None, "none")
    m = [[_bf_act(g[i][j], gate_act) * u[i][j] for j in range(len(g[0]))] for i in range(len(g))]
    return bf_linear(m, Wd, None, "none")


def bf_moe(x, ids, gw, experts, gate_act="gelu_tanh"):
    T, D = len(x), len(x[0])
    y = [[0.0] * D for _ in range(T)]
    for t in range(T):
        for j in range(len(ids[t])):
            Wg, Wu, Wd = experts[int(ids[t][j])]
            yt = bf_geglu([x[t]], Wg, Wu, Wd, gate_act)[0]
            for d in range(D):
                y[t][d] += float(gw[t][j]) * yt[d]
    return y


def bf_router(x, Wr, top_k):
    """Pure-Python router: dot products, then top_k by repeated scans for the
    largest remaining logit (the first, i.e. lower id, on a tie), then a
    softmax over the chosen ones with libm exp."""
    ids, gws = [], []
    for row in x:
        lg = [sum(float(a) * float(b) for a, b in zip(row, w)) for w in Wr]
        chosen = []
        for _ in range(top_k):
            best = None
            for e, v in enumerate(lg):
                if e in chosen:
                    continue
                if best is None or v > lg[best]:
                    best = e
            chosen.append(best)
        m = lg[chosen[0]]
        ex = [math.exp(lg[e] - m) for e in chosen]
        s = sum(ex)
        ids.append(chosen)
        gws.append([v / s for v in ex])
    return ids, gws


def _close(a, b, rtol=1e-12, atol=1e-13, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1.0)
    assert err <= rtol * scale + atol, f"{what}: max err {err:.3e} (scale {scale:.3e})"


def _bf16ish(rng, shape, scale=1.0):
    """Random values exactly representable in bf16 (8 significant bits)."""
    a = rng.standard_normal(shape) * scale
    e = np.floor(np.log2(np.maximum(np.abs(a), 1e-30)))
    return np.round(a / 2.0 ** (e - 7)) * 2.0 ** (e - 7)


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------
def check_linear_bruteforce(o):
    rng = np.random.default_rng(1234)
    for (M, K, N) in [(1, 1, 1), (2, 3, 5), (3, 8, 2), (5, 16, 8), (8, 8, 8), (16, 2, 3)]:
        x = _bf16ish(rng, (M, K))
        W = _bf16ish(rng, (N, K), 0.5)
        b = _bf16ish(rng, (N,), 0.5)
        for act in ("none", "gelu_erf", "gelu_tanh", "relu", "silu"):
            for bias in (None, b):
                ref = bf_linear(x.tolist(), W.tolist(), None if bias is None else bias.tolist(), act)
                _close(o.linear(x, W, bias, act), ref, what=f"linear {M}x{K}x{N} {act} bias={bias is not None}")


def check_mlp2_bruteforce(o):
    rng = np.random.default_rng(99)
    for (M, K, H, N) in [(1, 4, 6, 3), (3, 8, 5, 2), (4, 2, 8, 8)]:
        x = _bf16ish(rng, (M, K))
        W1 = _bf16ish(rng, (H, K), 0.5)
        b1 = _bf16ish(rng, (H,), 0.5)
        W2 = _bf16ish(rng, (N, H), 0.5)
        b2 = _bf16ish(rng, (N,), 0.5)
        for act in ("gelu_erf", "gelu_tanh", "none", "relu", "silu"):
            h = bf_linear(x.tolist(), W1.tolist(), b1.tolist(), act)
            ref = bf_linear(h, W2.tolist(), b2.tolist(), "none")
            _close(o.mlp2(x, W1, b1, W2, b2, act), ref, what=f"mlp2 {act}")


def check_geglu_bruteforce(o):
    rng = np.random.default_rng(7)
    for (M, D, H) in [(1, 3, 4), (2, 5, 7), (4, 8, 6)]:
        x = _bf16ish(rng, (M, D))
        Wg = _bf16ish(rng, (H, D), 0.7)
        Wu = _bf16ish(rng, (H, D), 0.7)
        Wd = _bf16ish(rng, (D, H), 0.7)
        ref = bf_geglu(x.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist())
        _close(o.geglu(x, Wg, Wu, Wd), ref, what=f"geglu {M}x{D}x{H}")
        for act in ("gelu_tanh", "gelu_erf", "silu", "relu", "none"):
            ref = bf_geglu(x.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist(), act)
            _close(o.glu(x, Wg, Wu, Wd, act), ref, what=f"glu {act} {M}x{D}x{H}")


def check_moe_bruteforce(o):
    rng = np.random.default_rng(5)
    T, D, H, E, k = 6, 4, 5, 3, 2
    x = _bf16ish(rng, (T, D))
    experts = [(_bf16ish(rng, (H, D), 0.7), _bf16ish(rng, (H, D), 0.7), _bf16ish(rng, (D, H), 0.7))
               for _ in range(E)]
    ids = np.array([[0, 1], [2, 0], [1, 2], [2, 1], [0, 2], [1, 1]], dtype=np.int32)  # last: duplicate id
    gw = rng.random((T, k))
    ref = bf_moe(x.tolist(), ids.tolist(), gw.tolist(),
                 [(a.tolist(), b.tolist(), c.tolist()) for a, b, c in experts])
    _close(o.moe_geglu(x, ids, gw, experts), ref, what="moe brute force")
    ref = bf_moe(x.tolist(), ids.tolist(), gw.tolist(),
                 [(a.tolist(), b.tolist(), c.tolist()) for a, b, c in experts], "silu")
    _close(o.moe_glu(x, ids, gw, experts, "silu"), ref, what="moe silu brute force")


def check_gelu_library(o):
    """The pages name torch's F.gelu (exact) and F.gelu(approximate="tanh")."""
    import torch
    import torch.nn.functional as F

    z = np.concatenate([np.linspace(-12, 12, 4801), [-1e-3, 1e-3, 0.0, 3.0, -3.0]])
    t = torch.from_numpy(z)
    _close(o.gelu_erf(z), F.gelu(t).numpy(), rtol=1e-14, atol=1e-15, what="gelu_erf vs F.gelu")
    _close(o.gelu_tanh(z), F.gelu(t, approximate="tanh").numpy(), rtol=1e-14, atol=1e-15,
           what="gelu_tanh vs F.gelu(tanh)")
    # activation() dispatches by name
    _close(o.activation(z, "gelu_erf"), F.gelu(t).numpy(), rtol=1e-14, atol=1e-15, what="act erf")
    _close(o.activation(z, "gelu_tanh"), F.gelu(t, approximate="tanh").numpy(), rtol=1e-14,
           atol=1e-15, what="act tanh")
    _close(o.activation(z, "none"), z, what="act none")


def check_gelu_closed_forms(o):
    # Phi(1) and Phi(-1): standard normal table values.
    assert abs(float(o.gelu_erf(1.0)) - 0.8413447460685429) < 1e-15
    assert abs(float(o.gelu_erf(-1.0)) + 0.15865525393145707) < 1e-15
    # libm erf, scalar, at a spread of points (incl. the negative tail).
    for v in (-6.0, -4.0, -2.5, -0.3, 0.7, 2.0, 5.0):
        ref = 0.5 * v * math.erfc(-v / math.sqrt(2.0))
        assert abs(float(o.gelu_erf(v)) - ref) <= 1e-15 * max(1.0, abs(ref)), v
    for g in (o.gelu_erf, o.gelu_tanh):
        assert float(g(0.0)) == 0.0
        assert float(g(10.0)) == 10.0           # gelu(x) -> x for x >> 0
        assert -1e-20 <= float(g(-10.0)) <= 0.0  # gelu(x) -> 0- for x << 0
        # odd-part identity: gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1; tanh odd)
        x = np.linspace(-6, 6, 1201)
        _close(g(x) - g(-x), x, rtol=1e-14, atol=1e-14, what="odd-part identity")
        # derivative 1/2 at 0
        h = 1e-6
        d = (float(g(h)) - float(g(-h))) / (2 * h)
        assert abs(d - 0.5) < 1e-9, d
    # the two variants differ, by at most ~4.73e-4, attained near |x| ~ 2.70
    # (their difference is even in x, a consequence of the odd-part identity)
    x = np.linspace(-8, 8, 160001)
    diff = np.abs(o.gelu_erf(x) - o.gelu_tanh(x))
    assert 4.70e-4 < diff.max() < 4.76e-4, diff.max()
    assert 2.6 < abs(x[diff.argmax()]) < 2.8


def check_silu_relu_closed_forms(o):
    """SiLU and ReLU against closed forms, identities and torch's F.silu/F.relu."""
    import torch
    import torch.nn.functional as F

    # sigmoid(1) = 1 / (1 + 1/e)
    assert abs(float(o.silu(1.0)) - 0.7310585786300049) < 1e-15
    assert abs(float(o.silu(-1.0)) + 0.2689414213699951) < 1e-15
    for a in (o.silu, o.relu):
        assert float(a(0.0)) == 0.0
        assert float(a(40.0)) == 40.0                 # -> x for x >> 0
        assert -1e-15 <= float(a(-40.0)) <= 0.0       # -> 0- for x << 0
        # odd-part identity a(x) - a(-x) = x (sigmoid(x) + sigmoid(-x) = 1; max(x,0) - max(-x,0) = x)
        x = np.linspace(-6, 6, 1201)
        _close(a(x) - a(-x), x, rtol=1e-14, atol=1e-14, what="odd-part identity")
    # SiLU: derivative 1/2 at 0; its minimum x* solves x sigmoid(x) = 1 + x, so
    # the minimum value is x* + 1 (x* = -1.278464542761074)
    h = 1e-6
    assert abs((float(o.silu(h)) - float(o.silu(-h))) / (2 * h) - 0.5) < 1e-9
    xs = -1.278464542761074
    assert abs(float(o.silu(xs)) - (xs + 1.0)) < 1e-14
    x = np.linspace(-3, 0, 300001)
    assert abs(x[np.argmin(o.silu(x))] - xs) < 2e-5
    # ReLU is exactly max(x, 0)
    x = np.linspace(-5, 5, 1001)
    assert np.array_equal(o.relu(x), np.maximum(x, 0.0))
    # library routines
    z = np.concatenate([np.linspace(-30, 30, 6001), [-1e-3, 1e-3, 0.0]])
    t = torch.from_numpy(z)
    _close(o.silu(z), F.silu(t).numpy(), rtol=1e-14, atol=1e-15, what="silu vs F.silu")
    _close(o.relu(z), F.relu(t).numpy(), rtol=0, atol=0, what="relu vs F.relu")
    _close(o.activation(z, "silu"), F.silu(t).numpy(), rtol=1e-14, atol=1e-15, what="act silu")
    _close(o.activation(z, "relu"), F.relu(t).numpy(), rtol=0, atol=0, what="act relu")


def check_glu_special_cases(o):
    """The gated block with each gate activation: identity weights give
    act(x) * x; the up projection is linear; gate and up are not symmetric;
    gelu_tanh reproduces the GeGLU block; the MoE form reduces to one expert."""
    rng = np.random.default_rng(31)
    x = _bf16ish(rng, (5, 6))
    I = np.eye(6)
    Wg, Wu, Wd = _bf16ish(rng, (9, 6)), _bf16ish(rng, (9, 6)), _bf16ish(rng, (6, 9))
    for act in ("silu", "relu", "gelu_erf", "gelu_tanh", "none"):
        ref = np.vectorize(lambda v: _bf_act(v, act) * v)(x)
        _close(o.glu(x, I, I, I, act), ref, what=f"glu identity {act}")
        a = o.glu(x, Wg, Wu, Wd, act)
        _close(o.glu(x, Wg, 2 * Wu, Wd, act), 2 * a, what=f"glu linear in up {act}")
        if act != "none":
            assert np.max(np.abs(a - o.glu(x, Wu, Wg, Wd, act))) > 1e-3, act
    _close(o.glu(x, Wg, Wu, Wd, "gelu_tanh"), o.geglu(x, Wg, Wu, Wd), what="glu tanh == geglu")
    experts = [(_bf16ish(rng, (7, 6), 0.6), _bf16ish(rng, (7, 6), 0.6), _bf16ish(rng, (6, 7), 0.6))
               for _ in range(3)]
    for e in range(3):
        ids = np.full((5, 1), e, dtype=np.int32)
        _close(o.moe_glu(x, ids, np.ones((5, 1)), experts, "silu"), o.glu(x, *experts[e], "silu"),
               what=f"moe_glu top1 expert {e}")


def check_router(o):
    """The router against a brute-force loop, closed forms and invariants."""
    rng = np.random.default_rng(41)
    for (T, D, E, k) in [(5, 4, 3, 2), (7, 8, 8, 2), (4, 6, 5, 5), (6, 3, 4, 1)]:
        x = _bf16ish(rng, (T, D))
        Wr = _bf16ish(rng, (E, D), 0.7)
        ids, gw, lg = o.moe_router(x, Wr, k)
        bids, bgw = bf_router(x.tolist(), Wr.tolist(), k)
        assert ids.tolist() == bids, (ids.tolist(), bids)
        _close(gw, bgw, what=f"router weights {T}x{D}x{E} k{k}")
        _close(lg, bf_linear(x.tolist(), Wr.tolist(), None, "none"), what="router logits")
        _close(gw.sum(axis=1), np.ones(T), what="router weights sum to 1")
        # chosen in descending logit order, all distinct
        sel = np.take_along_axis(lg, ids, axis=1)
        assert np.all(np.diff(sel, axis=1) <= 0)
        assert all(len(set(r)) == k for r in ids.tolist())
    # two experts, both chosen: the weights are sigmoid(a - b) and sigmoid(b - a)
    lg = np.array([[0.3, -1.2], [2.0, 2.5]])
    ids, gw = o.route_topk(lg, 2)
    assert ids.tolist() == [[0, 1], [1, 0]]
    _close(gw[:, 0], 1.0 / (1.0 + np.exp(-np.array([1.5, 0.5]))), what="router sigmoid form")
    # top-1: weight exactly 1; ties go to the lower id
    ids, gw = o.route_topk(np.array([[1.0, 3.0, 3.0, 0.0]]), 1)
    assert ids.tolist() == [[1]] and gw.tolist() == [[1.0]]
    ids, _ = o.route_topk(np.array([[0.5, 0.5, 0.5, 0.5]]), 3)
    assert ids.tolist() == [[0, 1, 2]]
    # permuting the experts' router rows permutes the chosen ids
    x = _bf16ish(rng, (9, 8))
    Wr = _bf16ish(rng, (6, 8))
    p = rng.permutation(6)
    ids, gw, _ = o.moe_router(x, Wr, 2)
    ids_p, gw_p, _ = o.moe_router(x, Wr[p], 2)
    assert np.array_equal(p[ids_p], ids)
    _close(gw_p, gw, what="router permutation")


def check_transpose_worked_example(o):
    """The page's strides-and-views example: with W = M ([out=3, in=2]) and
    x = I_2, nn.Linear's y = x @ W.T is exactly the printed M.t()."""
    g = _load("transpose_view.json")
    M = np.array(g["M"], dtype=np.float64)
    assert list(M.shape) == g["M_shape"]
    y = o.linear(np.eye(2), M, None, "none")
    assert y.tolist() == g["Mt"], y.tolist()
    assert y.flatten().tolist() == g["Mt_flatten"]
    # a single input row e_k picks out column k of W, i.e. row k of M.t()
    for k in range(2):
        e = np.zeros((1, 2))
        e[0, k] = 1.0
        assert o.linear(e, M, None, "none")[0].tolist() == g["Mt"][k]


def check_linear_special_cases(o):
    rng = np.random.default_rng(11)
    x = _bf16ish(rng, (7, 16))
    # identity weight, no bias, no activation -> y == x bitwise
    y = o.linear(x, np.eye(16), None, "none")
    assert np.array_equal(y, x)
    # W = 0 -> y = act(b) exactly
    b = _bf16ish(rng, (5,))
    for act in ("none", "gelu_erf", "gelu_tanh"):
        y = o.linear(x, np.zeros((5, 16)), b, act)
        ref = np.array([[_bf_act(float(v), act) for v in b]] * 7)
        _close(y, ref, rtol=1e-15, atol=1e-16, what=f"W=0 {act}")
    # one-hot rows: W[n] = e_{p(n)} -> y[:, n] = x[:, p(n)]
    p = np.array([3, 0, 15, 7, 7, 2])
    W = np.zeros((6, 16))
    W[np.arange(6), p] = 1.0
    assert np.array_equal(o.linear(x, W, None, "none"), x[:, p])
    # bias adds (not subtracts), per output column
    b6 = np.arange(1, 7, dtype=np.float64)
    assert np.array_equal(o.linear(x, W, b6, "none"), x[:, p] + b6[None, :])


def check_mlp2_bias_pins(o):
    rng = np.random.default_rng(3)
    x = _bf16ish(rng, (4, 8))
    b1 = _bf16ish(rng, (8,))
    # W1 = 0 -> h = act(b1); W2 = I, b2 = 0 -> y = act(b1) for every row
    for act in ("gelu_erf", "gelu_tanh"):
        y = o.mlp2(x, np.zeros((8, 8)), b1, np.eye(8), np.zeros(8), act)
        ref = np.array([[_bf_act(float(v), act) for v in b1]] * 4)
        _close(y, ref, rtol=1e-15, atol=1e-16, what="mlp2 W1=0")
    # the activation sits between the layers only: W1 = I, b1 = 0, W2 = -I, b2 = c
    c = _bf16ish(rng, (8,))
    y = o.mlp2(x, np.eye(8), None, -np.eye(8), c, "gelu_tanh")
    ref = -np.vectorize(lambda v: _bf_act(v, "gelu_tanh"))(x) + c[None, :]
    _close(y, ref, what="mlp2 act placement")


def check_geglu_special_cases(o):
    rng = np.random.default_rng(13)
    x = _bf16ish(rng, (5, 6))
    I = np.eye(6)
    # Wg = Wu = Wd = I -> y = gelu_tanh(x) * x
    ref = np.vectorize(lambda v: _bf_act(v, "gelu_tanh") * v)(x)
    _close(o.geglu(x, I, I, I), ref, what="geglu identity")
    W = _bf16ish(rng, (9, 6))
    Wd = _bf16ish(rng, (6, 9))
    assert np.array_equal(o.geglu(x, W, np.zeros((9, 6)), Wd), np.zeros((5, 6)))   # Wu = 0
    assert np.array_equal(o.geglu(x, W, W, np.zeros((6, 9))), np.zeros((5, 6)))    # Wd = 0
    # the gate goes through gelu, the up projection does not
    Wg = _bf16ish(rng, (9, 6))
    Wu = _bf16ish(rng, (9, 6))
    a = o.geglu(x, Wg, Wu, Wd)
    b = o.geglu(x, Wu, Wg, Wd)
    assert np.max(np.abs(a - b)) > 1e-3
    # gate = identity path: Wg = I, Wu = I (dim=hidden), Wd = I: elementwise gelu(x)*x
    # (already covered); up only linear: doubling Wu doubles y
    _close(o.geglu(x, Wg, 2 * Wu, Wd), 2 * a, what="geglu linear in up")


def check_fused_equals_unfused(o):
    """Fusion changes launches and traffic, not the mathematics: the one-call
    forms equal their compositions of Linears."""
    rng = np.random.default_rng(17)
    x = _bf16ish(rng, (6, 8))
    W1, b1 = _bf16ish(rng, (12, 8), 0.4), _bf16ish(rng, (12,), 0.4)
    W2, b2 = _bf16ish(rng, (5, 12), 0.4), _bf16ish(rng, (5,), 0.4)
    for act in ("gelu_erf", "gelu_tanh"):
        _close(o.mlp2(x, W1, b1, W2, b2, act),
               o.linear(o.linear(x, W1, b1, act), W2, b2, "none"), what="mlp2 == 2 linears")
    Wg, Wu, Wd = _bf16ish(rng, (12, 8), 0.4), _bf16ish(rng, (12, 8), 0.4), _bf16ish(rng, (8, 12), 0.4)
    m = o.linear(x, Wg, None, "gelu_tanh") * o.linear(x, Wu, None, "none")
    _close(o.geglu(x, Wg, Wu, Wd), o.linear(m, Wd, None, "none"), what="geglu == composition")


def check_moe_invariants(o):
    rng = np.random.default_rng(21)
    T, D, H, E = 9, 6, 7, 4
    x = _bf16ish(rng, (T, D))
    experts = [(_bf16ish(rng, (H, D), 0.6), _bf16ish(rng, (H, D), 0.6), _bf16ish(rng, (D, H), 0.6))
               for _ in range(E)]
    # top_k = 1, every token to expert e with weight 1 -> dense geglu of expert e
    for e in range(E):
        ids = np.full((T, 1), e, dtype=np.int32)
        _close(o.moe_geglu(x, ids, np.ones((T, 1)), experts), o.geglu(x, *experts[e]),
               what=f"moe top1 expert {e}")
    # weights (w, 1-w) on the same expert twice -> dense expert (linearity)
    w = rng.random(T)
    ids = np.full((T, 2), 2, dtype=np.int32)
    _close(o.moe_geglu(x, ids, np.stack([w, 1 - w], 1), experts), o.geglu(x, *experts[2]),
           what="moe split weight")
    # permuting tokens permutes output rows
    ids = rng.integers(0, E, size=(T, 2)).astype(np.int32)
    gw = rng.random((T, 2))
    y = o.moe_geglu(x, ids, gw, experts)
    p = rng.permutation(T)
    _close(o.moe_geglu(x[p], ids[p], gw[p], experts), y[p], what="moe permutation")
    # swapping the two slots of a token changes nothing
    _close(o.moe_geglu(x, ids[:, ::-1], gw[:, ::-1], experts), y, what="moe slot order")
    # zero gate weight removes an expert's contribution
    gw0 = gw.copy()
    gw0[:, 1] = 0.0
    y1 = o.moe_geglu(x, ids[:, :1], gw[:, :1], experts)
    _close(o.moe_geglu(x, ids, gw0, experts), y1, what="moe zero weight")
    # an expert fetched lazily through a callable gives the same result
    _close(o.moe_geglu(x, ids, gw, lambda e: experts[e]), y, what="moe callable")


def _torch_e4m3(codes):
    """torch's own float8_e4m3fn conversion of raw codes, to float64."""
    import torch

    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_e4m3_decode(o):
    codes = np.arange(256, dtype=np.uint8)
    v = o.e4m3_decode(codes)
    ref = _torch_e4m3(codes)
    assert np.array_equal(np.isnan(v), np.isnan(ref)), "e4m3 NaN codes differ from torch's"
    fin = ~np.isnan(ref)
    assert np.array_equal(v[fin], ref[fin]), "e4m3 values differ from torch's float8_e4m3fn"
    assert np.array_equal(np.signbit(v[fin]), np.signbit(ref[fin])), "e4m3 signs of zero differ"
    # closed forms of the encoding (sign, 4-bit exponent with bias 7, 3-bit mantissa)
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, val in known.items():
        assert v[c] == val, f"e4m3 code {c:#04x}: {v[c]} != {val}"
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.signbit(v[0x80])
    # positive codes are ordered by value; the sign bit only negates
    assert np.all(np.diff(v[:0x7F]) > 0), "e4m3 positive codes not increasing"
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


def check_w8_layers(o):
    rng = np.random.default_rng(23)
    M, K, H, N = 3, 16, 7, 5
    x = _bf16ish(rng, (M, K))
    q1, q2 = _finite_codes(rng, (H, K)), _finite_codes(rng, (N, H))
    s1, s2 = rng.random(H) * 0.02 + 0.005, rng.random(N) * 0.02 + 0.005
    b1, b2 = _bf16ish(rng, (H,)), _bf16ish(rng, (N,))
    W1 = s1[:, None] * _torch_e4m3(q1)
    W2 = s2[:, None] * _torch_e4m3(q2)
    for act in ("none", "gelu_tanh", "silu"):
        _close(o.linear_w8(x, q1, s1, b1, act), bf_linear(x, W1, b1, act), what=f"linear_w8 {act}")
    h = bf_linear(x, W1, b1, "gelu_erf")
    _close(o.mlp2_w8(x, q1, s1, b1, q2, s2, b2, "gelu_erf"), bf_linear(h, W2, b2, "none"),
           what="mlp2_w8")
    # gated: D = K, H hidden
    qg, qu, qd = _finite_codes(rng, (H, K)), _finite_codes(rng, (H, K)), _finite_codes(rng, (K, H))
    sg, su, sd = (rng.random(H) * 0.02 + 0.005, rng.random(H) * 0.02 + 0.005,
                  rng.random(K) * 0.02 + 0.005)
    Wg, Wu, Wd = (sg[:, None] * _torch_e4m3(qg), su[:, None] * _torch_e4m3(qu),
                  sd[:, None] * _torch_e4m3(qd))
    for act in ("gelu_tanh", "silu"):
        _close(o.glu_w8(x, qg, sg, qu, su, qd, sd, act), bf_geglu(x, Wg, Wu, Wd, act),
               what=f"glu_w8 {act}")
    # the row scale is linear: doubling it doubles a bias-free output
    _close(o.linear_w8(x, q1, 2 * s1), 2 * o.linear_w8(x, q1, s1), what="linear_w8 scale")


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------
def _bf_act_grad(z: float, act: str, h: float = 1e-6) -> float:
    """Central difference of the pure-Python activation (libm), a derivative
    that shares nothing with the oracle's closed-form act_grad."""
    if act == "relu":        # the kink: PyTorch's convention, 0 at z <= 0
        return 1.0 if z > 0.0 else 0.0
    return (_bf_act(z + h, act) - _bf_act(z - h, act)) / (2.0 * h)


def bf_linear_bwd(x, W, b, act, dy):
    """Pure-Python loops: z, dz = dy * act'(z) by central differences, then
    dx[m][k] = sum_n dz W[n][k], dW[n][k] = sum_m dz x[m][k], db[n] = sum_m dz."""
    M, K, N = len(x), len(x[0]), len(W)
    dz = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = sum(float(x[m][k]) * float(W[n][k]) for k in range(K)) + (float(b[n]) if b is not None else 0.0)
            dz[m][n] = float(dy[m][n]) * _bf_act_grad(s, act)
    dx = [[sum(dz[m][n] * float(W[n][k]) for n in range(N)) for k in range(K)] for m in range(M)]
    dW = [[sum(dz[m][n] * float(x[m][k]) for m in range(M)) for k in range(K)] for n in range(N)]
    db = [sum(dz[m][n] for m in range(M)) for n in range(N)] if b is not None else None
    return dx, dW, db


def check_act_grad_closed_forms(o):
    """Derivatives at points with known values, and the identities that follow
    from the odd-part identity a(x) - a(-x) = x: a'(x) + a'(-x) = 1."""
    phi1 = math.exp(-0.5) / math.sqrt(2.0 * math.pi)          # standard normal density at 1
    assert abs(float(o.act_grad(1.0, "gelu_erf")) - (0.8413447460685429 + phi1)) < 1e-15
    assert abs(float(o.act_grad(-1.0, "gelu_erf")) - (0.15865525393145707 - phi1)) < 1e-15
    for act in ("gelu_erf", "gelu_tanh", "silu"):
        assert float(o.act_grad(0.0, act)) == 0.5
        assert abs(float(o.act_grad(40.0, act)) - 1.0) < 1e-12     # a(x) -> x
        assert abs(float(o.act_grad(-40.0, act))) < 1e-9           # a(x) -> 0
        x = np.linspace(-7, 7, 1401)
        _close(o.act_grad(x, act) + o.act_grad(-x, act), np.ones_like(x), rtol=1e-13, atol=1e-13,
               what=f"{act}: a'(x) + a'(-x) = 1")
    # gelu_tanh'(1) from its formula by hand: s = sigmoid(2a), a = sqrt(2/pi)(1.044715)
    a = math.sqrt(2.0 / math.pi) * 1.044715
    sg = 1.0 / (1.0 + math.exp(-2.0 * a))
    want = sg + 2.0 * sg * (1.0 - sg) * math.sqrt(2.0 / math.pi) * (1.0 + 3 * 0.044715)
    assert abs(float(o.act_grad(1.0, "gelu_tanh")) - want) < 1e-14
    # SiLU's minimum x* = -1.278464542761074 (SiLU(x*) = x* + 1): derivative 0 there
    assert abs(float(o.act_grad(-1.278464542761074, "silu"))) < 1e-14
    assert list(o.act_grad(np.array([-1.0, 0.0, 1e-30, 3.0]), "relu")) == [0.0, 0.0, 1.0, 1.0]
    assert list(o.act_grad(np.array([-2.0, 0.0, 5.0]), "none")) == [1.0, 1.0, 1.0]


def check_act_grad_finite_differences(o):
    """Central differences of the (separately pinned) forward activations."""
    z = np.concatenate([np.linspace(-8, 8, 641), [-3.3, -0.01, 0.013, 2.7]])
    h = 1e-6
    for act in ("none", "gelu_erf", "gelu_tanh", "silu"):
        fd = (o.activation(z + h, act) - o.activation(z - h, act)) / (2 * h)
        _close(o.act_grad(z, act), fd, rtol=1e-8, atol=1e-8, what=f"{act}' vs central differences")
    zr = z[np.abs(z) > 1e-3]
    fd = (o.activation(zr + h, "relu") - o.activation(zr - h, "relu")) / (2 * h)
    _close(o.act_grad(zr, "relu"), fd, rtol=1e-8, atol=1e-8, what="relu' vs central differences")


def check_act_grad_library(o):
    """torch autograd (float64) through F.gelu, F.gelu(tanh), F.silu, F.relu."""
    import torch
    import torch.nn.functional as F

    z = np.concatenate([np.linspace(-10, 10, 2001), [0.0, -1e-4, 1e-4]])
    fns = {"gelu_erf": F.gelu, "gelu_tanh": lambda t: F.gelu(t, approximate="tanh"), "silu": F.silu,
           "relu": F.relu, "none": lambda t: t * 1.0}
    for act, fn in fns.items():
        t = torch.from_numpy(z.copy()).requires_grad_(True)
        fn(t).sum().backward()
        _close(o.act_grad(z, act), t.grad.numpy(), rtol=1e-13, atol=1e-14, what=f"{act}' vs torch autograd")


def check_linear_bwd_bruteforce(o):
    rng = np.random.default_rng(77)
    for (M, K, N, act, bias) in [(1, 1, 1, "none", True), (2, 3, 5, "gelu_erf", True), (3, 4, 2, "gelu_tanh", False),
                                 (4, 5, 3, "silu", True), (3, 3, 3, "relu", True), (5, 2, 4, "gelu_tanh", True)]:
        x = _bf16ish(rng, (M, K))
        W = _bf16ish(rng, (N, K), 0.5)
        b = _bf16ish(rng, (N,), 0.3) if bias else None
        dy = _bf16ish(rng, (M, N))
        dx, dW, db = o.linear_bwd(x, W, b, act, dy)
        bx, bW, bb = bf_linear_bwd(x.tolist(), W.tolist(), None if b is None else b.tolist(), act, dy.tolist())
        _close(dx, bx, rtol=1e-8, atol=1e-9, what=f"linear_bwd dx {M}x{K}x{N} {act}")
        _close(dW, bW, rtol=1e-8, atol=1e-9, what=f"linear_bwd dW {M}x{K}x{N} {act}")
        if bias:
            _close(db, bb, rtol=1e-8, atol=1e-9, what=f"linear_bwd db {act}")
        else:
            assert db is None


def _torch_grads(fn, arrays, dy):
    import torch

    ts = [None if a is None else torch.from_numpy(np.array(a, dtype=np.float64)).requires_grad_(True) for a in arrays]
    out = fn(*ts)
    out.backward(torch.from_numpy(np.asarray(dy, dtype=np.float64)))
    return [None if t is None else t.grad.numpy() for t in ts]


_TORCH_ACT = {
    "none": lambda t: t,
    "gelu_erf": lambda t: __import__("torch").nn.functional.gelu(t),
    "gelu_tanh": lambda t: __import__("torch").nn.functional.gelu(t, approximate="tanh"),
    "relu": lambda t: __import__("torch").nn.functional.relu(t),
    "silu": lambda t: __import__("torch").nn.functional.silu(t),
}


def check_backward_library(o):
    """linear_bwd, mlp2_bwd and glu_bwd against torch autograd in float64 (the
    forward written with torch's F.linear and activations)."""
    import torch.nn.functional as F

    rng = np.random.default_rng(5)
    M, K, H, N = 7, 12, 10, 6
    x = _bf16ish(rng, (M, K))
    for act in ("none", "gelu_erf", "gelu_tanh", "relu", "silu"):
        W = _bf16ish(rng, (N, K), 0.4)
        b = _bf16ish(rng, (N,), 0.2)
        dy = _bf16ish(rng, (M, N))
        gx, gW, gb = _torch_grads(lambda x_, W_, b_: _TORCH_ACT[act](F.linear(x_, W_, b_)), [x, W, b], dy)
        dx, dW, db = o.linear_bwd(x, W, b, act, dy)
        for a, r, n in ((dx, gx, "dx"), (dW, gW, "dW"), (db, gb, "db")):
            _close(a, r, rtol=1e-12, atol=1e-13, what=f"linear_bwd {n} {act} vs autograd")
        W1 = _bf16ish(rng, (H, K), 0.4)
        b1 = _bf16ish(rng, (H,), 0.2)
        W2 = _bf16ish(rng, (N, H), 0.4)
        b2 = _bf16ish(rng, (N,), 0.2)
        ref = _torch_grads(lambda x_, a_, c_, d_, e_: F.linear(_TORCH_ACT[act](F.linear(x_, a_, c_)), d_, e_),
                           [x, W1, b1, W2, b2], dy)
        got = o.mlp2_bwd(x, W1, b1, W2, b2, act, dy)
        for a, r, n in zip(got, [ref[0], ref[1], ref[2], ref[3], ref[4]], ("dx", "dW1", "db1", "dW2", "db2")):
            _close(a, r, rtol=1e-12, atol=1e-13, what=f"mlp2_bwd {n} {act} vs autograd")
        D = K
        Wg = _bf16ish(rng, (H, D), 0.4)
        Wu = _bf16ish(rng, (H, D), 0.4)
        Wd = _bf16ish(rng, (D, H), 0.4)
        dyd = _bf16ish(rng, (M, D))
        ref = _torch_grads(lambda x_, g_, u_, d_: F.linear(_TORCH_ACT[act](F.linear(x_, g_)) * F.linear(x_, u_), d_),
                           [x, Wg, Wu, Wd], dyd)
        got = o.glu_bwd(x, Wg, Wu, Wd, act, dyd)
        for a, r, n in zip(got, ref, ("dx", "dWg", "dWu", "dWd")):
            _close(a, r, rtol=1e-12, atol=1e-13, what=f"glu_bwd {n} {act} vs autograd")


def check_glu_bwd_directional(o):
    """<dy, glu(theta + e v) - glu(theta - e v)> / 2e = <grad, v> for a random
    direction v of each input (the forward glu is pinned separately)."""
    rng = np.random.default_rng(11)
    M, D, H = 5, 6, 8
    x = _bf16ish(rng, (M, D))
    Wg, Wu = _bf16ish(rng, (H, D), 0.5), _bf16ish(rng, (H, D), 0.5)
    Wd = _bf16ish(rng, (D, H), 0.5)
    dy = _bf16ish(rng, (M, D))
    e = 1e-6
    for act in ("gelu_tanh", "gelu_erf", "silu"):
        grads = o.glu_bwd(x, Wg, Wu, Wd, act, dy)
        args = [x, Wg, Wu, Wd]
        for i in range(4):
            v = rng.standard_normal(args[i].shape)
            plus = [a + e * v if j == i else a for j, a in enumerate(args)]
            minus = [a - e * v if j == i else a for j, a in enumerate(args)]
            fd = np.sum(dy * (o.glu(*plus, act) - o.glu(*minus, act))) / (2 * e)
            got = np.sum(grads[i] * v)
            assert abs(fd - got) <= 1e-7 * max(1.0, abs(got)), (act, i, fd, got)


def check_glu_bwd_sampled(o):
    """The sampled backward equals the full backward restricted to its rows
    and hidden units (it is a restriction of the same definitions)."""
    rng = np.random.default_rng(21)
    M, D, H = 9, 8, 12
    x, dy = _bf16ish(rng, (M, D)), _bf16ish(rng, (M, D))
    Wg, Wu, Wd = _bf16ish(rng, (H, D), 0.5), _bf16ish(rng, (H, D), 0.5), _bf16ish(rng, (D, H), 0.5)
    rows, hidden = np.array([0, 3, 8]), np.array([1, 2, 7, 11])
    for act in ("gelu_tanh", "silu"):
        full = o.glu_bwd(x, Wg, Wu, Wd, act, dy)
        got = o.glu_bwd_sampled(x, Wg, Wu, Wd, act, dy, rows, hidden)
        _close(got[0], full[0][rows], rtol=1e-13, atol=1e-14, what="sampled dx")
        _close(got[1], full[1][hidden], rtol=1e-13, atol=1e-14, what="sampled dWg")
        _close(got[2], full[2][hidden], rtol=1e-13, atol=1e-14, what="sampled dWu")
        _close(got[3], full[3][:, hidden], rtol=1e-13, atol=1e-14, what="sampled dWd")


def check_backward_special_cases(o):
    """Identity weights: dx = dy * act'(x) with W = I; W = 0 gives dx = 0 and
    dW = dz^T x with dz = dy * act'(b); the gated block's gradient through
    Wu = 0 vanishes for dx and dWg (m = 0 makes dWd = 0 too)."""
    rng = np.random.default_rng(3)
    M, K = 6, 5
    x = _bf16ish(rng, (M, K))
    dy = _bf16ish(rng, (M, K))
    I = np.eye(K)
    for act in ("gelu_erf", "silu"):
        dx, dW, db = o.linear_bwd(x, I, None, act, dy)
        _close(dx, dy * o.act_grad(x, act), rtol=1e-14, atol=1e-15, what=f"identity W dx {act}")
        b = _bf16ish(rng, (K,), 0.5)
        dx, dW, db = o.linear_bwd(x, np.zeros((K, K)), b, act, dy)
        dz = dy * o.act_grad(np.broadcast_to(b, (M, K)), act)
        _close(dx, np.zeros_like(dx), what="W=0 dx")
        _close(dW, dz.T @ x, rtol=1e-14, atol=1e-15, what="W=0 dW")
        _close(db, dz.sum(axis=0), rtol=1e-14, atol=1e-15, what="W=0 db")
    H = 4
    Wg = _bf16ish(rng, (H, K), 0.5)
    Wd = _bf16ish(rng, (K, H), 0.5)
    dx, dWg, dWu, dWd = o.glu_bwd(x, Wg, np.zeros((H, K)), Wd, "gelu_tanh", dy)
    for a, n in ((dx, "dx"), (dWg, "dWg"), (dWd, "dWd")):
        _close(a, np.zeros_like(a), what=f"Wu=0 {n}")
    assert np.max(np.abs(dWu)) > 1e-3


ALL_CHECKS = [
    check_act_grad_closed_forms,
    check_act_grad_finite_differences,
    check_act_grad_library,
    check_linear_bwd_bruteforce,
    check_backward_library,
    check_glu_bwd_directional,
    check_backward_special_cases,
    check_glu_bwd_sampled,
    check_linear_bruteforce,
    check_mlp2_bruteforce,
    check_geglu_bruteforce,
    check_moe_bruteforce,
    check_gelu_library,
    check_gelu_closed_forms,
    check_silu_relu_closed_forms,
    check_transpose_worked_example,
    check_linear_special_cases,
    check_mlp2_bias_pins,
    check_geglu_special_cases,
    check_glu_special_cases,
    check_fused_equals_unfused,
    check_moe_invariants,
    check_router,
    check_e4m3_decode,
    check_w8_layers,
]
