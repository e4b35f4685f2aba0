"""Plain fp64 CPU oracle for the fused transformer feed-forward path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library never imports it, shares no code with it, and must never fall back to it.

Every function computes the plain definition the pages give, in float64, on the
caller's (bf16-valued) inputs, with no rounding of any intermediate and no
blocking, fusion or reordering beyond a library matmul.  Fusion on the GPU
changes launches and memory traffic, never the mathematics (ainews.cool
"PyTorch fused MLP efficiency", section "technical deep dive": the fused form
loads X once and computes the same W1*X+b1 -> activation -> W2*(.)+b2 chain;
"Profiling in PyTorch (Part 2): From nn.Linear to a Fused MLP", section "The
fused Triton kernel": the fused kernel computes gelu(g)*u exactly as eager does).

Readings taken where the pages are silent (each is listed in the design doc):
  * GELU formulas: the pages name ``F.gelu(g, approximate="tanh")`` and plain
    "GELU" but print no formula; we take PyTorch's documented definitions
    (Hendrycks & Gimpel): exact  z*Phi(z) = z/2 * erfc(-z/sqrt 2)  and tanh
    z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))).
  * Intermediates (h, g, u, m) are NOT rounded: the oracle is the plain
    definition; the GPU's bf16 rounding of h/m is absorbed by the tolerance.
  * MoE: y[t] = sum_j gate_w[t, j] * geglu_{expert_ids[t, j]}(x[t]); duplicate
    expert ids within a token simply add.
  * ReLU is max(z, 0) (ainews.cool "technical deep dive" names ReLU for the
    two-layer MLP).  SiLU, z * sigmoid(z), is the gate activation of SwiGLU;
    the pages name three-Linear MLP blocks (LLaMA-3, Mixtral experts) without
    naming their gate activation, so the gated block takes it as an argument.

  * Backward pass: the pages profile the forward only; Liger's fused gelu*mul
    ("Profiling in PyTorch (Part 2)", section "Let's use hand tuned kernels":
    LigerGELUMulFunction) is an autograd Function, so its backward exists but
    is not described.  The gradients here are the chain rule applied to the
    forward definitions above, with the derivative of each activation written
    out from its formula (act_grad), and nothing rounded.

  * FP8 weights (decode): the pages only note that decode is bound by the
    weight bytes; the format is the OCP 8-bit floating point E4M3 encoding
    ("e4m3fn") with one scale per output row, and the functions here
    dequantise exactly and then call the bf16 definitions above.

Pins: tests/test_oracle_pins.py checks every function here against brute-force
loops, library routines, closed forms, a printed worked example and invariants.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc as _erfc
from scipy.special import expit as _expit

__all__ = [
    "ACTS",
    "gelu_erf",
    "gelu_tanh",
    "relu",
    "silu",
    "activation",
    "linear",
    "mlp2",
    "geglu",
    "glu",
    "moe_geglu",
    "moe_glu",
    "route_topk",
    "moe_router",
    "e4m3_decode",
    "dequant_w8",
    "linear_w8",
    "mlp2_w8",
    "glu_w8",
    "act_grad",
    "linear_bwd",
    "mlp2_bwd",
    "glu_bwd",
    "glu_bwd_sampled",
]

ACTS = ("none", "gelu_erf", "gelu_tanh", "relu", "silu")

_SQRT_HALF = np.sqrt(0.5)
_SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)
_GELU_TANH_CUBIC = 0.044715


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def gelu_erf(z):
    """Exact GELU, z * Phi(z), with Phi the standard normal CDF.

    The ainews.cool article ("technical deep dive" / "benchmark data") names a
    plain "GELU" activation for its 4096-wide MLP; PyTorch's default GELU is the
    exact one.  Phi(z) = erfc(-z/sqrt(2)) / 2, which keeps full relative accuracy
    in the negative tail where 1 + erf(.) would cancel.
    """
    z = _f64(z)
    return 0.5 * z * _erfc(-z * _SQRT_HALF)


def gelu_tanh(z):
    """Tanh-approximated GELU, as named by ``F.gelu(g, approximate="tanh")``.

    "Profiling in PyTorch (Part 2)", section "Stacking three Linears: the MLP"
    (the SimpleGeGLUMLP forward).  Formula: PyTorch's documented definition,
    z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))).
    """
    z = _f64(z)
    inner = _SQRT_2_OVER_PI * (z + _GELU_TANH_CUBIC * z * z * z)
    return 0.5 * z * (1.0 + np.tanh(inner))


def relu(z):
    """ReLU, max(z, 0): the activation of the two-layer MLP in ainews.cool
    "PyTorch fused MLP efficiency", section "technical deep dive"."""
    z = _f64(z)
    return np.where(z > 0.0, z, 0.0)


def silu(z):
    """SiLU (swish), z * sigmoid(z), with sigmoid from scipy's expit (stable in
    both tails).  The gate activation of SwiGLU blocks; see the module notes
    for why it is offered."""
    z = _f64(z)
    return z * _expit(z)


def activation(z, act: str):
    """The epilogue activation selected by name: none, gelu_erf, gelu_tanh,
    relu or silu.

    "Profiling in PyTorch (Part 2)", section "Why are there no separate mul and
    add kernels?": applying an activation is a classic GEMM epilogue.
    """
    if act == "none":
        return _f64(z)
    if act == "gelu_erf":
        return gelu_erf(z)
    if act == "gelu_tanh":
        return gelu_tanh(z)
    if act == "relu":
        return relu(z)
    if act == "silu":
        return silu(z)
    raise ValueError(f"unknown activation {act!r}; expected one of {ACTS}")


def linear(x, W, b=None, act: str = "none"):
    """y = act(x @ W^T + b), W stored [out, in] as nn.Linear stores it.

    "Profiling in PyTorch (Part 2)", section "From matmul-add to Linear"
    (y = x @ w.T + b) and section "Why are there no separate mul and add
    kernels?" (addmm: out = x @ weight.T + bias; bias/activation are the
    epilogue).  x is [M, K], W is [N, K], b is [N] or None; returns [M, N].
    """
    x = _f64(x)
    W = _f64(W)
    if x.ndim != 2 or W.ndim != 2 or x.shape[1] != W.shape[1]:
        raise ValueError(f"shape mismatch: x{x.shape} W{W.shape}")
    z = x @ W.T
    if b is not None:
        b = _f64(b)
        if b.shape != (W.shape[0],):
            raise ValueError(f"bias shape {b.shape} != ({W.shape[0]},)")
        z = z + b[None, :]
    return activation(z, act)


def mlp2(x, W1, b1, W2, b2, act: str):
    """Two-layer MLP: y = act(x W1^T + b1) W2^T + b2 (activation between layers only).

    ainews.cool "PyTorch fused MLP efficiency", section "technical deep dive":
    launch 1 computes W1*X+b1, launch 2 applies the activation, launch 3
    computes W2*(act(W1*X+b1))+b2; the fused form does the same chain in one
    launch.  x [M,K], W1 [H,K], b1 [H]|None, W2 [N,H], b2 [N]|None.
    """
    h = linear(x, W1, b1, act)
    return linear(h, W2, b2, "none")


def geglu(x, Wg, Wu, Wd):
    """GeGLU feed-forward: y = (gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T, no biases.

    "Profiling in PyTorch (Part 2)", section "Stacking three Linears: the MLP"
    (SimpleGeGLUMLP: gate_proj, up_proj, down_proj all bias=False;
    g = gate(x), u = up(x), h = gelu(g, tanh), m = h * u, y = down(m)).
    x [M,D], Wg/Wu [H,D], Wd [D,H].
    """
    g = linear(x, Wg)
    u = linear(x, Wu)
    m = gelu_tanh(g) * u
    return linear(m, Wd)


def glu(x, Wg, Wu, Wd, gate_act: str):
    """Gated feed-forward block with a named gate activation:
    y = (gate_act(x Wg^T) * (x Wu^T)) Wd^T, no biases.

    The GeGLU block above with its gelu replaced by gate_act ("silu": SwiGLU,
    "relu": ReGLU, "none": bilinear).  x [M,D], Wg/Wu [H,D], Wd [D,H].
    """
    g = linear(x, Wg)
    u = linear(x, Wu)
    m = activation(g, gate_act) * u
    return linear(m, Wd)


def moe_glu(x, expert_ids, gate_w, expert_weights, gate_act: str):
    """moe_geglu with each expert the gated block glu(..., gate_act)."""
    x = _f64(x)
    ids = np.asarray(expert_ids)
    w = _f64(gate_w)
    if ids.shape != w.shape or ids.ndim != 2 or ids.shape[0] != x.shape[0]:
        raise ValueError(f"routes shape mismatch: ids{ids.shape} w{w.shape} x{x.shape}")
    get = expert_weights if callable(expert_weights) else (lambda e: expert_weights[e])
    y = np.zeros_like(x)
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        Wg, Wu, Wd = get(int(e))
        ye = glu(x[tok], Wg, Wu, Wd, gate_act)
        np.add.at(y, tok, w[tok, slot][:, None] * ye)
    return y


def route_topk(logits, top_k: int):
    """Top-k routes from given router logits [T, E]: the top_k experts of each
    token by logit, largest first, a tie going to the lower expert id (a stable
    sort of the negated logits), and gate weights = softmax over those top_k
    logits.  Returns (ids int32 [T, top_k], gate_w float64 [T, top_k]).

    The decision is taken in the precision of the logits handed in: the tests
    hand in the kernel's own fp32 logits to check its integer ids exactly.
    """
    lg = _f64(logits)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(lg, ids, axis=1)
    e = np.exp(sel - sel[:, :1])
    return ids.astype(np.int32), e / e.sum(axis=1, keepdims=True)


def moe_router(x, Wr, top_k: int):
    """The MoE router: logits = x Wr^T, then route_topk.  ainews.cool "PyTorch
    fused MLP efficiency", section "architectural impact", routes each token to
    several experts; it gives no router formula, and this is the plain linear
    router with a softmax over the chosen logits.  x [T,D], Wr [E,D].
    Returns (ids, gate_w, logits)."""
    logits = linear(x, Wr)
    ids, gw = route_topk(logits, top_k)
    return ids, gw, logits


def moe_geglu(x, expert_ids, gate_w, expert_weights):
    """Top-k routed mixture of GeGLU experts with a weighted combine.

    ainews.cool "PyTorch fused MLP efficiency", section "architectural impact":
    an MoE layer routes each token to several experts, each expert being an
    MLP.  Here each expert is the GeGLU block above and
        y[t] = sum_j gate_w[t, j] * geglu_{expert_ids[t, j]}(x[t]).

    x [T,D]; expert_ids int [T,k]; gate_w [T,k];
    expert_weights: a sequence (or callable e -> (Wg, Wu, Wd)) of per-expert
    weights, fetched one expert at a time so only one expert's fp64 copy is
    resident.  Experts that receive no token are never fetched.
    """
    x = _f64(x)
    ids = np.asarray(expert_ids)
    w = _f64(gate_w)
    if ids.shape != w.shape or ids.ndim != 2 or ids.shape[0] != x.shape[0]:
        raise ValueError(f"routes shape mismatch: ids{ids.shape} w{w.shape} x{x.shape}")
    get = expert_weights if callable(expert_weights) else (lambda e: expert_weights[e])
    # A GeGLU expert maps dim -> dim, so y has x's shape.
    y = np.zeros_like(x)
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        Wg, Wu, Wd = get(int(e))
        ye = geglu(x[tok], Wg, Wu, Wd)
        # np.add.at: a token routed twice to the same expert adds both terms.
        np.add.at(y, tok, w[tok, slot][:, None] * ye)
    return y


# ---------------------------------------------------------------------------
# FP8 (E4M3) weights
# ---------------------------------------------------------------------------
def e4m3_decode(codes):
    """Value of each OCP FP8 E4M3 ("e4m3fn") code, as float64.

    The OCP 8-bit floating point specification (OFP8), format E4M3: bit 7 the
    sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the mantissa m.
    e = 0: subnormal, m/8 * 2^(1-7); otherwise (1 + m/8) * 2^(e-7).  There are
    no infinities; e = 15 with m = 7 is NaN (0x7F and 0xFF), so the largest
    finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = sign * mag
    return np.where((e == 15) & (c & 7 == 7), np.nan, v)


def dequant_w8(Wq, scale):
    """W[n, k] = scale[n] * e4m3(Wq[n, k]): per-output-row scaled FP8 weights."""
    Wq = np.asarray(Wq, dtype=np.uint8)
    scale = _f64(scale)
    if Wq.ndim != 2 or scale.shape != (Wq.shape[0],):
        raise ValueError(f"scale shape {scale.shape} does not match weights {Wq.shape}")
    return scale[:, None] * e4m3_decode(Wq)


def linear_w8(x, Wq, scale, b=None, act: str = "none"):
    """linear() on the dequantised FP8 weights: act(x W^T + b), W = scale * e4m3(Wq)."""
    return linear(x, dequant_w8(Wq, scale), b, act)


def mlp2_w8(x, W1q, s1, b1, W2q, s2, b2, act: str):
    """mlp2() on dequantised FP8 weights W1 = s1 * e4m3(W1q), W2 = s2 * e4m3(W2q)."""
    return mlp2(x, dequant_w8(W1q, s1), b1, dequant_w8(W2q, s2), b2, act)


def glu_w8(x, Wgq, sg, Wuq, su, Wdq, sd, gate_act: str):
    """glu() on dequantised FP8 weights (gate, up and down each with row scales)."""
    return glu(x, dequant_w8(Wgq, sg), dequant_w8(Wuq, su), dequant_w8(Wdq, sd), gate_act)


# ---------------------------------------------------------------------------
# Backward pass (gradients of the forward definitions above)
# ---------------------------------------------------------------------------
def act_grad(z, act: str):
    """d act(z) / dz, from each activation's formula:
      none       1
      gelu_erf   Phi(z) + z phi(z), phi the standard normal density
      gelu_tanh  (1 + tanh a)/2 + z/2 (1 - tanh^2 a) sqrt(2/pi) (1 + 3*0.044715 z^2),
                 a = sqrt(2/pi) (z + 0.044715 z^3)
      relu       1 where z > 0, else 0 (0 at z = 0, PyTorch's convention)
      silu       sigmoid(z) (1 + z (1 - sigmoid(z)))
    """
    z = _f64(z)
    if act == "none":
        return np.ones_like(z)
    if act == "gelu_erf":
        phi = np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
        return 0.5 * _erfc(-z * _SQRT_HALF) + z * phi
    if act == "gelu_tanh":
        a = _SQRT_2_OVER_PI * (z + _GELU_TANH_CUBIC * z * z * z)
        t = np.tanh(a)
        da = _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_TANH_CUBIC * z * z)
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * da
    if act == "relu":
        return np.where(z > 0.0, 1.0, 0.0)
    if act == "silu":
        sg = _expit(z)
        return sg * (1.0 + z * (1.0 - sg))
    raise ValueError(f"unknown activation {act!r}; expected one of {ACTS}")


def linear_bwd(x, W, b, act: str, dy):
    """Gradients of y = act(x W^T + b) (linear above) for an upstream gradient
    dy [M, N]:  z = x W^T + b,  dz = dy * act'(z),
        dx = dz W  [M, K],   dW = dz^T x  [N, K],   db = sum_m dz  [N] (None
    without a bias).  Returns (dx, dW, db)."""
    x = _f64(x)
    W = _f64(W)
    dy = _f64(dy)
    z = x @ W.T
    if b is not None:
        z = z + _f64(b)[None, :]
    if dy.shape != z.shape:
        raise ValueError(f"dy shape {dy.shape} != {z.shape}")
    dz = dy * act_grad(z, act)
    return dz @ W, dz.T @ x, (dz.sum(axis=0) if b is not None else None)


def mlp2_bwd(x, W1, b1, W2, b2, act: str, dy):
    """Gradients of y = act(x W1^T + b1) W2^T + b2 (mlp2 above): the second
    layer's backward on h = act(x W1^T + b1), then the first layer's with the
    gradient reaching h.  Returns (dx, dW1, db1, dW2, db2)."""
    h = linear(x, W1, b1, act)
    dh, dW2, db2 = linear_bwd(h, W2, b2, "none", dy)
    dx, dW1, db1 = linear_bwd(x, W1, b1, act, dh)
    return dx, dW1, db1, dW2, db2


def glu_bwd(x, Wg, Wu, Wd, gate_act: str, dy):
    """Gradients of the gated block y = (gate_act(x Wg^T) * (x Wu^T)) Wd^T
    (glu above; gelu_tanh gives GeGLU) for an upstream gradient dy [M, D]:
        g = x Wg^T, u = x Wu^T, m = act(g) * u,
        dWd = dy^T m,   dm = dy Wd,
        dg = dm * u * act'(g),   du = dm * act(g),
        dx = dg Wg + du Wu,   dWg = dg^T x,   dWu = du^T x.
    Returns (dx, dWg, dWu, dWd)."""
    x = _f64(x)
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    dy = _f64(dy)
    g = x @ Wg.T
    u = x @ Wu.T
    a = activation(g, gate_act)
    m = a * u
    dWd = dy.T @ m
    dm = dy @ Wd
    dg = dm * u * act_grad(g, gate_act)
    du = dm * a
    return dg @ Wg + du @ Wu, dg.T @ x, du.T @ x, dWd


def glu_bwd_sampled(x, Wg, Wu, Wd, gate_act: str, dy, rows, hidden):
    """Exactly the entries glu_bwd returns for a subset, without the full
    products (for full-size shapes):
      dx[rows]          needs dg, du of those token rows only (all hidden units);
      dWg[hidden], dWu[hidden], dWd[:, hidden]
                        need g, u, dm of those hidden units only (all tokens).
    Same definitions as glu_bwd; returns (dx_rows, dWg_h, dWu_h, dWd_h)."""
    x = _f64(x)
    Wg, Wu, Wd = _f64(Wg), _f64(Wu), _f64(Wd)
    dy = _f64(dy)
    rows = np.asarray(rows)
    hidden = np.asarray(hidden)
    # token rows: every hidden unit
    xr, dyr = x[rows], dy[rows]
    g, u = xr @ Wg.T, xr @ Wu.T
    a = activation(g, gate_act)
    dm = dyr @ Wd
    dx = (dm * u * act_grad(g, gate_act)) @ Wg + (dm * a) @ Wu
    # hidden units: every token
    g = x @ Wg[hidden].T
    u = x @ Wu[hidden].T
    a = activation(g, gate_act)
    dm = dy @ Wd[:, hidden]
    dg = dm * u * act_grad(g, gate_act)
    du = dm * a
    return dx, dg.T @ x, du.T @ x, dy.T @ (a * u)
