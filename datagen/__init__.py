"""Seeded synthetic inputs for the fused feed-forward workloads.

This module is the only code shared by the oracle side (tests) and the GPU
side (tests, bench).  It holds no arithmetic of the method itself: it draws
random numbers, rounds them to bf16 (round-to-nearest-even, the rounding the
inputs of both sides see), and describes the workload shapes and their
algorithmic FLOP / byte counts.

Workload shapes come from the pages where they give them:
  * Linear 32 -> 64 at batch 1024: "Profiling in PyTorch (Part 2)", section
    "From matmul-add to Linear" (the profiled command line).
  * 4096 -> 4096 -> 4096 GELU MLP at batch 1: ainews.cool "PyTorch fused MLP
    efficiency", section "benchmark data".
  * GeGLU dim 768 / hidden 3072 over batch 64 x seq 128 = 8192 tokens:
    "Profiling in PyTorch (Part 2)", sections "Stacking three Linears: the MLP"
    and "Why are there two kinds of GEMM kernels?".
The 8192/28672 FFN and the 8-expert top-2 MoE are the LLaMA-3-70B- and
Mixtral-shaped workloads the ainews.cool article alludes to ("technical deep
dive", "architectural impact").

Random streams: every tensor has its own PCG64 stream keyed by
(seed, workload family, tensor name), so the weights of a workload do not
depend on its token count.  Values are drawn in float32 and rounded to bf16.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "rne_bf16",
    "bf16_to_f32",
    "rng_for",
    "normal_bf16",
    "uniform_bf16",
    "make_inputs",
    "make_routes",
    "expert_weights",
    "router_weights",
]


# ---------------------------------------------------------------------------
# bf16 encoding (input preparation only)
# ---------------------------------------------------------------------------
def rne_bf16(a) -> np.ndarray:
    """float32 -> raw bf16 bits (uint16), round-to-nearest, ties to even.

    Finite inputs only (values beyond the bf16 range round to +-inf).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """raw bf16 bits (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------
def rng_for(seed: int, family: str, name: str) -> np.random.Generator:
    """An independent PCG64 stream for one tensor of one workload family."""
    key = zlib.crc32(f"{family}/{name}".encode())
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), key])))


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) drawn in float32, rounded to bf16 bits."""
    return rne_bf16(rng.standard_normal(size=shape, dtype=np.float32))


def uniform_bf16(rng: np.random.Generator, shape, bound: float) -> np.ndarray:
    """U(-bound, bound) drawn in float32, rounded to bf16 bits."""
    a = rng.random(size=shape, dtype=np.float32)
    a = (a * np.float32(2.0 * bound) - np.float32(bound)).astype(np.float32)
    return rne_bf16(a)


def e4m3_weights(rng: np.random.Generator, rows: int, cols: int, bound: float):
    """FP8 weights for the decode calls: E4M3 codes [rows, cols] (uint8) and one
    fp32 scale per row.  The codes are torch's float8_e4m3fn rounding of
    U(-224, 224) draws; scale[n] = bound / 224 * U(0.75, 1.25), so the
    represented weights scale[n] * e4m3(q) spread over about U(-bound, bound).
    NaN codes never occur (|draw| < 448)."""
    import torch

    u = rng.random(size=(rows, cols), dtype=np.float32) * np.float32(448.0) - np.float32(224.0)
    q = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    s = (np.float32(bound / 224.0) * (np.float32(0.75) + np.float32(0.5) * rng.random(rows, dtype=np.float32)))
    return q, s.astype(np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """One feed-forward workload.  All tensors row-major; weights [out, in].

    op: "mlp2" (x[M,K] -> W1[H,K],b1 -> act -> W2[N,H],b2),
        "geglu" (x[M,D]; Wg,Wu[H,D]; Wd[D,H]),
        "moe" (x[T,D]; E experts of geglu; top_k routes per token), or
        "route" (x[T,D]; router Wr[E,D] -> top_k ids and gate weights).
    """

    name: str
    op: str
    M: int              # tokens (T for moe)
    K: int              # input dim (D for geglu/moe)
    H: int              # hidden dim
    N: int              # output dim (D for geglu/moe)
    act: str = "none"   # activation between the layers (mlp2 only)
    bias: bool = False
    w1_bound: float = 0.0
    w2_bound: float = 0.0
    b1_bound: float = 0.0
    b2_bound: float = 0.0
    E: int = 0
    top_k: int = 0
    family: str = ""
    notes: str = field(default="", compare=False)

    # -- algorithmic work (what the method must do, once) -------------------
    @property
    def flops(self) -> int:
        """sum of 2*M*K*N over the method's GEMMs (epilogue flops excluded)."""
        if self.op == "mlp2":
            return 2 * self.M * (self.K * self.H + self.H * self.N)
        if self.op == "geglu":
            return 2 * self.M * 3 * self.K * self.H
        if self.op == "moe":
            return 2 * self.M * self.top_k * 3 * self.K * self.H
        if self.op == "route":
            return 2 * self.M * self.K * self.E
        if self.op == "glu_bwd":
            # dm = dy Wd, dx = dg Wg + du Wu, dWd = dy^T m, dWg = dg^T x, dWu = du^T x
            return 2 * self.M * 6 * self.K * self.H
        raise ValueError(self.op)

    @property
    def weight_bytes(self) -> int:
        if self.op == "mlp2":
            wb = 2 * (self.H * self.K + self.N * self.H)
            if self.bias:
                wb += 2 * (self.H + self.N)
            return wb
        if self.op in ("geglu", "glu_bwd"):
            return 2 * 3 * self.K * self.H
        if self.op == "moe":
            return self.E * 2 * 3 * self.K * self.H
        if self.op == "route":
            return 2 * self.E * self.K
        raise ValueError(self.op)

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: weights (+biases) + x + y (+ routes), each once."""
        b = self.weight_bytes + 2 * self.M * self.K + 2 * self.M * self.N
        if self.op == "glu_bwd":   # + the weight gradients written and dy read
            b += self.weight_bytes + 2 * self.M * self.N
        if self.op in ("moe", "route"):
            b += self.M * self.top_k * (4 + 4)  # int32 ids + fp32 gate weights
        return b


def _tiny() -> Workload:
    return Workload(
        name="tiny_mlp2_1024x32-64-32", op="mlp2", M=1024, K=32, H=64, N=32,
        act="gelu_tanh", bias=True,
        w1_bound=1 / math.sqrt(32), b1_bound=1 / math.sqrt(32),
        w2_bound=1 / math.sqrt(64), b2_bound=1 / math.sqrt(64), family="tiny")


def _decode(M: int) -> Workload:
    return Workload(
        name=f"decode_mlp2_4096x4096x4096_M{M}", op="mlp2", M=M, K=4096, H=4096,
        N=4096, act="gelu_erf", bias=True,
        w1_bound=1 / 64, w2_bound=1 / 64, b1_bound=1 / 64, b2_bound=1 / 64,
        family="decode")


def _geglu768() -> Workload:
    return Workload(
        name="geglu_8192tok_768-3072", op="geglu", M=8192, K=768, H=3072, N=768,
        w1_bound=1 / math.sqrt(768), w2_bound=1 / math.sqrt(3072), family="geglu768")


def _large(T: int) -> Workload:
    return Workload(
        name=f"geglu_large_8192-28672_T{T}", op="geglu", M=T, K=8192, H=28672, N=8192,
        w1_bound=1 / math.sqrt(8192), w2_bound=1 / math.sqrt(28672), family="large")


def _moe(T: int = 4096) -> Workload:
    return Workload(
        name=f"moe_geglu_8x4096-14336_T{T}_top2", op="moe", M=T, K=4096, H=14336, N=4096,
        w1_bound=1 / math.sqrt(4096), w2_bound=1 / math.sqrt(14336), E=8, top_k=2,
        family="moe")


def _router(T: int = 4096) -> Workload:
    """The router of the 8-expert MoE layer: x [T, 4096], Wr [8, 4096], top-2."""
    return Workload(
        name=f"moe_router_8x4096_T{T}_top2", op="route", M=T, K=4096, H=0, N=0,
        w1_bound=1 / math.sqrt(4096), E=8, top_k=2, family="moe")


def _glu_bwd(base: Workload) -> Workload:
    """The backward pass of a GeGLU workload (same family, so the same weights
    and x), with an upstream gradient dy ~ N(0, 1) of y's shape."""
    import dataclasses

    return dataclasses.replace(base, name=base.name + "_bwd", op="glu_bwd")


WORKLOADS = {
    "tiny": _tiny(),
    "decode1": _decode(1),
    "decode16": _decode(16),
    "geglu768": _geglu768(),
    "large1": _large(1),
    "large16": _large(16),
    "large4096": _large(4096),
    "moe": _moe(),
    "router": _router(),
    "geglu768_bwd": _glu_bwd(_geglu768()),
    "large4096_bwd": _glu_bwd(_large(4096)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------
def make_inputs(w: Workload, seed: int = 0, with_weights: bool = True) -> dict:
    """bf16-bit arrays (uint16) for a dense workload (mlp2 / geglu).

    mlp2: x, W1, b1, W2, b2 (biases only when w.bias);  geglu: x, Wg, Wu, Wd;
    glu_bwd: x, dy, Wg, Wu, Wd.
    """
    f = w.family
    out = {"x": normal_bf16(rng_for(seed, f, f"x{w.M}"), (w.M, w.K))}
    if w.op == "glu_bwd":   # the upstream gradient of a backward workload
        out["dy"] = normal_bf16(rng_for(seed, f, f"dy{w.M}"), (w.M, w.N))
    if not with_weights:
        return out
    if w.op == "mlp2":
        out["W1"] = uniform_bf16(rng_for(seed, f, "W1"), (w.H, w.K), w.w1_bound)
        out["W2"] = uniform_bf16(rng_for(seed, f, "W2"), (w.N, w.H), w.w2_bound)
        if w.bias:
            out["b1"] = uniform_bf16(rng_for(seed, f, "b1"), (w.H,), w.b1_bound)
            out["b2"] = uniform_bf16(rng_for(seed, f, "b2"), (w.N,), w.b2_bound)
    elif w.op in ("geglu", "glu_bwd"):
        out["Wg"] = uniform_bf16(rng_for(seed, f, "Wg"), (w.H, w.K), w.w1_bound)
        out["Wu"] = uniform_bf16(rng_for(seed, f, "Wu"), (w.H, w.K), w.w1_bound)
        out["Wd"] = uniform_bf16(rng_for(seed, f, "Wd"), (w.N, w.H), w.w2_bound)
    else:
        raise ValueError(f"make_inputs handles dense workloads, not {w.op}")
    return out


def make_routes(T: int, E: int, top_k: int, seed: int = 0, family: str = "moe"):
    """Top-k routes: distinct expert ids drawn uniformly per token, and gate
    weights = softmax over top_k N(0,1) logits (one logit per chosen expert).

    Returns (expert_ids int32 [T, top_k], gate_w float32 [T, top_k]).
    """
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    r = rng_for(seed, family, f"ids{T}")
    ids = np.argsort(r.random((T, E)), axis=1)[:, :top_k].astype(np.int32)
    logits = rng_for(seed, family, f"logits{T}").standard_normal((T, top_k), dtype=np.float32)
    z = logits.astype(np.float64)
    z = np.exp(z - z.max(axis=1, keepdims=True))
    gate = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(gate)


def router_weights(w: Workload, seed: int = 0):
    """bf16 bits of the router weight Wr [E, D] ~ U(+-1/sqrt(D)) of a MoE family."""
    return uniform_bf16(rng_for(seed, w.family, "Wr"), (w.E, w.K), 1 / math.sqrt(w.K))


def expert_weights(w: Workload, e: int, seed: int = 0):
    """bf16 bits of expert e: (Wg [H,D], Wu [H,D], Wd [D,H])."""
    f = w.family
    Wg = uniform_bf16(rng_for(seed, f, f"Wg{e}"), (w.H, w.K), w.w1_bound)
    Wu = uniform_bf16(rng_for(seed, f, f"Wu{e}"), (w.H, w.K), w.w1_bound)
    Wd = uniform_bf16(rng_for(seed, f, f"Wd{e}"), (w.N, w.H), w.w2_bound)
    return Wg, Wu, Wd
