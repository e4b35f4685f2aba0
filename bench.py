#!/usr/bin/env python3
"""Throughput of the fused feed-forward path on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--act ACT]

A step is one forward of the workload's whole feed-forward block through the
C ABI (one fmlp_* call) on synthetic seeded bf16 inputs already resident in
HBM.  --act replaces the workload's activation (two-layer MLPs) or its gate
activation (gated blocks and MoE: "silu" runs SwiGLU).

Default workload (the headline): the GeGLU feed-forward block of dim 8192 and
hidden 28672 at 4096 tokens, the largest configuration and the one bound by
the matrix cores (the flattened-token GEMM shapes of "Profiling in PyTorch
(Part 2)", section "Why are there two kinds of GEMM kernels?").  After it, the
same JSON line carries a "configs" table with every other workload timed on
its own: the tiny MLP, the 4096^3 decode MLP at 1 and 16 tokens (the 4096-wide
GELU MLP at batch 1 of ainews.cool "PyTorch fused MLP efficiency", section
"benchmark data"), the 768/3072 GeGLU, the large GeGLU at 1 and 16 tokens, the
MoE and the router.  Weights that would fit the 256 MB Infinity Cache rotate
through enough copies (>= 1 GiB) that every step reads them from HBM.

Prints ONE JSON line: metric/value (TFLOP/s), ms_per_step, the roofline of the
dominant kernel (HIP-event time over the timed region), the fp64 CPU oracle
timed on a bounded sample on this host's cores, and the configs table.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-MLP TFLOP/s & µs/forward (bf16) + % of MFMA or HBM roofline, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
COLD_BYTES = 1 << 30           # rotate weight copies until this many bytes (4x the 256 MB MALL)
# the page's fused 4096-wide GELU MLP at batch 1 on H100: 8.1 us (context only)
PAGE_H100_FUSED_US = 8.1

# the files each kernel is built from; the hash also covers their compile flags
KERNEL_SOURCES = {
    "decode_kernel": ["common.h", "kernels.h", "lds_dma.h", "exchange.h", "decode.hip"],
    "gemm_bf16_kernel": ["common.h", "kernels.h", "lds_dma.h", "gemm.hip", "moe.hip"],
    "small_mlp2_kernel": ["common.h", "kernels.h", "small_mlp.hip"],
    "moe_router_mfma_kernel": ["common.h", "kernels.h", "lds_dma.h", "moe.hip"],
    "decode_w8_kernel": ["common.h", "kernels.h", "lds_dma.h", "exchange.h", "decode_w8.h", "decode_w8.hip"],
    "decode_w8_two_kernel": ["common.h", "kernels.h", "lds_dma.h", "exchange.h", "decode_w8.h", "decode_w8.hip"],
    "decode_w8_split_kernel": ["common.h", "kernels.h", "lds_dma.h", "exchange.h", "decode_w8.h", "decode_w8.hip"],
    "glu_fused_kernel": ["common.h", "kernels.h", "lds_dma.h", "glu_fused.hip"],
}


def kernel_source_sha(kernel: str) -> str:
    from gemm_epilogue_bf16_amd import build as _build

    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gemm_epilogue_bf16_amd")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(pkg, "csrc", f), "rb") as fh:
            h.update(fh.read())
        h.update(" ".join(_build.EXTRA_FLAGS.get(f, [])).encode())
    # the include path names the checkout's location, which is not part of the build
    h.update(" ".join(f.replace(_build.ROOT, "<repo>") for f in _build.common_flags()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload set-up: returns a Case with bound launches (one per weight copy)
# ---------------------------------------------------------------------------
class Case:
    def __init__(self, w, calls, kernel, launches, path, copies, oracle_fn, oracle_sample):
        self.w = w
        self.calls = calls
        self.kernel = kernel          # dominant kernel (symbol prefix in traces)
        self.launches = launches      # kernel launches per step
        self.path = path
        self.copies = copies
        self.oracle_fn = oracle_fn    # () -> None, runs the oracle on the sample
        self.oracle_sample = oracle_sample  # (description, fraction of one step's flops)
        self.unfused = None           # per weight copy: the same forward as separate launches
        self.unfused_form = ("fmlp_linear (GEMM + bias + activation), then fmlp_linear (GEMM + bias)", 2)
        self.bytes = w.bytes          # algorithmic HBM bytes of one forward
        self.weights = "bf16"


def _dev(bits, torch, dev, dtype=None):
    import torch as _t
    if dtype is None:
        return _t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_t.bfloat16).to(dev)
    return _t.from_numpy(np.ascontiguousarray(bits)).to(dev)


_HOST_CACHE: dict = {}
_DEV_CACHE: dict = {}


def _inputs(w):
    """datagen.make_inputs, with the weights of a workload family generated
    once per process (the weights do not depend on the token count)."""
    import datagen

    key = (w.family, "geglu" if w.op == "glu_bwd" else w.op)   # a backward shares its forward's weights
    if key not in _HOST_CACHE:
        _HOST_CACHE[key] = {k: v for k, v in datagen.make_inputs(w, seed=0).items() if k != "x"}
    t = dict(_HOST_CACHE[key])
    t.update(datagen.make_inputs(w, seed=0, with_weights=False))   # x (and dy)
    return t


def _dev_weights(w, t, torch, dev):
    key = (w.family, "geglu" if w.op == "glu_bwd" else w.op)
    if key not in _DEV_CACHE:
        _DEV_CACHE[key] = {k: _dev(v, torch, dev) for k, v in t.items() if k not in ("x", "dy")}
    return _DEV_CACHE[key]


def _copies_for(weight_bytes: int, cold: bool) -> int:
    if not cold:
        return 1
    return max(1, -(-COLD_BYTES // weight_bytes))


def _setup_w8(w, cold: bool, dev, gate_act):
    """The decode workloads with FP8 E4M3 weights (one fp32 scale per row):
    same shapes, activations and biases as the bf16 workload; the weights are
    drawn as codes by datagen.e4m3_weights with the same bounds."""
    import torch

    import datagen
    import gemm_epilogue_bf16_amd as F
    import oracle

    if w.M > 16 or w.op not in ("mlp2", "geglu"):
        raise SystemExit("--weights fp8 is for the decode workloads (decode1, decode16, large1, large16)")
    f64 = lambda b: datagen.bf16_to_f32(b).astype(np.float64)  # noqa: E731
    t = datagen.make_inputs(w, seed=0, with_weights=False)
    if w.op == "mlp2" and w.bias:   # the bf16 workload's biases (same streams)
        t["b1"] = datagen.uniform_bf16(datagen.rng_for(0, w.family, "b1"), (w.H,), w.b1_bound)
        t["b2"] = datagen.uniform_bf16(datagen.rng_for(0, w.family, "b2"), (w.N,), w.b2_bound)
    x = _dev(t["x"], torch, dev)
    y = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
    if w.op == "mlp2":
        shapes = {"W1": (w.H, w.K, w.w1_bound), "W2": (w.N, w.H, w.w2_bound)}
    else:
        shapes = {"Wg": (w.H, w.K, w.w1_bound), "Wu": (w.H, w.K, w.w1_bound), "Wd": (w.N, w.H, w.w2_bound)}
    host = {k: datagen.e4m3_weights(datagen.rng_for(0, w.family, k + "_e4m3"), r, c, bd)
            for k, (r, c, bd) in shapes.items()}
    wbytes = sum(r * c + 4 * r for (r, c, _) in shapes.values())
    if w.op == "mlp2" and w.bias:
        wbytes += 2 * (w.H + w.N)
    R = _copies_for(wbytes, cold)
    sets = []
    for i in range(R):
        sets.append({k: (torch.from_numpy(q).to(dev), torch.from_numpy(sc).to(dev)) for k, (q, sc) in host.items()})
    ws = F.workspace_for(dev, int(F.lib().fmlp_w8_workspace_size(w.M, w.H)))
    calls = []
    rows = w.M
    cache = {}
    if w.op == "mlp2":
        b1 = _dev(t["b1"], torch, dev) if "b1" in t else None
        b2 = _dev(t["b2"], torch, dev) if "b2" in t else None
        for st in sets:
            calls.append(F.bind_mlp2_w8(x, *st["W1"], b1, *st["W2"], b2, w.act, out=y, workspace=ws))

        def fn():
            if not cache:
                cache.update({k: f64(v) for k, v in t.items()})
            c = cache
            return oracle.mlp2_w8(c["x"], *host["W1"], c.get("b1"), *host["W2"], c.get("b2"), w.act)
    else:
        act = gate_act or "gelu_tanh"
        for st in sets:
            calls.append(F.bind_glu_w8(x, *st["Wg"], *st["Wu"], *st["Wd"], act, out=y, workspace=ws))

        def fn():
            if not cache:
                cache.update({k: f64(v) for k, v in t.items()})
            return oracle.glu_w8(cache["x"], *host["Wg"], *host["Wu"], *host["Wd"], act)
    if w.M == 1 and w.H <= 4096:   # both layers in one launch (h exchanged as epoch-tagged words)
        # rows of at most 4096 codes: the two-role form (layer 2 held in registers during the exchange)
        kernel = "decode_w8_split_kernel" if w.K <= 4096 else "decode_w8_two_kernel"
        launches, p = 1, "FP8-weight decode, both layers in one launch"
    else:
        kernel, launches, p = "decode_w8_kernel", 2, "FP8-weight decode (one launch per layer)"
    case = Case(w, calls, kernel, launches, p, R, fn, (f"{rows} of {w.M} token rows, full weights", 1.0))
    case.bytes = wbytes + 2 * w.M * w.K + 2 * w.M * w.N
    case.weights = "fp8_e4m3, one fp32 scale per output row"
    return case


def setup_case(name: str, cold: bool, dev, path: str, act=None, w8: bool = False):
    import dataclasses

    import torch

    import datagen
    import gemm_epilogue_bf16_amd as F

    w = datagen.workload(name)
    gate_act = None
    if act is not None:
        if w.op == "mlp2":
            w = dataclasses.replace(w, act=act)
        else:
            gate_act = act
    f64 = lambda b: datagen.bf16_to_f32(b).astype(np.float64)  # noqa: E731
    R = _copies_for(w.weight_bytes, cold)

    if w8:
        return _setup_w8(w, cold, dev, gate_act)

    if w.op in ("mlp2", "geglu"):
        t = _inputs(w)
        x = _dev(t["x"], torch, dev)
        base = _dev_weights(w, t, torch, dev)
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
        y = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
        calls = []
        if w.op == "mlp2":
            ws = F.workspace_for(dev, F.fmlp_mlp2_workspace_size(w.M, w.K, w.H, w.N))
            for s in sets:
                calls.append(F.bind_mlp2(x, s["W1"], s.get("b1"), s["W2"], s.get("b2"), w.act, out=y, workspace=ws))
            # unfused: the page's launch-per-layer form, here two of our own
            # Linear launches (GEMM + bias + activation, then GEMM + bias)
            h_un = torch.empty(w.M, w.H, dtype=torch.bfloat16, device=dev)
            unfused = [(F.bind_linear(x, s["W1"], s.get("b1"), w.act, out=h_un),
                        F.bind_linear(h_un, s["W2"], s.get("b2"), "none", out=y)) for s in sets]
            if w.M <= 16:
                kernel, launches, p = "decode_kernel", 1, "persistent decode (1 launch)"
            elif max(w.K, w.H, w.N) <= 128:
                kernel, launches, p = "small_mlp2_kernel", 1, "small fused MLP (1 launch)"
            else:
                kernel, launches, p = "gemm_bf16_kernel", 2, "two tiled GEMMs"
            rows = min(w.M, 256)
            import oracle

            cache = {}

            def fn():
                if not cache:   # input decoding (bf16 bits -> float64), once, before timing
                    cache.update({k: f64(v) for k, v in t.items()})
                c = cache
                return oracle.mlp2(c["x"][:rows], c["W1"], c.get("b1"), c["W2"], c.get("b2"), w.act)
            sample = (f"{rows} of {w.M} token rows, full weights", rows / w.M)
            case = Case(w, calls, kernel, launches, p, R, fn, sample)
            case.unfused = unfused
            case.workspace = ws
            return case
        else:
            ws = F.workspace_for(dev, F.fmlp_geglu_workspace_size(w.M, w.K, w.H))
            for s in sets:
                if gate_act is None:
                    calls.append(F.bind_geglu(x, s["Wg"], s["Wu"], s["Wd"], out=y, workspace=ws))
                else:
                    calls.append(F.bind_glu(x, s["Wg"], s["Wu"], s["Wd"], gate_act, out=y, workspace=ws))
            if path == "fused":
                kernel, launches, p = "glu_fused_kernel", 1, "whole block in one launch, m kept on chip"
            elif w.M <= 16:
                kernel, launches, p = "decode_kernel", 1, "persistent decode (1 launch)"
            else:
                kernel, launches, p = "gemm_bf16_kernel", 2, "fused gate+up GEMM + down GEMM (2 launches)"
            unfused = None
            if w.M > 16 and gate_act is None and path in ("auto", "gemm"):
                # unfused: the page's eager GeGLU with our own GEMMs: g = gelu(x Wg^T) and
                # u = x Wu^T as two Linear launches, m = g * u as torch's elementwise
                # multiply (context: a library kernel), then the down projection
                g_un = torch.empty(w.M, w.H, dtype=torch.bfloat16, device=dev)
                u_un = torch.empty_like(g_un)
                m_un = torch.empty_like(g_un)
                unfused = [(F.bind_linear(x, s_["Wg"], None, "gelu_tanh", out=g_un),
                            F.bind_linear(x, s_["Wu"], None, "none", out=u_un),
                            (lambda: torch.mul(g_un, u_un, out=m_un)),
                            F.bind_linear(m_un, s_["Wd"], None, "none", out=y)) for s_ in sets]
            import oracle

            rows = min(w.M, 64 if w.K * w.H > 1e8 else 1024)
            cache = {}

            def fn():
                if not cache:   # input decoding (bf16 bits -> float64), once, before timing
                    cache.update({k: f64(v) for k, v in t.items()})
                c = cache
                if gate_act is not None:
                    return oracle.glu(c["x"][:rows], c["Wg"], c["Wu"], c["Wd"], gate_act)
                return oracle.geglu(c["x"][:rows], c["Wg"], c["Wu"], c["Wd"])
            sample = (f"{rows} of {w.M} token rows, full weights", rows / w.M)
        case = Case(w, calls, kernel, launches, p, R, fn, sample)
        case.workspace = ws
        if unfused is not None:
            case.unfused = unfused
            case.unfused_form = ("fmlp_linear (gate GEMM + tanh GELU), fmlp_linear (up GEMM), torch.mul, "
                                 "fmlp_linear (down GEMM)", 4)
        return case

    if w.op == "glu_bwd":
        # the gated block's backward: every gradient of a GeGLU forward for an
        # upstream gradient dy; the oracle times glu_bwd on the first rows tokens
        t = _inputs(w)
        x, dy = _dev(t["x"], torch, dev), _dev(t["dy"], torch, dev)
        base = _dev_weights(w, t, torch, dev)
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
        outs = (torch.empty_like(x), torch.empty_like(base["Wg"]), torch.empty_like(base["Wu"]),
                torch.empty_like(base["Wd"]))
        ws = torch.empty(int(F.lib().fmlp_glu_bwd_workspace_size(w.M, w.K, w.H)), dtype=torch.uint8, device=dev)
        calls = [F.bind_glu_bwd(x, s_["Wg"], s_["Wu"], s_["Wd"], "gelu_tanh", dy, out=outs, workspace=ws)
                 for s_ in sets]
        import oracle

        rows = 64 if w.K * w.H > 1e8 else 512
        cache = {}

        def fn():
            if not cache:
                cache.update({k: f64(v[:rows] if k in ("x", "dy") else v) for k, v in t.items()})
            c = cache
            return oracle.glu_bwd(c["x"], c["Wg"], c["Wu"], c["Wd"], "gelu_tanh", c["dy"])
        case = Case(w, calls, "gemm_bf16_kernel", 13,
                    "backward: dm GEMM, gate+up GEMM with the dGeGLU epilogue, dx GEMM over [dg|du], "
                    "3 weight-gradient GEMMs, 7 transposes (13 launches)", R, fn,
                    (f"{rows} of {w.M} token rows, full weights", rows / w.M))
        case.workspace = ws
        return case

    if w.op == "route":
        # x streams once per step; x copies rotate (>= 1 GiB) so it is read from HBM
        x_bits = datagen.make_inputs(datagen.workload("moe"), seed=0, with_weights=False)["x"]
        Wr_bits = datagen.router_weights(w, seed=0)
        xb = _dev(x_bits, torch, dev)
        Wr = _dev(Wr_bits, torch, dev)
        R = _copies_for(2 * w.M * w.K, cold)
        xs_d = [xb] + [xb.clone() for _ in range(R - 1)]
        ids_o = torch.empty(w.M, w.top_k, dtype=torch.int32, device=dev)
        gw_o = torch.empty(w.M, w.top_k, dtype=torch.float32, device=dev)
        calls = [F.bind_moe_route(xx, Wr, w.top_k, out=(ids_o, gw_o)) for xx in xs_d]
        import oracle

        toks = 1024
        cache = {}

        def fn():
            if not cache:
                cache["x"] = f64(x_bits[:toks])
                cache["Wr"] = f64(Wr_bits)
            return oracle.moe_router(cache["x"], cache["Wr"], w.top_k)
        return Case(w, calls, "moe_router_mfma_kernel", 1, "router: logits, top-k, softmax (1 launch)", R, fn,
                    (f"{toks} of {w.M} tokens", toks / w.M))

    # mixture of experts
    x_bits = datagen.make_inputs(w, seed=0, with_weights=False)["x"]
    ids, gw = datagen.make_routes(w.M, w.E, w.top_k, seed=0)
    experts = [datagen.expert_weights(w, e, seed=0) for e in range(w.E)]
    x = _dev(x_bits, torch, dev)
    Wg = torch.stack([_dev(e[0], torch, dev) for e in experts])
    Wu = torch.stack([_dev(e[1], torch, dev) for e in experts])
    Wd = torch.stack([_dev(e[2], torch, dev) for e in experts])
    ids_d = torch.from_numpy(ids).to(dev)
    gw_d = torch.from_numpy(gw).to(dev)
    y = torch.empty_like(x)
    ws = F.workspace_for(dev, F.fmlp_moe_workspace_size(w.M, w.K, w.H, w.E, w.top_k))
    if gate_act is None:
        calls = [F.bind_moe_geglu(x, ids_d, gw_d, Wg, Wu, Wd, out=y, workspace=ws)]
    else:
        calls = [F.bind_moe_glu(x, ids_d, gw_d, Wg, Wu, Wd, gate_act, out=y, workspace=ws)]
    import oracle

    toks = 32
    xs = datagen.bf16_to_f32(x_bits[:toks]).astype(np.float64)
    f64e = {}

    def get(e):
        if e not in f64e:
            f64e[e] = tuple(datagen.bf16_to_f32(a).astype(np.float64) for a in experts[e])
        return f64e[e]

    if gate_act is None:
        fn = lambda: oracle.moe_geglu(xs, ids[:toks], gw[:toks], get)  # noqa: E731
    else:
        fn = lambda: oracle.moe_glu(xs, ids[:toks], gw[:toks], get, gate_act)  # noqa: E731
    return Case(w, calls, "gemm_bf16_kernel", 6,
                "route (count, scan, place) + grouped gate+up + grouped down + combine",
                1, fn, (f"{toks} of {w.M} tokens (their experts' weights pre-converted)", toks / w.M))


def copy_calibration(dev, nbytes: int, reps: int):
    """A plain elementwise copy of known size (one read + one write of nbytes),
    run so that rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE can be scaled."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


# ---------------------------------------------------------------------------
def time_oracle(case: Case, seconds: float):
    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    case.oracle_fn()  # warm (BLAS init, page-in)
    n, t0 = 0, time.perf_counter()
    while True:
        case.oracle_fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_call = el / n
    flops = case.w.flops * case.oracle_sample[1]
    return {
        "value": round(flops / per_call / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{case.oracle_sample[0]}; {n} oracle calls in {el:.1f} s (fp64 numpy/OpenBLAS)",
        "us_per_forward_equiv": round(per_call / case.oracle_sample[1] * 1e6, 1),
        "cpu": platform.processor() or platform.machine(),
    }


def read_traffic(case: Case):
    """HBM bytes per step (all of a step's launches of the kernel) from
    committed rocprofv3 PMC summaries, if they were taken on the current
    sources of that kernel; else None."""
    p = os.path.join(ROOT, "profiles", f"{case.kernel}__{case.w.name}__traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha") != kernel_source_sha(case.kernel):
        return None
    return d.get("bytes_per_step", d.get("bytes_per_launch"))


EST_US = {"tiny": 5, "decode1": 12, "decode16": 12, "geglu768": 100, "large1": 250,
          "large16": 250, "large4096": 4000, "moe": 2500, "router": 8, "geglu768_bwd": 300,
          "large4096_bwd": 9000}
# every workload of the configuration table, in the order the rows are printed
CONFIG_ROWS = ["tiny", "decode1", "decode16", "geglu768", "large1", "large16", "large4096", "moe", "router",
               "geglu768_bwd", "large4096_bwd"]
# a workload timed again on another path (same inputs): the gated block in one
# launch with m on chip, against the default two launches of its own row
CONFIG_PATH_ROWS = [("geglu768", "fused")]


def run_timed(case: Case, K: int, W: int, path: str, stream, torch, F, unfused: bool = True) -> dict:
    """W untimed steps, then exactly K timed steps bracketed by synchronize on
    both sides (wall clock and HIP events on the stream the launches go to),
    then up to 200 single steps each between two events (per-step spread)."""
    R = len(case.calls)
    calls = case.calls
    with F.force_path(path):
        for i in range(W):
            calls[i % R]()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(K):
            calls[i % R]()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        res = {"wall_s": (t1 - t0) / K, "dev_s": ev0.elapsed_time(ev1) * 1e-3 / K}

        n_ev = min(K, 200)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        torch.cuda.synchronize()
        for i in range(n_ev):
            starts[i].record(stream)
            calls[i % R]()
            ends[i].record(stream)
        torch.cuda.synchronize()
        res["launch_ms"] = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])

        res["unfused_s"] = None
        if unfused and case.unfused is not None:
            for i in range(W):
                for c in case.unfused[i % R]:
                    c()
            torch.cuda.synchronize()
            u0 = time.perf_counter()
            for i in range(K):
                for c in case.unfused[i % R]:
                    c()
            torch.cuda.synchronize()
            res["unfused_s"] = (time.perf_counter() - u0) / K
    return res


def roofline_of(case: Case, kernel_s: float) -> dict:
    """Roofline of the step's dominant kernel family: algorithmic work of one
    step over the step's HIP-event time (for a one-launch step: the average
    launch duration, including the dispatch gap to the next launch)."""
    w = case.w
    if w.flops / case.bytes < 300.0:
        achieved = case.bytes / kernel_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    else:
        achieved = w.flops / kernel_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = read_traffic(case)
    return roof


def decode_timeouts(case: Case, F):
    """Barrier waits that gave up in the one-launch decode kernel (0 expected)."""
    ws = getattr(case, "workspace", None)
    if case.kernel not in ("decode_kernel", "decode_w8_two_kernel", "decode_w8_split_kernel") or ws is None:
        return None
    return F.barrier_timeouts(ws)


def config_row(name: str, dev, stream, torch, F, act=None, path: str = "auto") -> dict:
    """One row of the configuration table: the workload's forward timed on its
    own (cold weights), with its roofline fraction from HIP events."""
    case = setup_case(name, cold=True, dev=dev, path=path, act=act)
    est = EST_US[name]
    K = max(20, min(2000, int(0.4e6 / est)))
    r = run_timed(case, K, max(5, K // 10), path, stream, torch, F, unfused=False)
    roof = roofline_of(case, r["dev_s"])
    w = case.w
    row = {"workload": w.name, "tokens": w.M, "path": case.path, "launches": case.launches,
           "kernel": case.kernel, "steps": K,
           "us_per_forward": round(r["wall_s"] * 1e6, 3),
           "us_per_forward_device": round(r["dev_s"] * 1e6, 3),
           "tflops": round(w.flops / r["dev_s"] / 1e12, 2),
           "roofline": roof}
    t = decode_timeouts(case, F)
    if t is not None:
        row["barrier_timeouts"] = t
    del case
    torch.cuda.empty_cache()
    return row


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="large4096", choices=CONFIG_ROWS)
    ap.add_argument("--act", default=None, choices=["none", "gelu_erf", "gelu_tanh", "relu", "silu"],
                    help="activation of a two-layer MLP, or gate activation of a gated block")
    ap.add_argument("--warm", action="store_true", help="no weight rotation (weights may sit in the 256 MB cache)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "gemm", "small", "fused"],
                    help="fused: the gated block in one launch with m on chip (D <= 1024)")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                    help="fp8: the decode workloads with E4M3 weights and per-row scales")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused comparison (counter runs: one kernel variant only)")
    ap.add_argument("--no-configs", action="store_true",
                    help="only the headline workload (no table of the other workloads)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain copy of this many MiB (for PMC scaling) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the feed-forward path shards by tokens or by hidden columns; see DESIGN.md)",
              file=sys.stderr)
        return 2

    import torch

    import gemm_epilogue_bf16_amd as F

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev, args.copy_calibration << 20, 10)
        return 0

    case = setup_case(args.workload, cold=not args.warm, dev=dev, path=args.path, act=args.act,
                      w8=args.weights == "fp8")
    w = case.w
    K = args.steps if args.steps is not None else max(20, int(1.5e6 / EST_US[args.workload]))
    W = args.warmup if args.warmup is not None else max(5, K // 10)
    stream = torch.cuda.current_stream(dev)
    print(f"bench: {w.name}, {K} timed steps after {W} warm-up steps", file=sys.stderr, flush=True)
    r = run_timed(case, K, W, args.path, stream, torch, F, unfused=not args.no_unfused)
    wall_s, dev_s, launch_ms, unfused_s = r["wall_s"], r["dev_s"], r["launch_ms"], r["unfused_s"]
    per_launch_s = float(np.mean(launch_ms)) * 1e-3

    # one step = one forward; value = algorithmic TFLOP/s of the whole job
    value = w.flops / wall_s / 1e12
    kernel_s = dev_s
    roof = roofline_of(case, kernel_s)
    roof["kernel"] = case.kernel
    roof["launches_per_step"] = case.launches
    roof["algorithmic_flops"] = w.flops
    roof["algorithmic_bytes"] = case.bytes
    roof["us_per_step_events"] = round(kernel_s * 1e6, 3)
    roof["us_per_launch_bracketed"] = round(per_launch_s * 1e6, 3)
    roof["us_per_launch_p10_p50_p90"] = [round(float(v) * 1e3, 3) for v in np.percentile(launch_ms, [10, 50, 90])]
    timeouts = decode_timeouts(case, F)

    vs = None
    if (w.name.startswith("decode_mlp2_4096x4096x4096_M1") and args.act in (None, "gelu_erf")
            and case.weights == "bf16"):
        vs = round(value / (w.flops / (PAGE_H100_FUSED_US * 1e-6) / 1e12), 4)

    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "op": w.op,
            "tokens": w.M,
            "dims": {"in": w.K, "hidden": w.H, "out": w.N,
                     **({"experts": w.E, "top_k": w.top_k} if w.op in ("moe", "route") else {})},
            "act": (w.act if w.op == "mlp2" else "top-k + softmax" if w.op == "route"
                    else (f"{args.act} gate" if args.act else "gelu_tanh (GeGLU)")
                    + (", backward" if w.op == "glu_bwd" else "")),
            "bias": w.bias,
            "weight_format": case.weights,
            "weights": (f"cold: {case.copies} rotated copies of x ({case.copies * 2 * w.M * w.K / 2**20:.0f} MiB)"
                        if case.copies > 1 and w.op == "route" else
                        f"cold: {case.copies} rotated copies "
                        f"({case.copies * (case.bytes - 2 * w.M * (w.K + w.N)) / 2**20:.0f} MiB)"
                        if case.copies > 1 else "single copy"),
            "path": case.path,
            "parallelism": "single GPU",
        },
        "us_per_forward": round(wall_s * 1e6, 3),
        "us_per_forward_device": round(dev_s * 1e6, 3),
        "roofline": roof,
        "unfused": ({"launches": case.unfused_form[1], "us_per_forward": round(unfused_s * 1e6, 3),
                     "form": case.unfused_form[0]}
                    if unfused_s is not None else None),
        "baseline_note": ("vs_baseline = value / the page's H100 fused figure (8.1 us, same workload); "
                          "another machine, context only") if vs is not None else None,
    }
    if timeouts is not None:
        out["barrier_timeouts"] = timeouts
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = time_oracle(case, args.cpu_seconds)
    if not args.no_configs and args.weights == "bf16" and args.act is None and args.path == "auto":
        # the other workloads, each timed on its own after the headline
        del case
        rows = []
        for name in CONFIG_ROWS:
            if name == args.workload:
                continue
            print(f"bench: config row {name}", file=sys.stderr, flush=True)
            rows.append(config_row(name, dev, stream, torch, F))
        for name, path in CONFIG_PATH_ROWS:
            print(f"bench: config row {name} ({path} path)", file=sys.stderr, flush=True)
            rows.append(config_row(name, dev, stream, torch, F, path=path))
        out["configs"] = rows
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
