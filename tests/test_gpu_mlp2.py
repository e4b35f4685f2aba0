"""fmlp_mlp2 on the GPU against the fp64 oracle, on every path (persistent
decode, single-launch small MLP, two GEMMs), at the tiny and decode workloads'
full sizes and on random ragged shapes; plus fused == unfused and the bias pins."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bf16_ulp, bits_of, f64_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _dev_inputs(t):
    return {k: to_dev(v) for k, v in t.items()}


def _oracle(t, act):
    g = lambda k: None if k not in t else f64_of_bits(t[k])  # noqa: E731
    return oracle.mlp2(g("x"), g("W1"), g("b1"), g("W2"), g("b2"), act)


def _run(d, act, path="auto", ws=None):
    with F.force_path(path):
        y = F.fmlp_mlp2(d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), act, workspace=ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("path", ["auto", "small", "gemm"])
def test_tiny_workload_full(path):
    w = datagen.workload("tiny")
    t = datagen.make_inputs(w, seed=0)
    print(f"case {w.name} path={path}", flush=True)
    y = _run(_dev_inputs(t), w.act, path)
    assert_parity(y, _oracle(t, w.act), f"{w.name} {path}")


@pytest.mark.parametrize("name", ["decode1", "decode16"])
@pytest.mark.parametrize("path", ["auto", "gemm"])
def test_decode_workload_full(name, path):
    w = datagen.workload(name)
    t = datagen.make_inputs(w, seed=0)
    d = _dev_inputs(t)
    ws = F.workspace_for(DEV, F.fmlp_mlp2_workspace_size(w.M, w.K, w.H, w.N))
    print(f"case {w.name} path={path}", flush=True)
    y = _run(d, w.act, path, ws)
    assert_parity(y, _oracle(t, w.act), f"{w.name} {path}")
    assert F.barrier_timeouts(ws) == 0


SHAPES = [
    # (M, K, H, N)
    (1, 8, 8, 8), (1, 64, 200, 40), (3, 136, 520, 264), (16, 512, 256, 1024), (16, 1024, 4096, 64),
    (9, 4096, 1024, 4096), (17, 32, 64, 32), (40, 128, 128, 128), (100, 96, 40, 120),
    (16, 1024, 512, 16384), (1, 2048, 256, 12288),   # one-stage layer-2 tiles, several per block
    (257, 256, 512, 136), (600, 768, 1024, 392),
]


@pytest.mark.parametrize("M,K,H,N", SHAPES)
@pytest.mark.parametrize("act", ["gelu_erf", "gelu_tanh"])
def test_mlp2_random(M, K, H, N, act):
    rng = np.random.default_rng(M * 7919 + K * 31 + H * 3 + N)
    t = {"x": rand_bf16(rng, (M, K)),
         "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"), "b1": rand_bf16(rng, (H,), 0.3, "uniform"),
         "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"), "b2": rand_bf16(rng, (N,), 0.3, "uniform")}
    d = _dev_inputs(t)
    ref = _oracle(t, act)
    paths = ["auto", "gemm"]
    if M <= 16:
        paths.append("decode")
    if max(K, H, N) <= 128:
        paths.append("small")
    for p in paths:
        print(f"case mlp2 M={M} K={K} H={H} N={N} act={act} path={p}", flush=True)
        assert_parity(_run(d, act, p), ref, f"mlp2 {M}x{K}x{H}x{N} {p}")


@pytest.mark.parametrize("M,path", [(1, "decode"), (16, "decode"), (64, "small"), (300, "gemm")])
def test_mlp2_no_biases(M, path):
    rng = np.random.default_rng(M)
    K, H, N = 64, 128, 96
    t = {"x": rand_bf16(rng, (M, K)), "W1": rand_bf16(rng, (H, K), 0.125, "uniform"),
         "W2": rand_bf16(rng, (N, H), 0.09, "uniform")}
    print(f"case mlp2 no-bias M={M} path={path}", flush=True)
    assert_parity(_run(_dev_inputs(t), "gelu_tanh", path), _oracle(t, "gelu_tanh"), f"no-bias {path}")


@pytest.mark.parametrize("M,path", [(1, "decode"), (16, "decode"), (64, "small"), (300, "gemm")])
def test_mlp2_bias_pins(M, path):
    """W1 = 0 -> h = act(b1); W2 = I, b2 = 0 -> y = bf16(act(b1)) for every row."""
    rng = np.random.default_rng(M + 1)
    K = H = N = 64
    b1 = rand_bf16(rng, (H,), 2.0, "uniform")
    t = {"x": rand_bf16(rng, (M, K)), "W1": np.zeros((H, K), np.uint16), "b1": b1,
         "W2": datagen.rne_bf16(np.eye(N, H, dtype=np.float32)), "b2": np.zeros(N, np.uint16)}
    for act in ("gelu_erf", "gelu_tanh"):
        print(f"case mlp2 bias pin M={M} path={path} act={act}", flush=True)
        y = f64_of(_run(_dev_inputs(t), act, path))
        want = oracle.activation(f64_of_bits(b1), act)
        assert np.all(np.abs(y - want[None, :]) <= bf16_ulp(want)[None, :])


@pytest.mark.parametrize("M,path", [(1, "decode"), (16, "decode"), (300, "gemm"), (512, "small")])
def test_fused_equals_unfused(M, path):
    """One fused call == fmlp_linear(act) then fmlp_linear: both round h to
    bf16 once, at the same place."""
    rng = np.random.default_rng(M + 2)
    K, H, N = (128, 128, 64) if path == "small" else (512, 1024, 256)
    t = {"x": rand_bf16(rng, (M, K)),
         "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"), "b1": rand_bf16(rng, (H,), 0.3, "uniform"),
         "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"), "b2": rand_bf16(rng, (N,), 0.3, "uniform")}
    d = _dev_inputs(t)
    print(f"case fused==unfused M={M} path={path}", flush=True)
    fused = _run(d, "gelu_erf", path)
    h = F.fmlp_linear(d["x"], d["W1"], d["b1"], "gelu_erf")
    unfused = F.fmlp_linear(h, d["W2"], d["b2"], "none")
    torch.cuda.synchronize()
    a, b = f64_of(fused), f64_of(unfused)
    if path == "gemm":
        assert np.array_equal(bits_of(fused), bits_of(unfused))
    else:
        # different accumulation order: agree to the final rounding
        assert np.max(np.abs(a - b)) <= 2 * bf16_ulp(np.max(np.abs(b)))


def test_decode_determinism_and_repeat():
    """The persistent kernel is bitwise reproducible and its barrier words stay
    consistent over many back-to-back calls on one workspace."""
    w = datagen.workload("decode1")
    t = datagen.make_inputs(w, seed=0)
    d = _dev_inputs(t)
    ws = F.workspace_for(DEV, F.fmlp_mlp2_workspace_size(16, 4096, 4096, 4096))
    print("case decode repeat x50", flush=True)
    first = bits_of(_run(d, w.act, "decode", ws))
    gen0 = int(ws[:4].view(torch.int32).item())
    for _ in range(50):
        y = F.fmlp_mlp2(d["x"], d["W1"], d["b1"], d["W2"], d["b2"], w.act, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(y), first)
    hdr = ws[:12].view(torch.int32).cpu().numpy()
    assert hdr[0] == gen0 + 50, hdr          # one barrier generation per call
    assert hdr[2] == 0, hdr                  # no wait gave up


@pytest.mark.parametrize("K,H,N", [
    (64, 64, 4096),     # second layer wider than the first: not every block owns a layer-1 tile
    (256, 4104, 520),   # hidden size just past the word-flag limit
    (256, 4096, 520),   # at the limit: word-flag publish
    (512, 200, 40),     # word-flag publish, ragged tiles
    (2048, 1024, 512),  # word-flag publish on 64 blocks, half of them without a layer-2 tile
    (1024, 4096, 8192), # word-flag publish, two layer-2 tiles per block
    (1024, 4096, 520),  # word-flag publish, one-stage layer-1 tiles, most blocks own no layer-2 tile
])
def test_decode_one_token_publish_paths(K, H, N):
    """At one token the hidden vector is published either as epoch-tagged
    words or with per-block flags, depending on the shape; both must give the
    oracle's result and advance the barrier generation once per call."""
    rng = np.random.default_rng(K + H + N)
    t = {"x": rand_bf16(rng, (1, K)),
         "W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"), "b1": rand_bf16(rng, (H,), 0.2, "uniform"),
         "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"), "b2": rand_bf16(rng, (N,), 0.2, "uniform")}
    d = _dev_inputs(t)
    ws = F.workspace_for(DEV, F.fmlp_mlp2_workspace_size(1, K, H, N))
    print(f"case decode one-token publish K={K} H={H} N={N}", flush=True)
    gen0 = int(ws[:4].view(torch.int32).item())
    for _ in range(3):
        y = _run(d, "gelu_tanh", "decode", ws)
    ref = oracle.mlp2(*(f64_of_bits(t[k]) for k in ("x", "W1", "b1", "W2", "b2")), "gelu_tanh")
    assert_parity(y, ref, f"decode one token {K}/{H}/{N}")
    hdr = ws[:12].view(torch.int32).cpu().numpy()
    assert hdr[0] == gen0 + 3, hdr
    assert hdr[2] == 0, hdr


@pytest.mark.parametrize("M", [1, 16])
def test_decode_no_stale_hidden_vector(M):
    """Back-to-back persistent calls on alternating inputs into one output
    buffer: if a block read another XCD's h before it was visible (or a stale
    copy from the previous call), the result would carry the other input's h."""
    rng = np.random.default_rng(77 + M)
    K, H, N = 1024, 4096, 2048
    W1 = rand_bf16(rng, (H, K), K ** -0.5, "uniform")
    b1 = rand_bf16(rng, (H,), 0.2, "uniform")
    W2 = rand_bf16(rng, (N, H), H ** -0.5, "uniform")
    b2 = rand_bf16(rng, (N,), 0.2, "uniform")
    xs = [rand_bf16(rng, (M, K)), rand_bf16(rng, (M, K))]
    dW = {k: to_dev(v) for k, v in (("W1", W1), ("b1", b1), ("W2", W2), ("b2", b2))}
    dx = [to_dev(x) for x in xs]
    ws = F.workspace_for(DEV, F.fmlp_mlp2_workspace_size(M, K, H, N))
    outs = [torch.empty(M, N, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    print(f"case decode alternating inputs M={M}", flush=True)
    with F.force_path("decode"):
        want = []
        for i in range(2):
            F.fmlp_mlp2(dx[i], dW["W1"], dW["b1"], dW["W2"], dW["b2"], "gelu_erf", out=outs[i], workspace=ws)
            torch.cuda.synchronize()
            want.append(bits_of(outs[i]))
            ref = oracle.mlp2(f64_of_bits(xs[i]), f64_of_bits(W1), f64_of_bits(b1), f64_of_bits(W2),
                              f64_of_bits(b2), "gelu_erf")
            assert_parity(outs[i], ref, f"alternating input {i}")
        assert not np.array_equal(want[0], want[1])
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        for it in range(200):
            F.fmlp_mlp2(dx[it % 2], dW["W1"], dW["b1"], dW["W2"], dW["b2"], "gelu_erf", out=y, workspace=ws)
            if it % 20 == 19 or it < 4:
                torch.cuda.synchronize()
                assert np.array_equal(bits_of(y), want[it % 2]), f"iteration {it}"
    torch.cuda.synchronize()
    assert F.barrier_timeouts(ws) == 0
