"""The decode workspace on the GPU: the FP8 calls and the bf16 one-launch
decode calls share one workspace in any order, a header zeroed between calls
is harmless (every launch tags its h words and flags with a fresh epoch), and
the generation word moves by exactly one per one-launch decode call."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bits_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu


def _mlp2_inputs(rng, K, H, N):
    return {"W1": rand_bf16(rng, (H, K), K ** -0.5, "uniform"), "b1": rand_bf16(rng, (H,), 0.2, "uniform"),
            "W2": rand_bf16(rng, (N, H), H ** -0.5, "uniform"), "b2": rand_bf16(rng, (N,), 0.2, "uniform")}


def _ref(x, t, act):
    return oracle.mlp2(f64_of_bits(x), *(f64_of_bits(t[k]) for k in ("W1", "b1", "W2", "b2")), act)


def test_fp8_call_between_decode_calls_on_the_default_workspace():
    """A one-token bf16 decode call (word-flag publish: H = 4096), then a
    one-token two-layer FP8 call with ReLU at H = 4096 on the same cached
    workspace (one launch: it advances the same generation with the same
    word protocol), then the bf16 call again with a new x; then the FP8 call
    forced to its two-launch form, which keeps its h after the header and
    leaves the generation alone."""
    rng = np.random.default_rng(4096)
    K, H, N = 256, 4096, 512
    t = _mlp2_inputs(rng, K, H, N)
    d = {k: to_dev(v) for k, v in t.items()}
    xs = [rand_bf16(rng, (1, K)) for _ in range(2)]
    ws = F.workspace_for(DEV, max(F.fmlp_mlp2_workspace_size(1, K, H, N),
                                  int(F.lib().fmlp_w8_workspace_size(1, H))))
    q1, s1 = datagen.e4m3_weights(rng, H, K, K ** -0.5)
    q2, s2 = datagen.e4m3_weights(rng, N, H, H ** -0.5)
    dq = [torch.from_numpy(a).to(DEV) for a in (q1, s1, q2, s2)]
    print("case bf16 decode / fp8 mlp2 / bf16 decode on one workspace", flush=True)
    gen0 = F.decode_generation(ws)
    tmo0 = F.barrier_timeouts(ws)
    y0 = F.fmlp_mlp2(to_dev(xs[0]), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(y0, _ref(xs[0], t, "gelu_erf"), "bf16 decode, first x")
    assert F.decode_generation(ws) == (gen0 + 1) & 0xFFFFFFFF
    y8 = F.fmlp_mlp2_w8(to_dev(xs[1]), dq[0], dq[1], d["b1"], dq[2], dq[3], d["b2"], "relu")
    torch.cuda.synchronize()
    ref8 = oracle.mlp2_w8(f64_of_bits(xs[1]), q1, s1, f64_of_bits(t["b1"]), q2, s2, f64_of_bits(t["b2"]), "relu")
    assert_parity(y8, ref8, "fp8 mlp2 relu")
    assert F.decode_generation(ws) == (gen0 + 2) & 0xFFFFFFFF
    y1 = F.fmlp_mlp2(to_dev(xs[1]), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(y1, _ref(xs[1], t, "gelu_erf"), "bf16 decode, second x")
    assert F.decode_generation(ws) == (gen0 + 3) & 0xFFFFFFFF
    with F.force_path("gemm"):
        y8 = F.fmlp_mlp2_w8(to_dev(xs[0]), dq[0], dq[1], d["b1"], dq[2], dq[3], d["b2"], "relu")
    torch.cuda.synchronize()
    ref8 = oracle.mlp2_w8(f64_of_bits(xs[0]), q1, s1, f64_of_bits(t["b1"]), q2, s2, f64_of_bits(t["b2"]), "relu")
    assert_parity(y8, ref8, "fp8 mlp2 relu, two launches")
    assert F.decode_generation(ws) == (gen0 + 3) & 0xFFFFFFFF, "the two-launch FP8 form wrote the decode header"
    assert F.barrier_timeouts(ws) == tmo0


@pytest.mark.parametrize("M,K,H,N", [(1, 256, 4096, 512),    # word-flag publish (h words carry the epoch)
                                     (1, 256, 4104, 512),    # per-block flags at one token
                                     (16, 512, 2048, 1024)])  # per-block flags at 16 tokens
def test_header_zeroed_between_calls(M, K, H, N):
    """Zeroing only the 8 KB header between two calls with different x restarts
    the generation while the previous call's h words are still in the
    workspace; the second call must still compute from its own x."""
    rng = np.random.default_rng(M * 7 + H)
    t = _mlp2_inputs(rng, K, H, N)
    d = {k: to_dev(v) for k, v in t.items()}
    xs = [rand_bf16(rng, (M, K)) for _ in range(2)]
    ws = torch.zeros(F.fmlp_mlp2_workspace_size(M, K, H, N), dtype=torch.uint8, device=DEV)
    print(f"case header zeroed between calls M={M} K={K} H={H} N={N}", flush=True)
    outs = []
    with F.force_path("decode"):
        for i in range(2):
            y = F.fmlp_mlp2(to_dev(xs[i]), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_tanh", workspace=ws)
            torch.cuda.synchronize()
            assert F.decode_generation(ws) == 1
            assert F.barrier_timeouts(ws) == 0
            assert_parity(y, _ref(xs[i], t, "gelu_tanh"), f"call {i} after a zeroed header")
            outs.append(bits_of(y))
            ws[:8192].zero_()
            torch.cuda.synchronize()
    assert not np.array_equal(outs[0], outs[1])


def test_generation_moves_once_per_call_and_replays_differ():
    """Thirty back-to-back one-token calls alternating two inputs on one
    workspace: each output matches its own input, the generation advances by
    thirty and no wait gave up."""
    rng = np.random.default_rng(30)
    K, H, N = 512, 4096, 256
    t = _mlp2_inputs(rng, K, H, N)
    d = {k: to_dev(v) for k, v in t.items()}
    xs = [rand_bf16(rng, (1, K)) for _ in range(2)]
    dx = [to_dev(x) for x in xs]
    ws = torch.zeros(F.fmlp_mlp2_workspace_size(1, K, H, N), dtype=torch.uint8, device=DEV)
    print("case generation x30", flush=True)
    want = []
    for i in range(2):
        y = F.fmlp_mlp2(dx[i], d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(y, _ref(xs[i], t, "gelu_erf"), f"input {i}")
        want.append(bits_of(y))
    outs = [torch.empty(1, N, dtype=torch.bfloat16, device=DEV) for _ in range(30)]
    for i in range(30):
        F.fmlp_mlp2(dx[i % 2], d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", out=outs[i], workspace=ws)
    torch.cuda.synchronize()
    for i in range(30):
        assert np.array_equal(bits_of(outs[i]), want[i % 2]), f"call {i}"
    assert F.decode_generation(ws) == 32
    assert F.barrier_timeouts(ws) == 0


def test_backward_calls_leave_the_decode_header_alone():
    """A backward call between two one-token decode calls on the same cached
    workspace: the generation still moves by one per decode call and the
    timeout count stays put."""
    rng = np.random.default_rng(8)
    K, H, N = 256, 4096, 512
    t = _mlp2_inputs(rng, K, H, N)
    d = {k: to_dev(v) for k, v in t.items()}
    x = rand_bf16(rng, (1, K))
    ws = F.workspace_for(DEV, max(F.fmlp_mlp2_workspace_size(1, K, H, N),
                                  int(F.lib().fmlp_linear_bwd_workspace_size(64, K, H))))
    print("case decode / linear_bwd / decode on one workspace", flush=True)
    gen0, tmo0 = F.decode_generation(ws), F.barrier_timeouts(ws)
    F.fmlp_mlp2(to_dev(x), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    xb = to_dev(rand_bf16(rng, (64, K)))
    F.fmlp_linear_bwd(xb, d["W1"], d["b1"], "gelu_erf", to_dev(rand_bf16(rng, (64, H))), workspace=ws)
    y = F.fmlp_mlp2(to_dev(x), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(y, _ref(x, t, "gelu_erf"), "decode after a backward call")
    assert F.decode_generation(ws) == (gen0 + 2) & 0xFFFFFFFF
    assert F.barrier_timeouts(ws) == tmo0


@pytest.mark.parametrize("M,K,H,N", [(1, 512, 4096, 256), (16, 512, 2048, 1024), (1, 256, 4104, 512)])
def test_cooperative_decode_launch(M, K, H, N):
    """The opt-in cooperative launch of the one-launch decode: same results as
    the plain launch (bitwise), the generation moves once per call and no
    wait gives up; and the one-token FP8 two-layer launch the same way."""
    rng = np.random.default_rng(M * 5 + H)
    t = _mlp2_inputs(rng, K, H, N)
    d = {k: to_dev(v) for k, v in t.items()}
    x = rand_bf16(rng, (M, K))
    ws = torch.zeros(max(F.fmlp_mlp2_workspace_size(M, K, H, N), int(F.lib().fmlp_w8_workspace_size(M, H))),
                     dtype=torch.uint8, device=DEV)
    print(f"case cooperative decode M={M} K={K} H={H} N={N}", flush=True)
    plain = F.fmlp_mlp2(to_dev(x), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    torch.cuda.synchronize()
    gen0 = F.decode_generation(ws)
    with F.cooperative_decode():
        coop = F.fmlp_mlp2(to_dev(x), d["W1"], d["b1"], d["W2"], d["b2"], "gelu_erf", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(coop, _ref(x, t, "gelu_erf"), "cooperative launch")
    assert np.array_equal(bits_of(coop), bits_of(plain))
    assert F.decode_generation(ws) == (gen0 + 1) & 0xFFFFFFFF
    assert F.barrier_timeouts(ws) == 0
    if M == 1 and H % 16 == 0 and H <= 4096:
        q1, s1 = datagen.e4m3_weights(rng, H, K, K ** -0.5)
        q2, s2 = datagen.e4m3_weights(rng, N, H, H ** -0.5)
        dq = [torch.from_numpy(a).to(DEV) for a in (q1, s1, q2, s2)]
        y8 = F.fmlp_mlp2_w8(to_dev(x), dq[0], dq[1], d["b1"], dq[2], dq[3], d["b2"], "silu", workspace=ws)
        with F.cooperative_decode():
            y8c = F.fmlp_mlp2_w8(to_dev(x), dq[0], dq[1], d["b1"], dq[2], dq[3], d["b2"], "silu", workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(y8c), bits_of(y8))
        assert F.decode_generation(ws) == (gen0 + 3) & 0xFFFFFFFF
        assert F.barrier_timeouts(ws) == 0
