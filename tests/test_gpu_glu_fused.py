"""The gated block in one launch with m kept on chip (the "fused" path of
fmlp_glu / fmlp_geglu, model widths D <= 1024) against the fp64 oracle
(oracle.glu, oracle.geglu): ragged token counts (not multiples of the 64-row
block), D and H not multiples of a stage or sub-chunk, every gate activation,
one to eight parts of the hidden range (the part count follows from the token
count), the 8192-token 768/3072 GeGLU in full, bitwise determinism, agreement
with the two-launch path, and a workspace shared with the one-launch decode
(its header words untouched)."""
import numpy as np
import pytest
import torch

import datagen
import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bits_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu

ACTS = ["gelu_tanh", "gelu_erf", "silu", "relu", "none"]


def _inputs(seed, M, D, H):
    rng = np.random.default_rng(seed)
    return (rand_bf16(rng, (M, D)), rand_bf16(rng, (H, D), D ** -0.5, "uniform"),
            rand_bf16(rng, (H, D), D ** -0.5, "uniform"), rand_bf16(rng, (D, H), H ** -0.5, "uniform"))


def _parts(M, H):
    """The part count the library picks (one block per CU of a 256-CU device)."""
    m_tiles = -(-M // 64)
    subs = -(-H // 128)
    S = max(1, min(-(-256 // m_tiles), 8, subs))
    per = -(-subs // S)
    return -(-subs // per)


def _run(x, Wg, Wu, Wd, act, workspace=None):
    with F.force_path("fused"):
        y = F.fmlp_glu(*(to_dev(a) for a in (x, Wg, Wu, Wd)), act, workspace=workspace)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,D,H", [(1, 64, 128), (5, 96, 200), (63, 256, 520), (64, 8, 136), (130, 512, 1000),
                                   (257, 1024, 1024), (700, 768, 3072), (1000, 1000, 392), (3001, 320, 264)])
@pytest.mark.parametrize("act", ACTS)
def test_fused_glu_random(M, D, H, act):
    x, Wg, Wu, Wd = _inputs(M * 31 + D + H, M, D, H)
    print(f"case fused glu M={M} D={D} H={H} act={act} parts={_parts(M, H)}", flush=True)
    y = _run(x, Wg, Wu, Wd, act)
    ref = oracle.glu(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)), act)
    assert_parity(y, ref, f"fused glu {M}x{D}x{H} {act}")


@pytest.mark.parametrize("M,D,H", [(16384, 64, 384), (20000, 8, 128)])
def test_fused_glu_one_part(M, D, H):
    """256 or more token tiles: one part, no partials, bf16 y straight from the
    block."""
    assert _parts(M, H) == 1
    x, Wg, Wu, Wd = _inputs(M + D, M, D, H)
    print(f"case fused glu one part M={M} D={D} H={H}", flush=True)
    y = _run(x, Wg, Wu, Wd, "gelu_tanh")
    ref = oracle.geglu(*(f64_of_bits(a) for a in (x, Wg, Wu, Wd)))
    assert_parity(y, ref, f"fused glu {M}x{D}x{H} one part")


def test_fused_geglu768_full():
    """The 8192-token 768/3072 GeGLU workload (two parts of the hidden range),
    every output element."""
    w = datagen.workload("geglu768")
    t = datagen.make_inputs(w, seed=0)
    print(f"case {w.name} fused, full", flush=True)
    d = [to_dev(t[k]) for k in ("x", "Wg", "Wu", "Wd")]
    with F.force_path("fused"):
        y = F.fmlp_geglu(*d)
    torch.cuda.synchronize()
    ref = oracle.geglu(*(f64_of_bits(t[k]) for k in ("x", "Wg", "Wu", "Wd")))
    assert_parity(y, ref, f"{w.name} fused")


def test_fused_determinism_and_two_launch_agreement():
    M, D, H = 2000, 768, 3072
    x, Wg, Wu, Wd = _inputs(7, M, D, H)
    print("case fused determinism", flush=True)
    a = bits_of(_run(x, Wg, Wu, Wd, "gelu_tanh"))
    b = bits_of(_run(x, Wg, Wu, Wd, "gelu_tanh"))
    assert np.array_equal(a, b)
    with F.force_path("gemm"):
        y2 = F.fmlp_glu(*(to_dev(v) for v in (x, Wg, Wu, Wd)), "gelu_tanh")
    torch.cuda.synchronize()
    ref = oracle.geglu(*(f64_of_bits(v) for v in (x, Wg, Wu, Wd)))
    yf = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    assert_parity(yf, ref, "fused")
    assert_parity(y2, ref, "two launches")
    # both round m to bf16 once and y to bf16 once; they differ only in fp32
    # summation order
    diff = np.abs(yf.float().cpu().numpy() - y2.float().cpu().numpy())
    assert float(diff.max()) <= 2e-2 * float(np.abs(ref).max())


def test_fused_shares_a_workspace_with_decode():
    """A one-token decode call, then a fused call, then the decode call again
    on one workspace: the decode generation moves by one per decode call, and
    every output matches the oracle."""
    D, H = 512, 1024
    x1, Wg, Wu, Wd = _inputs(11, 1, D, H)
    xb = _inputs(12, 300, D, H)[0]
    d = [to_dev(a) for a in (Wg, Wu, Wd)]
    ws = F.workspace_for(DEV, max(F.fmlp_geglu_workspace_size(300, D, H), F.fmlp_geglu_workspace_size(1, D, H)))
    print("case decode / fused / decode on one workspace", flush=True)
    gen0, tmo0 = F.decode_generation(ws), F.barrier_timeouts(ws)
    ref1 = oracle.glu(*(f64_of_bits(a) for a in (x1, Wg, Wu, Wd)), "silu")
    y = F.fmlp_glu(to_dev(x1), *d, "silu", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(y, ref1, "decode before")
    with F.force_path("fused"):
        yb = F.fmlp_glu(to_dev(xb), *d, "silu", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(yb, oracle.glu(*(f64_of_bits(a) for a in (xb, Wg, Wu, Wd)), "silu"), "fused")
    y = F.fmlp_glu(to_dev(x1), *d, "silu", workspace=ws)
    torch.cuda.synchronize()
    assert_parity(y, ref1, "decode after")
    assert F.decode_generation(ws) == (gen0 + 2) & 0xFFFFFFFF
    assert F.barrier_timeouts(ws) == tmo0


def test_fused_rejects_wide_blocks():
    x = torch.zeros(4, 1032, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(64, 1032, dtype=torch.bfloat16, device=DEV)
    with F.force_path("fused"):
        with pytest.raises(F.FmlpError):
            F.fmlp_glu(x, W, W, W.t().contiguous(), "silu")
