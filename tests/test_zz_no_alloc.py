"""fmlp_glu_noalloc, the gated block with the library's own scratch array as
its workspace, against fmlp_glu with a caller's workspace (same kernels:
bitwise equal) and against the fp64 oracle, through the C ABI: two calls in a
row, the second smaller, on the large-token and the decode paths; a shape
beyond the scratch array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import gemm_epilogue_bf16_amd as F
import oracle
from gpu_util import DEV, assert_parity, bits_of, f64_of_bits, rand_bf16, to_dev

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _abi_noalloc(d, gate_act, M, D, H, y):
    L = F.lib()
    st = L.fmlp_glu_noalloc(d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr(), F.ACT[gate_act],
                            M, D, H, y.data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
    return st


def _abi_glu(d, gate_act, M, D, H, y):
    L = F.lib()
    need = int(L.fmlp_glu_workspace_size(M, D, H))
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    st = L.fmlp_glu(d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(), d[3].data_ptr(), F.ACT[gate_act], M, D, H,
                    y.data_ptr(), ws.data_ptr(), ctypes.c_size_t(ws.numel()),
                    torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("shapes,gate_act", [
    (((300, 512, 1024), (40, 256, 520)), "gelu_tanh"),   # two-GEMM path, then a smaller one
    (((16, 1024, 2048), (1, 512, 1024)), "silu"),        # one-launch decode path, then one token
    (((8192, 768, 3072), (5, 768, 3072)), "gelu_tanh"),  # the 768/3072 workload in full, then decode
])
def test_noalloc_matches_glu(shapes, gate_act):
    F.lib()
    for i, (M, D, H) in enumerate(shapes):
        rng = np.random.default_rng(M + D + H + i)
        x = rand_bf16(rng, (M, D))
        Wg = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
        Wu = rand_bf16(rng, (H, D), D ** -0.5, "uniform")
        Wd = rand_bf16(rng, (D, H), H ** -0.5, "uniform")
        d = [to_dev(a) for a in (x, Wg, Wu, Wd)]
        print(f"case glu_noalloc call {i}: M={M} D={D} H={H} {gate_act}", flush=True)
        y_na = torch.full((M, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        assert _abi_noalloc(d, gate_act, M, D, H, y_na) == 0, F.lib().fmlp_last_error()
        torch.cuda.synchronize()
        y_ws = torch.empty(M, D, dtype=torch.bfloat16, device=DEV)
        assert _abi_glu(d, gate_act, M, D, H, y_ws) == 0
        assert np.array_equal(bits_of(y_na), bits_of(y_ws)), "noalloc and workspace results differ"
        rows = np.arange(M) if M <= 512 else np.unique(np.linspace(0, M - 1, 300).astype(int))
        ref = oracle.glu(f64_of_bits(x[rows]), f64_of_bits(Wg), f64_of_bits(Wu), f64_of_bits(Wd), gate_act)
        assert_parity(y_na[torch.from_numpy(rows).to(DEV)], ref, f"glu_noalloc {M}x{D}x{H}")


def test_noalloc_refuses_beyond_the_scratch_array():
    L = F.lib()
    M, D, H = 4096, 8192, 28672     # m alone is 235 MB
    assert int(L.fmlp_glu_workspace_size(M, D, H)) > SCRATCH
    y = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    st = L.fmlp_glu_noalloc(w.data_ptr(), w.data_ptr(), w.data_ptr(), w.data_ptr(), 2, M, D, H, y.data_ptr(),
                            torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 5   # FMLP_E_WORKSPACE
    assert "FMLP_GLU_NOALLOC_SCRATCH_BYTES" in L.fmlp_last_error().decode()
    torch.cuda.synchronize()
    assert not torch.any(y != 0)
