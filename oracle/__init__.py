"""fp64 CPU oracle for the fused feed-forward path (test infrastructure only).

Importable only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  It shares no code with the GPU library (gemm_epilogue_bf16_amd), and the
GPU library never imports it.
"""
from .fmlp_oracle import (  # noqa: F401
    ACTS,
    act_grad,
    activation,
    dequant_w8,
    e4m3_decode,
    geglu,
    gelu_erf,
    gelu_tanh,
    glu,
    glu_bwd,
    glu_bwd_sampled,
    glu_w8,
    linear,
    linear_bwd,
    linear_w8,
    mlp2,
    mlp2_bwd,
    mlp2_w8,
    moe_geglu,
    moe_glu,
    moe_router,
    relu,
    route_topk,
    silu,
)
