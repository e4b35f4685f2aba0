"""fp64 CPU oracle for the fused feed-forward path (test infrastructure only).

Importable only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  It shares no code with the GPU library (gemm_epilogue_bf16_amd), and the
GPU library never imports it.
"""
from .fmlp_oracle import (  # noqa: F401
    ACTS,
    activation,
    geglu,
    gelu_erf,
    gelu_tanh,
    glu,
    linear,
    mlp2,
    moe_geglu,
    moe_glu,
    moe_router,
    relu,
    route_topk,
    silu,
)
