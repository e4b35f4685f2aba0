"""Workload shapes and algorithmic FLOP/byte counters against the numbers the
pages print (tests/golden/page_numbers.json, each entry cited)."""
import json
import os

import datagen as dg

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_geglu_tokens_flattened():
    g = G["geglu_tokens"]
    assert g["batch"] * g["seq"] == g["value"] == dg.workload("geglu768").M


def test_geglu_gemm_flops_match_page():
    g = G["geglu_gemm_gflop"]
    w = dg.workload("geglu768")
    assert (w.M, w.K, w.H) == (g["M"], g["K"], g["N"])
    one = 2 * w.M * w.K * w.H
    assert one == 38_654_705_664
    assert abs(one / 1e9 - g["value_approx"]) <= g["rel_tol"] * g["value_approx"]
    assert w.flops == 3 * one          # gate, up, down: same count each


def test_geglu_intermediate_bytes_match_page():
    g = G["geglu_intermediate_mb"]
    r, c = g["shape"]
    nbytes = r * c * 2
    assert nbytes == 50_331_648
    assert abs(nbytes / 1e6 - g["value_approx"]) <= g["rel_tol"] * g["value_approx"]


def test_linear_profile_shape_is_tiny_first_layer():
    g = G["linear_profile_shape"]
    w = dg.workload("tiny")
    assert (w.M, w.K, w.H) == (g["batch"], g["in_dim"], g["out_dim"])
    assert [w.H, w.K] == g["weight_shape"]


def test_h100_throughput_is_inverse_latency():
    # the reading taken of the page's table: its throughput rows are 1/latency
    g = G["h100_mlp_latency_us"]
    assert int(1e6 / g["unfused"]) == g["throughput_unfused_per_s"]
    assert int(1e6 / g["fused"]) == g["throughput_fused_per_s"]
    assert (g["launches_unfused"], g["launches_fused"]) == (3, 1)


def test_algorithmic_counts():
    assert dg.workload("tiny").flops == 8_388_608 and dg.workload("tiny").bytes == 139_456
    assert dg.workload("decode1").flops == 67_108_864 and dg.workload("decode1").bytes == 67_141_632
    assert dg.workload("decode16").bytes == 67_387_392
    assert dg.workload("geglu768").flops == 115_964_116_992
    assert dg.workload("large1").flops == 1_409_286_144
    assert dg.workload("large4096").flops == 5_772_436_045_824
    m = dg.workload("moe")
    assert m.flops == 2_886_218_022_912
    assert m.weight_bytes == 8 * 3 * 4096 * 14336 * 2


def test_backward_counts_are_twice_the_forward_products():
    for name in ("geglu768", "large4096"):
        f, b = dg.workload(name), dg.workload(name + "_bwd")
        assert (b.M, b.K, b.H, b.N, b.family) == (f.M, f.K, f.H, f.N, f.family)
        assert b.flops == 2 * f.flops
        assert b.bytes == 2 * 3 * 2 * f.K * f.H + 3 * 2 * f.M * f.K
