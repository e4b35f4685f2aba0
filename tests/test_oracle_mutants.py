"""Plant plausible mistakes in the oracle (on the CPU) and confirm that at least
one pin catches each.  This is what makes the pins worth trusting: a dropped
term, a wrong sign or index, a transposed operand, a swapped gate/up, or the
wrong GELU variant must all fail."""
import numpy as np
import pytest
from scipy.special import erfc

import oracle.fmlp_oracle as fo
from oracle_pins import ALL_CHECKS

_orig_linear = fo.linear
_orig_activation = fo.activation
_orig_gelu_erf = fo.gelu_erf
_orig_gelu_tanh = fo.gelu_tanh
_orig_moe = fo.moe_geglu
_orig_glu = fo.glu
_orig_route_topk = fo.route_topk


def _linear_no_bias(x, W, b=None, act="none"):
    return _orig_linear(x, W, None, act)


def _linear_bias_sub(x, W, b=None, act="none"):
    z = np.asarray(x, float) @ np.asarray(W, float).T
    if b is not None:
        z = z - np.asarray(b, float)[None, :]
    return fo.activation(z, act)


def _linear_square_transposed(x, W, b=None, act="none"):
    x = np.asarray(x, float)
    W = np.asarray(W, float)
    z = x @ W if W.shape[0] == W.shape[1] else x @ W.T
    if b is not None:
        z = z + np.asarray(b, float)[None, :]
    return fo.activation(z, act)


def _linear_act_before_bias(x, W, b=None, act="none"):
    z = fo.activation(np.asarray(x, float) @ np.asarray(W, float).T, act)
    if b is not None:
        z = z + np.asarray(b, float)[None, :]
    return z


def _gelu_erf_sign(z):
    z = np.asarray(z, float)
    return 0.5 * z * erfc(z * np.sqrt(0.5))


def _gelu_tanh_no_cubic(z):
    z = np.asarray(z, float)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2 / np.pi) * z))


def _gelu_tanh_wrong_const(z):
    z = np.asarray(z, float)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(1 / np.pi) * (z + 0.044715 * z ** 3)))


def _act_names_swapped(z, act):
    return _orig_activation(z, {"gelu_erf": "gelu_tanh", "gelu_tanh": "gelu_erf"}.get(act, act))


def _geglu_swapped(x, Wg, Wu, Wd):
    return _orig_linear(fo.gelu_tanh(_orig_linear(x, Wu)) * _orig_linear(x, Wg), Wd)


def _geglu_no_gelu(x, Wg, Wu, Wd):
    return _orig_linear(_orig_linear(x, Wg) * _orig_linear(x, Wu), Wd)


def _geglu_wrong_act(x, Wg, Wu, Wd):
    return _orig_linear(fo.gelu_erf(_orig_linear(x, Wg)) * _orig_linear(x, Wu), Wd)


def _silu_is_sigmoid(z):
    z = np.asarray(z, float)
    return 1.0 / (1.0 + np.exp(-z))


def _silu_double_slope(z):
    z = np.asarray(z, float)
    return z / (1.0 + np.exp(-2.0 * z))


def _relu_leaky(z):
    z = np.asarray(z, float)
    return np.where(z > 0, z, 0.01 * z)


def _glu_ignores_gate_act(x, Wg, Wu, Wd, gate_act):
    return _orig_glu(x, Wg, Wu, Wd, "gelu_tanh")


def _glu_gate_up_swapped(x, Wg, Wu, Wd, gate_act):
    return _orig_glu(x, Wu, Wg, Wd, gate_act)


def _route_softmax_over_all(logits, top_k):
    lg = np.asarray(logits, float)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :top_k]
    e = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), np.take_along_axis(p, ids, axis=1)


def _route_ties_to_higher(logits, top_k):
    lg = np.asarray(logits, float)[:, ::-1]
    ids, gw = _orig_route_topk(lg, top_k)
    return (lg.shape[1] - 1 - ids).astype(np.int32), gw


def _route_smallest(logits, top_k):
    return _orig_route_topk(-np.asarray(logits, float), top_k)


def _mlp2_act_twice(x, W1, b1, W2, b2, act):
    return _orig_linear(_orig_linear(x, W1, b1, act), W2, b2, act)


def _mlp2_drop_b2(x, W1, b1, W2, b2, act):
    return _orig_linear(_orig_linear(x, W1, b1, act), W2, None, "none")


def _moe_unweighted(x, ids, gw, ew):
    return _orig_moe(x, ids, np.ones_like(np.asarray(gw, float)), ew)


def _moe_first_slot(x, ids, gw, ew):
    ids = np.asarray(ids)
    return _orig_moe(x, ids[:, :1], np.asarray(gw, float)[:, :1], ew)


def _moe_dedup(x, ids, gw, ew):
    # overwrites instead of accumulating a token routed twice to one expert
    x = np.asarray(x, float)
    ids = np.asarray(ids)
    gw = np.asarray(gw, float)
    get = ew if callable(ew) else (lambda e: ew[e])
    y = np.zeros_like(x)
    for e in np.unique(ids):
        tok, slot = np.nonzero(ids == e)
        y[tok] += gw[tok, slot][:, None] * fo.geglu(x[tok], *get(int(e)))
    return y


_orig_e4m3 = fo.e4m3_decode
_orig_dequant = fo.dequant_w8


def _e4m3_bias8(codes):
    return _orig_e4m3(codes) * 0.5


def _e4m3_subnormal_as_normal(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = _orig_e4m3(c)
    e = (c.astype(np.int64) >> 3) & 15
    m = (c & 7).astype(np.float64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    return np.where(e == 0, sign * (1.0 + m / 8.0) * 2.0 ** -7, v)


def _e4m3_no_nan(codes):
    c = np.asarray(codes, dtype=np.uint8)
    v = _orig_e4m3(c)
    return np.where((c & 0x7F) == 0x7F, np.where(c & 0x80, -480.0, 480.0), v)


def _dequant_column_scale(Wq, scale):
    Wq = np.asarray(Wq, dtype=np.uint8)
    return fo.e4m3_decode(Wq) * np.asarray(scale, float)[None, :]


def _dequant_ignores_scale(Wq, scale):
    return fo.e4m3_decode(np.asarray(Wq, dtype=np.uint8))


_orig_act_grad = fo.act_grad
_orig_linear_bwd = fo.linear_bwd
_orig_glu_bwd = fo.glu_bwd


def _grad_erf_no_density_term(z, act):
    if act == "gelu_erf":
        return 0.5 * erfc(-np.asarray(z, float) * np.sqrt(0.5))
    return _orig_act_grad(z, act)


def _grad_tanh_no_cubic_term(z, act):
    if act == "gelu_tanh":
        z = np.asarray(z, float)
        t = np.tanh(np.sqrt(2 / np.pi) * (z + 0.044715 * z ** 3))
        return 0.5 * (1 + t) + 0.5 * z * (1 - t * t) * np.sqrt(2 / np.pi)
    return _orig_act_grad(z, act)


def _grad_silu_is_sigmoid(z, act):
    if act == "silu":
        return 1.0 / (1.0 + np.exp(-np.asarray(z, float)))
    return _orig_act_grad(z, act)


def _grad_relu_one_at_zero(z, act):
    if act == "relu":
        return np.where(np.asarray(z, float) >= 0, 1.0, 0.0)
    return _orig_act_grad(z, act)


def _grad_names_swapped(z, act):
    return _orig_act_grad(z, {"gelu_erf": "gelu_tanh", "gelu_tanh": "gelu_erf"}.get(act, act))


def _linear_bwd_no_act_grad(x, W, b, act, dy):
    return _orig_linear_bwd(x, W, b, "none", dy)


def _linear_bwd_dW_of_dy(x, W, b, act, dy):
    dx, dW, db = _orig_linear_bwd(x, W, b, act, dy)
    return dx, np.asarray(dy, float).T @ np.asarray(x, float), db


def _linear_bwd_dx_transposed_W(x, W, b, act, dy):
    dx, dW, db = _orig_linear_bwd(x, W, b, act, dy)
    W = np.asarray(W, float)
    if W.shape[0] == W.shape[1]:
        z = np.asarray(x, float) @ W.T + (0 if b is None else np.asarray(b, float))
        dx = (np.asarray(dy, float) * fo.act_grad(z, act)) @ W.T
    return dx, dW, db


def _linear_bwd_db_of_dy(x, W, b, act, dy):
    dx, dW, db = _orig_linear_bwd(x, W, b, act, dy)
    return dx, dW, (None if b is None else np.asarray(dy, float).sum(axis=0))


def _glu_bwd_dg_du_swapped(x, Wg, Wu, Wd, gate_act, dy):
    dx, dWg, dWu, dWd = _orig_glu_bwd(x, Wg, Wu, Wd, gate_act, dy)
    return dx, dWu, dWg, dWd


def _glu_bwd_gate_grad_on_up(x, Wg, Wu, Wd, gate_act, dy):
    x, Wg, Wu, Wd, dy = (np.asarray(a, float) for a in (x, Wg, Wu, Wd, dy))
    g, u = x @ Wg.T, x @ Wu.T
    a = fo.activation(g, gate_act)
    dm = dy @ Wd
    dg = dm * u
    du = dm * a * fo.act_grad(g, gate_act)
    return dg @ Wg + du @ Wu, dg.T @ x, du.T @ x, dy.T @ (a * u)


def _glu_bwd_dWd_of_u(x, Wg, Wu, Wd, gate_act, dy):
    dx, dWg, dWu, dWd = _orig_glu_bwd(x, Wg, Wu, Wd, gate_act, dy)
    return dx, dWg, dWu, np.asarray(dy, float).T @ (np.asarray(x, float) @ np.asarray(Wu, float).T)


def _glu_bwd_dx_gate_only(x, Wg, Wu, Wd, gate_act, dy):
    x, Wg, Wu, Wd, dy = (np.asarray(a, float) for a in (x, Wg, Wu, Wd, dy))
    _, dWg, dWu, dWd = _orig_glu_bwd(x, Wg, Wu, Wd, gate_act, dy)
    g, u = x @ Wg.T, x @ Wu.T
    dg = (dy @ Wd) * u * fo.act_grad(g, gate_act)
    return dg @ Wg, dWg, dWu, dWd


MUTANTS = {
    "act_grad_erf_without_z_phi": ("act_grad", _grad_erf_no_density_term),
    "act_grad_tanh_without_cubic_term": ("act_grad", _grad_tanh_no_cubic_term),
    "act_grad_silu_is_sigmoid": ("act_grad", _grad_silu_is_sigmoid),
    "act_grad_relu_one_at_zero": ("act_grad", _grad_relu_one_at_zero),
    "act_grad_names_swapped": ("act_grad", _grad_names_swapped),
    "linear_bwd_ignores_act_grad": ("linear_bwd", _linear_bwd_no_act_grad),
    "linear_bwd_dW_from_dy": ("linear_bwd", _linear_bwd_dW_of_dy),
    "linear_bwd_dx_through_W_transposed": ("linear_bwd", _linear_bwd_dx_transposed_W),
    "linear_bwd_db_from_dy": ("linear_bwd", _linear_bwd_db_of_dy),
    "glu_bwd_dWg_dWu_swapped": ("glu_bwd", _glu_bwd_dg_du_swapped),
    "glu_bwd_gate_grad_on_up": ("glu_bwd", _glu_bwd_gate_grad_on_up),
    "glu_bwd_dWd_from_u": ("glu_bwd", _glu_bwd_dWd_of_u),
    "glu_bwd_dx_gate_path_only": ("glu_bwd", _glu_bwd_dx_gate_only),
    "linear_drops_bias": ("linear", _linear_no_bias),
    "linear_subtracts_bias": ("linear", _linear_bias_sub),
    "linear_square_W_not_transposed": ("linear", _linear_square_transposed),
    "linear_act_before_bias": ("linear", _linear_act_before_bias),
    "gelu_erf_wrong_sign": ("gelu_erf", _gelu_erf_sign),
    "gelu_tanh_is_erf": ("gelu_tanh", _orig_gelu_erf),
    "gelu_erf_is_tanh": ("gelu_erf", _orig_gelu_tanh),
    "gelu_tanh_no_cubic": ("gelu_tanh", _gelu_tanh_no_cubic),
    "gelu_tanh_wrong_const": ("gelu_tanh", _gelu_tanh_wrong_const),
    "activation_names_swapped": ("activation", _act_names_swapped),
    "geglu_gate_up_swapped": ("geglu", _geglu_swapped),
    "geglu_no_gelu": ("geglu", _geglu_no_gelu),
    "geglu_erf_gelu": ("geglu", _geglu_wrong_act),
    "mlp2_act_after_both": ("mlp2", _mlp2_act_twice),
    "mlp2_drops_b2": ("mlp2", _mlp2_drop_b2),
    "moe_ignores_gate_w": ("moe_geglu", _moe_unweighted),
    "moe_first_slot_only": ("moe_geglu", _moe_first_slot),
    "moe_overwrites_duplicates": ("moe_geglu", _moe_dedup),
    "silu_is_sigmoid": ("silu", _silu_is_sigmoid),
    "silu_double_slope": ("silu", _silu_double_slope),
    "relu_leaky": ("relu", _relu_leaky),
    "glu_ignores_gate_act": ("glu", _glu_ignores_gate_act),
    "glu_gate_up_swapped": ("glu", _glu_gate_up_swapped),
    "router_softmax_over_all_experts": ("route_topk", _route_softmax_over_all),
    "router_ties_to_higher_id": ("route_topk", _route_ties_to_higher),
    "router_picks_smallest": ("route_topk", _route_smallest),
    "e4m3_exponent_bias_8": ("e4m3_decode", _e4m3_bias8),
    "e4m3_subnormals_as_normals": ("e4m3_decode", _e4m3_subnormal_as_normal),
    "e4m3_nan_codes_finite": ("e4m3_decode", _e4m3_no_nan),
    "w8_scale_per_column": ("dequant_w8", _dequant_column_scale),
    "w8_scale_ignored": ("dequant_w8", _dequant_ignores_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fo, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(fo)
        except Exception as e:  # AssertionError or a shape error
            caught.append(f"{check.__name__}: {type(e).__name__}")
    assert caught, f"planted mistake {name!r} passed every pin"
