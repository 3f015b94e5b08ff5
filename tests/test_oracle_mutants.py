"""Planted mistakes: each is a plausible slip in an implementation of the chain,
applied to a copy of the oracle's source on the CPU.  The pins must catch every one."""
import importlib.util
import os
import types

import pytest

from tests import _pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qkv_oracle.py")

MUTANTS = {
    "eps_outside_sqrt": [("1.0 / np.sqrt(mean_sq + eps)", "1.0 / np.sqrt(mean_sq) + eps")],
    "eps_dropped": [("1.0 / np.sqrt(mean_sq + eps)", "1.0 / np.sqrt(mean_sq)")],
    "sum_not_mean": [("np.mean(x * x, axis=-1)", "np.sum(x * x, axis=-1)")],
    "mean_over_head_slice": [("np.mean(x * x, axis=-1)", "np.mean(x[:, :16] * x[:, :16], axis=-1)")],
    "weight_dropped": [("* w_norm[None, :]", "* 1.0")],
    "one_plus_weight": [("* w_norm[None, :]", "* (1.0 + w_norm[None, :])")],
    "weight_transposed_use": [("@ np.asarray(w_qkv, dtype=np.float64)", "@ np.asarray(w_qkv, dtype=np.float64).T")],
    "bias_dropped": [("y = y + np.asarray(bias, dtype=np.float64)[None, :]", "y = y")],
    "bias_after_rotation": [
        ("y = project(a, w_qkv, bias)", "y = project(a, w_qkv, None)"),
        ("    return q, k, v\n",
         "    if bias is not None:\n        bb = np.asarray(bias, dtype=np.float64)\n"
         "        q = q + bb[None, :n_q]\n        k = k + bb[None, n_q:n_q + n_kv]\n"
         "        v = v + bb[None, n_q + n_kv:]\n    return q, k, v\n")],
    "rotation_sign": [("u * c - v * s, v * c + u * s", "u * c + v * s, v * c - u * s")],
    "interleaved_pairs": [("u, v = heads[..., :half], heads[..., half:]", "u, v = heads[..., 0::2], heads[..., 1::2]")],
    "cos_sin_swapped": [("c, s = np.cos(phi), np.sin(phi)", "s, c = np.cos(phi), np.sin(phi)")],
    "freq_exponent_halved": [("-2.0 * i / head_dim", "-1.0 * i / head_dim")],
    "freq_inverted": [("np.power(float(theta), -2.0 * i / head_dim)", "np.power(float(theta), 2.0 * i / head_dim)")],
    "position_is_token_index": [("np.asarray(pos, dtype=np.float64)[:, None]",
                                 "np.arange(len(pos), dtype=np.float64)[:, None]")],
    "v_rotated": [("v = y[:, n_q + n_kv:].copy()", "v = rope(y[:, n_q + n_kv:], pos, head_dim, theta)")],
    "k_not_rotated": [("k = rope(y[:, n_q:n_q + n_kv], pos, head_dim, theta)", "k = y[:, n_q:n_q + n_kv].copy()")],
    "q_not_rotated": [("q = rope(y[:, :n_q], pos, head_dim, theta)", "q = y[:, :n_q].copy()")],
    "cache_slot_wraps": [("if 0 <= s < out.shape[0]:", "s = s % out.shape[0]\n        if True:")],
    "cache_slot_off_by_one": [("out[s] = rows[t]", "out[(s + 1) % out.shape[0]] = rows[t]")],
    "cache_cleared": [("out = np.array(cache, dtype=np.float64, copy=True)",
                       "out = np.zeros_like(np.asarray(cache, dtype=np.float64))")],
    "cache_token_order_reversed": [("out[s] = rows[t]", "out[s] = rows[slots.shape[0] - 1 - t]")],
    "swiglu_gate_up_swapped": [("gate, up = y[:, :inter], y[:, inter:]", "up, gate = y[:, :inter], y[:, inter:]")],
    "swiglu_sigmoid_only": [("return silu(gate) * up", "return up / (1.0 + np.exp(-gate))")],
    "swiglu_silu_sign": [("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))")],
    "swiglu_no_norm": [("act = rms_norm(x, w_norm, eps)",
                        "act = np.asarray(x, dtype=np.float64) * np.asarray(w_norm, dtype=np.float64)")],
    "swiglu_interleaved_halves": [("gate, up = y[:, :inter], y[:, inter:]", "gate, up = y[:, 0::2], y[:, 1::2]")],
    "bwd_rotation_not_inverted": [("[gu * c + gv_ * s, gv_ * c - gu * s]", "[gu * c - gv_ * s, gv_ * c + gu * s]")],
    "bwd_norm_term_dropped": [("- (r ** 3 / H)[:, None] * x * inner[:, None]", "")],
    "bwd_norm_weight_missing_in_inner": [("inner = np.sum(ga * w[None, :] * x, axis=1)", "inner = np.sum(ga * x, axis=1)")],
    "bwd_dw_without_r": [("dw = np.sum(ga * x * r[:, None], axis=0)", "dw = np.sum(ga * x, axis=0)")],
    "bwd_dW_from_rotated_grads": [("dW = a.T @ gy", "dW = a.T @ np.concatenate([np.asarray(gq), np.asarray(gk), "
                                                    "np.asarray(gv)], axis=1)")],
    "bwd_scale_no_sqrt": [("sq = lambda m: np.sqrt(np.maximum(m, 0.0))", "sq = lambda m: np.maximum(m, 0.0)")],
    "bwd_scale_abs_sum_for_dW": [("sq((a * a).T @ (gy * gy))", "np.abs(a).T @ np.abs(gy)")],
    "bwd_scale_dx_norm_part_dropped": [
        ("\n                  + (r ** 3 / H)[:, None] * np.abs(x) * sq(np.sum((ga * w[None, :] * x) ** 2, axis=1))[:, None],",
         ",")],
    "bwd_scale_dw_without_r": [("sq(np.sum((ga * x * r[:, None]) ** 2, axis=0))", "sq(np.sum((ga * x) ** 2, axis=0))")],
    "bwd_scale_db_plain_sum": [("sq(np.sum(gy * gy, axis=0))", "np.abs(np.sum(gy, axis=0))")],
    "k_v_swapped": [("k = rope(y[:, n_q:n_q + n_kv], pos, head_dim, theta)",
                     "k = rope(y[:, n_q + n_kv:], pos, head_dim, theta)"),
                    ("v = y[:, n_q + n_kv:].copy()", "v = y[:, n_q:n_q + n_kv].copy()")],
}


def _mutant(subs):
    with open(ORACLE_SRC, encoding="utf-8") as f:
        src = f.read()
    for old, new in subs:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("qkv_oracle_mutant")
    exec(compile(src, "qkv_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(MUTANTS[name])
    caught = []
    for pin in _pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an exception (shape error, assertion) counts as caught
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    mod = _mutant([])
    for pin in _pins.ALL_PINS:
        pin(mod)
