"""The CPU oracle checked against hand examples, closed forms, invariants and brute
force (see tests/_pins.py for what each pin fixes)."""
import numpy as np
import pytest

from oracle import qkv_oracle
from tests import _pins
import workloads


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(qkv_oracle)


def _bf16_check(gpu_like, ref, tol):
    err = np.abs(gpu_like - ref) / (1.0 + np.abs(ref))
    return float(err.max())


def test_wrong_theta_is_visible_at_bf16_tolerance():
    """A path that used the other workload's theta must fail the 2e-2 parity check:
    mid-frequency pairs at positions in the thousands turn by visibly different angles."""
    wl = workloads.WORKLOADS[3].with_tokens(1, 4096)
    wl = workloads.Workload(**{**wl.__dict__, "hidden": 256, "num_q_heads": 2, "num_kv_heads": 1})
    inp = workloads.make_inputs(wl, seed=77)
    args = [inp["x"].double().numpy(), inp["w_norm"].double().numpy(), inp["w_qkv"].double().numpy(),
            None, inp["pos"].numpy()]
    good = qkv_oracle.qkv_forward(*args, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps, 5e5)
    bad = qkv_oracle.qkv_forward(*args, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps, 1e4)
    assert _bf16_check(bad[0], good[0], 2e-2) > 2e-2
    assert _bf16_check(bad[1], good[1], 2e-2) > 2e-2
    np.testing.assert_array_equal(bad[2], good[2])


def test_unnormalised_path_is_visible_with_scaled_rows():
    """Rows scaled by 10^U(-2,2) make a path that skipped the normalisation fail at
    bf16 tolerance (with x ~ N(0,1) alone, 1/rms is within about 1% of 1)."""
    rng = np.random.default_rng(5)
    T, H, nq, nkv, d = 64, 512, 2, 1, 128
    N = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, H)) * 10.0 ** rng.uniform(-2, 2, size=(T, 1))
    w = 1 + 0.1 * rng.standard_normal(H)
    W = 0.02 * rng.standard_normal((H, N))
    pos = np.arange(T)
    good = qkv_oracle.qkv_forward(x, w, W, None, pos, nq, nkv, d, 1e-6, 1e4)
    y = qkv_oracle.project(x * w[None, :], W, None)
    assert _bf16_check(y[:, (nq + nkv) * d:], good[2], 2e-2) > 2e-2


def test_rows_subset_matches_full():
    wl = workloads.WORKLOADS[1]
    inp = workloads.make_inputs(wl)
    a = [inp["x"].double().numpy(), inp["w_norm"].double().numpy(), inp["w_qkv"].double().numpy(),
         None, inp["pos"].numpy(), wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps, wl.rope_theta]
    full = qkv_oracle.qkv_forward(*a)
    rows = np.array([0, 3, 15])
    sub = qkv_oracle.qkv_forward_rows(rows, *a)
    for f, s in zip(full, sub):
        np.testing.assert_array_equal(f[rows], s)
