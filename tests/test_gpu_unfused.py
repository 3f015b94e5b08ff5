"""The chain's steps as separate kernels (qkv_rms_norm, qkv_rope, qkv_forward_unfused)
against the oracle, through the C ABI.

Bars: the normalised activations are the oracle's to within their one rounding to the
output dtype (bf16: 2^-8 relative, its unit roundoff; fp32: 1e-6 relative); the rotation's outputs to within
that rounding plus the fp32 cos/sin error (1e-5 of the row's largest input); the unfused
forward meets the fused forward's bar, |gpu - oracle| <= tol * (1 + |oracle|) with
tol = 1e-4 (fp32) and 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import transformer_rmsnorm_row_amd as qkv
import workloads
from oracle import qkv_oracle
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL = {"fp32": 1e-6, "bf16": 2.0 ** -8 * 1.001}


def dev_inputs(inp):
    b = None if inp["bias"] is None else inp["bias"].to(DEV)
    return inp["x"].to(DEV), inp["w_norm"].to(DEV), inp["w_qkv"].to(DEV), b, inp["pos"].to(DEV)


@pytest.mark.parametrize("cid,T", [(1, None), (2, None), (4, None), (3, 300), (5, 129)])
def test_rms_norm_step(cid, T):
    wl = workloads.WORKLOADS[cid]
    if T is not None:
        wl = wl.with_tokens(1, T)
    inp = workloads.make_inputs(wl, seed=11 + cid)
    with qkv.Plan.for_workload(wl) as plan:
        x, w, _, _, _ = dev_inputs(inp)
        got = P.to_f64(plan.rms_norm(x, w))
    ref = qkv_oracle.rms_norm(P.to_f64(inp["x"]), P.to_f64(inp["w_norm"]), wl.eps)
    bound = REL[wl.dtype] * np.abs(ref) + 1e-30
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"{wl.name}: worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"


@pytest.mark.parametrize("cid,T", [(1, None), (4, None), (3, 300), (5, 129)])
def test_rope_step(cid, T):
    """Bias and rotation alone, on a seeded stand-in for the projection output."""
    wl = workloads.WORKLOADS[cid]
    if T is not None:
        wl = wl.with_tokens(1, T)
    inp = workloads.make_inputs(wl, seed=23 + cid)
    g = torch.Generator().manual_seed(401 + cid)
    y0 = torch.randn(wl.tokens, wl.n_total, generator=g).to(wl.torch_dtype)
    with qkv.Plan.for_workload(wl) as plan:
        b = None if inp["bias"] is None else inp["bias"].to(DEV)
        got = P.to_f64(plan.rope(y0.to(DEV), b, inp["pos"].to(DEV)))
    y = P.to_f64(y0)
    if inp["bias"] is not None:
        y = y + P.to_f64(inp["bias"])[None, :]
    nq, nkv = wl.n_q, wl.n_kv
    pos = P.to_f64(inp["pos"])
    ref = np.concatenate([qkv_oracle.rope(y[:, :nq], pos, wl.head_dim, wl.rope_theta),
                          qkv_oracle.rope(y[:, nq:nq + nkv], pos, wl.head_dim, wl.rope_theta),
                          y[:, nq + nkv:]], axis=1)
    bound = REL[wl.dtype] * np.abs(ref) + 1e-5 * (1 + np.abs(y).max(axis=1, keepdims=True))
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"{wl.name}: worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"


@pytest.mark.parametrize("cid,T", [(1, None), (4, None), (3, 300), (5, 257), (4, 130)])
def test_forward_unfused(cid, T):
    wl = workloads.WORKLOADS[cid]
    if T is not None:
        wl = wl.with_tokens(1, T)
    inp = workloads.make_inputs(wl, seed=37 + cid)
    with qkv.Plan.for_workload(wl) as plan:
        (q, k, v), _ = plan.forward_unfused(*dev_inputs(inp))
        torch.cuda.synchronize()
    P.assert_parity((q, k, v), P.oracle_forward(wl, inp), P.TOL[wl.dtype], f"unfused {wl.name}")


def test_forward_unfused_full_size_sampled_rows():
    """The headline prefill shape, 8192 tokens, on sampled rows (ends, tile edges, random)."""
    wl = workloads.WORKLOADS[2]
    inp = workloads.make_inputs(wl)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 4096, wl.tokens - 1],
                                     np.random.default_rng(5).integers(0, wl.tokens, 57)]))
    with qkv.Plan.for_workload(wl) as plan:
        (q, k, v), _ = plan.forward_unfused(*dev_inputs(inp))
        torch.cuda.synchronize()
        got = tuple(t.float().cpu() for t in (q, k, v))
    P.assert_parity(got, P.oracle_forward(wl, inp, rows=rows), P.TOL["bf16"], "unfused full size", rows=rows)


def test_unfused_matches_fused_closely():
    """Both forms round the same products; on the GQA prefill shape (300 tokens) they differ
    by a few output roundings at most."""
    wl = workloads.WORKLOADS[3].with_tokens(1, 300)
    inp = workloads.make_inputs(wl, seed=3)
    with qkv.Plan.for_workload(wl) as plan:
        args = dev_inputs(inp)
        fused = plan.forward(*args)
        (q, k, v), _ = plan.forward_unfused(*args)
        torch.cuda.synchronize()
    for name, a, b in zip("QKV", fused, (q, k, v)):
        a, b = P.to_f64(a), P.to_f64(b)
        err = np.max(np.abs(a - b) / (1 + np.abs(a)))
        assert err < 2e-2, f"{name}: {err:.3e}"


@pytest.mark.parametrize("cid,T,d", [(1, None, None), (4, None, None), (3, 300, None), (5, 129, None),
                                     (10, 33, 64), (10, 40, 256)])
def test_head_norm_rope(cid, T, d):
    """The norm+rotation pass, read as a per-head RMSNorm of every Q and K head followed by
    the rotation: the oracle's rms_norm over each head's values, then its rope."""
    if cid == 10:
        wl = workloads.Workload(10, f"hnr_d{d}", 1, T, 1024, 4, 2, d, False, 1e4, 1e-6, "bf16", "per_seq")
    else:
        wl = workloads.WORKLOADS[cid]
        if T is not None:
            wl = wl.with_tokens(1, T)
    d = wl.head_dim
    inp = workloads.make_inputs(wl, seed=51 + cid)
    g = torch.Generator().manual_seed(509 + cid)
    y0 = torch.randn(wl.tokens, wl.n_total, generator=g).to(wl.torch_dtype)
    wq = (1 + 0.1 * torch.randn(d, generator=g)).to(wl.torch_dtype)
    wk = (1 + 0.1 * torch.randn(d, generator=g)).to(wl.torch_dtype)
    with qkv.Plan.for_workload(wl) as plan:
        got = P.to_f64(plan.head_norm_rope(y0.to(DEV), wq.to(DEV), wk.to(DEV), inp["pos"].to(DEV)))
    y, pos, T = P.to_f64(y0), P.to_f64(inp["pos"]), wl.tokens
    nq, nkv = wl.n_q, wl.n_kv

    def norm_rotate(block, w):
        heads = qkv_oracle.rms_norm(block.reshape(-1, d), P.to_f64(w), wl.eps).reshape(T, -1)
        return qkv_oracle.rope(heads, pos, d, wl.rope_theta)

    ref = np.concatenate([norm_rotate(y[:, :nq], wq), norm_rotate(y[:, nq:nq + nkv], wk), y[:, nq + nkv:]], axis=1)
    bound = REL[wl.dtype] * np.abs(ref) + 1e-5 * (1 + np.abs(ref).max(axis=1, keepdims=True))
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"{wl.name}: worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"
