"""Backward of the chain (qkv_backward) against the oracle's chain rule, through the C ABI.

Bar, derived from the arithmetic: every gradient element is a sum of many terms (over
tokens for dw_norm, dW and db; over output columns for dx) whose inputs are rounded
once -- for bf16 plans the unrotated gradient scaled by each token's r goes into the
fp32-accumulating GEMMs as bf16 (next to x itself), and the activation gradient they
give is rounded once to bf16 before the norm gradient -- so its error is relative to
the root-sum-square s of those terms, not to the sum itself, which can cancel.  The test requires
|gpu - oracle| <= tol * (1 + |oracle| + s) elementwise, tol = 1e-4 for fp32 plans and
2e-2 for bf16 plans (s from the oracle), and reports the plain (1 + |oracle|) ratio
too.  NaN/Inf fails.
"""
import dataclasses

import numpy as np
import pytest
import torch

import transformer_rmsnorm_row_amd as qkv
import workloads
from oracle import qkv_oracle
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(wl, inp, grads):
    with qkv.Plan.for_workload(wl) as plan:
        out = plan.backward(inp["x"].to(DEV), inp["w_norm"].to(DEV), inp["w_qkv"].to(DEV), inp["pos"].to(DEV),
                            grads["dq"].to(DEV), grads["dk"].to(DEV), grads["dv"].to(DEV))
        again = plan.backward(inp["x"].to(DEV), inp["w_norm"].to(DEV), inp["w_qkv"].to(DEV), inp["pos"].to(DEV),
                              grads["dq"].to(DEV), grads["dk"].to(DEV), grads["dv"].to(DEV))
        torch.cuda.synchronize()
    for a, b in zip(out, again):
        if a is not None:
            assert torch.equal(a, b), "backward is not deterministic"
    return out


def _oracle(wl, inp, grads):
    x, w, W, _, pos = P.oracle_inputs(inp)
    g = [P.to_f64(grads[k]) for k in ("dq", "dk", "dv")]
    return qkv_oracle.qkv_backward(x, w, W, pos, *g, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps,
                                   wl.rope_theta, with_bias=wl.has_bias, return_scales=True)


def _compare(wl, got, ref):
    tol = P.TOL[wl.dtype]
    refs, scales = ref
    lines, bad = [], []
    for name, g, r, sc in zip(("dx", "dw_norm", "dW", "db"), got, refs, scales):
        if r is None:
            assert g is None
            continue
        gv = P.to_f64(g)
        assert np.isfinite(gv).all(), f"{name}: NaN or Inf"
        ratio = np.abs(gv - r) / (1.0 + np.abs(r) + sc)
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        plain, _ = P.worst(gv, r)
        lines.append(f"{name}: {ratio[i]:.3e} (plain {plain:.3e}) at {i}")
        if not ratio[i] <= tol:
            bad.append(name)
    # every gradient is compared before failing, so a failure names all that are off
    assert not bad, f"{wl.name}: {', '.join(bad)} above {tol}: " + "; ".join(lines)
    return "; ".join(lines)


CASES = {
    "tiny_fp32": (workloads.WORKLOADS[1], {}),
    "bf16_bias_ragged": (workloads.WORKLOADS[5], dict(batch=1, seq=300, hidden=384, num_q_heads=4, num_kv_heads=2)),
    "gqa_1024": (workloads.WORKLOADS[3], dict(batch=1, seq=1024)),
    "decode_shape": (workloads.WORKLOADS[4], {}),
    "bf16_d64": (workloads.WORKLOADS[2], dict(batch=2, seq=100, hidden=256, num_q_heads=8, num_kv_heads=2,
                                               head_dim=64)),
    "fp32_d256": (workloads.WORKLOADS[1], dict(batch=1, seq=40, hidden=128, num_q_heads=2, num_kv_heads=1,
                                                head_dim=256)),
    # bf16 with N = 40 (not a multiple of 32): G = g W^T on the fp32-FMA tiles, and d = 8 takes
    # the 2-byte unrotate kernel
    "bf16_n40_d8": (workloads.WORKLOADS[3], dict(batch=1, seq=70, hidden=128, num_q_heads=3, num_kv_heads=1,
                                                  head_dim=8)),
    # the shape the benchmark times the backward on: Llama-7B, 4 x 2048 tokens, every
    # element of every gradient against the oracle's full chain rule
    "llama7b_full": (workloads.WORKLOADS[2], {}),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_parity(case):
    base, over = CASES[case]
    wl = dataclasses.replace(base, **over)
    inp = workloads.make_inputs(wl)
    grads = workloads.make_grads(wl)
    got = _run(wl, inp, grads)
    print(case, _compare(wl, got, _oracle(wl, inp, grads)))


def test_backward_bias_argument_must_match_plan():
    wl = dataclasses.replace(workloads.WORKLOADS[5], batch=1, seq=16, hidden=256, num_q_heads=2, num_kv_heads=1)
    lib = qkv.load_library()
    inp = workloads.make_inputs(wl)
    g = workloads.make_grads(wl)
    d = {k: v.to(DEV) for k, v in {**inp, **g}.items() if v is not None}
    T, H, N = wl.tokens, wl.hidden, wl.n_total
    dx = torch.empty((T, H), dtype=wl.torch_dtype, device=DEV)
    dw = torch.empty((H,), dtype=wl.torch_dtype, device=DEV)
    dW = torch.empty((H, N), dtype=wl.torch_dtype, device=DEV)
    with qkv.Plan.for_workload(wl) as plan:
        args = [d["x"].data_ptr(), d["w_norm"].data_ptr(), d["w_qkv"].data_ptr(), d["pos"].data_ptr(),
                d["dq"].data_ptr(), d["dk"].data_ptr(), d["dv"].data_ptr(), dx.data_ptr(), dw.data_ptr(),
                dW.data_ptr()]
        assert lib.qkv_backward(plan.handle, T, *args, None, None) == qkv.QKV_ERR_INVALID_ARG
        assert lib.qkv_backward(plan.handle, 0, *args, None, None) == qkv.QKV_OK
