"""qkv_forward_noalloc against qkv_forward, through the C ABI.

The no-allocation entry point keeps its scratch in the library's own device array,
shared by every call on the GPU.  Each case calls it twice in a row, the second time
with fewer tokens, and compares each call's Q, K, V with qkv_forward's (through a
plan) on the same inputs at the parity bar |a - b| <= tol * (1 + |b|) (tol 1e-4 for
fp32, 2e-2 for bf16); where both run the same kernel the outputs must be bit-identical.
Sampled rows are also checked against the oracle.
"""
import ctypes
import dataclasses

import numpy as np
import pytest
import torch

import transformer_rmsnorm_row_amd as qkv
import workloads
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# base workload and two calls (batch, seq, same kernel as the plan's forward); the second
# call is the smaller one
CASES = {
    # decode kernel in both entry points
    "decode_64_then_17": (workloads.WORKLOADS[4], [(64, 1, True), (17, 1, True)]),
    # 200 tokens: a plan runs the split-K prefill, the no-allocation call two decode
    # launches; 64 tokens: the decode kernel in both
    "decode_200_then_64": (workloads.WORKLOADS[4], [(200, 1, False), (64, 1, True)]),
    "tiny_fp32_16_then_5": (workloads.WORKLOADS[1], [(1, 16, True), (1, 5, True)]),
    # a plan runs the split-K prefill at these sizes, the no-allocation call the
    # single-launch prefill kernel
    "gqa_prefill_1000_then_300": (workloads.WORKLOADS[3], [(1, 1000, False), (1, 300, False)]),
    # 777 tokens: the single-launch prefill kernel in both; 129: the decode kernel in both
    "qwen_bias_777_then_129": (workloads.WORKLOADS[5], [(1, 777, True), (1, 129, True)]),
    # the full Llama-7B prefill, then a ragged smaller one: the single-launch prefill kernel
    "llama7b_8192_then_1111": (workloads.WORKLOADS[2], [(4, 2048, True), (1, 1111, True)]),
}


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def _call_noalloc(wl, d):
    lib = qkv.load_library()
    desc = qkv.PlanDesc(wl.tokens, wl.hidden, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                        qkv.QKV_BF16 if wl.dtype == "bf16" else qkv.QKV_F32, int(wl.has_bias), wl.eps, wl.rope_theta)
    T = wl.tokens
    q = torch.full((T, wl.n_q), float("nan"), dtype=wl.torch_dtype, device=DEV)
    k = torch.full((T, wl.n_kv), float("nan"), dtype=wl.torch_dtype, device=DEV)
    v = torch.full((T, wl.n_kv), float("nan"), dtype=wl.torch_dtype, device=DEV)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.qkv_forward_noalloc(ctypes.byref(desc), T, ptr(d["x"]), ptr(d["w_norm"]), ptr(d["w_qkv"]),
                                 ptr(d["bias"]), ptr(d["pos"]), ptr(q), ptr(k), ptr(v),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == qkv.QKV_OK, qkv.status_string(st)
    return q, k, v


def _check(wl, inp, same_kernel):
    d = _dev(inp)
    got = _call_noalloc(wl, d)
    with qkv.Plan.for_workload(wl) as plan:
        ref = plan.forward(d["x"], d["w_norm"], d["w_qkv"], d["bias"], d["pos"])
        torch.cuda.synchronize()
    tol = P.TOL[wl.dtype]
    lines = []
    for name, g, r in zip("QKV", got, ref):
        assert torch.isfinite(g).all(), f"{wl.name} {name}: non-finite output"
        if same_kernel:
            assert torch.equal(g, r), f"{wl.name} {name}: differs from qkv_forward running the same kernel"
        err, loc = P.worst(P.to_f64(g), P.to_f64(r))
        lines.append(f"{name} vs qkv_forward {err:.2e}")
        assert err <= tol, f"{wl.name} {name}: {err:.3e} > {tol} at {loc} against qkv_forward"
    rows = P.sample_rows(wl.tokens, 48, seed=wl.tokens)
    lines += P.assert_parity(got, P.oracle_forward(wl, inp, rows=rows), tol, wl.name + " (oracle)", rows=rows)
    return "; ".join(lines)


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_two_calls_match_qkv_forward(case):
    base, calls = CASES[case]
    for (b, s, same) in calls:
        wl = base.with_tokens(b, s)
        inp = workloads.make_inputs(wl, seed=1000 * base.cid + 31 * b + s)
        print(case, wl.tokens, _check(wl, inp, same), flush=True)
