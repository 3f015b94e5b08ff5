"""The key/value-cache form of the forward (qkv_forward_kv_cache) through the C ABI.

Bar: Q, and every cache row a valid slot names, within the parity tolerance of the
oracle (Q, K, V from the oracle's chain, the caches from its cache write); every other
cache row bit-for-bit as it was before the call.
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


def _cache(rows, width, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn((rows, width), generator=g).to(dtype)


def _slots(T, R, seed, drop=0.1, past_end=2):
    """Distinct rows of a cache of R rows for most tokens; some tokens padded (-1) and
    a few pointing past the end (both must write nothing)."""
    rng = np.random.default_rng(seed)
    s = rng.permutation(R)[:T].astype(np.int32)
    pad = rng.random(T) < drop
    s[pad] = -1
    far = rng.choice(T, size=min(past_end, T), replace=False)
    s[far] = R + rng.integers(0, 5, size=far.size)
    return s


def _dev(inp):
    b = None if inp["bias"] is None else inp["bias"].to(DEV)
    return inp["x"].to(DEV), inp["w_norm"].to(DEV), inp["w_qkv"].to(DEV), b, inp["pos"].to(DEV)


def _check_cache(name, got, init, expect, slots, tol):
    """Rows named by valid slots against the oracle; all others untouched."""
    R = init.shape[0]
    valid = np.array(sorted({int(s) for s in slots if 0 <= s < R}), dtype=np.int64)
    others = np.setdiff1d(np.arange(R), valid)
    err, loc = P.worst(P.to_f64(got)[valid], expect[valid])
    assert err <= tol, f"{name} cache rows: {err:.3e} at {loc}"
    assert torch.equal(got.cpu()[torch.from_numpy(others)], init[torch.from_numpy(others)]), \
        f"{name}: rows no slot names were modified"
    return f"{name}: {err:.3e} over {valid.size} rows"


CASES = {
    "generic": (workloads.WORKLOADS[1], {}, 40),
    "prefill": (workloads.WORKLOADS[3], dict(batch=1, seq=300, hidden=1152, num_q_heads=4, num_kv_heads=2), 700),
    "decode": (workloads.WORKLOADS[4], {}, 200),
    "decode_chunks": (workloads.WORKLOADS[4], dict(batch=150), 400),
    "prefill_d256": (workloads.WORKLOADS[3], dict(batch=1, seq=300, hidden=384, num_q_heads=4, num_kv_heads=2,
                                                  head_dim=256), 650),
    "prefill_d64": (workloads.WORKLOADS[3], dict(batch=1, seq=300, hidden=384, num_q_heads=8, num_kv_heads=2,
                                                 head_dim=64), 650),
    "prefill_split": (workloads.WORKLOADS[3], dict(batch=1, seq=300), 700),
}


@pytest.mark.parametrize("variant", sorted(CASES))
def test_cache_parity(variant):
    base, over, R = CASES[variant]
    wl = dataclasses.replace(base, **over)
    inp = workloads.make_inputs(wl)
    T, tol = wl.tokens, P.TOL[wl.dtype]
    slots = _slots(T, R, seed=wl.cid * 7 + 1)
    k0 = _cache(R, wl.n_kv, wl.torch_dtype, 11)
    v0 = _cache(R, wl.n_kv, wl.torch_dtype, 12)
    kc, vc = k0.to(DEV), v0.to(DEV)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(T) == ("prefill_split" if variant == "prefill_split" else variant.split("_")[0])
        q = plan.forward_kv_cache(*_dev(inp), torch.from_numpy(slots).to(DEV), kc, vc)
        torch.cuda.synchronize()
    rq, rk, rv = P.oracle_forward(wl, inp)
    err, loc = P.worst(P.to_f64(q), rq)
    assert err <= tol, f"Q: {err:.3e} at {loc}"
    print(_check_cache("K", kc, k0, qkv_oracle.kv_cache_write(P.to_f64(k0), slots, rk), slots, tol))
    print(_check_cache("V", vc, v0, qkv_oracle.kv_cache_write(P.to_f64(v0), slots, rv), slots, tol))


@pytest.mark.parametrize("cid", [3, 4])
def test_cache_rows_equal_dense_outputs(cid):
    """At full size, in the benchmark's launch configuration, the cache form writes
    exactly the dense forward's K and V rows (same kernels, same arithmetic) and the
    same Q; sampled rows also against the oracle."""
    wl = workloads.WORKLOADS[cid]
    inp = workloads.make_inputs(wl)
    T = wl.tokens
    R = T + 97
    slots = np.random.default_rng(cid).permutation(R)[:T].astype(np.int32)
    kc = torch.zeros((R, wl.n_kv), dtype=wl.torch_dtype, device=DEV)
    vc = torch.zeros_like(kc)
    args = _dev(inp)
    with qkv.Plan.for_workload(wl) as plan:
        q, k, v = plan.forward(*args)
        qc = plan.forward_kv_cache(*args, torch.from_numpy(slots).to(DEV), kc, vc)
        torch.cuda.synchronize()
    idx = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    assert torch.equal(qc, q)
    assert torch.equal(kc[idx], k)
    assert torch.equal(vc[idx], v)
    rows = P.sample_rows(T, 24, seed=cid)
    ref = P.oracle_forward(wl, inp, rows=rows)
    print(P.assert_parity((qc, kc[idx], vc[idx]), ref, P.TOL["bf16"], wl.name, rows=rows))


def test_rolling_cache_over_calls():
    """Generation into a rolling cache of capacity C (slot = pos mod C) in calls of 16
    consecutive positions: the cache ends up holding the last C positions, which read
    oldest to newest are the oracle's K and V of those positions."""
    wl = dataclasses.replace(workloads.WORKLOADS[4], batch=16)
    C, calls = 40, 4
    k0 = _cache(C, wl.n_kv, wl.torch_dtype, 21)
    v0 = _cache(C, wl.n_kv, wl.torch_dtype, 22)
    kc, vc = k0.to(DEV), v0.to(DEV)
    ek, ev = P.to_f64(k0), P.to_f64(v0)
    ks, vs = [], []
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(wl.tokens) == "decode"
        for c in range(calls):
            inp = workloads.make_inputs(wl, seed=900 + c)
            inp["pos"] = torch.arange(16 * c, 16 * c + 16, dtype=torch.int32)
            slots = qkv.ring_slots(inp["pos"], C)
            plan.forward_kv_cache(*_dev(inp), slots.to(DEV), kc, vc)
            _, rk, rv = P.oracle_forward(wl, inp)
            ek = qkv_oracle.kv_cache_write(ek, slots.numpy(), rk)
            ev = qkv_oracle.kv_cache_write(ev, slots.numpy(), rv)
            ks.append(rk)
            vs.append(rv)
        torch.cuda.synchronize()
    tol = P.TOL["bf16"]
    all_slots = np.arange(C)
    print(_check_cache("K", kc, k0, ek, all_slots, tol))
    print(_check_cache("V", vc, v0, ev, all_slots, tol))
    last = np.arange(16 * calls - C, 16 * calls)
    view = P.to_f64(kc)[last % C]
    err, loc = P.worst(view, np.concatenate(ks)[last])
    assert err <= tol, f"rolling view: {err:.3e} at {loc}"


def test_cache_argument_errors():
    wl = workloads.WORKLOADS[1]
    lib = qkv.load_library()
    inp = workloads.make_inputs(wl)
    x, w, W, b, pos = _dev(inp)
    T = wl.tokens
    q = torch.empty((T, wl.n_q), dtype=wl.torch_dtype, device=DEV)
    kc = torch.zeros((32, wl.n_kv), dtype=wl.torch_dtype, device=DEV)
    vc = torch.zeros_like(kc)
    slots = torch.arange(T, dtype=torch.int32, device=DEV)
    with qkv.Plan.for_workload(wl) as plan:
        h = plan.handle
        p = [x.data_ptr(), w.data_ptr(), W.data_ptr(), None, pos.data_ptr()]
        call = lambda s, rows, k, v: lib.qkv_forward_kv_cache(h, T, *p, s, rows, q.data_ptr(), k, v, None)
        assert call(slots.data_ptr(), 32, kc.data_ptr(), vc.data_ptr()) == qkv.QKV_OK
        assert call(None, 32, kc.data_ptr(), vc.data_ptr()) == qkv.QKV_ERR_INVALID_ARG
        assert call(slots.data_ptr() + 2, 32, kc.data_ptr(), vc.data_ptr()) == qkv.QKV_ERR_INVALID_ARG
        assert call(slots.data_ptr(), 0, kc.data_ptr(), vc.data_ptr()) == qkv.QKV_ERR_INVALID_ARG
        assert call(slots.data_ptr(), 32, None, vc.data_ptr()) == qkv.QKV_ERR_INVALID_ARG
        assert call(slots.data_ptr(), 32, kc.data_ptr() + 4, vc.data_ptr()) == qkv.QKV_ERR_INVALID_ARG
        big = (1 << 31) // (wl.n_kv * 4)
        assert call(slots.data_ptr(), big, kc.data_ptr(), vc.data_ptr()) == qkv.QKV_ERR_UNSUPPORTED
        torch.cuda.synchronize()
