"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bar: |gpu - oracle| <= tol * (1 + |oracle|) elementwise on Q, K and V separately,
tol = 1e-4 for the fp32 workload and 2e-2 for the bf16 ones; NaN or Inf fails.
"""
import dataclasses

import numpy as np
import pytest
import torch

import transformer_rmsnorm_row_amd as qkv
import workloads
from tests import _parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(plan, inp, stream=None):
    x = inp["x"].to(DEV)
    w = inp["w_norm"].to(DEV)
    W = inp["w_qkv"].to(DEV)
    b = None if inp["bias"] is None else inp["bias"].to(DEV)
    pos = inp["pos"].to(DEV)
    out = plan.forward(x, w, W, b, pos, stream=stream)
    torch.cuda.synchronize()
    return out


def shaped(wl, **kw):
    return dataclasses.replace(wl, **kw)


# ---------------------------------------------------------------- the five workloads

def test_tiny_fp32_full():
    wl = workloads.WORKLOADS[1]
    inp = workloads.make_inputs(wl)
    with qkv.Plan.for_workload(wl) as plan:
        got = run(plan, inp)
    ref = P.oracle_forward(wl, inp)
    print(P.assert_parity(got, ref, P.TOL["fp32"], wl.name))


def test_decode_full():
    wl = workloads.WORKLOADS[4]
    inp = workloads.make_inputs(wl)
    with qkv.Plan.for_workload(wl) as plan:
        got = run(plan, inp)
    ref = P.oracle_forward(wl, inp)
    print(P.assert_parity(got, ref, P.TOL["bf16"], wl.name))


@pytest.mark.parametrize("prepass", [False, True], ids=["one_launch", "prepass_opt_in"])
@pytest.mark.parametrize("cid", [2, 3, 5])
def test_prefill_full_size_sampled_rows(cid, prepass):
    """Full-size forward in the benchmark's launch configuration (and in the opt-in
    pre-pass form); the oracle evaluates a sample of rows (ends, every tile edge,
    random) one token at a time."""
    wl = workloads.WORKLOADS[cid]
    inp = workloads.make_inputs(wl)
    with qkv.Plan.for_workload(wl, prefill_prepass=prepass) as plan:
        assert plan.variant(wl.tokens) == "prefill"
        got = run(plan, inp)
    for t in got:
        assert torch.isfinite(t).all(), "non-finite output"
    rows = P.sample_rows(wl.tokens, 192, seed=cid)
    ref = P.oracle_forward(wl, inp, rows=rows)
    print(P.assert_parity(got, ref, P.TOL["bf16"], wl.name, rows=rows))


def test_prefill_largest_plan():
    """The largest token count a plan of the Llama-3-8B GQA shape accepts: kernels use
    32-bit byte offsets, so tokens x widest row (6144 columns) x 2 bytes stays below
    2^31.  One forward over 174761 tokens (1365 full 128-row panels and a ragged one:
    16392 tiles of 128 x 512, 64 rounds of the persistent grid and a partial one),
    sampled rows against the oracle; one token more is refused."""
    base = workloads.WORKLOADS[3]
    limit = (1 << 31) // (base.n_total * 2)
    wl = base.with_tokens(1, limit - 1)
    with pytest.raises(qkv.QKVError) as err:
        qkv.Plan.for_workload(wl, max_tokens=limit)
    assert err.value.status == qkv.QKV_ERR_UNSUPPORTED
    inp = workloads.make_inputs(wl, seed=4242)
    print(f"largest plan: T={wl.tokens}", flush=True)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(wl.tokens) == "prefill"
        got = run(plan, inp)
    rows = P.sample_rows(wl.tokens, 256, seed=11)
    idx = torch.as_tensor(rows, device=DEV)
    got_rows = tuple(t.index_select(0, idx) for t in got)
    for t in got_rows:
        assert torch.isfinite(t).all(), "non-finite output"
    # tokens are independent: the oracle over the sampled rows alone gives their outputs
    sub = dict(inp, x=inp["x"][rows], pos=inp["pos"][rows])
    ref = P.oracle_forward(wl, sub)
    print(P.assert_parity(got_rows, ref, P.TOL["bf16"], "largest plan"))


SPLIT_CASES = [
    # (workload, T, overrides): at most 128 tiles of 256 x 256, so K is split over two
    # workgroups per tile whose partial tiles the last to arrive adds
    (3, 257, {}),                  # GQA: 2 x 24 = 48 tiles; one real row in the last tile row
    (3, 777, {}),                  # 4 x 24 = 96 tiles
    (3, 1280, {}),                 # 5 x 24 = 120 tiles
    (5, 300, {}),                  # MHA with bias: 2 x 48 = 96 tiles
    (2, 500, {"hidden": 2048}),    # 96 tiles, 64 steps in 2 slices of 32
    (3, 300, {"hidden": 2048, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 64}),  # d = 64: 6 tiles
    (3, 300, {"hidden": 2048, "num_q_heads": 4, "num_kv_heads": 1, "head_dim": 256}),  # d = 256
]


@pytest.mark.parametrize("cid,T,over", SPLIT_CASES)
def test_prefill_split_k(cid, T, over):
    """The split-K form of the prefill kernel: full comparison with the oracle, and two
    forwards bit for bit equal (the partial tiles are added in slice order, whichever
    workgroup arrives last)."""
    wl = shaped(workloads.WORKLOADS[cid].with_tokens(1, T), **over)
    inp = workloads.make_inputs(wl, seed=11 * T + cid)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(T) == "prefill_split"
        got = run(plan, inp)
        again = run(plan, inp)
    for name, a, b in zip("QKV", got, again):
        assert torch.equal(a, b), f"{name} differs between two forwards"
    print(P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], f"{wl.name} split T={T}"))


PLAIN_SHAPE_CASES = [
    # (workload, T, overrides): plain (not split-K) prefill forwards on every head size of
    # the 128 x 512 single-launch kernel, and on the 256 x 256 normalise-on-load kernel,
    # which takes projections whose width is a multiple of 256 but not of 512; ragged T
    (3, 6000, {"hidden": 2048, "num_q_heads": 16, "num_kv_heads": 4, "head_dim": 64}),   # N = 1536
    (3, 3000, {"hidden": 2048, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 256}),   # N = 3072
    (5, 11000, {"hidden": 1024, "num_q_heads": 4, "num_kv_heads": 1}),                   # N = 768, bias
    # more tiles than the single-launch kernel's one workgroup per CU: some workgroups
    # take a second tile (288 tiles) or most do (480)
    (2, 1500, {}),                                                                        # Llama-7B shape
    (3, 5000, {}),                                                                        # GQA shape
]


@pytest.mark.parametrize("cid,T,over", PLAIN_SHAPE_CASES)
def test_prefill_plain_head_sizes_and_widths(cid, T, over):
    """Every element of Q, K and V against the oracle for plain prefill forwards of
    head size 64 and 256 (128 x 512 kernel), of a 768-wide projection (256 x 256
    kernel, normalising on load in one launch), and of tile counts that are not a
    multiple of the 128 x 512 kernel's grid."""
    wl = shaped(workloads.WORKLOADS[cid].with_tokens(1, T), **over)
    inp = workloads.make_inputs(wl, seed=13 * T + cid)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(T) == "prefill"
        got = run(plan, inp)
    print(P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], f"{wl.name} plain T={T}"))


PREPASS_CASES = [
    # (workload, T, overrides): the opt-in pre-pass form's 256 x 256 kernel on every head
    # size, ragged T, with bias; T large enough that the plain (not split-K) form runs
    (3, 1500, {"hidden": 1024}),                                                        # GQA, N = 6144
    (3, 6000, {"hidden": 2048, "num_q_heads": 16, "num_kv_heads": 4, "head_dim": 64}),  # N = 1536
    (3, 3000, {"hidden": 512, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 256}),   # N = 3072
    (5, 777, {"hidden": 1024}),                                                         # MHA + bias
    (2, 2500, {}),  # Llama-7B shape: 10 x 48 = 480 tiles, more than the persistent grid's workgroups
]


@pytest.mark.parametrize("cid,T,over", PREPASS_CASES)
def test_prefill_prepass_shapes(cid, T, over):
    """Every element of Q, K and V against the oracle for the opt-in pre-pass form
    (pre-pass, then the pre-normalised 256 x 256 kernel) at every head size."""
    wl = shaped(workloads.WORKLOADS[cid].with_tokens(1, T), **over)
    inp = workloads.make_inputs(wl, seed=17 * T + cid)
    with qkv.Plan.for_workload(wl, prefill_prepass=True) as plan:
        assert plan.variant(T) == "prefill"
        got = run(plan, inp)
    print(P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], f"{wl.name} pre-pass T={T}"))


def test_prefill_prepass_kv_cache():
    """The pre-pass form writing K and V into cache slots: the cache rows equal the dense
    forward's K and V bit for bit, unnamed rows stay untouched, Q is unchanged."""
    wl = shaped(workloads.WORKLOADS[3].with_tokens(1, 1500), hidden=1024)
    inp = workloads.make_inputs(wl, seed=4242)
    rows = 2048
    g = torch.Generator().manual_seed(5)
    slots = torch.randperm(rows, generator=g)[:wl.tokens].to(torch.int32)
    slots[::97] = -1          # some tokens write no K/V
    with qkv.Plan.for_workload(wl, prefill_prepass=True) as plan:
        assert plan.variant(wl.tokens) == "prefill"
        q, k, v = run(plan, inp)
        kc = torch.full((rows, wl.n_kv), 7.0, dtype=torch.bfloat16, device=DEV)
        vc = torch.full_like(kc, 7.0)
        args = [inp[n].to(DEV) for n in ("x", "w_norm", "w_qkv")]
        qc = plan.forward_kv_cache(*args, None, inp["pos"].to(DEV), slots.to(DEV), kc, vc)
        torch.cuda.synchronize()
    assert torch.equal(qc, q)
    keep = slots >= 0
    idx = slots[keep].long().to(DEV)
    assert torch.equal(kc[idx], k[keep.to(DEV)]) and torch.equal(vc[idx], v[keep.to(DEV)])
    untouched = torch.ones(rows, dtype=torch.bool)
    untouched[slots[keep].long()] = False
    assert bool((kc[untouched.to(DEV)] == 7.0).all()) and bool((vc[untouched.to(DEV)] == 7.0).all())


# ---------------------------------------------------------------- ragged sizes, full comparison

MEDIUM = [
    (2, 1, 300),     # MHA 32x128, two full 128-row blocks + tail
    (3, 1, 777),     # GQA 32/8, several 256-row tiles + ragged tail
    (5, 1, 513),     # MHA with bias, one row past two tiles
    (4, 1, 129),     # decode shape at a small prefill size
]


@pytest.mark.parametrize("cid,batch,seq", MEDIUM)
def test_ragged_full_comparison(cid, batch, seq):
    wl = workloads.WORKLOADS[cid].with_tokens(batch, seq)
    inp = workloads.make_inputs(wl, seed=31 * cid + seq)
    with qkv.Plan.for_workload(wl) as plan:
        got = run(plan, inp)
    ref = P.oracle_forward(wl, inp)
    print(P.assert_parity(got, ref, P.TOL[wl.dtype], wl.name))


@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 255, 256, 257])
@pytest.mark.parametrize("cid", [1, 3])
def test_token_count_edges(cid, T):
    base = workloads.WORKLOADS[cid]
    wl = base.with_tokens(1, T) if cid == 1 else shaped(base.with_tokens(1, T), hidden=512)
    inp = workloads.make_inputs(wl, seed=7 * T + cid)
    with qkv.Plan.for_workload(wl, max_tokens=300) as plan:
        got = run(plan, inp)
    ref = P.oracle_forward(wl, inp)
    P.assert_parity(got, ref, P.TOL[wl.dtype], f"{wl.name} T={T}")


@pytest.mark.parametrize("nq,nkv,d", [(4, 4, 64), (8, 2, 128), (2, 1, 256), (6, 3, 8), (3, 1, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_head_shapes(nq, nkv, d, dtype):
    wl = workloads.Workload(9, f"heads{nq}x{nkv}x{d}", 1, 100, 256, nq, nkv, d, True, 1e4, 1e-6, dtype, "per_seq")
    inp = workloads.make_inputs(wl, seed=nq * 100 + nkv * 10 + d)
    with qkv.Plan.for_workload(wl) as plan:
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL[dtype], wl.name)


@pytest.mark.parametrize("nq,nkv,d", [(8, 2, 64), (4, 1, 256), (16, 4, 64), (2, 1, 256)])
def test_prefill_head_sizes(nq, nkv, d):
    """Head sizes 64 and 256 on the MFMA prefill kernel (rotation partners d/2 apart,
    so a wave's two column blocks sit 32 or 128 columns apart), with bias and a ragged
    last row tile."""
    wl = workloads.Workload(12, f"prefill_d{d}_{nq}x{nkv}", 1, 300, 384, nq, nkv, d, True, 1e4, 1e-6, "bf16",
                            "per_seq")
    inp = workloads.make_inputs(wl, seed=7 * d + nq)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(wl.tokens) == "prefill"
        got = run(plan, inp)
    print(P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], wl.name))


@pytest.mark.parametrize("hidden", [128, 384, 640, 1152, 5120, 8192])
def test_prefill_hidden_sizes(hidden):
    """K extents that exercise the prefill kernel's loop structure: H = 128 runs only
    the final group of four 32-wide steps, the others one or more full groups first."""
    wl = workloads.Workload(11, f"prefill_h{hidden}", 1, 300, hidden, 4, 2, 128, True, 1e4, 1e-6, "bf16",
                            "per_seq")
    inp = workloads.make_inputs(wl, seed=hidden)
    with qkv.Plan.for_workload(wl) as plan:
        # 8 tiles: H = 5120 and 8192 split K over two workgroups per tile, the others cannot
        # (H / 32 steps must split into two multiples of 4)
        expect = "prefill_split" if hidden in (5120, 8192) else "prefill"
        assert plan.variant(wl.tokens) == expect
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], wl.name)


# ---------------------------------------------------------------- inputs the workloads cannot see

# shapes the special inputs run on, one per bf16 kernel: (tokens, hidden, variant)
PIN_SHAPES = {
    "decode": (96, 512, "decode"),            # two 64-token chunks
    "prefill": (300, 384, "prefill"),         # 12 K steps: no split
    "split": (300, 512, "prefill_split"),     # 8 tiles, 16 K steps in two slices
}


def _pin_case(kind, dtype="bf16", shape="decode"):
    T, H, _ = PIN_SHAPES[shape]
    bias = kind in ("big_bias", "zero_rows")
    wl = workloads.Workload(8, f"pin_{kind}_{shape}", 1, T, H, 4, 2, 128, bias, 1e4, 1e-6, dtype, "per_seq")
    inp = workloads.make_inputs(wl, seed=404)
    g = torch.Generator().manual_seed(405)
    dt = wl.torch_dtype
    if kind == "row_scaled":
        scale = 10.0 ** (torch.rand(wl.tokens, 1, generator=g) * 4 - 2)
        inp["x"] = (inp["x"].float() * scale).to(dt)
    elif kind == "small_rows":
        inp["x"] = (inp["x"].float() * 1e-3).to(dt)
    elif kind == "huge_rows":
        inp["x"] = (inp["x"].float() * 1e4).to(dt)
    elif kind == "zero_rows":
        # all-zero rows: 1/rms = 1/sqrt(eps), the normalised row is zero, and Q/K/V are the
        # bias (Q and K rotated); the first and last rows of every tile and chunk among them
        x = inp["x"].float()
        for t in {0, 1, 63, 64, 95, wl.tokens - 1, 255 % wl.tokens, 256 % wl.tokens}:
            x[t] = 0.0
        inp["x"] = x.to(dt)
    elif kind == "big_bias":
        inp["bias"] = torch.randn(wl.n_total, generator=g).to(dt)
    elif kind == "one_hot":
        W = torch.zeros(wl.hidden, wl.n_total)
        for j, (k0, n0) in enumerate([(0, 0), (H - 1, wl.n_q - 1), (17, wl.n_q), (300, wl.n_total - 1)]):
            W[k0, n0] = 1.0
        inp["w_qkv"] = W.to(dt)
    elif kind == "positions":
        base = torch.tensor([0, -1, -32768, 2**31 - 1, -(2**31), 1, 65535, 4096], dtype=torch.int32)
        inp["pos"] = base.repeat((wl.tokens + 7) // 8)[: wl.tokens].contiguous()
    return wl, inp


PIN_KINDS = ["row_scaled", "small_rows", "huge_rows", "zero_rows", "big_bias", "one_hot", "positions"]


@pytest.mark.parametrize("kind", PIN_KINDS)
@pytest.mark.parametrize("dtype,shape", [("bf16", "decode"), ("bf16", "prefill"), ("bf16", "split"),
                                         ("fp32", "decode")])
def test_pinning_inputs(kind, dtype, shape):
    wl, inp = _pin_case(kind, dtype, shape)
    with qkv.Plan.for_workload(wl) as plan:
        if dtype == "bf16":
            assert plan.variant(wl.tokens) == PIN_SHAPES[shape][2]
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL[dtype], f"{kind}/{dtype}/{shape}")


def test_eps_is_applied():
    """Rows with mean square ~1e-6: eps=1e-5 and eps=1e-6 give visibly different
    outputs, and each matches the oracle with its own eps."""
    wl, inp = _pin_case("small_rows", "fp32")
    outs = []
    for eps in (1e-6, 1e-5):
        w2 = dataclasses.replace(wl, eps=eps)
        with qkv.Plan.for_workload(w2) as plan:
            got = run(plan, inp)
        P.assert_parity(got, P.oracle_forward(w2, inp), P.TOL["fp32"], f"eps={eps}")
        outs.append(got[2].float().cpu())
    assert (outs[0] - outs[1]).abs().max() > 1e-2


# ---------------------------------------------------------------- row reduction alone

@pytest.mark.parametrize("cid", [1, 2])
def test_rms_inv_step(cid):
    from oracle import qkv_oracle
    wl = workloads.WORKLOADS[cid]
    inp = workloads.make_inputs(wl)
    with qkv.Plan.for_workload(wl) as plan:
        r = plan.rms_inv(inp["x"].to(DEV))
        torch.cuda.synchronize()
    ref = qkv_oracle.inv_rms(P.to_f64(inp["x"]), wl.eps)
    err = np.max(np.abs(P.to_f64(r) - ref) / np.abs(ref))
    assert err < 2e-6, err


# ---------------------------------------------------------------- properties at full size

@pytest.mark.parametrize("cid", [2, 4])
def test_deterministic(cid):
    wl = workloads.WORKLOADS[cid]
    inp = workloads.make_inputs(wl)
    with qkv.Plan.for_workload(wl) as plan:
        a = [t.clone() for t in run(plan, inp)]
        b = run(plan, inp)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_side_stream_and_output_reuse():
    wl = workloads.WORKLOADS[3].with_tokens(1, 384)
    inp = workloads.make_inputs(wl, seed=5)
    s = torch.cuda.Stream()
    with qkv.Plan.for_workload(wl) as plan:
        with torch.cuda.stream(s):
            got = run(plan, inp, stream=s)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], "side stream")


# ---------------------------------------------------------------- boundary behaviour with a device

def test_forward_argument_errors():
    wl = workloads.WORKLOADS[3].with_tokens(1, 64)
    inp = workloads.make_inputs(wl)
    lib = qkv.load_library()
    with qkv.Plan.for_workload(wl) as plan:
        x = inp["x"].to(DEV)
        w = inp["w_norm"].to(DEV)
        W = inp["w_qkv"].to(DEV)
        pos = inp["pos"].to(DEV)
        q = torch.empty(64, wl.n_q, dtype=torch.bfloat16, device=DEV)
        k = torch.empty(64, wl.n_kv, dtype=torch.bfloat16, device=DEV)
        v = torch.empty(64, wl.n_kv, dtype=torch.bfloat16, device=DEV)
        P_ = lambda t: t.data_ptr()
        h = plan.handle
        ok = lambda: lib.qkv_forward(h, 64, P_(x), P_(w), P_(W), None, P_(pos), P_(q), P_(k), P_(v), None)
        assert ok() == qkv.QKV_OK
        assert lib.qkv_forward(h, 65, P_(x), P_(w), P_(W), None, P_(pos), P_(q), P_(k), P_(v), None) == 1
        assert lib.qkv_forward(h, -1, P_(x), P_(w), P_(W), None, P_(pos), P_(q), P_(k), P_(v), None) == 1
        assert lib.qkv_forward(h, 64, P_(x) + 2, P_(w), P_(W), None, P_(pos), P_(q), P_(k), P_(v), None) == 1
        assert lib.qkv_forward(h, 64, P_(x), P_(w), P_(W), P_(w), P_(pos), P_(q), P_(k), P_(v), None) == 1
        assert lib.qkv_forward(h, 64, P_(x), P_(w), P_(W), None, None, P_(q), P_(k), P_(v), None) == 1
        assert lib.qkv_forward(h, 0, None, None, None, None, None, None, None, None, None) == qkv.QKV_OK
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 2, 17, 33, 63, 64])
def test_decode_token_counts(T):
    """The small-batch kernel at every token count it takes, GQA decode shape."""
    wl = workloads.WORKLOADS[4].with_tokens(T, 1)
    inp = workloads.make_inputs(wl, seed=900 + T)
    with qkv.Plan.for_workload(wl, max_tokens=64) as plan:
        assert plan.variant(T) == "decode"
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], f"decode T={T}")


@pytest.mark.parametrize("hidden,nq,nkv,bias", [(4096, 32, 32, True), (2048, 16, 4, False), (8192, 8, 2, True)])
def test_decode_shapes(hidden, nq, nkv, bias):
    wl = workloads.Workload(10, f"decode_{hidden}_{nq}x{nkv}", 24, 1, hidden, nq, nkv, 128, bias, 1e4, 1e-6,
                            "bf16", "uniform32768")
    inp = workloads.make_inputs(wl, seed=hidden + nq)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(wl.tokens) == "decode"
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], wl.name)


@pytest.mark.parametrize("T", [65, 100, 128, 150, 191, 192])
def test_decode_in_chunks(T):
    """65 to 192 tokens run the decode kernel once per 128-token chunk (fewer than a
    prefill tile's 256 rows would leave most compute units idle); full comparison with
    the oracle, and every 64 rows bit for bit equal to a forward of those 64 tokens alone
    (which the kernel's 64-token form computes)."""
    wl = workloads.WORKLOADS[4].with_tokens(T, 1)
    inp = workloads.make_inputs(wl, seed=700 + T)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(T) == "decode"
        got = run(plan, inp)
        P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], f"decode chunks T={T}")
        for t0 in range(0, T, 64):
            part = {k: (v[t0:t0 + 64] if k in ("x", "pos") else v) for k, v in inp.items()}
            one = run(plan, part)
            for name, g, o in zip("QKV", got, one):
                assert torch.equal(g[t0:t0 + 64], o), f"{name}: chunk at {t0} differs from its own forward"


def test_decode_chunk_boundary():
    """The decode kernel serves up to 192 tokens of a plan whose prefill kernel has a split-K
    form (a 128-token launch, then one of the 64-token form); from 193 on, the split-K
    prefill (while the tiles number at most 128: 24 per 256 tokens here)."""
    wl = workloads.WORKLOADS[4].with_tokens(1537, 1)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(192) == "decode"
        assert plan.variant(193) == "prefill_split"
        assert plan.variant(1280) == "prefill_split"   # 5 x 24 = 120 tiles
        assert plan.variant(1281) == "prefill"         # 6 x 24 = 144 tiles
        assert plan.variant(1) == "decode"


def test_decode_two_full_chunks():
    """Without a split-K prefill (hidden 1152: 36 steps of 32 do not split into two multiples
    of 4) the decode kernel keeps up to 256 tokens, two launches of its 128-token form; full
    comparison with the oracle at 256, and 257 goes to the plain prefill kernel."""
    wl = workloads.Workload(10, "decode_1152_8x2", 256, 1, 1152, 8, 2, 128, True, 1e4, 1e-6,
                            "bf16", "uniform32768")
    inp = workloads.make_inputs(wl, seed=1152)
    with qkv.Plan.for_workload(wl.with_tokens(257, 1)) as plan:
        assert plan.variant(256) == "decode"
        assert plan.variant(257) == "prefill"
        got = run(plan, inp)
    P.assert_parity(got, P.oracle_forward(wl, inp), P.TOL["bf16"], wl.name)


def test_plan_reuse_across_token_counts():
    """One plan serving forwards of different sizes in turn (plain prefill, split-K prefill
    with its partial tiles, decode with its partial sums, and plain again): each
    bit-identical to the same forward through a fresh plan of its own size."""
    base = workloads.WORKLOADS[3]
    with qkv.Plan.for_workload(base.with_tokens(1, 2048)) as plan:
        for T, variant in ((2048, "prefill"), (1537, "prefill"), (300, "prefill_split"), (64, "decode"),
                           (2048, "prefill")):
            wl = base.with_tokens(1, T)
            inp = workloads.make_inputs(wl, seed=T)
            assert plan.variant(T) == variant
            got = [t.clone() for t in run(plan, inp)]
            with qkv.Plan.for_workload(wl) as fresh:
                assert fresh.variant(T) == variant
                ref = run(fresh, inp)
            for name, g, r in zip("QKV", got, ref):
                assert torch.equal(g, r), f"T={T}: {name} differs from a fresh plan's forward"


def test_variant_names():
    for cid in (1, 2, 3, 4, 5):
        wl = workloads.WORKLOADS[cid]
        with qkv.Plan.for_workload(wl) as plan:
            v = plan.variant(wl.tokens)
            print(wl.name, v)
            if wl.dtype == "fp32":
                assert v == "generic"
            elif wl.tokens <= 64:
                assert v == "decode"
            else:
                assert v == "prefill"


@pytest.mark.parametrize("cid,T,variant", [(3, 300, "prefill_split"), (3, 2048, "prefill"), (3, 3000, "prefill"),
                                           (4, 150, "decode")])
def test_graph_replays(cid, T, variant):
    """A forward captured in a HIP graph (split-K prefill; plain prefill, one launch, with
    fewer and with more tiles than workgroups; decode over a 128-token and a 22-token
    chunk): each of several replays, with
    eager forwards of other inputs in between, writes exactly the eager result; the kernels
    leave their arrival counters at zero for the next call."""
    wl = workloads.WORKLOADS[cid].with_tokens(1, T) if cid == 3 else workloads.WORKLOADS[cid].with_tokens(T, 1)
    inp = workloads.make_inputs(wl, seed=31 + T)
    other = workloads.make_inputs(wl, seed=97 + T)
    dev = lambda i: (i["x"].to(DEV), i["w_norm"].to(DEV), i["w_qkv"].to(DEV),
                     None if i["bias"] is None else i["bias"].to(DEV), i["pos"].to(DEV))
    args, args2 = dev(inp), dev(other)
    with qkv.Plan.for_workload(wl) as plan:
        assert plan.variant(T) == variant
        ref = [t.clone() for t in plan.forward(*args)]
        out = plan.forward(*args)
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            plan.forward(*args, out=out, stream=stream)
        for i in range(4):
            for t in out:
                t.zero_()
            graph.replay()
            torch.cuda.synchronize()
            for name, g, r in zip("QKV", out, ref):
                assert torch.equal(g, r), f"replay {i}: {name} differs from the eager forward"
            plan.forward(*args2)  # eager work between replays
            torch.cuda.synchronize()
