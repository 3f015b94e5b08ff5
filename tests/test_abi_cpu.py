"""The C ABI without a GPU: the library loads, exports every entry point that
include/qkv.h declares, and rejects malformed arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import transformer_rmsnorm_row_amd as qkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkv.h")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qkv_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("qkv_plan_create", "qkv_forward", "qkv_plan_destroy", "qkv_status_string"):
        assert n in names
    assert set(names) == set(qkv.EXPORTS), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = qkv.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_and_variant_strings():
    lib = qkv.load_library()
    assert lib.qkv_status_string(0) == b"ok"
    assert lib.qkv_status_string(1) == b"invalid argument"
    assert lib.qkv_status_string(2).startswith(b"unsupported")
    assert lib.qkv_status_string(99) == b"unknown status"
    assert [lib.qkv_variant_name(i) for i in range(4)] == [b"generic", b"prefill", b"decode", b"prefill_split"]
    assert lib.qkv_variant_name(7) == b"unknown"


def _create(**over):
    lib = qkv.load_library()
    base = dict(max_tokens=16, hidden=64, num_q_heads=4, num_kv_heads=4, head_dim=16, dtype=0, has_bias=0,
                eps=1e-6, rope_theta=1e4)
    base.update(over)
    d = qkv.PlanDesc(**base)
    h = ctypes.c_void_p()
    st = lib.qkv_plan_create(ctypes.byref(d), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("over,expect", [
    (dict(max_tokens=0), qkv.QKV_ERR_INVALID_ARG),
    (dict(max_tokens=-5), qkv.QKV_ERR_INVALID_ARG),
    (dict(hidden=0), qkv.QKV_ERR_INVALID_ARG),
    (dict(num_q_heads=0), qkv.QKV_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), qkv.QKV_ERR_INVALID_ARG),
    (dict(num_q_heads=6, num_kv_heads=4), qkv.QKV_ERR_INVALID_ARG),
    (dict(head_dim=15), qkv.QKV_ERR_INVALID_ARG),
    (dict(head_dim=0), qkv.QKV_ERR_INVALID_ARG),
    (dict(dtype=2), qkv.QKV_ERR_INVALID_ARG),
    (dict(has_bias=2), qkv.QKV_ERR_INVALID_ARG),
    (dict(eps=-1.0), qkv.QKV_ERR_INVALID_ARG),
    (dict(eps=float("nan")), qkv.QKV_ERR_INVALID_ARG),
    (dict(rope_theta=0.0), qkv.QKV_ERR_INVALID_ARG),
    (dict(rope_theta=float("inf")), qkv.QKV_ERR_INVALID_ARG),
    (dict(flags=2), qkv.QKV_ERR_INVALID_ARG),
    (dict(flags=-1), qkv.QKV_ERR_INVALID_ARG),
    (dict(hidden=60), qkv.QKV_ERR_UNSUPPORTED),
    (dict(head_dim=6), qkv.QKV_ERR_UNSUPPORTED),
    (dict(max_tokens=1 << 40), qkv.QKV_ERR_UNSUPPORTED),
    (dict(hidden=1 << 16, num_q_heads=64, num_kv_heads=64, head_dim=256, dtype=1), qkv.QKV_ERR_UNSUPPORTED),
])
def test_bad_descriptor_rejected_before_any_hip_call(over, expect):
    st, h = _create(**over)
    assert st == expect
    assert h.value is None


def test_null_pointers_rejected():
    lib = qkv.load_library()
    h = ctypes.c_void_p()
    assert lib.qkv_plan_create(None, ctypes.byref(h)) == qkv.QKV_ERR_INVALID_ARG
    d = qkv.PlanDesc(16, 64, 4, 4, 16, 0, 0, 1e-6, 1e4)
    assert lib.qkv_plan_create(ctypes.byref(d), None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward(None, 4, *([None] * 8), None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_rms_inv(None, 4, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward_kv_cache(None, 4, *([None] * 6), 16, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_backward(None, 4, *([None] * 11), None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_rms_norm(None, 4, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_rope(None, 4, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward_unfused(None, 4, *([None] * 7), None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_head_norm_rope(None, 4, None, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    v = ctypes.c_int32()
    assert lib.qkv_plan_variant(None, 4, ctypes.byref(v)) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_plan_destroy(None) == qkv.QKV_OK


def test_unknown_handle_rejected():
    lib = qkv.load_library()
    fake = ctypes.create_string_buffer(256)
    assert lib.qkv_plan_destroy(ctypes.cast(fake, ctypes.c_void_p)) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward(ctypes.cast(fake, ctypes.c_void_p), 1, *([None] * 8), None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward_kv_cache(ctypes.cast(fake, ctypes.c_void_p), 1, *([None] * 6), 16,
                                    None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_rms_norm(ctypes.cast(fake, ctypes.c_void_p), 1, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_rope(ctypes.cast(fake, ctypes.c_void_p), 1, None, None, None, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_forward_unfused(ctypes.cast(fake, ctypes.c_void_p), 1, *([None] * 7),
                                   None) == qkv.QKV_ERR_INVALID_ARG


def test_valid_descriptor_without_gpu():
    """Without a device a valid descriptor gets past validation and fails at the first
    HIP call; with one it yields a plan."""
    lib = qkv.load_library()
    st, h = _create()
    if st == qkv.QKV_OK:
        assert lib.qkv_plan_destroy(h) == qkv.QKV_OK
        assert lib.qkv_plan_destroy(h) == qkv.QKV_ERR_INVALID_ARG
    else:
        assert st == qkv.QKV_ERR_HIP
        assert h.value is None


def test_ring_slots_helper():
    """Rolling-cache rows: position p of a cache of capacity C starting at row b is
    row b + p mod C (negative positions wrap the same way)."""
    import torch
    pos = torch.tensor([0, 1, 4, 5, 9, 10, -1], dtype=torch.int32)
    got = qkv.ring_slots(pos, 5, first_row=100)
    assert got.dtype == torch.int32
    assert got.tolist() == [100, 101, 104, 100, 104, 100, 104]
    with pytest.raises(ValueError):
        qkv.ring_slots(pos, 0)


def test_swiglu_arguments_rejected_before_any_hip_call():
    """The stateless gated-MLP call validates sizes, dtype, eps and pointers first; shapes
    the kernel does not implement are QKV_ERR_UNSUPPORTED, all without touching a GPU."""
    lib = qkv.load_library()
    fake = 1 << 20  # 16-byte aligned, never dereferenced: every case below fails validation
    ok_ptrs = [fake] * 4
    bf16 = qkv.QKV_BF16
    assert lib.qkv_swiglu_forward(0, 4096, 11008, bf16, 1e-6, *([None] * 4), None) == qkv.QKV_OK
    assert lib.qkv_swiglu_forward(-1, 4096, 11008, bf16, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 0, 11008, bf16, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, 7, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, bf16, -1.0, *ok_ptrs, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, bf16, float("nan"), *ok_ptrs, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, bf16, 1e-6, None, fake, fake, fake, None) == qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, bf16, 1e-6, fake + 2, fake, fake, fake, None) == \
        qkv.QKV_ERR_INVALID_ARG
    assert lib.qkv_swiglu_forward(4, 4096, 11008, qkv.QKV_F32, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_UNSUPPORTED
    assert lib.qkv_swiglu_forward(4, 4000, 11008, bf16, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_UNSUPPORTED
    assert lib.qkv_swiglu_forward(4, 4096, 11000, bf16, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_UNSUPPORTED
    assert lib.qkv_swiglu_forward(1 << 20, 4096, 11008, bf16, 1e-6, *ok_ptrs, None) == qkv.QKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("shape", [
    dict(hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=1),    # widest row: N = 6144
    dict(hidden=4096, num_q_heads=32, num_kv_heads=32, head_dim=128, dtype=1),   # N = 12288
    dict(hidden=8192, num_q_heads=8, num_kv_heads=8, head_dim=128, dtype=0),     # widest row: x, fp32
])
def test_token_limit_is_exact(shape):
    """Every kernel addresses a tensor with 32-bit byte offsets, so a plan's token count
    times its widest row (x, or the projection's N columns) times the element size must
    stay below 2^31: the first count at that bound is refused before any HIP call, and
    the count below it gets past validation."""
    elem = 2 if shape["dtype"] == 1 else 4
    n = (shape["num_q_heads"] + 2 * shape["num_kv_heads"]) * shape["head_dim"]
    limit = (1 << 31) // (max(n, shape["hidden"]) * elem)
    st, h = _create(max_tokens=limit, **shape)
    assert st == qkv.QKV_ERR_UNSUPPORTED and h.value is None
    st, h = _create(max_tokens=limit - 1, **shape)
    assert st in (qkv.QKV_OK, qkv.QKV_ERR_HIP)
    if st == qkv.QKV_OK:
        assert qkv.load_library().qkv_plan_destroy(h) == qkv.QKV_OK


@pytest.mark.parametrize("hidden", [8192, 4096])
def test_prepass_buffer_limit_is_exact(hidden):
    """The pre-pass form keeps bf16(x * w_norm) for max_tokens rows rounded up to whole
    256-row panels; that buffer is addressed with 32-bit byte offsets too, so the first
    token count whose padded buffer reaches 2^31 bytes is refused before any HIP call
    even where the tensors themselves stay below the bound, and the last count whose
    padded buffer fits gets past validation."""
    shape = dict(hidden=hidden, num_q_heads=8, num_kv_heads=8, head_dim=128, dtype=1)
    n = 3 * 8 * 128
    rows = (1 << 31) // (hidden * 2)              # padded rows that reach 2^31 bytes
    first_bad = rows - 255                         # rounds up to `rows`
    assert first_bad < (1 << 31) // (max(n, hidden) * 2)  # the tensors alone would pass
    st, h = _create(max_tokens=first_bad, **shape)
    assert st in (qkv.QKV_OK, qkv.QKV_ERR_HIP, qkv.QKV_ERR_OUT_OF_MEMORY)
    if st == qkv.QKV_OK:
        assert qkv.load_library().qkv_plan_destroy(h) == qkv.QKV_OK
    st, h = _create(max_tokens=first_bad, flags=qkv.QKV_PLAN_PREFILL_PREPASS, **shape)
    assert st == qkv.QKV_ERR_UNSUPPORTED and h.value is None
    st, h = _create(max_tokens=first_bad - 1, flags=qkv.QKV_PLAN_PREFILL_PREPASS, **shape)
    assert st in (qkv.QKV_OK, qkv.QKV_ERR_HIP, qkv.QKV_ERR_OUT_OF_MEMORY)
    if st == qkv.QKV_OK:
        assert qkv.load_library().qkv_plan_destroy(h) == qkv.QKV_OK


def _noalloc(desc, T, ptrs=None, bias=None):
    lib = qkv.load_library()
    p = ptrs if ptrs is not None else [16] * 8  # x, w_norm, w_qkv, pos, q, k, v (16-byte aligned dummies)
    return lib.qkv_forward_noalloc(None if desc is None else ctypes.byref(desc), T, p[0], p[1], p[2], bias, p[3],
                                   p[4], p[5], p[6], None)


def test_noalloc_rejects_bad_arguments_before_any_hip_call():
    """qkv_forward_noalloc validates the descriptor and every argument before it looks
    up its device array or launches anything (these calls run without a GPU)."""
    good = dict(max_tokens=16, hidden=64, num_q_heads=4, num_kv_heads=4, head_dim=16, dtype=0, has_bias=0,
                eps=1e-6, rope_theta=1e4)
    d = qkv.PlanDesc(**good)
    assert _noalloc(None, 4) == qkv.QKV_ERR_INVALID_ARG
    assert _noalloc(qkv.PlanDesc(**{**good, "head_dim": 15}), 4) == qkv.QKV_ERR_INVALID_ARG
    assert _noalloc(qkv.PlanDesc(**{**good, "hidden": 60}), 4) == qkv.QKV_ERR_UNSUPPORTED
    assert _noalloc(d, 0, ptrs=[None] * 8) == qkv.QKV_OK           # T == 0 touches nothing
    assert _noalloc(d, -1) == qkv.QKV_ERR_INVALID_ARG
    assert _noalloc(d, 17) == qkv.QKV_ERR_INVALID_ARG              # above max_tokens
    for i in range(7):
        ptrs = [16] * 8
        ptrs[i] = None
        assert _noalloc(d, 4, ptrs=ptrs) == qkv.QKV_ERR_INVALID_ARG
        ptrs[i] = 24 if i != 3 else 2                                  # misaligned
        assert _noalloc(d, 4, ptrs=ptrs) == qkv.QKV_ERR_INVALID_ARG
    assert _noalloc(d, 4, bias=16) == qkv.QKV_ERR_INVALID_ARG       # bias on a plan without one
    db = qkv.PlanDesc(**{**good, "has_bias": 1})
    assert _noalloc(db, 4) == qkv.QKV_ERR_INVALID_ARG              # missing bias
    # the pre-pass form needs plan scratch
    assert _noalloc(qkv.PlanDesc(**{**good, "flags": qkv.QKV_PLAN_PREFILL_PREPASS}), 4) == qkv.QKV_ERR_UNSUPPORTED
    # a rotary table larger than its slot in the device array
    big = qkv.PlanDesc(**{**good, "hidden": 2048, "num_q_heads": 1, "num_kv_heads": 1, "head_dim": 1040})
    assert _noalloc(big, 4) == qkv.QKV_ERR_UNSUPPORTED
