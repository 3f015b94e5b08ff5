"""Python binding of the MI355X fused RMSNorm -> QKV projection -> RoPE library.

Argument marshalling only: torch tensors become device pointers and the current
HIP stream, and every step of the computation runs in the HIP kernels of
``libqkv_mi355x.so`` behind the C ABI declared in ``include/qkv.h``.  There is no
other implementation to fall back to: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkv_mi355x.so")

QKV_OK, QKV_ERR_INVALID_ARG, QKV_ERR_UNSUPPORTED, QKV_ERR_HIP, QKV_ERR_OUT_OF_MEMORY = range(5)
QKV_F32, QKV_BF16 = 0, 1
VARIANTS = {0: "generic", 1: "prefill", 2: "decode", 3: "prefill_split"}

# Entry points of include/qkv.h: name -> (restype, argtypes)
_vp = ctypes.c_void_p
EXPORTS = {
    "qkv_plan_create": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
    "qkv_forward": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qkv_forward_kv_cache": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                            _vp, _vp, _vp, _vp]),
    "qkv_backward": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp]),
    "qkv_swiglu_forward": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_double, _vp, _vp, _vp, _vp, _vp]),
    "qkv_rms_inv": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp]),
    "qkv_rms_norm": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp]),
    "qkv_rope": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp]),
    "qkv_forward_unfused": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qkv_head_norm_rope": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp]),
    "qkv_forward_noalloc": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qkv_plan_variant": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)]),
    "qkv_plan_destroy": (ctypes.c_int, [_vp]),
    "qkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qkv_variant_name": (ctypes.c_char_p, [ctypes.c_int32]),
}


class PlanDesc(ctypes.Structure):
    """Mirror of ``qkv_plan_desc``."""
    _fields_ = [
        ("max_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("has_bias", ctypes.c_int32),
        ("eps", ctypes.c_double),
        ("rope_theta", ctypes.c_double),
        ("flags", ctypes.c_int32),
    ]


QKV_PLAN_PREFILL_PREPASS = 1


class QKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m transformer_rmsnorm_row_amd.build` "
                           "(or __graft_entry__.build()); there is no non-HIP implementation")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().qkv_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != QKV_OK:
        raise QKVError(status, where)


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return QKV_BF16
    if dtype == torch.float32:
        return QKV_F32
    raise ValueError(f"unsupported dtype {dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def swiglu_forward(x: torch.Tensor, w_norm: torch.Tensor, w_gate_up: torch.Tensor, eps: float,
                   out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """RMSNorm then SiLU(a @ W_gate) * (a @ W_up) in one launch; w_gate_up is [H, 2I]
    with the gate columns first.  Returns out [T, I] (bf16)."""
    lib = load_library()
    for name, t in (("x", x), ("w_norm", w_norm), ("w_gate_up", w_gate_up)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    T, H = x.shape
    if w_norm.shape != (H,) or w_gate_up.dim() != 2 or w_gate_up.shape[0] != H or w_gate_up.shape[1] % 2:
        raise ValueError("shapes must be x [T, H], w_norm [H], w_gate_up [H, 2I]")
    I = w_gate_up.shape[1] // 2
    if out is None:
        out = torch.empty((T, I), dtype=x.dtype, device=x.device)
    if out.shape != (T, I) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, I] tensor of x's dtype")
    _check(lib.qkv_swiglu_forward(T, H, I, _dtype_code(x.dtype), float(eps), _ptr(x), _ptr(w_norm),
                                  _ptr(w_gate_up), _ptr(out), _stream_handle(stream)), "qkv_swiglu_forward")
    return out


def forward_noalloc(desc: "PlanDesc", x: torch.Tensor, w_norm: torch.Tensor, w_qkv: torch.Tensor,
                    bias: Optional[torch.Tensor], pos: torch.Tensor,
                    out: Tuple[torch.Tensor, torch.Tensor, torch.Tensor],
                    stream: Optional[torch.cuda.Stream] = None):
    """qkv_forward_noalloc: the forward of a layer described by ``desc`` (a PlanDesc)
    into the caller's ``out = (q, k, v)``, with no plan and no device allocation (its
    scratch is the library's own device array).  Tensors must be contiguous, on the GPU
    and of the layer's shapes; the library validates the rest."""
    lib = load_library()
    q, k, v = out
    for name, t in (("x", x), ("w_norm", w_norm), ("w_qkv", w_qkv), ("pos", pos), ("q", q), ("k", k), ("v", v),
                    ("bias", bias)):
        if t is not None and (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _check(lib.qkv_forward_noalloc(ctypes.byref(desc), x.shape[0], _ptr(x), _ptr(w_norm), _ptr(w_qkv), _ptr(bias),
                                   _ptr(pos), _ptr(q), _ptr(k), _ptr(v), _stream_handle(stream)),
           "qkv_forward_noalloc")
    return q, k, v


def ring_slots(pos: torch.Tensor, capacity: int, first_row: int = 0) -> torch.Tensor:
    """Cache rows of a rolling (circular) key/value cache of ``capacity`` rows that
    starts at row ``first_row``: position p goes to ``first_row + p mod capacity``."""
    if capacity < 1:
        raise ValueError("capacity must be at least 1")
    return (first_row + torch.remainder(pos.to(torch.int64), capacity)).to(torch.int32)


class Plan:
    """A fused-chain plan for one layer shape (wraps ``qkv_plan_create``).

    ``forward(x, w_norm, w_qkv, bias, pos)`` queues one forward on the current
    stream and returns ``(q, k, v)``; ``q`` is ``[T, nq*head_dim]`` and ``k``, ``v``
    are ``[T, nkv*head_dim]``, dense and in the plan's dtype.
    """

    def __init__(self, *, max_tokens: int, hidden: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: torch.dtype = torch.bfloat16, has_bias: bool = False,
                 eps: float = 1e-6, rope_theta: float = 10000.0, prefill_prepass: bool = False):
        self._lib = load_library()
        self.dtype = dtype
        self.hidden = hidden
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.has_bias = bool(has_bias)
        self.max_tokens = max_tokens
        self.n_q = num_q_heads * head_dim
        self.n_kv = num_kv_heads * head_dim
        self.desc = PlanDesc(max_tokens, hidden, num_q_heads, num_kv_heads, head_dim,
                             _dtype_code(dtype), int(bool(has_bias)), float(eps), float(rope_theta),
                             QKV_PLAN_PREFILL_PREPASS if prefill_prepass else 0)
        handle = ctypes.c_void_p()
        _check(self._lib.qkv_plan_create(ctypes.byref(self.desc), ctypes.byref(handle)), "qkv_plan_create")
        self._handle = handle

    @classmethod
    def for_workload(cls, wl, max_tokens: Optional[int] = None, prefill_prepass: bool = False) -> "Plan":
        return cls(max_tokens=max_tokens or wl.tokens, hidden=wl.hidden, num_q_heads=wl.num_q_heads,
                   num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, dtype=wl.torch_dtype,
                   has_bias=wl.has_bias, eps=wl.eps, rope_theta=wl.rope_theta, prefill_prepass=prefill_prepass)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._handle is None:
            raise RuntimeError("plan already closed")
        return self._handle

    def variant(self, num_tokens: int) -> str:
        out = ctypes.c_int32(-1)
        _check(self._lib.qkv_plan_variant(self.handle, num_tokens, ctypes.byref(out)), "qkv_plan_variant")
        return VARIANTS.get(out.value, "unknown")

    def _check_tensor(self, t: torch.Tensor, name: str, shape, dtype) -> None:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def forward(self, x: torch.Tensor, w_norm: torch.Tensor, w_qkv: torch.Tensor,
                bias: Optional[torch.Tensor], pos: torch.Tensor,
                out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                stream: Optional[torch.cuda.Stream] = None):
        T = x.shape[0]
        H, N = self.hidden, self.n_q + 2 * self.n_kv
        self._check_tensor(x, "x", (T, H), self.dtype)
        self._check_tensor(w_norm, "w_norm", (H,), self.dtype)
        self._check_tensor(w_qkv, "w_qkv", (H, N), self.dtype)
        if bias is not None:
            self._check_tensor(bias, "bias", (N,), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        if out is None:
            q = torch.empty((T, self.n_q), dtype=self.dtype, device=x.device)
            k = torch.empty((T, self.n_kv), dtype=self.dtype, device=x.device)
            v = torch.empty((T, self.n_kv), dtype=self.dtype, device=x.device)
        else:
            q, k, v = out
            self._check_tensor(q, "q", (T, self.n_q), self.dtype)
            self._check_tensor(k, "k", (T, self.n_kv), self.dtype)
            self._check_tensor(v, "v", (T, self.n_kv), self.dtype)
        st = self._lib.qkv_forward(self.handle, T, _ptr(x), _ptr(w_norm), _ptr(w_qkv), _ptr(bias), _ptr(pos),
                                   _ptr(q), _ptr(k), _ptr(v), _stream_handle(stream))
        _check(st, "qkv_forward")
        return q, k, v

    def forward_kv_cache(self, x: torch.Tensor, w_norm: torch.Tensor, w_qkv: torch.Tensor,
                         bias: Optional[torch.Tensor], pos: torch.Tensor, slots: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, q: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """One forward whose K and V rows land in rows ``slots[t]`` of the caches
        (``[rows, nkv*head_dim]``, updated in place); returns Q.  Slots outside the
        cache write nothing."""
        T = x.shape[0]
        H, N = self.hidden, self.n_q + 2 * self.n_kv
        self._check_tensor(x, "x", (T, H), self.dtype)
        self._check_tensor(w_norm, "w_norm", (H,), self.dtype)
        self._check_tensor(w_qkv, "w_qkv", (H, N), self.dtype)
        if bias is not None:
            self._check_tensor(bias, "bias", (N,), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        self._check_tensor(slots, "slots", (T,), torch.int32)
        rows = k_cache.shape[0] if k_cache.dim() == 2 else -1
        self._check_tensor(k_cache, "k_cache", (rows, self.n_kv), self.dtype)
        self._check_tensor(v_cache, "v_cache", (rows, self.n_kv), self.dtype)
        if q is None:
            q = torch.empty((T, self.n_q), dtype=self.dtype, device=x.device)
        self._check_tensor(q, "q", (T, self.n_q), self.dtype)
        st = self._lib.qkv_forward_kv_cache(self.handle, T, _ptr(x), _ptr(w_norm), _ptr(w_qkv), _ptr(bias),
                                            _ptr(pos), _ptr(slots), rows, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _stream_handle(stream))
        _check(st, "qkv_forward_kv_cache")
        return q

    def backward(self, x: torch.Tensor, w_norm: torch.Tensor, w_qkv: torch.Tensor, pos: torch.Tensor,
                 dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                 stream: Optional[torch.cuda.Stream] = None):
        """Gradients (dx, dw_norm, dw_qkv, dbias or None) of a loss whose gradients with
        respect to Q, K, V are dq, dk, dv."""
        T = x.shape[0]
        H, N = self.hidden, self.n_q + 2 * self.n_kv
        self._check_tensor(x, "x", (T, H), self.dtype)
        self._check_tensor(w_norm, "w_norm", (H,), self.dtype)
        self._check_tensor(w_qkv, "w_qkv", (H, N), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        self._check_tensor(dq, "dq", (T, self.n_q), self.dtype)
        self._check_tensor(dk, "dk", (T, self.n_kv), self.dtype)
        self._check_tensor(dv, "dv", (T, self.n_kv), self.dtype)
        dx = torch.empty((T, H), dtype=self.dtype, device=x.device)
        dw = torch.empty((H,), dtype=self.dtype, device=x.device)
        dW = torch.empty((H, N), dtype=self.dtype, device=x.device)
        db = torch.empty((N,), dtype=self.dtype, device=x.device) if self.has_bias else None
        st = self._lib.qkv_backward(self.handle, T, _ptr(x), _ptr(w_norm), _ptr(w_qkv), _ptr(pos), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(dx), _ptr(dw), _ptr(dW), _ptr(db),
                                    _stream_handle(stream))
        _check(st, "qkv_backward")
        return dx, dw, dW, db

    def rms_inv(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        T = x.shape[0]
        self._check_tensor(x, "x", (T, self.hidden), self.dtype)
        if out is None:
            out = torch.empty((T,), dtype=torch.float32, device=x.device)
        self._check_tensor(out, "inv_rms", (T,), torch.float32)
        _check(self._lib.qkv_rms_inv(self.handle, T, _ptr(x), _ptr(out), _stream_handle(stream)), "qkv_rms_inv")
        return out

    def rms_norm(self, x: torch.Tensor, w_norm: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """The normalised activations [T, H] alone (qkv_rms_norm)."""
        T = x.shape[0]
        self._check_tensor(x, "x", (T, self.hidden), self.dtype)
        self._check_tensor(w_norm, "w_norm", (self.hidden,), self.dtype)
        if out is None:
            out = torch.empty_like(x)
        self._check_tensor(out, "xn", (T, self.hidden), self.dtype)
        _check(self._lib.qkv_rms_norm(self.handle, T, _ptr(x), _ptr(w_norm), _ptr(out), _stream_handle(stream)),
               "qkv_rms_norm")
        return out

    def rope(self, y: torch.Tensor, bias: Optional[torch.Tensor], pos: torch.Tensor,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Bias and rotation applied in place to a projection output y [T, N] (qkv_rope)."""
        T = y.shape[0]
        N = self.n_q + 2 * self.n_kv
        self._check_tensor(y, "y", (T, N), self.dtype)
        if bias is not None:
            self._check_tensor(bias, "bias", (N,), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        _check(self._lib.qkv_rope(self.handle, T, _ptr(bias), _ptr(pos), _ptr(y), _stream_handle(stream)),
               "qkv_rope")
        return y

    def head_norm_rope(self, y: torch.Tensor, w_qnorm: torch.Tensor, w_knorm: torch.Tensor, pos: torch.Tensor,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
        """Per-head RMSNorm of the Q and K heads of y [T, N], then their rotation, in place
        (qkv_head_norm_rope)."""
        T = y.shape[0]
        N = self.n_q + 2 * self.n_kv
        self._check_tensor(y, "y", (T, N), self.dtype)
        self._check_tensor(w_qnorm, "w_qnorm", (self.head_dim,), self.dtype)
        self._check_tensor(w_knorm, "w_knorm", (self.head_dim,), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        _check(self._lib.qkv_head_norm_rope(self.handle, T, _ptr(w_qnorm), _ptr(w_knorm), _ptr(pos), _ptr(y),
                                            _stream_handle(stream)), "qkv_head_norm_rope")
        return y

    def forward_unfused(self, x: torch.Tensor, w_norm: torch.Tensor, w_qkv: torch.Tensor,
                        bias: Optional[torch.Tensor], pos: torch.Tensor,
                        out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                        stream: Optional[torch.cuda.Stream] = None):
        """The chain as three steps (qkv_forward_unfused); returns (q, k, v) as column
        views of y [T, N], plus (xn, y) for reuse as ``out``."""
        T = x.shape[0]
        H, N = self.hidden, self.n_q + 2 * self.n_kv
        self._check_tensor(x, "x", (T, H), self.dtype)
        self._check_tensor(w_norm, "w_norm", (H,), self.dtype)
        self._check_tensor(w_qkv, "w_qkv", (H, N), self.dtype)
        if bias is not None:
            self._check_tensor(bias, "bias", (N,), self.dtype)
        self._check_tensor(pos, "pos", (T,), torch.int32)
        if out is None:
            xn = torch.empty((T, H), dtype=self.dtype, device=x.device)
            y = torch.empty((T, N), dtype=self.dtype, device=x.device)
        else:
            xn, y = out
            self._check_tensor(xn, "xn", (T, H), self.dtype)
            self._check_tensor(y, "y", (T, N), self.dtype)
        st = self._lib.qkv_forward_unfused(self.handle, T, _ptr(x), _ptr(w_norm), _ptr(w_qkv), _ptr(bias),
                                           _ptr(pos), _ptr(xn), _ptr(y), _stream_handle(stream))
        _check(st, "qkv_forward_unfused")
        nq, nkv = self.n_q, self.n_kv
        return (y[:, :nq], y[:, nq:nq + nkv], y[:, nq + nkv:]), (xn, y)

    def close(self) -> None:
        if self._handle is not None:
            _check(self._lib.qkv_plan_destroy(self._handle), "qkv_plan_destroy")
            self._handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if getattr(self, "_handle", None) is not None:
                self._lib.qkv_plan_destroy(self._handle)
                self._handle = None
        except Exception:
            pass
