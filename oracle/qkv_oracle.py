"""CPU oracle for the fused RMSNorm -> QKV projection -> rotary-embedding chain.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library and is deliberately slow and plain.

What it computes is the unfused definition of the attention-input chain that the
page "Liger-Kernel底层优化：新一代内核级推理加速引擎介绍" (Liger-Kernel low-level
optimisation: a new kernel-level inference acceleration engine) lists for one
Llama-style decoder layer in its opening section: normalise x with RMSNorm,
project it to q, k, v, then apply the rotary embedding to q and to k.  Where the
same page's fused-kernel listing (section "融合内核是如何工作的？来看一段简化版实现",
how the fused kernel works) is consistent with that chain it fixes the details:

  * step 1: sum of squares over the whole hidden size, divided by the hidden size,
    eps added inside the reciprocal square root;
  * step 2: each input element is scaled by that factor and by the learned
    weight before it enters the dot products with the projection weights; the
    bias is added to each dot product;
  * step 3: the rotation pairs feature i with feature i + head_dim/2 (the index
    is taken modulo head_dim/2).

Readings taken where the pages are silent or garbled (the fused listing mixes up
k and v, leaves q unrotated, indexes the tables by frequency only and uses the
opposite sign): rotate q and k (not v), by +angle, counter-clockwise; the
angle of pair i at position p is p * theta**(-2i/head_dim).

Everything is float64 on the exact input values (bf16 and fp32 inputs widen
to float64 without rounding); no intermediate result is rounded.  A library
matrix product serves as the projection step.
"""
from __future__ import annotations

import numpy as np


def inv_rms(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-token reciprocal root-mean-square, r[t] = 1/sqrt(mean_k x[t,k]^2 + eps).

    Fused-kernel listing, step 1: the mean is over the full hidden size and eps
    sits inside the square root.
    """
    x = np.asarray(x, dtype=np.float64)
    mean_sq = np.mean(x * x, axis=-1)
    return 1.0 / np.sqrt(mean_sq + eps)


def rms_norm(x: np.ndarray, w_norm: np.ndarray, eps: float) -> np.ndarray:
    """a[t,k] = x[t,k] * r[t] * w[k]  (fused-kernel listing, step 2: the
    normalised input element; the weight multiplies, it is not 1 + weight)."""
    x = np.asarray(x, dtype=np.float64)
    w_norm = np.asarray(w_norm, dtype=np.float64)
    return x * inv_rms(x, eps)[:, None] * w_norm[None, :]


def project(a: np.ndarray, w_qkv: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """y[t,n] = sum_k a[t,k] * W[k,n] (+ b[n]).

    The projection proj_qkv of the decoder-layer listing, with the weight held
    as one [hidden, N] matrix whose columns are the Q heads, then the K heads,
    then the V heads.  The bias is added before any rotation (fused-kernel
    listing: the bias add precedes step 3).
    """
    y = np.asarray(a, dtype=np.float64) @ np.asarray(w_qkv, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[t, i] = pos[t] * theta**(-2i/head_dim) for i < head_dim/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(y: np.ndarray, pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of every head in y [T, heads*head_dim].

    Feature i of a head pairs with feature i + head_dim/2 (fused-kernel listing,
    step 3); the pair (u, v) turns by +angle: (u cos - v sin, v cos + u sin).
    """
    T = y.shape[0]
    half = head_dim // 2
    heads = y.reshape(T, -1, head_dim)
    phi = rope_angles(pos, head_dim, theta)[:, None, :]
    c, s = np.cos(phi), np.sin(phi)
    u, v = heads[..., :half], heads[..., half:]
    out = np.concatenate([u * c - v * s, v * c + u * s], axis=-1)
    return out.reshape(T, -1)


def qkv_forward(x, w_norm, w_qkv, bias, pos, num_q_heads: int, num_kv_heads: int,
                head_dim: int, eps: float, theta: float):
    """The whole chain: (Q, K, V) in float64, Q [T, nq*d], K and V [T, nkv*d].

    Order as in the decoder-layer listing: rms_norm, proj_qkv, rotary on q,
    rotary on k; v leaves the projection unchanged.  Heads of different widths
    (grouped-query attention, fewer K/V heads than Q heads) only change how many
    columns each of the three outputs takes.
    """
    n_q = num_q_heads * head_dim
    n_kv = num_kv_heads * head_dim
    a = rms_norm(x, w_norm, eps)
    y = project(a, w_qkv, bias)
    assert y.shape[1] == n_q + 2 * n_kv, "W_qkv must have (nq + 2*nkv)*head_dim columns"
    q = rope(y[:, :n_q], pos, head_dim, theta)
    k = rope(y[:, n_q:n_q + n_kv], pos, head_dim, theta)
    v = y[:, n_q + n_kv:].copy()
    return q, k, v


def qkv_forward_rows(rows, x, w_norm, w_qkv, bias, pos, num_q_heads, num_kv_heads,
                     head_dim, eps, theta):
    """The same chain evaluated for a subset of tokens only (each token's
    outputs depend on its own row of x, its own position and the weights)."""
    rows = np.asarray(rows)
    return qkv_forward(np.asarray(x)[rows], w_norm, w_qkv, bias, np.asarray(pos)[rows],
                       num_q_heads, num_kv_heads, head_dim, eps, theta)


def kv_cache_write(cache, slots, rows):
    """Key/value cache after one forward writes its K (or V) rows into it.

    The RollingBuffer part of the page "Liger-Kernel内核级优化：FlashAttention与
    RollingBuffer详解" (Liger-Kernel kernel-level optimisation: FlashAttention and
    RollingBuffer explained) keeps keys and values in a buffer allocated once at its
    full size and writes new rows over old ones in place instead of concatenating.
    Which row a token lands in is the caller's choice, given as slots[t]: token t's
    row replaces cache row slots[t]; a slot outside [0, cache rows) writes nothing;
    every other row keeps its value.  (Reading: the page's ring reuse corresponds to
    slots[t] = pos[t] mod capacity; the slots themselves are an input here.)
    Returns a new float64 array; `cache` is not modified.
    """
    out = np.array(cache, dtype=np.float64, copy=True)
    rows = np.asarray(rows, dtype=np.float64)
    slots = np.asarray(slots)
    seen = set()
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if 0 <= s < out.shape[0]:
            assert s not in seen, "two tokens of one forward name the same slot"
            seen.add(s)
            out[s] = rows[t]
    return out


def silu(z):
    """SiLU (swish): z / (1 + exp(-z)); exp overflow for very negative z gives -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_parts(x, w_norm, w_gate_up, eps: float):
    """The gate and up sums (g, u), each [T, I] float64, before the SiLU and product."""
    act = rms_norm(x, w_norm, eps)
    y = act @ np.asarray(w_gate_up, dtype=np.float64)
    assert y.shape[1] % 2 == 0, "W_gate_up must have an even number of columns"
    inter = y.shape[1] // 2
    gate, up = y[:, :inter], y[:, inter:]
    return gate, up


def swiglu_forward(x, w_norm, w_gate_up, eps: float):
    """Gated MLP input of the decoder layer: out [T, I] in float64.

    The operator-fusion section ("算子融合") of the page "Liger-Kernel核心技术：
    RollingBuffer与融合算子详解" (Liger-Kernel core techniques: RollingBuffer and
    fused operators explained) describes the fused linear SwiGLU: the input times the
    gate weight and times the up weight, SiLU of the first times the second.  Here its
    input is the layer's RMSNorm output, computed as in qkv_forward, and the two
    weights are one [H, 2I] matrix with the gate columns first.  No bias.
    """
    gate, up = swiglu_parts(x, w_norm, w_gate_up, eps)
    return silu(gate) * up


def qkv_backward(x, w_norm, w_qkv, pos, gq, gk, gv, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, eps: float, theta: float, with_bias: bool = False,
                 return_scales: bool = False):
    """Gradients of the chain for upstream gradients gq, gk, gv of Q, K, V.

    The operator-fusion section ("算子融合") of the page "Liger-Kernel核心技术：
    RollingBuffer与融合算子详解" reports backward speed-ups for its fused kernels
    alongside the forward ones; the backward of this chain is the chain rule applied
    to the forward above, written out step by step in float64:

      * rotation: the transpose of a rotation by +angle is the rotation by -angle,
        so gy = (gu cos + gv sin, gv cos - gu sin) on each Q/K pair; gy = gv on V;
      * bias: db[n] = sum_t gy[t, n];
      * projection: dW = a^T gy, ga = gy W^T;
      * RMSNorm a = x r w with r = (mean x^2 + eps)^(-1/2), dr/dx_j = -r^3 x_j / H:
        dw[k] = sum_t ga[t,k] x[t,k] r[t];
        dx[t,j] = r w_j ga_j - (r^3 / H) x_j sum_k ga_k w_k x_k.

    Returns (dx, dw_norm, dw_qkv, dbias or None), float64.  With return_scales, also
    the root-sum-square of the terms that each element of those gradients sums, the
    scale that a sum of individually rounded terms is accurate to: over tokens for
    dw_norm (terms ga x r), dW (terms a gy) and db (terms gy); for dx, which is two
    separate sums, the root-sum-square of the first's terms r w_j gy_n W[j,n] (over
    output columns n) plus that of the second's terms (r^3/H) x_j ga_k w_k x_k (over k).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_norm, dtype=np.float64)
    W = np.asarray(w_qkv, dtype=np.float64)
    T, H = x.shape
    half = head_dim // 2
    phi = rope_angles(pos, head_dim, theta)[:, None, :]
    c, s = np.cos(phi), np.sin(phi)

    def unrotate(g):
        heads = np.asarray(g, dtype=np.float64).reshape(T, -1, head_dim)
        gu, gv_ = heads[..., :half], heads[..., half:]
        return np.concatenate([gu * c + gv_ * s, gv_ * c - gu * s], axis=-1).reshape(T, -1)

    gy = np.concatenate([unrotate(gq), unrotate(gk), np.asarray(gv, dtype=np.float64)], axis=1)
    assert gy.shape[1] == W.shape[1], "upstream gradients must cover every column of W_qkv"
    db = gy.sum(axis=0) if with_bias else None
    r = inv_rms(x, eps)
    a = x * r[:, None] * w[None, :]
    dW = a.T @ gy
    ga = gy @ W.T
    dw = np.sum(ga * x * r[:, None], axis=0)
    inner = np.sum(ga * w[None, :] * x, axis=1)
    dx = r[:, None] * w[None, :] * ga - (r ** 3 / H)[:, None] * x * inner[:, None]
    if return_scales:
        # root-sum-square of the terms each gradient element sums (see the docstring)
        sq = lambda m: np.sqrt(np.maximum(m, 0.0))
        scales = (r[:, None] * np.abs(w)[None, :] * sq((gy * gy) @ (W * W).T)
                  + (r ** 3 / H)[:, None] * np.abs(x) * sq(np.sum((ga * w[None, :] * x) ** 2, axis=1))[:, None],
                  sq(np.sum((ga * x * r[:, None]) ** 2, axis=0)),
                  sq((a * a).T @ (gy * gy)),
                  sq(np.sum(gy * gy, axis=0)) if with_bias else None)
        return (dx, dw, dW, db), scales
    return dx, dw, dW, db
