"""Pins for the CPU oracle: checks against facts fixed by the pages and by mathematics,
never against the oracle itself.

Each ``pin_*`` takes an implementation object ``o`` exposing the oracle's functions
(inv_rms, rms_norm, project, rope, qkv_forward) and raises AssertionError when the
implementation disagrees with the fact it pins.  The same pins run on the real
oracle (all must pass) and on deliberately broken copies of it (each copy must be
caught by at least one pin).

Sources of the facts:
  * hand-worked examples under tests/golden/ (each file names its passage);
  * closed forms: RMSNorm with unit weight has mean square m/(m+eps); a constant
    row maps to c/sqrt(c^2+eps); scaling x by alpha and eps by alpha^2 leaves the
    output unchanged;
  * rotations: angle 0 is the identity, every rotated pair keeps its length,
    rotations compose additively, and the per-head inner product of a rotated q and
    k depends only on the position difference;
  * brute force: triple loops in pure Python for the projection, and a complex-number
    formulation of the rotation, written independently of the oracle's code.
"""
from __future__ import annotations

import cmath
import math
import os
import random

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = [float(t) for t in val.split()]
    return out


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- RMSNorm

def pin_rmsnorm_hand_example(o):
    g = load_golden("rmsnorm_hand.txt")
    # the stored decimals are the closed form 1/sqrt(7.5) * x; re-derive them here too
    r_closed = 1.0 / math.sqrt(7.5)
    _close(g["inv_rms"], [r_closed], 1e-15, "golden inv_rms vs closed form")
    x = np.array([g["x"]])
    _close(o.inv_rms(x, g["eps"][0]), g["inv_rms"], 1e-13, "inv_rms hand example")
    _close(o.rms_norm(x, np.array(g["w"]), g["eps"][0])[0], g["a"], 1e-13, "rms_norm hand example")
    _close(o.rms_norm(x, np.array(g["w2"]), g["eps"][0])[0], g["a2"], 1e-13, "rms_norm weighted example")


def pin_rmsnorm_unit_weight_closed_form(o):
    rng = _rng(11)
    H = 96
    for eps in (1e-6, 1e-5, 0.5):
        x = rng.standard_normal((7, H)) * rng.uniform(0.01, 3.0, size=(7, 1))
        m = np.array([sum(float(v) * float(v) for v in row) / H for row in x])
        a = o.rms_norm(x, np.ones(H), eps)
        _close(np.mean(a * a, axis=1), m / (m + eps), 1e-12, f"unit-weight mean square, eps={eps}")


def pin_rmsnorm_scale_invariance(o):
    rng = _rng(12)
    H = 40
    x = rng.standard_normal((5, H))
    w = 1.0 + 0.1 * rng.standard_normal(H)
    eps = 1e-3
    for alpha in (1e-3, 7.0, 1e3):
        _close(o.rms_norm(alpha * x, w, alpha * alpha * eps), o.rms_norm(x, w, eps), 1e-12,
               f"scale invariance alpha={alpha}")


def pin_rmsnorm_constant_row(o):
    H = 24
    w = np.linspace(-2.0, 2.0, H)
    for c, eps in ((3.0, 1e-6), (1e-3, 1e-6), (1e-3, 1e-5), (-0.25, 0.0)):
        x = np.full((1, H), c)
        expect = c / math.sqrt(c * c + eps) * w
        _close(o.rms_norm(x, w, eps)[0], expect, 1e-12, f"constant row c={c} eps={eps}")


# --------------------------------------------------------------------------- projection

def _brute_project(a, W, b):
    T, H = len(a), len(a[0])
    N = len(W[0])
    y = [[0.0] * N for _ in range(T)]
    for t in range(T):
        for n in range(N):
            s = 0.0
            for k in range(H):
                s += float(a[t][k]) * float(W[k][n])
            y[t][n] = s + (float(b[n]) if b is not None else 0.0)
    return y


def pin_project_brute_force(o):
    rng = _rng(13)
    for (T, H, N) in ((3, 5, 12), (4, 8, 6), (1, 16, 24)):
        a = rng.standard_normal((T, H))
        W = rng.standard_normal((H, N))
        b = rng.standard_normal(N)
        _close(o.project(a, W, b), _brute_project(a, W, b), 1e-12, f"projection {T}x{H}x{N} with bias")
        _close(o.project(a, W, None), _brute_project(a, W, None), 1e-12, f"projection {T}x{H}x{N}")


def pin_onehot_layout(o):
    """A single nonzero weight W[k0, n0] = 1 routes a[:, k0] to output column n0;
    this pins the [H, N] orientation and the Q | K | V column split."""
    nq, nkv, d, H = 3, 1, 4, 6
    Nq, Nkv = nq * d, nkv * d
    N = Nq + 2 * Nkv
    rng = _rng(14)
    x = rng.standard_normal((2, H))
    w = 1.0 + 0.1 * rng.standard_normal(H)
    eps = 1e-6
    xd = np.asarray(x, dtype=np.float64)
    r = [1.0 / math.sqrt(sum(v * v for v in row) / H + eps) for row in xd]
    a = [[xd[t][k] * r[t] * w[k] for k in range(H)] for t in range(2)]
    pos0 = np.zeros(2, dtype=np.int64)
    for k0 in (0, 5):
        for n0 in (0, Nq - 1, Nq, Nq + Nkv - 1, Nq + Nkv, N - 1):
            W = np.zeros((H, N))
            W[k0, n0] = 1.0
            q, k, v = o.qkv_forward(x, w, W, None, pos0, nq, nkv, d, eps, 1e4)
            full = np.concatenate([q, k, v], axis=1)
            expect = np.zeros((2, N))
            for t in range(2):
                expect[t][n0] = a[t][k0]
            _close(full, expect, 1e-12, f"one-hot W[{k0},{n0}] at pos 0")
            assert q.shape == (2, Nq) and k.shape == (2, Nkv) and v.shape == (2, Nkv)


def pin_bias_closed_form(o):
    """W = 0: V equals the bias at every position; Q and K equal the bias turned
    by the position's angles (the bias is added before the rotation)."""
    nq, nkv, d, H = 2, 1, 4, 8
    Nq, Nkv = nq * d, nkv * d
    N = Nq + 2 * Nkv
    rng = _rng(15)
    b = rng.standard_normal(N)
    x = rng.standard_normal((3, H))
    pos = np.array([0, 1, 5])
    theta = 100.0
    q, k, v = o.qkv_forward(x, np.ones(H), np.zeros((H, N)), b, pos, nq, nkv, d, 1e-6, theta)
    for t, p in enumerate(pos):
        _close(v[t], b[Nq + Nkv:], 1e-13, "V equals bias")
        for (out, off, nh) in ((q, 0, nq), (k, Nq, nkv)):
            for h in range(nh):
                for i in range(d // 2):
                    ang = p * theta ** (-2.0 * i / d)
                    z = complex(b[off + h * d + i], b[off + h * d + i + d // 2]) * cmath.exp(1j * ang)
                    _close([out[t][h * d + i], out[t][h * d + i + d // 2]], [z.real, z.imag], 1e-12,
                           "rotated bias")


# --------------------------------------------------------------------------- rotary embedding

def pin_rope_hand_example(o):
    g = load_golden("rope_hand.txt")
    d, theta = int(g["head_dim"][0]), g["theta"][0]
    _close(g["e0"], [math.cos(1), 0, math.sin(1), 0], 1e-15, "golden e0 vs closed form")
    for j in range(4):
        e = np.zeros((1, d))
        e[0, j] = 1.0
        _close(o.rope(e, np.array([int(g["pos"][0])]), d, theta)[0], g[f"e{j}"], 1e-13, f"rope e{j} pos 1")
    e = np.zeros((1, d))
    e[0, 0] = 1.0
    _close(o.rope(e, np.array([2]), d, theta)[0], g["pos2_e0"], 1e-13, "rope e0 pos 2")


def pin_rope_identity_at_zero(o):
    rng = _rng(16)
    y = rng.standard_normal((4, 3 * 8))
    _close(o.rope(y, np.zeros(4, dtype=np.int64), 8, 1e4), y, 0.0, "rope at position 0")


def pin_rope_pair_norm(o):
    rng = _rng(17)
    d = 16
    y = rng.standard_normal((6, 2 * d))
    pos = np.array([0, 1, 7, 1000, 32767, 123456])
    out = o.rope(y, pos, d, 5e5)
    for t in range(6):
        for h in range(2):
            for i in range(d // 2):
                c0 = h * d + i
                c1 = c0 + d // 2
                _close(out[t, c0] ** 2 + out[t, c1] ** 2, y[t, c0] ** 2 + y[t, c1] ** 2, 1e-12, "pair norm")


def pin_rope_relative_position(o):
    """<rope(q, m), rope(k, n)> per head depends only on m - n."""
    rng = _rng(18)
    d = 8
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    for (m, n) in ((5, 2), (40, 3), (100, 100)):
        base = float(o.rope(q, np.array([m]), d, 1e4)[0] @ o.rope(k, np.array([n]), d, 1e4)[0])
        for shift in (1, 17, 3000):
            s = float(o.rope(q, np.array([m + shift]), d, 1e4)[0] @ o.rope(k, np.array([n + shift]), d, 1e4)[0])
            _close(s, base, 1e-11, f"relative position m={m} n={n} shift={shift}")


def pin_rope_composition(o):
    rng = _rng(19)
    d = 8
    y = rng.standard_normal((1, 2 * d))
    for (p1, p2) in ((3, 4), (100, 250), (7, 0)):
        two = o.rope(o.rope(y, np.array([p1]), d, 1e4), np.array([p2]), d, 1e4)
        one = o.rope(y, np.array([p1 + p2]), d, 1e4)
        _close(two, one, 1e-12, f"composition {p1}+{p2}")


def pin_v_untouched(o):
    rng = _rng(20)
    nq, nkv, d, H = 2, 2, 4, 8
    N = (nq + 2 * nkv) * d
    x = rng.standard_normal((1, H))
    w = np.ones(H)
    W = rng.standard_normal((H, N))
    _, _, v0 = o.qkv_forward(x, w, W, None, np.array([0]), nq, nkv, d, 1e-6, 1e4)
    for p in (1, 77, 30000):
        _, _, vp = o.qkv_forward(x, w, W, None, np.array([p]), nq, nkv, d, 1e-6, 1e4)
        _close(vp, v0, 0.0, f"V at position {p}")


# --------------------------------------------------------------------------- whole chain

def pin_chain_hand_example(o):
    g = load_golden("chain_hand.txt")
    W = np.array([g["W_row0"], g["W_row1"]])
    q, k, v = o.qkv_forward(np.array([g["x"]]), np.array(g["w"]), W, np.array(g["bias"]),
                            np.array([int(g["pos"][0])]), int(g["num_q_heads"][0]),
                            int(g["num_kv_heads"][0]), int(g["head_dim"][0]), g["eps"][0], g["theta"][0])
    _close(q[0], g["q"], 1e-13, "chain q")
    _close(k[0], g["k"], 1e-13, "chain k")
    _close(v[0], g["v"], 1e-13, "chain v")


def complex_chain(x, w, W, b, pos, nq, nkv, d, eps, theta):
    """Independent pure-Python formulation: each rotated pair is a complex number
    (u + i v) multiplied by exp(i * angle)."""
    T, H = len(x), len(x[0])
    N = len(W[0])
    Nq, Nkv = nq * d, nkv * d
    outs = []
    for t in range(T):
        ss = 0.0
        for kk in range(H):
            ss += float(x[t][kk]) ** 2
        r = (ss / H + eps) ** -0.5
        a = [float(x[t][kk]) * r * float(w[kk]) for kk in range(H)]
        y = []
        for n in range(N):
            s = 0.0
            for kk in range(H):
                s += a[kk] * float(W[kk][n])
            if b is not None:
                s += float(b[n])
            y.append(s)
        out = list(y)
        for (off, nh) in ((0, nq), (Nq, nkv)):
            for h in range(nh):
                for i in range(d // 2):
                    c = off + h * d + i
                    z = complex(y[c], y[c + d // 2]) * cmath.exp(1j * float(pos[t]) * float(theta) ** (-2.0 * i / d))
                    out[c], out[c + d // 2] = z.real, z.imag
        outs.append(out)
    outs = np.array(outs)
    return outs[:, :Nq], outs[:, Nq:Nq + Nkv], outs[:, Nq + Nkv:]


def pin_chain_against_complex(o):
    rng = random.Random(21)
    for (T, H, nq, nkv, d, bias, theta, eps) in ((5, 12, 2, 1, 4, True, 1e4, 1e-6),
                                                 (3, 16, 4, 2, 8, False, 5e5, 1e-5),
                                                 (2, 8, 1, 1, 2, True, 10.0, 0.0)):
        N = (nq + 2 * nkv) * d
        x = [[rng.gauss(0, 1) for _ in range(H)] for _ in range(T)]
        w = [1 + 0.1 * rng.gauss(0, 1) for _ in range(H)]
        W = [[rng.gauss(0, 0.3) for _ in range(N)] for _ in range(H)]
        b = [rng.gauss(0, 1) for _ in range(N)] if bias else None
        pos = [rng.randrange(0, 40000) for _ in range(T)]
        ref = complex_chain(x, w, W, b, pos, nq, nkv, d, eps, theta)
        got = o.qkv_forward(np.array(x), np.array(w), np.array(W), None if b is None else np.array(b),
                            np.array(pos), nq, nkv, d, eps, theta)
        for name, g_, r_ in zip("qkv", got, ref):
            _close(g_, r_, 1e-10, f"chain {name} vs complex formulation (T={T},H={H},d={d})")


def pin_kv_cache_rolling_window(o):
    """A rolling cache of capacity C fed one token at a time at slot pos mod C always
    holds, read from the oldest position to the newest, exactly the last C rows: the
    sliding window that keeps the newest tokens and drops the oldest, as the page's
    RollingBuffer part describes.  The window here is kept by plain list slicing."""
    rng = _rng(41)
    C, T, w = 5, 13, 3
    rows = rng.standard_normal((T, w))
    cache = np.full((C, w), 7.0)
    window = []
    for p in range(T):
        cache = o.kv_cache_write(cache, np.array([p % C]), rows[p:p + 1])
        window = (window + [rows[p]])[-C:]
        oldest = max(0, p - C + 1)
        view = np.stack([cache[q % C] for q in range(oldest, p + 1)])
        _close(view, np.stack(window), 0.0, "rolling view")


def pin_kv_cache_chunks_equal_single_steps(o):
    """Writing a chunk of up to C tokens in one call (distinct slots) leaves the same
    cache as writing them one by one."""
    rng = _rng(42)
    C, T, w = 8, 21, 4
    rows = rng.standard_normal((T, w))
    one = np.zeros((C, w))
    for p in range(T):
        one = o.kv_cache_write(one, np.array([p % C]), rows[p:p + 1])
    chunked = np.zeros((C, w))
    for start in range(0, T, 6):
        pos = np.arange(start, min(T, start + 6))
        chunked = o.kv_cache_write(chunked, pos % C, rows[pos])
    _close(chunked, one, 0.0, "chunked cache")


def pin_kv_cache_untouched_and_dropped(o):
    """Rows no slot names keep their values; slots -1 and past the end write nothing;
    a named row holds exactly the token's row."""
    rng = _rng(43)
    R, w = 6, 3
    cache = rng.standard_normal((R, w))
    rows = rng.standard_normal((5, w))
    slots = np.array([4, -1, 0, R, R + 3])
    out = o.kv_cache_write(cache, slots, rows)
    expect = cache.copy()
    expect[4] = rows[0]
    expect[0] = rows[2]
    _close(out, expect, 0.0, "cache rows")


def _silu_tanh(z):
    """SiLU through the identity sigmoid(z) = (1 + tanh(z/2)) / 2."""
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def pin_silu_values(o):
    """SiLU(0) = 0; SiLU(1) = e/(e+1); SiLU(z) - SiLU(-z) = z; the tanh form of the
    logistic function agrees everywhere."""
    _close(o.silu(np.array([0.0]))[0], 0.0, 0.0, "silu(0)")
    e = np.e
    _close(o.silu(np.array([1.0]))[0], e / (e + 1.0), 1e-15, "silu(1)")
    z = np.linspace(-30.0, 30.0, 241)
    _close(o.silu(z) - o.silu(-z), z, 1e-12, "odd part")
    _close(o.silu(z), _silu_tanh(z), 1e-12, "tanh form")


def pin_swiglu_brute_force(o):
    """Triple loops (row norm, both dot products, tanh-form SiLU) on a tiny case."""
    rng = _rng(51)
    T, H, inter, eps = 3, 8, 5, 1e-5
    x = rng.standard_normal((T, H)) * np.array([[0.1], [1.0], [7.0]])
    w = 1.0 + 0.1 * rng.standard_normal(H)
    W = 0.3 * rng.standard_normal((H, 2 * inter))
    ref = np.zeros((T, inter))
    for t in range(T):
        ms = sum(x[t, k] ** 2 for k in range(H)) / H
        r = 1.0 / np.sqrt(ms + eps)
        a = [x[t, k] * r * w[k] for k in range(H)]
        for j in range(inter):
            g = sum(a[k] * W[k, j] for k in range(H))
            u = sum(a[k] * W[k, inter + j] for k in range(H))
            ref[t, j] = _silu_tanh(g) * u
    _close(o.swiglu_forward(x, w, W, eps), ref, 1e-12, "swiglu brute force")


def pin_swiglu_onehot_layout(o):
    """Gate column j0 reads input feature k0 and up column j0 reads k1: output j0 is
    SiLU(a[:, k0]) * a[:, k1] and every other output is 0 (gate columns come first)."""
    rng = _rng(52)
    T, H, inter, eps = 4, 6, 3, 1e-6
    x = rng.standard_normal((T, H))
    w = np.ones(H)
    W = np.zeros((H, 2 * inter))
    k0, k1, j0 = 2, 5, 1
    W[k0, j0] = 1.0
    W[k1, inter + j0] = 1.0
    a = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
    expect = np.zeros((T, inter))
    expect[:, j0] = _silu_tanh(a[:, k0]) * a[:, k1]
    _close(o.swiglu_forward(x, w, W, eps), expect, 1e-12, "swiglu one-hot")


def pin_backward_finite_differences(o):
    """Every gradient of the backward against central differences of the forward on a
    tiny case (loss = sum of upstream gradient times output), with a bias."""
    rng = _rng(61)
    T, H, nq, nkv, d, eps, theta = 3, 8, 2, 1, 4, 1e-3, 100.0
    N = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, H))
    w = 1.0 + 0.2 * rng.standard_normal(H)
    W = 0.5 * rng.standard_normal((H, N))
    b = 0.3 * rng.standard_normal(N)
    pos = np.array([0, 5, 11])
    gq = rng.standard_normal((T, nq * d))
    gk = rng.standard_normal((T, nkv * d))
    gv = rng.standard_normal((T, nkv * d))

    def loss(x_, w_, W_, b_):
        q, k, v = o.qkv_forward(x_, w_, W_, b_, pos, nq, nkv, d, eps, theta)
        return float(np.sum(q * gq) + np.sum(k * gk) + np.sum(v * gv))

    def fd(arr, f):
        g = np.zeros_like(arr)
        h = 1e-6
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            g[idx] = (f(p) - f(m)) / (2 * h)
        return g

    dx, dw, dW, db = o.qkv_backward(x, w, W, pos, gq, gk, gv, nq, nkv, d, eps, theta, with_bias=True)
    _close(dx, fd(x, lambda v_: loss(v_, w, W, b)), 1e-6, "dx")
    _close(dw, fd(w, lambda v_: loss(x, v_, W, b)), 1e-6, "dw_norm")
    _close(dW, fd(W, lambda v_: loss(x, w, v_, b)), 1e-6, "dW")
    _close(db, fd(b, lambda v_: loss(x, w, W, v_)), 1e-6, "db")


def pin_backward_scale_invariance(o):
    """With eps = 0 the norm's output does not change when a row is scaled, so the input
    gradient of every token is orthogonal to that token's row: sum_j x_j dx_j = 0."""
    rng = _rng(62)
    T, H, nq, nkv, d = 4, 16, 2, 2, 8
    N = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, H)) * np.array([[0.01], [1.0], [3.0], [100.0]])
    w = 1.0 + 0.1 * rng.standard_normal(H)
    W = 0.2 * rng.standard_normal((H, N))
    pos = np.array([3, 0, 7, 1000])
    g = [rng.standard_normal((T, n)) for n in (nq * d, nkv * d, nkv * d)]
    dx, _, _, db = o.qkv_backward(x, w, W, pos, *g, nq, nkv, d, 0.0, 1e4)
    assert db is None
    dots = np.sum(dx * x, axis=1) / (np.linalg.norm(dx, axis=1) * np.linalg.norm(x, axis=1))
    _close(dots, np.zeros(T), 1e-12, "x . dx")


def pin_backward_scales_root_sum_square(o):
    """The tolerance scales of the backward (return_scales) against the root-sum-square
    of every gradient element's terms, each term enumerated one at a time with plain
    loops on a tiny case with a bias.  The terms come from the chain rule (rotation
    transposed, projection, norm); their sums must equal the oracle's gradients, which
    the finite-difference pin fixes independently, so the terms are the right ones
    before their squares are summed.  For dx the two sums (the weighted projection
    gradient, and the norm's inner product times its factor) are separate, and the
    scale is the sum of their two root-sum-squares."""
    rng = _rng(63)
    T, H, nq, nkv, d, eps, theta = 3, 8, 2, 1, 4, 1e-3, 100.0
    half = d // 2
    N = (nq + 2 * nkv) * d
    x = rng.standard_normal((T, H)) * np.array([[0.3], [1.0], [4.0]])
    w = 1.0 + 0.2 * rng.standard_normal(H)
    W = 0.5 * rng.standard_normal((H, N))
    pos = [0, 7, 19]
    gq = rng.standard_normal((T, nq * d))
    gk = rng.standard_normal((T, nkv * d))
    gv = rng.standard_normal((T, nkv * d))
    (dx, dw, dW, db), (s_dx, s_dw, s_dW, s_db) = o.qkv_backward(
        x, w, W, np.array(pos), gq, gk, gv, nq, nkv, d, eps, theta, with_bias=True, return_scales=True)

    # upstream gradient of the projection output: each Q/K pair (i, i + d/2) turned
    # back by its angle (the transpose of the forward rotation), V as it arrives
    g_up = np.concatenate([gq, gk, gv], axis=1)
    gy = [[0.0] * N for _ in range(T)]
    for t in range(T):
        for n in range(N):
            head_start = (n // d) * d
            i = (n - head_start) % half
            if n >= (nq + nkv) * d:
                gy[t][n] = float(g_up[t, n])
                continue
            ang = pos[t] * theta ** (-2.0 * i / d)
            u, v = g_up[t, head_start + i], g_up[t, head_start + i + half]
            if n - head_start < half:
                gy[t][n] = u * math.cos(ang) + v * math.sin(ang)
            else:
                gy[t][n] = v * math.cos(ang) - u * math.sin(ang)
    r = [1.0 / math.sqrt(sum(x[t, k] ** 2 for k in range(H)) / H + eps) for t in range(T)]
    act = [[x[t, k] * r[t] * w[k] for k in range(H)] for t in range(T)]
    ga = [[sum(gy[t][n] * W[k, n] for n in range(N)) for k in range(H)] for t in range(T)]

    def rss(terms):
        return math.sqrt(sum(v * v for v in terms))

    for n in range(N):
        terms = [gy[t][n] for t in range(T)]
        _close(sum(terms), db[n], 1e-12, "db terms")
        _close(rss(terms), s_db[n], 1e-12, "db scale")
    for k in range(H):
        for n in range(N):
            terms = [act[t][k] * gy[t][n] for t in range(T)]
            _close(sum(terms), dW[k, n], 1e-12, "dW terms")
            _close(rss(terms), s_dW[k, n], 1e-12, "dW scale")
        terms = [ga[t][k] * x[t, k] * r[t] for t in range(T)]
        _close(sum(terms), dw[k], 1e-12, "dw_norm terms")
        _close(rss(terms), s_dw[k], 1e-12, "dw_norm scale")
    for t in range(T):
        for j in range(H):
            first = [r[t] * w[j] * gy[t][n] * W[j, n] for n in range(N)]
            second = [-(r[t] ** 3 / H) * x[t, j] * ga[t][k] * w[k] * x[t, k] for k in range(H)]
            _close(sum(first) + sum(second), dx[t, j], 1e-12, "dx terms")
            _close(rss(first) + rss(second), s_dx[t, j], 1e-12, "dx scale")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
