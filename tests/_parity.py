"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare element by element."""
from __future__ import annotations

import numpy as np
import torch

from oracle import qkv_oracle

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_inputs(inp: dict):
    return (to_f64(inp["x"]), to_f64(inp["w_norm"]), to_f64(inp["w_qkv"]),
            None if inp["bias"] is None else to_f64(inp["bias"]), inp["pos"].numpy().astype(np.int64))


def oracle_forward(wl, inp: dict, rows=None):
    x, w, W, b, pos = oracle_inputs(inp)
    args = (wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps, wl.rope_theta)
    if rows is None:
        return qkv_oracle.qkv_forward(x, w, W, b, pos, *args)
    return qkv_oracle.qkv_forward_rows(rows, x, w, W, b, pos, *args)


def worst(gpu: np.ndarray, ref: np.ndarray):
    """max |gpu - ref| / (1 + |ref|) and where it occurs; NaN/Inf counts as infinite."""
    if gpu.shape != ref.shape:
        raise AssertionError(f"shape {gpu.shape} vs {ref.shape}")
    if gpu.size == 0:
        return 0.0, None
    ratio = np.abs(gpu - ref) / (1.0 + np.abs(ref))
    ratio = np.where(np.isfinite(gpu), ratio, np.inf)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return float(ratio[idx]), tuple(int(i) for i in idx)


def assert_parity(gpu_qkv, ref_qkv, tol: float, what: str, rows=None):
    msgs = []
    for name, g, r in zip("QKV", gpu_qkv, ref_qkv):
        g = to_f64(g) if isinstance(g, torch.Tensor) else g
        if rows is not None:
            g = g[rows]
        err, loc = worst(g, r)
        msgs.append(f"{name}: {err:.3e} at {loc}")
        assert err <= tol, f"{what}: {name} worst |gpu-oracle|/(1+|oracle|) = {err:.3e} > {tol} at {loc}"
    return msgs


def sample_rows(T: int, n: int, seed: int) -> np.ndarray:
    """The first and last 4 rows, the two rows on either side of every 256-row tile
    edge, plus random rows up to n in all (more than n when the fixed rows are)."""
    rng = np.random.default_rng(seed)
    fixed = set(range(min(T, 4))) | set(range(max(0, T - 4), T))
    for edge in range(256, T, 256):
        fixed |= {edge - 1, edge}
    extra = rng.choice(T, size=min(T, max(0, n - len(fixed))), replace=False)
    return np.array(sorted(fixed | set(int(e) for e in extra)))
