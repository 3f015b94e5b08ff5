#!/usr/bin/env python3
"""Throughput of the fused RMSNorm -> QKV projection -> RoPE forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one forward of the whole chain (row reduction, normalise-on-load
projection, bias, rotary embedding, single store of Q/K/V) over one batch of
seeded synthetic input already resident in HBM: for the prefill workloads one launch
of the 128 x 512 MFMA kernel, whose normalised activations never leave the chip.  W
untimed steps, then exactly K steps between two device synchronisations.  Prints one
JSON line.

The headline workload is the largest configuration, the Qwen-7B-shaped prefill with
QKV bias (2 x 8192 tokens).  Besides it the line carries:
  roofline      the forward's achieved rate against the MI355X peak of its bound
                (bf16 dense MFMA 2516.6 TFLOP/s for prefill, HBM 8 TB/s for decode), from
                HIP events on the stream the kernel runs on, plus the HBM traffic measured
                by rocprofv3 counters when it is current;
  configs       every configuration at full size: GPU time and rate, the fp64 oracle's
                full forward timed on the host cores, the worst parity ratio against it
                over every element of Q, K and V (with where it occurs), and SHA-256
                digests of the seeded inputs;
  prefill_prepass_opt_in  the same forward with the opt-in pre-pass form (two launches,
                normalised activations written to HBM and read back), timed beside it;
  decode        the 64-token decode step streaming its weight from HBM (8 weight
                copies rotated so the 256 MB last-level cache cannot hold them);
  other_workloads  two mid-size batches (512 tokens on the GQA shape, 128 decode tokens);
  tp8_shard     one GPU's share of the Llama-7B and GQA prefill forwards under 8-way head
                sharding (whole heads per GPU, no exchange on this path);
  unfused       the chain as three steps (RMSNorm kernel, rocBLAS GEMM, bias+RoPE
                kernel) against the fused forward, on the prefill and decode shapes;
  kv_cache, swiglu, backward  the built next steps (K/V into a cache, the gated MLP,
                the backward on the Llama-7B shape);
  prefill_zero_weight  the headline forward with an all-zero weight, a labelled
                diagnostic: how much of the prefill time is the clock lost to the
                matrix cores' power draw on random operands;
  cpu_baseline  the fp64 CPU oracle on the host cores, one full forward of the
                headline workload (a reported baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "fused RMSNorm+QKV+RoPE tokens/s; TFLOP/s %MFMA peak; decode HBM GB/s %peak"
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters.json")


# sources each kernel is built from: a counter reading stays valid while these are unchanged
# (a plain prefill forward is one launch of prefill_wide_kernel; the opt-in pre-pass form
# is the pre-pass of rownorm.hip, then prefill_kernel)
KERNEL_SOURCES = {
    "prefill_wide_kernel": ("prefill_wide.hip", "device_common.h", "launch.h"),
    "prefill_kernel": ("prefill.hip", "rownorm.hip", "device_common.h", "launch.h"),
    "prefill_pre_kernel": ("gemm.hip", "prefill_pre.h", "backward.h", "rownorm.hip", "device_common.h", "launch.h"),
    "decode_kernel": ("decode.hip", "device_common.h", "launch.h"),
}


def kernel_source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_rmsnorm_row_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per forward (every launch of one forward) of the workload from the
    committed rocprofv3 counter summary, scaled by the plain-copy calibration it holds;
    None unless the reading was taken on the kernels' current sources."""
    try:
        with open(COUNTER_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w or w.get("kernel") not in KERNEL_SOURCES:
        return None
    if w.get("kernel_digest") != kernel_source_digest(w["kernel"]):
        return None
    return int(w["hbm_bytes_per_forward"])


def time_forward(plan, bufs, steps: int, warmup: int):
    import torch
    x, w, W, b, pos, q, k, v = bufs
    for _ in range(warmup):
        plan.forward(x, w, W, b, pos, out=(q, k, v))
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        plan.forward(x, w, W, b, pos, out=(q, k, v))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / 1e3 / steps


def time_forward_kv_cache(qkv, wl, plan, bufs, steps: int, warmup: int, cap: int = 4096):
    """Seconds per forward of the key/value-cache form: each sequence owns `cap` cache
    rows and token t goes to its sequence's first row + pos[t] mod cap."""
    import torch
    x, w, W, b, pos, q, k, v = bufs
    cap = max(cap, wl.seq)  # distinct slots within a sequence
    seq_of = torch.arange(wl.tokens, device=x.device, dtype=torch.int32) // wl.seq
    slots = qkv.ring_slots(pos, cap) + seq_of * cap
    kc = torch.zeros((wl.batch * cap, wl.n_kv), dtype=q.dtype, device=x.device)
    vc = torch.zeros_like(kc)
    for _ in range(warmup):
        plan.forward_kv_cache(x, w, W, b, pos, slots, kc, vc, q=q)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        plan.forward_kv_cache(x, w, W, b, pos, slots, kc, vc, q=q)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def time_forward_cold(plan, bufs, calls: int = 50, flush_mib: int = 512):
    """Per-call times with the last-level cache flushed before each call: a 512 MiB
    buffer is rewritten between calls so x and W come from HBM.  Returns seconds."""
    import torch
    x, w, W, b, pos, q, k, v = bufs
    scratch = torch.empty(flush_mib << 20, dtype=torch.uint8, device=x.device)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(calls):
        scratch.fill_(i & 0xFF)
        start.record()
        plan.forward(x, w, W, b, pos, out=(q, k, v))
        end.record()
        end.synchronize()
        times.append(start.elapsed_time(end) / 1e3)
    del scratch
    return sorted(times)


def copy_bandwidth(mib: int = 1024, reps: int = 20) -> float:
    """Achievable HBM bandwidth of a plain device-to-device copy (bytes read + written
    per second), the practical ceiling the decode step is also reported against."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    seconds = start.elapsed_time(end) / 1e3 / reps
    return 2.0 * src.numel() / seconds


def device_inputs(wl, inp):
    import torch
    dev = "cuda:0"
    x = inp["x"].to(dev)
    w = inp["w_norm"].to(dev)
    W = inp["w_qkv"].to(dev)
    b = None if inp["bias"] is None else inp["bias"].to(dev)
    pos = inp["pos"].to(dev)
    q = torch.empty(wl.tokens, wl.n_q, dtype=wl.torch_dtype, device=dev)
    k = torch.empty(wl.tokens, wl.n_kv, dtype=wl.torch_dtype, device=dev)
    v = torch.empty(wl.tokens, wl.n_kv, dtype=wl.torch_dtype, device=dev)
    return x, w, W, b, pos, q, k, v


def decode_leg(qkv, workloads, replays: int = 125, copies: int = 8):
    """Decode step with the weight streamed from HBM: `copies` distinct (x, W) sets
    (8 x 51 MB > the 256 MB last-level cache), visited round-robin.  The forwards are
    captured once in a HIP graph and replayed, so the GPU time per call is not
    diluted by host launch latency (the decode kernel is a single ~10 us launch)."""
    import torch
    wl = workloads.BY_NAME["gqa_decode"]
    sets = []
    for c in range(copies):
        inp = workloads.make_inputs(wl, seed=1000 * wl.cid + 100 * c)
        sets.append(device_inputs(wl, inp))
    plan = qkv.Plan.for_workload(wl)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for s in sets:
            plan.forward(*s[:5], out=s[5:], stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for s in sets:
            plan.forward(*s[:5], out=s[5:], stream=stream)
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    per_call = start.elapsed_time(end) / 1e3 / (replays * copies)
    # warm-cache figure (one weight set, so the weight sits in the last-level cache),
    # labelled as such: never compared with HBM peak
    warm_graph = torch.cuda.CUDAGraph()
    s0 = sets[0]
    with torch.cuda.graph(warm_graph, stream=stream):
        for _ in range(copies):
            plan.forward(*s0[:5], out=s0[5:], stream=stream)
    warm_graph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        warm_graph.replay()
    end.record()
    torch.cuda.synchronize()
    warm = start.elapsed_time(end) / 1e3 / (replays * copies)
    # the same step writing K and V into a key/value cache (64 sequences x 4096 rows,
    # slot = sequence's first row + position mod 4096) instead of dense outputs
    cap = 4096
    kc = torch.zeros((wl.tokens * cap, wl.n_kv), dtype=wl.torch_dtype, device="cuda:0")
    vc = torch.zeros_like(kc)
    cache_slots = [qkv.ring_slots(s[4], cap) + torch.arange(wl.tokens, device="cuda:0", dtype=torch.int32) * cap
                   for s in sets]
    cache_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cache_graph, stream=stream):
        for s, sl in zip(sets, cache_slots):
            plan.forward_kv_cache(*s[:5], sl, kc, vc, q=s[5], stream=stream)
    cache_graph.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        cache_graph.replay()
    end.record()
    torch.cuda.synchronize()
    per_call_cache = start.elapsed_time(end) / 1e3 / (replays * copies)
    del kc, vc
    variant = plan.variant(wl.tokens)
    plan.close()
    nbytes = wl.algorithmic_bytes()
    gbs = nbytes / per_call / 1e9
    copy_gbs = copy_bandwidth() / 1e9
    return {
        "workload": wl.name, "tokens": wl.tokens, "variant": variant, "us_per_call": round(per_call * 1e6, 3),
        "calls_timed": replays * copies,
        "tokens_per_s": round(wl.tokens / per_call, 1), "algorithmic_bytes": nbytes,
        "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "copy_GBps": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4),
        "tflops": round(wl.flops() / per_call / 1e12, 2),
        "warm_cache_us_per_call": round(warm * 1e6, 3), "weight_copies_rotated": copies,
        "kv_cache_us_per_call": round(per_call_cache * 1e6, 3),
        "kv_cache_hbm_frac": round(nbytes / per_call_cache / 1e9 / PEAK_HBM_GBS, 4),
        "timing": "HIP graph of one forward per weight copy, replayed",
    }


def backward_leg(qkv, workloads, wl, bufs, steps: int = 10, warmup: int = 2):
    """The backward of the chain on the workload's shape: r, unrotate (scaled by r), the
    two GEMMs (this library's MFMA kernel, x itself as dW's operand), norm gradient and
    column sums."""
    import torch
    x, w, W, b, pos, q, k, v = bufs
    g = workloads.make_grads(wl)
    dq, dk, dv = (g[n].to(x.device) for n in ("dq", "dk", "dv"))
    plan = qkv.Plan.for_workload(wl)
    for _ in range(warmup):
        plan.backward(x, w, W, pos, dq, dk, dv)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        plan.backward(x, w, W, pos, dq, dk, dv)
    end.record()
    torch.cuda.synchronize()
    plan.close()
    sec = start.elapsed_time(end) / 1e3 / steps
    gemm_flops = 2 * wl.flops()
    return {"workload": wl.name, "us": round(sec * 1e6, 2), "gemm_flops": gemm_flops,
            "tflops": round(gemm_flops / sec / 1e12, 2), "mfma_frac": round(gemm_flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "dW = diag(w) x^T g and G = g W^T (g = r gy) on this library's 256 x 256 MFMA GEMM; r, "
                    "unrotate, norm gradient and column sums in its other kernels (no vendor library; the "
                    "normalised activations are never formed)"}


def _event_time(fn, steps: int, warmup: int) -> float:
    """Seconds per call of fn, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def unfused_leg(qkv, workloads, steps: int = 30, warmup: int = 5):
    """The chain as three separate steps (RMSNorm kernel -> rocBLAS GEMM -> bias+RoPE
    kernel, qkv_forward_unfused) against the fused forward, on the headline prefill
    shape and on the decode step (weight warm in the last-level cache for both), with
    the two unfused kernels also timed alone.  Algorithmic HBM bytes: fused = x + W +
    Q/K/V once; unfused adds xn written and read back, and y read and written again by
    the rotation."""
    import torch
    res = {}
    for name in ("llama7b_prefill", "gqa_decode"):
        wl = workloads.BY_NAME[name]
        x, w, W, b, pos, q, k, v = device_inputs(wl, workloads.make_inputs(wl))
        plan = qkv.Plan.for_workload(wl)
        _, bufs = plan.forward_unfused(x, w, W, b, pos)
        xn, y = bufs
        fused = _event_time(lambda: plan.forward(x, w, W, b, pos, out=(q, k, v)), steps, warmup)
        unfused = _event_time(lambda: plan.forward_unfused(x, w, W, b, pos, out=bufs), steps, warmup)
        pair = None
        if wl.tokens > 256:
            with qkv.Plan.for_workload(wl, prefill_prepass=True) as pp:
                if pp.variant(wl.tokens) == "prefill":
                    pair = _event_time(lambda: pp.forward(x, w, W, b, pos, out=(q, k, v)), steps, warmup)
        norm = _event_time(lambda: plan.rms_norm(x, w, out=xn), steps, warmup)
        rope = _event_time(lambda: plan.rope(y, b, pos), steps, warmup)
        wn = torch.ones(wl.head_dim, dtype=wl.torch_dtype, device=x.device)
        norm_rope = _event_time(lambda: plan.head_norm_rope(y, wn, wn, pos), steps, warmup)
        plan.close()
        T, H, N, e = wl.tokens, wl.hidden, wl.n_total, 2
        fused_bytes = wl.algorithmic_bytes()
        unfused_bytes = fused_bytes + 2 * T * H * e + 2 * T * N * e
        res[name] = {"tokens": T, "fused_us": round(fused * 1e6, 2), "unfused_us": round(unfused * 1e6, 2),
                     "unfused_over_fused": round(unfused / fused, 3),
                     "prepass_pair_us": None if pair is None else round(pair * 1e6, 2),
                     "unfused_over_prepass_pair": None if pair is None else round(unfused / pair, 3),
                     "rms_norm_us": round(norm * 1e6, 2), "rope_us": round(rope * 1e6, 2),
                     "head_norm_rope_us": round(norm_rope * 1e6, 2),
                     "gemm_us_by_difference": round((unfused - norm - rope) * 1e6, 2),
                     "rms_norm_hbm_GBps": round(2 * T * H * e / norm / 1e9, 1),
                     "rope_hbm_GBps": round(2 * T * N * e / rope / 1e9, 1),
                     "algorithmic_bytes_fused": fused_bytes, "algorithmic_bytes_unfused": unfused_bytes,
                     "kernels": "fused: 1 launch; opt-in pre-pass pair: pre-pass + 256 x 256 MFMA kernel; "
                                "unfused: norm kernel, rocBLAS GEMM, rotation kernel"}
        del x, w, W, b, pos, q, k, v, xn, y, bufs, wn
        torch.cuda.empty_cache()
    return res


def swiglu_leg(qkv, workloads, steps: int = 30, warmup: int = 5):
    """The gated-MLP forward (RMSNorm, gate|up GEMM, SiLU(g) * u) on the Llama-7B MLP
    shape, timed with HIP events on the current stream."""
    import torch
    wl = workloads.MLP_WORKLOADS["llama7b_mlp"]
    inp = workloads.make_mlp_inputs(wl)
    x, w, W = (inp[k].to("cuda:0") for k in ("x", "w_norm", "w_gate_up"))
    out = qkv.swiglu_forward(x, w, W, wl.eps)
    for _ in range(warmup):
        qkv.swiglu_forward(x, w, W, wl.eps, out=out)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        qkv.swiglu_forward(x, w, W, wl.eps, out=out)
    end.record()
    torch.cuda.synchronize()
    sec = start.elapsed_time(end) / 1e3 / steps
    tf = wl.flops() / sec / 1e12
    return {"workload": wl.name, "tokens": wl.tokens, "hidden": wl.hidden, "intermediate": wl.intermediate,
            "us": round(sec * 1e6, 2), "tokens_per_s": round(wl.tokens / sec, 1), "tflops": round(tf, 2),
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": wl.flops(),
            "algorithmic_bytes": wl.algorithmic_bytes()}


def _worst_ratio(gpu, ref):
    """max |gpu - ref| / (1 + |ref|) over one output tensor, with its (t, column);
    a non-finite GPU value counts as infinite."""
    import numpy as np
    ratio = np.abs(gpu - ref) / (1.0 + np.abs(ref))
    ratio = np.where(np.isfinite(gpu), ratio, np.inf)
    t, c = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return float(ratio[t, c]), int(t), int(c)


def _oracle_threads() -> int:
    try:
        import threadpoolctl
        return int(max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1))
    except Exception:
        return os.cpu_count() or 1


def _oracle_forward(wl, inp):
    """One full forward of the fp64 oracle on the host cores: (Q, K, V), seconds."""
    import numpy as np
    import torch
    from oracle import qkv_oracle
    to64 = lambda t: None if t is None else t.to(dtype=torch.float64).numpy()
    args = (to64(inp["x"]), to64(inp["w_norm"]), to64(inp["w_qkv"]), to64(inp["bias"]),
            inp["pos"].numpy().astype(np.int64), wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.eps,
            wl.rope_theta)
    t0 = time.perf_counter()
    out = qkv_oracle.qkv_forward(*args)
    return out, time.perf_counter() - t0


def configs_leg(qkv, workloads, steps: int = 30, warmup: int = 5, headline=None, oracle: bool = True):
    """Every configuration at full size, one record each: the GPU forward (back-to-back
    calls, HIP events on the current stream) against its bound, the fp64 oracle's
    full forward timed on the host cores, the worst |gpu - oracle| / (1 + |oracle|)
    over every element of Q, K and V with where it occurs (the oracle's outputs are the
    parity reference of this run), and SHA-256 digests of the seeded inputs.
    `headline` = (workload name, seconds per forward, (q, k, v)) reuses the headline's
    own timing and outputs instead of running it again."""
    import numpy as np
    import torch
    res = {}
    for wl in workloads.WORKLOADS.values():
        inp = workloads.make_inputs(wl)
        entry = {"tokens": wl.tokens,
                 "sha256_16": {k: workloads.digest(inp[k]) for k in ("x", "w_norm", "w_qkv", "bias", "pos")}}
        if headline is not None and headline[0] == wl.name:
            sec, outs, variant = headline[1], headline[2], headline[3]
            entry["timing"] = "the headline's own timed forwards"
        else:
            bufs = device_inputs(wl, inp)
            with qkv.Plan.for_workload(wl) as plan:
                variant = plan.variant(wl.tokens)
                _, sec = time_forward(plan, bufs, steps, warmup)
            outs = bufs[5:]
            del bufs
        flops, nbytes = wl.flops(), wl.algorithmic_bytes()
        entry.update({"variant": variant, "us": round(sec * 1e6, 2), "tokens_per_s": round(wl.tokens / sec, 1),
                      "tflops": round(flops / sec / 1e12, 3), "hbm_GBps": round(nbytes / sec / 1e9, 1)})
        if wl.tokens > 256:
            peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
            entry["mfma_frac"] = round(flops / sec / 1e12 / peak, 4)
        elif wl.dtype == "bf16":
            entry["hbm_frac_warm"] = round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4)
            entry.setdefault("timing", "weight warm in the last-level cache (the decode object streams it "
                                       "from HBM)")
        else:
            entry.setdefault("timing", "launch-bound (one fp32 kernel with the row reduction fused in)")
        if oracle:
            ref, osec = _oracle_forward(wl, inp)
            tol = 1e-4 if wl.dtype == "fp32" else 2e-2
            worst = None
            for name, g, r in zip("QKV", outs, ref):
                err, t, c = _worst_ratio(g.to("cpu", torch.float64).numpy(), r)
                if worst is None or err > worst[0]:
                    worst = (err, name, t, c)
            entry["oracle"] = {"seconds": round(osec, 3), "seconds_exact": osec, "cores": _oracle_threads(),
                               "tokens_per_s": round(wl.tokens / osec, 1),
                               "gflops_fp64": round(flops / osec / 1e9, 2)}
            entry["parity"] = {"max_ratio": float(f"{worst[0]:.4e}"), "tensor": worst[1], "t": worst[2],
                               "column": worst[3], "tol": tol, "ok": bool(worst[0] <= tol),
                               "compared": "every element of Q, K and V against the oracle's full forward"}
            del ref
        res[wl.name] = entry
        del outs
        torch.cuda.empty_cache()
    return res


def other_workloads_leg(qkv, workloads, steps: int = 30, warmup: int = 5):
    """Two mid-size batches on the configurations' shapes, back-to-back calls timed with
    HIP events on the current stream: 512 tokens of the GQA prefill shape (the prefill
    kernel's split-K form) and 128 sequences of the decode step (one launch of the
    decode kernel's 128-token form)."""
    import torch
    res = {}
    extra = [workloads.BY_NAME["llama3_8b_gqa_prefill"].with_tokens(1, 512),
             workloads.BY_NAME["gqa_decode"].with_tokens(128, 1)]
    for wl in extra:
        inp = workloads.make_inputs(wl)
        bufs = device_inputs(wl, inp)
        with qkv.Plan.for_workload(wl) as plan:
            variant = plan.variant(wl.tokens)
            _, sec = time_forward(plan, bufs, steps, warmup)
        flops, nbytes = wl.flops(), wl.algorithmic_bytes()
        res[wl.name] = {"tokens": wl.tokens, "variant": variant, "us": round(sec * 1e6, 2),
                        "tokens_per_s": round(wl.tokens / sec, 1), "tflops": round(flops / sec / 1e12, 3),
                        "hbm_GBps": round(nbytes / sec / 1e9, 1)}
        del bufs
        torch.cuda.empty_cache()
    return res


def shard_leg(qkv, workloads, steps: int = 30, warmup: int = 5):
    """One GPU's share under 8-way head sharding (tensor parallel, column-parallel W_qkv):
    each GPU takes whole Q heads and whole K/V heads, x is replicated, and there is no
    exchange on this path, so one GPU's time at the shard shape is the sharded forward's
    time.  Llama-7B: 4 Q + 4 K/V heads per GPU (N = 1536); Llama-3-8B GQA: 4 Q + 1 K/V
    head (N = 768); full T.  Compared with an eighth of the unsharded forward's time."""
    import dataclasses
    import torch
    res = {}
    for base_name, nq, nkv in (("llama7b_prefill", 4, 4), ("llama3_8b_gqa_prefill", 4, 1)):
        base = workloads.BY_NAME[base_name]
        wl = dataclasses.replace(base, name=base_name + "_tp8_shard", num_q_heads=nq, num_kv_heads=nkv)
        inp = workloads.make_inputs(wl)
        bufs = device_inputs(wl, inp)
        with qkv.Plan.for_workload(wl) as plan:
            variant = plan.variant(wl.tokens)
            _, sec = time_forward(plan, bufs, steps, warmup)
        flops = wl.flops()
        res[wl.name] = {"tokens": wl.tokens, "n": wl.n_total, "variant": variant, "us": round(sec * 1e6, 2),
                        "tflops": round(flops / sec / 1e12, 2),
                        "mfma_frac": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del bufs
        torch.cuda.empty_cache()
    return res


def prepass_leg(qkv, wl, bufs, steps: int = 30, warmup: int = 5):
    """The same forward through a plan with the opt-in pre-pass form
    (QKV_PLAN_PREFILL_PREPASS): a pre-pass writes bf16(x * w_norm) to HBM and the MFMA
    kernel streams it back, two launches.  Timed here beside the default single launch,
    which never writes the normalised activations."""
    with qkv.Plan.for_workload(wl, prefill_prepass=True) as plan:
        _, sec = time_forward(plan, bufs, steps, warmup)
    return sec


def zero_weight_leg(plan, bufs, steps: int = 30, warmup: int = 5):
    """The same forward with an all-zero weight: identical instructions and memory
    traffic, but matrix-core operands that never toggle.  The ratio to the seeded
    weight's time shows how much of the prefill time is set by the power the matrix
    cores draw on random data (the shader clock is managed down under that load)."""
    import torch
    x, w, W, b, pos, q, k, v = bufs
    Wz = torch.zeros_like(W)
    _, sec = time_forward(plan, (x, w, Wz, b, pos, q, k, v), steps, warmup)
    del Wz
    return sec


def cpu_baseline_leg(wl, inp, seconds=None):
    """The fp64 oracle, as it stands, on the host cores: one full forward (`seconds`:
    the configurations leg already timed that same forward in this run)."""
    dt = seconds if seconds is not None else _oracle_forward(wl, inp)[1]
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": round(wl.tokens / dt, 1), "unit": "tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "cpu_model": cpu,
            "sample": f"one full forward of {wl.name} ({wl.tokens} tokens) in fp64, {dt:.2f} s",
            "seconds": round(dt, 3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen7b_prefill_bias",
                    help="headline workload (default: the largest configuration, the Qwen-7B-shaped prefill)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's shape at this many tokens (one sequence) instead of its own")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle (the headline's baseline and each configuration's oracle and parity)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the key/value-cache, gated-MLP, backward, other-workload and zero-weight legs "
                         "(time only the workload's own forward)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cache-flushed per-call prefill timing (so a profiled run holds only the "
                         "timed back-to-back forwards)")
    ap.add_argument("--prefill-prepass", action="store_true",
                    help="time the opt-in two-launch prefill form (QKV_PLAN_PREFILL_PREPASS) as the step "
                         "instead of the single launch, e.g. to profile the pair")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (steps times), to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings against a known byte count")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": args.steps}))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every token is independent, so the work shards by tokens with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import transformer_rmsnorm_row_amd as qkv
    import workloads

    wl = workloads.BY_NAME[args.workload]
    if args.tokens:
        wl = wl.with_tokens(1, args.tokens)
    inp = workloads.make_inputs(wl)
    bufs = device_inputs(wl, inp)
    plan = qkv.Plan.for_workload(wl, prefill_prepass=args.prefill_prepass)
    variant = plan.variant(wl.tokens)
    prepass_form = args.prefill_prepass and variant == "prefill"
    print(f"[bench] {wl.name}: T={wl.tokens} H={wl.hidden} N={wl.n_total} variant={variant} "
          f"steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    wall, kernel_s = time_forward(plan, bufs, args.steps, args.warmup)
    # the headline's outputs, kept for its parity check against the oracle (the legs
    # below reuse the output buffers)
    head_out = None if args.no_extra or args.tokens else tuple(t.to("cpu") for t in bufs[5:])
    cold = None
    if wl.tokens > 256 and not args.no_cold:
        cold = time_forward_cold(plan, bufs)
    cache_s = None if args.no_extra else time_forward_kv_cache(qkv, wl, plan, bufs, args.steps, args.warmup)
    zero_s = prepass_s = None
    if not args.no_extra and wl.tokens > 256 and wl.dtype == "bf16":
        zero_s = zero_weight_leg(plan, bufs)
    plan.close()
    if not args.no_extra and variant == "prefill" and not prepass_form:
        prepass_s = prepass_leg(qkv, wl, bufs)

    flops = wl.flops()
    nbytes = wl.algorithmic_bytes()
    if wl.tokens <= 256:
        bound, achieved, peak, unit = "hbm", nbytes / kernel_s / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
        bound, achieved, unit = "mfma", flops / kernel_s / 1e12, "TFLOP/s"
    traffic = measured_traffic(wl.name + ("+prepass" if prepass_form else ""))
    # the launches of one forward, all inside the HIP-event window that gives kernel_us
    kernels = {"prefill": ("prenorm_kernel + prefill_pre_kernel (opt-in pre-pass form)" if prepass_form else
                           "prefill_wide_kernel (one launch, normalise-on-load)"),
               "prefill_split": "prefill_kernel (split-K form)",
               "decode": "decode_kernel", "generic": "generic kernel"}.get(variant, variant)
    out = {
        "metric": METRIC,
        "value": round(wl.tokens * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, 1+N(0,0.1) norm weight)",
        "config": {"workload": wl.name, "tokens": wl.tokens, "batch": wl.batch, "seq_len": wl.seq,
                   "hidden": wl.hidden, "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "bias": wl.has_bias, "rope_theta": wl.rope_theta, "eps": wl.eps,
                   "variant": variant, "prefill_prepass": prepass_form},
        "tflops": round(flops / kernel_s / 1e12, 2),
        "mfma_frac": round(flops / kernel_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_us": round(kernel_s * 1e6, 2), "kernels": kernels,
                     "algorithmic_bytes": nbytes, "flops": flops},
    }
    if cache_s is not None:
        out["kv_cache"] = {"us": round(cache_s * 1e6, 2), "tflops": round(flops / cache_s / 1e12, 2),
                           "time_vs_dense": round(cache_s / kernel_s, 4),
                           "cache": "K and V rows written to slot = sequence's first row + position mod C "
                                    "of [batch x C, kv_heads*head_dim] caches, C = max(4096, seq_len)"}
    if prepass_s is not None:
        out["prefill_prepass_opt_in"] = {
            "us": round(prepass_s * 1e6, 2), "time_vs_default": round(prepass_s / kernel_s, 4),
            "tflops": round(flops / prepass_s / 1e12, 2),
            "extra_hbm_bytes": 2 * wl.tokens * wl.hidden * 2,
            "note": "QKV_PLAN_PREFILL_PREPASS: pre-pass writes bf16(x * w_norm) to HBM, the 256 x 256 MFMA kernel "
                    "streams it back (two launches); the headline single launch never writes the normalised "
                    "activations"}
    if zero_s is not None:
        out["prefill_zero_weight"] = {
            "us": round(zero_s * 1e6, 2), "time_vs_seeded": round(zero_s / kernel_s, 4),
            "note": "same kernel and traffic with an all-zero weight (operands that do not toggle): the seeded "
                    "N(0,0.02) weight's extra time is the clock the matrix cores' power draw costs"}
    if cold:
        pct = lambda p: cold[min(len(cold) - 1, int(round(p * (len(cold) - 1))))]
        med = pct(0.5)
        out["prefill_cold"] = {
            "calls": len(cold), "median_us": round(med * 1e6, 2), "p10_us": round(pct(0.1) * 1e6, 2),
            "p90_us": round(pct(0.9) * 1e6, 2), "tflops_median": round(flops / med / 1e12, 2),
            "frac_median": round(flops / med / 1e12 / peak, 4),
            "timing": "each call event-bracketed after rewriting a 512 MiB buffer (last-level cache flushed)"}
    if not args.no_decode and wl.name != "gqa_decode":
        print("[bench] decode leg", file=sys.stderr, flush=True)
        out["decode"] = decode_leg(qkv, workloads)
    if not args.no_extra and wl.name != "gqa_decode":
        print("[bench] gated-MLP leg", file=sys.stderr, flush=True)
        out["swiglu"] = swiglu_leg(qkv, workloads)
        print("[bench] backward leg", file=sys.stderr, flush=True)
        bwl = workloads.BY_NAME["llama7b_prefill"]
        bbufs = device_inputs(bwl, workloads.make_inputs(bwl))
        out["backward"] = backward_leg(qkv, workloads, bwl, bbufs)
        del bbufs
        torch.cuda.empty_cache()
        print("[bench] unfused comparison leg", file=sys.stderr, flush=True)
        out["unfused"] = unfused_leg(qkv, workloads)
        print("[bench] other workloads leg", file=sys.stderr, flush=True)
        out["other_workloads"] = other_workloads_leg(qkv, workloads)
        print("[bench] 8-way head-sharding shard leg", file=sys.stderr, flush=True)
        out["tp8_shard"] = shard_leg(qkv, workloads)
    del bufs
    torch.cuda.empty_cache()
    if not args.no_extra:
        print("[bench] configurations leg (GPU, oracle, parity)", file=sys.stderr, flush=True)
        head = None if head_out is None or prepass_form else (wl.name, kernel_s, head_out, variant)
        out["configs"] = configs_leg(qkv, workloads, headline=head, oracle=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline leg", file=sys.stderr, flush=True)
        own = out.get("configs", {}).get(wl.name, {}).get("oracle") if head_out is not None else None
        out["cpu_baseline"] = cpu_baseline_leg(wl, inp, seconds=None if own is None else own["seconds_exact"])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
