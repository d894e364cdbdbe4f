#!/usr/bin/env python3
"""Attention-forward throughput on one MI355X.

One step = one attention forward (every kernel of the path) over the
workload's synthetic inputs, already resident in HBM.  Prints one JSON line:
TFLOP/s (4*B*Hq*Nq*Nkv*D, halved when causal), the fraction of the dense
bf16/fp16 MFMA peak, a parity check of sampled rows against the CPU oracle,
and that oracle's own throughput on the same rows (a reported baseline).

With ``--pass bwd`` a step is one gradient computation (attn_bwd: dQ, dK, dV
from the forward's output and log-sum-exp, computed once before timing) and
the algorithmic flops are 2.5 times the forward's (five products of the
forward's size: S again, dP, dV, dK, dQ); parity covers dQ of sampled rows.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
                    [--pass fwd|bwd]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "memory_efficient_tiled_amd", "csrc")
# the kernel sources each pass runs (a measurement taken on other sources is stale)
SOURCES = {"fwd": ("attn_common.h", "attn_tiles.h", "attn_plan.h", "attn_fwd_kernel.h",
                   "attn_fwd.hip", "attn_fwd_d64.hip", "attn_fwd_d80.hip", "attn_fwd_d96.hip",
                   "attn_fwd_d128.hip", "attn_fwd_d256.hip", "attn_fwd_d192v128.hip"),
           "bwd": ("attn_common.h", "attn_tiles.h", "attn_plan.h", "attn_bwd.hip"),
           # the FP8 kernel, and the plan and merge it shares with the 16-bit path
           "fp8": ("attn_common.h", "attn_tiles.h", "attn_plan.h", "attn_fwd_kernel.h",
                   "attn_fwd.hip", "attn_fwd_d128.hip", "attn_fwd_fp8.hip"),
           "ffn": ("attn_common.h", "attn_tiles.h", "ffn_chunked.hip")}
PROFILES = os.path.join(ROOT, "profiles")


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(pass_: str = "fwd") -> str:
    h = hashlib.sha256()
    for name in SOURCES[pass_]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, pass_: str = "fwd", kernels: str | None = None):
    """HBM bytes per step from a committed counter summary, if it was taken
    on the current kernel sources (``kernels``: the SOURCES key, default
    ``pass_``); otherwise None."""
    kernels = kernels or pass_
    path = os.path.join(PROFILES, f"attn_{pass_}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    t = re.search(r"hbm bytes per step:\s*`?([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != source_hash(kernels):
        return None
    return float(t.group(1))


class StreamOrderedPeak:
    """High-water mark of the library's workspace pool on the device
    (attn_workspace_pool; it serves every stream-ordered workspace): reset
    before the timed region, read after it, through the HIP runtime this
    process has already loaded (the one torch and the library share)."""

    USED_MEM_HIGH = 0x8   # hipMemPoolAttrUsedMemHigh

    def __init__(self, device_index: int = 0):
        import ctypes
        self.ok = False
        path = None
        with open("/proc/self/maps") as f:
            for ln in f:
                if "libamdhip64.so" in ln:
                    path = ln.split()[-1]
                    break
        if path is None:
            return
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        from memory_efficient_tiled_amd import binding
        import torch
        with torch.cuda.device(device_index):
            self.pool = ctypes.c_void_p(binding.workspace_pool())
        self.ok = True

    def reset(self):
        if self.ok:
            zero = self.ct.c_uint64(0)
            self.hip.hipMemPoolSetAttribute(self.pool, self.USED_MEM_HIGH, self.ct.byref(zero))

    def read(self):
        if not self.ok:
            return None
        v = self.ct.c_uint64(0)
        if self.hip.hipMemPoolGetAttribute(self.pool, self.USED_MEM_HIGH,
                                           self.ct.byref(v)) != 0:
            return None
        return int(v.value)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="0 = library choice")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="query rows per head for the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mask", choices=("none", "pad"), default="none",
                    help="pad: a boolean key-padding mask [B, 1, 1, Nkv] that keeps the "
                         "first 7/8 of the keys (timing only: no CPU leg)")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd", "ffn"), default="fwd",
                    help="time the forward (default) or the gradients")
    ap.add_argument("--ffn-chunk", type=int, default=None,
                    help="--pass ffn: token rows per chunk (default: the workload's; 0 = library)")
    ap.add_argument("--graph", action="store_true",
                    help="forward only: capture one step (attn_fwd_noalloc, which allocates "
                         "nothing) in a HIP graph and time its replays, as a serving loop "
                         "does for launch-bound shapes such as decode")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this size "
                         "(scales the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this attention forward runs on one GPU; --gpus "
              f"{args.gpus} is not supported (sharding over heads is described "
              "in the design notes, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": max(1, args.steps)}), flush=True)
        return

    from memory_efficient_tiled_amd import (attn_bwd, attn_fwd, attn_fwd_fp8, attn_fwd_noalloc,
                                            attn_fwd_num_splits, attn_fwd_plan, inputs)
    from memory_efficient_tiled_amd.binding import ATTN_BF16, ATTN_F16

    if args.pass_ == "ffn":
        return bench_ffn(args, torch, np)
    bwd = args.pass_ == "bwd"
    name = args.workload or inputs.HEADLINE
    w = inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    progress(f"workload {name}: {w.describe()}; pass {args.pass_}; generating inputs")
    want_cpu = not args.no_cpu_baseline and args.mask == "none"
    x = inputs.make_workload_inputs(w, seed=args.seed,
                                    sampled_rows=args.cpu_rows if want_cpu else None)

    fp8 = w.dtype == "fp8"
    if fp8 and args.pass_ == "bwd":
        raise SystemExit("bench.py: the FP8 path has no gradients")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if w.dtype == "bf16"
                             else np.ascontiguousarray(a))
        t = t.to(dev)
        if fp8:
            return t.view(torch.float8_e4m3fn)
        return t.view(torch.bfloat16) if w.dtype == "bf16" else t

    q, k, v = up(x.q), up(x.k), up(x.v)
    mask = None
    if args.mask == "pad":
        if w.dtype == "fp8":
            raise SystemExit("bench.py: the FP8 path takes no mask")
        mask = torch.zeros((w.B, 1, 1, w.Nkv), dtype=torch.bool, device=dev)
        mask[..., : w.Nkv - w.Nkv // 8] = True
    out = torch.empty((w.B, w.Hq, w.Nq, w.Dv), dtype=torch.bfloat16 if fp8 else q.dtype,
                      device=dev)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    dcode = ATTN_F16 if w.dtype == "f16" else ATTN_BF16
    # the FP8 path plans on the 256-row tiles; the count shown is the 16-bit path's
    splits = args.splits or (None if fp8 else attn_fwd_num_splits(
        w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, w.causal, dcode))
    progress(f"inputs on {torch.cuda.get_device_name(dev)}; split-KV count {splits}; "
             f"warmup {args.warmup}")

    def fwd_step():
        if fp8:
            attn_fwd_fp8(q, k, v, x.q_descale, x.k_descale, x.v_descale, causal=w.causal,
                         scale=w.scale, out=out, lse=lse, num_splits=args.splits)
        else:
            attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=out, lse=lse,
                     num_splits=args.splits, mask=mask)

    graph = None
    if args.graph:
        if bwd or fp8 or mask is not None or args.pass_ != "fwd":
            raise SystemExit("bench.py: --graph covers the 16-bit forward without a mask")
        # warm the library (device query, scratch address) outside the capture
        attn_fwd_noalloc(q, k, v, out, lse, causal=w.causal, scale=w.scale,
                         num_splits=args.splits)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            attn_fwd_noalloc(q, k, v, out, lse, causal=w.causal, scale=w.scale,
                             num_splits=args.splits)
        torch.cuda.synchronize()

    if bwd:
        dout = inputs.make_dout(x, seed=args.seed)
        g = up(dout)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fwd_step()

        def step():
            attn_bwd(q, k, v, out, lse, g, causal=w.causal, scale=w.scale,
                     dq=dq, dk=dk, dv=dv, mask=mask)
    elif graph is not None:
        step = graph.replay
    else:
        step = fwd_step

    stream = torch.cuda.current_stream(dev)
    # peak memory of the timed steps: torch's allocator (the outputs are
    # allocated before timing, so nothing is expected there) and the pool
    # that serves the library's stream-ordered workspace
    pool = StreamOrderedPeak(dev.index or 0)
    # one event between consecutive steps: the whole region gives the mean,
    # the gaps give per-step median and minimum.  Everything the host does
    # before timing happens before the warm-up, so the device idles as
    # little as possible between the warm-up and the first timed step.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    progress(f"warm-up {args.warmup} steps, then timing {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    torch_before = torch.cuda.memory_allocated(dev)
    pool.reset()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    torch_delta = torch.cuda.max_memory_allocated(dev) - torch_before
    pool_peak = pool.read()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    flops = w.bwd_flops if bwd else w.flops
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[w.dtype]
    progress(f"{ms:.4f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of peak); "
             f"wall {wall:.3f} s")

    kernels = "fp8" if fp8 else args.pass_
    traffic = measured_traffic(name, args.pass_, kernels)
    if w.bound == "hbm" and not bwd:
        # below the ridge (decode): algorithmic bytes against HBM bandwidth
        gbs = w.hbm_bytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": w.hbm_bytes}
    else:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                    "traffic": traffic}

    # memory: what the step needs beyond its inputs and preallocated outputs
    # is the plan's workspace (split partials; the gradients' Delta rows),
    # never anything of size Nq x Nkv
    esz = 1 if fp8 else 2
    out_bytes = (w.B * w.Hq * w.Nq * w.Dv * 2 + w.B * w.Hq * w.Nq * 4)
    in_bytes = esz * (w.B * w.Hq * w.Nq * w.D + w.B * w.Hkv * w.Nkv * (w.D + w.Dv))
    if bwd:
        ws_plan = None   # Delta rows, plus fp32 dK/dV partials when heads are split
    else:
        ws_plan = attn_fwd_plan(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv,
                                192 if w.Dv != w.D else w.D, w.causal, dcode,
                                args.splits).workspace_bytes
    score_bytes = 4.0 * w.B * w.Hq * w.Nq * w.Nkv
    memory = {"inputs_bytes": in_bytes, "outputs_bytes": out_bytes,
              "plan_workspace_bytes": None if ws_plan is None else int(ws_plan),
              "peak_torch_delta_bytes": int(torch_delta),
              "peak_stream_ordered_bytes": pool_peak,
              "score_matrix_fp32_bytes": score_bytes}
    if pool_peak is not None and not fp8 and not bwd:
        # the library allocates nothing but its workspace (2 MiB pool granularity)
        memory["within_workspace"] = bool(torch_delta == 0 and
                                          pool_peak <= ws_plan + (2 << 20))

    if bwd:
        metric = ("attention bwd (dQ, dK, dV) TFLOP/s and % of MI355X bf16 MFMA peak "
                  "(2.5x forward flops)")
    else:
        metric = ("attention fwd TFLOP/s and % of MI355X bf16 MFMA peak "
                  "(B=1,H=24,D=128,N=17K)")
    result = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms": {"mean": round(ms, 5), "median": round(per_step[len(per_step) // 2], 5),
                    "min": round(per_step[0], 5), "max": round(per_step[-1], 5)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{name}: {w.note}, {w.describe()}",
                   "pass": args.pass_,
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nkv": w.Nkv,
                   "D": w.D, "Dv": w.Dv, "causal": w.causal, "scale": w.scale, "seed": args.seed,
                   "k_offset_std": w.k_offset_std, "mask": args.mask,
                   "launch": "hip graph replay (attn_fwd_noalloc)" if graph is not None
                             else "eager",
                   "split_kv": None if bwd else splits,
                   "kernel_source": source_hash(kernels)},
        "roofline": roofline,
        "memory": memory,
    }

    if want_cpu:
        import oracle
        if bwd:
            cpu_leg_bwd(result, x, w, name, dout, dq, dk, dv, np, oracle)
        else:
            cpu_leg_fwd(result, x, w, name, out, lse, np, oracle)

    print(json.dumps(result), flush=True)


def cpu_leg_fwd(result, x, w, name, out, lse, np, oracle):
    """Parity of sampled output rows and the oracle's throughput on them:
    the oracle's streaming two-pass mode (attention_two_pass, key blocks of
    4096; it computes the scores twice, but throughput counts the
    algorithmic flops), with the time the whole workload would take at that
    rate, labelled as an extrapolation."""
    from tests.parity import gather_rows
    progress(f"oracle on {x.rows.shape[1]} rows x {w.Hq} heads")
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    l_gpu = lse.cpu().numpy().astype(np.float64)
    sc = oracle.scale_value(w.scale, w.D)
    G = w.Hq // w.Hkv
    c0 = time.perf_counter()
    o_ref = np.empty((w.B, w.Hq, x.rows.shape[1], w.Dv))
    l_ref = np.empty((w.B, w.Hq, x.rows.shape[1]))
    for b in range(w.B):
        for hk in range(w.Hkv):
            kh = oracle.decode(x.k[b:b + 1, hk:hk + 1], w.dtype) * x.k_descale
            vh = oracle.decode(x.v[b:b + 1, hk:hk + 1], w.dtype) * x.v_descale
            for g in range(G):
                h = hk * G + g
                qh = oracle.decode(x.q[b:b + 1, h:h + 1], w.dtype) * x.q_descale
                oh, lh = oracle.attention_two_pass(qh, kh, vh, sc, w.causal, rows=x.rows[h])
                o_ref[b, h], l_ref[b, h] = oh[0, 0], lh[0, 0]
    cpu_s = time.perf_counter() - c0
    rows = x.rows
    if w.causal:
        sample_flops = float(sum(2.0 * (w.D + w.Dv) * np.minimum(r + 1, w.Nkv).sum()
                                 for r in rows)) * w.B
    else:
        sample_flops = 2.0 * (w.D + w.Dv) * w.Nkv * rows.size * w.B
    o_s, l_s = gather_rows(o_gpu, rows), gather_rows(l_gpu, rows)
    err = np.abs(o_s - o_ref)
    if w.dtype == "fp8":   # the FP8 path's bound (tests/parity.py fp8_bounds)
        from tests.parity import fp8_bounds, half_ulp
        bd, mbd, lbd = fp8_bounds(x, w.scale, w.causal, rows=rows)
        hu = half_ulp(o_ref, "bf16")
        lerr = np.abs(l_s - l_ref)
        result["parity"] = {"rows_per_head": int(rows.shape[1]),
                            "max_abs_err": float(err.max()), "mean_abs_err": float(err.mean()),
                            "lse_max_abs_err": float(lerr.max()),
                            "tolerance": "fp8 bound (E4M3 probabilities, 8-bit score sums)",
                            "pass": bool(np.all(err <= bd + hu) and
                                         err.mean() <= float(np.mean(mbd + hu)) and
                                         np.all(lerr <= 1e-3 + lbd))}
        err = None
    if err is not None:
        result["parity"] = {"rows_per_head": int(rows.shape[1]),
                            "max_abs_err": float(err.max()),
                            "mean_abs_err": float(err.mean()),
                            "lse_max_abs_err": float(np.abs(l_s - l_ref).max()),
                            "pass": bool(err.max() <= 4e-3 and err.mean() <= 5e-4 and
                                         np.abs(l_s - l_ref).max() <= 1e-3)}
    result["cpu_baseline"] = {
        "value": round(sample_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
        "cores": blas_threads(), "kind": "oracle",
        "sample": f"{rows.shape[1]} query rows per head x {w.Hq} heads of {name} "
                  f"({sample_flops / 1e9:.1f} GFLOP algorithmic, {cpu_s:.1f} s, "
                  f"float64 numpy two-pass streaming oracle, {cpu_model()})",
        "extrapolated_full_workload_s": round(cpu_s * w.flops / sample_flops, 1)}
    progress(f"oracle {cpu_s:.1f} s; parity {result['parity']}")


def cpu_leg_bwd(result, x, w, name, dout, dq, dk, dv, np, oracle):
    """dQ of sampled query rows against the oracle, and the oracle's gradient
    throughput on them.  dQ of row i depends on row i's inputs and every key
    only, so the oracle runs on the sampled rows alone: every fourth row of
    the forward's sample (causal: the first rows, which keep their
    positions).  The sample's flops count the five products over those rows.
    Then dK and dV of every key of KV head 0 (batch 0), for which the oracle
    runs over all query rows of the G query heads that read it."""
    from tests.parity import gather_rows
    R = max(2, x.rows.shape[1] // 4)
    rows = (np.tile(np.arange(min(R, w.Nq)), (w.Hq, 1)) if w.causal else x.rows[:, ::4])
    progress(f"oracle gradients on {rows.shape[1]} rows x {w.Hq} heads")
    dq_gpu = gather_rows(dq.float().cpu().numpy().astype(np.float64), rows)
    sc = oracle.scale_value(w.scale, w.D)
    G = w.Hq // w.Hkv
    c0 = time.perf_counter()
    dq_ref = np.empty_like(dq_gpu)
    for b in range(w.B):
        for hk in range(w.Hkv):
            kh = oracle.decode(x.k[b:b + 1, hk:hk + 1], w.dtype)
            vh = oracle.decode(x.v[b:b + 1, hk:hk + 1], w.dtype)
            for gi in range(G):
                h = hk * G + gi
                qh = oracle.decode(x.q[b:b + 1, h:h + 1, rows[h]], w.dtype)
                gh = oracle.decode(dout[b:b + 1, h:h + 1, rows[h]], w.dtype)
                dqh, _, _ = oracle.attention_backward(qh, kh, vh, gh, sc, w.causal)
                dq_ref[b, h] = dqh[0, 0]
    cpu_s = time.perf_counter() - c0
    if w.causal:
        sample_flops = float(sum(2.0 * (3 * w.D + 2 * w.Dv) * np.minimum(r + 1, w.Nkv).sum()
                                 for r in rows)) * w.B
    else:
        sample_flops = 2.0 * (3 * w.D + 2 * w.Dv) * w.Nkv * rows.size * w.B
    err = np.abs(dq_gpu - dq_ref)
    rms = float(np.sqrt(np.mean(dq_ref ** 2)))
    u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -11
    parity = {"rows_per_head": int(rows.shape[1]), "tensor": "dq",
              "max_abs_err": float(err.max()),
              "mean_abs_err": float(err.mean()), "rms_ref": rms,
              "pass": bool(err.mean() <= 1.5 * u * rms)}
    # dK, dV of KV head 0: every key, the oracle over all rows of its group
    progress(f"oracle dK, dV of KV head 0 ({G} query heads x {w.Nq} rows)")
    c1 = time.perf_counter()
    _, dk_ref, dv_ref = oracle.attention_backward(
        oracle.decode(x.q[:1, :G], w.dtype), oracle.decode(x.k[:1, :1], w.dtype),
        oracle.decode(x.v[:1, :1], w.dtype), oracle.decode(dout[:1, :G], w.dtype),
        sc, w.causal)
    kv_s = time.perf_counter() - c1
    for tname, got_t, ref in (("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        got = got_t[:1, :1].float().cpu().numpy().astype(np.float64)
        e = np.abs(got - ref)
        r = float(np.sqrt(np.mean(ref ** 2)))
        parity[tname] = {"keys": int(w.Nkv), "max_abs_err": float(e.max()),
                         "mean_abs_err": float(e.mean()), "rms_ref": r,
                         "pass": bool(np.all(np.isfinite(got)) and e.mean() <= 1.5 * u * r)}
    parity["pass"] = bool(parity["pass"] and parity["dk"]["pass"] and parity["dv"]["pass"])
    parity["kv_head_oracle_s"] = round(kv_s, 2)
    result["parity"] = parity
    result["cpu_baseline"] = {
        "value": round(sample_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
        "cores": blas_threads(), "kind": "oracle",
        "sample": f"dQ of {rows.shape[1]} query rows per head x {w.Hq} heads of {name} "
                  f"({sample_flops / 1e9:.1f} GFLOP algorithmic, {cpu_s:.1f} s, "
                  f"float64 numpy, {cpu_model()})"}
    progress(f"oracle {cpu_s:.1f} s; parity {result['parity']}")



def bench_ffn(args, torch, np):
    """The chunked feed-forward block (FFN chunking): one ffn_chunked call per
    step over a 16-bit synthetic batch; roofline against the MFMA peak with
    the algorithmic flops of the two products (4 N Dm F); the CPU leg runs
    the float64 oracle on sampled rows."""
    from memory_efficient_tiled_amd import ffn_chunked, inputs
    name = args.workload or "dit-ffn-17160"
    w = inputs.FFN_WORKLOADS[name]
    dev = torch.device("cuda:0")
    progress(f"workload {name}: {w.describe()}; generating inputs")
    xi = inputs.make_ffn_inputs(w.N, w.Dm, w.F, w.dtype, seed=args.seed)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if w.dtype == "bf16"
                             else np.ascontiguousarray(a)).to(dev)
        return t.view(torch.bfloat16) if w.dtype == "bf16" else t

    x, w1, b1, w2, b2 = (up(a) for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2))
    y = torch.empty_like(x)
    chunk = w.chunk_rows if args.ffn_chunk is None else args.ffn_chunk
    ffn_chunked(x, w1, b1, w2, b2, chunk_rows=chunk, out=y, verify=True)

    def step():
        ffn_chunked(x, w1, b1, w2, b2, chunk_rows=chunk, out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    progress(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[w.dtype]
    result = {
        "metric": "chunked feed-forward block TFLOP/s and % of MI355X bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * tflops / peak, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{name}: {w.note}, {w.describe()}", "pass": "ffn",
                   "N": w.N, "Dm": w.Dm, "F": w.F, "chunk_rows": chunk,
                   "seed": args.seed, "kernel_source": source_hash("ffn")},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": measured_traffic(name, "ffn")},
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = np.unique(np.random.default_rng(args.seed).choice(w.N, 64, replace=False))
        dec = [oracle.decode(a, w.dtype) for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2)]
        progress(f"oracle on {rows.size} rows")
        c0 = time.perf_counter()
        ref = oracle.ffn(dec[0][rows], *dec[1:])
        cpu_s = time.perf_counter() - c0
        got = y.float().cpu().numpy().astype(np.float64)[rows]
        err = np.abs(got - ref)
        sample_flops = 4.0 * rows.size * w.Dm * w.F
        result["parity"] = {"rows": int(rows.size), "max_abs_err": float(err.max()),
                            "mean_abs_err": float(err.mean()),
                            "rms_ref": float(np.sqrt(np.mean(ref ** 2)))}
        result["cpu_baseline"] = {
            "value": round(sample_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{rows.size} rows of {name} ({sample_flops / 1e9:.1f} GFLOP, "
                      f"{cpu_s:.1f} s, float64 numpy, {cpu_model()})"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
