#!/usr/bin/env python3
"""Benchmark of the Hymba hybrid-head mixer on one MI355X.

One step = one prefill of the Hymba-1.5B-shaped sliding-window layer
(B=1, 2048 prompt rows + 128 meta rows, 25q/5kv x 64, window 1024, d_inner 3200,
d_state 16, bf16) through the library's C ABI: conv + selective scan, RoPE,
MFMA flash attention, fusion, plus the KV-cache and state hand-off outputs.
Inputs are seeded synthetic tensors already resident in HBM. Several input sets
are rotated so that back-to-back steps do not simply re-read the last step's
inputs from the 256 MB last-level cache.

Also reported, in the same JSON line: the decode step of 64 sequences over an
8192-row cache shared read-only by two layers (two mixer calls), per-kernel
durations from HIP events recorded between the library's launches, the
roofline of the dominant kernel, and the CPU oracle timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "hybrid-head mixer prefill tokens/s + decode µs/step; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
# VALU issue: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz lane-slots/s; a transcendental
# (v_exp_f32) issues at a quarter of the rate of an fma: four slots.
ALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
EXP_SLOTS = 4
SCAN_END_SLOTS_PER_ELEM = 3 + EXP_SLOTS   # mul(dt*A) + exp + mul(dt*u*B) + fma(h)
SCAN_OUT_SLOTS_PER_ELEM = 4 + EXP_SLOTS   # ... + fma(C.h)
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
KERNEL_SOURCES = ["common.hpp", "launch.hpp", "ssm_step.hpp", "mma.hpp", "ssm.hip", "ssd.hip", "attn.hip", "fuse.hip",
                  "api.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (plumbing for per-kernel timing)


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.all = []

    def array(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = ev.value
            self.all.append(ev.value)
        return arr

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(out.value)

    def close(self):
        for e in self.all:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.all = []


# ---------------------------------------------------------------------------
# algorithmic work of each kernel (each input read once, each output written once)


def visible_pairs(L, n_meta, window):
    total = 0
    for i in range(L):
        total += min(i + 1, n_meta + window) if window > 0 else i + 1
    return total


def prefill_work(cfg, chunk_rows):
    """Algorithmic work of each prefill kernel: every input read once, every
    output written once; ALU slots of the scan recurrence only."""
    es = 2 if cfg.act == "bf16" else 4
    B, L, D, N = cfg.batch, cfg.seq_rows, cfg.d_inner, cfg.d_state
    Hq, Hkv, hd, dv = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.head_dim_v
    rows = B * L
    nchunk = -(-L // chunk_rows)
    end_rows = B * (nchunk - 1) * chunk_rows           # every chunk but the last
    state = B * D * N * 4                                # one fp32 state set
    params = D * (N + 1 + 4) * 4                         # A, D, conv taps
    # end pass: x (with 3 rows of history per chunk), dt, B of its rows; end states + dt sums
    end_bytes = end_rows * (2 * D * es + N * es) + (nchunk - 1) * (state + B * D * 4) + params
    # carry chain: end states and dt sums in, carried-in states out
    carry_bytes = (nchunk - 1) * (state + B * D * 4) + nchunk * state + D * N * 4
    # output pass: x, dt, z, B, C, carried-in states; y, final state and conv history
    out_bytes = rows * (4 * D * es + 2 * N * es) + nchunk * state + state + B * D * 3 * es + params
    rope_bytes = rows * ((Hq + Hkv) * hd * es * 2 + Hkv * dv * es * 2)
    pairs = B * visible_pairs(L, cfg.n_meta, cfg.window)
    attn_flops = pairs * Hq * (2 * hd + 2 * dv)
    attn_bytes = rows * ((Hq + Hkv) * hd * es + Hkv * dv * es + D * es)
    fuse_bytes = rows * 3 * D * es + 2 * D * 4
    return {
        "ssm_chunk_end": {"bytes": end_bytes, "alu_slots": end_rows * D * N * SCAN_END_SLOTS_PER_ELEM},
        "ssm_chunk_carry": {"bytes": carry_bytes},
        "ssm_chunk_out": {"bytes": out_bytes, "alu_slots": rows * D * N * SCAN_OUT_SLOTS_PER_ELEM},
        "rope_prefill": {"bytes": rope_bytes},
        "attn_prefill": {"bytes": attn_bytes, "flops": attn_flops, "pairs": pairs},
        "fuse": {"bytes": fuse_bytes},
    }


def ssd_work(cfg):
    """Algorithmic work of the Mamba-2 form's three kernels (64-row chunks):
    every input read once, every output written once; the output pass's block
    products (the masked C B^T-weighted product and the entering-state term)
    as matrix-core flops, counted on each chunk's real rows."""
    es = 2 if cfg.act == "bf16" else 4
    B, L, D, N, H = cfg.batch, cfg.seq_rows, cfg.d_inner, cfg.d_state, cfg.ssm_heads
    P, Q = D // H, 64
    rows = B * L
    nchunk = -(-L // Q)
    state = B * D * N * 4
    params = (H + D * 5) * 4                              # A per head, D, conv taps
    in_rows = rows * (D * es + H * es)                    # x and dt
    state_bytes = in_rows + rows * N * es + nchunk * (state + B * D * 4) + params
    carry_bytes = nchunk * (state + B * D * 4) + (nchunk + 1) * state + H * 4
    out_bytes = in_rows + rows * (2 * D * es + 2 * N * es) + nchunk * state + state + B * D * 3 * es + params
    nr = [min(Q, L - k * Q) for k in range(nchunk)]
    flops = B * H * sum(2 * r * r * P + 2 * r * N * P for r in nr)
    return {"ssd_state": {"bytes": state_bytes}, "ssd_carry": {"bytes": carry_bytes},
            "ssd_out": {"bytes": out_bytes, "flops": flops}}


def decode_work(cfg):
    es = 2 if cfg.act == "bf16" else 4
    B, D, N = cfg.batch, cfg.d_inner, cfg.d_state
    Hq, Hkv, hd, dv = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.head_dim_v
    n_vis = min(cfg.cache_len + 1, cfg.n_meta + cfg.window) if cfg.window > 0 else cfg.cache_len + 1
    ssm_bytes = B * D * N * 4 * 2 + B * D * 3 * es * 2 + B * (3 * D + 2 * N) * es + B * D * es + D * (N + 5) * 4
    attn_bytes = B * Hkv * (n_vis - 1) * (hd + dv) * es + B * (Hq * hd + Hkv * (hd + dv)) * es
    comb_bytes = B * D * es * 3 + 2 * D * 4
    return {"ssm_decode": {"bytes": ssm_bytes}, "attn_decode": {"bytes": attn_bytes, "n_vis": n_vis},
            "decode_merge_fuse": {"bytes": comb_bytes},
            "total_bytes": ssm_bytes + attn_bytes + comb_bytes}


def kernel_report(name, avg_ms, work, act):
    t = avg_ms * 1e-3
    r = {"avg_us": round(avg_ms * 1e3, 2)}
    fr = {}
    if "bytes" in work:
        gbs = work["bytes"] / t / 1e9
        r["hbm_GBs"] = round(gbs, 1)
        fr["hbm"] = gbs / HBM_PEAK_GBS
    if "flops" in work:
        tf = work["flops"] / t / 1e12
        r["mfma_TFLOPs"] = round(tf, 1)
        fr["mfma"] = tf / MFMA_PEAK_TFLOPS[act]
    if "alu_slots" in work:
        ts = work["alu_slots"] / t / 1e12
        r["alu_Tslots"] = round(ts, 2)
        fr["alu"] = ts / ALU_PEAK_TSLOTS
    r["frac"] = {k: round(v, 4) for k, v in fr.items()}
    r["bound"] = max(fr, key=fr.get)
    return r


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_lm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# rocprofv3 kernel names -> the stage keys above (bf16 instances: the benchmark's dtype)
COUNTER_KERNELS = {
    "ssm_chunk_end": ("ssm_chunk_kernel<hymba::bf16, false>",),
    "ssm_chunk_carry": ("ssm_chunk_carry_kernel",),
    "ssm_chunk_out": ("ssm_chunk_kernel<hymba::bf16, true>",),
    "rope_prefill": ("rope_prefill_kernel<hymba::bf16>",),
    "attn_prefill": ("attn_prefill_kernel<hymba::bf16",),
    "fuse": ("fuse_rows_kernel<hymba::bf16",),
}


def summarize_counters(fetch_csv, write_csv, calib_mib, command):
    """HBM bytes per launch of each prefill kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each divided by what the
    same counter reads per KiB for the plain device copy of calib_mib MiB that
    the same command ran (the largest copy dispatch)."""
    import csv

    def per_kernel(path, counter):
        vals, copies = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name or "direct_copy" in name:
                copies.append(v)
            for key, pats in COUNTER_KERNELS.items():
                if any(p in name for p in pats):
                    vals.setdefault(key, []).append(v)
        return vals, copies

    fetch, fcopies = per_kernel(fetch_csv, "FETCH_SIZE")
    write, wcopies = per_kernel(write_csv, "WRITE_SIZE")
    true_kib = calib_mib * 1024.0
    ffac = max(fcopies) / true_kib
    wfac = max(wcopies) / true_kib
    kernels = {}
    for key in COUNTER_KERNELS:
        if key not in fetch or key not in write:
            continue
        f = sum(fetch[key]) / len(fetch[key])
        w = sum(write[key]) / len(write[key])
        kernels[key] = {"fetch_KiB": round(f, 1), "write_KiB": round(w, 1), "dispatches": len(fetch[key]),
                        "hbm_bytes_per_launch": int(round((f / ffac + w / wfac) * 1024))}
    return {"source_hash": source_hash(), "command": command,
            "calibration": {"copy_MiB": calib_mib, "fetch_KiB_per_true_KiB": round(ffac, 4),
                            "write_KiB_per_true_KiB": round(wfac, 4)},
            "kernels": kernels}


# ---------------------------------------------------------------------------


def bench_prefill(cfg, steps, warmup, n_sets, ev, serial=False):
    import torch
    import synth
    from harness import Prefill
    import attention_lm_amd as H

    log(f"[bench] prefill {cfg.name}: generating inputs")
    inp = synth.make_prefill_inputs(cfg)
    runs = [Prefill(cfg, inp, with_outputs=False, with_cache=True) for _ in range(n_sets)]
    for r in runs:   # hand-off outputs a real prefill writes: final SSM/conv state (KV cache is on)
        r.o["ssm_state_out"] = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda")
        r.o["conv_state_out"] = torch.empty((cfg.batch, cfg.d_inner, cfg.d_conv - 1), dtype=r.out.dtype, device="cuda")
    nst = len(H._lib.PREFILL_STAGES)

    def step(r, events=None):
        t = r.t
        H.hymba_mixer_prefill(r.desc, r.params, t["x"], t["z"], t["dt"], t["B"], t["C"], t["q"], t["k"], t["v"],
                              r.out, workspace=r.ws, stage_events=events, **r.o)

    log(f"[bench] prefill warmup {warmup}")
    wev = ev.array(2 * nst) if serial else None
    for i in range(warmup):
        step(runs[i % n_sets], wev)
    torch.cuda.synchronize()
    log(f"[bench] prefill timed {steps} steps")
    tev = [ev.array(2 * nst) for _ in range(steps)] if serial else [None] * steps
    t0 = time.perf_counter()
    for i in range(steps):
        step(runs[i % n_sets], tev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel durations: the same steps with stage events (stages serialized;
    # each kernel's dispatch records its own start and end)
    evs = [ev.array(2 * nst) for _ in range(steps)]
    for i in range(steps):
        step(runs[i % n_sets], evs[i])
    torch.cuda.synchronize()
    stage_ms = {name: sum(ev.ms(e[2 * j], e[2 * j + 1]) for e in evs) / steps
                for j, name in enumerate(H._lib.PREFILL_STAGES)}
    serial_ms = sum(ev.ms(e[0], e[2 * nst - 1]) for e in evs) / steps
    return wall / steps * 1e3, stage_ms, serial_ms


def bench_decode(cfg, steps, warmup, n_sets, ev):
    import torch
    import synth
    from harness import Decode
    import attention_lm_amd as H

    log(f"[bench] decode {cfg.name}: generating inputs")
    inp = synth.make_decode_inputs(cfg)
    runs = []
    for s in range(n_sets):
        runs.append(Decode(cfg, inp))
        log(f"[bench] decode set {s} on device")
    nst = len(H._lib.DECODE_STAGES)

    def step(r, events=None):
        for l in range(cfg.n_layers):
            L = r.layers[l]
            H.hymba_mixer_decode(r.desc, L["params"], L["x"], L["z"], L["dt"], L["B"], L["C"], L["q"], r.k_new,
                                 r.v_new, r.k_cache, r.v_cache, r.cache_len, L["ssm_state"], L["conv_state"],
                                 L["out"], workspace=r.ws, stage_events=None if events is None else events[l])

    for i in range(warmup):
        step(runs[i % n_sets])
    torch.cuda.synchronize()
    # the step as a caller runs it (no stage events: SSM step and attention concurrent)
    t0 = time.perf_counter()
    for i in range(steps):
        step(runs[i % n_sets])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call and per-stage durations: the same steps with stage events (stages
    # serialized; each kernel's dispatch records its own start and end)
    evs = [[ev.array(2 * nst) for _ in range(cfg.n_layers)] for _ in range(steps)]
    for i in range(steps):
        step(runs[i % n_sets], evs[i])
    torch.cuda.synchronize()
    per_layer_ms = [sum(ev.ms(evs[i][l][0], evs[i][l][2 * nst - 1]) for i in range(steps)) / steps
                    for l in range(cfg.n_layers)]
    stage_ms = {}
    for j, name in enumerate(H._lib.DECODE_STAGES):
        stage_ms[name] = [sum(ev.ms(evs[i][l][2 * j], evs[i][l][2 * j + 1]) for i in range(steps)) / steps
                          for l in range(cfg.n_layers)]
    return wall / steps * 1e3, per_layer_ms, stage_ms


def bench_continue(cfg, steps, warmup, ring, n_sets=3):
    """A prefill continued from its state: rows [M + W, L) of ``cfg`` after a
    first call over [0, M + W) (the chunk sees a full window of history), with
    the cache one row per position or the compact ring. Times the
    continuation call (inputs resident; state and cache are updated in place,
    so every call does the same work). Several sets (state, cache, inputs) are
    rotated, as in the prefill step, so that a call does not re-read the last
    call's data from the last-level cache."""
    import torch
    from harness import TORCH_DT, desc_for, dev
    import attention_lm_amd as H
    import synth

    per_row = ("x", "z", "dt", "B", "C", "q", "k", "v")
    M, W, L = cfg.n_meta, cfg.window, cfg.seq_rows
    a = M + W
    T = L - a
    act, dt_ = cfg.act, TORCH_DT[cfg.act]
    inp = synth.make_prefill_inputs(cfg)
    cap = M + W if ring else L
    par = {k: dev(inp[k]) for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")}
    params = H.make_params(par["A"], par["D"], par["conv_w"], par["beta_attn"], par["beta_ssm"])
    Hkv, D = cfg.n_kv_heads, cfg.d_inner
    d0 = desc_for(cfg.with_(n_tokens=a - M), cache_capacity=cap, cache_ring=ring)
    desc = desc_for(cfg.with_(n_tokens=T), cache_capacity=cap, cache_ring=ring)
    sets = []
    for _ in range(n_sets):
        kc = torch.zeros((cfg.batch, cap, Hkv, cfg.head_dim), dtype=dt_, device="cuda")
        vc = torch.zeros((cfg.batch, cap, Hkv, cfg.head_dim_v), dtype=dt_, device="cuda")
        state = torch.empty((cfg.batch, D, cfg.d_state), dtype=torch.float32, device="cuda")
        conv = torch.empty((cfg.batch, D, cfg.d_conv - 1), dtype=dt_, device="cuda")
        first = {k: dev(inp[k][:, :a], act) for k in per_row}
        out0 = torch.empty((cfg.batch, a, D), dtype=dt_, device="cuda")
        H.hymba_mixer_prefill(d0, params, *[first[k] for k in per_row], out0, ssm_state_out=state,
                              conv_state_out=conv, k_cache=kc, v_cache=vc)
        rest = {k: dev(inp[k][:, a:], act) for k in per_row}
        out = torch.empty((cfg.batch, T, D), dtype=dt_, device="cuda")
        ws = torch.empty(max(H.hymba_mixer_prefill_workspace_bytes(desc), 256), dtype=torch.uint8, device="cuda")
        sets.append((rest, out, state, conv, kc, vc, ws))

    def step(st):
        rest, out, state, conv, kc, vc, ws = st
        H.hymba_mixer_prefill_continue(desc, params, a, *[rest[k] for k in per_row], out, state, conv, kc, vc,
                                       workspace=ws)

    for i in range(warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    return {"us_per_call": round(us, 2), "tokens_per_s": round(cfg.batch * T / (us * 1e-6), 1),
            "cache_rows_per_seq": cap}


def bench_decode_ring(cfg, steps, warmup, n_sets=3):
    """The decode step over the compact cache: n_meta + window rows per
    sequence instead of cache_len, every sequence at position cache_len."""
    import torch
    from harness import Decode, desc_for
    import attention_lm_amd as H
    import synth

    cap = cfg.n_meta + cfg.window
    rcfg = cfg.with_(cache_capacity=cap, cache_len=cap)
    inp = synth.make_decode_inputs(rcfg)
    runs = []
    for _ in range(n_sets):   # rotated like the long-cache step, so no set stays in the last-level cache
        run = Decode(rcfg, inp)
        run.cache_len.fill_(cfg.cache_len)
        run.desc = desc_for(rcfg, cache_ring=True)
        run.ws = torch.empty(max(H.hymba_mixer_decode_workspace_bytes(run.desc), 256), dtype=torch.uint8,
                             device="cuda")
        runs.append(run)

    def step(run):
        for l in range(rcfg.n_layers):
            run.call(l, with_branches=False)

    for i in range(warmup):
        step(runs[i % n_sets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(runs[i % n_sets])
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    return {"us_per_step": round(us, 2), "cache_rows_per_seq": cap, "position": cfg.cache_len}


def cpu_baseline(cfg, min_seconds=10.0):
    import numpy as np
    import synth
    import oracle as O
    from threadpoolctl import threadpool_limits

    cores = min(16, len(os.sched_getaffinity(0)))
    inp = synth.make_prefill_inputs(cfg)
    reps = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while True:
            O.mixer_prefill(cfg, inp)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
    return {
        "value": round(cfg.batch * cfg.n_tokens * reps / el, 1),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{reps} full float64 oracle prefill(s) of the same workload ({cfg.batch}x{cfg.seq_rows} rows, "
                   f"all rows, attention and scan) in {el:.1f} s; BLAS threads={cores}, element-wise NumPy and the "
                   f"scan's time loop single-threaded; cpu={_cpu_model()}"),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated through the timed steps")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ssd", action="store_true", help="skip the prefill with the Mamba-2 form of the scan")
    ap.add_argument("--no-continue", action="store_true",
                    help="skip the continued prefill and the compact-cache decode")
    ap.add_argument("--serial", action="store_true",
                    help="time the prefill steps with the branches serialized (per-kernel events in every "
                         "step, as in the per-kernel pass): for profiles whose kernel averages must match")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="also run a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print per-kernel HBM bytes from two rocprofv3 --pmc counter CSVs (FETCH_SIZE, "
                         "WRITE_SIZE) of a run with --copy-calibration, and exit")
    ap.add_argument("--counter-command", default="", help="the command that produced the counter CSVs (recorded)")
    args = ap.parse_args()
    if args.summarize_counters:
        if not args.copy_calibration:
            ap.error("--summarize-counters needs the --copy-calibration size the counted run used")
        print(json.dumps(summarize_counters(*args.summarize_counters, args.copy_calibration, args.counter_command),
                         indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_lm_amd as H

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    H.load_library()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x3 for counter calibration")
        del src, dst
    ev = HipEvents()
    cfg = synth.config("swa_layer")
    ms, stage_ms, serial_ms = bench_prefill(cfg, args.steps, args.warmup, args.sets, ev, serial=args.serial)
    chunk_rows = H.hymba_mixer_prefill_chunk_rows(H.make_desc(
        batch=cfg.batch, n_meta=cfg.n_meta, n_tokens=cfg.n_tokens, d_inner=cfg.d_inner, n_q_heads=cfg.n_q_heads,
        n_kv_heads=cfg.n_kv_heads, window=cfg.window, act=cfg.act))
    work = prefill_work(cfg, chunk_rows)
    kernels = {k: kernel_report(k, stage_ms[k], work[k], cfg.act) for k in stage_ms}
    dom = max(stage_ms, key=stage_ms.get)
    kd = kernels[dom]
    bound = kd["bound"]
    if bound == "hbm":
        ach, peak, unit = kd["hbm_GBs"], HBM_PEAK_GBS, "GB/s"
    elif bound == "mfma":
        ach, peak, unit = kd["mfma_TFLOPs"], MFMA_PEAK_TFLOPS[cfg.act], "TFLOP/s"
    else:
        ach, peak, unit = kd["alu_Tslots"], round(ALU_PEAK_TSLOTS, 2), "Tslot/s"
    traffic = traffic_for(dom)
    roofline = {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic,
                "hbm_frac": kd["frac"].get("hbm")}

    res = {
        "metric": METRIC,
        "value": round(cfg.batch * cfg.n_tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic",
        "config": {"workload": cfg.workload, "batch": cfg.batch, "n_tokens": cfg.n_tokens, "n_meta": cfg.n_meta,
                   "d_inner": cfg.d_inner, "d_state": cfg.d_state, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "head_dim_v": cfg.head_dim_v,
                   "window": cfg.window, "input_sets": args.sets},
        "rows_per_s_incl_meta": round(cfg.batch * cfg.seq_rows / (ms * 1e-3), 1),
        "prefill_branches": "serialized" if args.serial else "concurrent",
        "serial_ms_per_step": round(serial_ms, 4),
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_decode:
        dcfg = synth.config("decode")
        dms, per_layer, dstage = bench_decode(dcfg, args.steps, args.warmup, 3, ev)
        dw = decode_work(dcfg)
        dk = {k: kernel_report(k, sum(v) / len(v), dw[k], dcfg.act) for k, v in dstage.items()}
        call_us = dms * 1e3 / dcfg.n_layers   # per call, as a caller runs them (branches concurrent)
        res["decode"] = {
            "workload": dcfg.workload,
            "us_per_step": round(dms * 1e3, 2),
            "layers_per_step": dcfg.n_layers,
            "branches": "one stream (SSM step, attention, epilogue in order)",
            "us_per_call_serialized": [round(x * 1e3, 2) for x in per_layer],
            "hbm_GBs_per_call": round(dw["total_bytes"] / (call_us * 1e-6) / 1e9, 1),
            "hbm_frac_per_call": round(dw["total_bytes"] / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_call": dw["total_bytes"],
            "kernels": dk,
        }
    if not args.no_ssd:
        scfg = cfg.with_(ssm_heads=50, name="swa_layer_ssd")
        log("[bench] prefill with the Mamba-2 form of the scan")
        sms, sstage, sserial = bench_prefill(scfg, args.steps, args.warmup, args.sets, ev)
        sw = ssd_work(scfg)
        names = {"ssm_chunk_end": "ssd_state", "ssm_chunk_carry": "ssd_carry", "ssm_chunk_out": "ssd_out"}
        sk = {}
        for k, v in sstage.items():
            n = names.get(k, k)
            sk[n] = kernel_report(n, v, sw[n] if n in sw else work[k], scfg.act)
        res["ssd"] = {
            "workload": f"{cfg.workload}, Mamba branch in the Mamba-2 form: 50 heads of 64 channels, "
                        f"one decay rate and step size per head",
            "tokens_per_s": round(scfg.batch * scfg.n_tokens / (sms * 1e-3), 1),
            "ms_per_step": round(sms, 4),
            "serial_ms_per_step": round(sserial, 4),
            "kernels": sk,
        }
    if not args.no_continue:
        log("[bench] prefill continuation")
        res["continue"] = {
            "workload": f"{cfg.workload}: rows {cfg.n_meta + cfg.window}..{cfg.seq_rows - 1} continuing a first "
                        f"call over rows 0..{cfg.n_meta + cfg.window - 1} (a full window of history)",
            "rows": bench_continue(cfg, args.steps, args.warmup, ring=False),
            "ring": bench_continue(cfg, args.steps, args.warmup, ring=True),
        }
        if not args.no_decode:
            log("[bench] decode over the compact cache")
            res["decode"]["ring"] = bench_decode_ring(synth.config("decode"), args.steps, args.warmup)
    ev.close()
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
