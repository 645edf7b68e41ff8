#!/usr/bin/env python3
"""Benchmark of the Hymba hybrid-head mixer on one MI355X.

Headline step = one prefill of the batched workload (B=16 sequences of 4096
prompt rows + 128 meta rows, 25q/5kv x 64, dv 128, window 1024, d_inner 3200,
d_state 16, dt = softplus(N(-3, 2)), bf16) through the library's C ABI: conv +
selective scan + gate, RoPE, MFMA flash attention, fusion, plus the KV-cache
and state hand-off outputs. It is the largest single-GPU workload; inputs are
seeded synthetic tensors already resident in HBM.

Also reported in the same JSON line, each timed the same way: the global
layer (B=1, 8192 + 128 rows, full causal attention), the sliding-window layer
(B=1, 2048 + 128 rows), the decode step of 64 sequences over an 8192-row cache
shared read-only by two layers (plain, and with the second layer's key
affine), per-kernel durations of every workload, the roofline of the headline's
dominant kernel, and the float64 CPU oracle timed on this host on a bounded
sample of the headline workload.

Timing: before every timed iteration a 512 MiB scratch buffer is written and
then read, outside the timed region, so the 256 MB last-level cache (MALL)
holds none of the step's data and no dirty lines of the flush; each iteration
is bracketed by HIP events on the stream the library runs on. 10 warm-up
iterations, then 50 timed; median with p10/p90. Per-kernel durations come from
a second pass in which every kernel's dispatch records its own start and end
events (branches serialized).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
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
FLUSH_BYTES = 512 << 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["common.hpp", "launch.hpp", "ssm_step.hpp", "mma.hpp", "ssm.hip", "ssd.hip", "attn.hip", "fuse.hip",
                  "api.hip"]
PREFILL_WORKLOADS = {"c3": "batched_prefill", "c2": "global_layer", "c1": "swa_layer"}
ALL_LEGS = ["c3", "c2", "c1", "decode", "decode_affine", "ssd", "ssd_batched", "continue"]


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


class Flush:
    """Evicts the last-level cache between timed iterations: a 512 MiB buffer
    is written (fill) and then read (a reduction), twice the 256 MB MALL, on
    the current stream. The read leaves the cache holding clean flush lines, so
    no write-back of the flush lands inside the next timed region."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.empty((), dtype=torch.int64, device="cuda")
        self.i = 0

    def __call__(self):
        import torch
        self.i += 1
        self.buf.fill_(self.i)
        torch.sum(self.buf, dim=0, dtype=torch.int64, out=self.sink)


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def timed(step, flush, steps, warmup):
    """warmup + steps iterations, each preceded by a cache flush outside the
    timed region and bracketed by events on the current stream. Returns
    per-iteration milliseconds and the wall time of the timed loop."""
    import torch
    for _ in range(warmup):
        flush()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def stats(ms):
    return {"median": round(pct(ms, 50), 4), "p10": round(pct(ms, 10), 4), "p90": round(pct(ms, 90), 4),
            "mean": round(sum(ms) / len(ms), 4)}


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
    if t <= 0:
        return r
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
    if fr:
        r["bound"] = max(fr, key=fr.get)
    return r


def _code_only(text):
    """A kernel source without its comments, trailing blanks and empty lines
    (the sources hold no string literal with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash():
    """Hash of the kernel sources' code (comments excluded): the counter
    summaries under profiles/ are valid while it is unchanged."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_lm_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counters_path(workload):
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.json")


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload, if it was taken on the current kernel sources; else None."""
    try:
        with open(counters_path(workload)) as f:
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
    "ssm_chunk_out": ("ssm_chunk_kernel<hymba::bf16, true>", "ssm_scan1_kernel<hymba::bf16>"),
    "rope_prefill": ("rope_prefill_kernel<hymba::bf16>",),
    "attn_prefill": ("attn_prefill_kernel<hymba::bf16",),
    "fuse": ("fuse_rows_kernel<hymba::bf16", "fuse_rows_stream_kernel<hymba::bf16"),
    "ssm_decode": ("ssm_decode_kernel<hymba::bf16>",),
    "ssm_attn_decode": ("attn_decode_wave_kernel",),
    "decode_merge_fuse": ("decode_combine_kernel<hymba::bf16",),
    "ssd_state": ("ssd_state_kernel",),
    "ssd_out": ("ssd_out_kernel",),
}


def summarize_counters(fetch_csv, write_csv, calib_mib, command):
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each divided by what the
    same counter reads per KiB for the plain device copy of calib_mib MiB that
    the same command ran (the largest runtime copy dispatch). On gfx950 the
    memory side serves reads as 128-byte requests, which FETCH_SIZE counts as
    64 bytes: the copy reads 0.5 KiB per true KiB, and every kernel's reads are
    scaled by that factor."""
    import csv

    def per_kernel(path, counter):
        vals, copies = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "__amd_rocclr_copyBuffer" in name:   # the runtime's device copy (hipMemcpy blit)
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


COMPUTE_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_TRANS_F32",
                    "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES",
                    "GRBM_GUI_ACTIVE"]
N_SIMD = 256 * 4
N_XCD = 8


def summarize_compute(csv_path, command):
    """Per-kernel compute counters from one rocprofv3 --pmc pass over
    COMPUTE_COUNTERS (values summed over the chip per dispatch; the GPU-active
    cycle count is summed over the 8 XCDs, so it is divided by 8): MFMA busy
    fraction of the SIMDs' cycles, cycles in which MFMA and other VALU work
    ran together, and instructions per launch (transcendental = v_exp_f32,
    v_rcp_f32 and the like)."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"]
        key = None
        for k, pats in COUNTER_KERNELS.items():
            if any(p in name for p in pats):
                key = k
        if key is None:
            continue
        d = per.setdefault(key, {}).setdefault(r.get("Dispatch_Id", r.get("Correlation_Id")), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for key, disp in per.items():
        rows = [v for v in disp.values() if all(c in v for c in COMPUTE_COUNTERS)]
        if not rows:
            continue
        avg = {c: sum(v[c] for v in rows) / len(rows) for c in COMPUTE_COUNTERS}
        cycles = avg["GRBM_GUI_ACTIVE"] / N_XCD   # reported summed over the XCDs
        act = cycles * N_SIMD
        out[key] = {
            "dispatches": len(rows),
            "gpu_active_cycles": round(cycles),
            "mfma_busy_frac": round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / act, 4) if act else None,
            "mfma_valu_coexec_frac": round(avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / act, 4) if act else None,
            "trans_f32_insts_per_launch": round(avg["SQ_INSTS_VALU_TRANS_F32"]),
            "valu_insts_per_launch": round(avg["SQ_INSTS_VALU"]),
            "mfma_insts_per_launch": round(avg["SQ_INSTS_MFMA"]),
            "salu_insts_per_launch": round(avg["SQ_INSTS_SALU"]),
            "wait_inst_any_frac_of_wave_cycles": round(avg["SQ_WAIT_INST_ANY"] / avg["SQ_WAVE_CYCLES"], 4)
            if avg["SQ_WAVE_CYCLES"] else None,
        }
    return {"source_hash": source_hash(), "command": command, "counters": COMPUTE_COUNTERS, "kernels": out}


def summarize_trace(stats_csv, title, command):
    """Markdown table of a rocprofv3 --kernel-trace --stats summary."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel trace: {title}", "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
             f"Kernel sources: {source_hash()} (bench.py source_hash).", "",
             "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        if len(name) > 90:
            name = name[:90]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


# ---------------------------------------------------------------------------


def bench_prefill(cfg, steps, warmup, ev, flush, stage_steps, serial=False):
    import torch
    import synth
    from harness import Prefill
    import attention_lm_amd as H

    log(f"[bench] prefill {cfg.name}: generating inputs")
    inp = synth.make_prefill_inputs(cfg)
    run = Prefill(cfg, inp, with_outputs=False, with_cache=True)
    del inp
    # hand-off outputs a real prefill writes: final SSM/conv state (the KV cache is on)
    run.o["ssm_state_out"] = torch.empty((cfg.batch, cfg.d_inner, cfg.d_state), dtype=torch.float32, device="cuda")
    run.o["conv_state_out"] = torch.empty((cfg.batch, cfg.d_inner, cfg.d_conv - 1), dtype=run.out.dtype,
                                          device="cuda")
    nst = len(H._lib.PREFILL_STAGES)

    def step(events=None):
        t = run.t
        H.hymba_mixer_prefill(run.desc, run.params, t["x"], t["z"], t["dt"], t["B"], t["C"], t["q"], t["k"],
                              t["v"], run.out, workspace=run.ws, stage_events=events, **run.o)

    sev = ev.array(2 * nst) if serial else None
    log(f"[bench] prefill {cfg.name}: {warmup} warm-up + {steps} timed iterations")
    ms, wall = timed(lambda: step(sev), flush, steps, warmup)
    # per-kernel durations: the same step with stage events (stages serialized;
    # each kernel's dispatch records its own start and end)
    evs = [ev.array(2 * nst) for _ in range(stage_steps)]
    for e in evs:
        flush()
        step(e)
    torch.cuda.synchronize()
    stage_ms = {name: [ev.ms(e[2 * j], e[2 * j + 1]) for e in evs] for j, name in enumerate(H._lib.PREFILL_STAGES)}
    serial_ms = [ev.ms(e[0], e[2 * nst - 1]) for e in evs]
    chunk_rows = H.hymba_mixer_prefill_chunk_rows(run.desc)
    del run
    torch.cuda.empty_cache()
    return ms, wall, stage_ms, serial_ms, chunk_rows


def prefill_leg(cfg, args, ev, flush, serial=False):
    ms, wall, stage_ms, serial_ms, chunk_rows = bench_prefill(cfg, args.steps, args.warmup, ev, flush,
                                                              args.stage_steps, serial)
    st = stats(ms)
    work = prefill_work(cfg, chunk_rows)
    kernels = {}
    for k, v in stage_ms.items():
        kernels[k] = kernel_report(k, sum(v) / len(v), work[k], cfg.act)
        kernels[k]["median_us"] = round(pct(v, 50) * 1e3, 2)
    leg = {
        "workload": cfg.workload,
        "tokens_per_s": round(cfg.batch * cfg.n_tokens / (st["median"] * 1e-3), 1),
        "rows_per_s_incl_meta": round(cfg.batch * cfg.seq_rows / (st["median"] * 1e-3), 1),
        "ms_per_step": st,
        "wall_ms_per_iteration_incl_flush": round(wall / len(ms) * 1e3, 4),
        "branches": "serialized" if serial else "concurrent",
        "serial_ms_per_step": stats(serial_ms),
        "scan_chunk_rows": chunk_rows,
        "work": {"bytes_whole_mixer": cfg.batch * cfg.seq_rows * _mixer_row_bytes(cfg),
                 "attn_flops": work["attn_prefill"]["flops"], "attn_pairs": work["attn_prefill"]["pairs"]},
        "kernels": kernels,
    }
    return leg


def _mixer_row_bytes(cfg):
    es = 2 if cfg.act == "bf16" else 4
    D, N = cfg.d_inner, cfg.d_state
    return (3 * D + 2 * N + (cfg.n_q_heads + cfg.n_kv_heads) * cfg.head_dim + cfg.n_kv_heads * cfg.head_dim_v
            + D) * es


def bench_decode(cfg, args, ev, flush):
    import torch
    import synth
    from harness import Decode
    import attention_lm_amd as H

    log(f"[bench] decode {cfg.name}: generating inputs")
    inp = synth.make_decode_inputs(cfg)
    run = Decode(cfg, inp)
    del inp
    nst = len(H._lib.DECODE_STAGES)

    def step(events=None):
        for l in range(cfg.n_layers):
            L = run.layers[l]
            H.hymba_mixer_decode(run.desc, L["params"], L["x"], L["z"], L["dt"], L["B"], L["C"], L["q"], run.k_new,
                                 run.v_new, run.k_cache, run.v_cache, run.cache_len, L["ssm_state"],
                                 L["conv_state"], L["out"], workspace=run.ws,
                                 stage_events=None if events is None else events[l])

    log(f"[bench] decode {cfg.name}: {args.warmup} warm-up + {args.steps} timed two-layer steps")
    ms, wall = timed(step, flush, args.steps, args.warmup)
    # per-call and per-stage durations: the same steps with stage events
    evs = [[ev.array(2 * nst) for _ in range(cfg.n_layers)] for _ in range(args.stage_steps)]
    for e in evs:
        flush()
        step(e)
    torch.cuda.synchronize()
    first = 2 if cfg.act == "bf16" else 0   # (bf16: the first stage is an empty event pair)
    per_layer = [[ev.ms(e[l][first], e[l][2 * nst - 1]) for e in evs] for l in range(cfg.n_layers)]
    stage_ms = {name: [[ev.ms(e[l][2 * j], e[l][2 * j + 1]) for e in evs] for l in range(cfg.n_layers)]
                for j, name in enumerate(H._lib.DECODE_STAGES)}
    del run
    torch.cuda.empty_cache()
    st = stats(ms)
    dw = decode_work(cfg)
    kernels = {}
    if cfg.act == "bf16":
        # the Mamba step runs inside the attention launch (workgroups of its
        # own); its stage records an empty event pair
        stage_ms = {"ssm_attn_decode": stage_ms["attn_decode"], "decode_merge_fuse": stage_ms["decode_merge_fuse"]}
        dw = dict(dw, ssm_attn_decode={"bytes": dw["ssm_decode"]["bytes"] + dw["attn_decode"]["bytes"]})
    for k, per in stage_ms.items():
        allv = [x for v in per for x in v]
        kernels[k] = kernel_report(k, sum(allv) / len(allv), dw[k], cfg.act)
        kernels[k]["per_layer_avg_us"] = [round(sum(v) / len(v) * 1e3, 2) for v in per]
    call_us = st["median"] * 1e3 / cfg.n_layers
    return {
        "workload": cfg.workload,
        "us_per_step": {k: round(v * 1e3, 2) for k, v in st.items()},
        "layers_per_step": cfg.n_layers,
        "us_per_call": round(call_us, 2),
        "us_per_call_serialized_stages": [round(sum(v) / len(v) * 1e3, 2) for v in per_layer],
        "bytes_per_call": dw["total_bytes"],
        "hbm_GBs_per_call": round(dw["total_bytes"] / (call_us * 1e-6) / 1e9, 1),
        "hbm_frac_per_call": round(dw["total_bytes"] / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "wall_us_per_iteration_incl_flush": round(wall / len(ms) * 1e6, 2),
        "kernels": kernels,
    }


def bench_continue(cfg, args, flush, ring):
    """A prefill continued from its state: rows [M + W, L) of ``cfg`` after a
    first call over [0, M + W) (the chunk sees a full window of history), with
    the cache one row per position or the compact ring. Times the continuation
    call (inputs resident; state and cache are updated in place, so every call
    does the same work)."""
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

    def step():
        H.hymba_mixer_prefill_continue(desc, params, a, *[rest[k] for k in per_row], out, state, conv, kc, vc,
                                       workspace=ws)

    ms, _ = timed(step, flush, args.steps, args.warmup)
    st = stats(ms)
    return {"us_per_call": {k: round(v * 1e3, 2) for k, v in st.items()},
            "tokens_per_s": round(cfg.batch * T / (st["median"] * 1e-3), 1), "cache_rows_per_seq": cap}


def bench_decode_ring(cfg, args, flush):
    """The decode step over the compact cache: n_meta + window rows per
    sequence instead of cache_len, every sequence at position cache_len."""
    from harness import Decode, desc_for
    import attention_lm_amd as H
    import torch
    import synth

    cap = cfg.n_meta + cfg.window
    rcfg = cfg.with_(cache_capacity=cap, cache_len=cap)
    inp = synth.make_decode_inputs(rcfg)
    run = Decode(rcfg, inp)
    run.cache_len.fill_(cfg.cache_len)
    run.desc = desc_for(rcfg, cache_ring=True)
    run.ws = torch.empty(max(H.hymba_mixer_decode_workspace_bytes(run.desc), 256), dtype=torch.uint8, device="cuda")

    def step():
        for l in range(rcfg.n_layers):
            run.call(l, with_branches=False)

    ms, _ = timed(step, flush, args.steps, args.warmup)
    st = stats(ms)
    return {"us_per_step": {k: round(v * 1e3, 2) for k, v in st.items()}, "cache_rows_per_seq": cap,
            "position": cfg.cache_len}


def cpu_baseline(cfg, min_seconds=12.0):
    """The float64 oracle on whole sequences of the workload (all rows: conv,
    scan, attention over every visible key, fusion), one sequence per repeat,
    until min_seconds have passed; prompt tokens per second."""
    import numpy as np
    import synth
    import oracle as O
    from threadpoolctl import threadpool_limits

    cores = min(16, len(os.sched_getaffinity(0)))
    one = cfg.with_(batch=1)   # each repeat: one sequence of the workload (its own seeded draws)
    reps = 0
    el = 0.0
    with threadpool_limits(limits=cores):
        while el < min_seconds:
            inp = synth.make_prefill_inputs(one.with_(seed=cfg.seed * 1000 + reps))
            t0 = time.perf_counter()
            O.mixer_prefill(one, inp)
            el += time.perf_counter() - t0
            reps += 1
    return {
        "value": round(one.n_tokens * reps / el, 1),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{reps} sequence(s) of the headline workload ({one.seq_rows} rows each: {one.n_meta} meta + "
                   f"{one.n_tokens} prompt, window {one.window}, d_inner {one.d_inner}, 25q/5kv), each a full "
                   f"float64 oracle prefill (all rows, scan and attention), {el:.1f} s of oracle time (input "
                   f"generation excluded); tokens/s = prompt rows / oracle time, the same unit as the GPU value; "
                   f"BLAS threads={cores}, element-wise NumPy and the scan's time loop single-threaded; "
                   f"cpu={_cpu_model()}"),
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
    ap.add_argument("--stage-steps", type=int, default=20, help="iterations of the per-kernel (evented) pass")
    ap.add_argument("--only", nargs="+", choices=ALL_LEGS, default=None,
                    help="run only these legs (c3 is the headline; without it no JSON headline is printed)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--serial", action="store_true",
                    help="time the prefill steps with the branches serialized (per-kernel events in every "
                         "step, as in the per-kernel pass): for profiles whose kernel averages must match")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="also run a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print per-kernel HBM bytes from two rocprofv3 --pmc counter CSVs (FETCH_SIZE, "
                         "WRITE_SIZE) of a run with --copy-calibration, and exit")
    ap.add_argument("--counter-command", default="", help="the command that produced the counter CSVs (recorded)")
    ap.add_argument("--summarize-compute", metavar="CSV",
                    help="print per-kernel compute counters (MFMA busy, transcendental and VALU instructions) from "
                         "one rocprofv3 --pmc pass over the COMPUTE_COUNTERS list, and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "TITLE"),
                    help="print a markdown table of a rocprofv3 --kernel-trace --stats summary, and exit")
    args = ap.parse_args()
    if args.summarize_compute:
        print(json.dumps(summarize_compute(args.summarize_compute, args.counter_command), indent=1))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.counter_command), end="")
        return
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
    legs = args.only or ALL_LEGS
    if args.copy_calibration:
        n = args.copy_calibration << 20
        # float32 elements: the copy moves 16-byte vectors per thread, the access
        # width of this library's kernels
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes x3 for counter calibration")
        del src, dst
    ev = HipEvents()
    flush = Flush()
    res = {}
    subs = {}
    for name in ("c3", "c2", "c1"):
        if name in legs:
            cfg = synth.config(PREFILL_WORKLOADS[name])
            subs[name] = (cfg, prefill_leg(cfg, args, ev, flush, serial=args.serial))
    if "decode" in legs:
        subs["decode"] = (synth.config("decode"), bench_decode(synth.config("decode"), args, ev, flush))
    if "decode_affine" in legs:
        subs["decode_affine"] = (synth.config("decode_affine"),
                                 bench_decode(synth.config("decode_affine"), args, ev, flush))
    for leg_name, base_name in (("ssd", "swa_layer"), ("ssd_batched", "batched_prefill")):
        if leg_name in legs:
            base = synth.config(base_name)
            scfg = base.with_(ssm_heads=50, name=f"{base_name}_ssd")
            leg = prefill_leg(scfg, args, ev, flush)
            sw = ssd_work(scfg)
            names = {"ssm_chunk_end": "ssd_state", "ssm_chunk_carry": "ssd_carry", "ssm_chunk_out": "ssd_out"}
            for k, n in names.items():
                kr = leg["kernels"].pop(k)
                leg["kernels"][n] = dict(kernel_report(n, kr["avg_us"] * 1e-3, sw[n], scfg.act),
                                         median_us=kr.get("median_us"))
            leg["workload"] = (f"{base.workload}, Mamba branch in the Mamba-2 form: 50 heads of 64 channels, one "
                               f"decay rate and step size per head")
            subs[leg_name] = (scfg, leg)
    if "continue" in legs:
        cfg = synth.config("swa_layer")
        log("[bench] prefill continuation")
        subs["continue"] = (cfg, {
            "workload": f"{cfg.workload}: rows {cfg.n_meta + cfg.window}..{cfg.seq_rows - 1} continuing a first "
                        f"call over rows 0..{cfg.n_meta + cfg.window - 1} (a full window of history)",
            "rows": bench_continue(cfg, args, flush, ring=False),
            "ring": bench_continue(cfg, args, flush, ring=True),
            "decode_ring": bench_decode_ring(synth.config("decode"), args, flush),
        })
    ev.close()

    if "c3" in subs:
        cfg, head = subs["c3"]
        kernels = head["kernels"]
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        kd = kernels[dom]
        bound = kd["bound"]
        if bound == "hbm":
            ach, peak, unit = kd["hbm_GBs"], HBM_PEAK_GBS, "GB/s"
        elif bound == "mfma":
            ach, peak, unit = kd["mfma_TFLOPs"], MFMA_PEAK_TFLOPS[cfg.act], "TFLOP/s"
        else:
            ach, peak, unit = kd["alu_Tslots"], round(ALU_PEAK_TSLOTS, 2), "Tslot/s"
        roofline = {"kernel": dom, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                    "frac": round(ach / peak, 4), "traffic": traffic_for(dom, cfg.name),
                    "hbm_frac": kd["frac"].get("hbm"), "avg_us": kd["avg_us"]}
        res = {
            "metric": METRIC,
            "value": head["tokens_per_s"],
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": head["ms_per_step"]["median"],
            "ms_per_step_p10": head["ms_per_step"]["p10"],
            "ms_per_step_p90": head["ms_per_step"]["p90"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": cfg.act,
            "data": "synthetic",
            "config": {"workload": cfg.workload, "batch": cfg.batch, "n_tokens": cfg.n_tokens,
                       "n_meta": cfg.n_meta, "d_inner": cfg.d_inner, "d_state": cfg.d_state,
                       "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                       "head_dim_v": cfg.head_dim_v, "window": cfg.window, "dt": "softplus(N(-3,2))"},
            "timing": "per iteration: 512 MiB cache flush (write + read) outside the timed region, HIP events "
                      "on the library's stream; median of the timed iterations (p10/p90 beside it)",
            "roofline": roofline,
            "headline": head,
        }
    else:
        res = {"metric": METRIC, "note": "headline leg (c3) not run"}
    for name in ("c2", "c1", "decode", "decode_affine", "ssd", "ssd_batched", "continue"):
        if name in subs:
            res[{"c2": "global_layer", "c1": "swa_layer"}.get(name, name)] = subs[name][1]
    if "c3" in subs and not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(subs["c3"][0])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
