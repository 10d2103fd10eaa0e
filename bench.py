#!/usr/bin/env python3
"""Throughput of the canvas denoise pass on one MI355X.

A step is one denoise pass of the whole hot path (embed, 30 decoder layers
with canvas attention + prompt-KV attention and the routed MoE, final norm,
tied LM head, argmax/confidence, lock-and-remask) over one batch of seeded
synthetic input: random-init bf16 weights (N(0, 0.02)), N(0, 1) prompt KV and
a uniformly drawn canvas.  Steps walk through the block's pass schedule
(steps_left = T, T-1, ..., 1) and restart it with a fresh canvas every T
passes, so every lock count of a block is exercised.

Prints one JSON line: canvas tokens/s per pass as ``value``, the resolved
tokens/s of whole blocks, the roofline of the dominant kernel (the grouped
gate|up expert GEMM, timed with HIP events on the library's stream) and the
CPU oracle's rate on a bounded sample of the same workload.  ``eb_sampler``
adds the entropy-bounded variant of the same workload: the pass time with
the sampler head (temperature, entropy, Gumbel-max sample) and the EB lock
step, and whole blocks that stop adaptively within 48 passes.  ``mxfp4_experts``
measures the same workload again with the expert matrices stored as MXFP4.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA

METRIC = "canvas tokens/sec per denoise pass; resolved tok/s (30-layer bf16, 1 MI355X)"

# HBM byte counters of the gate|up expert GEMM (rocprofv3 FETCH_SIZE / WRITE_SIZE
# runs, scaled by a plain copy of known size), valid for the kernel sources
# they were taken with
COUNTERS = os.path.join(ROOT, "profiles", "moe_gate_up_C3_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "canvas_denoising_moe_amd", "csrc", f) for f in ("gemm.hip", "common.h")]
GATE_UP_KERNEL = r"k_stream<unsigned short, \d+, \d+, 1, \d+, \d+, 0>"   # <T, MT, WN, EPI_GEGLU, R, LDS KB, bf16 W>
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib):
    """Per-launch HBM bytes of the gate|up GEMM from rocprofv3 counter runs
    (KiB per dispatch), each counter scaled by what it reads for a plain
    device copy of copy_mib MiB; written next to the other profiles."""
    import re
    import statistics
    known_kib = copy_mib * 1024.0

    def mean_kib(d, pattern, counter):
        v = [float(r["Counter_Value"]) for r in _counter_rows(d)
             if re.search(pattern, r["Kernel_Name"]) and r["Counter_Name"] == counter]
        if not v:
            raise SystemExit(f"no {counter} records of {pattern} under {d}")
        return statistics.fmean(v), len(v)

    cf, _ = mean_kib(copy_fetch_dir, re.escape(COPY_KERNEL), "FETCH_SIZE")
    cw, _ = mean_kib(copy_write_dir, re.escape(COPY_KERNEL), "WRITE_SIZE")
    f, nf = mean_kib(fetch_dir, GATE_UP_KERNEL, "FETCH_SIZE")
    w, nw = mean_kib(write_dir, GATE_UP_KERNEL, "WRITE_SIZE")
    out = {
        "kernel": "moe_grouped_gemm gate|up (k_stream, GeGLU epilogue), 30-layer 4096-prompt workload",
        "kernel_sources_sha256": kernel_sources_sha(),
        "copy_mib": copy_mib,
        "fetch_scale": known_kib / cf, "write_scale": known_kib / cw,
        "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w, "dispatches": [nf, nw],
        "fetch_bytes_per_launch": f * 1024.0 * known_kib / cf,
        "write_bytes_per_launch": w * 1024.0 * known_kib / cw,
    }
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(COUNTERS, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def measured_traffic():
    """HBM bytes per gate|up launch from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(COUNTERS) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    if c.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    return int(c["traffic_bytes_per_launch"])


def algorithmic(w, touched):
    """Algorithmic HBM bytes and flops of one pass and of one gate|up launch.

    ``touched[l]`` is the number of routed experts that received a token in
    layer l (weights of untouched experts need not be read)."""
    m = w.model
    M = w.batch * m.canvas_len
    H, D, F, E, K, V = m.hidden, m.head_dim, m.expert_ffn, m.n_experts, m.top_k, m.vocab
    qd, kvd = m.n_heads * D, m.n_kv_heads * D
    es = 2 if m.dtype == "bf16" else 4
    # expert matrices: MXFP4 stores 4 bits per weight plus one scale byte per 32
    ees = 0.5 + 1.0 / 32 if getattr(m, "expert_format", "native") == "mxfp4" else es
    byts = flops = 0.0
    gu_bytes = []
    for l in range(m.n_layers):
        Lw = m.kv_len(l, w.prompt_len)
        attn_w = (H * (qd + 2 * kvd) + qd * H + H * E) * es
        ex = (touched[l] + 1) * 3 * H * F * ees
        kv = w.batch * Lw * kvd * 2 * es
        norms = 4 * H * es
        byts += attn_w + ex + kv + norms
        gu_bytes.append((touched[l] + 1) * 2 * H * F * ees + M * H * es + (M * K + M) * F * es)
        flops += 2.0 * M * (H * (qd + 2 * kvd) + qd * H + H * E + (K + 1) * 3 * H * F)
        flops += 4.0 * M * m.n_heads * D * (Lw + m.canvas_len)
    if m.has_lm_head:
        byts += V * H * es + H * es + M * H * es
        flops += 2.0 * M * H * V
    gu_flops = 2.0 * (M * K + M) * H * 2 * F
    return byts, flops, sum(gu_bytes) / len(gu_bytes), gu_flops


def trace_touched(ctx, w, tokens, locked, tok0_d, lk0_d):
    """One whole block with the routing recorded: the number of routed experts
    that received a token, per pass of the block and per layer."""
    import numpy as np
    import torch
    m = w.model
    B, T = w.batch, w.n_steps
    M = B * m.canvas_len
    trace = torch.empty((m.n_layers, M, m.top_k), dtype=torch.int32, device=tokens.device)
    tokens.copy_(tok0_d)
    locked.copy_(lk0_d)
    ctx.set_trace(trace)
    out = []
    for t in range(T):
        ctx.denoise_step(tokens, locked, [T - t] * B)
        tr = trace.cpu().numpy()
        out.append([int(np.unique(tr[l]).size) for l in range(m.n_layers)])
    ctx.set_trace(None)
    return out


def pass_algorithmic(w, touched_by_pass, passes):
    """Mean algorithmic bytes and flops of the given passes of the block."""
    byts = flops = 0.0
    for s in passes:
        b, f, _, _ = algorithmic(w, touched_by_pass[s])
        byts += b
        flops += f
    return byts / len(passes), flops / len(passes)


def gate_up_bytes(w, touched_by_pass, passes):
    """Mean algorithmic bytes of one gate|up launch over every layer of the
    given passes."""
    return sum(algorithmic(w, touched_by_pass[s])[2] for s in passes) / len(passes)


def measure_workload(w, steps, warmup):
    """Pass time, resolved tokens of one block and the pass roofline of a
    second workload (its own context), plus its attention launches."""
    import numpy as np
    import torch

    import canvas_denoising_moe_amd as dg
    from canvas_denoising_moe_amd import binding as bd
    from synth import gen, upload

    m = w.model
    B, N, T = w.batch, m.canvas_len, w.n_steps
    M = B * N
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    ctx = dg.Context(m, max_batch=B, max_prompt_len=w.prompt_len, device=0)
    try:
        upload.load_context(ctx, w)
        torch.cuda.synchronize()
        load_s = time.perf_counter() - t0
        print(f"[bench] {w.name}: weights and prompt KV loaded in {load_s:.1f} s", file=sys.stderr, flush=True)
        tok0, lk0 = gen.canvas(w)
        tok0_d = torch.from_numpy(tok0).to(dev)
        lk0_d = torch.from_numpy(lk0).to(dev)
        tokens, locked = tok0_d.clone(), lk0_d.clone()
        touched_by_pass = trace_touched(ctx, w, tokens, locked, tok0_d, lk0_d)

        def step(i):
            s = i % T
            if s == 0:
                tokens.copy_(tok0_d)
                locked.copy_(lk0_d)
            ctx.denoise_step(tokens, locked, [T - s] * B)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        # attention launches (events add dispatch latency: outside the timed region)
        ctx.profile([bd.PROF_ATTN])
        for i in range(T):
            step(steps + i)
        torch.cuda.synchronize()
        ctx.profile(())
        n_at, ms_at = ctx.profile_read(bd.PROF_ATTN)
        tokens.copy_(tok0_d)
        locked.copy_(lk0_d)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.generate_block(tokens, locked, T)
        torch.cuda.synchronize()
        block_ms = (time.perf_counter() - t0) * 1e3
        assert bool(locked.all()), "block left unlocked positions"
    finally:
        ctx.close()
        torch.cuda.empty_cache()
    byts, flops = pass_algorithmic(w, touched_by_pass, [i % T for i in range(steps)])
    newly = int(M - lk0.sum())
    n_global = sum(1 for l in range(m.n_layers) if m.is_global(l))
    return {"workload": w.name, "batch": B, "prompt_len": w.prompt_len, "passes_per_block": T,
            "ms_per_step": round(ms, 4), "canvas_tok_s": round(M / (ms / 1e3), 1),
            "block_ms": round(block_ms, 3), "resolved_tok_s": round(newly / (block_ms / 1e3), 1),
            "pass_roofline": {"bytes": int(byts), "flops": int(flops),
                              "hbm_frac": round(byts / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                              "mfma_frac": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "attention_us_per_layer": round(ms_at / max(n_at, 1) * 1e3, 2),
            "attention_launches": n_at, "global_layers": n_global,
            "experts_touched_min": min(min(tp) for tp in touched_by_pass), "load_s": round(load_s, 1)}


def cpu_baseline(w):
    """The oracle (float64 numpy) timed on one whole denoise pass of the
    workload: every layer over every canvas position, the LM head, argmax and
    the lock step.  Weight generation and widening to float64 happen before
    each timed step and are not counted."""
    import numpy as np
    from oracle import model as om
    from oracle.inputs import prompt_kv_fn, weights_for
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    m = w.model
    M = w.batch * m.canvas_len
    W = weights_for(w)
    kvf = prompt_kv_fn(w)
    tok, lk = gen.canvas(w)
    rnd = om._rounder(m)
    t_total = 0.0
    t0 = time.perf_counter()
    x = W.embed_rows(tok.reshape(-1).astype(np.int64))
    t_total += time.perf_counter() - t0
    for l in range(m.n_layers):
        lw = {k: np.asarray(v) for k, v in W.layer(l).items()}  # widened outside the timing
        kv = [kvf(l, b) for b in range(w.batch)]
        t0 = time.perf_counter()
        x, _ = om.layer_forward(x, lw, m, l, kv, [w.prompt_len] * w.batch, rnd)
        t_total += time.perf_counter() - t0
        del lw, kv
    E = W.embed()
    t0 = time.perf_counter()
    h = rnd(om.rmsnorm(x, W.norm_final(), m.rms_eps))
    pred, conf = om.argmax_conf(om.lm_logits(h, E))
    om.lock_select(conf.reshape(w.batch, -1), pred.reshape(w.batch, -1), tok, lk, [w.n_steps] * w.batch)
    t_total += time.perf_counter() - t0
    sample = (f"oracle float64 on {cores} BLAS threads: one whole pass ({m.n_layers} layers, LM head, "
              f"argmax, lock) over all {M} canvas positions in {t_total:.1f} s")
    return {"value": M / t_total, "unit": "canvas tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample}


def measure_mxfp4(w0, steps, warmup):
    """The same workload with MXFP4 expert weights: pass time, the expert
    GEMMs' launch times and the gate|up roofline on its (4.25-bit) bytes."""
    import dataclasses

    import numpy as np
    import torch

    import canvas_denoising_moe_amd as dg
    from canvas_denoising_moe_amd import binding as bd
    from synth import gen, upload

    w = dataclasses.replace(w0, name=w0.name + "-mxfp4", model=dataclasses.replace(w0.model, expert_format="mxfp4"))
    m = w.model
    B, N, T = w.batch, m.canvas_len, w.n_steps
    M = B * N
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    ctx = dg.Context(m, max_batch=B, max_prompt_len=w.prompt_len, device=0)
    try:
        upload.load_context(ctx, w)
        torch.cuda.synchronize()
        load_s = time.perf_counter() - t0
        print(f"[bench] {w.name}: loaded and quantised in {load_s:.1f} s", file=sys.stderr, flush=True)
        tok0, lk0 = gen.canvas(w)
        tok0_d = torch.from_numpy(tok0).to(dev)
        lk0_d = torch.from_numpy(lk0).to(dev)
        tokens, locked = tok0_d.clone(), lk0_d.clone()
        touched_by_pass = trace_touched(ctx, w, tokens, locked, tok0_d, lk0_d)

        def step(i):
            s = i % T
            if s == 0:
                tokens.copy_(tok0_d)
                locked.copy_(lk0_d)
            ctx.denoise_step(tokens, locked, [T - s] * B)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        ctx.profile([bd.PROF_GATE_UP, bd.PROF_DOWN])
        prof_passes = [(steps + i) % T for i in range(4)]
        for i in range(4):
            step(steps + i)
        torch.cuda.synchronize()
        ctx.profile(())
        n_gu, ms_gu = ctx.profile_read(bd.PROF_GATE_UP)
        n_dn, ms_dn = ctx.profile_read(bd.PROF_DOWN)
    finally:
        ctx.close()
    gu_bytes = gate_up_bytes(w, touched_by_pass, prof_passes)
    gu_s = ms_gu / max(n_gu, 1) / 1e3
    ach = gu_bytes / gu_s / 1e9
    return {"workload": w.name, "ms_per_step": round(ms, 4), "canvas_tok_s": round(M / (ms / 1e3), 1),
            "gate_up_us": round(gu_s * 1e6, 2), "down_us": round(ms_dn / max(n_dn, 1) * 1e3, 2),
            "gate_up_roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_launch": int(gu_bytes)},
            "experts_touched_min": min(min(tp) for tp in touched_by_pass), "load_s": round(load_s, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="C3", help="C1..C5 (default C3: the 30-layer bf16 stack)")
    ap.add_argument("--blocks", type=int, default=2, help="whole blocks timed for resolved tok/s")
    ap.add_argument("--breakdown-steps", type=int, default=4,
                    help="extra passes after the timed region with every kernel class timed")
    ap.add_argument("--eb-blocks", type=int, default=1,
                    help="whole entropy-bounded blocks timed (at most 48 passes each)")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the variant with MXFP4 expert weights (a second context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--others", default="C4,C5",
                    help="further 30-layer workloads measured in their own contexts ('' for none)")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="only run 4 device copies of this many MiB (calibrates HBM byte counters) and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                              "COPY_WRITE_DIR"),
                    help="write the gate|up HBM traffic summary from rocprofv3 counter runs and exit")
    ap.add_argument("--copy-mib", type=int, default=512, help="size of the calibration copy")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: independent canvases shard with no exchange, see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import canvas_denoising_moe_amd as dg
    from canvas_denoising_moe_amd import binding as bd
    from synth import BY_ID, gen, upload

    if args.probe_copy_mib > 0:
        dev = torch.device("cuda", 0)
        nbytes = args.probe_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": 4}),
              flush=True)
        return

    w = BY_ID[args.workload]
    m = w.model
    B, N, T = w.batch, m.canvas_len, w.n_steps
    M = B * N
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    # room for the block commits timed at the end (each adds N cached positions)
    ctx = dg.Context(m, max_batch=B, max_prompt_len=w.prompt_len + 2 * N, device=0)
    upload.load_context(ctx, w, progress=True)
    torch.cuda.synchronize()
    init_s = time.perf_counter() - t0
    print(f"[bench] {w.name}: weights and prompt KV loaded in {init_s:.1f} s", file=sys.stderr, flush=True)

    tok0, lk0 = gen.canvas(w)
    tok0_d = torch.from_numpy(tok0).to(dev)
    lk0_d = torch.from_numpy(lk0).to(dev)
    tokens = tok0_d.clone()
    locked = lk0_d.clone()

    # routing of every pass of one block: experts that received tokens, per
    # pass of the block and layer (the weights of the others are not read)
    touched_by_pass = trace_touched(ctx, w, tokens, locked, tok0_d, lk0_d)

    def step(i):
        s = i % T
        if s == 0:
            tokens.copy_(tok0_d)
            locked.copy_(lk0_d)
        ctx.denoise_step(tokens, locked, [T - s] * B)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: only the dominant kernel carries (dispatch-bound) events, on
    # every launch of every 4th pass (each timed dispatch adds a few
    # microseconds of dispatch latency, so not every pass carries them)
    ctx.profile([bd.PROF_GATE_UP])
    ctx.profile((), keep=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % 4 == 0:
            ctx.profile([bd.PROF_GATE_UP], keep=True)
        step(i)
        if i % 4 == 0:
            ctx.profile((), keep=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ctx.profile(())
    n_gu, ms_gu = ctx.profile_read(bd.PROF_GATE_UP)
    ms_per_step = elapsed * 1e3 / args.steps
    value = M / (ms_per_step / 1e3)

    # per-kernel breakdown from extra passes with every class timed (events add
    # dispatch latency, so these passes are not part of the timed region)
    ctx.profile(True)
    for i in range(args.breakdown_steps):
        step(args.steps + i)
    torch.cuda.synchronize()
    ctx.profile(())
    prof = {k: ctx.profile_read(k) for k in (bd.PROF_GATE_UP, bd.PROF_DOWN, bd.PROF_ATTN,
                                              bd.PROF_LM_HEAD, bd.PROF_PASS)}

    # whole blocks (resolved tokens / block time), inputs restored outside the timing
    block_ms = []
    for _ in range(args.blocks):
        tokens.copy_(tok0_d)
        locked.copy_(lk0_d)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.generate_block(tokens, locked, T)
        torch.cuda.synchronize()
        block_ms.append((time.perf_counter() - t0) * 1e3)
        assert bool(locked.all()), "block left unlocked positions"
    newly = int(M - lk0.sum())
    block_med = float(np.median(block_ms)) if block_ms else float("nan")
    resolved = newly / (block_med / 1e3) if block_ms else float("nan")

    # entropy-bounded sampler: passes with the sampler head and the EB lock
    # step (timed alone, then with the LM head's launches timed), and whole
    # blocks that stop adaptively (one host read of the canvases' status per pass)
    eb_res = None
    if args.eb_blocks > 0:
        seeds = [1000 + b for b in range(B)]
        prev = torch.zeros((B, N), dtype=torch.int32, device=dev)
        status = torch.zeros(B, dtype=torch.int32, device=dev)
        eb_steps = min(args.steps, 8)

        def eb_run(k):
            tokens.copy_(tok0_d)
            locked.copy_(lk0_d)
            status.zero_()
            for t in range(k):
                ctx.eb_step(tokens, locked, t, 48, seeds, 0, prev, status)

        eb_run(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eb_run(eb_steps)
        torch.cuda.synchronize()
        eb_pass_ms = (time.perf_counter() - t0) * 1e3 / eb_steps
        ctx.profile([bd.PROF_LM_HEAD])
        eb_run(eb_steps)
        torch.cuda.synchronize()
        ctx.profile(())
        n_lm, ms_lm = ctx.profile_read(bd.PROF_LM_HEAD)
        eb_block_ms, eb_passes = [], None
        for _ in range(args.eb_blocks):
            tokens.copy_(tok0_d)
            locked.copy_(lk0_d)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            eb_passes = ctx.generate_block_eb(tokens, locked, seeds, 0, 48)
            torch.cuda.synchronize()
            eb_block_ms.append((time.perf_counter() - t0) * 1e3)
            assert bool(locked.all()), "EB block left unlocked positions"
        eb_med = float(np.median(eb_block_ms))
        eb_res = {"t_max": 48, "passes": eb_passes, "pass_ms": round(eb_pass_ms, 4),
                  "canvas_tok_s": round(M / (eb_pass_ms / 1e3), 1),
                  "lm_head_sampler_us": round(ms_lm / max(n_lm, 1) * 1e3, 2),
                  "block_ms": round(eb_med, 3), "resolved_tok_s": round(newly / (eb_med / 1e3), 1)}

    # block continuation: commit the resolved canvases to the prompt caches
    # (causal pass over the block + K/V append).  The first commit also sets
    # up the buffers the caches move between; the second is timed.  Last, as
    # it grows the context the passes above ran on.
    commit_ms = None
    if args.blocks > 0:
        ctx.commit_block(tokens)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ctx.commit_block(tokens)
        torch.cuda.synchronize()
        commit_ms = (time.perf_counter() - t0) * 1e3

    # the timed region's passes walk the block (pass i % T); the gate|up
    # launches carry events on every 4th pass
    timed = [i % T for i in range(args.steps)]
    byts, flops = pass_algorithmic(w, touched_by_pass, timed)
    gu_bytes = gate_up_bytes(w, touched_by_pass, [s for i, s in enumerate(timed) if i % 4 == 0])
    touched = [min(tp[l] for tp in touched_by_pass) for l in range(m.n_layers)]
    gu_avg_s = ms_gu / n_gu / 1e3
    achieved = gu_bytes / gu_avg_s / 1e9
    pass_n, pass_ms = prof[bd.PROF_PASS]
    kern = {"passes": pass_n, "pass_ms": round(pass_ms / max(pass_n, 1), 4)}
    for name, k in (("gate_up", bd.PROF_GATE_UP), ("down", bd.PROF_DOWN), ("attention", bd.PROF_ATTN),
                    ("lm_head", bd.PROF_LM_HEAD)):
        n, ms = prof[k]
        if n:
            kern[name] = {"launches": n, "avg_us": round(ms / n * 1e3, 2),
                          "share_of_pass": round(ms / pass_ms, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "canvas tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if m.dtype == "bf16" else "f32",
        "data": "synthetic (seeded random-init weights N(0,0.02), prompt KV N(0,1), uniform canvas)",
        "config": {"workload": w.name, "batch": B, "canvas_len": N, "layers": m.n_layers,
                   "prompt_len": w.prompt_len, "passes_per_block": T, "experts": m.n_experts,
                   "top_k": m.top_k, "vocab": m.vocab, "hidden": m.hidden},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "scope": "dominant kernel (the whole pass: pass_roofline)",
                     "kernel": "moe_grouped_gemm gate|up", "bytes_per_launch": int(gu_bytes),
                     "avg_launch_us": round(gu_avg_s * 1e6, 2)},
        "cpu_baseline": cpu,
        "resolved_tok_s": round(resolved, 1) if args.blocks > 0 else None,
        "block_ms": round(block_med, 3) if args.blocks > 0 else None,
        "commit_ms": round(commit_ms, 3) if commit_ms is not None else None,
        "resolved_tok_s_with_commit": round(newly / ((block_med + commit_ms) / 1e3), 1)
        if commit_ms is not None else None,
        "pass_roofline": {"bytes": int(byts), "flops": int(flops),
                          "hbm_frac": round(byts / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(flops / (ms_per_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels_breakdown": kern,
        "eb_sampler": eb_res,
        "experts_touched_min": min(touched),
        "init_s": round(init_s, 1),
    }
    ctx.close()
    if not args.no_mxfp4 and m.dtype == "bf16":
        torch.cuda.empty_cache()
        line["mxfp4_experts"] = measure_mxfp4(w, args.steps, args.warmup)
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        torch.cuda.empty_cache()
        line[name.lower()] = measure_workload(BY_ID[name], args.steps, args.warmup)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
