"""Benchmark of the KDA mixer core on one MI355X.

Default workload: the batched decode step, 256 sequences x 32 heads x head_dim 128, bf16
activations, fp32 state and conv rings, fresh activations for each of 128 consecutive
steps (all resident in HBM before timing).  One benchmark step = one kda_decode_step
launch over the whole batch.  Printed as one JSON line with:

* value      -- decode tokens/s per layer (256 x steps / time);
* roofline   -- the decode kernel against HBM: algorithmic bytes per launch / average
                launch duration (HIP events on the launch stream) vs 8 TB/s; `traffic` is
                the HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
                WRITE_SIZE, scaled by a copy-kernel calibration) when the stored
                measurement matches the current kernel source, else null;
* cpu_baseline -- the fp64 oracle timed on the host cores on a bounded sample of the
                same workload;
* prefill_scan_ab -- chunked prefill against the sequential-scan arm (kda_prefill_scan)
                on 256 prompts x 64 tokens x 32 heads;
* verify     -- the batched verify of speculative decoding on the same shape: 4 rows per
                sequence in one kda_decode_multi launch (tokens/s over all rows, HBM
                fraction at its algorithmic bytes);
* prefill    -- the chunked prefill on the 1 x 4096 x 32-head, 2 x 8192 x 96-head and
                16-sequence varlen x 64-head workloads, and on 2 x 8192 x 96 heads with
                the low-rank decay gate, the softplus gate, and both (3 warm-up runs, median of 20, each
                after a 768 MB write that flushes the 256 MB MALL): tokens/s, the fraction
                of HBM and of dense bf16 MFMA peak at the algorithmic byte and flop counts,
                and the roofline fraction max(bytes / HBM peak, flops / MFMA peak) / time;
                counter readings (HBM traffic, issued MFMA work) are attached from
                profiles/ when they were taken on the current kernel source.  The varlen
                entry also times its 32 decode steps from the returned states.

`--only-prefill` runs just the prefill part (for profiling); `--summarize-pmc` turns
rocprofv3 counter output into profiles/ summaries.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# Vector-ALU issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 fp32 instruction per SIMD
# every 2 cycles (the 157.3 TFLOP/s fp32 vector peak is 32 FMA lanes per SIMD and cycle;
# packed fp32 is not used).  Transcendentals (v_exp, v_rcp, ...) take 4 slots.
VALU_PEAK_INSTS = 256 * 4 * 2.4e9 / 2
D = 128

# Algorithmic HBM bytes per (token, head) of the decode step, bf16 io: fp32 state read and
# written once (2 x 128 x 128 x 4), fp32 ring of 3 planes x 128 channels x 3 taps read and
# written (2 x 4608), q/k/v/z/gate in (5 x 256), raw beta in (2), out (256).
DECODE_BYTES_PER_TOKEN_HEAD = 2 * D * D * 4 + 2 * 3 * D * 3 * 4 + 5 * D * 2 + 2 + D * 2
# Prefill, bf16 io: q/k/v/z/gate in, beta in, out; state/ring in and out are added per sequence.
PREFILL_BYTES_PER_TOKEN_HEAD = 5 * D * 2 + 2 + D * 2
IO_BYTES = {"bf16": 2, "f32": 4}
# Algorithmic prefill flops per (token, head) at chunk 64, the same count for every
# prefill workload whatever chunk the kernel uses: 6 d^2 + 5 C d + C^2 / 3.
PREFILL_FLOPS_PER_TOKEN_HEAD = 6 * D * D + 5 * 64 * D + 64 * 64 // 3
METRIC = "KDA tokens/s per layer (chunked prefill, decode); % of MFMA / HBM roofline"
DECODE_KERNEL = "decode_kernel"
PREFILL_KERNEL = "prefill_pc_kernel"  # the bf16 prefill kernel
PREFILL_WORKLOADS = ("tiny_prefill_fp32", "prefill_t4096_h32", "prefill_2x8192_h96", "varlen16_h64", "prefill_2x8192_h96_lowrank",
                     "prefill_2x8192_h96_softplus", "prefill_2x8192_h96_softplus_lowrank")


def kernel_source_hash(name: str) -> str:
    """Hash of the sources a kernel is built from, to tell whether stored counters are stale."""
    files = {"decode": ["kda_decode.hip", "kda_device.h", "kda_internal.h"],
             "prefill": ["kda_prefill.hip", "kda_prefill_pc.hip", "kda_mfma.h", "kda_device.h",
                         "kda_internal.h", "kda_api.cpp"]}[name]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_05_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_cores() -> int:
    """Threads for the oracle baseline: the cores this process may run on (its affinity
    mask), or fewer when the host's thread-count setting (OMP_NUM_THREADS) says so."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_info() -> dict:
    """The host CPU: model name, logical CPUs online, and the affinity mask's size."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = None
    return dict(model=model, nproc=os.cpu_count(), affinity=aff,
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"))


# --------------------------------------------------------------------------- decode

def bench_decode(steps: int, warmup: int, calibrate_copy: bool):
    import torch

    import gated_delta_rule_05_amd as kda
    import synthetic

    w = synthetic.WORKLOADS["decode_b256_h32"]
    dev = "cuda:0"
    dec = synthetic.make_workload(w.name, device=dev)
    layer = kda.Layer(**dec["layer"])
    B, H = w.batch, w.heads
    state, ring = dec["state"], dec["ring"]
    out = torch.empty((B, H * D), dtype=torch.bfloat16, device=dev)
    acts = [(dec["q"][s], dec["k"][s], dec["v"][s], dec["z"][s], dec["beta"][s], dec["gate"][s])
            for s in range(w.steps)]
    stream = torch.cuda.current_stream()

    def step(i):
        q, k, v, z, b, g = acts[i % w.steps]
        kda.decode_step(layer, q, k, v, z, b, g, state, ring, out=out, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    if calibrate_copy:
        copy_calibration()
    res = dict(B=B, H=H, ms_total=ms, ms_per_step=ms / steps,
               finite=bool(torch.isfinite(out.float()).all()))
    return res, dec


def bench_verify(dec, t: int = 4, reps: int = 32):
    """The batched verify of speculative decoding on the decode workload's shape: t rows
    per sequence in one kda_decode_multi launch (state and conv history stay in registers
    across the rows), ping-pong state buffers, median of `reps` launches.  Tokens/s counts
    all B * t rows; the algorithmic bytes are the state and ring once plus t rows of
    activations per (sequence, head)."""
    import torch

    import gated_delta_rule_05_amd as kda

    B, H = dec["q"].shape[1], dec["layer"]["num_heads"]
    layer = kda.Layer(**dec["layer"])
    rows = {n: dec[n][:t].transpose(0, 1).contiguous()
            for n in ("q", "k", "v", "z", "beta", "gate")}
    s0, r0 = dec["state"].clone(), dec["ring"].clone()
    s1, r1 = torch.empty_like(s0), torch.empty_like(r0)
    out = torch.empty((B, t, H * D), dtype=dec["q"].dtype, device=s0.device)
    stream = torch.cuda.current_stream()

    def run():
        kda.decode_multi(layer, rows["q"], rows["k"], rows["v"], rows["z"], rows["beta"],
                         rows["gate"], s0, r0, s1, r1, out=out, stream=stream)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    ms = times[len(times) // 2]
    act = 5 * D * 2 + 2 + D * 2
    nbytes = B * H * (2 * D * D * 4 + 2 * 3 * D * 3 * 4 + t * act)
    return dict(rows_per_sequence=t, batch=B, heads=H, ms=ms, tokens_per_s=B * t / (ms / 1e3),
                hbm_gbs=nbytes / (ms / 1e3) / 1e9, hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                algorithmic_bytes=nbytes)


def copy_calibration(nbytes: int = 1 << 30):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def decode_traffic(steps_hash: str):
    """Measured HBM bytes per decode launch from the stored counter summary, or None."""
    p = os.path.join(ROOT, "profiles", "decode_b256_h32_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        doc = json.load(f)
    if doc.get("source_hash") != steps_hash:
        return None
    return doc.get("bytes_per_launch")


# --------------------------------------------------------------------------- prefill

def prefill_algorithmic_bytes(w) -> int:
    """Bytes a prefill workload must move at least: the bf16 activation planes in and the
    output out per token-head, the state and ring once per sequence (in only when given);
    with the low-rank gate, z_low [T, 128] (shared by the heads) and f_b [H*128, 128] in
    place of the full-rank z plane."""
    N, H, T = len(w.seqlens), w.heads, sum(w.seqlens)
    e = IO_BYTES[w.io]
    nbytes = ((5 * D + 1 + D) * e * T * H + N * H * D * D * 4 * (2 if w.init_state else 1)
              + N * 3 * H * D * 3 * 4 * (2 if w.init_ring else 1))
    if w.low_rank_gate:
        nbytes += -D * e * T * H + D * e * T + H * D * D * e
    return nbytes


def bench_prefill(name: str, reps: int, warmup: int = 3, cpu: bool = True):
    import torch

    import gated_delta_rule_05_amd as kda
    import synthetic

    w = synthetic.WORKLOADS[name]
    dev = "cuda:0"
    prob = synthetic.make_workload(name, device=dev)
    layer = kda.Layer(**prob["layer"])
    cu_dev = prob["cu_seqlens"].to(dev)
    T = sum(w.seqlens)
    N = len(w.seqlens)
    dt = synthetic.torch_io_dtype(w.io)
    out = torch.empty((T, w.heads * D), dtype=dt, device=dev)
    st = torch.empty((N, w.heads, D, D), dtype=torch.float32, device=dev)
    rg = torch.empty((N, 3 * w.heads * D, 3), dtype=torch.float32, device=dev)
    flush = torch.empty(768 << 20, dtype=torch.uint8, device=dev)  # larger than the 256 MB MALL
    stream = torch.cuda.current_stream()
    ws_bytes = kda.prefill_workspace_bytes(layer, dt, prob["cu_seqlens"])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def run():
        kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"], prob["gate"],
                    cu_dev, prob["cu_seqlens"], state_in=prob["state_in"], ring_in=prob["ring_in"],
                    out=out, state_out=st, ring_out=rg, workspace=ws, stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    ms = times[len(times) // 2]
    H = w.heads
    nbytes = prefill_algorithmic_bytes(w)
    flops = PREFILL_FLOPS_PER_TOKEN_HEAD * T * H
    s = ms / 1e3
    res = dict(workload=name, sequences=N, tokens=T, heads=H, io=w.io,
               path="segment-parallel" if ws_bytes else "whole-sequence", workspace_bytes=ws_bytes,
               decay_gate=(("softplus, " if w.softplus_gate else "") +
                           ("low-rank (z_low f_b^T in the kernel)" if w.low_rank_gate else "full-rank z")),
               ms=ms, ms_min=times[0], reps=reps,
               tokens_per_s=T / s, hbm_gbs=nbytes / s / 1e9, hbm_frac=nbytes / s / 1e9 / HBM_PEAK_GBS,
               mfma_tflops=flops / s / 1e12, mfma_frac=flops / s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
               roofline_frac=max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) / s,
               algorithmic_bytes=nbytes, algorithmic_flops=flops,
               finite=bool(torch.isfinite(out.float()).all()))
    counters = prefill_counters(name)
    if counters:
        res["counters"] = counters
        # the kernel's actual bound: vector-ALU issue, from the counted instructions
        vi = counters.get("valu_insts_per_token_head")
        if vi:
            rate = vi * T * H / s
            res["alu_roofline"] = dict(bound="alu", achieved=rate, peak=VALU_PEAK_INSTS,
                                       unit="wave64 VALU instructions/s", frac=rate / VALU_PEAK_INSTS)
    if w.decode_after:
        res["decode_continuation"] = bench_decode_after(w, layer, st, rg, stream)
    del out, flush
    if cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(w, prob)
    del prob
    return res


def bench_scan_ab(name: str = "short256x64_h32", reps: int = 20):
    """The chunked prefill against the sequential-scan arm on a batch of short prompts:
    median of `reps` calls each, MALL flushed before each."""
    import torch

    import gated_delta_rule_05_amd as kda
    import synthetic

    w = synthetic.WORKLOADS[name]
    prob = synthetic.make_workload(name, device="cuda:0")
    layer = kda.Layer(**prob["layer"])
    cu_dev = prob["cu_seqlens"].to("cuda:0")
    flush = torch.empty(768 << 20, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = dict(workload=name, sequences=len(w.seqlens), tokens_per_sequence=w.seqlens[0], heads=w.heads)
    for arm in ("chunked", "scan"):
        def run():
            kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"], prob["gate"],
                        cu_dev, prob["cu_seqlens"], state_in=prob["state_in"], ring_in=prob["ring_in"],
                        scan=arm == "scan", stream=stream)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            flush.fill_(1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        ms = times[len(times) // 2]
        res[arm] = dict(ms=ms, tokens_per_s=sum(w.seqlens) / (ms / 1e3))
    return res


def bench_decode_after(w, layer, st, rg, stream):
    """The workload's decode continuation: w.decode_after steps over all its sequences from
    the returned states and rings (fresh activations per step, resident before timing)."""
    import torch

    import gated_delta_rule_05_amd as kda
    import synthetic

    N, H, steps = len(w.seqlens), w.heads, w.decode_after
    g = synthetic.gen(w.seed + 1, "cuda:0")
    acts = synthetic.activations(N, H, w.io, g, "cuda:0", lead=(steps,))
    out = torch.empty((N, H * D), dtype=torch.bfloat16, device="cuda:0")
    kda.decode_step(layer, acts["q"][0], acts["k"][0], acts["v"][0], acts["z"][0], acts["beta"][0],
                    acts["gate"][0], st, rg, out=out, stream=stream)  # warm-up
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        kda.decode_step(layer, acts["q"][i], acts["k"][i], acts["v"][i], acts["z"][i],
                        acts["beta"][i], acts["gate"][i], st, rg, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = DECODE_BYTES_PER_TOKEN_HEAD * N * H
    return dict(batch=N, heads=H, steps=steps, ms_per_step=ms, tokens_per_s=N / (ms / 1e3),
                hbm_gbs=nbytes / (ms / 1e3) / 1e9, hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS)


def prefill_counters(name: str):
    """Stored counter readings for a prefill workload, if taken on the current source."""
    p = os.path.join(ROOT, "profiles", "prefill_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        doc = json.load(f)
    if doc.get("source_hash") != kernel_source_hash("prefill"):
        return None
    return doc.get("workloads", {}).get(name)


# --------------------------------------------------------------------------- CPU baseline

PREFILL_CPU_SAMPLE = 2.0e6  # token-heads of oracle work per prefill workload (a few seconds)


def prefill_cpu_baseline(w, prob):
    """The fp64 oracle on the workload's own inputs, threaded over (sequence, head) units:
    every unit when the workload has at most PREFILL_CPU_SAMPLE token-heads, otherwise the
    first k heads of every sequence with k chosen to stay near that budget (all sequence
    lengths are kept).  Tokens/s per layer = sampled token-heads / H / time, i.e. the time
    scaled up from the sampled fraction of the units to the whole workload."""
    import oracle

    N, H, T = len(w.seqlens), w.heads, sum(w.seqlens)
    k = H if T * H <= PREFILL_CPU_SAMPLE else max(1, int(-(-PREFILL_CPU_SAMPLE * H // (T * H))))
    units = [(n, h) for n in range(N) for h in range(k)]
    p = prob["layer"]
    cpu = lambda x: None if x is None else x.detach().cpu()
    lay = oracle.Layer(H, D, cpu(p["conv_w"]), cpu(p["dt_bias"]), cpu(p["A_log"]), cpu(p["norm_w"]),
                       lower_bound=p["lower_bound"], l2_eps=p["l2_eps"], rms_eps=p["rms_eps"],
                       gate_kind=p.get("gate_kind", 0), f_b=cpu(p.get("f_b")))
    acts = {n: cpu(prob[n]) for n in ("q", "k", "v", "z", "beta", "gate")}
    st = None if prob.get("state_in") is None else cpu(prob["state_in"]).double().numpy()
    rg = None if prob.get("ring_in") is None else cpu(prob["ring_in"]).numpy()
    io = oracle.BF16 if w.io == "bf16" else oracle.F32
    cores = min(cpu_cores(), len(units))
    t = time.perf_counter()
    oracle.prefill_units(lay, io, prob["cu_seqlens"], acts["q"], acts["k"], acts["v"], acts["z"],
                         acts["beta"], acts["gate"], st, rg, units=units, nthreads=cores)
    el = time.perf_counter() - t
    th = k * T
    return {"value": th / H / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"all {N * H} units" if k == H else f"heads 0..{k - 1} of all {N} sequences "
                       f"({k} of {H} heads, scaled by {H / k:.2f})") +
                      f": {th} token-heads in {el:.2f} s"}


def cpu_baseline(dec, target_s: float = 10.0):
    """The fp64 oracle on a bounded sample of the decode workload: all heads of the first
    u sequences over all 128 steps (each sequence's 128 steps as one oracle sequence, the
    same math as 128 decode steps), threaded over (sequence, head) units; u grows until
    the sample takes about target_s seconds or covers the whole batch."""
    import numpy as np

    import oracle

    H = dec["layer"]["num_heads"]
    Hd = H * D
    steps = dec["q"].shape[0]
    B = dec["q"].shape[1]
    p = dec["layer"]
    lay = oracle.Layer(H, D, p["conv_w"].cpu().numpy(), p["dt_bias"].cpu().numpy(),
                       p["A_log"].cpu().numpy(), p["norm_w"].cpu().numpy(),
                       lower_bound=p["lower_bound"], l2_eps=p["l2_eps"], rms_eps=p["rms_eps"])
    cores = cpu_cores()

    def sample(u):
        acts = {n: dec[n][:, :u].transpose(0, 1).reshape(u * steps, -1).cpu()
                for n in ("q", "k", "v", "z", "gate", "beta")}
        st = dec["state"][:u].double().cpu().numpy()
        rg = dec["ring"][:u].cpu().numpy()
        cu = np.arange(u + 1, dtype=np.int64) * steps
        t = time.perf_counter()
        oracle.prefill_units(lay, oracle.BF16, cu, acts["q"], acts["k"], acts["v"], acts["z"],
                             acts["beta"], acts["gate"], st, rg, nthreads=cores)
        return time.perf_counter() - t

    u = 2
    el = sample(u)
    u2 = int(min(B, max(u, u * target_s / max(el, 1e-3))))
    if u2 > u:
        u, el = u2, sample(u2)
    token_heads = u * steps * H
    return {"value": u * steps / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{u} sequences x {H} heads x {steps} decode steps ({token_heads} "
                      f"token-heads) in {el:.1f} s"}


# --------------------------------------------------------------------------- PMC summaries

def _read_pmc(d: str, counter: str):
    """(kernel name, grid size, value) for every dispatch row of one counter, from
    rocprofv3's CSV output (--output-format csv) or its default SQLite database."""
    import csv
    import sqlite3
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0),
                                 float(r["Counter_Value"])))
    if not rows:
        for f in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
            con = sqlite3.connect(f)
            try:
                rows += [(k, int(g or 0), float(v)) for k, g, v in con.execute(
                    "select kernel_name, grid_size, value from counters_collection where counter_name = ?",
                    (counter,))]
            finally:
                con.close()
    return rows


def _copy_scale(rows):
    """Bytes per counted KiB, from the 1 GiB device copy (the largest copy dispatch)."""
    c = max((x for k, _, x in rows if "copyBuffer" in k), default=None)
    return (float(1 << 30) / (c * 1024), c) if c else (None, None)


def summarize_pmc(fetch_dir: str, write_dir: str):
    """Reads two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of
    `bench.py --decode-only --calibrate-copy` (decode steps only, so every decode-kernel
    dispatch is a one-row step), scales each by the same counter's reading on the 1 GiB
    copy kernel, and writes profiles/decode_b256_h32_pmc.json."""
    fetch = _read_pmc(fetch_dir, "FETCH_SIZE")
    write = _read_pmc(write_dir, "WRITE_SIZE")

    def mean_for(rows, pat):
        v = [x for k, _, x in rows if pat in k]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    f_dec, nf = mean_for(fetch, DECODE_KERNEL)
    w_dec, nw = mean_for(write, DECODE_KERNEL)
    f_scale, f_copy = _copy_scale(fetch)
    w_scale, w_copy = _copy_scale(write)
    fetched = f_dec * 1024 * f_scale if (f_dec and f_scale) else None
    written = w_dec * 1024 * w_scale if (w_dec and w_scale) else None
    alg = DECODE_BYTES_PER_TOKEN_HEAD * 256 * 32
    total = (fetched + written) if (fetched and written) else None
    doc = dict(kernel=DECODE_KERNEL, source_hash=kernel_source_hash("decode"),
               fetch_kib_per_dispatch=f_dec, write_kib_per_dispatch=w_dec, dispatches=[nf, nw],
               copy_fetch_kib=f_copy, copy_write_kib=w_copy, fetch_scale=f_scale,
               write_scale=w_scale, fetched_bytes=fetched, written_bytes=written,
               bytes_per_launch=total, algorithmic_bytes_per_launch=alg,
               traffic_over_algorithmic=(total / alg) if total else None)
    with open(os.path.join(ROOT, "profiles", "decode_b256_h32_pmc.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
    print(json.dumps(doc, indent=1))


def summarize_prefill_pmc(root: str):
    """Reads, for each prefill workload W, three rocprofv3 --pmc runs of
    `bench.py --only-prefill --prefill-workloads W --prefill-reps 1 --prefill-warmup 0
    --calibrate-copy` in ROOT/W_fetch (FETCH_SIZE), ROOT/W_write (WRITE_SIZE) and
    ROOT/W_mfma (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU, SQ_INSTS_MFMA).  Every
    dispatch of this library's kernels in a run belongs to the one prefill call (all
    passes of the segment-parallel path included); byte counters are scaled by the 1 GiB
    copy calibration.  Writes profiles/prefill_pmc.json: measured HBM bytes against the
    algorithmic bytes, and the bf16 MFMA work issued (512 flops per MOPS unit) against the
    algorithmic flops."""
    import synthetic

    out = {}
    scales = {}
    for name in PREFILL_WORKLOADS:
        d = {k: os.path.join(root, f"{name}_{k}") for k in ("fetch", "write", "mfma")}
        if not all(os.path.isdir(x) for x in d.values()):
            continue
        fetch = _read_pmc(d["fetch"], "FETCH_SIZE")
        write = _read_pmc(d["write"], "WRITE_SIZE")
        f_scale, f_copy = _copy_scale(fetch)
        w_scale, w_copy = _copy_scale(write)
        scales[name] = dict(fetch_scale=f_scale, write_scale=w_scale)

        def mine(k):
            return "kda::" in k and ("prefill" in k or "combine" in k)

        def total(rows):
            v = [x for k, _, x in rows if mine(k)]
            return sum(v) if v else None

        def kernels(rows):
            return sorted({re.findall(r"(\w+(?:<[\w, ]+>)?)\(", k)[0] for k, _, _ in rows if mine(k)})

        w = synthetic.WORKLOADS[name]
        N, H, T = len(w.seqlens), w.heads, sum(w.seqlens)
        f, wr = total(fetch), total(write)
        m = total(_read_pmc(d["mfma"], "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        va = total(_read_pmc(d["mfma"], "SQ_INSTS_VALU"))
        mf = total(_read_pmc(d["mfma"], "SQ_INSTS_MFMA"))
        alg = prefill_algorithmic_bytes(w)
        traffic = (f * 1024 * f_scale + wr * 1024 * w_scale) if (f and wr and f_scale and w_scale) else None
        out[name] = dict(kernels=kernels(fetch), hbm_bytes=traffic, algorithmic_bytes=alg,
                         traffic_over_algorithmic=(traffic / alg) if traffic else None,
                         mfma_flops_issued=(m * 512) if m else None,
                         algorithmic_flops=PREFILL_FLOPS_PER_TOKEN_HEAD * T * H,
                         valu_insts_per_token_head=(va / (T * H)) if va else None,
                         mfma_insts_per_token_head=(mf / (T * H)) if mf else None)
    doc = dict(kernel=PREFILL_KERNEL, source_hash=kernel_source_hash("prefill"),
               calibration=scales, workloads=out)
    with open(os.path.join(ROOT, "profiles", "prefill_pmc.json"), "w") as fh:
        json.dump(doc, fh, indent=1)
    print(json.dumps(doc, indent=1))


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the timed decode steps (no verify, prefill, A/B or CPU "
                         "baseline), so that a profile of the run holds decode steps alone")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--prefill-workloads", default=",".join(PREFILL_WORKLOADS))
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the prefill workloads and print their list")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-prefill-pmc", metavar="ROOT_DIR")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return 0
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(args.summarize_prefill_pmc)
        return 0
    if args.gpus != 1:
        print(f"bench.py: the KDA core runs on one GPU here; --gpus {args.gpus} is not supported "
              "(it shards by head or by sequence with no exchange between GPUs)",
              file=sys.stderr)
        return 2

    import torch
    import gated_delta_rule_05_amd as kda
    kda.load()  # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    workloads = [x for x in args.prefill_workloads.split(",") if x]

    def prefill_list():
        pf = []
        for name in workloads:
            pf.append(bench_prefill(name, args.prefill_reps, args.prefill_warmup,
                                    cpu=not args.no_cpu_baseline))
            torch.cuda.empty_cache()
        return pf

    if args.only_prefill:
        args.no_cpu_baseline = True
        pf = prefill_list()
        if args.calibrate_copy:
            copy_calibration()
        print(json.dumps({"prefill": pf}), flush=True)
        return 0

    dres, dec = bench_decode(args.steps, args.warmup, args.calibrate_copy)
    B, H = dres["B"], dres["H"]
    ms_step = dres["ms_per_step"]
    bytes_launch = DECODE_BYTES_PER_TOKEN_HEAD * B * H
    achieved = bytes_launch / (ms_step / 1e3) / 1e9
    traffic = decode_traffic(kernel_source_hash("decode"))
    line = {
        "metric": METRIC,
        "value": B * args.steps / (dres["ms_total"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_b256_h32", "batch": B, "heads": H, "head_dim": D,
                   "io": "bf16", "state": "f32", "activation_sets": 128},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": DECODE_KERNEL, "algorithmic_bytes_per_launch": bytes_launch},
    }
    if args.decode_only:
        print(json.dumps(line), flush=True)
        return 0
    line["verify"] = bench_verify(dec)
    if not args.no_prefill:
        line["prefill"] = prefill_list()
        line["prefill_scan_ab"] = bench_scan_ab()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(dec)
        line["cpu"] = cpu_info()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
