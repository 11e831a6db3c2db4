"""Benchmark of the blockwise-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-secondary]

A step is one pass of the hot path over one batch of synthetic input.  The
headline workload is one GPU's share of a causal ring at long context: a
16384-token query block (block 12 of 16 over a 262144-token sequence; GQA
64/8, head_dim 128, bf16) walks the K/V blocks in ring order 12, 11, ..., 0
with fp32 (m, l, O) state carried in HBM between calls -- one
``blockattn_fwd_block`` call per ring visit, the last visit with visible keys
finalising in the same call; blocks 13-15 lie in the causal future and make
no call.  ``value`` is algorithmic TFLOP/s (4 * D * Hq * visible (query, key)
pairs per step).

The line also carries the roofline of the dominant kernel (measured live with
HIP events around each launch, on the stream it runs on), its MFMA
utilisation and HBM bytes from the committed rocprofv3 counter runs when they
match the current kernel sources, the CPU oracle timed on a bounded sample
of the same workload, every workload's input SHA-256 and its errors against
the oracle, and secondary measurements of the other workloads (the 32K
causal prefill, fan-out decode and prefill, sharded merge, scaled merge,
backward, causal shard layouts) with a library bf16 GEMM timed the same way
as the board's sustained matrix-core rate under its power limit.
Prints exactly one JSON line (on stdout); progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import shutil
import subprocess
import threading
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
NOMINAL_MHZ = 2400.0        # the shader clock the published peaks assume
METRIC = "attention fwd TFLOP/s + MFMA util %; fan-out decode HBM GB/s (1 GPU)"
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def counters_record(key: str):
    """The committed rocprofv3 counter record of one kernel and workload
    (profiles/traffic.json), or None when it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(key)
    if not entry:
        return None
    from exact_blockwise_long_amd import build
    if entry.get("source_sha256") != build.sources_digest():
        return None
    return entry


def traffic_record(key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current sources."""
    entry = counters_record(key)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


class DevIO:
    """Host synthetic tensors to device tensors (the binding's from_host)."""

    def __init__(self, ba):
        self.ba = ba

    def to_device(self, t):
        return self.ba.from_host(t.storage, t.dtype == "bf16")


def input_sha256(tensors, names=("q", "k", "v")):
    """SHA-256 of each input's storage bits (NumPy does not promise stream stability across versions)."""
    return {n: t.sha256() for n, t in zip(names, tensors)}


FANOUT_NAMES = ("q", "prefix_k", "prefix_v", "suffix_k", "suffix_v")


class Timer:
    """HIP events on the current stream, i.e. the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def all_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def mean_ms(self):
        return float(np.mean(self.all_ms()))

    def median_ms(self):
        return float(np.median([a.elapsed_time(b) for a, b in self.pairs]))


def bench_prefill(torch, ba, H, w, steps, warmup, fused=True):
    """The 32K causal prefill: every visit of the query block in one call, then
    finalisation -- fused into the same call (blockattn_fwd_block_finalize), or
    as fwd_block + finalize."""
    log(f"inputs: {w.name}")
    q, k, v = w.make_inputs()
    sha = input_sha256((q, k, v))
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = [(kd[b * w.block_len:(b + 1) * w.block_len], vd[b * w.block_len:(b + 1) * w.block_len],
               b * w.block_len) for b in range(w.n_blocks)]
    st = ba.new_state(w.rows, w.head_dim)
    out = torch.empty(w.rows, w.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.rows, dtype=torch.float32, device="cuda")

    def step(timer=None):
        e0 = timer.start() if timer else None
        if fused:
            ba.fwd_block_finalize(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                                  causal=w.causal, out=out, lse=lse)
        else:
            ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                         causal=w.causal)
        if timer:
            timer.stop(e0)
        if not fused:
            ba.finalize(st, out=out, lse=lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    flops = w.flops()
    kernel_ms = timer.mean_ms()
    tf, ktf = flops / ms_step / 1e9, flops / kernel_ms / 1e9
    log(f"prefill{' (fused finalisation)' if fused else ''}: {ms_step:.3f} ms/step, walk kernel {kernel_ms:.3f} ms, "
        f"{tf:.1f} TFLOP/s")
    cnt = counters_record("walk_kernel_causal_prefill") or {}
    res = {"workload": w.name, "ms_per_step": round(ms_step, 4), "TFLOP/s": round(tf, 1),
           "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops_per_step": flops,
           "calls": "one blockattn_fwd_block_finalize call per step (every visit, then the finalised output)",
           "roofline": {"kernel": "walk_kernel<128>", "bound": "mfma", "achieved": round(ktf, 2),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ktf / PEAK_BF16_TFLOPS, 4),
                        "traffic": cnt.get("hbm_bytes_per_launch"), "mfma_util_pct": cnt.get("mfma_util_pct"),
                        "kernel_ms_mean": round(kernel_ms, 4)},
           "input_sha256": sha}
    return dict(result=res, q=q, k=k, v=v, out=out, lse=lse, step=step, kernel_ms=kernel_ms, flops=flops)


def bench_backward(torch, ba, H, w, steps, warmup):
    """Backward of the prefill workload: clear the fp32 accumulators, bwd_delta,
    then one bwd_block call over the forward's visits (the dQ walk and the
    dK/dV kernel).  Algorithmic work is five products per visible pair (scores
    recomputed once, dP, dV, dK, dQ: 2.5x the forward's); the kernels
    recompute scores and dP on both sides, seven products."""
    log(f"inputs: {w.name} (backward)")
    q, k, v = w.make_inputs()
    do = w.make_dout()
    sha = input_sha256((q, k, v, do), ("q", "k", "v", "dout"))
    qd, kd, vd, dod = H.to_device(q), H.to_device(k), H.to_device(v), H.to_device(do)
    del q, k, v, do
    L = w.block_len
    blocks = [(kd[b * L:(b + 1) * L], vd[b * L:(b + 1) * L], b * L) for b in range(w.n_blocks)]
    st = ba.new_state(w.rows, w.head_dim)
    ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)
    out, lse = ba.finalize(st)
    del st
    delta = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    dq = torch.empty(w.rows, w.head_dim, dtype=torch.float32, device="cuda")
    dkv = [(torch.empty(L, w.n_kv_heads, w.head_dim, dtype=torch.float32, device="cuda"),
            torch.empty(L, w.n_kv_heads, w.head_dim, dtype=torch.float32, device="cuda")) for _ in blocks]

    def step(timer=None):
        dq.zero_()
        for a, b in dkv:
            a.zero_()
            b.zero_()
        ba.bwd_delta(out, dod, delta)
        e0 = timer.start() if timer else None
        ba.bwd_block(qd, dod, lse, delta, blocks, w.order, dq, dkv, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                     causal=w.causal)
        if timer:
            timer.stop(e0)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kms = timer.mean_ms()
    alg = 2.5 * w.flops()
    tf, ktf = alg / ms / 1e9, alg / kms / 1e9
    log(f"backward: {ms:.3f} ms/step, bwd_block {kms:.3f} ms, {tf:.1f} TFLOP/s step, {ktf:.1f} TFLOP/s kernels")
    return {"workload": w.name + ", backward", "ms_per_step": round(ms, 3), "TFLOP/s": round(tf, 1),
            "bwd_block_ms_mean": round(kms, 3), "bwd_block_TFLOP/s": round(ktf, 1),
            "bwd_block_frac_of_bf16_peak": round(ktf / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flops_per_step": alg, "executed_mfma_flops_per_step": 3.5 * w.flops(),
            "step": "zero dq/dk/dv, bwd_delta, bwd_block (dq_kernel + dkdv_kernel)", "input_sha256": sha}


def _smi_sample():
    """One amd-smi reading: (mean GFX clock over the XCDs in MHz, socket power in W) or None."""
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                             text=True, timeout=10).stdout
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
        pw = g["power"]["socket_power"]["value"]
        return (sum(clk) / len(clk), float(pw)) if clk else None
    except Exception:  # the tool is absent or its output format differs: no clock record
        return None


def sample_clock(torch, step, seconds):
    """Shader clock and board power while `step` runs back to back for `seconds`.

    The headline kernel holds the board at its power limit, where the clock
    settles below the 2.4 GHz the nominal peak assumes; the bench reports the
    achieved rate against both.  Readings taken while the GPU idles (clock
    under 1 GHz, e.g. before the first launch lands) are dropped.
    """
    if shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            r = _smi_sample()
            if r is not None:
                samples.append(r)
            stop.wait(0.1)

    for _ in range(20):  # bring the clock up before sampling starts
        step()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    busy = [s for s in samples if s[0] >= 1000.0]
    if not busy:
        return None
    mhz = sum(s[0] for s in busy) / len(busy)
    watts = sum(s[1] for s in busy) / len(busy)
    log(f"clock during a sustained run: {mhz:.0f} MHz mean GFX clock, {watts:.0f} W socket power "
        f"({len(busy)} amd-smi readings)")
    return {"gfx_mhz_mean": round(mhz, 1), "socket_power_w_mean": round(watts, 1), "readings": len(busy),
            "source": f"amd-smi metric, {seconds:.0f} s of back-to-back steps after the timed region"}


def bench_ring_share(torch, ba, H, w, steps, warmup):
    """One GPU's share of a causal ring (the headline).  One blockattn_fwd_block
    call per ring visit, fp32 state carried in HBM between calls; the last
    visit whose block has visible keys calls blockattn_fwd_block_finalize
    instead and writes the output.  Visits of blocks wholly in the causal
    future make no call (the rule lets no key of theirs in).  Every launch is
    bracketed by HIP events on the stream it runs on."""
    log(f"inputs: {w.name}")
    q, k, v = w.make_inputs()
    sha = input_sha256((q, k, v))
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = [(kd[b * w.block_len:(b + 1) * w.block_len], vd[b * w.block_len:(b + 1) * w.block_len],
               b * w.block_len) for b in range(w.n_blocks)]
    st = ba.new_state(w.rows, w.head_dim)
    out = torch.empty(w.rows, w.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    visible = w.visited_nonempty()
    skipped = [b for b in w.order if b not in visible]
    last = len(visible) - 1
    kw = dict(n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)

    def step(timer=None):
        for i, j in enumerate(visible):
            e0 = timer.start() if timer else None
            if i < last:
                ba.fwd_block(qd, blocks, [j], st, reset=(i == 0), **kw)
            else:
                ba.fwd_block_finalize(qd, blocks, [j], st, reset=(i == 0), out=out, lse=lse, **kw)
            if timer:
                timer.stop(e0)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    launches = np.array(timer.all_ms()).reshape(steps, len(visible))
    kernel_ms_step = float(launches.sum(axis=1).mean())
    flops = w.flops()
    tf = flops / ms / 1e9
    ktf = flops / kernel_ms_step / 1e9
    log(f"ring share: {ms:.2f} ms/step, {len(visible)} launches {kernel_ms_step:.2f} ms, {tf:.1f} TFLOP/s "
        f"(kernels {ktf:.1f})")
    return dict(q=q, k=k, v=v, out=out, lse=lse, step=step, ms_step=ms, kernel_ms_step=kernel_ms_step,
                launch_ms_mean=float(launches.mean()), launch_ms_by_visit=launches.mean(axis=0).tolist(),
                flops=flops, visible=visible, skipped=skipped, sha=sha)


class Flusher:
    """Evicts L2 and the 256 MB infinity cache between timed calls by reading 1 GiB.

    A read (not a fill) so no dirty lines are left to be written back while
    the timed kernel runs.
    """

    def __init__(self, torch):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.sink.copy_(self.buf.amax())


def flush_buffer(torch):
    return Flusher(torch)


def bench_fanout(torch, ba, H, w, steps, warmup):
    log(f"inputs: {w.name}")
    ins = w.make_inputs()
    dev = [H.to_device(t) for t in ins]
    nb, Hq, D = dev[0].shape
    out = torch.empty(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nb, Hq, dtype=torch.float32, device="cuda")
    ws = torch.empty(ba.fanout_workspace_bytes(nb, Hq, w.n_kv_heads, D, w.prefix_len, w.suffix_len),
                     dtype=torch.uint8, device="cuda")
    flush = flush_buffer(torch)
    for _ in range(warmup):
        ba.fanout_prefix_decode(*dev, workspace=ws, out=out, lse=lse)
    timer = Timer(torch)
    for _ in range(steps):
        flush()
        e0 = timer.start()
        ba.fanout_prefix_decode(*dev, workspace=ws, out=out, lse=lse)
        timer.stop(e0)
    torch.cuda.synchronize()
    ms = timer.median_ms()
    gbs = w.bytes() / ms / 1e6
    log(f"fanout: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    res = {"workload": w.name, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": w.bytes(),
           "traffic_attention_kernel": traffic_record("fanout_kernel_fanout_decode"),
           "timing": "median over steps, HIP events around the call, 1 GiB read between calls evicts the caches",
           "input_sha256": input_sha256(ins, FANOUT_NAMES)}
    return dict(result=res, ins=ins, out=out, lse=lse)


def bench_fanout_paged(torch, ba, H, w, steps, warmup, page_len=256):
    """The fan-out decode workload with its prefix and private suffixes in a
    page pool (page_len-token pages, seeded random pool order), timed like
    bench_fanout; the algorithmic bytes are the same."""
    from exact_blockwise_long_amd import workloads as wl
    log(f"inputs: {w.name}, paged (page_len {page_len})")
    q, pk, pv, sk, sv = w.make_inputs()
    g = np.random.Generator(np.random.PCG64(w.seed + 500))
    n_pool, pp, sp = wl.paged_layout(g, w.n_branches, w.prefix_len, w.suffix_len, page_len)
    kpool = wl.scatter_pages(g, pk, sk, n_pool, pp, sp, page_len)
    vpool = wl.scatter_pages(g, pv, sv, n_pool, pp, sp, page_len)
    sha = {"q": q.sha256(), "k_pool": kpool.sha256(), "v_pool": vpool.sha256(),
           "prefix_pages": hashlib.sha256(pp.tobytes()).hexdigest(),
           "suffix_pages": hashlib.sha256(sp.tobytes()).hexdigest()}
    kd, vd = H.to_device(kpool), H.to_device(vpool)
    del pk, pv, sk, sv, kpool, vpool
    qd = H.to_device(q)
    ppd, spd = torch.from_numpy(pp).cuda(), torch.from_numpy(sp).cuda()
    nb, Hq, D = qd.shape
    out = torch.empty(nb, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nb, Hq, dtype=torch.float32, device="cuda")
    ws = torch.empty(ba.fanout_workspace_bytes(nb, Hq, w.n_kv_heads, D, w.prefix_len, w.suffix_len),
                     dtype=torch.uint8, device="cuda")
    flush = flush_buffer(torch)

    def call():
        ba.fanout_prefix_decode_paged(qd, kd, vd, ppd, spd, w.prefix_len, w.suffix_len, workspace=ws, out=out,
                                      lse=lse)

    for _ in range(warmup):
        call()
    timer = Timer(torch)
    for _ in range(steps):
        flush()
        e0 = timer.start()
        call()
        timer.stop(e0)
    torch.cuda.synchronize()
    ms = timer.median_ms()
    gbs = w.bytes() / ms / 1e6
    log(f"fanout paged: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"workload": w.name + f", paged (page_len {page_len}, random pool order)", "us": round(ms * 1e3, 2),
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "pool_pages": int(n_pool),
            "timing": "median over steps, HIP events around the call, 1 GiB read between calls evicts the caches",
            "input_sha256": sha}


def bench_shard_merge(torch, ba, H, w, steps, warmup):
    log(f"inputs: {w.name}")
    q, k, v = w.make_inputs()
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    sl = w.shard_len
    blocks = [(kd[i * sl:(i + 1) * sl], vd[i * sl:(i + 1) * sl], i * sl) for i in range(w.n_shards)]
    states = [ba.new_state(w.rows, w.head_dim) for _ in range(w.n_shards)]
    merged = ba.new_state(w.rows, w.head_dim)
    out = torch.empty(w.rows, w.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    flush = flush_buffer(torch)
    t_all, t_merge = Timer(torch), Timer(torch)

    def step(timed):
        e0 = t_all.start() if timed else None
        ba.shard_states(qd, blocks, states, n_kv_heads=1)
        e1 = t_merge.start() if timed else None
        ba.merge_states(states, merged)
        if timed:
            t_merge.stop(e1)
        ba.finalize(merged, out=out, lse=lse)
        if timed:
            t_all.stop(e0)

    for _ in range(warmup):
        step(False)
    for _ in range(steps):
        flush()
        step(True)
    torch.cuda.synchronize()
    ms = t_all.median_ms()
    gbs = w.sweep_bytes() / ms / 1e6
    merge_us = t_merge.median_ms() * 1e3
    log(f"shard merge: sweep {ms * 1e3:.1f} us ({gbs:.0f} GB/s), 32-way merge {merge_us:.1f} us")
    res = {"workload": w.name, "sweep_us": round(ms * 1e3, 2), "sweep_GB/s": round(gbs, 1),
           "sweep_frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "merge_us": round(merge_us, 2),
           "merge_bytes": w.merge_bytes(), "input_sha256": input_sha256((q, k, v))}
    return dict(result=res, q=q, k=k, v=v, out=out, lse=lse)


def bench_merge_scaled(torch, ba, steps, warmup, n_parts=32, rows=131072, D=128):
    """Merge kernel at a bandwidth-visible size: 32 parts x 131072 rows x D=128 fp32."""
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    parts = []
    for _ in range(n_parts):
        m = torch.randn(rows, device="cuda", generator=g) * 5
        l = torch.rand(rows, device="cuda", generator=g) + 0.5
        o = torch.randn(rows, D, device="cuda", generator=g)
        parts.append((m, l, o))
    h = hashlib.sha256()   # the bits of every part's m, l, O in order
    for t in (x for part in parts for x in part):
        h.update(t.cpu().numpy().tobytes())
    out = ba.new_state(rows, D)
    flush = flush_buffer(torch)
    for _ in range(warmup):
        ba.merge_states(parts, out)
    timer = Timer(torch)
    for _ in range(steps):
        flush()
        e0 = timer.start()
        ba.merge_states(parts, out)
        timer.stop(e0)
    torch.cuda.synchronize()
    ms = timer.median_ms()
    nbytes = (n_parts + 1) * rows * (D + 2) * 4
    gbs = nbytes / ms / 1e6
    log(f"merge scaled: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"workload": f"{n_parts}-way merge, {rows} rows, D={D}, fp32", "us": round(ms * 1e3, 2),
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "inputs": "torch CUDA generator, seed 6: per part m = 5 N(0,1), l = U(0.5, 1.5), O = N(0,1)",
            "input_sha256": {"parts_m_l_o": h.hexdigest()}}


def bench_fanout_prefill(torch, ba, H, w, steps, warmup):
    """Fan-out prefill of the private suffixes: every branch's new query rows of a
    KV head batched against each prefix chunk (one call), against the same work
    issued one branch at a time (the prefix then streams once per branch)."""
    log(f"inputs: {w.name}")
    ins = w.make_inputs()
    sha = input_sha256(ins, FANOUT_NAMES)
    q, pk, pv, sk, sv = [H.to_device(t) for t in ins]
    del ins
    nb, T, Hq, D = q.shape
    out = torch.empty(nb, T, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nb, T, Hq, dtype=torch.float32, device="cuda")
    ws = torch.empty(ba.fanout_prefill_workspace_bytes(nb, T, Hq, w.n_kv_heads, D, w.prefix_len, w.suffix_len),
                     dtype=torch.uint8, device="cuda")
    ws1 = torch.empty(ba.fanout_prefill_workspace_bytes(1, T, Hq, w.n_kv_heads, D, w.prefix_len, w.suffix_len),
                      dtype=torch.uint8, device="cuda")
    flush = flush_buffer(torch)

    def batched():
        ba.fanout_prefix_prefill(q, pk, pv, sk, sv, workspace=ws, out=out, lse=lse)

    def per_branch():
        for b in range(nb):
            ba.fanout_prefix_prefill(q[b:b + 1], pk, pv, sk[b:b + 1], sv[b:b + 1], workspace=ws1,
                                     out=out[b:b + 1], lse=lse[b:b + 1])

    res = {"workload": w.name, "algorithmic_flops": w.flops(), "algorithmic_bytes": w.bytes(), "input_sha256": sha}
    for name, fn in (("batched", batched), ("per_branch", per_branch)):
        for _ in range(warmup):
            fn()
        timer = Timer(torch)
        for _ in range(steps):
            flush()
            e0 = timer.start()
            fn()
            timer.stop(e0)
        torch.cuda.synchronize()
        ms = timer.median_ms()
        tf = w.flops() / ms / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "GB/s": round(w.bytes() / ms / 1e6, 1)}
        log(f"fanout prefill {name}: {ms * 1e3:.1f} us, {tf:.0f} TFLOP/s, {w.bytes() / ms / 1e6:.0f} GB/s")
    res["batching_speedup"] = round(res["per_branch"]["us"] / res["batched"]["us"], 3)
    res["timing"] = "median over steps, HIP events around the call(s), 1 GiB read between calls evicts the caches"
    return res


def bench_layouts(torch, ba, H, w, reps):
    """Load-balanced causal shares ("RingAttention and Context Parallelism", section 5):
    every device of an n-device causal ring emulated on this GPU, each (device, step)
    timed with HIP events.  The ring waits for its slowest device at every step, so the
    critical path is the sum over steps of the slowest device's time; efficiency is the
    busy time over n times that path."""
    from exact_blockwise_long_amd import layouts as L
    log(f"inputs: {w.name}")
    q, k, v = w.make_inputs()
    sha = input_sha256((q, k, v))
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    del q, k, v
    n = w.n_devices
    res = {"workload": w.name, "n_devices": n, "algorithmic_flops": w.flops(), "layouts": {}, "input_sha256": sha}
    for layout in L.LAYOUTS:
        calls = []
        for dev in range(n):
            c = []
            L.run_device(ba, torch, layout, qd, kd, vd, n, dev, n_kv_heads=w.n_kv_heads, calls_out=c)
            calls.append(c)
        torch.cuda.synchronize()
        times = np.zeros((reps, n, n))
        for r in range(reps):
            ev = []
            for dev in range(n):
                for t in range(n):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for tt, fn in calls[dev]:
                        if tt == t:
                            fn()
                    e1.record()
                    ev.append((dev, t, e0, e1))
            torch.cuda.synchronize()
            for dev, t, e0, e1 in ev:
                times[r, dev, t] = e0.elapsed_time(e1)
        tm = np.median(times, axis=0)            # [device, step] ms
        crit = float(tm.max(axis=0).sum())
        busy = float(tm.sum())
        per_dev = tm.sum(axis=1)
        tf = w.flops() / n / crit / 1e9
        res["layouts"][layout] = {
            "critical_path_ms": round(crit, 3), "busy_ms": round(busy, 3),
            "efficiency": round(busy / (n * crit), 4),
            "TFLOP/s_per_device": round(tf, 1),
            "device_ms_min_max": [round(float(per_dev.min()), 3), round(float(per_dev.max()), 3)]}
        log(f"layout {layout}: critical path {crit:.2f} ms, efficiency {busy / (n * crit):.3f}, "
            f"{tf:.0f} TFLOP/s per device, device totals {per_dev.min():.2f}..{per_dev.max():.2f} ms")
    res["timing"] = f"median of {reps} replays; HIP events around each (device, step) group of fwd_block calls"
    return res


def copy_calibration(torch, steps):
    """A plain device copy of 1 GiB, repeated: the known-size reference that scales
    the HBM FETCH_SIZE / WRITE_SIZE counters of the attention kernels."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"workload": "device copy of 1 GiB (torch copy_)", "bytes_read_per_copy": n * 4,
            "bytes_written_per_copy": n * 4, "copies": steps}


def gemm_reference(torch, steps, n=8192):
    """A library bf16 GEMM (torch.matmul, served by hipBLASLt) of n^3, timed
    like the headline step: the dense matrix-core rate this board sustains
    under its power limit, beside which the attention kernels' fraction of
    the nominal 2.5 PFLOP/s is read.  Not part of any step."""
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    reps = max(steps, 40)
    for _ in range(reps):  # bring the clock to its loaded state first
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / ms / 1e9
    log(f"library GEMM {n}^3 bf16: {ms:.3f} ms, {tf:.0f} TFLOP/s")
    return {"workload": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), back to back", "ms": round(ms, 4),
            "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def blas_threads():
    from threadpoolctl import threadpool_info
    return int(max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1]))


def errors(got, ref):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean())}


def lse_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(got - ref))
    return float(d.max())


def oracle_sampled(w, q, k, v, out, lse, fixed_tokens, budget_s, seed):
    """The oracle (fp64 NumPy, as it stands) on sampled query tokens of a blockwise
    workload, every query head of each: the tokens in ``fixed_tokens`` first,
    then seeded random ones, 8 at a time, until ``budget_s`` seconds of oracle
    time are spent.  Returns the oracle's rate (algorithmic FLOP of the sampled
    rows over its time), the extrapolated time of the whole block, and the
    GPU output's errors on the sampled rows."""
    from exact_blockwise_long_amd import synth
    from oracle import attention as ora

    T, Hq, D = w.q_len, w.n_q_heads, w.head_dim
    t0 = time.perf_counter()
    n_keys = min(w.kv_len, w.q_pos0 + T) if w.causal else w.kv_len   # keys past the last query are never visible
    k64 = synth.Tensor(k.storage[:n_keys], k.dtype).f64()
    v64 = synth.Tensor(v.storage[:n_keys], v.dtype).f64()
    prep_s = time.perf_counter() - t0
    g = np.random.Generator(np.random.PCG64(seed))
    rest = [t for t in g.permutation(T) if t not in set(fixed_tokens)]
    queue = list(fixed_tokens) + rest
    got = out.float().cpu().numpy().reshape(T, Hq, D)
    got_lse = lse.cpu().numpy().reshape(T, Hq)
    done, flops, err_max, err_sum, err_n, lse_max = 0, 0.0, 0.0, 0.0, 0, 0.0
    t0 = time.perf_counter()
    while done < len(queue) and (time.perf_counter() - t0 < budget_s or done < len(fixed_tokens)):
        toks = np.sort(np.asarray(queue[done:done + 8]))
        q64 = synth.Tensor(q.storage[toks], q.dtype).f64()
        a, _, _, l_ref = ora.attend(q64, k64, v64, w.scale, w.q_pos0 + toks, None, w.causal)
        vis = np.clip(w.q_pos0 + toks + 1, 0, n_keys) if w.causal else np.full(len(toks), n_keys)
        flops += 4.0 * D * Hq * float(vis.sum())
        d = np.abs(got[toks] - a)
        err_max = max(err_max, float(d.max()))
        err_sum += float(d.sum())
        err_n += d.size
        lse_max = max(lse_max, lse_errors(got_lse[toks], l_ref))
        done += len(toks)
    el = time.perf_counter() - t0
    rate = flops / el
    return {"tokens": done, "rows": done * Hq, "oracle_s": round(el, 2), "convert_s": round(prep_s, 2),
            "oracle_flops": flops, "oracle_TFLOP/s": rate / 1e12,
            "extrapolated_full_s": round(w.flops() / rate, 1),
            "errors": {"max_abs": err_max, "mean_abs": err_sum / max(err_n, 1), "lse_max_abs": lse_max}}


def cpu_baseline(w, check):
    """The line's cpu_baseline: the oracle's rate on the headline workload's sample."""
    return {"value": round(check["oracle_TFLOP/s"], 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{check['tokens']} of {w.q_len} query tokens ({check['rows']} (token, head) rows: tokens 0 "
                      f"and {w.q_len - 1}, row-tile and key-tile edges, then seeded random ones; every visible key) "
                      f"of the headline workload, fp64 NumPy, {check['oracle_s']:.1f} s; the whole block would "
                      f"take {check['extrapolated_full_s']:.0f} s at this rate (extrapolated); host has "
                      f"{os.cpu_count()} logical CPUs"}


def bench_tiny(torch, ba, H, w, steps, warmup, check):
    """The tiny fp32 workload: one fwd_block call over its 4 blocks in order
    1, 2, 3, 0, then finalize (fp32), timed with HIP events; and its errors
    against the oracle on every row (output, m, l, LSE)."""
    q, k, v = w.make_inputs()
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    L = w.block_len
    blocks = [(kd[b * L:(b + 1) * L], vd[b * L:(b + 1) * L], b * L) for b in range(w.n_blocks)]
    st = ba.new_state(w.rows, w.head_dim)
    out = torch.empty(w.rows, w.head_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.rows, dtype=torch.float32, device="cuda")

    def step():
        ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)
        ba.finalize(st, out=out, lse=lse)

    for _ in range(warmup):
        step()
    timer = Timer(torch)
    for _ in range(steps):
        e0 = timer.start()
        step()
        timer.stop(e0)
    torch.cuda.synchronize()
    us = timer.median_ms() * 1e3
    log(f"tiny exact f32: {us:.1f} us per fwd_block + finalize")
    res = {"workload": w.name, "us": round(us, 2), "step": "fwd_block (4 blocks, order 1,2,3,0) + finalize, fp32",
           "input_sha256": input_sha256((q, k, v))}
    if check:
        from oracle import attention as ora
        t0 = time.perf_counter()
        a, m, l, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), w.scale, w.q_pos0 + np.arange(w.q_len), None,
                                      w.causal)
        el = time.perf_counter() - t0
        T, Hq, D = w.q_len, w.n_q_heads, w.head_dim
        res["oracle"] = {"work": "full", "seconds": round(el, 3), "cores": blas_threads()}
        res["errors"] = {"out": errors(out.cpu().numpy().reshape(T, Hq, D), a),
                         "m_max_abs": float(np.abs(st[0].cpu().numpy().reshape(T, Hq) - m).max()),
                         "l_max_rel": float((np.abs(st[1].cpu().numpy().reshape(T, Hq) - l) / l).max()),
                         "lse_max_abs": lse_errors(lse.cpu().numpy().reshape(T, Hq), lse_ref)}
    return res


def check_fanout(w, r):
    """The fan-out decode against the oracle on every branch and head (full work)."""
    from oracle import attention as ora
    q, pk, pv, sk, sv = r["ins"]
    t0 = time.perf_counter()
    a, lse_ref = ora.fanout_decode(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), w.scale)
    el = time.perf_counter() - t0
    out = r["out"].float().cpu().numpy()
    lse = r["lse"].cpu().numpy()
    return {"oracle": {"work": "full", "seconds": round(el, 2), "cores": blas_threads()},
            "errors": dict(errors(out, a), lse_max_abs=lse_errors(lse, lse_ref))}


def check_shard_merge(w, r):
    """The sharded sweep, 32-way merge and finalize against the oracle on all 64 rows (full work)."""
    from oracle import attention as ora
    q, k, v = r["q"], r["k"], r["v"]
    t0 = time.perf_counter()
    a, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), w.scale)
    el = time.perf_counter() - t0
    nb, Hq, D = q.shape
    out = r["out"].float().cpu().numpy().reshape(nb, Hq, D)
    lse = r["lse"].cpu().numpy().reshape(nb, Hq)
    return {"oracle": {"work": "full", "seconds": round(el, 2), "cores": blas_threads()},
            "errors": dict(errors(out, a), lse_max_abs=lse_errors(lse, lse_ref))}


def strip_private(d):
    return {k: v for k, v in d.items() if not k.startswith("_")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    choices=["all", "ring_share", "causal_prefill", "tiny_exact", "fanout", "shard_merge",
                             "merge_scaled", "layouts", "fanout_prefill", "fanout_paged", "backward",
                             "copy_calibration", "gemm_reference"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing and error checks")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time on the headline workload's sample")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock sampling run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path: the ring is emulated as the K/V visit order on one device)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    from exact_blockwise_long_amd import blockattn as ba
    from exact_blockwise_long_amd import workloads as wl
    ba.load()
    H = DevIO(ba)
    log(f"device: {torch.cuda.get_device_name(0)}; HIP runtime {ba.hip_runtimes_loaded()}")
    check = not args.no_cpu

    secondary = {}
    only = args.workload
    if only not in ("all", "ring_share"):
        if only == "causal_prefill":
            r = bench_prefill(torch, ba, H, wl.CAUSAL_PREFILL, args.steps, args.warmup)
            secondary["causal_prefill"] = r["result"]
        if only == "tiny_exact":
            secondary["tiny_exact"] = bench_tiny(torch, ba, H, wl.TINY_EXACT, args.steps, args.warmup, check)
        if only == "fanout":
            secondary["fanout_decode"] = bench_fanout(torch, ba, H, wl.FANOUT_DECODE, args.steps,
                                                      args.warmup)["result"]
        if only == "shard_merge":
            secondary["shard_merge"] = bench_shard_merge(torch, ba, H, wl.SHARD_MERGE, args.steps,
                                                         args.warmup)["result"]
        if only == "merge_scaled":
            secondary["merge_scaled"] = bench_merge_scaled(torch, ba, args.steps, args.warmup)
        if only == "fanout_prefill":
            secondary["fanout_prefill"] = bench_fanout_prefill(torch, ba, H, wl.FANOUT_PREFILL, args.steps,
                                                               args.warmup)
        if only == "layouts":
            secondary["causal_ring_layouts"] = bench_layouts(torch, ba, H, wl.CAUSAL_RING_LAYOUTS,
                                                             max(1, args.steps // 10))
        if only == "fanout_paged":
            secondary["fanout_decode_paged"] = bench_fanout_paged(torch, ba, H, wl.FANOUT_DECODE, args.steps,
                                                                  args.warmup)
        if only == "backward":
            secondary["backward"] = bench_backward(torch, ba, H, wl.CAUSAL_PREFILL, args.steps, args.warmup)
        if only == "copy_calibration":
            secondary["copy_calibration"] = copy_calibration(torch, args.steps)
        if only == "gemm_reference":
            secondary["gemm_reference"] = gemm_reference(torch, args.steps)
        print(json.dumps({"metric": METRIC, "partial": only, "secondary": secondary}), flush=True)
        return

    # ---- headline: one GPU's ring share at 256K
    w = wl.RING_SHARE
    res = bench_ring_share(torch, ba, H, w, args.steps, args.warmup)
    value = res["flops"] / res["ms_step"] / 1e9
    achieved = res["flops"] / res["kernel_ms_step"] / 1e9
    cnt = counters_record("walk_kernel_ring_share") or {}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5, rounded to bf16)",
        "config": {"workload": w.name, "q_tokens": w.q_len, "q_pos0": w.q_pos0, "seq_len": w.kv_len,
                   "kv_blocks": w.n_blocks, "block_len": w.block_len, "order": w.order,
                   "calls_per_step": len(res["visible"]), "blocks_in_causal_future_no_call": res["skipped"],
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "causal": w.causal, "state": "fp32 (m, l, O) in HBM between calls",
                   "algorithmic_flops_per_step": w.flops(), "input_sha256": res["sha"]},
        "roofline": {"kernel": f"walk_kernel<128> ({len(res['visible'])} launches per step, one per visit)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": cnt.get("hbm_bytes_per_launch"),
                     "mfma_util_pct": cnt.get("mfma_util_pct"),
                     "counters_source": "profiles/traffic.json walk_kernel_ring_share (rocprofv3 --pmc, matching "
                                        "kernel sources)" if cnt else None,
                     "kernel_ms_per_step": round(res["kernel_ms_step"], 4),
                     "launch_ms_mean": round(res["launch_ms_mean"], 4),
                     "launch_ms_by_visit": [round(x, 4) for x in res["launch_ms_by_visit"]],
                     "achieved_is": "algorithmic FLOP per step / sum of the step's launch durations (HIP events)"},
    }
    if not args.no_clock:
        clk = sample_clock(torch, res["step"], 3.0)
        if clk is not None:
            peak_clk = PEAK_BF16_TFLOPS * clk["gfx_mhz_mean"] / NOMINAL_MHZ
            clk["peak_at_measured_clock"] = round(peak_clk, 1)
            clk["frac_at_measured_clock"] = round(achieved / peak_clk, 4)
            line["roofline"]["clock"] = clk
    oracle_checks = {}
    if check:
        log("oracle on a sample of the headline workload")
        fixed = [0, 31, 32, 127, 128, 8191, 8192, w.q_len - 33, w.q_len - 32, w.q_len - 1]
        chk = oracle_sampled(w, res["q"], res["k"], res["v"], res["out"], res["lse"], fixed, args.cpu_budget, 1234)
        oracle_checks["ring_share"] = chk
        line["cpu_baseline"] = cpu_baseline(w, chk)
        log(f"oracle: {chk['tokens']} tokens in {chk['oracle_s']} s, errors {chk['errors']}")
    del res

    if not args.no_secondary and only == "all":
        r = bench_prefill(torch, ba, H, wl.CAUSAL_PREFILL, args.steps, args.warmup)
        secondary["causal_prefill"] = r["result"]
        if check:
            w2 = wl.CAUSAL_PREFILL
            oracle_checks["causal_prefill"] = oracle_sampled(w2, r["q"], r["k"], r["v"], r["out"], r["lse"],
                                                             [0, 4095], 8.0, 4321)
        del r
        secondary["tiny_exact"] = bench_tiny(torch, ba, H, wl.TINY_EXACT, args.steps, args.warmup, check)
        r = bench_fanout(torch, ba, H, wl.FANOUT_DECODE, args.steps, args.warmup)
        secondary["fanout_decode"] = r["result"]
        if check:
            secondary["fanout_decode"].update(check_fanout(wl.FANOUT_DECODE, r))
        del r
        secondary["fanout_decode_paged"] = bench_fanout_paged(torch, ba, H, wl.FANOUT_DECODE, args.steps,
                                                               args.warmup)
        secondary["fanout_prefill"] = bench_fanout_prefill(torch, ba, H, wl.FANOUT_PREFILL, args.steps, args.warmup)
        r = bench_shard_merge(torch, ba, H, wl.SHARD_MERGE, args.steps, args.warmup)
        secondary["shard_merge"] = r["result"]
        if check:
            secondary["shard_merge"].update(check_shard_merge(wl.SHARD_MERGE, r))
        del r
        secondary["merge_scaled"] = bench_merge_scaled(torch, ba, args.steps, args.warmup)
        secondary["backward"] = bench_backward(torch, ba, H, wl.CAUSAL_PREFILL, args.steps, args.warmup)
        secondary["causal_ring_layouts"] = bench_layouts(torch, ba, H, wl.CAUSAL_RING_LAYOUTS, 2)
        ref = gemm_reference(torch, args.steps)
        ref["walk_kernel_vs_gemm"] = round(achieved / ref["TFLOP/s"], 4)
        secondary["gemm_reference"] = ref
    if secondary:
        line["secondary"] = secondary
    if oracle_checks:
        line["oracle_checks"] = oracle_checks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
