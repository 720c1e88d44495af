#!/usr/bin/env python3
"""Throughput of the YaRN-RoPE blockwise attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
                    [--workload all|prefill|gqa32k_{pi,ntk,yarn}|decode|decode_fp8|
                                decode_gqa|decode_gqa_fp8|sink_window|ring|copy]

One step is the whole prefill path on the Llama-7B-like 16k workload
(batch 1, 32 heads, d=128, 16384 tokens, bf16, YaRN s=4 from 4096):
  rope_tables_build (16384 rows)  ->  rope_apply (K, once)  ->
  attn_prefill_blockwise (Q rotated on load, causal, online softmax).
``value`` is algorithmic TFLOP/s of the step (4*d flop per visible
(query, key) pair, masked pairs not counted) with inputs resident in HBM.

Also measured in the same run, each with its roofline: the 32k grouped-query
prefill once per rescale method (PI, NTK-aware, YaRN at s=8), the sink +
window decode (64 sequences, cache 4 + 4096) with 32 heads and with 32 query
over 8 key/value heads, each over a bf16 and an E4M3 cache (HBM GB/s), the
interleaved pair layout, per-pair factor tables, the prefill under the
sink+window mask, one ring device's share (8 heads, 8 key blocks of 32768 at
query block 7), and the fp64 oracle on the host's cores over a bounded
sample (``cpu_baseline``).  Per-kernel durations come from HIP events
recorded on the stream the library launches on.  Prints one JSON line.

Warm-up: under sustained load the engine clock ramps up over about the
first 50 ms (the 16k attention kernel measured 2.5 ms on its first launch
and 1.67 ms from about the 25th on).  Every workload therefore runs its W
warm-up steps and then keeps warming, ten steps at a time, until at least
0.2 s of warm-up has passed; the line reports the steps that took
(``warmup_steps_run``).  The timed steps are exactly K.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "YaRN-RoPE causal prefill TFLOP/s @16k (frac bf16 peak); sink decode HBM GB/s"

# HBM bytes per launch from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE,
# KiB per dispatch), scaled by what the same counters read for a plain 1 GiB
# device copy (FETCH x1.99996, WRITE x1.0).  Each figure holds only for the
# kernel sources it was taken on: the sha256 over the listed files must match,
# else the line reports traffic null.
_PP = ("csrc/attn_pp.hip", "csrc/attn_frag.h", "csrc/common.h")
_DEC = ("csrc/decode.hip", "csrc/common.h")
MEASURED_TRAFFIC = {
    "attn_bf16_pp_kernel": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",
        "fetch_kib": 1041111, "write_kib": 131091},
    "attn_bf16_pp_kernel_gqa_prefill_32k_pi8": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",
        "fetch_kib": 1503660, "write_kib": 262182},
    "attn_bf16_pp_kernel_gqa_prefill_32k_ntk8": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",
        "fetch_kib": 1485341, "write_kib": 262182},
    "attn_bf16_pp_kernel_gqa_prefill_32k_yarn8": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",
        "fetch_kib": 1427001, "write_kib": 262182},
    "attn_bf16_pp_kernel_window": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",
        "fetch_kib": 532525, "write_kib": 131082},
    "decode_kernel": {"files": _DEC, "sha256": "0fde804d8eb30350beb5e885fc48e14b35e8afde00d371fbfbe708ecf865a16f",
        "fetch_kib": 2100179, "write_kib": 512},
    "decode_kernel_fp8": {"files": _DEC, "sha256": "0fde804d8eb30350beb5e885fc48e14b35e8afde00d371fbfbe708ecf865a16f",
        "fetch_kib": 1050510, "write_kib": 512},
    "decode_kernel_gqa": {"files": _DEC, "sha256": "0fde804d8eb30350beb5e885fc48e14b35e8afde00d371fbfbe708ecf865a16f",
        "fetch_kib": 526086, "write_kib": 1536},
    "decode_kernel_gqa_fp8": {"files": _DEC, "sha256": "0fde804d8eb30350beb5e885fc48e14b35e8afde00d371fbfbe708ecf865a16f",
        "fetch_kib": 264138, "write_kib": 2560},
    "attn_bf16_pp_kernel_ring": {"files": _PP, "sha256": "141d016353be8f28d00c408a954442f6e543fa7ac759020ac831322bee7703d8",  # per step of 8 launches
        "fetch_kib": 9391301, "write_kib": 1130850},
}
FETCH_FACTOR, WRITE_FACTOR = 1.99996, 1.0


def sources_sha256(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "yarn_rope_blockwise_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """Calibrated HBM bytes per launch, or None once the kernel has changed."""
    t = MEASURED_TRAFFIC[kernel]
    if t["sha256"] is None or sources_sha256(t["files"]) != t["sha256"]:
        return None
    return round(t["fetch_kib"] * 1024 * FETCH_FACTOR + t["write_kib"] * 1024 * WRITE_FACTOR)


def causal_flops(seq: int, heads: int, d: int, batch: int = 1) -> float:
    """4*d flop per visible (query, key) pair: QK^T and PV, 2 flop per MAC."""
    return 4.0 * d * heads * batch * seq * (seq + 1) / 2.0


def ring_flops(block: int, heads: int, d: int, full_blocks: int) -> float:
    return 4.0 * d * heads * (full_blocks * block * block + block * (block + 1) / 2.0)


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _upload(shape, seed):
    import torch
    from yarn_rope_blockwise_amd import synth
    _, bits = synth.normal(shape, seed, "bf16")
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


# The engine clock ramps up over about the first 50 ms of sustained load, so
# warm-up goes on past the W steps asked for until this much time has run.
WARMUP_MIN_S = 0.2


def warm(fn, warmup: int, min_s: float = WARMUP_MIN_S) -> int:
    """Run fn() `warmup` times, then more, in tens, until `min_s` seconds of
    warm-up have passed (synchronised).  Returns the number of calls made."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        fn()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            fn()
            n += 1
        torch.cuda.synchronize()
    return n


def run_prefill(steps: int, warmup: int, w=None):
    """One step of the prefill path on workload w (default the 16k one):
    table build, K rotation, attention with Q rotated on load."""
    import torch
    from yarn_rope_blockwise_amd import api
    from yarn_rope_blockwise_amd import workloads as W
    w = w or W.LLAMA_16K
    B, S, H, D = w.batch, w.seq, w.n_q_heads, w.head_dim
    q = _upload((B, S, H, D), 0)
    k = _upload((B, S, w.n_kv_heads, D), 1)
    v = _upload((B, S, w.n_kv_heads, D), 2)
    cfg = api.RopeConfig.of(w.rope)
    tab = torch.empty((S, D // 2, 2), dtype=torch.float32, device="cuda")
    k_rot = torch.empty_like(k)
    out = torch.empty_like(q)
    _, _, af = api.rope_tables_build(cfg, S, out=tab)
    scale = af / np.sqrt(D)
    ws = api.new_workspace()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.rope_tables_build(cfg, S, out=tab)
        if ev is not None:
            ev[1].record()
        api.rope_apply(k, tab, out=k_rot)
        if ev is not None:
            ev[2].record()
        api.attn_prefill_blockwise(q, k_rot, v, scale, cos_sin=tab, out=out, workspace=ws)
        if ev is not None:
            ev[3].record()

    n_warm = warm(step, warmup)
    evs = [_events(4) for _ in range(steps)]
    t0, t1 = _events(2)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    tab_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    rope_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    flops = causal_flops(S, H, D, B)
    return dict(total_ms=total_ms, ms_per_step=total_ms / steps, tables_ms=tab_ms,
                rope_k_ms=rope_ms, attn_ms=attn_ms, flops=flops, warmup_steps_run=n_warm,
                k_bytes=2 * k.numel() * 2 + S * D * 4)


def sink_window_pairs(seq: int, n_sink: int, window: int) -> int:
    """Visible (query, key) pairs per head under the sink+window mask."""
    t = np.arange(seq, dtype=np.int64)
    return int(np.sum(np.minimum(t + 1, window) + np.clip(t - window + 1, 0, n_sink)))


def run_sink_window_prefill(steps: int, warmup: int, n_sink: int = 4, window: int = 4096):
    """The 16k prefill's attention under 4 sinks + a 4096-token window
    (attn_prefill_sink_window), back-to-back launches, K rotated beforehand."""
    import torch
    from yarn_rope_blockwise_amd import api
    from yarn_rope_blockwise_amd import workloads as W
    w = W.LLAMA_16K
    B, S, H, D = w.batch, w.seq, w.n_q_heads, w.head_dim
    q = _upload((B, S, H, D), 0)
    k = _upload((B, S, w.n_kv_heads, D), 1)
    v = _upload((B, S, w.n_kv_heads, D), 2)
    tab, _, af = api.rope_tables_build(api.RopeConfig.of(w.rope), S)
    k_rot = api.rope_apply(k, tab)
    out = torch.empty_like(q)
    scale = af / np.sqrt(D)
    ws = api.new_workspace()

    def call():
        api.attn_prefill_sink_window(q, k_rot, v, scale, n_sink, window, cos_sin=tab, out=out,
                                     workspace=ws)

    warm(call, warmup)
    t0, t1 = _events(2)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    flops = 4.0 * D * H * B * sink_window_pairs(S, n_sink, window)
    return dict(ms=ms, flops=flops, n_sink=n_sink, window=window)


def run_gqa32k(steps: int, warmup: int, kinds=None):
    """The 32k grouped-query prefill (32 query / 8 key-value heads, base 5e5,
    s = 8 from 4096) once per rescale method (PI, NTK-aware, YaRN): the same
    inputs, each method's own tables and softmax scale; the step as for the
    16k workload (table build, K rotation, attention)."""
    from yarn_rope_blockwise_amd import workloads as W
    kinds = kinds or (W.PI, W.NTK, W.YARN)
    out = {}
    for kind in kinds:
        w = W.GQA_32K[kind]
        log(f"gqa 32k prefill, {w.name}")
        out[w.name] = run_prefill(steps, warmup, w)
    return out


def run_decode(steps: int, warmup: int, n_q_heads=None, n_kv_heads=None, fp8: bool = False):
    """The sink + window decode (64 sequences, 4 + 4096 cache), timed over
    back-to-back launches: bf16 cache through attn_decode_sink_window, or
    E4M3 codes with per-(sequence, head) scales through
    attn_decode_sink_window_fp8; head counts default to the workload's."""
    import torch
    from yarn_rope_blockwise_amd import api, synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.SINK_DECODE
    Hq = n_q_heads or w.n_q_heads
    Hkv = n_kv_heads or w.n_kv_heads
    C = w.n_sink + w.window
    q = _upload((w.batch, Hq, w.head_dim), 0)
    if fp8:
        kc = torch.from_numpy(synth.e4m3_codes((w.batch, Hkv, C, w.head_dim), 1)).cuda()
        vc = torch.from_numpy(synth.e4m3_codes((w.batch, Hkv, C, w.head_dim), 2)).cuda()
        ks = torch.from_numpy(synth.uniform_scales((w.batch, Hkv), 4)).cuda()
        vs = torch.from_numpy(synth.uniform_scales((w.batch, Hkv), 5)).cuda()
    else:
        kc = _upload((w.batch, Hkv, C, w.head_dim), 1)
        vc = _upload((w.batch, Hkv, C, w.head_dim), 2)
    lens = torch.full((w.batch,), C, dtype=torch.int32, device="cuda")
    rh = torch.from_numpy(synth.ring_heads(w.batch, w.window)).cuda()
    tab, _, af = api.rope_tables_build(api.RopeConfig.of(w.rope), C)
    scale = af / np.sqrt(w.head_dim)
    out = torch.empty_like(q)

    def call():
        if fp8:
            api.attn_decode_sink_window_fp8(q, kc, vc, lens, w.n_sink, w.window, tab, scale, rh,
                                            out, k_scale=ks, v_scale=vs)
        else:
            api.attn_decode_sink_window(q, kc, vc, lens, w.n_sink, w.window, tab, scale, rh, out)

    warm(call, warmup)
    # Back-to-back launches between two events: the host queues calls faster
    # than the GPU runs them, so no launch waits on the host (events around
    # each call would also time the host's call overhead while the GPU idles).
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    kv_bytes = 2 * kc.numel() * kc.element_size()
    other = q.numel() * 2 * 2 + lens.numel() * 4 * 2 + (2 * w.batch * Hkv * 4 if fp8 else 0)
    return dict(ms=ms, bytes=kv_bytes + other, kv_bytes=kv_bytes)


def run_interleaved(steps: int, warmup: int):
    """The interleaved pair layout: rope_apply_ex on the 16k K (268 MB moved) and the
    bf16 decode through attn_decode_sink_window_ex, each timed back to back; the
    half-split rope_apply on the same K, timed the same way."""
    import torch
    from yarn_rope_blockwise_amd import api, synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.LLAMA_16K
    k = _upload((w.batch, w.seq, w.n_kv_heads, w.head_dim), 1)
    tab, _, _ = api.rope_tables_build(api.RopeConfig.of(w.rope), w.seq)
    kr = torch.empty_like(k)

    def back_to_back(fn):
        warm(fn, warmup)
        ev = _events(2)
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    rope_ms = back_to_back(lambda: api.rope_apply_ex(k, tab, layout=api.LAYOUT_INTERLEAVED, out=kr))
    # the half-split pass timed the same way (in the prefill step it is one
    # launch between two others)
    rope_half_ms = back_to_back(lambda: api.rope_apply(k, tab, out=kr))
    rope_bytes = 2 * k.numel() * 2 + w.seq * w.head_dim * 4
    del k, kr
    d = W.SINK_DECODE
    C = d.n_sink + d.window
    q = _upload((d.batch, d.n_q_heads, d.head_dim), 0)
    kc = _upload((d.batch, d.n_kv_heads, C, d.head_dim), 1)
    vc = _upload((d.batch, d.n_kv_heads, C, d.head_dim), 2)
    lens = torch.full((d.batch,), C, dtype=torch.int32, device="cuda")
    rh = torch.from_numpy(synth.ring_heads(d.batch, d.window)).cuda()
    dtab, _, af = api.rope_tables_build(api.RopeConfig.of(d.rope), C)
    out = torch.empty_like(q)

    def call():
        api.attn_decode_sink_window_ex(q, kc, vc, lens, d.n_sink, d.window, dtab,
                                       af / np.sqrt(d.head_dim), layout=api.LAYOUT_INTERLEAVED,
                                       ring_head=rh, out=out)
    warm(call, 3 * warmup)
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    dec_ms = ev[0].elapsed_time(ev[1]) / steps
    dec_bytes = 2 * kc.numel() * 2 + q.numel() * 2 * 2 + lens.numel() * 4 * 2
    return dict(rope_ms=rope_ms, rope_half_ms=rope_half_ms, rope_bytes=rope_bytes, dec_ms=dec_ms,
                dec_bytes=dec_bytes)


def run_ring(steps: int, warmup: int):
    import torch
    from yarn_rope_blockwise_amd import api
    from yarn_rope_blockwise_amd import workloads as W
    w = W.RING_SHARE
    blk, nb, H, D = w.block, w.n_blocks, w.n_q_heads, w.head_dim
    S = blk * nb
    q = _upload((1, blk, H, D), 0)
    k = _upload((1, S, w.n_kv_heads, D), 1)
    v = _upload((1, S, w.n_kv_heads, D), 2)
    tab, _, af = api.rope_tables_build(api.RopeConfig.of(w.rope), S)
    scale = af / np.sqrt(D)
    k_raw = k
    k = api.rope_apply(k_raw, tab)          # every block is rotated once by its owner
    st = api.AccState.empty(1, blk, H, D)
    out = torch.empty_like(q)
    ws = api.new_workspace()
    order = W.ring_order(w)
    qi = w.q_block_index
    qoff = qi * blk
    own = slice(qi * blk, (qi + 1) * blk)

    def step(ev=None):
        # this device rotates its own key block once per pass; the other
        # blocks arrive already rotated by their owners
        if ev is not None:
            ev[0].record()
        api.rope_apply(k_raw[:, own], tab, pos_offset=qoff, out=k[:, own])
        for t, j in enumerate(order):
            if ev is not None:
                ev[t + 1].record()
            api.attn_block_accumulate(q, k[:, j * blk:(j + 1) * blk], v[:, j * blk:(j + 1) * blk],
                                      st, qoff, j * blk, scale, cos_sin=tab, first=(t == 0),
                                      finalize=(t == nb - 1), out=out, workspace=ws)
        if ev is not None:
            ev[nb + 1].record()

    warm(step, warmup)
    evs = [_events(nb + 2) for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    per_call = np.array([[e[t + 1].elapsed_time(e[t + 2]) for t in range(nb)] for e in evs]).mean(0)
    total = float(np.mean([e[0].elapsed_time(e[nb + 1]) for e in evs]))
    full = sum(1 for j in order if j < w.q_block_index)
    return dict(ms=total, per_call_ms=[round(float(x), 4) for x in per_call],
                flops=ring_flops(blk, H, D, full))


def run_factor_tables(steps: int, warmup: int):
    """Tables from a per-pair factor vector, 262144 rows x 64 pairs (the ring share's
    table size, 128 MiB), timed back to back; smaller tables time the host's call."""
    import torch
    from yarn_rope_blockwise_amd import api
    S, D = 262144, 128
    lam = np.sort(np.random.default_rng(7).uniform(1.0, 64.0, D // 2))
    tab = torch.empty((S, D // 2, 2), dtype=torch.float32, device="cuda")
    warm(lambda: api.rope_tables_build_factors(D, 1e4, lam, S, out=tab), warmup)
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        api.rope_tables_build_factors(D, 1e4, lam, S, out=tab)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    return dict(ms=ms, bytes=tab.numel() * 4)


def run_copy(steps: int):
    """A plain 1 GiB device-to-device copy: the reference for HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "launches": steps}


def _oracle_head(head: int, ready, go, results):
    """One process of the CPU baseline: draw one head of the 16k prefill's
    shape (seeded by head), wait at the barrier, run the fp64 oracle on it."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - the env vars already ask for one thread
        pass
    from oracle import attention as A
    from oracle import rope as R
    from yarn_rope_blockwise_amd import synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.LLAMA_16K
    S, D = w.seq, w.head_dim
    th = R.inv_freq(w.rope.kind, D, w.rope.base, w.rope.scale, w.rope.orig_ctx)
    sc = R.softmax_scale(w.rope.kind, w.rope.scale, D)
    qv, _ = synth.normal((1, S, 1, D), 1000 + head, "bf16")
    kv, _ = synth.normal((1, S, 1, D), 2000 + head, "bf16")
    vv, _ = synth.normal((1, S, 1, D), 3000 + head, "bf16")
    ready.wait()
    go.wait()
    t0 = time.perf_counter()
    A.prefill(qv, kv, vv, th, sc)
    results.put((head, time.perf_counter() - t0))


def cpu_baseline(max_procs: int = 32):
    """The fp64 oracle as it stands, on the 16k prefill's shape: one process
    per core this process may run on (os.sched_getaffinity), each with BLAS
    on one thread and one whole head (all 16384 causal rows, its own seeded
    inputs, drawn before the clock starts).  The clock runs from the
    barrier that releases every process to the last result."""
    import multiprocessing as mp
    from yarn_rope_blockwise_amd import workloads as W
    n = max(1, min(len(os.sched_getaffinity(0)), max_procs, W.LLAMA_16K.n_q_heads))
    ctx = mp.get_context("spawn")            # fresh interpreters: no GPU state inherited
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    ready, go = ctx.Barrier(n + 1), ctx.Barrier(n + 1)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_head, args=(h, ready, go, results)) for h in range(n)]
    try:
        for p_ in procs:
            p_.start()
        ready.wait()                          # every process has its inputs
        go.wait()
        t0 = time.perf_counter()
        per = [results.get() for _ in range(n)]
        wall = time.perf_counter() - t0
        for p_ in procs:
            p_.join()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    w = W.LLAMA_16K
    flops = causal_flops(w.seq, n, w.head_dim)
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": n,
            "kind": "oracle",
            "sample": f"{n} of {w.n_q_heads} heads of the 16k prefill shape (all 16384 causal "
                      f"rows each, fp64 numpy, own seeded inputs), one process per core with "
                      f"BLAS on 1 thread; {wall:.1f} s wall from the start barrier, "
                      f"slowest head {max(t for _, t in per):.1f} s"}


def roofline(bound, achieved, peak, unit, kernel, traffic_key=None, **per_launch):
    d = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4),
         "traffic": measured_traffic(traffic_key) if traffic_key else None, "kernel": kernel}
    d.update(per_launch)
    return d


def decode_entry(name, d, kernel, traffic_key):
    gbs = d["bytes"] / (d["ms"] * 1e-3) / 1e9
    return {"workload": name, "ms": round(d["ms"], 4), "GB/s": round(gbs, 1),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", kernel, traffic_key,
                                 bytes_per_launch=d["bytes"])}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip everything but the 16k step")
    ap.add_argument("--workload", default="all",
                    choices=["all", "prefill", "gqa32k_pi", "gqa32k_ntk", "gqa32k_yarn", "decode",
                             "decode_fp8", "decode_gqa", "decode_gqa_fp8", "sink_window", "ring",
                             "copy"],
                    help="run one workload alone (for profiling); the JSON line needs 'all'")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from yarn_rope_blockwise_amd import workloads as W

    dec_warm = max(3 * args.warmup, 10)
    if args.workload != "all":
        gqa = lambda k: run_prefill(args.steps, args.warmup, W.GQA_32K[k])  # noqa: E731
        only = {"prefill": lambda: run_prefill(args.steps, args.warmup),
                "gqa32k_pi": lambda: gqa(W.PI), "gqa32k_ntk": lambda: gqa(W.NTK),
                "gqa32k_yarn": lambda: gqa(W.YARN),
                "decode": lambda: run_decode(args.steps, dec_warm),
                "decode_fp8": lambda: run_decode(args.steps, dec_warm, fp8=True),
                "decode_gqa": lambda: run_decode(args.steps, dec_warm, 32, 8),
                "decode_gqa_fp8": lambda: run_decode(args.steps, dec_warm, 32, 8, fp8=True),
                "sink_window": lambda: run_sink_window_prefill(args.steps, args.warmup),
                "ring": lambda: run_ring(args.steps, 2),
                "copy": lambda: run_copy(args.steps)}[args.workload]()
        only.pop("per_call_ms", None)
        print(json.dumps({"workload": args.workload, **{k: v for k, v in only.items()}}))
        return

    log("prefill 16k: uploading inputs and timing")
    pre = run_prefill(args.steps, args.warmup)
    log(f"prefill done: {pre['ms_per_step']:.3f} ms/step, attention {pre['attn_ms']:.3f} ms")
    value = pre["flops"] / (pre["ms_per_step"] * 1e-3) / 1e12
    attn_tflops = pre["flops"] / (pre["attn_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": pre["warmup_steps_run"],
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b_prefill_16k_yarn4", "batch": 1, "seq": 16384,
                   "q_heads": 32, "kv_heads": 32, "head_dim": 128, "causal": True,
                   "rope": "yarn s=4 (4096->16384), base 1e4, alpha 1, beta 32",
                   "step": "rope_tables_build + rope_apply(K) + attn_prefill_blockwise"},
        "roofline": roofline("mfma", attn_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", "attn_bf16_pp_kernel",
                             "attn_bf16_pp_kernel", kernel_ms=round(pre["attn_ms"], 4),
                             flops_per_launch=pre["flops"]),
        "step_breakdown_ms": {"rope_tables_build": round(pre["tables_ms"], 4),
                              "rope_apply_k": round(pre["rope_k_ms"], 4),
                              "attn_prefill_blockwise": round(pre["attn_ms"], 4)},
    }
    if not args.no_extras:
        gq = run_gqa32k(max(args.steps // 2, 5), args.warmup)
        line["gqa_prefill_32k"] = {}
        for name, r in gq.items():
            k_tf = r["flops"] / (r["attn_ms"] * 1e-3) / 1e12
            line["gqa_prefill_32k"][name] = {
                "ms_per_step": round(r["ms_per_step"], 4),
                "TFLOP/s": round(r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12, 2),
                "roofline": roofline("mfma", k_tf, PEAK_BF16_TFLOPS, "TFLOP/s", "attn_bf16_pp_kernel",
                                     "attn_bf16_pp_kernel_" + name, kernel_ms=round(r["attn_ms"], 4),
                                     flops_per_launch=r["flops"])}
        log("decode: uploading caches and timing")
        steps_d = max(args.steps, 10)
        line["decode"] = decode_entry("sink_decode_b64_h32_4p4096", run_decode(steps_d, dec_warm),
                                      "decode_kernel", "decode_kernel")
        line["decode_fp8"] = decode_entry("sink_decode_b64_h32_4p4096_e4m3",
                                          run_decode(steps_d, dec_warm, fp8=True),
                                          "decode_kernel<fp8>", "decode_kernel_fp8")
        line["decode_gqa"] = decode_entry("sink_decode_b64_q32_kv8_4p4096",
                                          run_decode(steps_d, dec_warm, 32, 8),
                                          "decode_kernel<G=4>", "decode_kernel_gqa")
        line["decode_gqa_fp8"] = decode_entry("sink_decode_b64_q32_kv8_4p4096_e4m3",
                                              run_decode(steps_d, dec_warm, 32, 8, fp8=True),
                                              "decode_kernel<G=4, fp8>", "decode_kernel_gqa_fp8")
        log(f"decode done: {line['decode']['ms']:.3f} ms, gqa {line['decode_gqa']['ms']:.3f} ms")
        il = run_interleaved(steps_d, max(args.warmup, 10))
        line["interleaved_layout"] = {
            "rope_apply_ex_k16k": {"ms": round(il["rope_ms"], 4),
                                   "GB/s": round(il["rope_bytes"] / (il["rope_ms"] * 1e-3) / 1e9, 1)},
            "rope_apply_k16k_half_split": {"ms": round(il["rope_half_ms"], 4),
                                           "GB/s": round(il["rope_bytes"] / (il["rope_half_ms"] * 1e-3) / 1e9, 1)},
            "decode_ex_bf16": {"ms": round(il["dec_ms"], 4),
                               "GB/s": round(il["dec_bytes"] / (il["dec_ms"] * 1e-3) / 1e9, 1)}}
        ft = run_factor_tables(steps_d, 10)
        line["factor_tables"] = {"workload": "rope_tables_build_factors 262144 rows x 64 pairs",
                                 "ms": round(ft["ms"], 4),
                                 "GB/s": round(ft["bytes"] / (ft["ms"] * 1e-3) / 1e9, 1)}
        sw = run_sink_window_prefill(steps_d, args.warmup)
        sw_tf = sw["flops"] / (sw["ms"] * 1e-3) / 1e12
        line["sink_window_prefill"] = {
            "workload": "llama7b_prefill_16k_yarn4 attention, 4 sinks + 4096 window",
            "ms": round(sw["ms"], 4), "TFLOP/s": round(sw_tf, 2),
            "roofline": roofline("mfma", sw_tf, PEAK_BF16_TFLOPS, "TFLOP/s", "attn_bf16_pp_kernel<window>",
                                 "attn_bf16_pp_kernel_window", flops_per_launch=sw["flops"])}
        log(f"sink+window prefill done: {sw['ms']:.3f} ms")
        log("ring share: uploading blocks and timing")
        ring = run_ring(max(2, args.steps // 5), 2)
        log(f"ring share done: {ring['ms']:.3f} ms")
        ring_kernel_ms = float(sum(ring["per_call_ms"]))
        ring_tf = ring["flops"] / (ring_kernel_ms * 1e-3) / 1e12
        line["ring_share"] = {"workload": "ring_share_h8_8x32768_yarn8_qblock7",
                              "ms": round(ring["ms"], 3),
                              "TFLOP/s": round(ring["flops"] / (ring["ms"] * 1e-3) / 1e12, 2),
                              "per_call_ms": ring["per_call_ms"],
                              # the 8 accumulate launches of a step (the step also rotates the own block)
                              "roofline": roofline("mfma", ring_tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                                   "attn_bf16_pp_kernel<exact> x 8", "attn_bf16_pp_kernel_ring",
                                                   flops_per_step=ring["flops"], traffic_per="step of 8 launches")}
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample, one process per core")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
