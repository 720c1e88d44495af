#!/usr/bin/env python3
"""Throughput of the YaRN-RoPE blockwise attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
                    [--workload all|prefill|decode|ring|copy]

One step is the whole prefill path on the Llama-7B-like 16k workload
(batch 1, 32 heads, d=128, 16384 tokens, bf16, YaRN s=4 from 4096):
  rope_tables_build (16384 rows)  ->  rope_apply (K, once)  ->
  attn_prefill_blockwise (Q rotated on load, causal, online softmax).
``value`` is algorithmic TFLOP/s of the step (4*d flop per visible
(query, key) pair, masked pairs not counted) with inputs resident in HBM.

Also measured in the same run: the sink + window decode (64 sequences x 32
heads, cache 4 + 4096, HBM GB/s), one ring device's share (8 heads, 8 key
blocks of 32768 at query block 7), and the fp64 oracle on the host cores
over a bounded sample (``cpu_baseline``).  Per-kernel durations come from
HIP events recorded on the stream the library launches on.
Prints one JSON line.

Warm-up: under sustained load the engine clock ramps up over about the
first 50 ms (the 16k attention kernel measured 2.5 ms on its first launch
and 1.67 ms from about the 25th on), so the default is 30 untimed steps; the
decode and the ring share, timed after it, take their own warm-up of about
the same length.
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
# device copy (FETCH x1.99994, WRITE x1.0).  Each figure holds only for the
# kernel sources it was taken on: the sha256 over the listed files must match,
# else the line reports traffic null.
MEASURED_TRAFFIC = {
    "attn_bf16_pp_kernel": {
        "files": ("csrc/attn_pp.hip", "csrc/attn_frag.h", "csrc/common.h"),
        "sha256": "ce8e6c36e22a7e2c76919f55ab83bb5006d79a7ef3bcad54fbf6a901c3916ea5",
        "fetch_kib": 1060865, "write_kib": 131091},
    "decode_bf16_kernel": {
        "files": ("csrc/decode.hip", "csrc/common.h"),
        "sha256": "bb86e0e7d62bfd147d1ef7163969d9f4cb27d1676997f5cb425c4230aea4a39b",
        "fetch_kib": 2108966, "write_kib": 512},
    "decode_bf16_kernel_fp8": {
        "files": ("csrc/decode.hip", "csrc/common.h"),
        "sha256": "bb86e0e7d62bfd147d1ef7163969d9f4cb27d1676997f5cb425c4230aea4a39b",
        "fetch_kib": 1060697, "write_kib": 512},
    "attn_bf16_pp_kernel_window": {
        "files": ("csrc/attn_pp.hip", "csrc/attn_frag.h", "csrc/common.h"),
        "sha256": "ce8e6c36e22a7e2c76919f55ab83bb5006d79a7ef3bcad54fbf6a901c3916ea5",
        "fetch_kib": 733819, "write_kib": 131091},
}
FETCH_FACTOR, WRITE_FACTOR = 1.99994, 1.0


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


def run_prefill(steps: int, warmup: int):
    import torch
    from yarn_rope_blockwise_amd import api
    from yarn_rope_blockwise_amd import workloads as W
    w = W.LLAMA_16K
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
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
                rope_k_ms=rope_ms, attn_ms=attn_ms, flops=flops,
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

    for _ in range(warmup):
        call()
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


def run_decode(steps: int, warmup: int):
    import torch
    from yarn_rope_blockwise_amd import api, synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.SINK_DECODE
    C = w.n_sink + w.window
    q = _upload((w.batch, w.n_q_heads, w.head_dim), 0)
    kc = _upload((w.batch, w.n_kv_heads, C, w.head_dim), 1)
    vc = _upload((w.batch, w.n_kv_heads, C, w.head_dim), 2)
    lens = torch.full((w.batch,), C, dtype=torch.int32, device="cuda")
    rh = torch.from_numpy(synth.ring_heads(w.batch, w.window)).cuda()
    tab, _, af = api.rope_tables_build(api.RopeConfig.of(w.rope), C)
    scale = af / np.sqrt(w.head_dim)
    out = torch.empty_like(q)
    for _ in range(warmup):
        api.attn_decode_sink_window(q, kc, vc, lens, w.n_sink, w.window, tab, scale, rh, out)
    torch.cuda.synchronize()
    # Back-to-back launches between two events: the host queues calls faster
    # than the GPU runs them, so no launch waits on the host (events around
    # each call would also time the host's call overhead while the GPU idles).
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        api.attn_decode_sink_window(q, kc, vc, lens, w.n_sink, w.window, tab, scale, rh, out)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    kv_bytes = 2 * kc.numel() * 2
    other = q.numel() * 2 * 2 + lens.numel() * 4 * 2
    return dict(ms=ms, bytes=kv_bytes + other, kv_bytes=kv_bytes)


def run_decode_fp8(steps: int, warmup: int):
    """The decode workload with E4M3 K/V caches and per-(sequence, head) scales."""
    import torch
    from yarn_rope_blockwise_amd import api, synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.SINK_DECODE
    C = w.n_sink + w.window
    q = _upload((w.batch, w.n_q_heads, w.head_dim), 0)
    kc = torch.from_numpy(synth.e4m3_codes((w.batch, w.n_kv_heads, C, w.head_dim), 1)).cuda()
    vc = torch.from_numpy(synth.e4m3_codes((w.batch, w.n_kv_heads, C, w.head_dim), 2)).cuda()
    ks = torch.from_numpy(synth.uniform_scales((w.batch, w.n_kv_heads), 4)).cuda()
    vs = torch.from_numpy(synth.uniform_scales((w.batch, w.n_kv_heads), 5)).cuda()
    lens = torch.full((w.batch,), C, dtype=torch.int32, device="cuda")
    rh = torch.from_numpy(synth.ring_heads(w.batch, w.window)).cuda()
    tab, _, af = api.rope_tables_build(api.RopeConfig.of(w.rope), C)
    scale = af / np.sqrt(w.head_dim)
    out = torch.empty_like(q)

    def call():
        api.attn_decode_sink_window_fp8(q, kc, vc, lens, w.n_sink, w.window, tab, scale, rh,
                                        out, k_scale=ks, v_scale=vs)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    kv_bytes = 2 * kc.numel()
    other = q.numel() * 2 * 2 + lens.numel() * 4 * 2 + ks.numel() * 4 * 2
    return dict(ms=ms, bytes=kv_bytes + other, kv_bytes=kv_bytes)


def run_interleaved(steps: int, warmup: int):
    """The interleaved pair layout: rope_apply_ex on the 16k K (268 MB moved) and the
    bf16 decode through attn_decode_sink_window_ex, each timed back to back."""
    import torch
    from yarn_rope_blockwise_amd import api, synth
    from yarn_rope_blockwise_amd import workloads as W
    w = W.LLAMA_16K
    k = _upload((w.batch, w.seq, w.n_kv_heads, w.head_dim), 1)
    tab, _, _ = api.rope_tables_build(api.RopeConfig.of(w.rope), w.seq)
    kr = torch.empty_like(k)
    for _ in range(warmup):
        api.rope_apply_ex(k, tab, layout=api.LAYOUT_INTERLEAVED, out=kr)
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        api.rope_apply_ex(k, tab, layout=api.LAYOUT_INTERLEAVED, out=kr)
    ev[1].record()
    torch.cuda.synchronize()
    rope_ms = ev[0].elapsed_time(ev[1]) / steps
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
    for _ in range(3 * warmup):
        call()
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for _ in range(steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    dec_ms = ev[0].elapsed_time(ev[1]) / steps
    dec_bytes = 2 * kc.numel() * 2 + q.numel() * 2 * 2 + lens.numel() * 4 * 2
    return dict(rope_ms=rope_ms, rope_bytes=rope_bytes, dec_ms=dec_ms, dec_bytes=dec_bytes)


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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
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
    for _ in range(warmup):
        api.rope_tables_build_factors(D, 1e4, lam, S, out=tab)
    torch.cuda.synchronize()
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


def cpu_baseline(budget_s: float = 12.0):
    """The fp64 oracle as it stands, on the 16k workload, head by head."""
    from oracle import attention as A
    from oracle import rope as R
    from yarn_rope_blockwise_amd import synth
    from yarn_rope_blockwise_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = W.LLAMA_16K
    S, D = w.seq, w.head_dim
    th = R.inv_freq(w.rope.kind, D, w.rope.base, w.rope.scale, w.rope.orig_ctx)
    sc = R.softmax_scale(w.rope.kind, w.rope.scale, D)
    done = 0
    t0 = time.perf_counter()
    while done < w.n_q_heads and time.perf_counter() - t0 < budget_s:
        qv, _ = synth.normal((1, S, 1, D), 1000 + done, "bf16")
        kv, _ = synth.normal((1, S, 1, D), 2000 + done, "bf16")
        vv, _ = synth.normal((1, S, 1, D), 3000 + done, "bf16")
        A.prefill(qv, kv, vv, th, sc)
        done += 1
    el = time.perf_counter() - t0
    flops = causal_flops(S, done, D)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {w.n_q_heads} heads of the 16k prefill (all 16384 causal rows "
                      f"each, fp64 numpy), {el:.1f} s wall incl. input generation"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip decode and ring share")
    ap.add_argument("--workload", default="all",
                    choices=["all", "prefill", "decode", "decode_fp8", "sink_window", "ring",
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

    if args.workload != "all":
        only = {"prefill": lambda: run_prefill(args.steps, args.warmup),
                "decode": lambda: run_decode(args.steps, max(3 * args.warmup, 10)),
                "decode_fp8": lambda: run_decode_fp8(args.steps, max(3 * args.warmup, 10)),
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
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("attn_bf16_pp_kernel"),
                     "kernel": "attn_bf16_pp_kernel", "kernel_ms": round(pre["attn_ms"], 4),
                     "flops_per_launch": pre["flops"]},
        "step_breakdown_ms": {"rope_tables_build": round(pre["tables_ms"], 4),
                              "rope_apply_k": round(pre["rope_k_ms"], 4),
                              "attn_prefill_blockwise": round(pre["attn_ms"], 4)},
    }
    if not args.no_extras:
        log("decode: uploading caches and timing")
        dec = run_decode(max(args.steps, 10), max(3 * args.warmup, 10))
        log(f"decode done: {dec['ms']:.3f} ms")
        gbs = dec["bytes"] / (dec["ms"] * 1e-3) / 1e9
        line["decode"] = {"workload": "sink_decode_b64_h32_4p4096", "ms": round(dec["ms"], 4),
                          "GB/s": round(gbs, 1),
                          "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(gbs / PEAK_HBM_GBS, 4),
                                       "traffic": measured_traffic("decode_bf16_kernel"),
                                       "kernel": "decode_bf16_kernel",
                                       "bytes_per_launch": dec["bytes"]}}
        log("decode, fp8 cache: uploading caches and timing")
        d8 = run_decode_fp8(max(args.steps, 10), max(3 * args.warmup, 10))
        g8 = d8["bytes"] / (d8["ms"] * 1e-3) / 1e9
        line["decode_fp8"] = {"workload": "sink_decode_b64_h32_4p4096_e4m3", "ms": round(d8["ms"], 4),
                              "GB/s": round(g8, 1),
                              "roofline": {"bound": "hbm", "achieved": round(g8, 1),
                                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                           "frac": round(g8 / PEAK_HBM_GBS, 4),
                                           "traffic": measured_traffic("decode_bf16_kernel_fp8"),
                                           "kernel": "decode_bf16_kernel<fp8>",
                                           "bytes_per_launch": d8["bytes"]}}
        il = run_interleaved(max(args.steps, 10), max(args.warmup, 10))
        line["interleaved_layout"] = {
            "rope_apply_ex_k16k": {"ms": round(il["rope_ms"], 4),
                                   "GB/s": round(il["rope_bytes"] / (il["rope_ms"] * 1e-3) / 1e9, 1)},
            "decode_ex_bf16": {"ms": round(il["dec_ms"], 4),
                               "GB/s": round(il["dec_bytes"] / (il["dec_ms"] * 1e-3) / 1e9, 1)}}
        ft = run_factor_tables(max(args.steps, 10), 10)
        line["factor_tables"] = {"workload": "rope_tables_build_factors 262144 rows x 64 pairs",
                                 "ms": round(ft["ms"], 4),
                                 "GB/s": round(ft["bytes"] / (ft["ms"] * 1e-3) / 1e9, 1)}
        sw = run_sink_window_prefill(max(args.steps, 10), args.warmup)
        line["sink_window_prefill"] = {
            "workload": "llama7b_prefill_16k_yarn4 attention, 4 sinks + 4096 window",
            "ms": round(sw["ms"], 4), "flops_per_launch": sw["flops"],
            "TFLOP/s": round(sw["flops"] / (sw["ms"] * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(sw["flops"] / (sw["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("attn_bf16_pp_kernel_window")}
        log(f"sink+window prefill done: {sw['ms']:.3f} ms")
        log("ring share: uploading blocks and timing")
        ring = run_ring(max(2, args.steps // 5), 2)
        log(f"ring share done: {ring['ms']:.3f} ms")
        line["ring_share"] = {"workload": "ring_share_h8_8x32768_yarn8_qblock7",
                              "ms": round(ring["ms"], 3),
                              "TFLOP/s": round(ring["flops"] / (ring["ms"] * 1e-3) / 1e12, 2),
                              "per_call_ms": ring["per_call_ms"]}
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
