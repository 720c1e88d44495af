"""GPU parity: prefill under the sink+window mask (attn_prefill_sink_window)
against the fp64 oracle.

Key position n is visible to query position t iff n <= t and (n < n_sink or
n > t - window), the prefill counterpart of the cache of 14cs17 "Sliding
Window + Attention Sinks".  The kernel skips the key tiles between the sinks
and a query tile's window; the cases put that gap, a partial sink tile, the
window's edge and the ragged end in several places.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api, synth
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, draw, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu


def _setup(B, S, Hq, Hkv, D, rope, seed_base):
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), S)
    qv, q = draw((B, S, Hq, D), seed_base + 0, "bf16")
    kv, k = draw((B, S, Hkv, D), seed_base + 1, "bf16")
    vv, v = draw((B, S, Hkv, D), seed_base + 2, "bf16")
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    return tab, th, scale, (qv, kv, vv), (q, k, v)


CASES = [
    # B, S, Hq, Hkv, D, n_sink, window
    (1, 1000, 4, 2, 128, 4, 200),      # gap after the sink tile from query tile 1 on
    (1, 1000, 2, 2, 128, 0, 64),       # no sinks: the walk starts at the window
    (1, 1000, 2, 1, 128, 70, 129),     # partial second sink tile, window edge mid-tile
    (2, 777, 4, 4, 64, 4, 1),          # sinks and the diagonal only
    (1, 700, 8, 2, 64, 0, 1),          # each row sees itself
    (1, 1300, 2, 2, 128, 300, 257),    # several sink tiles, then a jump
    (1, 63, 2, 2, 128, 4, 16),         # shorter than one key tile (slow loads)
    (1, 65, 2, 2, 64, 1, 2),           # one full tile and a ragged one
    (1, 600, 2, 2, 128, 5000, 10),     # every key a sink: causal
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,n_sink,window", CASES)
def test_prefill_sink_window_small(B, S, Hq, Hkv, D, n_sink, window):
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(B, S, Hq, Hkv, D, rope, 50 + S + window)
    say(f"attn_prefill_sink_window B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} sink={n_sink} win={window}")
    kr = api.rope_apply(k, tab)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = api.attn_prefill_sink_window(q, kr, v, scale, n_sink, window, cos_sin=tab, lse=lse)
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale, n_sink=n_sink, window=window)
    err = max_abs(host(o), ref)
    assert err <= BF16_TOL, err
    # log-sum-exp per row against the oracle's state
    qr = R.rotate_bshd(qv, th, np.arange(S))
    krr = R.rotate_bshd(kv, th, np.arange(S))
    vis = A.sink_window_visible(n_sink, window)
    lse_h = host(lse)
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            _, m, l = A.attention_full(qr[b, :, h], krr[b, :, g], vv[b, :, g], scale,
                                       np.arange(S), np.arange(S), vis, return_state=True)
            # A row that sees a handful of keys has a log-sum-exp set by one
            # or two logits, each off by the bf16 rounding of the rotated Q
            # (|logit| * 2^-8 or so): the bf16 bound, not the 1e-2 that a
            # long causal row averages down to.
            assert max_abs(lse_h[b, h], m + np.log(l)) <= BF16_TOL


def test_prefill_sink_window_packed_qkv_views():
    # Pre-rotated Q, K, V as views into a packed [B, S, 3, H, D] buffer
    # (strided tokens and heads), cos_sin = NULL.
    require_gpu()
    import torch
    B, S, H, D = 2, 900, 2, 128
    qkv_v, qkv = draw((B, S, 3, H, D), 78, "bf16")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    say(f"attn_prefill_sink_window packed qkv views S={S} sink=8 window=300")
    o = api.attn_prefill_sink_window(q, k, v, 0.1, 8, 300)
    torch.cuda.synchronize()
    ref = A.prefill(qkv_v[:, :, 0], qkv_v[:, :, 1], qkv_v[:, :, 2], None, 0.1, n_sink=8,
                    window=300)
    assert max_abs(host(o), ref) <= BF16_TOL


def test_prefill_sink_window_wide_window_is_causal_prefill():
    # A window of S keys reaches every earlier key: the same tiles, masks and
    # order as the causal prefill, so the same bits.
    require_gpu()
    import torch
    S, D = 1500, 128
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, _, scale, _, (q, k, v) = _setup(1, S, 4, 2, D, rope, 7)
    say(f"attn_prefill_sink_window window=S vs attn_prefill_blockwise S={S}")
    kr = api.rope_apply(k, tab)
    a = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    b = api.attn_prefill_sink_window(q, kr, v, scale, 4, S, cos_sin=tab)
    c = api.attn_prefill_sink_window(q, kr, v, scale, 0, 10 * S, cos_sin=tab)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_prefill_sink_window_full_llama16k():
    # The 16k Llama-7B-like prefill (32 heads, d=128, YaRN s=4) with 4 sinks
    # and a 4096-token window, launched as the bench times it (with a
    # workspace): 512 sampled rows of four heads against the oracle.
    require_gpu()
    import torch
    w = W.LLAMA_16K
    n_sink, window = 4, 4096
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(w.batch, w.seq, w.n_q_heads, w.n_kv_heads,
                                                     w.head_dim, w.rope, 0)
    say(f"attn_prefill_sink_window {w.name} sink={n_sink} window={window}")
    kr = api.rope_apply(k, tab)
    del k
    o = api.attn_prefill_sink_window(q, kr, v, scale, n_sink, window, cos_sin=tab,
                                     workspace=api.new_workspace())
    torch.cuda.synchronize()
    edges = [0, 3, 4, 63, 64, 255, 256, window - 1, window, window + 1, window + 63, window + 64,
             w.seq // 2, w.seq - 257, w.seq - 1]
    worst = 0.0
    for h in (0, 13, 22, 31):
        rows = synth.sample_rows(w.seq, 512, 2000 + h, must=edges)
        got = host(o[0, rows, h])
        ref = A.prefill(qv, kv, vv, th, scale, rows=rows, heads=[h], n_sink=n_sink,
                        window=window)[0, :, 0]
        worst = max(worst, max_abs(got, ref))
    assert worst <= BF16_TOL, worst


def test_prefill_sink_window_full_gqa32k():
    # The 32k GQA prefill (YaRN s=8) with 4 sinks and an 8192-token window:
    # 512 sampled rows of four query heads from different key groups.
    require_gpu()
    import torch
    w = W.GQA_32K[W.YARN]
    n_sink, window = 4, 8192
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(w.batch, w.seq, w.n_q_heads, w.n_kv_heads,
                                                     w.head_dim, w.rope, 100)
    say(f"attn_prefill_sink_window {w.name} sink={n_sink} window={window}")
    kr = api.rope_apply(k, tab)
    del k
    o = api.attn_prefill_sink_window(q, kr, v, scale, n_sink, window, cos_sin=tab)
    torch.cuda.synchronize()
    edges = [0, 5, 255, 256, window - 1, window, window + 255, window + 256, w.seq - 1]
    worst = 0.0
    for h in (0, 9, w.n_q_heads // 2 + 1, w.n_q_heads - 1):
        rows = synth.sample_rows(w.seq, 512, 3000 + h, must=edges)
        got = host(o[0, rows, h])
        ref = A.prefill(qv, kv, vv, th, scale, rows=rows, heads=[h], n_sink=n_sink,
                        window=window)[0, :, 0]
        worst = max(worst, max_abs(got, ref))
    assert worst <= BF16_TOL, worst


# ---------------------------------------------------------------------------
# attn_prefill_sink_window_chunk: one chunk of queries at an offset against
# the sequence's keys, positions kept.
# ---------------------------------------------------------------------------

CHUNK_CASES = [
    # B, Sq, Sk, q_offset, Hq, Hkv, D, n_sink, window
    (1, 300, 1000, 700, 4, 2, 128, 4, 200),      # the last chunk of a 1000-token input
    (1, 256, 768, 512, 2, 2, 128, 4, 129),       # tile-aligned chunk, keys ending with it
    (2, 100, 900, 400, 4, 4, 64, 4, 64),         # keys past the chunk (masked)
    (1, 500, 300, 200, 2, 1, 128, 70, 129),      # keys ending inside the chunk: late rows see sinks only
    (1, 64, 5000, 4900, 2, 2, 128, 300, 257),    # several sink tiles, a long gap
    (1, 1, 4097, 4096, 2, 2, 128, 4, 4096),      # one query, a window of exactly 4096
]


def _chunk_setup(B, Sq, Sk, q_offset, Hq, Hkv, D, seed):
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    n_rows = max(q_offset + Sq, Sk, 1)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), n_rows)
    qv, q = draw((B, Sq, Hq, D), seed, "bf16")
    kv, k = draw((B, Sk, Hkv, D), seed + 1, "bf16")
    vv, v = draw((B, Sk, Hkv, D), seed + 2, "bf16")
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    return tab, th, scale, (qv, kv, vv), (q, k, v)


@pytest.mark.parametrize("B,Sq,Sk,q_offset,Hq,Hkv,D,n_sink,window", CHUNK_CASES)
def test_prefill_sink_window_chunk(B, Sq, Sk, q_offset, Hq, Hkv, D, n_sink, window):
    require_gpu()
    import torch
    tab, th, scale, (qv, kv, vv), (q, k, v) = _chunk_setup(B, Sq, Sk, q_offset, Hq, Hkv, D, 60 + Sq + q_offset)
    say(f"attn_prefill_sink_window_chunk B={B} Sq={Sq} Sk={Sk} q_offset={q_offset} Hq={Hq} Hkv={Hkv} D={D} "
        f"sink={n_sink} win={window}")
    kr = api.rope_apply(k, tab)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = api.attn_prefill_sink_window_chunk(q, kr, v, scale, n_sink, window, q_offset, cos_sin=tab, lse=lse,
                                           workspace=api.new_workspace())
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale, q_offset=q_offset, n_sink=n_sink, window=window)
    assert max_abs(host(o), ref) <= BF16_TOL
    q_pos, k_pos = q_offset + np.arange(Sq), np.arange(Sk)
    qr = R.rotate_bshd(qv, th, q_pos)
    krr = R.rotate_bshd(kv, th, k_pos)
    vis = A.sink_window_visible(n_sink, window)
    lse_h = host(lse)
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            _, m, l = A.attention_full(qr[b, :, h], krr[b, :, g], vv[b, :, g], scale, q_pos, k_pos, vis,
                                       return_state=True)
            assert max_abs(lse_h[b, h], m + np.log(l)) <= BF16_TOL


def test_prefill_sink_window_chunk_without_keys():
    # Sk = 0: every row sees no key; the output is 0 and the log-sum-exp
    # -inf, with no key or value buffer at all.
    require_gpu()
    import torch
    tab, _, scale, _, (q, _, _) = _chunk_setup(1, 33, 0, 10, 2, 2, 64, 5)
    say("attn_prefill_sink_window_chunk Sk=0")
    empty = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 33), dtype=torch.float32, device="cuda")
    o = torch.full_like(q, float("nan"))
    api.attn_prefill_sink_window_chunk(q, empty, empty, scale, 4, 16, 10, cos_sin=tab, out=o, lse=lse)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(o)) == 0
    assert bool(torch.all(torch.isneginf(lse)))


def test_prefill_sink_window_in_chunks():
    # A 2000-token input prefilled in four uneven chunks, each against the
    # keys up to its own end (the key and value tensors grow as the chunks
    # arrive): every row against the oracle, and against the one-call prefill.
    require_gpu()
    import torch
    S, Hq, Hkv, D, n_sink, window = 2000, 4, 2, 128, 4, 700
    tab, th, scale, (qv, kv, vv), (q, k, v) = _chunk_setup(1, S, S, 0, Hq, Hkv, D, 321)
    kr = api.rope_apply(k, tab)
    say(f"attn_prefill_sink_window S={S} in one call and in four chunks")
    whole = api.attn_prefill_sink_window(q, kr, v, scale, n_sink, window, cos_sin=tab)
    ref = A.prefill(qv, kv, vv, th, scale, n_sink=n_sink, window=window)
    bounds = [0, 512, 1100, 1700, S]
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        o = api.attn_prefill_sink_window_chunk(q[:, c0:c1], kr[:, :c1], v[:, :c1], scale, n_sink, window, c0,
                                               cos_sin=tab)
        torch.cuda.synchronize()
        got = host(o)
        assert max_abs(got, ref[:, c0:c1]) <= BF16_TOL, (c0, c1)
        assert max_abs(got, host(whole[:, c0:c1])) <= BF16_TOL, (c0, c1)
