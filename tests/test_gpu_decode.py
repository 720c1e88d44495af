"""GPU parity: attention-sink + sliding-window decode against the fp64 oracle."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api, synth
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, dev_tensor, draw, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, n_sink, window, lens, ring_heads, rope, seed=0):
    import torch
    C = n_sink + window
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), C)
    qv, q = draw((B, Hq, D), seed + 0, "bf16")
    kv, k = draw((B, Hkv, C, D), seed + 1, "bf16")
    vv, v = draw((B, Hkv, C, D), seed + 2, "bf16")
    lens_t = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    rh_t = None if ring_heads is None else torch.tensor(np.asarray(ring_heads, np.int32),
                                                         device="cuda")
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    return tab, th, scale, (qv, kv, vv), (q, k, v), lens_t, rh_t


def test_decode_full_sink_config():
    # 64 sequences x 32 heads, d=128, 4 sinks + 4096 window (cache full),
    # ring heads seeded, plain RoPE.
    require_gpu()
    import torch
    w = W.SINK_DECODE
    C = w.n_sink + w.window
    rh = synth.ring_heads(w.batch, w.window)
    tab, th, scale, (qv, kv, vv), (q, k, v), lens, rht = _case(
        w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.window, [C] * w.batch, rh,
        w.rope)
    say("attn_decode_sink_window B=64 H=32 C=4100 full size")
    o = api.attn_decode_sink_window(q, k, v, lens, w.n_sink, w.window, tab, scale, ring_head=rht)
    torch.cuda.synchronize()
    got = host(o)
    ref = A.decode_sink_window(qv, kv, vv, th, scale, w.n_sink, w.window, [C] * w.batch, rh)
    err = max_abs(got, ref)
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("cache", ["bf16", "e4m3"])
def test_decode_full_gqa_config(cache):
    # The decode workload with grouped-query heads: 64 sequences x 32 query
    # heads over 8 key/value heads (4 per group), 4 sinks + 4096 window, every
    # sequence checked.
    require_gpu()
    import torch
    w = W.SINK_DECODE
    C = w.n_sink + w.window
    Hq, Hkv = 32, 8
    rh = synth.ring_heads(w.batch, w.window, seed_base=10)
    if cache == "bf16":
        tab, th, scale, (qv, kv, vv), (q, k, v), lens, rht = _case(
            w.batch, Hq, Hkv, w.head_dim, w.n_sink, w.window, [C] * w.batch, rh, w.rope, seed=20)
        ks = vs = None
    else:
        tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(
            w.batch, Hq, Hkv, w.head_dim, w.n_sink, w.window, [C] * w.batch, rh, w.rope, seed=24)
        k, v, ks, vs, lens, rht = dv["k"], dv["v"], dv["ks"], dv["vs"], dv["lens"], dv["rh"]
    say(f"attn_decode_sink_window_ex {cache} B=64 Hq=32 Hkv=8 C=4100 full size")
    o = api.attn_decode_sink_window_ex(q, k, v, lens, w.n_sink, w.window, tab, scale,
                                       ring_head=rht, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ref = A.decode_sink_window(qv, kv, vv, th, scale, w.n_sink, w.window, [C] * w.batch, rh)
    err = max_abs(host(o), ref)
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_edge_cases(G, D):
    # len 0, len inside the sinks, a partly filled window, a full window with
    # ring heads at 0 / middle / last slot, and invalid len / ring head.
    require_gpu()
    import torch
    n_sink, window = 4, 300
    C = n_sink + window
    lens = [0, 1, 3, 4, 5, 150, C, C, C, C + 1, C]
    heads = [0, 0, 0, 0, 0, 7, 0, 123, window - 1, 0, window]
    B = len(lens)
    Hkv = 2
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v), lens_t, rh_t = _case(
        B, Hkv * G, Hkv, D, n_sink, window, lens, heads, rope, seed=40 + G + D)
    say(f"attn_decode_sink_window edge cases G={G} D={D}")
    o = api.attn_decode_sink_window(q, k, v, lens_t, n_sink, window, tab, scale, ring_head=rh_t)
    torch.cuda.synchronize()
    got = host(o)
    for b in range(B):
        bad = lens[b] < 0 or lens[b] > C or heads[b] < 0 or heads[b] >= window
        if bad:
            assert np.isnan(got[b]).all(), b
            continue
        ref = A.decode_sink_window(qv[b:b + 1], kv[b:b + 1], vv[b:b + 1], th, scale, n_sink,
                                   window, [lens[b]], [heads[b]])
        if lens[b] == 0:
            assert np.all(got[b] == 0)
        assert max_abs(got[b], ref[0]) <= BF16_TOL, b


def test_decode_streaming_equals_masked_attention():
    # Tokens streamed through the cache (sinks kept, window evicting) give
    # the masked attention over the logical sequence with re-indexed positions.
    require_gpu()
    import torch
    n_sink, window, H, D, T = 4, 100, 4, 128, 357
    C = n_sink + window
    rope = W.Rope(W.PLAIN, D)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), C)
    kseq, _ = synth.normal((T, H, D), 91, "bf16")
    vseq, _ = synth.normal((T, H, D), 92, "bf16")
    qv, q = draw((1, H, D), 93, "bf16")
    kc = np.zeros((1, H, C, D), np.float32)
    vc = np.zeros((1, H, C, D), np.float32)
    for t in range(T):
        slot = t if t < n_sink else n_sink + (t - n_sink) % window
        kc[0, :, slot] = kseq[t]
        vc[0, :, slot] = vseq[t]
    rh = (T - n_sink) % window
    kdev = torch.from_numpy(synth.bf16_bits_from_f32(kc).view(np.int16)).view(torch.bfloat16).cuda()
    vdev = torch.from_numpy(synth.bf16_bits_from_f32(vc).view(np.int16)).view(torch.bfloat16).cuda()
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    say("attn_decode_sink_window streamed T=357")
    o = api.attn_decode_sink_window(q, kdev, vdev, torch.tensor([C], dtype=torch.int32,
                                                                 device="cuda"),
                                    n_sink, window, tab, scale,
                                    ring_head=torch.tensor([rh], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    kept = np.r_[0:n_sink, T - window:T]
    pos = np.arange(len(kept))
    ck, sk = R.tables(th, pos)
    cq, sq = R.tables(th, [len(kept) - 1])
    ref = np.zeros((H, D))
    for h in range(H):
        kk = R.rotate_half(kseq[kept, h].astype(np.float64), ck, sk)
        qq = R.rotate_half(qv[0, h][None].astype(np.float64), cq, sq)
        ref[h] = A.attention_full(qq, kk, vseq[kept, h], scale, np.array([len(kept) - 1]), pos,
                                  A.all_visible)[0]
    assert max_abs(host(o[0]), ref) <= BF16_TOL


# ---------------------------------------------------------------------------
# attn_decode_sink_window_fp8: E4M3 K/V caches with per-(sequence, head) scales
# ---------------------------------------------------------------------------

def _fp8_case(B, Hq, Hkv, D, n_sink, window, lens, ring_heads, rope, seed=0, scales=True):
    import torch
    from oracle import fp8
    C = n_sink + window
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), C)
    qv, q = draw((B, Hq, D), seed + 0, "bf16")
    kc = synth.e4m3_codes((B, Hkv, C, D), seed + 1)
    vc = synth.e4m3_codes((B, Hkv, C, D), seed + 2)
    ks = synth.uniform_scales((B, Hkv), seed + 4) if scales else np.ones((B, Hkv), np.float32)
    vs = synth.uniform_scales((B, Hkv), seed + 5) if scales else np.ones((B, Hkv), np.float32)
    kv = fp8.e4m3_decode(kc) * ks.astype(np.float64)[:, :, None, None]
    vv = fp8.e4m3_decode(vc) * vs.astype(np.float64)[:, :, None, None]
    dev = dict(k=torch.from_numpy(kc).cuda(), v=torch.from_numpy(vc).cuda(),
               ks=torch.from_numpy(ks).cuda() if scales else None,
               vs=torch.from_numpy(vs).cuda() if scales else None,
               lens=torch.tensor(np.asarray(lens, np.int32), device="cuda"),
               rh=None if ring_heads is None else torch.tensor(np.asarray(ring_heads, np.int32),
                                                               device="cuda"))
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    return tab, th, scale, (qv, kv, vv), q, dev


def test_decode_fp8_full_sink_config():
    # The 64 x 32 x (4 + 4096) decode with the cache in E4M3 (half the bytes).
    require_gpu()
    import torch
    w = W.SINK_DECODE
    C = w.n_sink + w.window
    rh = synth.ring_heads(w.batch, w.window)
    tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(
        w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sink, w.window, [C] * w.batch, rh,
        w.rope, seed=70)
    say("attn_decode_sink_window_fp8 B=64 H=32 C=4100 full size")
    o = api.attn_decode_sink_window_fp8(q, dv["k"], dv["v"], dv["lens"], w.n_sink, w.window, tab,
                                        scale, ring_head=dv["rh"], k_scale=dv["ks"],
                                        v_scale=dv["vs"])
    torch.cuda.synchronize()
    got = host(o)
    ref = A.decode_sink_window(qv, kv, vv, th, scale, w.n_sink, w.window, [C] * w.batch, rh)
    err = max_abs(got, ref)
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_fp8_edge_cases(G, D):
    # The same lengths and ring heads as the bf16 edge cases, every sequence
    # checked; no scales given (1).
    require_gpu()
    import torch
    n_sink, window = 4, 300
    C = n_sink + window
    lens = [0, 1, 3, 4, 5, 150, C, C, C, C + 1, C]
    heads = [0, 0, 0, 0, 0, 7, 0, 123, window - 1, 0, window]
    B, Hkv = len(lens), 2
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(B, Hkv * G, Hkv, D, n_sink, window, lens,
                                                    heads, rope, seed=80 + G + D, scales=False)
    say(f"attn_decode_sink_window_fp8 edge cases G={G} D={D}")
    o = api.attn_decode_sink_window_fp8(q, dv["k"], dv["v"], dv["lens"], n_sink, window, tab,
                                        scale, ring_head=dv["rh"])
    torch.cuda.synchronize()
    got = host(o)
    for b in range(B):
        if lens[b] < 0 or lens[b] > C or heads[b] < 0 or heads[b] >= window:
            assert np.isnan(got[b]).all(), b
            continue
        ref = A.decode_sink_window(qv[b:b + 1], kv[b:b + 1], vv[b:b + 1], th, scale, n_sink,
                                   window, [lens[b]], [heads[b]])
        if lens[b] == 0:
            assert np.all(got[b] == 0)
        assert max_abs(got[b], ref[0]) <= BF16_TOL, b


def test_decode_fp8_nan_code_reaches_output():
    # A NaN code in a visible value row makes that head's output NaN; the
    # other heads of the sequence are untouched.
    require_gpu()
    import torch
    n_sink, window, D = 4, 60, 128
    C = n_sink + window
    rope = W.Rope(W.PLAIN, D, 1e4, 1.0, 4096)
    tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(1, 2, 2, D, n_sink, window, [C], None, rope,
                                                    seed=90)
    dv["v"][0, 1, 10, 5] = 0x7F
    say("attn_decode_sink_window_fp8 NaN code")
    o = api.attn_decode_sink_window_fp8(q, dv["k"], dv["v"], dv["lens"], n_sink, window, tab,
                                        scale, k_scale=dv["ks"], v_scale=dv["vs"])
    torch.cuda.synchronize()
    got = host(o)
    assert np.isnan(got[0, 1, 5]) and not np.isnan(got[0, 0]).any()


def test_decode_fp8_nan_key_code_reaches_output():
    # A NaN code in a visible key row makes that head's logit, and so its
    # whole output, NaN; the other head is untouched.
    require_gpu()
    import torch
    n_sink, window, D = 4, 60, 128
    C = n_sink + window
    rope = W.Rope(W.PLAIN, D, 1e4, 1.0, 4096)
    tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(1, 2, 2, D, n_sink, window, [C], None, rope,
                                                    seed=91)
    dv["k"][0, 1, 10, 5] = 0xFF
    say("attn_decode_sink_window_fp8 NaN key code")
    o = api.attn_decode_sink_window_fp8(q, dv["k"], dv["v"], dv["lens"], n_sink, window, tab,
                                        scale, k_scale=dv["ks"], v_scale=dv["vs"])
    torch.cuda.synchronize()
    got = host(o)
    assert np.isnan(got[0, 1]).all() and not np.isnan(got[0, 0]).any()


@pytest.mark.parametrize("G,D,IL", [(1, 128, False), (1, 64, False), (2, 128, True), (4, 128, False),
                                    (8, 64, True)])
def test_decode_fp8_every_code(G, D, IL):
    # Every non-NaN E4M3 code, subnormals and the largest included: each of
    # the 16 (sequence, key head) pairs draws its K and V codes from one
    # exponent field, with scales that bring its values to about 0.5 .. 0.94,
    # so every field is decoded at full relative weight; the queries are
    # multiplied by 8 (exact) so that the softmax is peaked and the output
    # follows the logits closely.
    require_gpu()
    import torch
    from oracle import fp8
    B, Hkv, n_sink, window = 2, 8, 4, 300
    Hq, C = Hkv * G, n_sink + window
    fields = np.arange(16).reshape(B, Hkv)
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), C)
    qv0, _ = draw((B, Hq, D), 95, "bf16")
    qv = qv0 * 8.0
    q = dev_tensor(qv, synth.bf16_bits_from_f32(qv.astype(np.float32)), "bf16")
    kc = synth.e4m3_codes_banded((B, Hkv, C, D), 96, fields)
    vc = synth.e4m3_codes_banded((B, Hkv, C, D), 97, fields[::-1])
    band = lambda f: (2.0 ** (7 - np.maximum(f, 1)) * 0.5).astype(np.float32)
    ks, vs = band(fields), band(fields[::-1])
    kv = fp8.e4m3_decode(kc) * ks.astype(np.float64)[:, :, None, None]
    vv = fp8.e4m3_decode(vc) * vs.astype(np.float64)[:, :, None, None]
    rh = np.array([17, window - 1], np.int32)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    say(f"attn_decode_sink_window_ex fp8 every code G={G} D={D} IL={IL}")
    o = api.attn_decode_sink_window_ex(
        q, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
        torch.tensor([C, C], dtype=torch.int32, device="cuda"), n_sink, window, tab, scale,
        ring_head=torch.from_numpy(rh).cuda(), k_scale=torch.from_numpy(ks).cuda(),
        v_scale=torch.from_numpy(vs).cuda(),
        layout=api.LAYOUT_INTERLEAVED if IL else api.LAYOUT_HALF)
    torch.cuda.synchronize()
    got = host(o)
    ref = A.decode_sink_window(qv, kv, vv, th, scale, n_sink, window, [C, C], rh,
                               layout="interleaved" if IL else "half")
    err = max_abs(got, ref)
    assert err <= BF16_TOL, err


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_offsets_at_the_top_of_32_bits(fp8):
    # One (sequence, head)'s cache spread out with an entry stride that puts
    # its last entry's bytes just under 2^32: the kernel's lane offsets (a
    # 24-bit product of entry and stride, plus the chunk) reach the top of
    # their 32-bit range, as far as the host's checks allow.
    require_gpu()
    import torch
    from oracle import fp8 as F
    n_sink, window, D = 4, 2044, 128
    C = n_sink + window
    esz, align = (1, 16) if fp8 else (2, 8)
    stride = ((2 ** 32 - 1 - D * esz) // ((C - 1) * esz)) // align * align
    span = (C - 1) * stride + D
    assert stride * esz < 2 ** 24 and span * esz <= 2 ** 32 - 1 and span * esz > 2 ** 32 - 4096
    rope = W.Rope(W.PLAIN, D, 1e4, 1.0, 4096)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), C)
    qv, q = draw((1, 1, D), 120, "bf16")
    rh = np.array([777], np.int32)
    if fp8:
        kc = synth.e4m3_codes((1, 1, C, D), 121)
        vc = synth.e4m3_codes((1, 1, C, D), 122)
        kv, vv = F.e4m3_decode(kc), F.e4m3_decode(vc)
        small_k, small_v = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
        dt = torch.uint8
    else:
        kv, small_k = draw((1, 1, C, D), 121, "bf16")
        vv, small_v = draw((1, 1, C, D), 122, "bf16")
        dt = torch.bfloat16
    say(f"attn_decode_sink_window_ex, entry stride {stride} elements, span {span * esz} bytes, fp8={fp8}")
    big_k = torch.empty(span, dtype=dt, device="cuda")
    big_v = torch.empty(span, dtype=dt, device="cuda")
    k = big_k.as_strided((1, 1, C, D), (0, 0, stride, 1))
    v = big_v.as_strided((1, 1, C, D), (0, 0, stride, 1))
    k.copy_(small_k)
    v.copy_(small_v)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    o = api.attn_decode_sink_window_ex(q, k, v, torch.tensor([C], dtype=torch.int32, device="cuda"),
                                       n_sink, window, tab, scale,
                                       ring_head=torch.from_numpy(rh).cuda())
    torch.cuda.synchronize()
    got = host(o)
    del k, v, big_k, big_v
    torch.cuda.empty_cache()
    ref = A.decode_sink_window(qv, kv, vv, th, scale, n_sink, window, [C], rh)
    assert max_abs(got, ref) <= BF16_TOL


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("G,D", [(1, 128), (2, 64), (4, 64), (8, 128)])
def test_decode_interleaved_layout(fp8, G, D):
    # Keys and the query rotated in the interleaved pair layout, bf16 or E4M3
    # cache, through attn_decode_sink_window_ex; lengths and ring heads as in
    # the edge cases.
    require_gpu()
    import torch
    n_sink, window = 4, 300
    C = n_sink + window
    lens = [0, 1, 5, 150, C, C, C]
    heads = [0, 0, 0, 7, 0, 123, window - 1]
    B, Hkv = len(lens), 2
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    if fp8:
        tab, th, scale, (qv, kv, vv), q, dv = _fp8_case(B, Hkv * G, Hkv, D, n_sink, window, lens,
                                                        heads, rope, seed=100 + G + D)
        k, v, ks, vs, lens_t, rh_t = dv["k"], dv["v"], dv["ks"], dv["vs"], dv["lens"], dv["rh"]
    else:
        tab, th, scale, (qv, kv, vv), (q, k, v), lens_t, rh_t = _case(
            B, Hkv * G, Hkv, D, n_sink, window, lens, heads, rope, seed=110 + G + D)
        ks = vs = None
    say(f"attn_decode_sink_window_ex interleaved fp8={fp8} G={G} D={D}")
    o = api.attn_decode_sink_window_ex(q, k, v, lens_t, n_sink, window, tab, scale,
                                       layout=api.LAYOUT_INTERLEAVED, ring_head=rh_t,
                                       k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    got = host(o)
    for b in range(B):
        ref = A.decode_sink_window(qv[b:b + 1], kv[b:b + 1], vv[b:b + 1], th, scale, n_sink,
                                   window, [lens[b]], [heads[b]], layout="interleaved")
        assert max_abs(got[b], ref[0]) <= BF16_TOL, b
