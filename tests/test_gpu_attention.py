"""GPU parity: blockwise prefill and the ring-step accumulate against the fp64 oracle.

Small cases compare every output element; the full-size workloads (the
launch configurations the bench times) compare seeded samples of query
rows, each of which the oracle computes on its own.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api, synth
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, F32_TOL, draw, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu


def _setup(B, S, Hq, Hkv, D, dtype, rope, seed_base=0, n_rows=None):
    tab, th, af = api.rope_tables_build(api.RopeConfig.of(rope), n_rows or S)
    qv, q = draw((B, S, Hq, D), seed_base + 0, dtype)
    kv, k = draw((B, S, Hkv, D), seed_base + 1, dtype)
    vv, v = draw((B, S, Hkv, D), seed_base + 2, dtype)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    return tab, th, scale, (qv, kv, vv), (q, k, v)


def test_prefill_tiny_fp32():
    # 1 x 1 head x d=64, S=512, fp32, YaRN s=4 from 128.
    require_gpu()
    import torch
    w = W.TINY
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(1, w.seq, 1, 1, w.head_dim, "f32", w.rope)
    say("attn_prefill_blockwise tiny fp32 S=512 d=64")
    kr = api.rope_apply(k, tab)
    o = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale)
    err = max_abs(host(o), ref)
    assert err <= F32_TOL, err


CASES = [
    # B, S, Hq, Hkv, D, causal, kind
    (1, 1, 1, 1, 128, True, W.YARN),
    (1, 63, 2, 2, 128, True, W.YARN),
    (1, 64, 2, 1, 128, True, W.PI),
    (2, 257, 4, 2, 128, True, W.NTK),
    (1, 1000, 2, 2, 128, True, W.YARN),
    (1, 1000, 2, 2, 128, False, W.YARN),
    (1, 700, 8, 2, 64, True, W.YARN),
    (1, 513, 2, 2, 64, False, W.PLAIN),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,kind", CASES)
def test_prefill_bf16_small(B, S, Hq, Hkv, D, causal, kind):
    require_gpu()
    import torch
    rope = W.Rope(kind, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(B, S, Hq, Hkv, D, "bf16", rope, seed_base=S)
    say(f"attn_prefill_blockwise bf16 B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    kr = api.rope_apply(k, tab)
    o = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab, causal=causal, lse=lse)
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale, causal=causal)
    err = max_abs(host(o), ref)
    assert err <= BF16_TOL, err
    # log-sum-exp per row against the oracle's (m, l)
    qr = R.rotate_bshd(qv, th, np.arange(S))
    krr = R.rotate_bshd(kv, th, np.arange(S))
    vis = A.causal_visible if causal else A.all_visible
    lse_h = host(lse)
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            _, m, l = A.attention_full(qr[b, :, h], krr[b, :, g], vv[b, :, g], scale,
                                       np.arange(S), np.arange(S), vis, return_state=True)
            assert max_abs(lse_h[b, h], m + np.log(l)) <= 1e-2


def test_prefill_prerotated_and_strided():
    # cos_sin = NULL: Q and K are taken as already rotated; inputs are views
    # into a packed [B, S, 3, H, D] buffer (strided tokens and heads).
    require_gpu()
    import torch
    B, S, H, D = 1, 300, 2, 128
    qkv_v, qkv = draw((B, S, 3, H, D), 77, "bf16")
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    say("attn_prefill_blockwise prerotated strided S=300")
    o = api.attn_prefill_blockwise(q, k, v, 0.1)
    torch.cuda.synchronize()
    ref = A.prefill(qkv_v[:, :, 0], qkv_v[:, :, 1], qkv_v[:, :, 2], None, 0.1)
    assert max_abs(host(o), ref) <= BF16_TOL


@pytest.mark.parametrize("kv_tok_stride", [0, 64])
def test_prefill_overlapping_key_rows(kv_tok_stride):
    # K and V as views whose token stride is below a row (0: one row
    # broadcast to every token; 64 elements: rows overlap by half).  The
    # kernel's fast DMA needs a stride of at least a row, so every tile goes
    # through the clamped load; the oracle sees the same overlapping values.
    require_gpu()
    import torch
    S, H, D = 300, 2, 128
    span = (S - 1) * kv_tok_stride + H * D
    qv, q = draw((1, S, H, D), 31, "bf16")
    kbuf_v, kbuf = draw((span,), 32, "bf16")
    vbuf_v, vbuf = draw((span,), 33, "bf16")
    shape, strides = (1, S, H, D), (span, kv_tok_stride, D, 1)
    k = torch.as_strided(kbuf, shape, strides)
    v = torch.as_strided(vbuf, shape, strides)
    kv = np.lib.stride_tricks.as_strided(kbuf_v, shape, [x * kbuf_v.itemsize for x in strides])
    vv = np.lib.stride_tricks.as_strided(vbuf_v, shape, [x * vbuf_v.itemsize for x in strides])
    say(f"attn_prefill_blockwise key/value token stride {kv_tok_stride} S={S}")
    o = api.attn_prefill_blockwise(q, k, v, 0.09)
    torch.cuda.synchronize()
    ref = A.prefill(qv, np.array(kv), np.array(vv), None, 0.09)
    assert max_abs(host(o), ref) <= BF16_TOL


def test_prefill_interleaved_layout_prerotated():
    # A model in the interleaved pair layout: Q and K rotated by rope_apply_ex,
    # then the prefill with cos_sin = NULL, against the oracle rotating
    # (2i, 2i+1) pairs in fp64.
    require_gpu()
    import torch
    B, S, Hq, Hkv, D = 1, 700, 4, 2, 128
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(B, S, Hq, Hkv, D, "bf16", rope, seed_base=55)
    say("attn_prefill_blockwise interleaved layout, pre-rotated S=700")
    qr = api.rope_apply_ex(q, tab, layout=api.LAYOUT_INTERLEAVED)
    kr = api.rope_apply_ex(k, tab, layout=api.LAYOUT_INTERLEAVED)
    o = api.attn_prefill_blockwise(qr, kr, v, scale)
    torch.cuda.synchronize()
    c, s = R.tables(th, np.arange(S))
    qi = R.rotate_interleaved(np.asarray(qv, np.float64), c[None, :, None, :], s[None, :, None, :])
    ki = R.rotate_interleaved(np.asarray(kv, np.float64), c[None, :, None, :], s[None, :, None, :])
    ref = A.prefill(qi, ki, vv, None, scale)
    assert max_abs(host(o), ref) <= BF16_TOL


def test_prefill_deterministic():
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, 128, 1e4, 4.0, 128)
    tab, th, scale, _, (q, k, v) = _setup(1, 2000, 4, 4, 128, "bf16", rope, seed_base=5)
    say("attn_prefill_blockwise determinism S=2000")
    kr = api.rope_apply(k, tab)
    o1 = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    o2 = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("S,Hq,Hkv", [(2000, 4, 4), (1300, 3, 1)])
def test_prefill_claimed_items_repeated(S, Hq, Hkv):
    # With a workspace the last 30 % of the grid claims its work items at
    # run time from a counter there, which each launch leaves as it found
    # it.  70 launches in a row through one workspace, each into a NaN-filled
    # output, must all write every row and equal the fixed schedule
    # (workspace NULL) bit for bit (grids of 32 and 18 blocks).
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, 128, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(1, S, Hq, Hkv, 128, "bf16", rope, seed_base=9)
    say(f"attn_prefill_blockwise claimed items S={S} Hq={Hq} x70")
    kr = api.rope_apply(k, tab)
    fixed = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    ws = api.new_workspace()
    torch.cuda.synchronize()
    assert not torch.isnan(fixed).any()
    rows = _sample_rows(S, 5, 24)
    ref = A.prefill(qv, kv, vv, th, scale, rows=rows)
    assert max_abs(host(fixed[0, rows]), ref[0]) <= BF16_TOL
    for i in range(70):
        o = torch.full_like(q, float("nan"))
        api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab, out=o, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, fixed), i
    assert int(ws.abs().sum()) == 0


def test_prefill_claims_from_a_nonzero_counter():
    # Ticket c stands for claimed item c mod n: whatever the counter holds
    # when the launch starts, every item is taken once, and the counter ends
    # at its starting value mod n (n = claims per launch: 32 blocks, the
    # last 10 claimed, here).
    require_gpu()
    import torch
    S, Hq = 2000, 4
    rope = W.Rope(W.YARN, 128, 1e4, 4.0, 128)
    tab, th, scale, _, (q, k, v) = _setup(1, S, Hq, Hq, 128, "bf16", rope, seed_base=19)
    say("attn_prefill_blockwise claims from a counter holding 1234567")
    kr = api.rope_apply(k, tab)
    fixed = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    ws = api.new_workspace()
    ws[0] = 1234567
    o = torch.full_like(q, float("nan"))
    api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab, out=o, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, fixed)
    n_blocks = 8 * Hq                      # 256-row query tiles x heads
    n_claims = n_blocks - n_blocks * 7 // 10
    assert int(ws[0]) == 1234567 % n_claims
    assert int(ws[1:].abs().sum()) == 0


def test_prefill_two_streams_at_once():
    # Two streams of default priority, each with its own workspace, run
    # prefills of different inputs at the same time (nothing orders one
    # stream's launches against the other's); each result equals the same
    # call run alone, bit for bit.  The library keeps no state between calls.
    require_gpu()
    import torch
    S, Hq, Hkv = 4096, 8, 8
    rope = W.Rope(W.YARN, 128, 1e4, 4.0, 1024)
    tab, th, scale, _, (q1, k1, v1) = _setup(1, S, Hq, Hkv, 128, "bf16", rope, seed_base=120)
    _, _, _, _, (q2, k2, v2) = _setup(1, S, Hq, Hkv, 128, "bf16", rope, seed_base=130)
    kr1, kr2 = api.rope_apply(k1, tab), api.rope_apply(k2, tab)
    say("attn_prefill_blockwise on two streams at once, S=4096 H=8")
    alone1 = api.attn_prefill_blockwise(q1, kr1, v1, scale, cos_sin=tab)
    alone2 = api.attn_prefill_blockwise(q2, kr2, v2, scale, cos_sin=tab)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1, ws2 = api.new_workspace(), api.new_workspace()
    outs1 = [torch.full_like(q1, float("nan")) for _ in range(6)]
    outs2 = [torch.full_like(q2, float("nan")) for _ in range(6)]
    torch.cuda.synchronize()
    for i in range(6):
        with torch.cuda.stream(s1):
            api.attn_prefill_blockwise(q1, kr1, v1, scale, cos_sin=tab, out=outs1[i], workspace=ws1)
        with torch.cuda.stream(s2):
            api.attn_prefill_blockwise(q2, kr2, v2, scale, cos_sin=tab, out=outs2[i], workspace=ws2)
    torch.cuda.synchronize()
    for i in range(6):
        assert torch.equal(outs1[i], alone1), i
        assert torch.equal(outs2[i], alone2), i
    assert int(ws1.abs().sum()) == 0 and int(ws2.abs().sum()) == 0


def _sample_rows(S, seed, count=40):
    edges = [0, 1, 2, 63, 64, 127, 128, 255, 256, 257, S // 2, S - 257, S - 256, S - 2, S - 1]
    return synth.sample_rows(S, count, seed, must=edges)


def _check_prefill_rows(w, heads, rows_per_head=40):
    import torch
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(w.batch, w.seq, w.n_q_heads, w.n_kv_heads,
                                                     w.head_dim, "bf16", w.rope)
    say(f"attn_prefill_blockwise {w.name} full size")
    kr = api.rope_apply(k, tab)
    del k
    o = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab, workspace=api.new_workspace())
    torch.cuda.synchronize()
    worst = 0.0
    for h in heads:
        rows = _sample_rows(w.seq, 1000 + h, rows_per_head)
        got = host(o[0, rows, h])
        ref = A.prefill(qv, kv, vv, th, scale, rows=rows, heads=[h])[0, :, 0]
        worst = max(worst, max_abs(got, ref))
    assert worst <= BF16_TOL, worst
    return worst


# Full-size checks: 2048 seeded rows per head (the first and last rows and
# the tile edges among them) on four heads, each row computed by the oracle
# on its own.
FULL_ROWS = 2048


def test_prefill_full_llama16k():
    require_gpu()
    _check_prefill_rows(W.LLAMA_16K, heads=[0, 13, 22, 31], rows_per_head=FULL_ROWS)


@pytest.mark.parametrize("kind", [W.PI, W.NTK, W.YARN], ids=["pi", "ntk", "yarn"])
def test_prefill_full_gqa32k(kind):
    require_gpu()
    _check_prefill_rows(W.GQA_32K[kind], heads=[0, 5, 17, 30], rows_per_head=FULL_ROWS)


# ---------------------------------------------------------------------------
# attn_block_accumulate (one ring device's share)
# ---------------------------------------------------------------------------

def _ring(w_blocks, blk, Hq, Hkv, D, dtype, rope, qi, seed_base=0):
    S = w_blocks * blk
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), S)
    qv, q = draw((1, blk, Hq, D), seed_base + 0, dtype)        # the local query block
    kv, k = draw((1, S, Hkv, D), seed_base + 1, dtype)         # the whole key sequence
    vv, v = draw((1, S, Hkv, D), seed_base + 2, dtype)
    k = api.rope_apply(k, tab)          # each block rotated once at its own positions
    kb = [k[:, j * blk:(j + 1) * blk] for j in range(w_blocks)]
    vb = [v[:, j * blk:(j + 1) * blk] for j in range(w_blocks)]
    kbv = [kv[:, j * blk:(j + 1) * blk] for j in range(w_blocks)]
    vbv = [vv[:, j * blk:(j + 1) * blk] for j in range(w_blocks)]
    return tab, th, q, qv, kb, vb, kbv, vbv


def _run_ring(q, kb, vb, tab, scale, qi, blk, order, state=None, finalize=True, workspace=None):
    out = None
    for t, j in enumerate(order):
        last = t == len(order) - 1
        out = api.attn_block_accumulate(q, kb[j], vb[j], state, qi * blk, j * blk, scale,
                                        cos_sin=tab, first=(t == 0), finalize=finalize and last,
                                        workspace=workspace)
    return out


def test_accumulate_tiny_ring_fp32():
    # The tiny fp32 problem fed as 8 blocks of 64 (query block 7, ring order).
    require_gpu()
    import torch
    w = W.TINY_RING
    tab, th, q, qv, kb, vb, kbv, vbv = _ring(w.n_blocks, w.block, 1, 1, w.head_dim, "f32",
                                             w.rope, w.q_block_index)
    scale = R.softmax_scale(w.rope.kind, w.rope.scale, w.head_dim)
    st = api.AccState.empty(1, w.block, 1, w.head_dim)
    order = W.ring_order(w)
    say("attn_block_accumulate tiny fp32 ring 8x64")
    o = _run_ring(q, kb, vb, tab, scale, w.q_block_index, w.block, order, st)
    torch.cuda.synchronize()
    offs = [j * w.block for j in range(w.n_blocks)]
    o_ref, m_ref, l_ref, acc_ref = A.ring_share(qv, kbv, vbv, th, scale,
                                                w.q_block_index * w.block, offs, order=order)
    assert max_abs(host(o), o_ref) <= F32_TOL
    np.testing.assert_allclose(host(st.m), m_ref, atol=1e-5)
    np.testing.assert_allclose(host(st.l), l_ref, rtol=1e-5)
    np.testing.assert_allclose(host(st.o_acc), acc_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("qi", [0, 2, 3])
def test_accumulate_bf16_ring_small(qi):
    require_gpu()
    import torch
    nb, blk, Hq, Hkv, D = 4, 300, 4, 2, 128
    rope = W.Rope(W.YARN, D, 1e4, 8.0, 300)
    tab, th, q, qv, kb, vb, kbv, vbv = _ring(nb, blk, Hq, Hkv, D, "bf16", rope, qi, seed_base=9)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    offs = [j * blk for j in range(nb)]
    order = [(qi - t) % nb for t in range(nb)]       # includes future blocks: no-ops
    st = api.AccState.empty(1, blk, Hq, D)
    say(f"attn_block_accumulate bf16 ring 4x300 qi={qi}")
    o = _run_ring(q, kb, vb, tab, scale, qi, blk, order, st)
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref, acc_ref = A.ring_share(qv, kbv, vbv, th, scale, qi * blk, offs,
                                                order=order)
    assert max_abs(host(o), o_ref) <= BF16_TOL
    np.testing.assert_allclose(host(st.m), m_ref, atol=2e-2)
    # order invariance on the GPU: ascending block order
    st2 = api.AccState.empty(1, blk, Hq, D)
    o2 = _run_ring(q, kb, vb, tab, scale, qi, blk, list(range(nb)), st2)
    torch.cuda.synchronize()
    assert max_abs(host(o2), o_ref) <= BF16_TOL


def test_prefill_fp32_d128():
    # The fp32 storage path at d = 128 (the tiny configuration is d = 64):
    # GQA 2:1, causal, ragged tail.
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, 128, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(1, 300, 2, 1, 128, "f32", rope, seed_base=130)
    say("attn_prefill_blockwise fp32 S=300 Hq=2 Hkv=1 d=128")
    kr = api.rope_apply(k, tab)
    o = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab)
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale)
    assert max_abs(host(o), ref) <= F32_TOL


def _ring_b(B, nb, blk, Hq, Hkv, D, rope, seed_base):
    S = nb * blk
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), S)
    qv, q = draw((B, blk, Hq, D), seed_base + 0, "bf16")
    kv, k = draw((B, S, Hkv, D), seed_base + 1, "bf16")
    vv, v = draw((B, S, Hkv, D), seed_base + 2, "bf16")
    k = api.rope_apply(k, tab)
    kb = [k[:, j * blk:(j + 1) * blk] for j in range(nb)]
    vb = [v[:, j * blk:(j + 1) * blk] for j in range(nb)]
    kbv = [kv[:, j * blk:(j + 1) * blk] for j in range(nb)]
    vbv = [vv[:, j * blk:(j + 1) * blk] for j in range(nb)]
    return tab, th, q, qv, kb, vb, kbv, vbv


@pytest.mark.parametrize("causal,D", [(False, 64), (True, 128)])
def test_accumulate_bf16_ring_batched(causal, D):
    # Two sequences in the batch, three key blocks; non-causal (every block
    # visible, none skipped) at d = 64, causal at d = 128, fed out of order.
    require_gpu()
    import torch
    B, nb, blk, Hq, Hkv, qi = 2, 3, 200, 4, 2, 1
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 150)
    tab, th, q, qv, kb, vb, kbv, vbv = _ring_b(B, nb, blk, Hq, Hkv, D, rope, 140 + D)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    order = [2, 0, 1]
    st = api.AccState.empty(B, blk, Hq, D)
    say(f"attn_block_accumulate bf16 B=2 3x200 causal={causal} d={D}")
    o = None
    for t, j in enumerate(order):
        o = api.attn_block_accumulate(q, kb[j], vb[j], st, qi * blk, j * blk, scale, cos_sin=tab,
                                      causal=causal, first=(t == 0), finalize=(t == nb - 1))
    torch.cuda.synchronize()
    o_ref, m_ref, l_ref, _ = A.ring_share(qv, kbv, vbv, th, scale, qi * blk,
                                          [j * blk for j in range(nb)], order=order, causal=causal)
    assert max_abs(host(o), o_ref) <= BF16_TOL
    np.testing.assert_allclose(host(st.m), m_ref, atol=2e-2)
    np.testing.assert_allclose(host(st.l), l_ref, rtol=2e-2)


def test_prefill_token_stride_past_the_fast_dma():
    # K and V with a token stride of 2^24 elements: 64 rows of it pass 2^31
    # bytes, so the per-tile DMA cannot use 32-bit lane offsets and every
    # tile takes the clamped per-lane-address load (about 5.3 GB per view).
    require_gpu()
    import torch
    S, Hq, Hkv, D = 160, 2, 1, 128
    stride = 1 << 24
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, scale, (qv, kv, vv), (q, k, v) = _setup(1, S, Hq, Hkv, D, "bf16", rope, seed_base=150)
    kr = api.rope_apply(k, tab)
    span = (S - 1) * stride + Hkv * D
    say(f"attn_prefill_blockwise K/V token stride {stride} elements, {2 * span} bytes per view")
    big_k = torch.empty(span, dtype=torch.bfloat16, device="cuda")
    big_v = torch.empty(span, dtype=torch.bfloat16, device="cuda")
    ks = big_k.as_strided((1, S, Hkv, D), (0, stride, D, 1))
    vs = big_v.as_strided((1, S, Hkv, D), (0, stride, D, 1))
    ks.copy_(kr)
    vs.copy_(v)
    o = api.attn_prefill_blockwise(q, ks, vs, scale, cos_sin=tab)
    torch.cuda.synchronize()
    got = host(o)
    del ks, vs, big_k, big_v
    torch.cuda.empty_cache()
    ref = A.prefill(qv, kv, vv, th, scale)
    assert max_abs(got, ref) <= BF16_TOL


def test_accumulate_rows_that_start_empty():
    # Query rows at positions 0..255 against a key block at positions
    # 100..399 (causal): rows below 100 see none of its keys while later rows
    # of the same wave do.  Their state stays empty (m = -inf, l = 0, o = 0);
    # the other rows match the oracle.
    require_gpu()
    import torch
    Sq, Sk, H, D, scale = 256, 300, 2, 128, 0.09
    qv, q = draw((1, Sq, H, D), 71, "bf16")
    kv, k = draw((1, Sk, H, D), 72, "bf16")
    vv, v = draw((1, Sk, H, D), 73, "bf16")
    st = api.AccState.empty(1, Sq, H, D)
    say("attn_block_accumulate rows that start empty: q 0..255, k 100..399")
    o = api.attn_block_accumulate(q, k, v, st, 0, 100, scale, first=True, finalize=True)
    torch.cuda.synchronize()
    got_o, got_m, got_l = host(o), host(st.m), host(st.l)
    for h in range(H):
        ref, m, l = A.attention_full(qv[0, :, h], kv[0, :, h], vv[0, :, h], scale, np.arange(Sq),
                                     100 + np.arange(Sk), A.causal_visible, return_state=True)
        assert max_abs(got_o[0, :, h], ref) <= BF16_TOL
        assert np.all(np.isneginf(got_m[0, h, :100])) and np.all(got_l[0, h, :100] == 0)
        np.testing.assert_allclose(got_m[0, h, 100:], m[100:], atol=2e-2)
        np.testing.assert_allclose(got_l[0, h, 100:], l[100:], rtol=2e-2)


def test_accumulate_resume_from_host_snapshot():
    require_gpu()
    import torch
    nb, blk, Hq, Hkv, D = 4, 256, 2, 2, 128
    rope = W.Rope(W.PI, D, 1e4, 4.0)
    qi = 3
    tab, th, q, qv, kb, vb, kbv, vbv = _ring(nb, blk, Hq, Hkv, D, "bf16", rope, qi, seed_base=21)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    order = [3, 2, 1, 0]
    st = api.AccState.empty(1, blk, Hq, D)
    say("attn_block_accumulate resume")
    o_ref = _run_ring(q, kb, vb, tab, scale, qi, blk, order, st)
    st2 = api.AccState.empty(1, blk, Hq, D)
    _run_ring(q, kb, vb, tab, scale, qi, blk, order[:2], st2, finalize=False)
    torch.cuda.synchronize()
    snap = [host(x) for x in (st2.o_acc, st2.m, st2.l)]
    st3 = api.AccState(*[torch.from_numpy(x.astype(np.float32)).cuda() for x in snap])
    o_res = None
    for t, j in enumerate(order[2:]):
        o_res = api.attn_block_accumulate(q, kb[j], vb[j], st3, qi * blk, j * blk, scale,
                                          cos_sin=tab, finalize=(t == 1))
    torch.cuda.synchronize()
    assert torch.equal(o_res, o_ref)


def test_accumulate_full_ring_share():
    # 8 heads, query block 7 of 8 blocks of 32768 tokens (positions up to
    # 262143), YaRN s=8 from 32768, fed in ring order 7, 6, ..., 0.
    require_gpu()
    import torch
    w = W.RING_SHARE
    tab, th, q, qv, kb, vb, kbv, vbv = _ring(w.n_blocks, w.block, w.n_q_heads, w.n_kv_heads,
                                             w.head_dim, "bf16", w.rope, w.q_block_index)
    scale = R.softmax_scale(w.rope.kind, w.rope.scale, w.head_dim)
    st = api.AccState.empty(1, w.block, w.n_q_heads, w.head_dim)
    order = W.ring_order(w)
    say("attn_block_accumulate ring share 8x32768 full size")
    o = _run_ring(q, kb, vb, tab, scale, w.q_block_index, w.block, order, st, workspace=api.new_workspace())
    torch.cuda.synchronize()
    offs = [j * w.block for j in range(w.n_blocks)]
    worst = 0.0
    for h in (0, 3, 5, 7):
        rows = _sample_rows(w.block, 50 + h, FULL_ROWS)
        o_ref, m_ref, _, _ = A.ring_share(qv, kbv, vbv, th, scale, w.q_block_index * w.block,
                                          offs, order=order, rows=rows, heads=[h])
        worst = max(worst, max_abs(host(o[0, rows, h]), o_ref[0, :, 0]))
        assert max_abs(host(st.m[0, h, rows]), m_ref[0, 0]) <= 2e-2
    assert worst <= BF16_TOL, worst
