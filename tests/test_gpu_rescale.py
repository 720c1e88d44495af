"""GPU parity on inputs that force the online softmax to rescale a non-empty
accumulator, in each bf16 attention path: the causal prefill (including
work items claimed at run time, diagonal quarters and a ragged end), the
ring step (the jump arriving in a later call, against the stored state) and
the sink+window prefill.

The merge that keeps blockwise attention exact is the running max and sum
("Ring attention" in the jovanaeducation guide; "Ring Attention" in the
14cs17 notes): when a later key block holds a larger logit, what was
accumulated so far is scaled by exp(m_old - m_new).  The inputs are built in
tests/stress_inputs.py so that row maxima jump by 10 to 30 log2 units after
a row's first quarter while the logits stay exact; each test first counts,
from the oracle's logits on the CPU, the rows that must take that path, and
fails if there are too few.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api, synth
from tests import stress_inputs as SI
from tests.gpu_helpers import BF16_TOL, dev_tensor, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / np.log(2.0)


def _qkv(B, S, Hq, Hkv, D, pattern, seed):
    qv, qb = synth.normal((B, S, Hq, D), seed, "bf16")
    k0, _ = synth.normal((B, S, Hkv, D), seed + 1, "bf16")
    kv, kb = SI.scaled_bf16(k0, SI.quarter_multipliers(S, pattern), axis=1)
    v0, _ = synth.normal((B, S, Hkv, D), seed + 2, "bf16")
    vv, vb = SI.scaled_bf16(v0, np.full(S, SI.V_SCALE), axis=1)
    return (qv, kv, vv), (qb, kb, vb)


def _upload(values, bits):
    return tuple(dev_tensor(x, b, "bf16") for x, b in zip(values, bits))


def _logits_log2(qr, kr, scale):
    return (scale * LOG2E) * (np.asarray(qr, np.float64) @ np.asarray(kr, np.float64).T)


PREFILL_CASES = [
    # B, S, Hq, Hkv, D, workspace, min rows with an event, min with one on the diagonal
    (1, 2000, 4, 2, 128, True, 4 * 1500, 4 * 24),   # 32 blocks: the last 10 claimed (rows < 768)
    (1, 700, 2, 2, 64, False, 2 * 450, 2 * 24),
    (2, 333, 2, 1, 128, False, 4 * 180, 4 * 24),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,ws,min_rows,min_diag", PREFILL_CASES)
def test_prefill_rescale_forced(B, S, Hq, Hkv, D, ws, min_rows, min_diag):
    require_gpu()
    import torch
    factors = SI.quarter_turn_factors(D)
    th = R.inv_freq_factors(D, 1e4, factors)
    (qv, kv, vv), bits = _qkv(B, S, Hq, Hkv, D, [1, 1, 1, 8], seed=300 + S)
    scale = SI.SCALE_EXACT
    # CPU: rows that must rescale a non-empty state (ascending quarters)
    pos = np.arange(S)
    qr = R.rotate_bshd(qv, th, pos)
    kr = R.rotate_bshd(kv, th, pos)
    vis = A.causal_visible(pos, pos)
    walk = SI.ascending_quarters(S)
    diag_q = pos // SI.QUARTER
    rows = diag = 0
    big_jump = 0.0
    claimed_rows = 0
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            lg = _logits_log2(qr[b, :, h], kr[b, :, g], scale)
            ev, jump, at = SI.rescale_events(lg, vis, walk)
            rows += int(np.sum(ev > 0))
            big_jump = max(big_jump, float(jump.max()))
            # an event in the row's own quarter (on the diagonal, masked)
            diag += int(np.sum(at[pos, diag_q]))
            if ws and b == 0:
                claimed_rows += int(np.sum(ev[:768] > 0))
    assert rows >= min_rows, rows
    assert diag >= min_diag, diag
    assert 10.0 <= big_jump, big_jump
    if ws:
        assert claimed_rows >= 300, claimed_rows
    say(f"attn_prefill_blockwise forced rescale B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} ws={ws} "
        f"rows={rows} diag={diag}")
    q, k, v = _upload((qv, kv, vv), bits)
    tab, th_gpu = api.rope_tables_build_factors(D, 1e4, factors, S)
    np.testing.assert_allclose(th_gpu, th, rtol=1e-14)
    k_rot = api.rope_apply(k, tab)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = api.attn_prefill_blockwise(q, k_rot, v, scale, cos_sin=tab, lse=lse,
                                   workspace=api.new_workspace() if ws else None)
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale)
    err = max_abs(host(o), ref)
    assert err <= BF16_TOL, err
    lse_h = host(lse)
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            _, m, l = A.attention_full(qr[b, :, h], kr[b, :, g], vv[b, :, g], scale, pos, pos,
                                       A.causal_visible, return_state=True)
            assert max_abs(lse_h[b, h], m + np.log(l)) <= 1e-2


@pytest.mark.parametrize("D", [128, 64])
def test_accumulate_rescale_forced_in_later_calls(D):
    # Query block 3 of 4 blocks of 300 tokens, fed in ring order 3, 2, 1, 0.
    # Block multipliers 1, 8, 1, 16 (in feed order): the row maxima jump in
    # the second call against the state the first stored, and again in the
    # fourth.  The calls that store the state track the exact max.
    require_gpu()
    import torch
    nb, blk, Hq, Hkv, qi = 4, 300, 4, 2, 3
    S = nb * blk
    factors = SI.quarter_turn_factors(D)
    th = R.inv_freq_factors(D, 1e4, factors)
    mult_of_block = {3: 1.0, 2: 8.0, 1: 1.0, 0: 16.0}
    qv, qb = synth.normal((1, blk, Hq, D), 400 + D, "bf16")
    k0, _ = synth.normal((1, S, Hkv, D), 401 + D, "bf16")
    kv, kb = SI.scaled_bf16(k0, np.repeat([mult_of_block[j] for j in range(nb)], blk), axis=1)
    v0, _ = synth.normal((1, S, Hkv, D), 402 + D, "bf16")
    vv, vb = SI.scaled_bf16(v0, np.full(S, SI.V_SCALE), axis=1)
    scale = SI.SCALE_EXACT
    order = [3, 2, 1, 0]
    qpos = qi * blk + np.arange(blk)
    # CPU: events per call, each call walking its block's quarters in order,
    # starting from the exact max the stored state carries in
    qr = R.rotate_half(np.asarray(qv[0], np.float64), *[x[:, None, :] for x in R.tables(th, qpos)])
    kr = R.rotate_bshd(kv, th, np.arange(S))[0]
    later_rows = 0
    jumps = []
    for h in range(Hq):
        g = A.kv_head(h, Hq, Hkv)
        lg = _logits_log2(qr[:, h], kr[:, g], scale)
        vis = A.causal_visible(qpos, np.arange(S))
        run_max = np.full(blk, -np.inf)
        ev_later = np.zeros(blk, np.int64)
        for t, j in enumerate(order):
            walk = [j * blk + w for w in SI.ascending_quarters(blk)]
            ev, jump, _ = SI.rescale_events(lg, vis, walk, start=run_max)
            if t > 0:
                ev_later += ev
                jumps.append(jump[ev > 0])
            keys = np.arange(j * blk, (j + 1) * blk)
            run_max = np.maximum(run_max, np.where(vis[:, keys], lg[:, keys], -np.inf).max(axis=1))
        later_rows += int(np.sum(ev_later > 0))
    jumps = np.concatenate(jumps)
    assert later_rows >= Hq * 280, later_rows
    assert np.median(jumps) >= 10.0, np.median(jumps)
    say(f"attn_block_accumulate forced rescale in later calls D={D} rows={later_rows}")
    tab, _ = api.rope_tables_build_factors(D, 1e4, factors, S)
    q = dev_tensor(qv, qb, "bf16")
    k = api.rope_apply(dev_tensor(kv, kb, "bf16"), tab)
    v = dev_tensor(vv, vb, "bf16")
    st = api.AccState.empty(1, blk, Hq, D)
    ws = api.new_workspace()
    mids = {}
    out = None
    for t, j in enumerate(order):
        out = api.attn_block_accumulate(q, k[:, j * blk:(j + 1) * blk], v[:, j * blk:(j + 1) * blk],
                                        st, qi * blk, j * blk, scale, cos_sin=tab, first=(t == 0),
                                        finalize=(t == nb - 1), workspace=ws)
        if t == 1:
            torch.cuda.synchronize()
            mids = {n: host(x).copy() for n, x in (("acc", st.o_acc), ("m", st.m), ("l", st.l))}
    torch.cuda.synchronize()
    kbl = [kv[:, j * blk:(j + 1) * blk] for j in range(nb)]
    vbl = [vv[:, j * blk:(j + 1) * blk] for j in range(nb)]
    offs = [j * blk for j in range(nb)]
    # state after the second call (the first jump), normalised
    _, m2, l2, acc2 = A.ring_share(qv, kbl, vbl, th, scale, qi * blk, offs, order=order[:2],
                                   finalize=False)
    np.testing.assert_allclose(mids["m"], m2, atol=1e-3)
    np.testing.assert_allclose(mids["l"], l2, rtol=2e-3)
    o2 = mids["acc"] / np.transpose(mids["l"], (0, 2, 1))[..., None]
    o2_ref = acc2 / np.transpose(l2, (0, 2, 1))[..., None]
    assert max_abs(o2, o2_ref) <= BF16_TOL
    # after the last call
    o_ref, m_ref, l_ref, _ = A.ring_share(qv, kbl, vbl, th, scale, qi * blk, offs, order=order)
    assert max_abs(host(out), o_ref) <= BF16_TOL
    np.testing.assert_allclose(host(st.m), m_ref, atol=1e-3)
    np.testing.assert_allclose(host(st.l), l_ref, rtol=2e-3)


def test_prefill_sink_window_rescale_forced():
    # 4 sinks, a window of 200, every fourth quarter of keys 8x larger.  The
    # walk folds the sink tile first, then the window's tiles in an order of
    # its own; a row certainly rescales when every big quarter it sees beats
    # every small key it sees by more than the threshold, whatever that order.
    require_gpu()
    import torch
    B, S, Hq, Hkv, D, n_sink, window = 1, 1000, 2, 1, 128, 4, 200
    factors = SI.quarter_turn_factors(D)
    th = R.inv_freq_factors(D, 1e4, factors)
    pattern = [1, 1, 1, 8]
    (qv, kv, vv), bits = _qkv(B, S, Hq, Hkv, D, pattern, seed=500)
    scale = SI.SCALE_EXACT
    pos = np.arange(S)
    qr = R.rotate_bshd(qv, th, pos)
    kr = R.rotate_bshd(kv, th, pos)
    vis = A.sink_window_visible(n_sink, window)(pos, pos)
    big = SI.quarter_multipliers(S, pattern) > 1
    sure = 0
    for h in range(Hq):
        lg = _logits_log2(qr[0, :, h], kr[0, :, A.kv_head(h, Hq, Hkv)], scale)
        small_max = np.where(vis & ~big[None, :], lg, -np.inf).max(axis=1)
        bigq_min = np.full(S, np.inf)
        any_big = np.zeros(S, bool)
        for keys in SI.ascending_quarters(S):
            if not big[keys[0]]:
                continue
            seen = vis[:, keys].any(axis=1)
            mx = np.where(vis[:, keys], lg[:, keys], -np.inf).max(axis=1)
            bigq_min = np.where(seen, np.minimum(bigq_min, mx), bigq_min)
            any_big |= seen
        sure += int(np.sum(any_big & (bigq_min > small_max + SI.TAU + 0.5)))
    assert sure >= Hq * 500, sure
    say(f"attn_prefill_sink_window forced rescale S={S} sink={n_sink} win={window} rows={sure}")
    q, k, v = _upload((qv, kv, vv), bits)
    tab, _ = api.rope_tables_build_factors(D, 1e4, factors, S)
    k_rot = api.rope_apply(k, tab)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = api.attn_prefill_sink_window(q, k_rot, v, scale, n_sink, window, cos_sin=tab, lse=lse,
                                     workspace=api.new_workspace())
    torch.cuda.synchronize()
    ref = A.prefill(qv, kv, vv, th, scale, n_sink=n_sink, window=window)
    assert max_abs(host(o), ref) <= BF16_TOL
    lse_h = host(lse)
    for h in range(Hq):
        g = A.kv_head(h, Hq, Hkv)
        _, m, l = A.attention_full(qr[0, :, h], kr[0, :, g], vv[0, :, g], scale, pos, pos,
                                   A.sink_window_visible(n_sink, window), return_state=True)
        assert max_abs(lse_h[0, h], m + np.log(l)) <= 1e-2
