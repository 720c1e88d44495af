"""fp64 CPU oracle: exact softmax attention, written twice, plus the
ring-attention share and the attention-sink + sliding-window decode.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it.

Two independent forms of the same definition:

A. ``attention_full`` materialises one query row's logits over all visible
   keys and applies softmax(Q K^T / sqrt(d_k)) V (tecvarsity Section 1, the
   MHSA relation).  Query rows are processed in chunks only to bound
   memory; each row's softmax is whole.
B. ``attention_online`` walks key blocks in any given order, keeping a
   running max m, running sum l and an unnormalised accumulator per row, and
   divides at the end.  The pages name this update without printing it
   (14cs17 "Ring Attention" ties it to FlashAttention's online softmax; the
   jovanaeducation guide, "Ring attention", has each device add in the
   share of every block that passes it); this is the textbook form (Milakov
   & Gimelshein 2018).

Masks:
* causal: key position <= query position (tecvarsity FAQ 2 states the
  block-level rule; inside a block the token-level rule is the reading).
* sink + window: the cache is {x_1..x_s} U {x_{t-w+1}..x_t} (14cs17
  "Sliding Window + Attention Sinks").

Conventions (readings): GQA groups are contiguous, kv_head = h // (Hq/Hkv).
Rows with no visible key give output 0, m = -inf, l = 0.  The state m, l is
in the natural-exp domain of the scaled logits.
"""
from __future__ import annotations

import numpy as np

from . import rope as _rope


def causal_visible(q_pos, k_pos):
    return k_pos[None, :] <= q_pos[:, None]


def all_visible(q_pos, k_pos):
    return np.ones((q_pos.shape[0], k_pos.shape[0]), dtype=bool)


def sink_window_visible(n_sink: int, window: int):
    """Token n is visible to query t iff n < n_sink or t - window < n <= t."""
    def f(q_pos, k_pos):
        t = q_pos[:, None]
        n = k_pos[None, :]
        return (n <= t) & ((n < n_sink) | (n > t - window))
    return f


def attention_full(q, k, v, softmax_scale, q_pos, k_pos, visible=causal_visible,
                   row_chunk: int = 1024, return_state: bool = False):
    """Form A for one head: q [Sq, D], k [Sk, D], v [Sk, Dv] -> o [Sq, Dv]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    Sq = q.shape[0]
    o = np.zeros((Sq, v.shape[1]), np.float64)
    m_out = np.full(Sq, -np.inf)
    l_out = np.zeros(Sq)
    for r0 in range(0, Sq, row_chunk):
        r1 = min(Sq, r0 + row_chunk)
        logits = softmax_scale * (q[r0:r1] @ k.T)
        vis = visible(q_pos[r0:r1], k_pos)
        logits = np.where(vis, logits, -np.inf)
        m = logits.max(axis=1)
        has = np.isfinite(m)
        e = np.zeros_like(logits)
        e[has] = np.exp(logits[has] - m[has, None])
        l = e.sum(axis=1)
        o[r0:r1][has] = (e[has] @ v) / l[has, None]
        m_out[r0:r1] = m
        l_out[r0:r1] = l
    if return_state:
        return o, m_out, l_out
    return o


def online_init(Sq: int, Dv: int):
    """Empty online-softmax state: m = -inf, l = 0, acc = 0."""
    return np.full(Sq, -np.inf), np.zeros(Sq), np.zeros((Sq, Dv))


def online_update(state, q, k_blk, v_blk, softmax_scale, q_pos, k_pos_blk, visible=causal_visible):
    """Fold one key block into (m, l, acc) for one head (form B).

    m_new = max(m, rowmax(s));  alpha = exp(m - m_new)
    l     = alpha * l + sum(exp(s - m_new))
    acc   = alpha * acc + exp(s - m_new) @ v
    Masked entries contribute nothing.
    """
    m, l, acc = state
    s = softmax_scale * (np.asarray(q, np.float64) @ np.asarray(k_blk, np.float64).T)
    vis = visible(np.asarray(q_pos), np.asarray(k_pos_blk))
    s = np.where(vis, s, -np.inf)
    m_new = np.maximum(m, s.max(axis=1)) if s.shape[1] else m.copy()
    live = np.isfinite(m_new)
    alpha = np.zeros_like(m)
    alpha[live] = np.exp(m[live] - m_new[live])     # exp(-inf) = 0 for a first hit
    p = np.zeros_like(s)
    p[live] = np.exp(s[live] - m_new[live, None])
    l = alpha * l + p.sum(axis=1)
    acc = alpha[:, None] * acc + p @ np.asarray(v_blk, np.float64)
    return m_new, l, acc


def online_finish(state):
    m, l, acc = state
    o = np.zeros_like(acc)
    nz = l > 0
    o[nz] = acc[nz] / l[nz, None]
    return o


def attention_online(q, k, v, softmax_scale, q_pos, k_pos, block: int = 64,
                     order=None, visible=causal_visible, return_state: bool = False):
    """Form B for one head: blocks of ``block`` keys, folded in ``order``."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    k_pos = np.asarray(k_pos)
    n_blocks = (k.shape[0] + block - 1) // block
    order = range(n_blocks) if order is None else order
    st = online_init(np.asarray(q).shape[0], v.shape[1])
    for j in order:
        sl = slice(j * block, min(k.shape[0], (j + 1) * block))
        st = online_update(st, q, k[sl], v[sl], softmax_scale, q_pos, k_pos[sl], visible)
    o = online_finish(st)
    if return_state:
        return o, st[0], st[1]
    return o


# ----------------------------------------------------------------------------
# Whole-layer forms on [B, S, H, D] arrays.
# ----------------------------------------------------------------------------

def kv_head(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    return h // (n_q_heads // n_kv_heads)


def prefill(q, k, v, theta, softmax_scale, causal=True, rows=None, heads=None,
            batches=None, q_offset: int = 0, k_offset: int = 0, n_sink: int = 0,
            window: int = 0):
    """Rotate Q and K (fp64) and run form A per (b, h).

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D].  Query token s sits at position
    q_offset + s, key token j at k_offset + j.  ``theta`` is None when Q, K
    are already rotated.  ``rows`` restricts the query rows computed (the
    result then has len(rows) rows).  ``window`` > 0 applies the sink+window
    mask (sink_window_visible; causal implied) in place of ``causal``: the
    prefill counterpart of the cache of 14cs17 "Sliding Window + Attention
    Sinks".  Returns o [B', len(rows), H', D]
    over the selected batches/heads.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else heads
    batches = range(B) if batches is None else batches
    q_pos = q_offset + rows
    k_pos = k_offset + np.arange(Sk)
    vis = causal_visible if causal else all_visible
    if window > 0:
        vis = sink_window_visible(n_sink, window)
    if theta is not None:
        cq, sq = _rope.tables(theta, q_pos)
        ck, sk = _rope.tables(theta, k_pos)
    out = np.zeros((len(batches), len(rows), len(heads), v.shape[3]))
    for bi, b in enumerate(batches):
        krot = {}
        for hi, h in enumerate(heads):
            g = kv_head(h, Hq, Hkv)
            if g not in krot:
                krot[g] = k[b, :, g] if theta is None else _rope.rotate_half(k[b, :, g], ck, sk)
            qq = q[b, rows, h] if theta is None else _rope.rotate_half(q[b, rows, h], cq, sq)
            out[bi, :, hi] = attention_full(qq, krot[g], v[b, :, g], softmax_scale,
                                            q_pos, k_pos, vis)
    return out


def ring_share(q, k_blocks, v_blocks, theta, softmax_scale, q_offset, k_offsets,
               order=None, causal=True, rows=None, heads=None, state_in=None,
               finalize=True):
    """One ring device's share: fold whole KV blocks (possibly from other
    devices) into its query block's online-softmax state.

    q [B, Sq, Hq, D] at positions q_offset + s; block j is k_blocks[j],
    v_blocks[j] [B, Sk, Hkv, D] at positions k_offsets[j] + t.  A block
    wholly in the future of every query (k_offset > last query position) is
    skipped (tecvarsity FAQ 2); the token-level causal mask applies inside.
    Returns (o, m, l, acc) with o/acc [B, R, H, D] and m/l [B, H, R].
    """
    q = np.asarray(q, np.float64)
    B, Sq, Hq, D = q.shape
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    heads = list(range(Hq)) if heads is None else list(heads)
    order = range(len(k_blocks)) if order is None else order
    q_pos = q_offset + rows
    vis = causal_visible if causal else all_visible
    Hkv = np.asarray(k_blocks[0]).shape[2]
    if theta is not None:
        cq, sq = _rope.tables(theta, q_pos)
    R, H = len(rows), len(heads)
    m = np.full((B, H, R), -np.inf)
    l = np.zeros((B, H, R))
    acc = np.zeros((B, R, H, D))
    if state_in is not None:
        m, l, acc = (np.array(x, np.float64) for x in state_in)
    last_q = q_offset + Sq - 1
    for j in order:
        if causal and k_offsets[j] > last_q:
            continue
        kb = np.asarray(k_blocks[j], np.float64)
        vb = np.asarray(v_blocks[j], np.float64)
        k_pos = k_offsets[j] + np.arange(kb.shape[1])
        if theta is not None:
            ck, sk = _rope.tables(theta, k_pos)
        for b in range(B):
            krot = {}
            for hi, h in enumerate(heads):
                g = kv_head(h, Hq, Hkv)
                if g not in krot:
                    krot[g] = kb[b, :, g] if theta is None else _rope.rotate_half(kb[b, :, g], ck, sk)
                qq = q[b, rows, h] if theta is None else _rope.rotate_half(q[b, rows, h], cq, sq)
                st = (m[b, hi], l[b, hi], acc[b, :, hi])
                mn, ln, an = online_update(st, qq, krot[g], vb[b, :, g], softmax_scale,
                                           q_pos, k_pos, vis)
                m[b, hi], l[b, hi], acc[b, :, hi] = mn, ln, an
    o = None
    if finalize:
        o = np.zeros_like(acc)
        for b in range(B):
            for hi in range(H):
                o[b, :, hi] = online_finish((m[b, hi], l[b, hi], acc[b, :, hi]))
    return o, m, l, acc


def cache_slot(e: int, n_sink: int, window: int, ring_head: int) -> int:
    """Slot holding the e-th cached entry (sinks first, then the window in
    recency order).  Sinks occupy slots 0..n_sink-1; the window is a ring
    buffer whose oldest entry sits at slot n_sink + ring_head."""
    if e < n_sink:
        return e
    return n_sink + (ring_head + e - n_sink) % window


def decode_sink_window(q, k_cache, v_cache, theta, softmax_scale, n_sink, window,
                       cache_len, ring_head=None, heads=None, layout="half"):
    """One new query per sequence against its sink + window cache.

    q [B, Hq, D] (un-rotated), k_cache/v_cache [B, Hkv, C, D] (un-rotated
    keys), C = n_sink + window.  Entry e (0 <= e < len) sits at position e
    (positions re-indexed inside the cache); the query sits at len - 1
    (its own key/value were appended first).  Every cached entry is
    visible: eviction already applied the sink + window rule.
    Returns o [B, H', D].
    """
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    heads = range(Hq) if heads is None else heads
    # pairs (i, i + d/2), or (2i, 2i+1) for layout "interleaved" (tecvarsity
    # Section 2 pairs the dimensions without fixing which)
    rotate = _rope.rotate_interleaved if layout == "interleaved" else _rope.rotate_half
    out = np.zeros((B, len(heads), np.asarray(v_cache).shape[3]))
    for b in range(B):
        L = int(cache_len[b])
        if L == 0:
            continue
        rh = 0 if ring_head is None else int(ring_head[b])
        slots = np.array([cache_slot(e, n_sink, window, rh) for e in range(L)])
        pos = np.arange(L)
        ck, sk = _rope.tables(theta, pos)
        cq, sq = _rope.tables(theta, [L - 1])
        for hi, h in enumerate(heads):
            g = kv_head(h, Hq, Hkv)
            kk = rotate(np.asarray(k_cache[b, g], np.float64)[slots], ck, sk)
            vv = np.asarray(v_cache[b, g], np.float64)[slots]
            qq = rotate(q[b, h][None, :], cq, sq)
            out[b, hi] = attention_full(qq, kk, vv, softmax_scale, np.array([L - 1]), pos,
                                        all_visible)[0]
    return out
