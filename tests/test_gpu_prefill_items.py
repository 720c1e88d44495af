"""GPU: prefill launches over many heads against launches over slices of 8.

A prefill launch has one work item per (batch, head, 256-row query tile).
Items go to blocks with the heads regrouped so that the blocks an XCD runs
together share key/value heads, the heaviest causal query tiles first, and
the last 30 % of blocks claim their items from the workspace counter.  An
item's arithmetic does not depend on the block that runs it, so a launch
over hundreds of heads (a thousand or more items) must give, bit for bit,
the output and log-sum-exp of launches over 8-head slices of the same
tensors (strided views); outputs start as NaN, so an item skipped or
written twice shows.  Sampled rows of a few heads are also checked against
the fp64 oracle.
"""
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api, synth
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, draw, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu

SLICE = 8                 # heads per reference launch

CASES = [
    # name, B, S, D, Hq, G (query heads per kv head), causal, n_sink, window
    ("causal_d128_ragged", 1, 800, 128, 512, 8, True, 0, 0),     # last query tile: wave 0 only
    ("causal_d64", 1, 1000, 64, 256, 1, True, 0, 0),
    ("full_d128", 1, 520, 128, 352, 4, False, 0, 0),
    ("causal_b2_d128", 2, 600, 128, 176, 8, True, 0, 0),
    ("sink_window_d128", 1, 1000, 128, 512, 8, True, 4, 300),
    ("window_d64_no_sinks", 1, 900, 64, 256, 2, True, 0, 129),
]


def _call(q, k, v, tab, scale, causal, n_sink, window, out, lse):
    if window:
        return api.attn_prefill_sink_window(q, k, v, scale, n_sink, window, cos_sin=tab, out=out, lse=lse,
                                            workspace=api.new_workspace())
    return api.attn_prefill_blockwise(q, k, v, scale, cos_sin=tab, causal=causal, out=out, lse=lse,
                                      workspace=api.new_workspace())


@pytest.mark.parametrize("name,B,S,D,Hq,G,causal,n_sink,window", CASES, ids=[c[0] for c in CASES])
def test_prefill_many_heads_match_slices(name, B, S, D, Hq, G, causal, n_sink, window):
    require_gpu()
    import torch
    Hkv = Hq // G
    assert SLICE % G == 0
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), S)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    qv, q = draw((B, S, Hq, D), 900 + S, "bf16")
    kv, k = draw((B, S, Hkv, D), 901 + S, "bf16")
    vv, v = draw((B, S, Hkv, D), 902 + S, "bf16")
    kr = api.rope_apply(k, tab)
    del k
    say(f"prefill {name}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} in one launch")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    _call(q, kr, v, tab, scale, causal, n_sink, window, o, lse)
    torch.cuda.synchronize()

    say(f"prefill {name}: the same heads {SLICE} at a time")
    o1 = torch.full_like(q, float("nan"))
    lse1 = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device="cuda")
    for h0 in range(0, Hq, SLICE):
        g0, g1 = h0 // G, (h0 + SLICE) // G
        ls = torch.empty((B, SLICE, S), dtype=torch.float32, device="cuda")
        _call(q[:, :, h0:h0 + SLICE], kr[:, :, g0:g1], v[:, :, g0:g1], tab, scale, causal, n_sink, window,
              o1[:, :, h0:h0 + SLICE], ls)
        lse1[:, h0:h0 + SLICE] = ls
    torch.cuda.synchronize()
    assert not torch.isnan(o).any()
    assert torch.equal(o, o1)
    assert torch.equal(lse, lse1)

    # sampled rows of a few heads against the oracle
    worst = 0.0
    for b in range(B):
        for h in (0, Hq // 3, Hq - 1):
            rows = synth.sample_rows(S, 24, 3000 + 7 * h + b, must=[0, 1, 255, 256, S - 1])
            g = h // G
            ref = A.prefill(qv[b:b + 1, :, h:h + 1], kv[b:b + 1, :, g:g + 1], vv[b:b + 1, :, g:g + 1], th, scale,
                            causal=causal, n_sink=n_sink, window=window, rows=rows)[0, :, 0]
            worst = max(worst, max_abs(host(o[b, rows, h]), ref))
    assert worst <= BF16_TOL, worst
