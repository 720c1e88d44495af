"""GPU check of attn_prefill_blockwise_noalloc, the variant for callers that
cannot allocate: through the C ABI its output equals attn_prefill_blockwise
(with a workspace of its own) bit for bit, on two calls in a row, the second
with a smaller input; the call leaves torch's allocation count unchanged
(the output buffer is the caller's)."""
import pytest

from oracle import attention as A
from oracle import rope as R
from yarn_rope_blockwise_amd import api
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, draw, host, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,Hq,Hkv", [(4096, 8, 4), (1500, 4, 2)])
def test_noalloc_prefill_equals_workspace_prefill(S, Hq, Hkv):
    # 128 and 24 workgroups: both grids claim their last items from the
    # counter, the second from the array the first call left behind.
    require_gpu()
    import torch
    D = 128
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 1024)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), S)
    scale = R.softmax_scale(rope.kind, rope.scale, D)
    qv, q = draw((1, S, Hq, D), 600 + S, "bf16")
    kv, k = draw((1, S, Hkv, D), 601 + S, "bf16")
    vv, v = draw((1, S, Hkv, D), 602 + S, "bf16")
    kr = api.rope_apply(k, tab)
    say(f"attn_prefill_blockwise_noalloc S={S} Hq={Hq} Hkv={Hkv}")
    ref = api.attn_prefill_blockwise(q, kr, v, scale, cos_sin=tab, workspace=api.new_workspace())
    out = torch.full_like(q, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(3):
        api.attn_prefill_blockwise_noalloc(q, kr, v, scale, cos_sin=tab, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert torch.cuda.memory_allocated() == before
    rows = [0, 1, 255, 256, S // 2, S - 1]
    assert max_abs(host(out[0, rows]), A.prefill(qv, kv, vv, th, scale, rows=rows)[0]) <= BF16_TOL
