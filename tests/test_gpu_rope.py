"""GPU parity: cos/sin tables and the pair-rotation pass against the fp64 oracle."""
import numpy as np
import pytest

from oracle import rope as R
from yarn_rope_blockwise_amd import api
from yarn_rope_blockwise_amd import workloads as W
from tests.gpu_helpers import (BF16_TOL, F32_TOL, TABLE_TOL, draw, host, max_abs, require_gpu,
                               say)

pytestmark = pytest.mark.gpu

TABLE_CASES = [
    ("tiny_yarn4", W.TINY.rope, 512),
    ("llama16k_yarn4", W.LLAMA_16K.rope, 16384),
    ("gqa32k_pi8", W.GQA_32K[W.PI].rope, 32768),
    ("gqa32k_ntk8", W.GQA_32K[W.NTK].rope, 32768),
    ("gqa32k_yarn8", W.GQA_32K[W.YARN].rope, 32768),
    ("decode_plain", W.SINK_DECODE.rope, 4100),
    ("ring_yarn8_262144", W.RING_SHARE.rope, 262144),
]


@pytest.mark.parametrize("name,rope,n", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_tables_match_oracle(name, rope, n):
    require_gpu()
    say(f"rope_tables_build {name} n_pos={n}")
    cfg = api.RopeConfig.of(rope)
    tab, th, af = api.rope_tables_build(cfg, n)
    got = host(tab)
    ref_th = R.inv_freq(rope.kind, rope.head_dim, rope.base, rope.scale, rope.orig_ctx,
                        rope.alpha, rope.beta)
    np.testing.assert_allclose(th, ref_th, rtol=1e-12, atol=0)
    assert af == pytest.approx(R.attn_factor(rope.kind, rope.scale), rel=1e-15)
    c, s = R.tables(ref_th, np.arange(n))
    err = max(max_abs(got[..., 0], c), max_abs(got[..., 1], s))
    assert err <= TABLE_TOL, err


@pytest.mark.parametrize("d,n,pos0", [(128, 16384, 0), (64, 4100, 12345)])
def test_factor_tables_match_oracle(d, n, pos0):
    # Per-pair factors (tecvarsity Section 4): a non-uniform vector, rows at
    # an offset; every entry against the fp64 oracle.
    require_gpu()
    say(f"rope_tables_build_factors d={d} n_pos={n} pos0={pos0}")
    lam = np.sort(np.random.default_rng(d + n).uniform(1.0, 64.0, d // 2))
    tab, th = api.rope_tables_build_factors(d, 1e4, lam, n, pos0=pos0)
    ref_th = R.inv_freq_factors(d, 1e4, lam)
    np.testing.assert_allclose(th, ref_th, rtol=1e-14, atol=0)
    got = host(tab)
    c, s = R.tables(ref_th, np.arange(pos0, pos0 + n))
    err = max(max_abs(got[..., 0], c), max_abs(got[..., 1], s))
    assert err <= TABLE_TOL, err


def test_factor_tables_uniform_equal_pi_tables():
    # lambda_i = s for every pair is PI: the two entry points give the same table, bitwise.
    require_gpu()
    import torch
    say("rope_tables_build_factors uniform vs PI")
    rope = W.GQA_32K[W.PI].rope
    tab_pi, _, _ = api.rope_tables_build(api.RopeConfig.of(rope), 8192)
    tab_f, _ = api.rope_tables_build_factors(rope.head_dim, rope.base,
                                             np.full(rope.head_dim // 2, rope.scale), 8192)
    torch.cuda.synchronize()
    assert torch.equal(tab_pi, tab_f)


def test_tables_offset_rows():
    require_gpu()
    rope = W.RING_SHARE.rope
    say("rope_tables_build pos0=229376 n_pos=4096")
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), 4096, pos0=229376)
    c, s = R.tables(th, 229376 + np.arange(4096))
    got = host(tab)
    assert max(max_abs(got[..., 0], c), max_abs(got[..., 1], s)) <= TABLE_TOL


@pytest.mark.parametrize("d,n,pos0", [(128, 1, 0), (64, 15, 7), (128, 17, 1000003), (64, 33, 262127),
                                      (128, 4111, 16)])
def test_tables_ragged_row_groups(d, n, pos0):
    # Rows are written 16 to a thread (the first from its reduced angle, the
    # rest by angle addition): counts and offsets that cut those groups
    # short, and positions far past the tables above, against the oracle.
    require_gpu()
    say(f"rope_tables_build_factors d={d} n_pos={n} pos0={pos0}")
    lam = np.linspace(1.0, 8.0, d // 2)
    tab, th = api.rope_tables_build_factors(d, 1e4, lam, n, pos0=pos0)
    got = host(tab)
    c, s = R.tables(th, pos0 + np.arange(n))
    assert max(max_abs(got[..., 0], c), max_abs(got[..., 1], s)) <= TABLE_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_apply(dtype, D):
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    B, S, H = 2, 300, 3
    say(f"rope_apply {dtype} D={D} B={B} S={S} H={H}")
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), 600)
    xv, x = draw((B, S, H, D), 7, dtype)
    y = api.rope_apply(x, tab, pos_offset=17)
    torch.cuda.synchronize()
    ref = R.rotate_bshd(xv, th, 17 + np.arange(S))
    err = max_abs(host(y), ref)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert err <= tol, err
    if dtype == "bf16":
        # elementwise within one bf16 ulp of the exact rotation (fp32 math, RNE store)
        ulp = 2.0 ** (np.floor(np.log2(np.abs(ref) + 1e-30)) - 7)
        assert np.all(np.abs(host(y) - ref) <= ulp + 2.0 ** -20)
    # in place gives the same bits
    x2 = x.clone()
    api.rope_apply(x2, tab, pos_offset=17, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2, y)


def test_rope_apply_strided_and_pos_ids():
    require_gpu()
    import torch
    D = 128
    rope = W.Rope(W.NTK, D, 5e5, 8.0)
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), 1000)
    xv, x = draw((2, 50, 6, D), 8, "bf16")
    xs = x[:, :, 1:5]                       # non-contiguous head slice
    pos = np.random.default_rng(3).integers(0, 1000, size=(2, 50)).astype(np.int32)
    pos[1, 7] = 1000                        # out of table range -> NaN row
    say("rope_apply strided heads + pos_ids")
    y = api.rope_apply(xs, tab, pos_ids=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got = host(y)
    assert np.isnan(got[1, 7]).all()
    ok = np.ones((2, 50), bool)
    ok[1, 7] = False
    pos_ok = np.where(ok, pos, 0)
    ref = R.rotate_bshd(xv[:, :, 1:5], th, pos_ok)
    assert max_abs(got[ok], ref[ok]) <= BF16_TOL


def test_rope_apply_full_size_keys():
    # K of the Llama-7B-like 16k prefill, rotated at positions 0..16383.
    require_gpu()
    import torch
    w = W.LLAMA_16K
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(w.rope), w.seq)
    kv, k = draw((1, w.seq, w.n_kv_heads, w.head_dim), 1, "bf16")
    say("rope_apply llama16k K [1,16384,32,128]")
    y = api.rope_apply(k, tab)
    torch.cuda.synchronize()
    rows = np.r_[0:8, 4090:4100, 16376:16384]
    got = host(y[0, rows])
    ref = R.rotate_bshd(kv[:, rows], th, rows)[0]
    assert max_abs(got, ref) <= BF16_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_apply_interleaved(dtype, D):
    # Adjacent pairs (x_{2i}, x_{2i+1}) through rope_apply_ex, strided rows
    # and per-token positions, against the oracle's interleaved rotation.
    require_gpu()
    import torch
    rope = W.Rope(W.YARN, D, 1e4, 4.0, 128)
    B, S, H = 2, 300, 3
    say(f"rope_apply_ex interleaved {dtype} D={D}")
    tab, th, _ = api.rope_tables_build(api.RopeConfig.of(rope), 700)
    xv, xb = draw((B, S, 2 * H, D), 9, dtype)
    x = xb[:, :, ::2]                                 # every other head: strided rows
    pos = np.random.default_rng(3).integers(0, 700, size=(B, S)).astype(np.int32)
    y = api.rope_apply_ex(x, tab, layout=api.LAYOUT_INTERLEAVED,
                          pos_ids=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = np.empty((B, S, H, D))
    for b in range(B):
        c, s = R.tables(th, pos[b])
        ref[b] = R.rotate_interleaved(np.asarray(xv[b, :, ::2], np.float64), c[:, None, :],
                                      s[:, None, :])
    err = max_abs(host(y), ref)
    assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL), err
