"""Host-side checks of libyrb.so that need no GPU.

* the library loads and exports every function include/yrb.h declares;
* the fp64 frequencies and temperature computed on the host by the library
  match the oracle;
* invalid arguments are rejected with the documented status before anything
  is launched (these calls never reach the HIP runtime).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import rope as R
from yarn_rope_blockwise_amd import api
from yarn_rope_blockwise_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "yrb.h")

OK, EINVAL, EUNSUP, EALIGN = 0, -1, -2, -3
FAKE = 0x10000          # 16-byte aligned non-null address; never dereferenced
MISALIGNED = 0x10008


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:YRB_API\s+)?(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", txt,
                                 flags=re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("rope_tables_build", "rope_tables_build_factors", "rope_apply", "attn_prefill_blockwise", "attn_prefill_sink_window",
              "attn_block_accumulate", "attn_decode_sink_window", "yrb_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = api.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.yrb_status_str(0) == b"ok"
    assert L.yrb_status_str(-2).startswith(b"unsupported")


def test_library_exports_nothing_else():
    # Built with hidden visibility: the functions the header declares are the
    # library's only exported code; internal launchers and kernels stay local.
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("needs nm")
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    assert funcs == set(declared_functions()), funcs ^ set(declared_functions())


@pytest.mark.parametrize("kind", [R.PLAIN, R.PI, R.NTK, R.YARN])
@pytest.mark.parametrize("w", [W.TINY.rope, W.LLAMA_16K.rope, W.GQA_32K[W.YARN].rope,
                               W.RING_SHARE.rope], ids=["tiny", "llama16k", "gqa32k", "ring"])
def test_host_frequencies_match_oracle(kind, w):
    cfg = api.RopeConfig(kind, w.head_dim, w.base, w.scale, w.orig_ctx, w.alpha, w.beta)
    th, af = api.rope_frequencies(cfg)
    ref = R.inv_freq(kind, w.head_dim, w.base, w.scale, w.orig_ctx, w.alpha, w.beta)
    np.testing.assert_allclose(th, ref, rtol=1e-14, atol=0)
    assert af == pytest.approx(R.attn_factor(kind, w.scale), rel=1e-15)


def _tables(cfg_kw, **over):
    kw = dict(kind=3, head_dim=128, base=1e4, scale=4.0, orig_ctx=4096, alpha=1.0, beta=32.0)
    kw.update(cfg_kw)
    c = api.YrbRopeConfig(**kw)
    a = dict(pos0=0, n_pos=0, cos_sin=None)
    a.update(over)
    return api.lib().rope_tables_build(ctypes.byref(c), a["pos0"], a["n_pos"], a["cos_sin"],
                                       None, None, None)


@pytest.mark.parametrize("kw,expect", [
    ({}, OK),
    ({"kind": 7}, EINVAL),
    ({"head_dim": 96}, EUNSUP),
    ({"head_dim": 130}, EUNSUP),
    ({"base": 1.0}, EINVAL),
    ({"scale": 0.0}, EINVAL),
    ({"scale": -2.0}, EINVAL),
    ({"alpha": 32.0, "beta": 1.0}, EINVAL),
    ({"orig_ctx": 0}, EINVAL),
])
def test_rope_tables_config_validation(kw, expect):
    assert _tables(kw) == expect


def test_rope_tables_pointer_validation():
    assert _tables({}, n_pos=4, cos_sin=None) == EINVAL
    assert _tables({}, n_pos=4, cos_sin=MISALIGNED) == EALIGN
    assert _tables({}, n_pos=-1) == EINVAL
    assert _tables({}, pos0=-5) == EINVAL


@pytest.mark.parametrize("d", [64, 128])
def test_host_factor_frequencies_match_oracle(d):
    lam = np.random.default_rng(d).uniform(1.0, 64.0, d // 2)
    th = api.rope_frequencies_factors(d, 5e5, lam)
    np.testing.assert_allclose(th, R.inv_freq_factors(d, 5e5, lam), rtol=1e-14, atol=0)
    # a uniform vector is PI, bitwise: the same fp64 division
    pi, _ = api.rope_frequencies(api.RopeConfig(R.PI, d, 1e4, 8.0, 4096, 1.0, 32.0))
    assert np.array_equal(api.rope_frequencies_factors(d, 1e4, np.full(d // 2, 8.0)), pi)


def _factors(head_dim=128, base=1e4, lam="ones", pos0=0, n_pos=0, cos_sin=None):
    if isinstance(lam, str):
        lam = np.ones(head_dim // 2)
    ptr = None if lam is None else np.ascontiguousarray(lam, np.float64).ctypes.data_as(api._dp)
    return api.lib().rope_tables_build_factors(head_dim, base, ptr, pos0, n_pos, cos_sin, None,
                                               None)


def test_rope_tables_factors_validation():
    assert _factors() == OK
    assert _factors(head_dim=96) == EUNSUP
    assert _factors(base=1.0) == EINVAL
    assert _factors(base=float("inf")) == EINVAL
    assert _factors(lam=None) == EINVAL
    for bad in (0.0, -2.0, float("nan"), float("inf")):
        lam = np.ones(64)
        lam[7] = bad
        assert _factors(lam=lam) == EINVAL
    assert _factors(n_pos=4, cos_sin=None) == EINVAL
    assert _factors(n_pos=4, cos_sin=MISALIGNED) == EALIGN
    assert _factors(pos0=-1) == EINVAL


def _strides(*v):
    return api._arr(v)


def test_rope_apply_validation():
    L = api.lib()
    s = _strides(8 * 128 * 32, 128 * 32, 128)
    args = dict(x=FAKE, y=FAKE, dtype=0, B=1, S=8, H=32, D=128, xs=s, ys=s, cs=FAKE, rows=8,
                off=0, pos=None, st=None)

    def call(**over):
        a = dict(args)
        a.update(over)
        return L.rope_apply(a["x"], a["y"], a["dtype"], a["B"], a["S"], a["H"], a["D"], a["xs"],
                            a["ys"], a["cs"], a["rows"], a["off"], a["pos"], a["st"])
    assert call(D=80) == EUNSUP
    assert call(dtype=5) == EUNSUP
    assert call(x=None) == EINVAL
    assert call(cs=None) == EINVAL
    assert call(x=MISALIGNED) == EALIGN
    assert call(xs=_strides(8 * 128 * 32, 128 * 32, 132)) == EALIGN     # 264-byte head stride
    assert call(rows=7) == EINVAL                                        # table too short
    assert call(off=1) == EINVAL                                         # off + S > rows
    assert call(B=-1) == EINVAL
    assert call(B=0) == OK                                               # nothing to do
    assert call(ys=_strides(8 * 128 * 32, 1 << 31, 128)) == EINVAL       # stride >= 2^31 elements


def _prefill(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, B=1, S=64, Hq=4, Hkv=2, D=128,
             strides=_strides(*([64 * 4 * 128, 4 * 128, 128] * 4)), cs=FAKE, rows=64,
             scale=0.1, causal=1, lse=None, ws=None)
    a.update(over)
    return L.attn_prefill_blockwise(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["B"], a["S"],
                                    a["Hq"], a["Hkv"], a["D"], a["strides"], a["cs"], a["rows"],
                                    ctypes.c_float(a["scale"]), a["causal"], a["lse"], a["ws"],
                                    None)


def test_prefill_validation():
    assert _prefill(Hq=3) == EINVAL            # Hq % Hkv
    assert _prefill(Hkv=0) == EINVAL
    assert _prefill(D=32) == EUNSUP
    assert _prefill(causal=2) == EINVAL
    assert _prefill(scale=0.0) == EINVAL
    assert _prefill(scale=float("nan")) == EINVAL
    assert _prefill(q=None) == EINVAL
    assert _prefill(cs=MISALIGNED) == EALIGN
    assert _prefill(rows=63) == EINVAL         # table shorter than S
    assert _prefill(o=MISALIGNED) == EALIGN
    big = 1 << 31                              # strides are indexed in 32 bits
    assert _prefill(strides=_strides(*([64 * 4 * 128, big, 128] + [64 * 4 * 128, 4 * 128, 128] * 3))) == EINVAL
    assert _prefill(strides=_strides(*([64 * 4 * 128, 4 * 128, 128] * 3 + [-128, 4 * 128, 128]))) == EINVAL
    assert _prefill(lse=MISALIGNED) == EALIGN
    assert _prefill(ws=MISALIGNED) == EALIGN
    assert _prefill(S=0) == OK
    assert _prefill(B=0) == OK


def _prefill_sw(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, B=1, S=64, Hq=4, Hkv=2, D=128,
             strides=_strides(*([64 * 4 * 128, 4 * 128, 128] * 4)), cs=FAKE, rows=64,
             scale=0.1, sink=4, win=32, lse=None, ws=None)
    a.update(over)
    return L.attn_prefill_sink_window(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["B"], a["S"],
                                      a["Hq"], a["Hkv"], a["D"], a["strides"], a["cs"], a["rows"],
                                      ctypes.c_float(a["scale"]), a["sink"], a["win"], a["lse"],
                                      a["ws"], None)


def test_prefill_sink_window_validation():
    # Every call fails before a launch (or has nothing to do).
    assert _prefill_sw(dtype=1) == EUNSUP      # bf16 only
    assert _prefill_sw(sink=-1) == EINVAL
    assert _prefill_sw(win=0) == EINVAL
    assert _prefill_sw(win=-5) == EINVAL
    assert _prefill_sw(S=1 << 30, rows=1 << 30) == EINVAL
    assert _prefill_sw(Hq=3) == EINVAL
    assert _prefill_sw(D=32) == EUNSUP
    assert _prefill_sw(scale=0.0) == EINVAL
    assert _prefill_sw(rows=63) == EINVAL
    assert _prefill_sw(q=None) == EINVAL
    assert _prefill_sw(o=MISALIGNED) == EALIGN
    assert _prefill_sw(ws=MISALIGNED) == EALIGN
    assert _prefill_sw(S=0) == OK
    assert _prefill_sw(B=0, sink=1 << 40, win=1 << 40) == OK


def _prefill_chunk(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, B=1, Sq=64, Sk=128, Hq=4, Hkv=2, D=128,
             strides=_strides(*([64 * 4 * 128, 4 * 128, 128] * 4)), qo=64, cs=FAKE, rows=128,
             scale=0.1, sink=4, win=32, lse=None, ws=None)
    a.update(over)
    return L.attn_prefill_sink_window_chunk(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["B"], a["Sq"],
                                            a["Sk"], a["Hq"], a["Hkv"], a["D"], a["strides"], a["qo"],
                                            a["cs"], a["rows"], ctypes.c_float(a["scale"]), a["sink"],
                                            a["win"], a["lse"], a["ws"], None)


def test_prefill_sink_window_chunk_validation():
    # Every call fails before a launch (or has nothing to do); calls whose
    # sizes pass stop at the misaligned q.
    assert _prefill_chunk(dtype=1) == EUNSUP
    assert _prefill_chunk(qo=-1) == EINVAL
    assert _prefill_chunk(Sk=-1) == EINVAL
    assert _prefill_chunk(Sq=-1) == EINVAL
    assert _prefill_chunk(sink=-1) == EINVAL
    assert _prefill_chunk(win=0) == EINVAL
    assert _prefill_chunk(rows=127) == EINVAL                    # q_offset + Sq > table rows
    assert _prefill_chunk(qo=(1 << 30) - 10, rows=1 << 31) == EINVAL
    assert _prefill_chunk(Sk=1 << 30) == EINVAL
    assert _prefill_chunk(k=None) == EINVAL                     # keys missing while Sk > 0
    assert _prefill_chunk(q=MISALIGNED, k=None, v=None, Sk=0) == EALIGN   # no keys: K/V may be NULL
    assert _prefill_chunk(q=MISALIGNED, cs=None, rows=0) == EALIGN        # q already rotated: no table
    assert _prefill_chunk(q=MISALIGNED, sink=1 << 40, win=1 << 40) == EALIGN
    assert _prefill_chunk(q=MISALIGNED) == EALIGN
    assert _prefill_chunk(Sq=0) == OK
    assert _prefill_chunk(B=0) == OK


def _accum(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=0, B=1, Sq=64, Sk=64, Hq=2, Hkv=2, D=64,
             strides=_strides(*([64 * 2 * 64, 2 * 64, 64] * 3)), qo=64, ko=0, cs=FAKE, rows=128,
             scale=0.1, causal=1, acc=FAKE, m=FAKE, l=FAKE, flags=1, out=None, os=None, ws=None)
    a.update(over)
    return L.attn_block_accumulate(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["Sq"], a["Sk"],
                                   a["Hq"], a["Hkv"], a["D"], a["strides"], a["qo"], a["ko"],
                                   a["cs"], a["rows"], ctypes.c_float(a["scale"]),
                                   a["causal"], a["acc"], a["m"], a["l"], a["flags"], a["out"],
                                   a["os"], a["ws"], None)


def test_accumulate_validation():
    assert _accum(flags=4) == EINVAL
    assert _accum(flags=2) == EINVAL            # FINALIZE without output / strides
    assert _accum(flags=2, out=FAKE) == EINVAL  # no output strides
    assert _accum(qo=-1) == EINVAL
    assert _accum(rows=127) == EINVAL           # q_offset + Sq > rows
    assert _accum(qo=2 ** 31 - 10) == EINVAL    # positions must fit 31 bits
    assert _accum(m=None) == EINVAL
    assert _accum(acc=MISALIGNED) == EALIGN
    assert _accum(cs=MISALIGNED) == EALIGN
    assert _accum(ws=MISALIGNED) == EALIGN
    assert _accum(dtype=2) == EUNSUP
    assert _accum(Sq=0) == OK


def _decode(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=0, B=2, Hq=4, Hkv=4, D=128, sink=4, win=60,
             qs=_strides(512, 128), cs=_strides(4 * 64 * 128, 64 * 128, 128),
             os=_strides(512, 128), len=FAKE, rh=None, tab=FAKE, rows=64, scale=0.1)
    a.update(over)
    return L.attn_decode_sink_window(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["B"], a["Hq"],
                                     a["Hkv"], a["D"], a["sink"], a["win"], a["qs"], a["cs"],
                                     a["os"], a["len"], a["rh"], a["tab"], a["rows"],
                                     ctypes.c_float(a["scale"]), None)


def test_decode_validation():
    assert _decode(dtype=1) == EUNSUP           # the decode path is bf16
    assert _decode(Hq=12, Hkv=4) == EUNSUP      # group of 3 query heads
    assert _decode(Hq=6, Hkv=4) == EINVAL
    assert _decode(win=0) == EINVAL
    assert _decode(sink=-1) == EINVAL
    assert _decode(rows=63) == EINVAL           # table shorter than the cache
    assert _decode(len=None) == EINVAL
    assert _decode(k=MISALIGNED) == EALIGN
    assert _decode(cs=_strides(4 * 64 * 128, 64 * 128, 100)) == EALIGN
    assert _decode(B=0) == OK
    # 32-bit offsets inside one (sequence, head): entries, entry stride, span.
    # A call within the limits stops at the next check (a misaligned query).
    assert _decode(sink=1, win=(1 << 24) - 1, rows=1 << 24, cs=_strides(0, 0, 0), q=MISALIGNED) == EALIGN
    assert _decode(sink=2, win=(1 << 24) - 1, rows=1 << 25, cs=_strides(0, 0, 0)) == EINVAL
    assert _decode(cs=_strides(0, 0, (1 << 23) - 8), q=MISALIGNED) == EALIGN
    assert _decode(cs=_strides(0, 0, 1 << 23)) == EINVAL                 # 2^24 bytes per entry
    # 2^14 entries of 2^18 bytes: the last byte at 2^32 - 2^18 + 255; one entry more passes 2^32
    assert _decode(win=(1 << 14) - 4, rows=1 << 15, cs=_strides(0, 0, 1 << 17), q=MISALIGNED) == EALIGN
    assert _decode(win=(1 << 14) - 3, rows=1 << 15, cs=_strides(0, 0, 1 << 17)) == EINVAL


def _decode_fp8(**over):
    L = api.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=2, Hq=4, Hkv=4, D=128, sink=4, win=60,
             qs=_strides(512, 128), cs=_strides(4 * 64 * 128, 64 * 128, 128),
             os=_strides(512, 128), len=FAKE, rh=None, ks=None, vs=None, tab=FAKE, rows=64,
             scale=0.1)
    a.update(over)
    return L.attn_decode_sink_window_fp8(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"],
                                         a["Hkv"], a["D"], a["sink"], a["win"], a["qs"], a["cs"],
                                         a["os"], a["len"], a["rh"], a["ks"], a["vs"], a["tab"],
                                         a["rows"], ctypes.c_float(a["scale"]), None)


def test_decode_fp8_validation():
    # every call here fails validation (or has B = 0), so nothing is launched
    assert _decode_fp8(B=0) == OK
    assert _decode_fp8(D=96) == EUNSUP
    assert _decode_fp8(Hq=12, Hkv=4) == EUNSUP
    assert _decode_fp8(win=0) == EINVAL
    assert _decode_fp8(rows=63) == EINVAL
    assert _decode_fp8(len=None) == EINVAL
    assert _decode_fp8(k=MISALIGNED) == EALIGN
    assert _decode_fp8(cs=_strides(4 * 64 * 128, 64 * 128, 136)) == EALIGN   # 136-byte slot stride
    assert _decode_fp8(ks=MISALIGNED) == EALIGN
    assert _decode_fp8(o=MISALIGNED) == EALIGN


def test_layout_validation():
    # an unknown layout or cache type is rejected before anything is launched
    L = api.lib()
    s = _strides(8 * 128 * 32, 128 * 32, 128)
    assert L.rope_apply_ex(FAKE, FAKE, 0, 1, 8, 32, 128, s, s, FAKE, 8, 0, None, 2, None) == EINVAL
    assert L.rope_apply_ex(FAKE, FAKE, 0, 0, 8, 32, 128, s, s, FAKE, 8, 0, None, 1, None) == OK
    qs, cs, os_ = _strides(512, 128), _strides(4 * 64 * 128, 64 * 128, 128), _strides(512, 128)
    args = (FAKE, FAKE, FAKE, FAKE)
    tail = (4, 4, 128, 4, 60, qs, cs, os_, FAKE, None, None, None, FAKE, 64,
            ctypes.c_float(0.1), None)
    assert L.attn_decode_sink_window_ex(*args, 0, 2, 2, *tail) == EINVAL     # layout 2
    assert L.attn_decode_sink_window_ex(*args, 1, 0, 2, *tail) == EUNSUP     # f32 cache
    assert L.attn_decode_sink_window_ex(*args, 0, 1, 0, *tail) == OK         # B = 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(api, "_lib", None)
    with pytest.raises(ImportError):
        api.lib()
