"""Pins for the fp64 RoPE oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than its own formula:
a worked example printed on the pages, complex-number identities, the
invariants the pages state for RoPE, closed-form regime boundaries, or the
special cases where a rescale must reduce to plain RoPE or to PI.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import rope as R
from yarn_rope_blockwise_amd import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def test_base_frequencies_geometric():
    # theta_0 = 1 and consecutive ratios are base**(-2/d): a geometric ladder
    # (tecvarsity Section 2, theta_i = b^(-2i/d)).
    for d, b in ((64, 1e4), (128, 1e4), (128, 5e5)):
        th = R.base_inv_freq(d, b)
        assert th.shape == (d // 2,)
        assert th[0] == 1.0
        logs = np.log(th)
        np.testing.assert_allclose(np.diff(logs), -2.0 * math.log(b) / d, rtol=0, atol=1e-12)


def test_rotation_is_complex_multiplication():
    # A half-split pair (x_i, x_{i+d/2}) is the complex number x_i + j x_{i+d/2};
    # RoPE multiplies it by exp(j p theta_i).
    rng = np.random.default_rng(11)
    d = 128
    x = rng.standard_normal((7, d))
    pos = np.array([0, 1, 5, 4095, 8000, 131071, 262143])
    th = R.inv_freq(R.YARN, d, 1e4, 8.0, 32768)
    c, s = R.tables(th, pos)
    y = R.rotate_half(x, c, s)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * np.outer(pos, th))
    np.testing.assert_allclose(y[:, : d // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, d // 2:], z.imag, atol=1e-12)
    # interleaved pairs: (x_{2i}, x_{2i+1})
    yi = R.rotate_interleaved(x, c, s)
    zi = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.outer(pos, th))
    np.testing.assert_allclose(yi[:, 0::2], zi.real, atol=1e-12)
    np.testing.assert_allclose(yi[:, 1::2], zi.imag, atol=1e-12)


@settings(max_examples=40, deadline=None)
@given(p=st.integers(0, 262143), kind=st.sampled_from([0, 1, 2, 3]),
       s=st.sampled_from([1.0, 2.0, 4.0, 8.0]))
def test_pair_norm_preserved(p, kind, s):
    # tecvarsity Section 2: the rotation preserves the norm.
    rng = np.random.default_rng(p)
    x = rng.standard_normal(128)
    th = R.inv_freq(kind, 128, 1e4, s, 4096)
    c, sn = R.tables(th, [p])
    y = R.rotate_half(x, c[0], sn[0])
    pair_x = x[:64] ** 2 + x[64:] ** 2
    pair_y = y[:64] ** 2 + y[64:] ** 2
    np.testing.assert_allclose(pair_y, pair_x, rtol=1e-12, atol=1e-12)


@settings(max_examples=40, deadline=None)
@given(m=st.integers(0, 200000), n=st.integers(0, 200000), c=st.integers(-1000, 60000),
       kind=st.sampled_from([0, 1, 2, 3]))
def test_relative_position_invariance(m, n, c, kind):
    # tecvarsity Section 2: <R_m q, R_n k> = q^T R_{n-m} k depends on n - m only.
    if m + c < 0 or n + c < 0:
        return
    rng = np.random.default_rng(m * 7 + n)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    th = R.inv_freq(kind, 128, 1e4, 8.0, 4096)

    def dot(a, b):
        ca, sa = R.tables(th, [a])
        cb, sb = R.tables(th, [b])
        return R.rotate_half(q, ca[0], sa[0]) @ R.rotate_half(k, cb[0], sb[0])

    # fp64 angle rounding at |angle| ~ 2.6e5 is ~3e-11 rad per entry.
    assert abs(dot(m, n) - dot(m + c, n + c)) <= 1e-8 * (np.abs(q) @ np.abs(k))
    # and equals q . R_{n-m} k
    cr, sr = R.tables(th, [n - m])
    assert abs(dot(m, n) - q @ R.rotate_half(k, cr[0], sr[0])) <= 1e-8 * (np.abs(q) @ np.abs(k))


def test_position_zero_is_identity():
    th = R.inv_freq(R.YARN, 128, 1e4, 4.0, 4096)
    c, s = R.tables(th, [0])
    x = np.random.default_rng(0).standard_normal(128)
    assert np.array_equal(R.rotate_half(x, c[0], s[0]), x)


def test_pi_worked_example(golden):
    # 14cs17 "Position Interpolation": 4K->8K, position 8000 behaves as 4000.
    g = golden("pi_worked_example.json")
    assert g["scale"] == g["target_ctx"] / g["train_ctx"]
    for d in (64, 128):
        plain = R.inv_freq(R.PLAIN, d, 1e4)
        pi = R.inv_freq(R.PI, d, 1e4, g["scale"], g["train_ctx"])
        c_pi, s_pi = R.tables(pi, [g["position"]])
        c_pl, s_pl = R.tables(plain, [g["interpolated_position"]])
        assert np.array_equal(c_pi, c_pl) and np.array_equal(s_pi, s_pl)   # bitwise


@pytest.mark.parametrize("kind", [R.PI, R.NTK, R.YARN])
@pytest.mark.parametrize("d,b", [(64, 1e4), (128, 1e4), (128, 5e5)])
def test_unit_scale_reduces_to_plain(kind, d, b):
    plain = R.inv_freq(R.PLAIN, d, b)
    th = R.inv_freq(kind, d, b, 1.0, 4096)
    if kind in (R.PI, R.NTK):
        assert np.array_equal(th, plain)
    else:
        np.testing.assert_allclose(th, plain, rtol=2.3e-16, atol=0)   # <= 1 ulp
    assert R.attn_factor(kind, 1.0) == 1.0


@pytest.mark.parametrize("d,b,s", [(128, 1e4, 8.0), (128, 5e5, 8.0), (64, 1e4, 4.0), (128, 1e4, 4.0)])
def test_ntk_endpoints(d, b, s):
    # High frequencies preserved, the lowest interpolated like PI (14cs17 "NTK-Aware Scaling").
    plain = R.inv_freq(R.PLAIN, d, b)
    ntk = R.inv_freq(R.NTK, d, b, s)
    assert ntk[0] == 1.0
    np.testing.assert_allclose(ntk[-1], plain[-1] / s, rtol=1e-13)
    # every pair's angle shrinks by at most s and the shrink grows monotonically
    ratio = plain / ntk
    assert np.all(ratio >= 1.0 - 1e-15) and np.all(ratio <= s * (1 + 1e-13))
    assert np.all(np.diff(ratio) >= -1e-12)


def test_exercises(golden):
    g = golden("exercises.json")
    e1 = g["exercise1"]
    th = R.base_inv_freq(e1["head_dim"], e1["base"])
    a = R.angles(th, [e1["position"]])[0, e1["pair"]]
    assert a == e1["angle_rad"]
    a_max = R.angles(th, [e1["train_ctx"]])[0, e1["pair"]]
    assert a_max == e1["train_max_angle_rad"]
    assert (a <= a_max) == e1["in_training_range"]
    e2 = g["exercise2"]
    s = e2["target_ctx"] / e2["train_ctx"]
    assert s == e2["scale"]
    b2 = R.ntk_base(e2["head_dim"], e2["base"], s)
    np.testing.assert_allclose(b2, e2["ntk_base_derived"], rtol=1e-12)


def _regime_bounds(d, b, L):
    """Closed-form pair indices where r_i = L/(2 pi b^(2i/d)) crosses beta=32 and alpha=1."""
    def i_at(r):
        return (d / 2.0) * math.log(L / (2 * math.pi * r)) / math.log(b)
    return i_at(32.0), i_at(1.0)


@pytest.mark.parametrize("w", [W.TINY, W.LLAMA_16K, W.GQA_32K[W.YARN], W.RING_SHARE],
                         ids=lambda w: w.name)
def test_yarn_regimes(w):
    # root18d / tecvarsity Section 3: short wavelengths untouched, long ones
    # fully interpolated, a blend in between.
    r = w.rope
    d = r.head_dim
    plain = R.inv_freq(R.PLAIN, d, r.base)
    pi = R.inv_freq(R.PI, d, r.base, r.scale)
    y = R.inv_freq(R.YARN, d, r.base, r.scale, r.orig_ctx)
    i_hi, i_lo = _regime_bounds(d, r.base, r.orig_ctx)
    idx = np.arange(d // 2)
    hi = idx < i_hi          # r > beta
    lo = idx > i_lo          # r < alpha
    mid = ~hi & ~lo
    assert np.array_equal(y[hi], plain[hi])
    assert np.array_equal(y[lo], pi[lo])
    assert np.all(y[mid] < plain[mid]) and np.all(y[mid] > pi[mid])
    # the blend moves monotonically from "no scaling" to "full scaling"
    ratio = plain / y
    assert np.all(np.diff(ratio) >= -1e-12)


def test_yarn_regime_counts_llama16k():
    # d=128, b=1e4, L_train=4096: pairs 0-20 plain, 21-45 ramp, 46-63 PI.
    i_hi, i_lo = _regime_bounds(128, 1e4, 4096)
    assert math.floor(i_hi) == 20 and math.floor(i_lo) == 45


def test_temperature(golden):
    g = golden("yarn_constants.json")
    for case in g["cases"]:
        assert R.attn_factor(R.YARN, case["scale"]) == case["mscale"] ** 2
    for s in (2.0, 4.0, 8.0, 32.0):
        ms = g["mscale_coeff"] * math.log(s) + 1.0
        assert R.attn_factor(R.YARN, s) == pytest.approx(ms * ms, rel=1e-15)
        # only YaRN carries a temperature
        for k in (R.PLAIN, R.PI, R.NTK):
            assert R.attn_factor(k, s) == 1.0
    # constants of the ramp: beta_fast = 32 (beta), beta_slow = 1 (alpha)
    th = R.base_inv_freq(128, 1e4)
    y_default = R.inv_freq(R.YARN, 128, 1e4, 4.0, 4096)
    y_named = R.inv_freq(R.YARN, 128, 1e4, 4.0, 4096, alpha=g["beta_slow"], beta=g["beta_fast"])
    assert np.array_equal(y_default, y_named)
    assert th.shape == y_default.shape


def test_temperature_fold_equivalence():
    # Applying attn_factor as a logit multiplier == scaling both q and k by
    # sqrt(attn_factor) (the listing's mscale on both rotations).
    from oracle import attention as A
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((40, 64)) for _ in range(3))
    f = R.attn_factor(R.YARN, 4.0)
    pos = np.arange(40)
    o1 = A.attention_full(q, k, v, f / 8.0, pos, pos)
    o2 = A.attention_full(q * math.sqrt(f), k * math.sqrt(f), v, 1 / 8.0, pos, pos)
    np.testing.assert_allclose(o1, o2, atol=1e-13)


def test_tables_bshd_positions():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 9, 3, 64))
    th = R.inv_freq(R.YARN, 64, 1e4, 4.0, 128)
    pos = np.arange(9) + 100
    y1 = R.rotate_bshd(x, th, pos)
    y2 = R.rotate_bshd(x, th, np.stack([pos, pos]))
    assert np.array_equal(y1, y2)
    c, s = R.tables(th, pos)
    np.testing.assert_allclose(y1[1, 4, 2], R.rotate_half(x[1, 4, 2], c[4], s[4]), atol=0)


# --- per-pair factor vectors (tecvarsity Section 4, LongRoPE) ---------------

def test_factor_vector_pi_worked_example(golden):
    # A uniform vector lambda_i = s is PI: the same worked example holds
    # bitwise (14cs17 "Position Interpolation": position 8000 behaves as 4000).
    g = golden("pi_worked_example.json")
    for d in (64, 128):
        th = R.inv_freq_factors(d, 1e4, np.full(d // 2, g["scale"]))
        assert np.array_equal(th, R.inv_freq(R.PI, d, 1e4, g["scale"]))
        c_f, s_f = R.tables(th, [g["position"]])
        c_pl, s_pl = R.tables(R.inv_freq(R.PLAIN, d, 1e4), [g["interpolated_position"]])
        assert np.array_equal(c_f, c_pl) and np.array_equal(s_f, s_pl)


def test_factor_vector_unit_is_plain_and_each_pair_is_its_own_pi():
    d, b = 128, 1e4
    assert np.array_equal(R.inv_freq_factors(d, b, np.ones(d // 2)), R.inv_freq(R.PLAIN, d, b))
    # non-uniform: pair i interpolated by its own lambda_i, others untouched
    lam = np.ones(d // 2)
    lam[[3, 40, 63]] = [2.0, 8.0, 64.0]
    th = R.inv_freq_factors(d, b, lam)
    plain = R.inv_freq(R.PLAIN, d, b)
    for i, s in ((3, 2.0), (40, 8.0), (63, 64.0)):
        assert th[i] == R.inv_freq(R.PI, d, b, s)[i]
    keep = np.setdiff1d(np.arange(d // 2), [3, 40, 63])
    assert np.array_equal(th[keep], plain[keep])
    # a position p with factor lambda sees the angle plain pair i has at p / lambda
    c, s_ = R.tables(th, [640])
    c2, s2 = R.tables(plain, [10])        # 640 / 64 for pair 63
    assert c[0, 63] == c2[0, 63] and s_[0, 63] == s2[0, 63]


def test_factor_vector_expresses_yarn():
    # YaRN's theta' written as a per-pair vector lambda_i = theta_i / theta'_i
    w = W.LLAMA_16K.rope
    yarn = R.inv_freq(R.YARN, w.head_dim, w.base, w.scale, w.orig_ctx, w.alpha, w.beta)
    lam = R.base_inv_freq(w.head_dim, w.base) / yarn
    assert np.all(lam >= 1.0 - 1e-15) and np.all(lam <= w.scale * (1 + 1e-15))
    np.testing.assert_allclose(R.inv_freq_factors(w.head_dim, w.base, lam), yarn, rtol=4.5e-16)


@pytest.mark.parametrize("bad", [0.0, -1.0, float("nan"), float("inf")])
def test_factor_vector_rejects_bad_values(bad):
    lam = np.ones(64)
    lam[5] = bad
    with pytest.raises(ValueError):
        R.inv_freq_factors(128, 1e4, lam)
    with pytest.raises(ValueError):
        R.inv_freq_factors(128, 1e4, np.ones(63))
