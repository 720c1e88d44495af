"""Inputs that force the online softmax's rescale of a non-empty accumulator
(no test functions here).

The running max that a blockwise kernel keeps per query row ("Ring
attention" in the jovanaeducation guide, "Ring Attention" in the 14cs17
notes) only has to rescale what it accumulated when a later key beats it.
With N(0,1) inputs that almost never happens by a wide margin, and the
kernels here move their exponent reference lazily: only when a 32-key
quarter's max exceeds it by more than TAU = 8 (log2 units).  These inputs
make it happen on purpose:

* keys of chosen 32-key quarters are multiplied by a power of two (exact in
  bf16), so their logits are that many times larger and a row's max jumps
  by 10 to 30 log2 units when the walk reaches them;
* the rope table turns every pair by a quarter turn per position (per-pair
  factors with theta'_i = pi/2), so cos and sin are 0 or +-1 and the
  rotation is a signed permutation, exact in bf16; with softmax_scale =
  2^-3 / log2(e) the scaled query is exact as well.  The logits the kernel
  forms are then those of the fp64 oracle up to fp32 accumulation, and the
  bf16 tolerance measures only the rounding of P and of the output, not the
  bf16 rounding of large logits.

`rescale_events` walks rows through their quarters in a given order and
counts the jumps past TAU of a reference that is already finite: each is a
rescale of a non-empty accumulator.  Tests assert a minimum count so that
they cannot pass without taking that path.
"""
from __future__ import annotations

import numpy as np

from yarn_rope_blockwise_amd import synth

TAU = 8.0                                  # log2 units
# Values are N(0,1) halved.  Logits this large put a row's softmax on one or
# two keys, so its output is close to a single value row; at |o| in [2, 4)
# the bf16 output rounding alone is up to 2^-8 and the bf16 rounding of P
# adds up to 2^-9 |v|, together above the 2e-2 bound that holds for the
# averaged outputs of N(0,1) inputs.  Halving V (exact) halves both.
V_SCALE = 0.5
QUARTER = 32
SCALE_EXACT = float(np.float32(0.125 / np.log2(np.e)))   # q * scale * log2(e) ~= q / 8


def quarter_turn_factors(head_dim: int, base: float = 1e4) -> np.ndarray:
    """lambda_i with theta_i / lambda_i = pi/2 for every pair (fp64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / head_dim) / (np.pi / 2.0)


def quarter_multipliers(n_keys: int, pattern) -> np.ndarray:
    """Multiplier of key j: pattern[(j // 32) % len(pattern)]."""
    j = np.arange(n_keys)
    return np.asarray(pattern, np.float64)[(j // QUARTER) % len(pattern)]


def scaled_bf16(values_f32, mult, axis: int):
    """values * mult along `axis` (powers of two: exact), as (values, bits)."""
    shape = [1] * values_f32.ndim
    shape[axis] = -1
    v = (np.asarray(values_f32, np.float32) * np.asarray(mult, np.float32).reshape(shape)).astype(np.float32)
    bits = synth.bf16_bits_from_f32(v)
    assert np.array_equal(synth.f32_from_bf16_bits(bits), v), "multipliers must keep bf16 values exact"
    return v, bits


def rescale_events(logits_log2, visible, walk, start=None):
    """Count rescales of a non-empty state.

    logits_log2 [R, K] (log2 units), visible [R, K] bool, walk: list of
    key-index arrays (quarters) in the order the kernel folds them, the same
    for every row.  A row's reference starts at -inf, or at `start` [R] (the
    exact max a ring step's stored state carries in), and a quarter whose
    visible max exceeds it by more than TAU moves it there; such a move from
    a finite reference is an event.  Returns (events per row, largest jump
    per row, [R, len(walk)] bool: where the events are)."""
    R = logits_log2.shape[0]
    ref = np.full(R, -np.inf) if start is None else np.asarray(start, np.float64).copy()
    events = np.zeros(R, np.int64)
    jump = np.zeros(R)
    at = np.zeros((R, len(walk)), bool)
    for n, keys in enumerate(walk):
        s = np.where(visible[:, keys], logits_log2[:, keys], -np.inf)
        mx = s.max(axis=1) if len(keys) else np.full(R, -np.inf)
        grow = mx > ref + TAU
        ev = grow & np.isfinite(ref)
        events += ev
        at[:, n] = ev
        jump = np.where(ev, np.maximum(jump, mx - ref), jump)
        ref = np.where(grow, mx, ref)
    return events, jump, at


def ascending_quarters(n_keys: int):
    return [np.arange(q0, min(n_keys, q0 + QUARTER)) for q0 in range(0, n_keys, QUARTER)]
