"""fp64 CPU oracle: RoPE frequencies under a context-extension rescale,
cos/sin tables and pair rotation.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it.

Every function below is the plain definition written out in float64, in the
notation of the pages it cites:

* "Context Window Scaling: YaRN, LongRoPE, and RingAttention Architectures"
  (tecvarsity), Section 2 "Formal RoPE Mechanics" and "The Failure of Naive
  Positional Interpolation", Section 3 "Decoupled Frequency Partitioning" and
  "Attention Entropy & Dynamic Temperature Scaling".
* "Context Length Extension" (14cs17 notes), sections "Notation", "Why Models
  Fail at Longer Contexts", "Position Interpolation", "NTK-Aware Scaling",
  "YaRN: Yet Another RoPE Extension".
* "Long-context extension: stretching attention past its training window"
  (root18d), section "Not every RoPE dimension needs the same treatment".

Readings taken where the pages are silent or garbled (each is listed with
its reason in the design notes):

* NTK-aware base: the formula is missing after "Scale the base frequency
  instead".  Reading: b' = b * s**(d/(d-2)), the base change that keeps the
  fastest pair (i = 0) unchanged and interpolates the slowest pair
  (i = d/2-1) by exactly s.  The exponent is a reading, not pinned by a
  printed value ("parity unpinned" for the exponent itself).
* YaRN ramp: r_i = L_train / lambda_i (rotations of pair i inside the
  training window), gamma_i = clamp((r_i - alpha)/(beta - alpha), 0, 1),
  theta'_i = (1 - gamma_i) theta_i / s + gamma_i theta_i, alpha = 1,
  beta = 32.  The base is not changed by YaRN.
* Temperature: logits are multiplied by (0.1 ln s + 1)**2 for YaRN with
  s > 1 (1 otherwise).  It is returned as ``attn_factor`` and applied through
  the softmax scale, never folded into the tables.
* Pairing: half-split pairs (i, i + d/2) (the tecvarsity listing
  concatenates the frequency vector with itself).  Interleaved pairs
  (2i, 2i+1) are provided here for completeness only.
"""
from __future__ import annotations

import math

import numpy as np

PLAIN, PI, NTK, YARN = 0, 1, 2, 3
KIND_NAMES = {PLAIN: "plain", PI: "pi", NTK: "ntk", YARN: "yarn"}


def base_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base**(-2i/d), i = 0 .. d/2-1.

    tecvarsity Section 2 "Formal RoPE Mechanics"; 14cs17 "Why Models Fail at
    Longer Contexts" (angle p / base**(2i/d)).
    """
    if head_dim <= 0 or head_dim % 2:
        raise ValueError("head_dim must be a positive even number")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def ntk_base(head_dim: int, base: float, scale: float) -> float:
    """NTK-aware base b' = b * s**(d/(d-2)) (reading; 14cs17 "NTK-Aware Scaling")."""
    return float(base) * float(scale) ** (head_dim / (head_dim - 2.0))


def wavelengths(theta: np.ndarray) -> np.ndarray:
    """lambda_i = 2 pi / theta_i = 2 pi b**(2i/d) (tecvarsity Section 3)."""
    return 2.0 * math.pi / theta


def yarn_ramp(theta: np.ndarray, orig_ctx: float, alpha: float, beta: float) -> np.ndarray:
    """gamma_i in [0, 1]: 1 leaves pair i unscaled, 0 interpolates it fully.

    r_i = L_train / lambda_i counts how many full turns pair i makes inside
    the training window.  Many turns (r > beta): high frequency, untouched.
    Less than one turn (r < alpha): low frequency, full interpolation.  In
    between the two treatments blend linearly in r.
    root18d "Not every RoPE dimension needs the same treatment";
    tecvarsity Section 3 "Decoupled Frequency Partitioning".
    """
    r = float(orig_ctx) / wavelengths(theta)
    return np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)


def inv_freq(kind: int, head_dim: int, base: float, scale: float = 1.0,
             orig_ctx: float = 4096.0, alpha: float = 1.0, beta: float = 32.0) -> np.ndarray:
    """theta'_i for one rescale method.

    PLAIN: theta.                     (tecvarsity Section 2)
    PI:    theta / s  (m' = m / s).   (tecvarsity Section 2 PI paragraph;
                                        14cs17 "Position Interpolation")
    NTK:   b'**(-2i/d), b' = ntk_base (14cs17 "NTK-Aware Scaling", reading)
    YARN:  (1-gamma) theta/s + gamma theta  (root18d; tecvarsity Section 3)
    """
    if scale <= 0:
        raise ValueError("scale must be > 0")
    theta = base_inv_freq(head_dim, base)
    if kind == PLAIN:
        return theta
    if kind == PI:
        return theta / scale
    if kind == NTK:
        return base_inv_freq(head_dim, ntk_base(head_dim, base, scale))
    if kind == YARN:
        if not alpha < beta:
            raise ValueError("alpha must be < beta")
        g = yarn_ramp(theta, orig_ctx, alpha, beta)
        return (1.0 - g) * (theta / scale) + g * theta
    raise ValueError(f"unknown rope kind {kind}")


def inv_freq_factors(head_dim: int, base: float, factors) -> np.ndarray:
    """theta'_i = theta_i / lambda_i for a per-pair scale vector lambda.

    tecvarsity Section 4 "Deep Dive into LongRoPE": one scale per dimension
    (found by search) instead of a single s or a ramp.  Reading: lambda_i
    stretches pair i's wavelength, as s does for every pair under PI, so
    lambda_i = s for all i is PI exactly.
    """
    lam = np.asarray(factors, dtype=np.float64).reshape(-1)
    if lam.size != head_dim // 2:
        raise ValueError("one factor per pair")
    if not np.all(np.isfinite(lam)) or not np.all(lam > 0):
        raise ValueError("factors must be finite and > 0")
    return base_inv_freq(head_dim, base) / lam


def attn_factor(kind: int, scale: float) -> float:
    """Logit multiplier: (0.1 ln s + 1)**2 for YaRN with s > 1, else 1.

    tecvarsity Section 3 "Attention Entropy & Dynamic Temperature Scaling"
    and its listing's ``get_mscale`` (0.1 ln s + 1, 1 for s <= 1), which
    multiplies both the query's and the key's rotation, hence the square.
    """
    if kind != YARN or scale <= 1.0:
        return 1.0
    ms = 0.1 * math.log(scale) + 1.0
    return ms * ms


def softmax_scale(kind: int, scale: float, head_dim: int) -> float:
    """attn_factor / sqrt(d): softmax(QK^T / sqrt(d_k)) with the temperature."""
    return attn_factor(kind, scale) / math.sqrt(head_dim)


def angles(theta: np.ndarray, positions) -> np.ndarray:
    """angle[p, i] = p * theta_i in float64."""
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    return pos * theta.reshape(1, -1)


def tables(theta: np.ndarray, positions):
    """(cos, sin) of p * theta_i, each [n_pos, d/2] float64 (tecvarsity Section 2)."""
    a = angles(theta, positions)
    return np.cos(a), np.sin(a)


def rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate half-split pairs (x_i, x_{i+d/2}) by the angle of their position.

    y_i       = x_i cos - x_{i+d/2} sin
    y_{i+d/2} = x_i sin + x_{i+d/2} cos
    (the 2x2 matrix [[cos, -sin], [sin, cos]] of tecvarsity Section 2.)
    ``x`` is [..., d]; ``cos``/``sin`` broadcast against [..., d/2].
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def rotate_interleaved(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Same rotation on interleaved pairs (x_{2i}, x_{2i+1})."""
    x = np.asarray(x, dtype=np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = a * cos - b * sin
    y[..., 1::2] = a * sin + b * cos
    return y


def rotate_bshd(x: np.ndarray, theta: np.ndarray, positions) -> np.ndarray:
    """Rotate x [B, S, H, D] with token s at ``positions[s]`` (or [B, S] array)."""
    x = np.asarray(x, dtype=np.float64)
    B, S, H, D = x.shape
    pos = np.asarray(positions)
    if pos.ndim == 1:
        c, s = tables(theta, pos)                   # [S, D/2]
        return rotate_half(x, c[None, :, None, :], s[None, :, None, :])
    out = np.empty_like(x)
    for b in range(B):
        c, s = tables(theta, pos[b])
        out[b] = rotate_half(x[b], c[:, None, :], s[:, None, :])
    return out
