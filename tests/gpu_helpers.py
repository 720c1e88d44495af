"""Helpers shared by the GPU parity tests (no test functions here)."""
import sys

import numpy as np

from yarn_rope_blockwise_amd import synth

BF16_TOL = 2e-2      # max-abs bound for bf16 outputs vs the fp64 oracle (spec)
F32_TOL = 1e-5       # max-abs bound for fp32 outputs vs the fp64 oracle (spec)
TABLE_TOL = 1e-6     # max-abs bound for fp32 cos/sin table entries (spec)


def say(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    import yarn_rope_blockwise_amd.api as api
    api.lib()        # fails loudly if the HIP library is missing


def dev_tensor(values_f32, bits, dtype: str):
    """Device tensor holding exactly the synthetic values."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(values_f32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def draw(shape, seed, dtype):
    v, b = synth.normal(shape, seed, dtype)
    return v, dev_tensor(v, b, dtype)


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to bf16 (via fp32) and widen again; for ulp reports."""
    x32 = np.asarray(x, np.float32)
    return synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(x32)).astype(np.float64)
