"""The workloads this library is tested and measured on, by name and size.

Plain data: shapes, dtypes and rescale parameters.  No arithmetic.
Rope kinds: 0 plain, 1 position interpolation (PI), 2 NTK-aware, 3 YaRN.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

PLAIN, PI, NTK, YARN = 0, 1, 2, 3


@dataclass(frozen=True)
class Rope:
    kind: int
    head_dim: int
    base: float = 10000.0
    scale: float = 1.0
    orig_ctx: int = 4096
    alpha: float = 1.0
    beta: float = 32.0


@dataclass(frozen=True)
class Prefill:
    name: str
    batch: int
    seq: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    rope: Rope
    causal: bool = True
    kv_block: int = 64          # block size of the blockwise oracle (form B)


@dataclass(frozen=True)
class Decode:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_sink: int
    window: int
    dtype: str
    rope: Rope


@dataclass(frozen=True)
class RingShare:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int                  # tokens per ring block (query and key/value)
    n_blocks: int
    q_block_index: int          # which device's query block
    dtype: str
    rope: Rope
    order: tuple = field(default=())   # feed order; default: ring order from own block down


# Tiny fp32 check: 1 x 1 head x d=64, seq 512, YaRN s=4 from 128, KV block 64.
TINY = Prefill("tiny_fp32_s512", 1, 512, 1, 1, 64, "f32",
               Rope(YARN, 64, 10000.0, 4.0, 128), kv_block=64)
# The same tiny problem fed as 8 ring blocks of 64 tokens.
TINY_RING = RingShare("tiny_ring_8x64", 1, 1, 1, 64, 64, 8, 7, "f32",
                      Rope(YARN, 64, 10000.0, 4.0, 128))

# Llama-7B-like layer prefill, 16k, YaRN s=4 from 4096.
LLAMA_16K = Prefill("llama7b_prefill_16k_yarn4", 1, 16384, 32, 32, 128, "bf16",
                    Rope(YARN, 128, 10000.0, 4.0, 4096))

# GQA 32/8 heads, 32k, base 5e5, s=8 from 4096: PI, NTK, YaRN.
GQA_32K = {
    k: Prefill(f"gqa_prefill_32k_{n}8", 1, 32768, 32, 8, 128, "bf16",
               Rope(k, 128, 500000.0, 8.0, 4096))
    for k, n in ((PI, "pi"), (NTK, "ntk"), (YARN, "yarn"))
}

# Streaming decode: 64 sequences x 32 heads, 4 sinks + 4096 window, plain RoPE.
SINK_DECODE = Decode("sink_decode_b64_4p4096", 64, 32, 32, 128, 4, 4096, "bf16",
                     Rope(PLAIN, 128, 10000.0, 1.0, 4096))

# One ring device's share: 8 heads, blocks of 32768, 8 blocks, YaRN s=8 from 32768.
RING_SHARE = RingShare("ring_share_8x32k_yarn8", 1, 8, 8, 128, 32768, 8, 7, "bf16",
                       Rope(YARN, 128, 10000.0, 8.0, 32768))


def ring_order(w: RingShare):
    """Ring order as seen by device i: its own block first, then i-1, i-2, ..."""
    if w.order:
        return list(w.order)
    i = w.q_block_index
    return [(i - t) % w.n_blocks for t in range(w.n_blocks)]


def shrink(w, **kw):
    return replace(w, **kw)
