"""YaRN-RoPE blockwise attention for MI355X (gfx950).

The compute path is the HIP library ``libyrb.so`` built from ``csrc/``; the
Python functions here only marshal torch tensors into its C ABI.  Importing
the bindings fails loudly when the library has not been built.
"""
__all__ = ["rope_tables_build", "rope_apply", "attn_prefill_blockwise",
           "attn_block_accumulate", "attn_decode_sink_window", "RopeConfig"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
