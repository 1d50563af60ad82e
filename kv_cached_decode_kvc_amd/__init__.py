"""MI355X (gfx950) KV-cache decode attention: append, block tables, split-KV
decode and speculative-verify attention, as hand-written HIP kernels behind
the C ABI declared in ``include/kvc.h``.

``kvc`` is the ctypes binding (one Python function per C entry point);
``synth`` generates seeded synthetic workloads; ``metrics`` counts the
algorithmic bytes and FLOPs of a step.  The shared library is loaded on the
first call into ``kvc`` and its absence is an error.
"""
from .kvc import (KVC_BF16, KVC_F32, EXPORTS, KvcError, cache_desc, kvc_append,
                  kvc_attn_partition, kvc_attn_partition_tokens, kvc_attn_reduce,
                  kvc_attn_workspace_bytes, kvc_block_table, kvc_cache_desc, kvc_decode_attn,
                  kvc_status_string, kvc_verify_attn, lib)

__all__ = ["KVC_BF16", "KVC_F32", "EXPORTS", "KvcError", "cache_desc", "kvc_append",
           "kvc_attn_partition", "kvc_attn_partition_tokens", "kvc_attn_reduce",
           "kvc_attn_workspace_bytes", "kvc_block_table", "kvc_cache_desc", "kvc_decode_attn",
           "kvc_status_string", "kvc_verify_attn", "lib"]
