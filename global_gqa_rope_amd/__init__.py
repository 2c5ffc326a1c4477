"""MI355X (gfx950) attention block of a Gemma-4-style decoder.

The computation runs in libgemma_attn.so (HIP kernels behind a C ABI, see
include/gemma_attn.h); `api` is its torch-facing binding and `workloads` the
seeded synthetic inputs.
"""

from .api import (  # noqa: F401
    GemmaAttnError,
    Int8Cache,
    Layer,
    PrerotatedCache,
    cache_bytes,
    gemma_attn_decode,
    gemma_attn_decode_workspace_size,
    gemma_attn_prefill,
    gemma_attn_prefill_workspace_size,
    kv_append,
    new_cache,
    workspace,
)
