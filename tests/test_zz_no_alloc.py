"""gemma_attn_decode_noalloc (the decode on the library's static per-GPU
scratch) against gemma_attn_decode with a workspace: two calls in a row, the
second smaller, for a global K=V layer and a local windowed layer."""

import numpy as np
import pytest
import torch

from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, device

pytestmark = pytest.mark.gpu


def _case(shape, lens, seed):
    dev = device()
    B, D, Hkv = len(lens), shape.head_dim, shape.n_kv_heads
    cap = shape.window if shape.window else int(max(lens))
    kc = W.normal((B, Hkv, cap, D), seed, "k_cache", torch.bfloat16, dev)
    vc = None if shape.kv_shared else W.normal((B, Hkv, cap, D), seed, "v_cache", torch.bfloat16, dev)
    q = W.normal((B, shape.n_q_heads, D), seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, seed, "g_q", False, torch.bfloat16, dev)
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    return q, g_q, kc, vc, seq


@pytest.mark.parametrize("shape,first,second", [
    (W.GLOBAL_LAYER, [40000, 5, 70001, 1024, 131072, 17], [3000, 1]),
    (W.LOCAL_LAYER, [5000, 1, 1024, 1025, 90000, 33, 64], [700, 2000]),
], ids=["global", "local"])
def test_noalloc_decode_matches_decode(shape, first, second):
    lay = api_layer(shape, torch.bfloat16)
    for i, lens in enumerate([first, second]):
        q, g_q, kc, vc, seq = _case(shape, lens, 90 + i)
        mx = int(max(lens))
        want = api.gemma_attn_decode(lay, q, g_q, kc, vc, seq, mx)
        got = torch.full_like(q, float("nan"))
        api.gemma_attn_decode_noalloc(lay, q, g_q, kc, vc, seq, mx, got)
        torch.cuda.synchronize()
        print(f"[noalloc] {shape.head_dim} call {i}: B={len(lens)} max_len={mx}", flush=True)
        assert torch.equal(got, want), f"call {i}: differs from gemma_attn_decode"


def test_noalloc_decode_rejects_oversized_plans():
    shape = W.GLOBAL_LAYER
    lay = api_layer(shape, torch.bfloat16)
    dev = device()
    B, D = 256, shape.head_dim
    q = torch.zeros((B, shape.n_q_heads, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((B, shape.n_kv_heads, 16, D), dtype=torch.bfloat16, device=dev)
    seq = torch.full((B,), 16, dtype=torch.int32, device=dev)
    with pytest.raises(api.GemmaAttnError, match="static scratch"):
        api.gemma_attn_decode_noalloc(lay, q, q[0, 0], kc, None, seq, 16, torch.empty_like(q))
