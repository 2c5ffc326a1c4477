"""Calls on a caller's stream: the binding allocates the output and the
workspace itself (from the current stream's pool) and marks them used by the
caller's stream, so the caching allocator does not hand them out again while
the kernels still run there.  Results on a side stream, with other work
allocating and writing on the current stream right after each call, equal
the current stream's bit for bit."""

import pytest
import torch

from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, device

pytestmark = pytest.mark.gpu


def _churn():
    # new allocations on the current stream, written at once: they would land
    # in a block freed too early and overwrite what the side stream still uses
    for _ in range(4):
        torch.full((1 << 22,), 7.0, device=device())


def test_prefill_and_decode_on_a_side_stream_match_the_current_stream():
    dev = device()
    shape = W.GLOBAL_LAYER
    B, S = 2, 700
    x = W.PrefillWorkload("streams", shape, B, S, torch.bfloat16, False, seed=31).draw(dev)
    lay = api_layer(shape, torch.bfloat16)
    kc0 = torch.zeros((B, shape.n_kv_heads, S, shape.head_dim), dtype=torch.bfloat16, device=dev)
    kc1 = torch.zeros_like(kc0)
    want = api.gemma_attn_prefill(lay, x["q"], x["k"], None, x["g_q"], x["g_k"], kc0)
    q = W.normal((B, shape.n_q_heads, shape.head_dim), 31, "q_dec", torch.bfloat16, dev)
    lens = torch.tensor([S, S - 123], dtype=torch.int32, device=dev)
    want_dec = api.gemma_attn_decode(lay, q, x["g_q"], kc0, None, lens, S)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = api.gemma_attn_prefill(lay, x["q"], x["k"], None, x["g_q"], x["g_k"], kc1, stream=side)
    _churn()
    got_dec = api.gemma_attn_decode(lay, q, x["g_q"], kc1, None, lens, S, stream=side)
    _churn()
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(got, want), "prefill on a side stream differs"
    assert torch.equal(kc1, kc0), "cache written on a side stream differs"
    assert torch.equal(got_dec, want_dec), "decode on a side stream differs"
