"""The decode step of a layer stack (kv_append then decode per layer, local and
global layers) captured into one HIP graph: every replay, with the program's
own eager work and synchronisations between replays, gives exactly the eager
step's outputs and caches.  None of the calls allocates or issues a memset, so
they can be captured; the appends write the same token at the same position on
every replay."""

import pytest
import torch

from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, device

pytestmark = pytest.mark.gpu


def _stack(B, ctx, seed):
    dev = device()
    layers = []
    for i, shape in enumerate([W.LOCAL_LAYER, W.E_LOCAL_LAYER, W.GLOBAL_LAYER]):
        D, Hkv = shape.head_dim, shape.n_kv_heads
        cap = shape.window if shape.window else max(ctx) + 1
        lens = torch.tensor(ctx, dtype=torch.int32) + 1
        lay = api_layer(shape, torch.bfloat16)
        layers.append({
            "lay": lay,
            "kc": W.normal((B, Hkv, cap, D), seed + i, "k_cache", torch.bfloat16, dev),
            "vc": None if shape.kv_shared else W.normal((B, Hkv, cap, D), seed + i, "v_cache", torch.bfloat16, dev),
            "seq": lens.to(dev), "pos": (lens - 1).to(dev), "max": int(lens.max()),
            "q": W.normal((B, shape.n_q_heads, D), seed + i, "q_dec", torch.bfloat16, dev),
            "kn": W.normal((B, Hkv, D), seed + i, "k_new", torch.bfloat16, dev),
            "vn": None if shape.kv_shared else W.normal((B, Hkv, D), seed + i, "v_new", torch.bfloat16, dev),
            "g_q": W.gains(D, seed + i, "g_q", False, torch.bfloat16, dev),
            "g_k": W.gains(D, seed + i, "g_k", False, torch.bfloat16, dev),
            "out": torch.empty((B, shape.n_q_heads, D), dtype=torch.bfloat16, device=dev),
            "ws": api.workspace(api.gemma_attn_decode_workspace_size(lay, B, int(lens.max())), dev),
        })
    return layers


def _step(layers):
    for L in layers:
        api.kv_append(L["lay"], L["kn"], L["vn"], L["g_k"], L["pos"], L["kc"], L["vc"])
        api.gemma_attn_decode(L["lay"], L["q"], L["g_q"], L["kc"], L["vc"], L["seq"], L["max"], L["out"], L["ws"])


def test_stack_step_replayed_as_a_graph_matches_eager():
    layers = _stack(2, [3000, 700], seed=95)
    _step(layers)
    torch.cuda.synchronize()
    want = [L["out"].clone() for L in layers]
    caches = [(L["kc"].clone(), None if L["vc"] is None else L["vc"].clone()) for L in layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(layers)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(layers)
    torch.cuda.synchronize()
    for rep in range(4):
        for L in layers:
            L["out"].fill_(float("nan"))                     # eager work between replays
        scratch = torch.randn(1 << 20, device=device()).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}: scratch {float(scratch):.3f}", flush=True)
        for i, L in enumerate(layers):
            assert torch.equal(L["out"], want[i]), f"replay {rep}, layer {i}: output differs from the eager step"
            assert torch.equal(L["kc"], caches[i][0]), f"replay {rep}, layer {i}: k cache differs"
            if L["vc"] is not None:
                assert torch.equal(L["vc"], caches[i][1]), f"replay {rep}, layer {i}: v cache differs"
    del g
