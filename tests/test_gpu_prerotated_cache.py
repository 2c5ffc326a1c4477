"""GPU parity of the pre-rotated ("1.25 d") K=V cache against the float64 oracle.

The cache holds the normalised, unrotated rows (the values, and the key's
unrotated dims) plus each row's leading 2 n_rot dims already rotated to its
position (oracle.prerotated_heads), the layout behind the pages' 37.5%
figure.  Expected decode outputs come from oracle.decode_from_prerotated_cache
on the stored values; heads the kernels write are compared with
oracle.prerotated_heads of the oracle's rows.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, assert_close, device, oracle_layer, to64

pytestmark = pytest.mark.gpu

SHAPES = {"global": W.GLOBAL_LAYER, "global_g4": replace(W.GLOBAL_LAYER, n_q_heads=16)}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def pre_layer(shape) -> api.Layer:
    return replace(api_layer(shape, torch.bfloat16), cache_format=2)


def filled_cache(shape, lens, seed, batches=None):
    """A pre-rotated cache of N(0, 1) rows with oracle heads (bf16), for the
    sequences in `batches` (all by default); other sequences' heads are zeros."""
    B, cap, D = len(lens), max(lens), shape.head_dim
    lay = pre_layer(shape)
    cache = api.new_cache(lay, B, cap, device())
    rows = W.normal((B, shape.n_kv_heads, cap, D), seed, "k_cache", torch.bfloat16, device())
    cache.rows().copy_(rows)
    ol = oracle_layer(shape)
    for b in (range(B) if batches is None else batches):
        h = O.prerotated_heads(ol, to64(rows[b]), np.arange(cap))
        cache.heads()[b].copy_(torch.from_numpy(h).to(torch.bfloat16))
    return lay, cache


@pytest.mark.parametrize("kind,lens", [
    ("global", [1, 17, 1024, 1025, 2600]),
    ("global", [4097, 3000]),
    ("global_g4", [1, 33, 1500]),
])
def test_prerotated_decode(kind, lens):
    shape, dev = SHAPES[kind], device()
    lay, cache = filled_cache(shape, lens, seed=91)
    B, D = len(lens), shape.head_dim
    q = W.normal((B, shape.n_q_heads, D), 91, "q_dec", torch.bfloat16, "cpu")
    g_q = W.gains(D, 91, "g_q", False, torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = api.gemma_attn_decode(lay, q.to(dev), g_q.to(dev), cache, None, seq.to(dev), max(lens))
    torch.cuda.synchronize()
    ref = O.decode_from_prerotated_cache(oracle_layer(shape), to64(q), to64(g_q), to64(cache.heads()),
                                         to64(cache.rows()), seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"pre-rotated {kind} decode {lens}")


def test_prerotated_multi_token_decode():
    """Two new tokens per sequence; the heads are the rows rotated (to bf16), so
    the K=V definition on the rows is the expected output."""
    shape, dev = W.GLOBAL_LAYER, device()
    lens = [2, 300, 1500]
    lay, cache = filled_cache(shape, lens, seed=93)
    B, D, T = len(lens), shape.head_dim, 2
    q = W.normal((B, T, shape.n_q_heads, D), 93, "q_dec", torch.bfloat16, "cpu")
    g_q = W.gains(D, 93, "g_q", False, torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = api.gemma_attn_decode_multi(lay, q.to(dev), g_q.to(dev), cache, None, seq.to(dev), max(lens))
    torch.cuda.synchronize()
    ref = O.decode_multi_from_cache(oracle_layer(shape), to64(q), to64(g_q), to64(cache.rows()), None,
                                    seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"pre-rotated 2-token decode {lens}")


def test_prerotated_prefill_and_append_write_rows_and_heads():
    shape, dev = W.GLOBAL_LAYER, device()
    B, S, cap = 2, 300, 320
    x = W.PrefillWorkload("pre", shape, B, S, torch.bfloat16, False, 95).draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = pre_layer(shape)
    cache = api.new_cache(lay, B, cap, dev)
    out = api.gemma_attn_prefill(lay, xd["q"], xd["k"], None, xd["g_q"], xd["g_k"], cache)
    native = torch.full((B, shape.n_kv_heads, cap, shape.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    out_native = api.gemma_attn_prefill(api_layer(shape, torch.bfloat16), xd["q"], xd["k"], None, xd["g_q"],
                                        xd["g_k"], native)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out_native.cpu())
    assert torch.equal(cache.rows()[:, :, :S].cpu(), native[:, :, :S].cpu())
    ol = oracle_layer(shape)
    rows, _ = O.expected_caches_after_prefill(ol, to64(x["k"]), None, to64(x["g_k"]), S)
    assert_close(cache.heads()[:, :, :S], O.prerotated_heads(ol, rows, np.arange(S)), torch.bfloat16,
                 "prefill heads")
    assert not cache.heads()[:, :, S:].any()
    # one new token per sequence at positions 300 and 319
    kn = W.normal((B, shape.n_kv_heads, shape.head_dim), 95, "k_new", torch.bfloat16, dev)
    pos = [S, cap - 1]
    api.kv_append(lay, kn, None, xd["g_k"], torch.tensor(pos, dtype=torch.int32, device=dev), cache)
    torch.cuda.synchronize()
    k_hat = O.qk_norm(to64(kn), to64(x["g_k"]), shape.norm_eps)             # [B,Hkv,d]
    for b, p in enumerate(pos):
        assert_close(cache.rows()[b, :, p], k_hat[b], torch.bfloat16, f"appended row b={b}")
        want = O.prerotated_heads(ol, k_hat[b][:, None], [p])[:, 0]
        assert_close(cache.heads()[b, :, p], want, torch.bfloat16, f"appended head b={b}")


def test_prerotated_chunked_prefill():
    shape, dev = W.GLOBAL_LAYER, device()
    B, S, cut = 2, 700, 300
    x = W.PrefillWorkload("prec", shape, B, S, torch.bfloat16, False, 97).draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = pre_layer(shape)
    cache = api.new_cache(lay, B, S, dev)
    outs = [api.gemma_attn_prefill_chunk(lay, a, xd["q"][:, a:b].contiguous(), xd["k"][:, a:b].contiguous(),
                                         xd["g_q"], xd["g_k"], cache) for a, b in [(0, cut), (cut, S)]]
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), None, to64(x["g_q"]), to64(x["g_k"]))
    assert_close(torch.cat(outs, dim=1), ref, torch.bfloat16, f"pre-rotated chunks [0,{cut}) [{cut},{S})")
    rows, _ = O.expected_caches_after_prefill(ol, to64(x["k"]), None, to64(x["g_k"]), S)
    assert_close(cache.heads(), O.prerotated_heads(ol, rows, np.arange(S)), torch.bfloat16, "chunked heads")


def test_prerotated_global_decode_full_size_sampled():
    """The global decode workload (B=16, contexts 4K..128K) on a pre-rotated
    cache: the shortest and the longest sequence against the oracle."""
    wl = W.CONFIGS["global_decode"]
    shape, dev = wl.layer, device()
    lens = wl.lengths()
    sample = [int(np.argmin(lens.numpy())), int(np.argmax(lens.numpy()))]
    lay, cache = filled_cache(shape, [wl.cache_cap()] * wl.batch, wl.seed, batches=sample)
    q = W.normal((wl.batch, shape.n_q_heads, shape.head_dim), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(shape.head_dim, wl.seed, "g_q", False, torch.bfloat16, dev)
    out = api.gemma_attn_decode(lay, q, g_q, cache, None, lens.to(dev), int(lens.max()))
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in sample:
        L = int(lens[b])
        ref = O.decode_from_prerotated_cache(ol, to64(q[b:b + 1]), to64(g_q), to64(cache.heads()[b:b + 1, :, :L]),
                                             to64(cache.rows()[b:b + 1, :, :L]), np.array([L]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"pre-rotated global decode B16 b={b} L={L}")


def test_prerotated_edge_cases():
    """Out-of-range append positions write neither rows nor heads; invalid
    decode lengths give NaN rows next to valid ones."""
    shape, dev = W.GLOBAL_LAYER, device()
    D, cap = shape.head_dim, 50
    lay = pre_layer(shape)
    cache = api.new_cache(lay, 3, cap, dev)
    kn = W.normal((3, shape.n_kv_heads, D), 2, "k_new", torch.bfloat16, dev)
    g = torch.ones(D, dtype=torch.bfloat16, device=dev)
    api.kv_append(lay, kn, None, g, torch.tensor([-1, cap, cap - 1], dtype=torch.int32, device=dev), cache)
    torch.cuda.synchronize()
    r, h = cache.rows().float().cpu(), cache.heads().float().cpu()
    assert not r[:2].any() and not h[:2].any() and not r[2, :, :cap - 1].any() and not h[2, :, :cap - 1].any()
    k_hat = O.qk_norm(to64(kn[2]), np.ones(D), 1e-6)
    assert_close(cache.rows()[2, :, cap - 1], k_hat, torch.bfloat16, "appended row")
    assert_close(cache.heads()[2, :, cap - 1], O.prerotated_heads(oracle_layer(shape), k_hat[:, None], [cap - 1])[:, 0],
                 torch.bfloat16, "appended head")
    lens = [0, 40, 100]
    lay, full = filled_cache(shape, [100] * 3, seed=5)
    q = W.normal((3, shape.n_q_heads, D), 5, "q_dec", torch.bfloat16, "cpu")
    bad = torch.tensor([0, 40, 101], dtype=torch.int32, device=dev)   # 0 and 101 are out of range
    out = api.gemma_attn_decode(lay, q.to(dev), g, full, None, bad, 100)
    o = out.float().cpu()
    assert torch.isnan(o[0]).all() and torch.isnan(o[2]).all()
    ref = O.decode_from_prerotated_cache(oracle_layer(shape), to64(q), np.ones(D), to64(full.heads()),
                                         to64(full.rows()), np.array(lens), batches=[1])
    assert_close(out[1:2], ref, torch.bfloat16, "pre-rotated: valid row next to invalid ones")
