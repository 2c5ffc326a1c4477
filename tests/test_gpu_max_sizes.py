"""GPU parity at the largest sizes the workloads reach: a 128K-position global
prefill and decode steps against 256K-position caches (bf16 and int8), each
checked on sampled rows the float64 oracle computes one by one."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, assert_close, device, oracle_layer, to64
from tests.test_gpu_parity import _sampled_prefill

pytestmark = pytest.mark.gpu

CTX_256K = 262144


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_global_prefill_128k_sampled_rows():
    wl = W.with_seq(W.CONFIGS["global_prefill_32k"], 131072)
    _sampled_prefill(wl, [0, 1, 65535, 100000, 131071], [0], "global prefill 128K")


def test_global_decode_256k_context():
    shape, dev = W.GLOBAL_LAYER, device()
    lens = torch.tensor([CTX_256K, 150001], dtype=torch.int32)
    B, D = len(lens), shape.head_dim
    kc = W.normal((B, shape.n_kv_heads, CTX_256K, D), 81, "k_cache", torch.bfloat16, dev)
    q = W.normal((B, shape.n_q_heads, D), 81, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, 81, "g_q", False, torch.bfloat16, dev)
    out = api.gemma_attn_decode(api_layer(shape, torch.bfloat16), q, g_q, kc, None, lens.to(dev), CTX_256K)
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in range(B):
        L = int(lens[b])
        ref = O.decode_from_cache(ol, to64(q[b:b + 1]), to64(g_q), to64(kc[b:b + 1, :, :L]), None, np.array([L]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"decode at {L} cached positions")


@pytest.mark.parametrize("dtype,q_rot,k_rot", [(torch.bfloat16, 1.0, 1.0), (torch.float32, 4.0, 2.0)],
                         ids=["bf16", "fp32"])
def test_global_decode_long_segments_keep_rope_angles(dtype, q_rot, k_rot):
    """B=32 sequences of 131072 cached positions on a global K=V layer: each of
    the 256 split-K workgroups streams ~4096 tiles, so a wave runs 1024 (bf16,
    four waves) or 2048 (fp32, two waves) tiles inside one segment and carries
    its keys' p-RoPE angles across all of them.  bf16: the workload's N(0, 1)
    data at the bf16 tolerance.  fp32: the rotated dims (0..127) of q scaled up
    4x and those of the cache 2x, so that the scores lean on the rotated pairs,
    at the fp32 tolerance of 1e-5; there an angle error that grows by ~1e-6
    rad per tile (fp32 rounding of the per-tile rotation step, compounded over
    2048 tiles) gives, in a float64 simulation, a relative error of 4e-4 and a
    largest error of 6e-5.  Checked: the first and last sequence."""
    shape, dev = W.GLOBAL_LAYER, device()
    B, L, D, Hkv = 32, 131072, shape.head_dim, shape.n_kv_heads
    lens = torch.full((B,), L, dtype=torch.int32)
    kc = W.normal((B, Hkv, L, D), 85, "k_cache", dtype, dev)
    q = W.normal((B, shape.n_q_heads, D), 85, "q_dec", dtype, dev)
    if q_rot != 1.0:
        q[..., :128].mul_(q_rot)
        kc[..., :128].mul_(k_rot)
    g_q = W.gains(D, 85, "g_q", False, dtype, dev)
    out = api.gemma_attn_decode(api_layer(shape, dtype), q, g_q, kc, None, lens.to(dev), L)
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in [0, B - 1]:
        ref = O.decode_from_cache(ol, to64(q[b:b + 1]), to64(g_q), to64(kc[b:b + 1]), None, np.array([L]))
        assert_close(out[b:b + 1], ref, dtype, f"decode {dtype} B=32 L={L} b={b} (long segments)")
    del kc


def test_int8_decode_256k_context():
    shape, dev = W.GLOBAL_LAYER, device()
    D = shape.head_dim
    lay = replace(api_layer(shape, torch.bfloat16), cache_format=1)
    cache = api.new_cache(lay, 1, CTX_256K, dev)
    c, s = W.int8_rows((1, shape.n_kv_heads, CTX_256K, D), 83, dev)
    cache.codes().copy_(c)
    cache.scales().copy_(s)
    del c, s
    q = W.normal((1, shape.n_q_heads, D), 83, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, 83, "g_q", False, torch.bfloat16, dev)
    lens = torch.tensor([CTX_256K], dtype=torch.int32, device=dev)
    out = api.gemma_attn_decode(lay, q, g_q, cache, None, lens, CTX_256K)
    torch.cuda.synchronize()
    rows = O.dequantize_rows(cache.codes().cpu().numpy(), cache.scales().cpu().numpy())
    ref = O.decode_from_cache(oracle_layer(shape), to64(q), to64(g_q), rows, None, np.array([CTX_256K]))
    assert_close(out, ref, torch.bfloat16, f"int8 decode at {CTX_256K} cached positions")


def test_local_prefill_256k_prompt():
    """A 256K-position local-layer prompt: one KV head's rows of v span 2^31
    bytes, so v is staged through the workspace instead of read in place.
    Early rows (every key they see lies in the first 5K positions) against the
    oracle, and the ring's last slots."""
    shape, dev = W.LOCAL_LAYER, device()
    S = CTX_256K
    wl = W.with_seq(W.CONFIGS["local_prefill_32k"], S, batch=1)
    x = wl.draw(dev)
    lay = api_layer(shape, torch.bfloat16)
    kc = torch.empty((1, shape.n_kv_heads, shape.window, shape.head_dim), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    out = api.gemma_attn_prefill(lay, x["q"], x["k"], x["v"], x["g_q"], x["g_k"], kc, vc)
    torch.cuda.synchronize()
    rows = [0, 1, 1023, 1024, 1025, 4097]
    hi = max(rows) + 1
    ref = O.prefill(oracle_layer(shape), to64(x["q"][:, torch.as_tensor(rows, device=dev)]), to64(x["k"][:, :hi]),
                    to64(x["v"][:, :hi]), to64(x["g_q"]), to64(x["g_k"]), rows=np.asarray(rows), q_at_rows=True)
    assert_close(out[:, torch.as_tensor(rows, device=dev)], ref, torch.bfloat16, f"local prefill 256K rows {rows}")
    # the ring holds the last W positions' values unchanged (slot = position mod W)
    last = torch.arange(S - 8, S, device=dev)
    assert torch.equal(vc[0, :, last % shape.window].permute(1, 0, 2).cpu(), x["v"][0, last].cpu())
