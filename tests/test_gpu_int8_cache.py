"""GPU parity of the int8 K=V cache (global layers) against the float64 oracle.

The cache keeps each row as int8 codes and one fp32 scale (the symmetric
per-row reading of the int8 KV cache in the 32K memory table of "Gemma 4
技术报告"); decode and a later prefill chunk read the rows back as codes x
scale.  Expected outputs come from the oracle on the rows the codes stand for
(oracle.dequantize_rows); codes the kernels write are compared with
oracle.quantize_rows, which decides them in float32 as the kernels do.
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

# The global K=V layer, and one with 4 query heads per KV head (the other
# group size the int8 decode is built for).
SHAPES = {"global": W.GLOBAL_LAYER, "global_g4": replace(W.GLOBAL_LAYER, n_q_heads=16)}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def q8_layer(shape) -> api.Layer:
    return replace(api_layer(shape, torch.bfloat16), cache_format=1)


def cache_from(lay, codes: torch.Tensor, scales: torch.Tensor) -> api.Int8Cache:
    """A device Int8Cache holding int8 codes [B,Hkv,cap,d] and scales [B,Hkv,cap]."""
    B, _, cap, _ = codes.shape
    c = api.new_cache(lay, B, cap, device())
    c.codes().copy_(codes)
    c.scales().copy_(scales)
    return c


def oracle_rows(codes: torch.Tensor, scales: torch.Tensor) -> np.ndarray:
    """The float64 rows a cache stands for."""
    return O.dequantize_rows(codes.cpu().numpy(), scales.cpu().numpy())


def quantised_normal_keys(shape, B, cap, seed):
    """Rows of N(0, 1) keys quantised by the oracle: int8 codes and scales."""
    keys = W.normal((B, shape.n_kv_heads, cap, shape.head_dim), seed, "k_cache", torch.float32, "cpu")
    keys[0, 0, 0] = 0.0                                   # an all-zero row: s = 0, codes 0
    c, s = O.quantize_rows(keys.numpy())
    return torch.from_numpy(c), torch.from_numpy(s)


def assert_codes_match(got_c, got_s, k_hat, what):
    """Kernel codes/scales against oracle.quantize_rows of the float64 rows k_hat.

    The kernel normalises in float32, a few ulp from the float64 rows, so a
    code may differ by one where x / s lies within 1e-3 of a rounding boundary;
    everywhere else it must be equal, and the scales agree to 1e-5 relative."""
    want_c, want_s = O.quantize_rows(k_hat)
    got_c = np.asarray(got_c, dtype=np.int16)
    got_s = np.asarray(got_s, dtype=np.float32)
    assert np.allclose(got_s, want_s, rtol=1e-5, atol=0), f"{what}: scales"
    diff = np.abs(got_c - want_c.astype(np.int16))
    s = np.where(want_s > 0, want_s.astype(np.float64), 1.0)[..., None]
    r = k_hat / s
    near = np.abs(np.abs(r - np.floor(r)) - 0.5) < 1e-3
    print(f"[parity] {what}: {int((diff > 0).sum())} of {diff.size} codes off by one "
          f"({int(near.sum())} near a boundary)", flush=True)
    assert diff.max() <= 1, f"{what}: a code differs by {diff.max()}"
    assert not np.any((diff > 0) & ~near), f"{what}: a code differs away from a rounding boundary"


@pytest.mark.parametrize("kind,lens,src", [
    ("global", [1, 17, 1024, 1025, 2600], "quantised"),
    ("global", [4097, 3000], "random"),
    ("global_g4", [1, 33, 1500], "quantised"),
    ("global_g4", [700, 2049], "random"),
])
def test_int8_decode(kind, lens, src):
    shape, dev = SHAPES[kind], device()
    B, cap, D = len(lens), max(lens), shape.head_dim
    if src == "quantised":
        codes, scales = quantised_normal_keys(shape, B, cap, seed=41)
    else:
        codes, scales = W.int8_rows((B, shape.n_kv_heads, cap, D), 43)
    lay = q8_layer(shape)
    cache = cache_from(lay, codes.to(dev), scales.to(dev))
    q = W.normal((B, shape.n_q_heads, D), 41, "q_dec", torch.bfloat16, "cpu")
    g_q = W.gains(D, 41, "g_q", False, torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = api.gemma_attn_decode(lay, q.to(dev), g_q.to(dev), cache, None, seq.to(dev), max(lens))
    torch.cuda.synchronize()
    ref = O.decode_from_cache(oracle_layer(shape), to64(q), to64(g_q), oracle_rows(codes, scales), None,
                              seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"int8 {kind} decode {lens} ({src})")


def test_int8_decode_equals_decode_of_the_expanded_cache():
    """Codes whose scales are all 1: the int8 decode reads the same bf16 tiles
    as a bf16 cache holding the codes, and the two decodes agree bit for bit
    (multiplying by a scale of 1 is exact)."""
    shape, dev = W.GLOBAL_LAYER, device()
    lens = [5, 1000, 1601]
    B, cap, D = len(lens), max(lens), shape.head_dim
    codes, _ = W.int8_rows((B, shape.n_kv_heads, cap, D), 47, dev)
    scales = torch.ones(B, shape.n_kv_heads, cap, dtype=torch.float32, device=dev)
    lay = q8_layer(shape)
    cache = cache_from(lay, codes, scales)
    expanded = codes.to(torch.bfloat16)
    q = W.normal((B, shape.n_q_heads, D), 47, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, 47, "g_q", False, torch.bfloat16, dev)
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    a = api.gemma_attn_decode(lay, q, g_q, cache, None, seq, max(lens))
    b = api.gemma_attn_decode(api_layer(shape, torch.bfloat16), q, g_q, expanded, None, seq, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), b.cpu())


@pytest.mark.parametrize("kind,T,lens", [("global", 2, [2, 300, 1500]), ("global_g4", 4, [4, 999])])
def test_int8_multi_token_decode(kind, T, lens):
    shape, dev = SHAPES[kind], device()
    B, cap, D = len(lens), max(lens), shape.head_dim
    codes, scales = quantised_normal_keys(shape, B, cap, seed=53)
    lay = q8_layer(shape)
    cache = cache_from(lay, codes.to(dev), scales.to(dev))
    q = W.normal((B, T, shape.n_q_heads, D), 53, "q_dec", torch.bfloat16, "cpu")
    g_q = W.gains(D, 53, "g_q", False, torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = api.gemma_attn_decode_multi(lay, q.to(dev), g_q.to(dev), cache, None, seq.to(dev), max(lens))
    torch.cuda.synchronize()
    ref = O.decode_multi_from_cache(oracle_layer(shape), to64(q), to64(g_q), oracle_rows(codes, scales), None,
                                    seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"int8 {kind} {T}-token decode {lens}")


def test_int8_kv_append_writes_codes_and_scales():
    shape, dev = W.GLOBAL_LAYER, device()
    B, cap, D = 3, 64, shape.head_dim
    lay = q8_layer(shape)
    codes, scales = W.int8_rows((B, shape.n_kv_heads, cap, D), 59, dev)
    cache = cache_from(lay, codes, scales)
    kn = W.normal((B, shape.n_kv_heads, D), 59, "k_new", torch.bfloat16, dev)
    g_k = W.gains(D, 59, "g_k", False, torch.bfloat16, dev)
    pos = [0, 37, 63]
    api.kv_append(lay, kn, None, g_k, torch.tensor(pos, dtype=torch.int32, device=dev), cache)
    torch.cuda.synchronize()
    k_hat = O.qk_norm(to64(kn), to64(g_k), shape.norm_eps)                   # [B,Hkv,d]
    got_c, got_s = cache.codes().cpu(), cache.scales().cpu()
    rows = [(b, p) for b, p in enumerate(pos)]
    assert_codes_match(np.stack([got_c[b, :, p].numpy() for b, p in rows]),
                       np.stack([got_s[b, :, p].numpy() for b, p in rows]), k_hat, "kv_append int8 rows")
    keep = torch.ones(B, cap, dtype=torch.bool)
    for b, p in rows:
        keep[b, p] = False
    assert torch.equal(cache.codes().cpu().permute(0, 2, 1, 3)[keep], codes.cpu().permute(0, 2, 1, 3)[keep])
    assert torch.equal(cache.scales().cpu().permute(0, 2, 1)[keep], scales.cpu().permute(0, 2, 1)[keep])


def _prefill(lay, xd, cache):
    return api.gemma_attn_prefill(lay, xd["q"], xd["k"], None, xd["g_q"], xd["g_k"], cache)


def test_int8_prefill_writes_codes_and_attends_at_full_precision():
    shape, dev = W.GLOBAL_LAYER, device()
    B, S, cap = 2, 300, 320
    x = W.PrefillWorkload("q8", shape, B, S, torch.bfloat16, False, 61).draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = q8_layer(shape)
    cache = api.new_cache(lay, B, cap, dev)
    out = _prefill(lay, xd, cache)
    native = torch.full((B, shape.n_kv_heads, cap, shape.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    out_native = _prefill(api_layer(shape, torch.bfloat16), xd, native)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out_native.cpu())
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), None, to64(x["g_q"]), to64(x["g_k"]))
    assert_close(out, ref, torch.bfloat16, "int8-cache prefill output")
    k_hat = O.qk_norm(to64(x["k"]), to64(x["g_k"]), shape.norm_eps).transpose(0, 2, 1, 3)   # [B,Hkv,S,d]
    assert_codes_match(cache.codes()[:, :, :S].cpu().numpy(), cache.scales()[:, :, :S].cpu().numpy(), k_hat,
                       "prefill int8 rows")
    assert not cache.codes()[:, :, S:].any() and not cache.scales()[:, :, S:].any()


@pytest.mark.parametrize("S,cut", [(700, 300), (1100, 1024)])
def test_int8_prefill_chunk_reads_the_quantised_prefix(S, cut):
    """The second chunk attends over the first chunk's rows as stored (codes x
    scale) and over its own keys at full precision."""
    shape, dev = W.GLOBAL_LAYER, device()
    B = 2
    x = W.PrefillWorkload("q8c", shape, B, S, torch.bfloat16, False, 67).draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = q8_layer(shape)
    cache = api.new_cache(lay, B, S, dev)
    outs = []
    for a, b in [(0, cut), (cut, S)]:
        outs.append(api.gemma_attn_prefill_chunk(lay, a, xd["q"][:, a:b].contiguous(), xd["k"][:, a:b].contiguous(),
                                                 xd["g_q"], xd["g_k"], cache))
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    first = O.prefill(ol, to64(x["q"][:, :cut]), to64(x["k"][:, :cut]), None, to64(x["g_q"]), to64(x["g_k"]))
    assert_close(outs[0], first, torch.bfloat16, f"int8 first chunk of {S}")
    k_hat = O.qk_norm(to64(x["k"]), to64(x["g_k"]), shape.norm_eps).transpose(0, 2, 1, 3)   # [B,Hkv,S,d]
    c, s = O.quantize_rows(k_hat[:, :, :cut])
    rows = np.concatenate([O.dequantize_rows(c, s), k_hat[:, :, cut:]], axis=2)
    second = O.decode_multi_from_cache(ol, to64(x["q"][:, cut:]), to64(x["g_q"]), rows, None, np.full(B, S))
    assert_close(outs[1], second, torch.bfloat16, f"int8 chunk [{cut}, {S}) after the cached prefix")
    assert_codes_match(cache.codes().cpu().numpy(), cache.scales().cpu().numpy(), k_hat, "chunked int8 rows")


def test_int8_global_decode_full_size_sampled():
    """The global decode workload (B=16, contexts 4K..128K) on an int8 cache of
    random codes and scales: the shortest and the longest sequence."""
    wl = W.CONFIGS["global_decode"]
    shape, dev = wl.layer, device()
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    lay = q8_layer(shape)
    cache = api.new_cache(lay, B, cap, dev)
    for b in range(B):   # per sequence, to bound the generator's scratch
        c, s = W.int8_rows((1, shape.n_kv_heads, cap, D), 71 + b, dev)
        cache.codes()[b:b + 1].copy_(c)
        cache.scales()[b:b + 1].copy_(s)
        del c, s
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    out = api.gemma_attn_decode(lay, q, g_q, cache, None, lens.to(dev), int(lens.max()))
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in [int(np.argmin(lens.numpy())), int(np.argmax(lens.numpy()))]:
        L = int(lens[b])
        rows = oracle_rows(cache.codes()[b:b + 1, :, :L], cache.scales()[b:b + 1, :, :L])
        ref = O.decode_from_cache(ol, to64(q[b:b + 1]), to64(g_q), rows, None, np.array([L]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"int8 global decode B16 b={b} L={L}")


def test_int8_edge_cases():
    """Out-of-range append positions write neither codes nor scales; invalid
    decode lengths give NaN rows next to valid ones."""
    shape, dev = W.GLOBAL_LAYER, device()
    D, cap = shape.head_dim, 50
    lay = q8_layer(shape)
    cache = api.new_cache(lay, 3, cap, dev)
    kn = W.normal((3, shape.n_kv_heads, D), 2, "k_new", torch.bfloat16, dev)
    g = torch.ones(D, dtype=torch.bfloat16, device=dev)
    api.kv_append(lay, kn, None, g, torch.tensor([-1, cap, cap - 1], dtype=torch.int32, device=dev), cache)
    torch.cuda.synchronize()
    c, s = cache.codes().cpu(), cache.scales().cpu()
    assert not c[:2].any() and not s[:2].any() and not c[2, :, :cap - 1].any() and not s[2, :, :cap - 1].any()
    assert_codes_match(c[2, :, cap - 1].numpy(), s[2, :, cap - 1].numpy(), O.qk_norm(to64(kn[2]), np.ones(D), 1e-6),
                       "appended int8 row")
    codes, scales = W.int8_rows((3, shape.n_kv_heads, 100, D), 3)
    full = cache_from(lay, codes.to(dev), scales.to(dev))
    q = W.normal((3, shape.n_q_heads, D), 3, "q_dec", torch.bfloat16, "cpu")
    bad = torch.tensor([0, 40, 101], dtype=torch.int32, device=dev)   # 0 and 101 are out of range
    out = api.gemma_attn_decode(lay, q.to(dev), g, full, None, bad, 100).float().cpu()
    assert torch.isnan(out[0]).all() and torch.isnan(out[2]).all()
    ref = O.decode_from_cache(oracle_layer(shape), to64(q), np.ones(D), oracle_rows(codes, scales), None,
                              np.array([0, 40, 100]), batches=[1])
    assert_close(out[1:2], ref, torch.bfloat16, "int8: valid row next to invalid ones")
