"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Oracle-sized cases compare every output element; the full-size workloads run
in the benchmark's launch configuration and compare sampled rows the oracle
computes one by one.  Every input is seeded and synthetic.
"""

import numpy as np
import pytest
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, assert_close, device, oracle_layer, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _prefill_case(shape, B, S, dtype, unit_gains, seed, cap=None):
    dev = device()
    wl = W.PrefillWorkload("case", shape, B, S, dtype, unit_gains, seed)
    x = wl.draw("cpu")
    lay = api_layer(shape, dtype)
    if shape.window:
        cap = shape.window
    elif cap is None:
        cap = S
    kc = torch.full((B, shape.n_kv_heads, cap, shape.head_dim), float("nan"), dtype=dtype, device=dev)
    vc = None if shape.kv_shared else torch.full_like(kc, float("nan"))
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    out = torch.full_like(xd["q"], float("nan"))
    api.gemma_attn_prefill(lay, xd["q"], xd["k"], xd["v"], xd["g_q"], xd["g_k"], kc, vc, out)
    torch.cuda.synchronize()
    return x, xd, out, kc, vc


# ---- the tiny fp32 case: prefill of 256 tokens, then 16 decode steps --------------

@pytest.mark.parametrize("name", ["tiny_global", "tiny_local"])
def test_tiny_fp32_prefill_then_decode(name):
    wl = W.CONFIGS[name]
    shape, S, steps = wl.layer, wl.seq_len, W.TINY_DECODE_STEPS
    T = S + steps
    full = W.with_seq(wl, T).draw("cpu")              # one sequence of S + 16 tokens
    dev = device()
    lay = api_layer(shape, torch.float32)
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(full["q"]), to64(full["k"]), None if full["v"] is None else to64(full["v"]),
                    to64(full["g_q"]), to64(full["g_k"]))
    cap = shape.window if shape.window else T
    kc = torch.full((1, shape.n_kv_heads, cap, shape.head_dim), float("nan"), device=dev)
    vc = None if shape.kv_shared else torch.full_like(kc, float("nan"))
    q = full["q"].to(dev)
    k = full["k"].to(dev)
    v = None if full["v"] is None else full["v"].to(dev)
    g_q, g_k = full["g_q"].to(dev), full["g_k"].to(dev)
    out = api.gemma_attn_prefill(lay, q[:, :S].contiguous(), k[:, :S].contiguous(),
                                 None if v is None else v[:, :S].contiguous(), g_q, g_k, kc, vc)
    assert_close(out, ref[:, :S], torch.float32, f"{name} prefill")
    okc, ovc = O.expected_caches_after_prefill(ol, to64(full["k"][:, :S]),
                                               None if v is None else to64(full["v"][:, :S]),
                                               to64(full["g_k"]), cap)
    filled = ~np.isnan(okc)
    assert_close(kc.cpu()[torch.from_numpy(filled)], okc[filled], torch.float32, f"{name} k cache")
    if vc is not None:
        assert_close(vc.cpu()[torch.from_numpy(filled)], ovc[filled], torch.float32, f"{name} v cache")
    ws = api.workspace(api.gemma_attn_decode_workspace_size(lay, 1, T), dev)
    for t in range(S, T):
        pos = torch.tensor([t], dtype=torch.int32, device=dev)
        api.kv_append(lay, k[:, t].contiguous(), None if v is None else v[:, t].contiguous(), g_k, pos, kc, vc)
        o = api.gemma_attn_decode(lay, q[:, t].contiguous(), g_q, kc, vc, pos + 1, T, ws=ws)
        assert_close(o, ref[:, t], torch.float32, f"{name} decode step {t}")


# ---- bf16 prefill at oracle-sized shapes (several tiles + ragged tails) -----------

PREFILL_CASES = [
    ("global_S300", W.GLOBAL_LAYER, 1, 300),
    ("global_S1000_B2", W.GLOBAL_LAYER, 2, 1000),
    ("local_W1024_S1100_B2", W.LOCAL_LAYER, 2, 1100),
    ("local_W64_S300", W.replace(W.LOCAL_LAYER, window=64), 1, 300),
    ("global_G4", W.replace(W.GLOBAL_LAYER, n_q_heads=16), 1, 200),
    ("local_G1_W100", W.replace(W.LOCAL_LAYER, n_q_heads=16, window=100), 1, 257),
    # 12 workgroups: the XCD-aware order of windowed layers with a grid that 8 does not divide
    ("local_Hkv3_W64", W.replace(W.LOCAL_LAYER, n_q_heads=6, n_kv_heads=3, window=64), 1, 200),
    # the smaller models' layer types: global without K=V (separate V cache), 512-token window
    ("e_global_separate_v", W.E_GLOBAL_LAYER, 2, 300),
    ("e_local_W512", W.E_LOCAL_LAYER, 1, 1100),
]


@pytest.mark.parametrize("name,shape,B,S", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_bf16_all_rows(name, shape, B, S):
    x, xd, out, kc, vc = _prefill_case(shape, B, S, torch.bfloat16, False, seed=11)
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), None if x["v"] is None else to64(x["v"]),
                    to64(x["g_q"]), to64(x["g_k"]))
    assert_close(out, ref, torch.bfloat16, f"{name} prefill")
    cap = kc.shape[2]
    okc, ovc = O.expected_caches_after_prefill(ol, to64(x["k"]), None if x["v"] is None else to64(x["v"]),
                                               to64(x["g_k"]), cap)
    filled = ~np.isnan(okc)
    assert_close(kc.cpu()[torch.from_numpy(filled)], okc[filled], torch.bfloat16, f"{name} k cache")
    assert torch.isnan(kc.cpu()[torch.from_numpy(~filled)]).all(), "prefill wrote cache slots it should not"
    if vc is not None:
        assert_close(vc.cpu()[torch.from_numpy(filled)], ovc[filled], torch.bfloat16, f"{name} v cache")


@pytest.mark.parametrize("kind,S", [("global", 1), ("local", 1), ("global", 33), ("local", 33),
                                    ("global", 32), ("local", 64)])
def test_prefill_short_and_ragged(kind, S):
    shape = W.GLOBAL_LAYER if kind == "global" else W.replace(W.LOCAL_LAYER, window=16)
    x, xd, out, kc, vc = _prefill_case(shape, 1, S, torch.bfloat16, False, seed=5)
    ref = O.prefill(oracle_layer(shape), to64(x["q"]), to64(x["k"]),
                    None if x["v"] is None else to64(x["v"]), to64(x["g_q"]), to64(x["g_k"]))
    assert_close(out, ref, torch.bfloat16, f"{kind} S={S}")


def test_window_of_one_returns_the_value():
    shape = W.replace(W.LOCAL_LAYER, window=1)
    x, xd, out, kc, vc = _prefill_case(shape, 1, 70, torch.float32, False, seed=3)
    want = np.repeat(to64(x["v"]), shape.n_q_heads // shape.n_kv_heads, axis=2)
    assert_close(out, want, torch.float32, "window 1")


# ---- bf16 decode at oracle-sized shapes -----------------------------------------

def _decode_case(shape, lens, dtype, seed, cap=None):
    dev = device()
    B = len(lens)
    D, Hkv = shape.head_dim, shape.n_kv_heads
    cap = shape.window if shape.window else (cap or max(lens))
    kc = W.normal((B, Hkv, cap, D), seed, "k_cache", dtype, "cpu")
    vc = None if shape.kv_shared else W.normal((B, Hkv, cap, D), seed, "v_cache", dtype, "cpu")
    q = W.normal((B, shape.n_q_heads, D), seed, "q_dec", dtype, "cpu")
    g_q = W.gains(D, seed, "g_q", False, dtype)
    lay = api_layer(shape, dtype)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = torch.full((B, shape.n_q_heads, D), float("nan"), dtype=dtype, device=dev)
    api.gemma_attn_decode(lay, q.to(dev), g_q.to(dev), kc.to(dev), None if vc is None else vc.to(dev),
                          seq.to(dev), max(lens), out=out)
    torch.cuda.synchronize()
    return q, g_q, kc, vc, seq, out


DECODE_SHAPES = {"global": W.GLOBAL_LAYER, "local": W.LOCAL_LAYER, "e_global": W.E_GLOBAL_LAYER,
                 "e_local": W.E_LOCAL_LAYER}


@pytest.mark.parametrize("kind,lens", [
    ("global", [1, 17, 1024, 1025, 2600]),
    ("global", [4097, 3000]),
    ("local", [5, 1024, 1025, 5000]),
    ("e_global", [1, 17, 1024, 1025, 2600]),
    ("e_local", [5, 512, 513, 3000]),
])
def test_decode_bf16(kind, lens):
    shape = DECODE_SHAPES[kind]
    q, g_q, kc, vc, seq, out = _decode_case(shape, lens, torch.bfloat16, seed=7)
    ref = O.decode_from_cache(oracle_layer(shape), to64(q), to64(g_q), to64(kc),
                              None if vc is None else to64(vc), seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"{kind} decode {lens}")


def test_layers_sharing_one_cache():
    """Cross-layer cache sharing (the smaller models reuse a layer's cache in
    later layers): a layer that only reads another layer's cache, with its own
    queries and gains, is attention over that cache."""
    shape = W.E_LOCAL_LAYER
    x, xd, out, kc, vc = _prefill_case(shape, 1, 700, torch.bfloat16, False, seed=17)   # the owner fills the ring
    dev = device()
    D = shape.head_dim
    q2 = W.normal((1, shape.n_q_heads, D), 23, "q_dec", torch.bfloat16, dev)
    g2 = W.gains(D, 23, "g_q", False, torch.bfloat16, dev)
    seq = torch.tensor([700], dtype=torch.int32, device=dev)
    got = api.gemma_attn_decode(api_layer(shape, torch.bfloat16), q2, g2, kc, vc, seq, 700)
    torch.cuda.synchronize()
    ref = O.decode_from_cache(oracle_layer(shape), to64(q2), to64(g2), to64(kc), to64(vc), np.array([700]))
    assert_close(got, ref, torch.bfloat16, "reader layer on the owner's cache")


def test_decode_invalid_lengths_write_nan_rows():
    shape = W.GLOBAL_LAYER
    lens = [0, 40, 100]            # cap = 100, max_seq_len = 100
    dev = device()
    D = shape.head_dim
    kc = W.normal((3, 4, 100, D), 1, "k_cache", torch.bfloat16, "cpu")
    q = W.normal((3, 32, D), 1, "q_dec", torch.bfloat16, "cpu")
    g = torch.ones(D, dtype=torch.bfloat16)
    lay = api_layer(shape, torch.bfloat16)
    bad = torch.tensor([0, 40, 101], dtype=torch.int32, device=dev)   # 0 and 101 are out of range
    out = api.gemma_attn_decode(lay, q.to(dev), g.to(dev), kc.to(dev), None, bad, 100)
    o = out.float().cpu()
    assert torch.isnan(o[0]).all() and torch.isnan(o[2]).all()
    ref = O.decode_from_cache(oracle_layer(shape), to64(q), to64(g), to64(kc), None, np.array(lens),
                              batches=[1])
    assert_close(out[1:2], ref, torch.bfloat16, "valid row next to invalid ones")


# ---- several new tokens per sequence at once (global K=V layers) ---------------------

def _multi_case(shape, lens, T, seed, dtype=torch.bfloat16):
    dev = device()
    B, D, cap = len(lens), shape.head_dim, max(lens)
    kc = W.normal((B, shape.n_kv_heads, cap, D), seed, "k_cache", dtype, "cpu")
    q = W.normal((B, T, shape.n_q_heads, D), seed, "q_dec", dtype, "cpu")
    g_q = W.gains(D, seed, "g_q", False, dtype)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = torch.full((B, T, shape.n_q_heads, D), float("nan"), dtype=dtype, device=dev)
    api.gemma_attn_decode_multi(api_layer(shape, dtype), q.to(dev), g_q.to(dev), kc.to(dev), None, seq.to(dev),
                                max(lens), out=out)
    torch.cuda.synchronize()
    return q, g_q, kc, seq, out


@pytest.mark.parametrize("hq,T,lens", [
    (32, 2, [2, 17, 1024, 1025, 2600]),     # G = 8: 16 columns
    (16, 3, [3, 40, 1500]),                  # G = 4: 12 columns, 4 padding
    (8, 8, [8, 33, 700, 2049]),              # G = 2: 16 columns
    (32, 1, [1, 100, 3000]),                 # one token through the multi-token call
    (32, 3, [3, 20, 1030, 2600]),            # G = 8: 24 columns, two passes (2 + 1 tokens)
    (32, 4, [4, 17, 1025, 4100]),            # G = 8: 32 columns, two passes (a 4-token draft)
    (32, 8, [8, 900, 2049]),                 # G = 8: 64 columns, four passes
])
def test_multi_token_decode_bf16(hq, T, lens):
    shape = W.replace(W.GLOBAL_LAYER, n_q_heads=hq)
    q, g_q, kc, seq, out = _multi_case(shape, lens, T, seed=13)
    ref = O.decode_multi_from_cache(oracle_layer(shape), to64(q), to64(g_q), to64(kc), None, seq.numpy())
    assert_close(out, ref, torch.bfloat16, f"multi-token decode G={hq // 4} T={T} {lens}")


def test_multi_token_decode_of_one_token_equals_decode():
    shape = W.GLOBAL_LAYER
    lens = [1, 555, 4100]
    q, g_q, kc, seq, out = _multi_case(shape, lens, 1, seed=21)
    dev = device()
    one = api.gemma_attn_decode(api_layer(shape, torch.bfloat16), q[:, 0].to(dev), g_q.to(dev), kc.to(dev), None,
                                seq.to(dev), max(lens))
    assert torch.equal(out[:, 0].cpu(), one.cpu()), "q_len = 1 must take exactly the single-token path"


def test_multi_token_decode_short_sequences_write_nan_rows():
    shape = W.GLOBAL_LAYER
    q, g_q, kc, seq, out = _multi_case(shape, [1, 2, 300], 2, seed=5)     # L = 1 < q_len = 2
    o = out.float().cpu()
    assert torch.isnan(o[0]).all()
    ref = O.decode_multi_from_cache(oracle_layer(shape), to64(q), to64(g_q), to64(kc), None, seq.numpy(),
                                    batches=[1, 2])
    assert_close(out[1:], ref, torch.bfloat16, "valid sequences next to a short one")


# ---- a later chunk of a prompt against the cached positions (global K=V) ------------

def _chunked(shape, B, S, cuts, seed):
    """Prefill positions 0 .. S-1 as consecutive chunks [cuts[i], cuts[i+1])."""
    dev = device()
    wl = W.PrefillWorkload("chunks", shape, B, S, torch.bfloat16, False, seed)
    x = wl.draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = api_layer(shape, torch.bfloat16)
    kc = torch.full((B, shape.n_kv_heads, S, shape.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(xd["q"], float("nan"))
    bounds = [0] + list(cuts) + [S]
    for a, b in zip(bounds[:-1], bounds[1:]):
        o = api.gemma_attn_prefill_chunk(lay, a, xd["q"][:, a:b].contiguous(), xd["k"][:, a:b].contiguous(),
                                         xd["g_q"], xd["g_k"], kc)
        out[:, a:b] = o
    torch.cuda.synchronize()
    return x, xd, out, kc


@pytest.mark.parametrize("S,cuts", [(700, [300]), (300, [37, 107, 299]), (1100, [1024])])
def test_prefill_in_chunks_equals_the_whole_prompt(S, cuts):
    shape = W.GLOBAL_LAYER
    x, xd, out, kc = _chunked(shape, 2, S, cuts, seed=31)
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), None, to64(x["g_q"]), to64(x["g_k"]))
    assert_close(out, ref, torch.bfloat16, f"chunks {cuts} of {S}")
    okc, _ = O.expected_caches_after_prefill(ol, to64(x["k"]), None, to64(x["g_k"]), S)
    assert_close(kc, okc, torch.bfloat16, "cache after the chunks")


def test_first_chunk_equals_prefill():
    shape = W.GLOBAL_LAYER
    x, xd, out, kc = _chunked(shape, 1, 333, [], seed=33)
    lay = api_layer(shape, torch.bfloat16)
    kc2 = torch.full_like(kc, float("nan"))
    whole = api.gemma_attn_prefill(lay, xd["q"], xd["k"], None, xd["g_q"], xd["g_k"], kc2)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), whole.cpu()) and torch.equal(kc.cpu(), kc2.cpu())


def test_kv_append_ignores_out_of_range_positions():
    shape = W.GLOBAL_LAYER
    dev = device()
    D = shape.head_dim
    kc = torch.zeros((3, 4, 50, D), dtype=torch.bfloat16, device=dev)
    kn = W.normal((3, 4, D), 2, "k_new", torch.bfloat16, dev)
    g = torch.ones(D, dtype=torch.bfloat16, device=dev)
    pos = torch.tensor([-1, 50, 49], dtype=torch.int32, device=dev)
    api.kv_append(api_layer(shape, torch.bfloat16), kn, None, g, pos, kc)
    c = kc.float().cpu()
    assert (c[0] == 0).all() and (c[1] == 0).all()
    want = O.qk_norm(to64(kn[2]), np.ones(D), 1e-6)
    assert_close(kc[2, :, 49], want, torch.bfloat16, "appended slot")
    assert (c[2, :, :49] == 0).all()


def test_results_are_deterministic():
    shape = W.GLOBAL_LAYER
    x, xd, out1, kc, vc = _prefill_case(shape, 1, 700, torch.bfloat16, False, seed=9)
    out2 = api.gemma_attn_prefill(api_layer(shape, torch.bfloat16), xd["q"], xd["k"], None, xd["g_q"],
                                  xd["g_k"])
    assert torch.equal(out1, out2)
    lens = [3000, 10]
    q, g_q, kc, vc, seq, d1 = _decode_case(shape, lens, torch.bfloat16, seed=4)
    dev = device()
    d2 = api.gemma_attn_decode(api_layer(shape, torch.bfloat16), q.to(dev), g_q.to(dev), kc.to(dev), None,
                               seq.to(dev), max(lens))
    assert torch.equal(d1, d2)


# ---- full-size workloads, sampled rows ---------------------------------------------

def _sampled_prefill(wl, rows, batches, what):
    shape, S = wl.layer, wl.seq_len
    dev = device()
    x = wl.draw(dev)
    lay = api_layer(shape, torch.bfloat16)
    cap = shape.window if shape.window else S
    kc = torch.empty((wl.batch, shape.n_kv_heads, cap, shape.head_dim), dtype=torch.bfloat16, device=dev)
    vc = None if shape.kv_shared else torch.empty_like(kc)
    out = api.gemma_attn_prefill(lay, x["q"], x["k"], x["v"], x["g_q"], x["g_k"], kc, vc)
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    r = torch.as_tensor(rows, device=dev)
    hi = int(max(rows)) + 1
    for b in batches:
        ref = O.prefill(ol, to64(x["q"][b:b + 1, r]), to64(x["k"][b:b + 1, :hi]),
                        None if x["v"] is None else to64(x["v"][b:b + 1, :hi]),
                        to64(x["g_q"]), to64(x["g_k"]), rows=np.asarray(rows), q_at_rows=True)
        assert_close(out[b:b + 1, r], ref, torch.bfloat16, f"{what} b={b} rows {list(rows)}")
    # cache: the last written slots of the first sampled sequence
    b = batches[0]
    okc, _ = O.expected_caches_after_prefill(ol, to64(x["k"][b:b + 1, S - 8:]) if shape.kv_shared else
                                             to64(x["k"][b:b + 1]), None if x["v"] is None else
                                             to64(x["v"][b:b + 1]), to64(x["g_k"]),
                                             8 if shape.kv_shared else cap)
    if shape.kv_shared:
        assert_close(kc[b:b + 1, :, S - 8:], okc, torch.bfloat16, f"{what} cache slots")
    else:
        assert_close(kc[b:b + 1], okc, torch.bfloat16, f"{what} k ring")


def test_global_prefill_32k_last_chunk_sampled_rows():
    """The 32K global prefill as 28K positions, then a 4K chunk against them."""
    wl = W.CONFIGS["global_prefill_32k"]
    shape, S, start = wl.layer, wl.seq_len, 28672
    dev = device()
    x = wl.draw(dev)
    lay = api_layer(shape, torch.bfloat16)
    kc = torch.empty((1, shape.n_kv_heads, S, shape.head_dim), dtype=torch.bfloat16, device=dev)
    api.gemma_attn_prefill(lay, x["q"][:, :start].contiguous(), x["k"][:, :start].contiguous(), None, x["g_q"],
                           x["g_k"], kc)
    out = api.gemma_attn_prefill_chunk(lay, start, x["q"][:, start:].contiguous(), x["k"][:, start:].contiguous(),
                                       x["g_q"], x["g_k"], kc)
    torch.cuda.synchronize()
    rows = [start, start + 1, start + 1000, S - 1]
    ref = O.prefill(oracle_layer(shape), to64(x["q"][:, torch.as_tensor(rows, device=dev)]), to64(x["k"]), None,
                    to64(x["g_q"]), to64(x["g_k"]), rows=np.asarray(rows), q_at_rows=True)
    got = out[:, torch.as_tensor([r - start for r in rows], device=dev)]
    assert_close(got, ref, torch.bfloat16, f"last chunk rows {rows}")


def test_global_prefill_32k_sampled_rows():
    _sampled_prefill(W.CONFIGS["global_prefill_32k"], [0, 1, 15, 16, 31, 32, 1023, 12345, 32767], [0],
                     "global prefill 32K")


def test_local_prefill_32k_sampled_rows():
    _sampled_prefill(W.CONFIGS["local_prefill_32k"], [0, 31, 1023, 1024, 1025, 4097, 9999], [0, 3],
                     "local prefill B4 32K")


def _sampled_decode(wl, sample, what, append=False):
    """One decode step (optionally with kv_append first) at full size."""
    shape = wl.layer
    dev = device()
    lens = wl.lengths()
    B = wl.batch
    cap = wl.cache_cap()
    D, Hkv = shape.head_dim, shape.n_kv_heads
    kc = W.normal((B, Hkv, cap, D), wl.seed, "k_cache", torch.bfloat16, dev)
    vc = None if shape.kv_shared else W.normal((B, Hkv, cap, D), wl.seed, "v_cache", torch.bfloat16, dev)
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    g_k = W.gains(D, wl.seed, "g_k", False, torch.bfloat16, dev)
    lay = api_layer(shape, torch.bfloat16)
    seq = lens.to(dev)
    if append:
        kn = W.normal((B, Hkv, D), wl.seed, "k_new", torch.bfloat16, dev)
        vn = None if shape.kv_shared else W.normal((B, Hkv, D), wl.seed, "v_new", torch.bfloat16, dev)
        api.kv_append(lay, kn, vn, g_k, seq - 1, kc, vc)
    out = api.gemma_attn_decode(lay, q, g_q, kc, vc, seq, int(lens.max()))
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in sample:
        L = int(lens[b])
        n = min(L, shape.window) if shape.window else L
        kb = to64(kc[b:b + 1, :, :n])
        vb = None if vc is None else to64(vc[b:b + 1, :, :n])
        ref = O.decode_from_cache(ol, to64(q[b:b + 1]), to64(g_q), kb, vb, np.array([L]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"{what} b={b} L={L}")
        if append:
            slot = (L - 1) % cap
            if shape.kv_shared:
                want = O.qk_norm(to64(kn[b]), to64(g_k), shape.norm_eps)
            else:
                want = O.rotate(O.qk_norm(to64(kn[b]), to64(g_k), shape.norm_eps), L - 1,
                                shape.rope_theta, shape.rope_fraction)
            assert_close(kc[b, :, slot], want, torch.bfloat16, f"{what} appended key b={b}")


def test_global_decode_full_size_sampled():
    wl = W.CONFIGS["global_decode"]
    lens = wl.lengths().numpy()
    _sampled_decode(wl, [int(np.argmin(lens)), int(np.argmax(lens))], "global decode B16")


def test_multi_token_decode_full_size_sampled():
    """Two new tokens per sequence on the global decode workload (B=16,
    contexts up to 128K): the shortest and the longest sequence against the oracle."""
    wl = W.CONFIGS["global_decode"]
    shape, dev = wl.layer, device()
    lens = wl.lengths()
    B, cap, D, T = wl.batch, wl.cache_cap(), shape.head_dim, 2
    kc = W.normal((B, shape.n_kv_heads, cap, D), wl.seed, "k_cache", torch.bfloat16, dev)
    q = W.normal((B, T, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    out = api.gemma_attn_decode_multi(api_layer(shape, torch.bfloat16), q, g_q, kc, None, lens.to(dev),
                                      int(lens.max()))
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    for b in [int(np.argmin(lens.numpy())), int(np.argmax(lens.numpy()))]:
        L = int(lens[b])
        ref = O.decode_multi_from_cache(ol, to64(q[b:b + 1]), to64(g_q), to64(kc[b:b + 1, :, :L]), None,
                                        np.array([L]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"multi-token decode B16 b={b} L={L}")
    del kc


def test_stack_decode_layers_full_size_sampled():
    _sampled_decode(W.CONFIGS["stack_decode_local"], [0, 31], "stack local layer", append=True)
    _sampled_decode(W.CONFIGS["stack_decode_global"], [5], "stack global layer", append=True)
