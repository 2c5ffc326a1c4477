"""GPU parity for every layer type when several new tokens are checked at once
(multi-token decode, as the main model checks drafted tokens) and when a
prompt is prefilled in chunks: windowed layers (ring caches) and global layers
with a separate V cache, beside the global K=V layers of test_gpu_parity.

Each case builds its caches through the library (prefill, kv_append) and
compares with the float64 oracle's prefill of the whole sequence: every token
checked at once, and every row of every chunk, is the row a prefill of the
whole prompt gives ("Gemma 4 Technical Report" notes, §2.6, MTP drafter)."""

import numpy as np
import pytest
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import api_layer, assert_close, device, oracle_layer, to64

pytestmark = pytest.mark.gpu

SHAPES = {"local": W.LOCAL_LAYER, "e_local": W.E_LOCAL_LAYER, "e_global": W.E_GLOBAL_LAYER}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _caches(shape, B, cap, dev):
    kc = torch.full((B, shape.n_kv_heads, cap, shape.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = None if shape.kv_shared else torch.full_like(kc, float("nan"))
    return kc, vc


@pytest.mark.parametrize("kind,S,T,extra", [
    ("local", 2056, 4, 0),       # ring of 1027 slots; new tokens at 2052..2055 sit in slots 1025, 1026, 0, 1
    ("local", 700, 2, 0),        # the ring has not wrapped yet
    ("local", 3000, 2, 5),       # a ring wider than it needs: its oldest slots are outside every window
    ("e_local", 1300, 4, 0),     # W = 512, G = 4: 16 columns
    ("e_local", 515, 3, 0),      # slots wrap within the three new tokens (ring of 514 slots)
    ("e_global", 1500, 4, 0),    # separate-V global layer, slot = position
    ("e_global", 40, 2, 0),
    ("local", 2100, 11, 0),      # 22 columns: two passes over the ring (8 + 3 tokens)
    ("e_global", 900, 7, 0),     # G = 4: 28 columns, two passes (4 + 3 tokens)
])
def test_multi_token_decode_every_layer_type(kind, S, T, extra):
    shape = SHAPES[kind]
    dev = device()
    B = 2
    wl = W.PrefillWorkload("drafts", shape, B, S, torch.bfloat16, False, seed=41)
    x = wl.draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = api_layer(shape, torch.bfloat16)
    cap = shape.window + T - 1 + extra if shape.window else S
    kc, vc = _caches(shape, B, cap, dev)
    # the older tokens by a prefill, then the T new ones by kv_append, as a decode step does
    api.gemma_attn_prefill(lay, xd["q"][:, :S - T].contiguous(), xd["k"][:, :S - T].contiguous(),
                           None if xd["v"] is None else xd["v"][:, :S - T].contiguous(), xd["g_q"], xd["g_k"],
                           kc, vc)
    for t in range(S - T, S):
        pos = torch.full((B,), t, dtype=torch.int32, device=dev)
        api.kv_append(lay, xd["k"][:, t].contiguous(), None if xd["v"] is None else xd["v"][:, t].contiguous(),
                      xd["g_k"], pos, kc, vc)
    seq = torch.full((B,), S, dtype=torch.int32, device=dev)
    out = api.gemma_attn_decode_multi(lay, xd["q"][:, S - T:].contiguous(), xd["g_q"], kc, vc, seq, S)
    torch.cuda.synchronize()
    ol = oracle_layer(shape)
    rows = np.arange(S - T, S)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), None if x["v"] is None else to64(x["v"]), to64(x["g_q"]),
                    to64(x["g_k"]), rows=rows)
    assert_close(out, ref, torch.bfloat16, f"{kind} S={S}: {T} tokens at once vs the prefill rows")
    # the same cache through the oracle's multi-token decode
    ref2 = O.decode_multi_from_cache(ol, to64(x["q"][:, S - T:]), to64(x["g_q"]), to64(kc),
                                     None if vc is None else to64(vc), np.full(B, S))
    assert_close(out, ref2, torch.bfloat16, f"{kind} S={S}: {T} tokens against the written cache")


def test_one_token_on_a_wide_ring_equals_the_prefill_row():
    """Single-token decode over a ring wider than the window masks the slots
    older than the window."""
    shape = W.E_LOCAL_LAYER
    dev = device()
    S, cap = 1400, shape.window + 37
    wl = W.PrefillWorkload("wide", shape, 1, S, torch.bfloat16, False, seed=43)
    x = wl.draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = api_layer(shape, torch.bfloat16)
    kc, vc = _caches(shape, 1, cap, dev)
    api.gemma_attn_prefill(lay, xd["q"][:, :S - 1].contiguous(), xd["k"][:, :S - 1].contiguous(),
                           xd["v"][:, :S - 1].contiguous(), xd["g_q"], xd["g_k"], kc, vc)
    pos = torch.tensor([S - 1], dtype=torch.int32, device=dev)
    api.kv_append(lay, xd["k"][:, S - 1].contiguous(), xd["v"][:, S - 1].contiguous(), xd["g_k"], pos, kc, vc)
    out = api.gemma_attn_decode(lay, xd["q"][:, S - 1].contiguous(), xd["g_q"], kc, vc, pos + 1, S)
    torch.cuda.synchronize()
    ref = O.prefill(oracle_layer(shape), to64(x["q"]), to64(x["k"]), to64(x["v"]), to64(x["g_q"]), to64(x["g_k"]),
                    rows=np.array([S - 1]))[:, 0]
    assert_close(out, ref, torch.bfloat16, "one token on a ring of W + 37 slots")


def _chunked(shape, B, S, cuts, cap, seed):
    dev = device()
    wl = W.PrefillWorkload("chunks", shape, B, S, torch.bfloat16, False, seed)
    x = wl.draw("cpu")
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    lay = api_layer(shape, torch.bfloat16)
    kc, vc = _caches(shape, B, cap, dev)
    out = torch.full_like(xd["q"], float("nan"))
    bounds = [0] + list(cuts) + [S]
    for a, b in zip(bounds[:-1], bounds[1:]):
        print(f"[chunks] {shape.window} chunk {a}..{b}", flush=True)
        out[:, a:b] = api.gemma_attn_prefill_chunk(
            lay, a, xd["q"][:, a:b].contiguous(), xd["k"][:, a:b].contiguous(), xd["g_q"], xd["g_k"], kc,
            v=None if xd["v"] is None else xd["v"][:, a:b].contiguous(), v_cache=vc)
    torch.cuda.synchronize()
    return x, out, kc, vc


@pytest.mark.parametrize("kind,S,cuts,extra", [
    ("local", 2200, [600, 1500], 0),     # the second chunk crosses W = 1024; the third starts past it
    ("local", 1300, [1030], 3),          # a ring of W + 3 slots; the chunk starts after a wrap
    ("local", 300, [37, 107, 299], 0),   # short chunks inside the first window
    ("e_local", 1300, [400, 900], 0),    # W = 512
    ("e_global", 700, [300], 0),         # separate-V global layer
    ("e_global", 300, [37, 107, 299], 0),
])
def test_prefill_in_chunks_every_layer_type(kind, S, cuts, extra):
    shape = SHAPES[kind]
    B = 2
    cap = shape.window + extra if shape.window else S
    x, out, kc, vc = _chunked(shape, B, S, cuts, cap, seed=47)
    ol = oracle_layer(shape)
    ref = O.prefill(ol, to64(x["q"]), to64(x["k"]), to64(x["v"]), to64(x["g_q"]), to64(x["g_k"]))
    assert_close(out, ref, torch.bfloat16, f"{kind} chunks {cuts} of {S} vs the whole prompt")
    okc, ovc = O.expected_caches_after_prefill(ol, to64(x["k"]), to64(x["v"]), to64(x["g_k"]), cap)
    filled = ~np.isnan(okc)
    assert filled.all() or shape.window == 0 or S < cap
    assert_close(kc.cpu()[torch.from_numpy(filled)], okc[filled], torch.bfloat16, f"{kind} k cache after chunks")
    assert_close(vc.cpu()[torch.from_numpy(filled)], ovc[filled], torch.bfloat16, f"{kind} v cache after chunks")


def test_local_chunks_equal_the_whole_prefill_bit_for_bit_in_the_first_chunk():
    """A first chunk (start = 0) is gemma_attn_prefill itself."""
    shape = W.LOCAL_LAYER
    x, out, kc, vc = _chunked(shape, 1, 500, [], shape.window, seed=49)
    dev = device()
    lay = api_layer(shape, torch.bfloat16)
    kc2, vc2 = _caches(shape, 1, shape.window, dev)
    xd = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    whole = api.gemma_attn_prefill(lay, xd["q"], xd["k"], xd["v"], xd["g_q"], xd["g_k"], kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), whole.cpu())
    filled = ~torch.isnan(kc2.float().cpu())
    assert torch.equal(kc.cpu()[filled], kc2.cpu()[filled]) and torch.equal(vc.cpu()[filled], vc2.cpu()[filled])


def test_kv_append_into_a_separate_v_global_cache():
    """Global layer without K=V: the appended key is stored normalised and
    rotated at slot = position, the value raw."""
    shape = W.E_GLOBAL_LAYER
    dev = device()
    B, S, D, Hkv = 3, 64, shape.head_dim, shape.n_kv_heads
    lay = api_layer(shape, torch.bfloat16)
    kc, vc = _caches(shape, B, S, dev)
    kn = W.normal((B, Hkv, D), 51, "k_new", torch.bfloat16, "cpu")
    vn = W.normal((B, Hkv, D), 51, "v_new", torch.bfloat16, "cpu")
    g_k = W.gains(D, 51, "g_k", False, torch.bfloat16)
    positions = np.array([0, 17, 63])
    api.kv_append(lay, kn.to(dev), vn.to(dev), g_k.to(dev), torch.tensor(positions, dtype=torch.int32, device=dev),
                  kc, vc)
    torch.cuda.synchronize()
    okc, ovc = O.expected_caches_after_append(oracle_layer(shape), np.full((B, Hkv, S, D), np.nan),
                                              np.full((B, Hkv, S, D), np.nan), to64(kn), to64(vn), to64(g_k),
                                              positions)
    for b, p in enumerate(positions):
        assert_close(kc[b, :, p], okc[b, :, p], torch.bfloat16, f"appended key at {p}")
        assert torch.equal(vc[b, :, p].cpu(), vn[b]), "the value is stored as given"
    untouched = np.isnan(okc)
    assert torch.isnan(kc.float().cpu()[torch.from_numpy(untouched)]).all()
