"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import pytest

from global_gqa_rope_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma_attn.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keywords = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in keywords})


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert {"gemma_attn_prefill", "gemma_attn_decode", "kv_append"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gemma_attn.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_version(lib):
    assert lib.gemma_attn_version().startswith(b"gemma_attn")


def L(hq=32, hkv=4, d=512, window=0, shared=1, theta=1e6, p=0.25, eps=1e-6, dtype=0, cache=0):
    return _lib.GaLayer(hq, hkv, d, window, shared, theta, p, eps, 0.0, dtype, cache)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def prefill(lib, layer, B=1, S=16, v=None, k_cache=None, v_cache=None, cap=0, ws=FAKE, ws_bytes=1 << 40,
            out=FAKE):
    return lib.gemma_attn_prefill(ctypes.byref(layer), B, S, FAKE, FAKE, v, FAKE, FAKE, k_cache,
                                  v_cache, cap, out, ws, ws_bytes, None)


@pytest.mark.parametrize("layer,status,msg", [
    (L(hkv=5), 1, "multiple"),
    (L(d=0), 1, "positive"),
    (L(d=513), 1, "even"),
    (L(p=0.3), 1, "whole number"),
    (L(p=1.5), 1, "rope_fraction"),
    (L(eps=0.0), 1, "norm_eps"),
    (L(theta=-1.0), 1, "rope_theta"),
    (L(dtype=7), 1, "dtype"),
    (L(d=128, p=1.0), 2, "head_dim"),
    (L(hq=48, hkv=3), 2, "1, 2, 4, 8"),
    (L(window=64), 2, "window 0"),
    (L(p=0.5), 2, "64 pairs"),
    (L(cache=3), 1, "cache_format"),
    (L(cache=2, dtype=1), 2, "pre-rotated cache"),
    (L(cache=2, hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0), 2, "pre-rotated cache"),
    (L(cache=1, dtype=1), 2, "int8 cache"),
    (L(cache=1, hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0), 2, "int8 cache"),
    (L(cache=1, hq=8, hkv=4), 2, "int8 cache"),
])
def test_layer_validation(lib, layer, status, msg):
    assert prefill(lib, layer) == status
    assert msg in lib.gemma_attn_last_error().decode()


def test_prefill_argument_validation(lib):
    g = L()
    assert prefill(lib, g, v=FAKE) == 1                      # K=V takes no v
    loc = L(hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0)
    assert prefill(lib, loc, v=None) == 1                    # local needs v
    assert prefill(lib, loc, v=FAKE, k_cache=FAKE, v_cache=FAKE, cap=512) == 1   # ring >= W
    assert "at least the window" in lib.gemma_attn_last_error().decode()
    assert prefill(lib, g, k_cache=FAKE, cap=8, S=16) == 1   # cache too small
    assert prefill(lib, g, k_cache=FAKE, v_cache=FAKE, cap=64) == 1
    assert prefill(lib, g, ws=None, ws_bytes=0) == 3
    need = lib.gemma_attn_prefill_workspace_size(ctypes.byref(g), 1, 16)
    assert need > 0
    assert prefill(lib, g, ws_bytes=need - 1) == 3
    assert prefill(lib, g, ws=ctypes.c_void_p(0x1001)) == 1  # alignment
    assert prefill(lib, g, out=ctypes.c_void_p(0x1008)) == 1  # rows move in 16-byte pieces
    assert "16-byte aligned" in lib.gemma_attn_last_error().decode()
    assert prefill(lib, g, B=-1) == 1
    assert prefill(lib, g, B=0) == 0 and prefill(lib, g, S=0) == 0   # no-ops, no launch


def test_decode_and_append_validation(lib):
    g = L()
    dec = lambda **kw: lib.gemma_attn_decode(
        ctypes.byref(kw.get("layer", g)), kw.get("B", 2), FAKE, FAKE, FAKE, kw.get("v", None),
        kw.get("cap", 4096), FAKE, kw.get("max_len", 4096), FAKE, kw.get("ws", FAKE),
        kw.get("ws_bytes", 1 << 40), None)
    assert dec(v=FAKE) == 1
    assert dec(max_len=0) == 1
    assert dec(cap=0) == 1
    assert dec(ws=None, ws_bytes=0) == 3
    assert dec(B=0) == 0
    assert lib.gemma_attn_decode_workspace_size(ctypes.byref(g), 2, 4096) == decode_ws(2, 4, 8, 512, 4096)
    assert lib.gemma_attn_decode_workspace_size(ctypes.byref(g), 2, 1000) == decode_ws(2, 4, 8, 512, 1000)
    app = lambda **kw: lib.kv_append(ctypes.byref(kw.get("layer", g)), 2, FAKE, kw.get("v", None),
                                     FAKE, kw.get("pos", FAKE), FAKE, kw.get("vc", None),
                                     kw.get("cap", 4096), None)
    assert app(v=FAKE) == 1
    assert app(pos=None) == 1
    loc = L(hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0)
    assert app(layer=loc, v=FAKE, vc=None, cap=1024) == 1


def test_multi_token_decode_validation(lib):
    g = L()                                                     # global K=V, G = 8
    loc = L(hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0)
    dec = lambda **kw: lib.gemma_attn_decode_multi(
        ctypes.byref(kw.get("layer", g)), 2, kw.get("T", 2), FAKE, FAKE, FAKE, kw.get("v", None),
        kw.get("cap", 4096), FAKE, 4096, FAKE, FAKE, 1 << 40, None)
    assert dec(T=0) == 1                                        # q_len >= 1
    assert dec(T=9) == 2                                        # 9 tokens x 8 heads > 64 columns
    assert "64 query columns" in lib.gemma_attn_last_error().decode()
    assert dec(layer=loc, T=2, v=FAKE, cap=1024) == 1           # a W-slot ring is too small for 2 tokens
    assert "1025 slots" in lib.gemma_attn_last_error().decode()
    wsz = lambda layer, B, T, n: lib.gemma_attn_decode_multi_workspace_size(ctypes.byref(layer), B, T, n)
    assert wsz(g, 2, 0, 4096) == 0 and wsz(g, 2, 9, 4096) == 0
    # 17..32 columns: two column groups of 16, each with its own partials (and half the
    # workgroups, which the size query does not depend on); more take several launches
    two_groups = 2 * decode_ws(2, 4, 16, 512, 4096) - 256
    assert wsz(g, 2, 3, 4096) == wsz(g, 2, 4, 4096) == wsz(g, 2, 8, 4096) == two_groups
    assert wsz(loc, 2, 2, 4096) == decode_ws(2, 16, 4, 256, 4096)     # 2 tokens x G = 2 columns per slot
    # one token is the single-token call; two tokens widen every slot to 2 G d outputs
    assert wsz(g, 2, 1, 4096) == lib.gemma_attn_decode_workspace_size(ctypes.byref(g), 2, 4096)
    assert wsz(g, 2, 2, 4096) == decode_ws(2, 4, 16, 512, 4096)
    g2 = L(hq=8, hkv=4, d=512, shared=1)                         # G = 2: up to 8 tokens
    assert wsz(g2, 3, 8, 1000) == decode_ws(3, 4, 16, 512, 1000)


def test_prefill_chunk_validation(lib):
    g = L()
    loc = L(hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0)
    ch = lambda **kw: lib.gemma_attn_prefill_chunk(
        ctypes.byref(kw.get("layer", g)), 1, kw.get("start", 64), kw.get("chunk", 16), FAKE, FAKE, kw.get("v", None),
        FAKE, FAKE, kw.get("kc", FAKE), kw.get("vc", None), kw.get("cap", 4096), FAKE, FAKE, 1 << 40, None)
    assert ch(layer=loc, cap=1024) == 1                         # a separate-V layer needs v
    assert ch(layer=loc, v=FAKE, cap=1024) == 1                 # ... and v_cache
    assert ch(layer=loc, v=FAKE, vc=FAKE, cap=1000) == 1        # a ring of at least W slots
    assert "at least the window" in lib.gemma_attn_last_error().decode()
    assert ch(v=FAKE) == 1                                      # K=V layers take no v
    assert ch(kc=None) == 1                                     # the cached positions live in k_cache
    assert ch(cap=79) == 1                                      # cap >= start + chunk
    assert ch(start=-1) == 1
    assert ch(chunk=0) == 0                                     # no-op
    wsz = lambda start, chunk: lib.gemma_attn_prefill_chunk_workspace_size(ctypes.byref(g), 2, start, chunk)
    # the workspace of a prefill of start + chunk positions
    assert wsz(1000, 37) == lib.gemma_attn_prefill_workspace_size(ctypes.byref(g), 2, 1037)
    assert wsz(0, 512) == lib.gemma_attn_prefill_workspace_size(ctypes.byref(g), 2, 512)


def test_workspace_sizes_follow_the_layout(lib):
    g = L()
    # tables (S_pad * 64 pairs, 8 B in fp32 and 4 B in fp16) + key rows
    # [B,Hkv,S_pad,128] (the rotated head of a K=V layer) + value rows
    # [B,Hkv,S_pad,512], bf16 + the largest squared key length of each
    # 32-row tile [B,Hkv,S_pad/32], fp32
    s_pad = 32768
    want = s_pad * 64 * (8 + 4) + 1 * 4 * s_pad * 128 * 2 + 1 * 4 * s_pad * 512 * 2 + 1 * 4 * (s_pad // 32) * 4
    assert lib.gemma_attn_prefill_workspace_size(ctypes.byref(g), 1, 32768) == want
    loc = L(hq=32, hkv=16, d=256, window=1024, shared=0, theta=1e4, p=1.0)
    # at most 1024 / waves workgroups: the scratch stops growing with max_seq_len
    assert lib.gemma_attn_decode_workspace_size(ctypes.byref(loc), 32, 65537) == decode_ws(32, 16, 2, 256, 65537)
    assert decode_ws(32, 16, 2, 256, 65537) == decode_ws(32, 16, 2, 256, 1024)


def decode_ws(B, hkv, G, d, keys, waves=4):
    """Decode scratch: B+1 int32 tile offsets padded to 256 B, then one fp32
    slot of G*d outputs + 64 (max, sum) words per wave and (workgroup, segment)
    pair: waves * (P + B*hkv) slots for the largest grid P the launch may pick,
    P = min(1024 / waves, ceil(B * hkv * ceil(keys / 16) / (2 * waves)))."""
    tiles = B * hkv * -(-keys // 16)
    P = min(1024 // waves, -(-tiles // (2 * waves)))
    prefix = -(-(B + 1) * 4 // 256) * 256
    return prefix + waves * (P + B * hkv) * (G * d + 64) * 4


def test_cache_bytes(lib):
    g = L()
    assert lib.gemma_attn_cache_bytes(ctypes.byref(g), 2, 100) == 2 * 4 * 100 * 512 * 2
    q8 = L(cache=1)
    # codes [B,Hkv,cap,d] bytes, padded to 256 B, then one fp32 scale per row
    codes = 2 * 4 * 100 * 512
    assert lib.gemma_attn_cache_bytes(ctypes.byref(q8), 2, 100) == -(-codes // 256) * 256 + 2 * 4 * 100 * 4
    e = L(hq=8, hkv=2, cache=1)
    codes = 3 * 2 * 7 * 512
    assert lib.gemma_attn_cache_bytes(ctypes.byref(e), 3, 7) == -(-codes // 256) * 256 + 3 * 2 * 7 * 4
    pre = L(cache=2)
    # rows [B,Hkv,cap,d] bf16 (the native K=V cache), then heads [B,Hkv,cap,2 n_rot] bf16
    rows = 2 * 4 * 100 * 512 * 2
    assert lib.gemma_attn_cache_bytes(ctypes.byref(pre), 2, 100) == -(-rows // 256) * 256 + 2 * 4 * 100 * 128 * 2
    assert lib.gemma_attn_cache_bytes(ctypes.byref(L(cache=5)), 1, 1) == 0   # invalid layer


def test_int8_cache_alignment_is_checked(lib):
    q8 = L(cache=1)
    odd = ctypes.c_void_p(0x1008)
    st = lib.gemma_attn_decode(ctypes.byref(q8), 1, FAKE, FAKE, odd, None, 64, FAKE, 64, FAKE, FAKE, 1 << 40, None)
    assert st == 1 and "16-byte" in lib.gemma_attn_last_error().decode()
    pos = FAKE
    st = lib.kv_append(ctypes.byref(q8), 1, FAKE, None, FAKE, pos, odd, None, 64, None)
    assert st == 1 and "16-byte" in lib.gemma_attn_last_error().decode()


def test_binding_checks_cache_formats():
    """The torch binding rejects a cache of the wrong kind before any call."""
    from dataclasses import replace

    import torch

    from global_gqa_rope_amd import api
    from global_gqa_rope_amd import workloads as W

    base = api.Layer.from_shape(W.GLOBAL_LAYER, torch.bfloat16)
    q8, pre = replace(base, cache_format=1), replace(base, cache_format=2)
    q = torch.zeros(2, 32, 512, dtype=torch.bfloat16)
    plain = torch.zeros(2, 4, 16, 512, dtype=torch.bfloat16)
    for lay, kind in ((q8, "Int8Cache"), (pre, "PrerotatedCache")):
        with pytest.raises(ValueError, match=kind):
            api.gemma_attn_decode(lay, q, q[0, 0], plain, None, torch.zeros(2, dtype=torch.int32), 16)
    c8 = api.new_cache(q8, 2, 16, "cpu")
    cp = api.new_cache(pre, 2, 16, "cpu")
    assert c8.buf.numel() == api.cache_bytes(q8, 2, 16) and cp.buf.numel() == api.cache_bytes(pre, 2, 16)
    assert cp.rows().shape == (2, 4, 16, 512) and cp.heads().shape == (2, 4, 16, 128)
    with pytest.raises(ValueError, match="Int8Cache"):
        api.gemma_attn_decode(q8, q, q[0, 0], cp, None, torch.zeros(2, dtype=torch.int32), 16)
    with pytest.raises(ValueError, match="another batch"):          # made for B=2, used with B=3
        api.gemma_attn_decode(q8, torch.zeros(3, 32, 512, dtype=torch.bfloat16), q[0, 0], c8, None,
                              torch.zeros(3, dtype=torch.int32), 16)
    with pytest.raises(ValueError, match="device tensor"):           # the binding only passes device memory
        api.gemma_attn_decode(q8, q, q[0, 0], c8, None, torch.zeros(2, dtype=torch.int32), 16)
    with pytest.raises(api.GemmaAttnError, match="int8 cache"):      # no int8 cache for local layers
        api.new_cache(replace(api.Layer.from_shape(W.LOCAL_LAYER, torch.bfloat16), cache_format=1), 1, 8, "cpu")


def test_calibration_probe_validation(lib):
    """The measurement probes reject bad arguments on the host."""
    sink = FAKE
    assert lib.gemma_attn_calibrate_mfma(None, 8, 4, 1, sink, None) == 1
    assert lib.gemma_attn_calibrate_mfma(FAKE, 0, 4, 1, sink, None) == 1
    assert lib.gemma_attn_calibrate_mfma(FAKE, 8, 4, 0, sink, None) == 1
    assert lib.gemma_attn_calibrate_stream(FAKE, 24, 1, sink, None) == 1        # not a multiple of 16
    assert "multiple of 16" in lib.gemma_attn_last_error().decode()
    assert lib.gemma_attn_calibrate_stream(FAKE, 32, 1, None, None) == 1
