"""Torch-facing binding of the C ABI: argument marshalling only.

Every function here checks tensor devices, dtypes and shapes, passes raw
device pointers and the current HIP stream to libgemma_attn.so, and raises
GemmaAttnError on a non-OK status.  No step of the computation runs here.
Names follow the C entry points.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import GaLayer, GemmaAttnError  # noqa: F401

_DTYPES = {torch.bfloat16: _lib.GA_BF16, torch.float32: _lib.GA_F32}


@dataclass(frozen=True)
class Layer:
    """Python mirror of ga_layer."""

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    kv_shared: bool
    rope_theta: float
    rope_fraction: float
    norm_eps: float = 1e-6
    softmax_scale: float = 0.0     # <= 0: 1/sqrt(head_dim)
    dtype: torch.dtype = torch.bfloat16
    cache_format: int = 0          # GA_CACHE_NATIVE; 1 = GA_CACHE_INT8, 2 = GA_CACHE_PREROTATED (global K=V, bf16)

    def struct(self) -> GaLayer:
        return GaLayer(self.n_q_heads, self.n_kv_heads, self.head_dim, self.window,
                       int(self.kv_shared), self.rope_theta, self.rope_fraction, self.norm_eps,
                       self.softmax_scale, _DTYPES[self.dtype], int(self.cache_format))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @staticmethod
    def from_shape(shape, dtype: torch.dtype, softmax_scale: float = 0.0) -> "Layer":
        return Layer(shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.window,
                     shape.kv_shared, shape.rope_theta, shape.rope_fraction, shape.norm_eps,
                     softmax_scale, dtype)


def _ptr(t: torch.Tensor | None, name: str, layer: Layer | None = None, shape=None,
         dtype=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    want = dtype if dtype is not None else (layer.dtype if layer is not None else None)
    if want is not None and t.dtype != want:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {want}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


@dataclass(frozen=True)
class Int8Cache:
    """A GA_CACHE_INT8 cache: one uint8 buffer of gemma_attn_cache_bytes bytes
    holding the int8 codes and then the per-row fp32 scales."""

    buf: torch.Tensor
    batch: int
    cap: int
    n_kv_heads: int
    head_dim: int

    def codes(self) -> torch.Tensor:
        """Codes [B, Hkv, cap, d] (an int8 view)."""
        n = self.batch * self.n_kv_heads * self.cap * self.head_dim
        return self.buf[:n].view(torch.int8).view(self.batch, self.n_kv_heads, self.cap, self.head_dim)

    def scales(self) -> torch.Tensor:
        """Row scales [B, Hkv, cap] (a view)."""
        n = self.batch * self.n_kv_heads * self.cap * self.head_dim
        off = (n + 255) // 256 * 256
        rows = self.batch * self.n_kv_heads * self.cap
        return self.buf[off:off + 4 * rows].view(torch.float32).view(self.batch, self.n_kv_heads, self.cap)


@dataclass(frozen=True)
class PrerotatedCache:
    """A GA_CACHE_PREROTATED cache: one uint8 buffer of gemma_attn_cache_bytes
    bytes holding the K=V rows and then each row's rotated head."""

    buf: torch.Tensor
    batch: int
    cap: int
    n_kv_heads: int
    head_dim: int
    head_width: int                # 2 n_rot
    dtype: torch.dtype = torch.bfloat16

    def rows(self) -> torch.Tensor:
        """Normalised, unrotated rows [B, Hkv, cap, d] (a view)."""
        n = self.batch * self.n_kv_heads * self.cap * self.head_dim
        return self.buf[:n * 2].view(self.dtype).view(self.batch, self.n_kv_heads, self.cap, self.head_dim)

    def heads(self) -> torch.Tensor:
        """Rotated heads [B, Hkv, cap, 2 n_rot] (a view)."""
        off = (self.batch * self.n_kv_heads * self.cap * self.head_dim * 2 + 255) // 256 * 256
        n = self.batch * self.n_kv_heads * self.cap * self.head_width
        return self.buf[off:off + 2 * n].view(self.dtype).view(self.batch, self.n_kv_heads, self.cap,
                                                                 self.head_width)


def cache_bytes(layer: Layer, batch: int, cap: int) -> int:
    n = int(_lib.load().gemma_attn_cache_bytes(ctypes.byref(layer.struct()), batch, cap))
    if n == 0 and batch > 0 and cap > 0:
        raise GemmaAttnError(2, _lib.load().gemma_attn_last_error().decode(errors="replace"))
    return n


def new_cache(layer: Layer, batch: int, cap: int, device):
    """A zeroed cache for this layer: a [B, Hkv, cap, d] tensor, or an Int8Cache."""
    if layer.cache_format == _lib.GA_CACHE_INT8:
        buf = torch.zeros(cache_bytes(layer, batch, cap), dtype=torch.uint8, device=device)
        return Int8Cache(buf, batch, cap, layer.n_kv_heads, layer.head_dim)
    if layer.cache_format == _lib.GA_CACHE_PREROTATED:
        buf = torch.zeros(cache_bytes(layer, batch, cap), dtype=torch.uint8, device=device)
        width = 2 * round(layer.head_dim * layer.rope_fraction / 2)
        return PrerotatedCache(buf, batch, cap, layer.n_kv_heads, layer.head_dim, width, layer.dtype)
    return torch.zeros(batch, layer.n_kv_heads, cap, layer.head_dim, dtype=layer.dtype, device=device)


def _cache(layer: Layer, cache, name: str, batch: int) -> tuple[int | None, int]:
    """(pointer, cache_cap) of a cache argument (None: (None, 0))."""
    if cache is None:
        return None, 0
    if layer.cache_format in (_lib.GA_CACHE_INT8, _lib.GA_CACHE_PREROTATED):
        kind = Int8Cache if layer.cache_format == _lib.GA_CACHE_INT8 else PrerotatedCache
        if not isinstance(cache, kind):
            raise ValueError(f"{name}: this layer's cache format takes a {kind.__name__}")
        if cache.batch != batch or cache.n_kv_heads != layer.n_kv_heads or cache.head_dim != layer.head_dim:
            raise ValueError(f"{name}: cache made for another batch or layer")
        if cache.buf.numel() < cache_bytes(layer, batch, cache.cap):
            raise ValueError(f"{name}: cache buffer too small")
        return _ptr(cache.buf, name, dtype=torch.uint8), cache.cap
    cap = cache.shape[2]
    return _ptr(cache, name, layer, (batch, layer.n_kv_heads, cap, layer.head_dim)), cap


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def gemma_attn_prefill_workspace_size(layer: Layer, batch: int, seq_len: int) -> int:
    return int(_lib.load().gemma_attn_prefill_workspace_size(ctypes.byref(layer.struct()), batch, seq_len))


def gemma_attn_decode_workspace_size(layer: Layer, batch: int, max_seq_len: int) -> int:
    return int(_lib.load().gemma_attn_decode_workspace_size(ctypes.byref(layer.struct()), batch, max_seq_len))


def workspace(nbytes: int, device) -> torch.Tensor:
    """Caller-owned scratch (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _on_stream(t: torch.Tensor, stream) -> torch.Tensor:
    """Mark a tensor this binding allocated as used by `stream` (when one is given).

    Allocations come from the current stream's pool.  A kernel enqueued on
    another stream may still use the block after the binding returns and drops
    its reference; record_stream keeps the caching allocator from handing the
    block out again until that stream's work has finished.
    """
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def gemma_attn_prefill(layer: Layer, q, k, v, q_gain, k_gain, k_cache=None, v_cache=None,
                       out=None, ws=None, stream=None) -> torch.Tensor:
    B, S, Hq, d = q.shape
    Hkv = layer.n_kv_heads
    if out is None:
        out = _on_stream(torch.empty_like(q), stream)
    need = gemma_attn_prefill_workspace_size(layer, B, S)
    if ws is None:
        ws = _on_stream(workspace(need, q.device), stream)
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, vcap = _cache(layer, v_cache, "v_cache", B)
    if v_cache is not None and vcap != cap:
        raise ValueError("k_cache and v_cache differ in capacity")
    st = _lib.load().gemma_attn_prefill(
        ctypes.byref(layer.struct()), B, S,
        _ptr(q, "q", layer, (B, S, Hq, d)), _ptr(k, "k", layer, (B, S, Hkv, d)),
        _ptr(v, "v", layer, (B, S, Hkv, d)), _ptr(q_gain, "q_gain", layer, (d,)),
        _ptr(k_gain, "k_gain", layer, (d,)), kc, vc,
        cap, _ptr(out, "out", layer, (B, S, Hq, d)), _ptr(ws, "workspace", dtype=torch.uint8),
        ws.numel(), _stream(stream))
    _lib.check(st)
    return out


def gemma_attn_prefill_chunk_workspace_size(layer: Layer, batch: int, start: int, chunk: int) -> int:
    return int(_lib.load().gemma_attn_prefill_chunk_workspace_size(ctypes.byref(layer.struct()), batch, start,
                                                                     chunk))


def gemma_attn_prefill_chunk(layer: Layer, start: int, q, k, q_gain, k_gain, k_cache, out=None, ws=None,
                             stream=None, v=None, v_cache=None) -> torch.Tensor:
    """Positions start .. start + chunk - 1 against the positions already in the caches."""
    B, T, Hq, d = q.shape
    Hkv = layer.n_kv_heads
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, vcap = _cache(layer, v_cache, "v_cache", B)
    if v_cache is not None and vcap != cap:
        raise ValueError("k_cache and v_cache differ in capacity")
    if out is None:
        out = _on_stream(torch.empty_like(q), stream)
    if ws is None:
        ws = _on_stream(workspace(gemma_attn_prefill_chunk_workspace_size(layer, B, start, T), q.device), stream)
    st = _lib.load().gemma_attn_prefill_chunk(
        ctypes.byref(layer.struct()), B, int(start), T, _ptr(q, "q", layer, (B, T, Hq, d)),
        _ptr(k, "k", layer, (B, T, Hkv, d)), _ptr(v, "v", layer, (B, T, Hkv, d)),
        _ptr(q_gain, "q_gain", layer, (d,)), _ptr(k_gain, "k_gain", layer, (d,)), kc, vc, cap,
        _ptr(out, "out", layer, (B, T, Hq, d)), _ptr(ws, "workspace", dtype=torch.uint8), ws.numel(),
        _stream(stream))
    _lib.check(st)
    return out


def kv_append(layer: Layer, k_new, v_new, k_gain, positions, k_cache, v_cache=None,
              stream=None) -> None:
    B, Hkv, d = k_new.shape
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, _ = _cache(layer, v_cache, "v_cache", B)
    st = _lib.load().kv_append(
        ctypes.byref(layer.struct()), B, _ptr(k_new, "k_new", layer, (B, Hkv, d)),
        _ptr(v_new, "v_new", layer, (B, Hkv, d)), _ptr(k_gain, "k_gain", layer, (d,)),
        _ptr(positions, "positions", dtype=torch.int32, shape=(B,)),
        kc, vc, cap, _stream(stream))
    _lib.check(st)


def gemma_attn_decode(layer: Layer, q, q_gain, k_cache, v_cache, seq_lens, max_seq_len: int,
                      out=None, ws=None, stream=None) -> torch.Tensor:
    B, Hq, d = q.shape
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, _ = _cache(layer, v_cache, "v_cache", B)
    if out is None:
        out = _on_stream(torch.empty_like(q), stream)
    if ws is None:
        ws = _on_stream(workspace(gemma_attn_decode_workspace_size(layer, B, max_seq_len), q.device), stream)
    st = _lib.load().gemma_attn_decode(
        ctypes.byref(layer.struct()), B, _ptr(q, "q", layer, (B, Hq, d)),
        _ptr(q_gain, "q_gain", layer, (d,)), kc, vc, cap,
        _ptr(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,)), int(max_seq_len),
        _ptr(out, "out", layer, (B, Hq, d)), _ptr(ws, "workspace", dtype=torch.uint8), ws.numel(),
        _stream(stream))
    _lib.check(st)
    return out


def gemma_attn_decode_noalloc(layer: Layer, q, q_gain, k_cache, v_cache, seq_lens, max_seq_len: int, out,
                              stream=None) -> torch.Tensor:
    """gemma_attn_decode on the library's static per-GPU scratch: neither this
    binding nor the library allocates device memory, so `out` is required."""
    B, Hq, d = q.shape
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, _ = _cache(layer, v_cache, "v_cache", B)
    st = _lib.load().gemma_attn_decode_noalloc(
        ctypes.byref(layer.struct()), B, _ptr(q, "q", layer, (B, Hq, d)),
        _ptr(q_gain, "q_gain", layer, (d,)), kc, vc, cap,
        _ptr(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,)), int(max_seq_len),
        _ptr(out, "out", layer, (B, Hq, d)), _stream(stream))
    _lib.check(st)
    return out


def gemma_attn_decode_multi_workspace_size(layer: Layer, batch: int, q_len: int, max_seq_len: int) -> int:
    return int(_lib.load().gemma_attn_decode_multi_workspace_size(ctypes.byref(layer.struct()), batch, q_len,
                                                                    max_seq_len))


def gemma_attn_decode_multi(layer: Layer, q, q_gain, k_cache, v_cache, seq_lens, max_seq_len: int,
                            out=None, ws=None, stream=None) -> torch.Tensor:
    """q [B, q_len, Hq, d]: the last q_len positions of each sequence against its cache."""
    B, T, Hq, d = q.shape
    kc, cap = _cache(layer, k_cache, "k_cache", B)
    vc, _ = _cache(layer, v_cache, "v_cache", B)
    if out is None:
        out = _on_stream(torch.empty_like(q), stream)
    if ws is None:
        ws = _on_stream(workspace(gemma_attn_decode_multi_workspace_size(layer, B, T, max_seq_len), q.device),
                        stream)
    st = _lib.load().gemma_attn_decode_multi(
        ctypes.byref(layer.struct()), B, T, _ptr(q, "q", layer, (B, T, Hq, d)),
        _ptr(q_gain, "q_gain", layer, (d,)), kc, vc, cap,
        _ptr(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,)), int(max_seq_len),
        _ptr(out, "out", layer, (B, T, Hq, d)), _ptr(ws, "workspace", dtype=torch.uint8), ws.numel(),
        _stream(stream))
    _lib.check(st)
    return out


# ---- kernel timing hooks ------------------------------------------------------
KERNEL_IDS = {"prefill_attn": 0, "prefill_prep": 1, "decode_splitk": 2, "decode_merge": 3,
              "kv_append": 4}


def profile_enable(on: bool = True) -> None:
    _lib.load().gemma_attn_profile_enable(1 if on else 0)


def profile_reset() -> None:
    _lib.load().gemma_attn_profile_reset()


def profile_read(kernel: str) -> tuple[float, int]:
    """(total ms, launch count) of one kernel since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int()
    if _lib.load().gemma_attn_profile_read(KERNEL_IDS[kernel], ctypes.byref(ms), ctypes.byref(n)) != 0:
        raise RuntimeError("reading the kernel timing events failed")
    return ms.value, n.value
