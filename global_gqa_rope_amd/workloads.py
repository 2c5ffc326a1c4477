"""Seeded synthetic workloads: shapes and random draws only.

This module holds no attention arithmetic.  Tests, the benchmark and the smoke
check use it to draw the inputs; both the GPU path and the oracle then consume
exactly the same tensors.

Recipe (every tensor has its own generator, so draws do not depend on order):
    generator seed = 1_000_003 * seed + tag   (tag fixed per tensor role)
    float32 draws with torch's Philox/MT generator, then a round-to-nearest-even
    cast to bfloat16 for the bf16 workloads.
Small workloads draw on the CPU and are copied to the device; large ones draw
directly on the device (same recipe, the device generator's stream).

Shapes follow the pages: local layers 2 query heads per KV head with head dim
256 and a window of 1024, global layers 8 query heads per KV head with head dim
512 and a single K=V tensor ("Gemma 4多模态大模型架构详解", sections
"交错层（局部与全局注意力）", "分组查询注意力" and "K=V"); RoPE base 10k locally,
p-RoPE with p = 0.25 and base 1M globally ("Gemma 4 Technical Report" notes,
§2 "Long-context efficiency").  The 32K context is the length of the memory
table of "Gemma 4 技术报告：开源全模态密集 + MoE 模型家族…", section
"显存占用（32k 上下文，文本 only，int8 KV cache）"; 256K is the 31B context of
the "Gemma 4 架構與多模態拆解" talk notes, chapter "31B Dense".
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import torch

TAGS = {"q": 1, "k": 2, "v": 3, "g_q": 4, "g_k": 5, "lens": 6, "k_cache": 7,
        "v_cache": 8, "k_new": 9, "v_new": 10, "q_dec": 11, "q8_codes": 12, "q8_scales": 13}


@dataclass(frozen=True)
class LayerShape:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int            # 0 = global (full causal)
    kv_shared: bool
    rope_theta: float
    rope_fraction: float
    norm_eps: float = 1e-6


GLOBAL_LAYER = LayerShape(32, 4, 512, 0, True, 1e6, 0.25)
LOCAL_LAYER = LayerShape(32, 16, 256, 1024, False, 1e4, 1.0)
TINY_GLOBAL = LayerShape(8, 1, 512, 0, True, 1e6, 0.25)
# The smaller on-device models' layer types: 512-token windows, and global
# layers with a separate V cache (no K=V).  Head counts are assumptions of the
# same kind as the workloads above (8 query heads, 2 KV heads).
E_LOCAL_LAYER = LayerShape(8, 2, 256, 512, False, 1e4, 1.0)
E_GLOBAL_LAYER = LayerShape(8, 2, 512, 0, False, 1e6, 0.25)
TINY_LOCAL = LayerShape(4, 2, 256, 64, False, 1e4, 1.0)


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * int(seed) + TAGS[tag])
    return g


def normal(shape, seed: int, tag: str, dtype=torch.bfloat16, device="cpu",
           mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    """N(mean, std) float32 draws, rounded (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(seed, tag, device),
                    dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def gains(d: int, seed: int, tag: str, unit: bool, dtype, device="cpu"):
    """QKNorm gain vector: all ones, or N(1, 0.1)."""
    if unit:
        return torch.ones(d, dtype=dtype, device=device)
    return normal((d,), seed, tag, dtype, device, mean=1.0, std=0.1)


def int8_rows(shape, seed: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """A filled int8 K=V cache of rows shape[:-1] x shape[-1] codes: codes
    uniform in [-127, 127] (int8), and one scale per row uniform in
    [0.01, 0.03] (float32; rows of rms near 1 give scales of about 0.025)."""
    codes = torch.randint(-127, 128, tuple(shape), generator=_gen(seed, "q8_codes", device), dtype=torch.int8,
                          device=device)
    scales = torch.rand(tuple(shape[:-1]), generator=_gen(seed, "q8_scales", device), dtype=torch.float32,
                        device=device)
    return codes, scales.mul_(0.02).add_(0.01)


def uniform_lengths(n: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """n integers drawn uniformly from [lo, hi], both ends included (CPU, int32)."""
    g = _gen(seed, "lens", "cpu")
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    layer: LayerShape
    batch: int
    seq_len: int
    dtype: torch.dtype
    unit_gains: bool
    seed: int = 0

    def draw(self, device="cpu"):
        L, B, S = self.layer, self.batch, self.seq_len
        d = L.head_dim
        out = {
            "q": normal((B, S, L.n_q_heads, d), self.seed, "q", self.dtype, device),
            "k": normal((B, S, L.n_kv_heads, d), self.seed, "k", self.dtype, device),
            "v": None if L.kv_shared else
                 normal((B, S, L.n_kv_heads, d), self.seed, "v", self.dtype, device),
            "g_q": gains(d, self.seed, "g_q", self.unit_gains, self.dtype, device),
            "g_k": gains(d, self.seed, "g_k", self.unit_gains, self.dtype, device),
        }
        return out

    def flops(self) -> float:
        """Algorithmic flops: 4*d per (query head, visible key) pair."""
        L, S = self.layer, self.seq_len
        if L.window == 0:
            pairs = S * (S + 1) // 2
        else:
            W = L.window
            pairs = sum(min(i + 1, W) for i in range(min(S, W))) + max(0, S - W) * W
        return 4.0 * self.batch * L.n_q_heads * L.head_dim * pairs


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step per sequence against an existing cache."""

    name: str
    layer: LayerShape
    batch: int
    ctx_lo: int            # cached tokens before the step, drawn from [lo, hi]
    ctx_hi: int
    dtype: torch.dtype
    seed: int = 0

    def lengths(self) -> torch.Tensor:
        """Valid keys per sequence after appending the new token (context + 1)."""
        if self.ctx_lo == self.ctx_hi:
            ctx = torch.full((self.batch,), self.ctx_lo, dtype=torch.int32)
        else:
            ctx = uniform_lengths(self.batch, self.ctx_lo, self.ctx_hi, self.seed)
        return ctx + 1

    def cache_cap(self) -> int:
        if self.layer.window:
            return self.layer.window
        return self.ctx_hi + 1

    def kv_bytes(self, lens) -> int:
        """Algorithmic cache bytes one step reads (each cached element once)."""
        L = self.layer
        elem = torch.tensor([], dtype=self.dtype).element_size()
        per_key = L.n_kv_heads * L.head_dim * elem * (1 if L.kv_shared else 2)
        if L.window:
            return int(sum(min(int(n), L.window) for n in lens)) * per_key
        return int(sum(int(n) for n in lens)) * per_key


CONFIGS = {
    "tiny_global": PrefillWorkload("tiny_global", TINY_GLOBAL, 1, 256, torch.float32, True),
    "tiny_local": PrefillWorkload("tiny_local", TINY_LOCAL, 1, 256, torch.float32, True),
    "global_prefill_32k": PrefillWorkload("global_prefill_32k", GLOBAL_LAYER, 1, 32768,
                                          torch.bfloat16, False),
    "local_prefill_32k": PrefillWorkload("local_prefill_32k", LOCAL_LAYER, 4, 32768,
                                         torch.bfloat16, False),
    "global_decode": DecodeWorkload("global_decode", GLOBAL_LAYER, 16, 4096, 131072,
                                    torch.bfloat16),
    "stack_decode_local": DecodeWorkload("stack_decode_local", LOCAL_LAYER, 32, 65536,
                                         65536, torch.bfloat16),
    "stack_decode_global": DecodeWorkload("stack_decode_global", GLOBAL_LAYER, 32, 65536,
                                          65536, torch.bfloat16),
    # the longest context the pages give (256K): every sequence at 262144 keys
    "long_decode": DecodeWorkload("long_decode", GLOBAL_LAYER, 4, 262143, 262143, torch.bfloat16),
    # a 4:1 stack of the smaller models' layer types (512-token windows, a
    # global layer with a separate V cache)
    "e_stack_local": DecodeWorkload("e_stack_local", E_LOCAL_LAYER, 32, 65536, 65536, torch.bfloat16),
    "e_stack_global": DecodeWorkload("e_stack_global", E_GLOBAL_LAYER, 32, 65536, 65536, torch.bfloat16),
}

TINY_DECODE_STEPS = 16


def with_seq(w: PrefillWorkload, seq_len: int, batch: int | None = None, **kw):
    """The same workload at another length (parity cases at oracle-sized shapes)."""
    return replace(w, seq_len=seq_len, batch=w.batch if batch is None else batch, **kw)
