"""Plain float64 definitions of the attention block (test infrastructure only).

Conventions where the pages leave a step open (each one is listed with its
reason in the design notes of this repository):

* rotary pairs are adjacent dims (2i, 2i+1); "the first p of the pairs" is then
  the first p*d dims;
* pair i rotates by the angle pos * theta**(-2i/d) (the ladder of the full head
  dim, truncated to the first p*d/2 pairs: the low frequencies are the ones
  dropped), counter-clockwise;
* pairs past the rotated fraction are left exactly as they are (angle 0);
* positions are 0-based; QKNorm is x / sqrt(mean(x^2) + eps) * gain;
* query head h reads KV head h // G (contiguous groups);
* a window of W keeps keys j with i - W < j <= i (W keys including the query);
* global (K=V) layers use the normalised, unrotated key as the value; local
  layers use the raw v;
* caches: global layers keep one tensor holding the normalised, unrotated key of
  every position (slot = position); local layers keep a ring of W slots
  (slot = position mod W) holding the normalised and rotated key and the raw v.
"""

from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np


@dataclass(frozen=True)
class OracleLayer:
    """Shape and constants of one attention layer, oracle side."""

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int            # 0 = full causal (global layer); W > 0 = sliding window
    kv_shared: bool        # True = keys reused as values (global layers)
    rope_theta: float
    rope_fraction: float   # p: 1.0 on local layers, 0.25 on global layers
    norm_eps: float = 1e-6
    softmax_scale: float | None = None   # None = 1/sqrt(head_dim)

    @property
    def group(self) -> int:
        if self.n_q_heads % self.n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        if self.softmax_scale is None:
            return 1.0 / math.sqrt(self.head_dim)
        return float(self.softmax_scale)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --- QKNorm ------------------------------------------------------------------
# "Gemma 4 Technical Report" notes, §2 Model Architecture: QKNorm alongside
# pre- and post-norm RMSNorm.  RMSNorm of one head vector, then the gain.

def qk_norm(x, gain, eps: float) -> np.ndarray:
    """RMS-normalise the last axis of ``x`` and multiply by ``gain`` (length d)."""
    x = _f64(x)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * _f64(gain)


# --- RoPE and p-RoPE ---------------------------------------------------------
# "Gemma 4多模态大模型架构详解", section "p-RoPE（低频剪枝旋转位置编码）": the
# vector is cut into pairs, each pair is a 2-D vector rotated by an angle that
# shrinks from the first pair to the last; with p = 0.25 only the first quarter
# of the pairs carry position and the rest are left alone.  Base 1M on global
# layers, 10k on local layers ("Gemma 4 Technical Report" notes, §2).

def rotated_pairs(head_dim: int, fraction: float) -> int:
    """Number of rotated pairs, p * d / 2; it must be a whole number."""
    n = fraction * head_dim / 2.0
    if n < 0 or abs(n - round(n)) > 1e-9 or head_dim % 2:
        raise ValueError(f"p*d/2 = {n} is not a whole number of pairs")
    return int(round(n))


def rope_frequencies(head_dim: int, theta: float, fraction: float) -> np.ndarray:
    """Angular frequency of each rotated pair i: theta ** (-2 i / d)."""
    i = np.arange(rotated_pairs(head_dim, fraction), dtype=np.float64)
    return float(theta) ** (-2.0 * i / head_dim)


def rotate(x, positions, theta: float, fraction: float) -> np.ndarray:
    """Rotate pairs (2i, 2i+1), i < p*d/2, of ``x[..., d]`` by positions * omega_i.

    ``positions`` broadcasts against ``x.shape[:-1]``.  Dims from 2*(p*d/2) on
    are copied unchanged.
    """
    x = _f64(x)
    d = x.shape[-1]
    omega = rope_frequencies(d, theta, fraction)
    n = omega.size
    angle = _f64(positions)[..., None] * omega          # [..., n]
    c, s = np.cos(angle), np.sin(angle)
    y = x.copy()
    even = x[..., 0:2 * n:2]
    odd = x[..., 1:2 * n:2]
    y[..., 0:2 * n:2] = even * c - odd * s
    y[..., 1:2 * n:2] = even * s + odd * c
    return y


# --- Softmax attention -------------------------------------------------------
# Causal attention: every token attends to all earlier tokens (global) or to
# the last W tokens only (local).  "Gemma 4多模态大模型架构详解", section
# "交错层（局部与全局注意力）".

def masked_softmax_attention(q_rot, q_pos, k_rot, values, k_pos, scale: float,
                             window: int) -> np.ndarray:
    """One head: rows of q_rot [Sq, d] at q_pos against keys k_rot [Sk, d] at k_pos.

    Key j is visible to query i when k_pos[j] <= q_pos[i] and, for window > 0,
    k_pos[j] > q_pos[i] - window.  Softmax over the visible keys.
    """
    q_rot, k_rot, values = _f64(q_rot), _f64(k_rot), _f64(values)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    scores = scale * (q_rot @ k_rot.T)
    visible = k_pos[None, :] <= q_pos[:, None]
    if window > 0:
        visible &= k_pos[None, :] > q_pos[:, None] - window
    if not visible.any(axis=1).all():
        raise ValueError("a query row has no visible key")
    scores = np.where(visible, scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    weights = np.exp(scores)
    weights /= weights.sum(axis=1, keepdims=True)
    return weights @ values


# --- The layer ---------------------------------------------------------------

def _check_shapes(layer: OracleLayer, q, k, v):
    B, S, Hkv, d = k.shape
    Hq = q.shape[2]
    if Hq != layer.n_q_heads or d != layer.head_dim or q.shape[0] != B or q.shape[3] != d:
        raise ValueError("q shape does not match the layer")
    if Hkv != layer.n_kv_heads:
        raise ValueError("k shape does not match the layer")
    if layer.kv_shared:
        if v is not None:
            raise ValueError("K=V layer takes no separate v")
    elif v is None or v.shape != k.shape:
        raise ValueError("local layer needs v shaped like k")
    return B, S, Hq, d


def prefill(layer: OracleLayer, q, k, v, g_q, g_k, rows=None,
            row_block: int = 512, q_at_rows: bool = False) -> np.ndarray:
    """Attention output for a whole prompt.

    q [B,S,Hq,d], k [B,S,Hkv,d] and v [B,S,Hkv,d] (None for K=V) are the raw
    post-projection tensors.  Returns out [B, len(rows), Hq, d] for the query
    positions ``rows`` (all positions by default).  With ``q_at_rows`` the
    caller passes q only at those rows, q [B, len(rows), Hq, d].  Rows are
    evaluated ``row_block`` at a time; each row is its own softmax, so this is
    the definition evaluated row by row.
    """
    B, S, Hq, d = _check_shapes(layer, q, k, v)
    G = layer.group
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    if q_at_rows and q.shape[1] != rows.size:
        raise ValueError("q_at_rows: q must hold exactly the requested rows")
    if not q_at_rows and q.shape[1] != S:
        raise ValueError("q and k must have the same length")
    positions = np.arange(S)

    k_hat = qk_norm(k, g_k, layer.norm_eps)                          # [B,S,Hkv,d]
    k_rot = rotate(k_hat, positions[None, :, None], layer.rope_theta,
                   layer.rope_fraction)
    values = k_hat if layer.kv_shared else _f64(v)

    out = np.empty((B, rows.size, Hq, d), dtype=np.float64)
    for start in range(0, rows.size, row_block):
        r = rows[start:start + row_block]
        q_r = q[:, start:start + row_block] if q_at_rows else q[:, r]
        q_hat = qk_norm(q_r, g_q, layer.norm_eps)                   # [B,r,Hq,d]
        q_rot = rotate(q_hat, r[None, :, None], layer.rope_theta,
                       layer.rope_fraction)
        lo = 0 if layer.window == 0 else max(0, int(r.min()) - layer.window + 1)
        hi = int(r.max()) + 1
        kp = positions[lo:hi]
        for b in range(B):
            for h in range(Hq):
                c = h // G
                out[b, start:start + r.size, h] = masked_softmax_attention(
                    q_rot[b, :, h], r, k_rot[b, lo:hi, c], values[b, lo:hi, c],
                    kp, layer.scale, layer.window)
    return out


# --- Caches ------------------------------------------------------------------
# Global layers: one tensor serves as keys and values, stored normalised and
# unrotated; p-RoPE is applied when the scores are formed.  Local layers: a
# ring of cache_cap >= W slots (slot = position mod cache_cap) for the
# normalised, rotated key and the raw value.  W slots hold every key the
# newest token sees; checking T new tokens at once needs W + T - 1, since the
# earliest of them still sees T - 1 positions the later ones pushed out of a
# W-slot ring.

def expected_caches_after_prefill(layer: OracleLayer, k, v, g_k, cache_cap: int):
    """Cache contents [B,Hkv,cap,d] after a prompt of S tokens (unwritten = nan)."""
    k = _f64(k)
    B, S, Hkv, d = k.shape
    k_hat = qk_norm(k, g_k, layer.norm_eps)
    kc = np.full((B, Hkv, cache_cap, d), np.nan)
    if layer.kv_shared:
        if S > cache_cap:
            raise ValueError("prompt longer than the cache")
        kc[:, :, :S] = k_hat.transpose(0, 2, 1, 3)
        return kc, None
    # Separate V: keys stored rotated.  Windowed layers keep a ring of
    # cache_cap >= W slots (slot = position mod cache_cap); global ones every
    # position (slot = position), as the E2B/E4B global layers without K=V need.
    if layer.window > 0 and cache_cap < layer.window:
        raise ValueError("a local cache has at least W slots")
    if layer.window == 0 and S > cache_cap:
        raise ValueError("prompt longer than the cache")
    positions = np.arange(S)
    k_rot = rotate(k_hat, positions[None, :, None], layer.rope_theta,
                   layer.rope_fraction)
    vc = np.full_like(kc, np.nan)
    for p in range(max(0, S - cache_cap), S):
        kc[:, :, p % cache_cap] = k_rot[:, p]
        vc[:, :, p % cache_cap] = _f64(v)[:, p]
    return kc, vc


def expected_caches_after_append(layer: OracleLayer, k_cache, v_cache, k_new,
                                 v_new, g_k, positions):
    """Write one new token per sequence (k_new [B,Hkv,d]) at ``positions[b]``."""
    kc = _f64(k_cache).copy()
    vc = None if v_cache is None else _f64(v_cache).copy()
    k_hat = qk_norm(k_new, g_k, layer.norm_eps)                      # [B,Hkv,d]
    cap = kc.shape[2]
    for b, p in enumerate(np.asarray(positions, dtype=np.int64)):
        if layer.kv_shared:
            kc[b, :, p] = k_hat[b]
        else:
            kc[b, :, p % cap] = rotate(k_hat[b], p, layer.rope_theta,
                                       layer.rope_fraction)
            vc[b, :, p % cap] = _f64(v_new)[b]
    return kc, vc


def ring_positions(seq_len: int, cache_cap: int) -> np.ndarray:
    """Positions held by the min(L, cap) filled slots of a ring after L tokens:
    slot s holds the latest position congruent to s mod cap."""
    L = int(seq_len)
    return np.array([L - 1 - ((L - 1 - s) % cache_cap) for s in range(min(L, cache_cap))], dtype=np.int64)


def decode_from_cache(layer: OracleLayer, q, g_q, k_cache, v_cache, seq_lens,
                      batches=None) -> np.ndarray:
    """One decode step per sequence: q [B,Hq,d] raw, query position L_b - 1.

    ``seq_lens[b]`` counts the valid keys including the new token.  Global
    layers read slots 0..L_b-1 (slot j = position j): K=V caches are rotated on
    the fly, separate-V caches hold rotated keys.  Local layers read the
    min(L_b, cap) filled ring slots, whose keys are stored already rotated, and
    see those inside the window.  Returns out [len(batches), Hq, d].
    """
    G = layer.group
    batches = range(q.shape[0]) if batches is None else batches
    out = []
    for b in batches:
        L = int(seq_lens[b])
        qpos = np.array([L - 1])
        q_hat = qk_norm(q[b], g_q, layer.norm_eps)                  # [Hq,d]
        q_rot = rotate(q_hat, L - 1, layer.rope_theta, layer.rope_fraction)
        rows = np.empty((layer.n_q_heads, layer.head_dim))
        if layer.kv_shared:
            kpos = np.arange(L)
            for c in range(layer.n_kv_heads):
                keys = _f64(k_cache[b, c, :L])
                k_rot = rotate(keys, kpos, layer.rope_theta, layer.rope_fraction)
                for h in range(c * G, (c + 1) * G):
                    rows[h] = masked_softmax_attention(q_rot[h:h + 1], qpos, k_rot,
                                                       keys, kpos, layer.scale, 0)[0]
        elif layer.window == 0:
            # global layer with a separate V: slot = position, keys stored rotated
            kpos = np.arange(L)
            for h in range(layer.n_q_heads):
                rows[h] = masked_softmax_attention(
                    q_rot[h:h + 1], qpos, k_cache[b, h // G, :L], v_cache[b, h // G, :L], kpos, layer.scale, 0)[0]
        else:
            kpos = ring_positions(L, k_cache.shape[2])
            n = kpos.size
            for h in range(layer.n_q_heads):
                rows[h] = masked_softmax_attention(
                    q_rot[h:h + 1], qpos, k_cache[b, h // G, :n],
                    v_cache[b, h // G, :n], kpos, layer.scale, layer.window)[0]
        out.append(rows)
    return np.stack(out)


def decode_multi_from_cache(layer: OracleLayer, q, g_q, k_cache, v_cache, seq_lens,
                            batches=None) -> np.ndarray:
    """Several new tokens per sequence against the cache, each causally.

    q [B,T,Hq,d] raw; token j of sequence b sits at position L_b - T + j, where
    ``seq_lens[b]`` = L_b counts the valid keys including all T new tokens, and
    attends to the cached keys at positions up to its own (and, on windowed
    layers, above its own minus W).  Global layers: slot = position; a K=V
    cache's unrotated keys are rotated on the fly and used unrotated as values,
    a separate-V cache holds rotated keys.  Windowed layers: a ring of cap
    slots holding rotated keys, which must still hold every key the earliest
    token sees (cap >= W + T - 1 once the ring has wrapped).  This is the check
    of tokens proposed by the MTP drafter ("Gemma 4 Technical Report" notes,
    section 2.6): each is attention at its own position, the definition of
    ``prefill`` row by row.  Returns out [len(batches), T, Hq, d].
    """
    G, T = layer.group, q.shape[1]
    batches = range(q.shape[0]) if batches is None else batches
    out = []
    for b in batches:
        L = int(seq_lens[b])
        if L < T:
            raise ValueError("fewer keys than new tokens")
        qpos = L - T + np.arange(T)
        q_hat = qk_norm(q[b], g_q, layer.norm_eps)                             # [T,Hq,d]
        q_rot = rotate(q_hat, qpos[:, None], layer.rope_theta, layer.rope_fraction)
        if layer.window:
            kpos = ring_positions(L, k_cache.shape[2])
            if kpos.min() > max(0, int(qpos[0]) - layer.window + 1):
                raise ValueError("the ring no longer holds keys the earliest new token sees")
        else:
            kpos = np.arange(L)
        n = kpos.size
        rows = np.empty((T, layer.n_q_heads, layer.head_dim))
        for c in range(layer.n_kv_heads):
            stored = _f64(k_cache[b, c, :n])
            if layer.kv_shared:
                keys, vals = rotate(stored, kpos, layer.rope_theta, layer.rope_fraction), stored
            else:
                keys, vals = stored, _f64(v_cache[b, c, :n])
            for h in range(c * G, (c + 1) * G):
                rows[:, h] = masked_softmax_attention(q_rot[:, h], qpos, keys, vals, kpos, layer.scale,
                                                      layer.window)
        out.append(rows)
    return np.stack(out)


# --- int8 K=V cache ------------------------------------------------------------
# The pages' 32K memory table counts the KV cache in int8 (table "显存占用（32k
# 上下文，文本 only，int8 KV cache）" of "Gemma 4 技术报告：开源全模态密集 + MoE 模型家族，
# 长上下文与端侧高效是本代核心").  They do not say how values map to int8; the
# reading taken here is symmetric scaling per cached row (one position of one
# KV head): codes c_i = round-half-even(x_i / s) with s = max_i |x_i| / 127,
# standing for c_i * s.  The code is an integer decided by floating point, so
# it is computed in float32, the precision the kernels use.

def quantize_rows(x):
    """int8 codes [..., d] and float32 scales [...] of rows x[..., d]."""
    x32 = np.asarray(x, dtype=np.float32)
    s = np.max(np.abs(x32), axis=-1) / np.float32(127.0)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    c = np.rint(x32 / safe[..., None])
    c = np.where(s[..., None] > 0, np.clip(c, -127, 127), 0.0)
    return c.astype(np.int8), s.astype(np.float32)


def dequantize_rows(codes, scales) -> np.ndarray:
    """The rows int8 codes and their scales stand for: c_i * s."""
    return np.asarray(codes, dtype=np.float64) * _f64(scales)[..., None]


# --- Pre-rotated ("1.25 d") global cache ---------------------------------------
# The layout behind the pages' 37.5% figure (reading R12): per token, the
# rotated leading 2 n_rot dims of the normalised key, plus the normalised,
# unrotated d-dim row, which is the value and also supplies the key's remaining
# dims.  It stores (1 + p) d values per token instead of the K=V tensor's d, and
# needs no rotation when scores are formed.

def prerotated_heads(layer: OracleLayer, rows, positions) -> np.ndarray:
    """The cached heads of normalised, unrotated rows [..., P, d] at positions [P]:
    their leading 2 n_rot dims rotated to their positions."""
    n = 2 * rotated_pairs(layer.head_dim, layer.rope_fraction)
    rotated = rotate(_f64(rows), np.asarray(positions), layer.rope_theta, layer.rope_fraction)
    return rotated[..., :n]


def decode_from_prerotated_cache(layer: OracleLayer, q, g_q, heads, rows, seq_lens,
                                 batches=None) -> np.ndarray:
    """One decode step per sequence against a pre-rotated global cache:
    heads [B,Hkv,cap,2 n_rot] (rotated), rows [B,Hkv,cap,d] (unrotated).

    Key j of KV head c is [heads[b,c,j], rows[b,c,j,2 n_rot:]], already at its
    position; its value is rows[b,c,j].  q [B,Hq,d] raw at position L_b - 1.
    Returns out [len(batches), Hq, d]."""
    if not layer.kv_shared or layer.window:
        raise ValueError("the pre-rotated cache is a global K=V layer layout")
    G = layer.group
    n = 2 * rotated_pairs(layer.head_dim, layer.rope_fraction)
    batches = range(q.shape[0]) if batches is None else batches
    out = []
    for b in batches:
        L = int(seq_lens[b])
        qpos = np.array([L - 1])
        q_rot = rotate(qk_norm(q[b], g_q, layer.norm_eps), L - 1, layer.rope_theta, layer.rope_fraction)
        kpos = np.arange(L)
        res = np.empty((layer.n_q_heads, layer.head_dim))
        for c in range(layer.n_kv_heads):
            vals = _f64(rows[b, c, :L])
            keys = np.concatenate([_f64(heads[b, c, :L]), vals[:, n:]], axis=-1)
            for h in range(c * G, (c + 1) * G):
                res[h] = masked_softmax_attention(q_rot[h:h + 1], qpos, keys, vals, kpos, layer.scale, 0)[0]
        out.append(res)
    return np.stack(out)


def cache_bytes_per_token(head_dim: int, fraction: float, layout: str,
                          bytes_per_elem: float = 1.0) -> float:
    """Bytes one KV head caches per token under three global-layer layouts.

    ``separate``: K and V, 2d.  ``prerotated``: the rotated p*d dims of K plus the
    unrotated d dims used as V, (1+p)*d.  ``shared``: one unrotated K=V tensor, d
    (p-RoPE applied when the scores are formed).
    """
    if layout == "separate":
        n = 2 * head_dim
    elif layout == "prerotated":
        n = head_dim + 2 * rotated_pairs(head_dim, fraction)
    elif layout == "shared":
        n = head_dim
    else:
        raise ValueError(layout)
    return n * bytes_per_elem
