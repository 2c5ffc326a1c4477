"""GPU parity of the prefill attention on both of its softmax paths.

The prefill kernel skips the running row max for a wave whose scores are
bounded by |q~| max|k~| <= 40 (log2 units, q~ including the softmax scale,
the maximum over the key tiles the workgroup reads).  QKNorm keeps both
lengths near sqrt(d) times the gains' rms, so at the default 1/sqrt(d) scale
every wave of the seeded workloads takes that path (the other parity tests).
Here the gains are shaped so that some rows' bounds are far larger while their
scores stay ordinary: queries get a large gain on dims 2-3 where every key is
zero (key gain 0), keys get a large gain on dims 0-1 where every query is zero
(query gain 0); other rows hold zeros in the dims of the large gains.  Rotation keeps each pair within its two dims, so those parts
never meet in a score.  A few query rows (one wave's positions) put their
energy in dims 2-3, and one key row in dims 0-1: that wave, and every
workgroup whose tiles reach that key, take the online max, next to waves of
the same workgroup and other workgroups that do not.  Every output element is
compared with the float64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd import workloads as W
from tests.gpu_helpers import assert_close, device, oracle_layer, to64

pytestmark = pytest.mark.gpu

BOUND = 40.0
LOG2E = 1.4426950408889634


def _normed_lengths(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """|x / rms(x) * g| along the last axis (the rotation keeps lengths)."""
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return np.linalg.norm(x / rms * g, axis=-1)


def _shaped_inputs(shape, B, S, q_rows, k_row, seed=23):
    x = W.PrefillWorkload("bound", shape, B, S, torch.bfloat16, False, seed).draw("cpu")
    g_q, g_k = x["g_q"].clone(), x["g_k"].clone()
    g_q[0:2] = 0.0
    g_q[2:4] = 8.0
    g_k[0:2] = 8.0
    g_k[2:4] = 0.0
    # values below 2 in magnitude: at |o| near 4 the bf16 roundings of q, k,
    # v, P and the output alone reach 2e-2 on some rows (the arithmetic itself,
    # on either softmax path); this test is about the paths
    if shape.kv_shared:
        g_k[4:] *= 0.45
    else:
        x["v"] = x["v"] * 0.5
    q, k = x["q"].clone(), x["k"].clone()
    q[..., 2:4] = 0.0                              # other rows stay clear of the large gains
    k[..., 0:2] = 0.0
    q[0, q_rows, :, :] = 0.0
    q[0, q_rows, :, 2:4] = 1.0                     # all of these rows' length in dims 2-3
    k[0, k_row, 0, :] = 0.0
    k[0, k_row, 0, 0:2] = 1.0                      # one key row of head 0 in dims 0-1
    x.update(q=q, k=k, g_q=g_q, g_k=g_k)
    return x


# (layer, S, query rows of one wave, the long key row)
#  local, window 100: workgroups of 128 positions, waves of 32 positions (wave 2
#    of workgroup 0 = positions 64..95); key 200 lies in the tiles of workgroups
#    1 and 2 of head 0
#  global: workgroups of 16 positions, waves of 4 (wave 2 of workgroup 2 =
#    positions 40..43); key 200 is read by every workgroup from position 200 on
CASES = [
    ("local", W.replace(W.LOCAL_LAYER, window=100), 300, list(range(64, 96)), 200),
    ("global", W.GLOBAL_LAYER, 300, list(range(40, 44)), 200),
]


@pytest.mark.parametrize("kind,shape,S,q_rows,k_row", CASES, ids=[c[0] for c in CASES])
def test_prefill_on_both_softmax_paths(kind, shape, S, q_rows, k_row):
    B = 2
    x = _shaped_inputs(shape, B, S, q_rows, k_row)
    scale = shape.head_dim ** -0.5 * LOG2E
    qn = _normed_lengths(to64(x["q"]), to64(x["g_q"]), shape.norm_eps) * scale       # [B,S,Hq]
    kn = _normed_lengths(to64(x["k"]), to64(x["g_k"]), shape.norm_eps)               # [B,S,Hkv]
    ordinary = np.ones(S, bool)
    ordinary[q_rows] = False
    kn_plain = kn.copy()
    kn_plain[0, k_row, 0] = 0.0
    print(f"[bound] {kind}: ordinary rows {qn[:, ordinary].max() * kn_plain.max():.1f}, "
          f"shaped query rows {qn[0, q_rows].min() * kn_plain.max():.1f}, "
          f"with the long key {qn[:, ordinary].min() * kn[0, k_row, 0]:.1f}", flush=True)
    assert qn[:, ordinary].max() * kn_plain.max() < 0.9 * BOUND
    assert qn[0, q_rows].min() * kn_plain.max() > 1.5 * BOUND
    assert qn[:, ordinary].min() * kn[0, k_row, 0] > 1.5 * BOUND

    dev = device()
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    cap = shape.window if shape.window else S
    kc = torch.zeros((B, shape.n_kv_heads, cap, shape.head_dim), dtype=torch.bfloat16, device=dev)
    vc = None if shape.kv_shared else torch.zeros_like(kc)
    xd = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    out = torch.full_like(xd["q"], float("nan"))
    api.gemma_attn_prefill(lay, xd["q"], xd["k"], xd["v"], xd["g_q"], xd["g_k"], kc, vc, out)
    torch.cuda.synchronize()
    ref = O.prefill(oracle_layer(shape), to64(x["q"]), to64(x["k"]),
                    None if x["v"] is None else to64(x["v"]), to64(x["g_q"]), to64(x["g_k"]))
    err = np.abs(to64(out) - ref)
    worst = np.unravel_index(int(err.argmax()), err.shape)
    print(f"[parity] {kind}: largest error at (b, row, head, dim) {tuple(int(i) for i in worst)}: "
          f"got {float(to64(out)[worst]):.5f}, want {ref[worst]:.5f}", flush=True)
    assert_close(out, ref, torch.bfloat16, f"{kind} prefill, shaped gains")


def test_chunk_bound_counts_the_cached_prefix_keys():
    """A later chunk's bound takes the key lengths of the cached prefix rows it
    reads, not only its own.  One prefix key (position 150) puts all its
    length in dims 200-201 (unrotated at p = 0.25) and was cached with a key
    gain of 6 there, so its normalised length is ~136 against ~23 for every
    other key.  Four chunk queries put all their length in the same two dims
    (ordinary query gains, length ~1.45 after the scale): their score with
    that key is ~197 (log2 units), and 2^197 overflows fp32, so those rows come
    out finite only if the bound counts the cached key (with the chunk's own
    keys it is ~33, under the 40 of the fixed path).  Every other query and
    key holds zeros in dims 200-201, so no other score changes.  Global layer
    with a separate V cache; the oracle is the multi-token decode over the
    expected cache (prefix rows with the prefix's gains, chunk rows with the
    chunk's)."""
    shape = W.E_GLOBAL_LAYER
    B, S, start, src = 1, 500, 300, 150
    dev = device()
    x = W.PrefillWorkload("bound_chunk", shape, B, S, torch.bfloat16, False, seed=41).draw("cpu")
    g_big = x["g_k"].clone()
    g_big[200:202] = 6.0
    q, k = x["q"].clone(), x["k"].clone()
    q[..., 200:202] = 0.0
    k[..., 200:202] = 0.0
    k[0, src, :, :] = 0.0
    k[0, src, :, 200:202] = 1.0
    aligned = [start + 7, start + 40, start + 150, start + 199]
    for row in aligned:
        q[0, row, :, :] = 0.0
        q[0, row, :, 200:202] = 1.0
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    kc = torch.zeros((B, shape.n_kv_heads, S, shape.head_dim), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    qd, kd, vd = q.to(dev), k.to(dev), x["v"].to(dev)
    gq, gk, gbd = x["g_q"].to(dev), x["g_k"].to(dev), g_big.to(dev)
    api.gemma_attn_prefill_chunk(lay, 0, qd[:, :start], kd[:, :start], gq, gbd, kc, v=vd[:, :start], v_cache=vc)
    out = api.gemma_attn_prefill_chunk(lay, start, qd[:, start:], kd[:, start:], gq, gk, kc, v=vd[:, start:],
                                       v_cache=vc)
    torch.cuda.synchronize()

    ol = oracle_layer(shape)
    k64, v64 = to64(k), to64(x["v"])
    kc_pre, _ = O.expected_caches_after_prefill(ol, k64[:, :start], v64[:, :start], to64(g_big), S)
    kc_ref, vc_ref = O.expected_caches_after_prefill(ol, k64, v64, to64(x["g_k"]), S)
    kc_ref[:, :, :start] = kc_pre[:, :, :start]
    ref = O.decode_multi_from_cache(ol, to64(q[:, start:]), to64(x["g_q"]), kc_ref, vc_ref, np.array([S]))
    scale = shape.head_dim ** -0.5 * LOG2E
    qn = _normed_lengths(to64(q[0, start:]), to64(x["g_q"]), shape.norm_eps) * scale
    kn_pre = _normed_lengths(k64[0, :start], to64(g_big), shape.norm_eps)
    kn_own = _normed_lengths(k64[0, start:], to64(x["g_k"]), shape.norm_eps)
    print(f"[bound] chunk: with the cached key {qn.max() * kn_pre.max():.1f}, "
          f"with the chunk's own keys {qn.max() * kn_own.max():.1f}", flush=True)
    assert qn.max() * kn_own.max() < 0.9 * BOUND and qn.max() * kn_pre.max() > 128
    assert torch.isfinite(out).all(), "non-finite outputs: a bound without the cached rows"
    assert_close(out, ref, torch.bfloat16, "global separate-V chunk against a long cached key")
