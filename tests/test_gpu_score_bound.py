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
