"""Pins for the float64 oracle (CPU only).

Each test ties an oracle function to something other than itself: a value the
pages print, a closed form, an invariant, a library routine in a special case,
or a scalar brute force on tiny inputs written separately below.  Together they
are chosen so that a plausible slip in the oracle (a dropped eps or gain, a sign
or index error in the rotation, the wrong GQA head, an off-by-one window, the
rotated key used as value, a transposed product) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(1234)


def layer(hq=4, hkv=2, d=8, window=0, kv_shared=False, theta=1e4, p=1.0,
          eps=1e-6, scale=None):
    return O.OracleLayer(hq, hkv, d, window, kv_shared, theta, p, eps, scale)


# ---------------------------------------------------------------- QKNorm ----

def test_qknorm_hand_values():
    # x = (3, 4): mean square 12.5, rms = 3.5355339059327378
    y = O.qk_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(y, [0.848528137423857, 1.131370849898476], atol=1e-15)
    # gains multiply after normalisation, dim by dim
    y = O.qk_norm(np.array([3.0, 4.0]), np.array([2.0, 0.5]), 0.0)
    assert np.allclose(y, [1.697056274847714, 0.565685424949238], atol=1e-15)


def test_qknorm_mean_square_closed_form():
    x = RNG.normal(size=(5, 3, 64)) * 3.0
    eps = 1e-2
    y = O.qk_norm(x, np.ones(64), eps)
    m = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), m / (m + eps), rtol=1e-13)


def test_qknorm_scale_invariance():
    x = RNG.normal(size=(7, 32))
    g = RNG.normal(1.0, 0.1, size=32)
    assert np.allclose(O.qk_norm(x, g, 0.0), O.qk_norm(5.5 * x, g, 0.0), rtol=1e-13)


# ------------------------------------------------------------------ RoPE ----

def test_rope_hand_values():
    # d = 4, base 1e4, full rotation: omega = (1, 1e4**-0.5 = 0.01)
    assert np.allclose(O.rope_frequencies(4, 1e4, 1.0), [1.0, 0.01], rtol=1e-15)
    y = O.rotate(np.array([1.0, 0.0, 1.0, 0.0]), 1, 1e4, 1.0)
    assert np.allclose(y, [0.5403023058681398, 0.8414709848078965,
                           0.9999500004166653, 0.009999833334166664], atol=1e-15)
    # counter-clockwise: (0, 1) turns towards negative first coordinate
    y = O.rotate(np.array([0.0, 1.0, 0.0, 0.0]), 1, 1e4, 1.0)
    assert np.allclose(y[:2], [-0.8414709848078965, 0.5403023058681398], atol=1e-15)


def test_p_rope_frequency_ladder():
    # global layer: d = 512, base 1e6, p = 0.25 -> 64 rotated pairs (128 dims)
    w = O.rope_frequencies(512, 1e6, 0.25)
    assert w.size == 64 and O.rotated_pairs(512, 0.25) == 64
    assert w[0] == 1.0
    assert abs(w[32] - 10 ** -0.75) < 1e-15          # 1e6 ** (-64/512) = 10**-0.75
    assert np.all(np.diff(w) < 0)
    # pruning keeps the high-frequency end of the full ladder
    full = O.rope_frequencies(512, 1e6, 1.0)
    assert np.array_equal(w, full[:64])
    assert w.min() > full[64:].max()
    # local layer: all 128 pairs of d = 256
    assert O.rope_frequencies(256, 1e4, 1.0).size == 128
    with pytest.raises(ValueError):
        O.rotated_pairs(10, 0.25)


def test_rope_position_zero_is_identity_and_norm_preserved():
    x = RNG.normal(size=(6, 512))
    assert np.array_equal(O.rotate(x, np.zeros(6), 1e6, 0.25), x)
    y = O.rotate(x, np.arange(6) * 977, 1e6, 0.25)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # every rotated pair keeps its own length
    pairs_x = np.hypot(x[:, 0:128:2], x[:, 1:128:2])
    pairs_y = np.hypot(y[:, 0:128:2], y[:, 1:128:2])
    assert np.allclose(pairs_x, pairs_y, rtol=1e-13)


def test_p_rope_leaves_unrotated_dims_bit_identical():
    x = RNG.normal(size=(9, 512))
    y = O.rotate(x, np.arange(9) * 12345 + 7, 1e6, 0.25)
    assert np.array_equal(y[:, 128:], x[:, 128:])
    assert not np.allclose(y[:, :128], x[:, :128])
    assert np.array_equal(O.rotate(x, np.arange(9) + 3, 1e6, 0.0), x)


def test_rope_scores_depend_on_relative_position_only():
    q = RNG.normal(size=256)
    k = RNG.normal(size=256)
    for p in (0.25, 1.0):
        s0 = O.rotate(q, 40, 1e4, p) @ O.rotate(k, 13, 1e4, p)
        s1 = O.rotate(q, 40 + 5000, 1e4, p) @ O.rotate(k, 13 + 5000, 1e4, p)
        assert abs(s0 - s1) < 1e-11


def _rotate_half_split(x, pos, theta, p):
    """Other pairing convention: pair i is (i, i + n) inside the first 2n dims."""
    d = x.shape[-1]
    n = int(round(p * d / 2))
    y = x.copy()
    for i in range(n):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        y[i] = x[i] * c - x[i + n] * s
        y[i + n] = x[i] * s + x[i + n] * c
    return y


def test_pairing_conventions_differ_by_a_fixed_permutation():
    d, p, theta, pos = 512, 0.25, 1e6, 3001
    n = int(p * d / 2)
    perm = np.arange(d)                       # adjacent index -> half-split index
    perm[0:2 * n:2] = np.arange(n)
    perm[1:2 * n:2] = np.arange(n) + n
    x = RNG.normal(size=d)
    adj_in = np.empty(d)
    adj_in[:] = x[perm]
    adj_out = O.rotate(adj_in, pos, theta, p)
    half = _rotate_half_split(x, pos, theta, p)
    assert np.allclose(half[perm], adj_out, atol=1e-13)


# -------------------------------------------------------- brute force ----

def _brute_force_layer(lay, q, k, v, g_q, g_k):
    """Scalar loops straight from the definitions, for S, d <= 8."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    n = int(round(lay.rope_fraction * d / 2))
    scale = lay.scale

    def norm(vec, g):
        ms = sum(t * t for t in vec) / d
        r = 1.0 / math.sqrt(ms + lay.norm_eps)
        return [vec[i] * r * g[i] for i in range(d)]

    def rot(vec, pos):
        out = list(vec)
        for i in range(n):
            a = pos * lay.rope_theta ** (-2.0 * i / d)
            out[2 * i] = vec[2 * i] * math.cos(a) - vec[2 * i + 1] * math.sin(a)
            out[2 * i + 1] = vec[2 * i] * math.sin(a) + vec[2 * i + 1] * math.cos(a)
        return out

    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            c = h // G
            for i in range(S):
                qi = rot(norm(list(q[b, i, h]), g_q), i)
                js = [j for j in range(S) if j <= i and (lay.window == 0 or j > i - lay.window)]
                scores = []
                vals = []
                for j in js:
                    kh = norm(list(k[b, j, c]), g_k)
                    kj = rot(kh, j)
                    scores.append(scale * sum(qi[t] * kj[t] for t in range(d)))
                    vals.append(kh if lay.kv_shared else list(v[b, j, c]))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for t in range(d):
                    out[b, i, h, t] = sum(w[u] * vals[u][t] for u in range(len(js))) / tot
    return out


@pytest.mark.parametrize("kv_shared,window,p", [(True, 0, 0.25), (False, 3, 1.0),
                                                (False, 0, 0.5), (True, 2, 1.0)])
def test_prefill_matches_brute_force(kv_shared, window, p):
    lay = layer(hq=4, hkv=2, d=8, window=window, kv_shared=kv_shared, theta=10.0, p=p,
                eps=1e-3)
    B, S = 2, 7
    q = RNG.normal(size=(B, S, 4, 8))
    k = RNG.normal(size=(B, S, 2, 8))
    v = None if kv_shared else RNG.normal(size=(B, S, 2, 8))
    g_q = RNG.normal(1.0, 0.3, size=8)
    g_k = RNG.normal(1.0, 0.3, size=8)
    got = O.prefill(lay, q, k, v, g_q, g_k, row_block=3)
    want = _brute_force_layer(lay, q, k, v, g_q, g_k)
    assert np.allclose(got, want, atol=1e-12)


# ---------------------------------------------------- special cases ----

def test_single_token_returns_its_value():
    lay = layer(d=16, kv_shared=False)
    q = RNG.normal(size=(1, 1, 4, 16))
    k = RNG.normal(size=(1, 1, 2, 16))
    v = RNG.normal(size=(1, 1, 2, 16))
    out = O.prefill(lay, q, k, v, np.ones(16), np.ones(16))
    assert np.allclose(out[0, 0, 0], v[0, 0, 0]) and np.allclose(out[0, 0, 3], v[0, 0, 1])


def test_identical_keys_average_the_values():
    # with p = 0 and one key repeated, every visible key has the same score
    lay = layer(d=16, p=0.0)
    S = 11
    q = RNG.normal(size=(1, S, 4, 16))
    k = np.broadcast_to(RNG.normal(size=(1, 1, 2, 16)), (1, S, 2, 16))
    v = RNG.normal(size=(1, S, 2, 16))
    out = O.prefill(lay, q, k, v, np.ones(16), np.ones(16))
    want = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.allclose(out[:, :, ::2], want, atol=1e-13)


def _sdpa64(qt, kt, vt, scale, mask):
    """torch scaled_dot_product_attention on CPU in float64 ([H,S,d] tensors)."""
    f = torch.nn.functional.scaled_dot_product_attention
    return f(torch.from_numpy(qt), torch.from_numpy(kt), torch.from_numpy(vt),
             attn_mask=torch.from_numpy(mask), scale=scale).numpy()


@pytest.mark.parametrize("window", [0, 5])
def test_no_rotation_matches_torch_sdpa(window):
    d, S = 32, 40
    lay = layer(hq=6, hkv=3, d=d, window=window, p=0.0, eps=1e-6, scale=0.37)
    q = RNG.normal(size=(1, S, 6, d))
    k = RNG.normal(size=(1, S, 3, d))
    v = RNG.normal(size=(1, S, 3, d))
    g = RNG.normal(1, 0.1, size=d)
    out = O.prefill(lay, q, k, v, g, g)
    qh = O.qk_norm(q, g, 1e-6)[0].transpose(1, 0, 2)
    kh = O.qk_norm(k, g, 1e-6)[0].transpose(1, 0, 2)
    kh = np.repeat(kh, 2, axis=0)
    vv = np.repeat(v[0].transpose(1, 0, 2), 2, axis=0)
    i = np.arange(S)
    mask = i[None, :] <= i[:, None]
    if window:
        mask &= i[None, :] > i[:, None] - window
    ref = _sdpa64(np.ascontiguousarray(qh), np.ascontiguousarray(kh),
                  np.ascontiguousarray(vv), 0.37, mask)
    assert np.allclose(out[0].transpose(1, 0, 2), ref, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    d, S, G = 16, 9, 4
    lay = layer(hq=8, hkv=2, d=d, theta=100.0, p=0.5)
    mha = layer(hq=8, hkv=8, d=d, theta=100.0, p=0.5)
    q = RNG.normal(size=(2, S, 8, d))
    k = RNG.normal(size=(2, S, 2, d))
    v = RNG.normal(size=(2, S, 2, d))
    g = np.ones(d)
    a = O.prefill(lay, q, k, v, g, g)
    b = O.prefill(mha, q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), g, g)
    assert np.allclose(a, b, atol=1e-13)


def test_window_special_cases():
    d, S = 8, 12
    q = RNG.normal(size=(1, S, 2, d))
    k = RNG.normal(size=(1, S, 1, d))
    v = RNG.normal(size=(1, S, 1, d))
    g = np.ones(d)
    full = O.prefill(layer(hq=2, hkv=1, d=d, window=0), q, k, v, g, g)
    wide = O.prefill(layer(hq=2, hkv=1, d=d, window=S), q, k, v, g, g)
    assert np.allclose(full, wide, atol=1e-14)
    one = O.prefill(layer(hq=2, hkv=1, d=d, window=1), q, k, v, g, g)
    assert np.allclose(one[0, :, 0], v[0, :, 0]) and np.allclose(one[0, :, 1], v[0, :, 0])


def test_window_of_four_sees_the_last_four_tokens(golden_dir):
    W = json.load(open(os.path.join(golden_dir, "page_constants.json")))["window_example"]["value"]
    # a probe value per key makes the visible set readable from the output
    S, d = 10, 4
    q = np.zeros((1, S, 1, d))
    k = np.zeros((1, S, 1, d))
    v = np.zeros((1, S, 1, d))
    v[0, :, 0, 0] = 2.0 ** np.arange(S)
    out = O.prefill(layer(hq=1, hkv=1, d=d, window=W, p=0.0), q, k, v,
                    np.ones(d), np.ones(d))
    for i in range(S):
        vis = [j for j in range(S) if i - W < j <= i]
        assert len(vis) == min(i + 1, 4)
        assert abs(out[0, i, 0, 0] - sum(2.0 ** j for j in vis) / len(vis)) < 1e-12


def test_keys_as_values_uses_normalised_unrotated_key():
    d, S = 16, 10
    shared = layer(hq=4, hkv=1, d=d, kv_shared=True, theta=1e6, p=0.25)
    sep = layer(hq=4, hkv=1, d=d, kv_shared=False, theta=1e6, p=0.25)
    q = RNG.normal(size=(1, S, 4, d))
    k = RNG.normal(size=(1, S, 1, d))
    g_q = RNG.normal(1, 0.1, size=d)
    g_k = RNG.normal(1, 0.1, size=d)
    a = O.prefill(shared, q, k, None, g_q, g_k)
    b = O.prefill(sep, q, k, O.qk_norm(k, g_k, 1e-6), g_q, g_k)
    assert np.allclose(a, b, atol=1e-14)
    with pytest.raises(ValueError):
        O.prefill(shared, q, k, k, g_q, g_k)


def test_softmax_scale_default_is_inverse_sqrt_head_dim():
    assert layer(d=512).scale == 1 / math.sqrt(512)
    assert layer(d=256, scale=0.5).scale == 0.5


# --------------------------------------------------- decode and caches ----

def test_ring_positions_hand_values():
    # 10 tokens in a 4-slot ring: slots 0..3 hold positions 8, 9, 6, 7
    assert O.ring_positions(10, 4).tolist() == [8, 9, 6, 7]
    assert O.ring_positions(3, 4).tolist() == [0, 1, 2]
    assert O.ring_positions(8, 4).tolist() == [4, 5, 6, 7]


@pytest.mark.parametrize("kind", ["global", "global_separate_v", "local", "local_wide_ring"])
def test_decode_from_cache_equals_prefill_row(kind):
    d = 32
    if kind == "global":
        lay = layer(hq=8, hkv=1, d=d, kv_shared=True, theta=1e6, p=0.25)
    elif kind == "global_separate_v":         # E2B/E4B global layers: no K=V
        lay = layer(hq=8, hkv=2, d=d, kv_shared=False, theta=1e6, p=0.25)
    else:
        lay = layer(hq=4, hkv=2, d=d, window=6, theta=1e4, p=1.0)
    B, T = 2, 15                      # T > W exercises the ring wrap
    hkv = lay.n_kv_heads
    q = RNG.normal(size=(B, T, lay.n_q_heads, d))
    k = RNG.normal(size=(B, T, hkv, d))
    v = None if lay.kv_shared else RNG.normal(size=(B, T, hkv, d))
    g_q = RNG.normal(1, 0.1, size=d)
    g_k = RNG.normal(1, 0.1, size=d)
    full = O.prefill(lay, q, k, v, g_q, g_k)
    # a ring wider than the window keeps older keys, which the window must mask
    cap = (lay.window + 3 if kind == "local_wide_ring" else lay.window) if lay.window else T
    kc, vc = O.expected_caches_after_prefill(lay, k[:, :T - 4],
                                             None if v is None else v[:, :T - 4], g_k, cap)
    for t in range(T - 4, T):
        kc, vc = O.expected_caches_after_append(lay, kc, vc, k[:, t],
                                                None if v is None else v[:, t], g_k,
                                                np.full(B, t))
        got = O.decode_from_cache(lay, q[:, t], g_q, kc, vc, np.full(B, t + 1))
        assert np.allclose(got, full[:, t], atol=1e-13)


@pytest.mark.parametrize("kind,group", [("global", 8), ("global", 2), ("global_separate_v", 4), ("local", 2),
                                        ("local", 4)])
def test_multi_token_decode_equals_the_prefill_rows(kind, group):
    """Several new tokens at once: token j is the prefill row at its position,
    over a cache built by a prefill of the older tokens plus appends.  The
    local case uses a ring of W + T - 1 = 8 slots and new tokens at positions
    7, 8, 9, whose slots (7, 0, 1) wrap inside the new tokens."""
    d = 32
    B, S, T = 2, 13, 3
    if kind == "global":
        lay = layer(hq=2 * group, hkv=2, d=d, kv_shared=True, theta=1e6, p=0.25)
    elif kind == "global_separate_v":
        lay = layer(hq=2 * group, hkv=2, d=d, kv_shared=False, theta=1e6, p=0.25)
    else:
        lay = layer(hq=2 * group, hkv=2, d=d, window=6, theta=1e4, p=1.0)
        S = 10
    cap = lay.window + T - 1 if lay.window else S
    q = RNG.normal(size=(B, S, lay.n_q_heads, d))
    k = RNG.normal(size=(B, S, lay.n_kv_heads, d))
    v = None if lay.kv_shared else RNG.normal(size=(B, S, lay.n_kv_heads, d))
    g_q = RNG.normal(1, 0.1, size=d)
    g_k = RNG.normal(1, 0.1, size=d)
    full = O.prefill(lay, q, k, v, g_q, g_k)
    kc, vc = O.expected_caches_after_prefill(lay, k[:, :S - T], None if v is None else v[:, :S - T], g_k, cap)
    for t in range(S - T, S):
        kc, vc = O.expected_caches_after_append(lay, kc, vc, k[:, t], None if v is None else v[:, t], g_k,
                                                np.full(B, t))
    got = O.decode_multi_from_cache(lay, q[:, S - T:], g_q, kc, vc, np.full(B, S))
    assert np.allclose(got, full[:, S - T:], atol=1e-13)
    # one token is the single-token decode
    one = O.decode_multi_from_cache(lay, q[:, S - 1:], g_q, kc, vc, np.full(B, S))
    assert np.allclose(one[:, 0], O.decode_from_cache(lay, q[:, S - 1], g_q, kc, vc, np.full(B, S)), atol=1e-13)


def test_multi_token_decode_masks_the_later_new_tokens():
    """Token 0 of two new tokens must not see the second token's key: changing
    that key leaves token 0's output bit-identical and changes token 1's."""
    d = 8
    lay = layer(hq=2, hkv=1, d=d, kv_shared=True, theta=1e6, p=0.25)
    q = RNG.normal(size=(1, 2, 2, d))
    kc = RNG.normal(size=(1, 1, 6, d))
    g = np.ones(d)
    a = O.decode_multi_from_cache(lay, q, g, kc, None, np.array([6]))
    kc2 = kc.copy()
    kc2[0, 0, 5] += 1.0                               # the key of the second new token (position 5)
    b = O.decode_multi_from_cache(lay, q, g, kc2, None, np.array([6]))
    assert np.array_equal(a[:, 0], b[:, 0]) and not np.allclose(a[:, 1], b[:, 1])
    # a W-slot ring after 6 tokens holds positions 3..5: the first of two new
    # tokens (position 4, window 3) needs position 2, which it no longer holds
    loc = layer(hq=2, hkv=1, d=d, window=3, theta=1e4, p=1.0)
    with pytest.raises(ValueError):
        O.decode_multi_from_cache(loc, q, g, kc[:, :, :3], kc[:, :, :3], np.array([6]))
    O.decode_multi_from_cache(loc, q, g, kc[:, :, :4], kc[:, :, :4], np.array([6]))   # W + 1 slots suffice


def test_int8_rows_hand_values_and_bounds():
    x = np.array([[1.27, -0.635, 0.0, 0.005], [0.0, 0.0, 0.0, 0.0]])
    c, s = O.quantize_rows(x)
    assert s.dtype == np.float32 and c.dtype == np.int8
    assert np.isclose(s[0], 0.01) and s[1] == 0
    assert c[0].tolist() == [127, -64, 0, 0]                 # -63.5 and 0.5 round half to even
    assert (c[1] == 0).all() and (O.dequantize_rows(c, s)[1] == 0).all()
    rows = RNG.normal(size=(64, 512))
    c, s = O.quantize_rows(rows)
    assert (np.abs(c).max(axis=1) == 127).all()              # the largest element maps to +-127
    err = np.abs(O.dequantize_rows(c, s) - rows)
    assert (err <= s[:, None] * (0.5 + 1e-5)).all()          # half a step at most
    # int8 halves the bf16 bytes of a cached row (the scale adds 4 bytes a row)
    assert c[0].nbytes + 4 == 512 + 4 and c[0].nbytes * 2 == 512 * 2


def test_global_cache_holds_one_unrotated_normalised_tensor():
    lay = layer(hq=8, hkv=1, d=16, kv_shared=True, theta=1e6, p=0.25)
    k = RNG.normal(size=(1, 5, 1, 16))
    g = RNG.normal(1, 0.1, size=16)
    kc, vc = O.expected_caches_after_prefill(lay, k, None, g, 8)
    assert vc is None
    assert np.allclose(kc[0, 0, :5], O.qk_norm(k[0, :, 0], g, 1e-6))
    assert np.isnan(kc[0, 0, 5:]).all()


def test_cache_layouts_reproduce_the_pages_global_reduction(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "page_constants.json")))
    p = c["rope_fraction_global"]["value"]
    d = c["head_dim_global"]["value"]
    sep = O.cache_bytes_per_token(d, p, "separate")
    pre = O.cache_bytes_per_token(d, p, "prerotated")
    shared = O.cache_bytes_per_token(d, p, "shared")
    assert 1 - pre / sep == pytest.approx(c["global_kv_reduction"]["value"], abs=1e-12)
    assert 1 - shared / sep == 0.5


def test_cache_layout_is_consistent_with_the_32k_memory_table(golden_dir):
    """31B at 32K with an int8 cache: W-slot local rings plus one K=V tensor.

    The layer count, window and 5:1 ratio come from the pages; the head counts
    (16 KV heads of 256 on local layers, 4 K=V heads of 512 on global layers)
    are the workload's, an assumption.  Only the single-tensor layout lands
    within 2% of the table's figure.
    """
    c = json.load(open(os.path.join(golden_dir, "page_constants.json")))
    mem = json.load(open(os.path.join(golden_dir, "kv_memory_32k.json")))
    n_layers = c["layers_31b"]["value"]
    n_global = n_layers // (c["local_to_global_ratio"]["value"] + 1)
    n_local = n_layers - n_global
    W = c["window_large_models"]["value"]
    ctx = mem["context_tokens"]
    local = n_local * 16 * W * O.cache_bytes_per_token(256, 1.0, "separate")

    def total(layout):
        return (local + n_global * 4 * ctx *
                O.cache_bytes_per_token(512, c["rope_fraction_global"]["value"], layout)) / 1e9

    target = mem["plus_kv_gb"]["31B"]
    assert abs(total("shared") - target) / target < 0.02
    assert abs(total("prerotated") - target) / target > 0.1
    assert abs(total("separate") - target) / target > 0.5


# ----------------------------------------------- pre-rotated ("1.25 d") cache ----

def test_prerotated_heads_hand_values():
    lay = layer(hq=2, hkv=1, d=8, kv_shared=True, theta=1e4, p=0.5)   # 2 rotated pairs: w0 = 1, w1 = 0.1
    x = np.array([[1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0]] * 2)
    h = O.prerotated_heads(lay, x, [0, 2])
    assert h.shape == (2, 4)
    assert np.array_equal(h[0], x[0, :4])                                  # position 0: unrotated
    c0, s0, c1, s1 = np.cos(2.0), np.sin(2.0), np.cos(0.2), np.sin(0.2)
    want = [1 * c0 - 2 * s0, 1 * s0 + 2 * c0, 3 * c1 - 4 * s1, 3 * s1 + 4 * c1]
    assert np.allclose(h[1], want, atol=1e-15)
    # heads plus rows are the (1 + p) d values per token of the "prerotated" layout
    lay512 = layer(hq=8, hkv=1, d=512, kv_shared=True, theta=1e6, p=0.25)
    h512 = O.prerotated_heads(lay512, RNG.normal(size=(3, 512)), [0, 1, 2])
    assert h512.shape[-1] + 512 == O.cache_bytes_per_token(512, 0.25, "prerotated")


def test_prerotated_decode_equals_prefill_rows():
    """Heads built at each slot's position from the K=V rows, read as keys
    [head, row[2 n_rot:]] with the row as value: the prefill row again."""
    d = 32
    lay = layer(hq=8, hkv=2, d=d, kv_shared=True, theta=1e6, p=0.25)
    B, T = 2, 13
    q = RNG.normal(size=(B, T, lay.n_q_heads, d))
    k = RNG.normal(size=(B, T, lay.n_kv_heads, d))
    g_q = RNG.normal(1, 0.1, size=d)
    g_k = RNG.normal(1, 0.1, size=d)
    full = O.prefill(lay, q, k, None, g_q, g_k)
    rows, _ = O.expected_caches_after_prefill(lay, k, None, g_k, T)
    heads = O.prerotated_heads(lay, rows, np.arange(T))
    for t in (0, 5, T - 1):
        got = O.decode_from_prerotated_cache(lay, q[:, t], g_q, heads, rows, np.full(B, t + 1))
        assert np.allclose(got, full[:, t], atol=1e-13)
    # heads that were not rotated give other scores
    wrong = O.decode_from_prerotated_cache(lay, q[:, T - 1], g_q, rows[..., :heads.shape[-1]], rows,
                                           np.full(B, T))
    assert not np.allclose(wrong, full[:, T - 1], atol=1e-6)
