"""Pins for the oracle's attention: closed forms, special cases and brute force.

Each pin reaches the oracle from a different route than the oracle's own code:
  * RoPE is rebuilt here with complex arithmetic (a vector at position n is the complex
    vector x_k + i x_{k+D/2} times exp(i n omega_k)), not with the oracle's rotation;
  * special cases reduce to a library causal attention (torch SDPA, float64, CPU):
    G = 1 (in-window: exactly the base model; review page, Key idea), w0 >= L (every pair
    local), w0 = 0 (every pair remote, i.e. RoPE at aliased positions f(x));
  * per-pair pure-Python loops score each pair from its *relative* position (i - j for a
    local pair, f(i) - f(j) for a remote one; review page, Method), with no rotation of
    vectors at all;
  * the pages' three-pass inclusion-exclusion merge (review page, Method; gist.science
    summary, Methodologie section 2) must equal the direct definition;
  * decode at length L equals the last row of prefill at length L.
"""
import cmath
import math

import numpy as np
import pytest
import torch

from oracle import (bifocal_attention, bifocal_decode, bifocal_decode_steps, decode_step_from_raw, group_size,
                    raw_bifocal_attention, rope_frequencies, rotate_pairs, three_pass_attention)


# --------------------------------------------------------------------------------------
# Independent RoPE via complex numbers
# --------------------------------------------------------------------------------------
def _freqs(D, theta):
    # Same textbook definition as the oracle, reached through exp/log instead of a power.
    return np.array([math.exp(-(2.0 * k / D) * math.log(theta)) for k in range(D // 2)])


def rope_complex(x, positions, theta):
    """x [B, L, H, D]; positions [L] -> x rotated at those positions, via complex multiply."""
    D = x.shape[-1]
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    ph = np.exp(1j * np.outer(np.asarray(positions, dtype=np.float64), _freqs(D, theta)))
    zr = z * ph[None, :, None, :]
    return np.concatenate([zr.real, zr.imag], axis=-1)


def sdpa_causal(q, k, v):
    """Library causal attention in float64: q [B, L, Hq, D], k/v [B, L, Hkv, D] (GQA expanded)."""
    B, L, Hq, D = q.shape
    rep = Hq // k.shape[2]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, rep, axis=2).transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, rep, axis=2).transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.numpy().transpose(0, 2, 1, 3)


def _rand(seed, B, L, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, L, Hq, D)), rng.standard_normal((B, L, Hkv, D)),
            rng.standard_normal((B, L, Hkv, D)))


# --------------------------------------------------------------------------------------
# Rotation
# --------------------------------------------------------------------------------------
def test_rotation_matches_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 37, 2, 16))
    pos = rng.integers(-50000, 50000, size=37)
    omega = rope_frequencies(16, 1.0e6)
    mine = rotate_pairs(x, (pos[:, None] * omega[None, :])[None, :, None, :])
    np.testing.assert_allclose(mine, rope_complex(x, pos, 1.0e6), rtol=0, atol=1e-12)


def test_rotation_composes_additively_and_preserves_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 32))
    a = rng.uniform(-100, 100, size=(5, 16))
    b = rng.uniform(-100, 100, size=(5, 16))
    np.testing.assert_allclose(rotate_pairs(rotate_pairs(x, a), b), rotate_pairs(x, a + b), atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(rotate_pairs(x, a), axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(rotate_pairs(x, np.zeros((5, 16))), x)  # zero offset is the identity, bit for bit


def test_frequencies_textbook_endpoints():
    w = rope_frequencies(128, 1.0e6)
    assert w[0] == 1.0
    np.testing.assert_allclose(w, _freqs(128, 1.0e6), rtol=1e-14)
    assert np.all(np.diff(w) < 0)


# --------------------------------------------------------------------------------------
# Special cases against a library causal attention
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,wp,w0", [(64, 64, 8), (100, 128, 16), (33, 40, 0)])
def test_in_window_is_plain_causal_attention(L, wp, w0):
    assert group_size(L, wp) == 1
    q, k, v = _rand(2, 1, L, 4, 2, 16)
    o, _ = bifocal_attention(q, k, v, w0=w0, w_pretrained=wp, theta=1e4)
    np.testing.assert_allclose(o, sdpa_causal(q, k, v), rtol=0, atol=1e-12)
    # Bit-identical to the oracle's own all-local run: with G = 1 the correction is exactly 0.
    o_local, _ = bifocal_attention(q, k, v, w0=L + 5, w_pretrained=wp, theta=1e4)
    assert np.array_equal(o, o_local)


@pytest.mark.parametrize("L,wp", [(96, 20), (70, 16)])
def test_all_local_window_is_plain_causal_attention(L, wp):
    assert group_size(L, wp) > 1
    q, k, v = _rand(3, 2, L, 2, 1, 8)
    o, _ = bifocal_attention(q, k, v, w0=L, w_pretrained=wp, theta=1e4)
    np.testing.assert_allclose(o, sdpa_causal(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,wp,D", [(96, 20, 8), (65, 16, 16)])
def test_zero_window_is_rope_attention_at_aliased_positions(L, wp, D):
    G = group_size(L, wp)
    assert G > 1
    qr, kr, v = _rand(4, 1, L, 4, 2, D)
    pos = np.arange(L)
    q = rope_complex(qr, pos, 1e4)
    k = rope_complex(kr, pos, 1e4)
    o, _ = bifocal_attention(q, k, v, w0=0, w_pretrained=wp, theta=1e4)
    want = sdpa_causal(rope_complex(qr, pos // G, 1e4), rope_complex(kr, pos // G, 1e4), v)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------------------
# Per-pair brute force (relative positions, pure Python)
# --------------------------------------------------------------------------------------
def brute_force(qr, kr, v, w0, wp, theta):
    """qr/kr raw [B, L, H, D]; every pair scored from its relative position."""
    B, L, Hq, D = qr.shape
    Hkv = kr.shape[2]
    half = D // 2
    G = 1
    while L > G * wp:
        G += 1
    freqs = [theta ** (-2.0 * kk / D) for kk in range(half)]
    out = np.zeros((B, L, Hq, D))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            kv = h * Hkv // Hq
            for i in range(L):
                scores = []
                for j in range(i + 1):
                    rel = (i - j) if (i - j) < w0 else (i // G - j // G)
                    acc = 0.0
                    for kk in range(half):
                        zq = complex(qr[b, i, h, kk], qr[b, i, h, kk + half])
                        zk = complex(kr[b, j, kv, kk], kr[b, j, kv, kk + half])
                        acc += (zq * zk.conjugate() * cmath.exp(1j * rel * freqs[kk])).real
                    scores.append(acc / math.sqrt(D))
                m = max(scores)
                ws = [math.exp(s - m) for s in scores]
                tot = sum(ws)
                for j, w in enumerate(ws):
                    out[b, i, h] += (w / tot) * v[b, j, kv]
                lse[b, h, i] = m + math.log(tot)
    return out, lse


BRUTE_CASES = [
    # (L, D, Hq, Hkv, wp, w0, theta)
    (40, 8, 2, 1, 12, 5, 1e4),    # G = 4
    (33, 8, 2, 2, 16, 1, 100.0),  # G = 3, w0 = 1: only the diagonal is local
    (28, 8, 4, 2, 9, 0, 1e4),     # G = 4, all remote
    (24, 8, 1, 1, 7, 24, 1e4),    # w0 = L: all local
    (30, 16, 2, 1, 10, 7, 1e6),   # G = 3, D = 16, large theta
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_per_pair_brute_force(case):
    L, D, Hq, Hkv, wp, w0, theta = case
    qr, kr, v = _rand(10 + L, 1, L, Hq, Hkv, D)
    pos = np.arange(L)
    q = rope_complex(qr, pos, theta)
    k = rope_complex(kr, pos, theta)
    want_o, want_lse = brute_force(qr, kr, v, w0, wp, theta)
    o, lse = bifocal_attention(q, k, v, w0=w0, w_pretrained=wp, theta=theta)
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-11)
    o3, lse3 = three_pass_attention(q, k, v, w0=w0, w_pretrained=wp, theta=theta)
    np.testing.assert_allclose(o3, want_o, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse3, want_lse, rtol=0, atol=1e-10)
    o_raw, _ = raw_bifocal_attention(qr, kr, v, w0=w0, w_pretrained=wp, theta=theta)
    np.testing.assert_allclose(o_raw, want_o, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------------------
# Formulations against each other at larger sizes
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L,wp,w0", [(512, 128, 32), (300, 64, 100), (257, 50, 0)])
def test_three_pass_merge_equals_direct_definition(L, wp, w0):
    q, k, v = _rand(20, 1, L, 2, 1, 32)
    o, lse = bifocal_attention(q, k, v, w0=w0, w_pretrained=wp, theta=1e4)
    o3, lse3, parts = three_pass_attention(q, k, v, w0=w0, w_pretrained=wp, theta=1e4, return_parts=True)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse3, lse, rtol=0, atol=1e-10)
    # B covers C's pairs, so LSE_B >= LSE_C everywhere (merge weights stay non-negative).
    assert np.all(parts["B"][1] >= parts["C"][1] - 1e-12)


def test_raw_definition_equals_correction_rotation_path():
    L, wp, w0, theta = 200, 48, 24, 1e6
    qr, kr, v = _rand(21, 1, L, 4, 2, 16)
    pos = np.arange(L)
    o_raw, lse_raw = raw_bifocal_attention(qr, kr, v, w0=w0, w_pretrained=wp, theta=theta)
    o, lse = bifocal_attention(rope_complex(qr, pos, theta), rope_complex(kr, pos, theta), v,
                               w0=w0, w_pretrained=wp, theta=theta)
    np.testing.assert_allclose(o, o_raw, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_raw, rtol=0, atol=1e-11)


def test_row_subset_equals_full_rows():
    q, k, v = _rand(22, 1, 150, 2, 2, 8)
    o, lse = bifocal_attention(q, k, v, w0=10, w_pretrained=40, theta=1e4)
    rows = [149, 0, 77, 10, 11]
    o2, lse2 = bifocal_attention(q, k, v, w0=10, w_pretrained=40, theta=1e4, rows=rows, block=2)
    # Only the BLAS summation order differs (a shorter key range per block).
    np.testing.assert_allclose(o2, o[:, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, rows], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("L", [47, 48, 49, 50])
def test_decode_equals_last_prefill_row_across_group_flip(L):
    # w_pretrained = 16: G = 3 up to L = 48 and 4 from L = 49.
    wp, w0, theta = 16, 6, 1e4
    rng = np.random.default_rng(30)
    cap = 52
    kc = rng.standard_normal((1, cap, 2, 8))
    vc = rng.standard_normal((1, cap, 2, 8))
    qs = rng.standard_normal((1, L, 4, 8))
    o_dec, lse_dec = bifocal_decode(qs[:, L - 1], kc, vc, L=L, w0=w0, w_pretrained=wp, theta=theta)
    o_pre, lse_pre = bifocal_attention(qs, kc[:, :L], vc[:, :L], w0=w0, w_pretrained=wp, theta=theta, rows=[L - 1])
    np.testing.assert_allclose(o_dec, o_pre[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_dec, lse_pre[:, :, 0], rtol=0, atol=1e-12)


def test_decode_matches_brute_force():
    L, wp, w0, theta = 35, 9, 4, 1e4
    qr, kr, v = _rand(31, 1, L, 2, 1, 8)
    pos = np.arange(L)
    want, want_lse = brute_force(qr, kr, v, w0, wp, theta)
    q = rope_complex(qr, pos, theta)
    k = rope_complex(kr, pos, theta)
    o, lse = bifocal_decode(q[:, L - 1], k, v, L=L, w0=w0, w_pretrained=wp, theta=theta)
    np.testing.assert_allclose(o, want[:, L - 1], rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, want_lse[:, :, L - 1], rtol=0, atol=1e-11)


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_decode_step_from_raw_is_last_row_of_brute_force(case):
    # The cache holds keys 0 .. p-1 at their base positions (complex rotation) plus garbage at
    # row p and beyond; the step itself must rotate the new raw key and query at p and append.
    L, D, Hq, Hkv, wp, w0, theta = case
    qr, kr, v = _rand(40 + L, 2, L, Hq, Hkv, D)
    p = L - 1
    want_o, want_lse = brute_force(qr, kr, v, w0, wp, theta)
    cap = L + 3
    rng = np.random.default_rng(L)
    kc = rng.standard_normal((2, cap, Hkv, D))
    vc = rng.standard_normal((2, cap, Hkv, D))
    kc[:, :p] = rope_complex(kr[:, :p], np.arange(p), theta)
    vc[:, :p] = v[:, :p]
    o, lse, kc2, vc2 = decode_step_from_raw(qr[:, p], kr[:, p], v[:, p], kc, vc, L=L, w0=w0, w_pretrained=wp,
                                            theta=theta)
    np.testing.assert_allclose(o, want_o[:, p], rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, want_lse[:, :, p], rtol=0, atol=1e-11)
    np.testing.assert_allclose(kc2[:, p], rope_complex(kr[:, p:L], [p], theta)[:, 0], rtol=0, atol=1e-12)
    assert np.array_equal(vc2[:, p], v[:, p])
    # Rows other than p are untouched, and the inputs are not modified in place.
    keep = [r for r in range(cap) if r != p]
    assert np.array_equal(kc2[:, keep], kc[:, keep]) and np.array_equal(vc2[:, keep], vc[:, keep])


# --------------------------------------------------------------------------------------
# Decode steps over one cache (each step its own length and G)
# --------------------------------------------------------------------------------------
def test_decode_steps_match_brute_force_across_group_flips():
    """Every step of a run whose length crosses two changes of G equals the last row of the
    per-pair brute force at that length (raw query at p = L - 1, keys at base positions)."""
    L_max, wp, w0, theta, D, Hq, Hkv = 38, 9, 4, 1e4, 8, 4, 2
    qr, kr, v = _rand(90, 2, L_max, Hq, Hkv, D)
    kc = rope_complex(kr, np.arange(L_max), theta)
    lengths = [1, 2, 9, 10, 18, 19, 27, 28, 37, 38]  # G = 1 .. 5, w0 edge at L = 5
    qs = np.stack([rope_complex(qr[:, L - 1:L], [L - 1], theta)[:, 0] for L in lengths])
    o, lse = bifocal_decode_steps(qs, kc, v, lengths=lengths, w0=w0, w_pretrained=wp, theta=theta, block=3)
    for t, L in enumerate(lengths):
        want_o, want_lse = brute_force(qr[:, :L], kr[:, :L], v[:, :L], w0, wp, theta)
        np.testing.assert_allclose(o[t], want_o[:, L - 1], rtol=0, atol=1e-11)
        np.testing.assert_allclose(lse[t], want_lse[:, :, L - 1], rtol=0, atol=1e-11)


@pytest.mark.parametrize("w0", [0, 1, 7, 1000])
def test_decode_steps_equal_single_decodes(w0):
    rng = np.random.default_rng(91 + w0)
    B, cap, Hq, Hkv, D, wp, theta = 2, 300, 6, 2, 16, 64, 1e6
    kc = rng.standard_normal((B, cap, Hkv, D))
    vc = rng.standard_normal((B, cap, Hkv, D))
    lengths = [300, 1, 64, 65, 128, 129, 200, 257]  # unordered, G from 1 to 5
    qs = rng.standard_normal((len(lengths), B, Hq, D))
    o, lse = bifocal_decode_steps(qs, kc, vc, lengths=lengths, w0=w0, w_pretrained=wp, theta=theta, block=2)
    for t, L in enumerate(lengths):
        o1, lse1 = bifocal_decode(qs[t], kc, vc, L=L, w0=w0, w_pretrained=wp, theta=theta)
        np.testing.assert_allclose(o[t], o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[t], lse1, rtol=0, atol=1e-12)


def test_row_blocks_and_workers_do_not_change_the_rows():
    q, k, v = _rand(23, 2, 200, 4, 2, 16)
    o1, l1 = bifocal_attention(q, k, v, w0=12, w_pretrained=48, theta=1e4, workers=1, block=200)
    o2, l2 = bifocal_attention(q, k, v, w0=12, w_pretrained=48, theta=1e4, workers=4, block=7)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
