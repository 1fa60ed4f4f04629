"""CPU oracle for Dynamic Bifocal RoPE attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU library (C-ABI + HIP kernels) never calls it and shares no
code with it; the product path raises if its HIP library is missing.

Everything here is float64 numpy, written from the method as the Jet-Long pages define it.
Sources are cited by page and section:

  [review]  "Paper Review -- Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
            RoPE" (romaanj.github.io), sections Method, Key idea, Results.
  [gist]    "Technische Samenvatting: Jet-Long" (gist.science), Methodologie sections 1
            (Dynamische Bifocale RoPE) and 2 (Efficientiemechanismen voor Inferentie).
  [atlas]   Jet-Long summary on atlas.scime.ai, section Approach.

What is computed (all readings of open points are listed in the design notes):
  * G = max(1, ceil(L / w_pretrained)), recomputed from the current length L, and the
    aliasing map f(x) = floor(x / G)  ([review] Method; [gist] section 1 formulas).
  * A pair (i, j), j <= i, is LOCAL when 0 <= i - j < w0 and keeps its ordinary RoPE score
    (positions i and j); it is REMOTE when i - j >= w0 and is scored as if the query sat
    at f(i) and the key at f(j)  ([review] Method; [gist] section 1, local/remote window).
  * Inputs are post-base-RoPE vectors (the cache keeps keys rotated at their absolute
    positions). Remote vectors are rebuilt by an extra rotation by Delta_x = f(x) - x,
    since RoPE rotations compose additively ([gist] section 2, correction rotation).
  * One causal softmax over the per-pair scores, scale 1/sqrt(D).
  * The pages obtain the same output from three attentions merged by inclusion-exclusion
    with log-sum-exp weights ([review] Method; [gist] section 2): `three_pass_attention`
    writes that merge out literally as a second formulation.

RoPE convention (not fixed by the pages): half-split pairs (d, d + D/2) and frequencies
omega_k = theta ** (-2k/D), k < D/2; a vector at position n is rotated pairwise by n*omega_k.

Parity pins (tests/test_oracle_*.py): brute-force enumeration of G and f, the remote
range invariant, G = 1 against a library causal attention, w0 >= L and w0 = 0 against
library causal attention on base/aliased RoPE built with complex arithmetic, the
three-pass merge, a raw-input definitional path, per-pair Python loops, and
decode == last prefill row.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "group_size",
    "aliased_positions",
    "correction_offsets",
    "rope_frequencies",
    "rotate_pairs",
    "bifocal_attention",
    "bifocal_decode",
    "bifocal_decode_steps",
    "three_pass_attention",
    "raw_bifocal_attention",
    "decode_step_from_raw",
]


# ---------------------------------------------------------------------------------------
# Position arithmetic ([review] Method; [gist] Methodologie section 1, Dynamische Groepering)
# ---------------------------------------------------------------------------------------
def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)), in exact integer arithmetic."""
    L = int(L)
    w_pretrained = int(w_pretrained)
    if L < 1 or w_pretrained < 1:
        raise ValueError("L and w_pretrained must be >= 1")
    return max(1, -(-L // w_pretrained))


def aliased_positions(L: int, G: int) -> np.ndarray:
    """f(x) = floor(x / G) for x = 0 .. L-1 (int64)."""
    return np.arange(int(L), dtype=np.int64) // int(G)


def correction_offsets(L: int, G: int) -> np.ndarray:
    """Delta_x = f(x) - x (<= 0): the extra rotation that moves a base-position vector to f(x)."""
    x = np.arange(int(L), dtype=np.int64)
    return x // int(G) - x


# ---------------------------------------------------------------------------------------
# RoPE rotation (half-split pairs)
# ---------------------------------------------------------------------------------------
def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_k = theta ** (-2k / D), k = 0 .. D/2 - 1 (float64)."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * k / head_dim)


def rotate_pairs(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each pair (x_k, x_{k+D/2}) by angles[..., k] (float64).

    x' _k       = x_k cos(a) - x_{k+D/2} sin(a)
    x' _{k+D/2} = x_k sin(a) + x_{k+D/2} cos(a)
    `angles` broadcasts against x[..., :D/2].
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    c = np.cos(angles)
    s = np.sin(angles)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def _remote_vectors(x: np.ndarray, L: int, G: int, theta: float) -> np.ndarray:
    """Correction rotation of post-RoPE vectors x [B, L, H, D] by Delta_n * omega (per position n)."""
    omega = rope_frequencies(x.shape[-1], theta)
    delta = correction_offsets(L, G).astype(np.float64)
    angles = delta[:, None] * omega[None, :]  # [L, D/2]
    return rotate_pairs(x, angles[None, :, None, :])


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, L, H, D] arrays")
    B, L, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] < L or k.shape[3] != D:
        raise ValueError("k/v shape mismatch")
    if Hq % k.shape[2] != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return B, L, Hq, k.shape[2], D


# ---------------------------------------------------------------------------------------
# Direct definition: per-pair score matrix, one causal softmax
# ---------------------------------------------------------------------------------------
def _run_jobs(fn, jobs, workers):
    """Run fn(*job) for every job on a thread pool with one BLAS thread per worker.

    Only the schedule is parallel: each job writes its own disjoint slice of the outputs."""
    jobs = list(jobs)
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers <= 1 or len(jobs) <= 1:
        for job in jobs:
            fn(*job)
        return
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(fn, *job) for job in jobs]:
                f.result()


def bifocal_attention(q, k, v, *, w0: int, w_pretrained: int, theta: float,
                      rows: Optional[Sequence[int]] = None, block: int = 64, workers: Optional[int] = None):
    """Dynamic bifocal attention from the per-pair definition.

    q: [B, L, Hq, D], k/v: [B, L, Hkv, D]; q and k post-base-RoPE at their absolute
    positions. Query head h reads KV head h // (Hq / Hkv).
    `rows` optionally restricts the computed query rows (any order); keys are always
    0 .. i for row i, and G is always taken from the full length L.
    Only the requested rows (and the keys they reach) are converted to float64.
    Rows are taken in ascending order in blocks of `block`, on `workers` threads (default:
    the host's cores, at most 16) over (sequence, KV head, row block).
    Returns (O [B, R, Hq, D] float64, LSE [B, Hq, R] float64, natural log), R = len(rows).
    """
    B, L, Hq, Hkv, D = _check_shapes(q, k, v)
    if w0 < 0:
        raise ValueError("w0 must be >= 0")
    G = group_size(L, w_pretrained)
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return np.zeros((B, 0, Hq, D)), np.zeros((B, Hq, 0))
    if rows.min() < 0 or rows.max() >= L:
        raise ValueError("row out of range")
    nk = int(rows.max()) + 1
    omega = rope_frequencies(D, theta)
    delta = correction_offsets(L, G).astype(np.float64)
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    order = np.argsort(rows, kind="stable")
    srt = rows[order]
    q_base = np.asarray(q[:, srt], dtype=np.float64)  # [B, R, Hq, D]
    q_rem = rotate_pairs(q_base, (delta[srt][:, None] * omega[None, :])[None, :, None, :])
    out = np.zeros((B, rows.size, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, rows.size), dtype=np.float64)
    # Base keys, remote keys (corrected by Delta_j) and values of each KV head, contiguous.
    kv_base, kv_rem, kv_val = {}, {}, {}

    def prepare(b, kv):
        kb = np.ascontiguousarray(k[b, :nk, kv], dtype=np.float64)
        kv_base[b, kv] = kb
        kv_rem[b, kv] = rotate_pairs(kb, delta[:nk, None] * omega[None, :])
        kv_val[b, kv] = np.ascontiguousarray(v[b, :nk, kv], dtype=np.float64)

    def row_block(b, kv, start):
        sl = slice(start, start + block)
        r = srt[sl]
        nkeys = int(r[-1]) + 1
        j = np.arange(nkeys, dtype=np.int64)
        rel = r[:, None] - j[None, :]  # i - j
        local = (rel >= 0) & (rel < w0)
        remote = rel >= w0
        for h in range(Hq):
            if h // group != kv:
                continue
            s_base = (q_base[b, sl, h] @ kv_base[b, kv][:nkeys].T) * scale
            s_rem = (q_rem[b, sl, h] @ kv_rem[b, kv][:nkeys].T) * scale
            s = np.where(local, s_base, np.where(remote, s_rem, -np.inf))
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, order[sl], h, :] = (p @ kv_val[b, kv][:nkeys]) / l
            lse[b, h, order[sl]] = (m + np.log(l))[:, 0]

    pairs = [(b, kv) for b in range(B) for kv in range(Hkv)]
    _run_jobs(prepare, pairs, workers)
    _run_jobs(row_block, [(b, kv, s0) for b, kv in pairs for s0 in range(0, rows.size, block)], workers)
    return out, lse


def bifocal_decode(q, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int, theta: float):
    """One decode step: the query at position p = L - 1 against cached keys 0 .. L-1.

    q: [B, Hq, D] post-base-RoPE at p; caches [B, Lcap, Hkv, D] with base-position keys.
    G is recomputed from this step's L ([review] Method: G follows the current length).
    Returns (o [B, Hq, D], lse [B, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if k_cache.shape[1] < L or L < 1:
        raise ValueError("L outside the cache")
    G = group_size(L, w_pretrained)
    p = L - 1
    omega = rope_frequencies(D, theta)
    delta = correction_offsets(L, G).astype(np.float64)
    kb = np.asarray(k_cache[:, :L], dtype=np.float64)
    vb = np.asarray(v_cache[:, :L], dtype=np.float64)
    k_rem = rotate_pairs(kb, (delta[:, None] * omega[None, :])[None, :, None, :])
    q_rem = rotate_pairs(q, (delta[p] * omega)[None, None, :])
    j = np.arange(L, dtype=np.int64)
    local = (p - j) < w0
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            kv = h // group
            s = np.where(local, kb[b, :, kv, :] @ q[b, h], k_rem[b, :, kv, :] @ q_rem[b, h]) * scale
            m = s.max()
            e = np.exp(s - m)
            out[b, h] = (e @ vb[b, :, kv, :]) / e.sum()
            lse[b, h] = m + math.log(e.sum())
    return out, lse


def bifocal_decode_steps(q_steps, k_cache, v_cache, *, lengths, w0: int, w_pretrained: int, theta: float,
                         block: int = 64, workers: Optional[int] = None):
    """A sequence of decode steps over one cache: step t's query q_steps[t], post-base-RoPE at
    p_t = lengths[t] - 1, attends cached keys 0 .. p_t with its own group size
    G_t = max(1, ceil(lengths[t] / w_pretrained)) ([review] Method: G follows the current
    length). A key is local iff p_t - j < w0, else remote (aliased positions f(p_t), f(j)).

    Each step is the decode of `bifocal_decode` at L = lengths[t]; here the steps that share a
    group size share the corrected keys, and the steps of a block of `block` are scored as the
    rows of one matrix, on `workers` threads over (group size, sequence, KV head, step block).
    q_steps [T, B, Hq, D]; caches [B, Lcap, Hkv, D]. Returns (o [T, B, Hq, D], lse [T, B, Hq]).
    """
    q_steps = np.asarray(q_steps, dtype=np.float64)
    T, B, Hq, D = q_steps.shape
    lengths = np.asarray(lengths, dtype=np.int64).reshape(T)
    Hkv = k_cache.shape[2]
    if T == 0:
        return np.zeros((0, B, Hq, D)), np.zeros((0, B, Hq))
    if lengths.min() < 1 or lengths.max() > k_cache.shape[1]:
        raise ValueError("L outside the cache")
    if w0 < 0:
        raise ValueError("w0 must be >= 0")
    omega = rope_frequencies(D, theta)
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    G_of = np.array([group_size(int(L), w_pretrained) for L in lengths], dtype=np.int64)
    nk = int(lengths.max())
    out = np.zeros((T, B, Hq, D), dtype=np.float64)
    lse = np.zeros((T, B, Hq), dtype=np.float64)
    kv_base, kv_val = {}, {}

    def prepare(b, kv):
        kv_base[b, kv] = np.ascontiguousarray(k_cache[b, :nk, kv], dtype=np.float64)
        kv_val[b, kv] = np.ascontiguousarray(v_cache[b, :nk, kv], dtype=np.float64)

    def steps_of_group(G, b, kv):
        st = np.nonzero(G_of == G)[0]
        n_g = int(lengths[st].max())
        delta = correction_offsets(n_g, G).astype(np.float64)
        k_rem = rotate_pairs(kv_base[b, kv][:n_g], delta[:, None] * omega[None, :])
        for s0 in range(0, st.size, block):
            t = st[s0:s0 + block]
            p = lengths[t] - 1  # query positions
            nkeys = int(p.max()) + 1
            j = np.arange(nkeys, dtype=np.int64)
            rel = p[:, None] - j[None, :]  # p_t - j
            local = (rel >= 0) & (rel < w0)
            remote = rel >= w0
            for h in range(Hq):
                if h // group != kv:
                    continue
                qb = q_steps[t, b, h]  # [S, D]
                qr = rotate_pairs(qb, delta[p][:, None] * omega[None, :])
                s_base = (qb @ kv_base[b, kv][:nkeys].T) * scale
                s_rem = (qr @ k_rem[:nkeys].T) * scale
                s = np.where(local, s_base, np.where(remote, s_rem, -np.inf))
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                out[t, b, h] = (e @ kv_val[b, kv][:nkeys]) / l
                lse[t, b, h] = (m + np.log(l))[:, 0]

    pairs = [(b, kv) for b in range(B) for kv in range(Hkv)]
    _run_jobs(prepare, pairs, workers)
    _run_jobs(steps_of_group, [(int(G), b, kv) for G in np.unique(G_of) for b, kv in pairs], workers)
    return out, lse


# ---------------------------------------------------------------------------------------
# Second formulation: three attentions merged by inclusion-exclusion
# ([review] Method: passes A, B, C and the merge; [gist] section 2, Inclusie-Exclusie)
# ---------------------------------------------------------------------------------------
def _windowed_attention(qx, kx, v, window: Optional[int], rows: np.ndarray, group: int):
    """Softmax attention over keys j with 0 <= i - j (< window when window is not None).

    Returns (O [B, R, Hq, D], LSE [B, Hq, R]); rows with no key get O = 0, LSE = -inf.
    """
    B, _, Hq, D = qx.shape
    scale = 1.0 / math.sqrt(D)
    nkeys = int(rows.max()) + 1
    rel = rows[:, None] - np.arange(nkeys)[None, :]
    allowed = rel >= 0
    if window is not None:
        allowed &= rel < window
    out = np.zeros((B, rows.size, Hq, D))
    lse = np.full((B, Hq, rows.size), -np.inf)
    has_key = allowed.any(axis=1)
    for b in range(B):
        for h in range(Hq):
            kv = h // group
            s = np.where(allowed, (qx[b, rows, h] @ kx[b, :nkeys, kv].T) * scale, -np.inf)
            m = np.where(has_key, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            safe = np.where(has_key, l, 1.0)
            out[b, :, h] = np.where(has_key[:, None], (e @ v[b, :nkeys, kv]) / safe[:, None], 0.0)
            lse[b, h] = np.where(has_key, m + np.log(safe), -np.inf)
    return out, lse


def three_pass_attention(q, k, v, *, w0: int, w_pretrained: int, theta: float,
                         rows: Optional[Sequence[int]] = None, return_parts: bool = False):
    """O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C), weights from log-sum-exps.

    A: sliding window (0 <= i-j < w0) on base vectors; B: full causal on remote vectors;
    C: sliding window on remote vectors. W_X = exp(LSE_X - M), M = max(LSE_A, LSE_B).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, Hkv, D = _check_shapes(q, k, v)
    G = group_size(L, w_pretrained)
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    group = Hq // Hkv
    q_rem = _remote_vectors(q, L, G, theta)
    k_rem = _remote_vectors(k, L, G, theta)
    o_a, lse_a = _windowed_attention(q, k, v, w0, rows, group)
    o_b, lse_b = _windowed_attention(q_rem, k_rem, v, None, rows, group)
    o_c, lse_c = _windowed_attention(q_rem, k_rem, v, w0, rows, group)
    m = np.maximum(lse_a, lse_b)  # LSE_B >= LSE_C: C's pairs are a subset of B's
    w_a = np.exp(lse_a - m)
    w_b = np.exp(lse_b - m)
    w_c = np.exp(lse_c - m)
    tr = lambda w: np.transpose(w, (0, 2, 1))[..., None]  # [B, Hq, R] -> [B, R, Hq, 1]
    num = tr(w_a) * o_a + tr(w_b) * o_b - tr(w_c) * o_c
    den = w_a + w_b - w_c
    out = num / tr(den)
    lse = m + np.log(den)
    if return_parts:
        return out, lse, {"A": (o_a, lse_a), "B": (o_b, lse_b), "C": (o_c, lse_c)}
    return out, lse


# ---------------------------------------------------------------------------------------
# Third formulation: from raw (pre-RoPE) vectors, positions applied per pair
# ---------------------------------------------------------------------------------------
def raw_bifocal_attention(q_raw, k_raw, v, *, w0: int, w_pretrained: int, theta: float):
    """The definition on raw vectors: a local pair scores R(i)q . R(j)k, a remote pair
    R(f(i))q . R(f(j))k. No correction rotation is involved.
    Returns (O [B, L, Hq, D], LSE [B, Hq, L]).
    """
    q_raw = np.asarray(q_raw, dtype=np.float64)
    k_raw = np.asarray(k_raw, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, Hkv, D = _check_shapes(q_raw, k_raw, v)
    G = group_size(L, w_pretrained)
    omega = rope_frequencies(D, theta)
    pos = np.arange(L, dtype=np.float64)
    fpos = aliased_positions(L, G).astype(np.float64)
    at = lambda x, p: rotate_pairs(x, (p[:, None] * omega[None, :])[None, :, None, :])
    q_base, k_base = at(q_raw, pos), at(k_raw, pos)
    q_alias, k_alias = at(q_raw, fpos), at(k_raw, fpos)
    rows = np.arange(L)
    rel = rows[:, None] - rows[None, :]
    local = (rel >= 0) & (rel < w0)
    remote = rel >= w0
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, L, Hq, D))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            kv = h // group
            s = np.where(local, q_base[b, :, h] @ k_base[b, :, kv].T,
                         np.where(remote, q_alias[b, :, h] @ k_alias[b, :, kv].T, -np.inf)) * scale
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            out[b, :, h] = (e @ v[b, :, kv]) / l
            lse[b, h] = (m + np.log(l))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------------------
# Decode step on the new token's raw vectors ([review] Method: keys are cached at their base
# positions; [gist] section 2: the cache is never rewritten when G changes)
# ---------------------------------------------------------------------------------------
def decode_step_from_raw(q_raw, k_raw, v_new, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int,
                         theta: float):
    """The new token sits at position p = L - 1: its raw query and key get base RoPE at p
    (angle p * omega_k), the rotated key and the value enter the cache at row p, and the step
    is then `bifocal_decode` at length L.

    q_raw [B, Hq, D]; k_raw, v_new [B, Hkv, D]; caches [B, Lcap, Hkv, D] (rows < p used).
    Returns (o, lse, k_cache', v_cache') with the updated caches as new float64 arrays.
    """
    q_raw = np.asarray(q_raw, dtype=np.float64)
    k_raw = np.asarray(k_raw, dtype=np.float64)
    D = q_raw.shape[-1]
    p = L - 1
    angles = p * rope_frequencies(D, theta)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    kc[:, p] = rotate_pairs(k_raw, angles)
    vc[:, p] = np.asarray(v_new, dtype=np.float64)
    o, lse = bifocal_decode(rotate_pairs(q_raw, angles), kc, vc, L=L, w0=w0, w_pretrained=w_pretrained, theta=theta)
    return o, lse, kc, vc
