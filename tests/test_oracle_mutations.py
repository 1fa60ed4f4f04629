"""The oracle's pins must catch plausible mistakes planted in the oracle (CPU only).

Each mutation edits one expression of the oracle's source text, loads the edited copy as
a throw-away module and runs it against the pins of tests/test_oracle_attention.py and
tests/test_oracle_positions.py (brute force, library causal attention, golden G values).
A mutation that no pin notices would mean the pins leave that part of the oracle open.
"""
import os
import types

import numpy as np
import pytest

from tests.test_oracle_attention import _rand, brute_force, rope_complex, sdpa_causal

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "bifocal_oracle.py")

MUTATIONS = [
    ("rotation sign", "x1 * c - x2 * s", "x1 * c + x2 * s"),
    ("rotation transposed", "x1 * s + x2 * c", "x2 * s + x1 * c"),
    ("window boundary off by one", "rel = r[:, None] - j[None, :]  # i - j\n        local = (rel >= 0) & (rel < w0)",
     "rel = r[:, None] - j[None, :]  # i - j\n        local = (rel >= 0) & (rel <= w0)"),
    ("remote boundary off by one", "        remote = rel >= w0\n        for h in range(Hq):",
     "        remote = rel > w0\n        for h in range(Hq):"),
    ("floor instead of ceil in G", "return max(1, -(-L // w_pretrained))", "return max(1, L // w_pretrained)"),
    ("dropped query correction",
     "q_rem = rotate_pairs(q_base, (delta[srt][:, None] * omega[None, :])[None, :, None, :])", "q_rem = q_base"),
    ("correction sign", "return x // int(G) - x", "return x - x // int(G)"),
    ("frequency exponent", "-2.0 * k / head_dim", "-1.0 * k / head_dim"),
    ("score scale", "scale = 1.0 / math.sqrt(D)\n    order = np.argsort", "scale = 1.0 / D\n    order = np.argsort"),
    ("GQA mapping", "if h // group != kv:\n                continue\n            s_base = (q_base",
     "if h % Hkv != kv:\n                continue\n            s_base = (q_base"),
    ("lse drops the max", "lse[b, h, order[sl]] = (m + np.log(l))[:, 0]", "lse[b, h, order[sl]] = np.log(l)[:, 0]"),
    ("new token rotated at L", "angles = p * rope_frequencies(D, theta)", "angles = L * rope_frequencies(D, theta)"),
    ("new value not appended", "vc[:, p] = np.asarray(v_new, dtype=np.float64)", "vc[:, p] = vc[:, p]"),
    ("new query left raw", "bifocal_decode(rotate_pairs(q_raw, angles), kc", "bifocal_decode(q_raw, kc"),
    ("decode steps: one G for every step", "G_of = np.array([group_size(int(L), w_pretrained) for L in lengths]",
     "G_of = np.array([group_size(int(lengths.max()), w_pretrained) for L in lengths]"),
    ("decode steps: window off by one", "rel = p[:, None] - j[None, :]  # p_t - j\n            local = (rel >= 0) & (rel < w0)",
     "rel = p[:, None] - j[None, :]  # p_t - j\n            local = (rel >= 0) & (rel <= w0)"),
    ("decode steps: query one position early", "p = lengths[t] - 1  # query positions", "p = lengths[t] - 2  # query positions"),
    ("decode steps: dropped query correction", "qr = rotate_pairs(qb, delta[p][:, None] * omega[None, :])", "qr = qb"),
]


def _load_mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), SRC + "<mutant>", "exec"), mod.__dict__)
    return mod


def _pins_pass(m) -> bool:
    """True if the (possibly mutated) oracle passes a compact set of the pins.

    A mutant that raises is reported by the caller, not counted as caught."""
    if True:
        # Golden G values (review page, Validation/Significance; atlas summary, Approach).
        if m.group_size(131072, 32768) != 4 or m.group_size(32769, 32768) != 2 or m.group_size(8, 32768) != 1:
            return False
        for L, D, Hq, Hkv, wp, w0, theta in [(30, 8, 4, 2, 8, 5, 1e4), (26, 8, 2, 1, 9, 0, 1e4)]:
            qr, kr, v = _rand(50 + L, 1, L, Hq, Hkv, D)
            pos = np.arange(L)
            q, k = rope_complex(qr, pos, theta), rope_complex(kr, pos, theta)
            want_o, want_lse = brute_force(qr, kr, v, w0, wp, theta)
            o, lse = m.bifocal_attention(q, k, v, w0=w0, w_pretrained=wp, theta=theta)
            if not (np.allclose(o, want_o, atol=1e-9, rtol=0) and np.allclose(lse, want_lse, atol=1e-9, rtol=0)):
                return False
        # Decode step on raw new-token vectors against the last brute-force row.
        L, D, Hq, Hkv, wp, w0, theta = 29, 8, 4, 2, 8, 5, 1e4
        qr, kr, v = _rand(70, 1, L, Hq, Hkv, D)
        want_o, _ = brute_force(qr, kr, v, w0, wp, theta)
        kc = rope_complex(kr, np.arange(L), theta)
        kc[:, L - 1] = 0.0
        vc = v.copy()
        vc[:, L - 1] = 0.0
        o, _, _, _ = m.decode_step_from_raw(qr[:, L - 1], kr[:, L - 1], v[:, L - 1], kc, vc, L=L, w0=w0,
                                            w_pretrained=wp, theta=theta)
        if not np.allclose(o, want_o[:, L - 1], atol=1e-9, rtol=0):
            return False
        # A run of decode steps across a change of G against the last brute-force row at each length.
        wp, w0, theta, D, Hq, Hkv = 8, 5, 1e4, 8, 4, 2
        qr, kr, v = _rand(80, 1, 34, Hq, Hkv, D)
        kc = rope_complex(kr, np.arange(34), theta)
        lengths = [15, 16, 17, 25, 33, 34]  # G = 2, 2, 3, 4, 5, 5
        qs = np.stack([rope_complex(qr[:, L - 1:L], [L - 1], theta)[:, 0] for L in lengths])
        o, lse = m.bifocal_decode_steps(qs, kc, v, lengths=lengths, w0=w0, w_pretrained=wp, theta=theta, block=4)
        for t, L in enumerate(lengths):
            want_o, want_lse = brute_force(qr[:, :L], kr[:, :L], v[:, :L], w0, wp, theta)
            if not (np.allclose(o[t], want_o[:, L - 1], atol=1e-9, rtol=0)
                    and np.allclose(lse[t], want_lse[:, :, L - 1], atol=1e-9, rtol=0)):
                return False
        # G = 1 against library causal attention.
        q, k, v = _rand(60, 1, 40, 4, 2, 16)
        o, _ = m.bifocal_attention(q, k, v, w0=8, w_pretrained=64, theta=1e4)
        return bool(np.allclose(o, sdpa_causal(q, k, v), atol=1e-9, rtol=0))


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass(_load_mutant("import math", "import math"))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert not _pins_pass(_load_mutant(old, new)), f"pins did not catch: {name}"
