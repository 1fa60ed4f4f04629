"""Pins for the oracle's position arithmetic: G, f and the remote-range guarantee.

Sources: review page "Paper Review -- Jet-Long", section Method (G and f); gist.science
technical summary, Methodologie section 1 (the G and f formulas, and that every remote
rotation stays on the pretrained grid with minimal compression); atlas.scime.ai summary,
Approach (G is the minimal integer compression that keeps remote relative positions in
the pretrained range).
"""
import os

import numpy as np
import pytest

from oracle import aliased_positions, correction_offsets, group_size

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "group_size.txt")


def _max_remote_relative(L: int, g: int) -> int:
    """Largest f(i) - f(j) over all pairs j <= i < L, enumerated pair by pair (numpy)."""
    x = np.arange(L)
    fx = x // g
    d = fx[:, None] - fx[None, :]
    return int(d[np.tril_indices(L)].max())


def _brute_force_group_size(L: int, w_pretrained: int) -> int:
    """Smallest integer g >= 1 such that every pair's aliased distance is < w_pretrained."""
    g = 1
    while _max_remote_relative(L, g) >= w_pretrained:
        g += 1
    return g


def test_group_size_matches_brute_force_enumeration():
    mismatches = []
    for L in range(1, 130):
        for wp in range(1, 33):
            if group_size(L, wp) != _brute_force_group_size(L, wp):
                mismatches.append((L, wp))
    assert not mismatches, mismatches[:10]


def test_group_size_golden_values():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            L, wp, G, _src = line.split(maxsplit=3)
            rows.append((int(L), int(wp), int(G)))
    assert len(rows) >= 6
    for L, wp, G in rows:
        assert group_size(L, wp) == G, (L, wp, G)


def test_group_size_rejects_bad_arguments():
    for L, wp in [(0, 10), (-3, 10), (10, 0), (10, -1)]:
        with pytest.raises(ValueError):
            group_size(L, wp)


def test_aliased_positions_by_repeated_subtraction():
    for L, G in [(1, 1), (17, 1), (50, 3), (64, 4), (97, 7)]:
        expect = []
        for x in range(L):
            n, r = 0, x
            while r >= G:
                r -= G
                n += 1
            expect.append(n)
        assert aliased_positions(L, G).tolist() == expect
        assert (correction_offsets(L, G) == np.array(expect) - np.arange(L)).all()


@pytest.mark.parametrize("L,wp,w0", [(200, 64, 16), (513, 128, 32), (1000, 250, 0), (97, 13, 5), (64, 64, 8)])
def test_remote_relative_positions_stay_in_pretrained_range(L, wp, w0):
    G = group_size(L, wp)
    f = aliased_positions(L, G)
    i, j = np.tril_indices(L)
    remote = (i - j) >= w0
    rel = f[i[remote]] - f[j[remote]]
    assert rel.size == 0 or (rel.min() >= 0 and rel.max() < wp)
    assert rel.size == 0 or rel.max() == (L - 1) // G
    # Minimality: with one group fewer some remote pair leaves the range (when G > 1 and
    # the farthest pair is remote).
    if G > 1 and (L - 1) >= w0:
        assert _max_remote_relative(L, G - 1) >= wp


def test_group_size_flip_in_the_decode_workload():
    # A 98000..98512 decode crosses 3 * 32768: G goes 3 -> 4 between these lengths.
    assert group_size(98304, 32768) == 3 == _closed_form_check(98304, 32768)
    assert group_size(98305, 32768) == 4 == _closed_form_check(98305, 32768)


def _closed_form_check(L, wp):
    # (L-1)//g < wp  <=>  L <= g * wp; smallest such g >= 1.
    g = 1
    while L > g * wp:
        g += 1
    return g
