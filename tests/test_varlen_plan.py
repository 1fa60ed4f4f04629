"""Host-side check of the per-sequence-length decode plan that the split kernel runs on the device.

The 32-key blocks of all sequences are laid end to end, and workgroup w of a grid of nwg takes the
run [w nb, (w + 1) nb) with nb = ceil(total / nwg). Its run crosses one or more segments (the part
of one sequence inside the run), and segment (w, b) writes partial record w + b. The workgroup
holding a sequence's first block records (first workgroup, count) for the reduce.

`lane_plan` restates, step by step, how one 64-lane wave finds a workgroup's run: per-lane sums over
contiguous groups of sequences, a scan over the lanes, then a scan over the chosen lane's sequences.
`direct_plan` is the definition through a prefix sum and a search. The tests check that the two
agree, that the runs cover every block of every sequence exactly once, that no workgroup carries
more than nb blocks, and that the record indices are distinct and below nwg + B."""
import numpy as np

CUS = 256       # workgroups that fill the chip once (one 8-wave workgroup per CU)
KV_WAVES = 8    # KV heads per workgroup
LANES = 64


def grid(n_kv_heads):
    groups = -(-n_kv_heads // KV_WAVES)
    return -(-CUS // groups)


def blocks_of(lens, max_len):
    L = np.clip(np.asarray(lens, dtype=np.int64), 1, max_len)
    return (L + 31) // 32


def direct_plan(blocks, nwg, w):
    """(b0, start, remaining, P0, nb) of workgroup w, from the definition."""
    P = np.concatenate([[0], np.cumsum(blocks)])
    total = int(P[-1])
    nb = -(-total // nwg)
    first = w * nb
    if first >= total:
        return -1, 0, 0, 0, nb
    b0 = int(np.searchsorted(P, first, side="right") - 1)
    return b0, int(first - P[b0]), int(min(nb, total - first)), int(P[b0]), nb


def lane_plan(blocks, nwg, w):
    """The wave's computation, lane by lane."""
    B = len(blocks)
    m = -(-B // LANES)
    lo = np.minimum(np.arange(LANES) * m, B)
    hi = np.minimum(lo + m, B)
    sums = np.array([int(blocks[lo[l]:hi[l]].sum()) for l in range(LANES)], dtype=np.int64)
    incl = np.cumsum(sums)
    total = int(incl[-1])
    nb = -(-total // nwg)
    first = w * nb
    if first >= total:
        return -1, 0, 0, 0, nb
    excl = incl - sums
    hit = np.nonzero((first >= excl) & (first < incl))[0]
    src = int(hit[0])
    base = int(excl[src])
    for j0 in range(lo[src], hi[src], LANES):
        j = np.arange(j0, min(j0 + LANES, hi[src]))
        n = blocks[j]
        inc = base + np.cumsum(n)
        ex = inc - n
        f = np.nonzero((first >= ex) & (first < ex + n))[0]
        if f.size:
            sj = int(f[0])
            b0 = int(j[sj])
            return b0, int(first - ex[sj]), int(min(nb, total - first)), int(ex[sj]), nb
        base = int(inc[-1])
    raise AssertionError("no sequence holds the run's first block")


def segments(blocks, nwg):
    """Every (workgroup, sequence, first local block, blocks) segment, walking each run as the
    kernel does; plus the (first, count) pair each sequence's first workgroup records."""
    segs, info = [], {}
    for w in range(nwg):
        b, start, rem, P, nb = direct_plan(blocks, nwg, w)
        while rem > 0:
            nbk = int(blocks[b])
            take = min(nbk - start, rem)
            if start == 0:
                info[b] = (w, (P + nbk - 1) // nb - w + 1)
            segs.append((w, b, start, take))
            rem -= take
            P += nbk
            b += 1
            start = 0
    return segs, info


def check(lens, max_len, n_kv_heads):
    blocks = blocks_of(lens, max_len)
    B, nwg = len(blocks), grid(n_kv_heads)
    segs, info = segments(blocks, nwg)
    nb = -(-int(blocks.sum()) // nwg)
    # Each sequence's blocks are covered exactly once, in order.
    covered = [[] for _ in range(B)]
    per_wg = np.zeros(nwg, dtype=np.int64)
    for w, b, start, take in segs:
        assert take >= 1
        covered[b].append((start, take))
        per_wg[w] += take
    for b in range(B):
        at = 0
        for start, take in covered[b]:
            assert start == at
            at += take
        assert at == blocks[b]
    assert per_wg.max() <= nb
    # Records w + b: distinct, below nwg + B.
    rec = [w + b for w, b, _, _ in segs]
    assert len(set(rec)) == len(rec) and max(rec) < nwg + B
    # The reduce's (first, count) of each sequence names exactly its segments' workgroups.
    for b in range(B):
        first, count = info[b]
        assert [w for w, bb, _, _ in segs if bb == b] == list(range(first, first + count))


def test_lane_plan_matches_definition():
    rng = np.random.default_rng(21)
    for _ in range(3000):
        B = int(rng.integers(1, 5000))
        max_len = int(rng.integers(1, 1 << 17))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(1, max_len + 1, size=B)
        elif kind == 1:
            lens = np.full(B, max_len)
        else:  # one long sequence among short ones
            lens = rng.integers(1, max(2, max_len // 100), size=B)
            lens[rng.integers(0, B)] = max_len
        blocks = blocks_of(lens, max_len)
        nwg = grid(int(rng.choice([1, 8, 16, 32])))
        for w in {0, nwg - 1, *rng.integers(0, nwg, size=6).tolist()}:
            assert lane_plan(blocks, nwg, w) == direct_plan(blocks, nwg, w)


def test_bench_mix():
    # 16K, 48K, 98512 and 128K keys, 8 KV heads: 9223 blocks, runs of 37 blocks over 250 workgroups.
    blocks = blocks_of([16384, 49152, 98512, 131072], 131072)
    assert int(blocks.sum()) == 9223
    segs, info = segments(blocks, 256)
    assert max(w for w, _, _, _ in segs) == 249
    assert info == {0: (0, 14), 1: (13, 43), 2: (55, 84), 3: (138, 112)}
    check([16384, 49152, 98512, 131072], 131072, 8)


def test_edge_batches():
    check([1], 1, 8)
    check([1] * 300, 1, 8)
    check([131072] * 255, 131072, 8)
    check([131072] * 257, 131072, 8)
    check([5, 131072], 131072, 8)
    check([0, -3, 7], 100, 8)          # lengths clamp to [1, max_len]
    check([40000] * 70, 40000, 32)     # 4 KV-head groups: 64 workgroups
    check(list(range(1, 3000)), 3000, 8)


def test_random_batches():
    rng = np.random.default_rng(20)
    for _ in range(300):
        B = int(rng.integers(1, 700))
        max_len = int(rng.integers(1, 1 << 17))
        lens = rng.integers(1, max_len + 1, size=B)
        check(lens.tolist(), max_len, int(rng.choice([1, 2, 8, 16, 32])))
