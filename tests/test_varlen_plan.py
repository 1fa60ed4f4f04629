"""Host-side check of the per-sequence-length decode plan: the chunk rule the split and reduce
kernels evaluate on the device (one chunk length for the whole batch, from the device-side
lengths), restated here and run over random batches. It must cover every key of every sequence
with chunks that are multiples of the 32-key block and never need more workgroups than the
grid's slots."""
import numpy as np

CUS = 256       # workgroups that fill the chip once (one 8-wave workgroup per CU)
KV_WAVES = 8    # KV heads per workgroup


def slots_for(batch, n_kv_heads):
    groups = -(-n_kv_heads // KV_WAVES)
    return -(-CUS // groups) + batch


def plan(lens, max_len, n_kv_heads):
    B = len(lens)
    slots = slots_for(B, n_kv_heads)
    L = np.clip(np.asarray(lens, dtype=np.int64), 1, max_len)
    total = int(L.sum())
    per = -(-total // (slots - B))
    cap = -(-max_len // 32) * 32
    chunk = min(cap, max(32, -(-per // 32) * 32))
    counts = -(-L // chunk)
    return slots, chunk, counts, L


def check(lens, max_len, n_kv_heads):
    slots, chunk, counts, L = plan(lens, max_len, n_kv_heads)
    assert chunk % 32 == 0 and chunk >= 32
    assert np.all(counts * chunk >= L) and np.all((counts - 1) * chunk < L)  # covered, no empty chunk
    assert counts.sum() <= slots


def test_bench_mix():
    # 16K, 48K, 98512 and 128K keys, 8 KV heads: 251 chunks of 1184 keys in 260 slots.
    slots, chunk, counts, _ = plan([16384, 49152, 98512, 131072], 131072, 8)
    assert (slots, chunk) == (260, 1184)
    assert counts.tolist() == [14, 42, 84, 111]


def test_edge_batches():
    check([1], 1, 8)
    check([1] * 300, 1, 8)
    check([131072] * 255, 131072, 8)
    check([131072] * 256, 131072, 8)
    check([5, 131072], 131072, 8)
    check([0, -3, 7], 100, 8)          # lengths clamp to [1, max_len]
    check([40000] * 70, 40000, 32)     # 4 KV-head groups: 64 workgroups per round


def test_random_batches():
    rng = np.random.default_rng(20)
    for _ in range(20000):
        B = int(rng.integers(1, 600))
        max_len = int(rng.integers(1, 1 << 17))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(1, max_len + 1, size=B)
        elif kind == 1:
            lens = np.full(B, max_len)
        else:  # one long sequence among short ones
            lens = rng.integers(1, max(2, max_len // 100), size=B)
            lens[rng.integers(0, B)] = max_len
        check(lens.tolist(), max_len, int(rng.choice([1, 2, 8, 16, 32])))
