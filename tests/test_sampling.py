"""The output sample of the large parity cases (tests/parity.py, CPU only): it holds the seeded random
floor plus, for every expert, the first and last token and both tokens at each boundary of its GPU tiles."""
import numpy as np

from parity import SAMPLE_FLOOR, output_rows, sample_rows, tile_height


def test_tile_height_rule():
    # even split over ceil(n / 256) tiles, rounded up to 32 rows, never above 256
    assert tile_height(1) == 32 and tile_height(256) == 256 and tile_height(257) == 160
    assert tile_height(963) == 256 and tile_height(600) == 224
    for n in range(1, 3000, 7):
        h = tile_height(n)
        nt = -(-n // 256)
        assert h % 32 == 0 and h <= 256 and -(-n // h) == nt


def test_sample_covers_expert_ends_and_tile_boundaries():
    rng = np.random.default_rng(3)
    T, E, k = 5000, 40, 4
    # skewed routing: expert 0 in every token, others random
    ids = np.stack([np.concatenate([[0], rng.choice(np.arange(1, E), k - 1, replace=False)]) for _ in range(T)])
    rows = set(sample_rows(ids, 100, seed=1).tolist())
    assert len(rows) >= 100
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0]
        if toks.size == 0:
            continue
        assert toks[0] in rows and toks[-1] in rows
        ht = tile_height(toks.size)
        for b in range(ht, toks.size, ht):
            assert toks[b - 1] in rows and toks[b] in rows
    # expert 0 has 5000 rows: 19 tiles of 256 (rows 0..4863) and a last tile of 136
    assert all(b in rows for b in (255, 256, 4863, 4864, 4999))


def test_output_rows_floor():
    rng = np.random.default_rng(0)
    ids = np.stack([rng.choice(64, 4, replace=False) for _ in range(8192)])
    assert output_rows(8192, ids, 0, full=True).size == 8192
    assert output_rows(SAMPLE_FLOOR, ids[:SAMPLE_FLOOR], 0, full=False).size == SAMPLE_FLOOR
    s = output_rows(8192, ids, 0, full=False)
    assert s.size >= SAMPLE_FLOOR and np.all(np.diff(s) > 0)
