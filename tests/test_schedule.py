"""The workspace-schedule reader the GPU tests use to find stored partials (CPU)."""
import numpy as np

from tests.schedule import workspace_segments


def test_segments_tile_every_sequence_in_order():
    rng = np.random.default_rng(22)
    for _ in range(30):
        lens = [int(x) for x in rng.integers(0, 300, size=int(rng.integers(1, 9)))]
        P = int(rng.choice([16, 32, 64]))
        n_wg = int(rng.integers(1, 12))
        segs = workspace_segments(lens, P, n_wg)
        nu = [-(-n // P) for n in lens]
        k = -(-sum(nu) // n_wg) if sum(nu) else 0
        per_wg = {}
        for w, b, lo, hi in segs:
            assert 0 <= w < n_wg and 0 <= lo < hi <= lens[b]
            assert lo % P == 0
            per_wg[w] = per_wg.get(w, 0) + -(-hi // P) - lo // P
        assert all(v <= k for v in per_wg.values())
        for b, n in enumerate(lens):
            mine = [(w, lo, hi) for w, bb, lo, hi in segs if bb == b]
            assert [x[0] for x in mine] == sorted(x[0] for x in mine)
            pos = 0
            for _, lo, hi in mine:
                assert lo == pos
                pos = hi
            assert pos == n


def test_segments_worked_case():
    # lengths 40 and 8 with 16-token units: 3 + 1 units; 2 runs take 2 units each
    assert workspace_segments([40, 8], 16, 2) == [(0, 0, 0, 32), (1, 0, 32, 40), (1, 1, 0, 8)]
    assert workspace_segments([0, 0], 16, 4) == []
