"""The seeded input generators: shapes, determinism, and the property each stress
distribution is there for (no GPU)."""

import math

import numpy as np

from workloads import WORKLOADS, custom, generate


def test_shapes_and_determinism():
    w = custom(2, 4, 2, 100, 192, 128)
    q, k, v = generate(w, seed=3)
    assert q.shape == (2, 4, 100, 192) and k.shape == (2, 2, 100, 192) and v.shape == (2, 2, 100, 128)
    assert q.dtype == k.dtype == v.dtype == np.float32
    q2, k2, v2 = generate(w, seed=3)
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    assert not np.array_equal(q, generate(w, seed=4)[0])
    assert set(WORKLOADS) >= {"tiny", "mha4k", "gqa32k", "mla32k", "act16k"}


def test_rising_scores_outgrow_a_lazy_reference_many_times():
    # base-2 logits of the last row, tile maxima over 64 keys: starting from the ceiling
    # of the first tile's maximum, count how often a tile's maximum exceeds the current
    # reference by more than the kernels' lazy threshold of 24 binades (each such tile
    # moves the reference to its ceiling)
    for dqk in (128, 192):
        w = custom(1, 2, 1, 2048, dqk, 128, dist="rising", wid=950)
        q, k, _ = generate(w, seed=0)
        for h in range(2):
            x = (k[0, 0].astype(np.float64) @ q[0, h, -1].astype(np.float64)) * math.log2(math.e) / math.sqrt(dqk)
            tile_max = x.reshape(-1, 64).max(axis=1)
            growth = (tile_max[-1] - tile_max[0]) / (len(tile_max) - 1)
            assert 4.0 < growth < 6.0  # about 5 binades per tile
            ref, moves = math.ceil(tile_max[0]), 0
            for m in tile_max[1:]:
                if m > ref + 24:
                    ref, moves = math.ceil(m), moves + 1
            assert moves >= 5
