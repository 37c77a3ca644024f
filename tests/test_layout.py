"""The expanded-cache layout that gqla_expand_cache writes and gqla_decode_gqa reads
(declared in include/gqla.h): the test-side converters must place every element where
the header's formulas say, including a partial last key slab."""
import numpy as np
import pytest

from gpu_util import expanded_to_logical, logical_to_expanded


@pytest.mark.parametrize("dqk,dv", [(48, 32), (128, 128), (192, 128)])
def test_expanded_layout_positions(dqk, dv):
    NB, G = 3, 2
    K = np.zeros((NB, G, 64, dqk))
    V = np.zeros((NB, G, 64, dv))
    # value = a unique code of (block, group, slot, feature)
    for p in range(NB):
        for g in range(G):
            K[p, g] = (p * 10 + g) * 1e6 + np.arange(64)[:, None] * 1e3 + np.arange(dqk)[None, :]
            V[p, g] = -((p * 10 + g) * 1e6 + np.arange(64)[:, None] * 1e3 + np.arange(dv)[None, :])
    flat = logical_to_expanded(K, V)
    assert flat.shape == (NB * G * 64 * (dqk + dv),)
    chunk = flat.reshape(NB, G, -1)
    rng = np.random.default_rng(7)
    for _ in range(200):
        p, g, r = rng.integers(NB), rng.integers(G), rng.integers(64)
        f = rng.integers(dqk)
        w = min(32, dqk - 32 * (f // 32))
        assert chunk[p, g, 2048 * (f // 32) + r * w + f % 32] == K[p, g, r, f]
        f = rng.integers(dv)
        assert chunk[p, g, 64 * dqk + 32 * dv * (r // 32) + 32 * f + r % 32] == V[p, g, r, f]
    K2, V2 = expanded_to_logical(flat, NB, G, dqk, dv)
    assert np.array_equal(K2, K) and np.array_equal(V2, V)
