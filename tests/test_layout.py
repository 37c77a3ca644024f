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


@pytest.mark.parametrize("dqk,dv,dr", [(48, 32, 16), (128, 128, 64), (192, 128, 64)])
def test_shared_rope_layout_positions(dqk, dv, dr):
    """rope_shared = 1: per block the RoPE keys once (slabs over d_R), then per group the
    d_n key features in slabs and V in 32-slot halves."""
    from gpu_util import expanded_block_values
    NB, G = 3, 2
    dn = dqk - dr
    K = np.zeros((NB, G, 64, dqk))
    V = np.zeros((NB, G, 64, dv))
    for p in range(NB):
        for g in range(G):
            K[p, g] = (p * 10 + g) * 1e6 + np.arange(64)[:, None] * 1e3 + np.arange(dqk)[None, :]
            V[p, g] = -((p * 10 + g) * 1e6 + np.arange(64)[:, None] * 1e3 + np.arange(dv)[None, :])
        K[p, :, :, dn:] = K[p, 0, :, dn:]          # the key is shared across groups
    flat = logical_to_expanded(K, V, rope_shared=True, dr=dr)
    per_block = expanded_block_values(G, dqk, dv, True, dr)
    assert per_block == 64 * (dr + G * (dn + dv)) and flat.shape == (NB * per_block,)
    blk = flat.reshape(NB, per_block)
    rng = np.random.default_rng(8)
    for _ in range(200):
        p, g, r = rng.integers(NB), rng.integers(G), rng.integers(64)
        f = rng.integers(dr)
        w = min(32, dr - 32 * (f // 32))
        assert blk[p, 2048 * (f // 32) + r * w + f % 32] == K[p, g, r, dn + f]
        f = rng.integers(dn)
        w = min(32, dn - 32 * (f // 32))
        assert blk[p, 64 * dr + g * 64 * (dn + dv) + 2048 * (f // 32) + r * w + f % 32] == K[p, g, r, f]
        f = rng.integers(dv)
        assert blk[p, 64 * dr + g * 64 * (dn + dv) + 64 * dn + 32 * dv * (r // 32) + 32 * f + r % 32] == V[p, g, r, f]
    K2, V2 = expanded_to_logical(flat, NB, G, dqk, dv, rope_shared=True, dr=dr)
    assert np.array_equal(K2, K) and np.array_equal(V2, V)
