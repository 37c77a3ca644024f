"""gqla_pick_path (host arithmetic, no GPU): argument checks and the properties its
cost model must have — work grows with context, the GQA cost with the number of groups,
the absorb cost with H * s_q — and the clear-cut choices at the two ends."""
import pytest

import decode_attention_02_amd as G
from decode_attention_02_amd import _lib


def dims(H=128, Gr=16, s_q=1, B=64, dn=128, dv=128, rope_shared=0):
    return G.Dims(batch=B, num_heads=H, num_groups=Gr, latent_rank=512, rope_dim=64, nope_dim=dn,
                  v_dim=dv, s_q=s_q, rope_shared=rope_shared)


def test_rejects_bad_context_totals():
    d = dims(s_q=2, B=4)
    with pytest.raises(_lib.GqlaError):
        G.gqla_pick_path(d, 4 * 2 - 1, 100)        # below B * s_q
    with pytest.raises(_lib.GqlaError):
        G.gqla_pick_path(d, 4 * 100 + 1, 100)      # above B * max_ctx
    with pytest.raises(_lib.GqlaError):
        G.gqla_pick_path(d, 8, 1)                  # max_ctx < s_q


def test_estimates_grow_with_context():
    d = dims()
    _, (a1, g1) = G.gqla_pick_path(d, 64 * 4096, 4096)
    _, (a2, g2) = G.gqla_pick_path(d, 64 * 8192, 8192)
    assert 0 < a1 < a2 and 0 < g1 < g2
    assert 1.6 < a2 / a1 < 2.1 and 1.6 < g2 / g1 < 2.1


def test_gqa_cost_follows_groups_absorb_cost_does_not():
    # same 128 heads, 4x the groups: 4x the expanded-cache bytes, same latent work
    _, (a4, g4) = G.gqla_pick_path(dims(Gr=4), 64 * 8192, 8192)
    _, (a16, g16) = G.gqla_pick_path(dims(Gr=16), 64 * 8192, 8192)
    assert g16 > 3.0 * g4
    assert abs(a16 - a4) < 1e-3 * a4


def test_absorb_cost_follows_query_rows():
    est = {s: G.gqla_pick_path(dims(s_q=s), 64 * 8192, 8192)[1] for s in (2, 8)}
    assert est[8][0] > 3.0 * est[2][0]      # MFMA-bound: ~4x the head-products
    assert est[8][1] < 1.2 * est[2][1]      # bandwidth-bound: same bytes


def test_clear_cut_choices():
    # one query row of 128 heads: the latent (1152 B/token) against 16 groups (10240 B/token)
    assert G.gqla_pick_path(dims(s_q=1), 64 * 8192, 8192)[0] == G.GQLA_PATH_ABSORB
    # sixteen query rows: the absorb path's head-products dominate
    assert G.gqla_pick_path(dims(s_q=16), 64 * 8192, 8192)[0] == G.GQLA_PATH_GQA


def test_shared_rope_layout_lowers_only_the_gqa_estimate():
    # LLaMA-3-8B shape: the RoPE key once per block instead of once per group cuts the
    # expanded bytes per token from 8 * 256 to 8 * 192 + 64 values (-22%)
    base = dict(H=32, Gr=8, s_q=2, B=32, dn=64, dv=128)
    _, (a0, g0) = G.gqla_pick_path(dims(**base), 32 * 8192, 8192)
    _, (a1, g1) = G.gqla_pick_path(dims(**base, rope_shared=1), 32 * 8192, 8192)
    assert a1 == a0
    assert 0.7 * g0 < g1 < 0.95 * g0
