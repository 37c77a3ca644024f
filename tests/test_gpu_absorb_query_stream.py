"""GPU parity of gqla_absorb_query at row counts that take its streaming form (the W_UK^g
slice held in registers, 64-row tiles with the next tile's queries in flight) against the
fp64 oracle: two groups of eight heads (nope 128) and eight groups of four (nope 64), a
ragged last tile, and per-workgroup tile runs of even and odd length. The RoPE part is a copy
and must match bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from oracle import gqla_ref as R
from workloads.generate import bf16_bits_to_f64, f64_to_bf16_bits

from gpu_util import TOL, log, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


# (H, G, d_n, B, s_q): rows * H / G rows per group over 64-row tiles; with G groups and four
# 128-feature slices, 512 / (4 G) workgroups per (group, slice) take tiles x, x + 512 / (4 G), ...
@pytest.mark.parametrize("H,Gr,dn,B,s_q", [
    (16, 2, 128, 4101, 2),   # 1026 tiles per group (the last 16 rows): 17 or 16 per workgroup
    (32, 8, 64, 4100, 1),    # 257 tiles per group (the last 16 rows): 17 or 16 per workgroup
])
def test_absorb_query_stream_matches_oracle(H, Gr, dn, B, s_q):
    dc, dr = 512, 64
    rng = np.random.default_rng(zlib.crc32(f"absorb_query_stream/{H}/{Gr}/{dn}/{B}/{s_q}".encode()))
    qn_bits = f64_to_bf16_bits(rng.standard_normal((B, s_q, H, dn)))
    qr_bits = f64_to_bf16_bits(rng.standard_normal((B, s_q, H, dr)))
    wk_bits = f64_to_bf16_bits(rng.standard_normal((Gr, dn, dc)) * dn ** -0.5)
    d = G.Dims(batch=B, num_heads=H, num_groups=Gr, latent_rank=dc, rope_dim=dr, nope_dim=dn, v_dim=128, s_q=s_q,
               dtype=G.GQLA_BF16)
    q_abs = torch.full((B, s_q, H, dc + dr), float("nan"), dtype=torch.bfloat16, device="cuda")
    log(f"absorb_query stream H={H} G={Gr} d_n={dn} rows={B * s_q}")
    G.gqla_absorb_query(d, to_dev(qn_bits, "bf16"), to_dev(qr_bits, "bf16"), to_dev(wk_bits, "bf16"), q_abs)
    got = to_host(q_abs)
    ref = R.absorb_query(bf16_bits_to_f64(qn_bits), bf16_bits_to_f64(qr_bits), bf16_bits_to_f64(wk_bits))
    assert np.isfinite(got).all()
    e = rel_err(got[..., :dc], ref[..., :dc])
    log(f"  rel err {e:.2e}")
    assert e <= TOL["bf16"]
    assert np.array_equal(got[..., dc:], ref[..., dc:])
