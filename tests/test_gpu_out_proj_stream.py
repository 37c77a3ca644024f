"""GPU parity of gqla_out_proj at row counts that take its streaming form (four-wave
workgroups, one per CU, sharing each 16-row tile of o_lat through an LDS ring three tiles
deep) against the fp64 oracle's value projection: two and eight groups, a ragged last tile,
and per-workgroup tile runs that end on, and inside, the ring's unrolled round of four."""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from oracle import gqla_ref as R
from workloads.generate import bf16_bits_to_f64, f64_to_bf16_bits

from gpu_util import TOL, log, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


# (H, G, rows = B * s_q): rows * H / G rows per group over 16-row tiles; 256 / G workgroups
# per group take tiles x, x + 256 / G, ...
@pytest.mark.parametrize("H,Gr,B,s_q", [
    (16, 2, 2048, 1),    # 1024 tiles per group: 8 per workgroup, two whole rounds
    (16, 2, 2565, 1),    # 1283 tiles per group, the last with 8 of 16 rows: 10 or 11 per workgroup
    (32, 8, 1111, 1),    # 8 groups of 4 heads: 278 tiles per group (the last 12 rows): 8 or 9 per workgroup
])
def test_out_proj_stream_matches_oracle(H, Gr, B, s_q):
    dc, dv = 512, 128
    rng = np.random.default_rng(zlib.crc32(f"out_proj_stream/{H}/{Gr}/{B}/{s_q}".encode()))
    o_lat = rng.standard_normal((B, s_q, H, dc)).astype(np.float32)
    w_bits = f64_to_bf16_bits(rng.standard_normal((Gr, dv, dc)) * dc ** -0.5)
    w_uv = bf16_bits_to_f64(w_bits)
    d = G.Dims(batch=B, num_heads=H, num_groups=Gr, latent_rank=dc, rope_dim=64, nope_dim=128, v_dim=dv, s_q=s_q,
               dtype=G.GQLA_BF16)
    out = torch.full((B, s_q, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    log(f"out_proj stream H={H} G={Gr} rows={B * s_q}")
    G.gqla_out_proj(d, to_dev(o_lat, "f32"), to_dev(w_bits, "bf16"), out)
    got = to_host(out)
    ref = R.out_projection(o_lat.astype(np.float64), w_uv)
    assert np.isfinite(got).all()
    e = rel_err(got, ref)
    log(f"  rel err {e:.2e}")
    assert e <= TOL["bf16"]
