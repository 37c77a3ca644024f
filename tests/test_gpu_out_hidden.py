"""GPU parity of the output side (gqla_out_hidden, gqla_fold_out_weight) against the fp64
oracle, on seeded host inputs: W_O over the heads' outputs, the fold of W_UV^g into W_O, and
the folded projection over the absorb path's fp32 latent outputs. Row counts cover one row,
a ragged last 16-row tile and several row passes; hidden sizes cover the module's
H * head_dim, untied sizes (every weight-streaming form: per-wave register chunks, and from
hidden 8192 up 64-row LDS-staged chunks, 512 bytes of each row when the contraction is whole
256-element chunks, else 256) and one that is not a multiple of 16 (generic kernel)."""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from oracle import gqla_ref as R
from workloads.generate import bf16_bits_to_f64, f64_to_bf16_bits

from gpu_util import TOL, log, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu

# name: (H, G, d_c, d_v, dtype)
SHAPES = {
    "tiny-fp32": (8, 2, 64, 32, "f32"),
    "llama3-8b": (32, 8, 512, 128, "bf16"),
    "dsv3": (128, 16, 512, 128, "bf16"),
    "dsv3-tp8share": (16, 2, 512, 128, "bf16"),
    # head counts whose contraction H * d_v is 1 and 19 chunks of 128 (not whole 256-element
    # chunks: the LDS-staged form with 128-element chunks, its 4-chunk ring ending in a tail
    # of 1 and 3 chunks) ...
    "h1": (1, 1, 512, 128, "bf16"),
    "h19": (19, 1, 512, 128, "bf16"),
    # ... and 1, 3, 5, 7 and 11 chunks of 256 (the 512-byte-run form, with rings of 4 chunks
    # at 64 rows per workgroup and of 8 at 16 and 32: no whole ring, or tails after one)
    "h2": (2, 1, 512, 128, "bf16"),
    "h6": (6, 2, 512, 128, "bf16"),
    "h10": (10, 2, 512, 128, "bf16"),
    "h14": (14, 2, 512, 128, "bf16"),
    "h22": (22, 2, 512, 128, "bf16"),
}


def _stored(rng, shape, scale, dtype):
    """Seeded Gaussian rounded once to the storage type: (values as fp64, device tensor)."""
    x = rng.standard_normal(shape) * scale
    if dtype == "bf16":
        bits = f64_to_bf16_bits(x)
        return bf16_bits_to_f64(bits), to_dev(bits, "bf16")
    x32 = x.astype(np.float32)
    return x32.astype(np.float64), to_dev(x32, "f32")


def _dims(H, Gr, dc, dv, dtype, B, s_q):
    return G.Dims(batch=B, num_heads=H, num_groups=Gr, latent_rank=dc, rope_dim=16 if dtype == "f32" else 64,
                  nope_dim=32 if dtype == "f32" else 128, v_dim=dv, s_q=s_q,
                  dtype=G.GQLA_BF16 if dtype == "bf16" else G.GQLA_F32)


@pytest.mark.parametrize("name,hidden,B,s_q", [
    ("tiny-fp32", 256, 2, 2), ("tiny-fp32", 100, 3, 1),
    ("llama3-8b", 4096, 32, 1), ("llama3-8b", 4096, 3, 2), ("llama3-8b", 4096, 1, 1), ("llama3-8b", 4100, 5, 1),
    ("dsv3", 7168, 40, 2), ("dsv3", 16384, 2, 1),
    # 64-row LDS-staged form (hidden a multiple of 64, >= 128 workgroups): 1, 2 and 4 row
    # tiles, a ragged last tile, and two passes over the rows
    ("dsv3", 16384, 64, 1), ("dsv3", 8192, 70, 1), ("llama3-8b", 8192, 20, 1), ("llama3-8b", 16384, 13, 1),
    ("h1", 8192, 5, 1), ("h10", 8192, 33, 1), ("h19", 16384, 17, 1),
    ("h2", 8192, 3, 1), ("h6", 8192, 40, 1), ("h14", 16384, 64, 1), ("h14", 8192, 80, 1),
    ("h6", 7168, 40, 1), ("h10", 7200, 20, 1), ("h14", 4096, 33, 1), ("h2", 6144, 17, 1), ("h22", 4096, 24, 1),
    ("dsv3-tp8share", 2048, 9, 2),
])
def test_out_hidden_matches_oracle(name, hidden, B, s_q):
    H, Gr, dc, dv, dtype = SHAPES[name]
    rng = np.random.default_rng(zlib.crc32(f"{name}/{hidden}/{B}/{s_q}".encode()))
    d = _dims(H, Gr, dc, dv, dtype, B, s_q)
    out, out_d = _stored(rng, (B, s_q, H, dv), 1.0, dtype)
    w_o, w_o_d = _stored(rng, (hidden, H * dv), (H * dv) ** -0.5, dtype)
    w_uv, w_uv_d = _stored(rng, (Gr, dv, dc), dc ** -0.5, dtype)
    o_lat = rng.standard_normal((B, s_q, H, dc)).astype(np.float32)
    o_lat_d = to_dev(o_lat, "f32")
    o_lat = o_lat.astype(np.float64)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL[dtype]
    log(f"out_hidden {name} hidden={hidden} rows={B * s_q}")

    y = torch.empty(B, s_q, hidden, dtype=tdt, device="cuda")
    G.gqla_out_hidden(d, hidden, False, out_d, w_o_d, y)
    e = rel_err(to_host(y), R.hidden_projection(out, w_o))
    log(f"  unfolded {e:.2e}")
    assert e <= tol

    w_fold = torch.empty(hidden, H * dc, dtype=tdt, device="cuda")
    G.gqla_fold_out_weight(d, hidden, w_o_d, w_uv_d, w_fold)
    # The oracle folds a sample of output features where the whole fold would be large
    # (every output feature is its own row of W_O and of the folded weight).
    n_s = np.arange(hidden) if hidden * H * dc <= 1 << 24 else np.sort(rng.choice(hidden, 48, replace=False))
    wf_ref = R.fold_out_weight(w_o[n_s], w_uv, H)
    e = rel_err(to_host(w_fold)[n_s], wf_ref)
    log(f"  fold weight {e:.2e} ({len(n_s)} output features)")
    assert e <= tol

    yf = torch.empty(B, s_q, hidden, dtype=tdt, device="cuda")
    G.gqla_out_hidden(d, hidden, True, o_lat_d, w_fold, yf)
    got_f = to_host(yf)[..., n_s]
    e = rel_err(got_f, R.folded_hidden_projection(o_lat, wf_ref))
    log(f"  folded {e:.2e}")
    assert e <= tol
    # the fold changes nothing: the same rows through W_UV^g then W_O
    e = rel_err(got_f, R.hidden_projection(R.out_projection(o_lat, w_uv), w_o[n_s]))
    assert e <= tol


def test_out_hidden_rejects_bad_arguments():
    H, Gr, dc, dv, dtype = SHAPES["llama3-8b"]
    d = _dims(H, Gr, dc, dv, dtype, 2, 1)
    x = torch.zeros(2, 1, H, dv, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, H * dv, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(2, 1, 64, dtype=torch.bfloat16, device="cuda")
    for hidden in (0, 70000):
        with pytest.raises(G.GqlaError):
            G.gqla_out_hidden(d, hidden, False, x, w, y)
    with pytest.raises(G.GqlaError):
        G.gqla_fold_out_weight(d, 0, w, w, w)
