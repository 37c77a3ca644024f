"""Guard bands and metadata validation, through the C ABI.

Every output buffer of every compute entry point (q_abs, o_lat, lse, out, the split
workspace, the expanded cache, the caches the append writes, y and W_fold) is allocated
with a band of sentinel words before and after it. After the calls the bands must be
bit-identical: a kernel that writes past either end of an output shows up here, where
NaN-prefilled outputs only catch elements that are never written. The paged caches are
tokens in fixed-size blocks ("Grouped Query Attention (GQA)", section "GQA et techniques
connexes", PagedAttention); gqla_validate_paged is the synchronous check of that metadata.
"""
import numpy as np
import pytest
import torch

import decode_attention_02_amd as G
from workloads import generate, workload

from gpu_util import log, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

BAND = 1024          # sentinel elements on each side of every output
SENT16 = 0x5A5B      # bf16 sentinel bits (a finite value no kernel here produces)
SENT32 = 0x5A5B5C5D  # fp32 sentinel bits


class Bands:
    """Outputs with sentinel bands around them."""

    def __init__(self):
        self.items = []

    def alloc(self, name, shape, dtype, fill=float("nan")):
        n = int(np.prod(shape))
        flat = torch.empty(BAND + n + BAND, dtype=dtype, device="cuda")
        bits = flat.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)
        sent = SENT16 if dtype == torch.bfloat16 else SENT32
        bits[:BAND] = sent
        bits[BAND + n:] = sent
        body = flat[BAND:BAND + n]
        if fill is not None:
            body.fill_(fill)
        self.items.append((name, flat, n, sent))
        return body.view(shape)

    def check(self):
        torch.cuda.synchronize()
        for name, flat, n, sent in self.items:
            bits = flat.view(torch.int16 if flat.dtype == torch.bfloat16 else torch.int32)
            u = np.uint16 if flat.dtype == torch.bfloat16 else np.uint32
            for side, band in (("before", bits[:BAND]), ("after", bits[BAND + n:])):
                band = band.cpu().numpy().view(u)
                bad = np.nonzero(band != sent)[0]
                assert len(bad) == 0, f"{name}: {len(bad)} words written {side} the buffer (first at {bad[0]})"


CASES = [  # workload, s_q, context lengths, splits, expanded layout shares the RoPE key
    ("tiny-fp32", 2, [64, 2, 130, 65], 3, False),
    ("tiny-fp32", 1, [64, 1, 200], 0, True),
    ("llama3-8b-b32-ctx8k", 2, [129, 700, 2], 0, True),
    ("llama3-8b-b32-ctx8k", 1, [129, 700, 2], 3, False),
    ("dsv3-b64-ctx8k", 2, [300, 65], 0, False),
    ("dsv3-b64-ctx8k", 1, [300, 65, 1000], 4, True),
    ("dsv3-tp8share-ctx16k", 2, [513, 40], 0, True),
]


@pytest.mark.parametrize("name,s_q,ctx,splits,shared", CASES)
def test_outputs_keep_their_guard_bands(name, s_q, ctx, splits, shared):
    w = workload(name)
    x = generate(w, s_q, batch=len(ctx), ctx_lens=ctx, shuffled=True, extra_blocks=1)
    log(f"guards {name} s_q={s_q} ctx={ctx} splits={splits} rope_shared={shared}")
    B, H = len(ctx), w.heads
    dt = torch_dtype(x.dtype)
    dims = G.Dims(batch=B, num_heads=H, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                  nope_dim=w.nope, v_dim=w.v, s_q=s_q, dtype=G.GQLA_BF16 if x.dtype == "bf16" else G.GQLA_F32,
                  rope_shared=int(shared))
    table = torch.from_numpy(x.block_table).cuda()
    lens = torch.from_numpy(x.ctx_lens).cuda()
    paged = G.Paged(table, lens, int(max(ctx)), x.num_blocks, splits)
    bands = Bands()
    w_uk, w_uv = to_dev(x.w_uk, x.dtype), to_dev(x.w_uv, x.dtype)
    q_nope, q_rope, q = to_dev(x.q_nope, x.dtype), to_dev(x.q_rope, x.dtype), to_dev(x.q, x.dtype)

    def ws(path):
        n = G.gqla_workspace_bytes(dims, path, table.shape[1], paged.max_ctx_len, x.num_blocks, splits)
        return bands.alloc(f"workspace[{path}]", (max(n, 4) // 4,), torch.float32) if n else None

    # MQA-absorb path
    q_abs = bands.alloc("q_abs", (B, s_q, H, w.latent + w.rope), dt)
    o_lat = bands.alloc("o_lat", (B, s_q, H, w.latent), torch.float32)
    lse_a = bands.alloc("lse(absorb)", (B, s_q, H), torch.float32)
    out_a = bands.alloc("out(absorb)", (B, s_q, H, w.v), dt)
    G.gqla_absorb_query(dims, q_nope, q_rope, w_uk, q_abs)
    G.gqla_decode_absorb(dims, paged, q_abs, to_dev(x.latent_cache, x.dtype), ws(G.GQLA_PATH_ABSORB), o_lat, lse_a)
    G.gqla_out_proj(dims, o_lat, w_uv, out_a)
    # GQA path: expansion of every block, decode
    per_block = 64 * G.gqla_cache_bytes_per_token(dims, G.GQLA_PATH_GQA) // (2 if x.dtype == "bf16" else 4)
    expanded = bands.alloc("expanded", (x.num_blocks * per_block,), dt)
    latent = bands.alloc("latent", x.latent_cache.shape, dt, fill=None)
    latent.copy_(to_dev(x.latent_cache, x.dtype))
    ids = torch.arange(x.num_blocks, dtype=torch.int32, device="cuda")
    G.gqla_expand_cache(dims, latent, w_uk, w_uv, ids, x.num_blocks, expanded)
    out_g = bands.alloc("out(gqa)", (B, s_q, H, w.v), dt)
    lse_g = bands.alloc("lse(gqa)", (B, s_q, H), torch.float32)
    G.gqla_decode_gqa(dims, paged, q, expanded, ws(G.GQLA_PATH_GQA), out_g, lse_g)
    # append of the s_q newest tokens into both caches (in place)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    c_new = torch.randn(B, s_q, w.latent, generator=gen, device="cuda").to(dt)
    kr_new = torch.randn(B, s_q, w.rope, generator=gen, device="cuda").to(dt)
    G.gqla_append_tokens(dims, paged, c_new, kr_new, 10000.0, w_uk, w_uv, latent, expanded)
    # output side: W_O over the heads' outputs, the fold, the folded projection
    hidden = H * w.v
    w_o = (torch.randn(hidden, H * w.v, generator=gen, device="cuda") * (H * w.v) ** -0.5).to(dt)
    y = bands.alloc("y", (B * s_q, hidden), dt)
    G.gqla_out_hidden(dims, hidden, False, out_g, w_o, y)
    w_fold = bands.alloc("w_fold", (hidden, H * w.latent), dt)
    G.gqla_fold_out_weight(dims, hidden, w_o, w_uv, w_fold)
    y2 = bands.alloc("y(folded)", (B * s_q, hidden), dt)
    G.gqla_out_hidden(dims, hidden, True, o_lat, w_fold, y2)
    bands.check()
    for t in (q_abs, o_lat, out_a, out_g, y, y2):
        assert torch.isfinite(t.float()).all()


def _validate(name, ctx, table_edit=None, lens_edit=None, max_ctx=None):
    w = workload(name)
    x = generate(w, 2, batch=len(ctx), ctx_lens=ctx, shuffled=True)
    table_h, lens_h = x.block_table.copy(), x.ctx_lens.copy()
    if table_edit:
        table_edit(table_h)
    if lens_edit:
        lens_edit(lens_h)
    dims = G.Dims(batch=len(ctx), num_heads=w.heads, num_groups=w.groups, latent_rank=w.latent, rope_dim=w.rope,
                  nope_dim=w.nope, v_dim=w.v, s_q=2)
    paged = G.Paged(torch.from_numpy(table_h).cuda(), torch.from_numpy(lens_h).cuda(),
                    int(max(ctx)) if max_ctx is None else max_ctx, x.num_blocks)
    G.gqla_validate_paged(dims, paged)


def test_validate_paged_accepts_a_good_table():
    _validate("dsv3-b64-ctx8k", [130, 64, 2, 65])


def _expect_invalid(match, **kw):
    with pytest.raises(G.GqlaError) as e:
        _validate("dsv3-b64-ctx8k", [130, 64, 2, 65], **kw)
    assert e.value.status == -1   # GQLA_ERR_INVALID_ARG
    msg = str(e.value)
    log(f"  rejected: {msg}")
    assert match in msg, msg


def test_validate_paged_names_an_out_of_pool_block():
    def edit(t):
        t[2, 0] = 10_000   # the pool holds 7 blocks
    _expect_invalid("block_table[2][0] = 10000", table_edit=edit)


def test_validate_paged_names_a_negative_block():
    def edit(t):
        t[0, 2] = -1       # third block of sequence 0 (130 tokens use 3 blocks)
    _expect_invalid("block_table[0][2] = -1", table_edit=edit)


def test_validate_paged_names_an_over_long_context():
    def edit(lens):
        lens[1] = 131      # beyond max_ctx_len = 130
    _expect_invalid("ctx_lens[1] = 131", lens_edit=edit)


def test_validate_paged_names_a_context_shorter_than_s_q():
    def edit(lens):
        lens[3] = 1        # s_q = 2 new tokens need L >= 2
    _expect_invalid("ctx_lens[3] = 1", lens_edit=edit)
