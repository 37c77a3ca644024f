"""Host-side checks of the C ABI: the library loads, exports what include/gqla.h
declares, validates arguments before launching anything, and plans splits. No GPU."""
import ctypes
import os
import re

import pytest

import decode_attention_02_amd as G
from decode_attention_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _dims(**kw):
    base = dict(batch=32, num_heads=32, num_groups=8, latent_rank=512, rope_dim=64, nope_dim=64,
                v_dim=128, s_q=1, dtype=G.GQLA_BF16)
    base.update(kw)
    return G.Dims(**base)


def test_every_declared_symbol_is_exported():
    header = open(os.path.join(ROOT, "include", "gqla.h")).read()
    declared = set(re.findall(r"\b(gqla_[a-z_]+)\s*\(", header))
    assert {"gqla_absorb_query", "gqla_decode_absorb", "gqla_expand_cache", "gqla_decode_gqa",
            "gqla_out_proj"} <= declared
    lib = ctypes.CDLL(G.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(G.EXPORTED)
    assert "gfx950" in G.gqla_version()


def test_cache_bytes_per_token_matches_printed_ratio():
    d = _dims()
    absorb = G.gqla_cache_bytes_per_token(d, G.GQLA_PATH_ABSORB)
    gqa = G.gqla_cache_bytes_per_token(d, G.GQLA_PATH_GQA)
    assert (absorb, gqa) == (576 * 2, 2048 * 2)
    assert absorb / gqa == 0.28125
    ds = _dims(num_heads=128, num_groups=16, nope_dim=128)
    assert G.gqla_cache_bytes_per_token(ds, G.GQLA_PATH_GQA) == 10240
    assert G.gqla_cache_bytes_per_token(_dims(num_heads=16, num_groups=2, nope_dim=128), G.GQLA_PATH_GQA) == 1280
    assert G.gqla_cache_bytes_per_token(_dims(dtype=G.GQLA_F32), G.GQLA_PATH_ABSORB) == 576 * 4
    assert G.gqla_cache_bytes_per_token(_dims(num_groups=5), G.GQLA_PATH_GQA) == 0
    assert G.gqla_cache_bytes_per_token(d, 7) == 0


@pytest.mark.parametrize("bad,msg", [
    (dict(num_groups=5), "must divide"),
    (dict(s_q=0), "s_q"),
    (dict(block_size=32), "block_size"),
    (dict(dtype=3), "dtype"),
    (dict(latent_rank=0), "positive"),
    (dict(rope_dim=-1), "positive"),
])
def test_invalid_dims_rejected_before_launch(bad, msg):
    with pytest.raises(G.GqlaError) as e:
        G.gqla_num_splits(_dims(**bad), G.GQLA_PATH_GQA, 128, 8192, 4096)
    assert e.value.status == _lib.GQLA_ERR_INVALID_ARG and msg in str(e.value)
    # the compute entry points reject the same dims without touching the device
    d = _dims(**bad).c()
    assert _lib.LIB.gqla_absorb_query(ctypes.byref(d), 1, 1, 1, 1, None) == _lib.GQLA_ERR_INVALID_ARG
    assert _lib.LIB.gqla_out_proj(ctypes.byref(d), 1, 1, 1, None) == _lib.GQLA_ERR_INVALID_ARG
    assert _lib.LIB.gqla_expand_cache(ctypes.byref(d), 1, 1, 1, 1, 1, 1, 1, None) == _lib.GQLA_ERR_INVALID_ARG
    p = _lib.gqla_paged(1, 1, 128, 8192, 4096, 0)
    assert _lib.LIB.gqla_decode_absorb_out(ctypes.byref(d), ctypes.byref(p), 1, 1, 1, 1, 1 << 30, 1, 1, None,
                                           None) == _lib.GQLA_ERR_INVALID_ARG


def test_invalid_paging_and_path_rejected():
    d = _dims()
    with pytest.raises(G.GqlaError, match="exceeds"):
        G.gqla_num_splits(d, G.GQLA_PATH_GQA, 10, 10 * 64 + 1, 100)
    with pytest.raises(G.GqlaError, match="max_ctx_len"):
        G.gqla_num_splits(_dims(s_q=2), G.GQLA_PATH_GQA, 10, 1, 100)
    with pytest.raises(G.GqlaError, match="unknown path"):
        G.gqla_num_splits(d, 2, 10, 64, 100)
    with pytest.raises(G.GqlaError, match="num_splits"):
        G.gqla_num_splits(d, G.GQLA_PATH_GQA, 10, 64, 100, num_splits=-1)
    dc = d.c()
    p = _lib.gqla_paged(None, None, 128, 8192, 4096, 0)
    assert _lib.LIB.gqla_decode_gqa(ctypes.byref(dc), ctypes.byref(p), 1, 1, None, 0, 1, None, None) \
        == _lib.GQLA_ERR_INVALID_ARG
    assert _lib.LIB.gqla_decode_absorb(ctypes.byref(dc), None, 1, 1, None, 0, 1, None, None) \
        == _lib.GQLA_ERR_INVALID_ARG
    assert _lib.LIB.gqla_decode_absorb_out(ctypes.byref(dc), None, 1, 1, 1, 1, 1 << 30, 1, 1, None, None) \
        == _lib.GQLA_ERR_INVALID_ARG
    # null tensors
    assert _lib.LIB.gqla_absorb_query(ctypes.byref(dc), None, 1, 1, 1, None) == _lib.GQLA_ERR_INVALID_ARG
    assert b"null" in _lib.LIB.gqla_last_error()
    pv = _lib.gqla_paged(1, 1, 128, 8192, 4096, 0)
    for nulled in range(5):   # q_abs, latent_cache, w_uv, o_lat, out
        args = [1, 1, 1, 1, 1 << 30, 1, 1]
        args[[0, 1, 2, 5, 6][nulled]] = None
        assert _lib.LIB.gqla_decode_absorb_out(ctypes.byref(dc), ctypes.byref(pv), *args, None, None) \
            == _lib.GQLA_ERR_INVALID_ARG
        assert b"null" in _lib.LIB.gqla_last_error()
    # zero blocks to expand is a no-op, negative is an error
    assert _lib.LIB.gqla_expand_cache(ctypes.byref(dc), None, None, None, None, 0, 1, None, None) == 0
    assert _lib.LIB.gqla_expand_cache(ctypes.byref(dc), 1, 1, 1, 1, -1, 1, 1, None) == _lib.GQLA_ERR_INVALID_ARG


def test_workspace_too_small_rejected_before_launch():
    d = _dims().c()
    p = _lib.gqla_paged(1, 1, 128, 8192, 4096, 4)
    st = _lib.LIB.gqla_decode_gqa(ctypes.byref(d), ctypes.byref(p), 1, 1, 1, 16, 1, None, None)
    assert st == _lib.GQLA_ERR_WORKSPACE
    # the fused absorb entry point checks the same workspace before its first launch
    ds = _dims(dtype=G.GQLA_BF16).c()
    st = _lib.LIB.gqla_decode_absorb_out(ctypes.byref(ds), ctypes.byref(p), 1, 1, 1, 1, 16, 1, 1, None, None)
    assert st == _lib.GQLA_ERR_WORKSPACE


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("B,H,Gr,s_q,ctx", [(32, 32, 8, 1, 8192), (32, 32, 8, 2, 8192), (64, 128, 16, 2, 8192),
                                            (8, 128, 16, 2, 65536), (10240, 16, 2, 2, 16384), (2, 8, 2, 2, 64),
                                            (3, 32, 8, 2, 1), (1, 16, 2, 1, 64 * 1000 + 5)])
def test_split_plan_covers_context(path, B, H, Gr, s_q, ctx):
    ctx = max(ctx, s_q)
    d = _dims(batch=B, num_heads=H, num_groups=Gr, s_q=s_q, nope_dim=128 if H >= 16 else 64)
    nblk = (ctx + 63) // 64
    for forced in (0, 1, 3, 7, 10**6):
        n = G.gqla_num_splits(d, path, nblk, ctx, B * nblk, num_splits=forced)
        assert 1 <= n <= min(nblk, 1024)
        if forced:
            assert n <= forced
        if path == G.GQLA_PATH_GQA and not forced and B * Gr < 256 and nblk >= 16:
            # length-balanced plan: n counts partial slots per row, bounded by the runs a
            # sequence can meet (runs of at least 8 blocks, ceil(256 / G) of them per group)
            assert 2 <= n <= min(-(-256 // Gr) + 1, -(-nblk // 8) + 1)
        else:
            bps = -(-nblk // n)
            assert (n - 1) * bps < nblk <= n * bps   # no empty trailing split
        ws = G.gqla_workspace_bytes(d, path, nblk, ctx, B * nblk, num_splits=forced)
        dvo = 128 if path == 1 else 512
        assert ws == (0 if n == 1 else B * s_q * H * n * (dvo + 1) * 4)
