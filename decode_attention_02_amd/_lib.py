"""ctypes binding of libgqla.so (argument marshalling only).

Each wrapper carries the name of the C entry point it calls, takes torch tensors that
already live on the GPU, and passes their device pointers and the current HIP stream.
No step of the computation happens here; if the library is missing the import fails.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqla.so")

GQLA_OK, GQLA_ERR_INVALID_ARG, GQLA_ERR_UNSUPPORTED, GQLA_ERR_WORKSPACE, GQLA_ERR_HIP = 0, -1, -2, -3, -4
GQLA_F32, GQLA_BF16 = 0, 1
GQLA_PATH_ABSORB, GQLA_PATH_GQA = 0, 1

EXPORTED = ("gqla_absorb_query", "gqla_decode_absorb", "gqla_out_proj", "gqla_expand_cache",
            "gqla_decode_gqa", "gqla_num_splits", "gqla_workspace_bytes",
            "gqla_cache_bytes_per_token", "gqla_validate_paged", "gqla_status_string",
            "gqla_last_error", "gqla_version", "gqla_pick_path", "gqla_append_tokens",
            "gqla_out_hidden", "gqla_fold_out_weight", "gqla_decode_absorb_noalloc",
            "gqla_decode_absorb_out", "gqla_stream_read")
NOALLOC_SCRATCH_BYTES = 64 << 20   # GQLA_NOALLOC_SCRATCH_BYTES


class GqlaError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {status}: {msg}")
        self.status = status


class gqla_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("latent_rank", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("nope_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("s_q", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_shared", ctypes.c_int32)]


class gqla_paged(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("ctx_lens", ctypes.c_void_p),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("num_splits", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with decode_attention_02_amd/build.py "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, P = ctypes.POINTER(gqla_dims), ctypes.POINTER(gqla_paged)
    sig = {
        "gqla_absorb_query": [D, vp, vp, vp, vp, vp],
        "gqla_decode_absorb": [D, P, vp, vp, vp, sz, vp, vp, vp],
        "gqla_decode_absorb_noalloc": [D, P, vp, vp, vp, vp, vp],
        "gqla_decode_absorb_out": [D, P, vp, vp, vp, vp, sz, vp, vp, vp, vp],
        "gqla_out_proj": [D, vp, vp, vp, vp],
        "gqla_expand_cache": [D, vp, vp, vp, vp, i64, i64, vp, vp],
        "gqla_decode_gqa": [D, P, vp, vp, vp, sz, vp, vp, vp],
        "gqla_num_splits": [D, P, i32, ctypes.POINTER(i32)],
        "gqla_workspace_bytes": [D, P, i32, ctypes.POINTER(sz)],
        "gqla_validate_paged": [D, P, vp],
        "gqla_pick_path": [D, i64, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float)],
        "gqla_append_tokens": [D, P, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp],
        "gqla_out_hidden": [D, i32, i32, vp, vp, vp, vp],
        "gqla_fold_out_weight": [D, i32, vp, vp, vp, vp],
        "gqla_stream_read": [vp, sz, vp, i32, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.gqla_cache_bytes_per_token.argtypes = [D, i32]
    lib.gqla_cache_bytes_per_token.restype = i64
    lib.gqla_status_string.argtypes = [ctypes.c_int]
    lib.gqla_status_string.restype = ctypes.c_char_p
    lib.gqla_last_error.argtypes = []
    lib.gqla_last_error.restype = ctypes.c_char_p
    lib.gqla_version.argtypes = []
    lib.gqla_version.restype = ctypes.c_char_p
    return lib


LIB = _load()


def _check(status: int, where: str) -> None:
    if status != GQLA_OK:
        raise GqlaError(status, where, LIB.gqla_last_error().decode())


@dataclass
class Dims:
    batch: int
    num_heads: int
    num_groups: int
    latent_rank: int
    rope_dim: int
    nope_dim: int
    v_dim: int
    s_q: int
    dtype: int = GQLA_BF16
    block_size: int = 64
    softmax_scale: float = 0.0
    rope_shared: int = 0

    def c(self) -> gqla_dims:
        return gqla_dims(self.batch, self.num_heads, self.num_groups, self.latent_rank,
                         self.rope_dim, self.nope_dim, self.v_dim, self.s_q, self.block_size,
                         self.dtype, self.softmax_scale, self.rope_shared)


@dataclass
class Paged:
    block_table: torch.Tensor   # int32 [B][max_blocks], device
    ctx_lens: torch.Tensor      # int32 [B], device
    max_ctx_len: int
    num_blocks: int
    num_splits: int = 0

    def c(self) -> gqla_paged:
        for t in (self.block_table, self.ctx_lens):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("block_table and ctx_lens must be contiguous int32")
        return gqla_paged(_ptr(self.block_table), _ptr(self.ctx_lens), self.block_table.shape[1],
                          self.max_ctx_len, self.num_blocks, self.num_splits)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgqla must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def gqla_absorb_query(dims: Dims, q_nope, q_rope, w_uk, q_abs, stream=None) -> None:
    d = dims.c()
    _check(LIB.gqla_absorb_query(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(q_abs),
                                 _stream(stream)), "gqla_absorb_query")


def gqla_decode_absorb(dims: Dims, paged: Paged, q_abs, latent_cache, workspace, o_lat, lse=None,
                       stream=None) -> None:
    d, p = dims.c(), paged.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.gqla_decode_absorb(ctypes.byref(d), ctypes.byref(p), _ptr(q_abs), _ptr(latent_cache),
                                  _ptr(workspace), ws_bytes, _ptr(o_lat), _ptr(lse), _stream(stream)),
           "gqla_decode_absorb")


def gqla_decode_absorb_noalloc(dims: Dims, paged: Paged, q_abs, latent_cache, o_lat, lse=None,
                               stream=None) -> None:
    """gqla_decode_absorb with the split partials in the library's fixed scratch array."""
    d, p = dims.c(), paged.c()
    _check(LIB.gqla_decode_absorb_noalloc(ctypes.byref(d), ctypes.byref(p), _ptr(q_abs), _ptr(latent_cache),
                                          _ptr(o_lat), _ptr(lse), _stream(stream)),
           "gqla_decode_absorb_noalloc")


def gqla_decode_absorb_out(dims: Dims, paged: Paged, q_abs, latent_cache, w_uv, workspace, o_lat, out, lse=None,
                           stream=None) -> None:
    """gqla_decode_absorb then gqla_out_proj in one call (split combine fused with W_UV^g)."""
    d, p = dims.c(), paged.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.gqla_decode_absorb_out(ctypes.byref(d), ctypes.byref(p), _ptr(q_abs), _ptr(latent_cache), _ptr(w_uv),
                                      _ptr(workspace), ws_bytes, _ptr(o_lat), _ptr(out), _ptr(lse), _stream(stream)),
           "gqla_decode_absorb_out")


def gqla_out_proj(dims: Dims, o_lat, w_uv, out, stream=None) -> None:
    d = dims.c()
    _check(LIB.gqla_out_proj(ctypes.byref(d), _ptr(o_lat), _ptr(w_uv), _ptr(out), _stream(stream)),
           "gqla_out_proj")


def gqla_expand_cache(dims: Dims, latent_cache, w_uk, w_uv, block_ids, num_blocks: int, expanded_cache,
                      stream=None) -> None:
    d = dims.c()
    if block_ids.dtype != torch.int32:
        raise ValueError("block_ids must be int32")
    _check(LIB.gqla_expand_cache(ctypes.byref(d), _ptr(latent_cache), _ptr(w_uk), _ptr(w_uv), _ptr(block_ids),
                                 block_ids.numel(), num_blocks, _ptr(expanded_cache), _stream(stream)),
           "gqla_expand_cache")


def gqla_decode_gqa(dims: Dims, paged: Paged, q, expanded_cache, workspace, out, lse=None,
                    stream=None) -> None:
    d, p = dims.c(), paged.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.gqla_decode_gqa(ctypes.byref(d), ctypes.byref(p), _ptr(q), _ptr(expanded_cache),
                               _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(stream)),
           "gqla_decode_gqa")


def _host_paged(max_blocks: int, max_ctx_len: int, num_blocks: int, num_splits: int) -> gqla_paged:
    return gqla_paged(None, None, max_blocks, max_ctx_len, num_blocks, num_splits)


def gqla_num_splits(dims: Dims, path: int, max_blocks: int, max_ctx_len: int, num_blocks: int,
                    num_splits: int = 0) -> int:
    d, p, n = dims.c(), _host_paged(max_blocks, max_ctx_len, num_blocks, num_splits), ctypes.c_int32()
    _check(LIB.gqla_num_splits(ctypes.byref(d), ctypes.byref(p), path, ctypes.byref(n)), "gqla_num_splits")
    return n.value


def gqla_workspace_bytes(dims: Dims, path: int, max_blocks: int, max_ctx_len: int, num_blocks: int,
                         num_splits: int = 0) -> int:
    d, p, n = dims.c(), _host_paged(max_blocks, max_ctx_len, num_blocks, num_splits), ctypes.c_size_t()
    _check(LIB.gqla_workspace_bytes(ctypes.byref(d), ctypes.byref(p), path, ctypes.byref(n)),
           "gqla_workspace_bytes")
    return n.value


def gqla_cache_bytes_per_token(dims: Dims, path: int) -> int:
    d = dims.c()
    return LIB.gqla_cache_bytes_per_token(ctypes.byref(d), path)


def gqla_append_tokens(dims: Dims, paged: Paged, c_new, kr_new, rope_theta: float, w_uk, w_uv, latent_cache,
                       expanded_cache=None, stream=None) -> None:
    d, p = dims.c(), paged.c()
    _check(LIB.gqla_append_tokens(ctypes.byref(d), ctypes.byref(p), _ptr(c_new), _ptr(kr_new), ctypes.c_float(rope_theta),
                                  _ptr(w_uk), _ptr(w_uv), _ptr(latent_cache), _ptr(expanded_cache), _stream(stream)),
           "gqla_append_tokens")


def gqla_out_hidden(dims: Dims, hidden: int, folded: bool, x, w, y, stream=None) -> None:
    """y = x W^T: W_O over the heads' outputs (folded=False) or the folded weight over the
    absorb path's latent outputs (folded=True)."""
    d = dims.c()
    _check(LIB.gqla_out_hidden(ctypes.byref(d), hidden, int(bool(folded)), _ptr(x), _ptr(w), _ptr(y), _stream(stream)),
           "gqla_out_hidden")


def gqla_fold_out_weight(dims: Dims, hidden: int, w_o, w_uv, w_fold, stream=None) -> None:
    d = dims.c()
    _check(LIB.gqla_fold_out_weight(ctypes.byref(d), hidden, _ptr(w_o), _ptr(w_uv), _ptr(w_fold), _stream(stream)),
           "gqla_fold_out_weight")


def gqla_pick_path(dims: Dims, total_ctx: int, max_ctx: int):
    """(path, (absorb_us, gqa_us)): the decode path the MI355X cost model picks."""
    d = dims.c()
    path = ctypes.c_int32()
    est = (ctypes.c_float * 2)()
    _check(LIB.gqla_pick_path(ctypes.byref(d), ctypes.c_int64(total_ctx), ctypes.c_int32(max_ctx),
                              ctypes.byref(path), est), "gqla_pick_path")
    return path.value, (float(est[0]), float(est[1]))


def gqla_validate_paged(dims: Dims, paged: Paged, stream=None) -> None:
    d, p = dims.c(), paged.c()
    _check(LIB.gqla_validate_paged(ctypes.byref(d), ctypes.byref(p), _stream(stream)), "gqla_validate_paged")


def gqla_stream_read(src, partial, num_wgs: int, stream=None) -> None:
    """Read every byte of the device tensor `src` with the decodes' streaming loads;
    partial (fp32, at least num_wgs elements) receives one sum per workgroup."""
    if partial.dtype != torch.float32 or partial.numel() < num_wgs:
        raise ValueError("partial must be fp32 with at least num_wgs elements")
    _check(LIB.gqla_stream_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(src.numel() * src.element_size()),
                                ctypes.c_void_p(partial.data_ptr()), ctypes.c_int32(num_wgs), _stream(stream)),
           "gqla_stream_read")


def gqla_version() -> str:
    return LIB.gqla_version().decode()
