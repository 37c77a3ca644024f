"""The five GQLA decode workloads, named by what they are.

Dimension names follow the GQLA pages: H query heads split into G groups of
gs = H / G heads that share one key/value up-projection (W_UK^g, W_UV^g); a joint
latent of d_c values plus a decoupled RoPE key of d_R values is cached per token;
queries carry d_n "nope" values plus d_R RoPE values; values have d_v entries.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int          # H
    groups: int         # G
    latent: int         # d_c
    rope: int           # d_R
    nope: int           # d_n
    v: int              # d_v
    batch: int          # B
    ctx: Tuple[int, int]  # (lo, hi) inclusive; lo == hi for a fixed context length
    s_q: Tuple[int, ...]  # query rows per sequence that the workload runs
    dtype: str          # "f32" or "bf16"
    shuffled: bool      # block table is a seeded permutation of the pool
    seed: int
    paths: Tuple[str, ...] = ("absorb", "gqa")
    note: str = ""

    @property
    def group_size(self) -> int:
        return self.heads // self.groups

    @property
    def qk(self) -> int:
        return self.nope + self.rope

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # Tiny layer for CPU-scale checks: 8 heads in 2 groups, latent 64 + RoPE 16.
    "tiny-fp32": Workload(
        "tiny-fp32", heads=8, groups=2, latent=64, rope=16, nope=32, v=32, batch=2,
        ctx=(64, 64), s_q=(1, 2), dtype="f32", shuffled=False, seed=1000,
        paths=("absorb", "gqa", "naive")),
    # LLaMA-3-8B attention converted to GQLA: 32 heads in 8 groups of 4, 512 + 64 latent.
    "llama3-8b-b32-ctx8k": Workload(
        "llama3-8b-b32-ctx8k", heads=32, groups=8, latent=512, rope=64, nope=64, v=128,
        batch=32, ctx=(8192, 8192), s_q=(1, 2), dtype="bf16", shuffled=False, seed=1001,
        note="absorb path at s_q=1, GQA path at s_q=2"),
    # DeepSeek-V3 attention shape: 128 heads in 16 groups of 8.
    "dsv3-b64-ctx8k": Workload(
        "dsv3-b64-ctx8k", heads=128, groups=16, latent=512, rope=64, nope=128, v=128,
        batch=64, ctx=(8192, 8192), s_q=(1, 2), dtype="bf16", shuffled=True, seed=1002),
    # Long context, DeepSeek-V3 shape, per-sequence lengths uniform in [32768, 65536].
    "dsv3-b8-ctx32k-64k": Workload(
        "dsv3-b8-ctx32k-64k", heads=128, groups=16, latent=512, rope=64, nope=128, v=128,
        batch=8, ctx=(32768, 65536), s_q=(2,), dtype="bf16", shuffled=True, seed=1003),
    # One eighth of the DeepSeek-V3 heads (16 heads, 2 groups) at 16K context; the batch
    # is sized so the expanded cache fills about 200 GiB of HBM.
    "dsv3-tp8share-ctx16k": Workload(
        "dsv3-tp8share-ctx16k", heads=16, groups=2, latent=512, rope=64, nope=128, v=128,
        batch=10240, ctx=(16384, 16384), s_q=(2,), dtype="bf16", shuffled=True, seed=1004),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
