"""Checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

from workloads import WORKLOADS, bf16_bits_to_f64, f64_to_bf16_bits, generate, workload


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38]])
    ours = f64_to_bf16_bits(x)
    theirs = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(bf16_bits_to_f64(ours), torch.from_numpy(theirs.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_workload_shapes():
    for w in WORKLOADS.values():
        assert w.heads % w.groups == 0
    t = workload("dsv3-tp8share-ctx16k")
    per_tok = t.groups * (t.qk + t.v) * 2
    assert t.batch == 200 * 2**30 // (t.ctx[0] * per_tok) == 10240


def test_generator_is_seeded_and_paged():
    w = workload("dsv3-b8-ctx32k-64k")
    a = generate(w, 2, batch=3, ctx_lens=[70, 2, 129])
    b = generate(w, 2, batch=3, ctx_lens=[70, 2, 129])
    assert np.array_equal(a.latent_cache.view(np.uint16), b.latent_cache.view(np.uint16))
    assert a.num_blocks == 2 + 1 + 3
    assert sorted(a.block_table[a.block_table >= 0].tolist()) == list(range(6))
    assert (a.block_table[1, 1:] == -1).all()
    # slots past the end of a sequence are NaN
    last = a.block_table[0, 1]
    assert np.isnan(a.f64(a.latent_cache[last, 70 - 64:])).all()
    lens = generate(w, 2).ctx_lens
    assert lens.min() >= 32768 and lens.max() <= 65536 and len(set(lens.tolist())) > 1
