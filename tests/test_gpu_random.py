"""Randomised parity of both decode paths against the oracle: seeded random batch sizes,
ragged context lengths (s_q up to 3000 tokens), split counts (automatic, 1 to 9), both
expanded-cache layouts, shuffled block tables with spare blocks, on every workload shape.
Each case is printed before its GPU calls, with everything needed to rerun it."""
import numpy as np
import pytest

from gpu_util import TOL, Run, log, oracle_paths, rel_err
from workloads import generate, workload

SHAPES = [("llama3-8b-b32-ctx8k", [1, 2, 4, 8]), ("dsv3-b64-ctx8k", [1, 2, 4]),
          ("dsv3-tp8share-ctx16k", [1, 2]), ("tiny-fp32", [1, 2])]


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        name, sqs = SHAPES[rng.integers(len(SHAPES))]
        s_q = int(rng.choice(sqs))
        B = int(rng.integers(1, 9))
        max_len = int(rng.choice([70, 300, 1500, 3000]))
        yield dict(name=name, s_q=s_q, lens=[int(rng.integers(s_q, max_len + 1)) for _ in range(B)],
                   splits=int(rng.choice([0, 0, 1, 2, 3, 5, 9])), shared=bool(rng.integers(2)),
                   extra=int(rng.integers(0, 4)), seed=int(rng.integers(1 << 30)))


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [101, 202, 303, 404])
def test_random_cases_match_oracle(seed):
    for i, c in enumerate(_cases(seed, 12)):
        log(f"case {seed}/{i}: {c}")
        x = generate(workload(c["name"]), c["s_q"], batch=len(c["lens"]), ctx_lens=c["lens"], shuffled=True,
                     extra_blocks=c["extra"], seed=c["seed"])
        run = Run(x, c["splits"], c["shared"])
        got_a, got_g = run.absorb(), run.gqa()
        ref = oracle_paths(x)
        tol = TOL["bf16"] if x.dtype == "bf16" else TOL["f32"]
        for b in ref:
            errs = (rel_err(got_a["out"][b], ref[b]["absorb_out"]), rel_err(got_a["o_lat"][b], ref[b]["o_lat"]),
                    rel_err(got_g["out"][b], ref[b]["out"]))
            lse_err = max(float(np.max(np.abs(got_a["lse"][b] - ref[b]["absorb_lse"]))),
                          float(np.max(np.abs(got_g["lse"][b] - ref[b]["lse"]))))
            scale = max(1.0, float(np.max(np.abs(ref[b]["lse"]))))
            assert max(errs) <= tol and lse_err <= tol * scale, (seed, i, b, errs, lse_err)
