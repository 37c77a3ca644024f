"""The path picker against measurement: on two DeepSeek-V3 head-share cases where the
paths differ clearly on MI355X (absorb ahead at s_q = 1, GQA ahead at s_q = 4), the picked
path must be within 15% of the faster measured one."""
import pytest
import torch

from decode_attention_02_amd import crossover

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("s_q", [1, 4])
def test_picked_path_is_near_the_faster_one(s_q):
    log(f"picker dsv3 (R=4) s_q={s_q}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    r = crossover.run_case("dsv3 (R=4)", s_q, batch=64, ctx=8192, reps=5, gen=gen)
    log(f"  absorb {r['absorb_us']:.1f} us, gqa {r['gqa_us']:.1f} us, picked {r['picked']}")
    assert r["picked_cost"] <= 0.15
