"""gqla_stream_read, the streaming-read helper the benchmark's read ceiling comes from: every
16-byte word of the buffer is read exactly once for any workgroup count (a span tail and a
sub-span buffer included), and bad arguments are refused before any launch."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 32768, 32768 * 5 + 48, (8 << 20) + 16 * 37])
@pytest.mark.parametrize("wgs", [1, 7, 256, 4096])
def test_stream_read_sums_every_word_once(nbytes, wgs):
    import decode_attention_02_amd as G
    n = nbytes // 4
    # distinct small integers so a word read twice or skipped changes the exact fp32 sum
    src = (torch.arange(n, device="cuda", dtype=torch.int64) % 7 + 1).to(torch.float32)
    partial = torch.full((wgs,), float("nan"), dtype=torch.float32, device="cuda")
    G.gqla_stream_read(src, partial, wgs)
    torch.cuda.synchronize()
    want = float(src.double().sum())
    assert not torch.isnan(partial).any()
    assert float(partial.double().sum()) == want


def test_stream_read_rejects_bad_arguments():
    import decode_attention_02_amd as G
    src = torch.ones(64, dtype=torch.float32, device="cuda")
    partial = torch.empty(4, dtype=torch.float32, device="cuda")
    with pytest.raises(G.GqlaError):
        G.gqla_stream_read(src[1:], partial, 4)          # 252 bytes: not a multiple of 16
    with pytest.raises(G.GqlaError):
        G.gqla_stream_read(src, partial, 0)
    with pytest.raises(ValueError):
        G.gqla_stream_read(src, partial, 8)              # partial too short
