"""GPU check of the streaming-read measurement kernel behind bench.py's
read ceiling: in both read patterns every 16-byte piece of the range is
read (a single piece whose words XOR to the fold's trigger value, anywhere
in the buffer, reaches the sink; an all-zero buffer leaves it untouched)."""
import pytest
import torch

from decode_attention_14_amd import binding as fd
from gpu_cases import say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

TRIGGER = 0x6a09e667  # the fold value that reaches the sink (fd_decode.hip)


@pytest.mark.parametrize("pattern", [0, 1])
@pytest.mark.parametrize("nbytes,workgroups", [(16 * 1000, 3), (1 << 20, 0), (1 << 22, 256), (16 * 4097, 7)])
def test_stream_read_reads_every_piece(pattern, nbytes, workgroups):
    say(f"[case] stream read pattern {pattern}, {nbytes} B, {workgroups} workgroups")
    n16 = nbytes // 16
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    fd.stream_read(buf, workgroups=workgroups, sink=sink, pattern=pattern)
    torch.cuda.synchronize()
    assert sink.item() == 0
    for piece in (0, 1, n16 // 2, n16 - 1):
        buf.zero_()
        buf[4 * piece + 2] = TRIGGER
        sink.zero_()
        fd.stream_read(buf, workgroups=workgroups, sink=sink, pattern=pattern)
        torch.cuda.synchronize()
        assert sink.item() == TRIGGER, (pattern, nbytes, workgroups, piece)
