"""The streaming-read hook that measures the HBM read ceiling: every byte is
read exactly once, each workgroup its own contiguous chunk (checked through
the per-workgroup XOR words, computed here in numpy)."""
import numpy as np
import pytest

import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _expected(words: np.ndarray, wgs: int) -> np.ndarray:
    """Per-workgroup XOR: chunk w holds 16-byte words [w*per, (w+1)*per)."""
    n16 = words.size // 4
    per = -(-n16 // wgs) if n16 else 0
    out = np.zeros(wgs, dtype=np.uint32)
    for w in range(wgs):
        lo, hi = min(n16, w * per), min(n16, (w + 1) * per)
        if hi > lo:
            out[w] = np.bitwise_xor.reduce(words[4 * lo:4 * hi])
    return out


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 16, 8192 * 16 * 3 + 48, 1 << 22, (64 << 20) + 1024])
def test_stream_read_reads_each_byte_once(nbytes):
    import ternary_weight_base_amd as tq
    say(f"stream read {nbytes} B")
    W = tq.TQ_STREAM_READ_WGS
    words = synth.normal_f32(synth.seed(950, nbytes % 9973), nbytes // 4).view(np.uint32)
    src = dev(words.view(np.int32))
    sink = torch.full((W + 5,), -1, dtype=torch.int32, device="cuda")
    tq.tq_debug_stream_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:W], _expected(words, W))
    assert np.all(got[W:] == np.uint32(0xFFFFFFFF))  # nothing past the sink's used words
