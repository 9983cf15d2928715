"""tq_gemv_noalloc (the allocation-free tq_gemv: its workspace is the
library's fixed device scratch array) against tq_gemv with a workspace of
its own, through the C ABI: two calls in a row, the second on a smaller
input, each bit-identical with tq_gemv and within tolerance of the oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import B3, TB, FMTS, acts_f16, assert_close, dev, say, upload_blob, weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)


def _call(tq, fmt, M, N, K, seed):
    t, s = weights(N, K, seed)
    W = upload_blob(fmt, t, s)
    x = dev(acts_f16(M, K, seed + 1))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    tq.tq_quant_act(x, q, a)
    need = tq.tq_gemv_workspace_bytes(fmt, M, N, K)
    assert 0 < need <= tq.lib.tq_noalloc_scratch_bytes()
    y0 = torch.full((M, N), float("nan"), device="cuda")
    y1 = torch.full((M, N), float("nan"), device="cuda")
    ws = torch.zeros((need + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    rc = tq.lib.tq_gemv_noalloc(fmt, M, N, K, W.data_ptr(), q.data_ptr(), a.data_ptr(), y1.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0, tq.tq_status_str(rc)
    tq.tq_gemv(fmt, M, N, K, W, q, a, y0, ws)
    torch.cuda.synchronize()
    y0, y1 = y0.cpu().numpy(), y1.cpu().numpy()
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), "differs from tq_gemv"
    assert_close(y1, oracle.gemv(t, s, q.cpu().numpy(), a.cpu().numpy()), f"noalloc {FMTS[fmt]} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_noalloc_two_calls_second_smaller(fmt):
    import ternary_weight_base_amd as tq
    # first: 8 tokens on the down shape (MFMA GEMV, K split into 3 chunks
    # meeting through the workspace); second, smaller: one token, 2048 rows
    # x 8192 (8 K chunks meeting through the counter and partial sums)
    say(f"noalloc {FMTS[fmt]} 8x5120x17408 then 1x2048x8192")
    _call(tq, fmt, 8, 5120, 17408, 9100)
    _call(tq, fmt, 1, 2048, 8192, 9200)
