"""One workspace serves calls of every shape and entry point in stream
order: each call leaves it zero-filled, so the outputs equal those of calls
that each had a fresh workspace, bit for bit.  The sequence interleaves the
one-token K-chunk meets (exchange with 3 and 4 chunks, counter with 8), the
equal split of gate/up, the Hadamard-rotated output (counter meet), the
small-batch MFMA GEMV's split-K and the GEMM's split-K."""
import numpy as np
import pytest

import synth
from gpu_util import B3, TB, FMTS, dev, say, upload_blob, weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quant(tq, x):
    q = torch.empty(x.shape, dtype=torch.int8, device="cuda")
    a = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    tq.tq_quant_act(x, q, a)
    return q, a


@pytest.mark.parametrize("fmt", [B3, TB])
def test_one_workspace_for_every_call(fmt):
    import ternary_weight_base_amd as tq
    say(f"shared workspace {FMTS[fmt]}")
    calls = []  # (name, workspace bytes, fn(ws) -> output)

    def gemv(M, N, K, seed):
        W = upload_blob(fmt, *weights(N, K, seed))
        q, a = _quant(tq, dev(synth.normal_f16(synth.seed(seed, 9), M, K)))
        nb = tq.tq_gemv_workspace_bytes(fmt, M, N, K)

        def run(ws):
            y = torch.full((M, N), float("nan"), device="cuda")
            tq.tq_gemv(fmt, M, N, K, W, q, a, y, ws)
            return y
        calls.append((f"gemv M={M} {N}x{K}", nb, run))

    def gate_up(N, K, seed):
        Wg, Wu = upload_blob(fmt, *weights(N, K, seed)), upload_blob(fmt, *weights(N, K, seed + 1))
        q, a = _quant(tq, dev(synth.normal_f16(synth.seed(seed, 9), 1, K)))
        nb = tq.tq_gemv_workspace_bytes(fmt, 1, N, K)

        def run(ws):
            h = torch.full((1, N), float("nan"), device="cuda")
            tq.tq_gemv_gate_up_swiglu(fmt, 1, N, K, Wg, Wu, q, a, h, ws)
            return h
        calls.append((f"gate/up {N}x{K}", nb, run))

    def rotated(N, K, seed):
        W = upload_blob(fmt, *weights(N, K, seed))
        x = dev(synth.normal_f16(synth.seed(seed, 9), K))
        s = dev(synth.signs(synth.seed(seed, 8), N))
        nb = tq.tq_gemv_quant_workspace_bytes(fmt, N, K, False)

        def run(ws):
            y = torch.full((N,), float("nan"), device="cuda")
            yb = torch.full(((N + 63) // 64,), float("nan"), device="cuda")
            tq.tq_gemv_quant(fmt, N, K, W, None, x, y, y_bmax=yb, ws=ws, y_signs=s)
            return torch.cat([y, yb])
        calls.append((f"rotated {N}x{K}", nb, run))

    def gemm(M, N, K, seed):
        W = upload_blob(fmt, *weights(N, K, seed))
        q, a = _quant(tq, dev(synth.normal_f16(synth.seed(seed, 9), M, K)))
        nb = tq.tq_gemm_workspace_bytes(fmt, M, N, K)
        assert nb > 0

        def run(ws):
            y = torch.full((M, N), float("nan"), device="cuda")
            tq.tq_gemm(fmt, M, N, K, W, q, a, y, ws)
            return y
        calls.append((f"gemm M={M} {N}x{K}", nb, run))

    gemv(1, 5120, 8192, 7000)       # 3 K chunks: exchange
    gate_up(17408, 5120, 7010)      # equal split: exchange
    gemv(1, 2048, 8192, 7020)       # 8 K chunks: counter
    rotated(5120, 8192, 7030)       # rotated output: counter
    gemv(4, 5120, 17408, 7040)      # MFMA GEMV, split-K
    gemm(128, 5120, 17408, 7050)    # GEMM, split-K
    gemm(330, 5120, 17408, 7070)    # GEMM, 128-row tiles, ragged last tile, 3-way split-K
    gemm(48, 5120, 17408, 7080)     # GEMM, 64-row tiles, 12-way split-K
    gemv(1, 4096, 8192, 7060)       # 4 K chunks: exchange, two tree levels

    def fresh(nb):
        return torch.zeros(max(4, (nb + 15) // 16 * 4), dtype=torch.int32, device="cuda")

    ref = []
    for name, nb, run in calls:
        ref.append(run(fresh(nb)).cpu().numpy())
    torch.cuda.synchronize()
    shared = fresh(max(nb for _, nb, _ in calls))
    for rep in range(2):
        outs = [run(shared) for _, _, run in calls]
        torch.cuda.synchronize()
        for (name, _, _), o, r in zip(calls, outs, ref):
            assert np.array_equal(o.cpu().numpy().view(np.uint32), r.view(np.uint32)), f"{name}, pass {rep}"
        assert not shared.any().item(), f"workspace left non-zero after pass {rep}"


def test_workspace_clear_and_check():
    """tq_workspace_check counts the non-zero 32-bit words exactly;
    tq_workspace_clear zeroes every byte of the range and nothing past it."""
    import ternary_weight_base_amd as tq
    say("workspace clear/check")
    rng = np.random.default_rng(7)
    for words in (4, 64, 1000, 262144 + 4):  # up to 1 MiB, one ragged tail of the grid
        host = rng.integers(-3, 3, size=words + 4, dtype=np.int32)
        host[-4:] = 5  # guard words past the range
        buf = dev(host)
        cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        tq.tq_workspace_check(buf[:words], cnt)
        torch.cuda.synchronize()
        assert int(cnt.item()) == int(np.count_nonzero(host[:words]))
        tq.tq_workspace_clear(buf[:words])
        tq.tq_workspace_check(buf[:words], cnt)
        torch.cuda.synchronize()
        assert int(cnt.item()) == 0
        out = buf.cpu().numpy()
        assert not out[:words].any() and (out[words:] == 5).all()


@pytest.mark.parametrize("fmt", [B3, TB])
def test_poisoned_workspace_is_detected_and_cleared(fmt):
    """A workspace holding stale words (as a call that did not complete
    would leave it) is reported by tq_workspace_check; after
    tq_workspace_clear a split-K call gives the same output, bit for bit, as
    on a fresh workspace, and leaves the workspace zero again."""
    import ternary_weight_base_amd as tq
    say(f"poisoned workspace {FMTS[fmt]}")
    N, K = 5120, 17408  # K chunks that meet through the workspace
    W = upload_blob(fmt, *weights(N, K, 31))
    q, a = _quant(tq, dev(synth.normal_f16(synth.seed(31, 9), 1, K)))
    nb = tq.tq_gemv_workspace_bytes(fmt, 1, N, K)
    assert nb > 0
    fresh = torch.zeros((nb + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    y0 = torch.full((1, N), float("nan"), device="cuda")
    tq.tq_gemv(fmt, 1, N, K, W, q, a, y0, fresh)
    ws = torch.zeros_like(fresh)
    ws[::97] = 12345  # stale counters / sums
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    tq.tq_workspace_check(ws, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == int((ws != 0).sum().item()) > 0
    tq.tq_workspace_clear(ws)
    y1 = torch.full((1, N), float("nan"), device="cuda")
    tq.tq_gemv(fmt, 1, N, K, W, q, a, y1, ws)
    tq.tq_workspace_check(ws, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
