"""GPU parity of tq_gemv_quant (quantiser fused into the one-token
projection) against the oracle: quantise the same input with the oracle's
quantiser (bit-exact by construction), then its GEMV / SwiGLU."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import B3, TB, FMTS, assert_close, dev, say, weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)


def _block_max(v):
    v = np.abs(np.asarray(v, dtype=np.float32).ravel())
    pad = (-v.size) % 64
    return np.pad(v, (0, pad)).reshape(-1, 64).max(axis=1)


def _run(fmt, N, K, x, gate_up, seed, x_bmax=None):
    import ternary_weight_base_amd as tq
    tg, sg = weights(N, K, seed)
    Wg = dev(tq.tq_pack(fmt, tg, sg))
    Wu, tu, su = None, None, None
    if gate_up:
        tu, su = weights(N, K, seed + 1000)
        Wu = dev(tq.tq_pack(fmt, tu, su))
    y = torch.full((N,), float("nan"), device="cuda")
    yb = torch.full(((N + 63) // 64,), float("nan"), device="cuda")
    nbytes = tq.tq_gemv_quant_workspace_bytes(fmt, N, K, gate_up)
    ws = torch.zeros(max(4, (nbytes + 15) // 16 * 4), dtype=torch.int32, device="cuda")
    xb = None if x_bmax is None else dev(x_bmax)
    tq.tq_gemv_quant(fmt, N, K, Wg, Wu, dev(x), y, x_bmax=xb, y_bmax=yb, ws=ws)
    torch.cuda.synchronize()
    y, yb = y.cpu().numpy(), yb.cpu().numpy()
    q, s = oracle.quant(np.asarray(x).reshape(1, K))
    ref = oracle.gemv(tg, sg, q, s)
    if gate_up:
        ref = oracle.swiglu(ref, oracle.gemv(tu, su, q, s))
    return y, yb, ref.ravel()


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("gate_up", [False, True])
@pytest.mark.parametrize("N,K", [(640, 1024), (1152, 640), (4160, 2048), (300, 17408)])
def test_gemv_quant_f16(fmt, gate_up, N, K):
    say(f"gemv_quant f16 {FMTS[fmt]} gate_up={gate_up} {N}x{K}")
    x = synth.normal_f16(synth.seed(61, N, K), K)
    y, yb, ref = _run(fmt, N, K, x, gate_up, 61)
    assert_close(y, ref, "y")
    assert np.array_equal(yb, _block_max(y)), "block maxima of y"


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("gate_up", [False, True])
def test_gemv_quant_f32_with_block_maxima(fmt, gate_up):
    """fp32 input: the absmax comes from the given block maxima; a chained
    call (the maxima written by the previous projection) matches the oracle
    on the same fp32 vector."""
    say(f"gemv_quant f32 {FMTS[fmt]} gate_up={gate_up}")
    N, K = 1280, 2560
    x = synth.normal_f32(synth.seed(62, K), K) * np.float32(3.0)
    y, _, ref = _run(fmt, N, K, x, gate_up, 62, x_bmax=_block_max(x))
    assert_close(y, ref, "y")


def test_gemv_quant_chained():
    """Two projections chained through y_bmax: the second consumes the
    first's fp32 output and maxima, as the decode stack does."""
    import ternary_weight_base_amd as tq
    say("gemv_quant chained")
    N1, K1, N2 = 2048, 1024, 640
    t1, s1 = weights(N1, K1, 63)
    t2, s2 = weights(N2, N1, 64)
    W1, W2 = dev(tq.tq_pack(B3, t1, s1)), dev(tq.tq_pack(B3, t2, s2))
    x = synth.normal_f16(synth.seed(63), K1)
    y1 = torch.empty(N1, device="cuda")
    b1 = torch.empty(N1 // 64, device="cuda")
    y2 = torch.empty(N2, device="cuda")
    ws = torch.zeros(1 << 18, dtype=torch.int32, device="cuda")
    tq.tq_gemv_quant(B3, N1, K1, W1, None, dev(x), y1, y_bmax=b1, ws=ws)
    tq.tq_gemv_quant(B3, N2, N1, W2, None, y1, y2, x_bmax=b1, ws=ws)
    torch.cuda.synchronize()
    y1h = y1.cpu().numpy()
    q, s = oracle.quant(y1h.reshape(1, N1))  # stage-isolated: the GPU's y1
    assert_close(y2.cpu().numpy(), oracle.gemv(t2, s2, q, s).ravel(), "chained")


def test_gemv_quant_zero_input():
    say("gemv_quant zero input")
    N, K = 640, 1024
    x = np.zeros(K, dtype=np.float16)
    y, yb, ref = _run(B3, N, K, x, True, 65)
    assert np.all(y == 0) and np.all(yb == 0)


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("case", ["gate_up_f16", "gate_up_f32", "down_f32"])
def test_gemv_quant_full_ffn_shapes(fmt, case):
    """The FFN block's launches at full size: gate/up 2 x 17408 x 5120 (the
    equal item split over 256 workgroups) on an fp16 or an fp32 input, and
    down 5120 x 17408 (K chunks) on an fp32 input with block maxima."""
    say(f"gemv_quant full {FMTS[fmt]} {case}")
    if case == "down_f32":
        N, K, gate_up = 5120, 17408, False
    else:
        N, K, gate_up = 17408, 5120, True
    if case == "gate_up_f16":
        x, xb = synth.normal_f16(synth.seed(66, K), K), None
    else:
        x = synth.normal_f32(synth.seed(67, K), K)
        xb = _block_max(x)
    y, yb, ref = _run(fmt, N, K, x, gate_up, 68, x_bmax=xb)
    assert_close(y, ref, "y")
    assert np.array_equal(yb, _block_max(y)), "block maxima of y"


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("N,K,gate_up", [(17408, 5120, True), (5120, 17408, False)])
def test_exchange_meet_deterministic(fmt, N, K, gate_up):
    """The pieces of a cut block meet by exchange in whatever order they
    arrive; 20 runs of the 27B gate/up (two pieces per block, equal split)
    and down (three K chunks, a two-level tree) give the same y and block
    maxima bit for bit, the maxima are those of y, and the workspace ends
    zero."""
    import ternary_weight_base_amd as tq
    say(f"exchange determinism {FMTS[fmt]} {N}x{K}")
    Wg = dev(tq.tq_pack(fmt, *weights(N, K, 63)))
    Wu = dev(tq.tq_pack(fmt, *weights(N, K, 64))) if gate_up else None
    x = synth.normal_f32(synth.seed(65, K), K)
    xb = dev(_block_max(x))
    x = dev(x)
    nbytes = tq.tq_gemv_quant_workspace_bytes(fmt, N, K, gate_up)
    assert nbytes > 0
    ws = torch.zeros(max(4, (nbytes + 15) // 16 * 4), dtype=torch.int32, device="cuda")
    ys, bs = [], []
    for _ in range(20):
        y = torch.full((N,), float("nan"), device="cuda")
        yb = torch.full(((N + 63) // 64,), float("nan"), device="cuda")
        tq.tq_gemv_quant(fmt, N, K, Wg, Wu, x, y, x_bmax=xb, y_bmax=yb, ws=ws)
        ys.append(y)
        bs.append(yb)
    torch.cuda.synchronize()
    y0, b0 = ys[0].cpu().numpy(), bs[0].cpu().numpy()
    assert np.array_equal(b0, _block_max(y0))
    for y, yb in zip(ys[1:], bs[1:]):
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y0.view(np.uint32))
        assert np.array_equal(yb.cpu().numpy().view(np.uint32), b0.view(np.uint32))
    assert not ws.any().item()
