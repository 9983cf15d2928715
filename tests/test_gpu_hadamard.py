"""GPU parity of the online Hadamard rotation of the FFN input: the standalone
rotate + quantise call (bit-exact with the oracle: q and the scale), and the
rotation folded into a projection's output (tq_gemv_quant's y_signs) and into
the decode stack (ffn_signs), checked through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import B3, TB, FMTS, assert_close, dev, say, upload_blob, weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)


def _tq():
    import ternary_weight_base_amd as tq
    return tq


def _hq_gpu(x, signs):
    tq = _tq()
    M, K = x.shape
    q = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
    a = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_hadamard_quant_act(dev(x), dev(signs), q, a)
    torch.cuda.synchronize()
    return q.cpu().numpy(), a.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 64), (1, 5120), (3, 17408), (16, 8192), (512, 1024), (2, 192),
                                 (2, 40960)])
def test_hadamard_quant_bit_exact(dtype, M, K):
    say(f"hadamard quant {dtype} M={M} K={K}")
    gen = synth.normal_f16 if dtype == "f16" else synth.normal_f32
    x = gen(synth.seed(700, M, K), M, K)
    s = synth.signs(synth.seed(701, K), K)
    q, a = _hq_gpu(x, s)
    q_ref, a_ref = oracle.quant(oracle.hadamard(x, s))
    assert np.array_equal(a.view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_hadamard_quant_special_rows():
    """A zero row (scale 0, q 0), a one-hot row (every rotated value +-1/8:
    q = +-127 with the signs' pattern), and flipped signs (q negated)."""
    say("hadamard quant special rows")
    K = 256
    x = np.zeros((3, K), dtype=np.float32)
    x[1, 70] = 3.0
    x[2] = synth.normal_f32(synth.seed(702, 1), K)
    s = synth.signs(synth.seed(703, K), K)
    q, a = _hq_gpu(x, s)
    assert a[0] == 0 and np.all(q[0] == 0)
    assert np.all(q[1, :64] == 0) and np.all(q[1, 128:] == 0)
    H = oracle.hadamard(x[1:2], s)[0]
    assert np.all(np.abs(H[64:128]) == np.float32(0.375))
    assert np.array_equal(q[1, 64:128], np.where(H[64:128] > 0, 127, -127).astype(np.int8))
    q2, a2 = _hq_gpu(x, (-s).astype(np.int8))
    assert np.array_equal(q2[2], -q[2]) and a2[2] == a[2]


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("N,K", [(5120, 8192), (640, 1024), (128, 384)])
def test_projection_output_rotation(fmt, N, K):
    """tq_gemv_quant with y_signs stores diag(s) H_64 y / 8: bit-exact with
    the oracle's rotation of the same launch's unrotated y, within tolerance
    of the oracle's own chain; y_bmax holds the rotated blocks' maxima."""
    say(f"projection rotation {FMTS[fmt]} N={N} K={K}")
    tq = _tq()
    t, sc = weights(N, K, 710 + N)
    W = upload_blob(fmt, t, sc)
    x = synth.normal_f16(synth.seed(711, K), K)
    s = synth.signs(synth.seed(712, N), N)
    ws = torch.zeros(max(4, (tq.tq_gemv_quant_workspace_bytes(fmt, N, K) + 15) // 16 * 4),
                     dtype=torch.int32, device="cuda")
    y0 = torch.full((N,), float("nan"), device="cuda")
    y1 = torch.full((N,), float("nan"), device="cuda")
    b1 = torch.full((N // 64,), float("nan"), device="cuda")
    tq.tq_gemv_quant(fmt, N, K, W, None, dev(x), y0, ws=ws)
    tq.tq_gemv_quant(fmt, N, K, W, None, dev(x), y1, y_bmax=b1, ws=ws, y_signs=dev(s))
    torch.cuda.synchronize()
    y0, y1, b1 = y0.cpu().numpy(), y1.cpu().numpy(), b1.cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), oracle.hadamard(y0, s).view(np.uint32))
    q, a = oracle.quant(x[None, :])
    assert_close(y1[None, :], oracle.hadamard(oracle.gemv(t, sc, q, a), s), "rotated y")
    assert np.array_equal(b1, np.abs(y1).reshape(-1, 64).max(axis=1))


@pytest.mark.parametrize("fmt", [B3, TB])
def test_decode_stack_ffn_rotation(fmt):
    """The stack with ffn_signs: y_o is the rotated O output, gate/up consume
    it (stage-isolated: the oracle quantises the GPU's y_o, as the other
    stack tests do), and the other stages are unchanged."""
    say(f"stack ffn rotation {FMTS[fmt]}")
    tq = _tq()
    L, hidden, inter, qkv_out, o_in = 2, 640, 1152, 1280, 1024
    shapes = {"qkv": (qkv_out, hidden), "o": (hidden, o_in), "gate": (inter, hidden),
              "up": (inter, hidden), "down": (hidden, inter)}
    host, devw = [], []
    for l in range(L):
        hw, dw = {}, []
        for i, (name, (N, K)) in enumerate(shapes.items()):
            t = synth.trits(synth.seed(720, l, i, 1), N, K)
            s = synth.scales(synth.seed(720, l, i, 2), N, K)
            hw[name] = (t, s)
            dw.append(dev(tq.tq_pack(fmt, t, s)))
        host.append(hw)
        devw.append(dw)
    x = synth.normal_f16(synth.seed(721, 1), L, hidden)
    a = synth.normal_f16(synth.seed(721, 2), L, o_in)
    signs = synth.signs(synth.seed(722, 1), L * hidden).reshape(L, hidden)
    outs = [torch.full((L, n), float("nan"), device="cuda") for n in (qkv_out, hidden, inter, hidden)]
    nbytes = tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    tq.tq_decode_stack(fmt, L, hidden, inter, qkv_out, o_in, devw, dev(x), dev(a), *outs, ws,
                       ffn_signs=dev(signs))
    torch.cuda.synchronize()
    y_qkv, y_o, h, y_out = (t.cpu().numpy() for t in outs)
    for l, hw in enumerate(host):
        q, sc = oracle.quant(x[l:l + 1])
        assert_close(y_qkv[l:l + 1], oracle.gemv(*hw["qkv"], q, sc), f"qkv[{l}]")
        q, sc = oracle.quant(a[l:l + 1])
        assert_close(y_o[l:l + 1], oracle.hadamard(oracle.gemv(*hw["o"], q, sc), signs[l]), f"o[{l}]")
        q, sc = oracle.quant(y_o[l:l + 1])
        h_ref = oracle.swiglu(oracle.gemv(*hw["gate"], q, sc), oracle.gemv(*hw["up"], q, sc))
        assert_close(h[l:l + 1], h_ref, f"h[{l}]")
        q, sc = oracle.quant(h[l:l + 1])
        assert_close(y_out[l:l + 1], oracle.gemv(*hw["down"], q, sc), f"down[{l}]")
