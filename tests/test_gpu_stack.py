"""GPU parity of the decode stack against the oracle, layer by layer:
tq_decode_stack (one fused quantise+project launch per projection) and
tq_decode_stack_persistent (one launch per 32 layers), which must agree bit
for bit.  Each stage is checked on the GPU's own input
of that stage (stage-isolated), because chained fp32 stages cannot be
bit-exact end-to-end (an ulp of difference can move an int8 across a
rounding tie); the chain as a whole is checked within the same tolerance."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import B3, B3R, BP, TB, FMTS, assert_close, dev, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)


def _run_stack(fmt, L, hidden, inter, qkv_out, o_in, seed, zero_layers=(), persistent=False,
               ffn_signs=None):
    import ternary_weight_base_amd as tq
    shapes = {"qkv": (qkv_out, hidden), "o": (hidden, o_in), "gate": (inter, hidden),
              "up": (inter, hidden), "down": (hidden, inter)}
    host, devw = [], []
    for l in range(L):
        hw, dw = {}, []
        for i, (name, (N, K)) in enumerate(shapes.items()):
            t = synth.trits(synth.seed(seed, l, i, 1), N, K)
            s = synth.scales(synth.seed(seed, l, i, 2), N, K)
            hw[name] = (t, s)
            dw.append(dev(tq.tq_pack(fmt, t, s)))
        host.append(hw)
        devw.append(dw)
    x = synth.normal_f16(synth.seed(seed, 99, 1), L, hidden)
    a = synth.normal_f16(synth.seed(seed, 99, 2), L, o_in)
    for l in zero_layers:  # absmax 0 all along the layer's chain
        x[l] = 0
        a[l] = 0
    y_qkv = torch.full((L, qkv_out), float("nan"), device="cuda")
    y_o = torch.full((L, hidden), float("nan"), device="cuda")
    h = torch.full((L, inter), float("nan"), device="cuda")
    y_out = torch.full((L, hidden), float("nan"), device="cuda")
    nbytes = tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    outs = []
    sg = None if ffn_signs is None else dev(ffn_signs)
    for rep in range(2):  # twice: the workspace must come back ready for reuse
        tq.tq_decode_stack(fmt, L, hidden, inter, qkv_out, o_in, devw, dev(x), dev(a),
                           y_qkv, y_o, h, y_out, ws, persistent=persistent, ffn_signs=sg)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (y_qkv, y_o, h, y_out)])
        assert tq.stack_timeouts(ws) == 0, "a wait of the persistent kernel gave up"
        # all but the block maxima of y_o and h (the last two sections) left zero
        r256 = lambda n: (n + 255) // 256 * 256
        keep = r256((hidden + 63) // 64 * 4) + r256((inter + 63) // 64 * 4)
        assert not ws[:(nbytes - keep) // 4].any().item(), "workspace not left zero"
    for r0, r1 in zip(*outs):
        assert np.array_equal(r0.view(np.uint32), r1.view(np.uint32)), "not deterministic"
    return host, x, a, outs[0]


def _check_layers(host, x, a, outs, what):
    y_qkv, y_o, h, y_out = outs
    for l, hw in enumerate(host):
        q, s = oracle.quant(x[l:l + 1])
        assert_close(y_qkv[l:l + 1], oracle.gemv(*hw["qkv"], q, s), f"{what} qkv[{l}]")
        q, s = oracle.quant(a[l:l + 1])
        assert_close(y_o[l:l + 1], oracle.gemv(*hw["o"], q, s), f"{what} o[{l}]")
        q, s = oracle.quant(y_o[l:l + 1])  # stage-isolated: the GPU's y_o
        h_ref = oracle.swiglu(oracle.gemv(*hw["gate"], q, s), oracle.gemv(*hw["up"], q, s))
        assert_close(h[l:l + 1], h_ref, f"{what} h[{l}]")
        q, s = oracle.quant(h[l:l + 1])  # stage-isolated: the GPU's h
        assert_close(y_out[l:l + 1], oracle.gemv(*hw["down"], q, s), f"{what} down[{l}]")


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
@pytest.mark.parametrize("L,hidden,inter,qkv_out,o_in", [(3, 640, 1152, 1280, 1024),
                                                          (2, 384, 2176, 1600, 768)])
def test_decode_stack_small(fmt, L, hidden, inter, qkv_out, o_in):
    say(f"stack {FMTS[fmt]} L={L} {hidden}/{inter}/{qkv_out}/{o_in}")
    host, x, a, outs = _run_stack(fmt, L, hidden, inter, qkv_out, o_in, 11 + L)
    _check_layers(host, x, a, outs, FMTS[fmt])


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
def test_decode_stack_full_shapes_two_layers(fmt):
    """The 27B-shaped layer (hidden 5120, intermediate 17408, QKV 10240, O 8192),
    two layers."""
    say(f"stack {FMTS[fmt]} full shapes L=2")
    host, x, a, outs = _run_stack(fmt, 2, 5120, 17408, 10240, 8192, 5)
    _check_layers(host, x, a, outs, "full")


def test_decode_stack_matches_separate_calls():
    """The fused launches compute what tq_quant_act followed by
    tq_gemv_gate_up_swiglu computes: the quantised input is bit-identical and
    the kernel and its split are the same, so the outputs are too."""
    import ternary_weight_base_amd as tq
    say("stack vs separate calls")
    L, hidden, inter, qkv_out, o_in = 2, 640, 1152, 1280, 1024
    host, x, a, outs = _run_stack(B3, L, hidden, inter, qkv_out, o_in, 21)
    y_o = outs[1]
    for l, hw in enumerate(host):
        Wg = dev(tq.tq_pack(B3, *hw["gate"]))
        Wu = dev(tq.tq_pack(B3, *hw["up"]))
        q = torch.empty((1, hidden), dtype=torch.int8, device="cuda")
        sc = torch.empty(1, dtype=torch.float32, device="cuda")
        tq.tq_quant_act(dev(y_o[l:l + 1]), q, sc)
        hh = torch.empty((1, inter), dtype=torch.float32, device="cuda")
        tq.tq_gemv_gate_up_swiglu(B3, 1, inter, hidden, Wg, Wu, q, sc, hh, tq.workspace(B3, 1, inter, hidden))
        torch.cuda.synchronize()
        assert np.array_equal(outs[2][l:l + 1].view(np.uint32), hh.cpu().numpy().view(np.uint32)), l


def test_decode_stack_zero_inputs():
    """All-zero layer inputs give all-zero outputs down the whole chain
    (absmax 0 -> scale 0, q 0), and do not disturb the neighbouring layers."""
    say("stack zero layers")
    host, x, a, outs = _run_stack(B3, 3, 640, 1152, 1280, 1024, 31, zero_layers=(1,))
    for t in outs:
        assert np.all(t[1] == 0)
    _check_layers(host, x, a, outs, "zero")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_decode_stack_long_rows(fmt):
    """An fp16 input longer than one absmax pass (o_in 9216 > 8192) and a
    producer with more than 320 row blocks (inter 20608: h's block maxima
    take a second pass)."""
    say(f"stack long rows {FMTS[fmt]}")
    host, x, a, outs = _run_stack(fmt, 1, 256, 20608, 384, 9216, 41)
    _check_layers(host, x, a, outs, "long")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_decode_stack_split_k_everywhere(fmt):
    """Every stage splits K over workgroups (16..40 groups per row), and the
    gate/up stage has 80 row blocks: the split-K counters of one launch and
    the partial sums of the others share the workspace without overlapping."""
    say(f"stack split-K {FMTS[fmt]}")
    host, x, a, outs = _run_stack(fmt, 2, 2048, 5120, 1024, 2048, 51)
    _check_layers(host, x, a, outs, "splitk")


@pytest.mark.parametrize("fmt", [B3, TB, BP])
@pytest.mark.parametrize("L,hidden,inter,qkv_out,o_in", [(3, 640, 1152, 1280, 1024),
                                                          (2, 2048, 5120, 1024, 2048),
                                                          (1, 256, 20608, 384, 9216),
                                                          (2, 5120, 17408, 10240, 8192),
                                                          (33, 256, 512, 384, 256)])
def test_persistent_matches_launches(fmt, L, hidden, inter, qkv_out, o_in):
    """The persistent kernel and the per-projection launches run the same
    plans, quantiser, integer cores and meets: every output equal bit for
    bit (27B shapes; split K everywhere; long rows; 33 layers = two
    persistent launches)."""
    say(f"persistent vs launches {FMTS[fmt]} L={L} {hidden}/{inter}/{qkv_out}/{o_in}")
    _, _, _, p = _run_stack(fmt, L, hidden, inter, qkv_out, o_in, 61 + L)
    _, _, _, q = _run_stack(fmt, L, hidden, inter, qkv_out, o_in, 61 + L, persistent=True)
    for name, u, v in zip(("y_qkv", "y_o", "h", "y_out"), p, q):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), name


@pytest.mark.parametrize("fmt", [B3, TB])
def test_persistent_repeated_calls_identical(fmt):
    """100 calls of the persistent kernel on one input give identical outputs.
    Regression: the block maxima of gate/up's output (read by down's
    quantiser) once took a wave ballot with only lane 0 active, so a piece of
    a cut block whose finished rows did not include row 0 dropped its
    maximum -- about one call in 70 quantised h with a smaller absmax."""
    import ternary_weight_base_amd as tq
    say(f"persistent repeated {FMTS[fmt]}")
    L, hidden, inter, qkv_out, o_in, seed = 2, 2048, 5120, 1024, 2048, 63
    shapes = [(qkv_out, hidden), (hidden, o_in), (inter, hidden), (inter, hidden), (hidden, inter)]
    devw = [[dev(tq.tq_pack(fmt, synth.trits(synth.seed(seed, l, i, 1), N, K),
                            synth.scales(synth.seed(seed, l, i, 2), N, K)))
             for i, (N, K) in enumerate(shapes)] for l in range(L)]
    x = dev(synth.normal_f16(synth.seed(seed, 99, 1), L, hidden))
    a = dev(synth.normal_f16(synth.seed(seed, 99, 2), L, o_in))
    outs = [torch.full((L, n), float("nan"), device="cuda") for n in (qkv_out, hidden, inter, hidden)]
    nbytes = tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    ref = None
    for it in range(100):
        tq.tq_decode_stack(fmt, L, hidden, inter, qkv_out, o_in, devw, x, a, *outs, ws, persistent=True)
        cur = torch.cat([o.flatten() for o in outs]).view(torch.int32)
        if ref is None:
            ref = cur.clone()
        else:
            assert torch.equal(cur, ref), f"call {it} differs"
    assert tq.stack_timeouts(ws) == 0


@pytest.mark.parametrize("fmt", [B3, TB])
def test_persistent_ffn_rotation_matches_launches(fmt):
    """With the FFN input rotated in O's epilogue (counter meet), full shapes."""
    say(f"persistent rotation {FMTS[fmt]}")
    signs = synth.signs(synth.seed(71, 1), 2 * 5120).reshape(2, 5120)
    _, _, _, p = _run_stack(fmt, 2, 5120, 17408, 10240, 8192, 71, ffn_signs=signs)
    _, _, _, q = _run_stack(fmt, 2, 5120, 17408, 10240, 8192, 71, ffn_signs=signs, persistent=True)
    for name, u, v in zip(("y_qkv", "y_o", "h", "y_out"), p, q):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), name


def test_persistent_wait_limit_gives_up_and_exits():
    """Failure handling of the bounded waits, forced from the host: a wait
    limit of one real-time tick (set in the workspace header) makes the
    persistent kernel's waits give up; the launch still ends normally and
    reports them in the workspace's first word.  A fresh workspace then
    gives correct results again."""
    import ternary_weight_base_amd as tq
    say("persistent wait limit")
    L, hidden, inter, qkv_out, o_in = 2, 640, 1152, 1280, 1024
    shapes = {"qkv": (qkv_out, hidden), "o": (hidden, o_in), "gate": (inter, hidden),
              "up": (inter, hidden), "down": (hidden, inter)}
    devw = [[dev(tq.tq_pack(B3, synth.trits(synth.seed(81, l, i, 1), N, K),
                            synth.scales(synth.seed(81, l, i, 2), N, K)))
             for i, (N, K) in enumerate(shapes.values())] for l in range(L)]
    x = dev(synth.normal_f16(synth.seed(81, 9, 1), L, hidden))
    a = dev(synth.normal_f16(synth.seed(81, 9, 2), L, o_in))
    outs = [torch.empty((L, n), device="cuda") for n in (qkv_out, hidden, inter, hidden)]
    nbytes = tq.tq_decode_stack_workspace_bytes(B3, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    ws[2] = 1  # wait limit: one tick (words 2..3, little endian)
    tq.tq_decode_stack(B3, L, hidden, inter, qkv_out, o_in, devw, x, a, *outs, ws, persistent=True)
    torch.cuda.synchronize()
    assert tq.stack_timeouts(ws) > 0
    ws.zero_()
    tq.tq_decode_stack(B3, L, hidden, inter, qkv_out, o_in, devw, x, a, *outs, ws, persistent=True)
    torch.cuda.synchronize()
    assert tq.stack_timeouts(ws) == 0
    ref = [t.clone() for t in outs]
    tq.tq_decode_stack(B3, L, hidden, inter, qkv_out, o_in, devw, x, a, *outs, ws)
    torch.cuda.synchronize()
    for u, v in zip(ref, outs):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))
