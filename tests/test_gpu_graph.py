"""The C-ABI calls captured in a HIP graph: each replay must reproduce the
eager result bit for bit (the split-K counters are left zero by every launch,
so a replay finds them as the first call did).  Replays are interleaved with
the program's own eager work and synchronisations."""
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


def _replays_match(fn, outs, n=3):
    """Run fn eagerly, capture it, replay n times with other work between the
    replays; every replay's outputs equal the eager ones bit for bit."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(n):
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else 99)
        junk.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            a, b = o.cpu().numpy(), e.cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {r}"


@pytest.mark.parametrize("fmt", [B3, TB])
def test_graph_decode_stack(fmt):
    """Every split mode in one stack: K chunks (O, down), the equal item
    split of a gate/up with 314 row blocks, and the FFN rotation."""
    import ternary_weight_base_amd as tq
    say(f"graph stack {FMTS[fmt]}")
    L, hidden, inter, qkv_out, o_in = 2, 256, 20096, 384, 2048
    shapes = ((qkv_out, hidden), (hidden, o_in), (inter, hidden), (inter, hidden), (hidden, inter))
    devw = [[upload_blob(fmt, *weights(N, K, 900 + 10 * l + i)) for i, (N, K) in enumerate(shapes)]
            for l in range(L)]
    x = dev(synth.normal_f16(synth.seed(901, 1), L, hidden))
    a = dev(synth.normal_f16(synth.seed(901, 2), L, o_in))
    signs = dev(synth.signs(synth.seed(901, 3), L * hidden).reshape(L, hidden))
    outs = [torch.empty((L, n), device="cuda") for n in (qkv_out, hidden, inter, hidden)]
    nb = tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nb + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    layers = tq.stack_layers(devw)
    _replays_match(lambda: tq.tq_decode_stack(fmt, L, hidden, inter, qkv_out, o_in, layers, x, a,
                                              *outs, ws, ffn_signs=signs), outs)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_graph_gemv_and_quant(M):
    """Quantiser, GEMV (one token: the projection kernel; 4 and 16 tokens:
    the MFMA kernel, split-K) and the fused gate/up, captured together."""
    import ternary_weight_base_amd as tq
    say(f"graph gemv M={M}")
    N, K = 5120, 8192
    W = upload_blob(B3, *weights(N, K, 910))
    Wg = upload_blob(B3, *weights(2048, 5120, 911))
    Wu = upload_blob(B3, *weights(2048, 5120, 912))
    x = dev(synth.normal_f16(synth.seed(913, M), M, K))
    x2 = dev(synth.normal_f16(synth.seed(914, M), M, 5120))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    q2 = torch.empty((M, 5120), dtype=torch.int8, device="cuda")
    a = torch.empty(M, device="cuda")
    a2 = torch.empty(M, device="cuda")
    y = torch.empty((M, N), device="cuda")
    h = torch.empty((M, 2048), device="cuda")
    ws = tq.workspace(B3, M, N, K)
    ws2 = tq.workspace(B3, M, 2048, 5120)

    def fn():
        tq.tq_quant_act(x, q, a)
        tq.tq_gemv(B3, M, N, K, W, q, a, y, ws)
        tq.tq_quant_act(x2, q2, a2)
        tq.tq_gemv_gate_up_swiglu(B3, M, 2048, 5120, Wg, Wu, q2, a2, h, ws2)
    _replays_match(fn, [q, a, y, q2, a2, h])


def test_graph_gemm_and_hadamard():
    import ternary_weight_base_amd as tq
    say("graph gemm + hadamard")
    M, N, K = 512, 1024, 5120
    W = upload_blob(TB, *weights(N, K, 920))
    x = dev(synth.normal_f16(synth.seed(921, 1), M, K))
    s = dev(synth.signs(synth.seed(921, 2), K))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a = torch.empty(M, device="cuda")
    y = torch.empty((M, N), device="cuda")
    ws = tq.workspace(TB, M, N, K)  # 64 output tiles: K split in chunks

    def fn():
        tq.tq_hadamard_quant_act(x, s, q, a)
        tq.tq_gemm(TB, M, N, K, W, q, a, y, ws)
    _replays_match(fn, [q, a, y])


def test_graph_workspace_clear_and_check():
    """The workspace helpers captured in a graph: a stale workspace (filled
    by a kernel inside the graph) is counted, cleared, and counted again as
    zero on every replay."""
    import ternary_weight_base_amd as tq
    say("graph workspace clear/check")
    words = 70000
    ws = torch.zeros(words, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    cnt2 = torch.zeros(1, dtype=torch.int32, device="cuda")

    def fn():
        ws.fill_(7)
        tq.tq_workspace_check(ws, cnt)
        tq.tq_workspace_clear(ws)
        tq.tq_workspace_check(ws, cnt2)
    _replays_match(fn, [cnt, cnt2, ws])
    assert int(cnt.item()) == words and int(cnt2.item()) == 0 and not ws.any().item()
