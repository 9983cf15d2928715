"""GPU parity of the batch decode stack (tq_decode_stack_batch: 1..4 token
rows per launch).  Each row must equal, bit for bit, tq_decode_stack run on
that row alone (same plans, quantiser, integer core, fp32 order and meets;
only the weight groups are shared between the rows), and each stage is
checked against the oracle on the GPU's own input of that stage
(stage-isolated, as in the one-token stack tests)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import B3, TB, FMTS, assert_close, dev, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)


def _weights(fmt, L, hidden, inter, qkv_out, o_in, seed):
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
    return host, devw


def _outs(L, R, dims):
    return [torch.full((L, R, n), float("nan"), device="cuda") for n in dims]


def _run(fmt, R, L, hidden, inter, qkv_out, o_in, seed, zero_rows=(), signs=None):
    """Runs the batch stack (twice: the workspace must come back ready) and,
    per row, the one-token stack; asserts bit identity.  Returns the host
    weights, the inputs and the batch outputs as numpy [L][R][N]."""
    import ternary_weight_base_amd as tq
    host, devw = _weights(fmt, L, hidden, inter, qkv_out, o_in, seed)
    x = synth.normal_f16(synth.seed(seed, 99, 1), L, R, hidden)
    a = synth.normal_f16(synth.seed(seed, 99, 2), L, R, o_in)
    for r in zero_rows:  # absmax 0 all along the row's chain
        x[:, r] = 0
        a[:, r] = 0
    dims = (qkv_out, hidden, inter, hidden)
    sg = None if signs is None else dev(signs)
    nbytes = tq.tq_decode_stack_batch_workspace_bytes(fmt, R, L, hidden, inter, qkv_out, o_in)
    assert nbytes >= tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws = torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    xd, ad = dev(x), dev(a)
    runs = []
    for rep in range(2):
        outs = _outs(L, R, dims)
        tq.tq_decode_stack_batch(fmt, R, L, hidden, inter, qkv_out, o_in, devw, xd, ad, *outs, ws,
                                 ffn_signs=sg)
        torch.cuda.synchronize()
        runs.append([t.cpu().numpy() for t in outs])
        r256 = lambda n: (n + 255) // 256 * 256
        keep = r256(R * ((hidden + 63) // 64) * 4) + r256(R * ((inter + 63) // 64) * 4)
        assert not ws[:(nbytes - keep) // 4].any().item(), "workspace not left zero"
    for u, v in zip(*runs):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), "not deterministic"
    batch = runs[0]
    # each row alone through the one-token stack
    nb1 = tq.tq_decode_stack_workspace_bytes(fmt, L, hidden, inter, qkv_out, o_in)
    ws1 = torch.zeros((nb1 + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    for r in range(R):
        one = [torch.full((L, n), float("nan"), device="cuda") for n in dims]
        tq.tq_decode_stack(fmt, L, hidden, inter, qkv_out, o_in, devw, dev(x[:, r].copy()),
                           dev(a[:, r].copy()), *one, ws1, ffn_signs=sg)
        torch.cuda.synchronize()
        for name, u, v in zip(("y_qkv", "y_o", "h", "y_out"), batch, one):
            assert np.array_equal(u[:, r].view(np.uint32), v.cpu().numpy().view(np.uint32)), \
                f"row {r} {name} differs from the one-token stack"
    return host, x, a, batch


def _check(host, x, a, batch, rows, what, signs=None):
    """Stage-isolated oracle checks of the listed (layer, row) pairs."""
    y_qkv, y_o, h, y_out = batch
    for l, r in rows:
        hw = host[l]
        q, s = oracle.quant(x[l, r:r + 1])
        assert_close(y_qkv[l, r:r + 1], oracle.gemv(*hw["qkv"], q, s), f"{what} qkv[{l},{r}]")
        q, s = oracle.quant(a[l, r:r + 1])
        yo_ref = oracle.gemv(*hw["o"], q, s)
        if signs is not None:
            yo_ref = oracle.hadamard(yo_ref, signs[l])
        assert_close(y_o[l, r:r + 1], yo_ref, f"{what} o[{l},{r}]")
        q, s = oracle.quant(y_o[l, r:r + 1])  # the GPU's y_o
        h_ref = oracle.swiglu(oracle.gemv(*hw["gate"], q, s), oracle.gemv(*hw["up"], q, s))
        assert_close(h[l, r:r + 1], h_ref, f"{what} h[{l},{r}]")
        q, s = oracle.quant(h[l, r:r + 1])  # the GPU's h
        assert_close(y_out[l, r:r + 1], oracle.gemv(*hw["down"], q, s), f"{what} down[{l},{r}]")


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_batch_small(fmt, R):
    """Small layers (QKV 1280 rows = 20 blocks, gate/up 1152 = 18 blocks,
    K chunks met by exchange), rows 1..4 (1: the one-token kernels)."""
    say(f"batch stack {FMTS[fmt]} R={R} small")
    host, x, a, out = _run(fmt, R, 2, 640, 1152, 1280, 1024, 100 + R)
    _check(host, x, a, out, [(l, r) for l in range(2) for r in range(R)], f"R={R}")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_batch_ragged_and_other_shapes(fmt):
    """A ragged last row block (QKV N = 1000: 15 blocks and 40 rows) and
    the second small layer shape."""
    say(f"batch stack {FMTS[fmt]} R=3 ragged")
    host, x, a, out = _run(fmt, 3, 2, 384, 2176, 1000, 768, 131)
    _check(host, x, a, out, [(0, 0), (1, 2)], "ragged")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_batch_split_k_everywhere(fmt):
    """Every stage splits K over workgroups; the split-K meets of the rows
    share the block counters."""
    say(f"batch stack {FMTS[fmt]} R=4 split-K")
    host, x, a, out = _run(fmt, 4, 2, 2048, 5120, 1024, 2048, 141)
    _check(host, x, a, out, [(0, 3), (1, 1)], "splitk")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_batch_full_shapes(fmt):
    """The 27B-shaped layer (hidden 5120, intermediate 17408, QKV 10240,
    O 8192) with 4 rows: gate/up on the equal split (exchange meet with
    two pieces per cut block), the others on K chunks."""
    say(f"batch stack {FMTS[fmt]} R=4 full shapes")
    host, x, a, out = _run(fmt, 4, 1, 5120, 17408, 10240, 8192, 151)
    _check(host, x, a, out, [(0, 0), (0, 3)], "full")


@pytest.mark.parametrize("fmt", [B3, TB])
def test_batch_ffn_rotation(fmt):
    """FFN input rotated online in O's epilogue (counter meet), 3 rows."""
    say(f"batch stack {FMTS[fmt]} R=3 rotation")
    L, hidden = 2, 640
    signs = synth.signs(synth.seed(161, 1), L * hidden).reshape(L, hidden)
    host, x, a, out = _run(fmt, 3, L, hidden, 1152, 1280, 1024, 161, signs=signs)
    _check(host, x, a, out, [(0, 1), (1, 2)], "rotation", signs=signs)


def test_batch_zero_row_and_long_rows():
    """A row of zeros between live rows (its scale 0, every output 0, the
    neighbours untouched); fp16 input longer than one absmax pass (o_in 9216)
    and 322 row blocks of h."""
    say("batch stack zero row + long rows")
    host, x, a, out = _run(B3, 3, 1, 256, 20608, 384, 9216, 171, zero_rows=(1,))
    for t in out:
        assert np.all(t[:, 1] == 0)
    _check(host, x, a, out, [(0, 0), (0, 2)], "long")
