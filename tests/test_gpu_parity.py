"""GPU parity: every HIP entry point against the CPU oracle, through the C ABI.

Bit-exact: decoded trits, int8 activations and their scales, int32 group
sums.  fp32 outputs: max abs err <= 1e-3 * max|y_ref| and relative L2 <= 1e-5.
Sizes span several tiles with ragged tails, plus the full benchmark shapes.
"""
import numpy as np
import pytest

import oracle
from gpu_util import B3, B3R, BP, TB, FMTS, ONE_TOKEN_ONLY, acts_f16, assert_close, dev, say, upload_blob, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)
    yield


def _tq():
    import ternary_weight_base_amd as tq
    return tq


def _quant_gpu(x_np):
    tq = _tq()
    M, K = x_np.shape
    x = dev(x_np)
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    tq.tq_quant_act(x, q, a)
    torch.cuda.synchronize()
    return q, a


# ------------------------------------------------------------- quantiser ---

@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 128), (1, 1024), (3, 5120), (16, 8192), (2, 17408), (512, 5120)])
def test_quant_bitexact(dtype, M, K):
    say(f"quant {dtype} M={M} K={K}")
    x = acts_f16(M, K, 1000 + M * 3 + K)
    if dtype == "f32":
        x = (x.astype(np.float32) * np.float32(3.7)).astype(np.float32)
    q, a = _quant_gpu(x)
    qr, ar = oracle.quant(x)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), ar.view(np.uint32))


def test_quant_special_rows():
    K = 256
    x = np.zeros((5, K), np.float32)
    x[1, :4] = [1.0, -0.5, 0.25, 0.0]       # a tie at -63.5
    x[2, :2] = [2.0, 1.0]                    # a tie at 63.5
    x[3] = np.linspace(-3, 3, K, dtype=np.float32)
    x[4, 7] = -1e-30                         # tiny but fine (127/a finite)
    for arr in (x, x.astype(np.float16)):
        say(f"quant special {arr.dtype}")
        q, a = _quant_gpu(arr)
        qr, ar = oracle.quant(arr)
        assert np.array_equal(q.cpu().numpy(), qr)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), ar.view(np.uint32))


# --------------------------------------------------------------- decoder ---

@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
@pytest.mark.parametrize("N,K", [(1, 128), (64, 1024), (65, 384), (100, 640), (1024, 1024), (300, 5120)])
def test_debug_unpack_bitexact(fmt, N, K):
    say(f"unpack {FMTS[fmt]} N={N} K={K}")
    tq = _tq()
    t, s = weights(N, K, 2000 + N + K)
    W = upload_blob(fmt, t, s)
    out = torch.full((N, K), 7, dtype=torch.int8, device="cuda")
    tq.tq_debug_unpack(fmt, N, K, W, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), t)


# ------------------------------------------------------------ group sums ---

@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("N,K", [(100, 640), (1024, 1024), (130, 17408)])
def test_group_sums_gemv_bitexact(fmt, M, N, K):
    say(f"sums gemv {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    t, s = weights(N, K, 3000 + N + K)
    x = acts_f16(M, K, 3100 + M)
    qr, _ = oracle.quant(x)
    W = upload_blob(fmt, t, s)
    S = torch.full((M, N, K // 128), 12345, dtype=torch.int32, device="cuda")
    tq.tq_debug_group_sums(fmt, M, N, K, W, dev(qr), S, use_gemm_path=False)
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), oracle.group_sums(t, qr))


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M", [1, 17, 130, 512])
def test_group_sums_gemm_bitexact(fmt, M):
    N, K = 130, 640
    say(f"sums gemm {FMTS[fmt]} M={M}")
    tq = _tq()
    t, s = weights(N, K, 3500 + M)
    x = acts_f16(M, K, 3600 + M)
    qr, _ = oracle.quant(x)
    W = upload_blob(fmt, t, s)
    S = torch.full((M, N, K // 128), 12345, dtype=torch.int32, device="cuda")
    tq.tq_debug_group_sums(fmt, M, N, K, W, dev(qr), S, use_gemm_path=True)
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), oracle.group_sums(t, qr))


# ------------------------------------------------------------------ GEMV ---

def _gemv_gpu(fmt, M, N, K, W, q, a):
    tq = _tq()
    ws = tq.workspace(fmt, M, N, K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_gemv(fmt, M, N, K, W, q, a, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ws


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 1024, 1024), (1, 65, 384), (3, 100, 640),
                                   (1, 10240, 5120), (1, 5120, 8192), (1, 5120, 17408),
                                   (2, 5120, 17408), (4, 1000, 2048), (8, 257, 1024),
                                   (16, 300, 5120), (8, 5120, 17408), (16, 10240, 5120),
                                   (2, 5120, 8192), (4, 5120, 8192), (16, 5120, 8192),
                                   (4, 10240, 5120), (4, 5120, 17408),
                                   (1, 8192, 4096), (1, 4096, 8192), (1, 4136, 8192), (1, 2048, 8192),
                                   (1, 20000, 640)])
def test_gemv_vs_oracle(fmt, M, N, K):
    """One token: the K-chunk splits meet by exchange (2 chunks at 8192 rows,
    a full two-level tree of 4 at 4096, 3 with a ragged 40-row tail block at
    4136) or through the counter (8 chunks at 2048 rows); 20000 rows take 313
    workgroups, more than one per CU (B3: the SGPR activation form)."""
    say(f"gemv {FMTS[fmt]} M={M} N={N} K={K}")
    t, s = weights(N, K, 4000 + N + K)
    x = acts_f16(M, K, 4100 + M + K)
    q, a = _quant_gpu(x)
    qn, an = q.cpu().numpy(), a.cpu().numpy()
    W = upload_blob(fmt, t, s)
    y, ws = _gemv_gpu(fmt, M, N, K, W, q, a)
    assert_close(y, oracle.gemv(t, s, qn, an), f"gemv {FMTS[fmt]} {M}x{N}x{K}")
    if ws is not None:  # the whole workspace is handed back zeroed for the next call
        assert not ws.any().item()


@pytest.mark.parametrize("fmt", ONE_TOKEN_ONLY)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 65, 384), (1, 1024, 1024), (1, 10240, 5120),
                                   (1, 5120, 8192), (1, 5120, 17408)])
def test_gemv_one_token_layouts(fmt, M, N, K):
    """The bit-plane layout (BP) and the row-major B3 groups (B3R) on the
    one-token projection kernel."""
    say(f"gemv {FMTS[fmt]} N={N} K={K}")
    t, s = weights(N, K, 4300 + N + K)
    q, a = _quant_gpu(acts_f16(M, K, 4400 + K))
    W = upload_blob(fmt, t, s)
    y, _ = _gemv_gpu(fmt, M, N, K, W, q, a)
    assert_close(y, oracle.gemv(t, s, q.cpu().numpy(), a.cpu().numpy()), f"gemv {FMTS[fmt]} {N}x{K}")


@pytest.mark.parametrize("fmt", ONE_TOKEN_ONLY)
@pytest.mark.parametrize("N,K", [(17408, 5120), (130, 640)])
def test_gate_up_swiglu_one_token_layouts(fmt, N, K):
    say(f"swiglu {FMTS[fmt]} N={N} K={K}")
    tq = _tq()
    BP = fmt
    tg, sg = weights(N, K, 4500 + N)
    tu, su = weights(N, K, 4501 + N)
    q, a = _quant_gpu(acts_f16(1, K, 4600))
    qn, an = q.cpu().numpy(), a.cpu().numpy()
    h = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_gemv_gate_up_swiglu(BP, 1, N, K, upload_blob(BP, tg, sg), upload_blob(BP, tu, su), q, a, h,
                              tq.workspace(BP, 1, N, K))
    torch.cuda.synchronize()
    ref = oracle.swiglu(oracle.gemv(tg, sg, qn, an), oracle.gemv(tu, su, qn, an))
    assert_close(h.cpu().numpy(), ref, f"swiglu {FMTS[fmt]}")


def test_gemv_zero_weights_and_zero_activations():
    tq = _tq()
    N, K = 70, 512
    for fmt in (B3, TB):
        say(f"gemv zeros {FMTS[fmt]}")
        t = np.zeros((N, K), np.int8)
        s = np.full((N, K // 128), 0x3C00, np.uint16)
        W = upload_blob(fmt, t, s)
        q, a = _quant_gpu(acts_f16(2, K, 5))
        y, _ = _gemv_gpu(fmt, 2, N, K, W, q, a)
        assert np.all(y == 0)
        t, s = weights(N, K, 6)
        W = upload_blob(fmt, t, s)
        q, a = _quant_gpu(np.zeros((1, K), np.float16))
        y, _ = _gemv_gpu(fmt, 1, N, K, W, q, a)
        assert np.all(y == 0)


def test_gemv_deterministic_across_runs():
    tq = _tq()
    N, K = 5120, 17408
    t, s = weights(N, K, 4444)
    W = upload_blob(B3, t, s)
    q, a = _quant_gpu(acts_f16(1, K, 4445))
    say("gemv determinism")
    y1, _ = _gemv_gpu(B3, 1, N, K, W, q, a)
    y2, _ = _gemv_gpu(B3, 1, N, K, W, q, a)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    q, a = _quant_gpu(acts_f16(8, K, 4446))  # several tokens: the MFMA path
    y1, _ = _gemv_gpu(B3, 8, N, K, W, q, a)
    y2, _ = _gemv_gpu(B3, 8, N, K, W, q, a)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# ------------------------------------------------------ fused gate/up -----

@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M,N,K", [(1, 17408, 5120), (1, 130, 640), (4, 1000, 1024), (16, 200, 2048),
                                   (8, 17408, 5120), (1, 20000, 640), (1, 30000, 1024), (1, 16448, 128),
                                   (1, 8192, 4096), (1, 12800, 2048)])
def test_gate_up_swiglu_vs_oracle(fmt, M, N, K):
    """One token with 257..512 row blocks takes the equal item split over
    256 workgroups, whose ranges cross blocks (ragged 20000 rows, 5 and 8
    groups per row; 257 blocks of one group); with fewer blocks K is cut
    into chunks (4 at 8192 rows, 2 at 12800) that meet by exchange."""
    say(f"swiglu {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    tg, sg = weights(N, K, 5000 + N)
    tu, su = weights(N, K, 5001 + N)
    q, a = _quant_gpu(acts_f16(M, K, 5100 + M))
    qn, an = q.cpu().numpy(), a.cpu().numpy()
    Wg, Wu = upload_blob(fmt, tg, sg), upload_blob(fmt, tu, su)
    ws = tq.workspace(fmt, M, N, K)
    h = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_gemv_gate_up_swiglu(fmt, M, N, K, Wg, Wu, q, a, h, ws)
    torch.cuda.synchronize()
    ref = oracle.swiglu(oracle.gemv(tg, sg, qn, an), oracle.gemv(tu, su, qn, an))
    assert_close(h.cpu().numpy(), ref, "swiglu")
    if ws is not None:
        assert not ws.any().item()


# ------------------------------------------------------------------ GEMM ---

@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M,N,K", [(17, 130, 640), (40, 1000, 5120), (200, 64, 1024), (512, 1000, 5120)])
def test_gemm_vs_oracle(fmt, M, N, K):
    say(f"gemm {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    t, s = weights(N, K, 6000 + M + N)
    q, a = _quant_gpu(acts_f16(M, K, 6100 + M))
    W = upload_blob(fmt, t, s)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_gemm(fmt, M, N, K, W, q, a, y, tq.workspace(fmt, M, N, K))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.gemv(t, s, q.cpu().numpy(), a.cpu().numpy()), "gemm")


def _tile_rows(M):
    """Token rows that touch every 16-row token tile (one row of each, at a
    position that moves from tile to tile) and the edges of every 64-row
    stretch."""
    rows = {0, 15, 16, 63, M - 1}
    for t in range((M + 15) // 16):
        rows.add(16 * t + (7 * t) % 16)
    for edge in range(64, M, 64):
        rows |= {edge - 1, edge}
    return np.array(sorted(r for r in rows if 0 <= r < M))


def _gemm_full_check(fmt, M, N, K, seed):
    """y prefilled with NaN: every element must be written (all finite), and
    the token rows touching every token tile match the oracle over all N
    output columns."""
    tq = _tq()
    t, s = weights(N, K, seed)
    q, a = _quant_gpu(acts_f16(M, K, seed + 100))
    W = upload_blob(fmt, t, s)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = tq.workspace(fmt, M, N, K)
    tq.tq_gemm(fmt, M, N, K, W, q, a, y, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all().item(), "some output element never written"
    rows = _tile_rows(M)
    qn, an = q.cpu().numpy(), a.cpu().numpy()
    ref = oracle.gemv(t, s, qn[rows], an[rows])
    assert_close(y.cpu().numpy()[rows], ref, f"gemm {FMTS[fmt]} {M}x{N}x{K}")
    if ws is not None:
        assert not ws.any().item()


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M,N,K", [(330, 5120, 17408), (400, 5120, 17408), (512, 14336, 1024)])
def test_gemm_wide_tile_full(fmt, M, N, K):
    """256-token tiles with a ragged last tile and a 3-way K split (M = 400),
    128-token tiles with a 3-way split (M = 330), and 448 256-token tiles
    with no split (short K)."""
    say(f"gemm wide {FMTS[fmt]} M={M} N={N} K={K}")
    _gemm_full_check(fmt, M, N, K, 6700 + M)


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_gemm_prefill_full_size(fmt, N, K):
    """The prefill shapes at full size (M = 512)."""
    say(f"gemm full {FMTS[fmt]} N={N} K={K}")
    _gemm_full_check(fmt, 512, N, K, 6500 + N)


# ------------------------------------------- ternariser -> pack -> GPU -----

@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
def test_ternarize_pack_gpu_end_to_end(fmt):
    """fp32 weights -> tq_ternarize (host) -> tq_pack -> GPU projections,
    against oracle.ternarize -> oracle.gemv: trits and scales bit-identical,
    outputs within tolerance (one token, the fused gate/up, 4 tokens, and a
    64-token GEMM)."""
    import synth
    tq = _tq()
    N, K = 5120, 8192
    say(f"ternarize e2e {FMTS[fmt]}")
    w = synth.normal_f32(synth.seed(8100, 1), N, K)
    w[::5] *= np.float32(0.02)   # rows of small weights: scales near the fp16 subnormal range
    t, s = tq.tq_ternarize(w)
    tr, sr = oracle.ternarize(w)
    assert np.array_equal(t, tr) and np.array_equal(s, sr)
    W = upload_blob(fmt, t, s)
    Ms = (1,) if fmt in ONE_TOKEN_ONLY else (1, 4, 64)
    for M in Ms:
        q, a = _quant_gpu(acts_f16(M, K, 8200 + M))
        qn, an = q.cpu().numpy(), a.cpu().numpy()
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_gemm(fmt, M, N, K, W, q, a, y, tq.workspace(fmt, M, N, K)) if M > 1 else \
            tq.tq_gemv(fmt, M, N, K, W, q, a, y, tq.workspace(fmt, M, N, K))
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), oracle.gemv(tr, sr, qn, an), f"ternarised M={M}")
    # gate/up from two ternarised matrices on one shared input
    wu = synth.normal_f32(synth.seed(8100, 2), N, K)
    tu, su = tq.tq_ternarize(wu)
    tur, sur = oracle.ternarize(wu)
    assert np.array_equal(tu, tur) and np.array_equal(su, sur)
    q, a = _quant_gpu(acts_f16(1, K, 8300))
    qn, an = q.cpu().numpy(), a.cpu().numpy()
    h = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_gemv_gate_up_swiglu(fmt, 1, N, K, W, upload_blob(fmt, tu, su), q, a, h,
                              tq.workspace(fmt, 1, N, K))
    torch.cuda.synchronize()
    ref = oracle.swiglu(oracle.gemv(tr, sr, qn, an), oracle.gemv(tur, sur, qn, an))
    assert_close(h.cpu().numpy(), ref, "ternarised gate/up")
