"""Bit-exact parity of the integer core in the kernels the product runs.

The group-sum hooks (tq_debug_group_sums, tq_debug_gate_up_sums,
tq_debug_gemv_quant_sums, tq_debug_gemv_quant_rows_sums) launch the very
kernel, plan and decode path of the matching product call -- the one-token
projection kernel in both activation forms, the MFMA GEMV for 2..16 tokens,
the GEMM with its 64/128/256-row tiles and K chunks, the fused quantiser of
the stack's launches and of the batch stack's 2..4-row launches -- with the scaling
replaced by a store of S[m][n][g] = sum_i t[n][128g+i] * q[m][128g+i].  Every
S is compared element by element with the oracle's plain int32 sum
(oracle.group_sums), at the 27B shapes and on ragged shapes.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import B3, B3R, BP, ONE_TOKEN_ONLY, TB, FMTS, acts_f16, dev, say, weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SENTINEL = 0x7FFFFFFF  # |S| <= 16256: never a sum


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.set_threads(8)
    yield
    _weights.cache_clear()
    _blob.cache_clear()
    torch.cuda.empty_cache()


def _tq():
    import ternary_weight_base_amd as tq
    return tq


@functools.lru_cache(maxsize=8)
def _weights(N, K, seed):
    return weights(N, K, seed)


@functools.lru_cache(maxsize=6)
def _blob(fmt, N, K, seed):
    return dev(_tq().tq_pack(fmt, *_weights(N, K, seed)))


def _int8_acts(M, K, seed):
    q, _ = oracle.quant(acts_f16(M, K, seed))
    return q


def _sums(M, N, K, nmat=1):
    return torch.full((nmat, M, N, K // 128), SENTINEL, dtype=torch.int32, device="cuda")


# The 27B decode shapes (N, K): QKV, O, down, and gate (one matrix: 272 row
# blocks, more workgroups than CUs -> the SGPR activation form), plus ragged
# shapes with a partial last block.
SHAPES = [(10240, 5120), (5120, 8192), (5120, 17408), (17408, 5120), (100, 640), (65, 384)]
# (format, tokens): BP and B3R run on the one-token kernel only
FMT_M = [(f, m) for f in (B3, TB, BP, B3R) for m in (1, 2, 4, 8, 16) if f not in ONE_TOKEN_ONLY or m == 1]


@pytest.mark.parametrize("fmt,M", FMT_M)
@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv_group_sums(fmt, M, N, K):
    say(f"gemv sums {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    seed = 7000 + N + K
    t, _ = _weights(N, K, seed)
    q = _int8_acts(M, K, 7100 + M + K)
    S = _sums(M, N, K)
    tq.tq_debug_group_sums(fmt, M, N, K, _blob(fmt, N, K, seed), dev(q), S, use_gemm_path=False)
    torch.cuda.synchronize()
    assert np.array_equal(S[0].cpu().numpy(), oracle.group_sums(t, q))


@pytest.mark.parametrize("fmt,M", FMT_M)
@pytest.mark.parametrize("N,K", [(17408, 5120), (20000, 640), (8192, 4096), (130, 640)])
def test_gate_up_group_sums(fmt, M, N, K):
    """The fused gate/up kernel: the equal item split over 256 workgroups
    (17408 and the ragged 20000 rows), K chunks (8192 rows), one block."""
    say(f"gate/up sums {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    tg, _ = _weights(N, K, 7200 + N)
    tu, _ = _weights(N, K, 7201 + N)
    q = _int8_acts(M, K, 7300 + M)
    S = _sums(M, N, K, nmat=2)
    tq.tq_debug_gate_up_sums(fmt, M, N, K, _blob(fmt, N, K, 7200 + N), _blob(fmt, N, K, 7201 + N),
                             dev(q), S)
    torch.cuda.synchronize()
    Sh = S.cpu().numpy()
    assert np.array_equal(Sh[0], oracle.group_sums(tg, q)), "gate"
    assert np.array_equal(Sh[1], oracle.group_sums(tu, q)), "up"


def _block_max(v):
    v = np.abs(np.asarray(v, dtype=np.float32).ravel())
    return v.reshape(-1, 64).max(axis=1)


# The decode stack's four launches: (N, K, input dtype, gate/up)
STACK_LAUNCHES = [(10240, 5120, "f16", False), (5120, 8192, "f16", False),
                  (17408, 5120, "f32", True), (5120, 17408, "f32", False), (1152, 640, "f32", True)]


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
@pytest.mark.parametrize("N,K,dtype,gate_up", STACK_LAUNCHES)
def test_gemv_quant_group_sums(fmt, N, K, dtype, gate_up):
    """The quantiser fused into the stack's projection launches: the int8
    codes it derives inside the launch (seen through S) and its activation
    scale equal the oracle quantiser's bit for bit."""
    say(f"gemv_quant sums {FMTS[fmt]} {N}x{K} {dtype} gate_up={gate_up}")
    tq = _tq()
    seed = 7400 + N + K
    x = synth.normal_f16(synth.seed(seed, 3), K)
    if dtype == "f32":  # an fp32 producer output: spread beyond the fp16 grid
        x = (x.astype(np.float32) * np.float32(3.3)
             + synth.normal_f32(synth.seed(seed, 4), K) * np.float32(1e-3)).astype(np.float32)
    xb = dev(_block_max(x)) if dtype == "f32" else None
    t, _ = _weights(N, K, seed)
    Wu, tu = None, None
    if gate_up:
        tu, _ = _weights(N, K, seed + 1)
        Wu = _blob(fmt, N, K, seed + 1)
    nmat = 2 if gate_up else 1
    S = torch.full((nmat, N, K // 128), SENTINEL, dtype=torch.int32, device="cuda")
    a = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_debug_gemv_quant_sums(fmt, N, K, _blob(fmt, N, K, seed), Wu, dev(x), S, x_bmax=xb, a_scale=a)
    torch.cuda.synchronize()
    q, sc = oracle.quant(x.reshape(1, K))
    assert a.cpu().numpy().view(np.uint32)[0] == sc.view(np.uint32)[0], "activation scale"
    Sh = S.cpu().numpy()
    assert np.array_equal(Sh[0], oracle.group_sums(t, q)[0])
    if gate_up:
        assert np.array_equal(Sh[1], oracle.group_sums(tu, q)[0])


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("rows", [2, 3, 4])
@pytest.mark.parametrize("N,K,dtype,gate_up", STACK_LAUNCHES)
def test_gemv_quant_rows_group_sums(fmt, rows, N, K, dtype, gate_up):
    """The batch stack's launches (tq_decode_stack_batch: each weight group
    decoded once and dotted with every token row): per row, the int8 codes
    the fused quantiser derives and the integer sums equal the oracle's bit
    for bit, and so does each row's activation scale.  One row is all zero
    (scale 0, every sum 0) when there are more than two."""
    say(f"gemv_quant rows sums {FMTS[fmt]} rows={rows} {N}x{K} {dtype} gate_up={gate_up}")
    tq = _tq()
    seed = 7700 + N + K + rows
    x = synth.normal_f16(synth.seed(seed, 3), rows, K)
    if dtype == "f32":
        x = (x.astype(np.float32) * np.float32(3.3)
             + synth.normal_f32(synth.seed(seed, 4), rows, K) * np.float32(1e-3)).astype(np.float32)
    if rows > 2:
        x[1] = 0
    xb = dev(np.stack([_block_max(x[r]) for r in range(rows)])) if dtype == "f32" else None
    t, _ = _weights(N, K, seed)
    Wu, tu = None, None
    if gate_up:
        tu, _ = _weights(N, K, seed + 1)
        Wu = _blob(fmt, N, K, seed + 1)
    nmat = 2 if gate_up else 1
    S = torch.full((nmat, rows, N, K // 128), SENTINEL, dtype=torch.int32, device="cuda")
    a = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_debug_gemv_quant_rows_sums(fmt, rows, N, K, _blob(fmt, N, K, seed), Wu, dev(x), S, x_bmax=xb,
                                     a_scale=a)
    torch.cuda.synchronize()
    q, sc = oracle.quant(x)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), sc.view(np.uint32)), "activation scales"
    Sh = S.cpu().numpy()
    ref = oracle.group_sums(t, q)  # [rows][N][G]
    for r in range(rows):
        assert np.array_equal(Sh[0, r], ref[r]), f"row {r}"
    if gate_up:
        refu = oracle.group_sums(tu, q)
        for r in range(rows):
            assert np.array_equal(Sh[1, r], refu[r]), f"up row {r}"
    if rows > 2:
        assert sc[1] == 0 and not Sh[:, 1].any()


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


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M", [5, 17, 64, 400, 512])
@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_gemm_group_sums(fmt, M, N, K):
    """The prefill GEMM's own plan: 64-row tiles with K chunks for M <= 64,
    128- or 256-row tiles (a ragged last tile at M = 400) above.  Every
    element is written (no sentinel left); the sums of token rows touching
    every 16-row stretch and every tile edge equal the oracle's over all N
    and all groups."""
    say(f"gemm sums {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    seed = 7500 + N
    t, _ = _weights(N, K, seed)
    q = _int8_acts(M, K, 7600 + M)
    S = _sums(M, N, K)
    tq.tq_debug_group_sums(fmt, M, N, K, _blob(fmt, N, K, seed), dev(q), S, use_gemm_path=True)
    torch.cuda.synchronize()
    assert not (S == SENTINEL).any().item(), "some group sum never written"
    rows = _tile_rows(M)
    got = S[0][torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got, oracle.group_sums(t, q[rows]))
    del S
    torch.cuda.empty_cache()


# ------------------------------------------------------------ edge values ---

def _edge_weights(N, K, seed):
    """Trits with whole groups of +1 and of -1 (so |S| reaches 127 * 128 =
    16256 against +-127 activations) mixed with random groups, and fp16
    scales covering zero, negative, subnormal and the largest finite value."""
    t, s = weights(N, K, seed)
    G = K // 128
    t = t.reshape(N, G, 128)
    t[0::3, 0::2] = 1
    t[1::3, 1::2] = -1
    t = t.reshape(N, K)
    s = s.copy()
    special = np.array([0x0000, 0x8000, 0x0001, 0x83FF, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00, 0x0400],
                       dtype=np.uint16)  # +-0, subnormals, +-65504, +-1, the smallest normal
    s.flat[::7] = special[np.arange(s.flat[::7].size) % special.size]
    return t, s


def _edge_acts(M, K, seed):
    """int8 activations at the extremes: +-127 everywhere, with random rows mixed in."""
    rng = np.random.default_rng(seed)
    q = np.where(rng.random((M, K)) < 0.5, 127, -127).astype(np.int8)
    q[0] = 127
    if M > 1:
        q[1] = -127
    if M > 2:
        q[2] = _int8_acts(1, K, seed)[0]
    return q


@pytest.mark.parametrize("fmt,M", [(f, m) for f in (B3, TB, BP, B3R) for m in (1, 3, 16)
                                   if f not in ONE_TOKEN_ONLY or m == 1])
@pytest.mark.parametrize("N,K", [(200, 1024), (5120, 8192)])
def test_edge_values_gemv(fmt, M, N, K):
    """Extreme sums and special scales through tq_gemv: the int32 sums are
    bit-exact and the fp32 outputs within tolerance."""
    from gpu_util import assert_close
    say(f"edge gemv {FMTS[fmt]} M={M} N={N} K={K}")
    tq = _tq()
    t, s = _edge_weights(N, K, 7700 + N)
    q = _edge_acts(M, K, 7800 + M)
    a = np.linspace(0.5, 2.0, M).astype(np.float32)
    W = dev(tq.tq_pack(fmt, t, s))
    S = _sums(M, N, K)
    tq.tq_debug_group_sums(fmt, M, N, K, W, dev(q), S, use_gemm_path=False)
    y = torch.full((M, N), float("nan"), device="cuda")
    tq.tq_gemv(fmt, M, N, K, W, dev(q), dev(a), y, tq.workspace(fmt, M, N, K))
    torch.cuda.synchronize()
    S_ref = oracle.group_sums(t, q)
    assert np.abs(S_ref).max() == 16256
    assert np.array_equal(S[0].cpu().numpy(), S_ref)
    assert_close(y.cpu().numpy(), oracle.gemv(t, s, q, a), "edge gemv")


@pytest.mark.parametrize("fmt", [B3, TB])
@pytest.mark.parametrize("M", [40, 300])
def test_edge_values_gemm(fmt, M):
    from gpu_util import assert_close
    N, K = 1000, 2048
    say(f"edge gemm {FMTS[fmt]} M={M}")
    tq = _tq()
    t, s = _edge_weights(N, K, 7900)
    q = _edge_acts(M, K, 7901)
    a = np.linspace(0.5, 2.0, M).astype(np.float32)
    W = dev(tq.tq_pack(fmt, t, s))
    S = _sums(M, N, K)
    tq.tq_debug_group_sums(fmt, M, N, K, W, dev(q), S, use_gemm_path=True)
    y = torch.full((M, N), float("nan"), device="cuda")
    tq.tq_gemm(fmt, M, N, K, W, dev(q), dev(a), y, tq.workspace(fmt, M, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(S[0].cpu().numpy(), oracle.group_sums(t, q))
    assert_close(y.cpu().numpy(), oracle.gemv(t, s, q, a), "edge gemm")


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
def test_edge_values_gate_up(fmt):
    from gpu_util import assert_close
    N, K = 17408, 5120
    say(f"edge gate/up {FMTS[fmt]}")
    tq = _tq()
    tg, sg = _edge_weights(N, K, 8000)
    tu, su = _edge_weights(N, K, 8001)
    q = _edge_acts(1, K, 8002)
    a = np.array([1e-3], np.float32)  # keeps silu's argument and the product finite
    Wg, Wu = dev(tq.tq_pack(fmt, tg, sg)), dev(tq.tq_pack(fmt, tu, su))
    h = torch.full((1, N), float("nan"), device="cuda")
    tq.tq_gemv_gate_up_swiglu(fmt, 1, N, K, Wg, Wu, dev(q), dev(a), h, tq.workspace(fmt, 1, N, K))
    torch.cuda.synchronize()
    ref = oracle.swiglu(oracle.gemv(tg, sg, q, a), oracle.gemv(tu, su, q, a))
    assert_close(h.cpu().numpy(), ref, "edge gate/up")
