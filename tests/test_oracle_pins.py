"""Pins for the CPU oracle: closed forms, hand-worked examples, brute force and
library routines (numpy / torch), never the oracle checked against itself.

Each group of tests names the definition it pins.  Hand-worked values live in
tests/golden/hand_examples.json; the pages' own size figures in
tests/golden/pages_sizes.json.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
B3, TB, BP = oracle.FMT_B3, oracle.FMT_2B, oracle.FMT_BP


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _one_group(trits_head, fill=0, fmt=B3):
    """A 1x128 row whose first trits are given, rest `fill`; scale 1.0."""
    t = np.full((1, 128), fill, dtype=np.int8)
    t[0, : len(trits_head)] = trits_head
    s = np.array([[0x3C00]], dtype=np.uint16)
    return t, s


# ---------------------------------------------------------------- fp16 ----

def test_half_to_float_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_synth_f16_rounding_matches_numpy():
    rng = np.random.default_rng(5)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                           [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26]])
    for v in vals:
        assert synth.f16_bits(v) == int(np.array([v]).astype(np.float16).view(np.uint16)[0]), v


# ---------------------------------------------------------------- B3 ------

def test_b3_hand_bytes():
    g = _gold("hand_examples.json")
    for ex in g["b3_bytes"]:
        t, s = _one_group(ex["trits"])
        blob = oracle.pack(B3, t, s)
        assert blob[0] == ex["byte"], ex
    for ex in g["b3_tail_bytes"]:
        t = np.zeros((1, 128), dtype=np.int8)
        t[0, 125:] = ex["trits"]
        blob = oracle.pack(B3, t, np.array([[0x3C00]], dtype=np.uint16))
        assert blob[25] == ex["byte"], ex


def test_b3_closed_form_groups():
    for fill, body, tail in ((0, 121, 121), (1, 242, 134), (-1, 0, 108)):
        t = np.full((1, 128), fill, dtype=np.int8)
        blob = oracle.pack(B3, t, np.array([[0x3C00]], dtype=np.uint16))
        assert list(blob[:25]) == [body] * 25 and blob[25] == tail
        assert list(blob[26:28]) == [0x00, 0x3C]  # scale, little-endian


def test_b3_all_243_patterns_vs_python_base3():
    """Every 5-trit pattern, at the first and at the last full byte of a group,
    equals Python's int(str, 3) of the digits written most-significant first."""
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T
    seen = set()
    for p in pats:
        expect = int("".join(str(d + 1) for d in p[::-1]), 3)
        for j in (0, 24):
            t = np.zeros((1, 128), dtype=np.int8)
            t[0, 5 * j: 5 * j + 5] = p
            blob = oracle.pack(B3, t, np.array([[0x3C00]], dtype=np.uint16))
            assert blob[j] == expect
        seen.add(expect)
    assert seen == set(range(243))  # a bijection onto 0..242


def test_b3_all_27_tail_patterns():
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 3, indexing="ij")).reshape(3, -1).T
    for p in pats:
        t = np.zeros((1, 128), dtype=np.int8)
        t[0, 125:] = p
        blob = oracle.pack(B3, t, np.array([[0x3C00]], dtype=np.uint16))
        assert blob[25] == int("11" + "".join(str(d + 1) for d in p[::-1]), 3)


def test_b3_every_byte_value_roundtrip_and_rejects():
    for v in range(256):
        for j in (0, 13, 24, 25):
            blob = oracle.pack(B3, np.zeros((1, 128), np.int8), np.array([[0x3C00]], np.uint16))
            blob[j] = v
            rc, t, s = oracle.unpack(B3, blob, 1, 128)
            if j < 25:
                valid = v < 243
            else:
                valid = v < 243 and (v // 27) % 3 == 1 and v // 81 == 1
            assert (rc == 0) == valid, (v, j, rc)
            if valid:
                assert np.array_equal(oracle.pack(B3, t, s), blob)


def test_b3_random_roundtrip_and_layout():
    N, K = 7, 640
    t = synth.trits(synth.seed(91), N, K)
    s = synth.scales(synth.seed(92), N, K)
    blob = oracle.pack(B3, t, s)
    G = K // 128
    assert blob.size == N * G * 28 == oracle.packed_bytes(B3, N, K)
    rc, t2, s2 = oracle.unpack(B3, blob, N, K)
    assert rc == 0 and np.array_equal(t, t2) and np.array_equal(s, s2)
    # scale region: [N][G] little-endian after the trit region
    assert np.array_equal(blob[N * G * 26:].view(np.uint16).reshape(N, G), s)
    # group (n, g) owns bytes (n*G+g)*26: re-pack one group alone and compare
    n, g = 5, 3
    one = oracle.pack(B3, np.ascontiguousarray(t[n: n + 1, 128 * g: 128 * g + 128]),
                      s[n: n + 1, g: g + 1])
    assert np.array_equal(blob[(n * G + g) * 26:(n * G + g + 1) * 26], one[:26])


def test_pack_rejects_bad_inputs():
    t = np.zeros((2, 256), np.int8)
    s = np.full((2, 2), 0x3C00, np.uint16)
    bad = t.copy()
    bad[1, 7] = 2
    for fmt in (B3, TB, BP):
        with pytest.raises(oracle.OracleError):
            oracle.pack(fmt, bad, s)
        for nonfinite in (0x7C00, 0xFC00, 0x7E00):
            s2 = s.copy()
            s2[0, 1] = nonfinite
            with pytest.raises(oracle.OracleError):
                oracle.pack(fmt, t, s2)
        with pytest.raises(oracle.OracleError):
            oracle.pack(fmt, np.zeros((1, 200), np.int8), np.zeros((1, 1), np.uint16))
    assert oracle.packed_bytes(B3, 1, 100) == 0 and oracle.packed_bytes(TB, 0, 128) == 0


# ---------------------------------------------------------------- 2B ------

def test_2b_hand_and_all_81_bytes():
    for ex in _gold("hand_examples.json")["twobit_bytes"]:
        t, s = _one_group(ex["trits"])
        assert oracle.pack(TB, t, s)[0] == ex["byte"]
    for fill, byte in ((0, 0x55), (1, 0xAA), (-1, 0x00)):
        blob = oracle.pack(TB, np.full((1, 128), fill, np.int8), np.array([[0x3C00]], np.uint16))
        assert list(blob[:32]) == [byte] * 32
    valid = 0
    for v in range(256):
        blob = oracle.pack(TB, np.zeros((1, 128), np.int8), np.array([[0x3C00]], np.uint16))
        blob[9] = v
        rc, t, _ = oracle.unpack(TB, blob, 1, 128)
        fields = [(v >> (2 * i)) & 3 for i in range(4)]
        assert (rc == 0) == (3 not in fields)
        if rc == 0:
            valid += 1
            assert list(t[0, 36:40]) == [f - 1 for f in fields]
    assert valid == 81


def test_2b_random_roundtrip():
    N, K = 5, 384
    t = synth.trits(synth.seed(93), N, K)
    s = synth.scales(synth.seed(94), N, K)
    blob = oracle.pack(TB, t, s)
    assert blob.size == N * 3 * 34
    rc, t2, s2 = oracle.unpack(TB, blob, N, K)
    assert rc == 0 and np.array_equal(t, t2) and np.array_equal(s, s2)


# ---------------------------------------------------------------- BP ------

def test_bp_bit_positions_and_fills():
    """Trit k of a group: nonzero plane byte k // 8, bit k % 8; the sign
    plane 16 bytes later; fills of 0, +1 and -1."""
    s1 = np.array([[0x3C00]], np.uint16)
    for k in (0, 1, 7, 8, 63, 100, 127):
        for v in (1, -1):
            t = np.zeros((1, 128), np.int8)
            t[0, k] = v
            blob = oracle.pack(BP, t, s1)
            ref = np.zeros(32, np.uint8)
            ref[k // 8] = 1 << (k % 8)
            if v < 0:
                ref[16 + k // 8] = 1 << (k % 8)
            assert np.array_equal(blob[:32], ref), (k, v)
    for fill, nz, sg in ((0, 0x00, 0x00), (1, 0xFF, 0x00), (-1, 0xFF, 0xFF)):
        blob = oracle.pack(BP, np.full((1, 128), fill, np.int8), s1)
        assert list(blob[:16]) == [nz] * 16 and list(blob[16:32]) == [sg] * 16
    assert list(oracle.pack(BP, np.zeros((1, 128), np.int8), s1)[32:34]) == [0x00, 0x3C]


def test_bp_all_byte_pairs():
    """Every (nonzero, sign) byte pair: accepted exactly when no sign bit
    sits on a zero trit (3^8 = 6561 pairs), decoded bit by bit."""
    s1 = np.array([[0x3C00]], np.uint16)
    base = oracle.pack(BP, np.zeros((1, 128), np.int8), s1)
    valid = 0
    for nz in range(256):
        for sg in range(256):
            blob = base.copy()
            blob[5], blob[21] = nz, sg
            rc, t, _ = oracle.unpack(BP, blob, 1, 128)
            ok = (sg & ~nz) == 0
            assert (rc == 0) == ok
            if ok:
                valid += 1
                ref = [(-1 if (sg >> i) & 1 else 1) if (nz >> i) & 1 else 0 for i in range(8)]
                assert list(t[0, 40:48]) == ref
    assert valid == 6561


def test_bp_random_roundtrip():
    N, K = 5, 384
    t = synth.trits(synth.seed(95), N, K)
    s = synth.scales(synth.seed(96), N, K)
    blob = oracle.pack(BP, t, s)
    assert blob.size == N * 3 * 34 and blob.size == oracle.packed_bytes(BP, N, K)
    rc, t2, s2 = oracle.unpack(BP, blob, N, K)
    assert rc == 0 and np.array_equal(t, t2) and np.array_equal(s, s2)


def test_format_sizes_vs_pages():
    g = _gold("pages_sizes.json")
    b3_bpw = 28 * 8 / 128
    tb_bpw = 34 * 8 / 128
    assert abs(b3_bpw - g["effective_bits_per_weight_with_fp16_group_scales"]["value"]) < 0.02
    # five trits per byte sits just above the entropy bound log2(3)
    assert math.log2(3) <= 8 / 5 and abs(math.log2(3) - g["entropy_bits_per_trit"]["value"]) < 0.01
    assert 8 / 4 == g["two_bit_aligned_storage_bits"]["value"]
    r = g["pq2_gb_over_ptq1_0_gb"]
    assert abs(tb_bpw / b3_bpw - r["pq2_gb"] / r["ptq1_0_gb"]) < 0.01 * (r["pq2_gb"] / r["ptq1_0_gb"])


# ---------------------------------------------------------------- quant ---

def test_quant_hand_examples():
    for ex in _gold("hand_examples.json")["quant"]:
        x = np.array([ex["x"]], dtype=np.float16)
        q, sc = oracle.quant(x)
        assert list(q[0]) == ex["q"], ex
        if ex.get("scale_is_1_over_127"):
            assert sc[0] == np.float32(1.0) / np.float32(127.0)
        if "scale" in ex:
            assert sc[0] == ex["scale"]


def _numpy_quant_f32(x32):
    a = np.abs(x32).max(axis=-1, keepdims=True).astype(np.float32)
    inv = np.float32(127.0) / a
    q = np.clip(np.rint((x32 * inv).astype(np.float32)), -127, 127).astype(np.int8)
    return q, (a / np.float32(127.0)).astype(np.float32)[..., 0]


def test_quant_bruteforce_all_fp16_pairs():
    """K=2, x0 = +-1, x1 = every finite fp16: covers |x1| <= 1 and the regime
    where x1 becomes the absmax.  Compared with numpy float32 arithmetic."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x1 = bits.view(np.float16)
    x1 = x1[np.isfinite(x1)]
    assert x1.size == 63488
    for x0 in (1.0, -1.0):
        x = np.stack([np.full(x1.size, x0, np.float16), x1], axis=1)
        q, sc = oracle.quant(x)
        qr, scr = _numpy_quant_f32(x.astype(np.float32))
        assert np.array_equal(q, qr)
        assert np.array_equal(sc.view(np.uint32), scr.view(np.uint32))


def test_quant_invariants():
    x = synth.normal_f32(synth.seed(95), 64, 1000)
    q, sc = oracle.quant(x)
    am = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), am]) == 127)
    assert np.all(np.abs(q).max(axis=1) == 127)
    qn, scn = oracle.quant(-x)
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    for k in (-3, 5):
        qk, sck = oracle.quant((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qk, q)
        assert np.allclose(sck, sc * 2.0 ** k, rtol=0, atol=0)
    # fp16 input equals fp32 input of the widened values
    xh = synth.normal_f16(synth.seed(96), 8, 640)
    assert np.array_equal(oracle.quant(xh)[0], oracle.quant(xh.astype(np.float32))[0])


def test_quant_rejects_nonfinite():
    for bad in (np.inf, -np.inf, np.nan):
        x = np.array([[1.0, bad, 0.5]], dtype=np.float32)
        with pytest.raises(oracle.OracleError):
            oracle.quant(x)
    with pytest.raises(oracle.OracleError):  # 127/a overflows
        oracle.quant(np.array([[1e-39, 0.0]], dtype=np.float32))


# ------------------------------------------------------- integer core -----

def test_group_sums_vs_numpy_int64():
    M, N, K = 3, 9, 512
    t = synth.trits(synth.seed(97), N, K)
    q, _ = oracle.quant(synth.normal_f16(synth.seed(98), M, K))
    S = oracle.group_sums(t, q)
    G = K // 128
    ref = np.einsum("ngi,mgi->mng", t.reshape(N, G, 128).astype(np.int64),
                    q.reshape(M, G, 128).astype(np.int64))
    assert np.array_equal(S.astype(np.int64), ref)
    assert np.abs(S).max() <= 127 * 128


def test_group_sums_special_cases():
    K = 256
    q, _ = oracle.quant(synth.normal_f16(synth.seed(99), 1, K))
    assert not oracle.group_sums(np.zeros((2, K), np.int8), q).any()
    for sign in (1, -1):
        for k in (0, 127, 128, 255):
            t = np.zeros((1, K), np.int8)
            t[0, k] = sign
            S = oracle.group_sums(t, q)[0, 0]
            expect = np.zeros(2, np.int64)
            expect[k // 128] = sign * int(q[0, k])
            assert np.array_equal(S, expect)
        S = oracle.group_sums(np.full((1, K), sign, np.int8), q)[0, 0]
        assert np.array_equal(S, sign * q[0].reshape(2, 128).astype(np.int64).sum(1))
    # additivity over disjoint supports
    a = synth.trits(synth.seed(100), 1, K)
    b = np.where(a == 0, synth.trits(synth.seed(101), 1, K), 0).astype(np.int8)
    assert np.array_equal(oracle.group_sums(a + b, q),
                          oracle.group_sums(a, q) + oracle.group_sums(b, q))


# ------------------------------------------------------------ output ------

def _deq_ref(t, s, q, a):
    """float64 dequantize-then-matmul: W[n,k] = s[n,k//128] * t[n,k]."""
    sf = s.view(np.float16).astype(np.float64)
    W = t.astype(np.float64) * np.repeat(sf, 128, axis=1)
    return (q.astype(np.float64) @ W.T) * a.astype(np.float64)[:, None]


def test_gemv_vs_float64_dequant_matmul():
    M, N, K = 4, 33, 1024
    t = synth.trits(synth.seed(102), N, K)
    s = synth.scales(synth.seed(103), N, K)
    q, a = oracle.quant(synth.normal_f16(synth.seed(104), M, K))
    y = oracle.gemv(t, s, q, a)
    ref = _deq_ref(t, s, q, a)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())
    # rounding is the only difference: one fp32 rounding of the double value
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2.0 ** -23
    # With scales in [0.005, 0.05] every term s*t*q is a multiple of 2^-18 below
    # 2^13, so both double sums are exact whatever their order, and the result
    # is the exact value times a, rounded once to double and once to fp32.
    assert np.array_equal(y, ref.astype(np.float32))


def test_gemv_long_k_exact_rounding():
    """K=17408 (136 groups): the scaled group sums need more than 24 bits, so
    only an accumulation wider than fp32 reproduces the once-rounded value."""
    M, N, K = 2, 24, 17408
    t = synth.trits(synth.seed(112), N, K)
    s = synth.scales(synth.seed(113), N, K)
    q, a = oracle.quant(synth.normal_f16(synth.seed(114), M, K))
    y = oracle.gemv(t, s, q, a)
    assert np.array_equal(y, _deq_ref(t, s, q, a).astype(np.float32))


def test_gemv_unit_scales_is_exact_integer_matmul():
    M, N, K = 2, 17, 384
    t = synth.trits(synth.seed(105), N, K)
    s = np.full((N, K // 128), 0x3C00, np.uint16)
    q, _ = oracle.quant(synth.normal_f16(synth.seed(106), M, K))
    y = oracle.gemv(t, s, q, np.ones(M, np.float32))
    ref = q.astype(np.int64) @ t.astype(np.int64).T
    assert np.array_equal(y.astype(np.int64), ref)


def test_gemv_hand_example():
    ex = _gold("hand_examples.json")["gemv_k128"]
    t = np.zeros((1, 128), np.int8)
    t[0, 0], t[0, 1] = 1, -1
    s = np.array([[0x3800]], np.uint16)  # 0.5
    x = np.zeros((1, 128), np.float16)
    x[0, :3] = [1.0, -0.5, 0.25]
    q, a = oracle.quant(x)
    assert oracle.group_sums(t, q)[0, 0, 0] == ex["S"]
    y = oracle.gemv(t, s, q, a)[0, 0]
    assert abs(y - ex["y"]) <= 1e-7


def test_gemv_rows_and_packed_agree_with_gemv():
    M, N, K = 2, 21, 768
    t = synth.trits(synth.seed(107), N, K)
    s = synth.scales(synth.seed(108), N, K)
    q, a = oracle.quant(synth.normal_f16(synth.seed(109), M, K))
    y = oracle.gemv(t, s, q, a)
    rows = np.array([0, 20, 7, 7])
    assert np.array_equal(oracle.gemv_rows(t, s, q, a, rows), y[:, rows])
    for fmt in (B3, TB, BP):
        assert np.array_equal(oracle.project_packed(fmt, oracle.pack(fmt, t, s), N, K, q, a), y)
    oracle.set_threads(4)
    try:
        assert np.array_equal(oracle.gemv(t, s, q, a), y)
    finally:
        oracle.set_threads(1)


# ----------------------------------------------------------- swiglu -------

def test_swiglu_vs_torch_silu_float64():
    g = synth.normal_f32(synth.seed(110), 4096) * np.float32(6)
    u = synth.normal_f32(synth.seed(111), 4096)
    h = oracle.swiglu(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64)))
           * torch.from_numpy(u.astype(np.float64))).numpy()
    assert np.allclose(h, ref, rtol=2.0 ** -23, atol=1e-37)
    assert np.array_equal(h, ref.astype(np.float32))


def test_swiglu_special_values():
    g = np.array([0.0, 80.0, -80.0, 1.0], np.float32)
    u = np.array([3.0, 2.0, 1.0, 1.0], np.float32)
    h = oracle.swiglu(g, u)
    assert h[0] == 0.0
    assert h[1] == np.float32(160.0)
    assert h[2] <= 0.0 and abs(h[2]) < 1e-30
    assert abs(h[3] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-7


# ------------------------------------------- Hadamard rotation (FFN input) ----
# Pinned against Sylvester's matrix built by scipy.linalg.hadamard (a library
# routine), closed forms for one-hot inputs, orthogonality and the invariance
# of W x under a joint rotation of W's columns and x.

def _sylvester64():
    from scipy.linalg import hadamard
    return hadamard(64).astype(np.float64)


def test_hadamard_one_hot_closed_form():
    """e_j -> s_i (-1)^popcount(i & j) / 8 inside j's block, zero elsewhere."""
    K = 192
    s = synth.signs(synth.seed(9, 1), K)
    for j in (0, 1, 5, 63, 64, 100, 191):
        x = np.zeros(K, dtype=np.float32)
        x[j] = 1.0
        y = oracle.hadamard(x, s)
        b0 = (j // 64) * 64
        ref = np.zeros(K, dtype=np.float32)
        for i in range(64):
            ref[b0 + i] = s[b0 + i] * (-1.0 if bin(i & (j - b0)).count("1") % 2 else 1.0) / 8.0
        assert np.array_equal(y, ref), j


def test_hadamard_vs_scipy_matrix():
    """Block-diagonal diag(s) H_64 / 8 as a float64 matrix product, rounded once;
    N(0,1) inputs keep every double sum exact, so the results are equal."""
    H = _sylvester64()
    M, K = 3, 320
    x = synth.normal_f32(synth.seed(9, 2), M, K)
    s = synth.signs(synth.seed(9, 3), K)
    y = oracle.hadamard(x, s)
    ref = np.empty((M, K), dtype=np.float64)
    for b in range(K // 64):
        blk = x[:, 64 * b:64 * b + 64].astype(np.float64)
        ref[:, 64 * b:64 * b + 64] = (blk @ H.T) / 8.0 * s[64 * b:64 * b + 64]
    assert np.array_equal(y, ref.astype(np.float32))


def test_hadamard_fp16_input_widened_exactly():
    K = 128
    xh = synth.normal_f16(synth.seed(9, 4), 2, K)
    s = synth.signs(synth.seed(9, 5), K)
    assert np.array_equal(oracle.hadamard(xh, s), oracle.hadamard(xh.astype(np.float32), s))


def test_hadamard_orthogonal():
    """Parseval per block, and the inverse H diag(s) / 8 returns the input."""
    H = _sylvester64()
    K = 256
    x = synth.normal_f32(synth.seed(9, 6), K)
    s = synth.signs(synth.seed(9, 7), K)
    y = oracle.hadamard(x, s).astype(np.float64)
    for b in range(K // 64):
        xb, yb = x[64 * b:64 * b + 64].astype(np.float64), y[64 * b:64 * b + 64]
        assert math.isclose((yb ** 2).sum(), (xb ** 2).sum(), rel_tol=1e-6)
        back = H @ (yb * s[64 * b:64 * b + 64]) / 8.0
        assert np.allclose(back, xb, rtol=0, atol=1e-6)
    assert np.allclose(H @ H, 64.0 * np.eye(64))


def test_hadamard_joint_rotation_invariance():
    """W x = (W R^T)(R x) for R = diag(s) H / 8 per block."""
    H = _sylvester64()
    K, N = 128, 7
    rng = np.random.default_rng(3)
    W = rng.standard_normal((N, K))
    x = synth.normal_f32(synth.seed(9, 8), K)
    s = synth.signs(synth.seed(9, 9), K)
    R = np.zeros((K, K))
    for b in range(K // 64):
        R[64 * b:64 * b + 64, 64 * b:64 * b + 64] = np.diag(s[64 * b:64 * b + 64].astype(np.float64)) @ H / 8.0
    y = oracle.hadamard(x, s).astype(np.float64)
    assert np.allclose((W @ R.T) @ y, W @ x.astype(np.float64), rtol=0, atol=1e-5)


def test_hadamard_blocks_independent_and_rejects():
    K = 192
    s = synth.signs(synth.seed(9, 10), K)
    x = synth.normal_f32(synth.seed(9, 11), K)
    x2 = x.copy()
    x2[70] += 1.0
    d = oracle.hadamard(x2, s) != oracle.hadamard(x, s)
    assert d[64:128].any() and not d[:64].any() and not d[128:].any()
    with pytest.raises(oracle.OracleError):
        oracle.hadamard(np.zeros(100, np.float32), np.ones(100, np.int8))
    bad = s.copy()
    bad[5] = 0
    with pytest.raises(oracle.OracleError):
        oracle.hadamard(x, bad)
    xn = x.copy()
    xn[3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.hadamard(xn, s)


# ------------------------------------------------------- ternarisation ----
# Pinned against a float64 brute force over every support size (numpy), the
# closed forms of constant, single-weight and zero groups, sign and scale
# invariances, and numpy's float16 rounding.

def _brute_ternarize_group(wg):
    """Least-squares ternary fit of one group: every support size k of the
    k largest magnitudes (stable order), residual computed directly."""
    order = np.argsort(-np.abs(wg.astype(np.float64)), kind="stable")
    w64 = wg.astype(np.float64)
    best = (np.sum(w64 ** 2), 0, np.zeros(128, np.int8), 0.0)
    for k in range(1, 129):
        sup = order[:k]
        t = np.zeros(128, np.int8)
        t[sup] = np.sign(w64[sup]).astype(np.int8)
        s = np.abs(w64[sup]).sum() / k
        res = np.sum((w64 - s * t) ** 2)
        if res < best[0]:
            best = (res, k, t, s)
    return best[2], np.float16(best[3]).view(np.uint16)


def test_ternarize_vs_bruteforce():
    N, K = 3, 384
    w = synth.normal_f32(synth.seed(31, 1), N, K) * np.float32(0.02)
    t, s = oracle.ternarize(w)
    for n in range(N):
        for g in range(K // 128):
            tr, sr = _brute_ternarize_group(w[n, 128 * g:128 * g + 128])
            assert np.array_equal(t[n, 128 * g:128 * g + 128], tr), (n, g)
            assert s[n, g] == sr, (n, g)


def test_ternarize_heavy_tails_vs_bruteforce():
    """A few large weights among small ones: a small support wins."""
    w = synth.normal_f32(synth.seed(31, 2), 2, 128) * np.float32(0.01)
    w[0, [3, 50, 99]] = [4.0, -5.0, 4.5]
    w[1, :] = np.float32(0.001)
    w[1, 7] = -2.0
    t, s = oracle.ternarize(w)
    for n in range(2):
        tr, sr = _brute_ternarize_group(w[n])
        assert np.array_equal(t[n], tr) and s[n, 0] == sr
    assert np.count_nonzero(t[1]) == 1 and t[1, 7] == -1
    assert s[1, 0] == np.float16(2.0).view(np.uint16)


def test_ternarize_closed_forms():
    c = np.float32(0.03125)
    w = np.zeros((3, 128), np.float32)
    w[0] = c * np.where(np.arange(128) % 3 == 0, -1, 1)  # constant magnitude: full support
    w[1, 17] = -0.75                                      # a single weight
    t, s = oracle.ternarize(w)                            # row 2: all zero
    assert np.array_equal(t[0], np.where(np.arange(128) % 3 == 0, -1, 1).astype(np.int8))
    assert s[0, 0] == np.float16(c).view(np.uint16)
    assert np.count_nonzero(t[1]) == 1 and t[1, 17] == -1 and s[1, 0] == np.float16(0.75).view(np.uint16)
    assert not t[2].any() and s[2, 0] == 0


def test_ternarize_invariances():
    w = synth.normal_f32(synth.seed(31, 3), 2, 256) * np.float32(0.05)
    t, s = oracle.ternarize(w)
    tn, sn = oracle.ternarize(-w)
    assert np.array_equal(tn, -t) and np.array_equal(sn, s)
    t2, s2 = oracle.ternarize(w * np.float32(2.0))
    assert np.array_equal(t2, t)
    assert np.array_equal(s2.view(np.float16).astype(np.float64), 2.0 * s.view(np.float16).astype(np.float64))
    perm = np.random.default_rng(5).permutation(128)
    tp, sp = oracle.ternarize(np.ascontiguousarray(w[:, perm]))
    assert np.array_equal(tp, t[:, perm]) and np.array_equal(sp[:, 0], s[:, 0])


def test_ternarize_scale_rounding_vs_numpy_float16():
    """The scale of a one-weight group is |w| rounded to fp16: compared with
    numpy's float16 conversion on exact midpoints (ties to even), subnormals,
    values near the top of the range, and random values."""
    rng = np.random.default_rng(7)
    h = rng.integers(1, 0x7BFF, 400).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals = np.concatenate([(lo + hi) / 2, lo, rng.random(200) * 60000, rng.random(100) * 6e-5,
                           [65504.0, 65519.0, 2.0 ** -24, 2.0 ** -25 * 1.5, 2.0 ** -14]]).astype(np.float32)
    w = np.zeros((vals.size, 128), np.float32)
    w[:, 0] = vals
    t, s = oracle.ternarize(w)
    ref = vals.astype(np.float64).astype(np.float16).view(np.uint16)
    assert np.array_equal(s[:, 0], ref)


def test_ternarize_rejects():
    with pytest.raises(oracle.OracleError):
        oracle.ternarize(np.full((1, 128), np.nan, np.float32))
    w = np.zeros((1, 128), np.float32)
    w[0, 0] = 65520.0  # rounds past the largest fp16
    with pytest.raises(oracle.OracleError):
        oracle.ternarize(w)
    with pytest.raises(oracle.OracleError):
        oracle.ternarize(np.zeros((1, 100), np.float32))
