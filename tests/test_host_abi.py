"""Host-side tests of libtq (no GPU): the library loads and exports every
symbol include/tq.h declares; the packer follows the documented layout and
round-trips; every argument error is reported before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import ternary_weight_base_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
B3, TB, BP, B3R = tq.TQ_FMT_B3, tq.TQ_FMT_2B, tq.TQ_FMT_BP, tq.TQ_FMT_B3R


def _header_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(tq.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(tq.EXPORTS)


def test_status_strings():
    for code in range(0, -9, -1):
        assert tq.tq_status_str(code) not in ("", "unknown status")
    assert tq.tq_status_str(-100) == "unknown status"


def _rand(N, K, seed):
    return synth.trits(synth.seed(seed, 1), N, K), synth.scales(synth.seed(seed, 2), N, K)


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (64, 1024), (65, 384), (130, 640), (200, 128)])
def test_pack_roundtrip_and_size(fmt, N, K):
    t, s = _rand(N, K, N * 7 + K)
    blob = tq.tq_pack(fmt, t, s)
    P = 28 if fmt in (B3, B3R) else 34
    align = {B3: 4, B3R: 1}.get(fmt, 8)
    nb = (N + 63) // 64
    w = N - 64 * (nb - 1)
    rows = 64 * (nb - 1) + (w + align - 1) // align * align
    assert blob.size == tq.tq_packed_bytes(fmt, N, K) == rows * (K // 128) * P
    t2, s2 = tq.tq_unpack(fmt, blob, N, K)
    assert np.array_equal(t, t2) and np.array_equal(s, s2)


def _device_group_bytes(fmt, blob, N, K, n, g):
    """The (row n, group g) bytes and scale, located as include/tq.h describes."""
    G = K // 128
    if fmt == B3R:  # row-major: row n's group g at (n G + g) 28, 26 bytes then the scale
        a = (n * G + g) * 28
        return blob[a: a + 26], int(blob[a + 26]) | (int(blob[a + 27]) << 8)
    P = 28 if fmt == B3 else 34
    align = 4 if fmt == B3 else 8
    nb = (N + 63) // 64
    b, r = divmod(n, 64)
    w = N - 64 * (nb - 1)
    Wb = 64 if b < nb - 1 else (w + align - 1) // align * align
    gb = 64 * b * G * P + g * Wb * P
    if fmt == B3:
        body = np.concatenate([blob[gb + r * 16: gb + r * 16 + 16],
                               blob[gb + Wb * 16 + r * 12: gb + Wb * 16 + r * 12 + 10]])
        sc = blob[gb + Wb * 16 + r * 12 + 10: gb + Wb * 16 + r * 12 + 12]
    else:
        body = np.concatenate([blob[gb + r * 16: gb + r * 16 + 16],
                               blob[gb + Wb * 16 + r * 16: gb + Wb * 16 + r * 16 + 16]])
        sc = blob[gb + Wb * 32 + r * 2: gb + Wb * 32 + r * 2 + 2]
    return body, int(sc[0]) | (int(sc[1]) << 8)


def _decode_b3_doc(body):
    """Decode 26 device bytes by the rule written in include/tq.h, using
    Python's base-3 string conversion."""
    t = np.full(128, 99, dtype=np.int64)
    for j, v in enumerate(body):
        assert v < 243
        digits = [int(c) for c in np.base_repr(int(v), 3).rjust(5, "0")][::-1]
        if j < 25:
            for i in range(4):
                t[4 * j + i] = digits[i] - 1
            t[100 + j] = digits[4] - 1
        else:
            assert digits[0] == 1 and digits[4] == 1
            t[125:128] = np.array(digits[1:4]) - 1
    return t


def _decode_bp_doc(body):
    """Byte 4w + b, bit s of each plane is k = 32w + 4s + b (include/tq.h)."""
    t = np.full(128, 99, dtype=np.int64)
    for j in range(16):
        w, b = divmod(j, 4)
        for s in range(8):
            nz, neg = (int(body[j]) >> s) & 1, (int(body[16 + j]) >> s) & 1
            assert not (neg and not nz)
            t[32 * w + 4 * s + b] = (-1 if neg else 1) if nz else 0
    return t


def _decode_2b_doc(body):
    t = np.full(128, 99, dtype=np.int64)
    for byte_idx, v in enumerate(body):
        m, c = divmod(byte_idx, 4)
        for s in range(4):
            code = (int(v) >> (2 * s)) & 3
            assert code != 3
            t[16 * m + 4 * s + c] = code - 1
    return t


@pytest.mark.parametrize("fmt", [B3, TB, BP, B3R])
def test_pack_matches_documented_layout(fmt):
    N, K = 70, 384
    t, s = _rand(N, K, 5 + fmt)
    blob = tq.tq_pack(fmt, t, s)
    for n in (0, 1, 63, 64, 69):
        for g in range(K // 128):
            body, sc = _device_group_bytes(fmt, blob, N, K, n, g)
            dec = {B3: _decode_b3_doc, TB: _decode_2b_doc, BP: _decode_bp_doc, B3R: _decode_b3_doc}[fmt](body)
            assert np.array_equal(dec, t[n, 128 * g: 128 * g + 128]), (n, g)
            assert sc == s[n, g]


def test_pack_same_information_as_oracle_canonical():
    N, K = 33, 512
    t, s = _rand(N, K, 77)
    for fmt in (B3, TB, BP):
        rc, t1, s1 = oracle.unpack(fmt, oracle.pack(fmt, t, s), N, K)
        t2, s2 = tq.tq_unpack(fmt, tq.tq_pack(fmt, t, s), N, K)
        assert rc == 0 and np.array_equal(t1, t2) and np.array_equal(s1, s2)
    # B3R holds exactly B3's group bytes and scales, in row-major group order
    b3, b3r = tq.tq_pack(B3, t, s), tq.tq_pack(B3R, t, s)
    for n in range(N):
        for g in range(K // 128):
            u, su = _device_group_bytes(B3, b3, N, K, n, g)
            v, sv = _device_group_bytes(B3R, b3r, N, K, n, g)
            assert np.array_equal(u, v) and su == sv
    t3, s3 = tq.tq_unpack(B3R, b3r, N, K)
    assert np.array_equal(t3, t) and np.array_equal(s3, s)


def test_b3_closed_form_device_bytes():
    # all-zero trits -> every full byte 121 (digits all 1); the tail byte too
    N, K = 4, 128
    blob = tq.tq_pack(B3, np.zeros((N, K), np.int8), np.full((N, 1), 0x3C00, np.uint16))
    body, sc = _device_group_bytes(B3, blob, N, K, 2, 0)
    assert list(body) == [121] * 26 and sc == 0x3C00
    blob = tq.tq_pack(B3, np.ones((N, K), np.int8), np.zeros((N, 1), np.uint16))
    body, _ = _device_group_bytes(B3, blob, N, K, 1, 0)
    assert list(body[:25]) == [242] * 25 and body[25] == 1 + 2 * 3 + 2 * 9 + 2 * 27 + 81


def test_unpack_rejects_noncanonical():
    N, K = 5, 256
    t, s = _rand(N, K, 9)
    blob = tq.tq_pack(B3, t, s)
    for pos, val in ((0, 243), (17, 255)):
        bad = blob.copy()
        bad[pos] = val
        with pytest.raises(tq.TQError) as e:
            tq.tq_unpack(B3, bad, N, K)
        assert e.value.status == -5
    # tail byte with a non-unit padding digit (digit 0 = 0)
    bad = blob.copy()
    off = 8 * 16 + 0 * 12 + 9  # block 0 (padded to 8 rows), group 0, row 0, device byte 25
    assert bad[off] % 3 == 1
    bad[off] -= 1
    with pytest.raises(tq.TQError):
        tq.tq_unpack(B3, bad, N, K)
    # padding rows must stay zero trits / zero scale
    bad = blob.copy()
    bad[8 * 16 + 5 * 12 + 10] = 1  # scale of padding row 5 (rows 5..7 pad)
    with pytest.raises(tq.TQError):
        tq.tq_unpack(B3, bad, N, K)
    blob2 = tq.tq_pack(TB, t, s)
    bad = blob2.copy()
    bad[3] = 0xFF
    with pytest.raises(tq.TQError):
        tq.tq_unpack(TB, bad, N, K)
    # BP: a sign bit on a zero trit (row 0, group 0: nonzero byte 2 at 2, sign byte at 8*16 + 2)
    blobp = tq.tq_pack(BP, np.zeros((N, K), np.int8), s)
    badp = blobp.copy()
    badp[8 * 16 + 2] = 0x10
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(BP, badp, N, K)
    assert e.value.status == -5
    # non-finite scale
    bad = blob.copy()
    bad[8 * 16 + 1 * 12 + 11] = 0x7C
    bad[8 * 16 + 1 * 12 + 10] = 0x00
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(B3, bad, N, K)
    assert e.value.status == -4
    # B3R: a byte >= 243 (row 1, group 1, byte 3) and a bad padding digit in byte 25
    blobr = tq.tq_pack(B3R, t, s)
    bad = blobr.copy()
    bad[(1 * (K // 128) + 1) * 28 + 3] = 250
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(B3R, bad, N, K)
    assert e.value.status == -5
    bad = blobr.copy()
    assert bad[25] % 3 == 1
    bad[25] -= 1
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(B3R, bad, N, K)
    assert e.value.status == -5


def test_pack_rejects_bad_arguments():
    L = tq.lib
    t = np.zeros((2, 256), np.int8)
    s = np.full((2, 2), 0x3C00, np.uint16)
    out = np.empty(tq.tq_packed_bytes(B3, 2, 256), np.uint8)
    P = lambda a: a.ctypes.data
    assert L.tq_pack(B3, 2, 256, None, P(s), P(out), out.size) == -1
    assert L.tq_pack(B3, 2, 200, P(t), P(s), P(out), out.size) == -2
    assert L.tq_pack(B3, 0, 256, P(t), P(s), P(out), out.size) == -2
    assert L.tq_pack(7, 2, 256, P(t), P(s), P(out), out.size) == -5
    assert L.tq_pack(B3, 2, 256, P(t), P(s), P(out), out.size - 1) == -7
    t2 = t.copy()
    t2[1, 3] = 2
    assert L.tq_pack(B3, 2, 256, P(t2), P(s), P(out), out.size) == -4
    s2 = s.copy()
    s2[0, 0] = 0x7E00
    out2 = np.empty(tq.tq_packed_bytes(TB, 2, 256), np.uint8)
    assert L.tq_pack(TB, 2, 256, P(t), P(s2), P(out2), out2.size) == -4
    assert tq.tq_packed_bytes(B3, 2, 100) == 0 and tq.tq_packed_bytes(9, 2, 128) == 0


# Device entry points: every check below fails on the host, before any launch,
# so these run without a GPU.  Fake device addresses are never dereferenced.
FAKE = 0x10000  # 16-byte aligned
MIS = 0x10004   # 4-byte but not 16-byte aligned
ODD = 0x10002   # not even 4-byte aligned


def test_device_entry_points_validate_on_host():
    L = tq.lib
    # quant
    assert L.tq_quant_act(5, 1, 128, FAKE, FAKE, FAKE, None) == -6
    assert L.tq_quant_act(0, 0, 128, FAKE, FAKE, FAKE, None) == -2
    assert L.tq_quant_act(0, 1, 100, FAKE, FAKE, FAKE, None) == -2
    assert L.tq_quant_act(0, 1, 128, None, FAKE, FAKE, None) == -1
    assert L.tq_quant_act(0, 1, 128, MIS, FAKE, FAKE, None) == -3
    assert L.tq_quant_act(0, 1, 128, FAKE, FAKE, ODD, None) == -3
    # gemv
    assert L.tq_gemv(B3, 0, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2
    assert L.tq_gemv(B3, 17, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2
    assert L.tq_gemv(B3, 1, 64, 130, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2
    assert L.tq_gemv(4, 1, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
    assert L.tq_gemv(B3, 1, 64, 128, None, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert L.tq_gemv(B3, 1, 64, 128, FAKE, MIS, FAKE, FAKE, None, 0, None) == -3
    # a shape that splits K across workgroups needs a workspace of the stated size
    need = tq.tq_gemv_workspace_bytes(B3, 1, 5120, 17408)
    assert need > 0
    assert L.tq_gemv(B3, 1, 5120, 17408, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert L.tq_gemv(B3, 1, 5120, 17408, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == -7
    assert L.tq_gemv_gate_up_swiglu(B3, 1, 5120, 17408, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    need - 1, None) == -7
    assert L.tq_gemv(B3, 1, 5120, 17408, FAKE, FAKE, FAKE, FAKE, MIS, need, None) == -3
    assert L.tq_gemv_gate_up_swiglu(B3, 1, 64, 128, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == -1
    # BP and B3R run on the one-token kernel only
    for f in (BP, B3R):
        assert L.tq_gemv(f, 2, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
        assert L.tq_gemm(f, 512, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
        assert L.tq_debug_group_sums(f, 1, 64, 128, FAKE, FAKE, FAKE, 1, None) == -5
    assert L.tq_debug_unpack(4, 64, 128, FAKE, FAKE, None) == -5
    assert L.tq_gemv(BP, 2, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
    assert L.tq_gemm(BP, 512, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
    assert L.tq_debug_group_sums(BP, 2, 64, 128, FAKE, FAKE, FAKE, 0, None) == -5
    assert L.tq_debug_group_sums(BP, 1, 64, 128, FAKE, FAKE, FAKE, 1, None) == -5
    assert L.tq_debug_gate_up_sums(BP, 2, 64, 128, FAKE, FAKE, FAKE, FAKE, None) == -5
    assert L.tq_debug_unpack(5, 64, 128, FAKE, FAKE, None) == -5
    assert tq.tq_gemv_workspace_bytes(BP, 2, 5120, 8192) == 0
    assert tq.tq_gemv_workspace_bytes(BP, 1, 5120, 8192) > 0
    # gemm
    assert L.tq_gemm(B3, 0, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2
    assert L.tq_gemm(B3, 512, 64, 96, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -2
    assert L.tq_gemm(B3, 512, 64, 128, FAKE, MIS, FAKE, FAKE, None, 0, None) == -3
    assert L.tq_gemm(B3, 512, 64, 128, FAKE, FAKE, ODD, FAKE, None, 0, None) == -3
    assert L.tq_gemm(4, 512, 64, 128, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
    gneed = tq.tq_gemm_workspace_bytes(B3, 512, 5120, 17408)  # split K: a workspace is needed
    assert L.tq_gemm(B3, 512, 5120, 17408, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert L.tq_gemm(B3, 512, 5120, 17408, FAKE, FAKE, FAKE, FAKE, MIS, gneed, None) == -3
    assert L.tq_gemm(B3, 512, 5120, 17408, FAKE, FAKE, FAKE, FAKE, FAKE, gneed - 1, None) == -7
    # debug hooks
    assert L.tq_debug_unpack(B3, 64, 128, FAKE, None, None) == -1
    assert L.tq_debug_unpack(B3, 0, 128, FAKE, FAKE, None) == -2
    assert L.tq_debug_group_sums(B3, 17, 64, 128, FAKE, FAKE, FAKE, 0, None) == -2
    assert L.tq_debug_group_sums(B3, 1, 64, 128, FAKE, FAKE, ODD, 1, None) == -3
    assert L.tq_debug_group_sums(B3, 1, 64, 128, FAKE, MIS, FAKE, 1, None) == -3
    assert L.tq_debug_gate_up_sums(B3, 1, 64, 128, FAKE, None, FAKE, FAKE, None) == -1
    assert L.tq_debug_gate_up_sums(B3, 17, 64, 128, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert L.tq_debug_gate_up_sums(B3, 1, 64, 128, FAKE, MIS, FAKE, FAKE, None) == -3
    # the allocation-free GEMV: every rejection before any device work
    NA = L.tq_gemv_noalloc
    assert NA(B3, 1, 5120, 17408, None, FAKE, FAKE, FAKE, None) == -1
    assert NA(B3, 8, 5120, 17408, FAKE, MIS, FAKE, FAKE, None) == -3
    assert NA(B3, 8, 5120, 17408, FAKE, FAKE, FAKE, ODD, None) == -3
    assert NA(B3, 17, 5120, 17408, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert NA(9, 1, 5120, 17408, FAKE, FAKE, FAKE, FAKE, None) == -5
    assert L.tq_noalloc_scratch_bytes() == 4 << 20
    # fused-quantiser sums: (fmt, N, K, W, Wu, x_dtype, x, x_bmax, x_nb, S, a_scale, stream)
    Q = L.tq_debug_gemv_quant_sums
    assert Q(B3, 64, 256, FAKE, None, 0, FAKE, None, 0, None, None, None) == -1
    assert Q(B3, 64, 256, FAKE, None, 1, FAKE, None, 4, FAKE, None, None) == -1
    assert Q(B3, 64, 256, FAKE, None, 2, FAKE, None, 0, FAKE, None, None) == -6
    assert Q(B3, 64, 256, FAKE, None, 1, FAKE, FAKE, 3, FAKE, None, None) == -2
    assert Q(7, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -5
    assert Q(B3, 64, 256, FAKE, None, 0, MIS, None, 0, FAKE, None, None) == -3
    assert Q(B3, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, ODD, None) == -3


@pytest.mark.parametrize("name", ["tq_decode_stack", "tq_decode_stack_persistent"])
def test_decode_stack_validates_on_host(name):
    class _L:  # the function under test in place of tq_decode_stack
        tq_decode_stack = getattr(tq.lib, name)
    L = _L
    args = (B3, 2, 640, 1152, 1280, 1024)
    need = tq.tq_decode_stack_workspace_bytes(*args)
    assert need > 0
    assert tq.tq_decode_stack_workspace_bytes(B3, 0, 640, 1152, 1280, 1024) == 0
    assert tq.tq_decode_stack_workspace_bytes(B3, 2, 600, 1152, 1280, 1024) == 0
    good = (tq.TqLayer * 2)(*[tq.TqLayer(FAKE, FAKE, FAKE, FAKE, FAKE)] * 2)
    bad = (tq.TqLayer * 2)(tq.TqLayer(FAKE, FAKE, FAKE, FAKE, FAKE), tq.TqLayer(FAKE, None, FAKE, FAKE, FAKE))
    mis = (tq.TqLayer * 2)(tq.TqLayer(FAKE, FAKE, FAKE, FAKE, FAKE), tq.TqLayer(FAKE, FAKE, MIS, FAKE, FAKE))
    c = lambda a: ctypes.cast(a, ctypes.c_void_p)
    outs = (FAKE,) * 4
    # (..., y_qkv, y_o, h, y_out, ffn_signs, ws, ws_bytes, stream)
    assert L.tq_decode_stack(*args, c(good), FAKE, FAKE, *outs, None, FAKE, need - 1, None) == -7
    assert L.tq_decode_stack(*args, c(bad), FAKE, FAKE, *outs, None, FAKE, need, None) == -1
    assert L.tq_decode_stack(*args, c(mis), FAKE, FAKE, *outs, None, FAKE, need, None) == -3
    assert L.tq_decode_stack(*args, c(good), MIS, FAKE, *outs, None, FAKE, need, None) == -3
    assert L.tq_decode_stack(*args, c(good), FAKE, FAKE, FAKE, ODD, FAKE, FAKE, None, FAKE, need,
                             None) == -3
    assert L.tq_decode_stack(*args, None, FAKE, FAKE, *outs, None, FAKE, need, None) == -1
    assert L.tq_decode_stack(5, 2, 640, 1152, 1280, 1024, c(good), FAKE, FAKE, *outs, None, FAKE,
                             need, None) == -5
    assert L.tq_decode_stack(*args, c(good), FAKE, FAKE, *outs, FAKE, FAKE, need - 1, None) == -7


def test_decode_stack_batch_validates_on_host():
    """Every rejection of tq_decode_stack_batch happens on the host."""
    L = tq.lib
    args = (2, 640, 1152, 1280, 1024)  # layers, hidden, inter, qkv_out, o_in
    W = tq.tq_decode_stack_batch_workspace_bytes
    need = {r: W(B3, r, *args) for r in (1, 2, 3, 4)}
    assert need[1] == tq.tq_decode_stack_workspace_bytes(B3, *args)
    assert need[1] <= need[2] <= need[3] <= need[4] and need[1] < need[4]
    assert W(B3, 0, *args) == 0 and W(B3, 5, *args) == 0
    assert W(BP, 2, *args) == 0 and W(B3R, 2, *args) == 0 and W(9, 2, *args) == 0
    assert W(TB, 2, *args) > 0
    assert W(B3, 2, 2, 600, 1152, 1280, 1024) == 0
    good = (tq.TqLayer * 2)(*[tq.TqLayer(FAKE, FAKE, FAKE, FAKE, FAKE)] * 2)
    bad = (tq.TqLayer * 2)(tq.TqLayer(FAKE, FAKE, FAKE, FAKE, FAKE), tq.TqLayer(FAKE, None, FAKE, FAKE, FAKE))
    c = lambda a: ctypes.cast(a, ctypes.c_void_p)
    outs = (FAKE,) * 4
    S = L.tq_decode_stack_batch
    # (fmt, rows, layers, hidden, inter, qkv_out, o_in, weights, x_in, a_in, y_qkv, y_o, h, y_out,
    #  ffn_signs, ws, ws_bytes, stream)
    assert S(B3, 3, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[3] - 1, None) == -7
    assert S(B3, 4, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[1], None) == -7
    assert S(B3, 0, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[4], None) == -2
    assert S(B3, 5, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[4], None) == -2
    assert S(BP, 2, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[4], None) == -5
    assert S(B3R, 2, *args, c(good), FAKE, FAKE, *outs, None, FAKE, need[4], None) == -5
    assert S(B3, 2, *args, c(bad), FAKE, FAKE, *outs, None, FAKE, need[2], None) == -1
    assert S(B3, 2, *args, None, FAKE, FAKE, *outs, None, FAKE, need[2], None) == -1
    assert S(B3, 2, *args, c(good), MIS, FAKE, *outs, None, FAKE, need[2], None) == -3
    assert S(B3, 2, *args, c(good), FAKE, FAKE, FAKE, ODD, FAKE, FAKE, None, FAKE, need[2], None) == -3
    assert S(B3, 2, 2, 640, 1152, 1280, 1000, c(good), FAKE, FAKE, *outs, None, FAKE, need[4],
             None) == -2


def test_gemv_quant_rows_sums_validates_on_host():
    """Every rejection of tq_debug_gemv_quant_rows_sums happens on the host."""
    Q = tq.lib.tq_debug_gemv_quant_rows_sums
    # (fmt, rows, N, K, W, Wu, x_dtype, x, x_bmax, x_nb, S, a_scale, stream)
    assert Q(B3, 2, 64, 256, FAKE, None, 0, FAKE, None, 0, None, None, None) == -1
    assert Q(B3, 2, 64, 256, None, None, 0, FAKE, None, 0, FAKE, None, None) == -1
    assert Q(B3, 2, 64, 256, FAKE, None, 1, FAKE, None, 4, FAKE, None, None) == -1
    assert Q(BP, 2, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -5
    assert Q(B3R, 2, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -5
    assert Q(B3, 2, 64, 256, FAKE, None, 2, FAKE, None, 0, FAKE, None, None) == -6
    assert Q(B3, 0, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -2
    assert Q(B3, 5, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -2
    assert Q(B3, 2, 64, 200, FAKE, None, 0, FAKE, None, 0, FAKE, None, None) == -2
    assert Q(B3, 2, 64, 256, FAKE, None, 1, FAKE, FAKE, 3, FAKE, None, None) == -2
    assert Q(B3, 2, 64, 256, FAKE, None, 0, MIS, None, 0, FAKE, None, None) == -3
    assert Q(B3, 2, 64, 256, FAKE, None, 0, FAKE, None, 0, ODD, None, None) == -3
    assert Q(B3, 2, 64, 256, FAKE, None, 0, FAKE, None, 0, FAKE, ODD, None) == -3


def test_gemv_quant_validates_on_host():
    """Every rejection of tq_gemv_quant happens on the host (no GPU here:
    the device pointers are never dereferenced)."""
    L = tq.lib
    F16, F32 = tq.TQ_F16, tq.TQ_F32
    N, K = 5120, 8192
    need = tq.tq_gemv_quant_workspace_bytes(B3, N, K)
    assert need > 0 and tq.tq_gemv_quant_workspace_bytes(B3, N, K, True) > need
    assert tq.tq_gemv_quant_workspace_bytes(B3, N, 1000) == 0
    call = lambda fmt=B3, n=N, k=K, W=FAKE, Wu=None, dt=F16, x=FAKE, xb=None, nb=0, y=FAKE, yb=None, \
        sg=None, ws=FAKE, wsb=need: L.tq_gemv_quant(fmt, n, k, W, Wu, dt, x, xb, nb, y, yb, sg, ws,
                                                    wsb, None)
    assert call(W=None) == -1
    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(dt=F32) == -1                       # fp32 input needs its block maxima
    assert call(fmt=4) == -5
    assert call(dt=7) == -6
    assert call(k=1000) == -2
    assert call(dt=F32, xb=FAKE, nb=K // 64 - 1) == -2  # wrong maxima count
    assert call(x=MIS) == -3
    assert call(W=MIS) == -3
    assert call(Wu=MIS) == -3
    assert call(y=ODD) == -3
    assert call(dt=F32, xb=ODD, nb=K // 64) == -3
    assert call(yb=ODD) == -3
    assert call(ws=None) == -1
    assert call(ws=MIS) == -3
    assert call(wsb=need - 1) == -7
    assert call(sg=FAKE, Wu=FAKE) == -2             # the rotation takes one matrix
    assert call(sg=FAKE, n=N - 64 + 32) == -2        # ... and whole 64-row blocks
    assert call(sg=FAKE, wsb=need - 1) == -7


def test_hadamard_quant_validates_on_host():
    L = tq.lib
    F16, F32 = tq.TQ_F16, tq.TQ_F32
    call = lambda dt=F16, m=2, k=5120, x=FAKE, sg=FAKE, q=FAKE, a=FAKE: \
        L.tq_hadamard_quant_act(dt, m, k, x, sg, q, a, None)
    assert call(x=None) == -1
    assert call(sg=None) == -1
    assert call(q=None) == -1
    assert call(a=None) == -1
    assert call(dt=5) == -6
    assert call(m=0) == -2
    assert call(k=32) == -2
    assert call(k=5120 + 32) == -2
    assert call(x=MIS) == -3
    assert call(sg=MIS) == -3
    assert call(q=MIS) == -3
    assert call(a=ODD) == -3


def test_stream_read_validates_on_host():
    L = tq.lib
    W = tq.TQ_STREAM_READ_WGS
    call = lambda src=FAKE, n=1 << 20, sink=FAKE, sw=W: L.tq_debug_stream_read(src, n, sink, sw, None)
    assert call(src=None) == -1
    assert call(sink=None) == -1
    assert call(n=24) == -2
    assert call(sw=W - 1) == -7
    assert call(src=MIS) == -3
    assert call(sink=ODD) == -3


def test_workspace_upkeep_validates_on_host():
    L = tq.lib
    clear = lambda ws=FAKE, n=1 << 20: L.tq_workspace_clear(ws, n, None)
    check = lambda ws=FAKE, n=1 << 20, cnt=FAKE: L.tq_workspace_check(ws, n, cnt, None)
    assert clear(ws=None) == -1
    assert clear(n=24) == -2
    assert clear(ws=MIS) == -3
    assert clear(ws=None, n=0) == 0  # nothing to clear: no launch
    assert check(ws=None) == -1
    assert check(cnt=None) == -1
    assert check(n=40) == -2
    assert check(ws=MIS) == -3
    assert check(cnt=ODD) == -3


def test_workspace_sizes():
    assert tq.tq_gemv_workspace_bytes(B3, 1, 1024, 1024) == 0
    for N, K in ((5120, 8192), (5120, 17408), (10240, 5120)):
        assert tq.tq_gemv_workspace_bytes(B3, 1, N, K) > 0
    assert tq.tq_gemm_workspace_bytes(B3, 512, 17408, 5120) == 0   # 1088 tiles: no K split
    assert tq.tq_gemm_workspace_bytes(B3, 512, 5120, 17408) > 0    # 320 tiles: K in chunks
    assert tq.tq_gemv_workspace_bytes(B3, 17, 1024, 1024) == 0  # out of range
