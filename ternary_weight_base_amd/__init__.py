"""Python binding of libtq (ternary-weight GEMV/GEMM for AMD gfx950).

Argument marshalling only: every step of the computation runs in libtq's HIP
kernels (or, for packing, in its host C++ code).  PyTorch supplies device
memory and streams.  The functions carry the C ABI's names (see
include/tq.h); device tensors must be contiguous, on the GPU and 16-byte
aligned.  If libtq.so is missing the import fails loudly -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_FMT_B3 = 0
TQ_FMT_2B = 1
TQ_FMT_BP = 2
TQ_FMT_B3R = 3  # B3 bytes in row-major group order (the layout without the re-tiling)
TQ_F16 = 0
TQ_F32 = 1
TQ_STREAM_READ_WGS = 8192
GROUP = 128
GEMV_MAX_M = 16
STACK_MAX_ROWS = 4

_STATUS = {0: "TQ_OK", -1: "TQ_ERR_NULL", -2: "TQ_ERR_SHAPE", -3: "TQ_ERR_ALIGN",
           -4: "TQ_ERR_VALUE", -5: "TQ_ERR_FORMAT", -6: "TQ_ERR_DTYPE", -7: "TQ_ERR_SIZE",
           -8: "TQ_ERR_HIP"}

EXPORTS = ("tq_status_str", "tq_packed_bytes", "tq_pack", "tq_unpack", "tq_quant_act",
           "tq_gemv_workspace_bytes", "tq_gemv", "tq_gemv_gate_up_swiglu",
           "tq_gemm_workspace_bytes", "tq_gemm", "tq_debug_unpack", "tq_debug_group_sums",
           "tq_gemv_quant_workspace_bytes", "tq_gemv_quant",
           "tq_decode_stack_workspace_bytes", "tq_decode_stack", "tq_hadamard_quant_act",
           "tq_ternarize", "tq_debug_stream_read", "tq_debug_gate_up_sums",
           "tq_debug_gemv_quant_sums", "tq_decode_stack_persistent",
           "tq_gemv_noalloc", "tq_noalloc_scratch_bytes",
           "tq_decode_stack_batch_workspace_bytes", "tq_decode_stack_batch",
           "tq_debug_gemv_quant_rows_sums", "tq_workspace_clear", "tq_workspace_check")


class TqLayer(ctypes.Structure):
    """Packed weights of one layer (device addresses), as tq_layer in tq.h."""
    _fields_ = [("qkv", ctypes.c_void_p), ("o", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtq.so not built ({LIB_PATH}); run ternary_weight_base_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "tq_status_str": ([I], ctypes.c_char_p),
        "tq_packed_bytes": ([I, I64, I64], SZ),
        "tq_pack": ([I, I64, I64, P, P, P, SZ], I),
        "tq_unpack": ([I, I64, I64, P, SZ, P, P], I),
        "tq_quant_act": ([I, I64, I64, P, P, P, P], I),
        "tq_gemv_workspace_bytes": ([I, I64, I64, I64], SZ),
        "tq_gemv": ([I, I64, I64, I64, P, P, P, P, P, SZ, P], I),
        "tq_gemv_gate_up_swiglu": ([I, I64, I64, I64, P, P, P, P, P, P, SZ, P], I),
        "tq_gemm_workspace_bytes": ([I, I64, I64, I64], SZ),
        "tq_gemm": ([I, I64, I64, I64, P, P, P, P, P, SZ, P], I),
        "tq_debug_unpack": ([I, I64, I64, P, P, P], I),
        "tq_debug_group_sums": ([I, I64, I64, I64, P, P, P, I, P], I),
        "tq_gemv_quant_workspace_bytes": ([I, I64, I64, I], SZ),
        "tq_gemv_quant": ([I, I64, I64, P, P, I, P, P, I64, P, P, P, P, SZ, P], I),
        "tq_decode_stack_workspace_bytes": ([I, I64, I64, I64, I64, I64], SZ),
        "tq_decode_stack": ([I, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, SZ, P], I),
        "tq_decode_stack_persistent": ([I, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, SZ, P], I),
        "tq_decode_stack_batch_workspace_bytes": ([I, I64, I64, I64, I64, I64, I64], SZ),
        "tq_debug_gemv_quant_rows_sums": ([I, I64, I64, I64, P, P, I, P, P, I64, P, P, P], I),
        "tq_decode_stack_batch": ([I, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, SZ, P], I),
        "tq_gemv_noalloc": ([I, I64, I64, I64, P, P, P, P, P], I),
        "tq_noalloc_scratch_bytes": ([], SZ),
        "tq_hadamard_quant_act": ([I, I64, I64, P, P, P, P, P], I),
        "tq_ternarize": ([I64, I64, P, P, P], I),
        "tq_debug_stream_read": ([P, SZ, P, I64, P], I),
        "tq_debug_gate_up_sums": ([I, I64, I64, I64, P, P, P, P, P], I),
        "tq_debug_gemv_quant_sums": ([I, I64, I64, P, P, I, P, P, I64, P, P, P], I),
        "tq_workspace_clear": ([P, SZ, P], I),
        "tq_workspace_check": ([P, SZ, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def _check(rc: int, what: str):
    if rc != 0:
        raise TQError(rc, what)


def _ptr(t) -> int:
    """Device address of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def tq_status_str(status: int) -> str:
    return lib.tq_status_str(status).decode()


# ---- host: packed format ------------------------------------------------

def tq_packed_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib.tq_packed_bytes(fmt, N, K))


def tq_pack(fmt: int, trits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """trits int8 [N][K], scales fp16 bits uint16 [N][K/128] -> packed uint8 blob (host)."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = t.shape
    nbytes = tq_packed_bytes(fmt, N, K)
    out = np.empty(max(nbytes, 1), dtype=np.uint8)
    _check(lib.tq_pack(fmt, N, K, t.ctypes.data, s.ctypes.data, out.ctypes.data, nbytes),
           "tq_pack")
    return out


def tq_ternarize(w: np.ndarray):
    """fp32 weights [N][K] (host) -> (trits int8 [N][K], fp16 scale bits uint16 [N][K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    t = np.empty((N, K), dtype=np.int8)
    s = np.empty((N, max(K // GROUP, 1)), dtype=np.uint16)
    _check(lib.tq_ternarize(N, K, w.ctypes.data, t.ctypes.data, s.ctypes.data), "tq_ternarize")
    return t, s


def tq_unpack(fmt: int, blob: np.ndarray, N: int, K: int):
    """Inverse of tq_pack -> (trits int8 [N][K], scales uint16 [N][K/128])."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    t = np.empty((N, K), dtype=np.int8)
    s = np.empty((N, K // GROUP), dtype=np.uint16)
    _check(lib.tq_unpack(fmt, N, K, b.ctypes.data, b.size, t.ctypes.data, s.ctypes.data),
           "tq_unpack")
    return t, s


# ---- device ---------------------------------------------------------------

def tq_quant_act(x, q, a_scale, stream=None) -> None:
    """x [M][K] fp16/fp32 (device) -> q int8 [M][K], a_scale fp32 [M]."""
    import torch
    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(x.dtype, -1)
    M, K = x.shape
    _check(lib.tq_quant_act(dtype, M, K, _ptr(x), _ptr(q), _ptr(a_scale), _stream(stream)),
           "tq_quant_act")


def tq_hadamard_quant_act(x, signs, q, a_scale, stream=None) -> None:
    """x [M][K] fp16/fp32 (device), signs int8 [K] -> q int8 [M][K], a_scale
    fp32 [M] of the block-64 Hadamard-rotated rows."""
    import torch
    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(x.dtype, -1)
    M, K = x.shape
    _check(lib.tq_hadamard_quant_act(dtype, M, K, _ptr(x), _ptr(signs), _ptr(q), _ptr(a_scale),
                                     _stream(stream)), "tq_hadamard_quant_act")


def tq_gemv_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return int(lib.tq_gemv_workspace_bytes(fmt, M, N, K))


def tq_gemm_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return int(lib.tq_gemm_workspace_bytes(fmt, M, N, K))


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def tq_gemv(fmt, M, N, K, W, q, a_scale, y, ws=None, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib.tq_gemv(fmt, M, N, K, _ptr(W), _ptr(q), _ptr(a_scale), _ptr(y), wp, wb,
                       _stream(stream)), "tq_gemv")


def tq_gemv_noalloc(fmt, M, N, K, W, q, a_scale, y, stream=None) -> None:
    """tq_gemv with the library's own fixed device scratch array as workspace."""
    _check(lib.tq_gemv_noalloc(fmt, M, N, K, _ptr(W), _ptr(q), _ptr(a_scale), _ptr(y), _stream(stream)),
           "tq_gemv_noalloc")


def tq_gemv_gate_up_swiglu(fmt, M, N, K, Wg, Wu, q, a_scale, h, ws=None, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib.tq_gemv_gate_up_swiglu(fmt, M, N, K, _ptr(Wg), _ptr(Wu), _ptr(q), _ptr(a_scale),
                                      _ptr(h), wp, wb, _stream(stream)), "tq_gemv_gate_up_swiglu")


def tq_gemm(fmt, M, N, K, W, q, a_scale, y, ws=None, stream=None) -> None:
    wp, wb = _ws(ws)
    _check(lib.tq_gemm(fmt, M, N, K, _ptr(W), _ptr(q), _ptr(a_scale), _ptr(y), wp, wb,
                       _stream(stream)), "tq_gemm")


def tq_debug_unpack(fmt, N, K, W, trits, stream=None) -> None:
    _check(lib.tq_debug_unpack(fmt, N, K, _ptr(W), _ptr(trits), _stream(stream)),
           "tq_debug_unpack")


def tq_debug_group_sums(fmt, M, N, K, W, q, S, use_gemm_path=False, stream=None) -> None:
    _check(lib.tq_debug_group_sums(fmt, M, N, K, _ptr(W), _ptr(q), _ptr(S), int(use_gemm_path),
                                   _stream(stream)), "tq_debug_group_sums")


def tq_debug_gate_up_sums(fmt, M, N, K, Wg, Wu, q, S, stream=None) -> None:
    """S int32 [2][M][N][K/128]: the gate and up group sums of tq_gemv_gate_up_swiglu's kernel."""
    _check(lib.tq_debug_gate_up_sums(fmt, M, N, K, _ptr(Wg), _ptr(Wu), _ptr(q), _ptr(S),
                                     _stream(stream)), "tq_debug_gate_up_sums")


def tq_debug_gemv_quant_sums(fmt, N, K, W, Wu, x, S, x_bmax=None, a_scale=None, stream=None) -> None:
    """S int32 [nmat][N][K/128] (and a_scale fp32 [1]) from tq_gemv_quant's kernel,
    which quantises x (fp16 [K], or fp32 [K] with x_bmax) inside the launch."""
    import torch
    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(x.dtype, -1)
    nb = 0 if x_bmax is None else x_bmax.numel()
    _check(lib.tq_debug_gemv_quant_sums(fmt, N, K, _ptr(W), _ptr(Wu), dtype, _ptr(x), _ptr(x_bmax), nb,
                                        _ptr(S), _ptr(a_scale), _stream(stream)),
           "tq_debug_gemv_quant_sums")


def tq_debug_gemv_quant_rows_sums(fmt, rows, N, K, W, Wu, x, S, x_bmax=None, a_scale=None,
                                  stream=None) -> None:
    """S int32 [nmat][rows][N][K/128] (and a_scale fp32 [rows]) from the batch
    stack's kernel over `rows` token rows of x (fp16 [rows][K], or fp32 with
    x_bmax [rows][K/64])."""
    import torch
    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(x.dtype, -1)
    nb = 0 if x_bmax is None else K // 64
    _check(lib.tq_debug_gemv_quant_rows_sums(fmt, rows, N, K, _ptr(W), _ptr(Wu), dtype, _ptr(x),
                                             _ptr(x_bmax), nb, _ptr(S), _ptr(a_scale), _stream(stream)),
           "tq_debug_gemv_quant_rows_sums")


def tq_workspace_clear(ws, stream=None) -> None:
    """Zero-fill a workspace tensor (device, 16-byte aligned, size a multiple
    of 16 bytes) on the stream: the state every workspace-taking call expects."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.tq_workspace_clear(_ptr(ws), nbytes, _stream(stream)), "tq_workspace_clear")


def tq_workspace_check(ws, count, stream=None) -> None:
    """count (device int32/uint32 [>= 1]) receives the number of non-zero
    32-bit words of the workspace tensor ws (0: fit for the next call)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.tq_workspace_check(_ptr(ws), nbytes, _ptr(count), _stream(stream)), "tq_workspace_check")


def tq_debug_stream_read(src, sink, stream=None) -> None:
    """Read every byte of src (device tensor, size a multiple of 16) once;
    sink (int32/uint32 [>= TQ_STREAM_READ_WGS]) receives per-workgroup XORs."""
    nbytes = src.numel() * src.element_size()
    _check(lib.tq_debug_stream_read(_ptr(src), nbytes, _ptr(sink), sink.numel(), _stream(stream)),
           "tq_debug_stream_read")


def tq_gemv_quant_workspace_bytes(fmt, N, K, gate_up=False) -> int:
    return int(lib.tq_gemv_quant_workspace_bytes(fmt, N, K, int(bool(gate_up))))


def tq_gemv_quant(fmt, N, K, W, Wu, x, y, x_bmax=None, y_bmax=None, ws=None, stream=None,
                  y_signs=None) -> None:
    """y = W . quant(x) (or SwiGLU of W, Wu) for one token x [K] fp16 / fp32
    (device); fp32 x needs x_bmax, its K/64 block maxima.  y_signs (int8 [N])
    stores y Hadamard-rotated per 64-row block."""
    import torch
    dtype = {torch.float16: TQ_F16, torch.float32: TQ_F32}.get(x.dtype, -1)
    nb = 0 if x_bmax is None else x_bmax.numel()
    wp, wb = _ws(ws)
    _check(lib.tq_gemv_quant(fmt, N, K, _ptr(W), _ptr(Wu), dtype, _ptr(x), _ptr(x_bmax), nb,
                             _ptr(y), _ptr(y_bmax), _ptr(y_signs), wp, wb, _stream(stream)),
           "tq_gemv_quant")


def tq_decode_stack_workspace_bytes(fmt, layers, hidden, inter, qkv_out, o_in) -> int:
    return int(lib.tq_decode_stack_workspace_bytes(fmt, layers, hidden, inter, qkv_out, o_in))


def tq_decode_stack(fmt, layers, hidden, inter, qkv_out, o_in, weights, x_in, a_in,
                    y_qkv, y_o, h, y_out, ws, stream=None, ffn_signs=None, persistent=False) -> None:
    """weights: list of (qkv, o, gate, up, down) device tensors per layer (or a
    ctypes array of TqLayer built once with stack_layers()).  ffn_signs (int8
    [layers][hidden]) rotates the FFN input online.  persistent=True calls
    tq_decode_stack_persistent (one launch per 32 layers) instead of one
    launch per projection."""
    arr = weights if isinstance(weights, ctypes.Array) else stack_layers(weights)
    wp, wb = _ws(ws)
    fn = lib.tq_decode_stack_persistent if persistent else lib.tq_decode_stack
    _check(fn(fmt, layers, hidden, inter, qkv_out, o_in, ctypes.cast(arr, ctypes.c_void_p),
              _ptr(x_in), _ptr(a_in), _ptr(y_qkv), _ptr(y_o), _ptr(h), _ptr(y_out), _ptr(ffn_signs),
              wp, wb, _stream(stream)), "tq_decode_stack_persistent" if persistent else "tq_decode_stack")


def tq_decode_stack_batch_workspace_bytes(fmt, rows, layers, hidden, inter, qkv_out, o_in) -> int:
    return int(lib.tq_decode_stack_batch_workspace_bytes(fmt, rows, layers, hidden, inter, qkv_out, o_in))


def tq_decode_stack_batch(fmt, rows, layers, hidden, inter, qkv_out, o_in, weights, x_in, a_in,
                          y_qkv, y_o, h, y_out, ws, stream=None, ffn_signs=None) -> None:
    """tq_decode_stack for `rows` token rows per launch: x_in [layers][rows][hidden],
    a_in [layers][rows][o_in], outputs [layers][rows][N]."""
    arr = weights if isinstance(weights, ctypes.Array) else stack_layers(weights)
    wp, wb = _ws(ws)
    _check(lib.tq_decode_stack_batch(fmt, rows, layers, hidden, inter, qkv_out, o_in,
                                     ctypes.cast(arr, ctypes.c_void_p), _ptr(x_in), _ptr(a_in),
                                     _ptr(y_qkv), _ptr(y_o), _ptr(h), _ptr(y_out), _ptr(ffn_signs),
                                     wp, wb, _stream(stream)), "tq_decode_stack_batch")


def stack_timeouts(ws) -> int:
    """Waits of the persistent decode stack that gave up (the workspace's first
    32-bit word; 0 after correct calls).  Synchronises with the device."""
    return int(ws.view(-1)[0:1].view(-1).cpu().numpy().view("uint32")[0]) if ws is not None else 0


def stack_layers(weights):
    """Host array of TqLayer from [(qkv, o, gate, up, down), ...] device tensors."""
    arr = (TqLayer * len(weights))()
    for i, w in enumerate(weights):
        arr[i] = TqLayer(*[_ptr(t) for t in w])
    return arr


def workspace(fmt: int, M: int, N: int, K: int, device="cuda"):
    """A zero-filled workspace tensor sized for tq_gemv / tq_gemm on this shape
    (None when the shape needs none).  Allocation is the caller's: this helper
    uses torch, never the library."""
    import torch
    nbytes = max(tq_gemv_workspace_bytes(fmt, min(M, GEMV_MAX_M), N, K),
                 tq_gemm_workspace_bytes(fmt, M, N, K))
    if nbytes == 0:
        return None
    return torch.zeros((nbytes + 15) // 16 * 4, dtype=torch.int32, device=device)
