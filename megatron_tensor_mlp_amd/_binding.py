"""ctypes binding of libtpmlp (argument marshalling only).

Each ``tp_*`` function here has the name of the C entry point it calls.  It
reads sizes and leading dimensions off the torch tensors, checks that the
buffers are large enough for those sizes (the C library cannot see buffer
extents), and passes raw device pointers plus the current torch HIP stream.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded before libtpmlp so the process uses one HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtpmlp.so")

DTYPE = {torch.float32: 0, torch.bfloat16: 1}
ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "gelu_erf": 3, "swiglu": 4}
STATUS = ["TP_OK", "TP_ERR_NULL_POINTER", "TP_ERR_BAD_SHAPE", "TP_ERR_NOT_DIVISIBLE",
          "TP_ERR_BAD_SHARD", "TP_ERR_MISALIGNED", "TP_ERR_BAD_DTYPE", "TP_ERR_BAD_ACT",
          "TP_ERR_WORKSPACE", "TP_ERR_HIP"]


class TpError(RuntimeError):
    def __init__(self, status: int, message: str):
        name = STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


_lib = None


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libtpmlp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m megatron_tensor_mlp_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    ci = ctypes.c_int
    lib.tp_col_linear.argtypes = [ci, ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp, i64, vp,
                                  vp, i64, vp, sz, vp]
    lib.tp_row_linear.argtypes = [ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp, i64, vp, sz,
                                  vp]
    lib.tp_mlp_shard.argtypes = [ci, ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp, i64, vp,
                                 vp, i64, vp, i64, vp, i64, vp, sz, vp]
    lib.tp_mlp_shard_noalloc.argtypes = [ci, ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp,
                                         i64, vp, vp, i64, vp, i64, vp, i64, vp]
    lib.tp_partial_sum.argtypes = [i64, i64, i32, ctypes.POINTER(vp), i64, vp, vp, i64, vp]
    lib.tp_mlp_simulated.argtypes = [ci, ci, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64, vp,
                                     vp, i64, vp, vp, vp, vp, i64, vp, sz, vp]
    lib.tp_workspace_bytes.argtypes = [ci, ci, i64, i64, i64, i32]
    lib.tp_workspace_bytes.restype = sz
    lib.tp_shard_bounds.argtypes = [i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.tp_status_string.argtypes = [ci]
    lib.tp_status_string.restype = ctypes.c_char_p
    lib.tp_last_error_message.argtypes = []
    lib.tp_last_error_message.restype = ctypes.c_char_p
    lib.tp_abi_version.argtypes = []
    lib.tp_abi_version.restype = i32
    lib.tp_calib_mfma_bf16.argtypes = [i32, i64, vp, i32, vp]
    lib.tp_calib_hbm_read.argtypes = [vp, i64, vp, i32, vp]
    lib.tp_qkv_linear.argtypes = [ci, i64, i64, i32, i32, i64, i32, i32, vp, i64, vp, i64, vp,
                                  vp, i64, vp, sz, vp]
    lib.tp_qkv_workspace_bytes.argtypes = [ci, i64, i64, i32, i32, i64, i32]
    lib.tp_qkv_workspace_bytes.restype = sz
    lib.tp_col_linear_train.argtypes = [ci, ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp,
                                        i64, vp, vp, i64, vp, i64, vp]
    lib.tp_mlp_shard_backward.argtypes = [ci, ci, i64, i64, i64, i32, i32, vp, i64, vp, i64, vp,
                                          i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp,
                                          i64, vp, i64, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.tp_attention.argtypes = [ci, i64, i64, i32, i32, i64, i32, vp, i64, vp, i64, vp, i64,
                                 vp, i64, vp]
    lib.tp_backward_workspace_bytes.argtypes = [ci, ci, i64, i64, i64, i32, i32]
    lib.tp_backward_workspace_bytes.restype = sz
    cf = ctypes.c_float
    lib.tp_residual_layernorm.argtypes = [i64, i64, i32, ctypes.POINTER(vp), i64, vp, vp, i64, vp,
                                          i64, vp, vp, cf, vp, i64, vp]
    lib.tp_block_simulated.argtypes = [ci, ci, i64, i64, i64, i32, i32, i64, i64, i32, i32, cf,
                                       vp, i64, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp, vp, i64,
                                       vp, i64, vp, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.tp_block_workspace_bytes.argtypes = [ci, ci, i64, i64, i64, i32, i32, i64, i64, i32]
    lib.tp_block_workspace_bytes.restype = sz
    for name in ("tp_col_linear", "tp_row_linear", "tp_mlp_shard", "tp_partial_sum",
                 "tp_mlp_simulated", "tp_shard_bounds", "tp_calib_mfma_bf16", "tp_qkv_linear",
                 "tp_col_linear_train", "tp_mlp_shard_backward", "tp_attention",
                 "tp_residual_layernorm", "tp_block_simulated"):
        getattr(lib, name).restype = ci
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = library().tp_last_error_message().decode()
        raise TpError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ld(t, rows: int, cols: int, name: str) -> int:
    """Leading dimension of a row-major 2-D view, after checking it spans rows x cols."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} is {tuple(t.shape)}, needs at least ({rows}, {cols})")
    if rows > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], cols)


def _dt(t) -> int:
    if t.dtype not in DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPE[t.dtype]


def _act(act) -> int:
    return ACT[act] if isinstance(act, str) else int(act)


def tp_abi_version() -> int:
    return library().tp_abi_version()


def tp_calib_mfma_bf16(gaussian: bool, iters: int, stats, stream=None):
    """Enqueue the MFMA calibration kernel (include/tpmlp_calib.h): one
    workgroup per pair of entries of `stats` (a device int64 tensor of 2*nwg)."""
    if stats.dtype != torch.int64 or not stats.is_cuda or stats.numel() % 2:
        raise ValueError("stats must be a device int64 tensor of even length")
    _check(library().tp_calib_mfma_bf16(1 if gaussian else 0, iters, _ptr(stats),
                                        stats.numel() // 2, _stream(stream)))


def tp_calib_hbm_read(buf, sink, nbytes: int | None = None, stream=None):
    """Enqueue the streaming-read calibration kernel (include/tpmlp_calib.h) over
    the first nbytes (default all) of the device tensor `buf`; one workgroup per
    entry of `sink` (a device int32 tensor)."""
    if not sink.is_cuda or sink.dtype != torch.int32:
        raise ValueError("sink must be a device int32 tensor")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check(library().tp_calib_hbm_read(_ptr(buf), n, _ptr(sink), sink.numel(), _stream(stream)))


def tp_shard_bounds(k: int, i: int, p: int):
    """(c0, s): the block [c0, c0 + s) that shard i of p owns of a dimension of size k."""
    c0, s = ctypes.c_int64(), ctypes.c_int64()
    _check(library().tp_shard_bounds(k, i, p, ctypes.byref(c0), ctypes.byref(s)))
    return c0.value, s.value


def tp_workspace_bytes(dtype, act, T: int, d: int, k: int, p: int) -> int:
    dt = DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return library().tp_workspace_bytes(dt, _act(act), T, d, k, p)


_ws_cache: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """A zero-filled device buffer of at least nbytes, cached per device.  The
    library leaves its arrival counters zero after every call, so the buffer
    can be reused by later calls on the same stream."""
    if nbytes <= 0:
        return None
    dev = torch.device(device)
    buf = _ws_cache.get(dev)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[dev] = buf
    return buf


def _ws_args(ws, need, device):
    if ws is None:
        ws = workspace(need, device)
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def tp_col_linear(X, W1, i: int, p: int, Y, act="gelu_tanh", Wu=None, b1=None, ws=None,
                  stream=None):
    """Y <- act(X W1[:, i*s:(i+1)*s] + b1[i*s:(i+1)*s]) (or the SwiGLU pair), s = k/p."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldy = _ld(Y, T, s, "Y")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    need = tp_workspace_bytes(X.dtype, a, T, d, k, p)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_col_linear(_dt(X), a, T, d, k, i, p, _ptr(X), ldx, _ptr(W1), ldw1,
                                   _ptr(Wu), ldwu, _ptr(b1), _ptr(Y), ldy, wsp, wsn,
                                   _stream(stream)))
    return Y


def tp_row_linear(Y, W2, i: int, p: int, Z, ws=None, stream=None):
    """Z <- Y W2[i*s:(i+1)*s, :] (fp32 partial, no bias), s = k/p."""
    k, d = W2.shape
    T = Y.shape[0]
    s = k // p if p > 0 else 0
    ldy = _ld(Y, T, s, "Y")
    ldw2 = _ld(W2, k, d, "W2")
    ldz = _ld(Z, T, d, "Z")
    need = tp_workspace_bytes(Y.dtype, 0, T, d, k, p)
    wsp, wsn = _ws_args(ws, need, Y.device)
    _check(library().tp_row_linear(_dt(Y), T, d, k, i, p, _ptr(Y), ldy, _ptr(W2), ldw2, _ptr(Z),
                                   ldz, wsp, wsn, _stream(stream)))
    return Z


def tp_mlp_shard(X, W1, W2, i: int, p: int, Y, Z, act="gelu_tanh", Wu=None, b1=None, ws=None,
                 stream=None):
    """Y <- column step of shard i, Z <- row step (fp32 partial)."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldw2 = _ld(W2, k, d, "W2")
    ldy = _ld(Y, T, s, "Y")
    ldz = _ld(Z, T, d, "Z")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    need = tp_workspace_bytes(X.dtype, a, T, d, k, p)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_mlp_shard(_dt(X), a, T, d, k, i, p, _ptr(X), ldx, _ptr(W1), ldw1,
                                  _ptr(Wu), ldwu, _ptr(b1), _ptr(W2), ldw2, _ptr(Y), ldy,
                                  _ptr(Z), ldz, wsp, wsn, _stream(stream)))
    return Y, Z


def tp_mlp_shard_noalloc(X, W1, W2, i: int, p: int, Y, Z, act="gelu_tanh", Wu=None, b1=None,
                         stream=None):
    """tp_mlp_shard with the library's static scratch instead of a workspace (for
    callers that cannot allocate): Y <- column step of shard i, Z <- row step."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldw2 = _ld(W2, k, d, "W2")
    ldy = _ld(Y, T, s, "Y")
    ldz = _ld(Z, T, d, "Z")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    _check(library().tp_mlp_shard_noalloc(_dt(X), a, T, d, k, i, p, _ptr(X), ldx, _ptr(W1), ldw1,
                                          _ptr(Wu), ldwu, _ptr(b1), _ptr(W2), ldw2, _ptr(Y), ldy,
                                          _ptr(Z), ldz, _stream(stream)))
    return Y, Z


def tp_partial_sum(parts, Z, b2=None, stream=None):
    """Z <- ((parts[0] + parts[1]) + ...) (+ b2); parts are fp32 [T, d] views with one ld."""
    p = len(parts)
    T, d = Z.shape
    ldp = _ld(parts[0], T, d, "parts[0]") if p else d
    for q, t in enumerate(parts):
        if _ld(t, T, d, f"parts[{q}]") != ldp:
            raise ValueError("all partials must share one leading dimension")
    ldz = _ld(Z, T, d, "Z")
    if b2 is not None and b2.numel() < d:
        raise ValueError("b2 is shorter than d")
    arr = (ctypes.c_void_p * max(p, 1))(*[t.data_ptr() for t in parts])
    _check(library().tp_partial_sum(T, d, p, arr, ldp, _ptr(b2), _ptr(Z), ldz, _stream(stream)))
    return Z


def tp_mlp_simulated(X, W1, W2, p: int, Y, Zp, Z, act="gelu_tanh", Wu=None, b1=None, b2=None,
                     ws=None, stream=None):
    """All p shards on this device: Y [p, T, k/p], Zp [p, T, d] fp32, Z [T, d] fp32."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldw2 = _ld(W2, k, d, "W2")
    if not Y.is_contiguous() or Y.numel() < p * T * s:
        raise ValueError("Y must be a contiguous [p, T, k/p] buffer")
    if not Zp.is_contiguous() or Zp.numel() < p * T * d or Zp.dtype != torch.float32:
        raise ValueError("Zp must be a contiguous fp32 [p, T, d] buffer")
    ldz = _ld(Z, T, d, "Z")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    need = tp_workspace_bytes(X.dtype, a, T, d, k, p)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_mlp_simulated(_dt(X), a, T, d, k, p, _ptr(X), ldx, _ptr(W1), ldw1,
                                      _ptr(Wu), ldwu, _ptr(b1), _ptr(W2), ldw2, _ptr(b2),
                                      _ptr(Y), _ptr(Zp), _ptr(Z), ldz, wsp, wsn,
                                      _stream(stream)))
    return Z


def tp_qkv_workspace_bytes(dtype, T: int, d: int, Hq: int, Hkv: int, dh: int, p: int) -> int:
    dt = DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return library().tp_qkv_workspace_bytes(dt, T, d, Hq, Hkv, dh, p)


def tp_qkv_linear(X, Wqkv, Hq: int, Hkv: int, dh: int, i: int, p: int, QKV, bqkv=None, ws=None,
                  stream=None):
    """QKV <- [Q_i | K_i | V_i]: the query, key and value heads of head shard i of p
    projected from X; Wqkv is the full packed [d, (Hq + 2 Hkv) dh] weight."""
    T, d = X.shape
    ncol = (Hq + 2 * Hkv) * dh
    nout = ncol // p if p > 0 else 0
    ldx = _ld(X, T, d, "X")
    ldw = _ld(Wqkv, d, ncol, "Wqkv")
    ldo = _ld(QKV, T, nout, "QKV")
    if bqkv is not None and bqkv.numel() < ncol:
        raise ValueError("bqkv is shorter than (Hq + 2 Hkv) dh")
    need = tp_qkv_workspace_bytes(X.dtype, T, d, Hq, Hkv, dh, p)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_qkv_linear(_dt(X), T, d, Hq, Hkv, dh, i, p, _ptr(X), ldx, _ptr(Wqkv), ldw,
                                   _ptr(bqkv), _ptr(QKV), ldo, wsp, wsn, _stream(stream)))
    return QKV


def tp_col_linear_train(X, W1, i: int, p: int, Y, H, act="gelu_tanh", Wu=None, b1=None,
                        stream=None):
    """tp_col_linear, also writing the pre-activation H [T, k/p] (SwiGLU: [G | U], [T, 2k/p])."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldy = _ld(Y, T, s, "Y")
    ldh = _ld(H, T, 2 * s if a == ACT["swiglu"] else s, "H")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    _check(library().tp_col_linear_train(_dt(X), a, T, d, k, i, p, _ptr(X), ldx, _ptr(W1), ldw1,
                                         _ptr(Wu), ldwu, _ptr(b1), _ptr(Y), ldy, _ptr(H), ldh,
                                         _stream(stream)))
    return Y, H


def tp_backward_workspace_bytes(dtype, act, T: int, d: int, k: int, p: int, with_db1: bool) -> int:
    dt = DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return library().tp_backward_workspace_bytes(dt, _act(act), T, d, k, p, 1 if with_db1 else 0)


def tp_mlp_shard_backward(X, W1, W2, H, Y, dZ, i: int, p: int, dH, dXp, dW1, dW2,
                          act="gelu_tanh", Wu=None, dWu=None, db1=None, ws=None, stream=None):
    """Backward pass of shard i: dH (dt), dXp [T, d], dW1 [d, k/p], dWu, db1 [k/p], dW2 [k/p, d]
    (fp32), from X, the full weights, the saved H and Y, and dZ [T, d] (dt)."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p if p > 0 else 0
    a = _act(act)
    hw = 2 * s if a == ACT["swiglu"] else s
    ldx = _ld(X, T, d, "X")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldw2 = _ld(W2, k, d, "W2")
    ldh = _ld(H, T, hw, "H")
    ldy = _ld(Y, T, s, "Y")
    lddz = _ld(dZ, T, d, "dZ")
    lddh = _ld(dH, T, hw, "dH")
    lddx = _ld(dXp, T, d, "dXp")
    lddw1 = _ld(dW1, d, s, "dW1")
    lddwu = _ld(dWu, d, s, "dWu") if dWu is not None else 0
    lddw2 = _ld(dW2, s, d, "dW2")
    for name, t in (("dXp", dXp), ("dW1", dW1), ("dW2", dW2), ("dWu", dWu), ("db1", db1)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if db1 is not None and db1.numel() < s:
        raise ValueError("db1 is shorter than k/p")
    need = tp_backward_workspace_bytes(X.dtype, a, T, d, k, p, db1 is not None)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_mlp_shard_backward(
        _dt(X), a, T, d, k, i, p, _ptr(X), ldx, _ptr(W1), ldw1, _ptr(Wu), ldwu, _ptr(W2), ldw2,
        _ptr(H), ldh, _ptr(Y), ldy, _ptr(dZ), lddz, _ptr(dH), lddh, _ptr(dXp), lddx, _ptr(dW1),
        lddw1, _ptr(dWu), lddwu, _ptr(db1), _ptr(dW2), lddw2, wsp, wsn, _stream(stream)))
    return dH, dXp, dW1, dW2


def tp_attention(Q, K, V, O, Hq: int, Hkv: int, dh: int, S: int | None = None, causal=True,
                 stream=None):
    """O <- per-head softmax(Q K^T / sqrt(dh)) V (bf16) over sequences of S tokens (default:
    one sequence of T).  Q, O: [T, Hq dh] views, K, V: [T, Hkv dh] views (e.g. the column
    blocks of tp_qkv_linear's output)."""
    T = Q.shape[0]
    S = T if S is None else S
    if S < 0 or (S > 0 and T % S) or (S == 0 and T > 0):
        raise ValueError("T must be a whole number of sequences of S tokens")
    nseq = T // S if S > 0 else 0
    ldq = _ld(Q, T, Hq * dh, "Q")
    ldk = _ld(K, T, Hkv * dh, "K")
    ldv = _ld(V, T, Hkv * dh, "V")
    ldo = _ld(O, T, Hq * dh, "O")
    _check(library().tp_attention(_dt(Q), nseq, S, Hq, Hkv, dh, 1 if causal else 0, _ptr(Q), ldq,
                                  _ptr(K), ldk, _ptr(V), ldv, _ptr(O), ldo, _stream(stream)))
    return O


def _vec(t, n: int, name: str):
    """A 1-D fp32 parameter vector of at least n elements, or None."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous fp32 vector of at least {n} elements")
    return t


def tp_residual_layernorm(parts=(), X=None, A=None, bias=None, R=None, gamma=None, beta=None,
                          eps: float = 1e-5, stream=None):
    """x = (((parts[0] + ...) + bias) + R) in fp32, left to right; X <- x (fp32 [T, d]);
    A <- LayerNorm(x) * gamma + beta (bf16 [T, d]).  Returns (X, A)."""
    ref = next((t for t in (list(parts) + [R, X, A]) if t is not None), None)
    if ref is None:
        raise ValueError("no tensor to take the shape from")
    T, d = ref.shape
    p = len(parts)
    ldp = _ld(parts[0], T, d, "parts[0]") if p else d
    for q, t in enumerate(parts):
        if t.dtype != torch.float32 or _ld(t, T, d, f"parts[{q}]") != ldp:
            raise ValueError("partials must be fp32 and share one leading dimension")
    ldr = _ld(R, T, d, "R") if R is not None else d
    ldx = _ld(X, T, d, "X") if X is not None else d
    lda = _ld(A, T, d, "A") if A is not None else d
    for name, t in (("R", R), ("X", X)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be fp32")
    if A is not None and A.dtype != torch.bfloat16:
        raise ValueError("A must be bf16")
    _vec(bias, d, "bias"), _vec(gamma, d, "gamma"), _vec(beta, d, "beta")
    arr = (ctypes.c_void_p * max(p, 1))(*[t.data_ptr() for t in parts])
    _check(library().tp_residual_layernorm(T, d, p, arr, ldp, _ptr(bias), _ptr(R), ldr, _ptr(X),
                                           ldx, _ptr(gamma), _ptr(beta), float(eps), _ptr(A), lda,
                                           _stream(stream)))
    return X, A


def tp_block_workspace_bytes(dtype, act, nseq: int, S: int, d: int, Hq: int, Hkv: int, dh: int,
                             k: int, p: int) -> int:
    dt = DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return library().tp_block_workspace_bytes(dt, _act(act), nseq, S, d, Hq, Hkv, dh, k, p)


def tp_block_simulated(X, Hq: int, Hkv: int, dh: int, p: int, ln1, Wqkv, WO, ln2, W1, W2, Out,
                       S=None, causal=True, eps: float = 1e-5, act="gelu_tanh", bqkv=None,
                       bO=None, Wu=None, b1=None, b2=None, ws=None, stream=None):
    """One pre-LayerNorm transformer block of p tensor-parallel shards on this device.
    X, Out fp32 [T, d] (T = nseq * S); ln1, ln2 = (gamma, beta) fp32 [d]; Wqkv, WO, W1,
    (Wu,) W2 bf16 full matrices; bO, b2 fp32 [d] or None; bqkv, b1 bf16 or None."""
    T, d = X.shape
    S = T if S is None else S
    if S <= 0 or T % S:
        raise ValueError("T must be a whole number of sequences of S tokens")
    nseq = T // S
    k = W1.shape[1]
    a = _act(act)
    ncol = (Hq + 2 * Hkv) * dh
    if X.dtype != torch.float32 or Out.dtype != torch.float32:
        raise ValueError("X and Out must be fp32")
    ldx = _ld(X, T, d, "X")
    ldout = _ld(Out, T, d, "Out")
    ldq = _ld(Wqkv, d, ncol, "Wqkv")
    ldo = _ld(WO, Hq * dh, d, "WO")
    ldw1 = _ld(W1, d, k, "W1")
    ldwu = _ld(Wu, d, k, "Wu") if Wu is not None else 0
    ldw2 = _ld(W2, k, d, "W2")
    for name, t, n in (("ln1 gamma", ln1[0], d), ("ln1 beta", ln1[1], d), ("ln2 gamma", ln2[0], d),
                       ("ln2 beta", ln2[1], d), ("bO", bO, d), ("b2", b2, d)):
        _vec(t, n, name)
    if bqkv is not None and bqkv.numel() < ncol:
        raise ValueError("bqkv is shorter than (Hq + 2 Hkv) dh")
    if b1 is not None and b1.numel() < k:
        raise ValueError("b1 is shorter than k")
    need = tp_block_workspace_bytes(Wqkv.dtype, a, nseq, S, d, Hq, Hkv, dh, k, p)
    wsp, wsn = _ws_args(ws, need, X.device)
    _check(library().tp_block_simulated(
        _dt(Wqkv), a, nseq, S, d, Hq, Hkv, dh, k, p, 1 if causal else 0, float(eps), _ptr(X), ldx,
        _ptr(ln1[0]), _ptr(ln1[1]), _ptr(Wqkv), ldq, _ptr(bqkv), _ptr(WO), ldo, _ptr(bO),
        _ptr(ln2[0]), _ptr(ln2[1]), _ptr(W1), ldw1, _ptr(Wu), ldwu, _ptr(b1), _ptr(W2), ldw2,
        _ptr(b2), _ptr(Out), ldout, wsp, wsn, _stream(stream)))
    return Out
