"""Host-side tests of the C ABI: the library loads, exports what include/*.h
declare, does its shard bookkeeping, and rejects bad arguments before any
launch.  No GPU is used: the error-path cases pass fake (never dereferenced)
pointers and are skipped whenever a GPU is visible, so no kernel can ever see
them."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import megatron_tensor_mlp_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpmlp.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-pointer error paths run only where no GPU is visible")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tp_col_linear", "tp_row_linear", "tp_mlp_shard", "tp_partial_sum",
              "tp_mlp_simulated", "tp_workspace_bytes", "tp_shard_bounds", "tp_status_string",
              "tp_last_error_message", "tp_abi_version", "tp_calib_mfma_bf16", "tp_qkv_linear",
              "tp_qkv_workspace_bytes", "tp_attention", "tp_residual_layernorm",
              "tp_block_simulated", "tp_block_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = tp.library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", tp.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (tp_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_library_is_gfx950():
    """The fat binary carries gfx950 code objects (the offload bundle's target id)."""
    blob = open(tp.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_abi_version_matches_header():
    m = re.search(r"#define TPMLP_ABI_VERSION (\d+)", open(HEADER).read())
    assert tp.tp_abi_version() == int(m.group(1))


def test_status_strings():
    lib = tp.library()
    for code, name in enumerate(tp._binding.STATUS):
        assert lib.tp_status_string(code).decode() == name
    assert lib.tp_status_string(99).decode() == "TP_UNKNOWN_STATUS"


def test_shard_bounds_llama_tp8(golden):
    """'What is Tensor Parallelism?', Llama 3.1 70B worked example: 3584 columns per GPU."""
    g = golden("llama70b_tp8_shapes.txt")
    k, p, s = int(g["ffn_size"]), int(g["tp"]), int(g["ffn_columns_per_gpu"])
    for i in range(p):
        assert tp.tp_shard_bounds(k, i, p) == (i * s, s)


def test_shard_bounds_errors():
    """'Tensor Parallelism Explained', section 4: 64 heads over TP = 5 fails at startup;
    the same divisibility rule applies to the sharded hidden dimension."""
    with pytest.raises(tp.TpError) as e:
        tp.tp_shard_bounds(64, 0, 5)
    assert e.value.name == "TP_ERR_NOT_DIVISIBLE"
    assert "divisible" in str(e.value)
    for p in (1, 2, 4, 8):
        assert tp.tp_shard_bounds(64, p - 1, p) == ((p - 1) * (64 // p), 64 // p)
    for (k, i, p) in ((64, 4, 4), (64, -1, 4), (64, 0, 0), (64, 0, 65)):
        with pytest.raises(tp.TpError) as e:
            tp.tp_shard_bounds(k, i, p)
        assert e.value.name == "TP_ERR_BAD_SHARD"


def test_workspace_bytes():
    bf16 = torch.bfloat16
    # many tokens, many tiles: tiled path, no workspace
    assert tp.tp_workspace_bytes(bf16, "swiglu", 4096, 8192, 28672, 8) == 0
    assert tp.tp_workspace_bytes(torch.float32, "gelu_tanh", 4, 512, 2048, 4) == 0
    # decode shapes split K and need partial sums + arrival counters
    for T in (1, 8, 64):
        assert tp.tp_workspace_bytes(bf16, "swiglu", T, 8192, 28672, 8) > 0
    # invalid arguments report 0
    assert tp.tp_workspace_bytes(bf16, "swiglu", 8, 8192, 28672, 5) == 0
    assert tp.tp_workspace_bytes(bf16, 9, 8, 8192, 28672, 8) == 0


# --- fake-pointer error paths (validation happens before any launch) --------
A = 0x10000  # 16-byte aligned, never dereferenced
MIS = A + 2  # misaligned
P = ctypes.c_void_p


def col(dt=1, act=2, T=4, d=64, k=128, i=0, p=2, X=A, ldx=64, W1=A, ldw1=128, Wu=None, ldwu=0,
        b1=None, Y=A, ldy=64, ws=None, wsb=0):
    return tp.library().tp_col_linear(dt, act, T, d, k, i, p, P(X), ldx, P(W1), ldw1, P(Wu), ldwu,
                                      P(b1), P(Y), ldy, P(ws), wsb, None)


def status_name(code):
    return tp._binding.STATUS[code]


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(k=129, ldw1=136), "TP_ERR_NOT_DIVISIBLE"),   # k % p != 0
    (dict(i=2), "TP_ERR_BAD_SHARD"),
    (dict(i=-1), "TP_ERR_BAD_SHARD"),
    (dict(p=0), "TP_ERR_BAD_SHARD"),
    (dict(p=65, k=65 * 8, ldw1=65 * 8), "TP_ERR_BAD_SHARD"),
    (dict(T=-1), "TP_ERR_BAD_SHAPE"),
    (dict(d=0), "TP_ERR_BAD_SHAPE"),
    (dict(k=0), "TP_ERR_BAD_SHAPE"),
    (dict(X=None), "TP_ERR_NULL_POINTER"),
    (dict(W1=None), "TP_ERR_NULL_POINTER"),
    (dict(Y=None), "TP_ERR_NULL_POINTER"),
    (dict(X=MIS), "TP_ERR_MISALIGNED"),
    (dict(ldx=60), "TP_ERR_BAD_SHAPE"),
    (dict(ldx=68), "TP_ERR_MISALIGNED"),
    (dict(d=60, ldx=64), "TP_ERR_MISALIGNED"),       # d not a multiple of 8 (bf16)
    (dict(k=136, ldw1=136), "TP_ERR_MISALIGNED"),    # k/p = 68
    (dict(ldy=32), "TP_ERR_BAD_SHAPE"),
    (dict(dt=7), "TP_ERR_BAD_DTYPE"),
    (dict(act=9), "TP_ERR_BAD_ACT"),
    (dict(act=4), "TP_ERR_NULL_POINTER"),             # SwiGLU without Wu
    (dict(act=4, Wu=A, ldwu=128, b1=A), "TP_ERR_BAD_ACT"),  # bias with SwiGLU
    (dict(b1=MIS), "TP_ERR_MISALIGNED"),
    (dict(T=1, d=8192, ldx=8192, k=28672, ldw1=28672, p=8, ldy=3584), "TP_ERR_WORKSPACE"),
    (dict(T=100, ldx=1 << 21), "TP_ERR_BAD_SHAPE"),     # beyond the tiled kernels' offsets
    (dict(T=4, ldw1=1 << 23), "TP_ERR_BAD_SHAPE"),      # beyond the few-token kernels' offsets
])
def test_col_linear_rejects(kw, expect):
    assert status_name(col(**kw)) == expect
    assert tp.library().tp_last_error_message().decode() != ""


@no_gpu
def test_fp32_alignment_rule_is_four():
    # fp32: d = 60 is allowed (multiple of 4), but a misaligned ld is not
    assert status_name(col(dt=0, d=60, ldx=60, T=0)) == "TP_OK"
    assert status_name(col(dt=0, ldx=66)) == "TP_ERR_MISALIGNED"


@no_gpu
def test_zero_tokens_launch_nothing():
    assert status_name(col(T=0)) == "TP_OK"
    lib = tp.library()
    assert lib.tp_last_error_message().decode() == ""
    st = lib.tp_row_linear(1, 0, 64, 128, 0, 2, P(A), 64, P(A), 64, P(A), 64, None, 0, None)
    assert status_name(st) == "TP_OK"
    # with no tokens the token-sized buffers may be NULL (empty torch tensors are)
    assert status_name(col(T=0, X=None, Y=None)) == "TP_OK"
    st = lib.tp_row_linear(1, 0, 64, 128, 0, 2, None, 64, P(A), 64, None, 64, None, 0, None)
    assert status_name(st) == "TP_OK"
    assert status_name(col(T=0, W1=None)) == "TP_ERR_NULL_POINTER"


@no_gpu
@pytest.mark.parametrize("args,expect", [
    (dict(k=129), "TP_ERR_NOT_DIVISIBLE"),
    (dict(Z=None), "TP_ERR_NULL_POINTER"),
    (dict(ldz=60), "TP_ERR_BAD_SHAPE"),
    (dict(ldw2=60), "TP_ERR_BAD_SHAPE"),
    (dict(Y=MIS), "TP_ERR_MISALIGNED"),
])
def test_row_linear_rejects(args, expect):
    a = dict(dt=1, T=4, d=64, k=128, i=0, p=2, Y=A, ldy=64, W2=A, ldw2=64, Z=A, ldz=64)
    a.update(args)
    st = tp.library().tp_row_linear(a["dt"], a["T"], a["d"], a["k"], a["i"], a["p"], P(a["Y"]),
                                    a["ldy"], P(a["W2"]), a["ldw2"], P(a["Z"]), a["ldz"], None, 0,
                                    None)
    assert status_name(st) == expect


@no_gpu
def test_partial_sum_rejects():
    lib = tp.library()
    arr = (ctypes.c_void_p * 3)(A, A, None)
    assert status_name(lib.tp_partial_sum(4, 64, 3, arr, 64, None, P(A), 64, None)) \
        == "TP_ERR_NULL_POINTER"
    arr = (ctypes.c_void_p * 2)(A, MIS)
    assert status_name(lib.tp_partial_sum(4, 64, 2, arr, 64, None, P(A), 64, None)) \
        == "TP_ERR_MISALIGNED"
    arr = (ctypes.c_void_p * 2)(A, A)
    assert status_name(lib.tp_partial_sum(4, 62, 2, arr, 64, None, P(A), 64, None)) \
        == "TP_ERR_MISALIGNED"
    assert status_name(lib.tp_partial_sum(4, 64, 0, arr, 64, None, P(A), 64, None)) \
        == "TP_ERR_BAD_SHARD"
    assert status_name(lib.tp_partial_sum(4, 64, 65, arr, 64, None, P(A), 64, None)) \
        == "TP_ERR_BAD_SHARD"
    assert status_name(lib.tp_partial_sum(0, 64, 2, arr, 64, None, P(A), 64, None)) == "TP_OK"


@no_gpu
def test_simulated_rejects_page_example_degree():
    """p = 5 does not divide k = 320 ... but 320 / 5 = 64 does; the page's 64 over 5
    is the failing case: k = 64, p = 5."""
    lib = tp.library()
    st = lib.tp_mlp_simulated(1, 2, 4, 64, 64, 5, P(A), 64, P(A), 64, None, 0, None, P(A), 64,
                              None, P(A), P(A), P(A), 64, None, 0, None)
    assert status_name(st) == "TP_ERR_NOT_DIVISIBLE"


@no_gpu
def test_calibration_errors():
    lib = tp.library()
    assert status_name(lib.tp_calib_mfma_bf16(1, 0, P(A), 4, None)) == "TP_ERR_BAD_SHAPE"
    assert status_name(lib.tp_calib_mfma_bf16(1, 10, P(A), 0, None)) == "TP_ERR_BAD_SHAPE"
    assert status_name(lib.tp_calib_mfma_bf16(0, 10, None, 4, None)) == "TP_ERR_NULL_POINTER"


# --- attention projections ---------------------------------------------------
def qkv(dt=1, T=4, d=64, Hq=8, Hkv=2, dh=16, i=0, p=2, X=A, ldx=64, W=A, ldw=192, b=None, O=A,
        ldo=96, ws=None, wsb=0):
    return tp.library().tp_qkv_linear(dt, T, d, Hq, Hkv, dh, i, p, P(X), ldx, P(W), ldw, P(b),
                                      P(O), ldo, P(ws), wsb, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(Hkv=1, ldw=160), "TP_ERR_NOT_DIVISIBLE"),     # 1 key/value head over 2 GPUs
    (dict(Hq=5, ldw=144, ldo=72), "TP_ERR_NOT_DIVISIBLE"),
    (dict(i=2), "TP_ERR_BAD_SHARD"),
    (dict(p=0), "TP_ERR_BAD_SHARD"),
    (dict(p=65), "TP_ERR_BAD_SHARD"),
    (dict(T=-1), "TP_ERR_BAD_SHAPE"),
    (dict(d=0), "TP_ERR_BAD_SHAPE"),
    (dict(Hq=0), "TP_ERR_BAD_SHAPE"),
    (dict(Hkv=0), "TP_ERR_BAD_SHAPE"),
    (dict(dh=0), "TP_ERR_BAD_SHAPE"),
    (dict(dh=12, ldw=144, ldo=72), "TP_ERR_MISALIGNED"),   # head width not a multiple of 8
    (dict(d=60), "TP_ERR_MISALIGNED"),
    (dict(ldw=184), "TP_ERR_BAD_SHAPE"),              # narrower than (Hq + 2 Hkv) dh
    (dict(ldo=88), "TP_ERR_BAD_SHAPE"),               # narrower than the shard's columns
    (dict(ldx=60), "TP_ERR_BAD_SHAPE"),
    (dict(X=None), "TP_ERR_NULL_POINTER"),
    (dict(W=None), "TP_ERR_NULL_POINTER"),
    (dict(O=None), "TP_ERR_NULL_POINTER"),
    (dict(b=MIS), "TP_ERR_MISALIGNED"),
    (dict(dt=5), "TP_ERR_BAD_DTYPE"),
    (dict(T=1, d=8192, ldx=8192, Hq=64, Hkv=8, dh=128, ldw=10240, p=8, ldo=1280),
     "TP_ERR_WORKSPACE"),
    (dict(T=4, ldw=1 << 23), "TP_ERR_BAD_SHAPE"),      # beyond the few-token kernels' offsets
])
def test_qkv_linear_rejects(kw, expect):
    assert status_name(qkv(**kw)) == expect
    assert tp.library().tp_last_error_message().decode() != ""


@no_gpu
def test_qkv_zero_tokens_and_fp32_alignment():
    assert status_name(qkv(T=0, X=None, O=None)) == "TP_OK"
    assert status_name(qkv(T=0, W=None)) == "TP_ERR_NULL_POINTER"
    # fp32: a head width of 12 is allowed (multiple of 4)
    assert status_name(qkv(dt=0, T=0, dh=12, ldw=144, ldo=72)) == "TP_OK"


# The tiled path's split-K plan, seen through the workspace it needs: the
# counter area, then one 256 x 256 fp32 partial slot per tile and k-range.
CTR = 256 << 10
SLOT = 256 * 256 * 4


def test_tiled_split_k_plan():
    """A many-token GEMM of t <= 120 tiles of 256 rows splits K into
    S = min(240 // t, 4 (8 when t <= 20), K // 768) k-ranges per tile, if
    that is 2 or more."""
    bf16 = torch.bfloat16
    qkv = lambda *a: tp.tp_qkv_workspace_bytes(bf16, *a)  # noqa: E731
    # Llama-70B QKV shard, T = 4096: 16 x 5 tiles, 3 k-ranges of d = 8192
    assert qkv(4096, 8192, 64, 8, 128, 8) == CTR + 80 * 3 * SLOT
    # T = 2048: 8 x 5 tiles, 4 ranges (6 would fit: at most 4 above 20 tiles)
    assert qkv(2048, 8192, 64, 8, 128, 8) == CTR + 40 * 4 * SLOT
    # 4 x 5 tiles: 12 would fit, 8 at most
    assert qkv(1000, 8192, 8, 1, 128, 1) == CTR + 20 * 8 * SLOT
    # 120 tiles (4 x 30) split in 2; 121 (11 x 11) not at all
    assert qkv(1024, 8192, 58, 1, 128, 1) == CTR + 120 * 2 * SLOT
    assert qkv(2816, 8192, 20, 1, 128, 1) == 0
    # K: 2 ranges need K >= 1536
    assert qkv(4096, 3072, 64, 8, 128, 8) == CTR + 80 * 3 * SLOT
    assert qkv(4096, 1528, 64, 8, 128, 8) == 0
    assert tp.tp_qkv_workspace_bytes(torch.float32, 4096, 8192, 64, 8, 128, 8) == 0
    # MLP shard, T = 300, Llama-70B width: column 2 x 28 tiles in 4 ranges,
    # row 2 x 32 tiles in 3 (K = 3584); the larger of the two
    mlp = lambda *a: tp.tp_workspace_bytes(bf16, *a)  # noqa: E731
    assert mlp("swiglu", 300, 8192, 3584, 1) == CTR + 56 * 4 * SLOT
    # the same shard as one of p = 8 (the simulated launches group 8 x 56
    # tiles and do not split)
    assert mlp("swiglu", 300, 8192, 28672, 8) == CTR + 56 * 4 * SLOT
    # one tile, K = 12296: 8 ranges; the simulated launch groups the 4 shards'
    # tiles (4 x 8 slots)
    assert mlp("none", 65, 12296, 1024, 4) == CTR + 4 * 8 * SLOT
    # the headline shard: 448 and 512 tiles, no split
    assert mlp("swiglu", 4096, 8192, 28672, 8) == 0


def test_qkv_workspace_bytes():
    bf16 = torch.bfloat16
    assert tp.tp_qkv_workspace_bytes(bf16, 4096, 4096, 32, 32, 128, 4) == 0  # 16 x 12 tiles
    for T in (1, 8, 64):
        assert tp.tp_qkv_workspace_bytes(bf16, T, 8192, 64, 8, 128, 8) > 0
    assert tp.tp_qkv_workspace_bytes(torch.float32, 8, 8192, 64, 8, 128, 8) == 0
    # invalid arguments report 0 and leave the last error message alone
    lib = tp.library()
    assert status_name(lib.tp_shard_bounds(64, 0, 5, ctypes.byref(ctypes.c_int64()),
                                           ctypes.byref(ctypes.c_int64()))) \
        == "TP_ERR_NOT_DIVISIBLE"
    msg = lib.tp_last_error_message().decode()
    assert tp.tp_qkv_workspace_bytes(bf16, 8, 8192, 64, 8, 128, 16) == 0   # 8 kv heads / 16
    assert tp.tp_qkv_workspace_bytes(bf16, 8, 8192, 64, 8, 120, 8) > 0     # dh = 120 is aligned
    assert tp.tp_qkv_workspace_bytes(bf16, 8, 8192, 64, 8, 100, 8) == 0    # dh = 100 misaligned
    assert lib.tp_last_error_message().decode() == msg


# --- training forward and backward --------------------------------------------
def train(dt=1, act=2, T=4, d=64, k=128, i=0, p=2, X=A, ldx=64, W1=A, ldw1=128, Wu=None, ldwu=0,
          b1=None, Y=A, ldy=64, H=A, ldh=64):
    return tp.library().tp_col_linear_train(dt, act, T, d, k, i, p, P(X), ldx, P(W1), ldw1, P(Wu),
                                            ldwu, P(b1), P(Y), ldy, P(H), ldh, None)


def bwd(dt=1, act=2, T=4, d=64, k=128, i=0, p=2, X=A, ldx=64, W1=A, ldw1=128, Wu=None, ldwu=0,
        W2=A, ldw2=64, H=A, ldh=64, Y=A, ldy=64, dZ=A, lddz=64, dH=A, lddh=64, dXp=A, lddx=64,
        dW1=A, lddw1=64, dWu=None, lddwu=0, db1=None, dW2=A, lddw2=64, ws=None, wsb=0):
    return tp.library().tp_mlp_shard_backward(
        dt, act, T, d, k, i, p, P(X), ldx, P(W1), ldw1, P(Wu), ldwu, P(W2), ldw2, P(H), ldh, P(Y),
        ldy, P(dZ), lddz, P(dH), lddh, P(dXp), lddx, P(dW1), lddw1, P(dWu), lddwu, P(db1), P(dW2),
        lddw2, P(ws), wsb, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(H=None), "TP_ERR_NULL_POINTER"),
    (dict(ldh=60), "TP_ERR_BAD_SHAPE"),
    (dict(act=4, Wu=A, ldwu=128), "TP_ERR_BAD_SHAPE"),     # SwiGLU keeps [G | U]: ldh >= 2 k/p
    (dict(k=129, ldw1=136), "TP_ERR_NOT_DIVISIBLE"),
    (dict(H=MIS), "TP_ERR_MISALIGNED"),
])
def test_col_linear_train_rejects(kw, expect):
    assert status_name(train(**kw)) == expect


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(k=129, ldw1=136), "TP_ERR_NOT_DIVISIBLE"),
    (dict(i=2), "TP_ERR_BAD_SHARD"),
    (dict(dZ=None), "TP_ERR_NULL_POINTER"),
    (dict(dW1=None), "TP_ERR_NULL_POINTER"),
    (dict(dW2=None), "TP_ERR_NULL_POINTER"),
    (dict(act=4, Wu=A, ldwu=128, ldh=128, lddh=128), "TP_ERR_NULL_POINTER"),   # no dWu
    (dict(act=4, Wu=A, ldwu=128, dWu=A, lddwu=64), "TP_ERR_BAD_SHAPE"),        # dH narrower than 2s
    (dict(act=4, Wu=A, ldwu=128, dWu=A, lddwu=64, ldh=128, lddh=128, db1=A),
     "TP_ERR_BAD_ACT"),                                                         # no db1 with SwiGLU
    (dict(lddw2=60), "TP_ERR_BAD_SHAPE"),
    (dict(lddw1=60), "TP_ERR_BAD_SHAPE"),
    (dict(lddx=60), "TP_ERR_BAD_SHAPE"),
    (dict(ldw2=60), "TP_ERR_BAD_SHAPE"),
    (dict(dXp=MIS), "TP_ERR_MISALIGNED"),
    (dict(db1=A), "TP_ERR_WORKSPACE"),                     # the bias gradient needs a workspace
    (dict(dt=3), "TP_ERR_BAD_DTYPE"),
])
def test_backward_rejects(kw, expect):
    assert status_name(bwd(**kw)) == expect
    assert tp.library().tp_last_error_message().decode() != ""


def test_backward_workspace_bytes():
    bf16 = torch.bfloat16
    assert tp.tp_backward_workspace_bytes(bf16, "gelu_tanh", 4096, 8192, 28672, 8, True) \
        == (256 << 10) + 64 * 3584 * 4
    assert tp.tp_backward_workspace_bytes(bf16, "gelu_tanh", 4096, 8192, 28672, 8, False) == 0
    assert tp.tp_backward_workspace_bytes(bf16, "swiglu", 4096, 8192, 28672, 8, True) == 0
    assert tp.tp_backward_workspace_bytes(bf16, "gelu_tanh", 4096, 8192, 28672, 5, True) == 0


def attn(dt=1, nseq=1, S=64, Hq=4, Hkv=2, dh=128, causal=1, Q=A, ldq=1024, K=A, ldk=1024, V=A,
         ldv=1024, O=A, ldo=512):
    return tp.library().tp_attention(dt, nseq, S, Hq, Hkv, dh, causal, P(Q), ldq, P(K), ldk, P(V),
                                     ldv, P(O), ldo, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(dt=0), "TP_ERR_BAD_DTYPE"),          # bf16 only
    (dict(Hkv=3), "TP_ERR_NOT_DIVISIBLE"),
    (dict(dh=96, ldq=384, ldo=384), "TP_ERR_BAD_SHAPE"),
    (dict(Hq=0), "TP_ERR_BAD_SHAPE"),
    (dict(S=-1), "TP_ERR_BAD_SHAPE"),
    (dict(ldo=500), "TP_ERR_BAD_SHAPE"),
    (dict(ldk=200), "TP_ERR_BAD_SHAPE"),
    (dict(ldq=1028), "TP_ERR_MISALIGNED"),
    (dict(Q=None), "TP_ERR_NULL_POINTER"),
    (dict(V=MIS), "TP_ERR_MISALIGNED"),
])
def test_attention_rejects(kw, expect):
    assert status_name(attn(**kw)) == expect


@no_gpu
def test_attention_empty_is_ok():
    assert status_name(attn(nseq=0, Q=None, K=None, V=None, O=None)) == "TP_OK"
    assert status_name(attn(S=0, Q=None, K=None, V=None, O=None)) == "TP_OK"


def rln(T=4, d=64, p=2, parts=(A, A), ldp=64, bias=None, R=A, ldr=64, X=A, ldx=64, gamma=A,
        beta=A, eps=1e-5, Aout=A, lda=64):
    arr = (P * max(len(parts), 1))(*[P(x) for x in parts])
    return tp.library().tp_residual_layernorm(T, d, p, arr if parts is not None else None, ldp,
                                              P(bias), P(R), ldr, P(X), ldx, P(gamma), P(beta),
                                              eps, P(Aout), lda, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(T=-1), "TP_ERR_BAD_SHAPE"),
    (dict(d=0), "TP_ERR_BAD_SHAPE"),
    (dict(d=16392, ldp=16392, ldr=16392, ldx=16392, lda=16392), "TP_ERR_BAD_SHAPE"),  # > 16384
    (dict(d=60), "TP_ERR_MISALIGNED"),
    (dict(p=65), "TP_ERR_BAD_SHARD"),
    (dict(p=-1), "TP_ERR_BAD_SHARD"),
    (dict(p=0, parts=(), R=None), "TP_ERR_BAD_SHAPE"),          # nothing to add
    (dict(X=None, Aout=None, gamma=None, beta=None), "TP_ERR_BAD_SHAPE"),  # no output
    (dict(gamma=None), "TP_ERR_NULL_POINTER"),                  # A without gamma
    (dict(beta=None), "TP_ERR_NULL_POINTER"),
    (dict(eps=-1.0), "TP_ERR_BAD_SHAPE"),
    (dict(eps=float("inf")), "TP_ERR_BAD_SHAPE"),
    (dict(ldp=60), "TP_ERR_BAD_SHAPE"),
    (dict(lda=68), "TP_ERR_MISALIGNED"),
    (dict(parts=(A, None)), "TP_ERR_NULL_POINTER"),
    (dict(R=MIS), "TP_ERR_MISALIGNED"),
    (dict(bias=MIS), "TP_ERR_MISALIGNED"),
])
def test_residual_layernorm_rejects(kw, expect):
    assert status_name(rln(**kw)) == expect


@no_gpu
def test_residual_layernorm_empty_is_ok():
    assert status_name(rln(T=0, parts=(None, None), R=None, X=None, Aout=A)) == "TP_OK"
    assert status_name(rln(T=0, parts=(None, None), R=None, X=None, Aout=None, gamma=None,
                           beta=None)) == "TP_OK"


def blk(dt=1, act=2, nseq=1, S=64, d=64, Hq=4, Hkv=2, dh=64, k=128, p=2, causal=1, eps=1e-5,
        X=A, ldx=64, g1=A, b1n=A, Wqkv=A, ldq=512, bqkv=None, WO=A, ldo=64, bO=None, g2=A, b2n=A,
        W1=A, ldw1=128, Wu=None, ldwu=0, b1=None, W2=A, ldw2=64, b2=None, Out=A, ldout=64,
        ws=A, wsb=1 << 40):
    return tp.library().tp_block_simulated(
        dt, act, nseq, S, d, Hq, Hkv, dh, k, p, causal, eps, P(X), ldx, P(g1), P(b1n), P(Wqkv),
        ldq, P(bqkv), P(WO), ldo, P(bO), P(g2), P(b2n), P(W1), ldw1, P(Wu), ldwu, P(b1), P(W2),
        ldw2, P(b2), P(Out), ldout, P(ws), wsb, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(dt=0), "TP_ERR_BAD_DTYPE"),
    (dict(act=9), "TP_ERR_BAD_ACT"),
    (dict(S=-1), "TP_ERR_BAD_SHAPE"),
    (dict(dh=96, ldq=768), "TP_ERR_BAD_SHAPE"),
    (dict(Hkv=3, ldq=640), "TP_ERR_NOT_DIVISIBLE"),            # Hq % Hkv
    (dict(p=4, Hq=4, Hkv=2), "TP_ERR_NOT_DIVISIBLE"),          # Hkv % p
    (dict(k=129, ldw1=136), "TP_ERR_NOT_DIVISIBLE"),
    (dict(p=0), "TP_ERR_BAD_SHARD"),
    (dict(d=60, ldx=64, ldo=64, ldw2=64, ldout=64), "TP_ERR_MISALIGNED"),
    (dict(d=16392, ldx=16392, ldo=16392, ldw2=16392, ldout=16392), "TP_ERR_BAD_SHAPE"),
    (dict(g2=None), "TP_ERR_NULL_POINTER"),
    (dict(X=None), "TP_ERR_NULL_POINTER"),
    (dict(Out=MIS), "TP_ERR_MISALIGNED"),
    (dict(eps=-1.0), "TP_ERR_BAD_SHAPE"),
    (dict(ldq=500), "TP_ERR_BAD_SHAPE"),                       # below (Hq + 2 Hkv) dh
    (dict(ldout=60), "TP_ERR_BAD_SHAPE"),
    (dict(act=4), "TP_ERR_NULL_POINTER"),                      # SwiGLU without Wu
    (dict(act=4, Wu=A, ldwu=128, b1=A), "TP_ERR_BAD_ACT"),     # column bias with SwiGLU
    (dict(ws=None, wsb=0), "TP_ERR_WORKSPACE"),
    (dict(wsb=1024), "TP_ERR_WORKSPACE"),
])
def test_block_rejects(kw, expect):
    assert status_name(blk(**kw)) == expect


@no_gpu
def test_block_empty_is_ok_and_workspace_sizes():
    assert status_name(blk(S=0, X=None, Out=None, ws=None, wsb=0)) == "TP_OK"
    bf16 = torch.bfloat16
    # T = 4096: counter area, LN output, QKV and attention output of all heads, the 8 hidden
    # shards and the 8 partials plus X1 (all 256-byte multiples here)
    T, d, s = 4096, 8192, 3584
    expect = (256 << 10) + T * d * 2 + T * 10240 * 2 + T * 8192 * 2 + 8 * T * s * 2 + T * d * 4 \
        + 8 * T * d * 4
    assert tp.tp_block_workspace_bytes(bf16, "swiglu", 1, T, d, 64, 8, 128, 28672, 8) == expect
    assert tp.tp_block_workspace_bytes(bf16, "swiglu", 1, 0, d, 64, 8, 128, 28672, 8) == 0
    assert tp.tp_block_workspace_bytes(torch.float32, "swiglu", 1, T, d, 64, 8, 128, 28672, 8) == 0
    assert tp.tp_block_workspace_bytes(bf16, "swiglu", 1, T, d, 64, 8, 96, 28672, 8) == 0


# --- the entry point that allocates nothing ---------------------------------
def noalloc(dt=1, act=4, T=64, d=8192, k=65536, i=0, p=1, X=A, ldx=8192, W1=A, ldw1=65536, Wu=A,
            ldwu=65536, b1=None, W2=A, ldw2=8192, Y=A, ldy=65536, Z=A, ldz=8192):
    return tp.library().tp_mlp_shard_noalloc(dt, act, T, d, k, i, p, P(X), ldx, P(W1), ldw1,
                                             P(Wu), ldwu, P(b1), P(W2), ldw2, P(Y), ldy, P(Z),
                                             ldz, None)


def test_static_scratch_limit_is_declared():
    m = re.search(r"#define TP_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == 16 << 20


@no_gpu
def test_noalloc_rejects_sizes_beyond_the_static_scratch():
    """A SwiGLU few-token shard with 65536 hidden columns needs 32.25 MiB of split-K
    scratch (tp_workspace_bytes), more than the 16 MiB static array: TP_ERR_WORKSPACE
    before anything is touched; 16384 columns fit (and T = 0 launches nothing)."""
    assert tp.tp_workspace_bytes(torch.bfloat16, "swiglu", 64, 8192, 65536, 1) > 16 << 20
    rc = noalloc()
    assert status_name(rc) == "TP_ERR_WORKSPACE"
    assert "static scratch" in tp.library().tp_last_error_message().decode()
    assert status_name(noalloc(T=0, X=None, Y=None, Z=None)) == "TP_OK"


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(p=3), "TP_ERR_NOT_DIVISIBLE"),
    (dict(i=1), "TP_ERR_BAD_SHARD"),
    (dict(Wu=None), "TP_ERR_NULL_POINTER"),
    (dict(W2=MIS), "TP_ERR_MISALIGNED"),
    (dict(ldz=8000), "TP_ERR_BAD_SHAPE"),
    (dict(act=2, b1=A, Wu=None, ldwu=0, T=-1), "TP_ERR_BAD_SHAPE"),
])
def test_noalloc_validates_like_the_workspace_entry_point(kw, expect):
    assert status_name(noalloc(**kw)) == expect
