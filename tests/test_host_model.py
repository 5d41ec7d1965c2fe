"""Host-side bounds model of every launch the C ABI makes, under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only, no GPU).

The library's host code (api.cpp and the launch code of every kernel source,
compiled for the host only) is linked, instrumented, against a stand-in for
the HIP runtime (tests/hostcheck/fake_hip.cpp) and a driver that calls the C
ABI on fake device buffers sized exactly to each operand's documented shape
(tests/hostcheck/driver.cpp).  Every kernel launch reaches a bounds model
(tests/hostcheck/model.cpp) instead of a GPU:
  - tiled GEMM launches lane by lane, with the kernel's own addressing code
    (csrc/tiled_geometry.hpp): each workgroup's tile (all tiles exactly once),
    every buffer-to-LDS load's bytes at its first and last live k-step (with
    the QKV column map and split B^T operands), offsets inside the descriptor
    range, each stage's LDS filled once, and every epilogue store and read;
  - few-token GEMM launches lane by lane (csrc/decode_geometry.hpp): each
    workgroup's column block and k-range (all exactly once), the weight and
    token loads at their first and last live stage, each stage's LDS filled
    once, the split-K partial stores and loads (no two workgroups' stores
    overlapping), the arrival counter, and the output stores;
  - every other launch at the level of its arguments (operand extents,
    attention, reductions, LayerNorm, column sums).
The cases are the GPU tests' shapes, the full-size workloads, empty inputs,
padded leading dimensions, and rejected arguments (which must launch nothing).
A run with every buffer two bytes short must report findings: the model sees
the last element of the operands.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from megatron_tensor_mlp_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "hostcheck")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
CPP_SOURCES = [os.path.join(build.CSRC, s) for s in build.SOURCES if s.endswith(".cpp")] + [
    os.path.join(HC, s) for s in ("fake_hip.cpp", "model.cpp", "driver.cpp")]
# Instrumentation of host code only: for hipcc each sanitizer flag goes to the
# host compilation; the plain C++ sources are built with the same LLVM clang.
SAN = ["address", "undefined"]
HIP_SAN = [f for s in SAN for f in ("-Xarch_host", "-fsanitize=" + s)]
CXX_SAN = ["-fsanitize=" + ",".join(SAN), "-fno-sanitize-recover=undefined"]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-3000:]
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(CLANG) and shutil.which(build.hipcc())):
        pytest.skip("ROCm clang/hipcc not found")
    out = tmp_path_factory.mktemp("hostcheck")

    def hip_obj(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        _run([build.hipcc(), "--offload-arch=" + build.ARCH, "--offload-host-only", *COMMON,
              *HIP_SAN, "-c", os.path.join(build.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(8) as ex:
        hip_objs = list(ex.map(hip_obj, HIP_SOURCES))
        cxx_objs = list(ex.map(lambda s: cxx_obj(s, out), CPP_SOURCES))
    # A host-only object refers to its (absent) device code image by a symbol;
    # the stand-in runtime never reads it, so each gets an empty definition.
    names = set()
    for o in hip_objs:
        names |= set(re.findall(r"__hip_fatbin_[0-9a-f]+", _run(["nm", "-u", o]).stdout))
    stub = out / "fatbins.cpp"
    stub.write_text("".join(f'extern "C" const char {n}[64] = {{0}};\n' for n in sorted(names)))
    _run([CLANG, *COMMON, "-c", str(stub), "-o", str(out / "fatbins.o")])
    objs = hip_objs + cxx_objs + [str(out / "fatbins.o")]
    exe = str(out / "driver")
    _run([CLANG, *CXX_SAN, "-o", exe, *objs])
    return Built(exe, objs, out)


class Built:
    def __init__(self, exe, objs, out):
        self.exe, self.objs, self.out = exe, objs, out


def cxx_obj(src, out, include_first=None):
    obj = str(out / (os.path.basename(src) + ".o"))
    inc = ([f"-I{include_first}"] if include_first else []) + [
        "-I" + build.CSRC, "-I" + os.path.join(ROCM, "include")]
    _run([CLANG, *COMMON, *CXX_SAN, "-D__HIP_PLATFORM_AMD__", *inc, "-c", src, "-o", obj])
    return obj


def run_driver(exe, lines, timeout=600):
    exe = exe.exe if isinstance(exe, Built) else exe
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       timeout=timeout, env=env)
    return r


def gpu_test_cases():
    """The shapes the GPU tests run, as driver lines."""
    from tests import test_gpu_attn as ga
    from tests import test_gpu_backward as gb
    from tests import test_gpu_block as gk
    from tests import test_gpu_edges as ge
    from tests import test_gpu_parity as gp
    from tests import test_zz_no_alloc as gz

    out = []
    for T, d, k, p, act in gp.CASES + ge.WIDE:
        for i in sorted({0, p - 1}):
            bias = "" if act == "swiglu" else " bias=1"
            out.append(f"shard bf16 {act} {T} {d} {k} {i} {p}{bias}")
    for T, d, k, p, act, _ in gp.DECODE_CASES:
        for i in sorted({0, p - 1}):
            out.append(f"shard bf16 {act} {T} {d} {k} {i} {p}" + ("" if act == "swiglu" else " bias=1"))
    for T, d, k, act, _ in gp.TILE256_CASES:
        out.append(f"shard bf16 {act} {T} {d} {k} 0 1" + ("" if act == "swiglu" else " bias=1"))
    for T, d, k, p, act, _ in gp.SPLIT_CASES:
        out.append(f"shard bf16 {act} {T} {d} {k} {p - 1} {p}" + ("" if act == "swiglu" else " bias=1"))
    for T, d, k, p, act, _ in gp.SIM_SPLIT_CASES:
        out.append(f"sim bf16 {act} {T} {d} {k} {p}" + ("" if act == "swiglu" else " bias=1"))
    out.append("qkv bf16 1000 8192 8 1 128 0 1 bias=1")
    for T1, T2, d, k, p, act in gz.CASES:
        for T in (T1, T2):
            out.append(f"noalloc bf16 {act} {T} {d} {k} {p - 1} {p}"
                       + ("" if act == "swiglu" else " bias=1"))
    for T, d, Hq, Hkv, dh, p, bias, _ in ga.QKV_CASES:
        for i in sorted({0, p - 1}):
            out.append(f"qkv bf16 {T} {d} {Hq} {Hkv} {dh} {i} {p} bias={int(bias)}")
    for nseq, S, Hq, Hkv, dh, causal, _ in ga.ATTN_CASES:
        out.append(f"attn {nseq} {S} {Hq} {Hkv} {dh} {int(causal)}")
    for T, d, k, p, act, bias in gb.CASES:
        for i in sorted({0, p - 1}):
            out.append(f"train bf16 {act} {T} {d} {k} {i} {p} bias={int(bias)}")
            out.append(f"bwd bf16 {act} {T} {d} {k} {i} {p} db1={int(bias)}")
    for T, d, p, bias, res, ln, _ in gk.ROW_CASES:
        out.append(f"rln {T} {d} {p} bias={int(bias)} R={int(res)} ln={int(ln)}")
    for nseq, S, d, Hq, Hkv, dh, k, p, act, causal, _ in gk.BLOCK_CASES:
        out.append(f"block {act} {nseq} {S} {d} {Hq} {Hkv} {dh} {k} {p} {int(causal)} "
                   f"bias={int(act != 'swiglu')}")
    for p in (1, 3, 8, 17, 64):
        for b2 in (0, 1):
            out.append(f"psum 257 264 {p} b2={b2}")
    return out


# Full-size workloads, empty inputs, padded leading dimensions, fp32.
EXTRA = [
    "shard bf16 swiglu 4096 8192 28672 7 8",          # Llama-70B TP=8 prefill shard
    "shard bf16 swiglu 1 8192 28672 0 8",             # decode T = 1, 8, 64
    "shard bf16 swiglu 8 8192 28672 7 8",
    "shard bf16 swiglu 64 8192 28672 3 8",
    "noalloc bf16 swiglu 64 8192 28672 7 8",
    "shard bf16 gelu_tanh 2048 12288 49152 7 8 bias=1",  # GPT-3 175B width at TP = 8
    "sim bf16 swiglu 512 8192 28672 8 b2=1",          # simulated TP = 8, full weights
    "sim bf16 gelu_tanh 300 264 1024 4 bias=1",
    "sim bf16 swiglu 20 264 1024 4",
    "qkv bf16 4096 8192 64 8 128 5 8",                # Llama-70B head shard
    "qkv bf16 1 8192 64 8 128 7 8",
    "attn 1 4096 8 1 128 1",
    "attn 1 16384 8 1 128 1",
    "train bf16 swiglu 4096 8192 28672 7 8",
    "bwd bf16 swiglu 4096 8192 28672 7 8",
    "bwd bf16 gelu_tanh 300 264 1024 3 4 db1=1 pad=8",
    "block swiglu 1 512 8192 64 8 128 28672 8 1 inplace=1",
    "shard bf16 swiglu 300 8192 3584 0 1 nows=1",     # no workspace: the tiled GEMMs run unsplit
    "col bf16 gelu_tanh 257 4104 2048 0 1 bias=1 nows=1",
    "row bf16 300 8192 3584 0 1 nows=1",
    "qkv bf16 1000 8192 8 1 128 0 1 bias=1 nows=1",
    "sim bf16 swiglu 300 8192 2048 4 nows=1",
    "shard bf16 swiglu 300 264 1024 2 4 pad=8",       # padded leading dimensions
    "shard bf16 gelu_erf 17 264 1024 0 4 bias=1 pad=16",
    "qkv bf16 300 264 8 2 64 1 2 bias=1 pad=8",
    "attn 2 65 2 2 64 0 pad=8",
    "psum 300 264 8 b2=1 pad=8 inplace=1",
    "shard f32 gelu_tanh 64 16 32 1 4 bias=1",         # fp32 path (Day 41 shapes)
    "shard f32 swiglu 300 264 1024 3 4",
    "sim f32 gelu_erf 64 16 32 4 bias=1 b2=1",
    "bwd f32 gelu_tanh 65 264 1024 1 4 db1=1",
    "shard bf16 swiglu 0 264 1024 1 4",               # no tokens: nothing to launch
    "sim bf16 gelu_tanh 0 264 1024 4",
    "qkv bf16 0 264 8 2 64 0 2",
    "bwd bf16 swiglu 0 264 1024 0 4",
    "psum 0 264 4",
    "rln 0 264 2",
    # rejected arguments: nothing may be launched
    "! col bf16 swiglu 10 8 12 0 5",                  # k % p != 0
    "! shard bf16 swiglu 10 8 12 4 4",                # i outside [0, p)
    "! shard bf16 swiglu 10 12 1024 0 4",             # d not a multiple of 8
    "! shard bf16 swiglu 10 264 1024 0 4 bias=1",     # bias with SwiGLU
    "! qkv bf16 10 264 8 3 64 0 2",                   # Hkv % p != 0
    "! block swiglu 1 16 24 4 2 96 64 2 1",           # dh neither 64 nor 128
    "! noalloc bf16 swiglu 64 8192 65536 0 1",        # partials beyond the static scratch
    "! shard bf16 swiglu 64 8192 28672 0 8 nows=1",   # few tokens: the workspace is required
]


def test_every_launch_stays_in_bounds(driver):
    lines = gpu_test_cases() + EXTRA
    r = run_driver(driver, lines)
    tail = "\n".join(r.stdout.splitlines()[-40:]) + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, tail
    done = re.search(r"DONE cases (\d+) failed (\d+)", r.stdout)
    assert done and int(done.group(1)) == len(lines) and done.group(2) == "0", tail
    stats = [re.search(r"launches (\d+) tiled (\d+) decode (\d+) other (\d+) accesses (\d+)", x)
             for x in r.stdout.splitlines() if x.startswith("CASE")]
    tiled = sum(int(m.group(2)) for m in stats)
    decode = sum(int(m.group(3)) for m in stats)
    other = sum(int(m.group(4)) for m in stats)
    assert tiled >= 100 and decode >= 50 and other >= 50, (tiled, decode, other)


def test_split_k_launches_are_modelled(driver):
    """The shapes that split K launch the split instantiation (bool template
    argument 1), and the model checks them without findings."""
    from tests import test_gpu_parity as gp
    lines = [f"shard bf16 {act} {T} {d} {k} {p - 1} {p}" + ("" if act == "swiglu" else " bias=1")
             for T, d, k, p, act, _ in gp.SPLIT_CASES]
    lines.append("qkv bf16 4096 8192 64 8 128 5 8")
    r = run_driver(driver, [x + " kernels=1" for x in lines])
    out = r.stdout
    assert re.search(r"DONE cases \d+ failed 0", out), out[-3000:] + r.stderr[-2000:]
    split = [x for x in out.splitlines()
             if x.startswith("KERNEL") and "gemm_bf16_tiled_kernel" in x and "Lb1E" in x]
    # every case has at least one split launch (the column step, or the QKV)
    assert len(split) >= len(lines), out[-3000:]


def test_model_sees_the_last_element(driver):
    """Every buffer two bytes short of its operand's extent: each case must
    report a finding (so an access to an operand's last element is seen)."""
    lines = ["shard bf16 swiglu 300 264 1024 2 4", "shard bf16 gelu_tanh 17 264 1024 0 4 bias=1",
             "qkv bf16 300 264 8 2 64 1 2 bias=1", "bwd bf16 swiglu 300 264 1024 3 4",
             "attn 1 200 4 2 128 1", "psum 7 264 3 b2=1", "rln 7 264 3 bias=1"]
    r = run_driver(driver, [x + " shrink=2" for x in lines])
    cases = [x for x in r.stdout.splitlines() if x.startswith("CASE")]
    assert len(cases) == len(lines), r.stdout[-2000:] + r.stderr[-2000:]
    for c in cases:
        assert "FAILED" in c and int(re.search(r"findings (\d+)", c).group(1)) > 0, c


# Planted mistakes in a copy of the shared addressing code (the bounds model is
# rebuilt against the copy; the library itself is untouched): for the tiled
# GEMM a dropped row check on A, a column check that lets one 16-byte unit past
# N through, a tile order that is not a bijection, split-K partial groups that
# overlap and k-ranges that are not whole k-steps; for the few-token GEMM
# a dropped token-row check, a weight column check one unit late, and partial
# slots of half their size.  Each must produce findings.
MUTANTS = [
    ("A rows past M not masked", "tiled_geometry.hpp",
     "off = (m0 + r < p.M) ? (uint32_t)((r * p.lda + 8 * lu) * 2) : OOB_OFF;",
     "off = (uint32_t)((r * p.lda + 8 * lu) * 2);",
     ["shard bf16 swiglu 300 264 1024 2 4", "shard bf16 gelu_tanh 1000 520 8504 0 1 bias=1"]),
    ("B column check off by one unit", "tiled_geometry.hpp",
     "off = (col < p.N) ? (uint32_t)((kr * ld + src_col(p, col)) * 2) : OOB_OFF;",
     "off = (col < p.N + 8) ? (uint32_t)((kr * ld + src_col(p, col)) * 2) : OOB_OFF;",
     ["shard bf16 gelu_erf 257 520 768 1 2 bias=1", "qkv bf16 300 264 8 2 64 1 2 bias=1"]),
    ("tile order not a bijection", "tiled_geometry.hpp",
     "const int t = xcd * q + (xcd < r ? xcd : r) + idx;",
     "const int t = xcd * q + idx;",
     ["shard bf16 swiglu 300 264 1024 2 4", "shard bf16 relu 1000 8456 1024 0 1 bias=1"]),
    ("split-K slot groups overlap", "tiled_geometry.hpp",
     "* 64 + lane) * 16);",
     "* 64 + lane) * 8);",
     ["qkv bf16 1000 8192 8 1 128 0 1 bias=1", "shard bf16 none 65 12296 1024 3 4 bias=1"]),
    ("split-K k-range not whole steps", "tiled_geometry.hpp",
     "return (per + BK - 1) / BK * BK;",
     "return per;",
     ["shard bf16 none 65 12296 1024 3 4 bias=1", "shard bf16 gelu_tanh 257 4104 2048 0 1 bias=1"]),
    ("few-token rows past M not masked", "decode_geometry.hpp",
     "off = (r < p.M && r < 16 * MB) ? (uint32_t)((r * p.lda + k) * 2) : OOB_OFF;",
     "off = (r < 16 * MB) ? (uint32_t)((r * p.lda + k) * 2) : OOB_OFF;",
     ["shard bf16 swiglu 1 264 1024 0 4", "shard bf16 gelu_erf 17 1032 1536 3 4 bias=1"]),
    ("few-token weight columns past N", "decode_geometry.hpp",
     "off = col < p.N ? (uint32_t)((r * ldw + src_col(p, col)) * 2) : OOB_OFF;",
     "off = col < p.N + 8 ? (uint32_t)((r * ldw + src_col(p, col)) * 2) : OOB_OFF;",
     ["shard bf16 relu 40 520 1000 0 1 bias=1", "qkv bf16 8 520 12 4 40 3 4 bias=1"]),
    ("few-token partial slots overlap", "decode_geometry.hpp",
     "return (uint32_t)((q * S + s) * (PF * 4));",
     "return (uint32_t)((q * S + s) * (PF * 2));",
     ["shard bf16 swiglu 3 264 16384 0 1", "shard bf16 none 33 264 1024 1 4"]),
]


@pytest.fixture(scope="module")
def mutant_outcomes(driver, tmp_path_factory):
    """Every mutant's bounds model built (in parallel) and run on its cases;
    what -> (case lines of the output, full output)."""
    def one(m):
        what, fname, old, new, lines = m
        d = tmp_path_factory.mktemp("mutant")
        src = open(os.path.join(build.CSRC, fname)).read()
        assert src.count(old) == 1, what
        (d / fname).write_text(src.replace(old, new))  # found before csrc/'s copy
        model = cxx_obj(os.path.join(HC, "model.cpp"), d, include_first=str(d))
        objs = [o for o in driver.objs if not o.endswith("model.cpp.o")] + [model]
        exe = str(d / "driver")
        _run([CLANG, *CXX_SAN, "-o", exe, *objs])
        r = run_driver(exe, lines)
        return what, ([x for x in r.stdout.splitlines() if x.startswith("CASE")],
                      r.stdout[-2000:] + r.stderr[-2000:])
    with ThreadPoolExecutor(len(MUTANTS)) as ex:
        return dict(ex.map(one, MUTANTS))


@pytest.mark.parametrize("what,fname,old,new,lines", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_model_catches_planted_addressing_mistakes(mutant_outcomes, what, fname, old, new, lines):
    cases, out = mutant_outcomes[what]
    assert len(cases) == len(lines), out
    assert any(int(re.search(r"findings (\d+)", c).group(1)) > 0 for c in cases), out
