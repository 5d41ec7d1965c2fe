"""The pins catch planted mistakes: each mutant below is a copy of oracle.c with
one plausible error (a dropped term, a wrong sign, constant, index or operand
order, a swapped gate/up, a mis-sliced bias), built with gcc; the CPU pin suite
(tests/test_oracle_pins.py) run against it in a subprocess must fail.  All of
this happens on the CPU; the GPU path is not involved."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, which occurrence: 0 = first, -1 = all)
MUTANTS = [
    ("gelu_tanh drops the cubic term", "tanh(c * (x + 0.044715 * x * x * x))", "tanh(c * x)", 0),
    ("gelu_tanh wrong coefficient", "0.044715 * x * x * x)))", "0.04715 * x * x * x)))", 0),
    ("gelu_erf wrong scale", "erf(x / sqrt(2.0))", "erf(x / 2.0)", 0),
    ("silu wrong sign", "return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));", 0),
    ("relu leaks", "return x > 0.0 ? x : 0.0;", "return x > 0.0 ? x : 0.01 * x;", 0),
    ("column shards in reverse order", "const int64_t s = k / p, c0 = (int64_t)i * s;",
     "const int64_t s = k / p, c0 = (int64_t)(p - 1 - i) * s;", 0),
    ("column bias not sliced", "const double v = b1 ? h[j] + b1[c0 + j] : h[j];",
     "const double v = b1 ? h[j] + b1[j] : h[j];", 0),
    ("swiglu gate and up swapped", "h[j] = act_scalar_f64(OR_ACT_SWIGLU, h[j]) * u[j];",
     "h[j] = act_scalar_f64(OR_ACT_SWIGLU, u[j]) * h[j];", 0),
    ("row shard reads W2 transposed",
     "const double *w = W2 + (c0 + j) * d;\n      for (int64_t n = 0; n < d; ++n) z[n] += yv * w[n];",
     "for (int64_t n = 0; n < d; ++n) z[n] += yv * W2[n * k + c0 + j];", 0),
    ("partial sum drops the last shard", "for (int32_t q = 1; q < p; ++q) acc += parts[(int64_t)q * n + e];",
     "for (int32_t q = 1; q < p - 1; ++q) acc += parts[(int64_t)q * n + e];", 0),
    ("partial sum forgets b2", "if (b2) acc += b2[e % d];", "", 0),
    ("unsharded MLP reads W2 transposed", "z[n] += yv * W2[j * d + n];", "z[n] += yv * W2[n * k + j];", 0),
    ("fp32 linear reads W transposed", "h[j] += xv * W[c * k + j];", "h[j] += xv * W[j * d + c];", 0),
    ("fp32 column shard wrong offset", "const float *w = W1 + c * k + c0;",
     "const float *w = W1 + c * k + (c0 > 0 ? c0 - 1 : c0);", 0),
    ("qkv key and value blocks swapped",
     "(part == 1 ? (int64_t)Hq * dh : ((int64_t)Hq + Hkv) * dh)",
     "(part == 2 ? (int64_t)Hq * dh : ((int64_t)Hq + Hkv) * dh)", 0),
    ("qkv heads of the mirrored shard",
     "for (int64_t h = (int64_t)i * per_gpu; h < ((int64_t)i + 1) * per_gpu; ++h)",
     "for (int64_t h = (int64_t)(p - 1 - i) * per_gpu; h < ((int64_t)(p - 1 - i) + 1) * per_gpu; ++h)", 0),
    ("qkv key/value shard i starts at head i",
     "for (int64_t h = (int64_t)i * per_gpu; h < ((int64_t)i + 1) * per_gpu; ++h)",
     "for (int64_t h = (part == 0 ? (int64_t)i * per_gpu : i);"
     " h < (part == 0 ? (int64_t)i * per_gpu : i) + per_gpu; ++h)", 0),
    ("qkv bias not mapped", "QKV[t * nout + n] = b ? acc + b[src[n]] : acc;",
     "QKV[t * nout + n] = b ? acc + b[n] : acc;", 0),
    ("gelu_tanh derivative drops the sech^2 factor", "0.5 * x * (1.0 - t * t) * c *",
     "0.5 * x * c *", 0),
    ("gelu_erf derivative drops the x factor", "x * exp(-0.5 * x * x) / sqrt(2.0 * M_PI)",
     "exp(-0.5 * x * x) / sqrt(2.0 * M_PI)", 0),
    ("silu derivative wrong sign", "return s * (1.0 + x * (1.0 - s));", "return s * (1.0 + x * s);", 0),
    ("swiglu up gradient uses the up value", "dH[t * hw + s + j] = dy * sg;",
     "dH[t * hw + s + j] = dy * u;", 0),
    ("row weight gradient from the pre-activation", "a += Y[t * s + j] * dZ[t * d + n];",
     "a += H[t * s + j] * dZ[t * d + n];", 0),
    ("hidden gradient reads W2 transposed", "dy += dZ[t * d + n] * W2[(c0 + j) * d + n];",
     "dy += dZ[t * d + n] * W2[n * k + c0 + j];", 0),
    ("input gradient drops the up term",
     "acc += dH[t * hw + s + j] * Wu[c * k + c0 + j];", "", 0),
    ("input gradient ignores the shard offset", "acc += dH[t * hw + j] * W1[c * k + c0 + j];",
     "acc += dH[t * hw + j] * W1[c * k + j];", 0),
    ("bias gradient drops the first token", "for (int64_t t = 0; t < T; ++t) a += dH[t * hw + j];",
     "for (int64_t t = 1; t < T; ++t) a += dH[t * hw + j];", 0),
    ("attention without the 1/sqrt(dh) scale", "const double scale = 1.0 / sqrt((double)dh);",
     "const double scale = 1.0;", 0),
    ("attention mask hides the diagonal", "const int64_t nk = causal ? t + 1 : S;",
     "const int64_t nk = causal ? (t > 0 ? t : 1) : S;", 0),
    ("grouped heads interleaved", "const int64_t c = h / group;", "const int64_t c = h % Hkv;", 0),
    ("attention ignores the sequence start", "const int64_t tk = b * S + j;", "const int64_t tk = j;", 0),
    ("layernorm without the mean", "Y[t * d + c] = (x[c] - mu) * rstd * gamma[c] + beta[c];",
     "Y[t * d + c] = x[c] * rstd * gamma[c] + beta[c];", 0),
    ("layernorm unbiased variance", "const double var = sq / (double)d;",
     "const double var = sq / (double)(d - 1);", 0),
    ("layernorm eps outside the root", "const double rstd = 1.0 / sqrt(var + eps);",
     "const double rstd = 1.0 / (sqrt(var) + eps);", 0),
    ("block drops the attention residual",
     "x1[n] = X[t * d + n] + (bO ? x1[n] + bO[n] : x1[n]);", "x1[n] = bO ? x1[n] + bO[n] : x1[n];", 0),
    ("block drops the FFN residual", "Out[e] = X1[e] + Z[e];", "Out[e] = Z[e];", 0),
    ("block's second LayerNorm takes the first one's parameters",
     "oracle_layernorm_f64(nrows, d, X1, ln2_g, ln2_b, eps, B)",
     "oracle_layernorm_f64(nrows, d, X1, ln1_g, ln1_b, eps, B)", 0),
    ("block's FFN swaps gate and up", "act_scalar_f64(OR_ACT_SWIGLU, hid[j]) * up[j]",
     "act_scalar_f64(OR_ACT_SWIGLU, up[j]) * hid[j]", 0),
    ("bf16 rounding truncates", "b += 0x7fffu + ((b >> 16) & 1u);", "", 0),
    ("fp32 gelu_tanh drops the cubic term", "tanhf(c * (x + 0.044715f * x * x * x))",
     "tanhf(c * x)", 0),
    ("fp32 silu wrong sign", "return x / (1.0f + expf(-x));", "return x / (1.0f + expf(x));", 0),
    ("fp32 gelu_erf wrong scale", "erff(x / sqrtf(2.0f))", "erff(x / 2.0f)", 0),
    ("block's output projection reads WO transposed", "const double *w = WO + j * d;\n      for (int64_t n = 0; n < d; ++n) x1[n] += ov * w[n];",
     "for (int64_t n = 0; n < d; ++n) x1[n] += ov * WO[n * qw + j];", 0),
]


def build_mutant(text, old, new, which, out):
    assert old in text, old
    if which == 0:
        text = text.replace(old, new, 1)
    else:
        text = text.replace(old, new)
    src = out + ".c"
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-ffp-contract=off", "-std=c11", "-D_DEFAULT_SOURCE",
                    "-fPIC", "-shared", "-o", out, src, "-lm"], check=True)


def run_pins(lib):
    env = dict(os.environ, TPMLP_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


CONTROL = ("unmutated copy", "#include <math.h>", "#include <math.h>", 0)


@pytest.fixture(scope="module")
def outcomes():
    """Every mutant (and an unchanged copy) built and run against the pins, in
    parallel subprocesses; name -> (return code, tail of the output)."""
    text = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        def one(m):
            name, old, new, which = m
            lib = os.path.join(tmp, "lib%d.so" % abs(hash(name)))
            build_mutant(text, old, new, which, lib)
            r = run_pins(lib)
            return name, (r.returncode, r.stdout[-2000:])
        workers = max(1, min(8, (os.cpu_count() or 2)))
        with ThreadPoolExecutor(workers) as ex:
            return dict(ex.map(one, MUTANTS + [CONTROL]))


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(outcomes, name, old, new, which):
    rc, out = outcomes[name]
    assert rc != 0, f"mutant '{name}' survived the pins:\n{out}"


def test_unmutated_copy_passes(outcomes):
    """Control: the same procedure on an unchanged copy passes the pins."""
    rc, out = outcomes[CONTROL[0]]
    assert rc == 0, out
