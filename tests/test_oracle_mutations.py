"""Mutation test of the oracle (CPU only): copies of oracle/kvq_oracle.c, each
with one plausible mistake planted, are compiled like the oracle and the
oracle's pin tests are run against each copy in a subprocess (the copy loaded
through KVQ_ORACLE_LIB). Every mutant must fail at least one pin, and the
unmodified source, built the same way, must pass them all. The mistakes span
the codecs (rounding, divisors, ties, clamps, zero points, nibble placement,
static scales), the layout (bytes per token, slots, heads, staging), attention
(softmax scale, causal and window limits, value scales) and the pool."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")
PINS = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
              if f.startswith("test_oracle_") and f.endswith(".py")
              and f not in ("test_oracle_mutations.py", "test_oracle_quant_error.py"))

# (name, text in the source, replacement, which occurrence)
MUTANTS = [
    ("INT8 ties away from zero", "float r = rintf(x[i] / sc);", "float r = roundf(x[i] / sc);", 0),
    ("divisor 2^(bits-1)", "float sc = a / (float)qmax;", "float sc = a / (float)(qmax + 1);", 0),
    ("E4M3 ties to the upper code", "pick = (k % 2 == 0) ? k : k + 1;", "pick = k + 1;", 0),
    ("E4M3 scale from 240", "float sc = a / 448.0f;", "float sc = a / 240.0f;", 0),
    ("zero point sign", "float zf = rintf(-mn / sc);", "float zf = rintf(mn / sc);", 0),
    ("asymmetric range not widened to 0", "float mn = 0.0f, mx = 0.0f;",
     "float mn = x[0], mx = x[0];", 0),
    ("asymmetric step /16", "float sc = (mx - mn) / 15.0f;", "float sc = (mx - mn) / 16.0f;", 0),
    ("plain nibble packing", "int byte = n * r + i;", "int byte = e / 2;", 0),
    ("INT4 symmetric offset instead of sign", "int qv = nib[e] >= 8 ? (int)nib[e] - 16 : (int)nib[e];",
     "int qv = (int)nib[e] - 8;", 0),
    ("value scale dropped", "for (int e = 0; e < d; ++e) out[e] = (float)((const int8_t*)row)[e] * s;",
     "for (int e = 0; e < d; ++e) out[e] = (float)((const int8_t*)row)[e] * (side ? 1.0f : s);", 0),
    ("query head to KV head h % H", "  int g = h / G;\n", "  int g = h % H;\n", 0),
    ("softmax scale 1/d", "J.sm = sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)L->head_dim);",
     "J.sm = sm_scale != 0.0 ? sm_scale : 1.0 / (double)L->head_dim;", 0),
    ("last token dropped", "J->lens[b], 0, J->lens[b], J->sm, &m, &l, acc);",
     "J->lens[b], 0, J->lens[b] - (J->lens[b] > 0), J->sm, &m, &l, acc);", 0),
    ("bytes per token: 16-bit codes for all", "per_layer += H * d * code_bits(side_code(L, side)) / 8;",
     "per_layer += H * d * 16 / 8;", 0),
    ("blocks taken from the stack top down", "row[have + k] = stack[*top - off - need + k];",
     "row[have + k] = stack[*top - off - 1 - k];", 0),
    ("slot offset off by one", "slots[tok++] = (int64_t)row[pos / bs] * bs + pos % bs;",
     "slots[tok++] = (int64_t)row[pos / bs] * bs + (pos + 1) % bs;", 0),
    ("release pushes blocks reversed", "stack[pos++] = tables[(int64_t)b * max_blocks + k];",
     "stack[pos++] = tables[(int64_t)b * max_blocks + (nblk - 1 - k)];", 0),
    ("causal limit excludes the query's own position", "return t <= p && (J->window <= 0",
     "return t < p && (J->window <= 0", 0),
    ("window one position too long", "t >= p + 1 - J->window", "t >= p - J->window", 0),
    ("per-channel block quantized one row early", "if (off != bs - 1) return;",
     "if (off != bs - 2) return;", 0),
    ("per-channel tail boundary", "pos >= (context_len / bs) * bs", "pos > (context_len / bs) * bs", 0),
    ("static INT8 ties away from zero", "float r = rintf(x[i] / s);", "float r = roundf(x[i] / s);", 0),
    ("static E4M3 through a reciprocal", "q[i] = orc_e4m3_encode(x[i] / s);",
     "q[i] = orc_e4m3_encode(x[i] * (1.0f / s));", 0),
    ("static asymmetric clamp at 7", "if (r > 15.0f) r = 15.0f;", "if (r > 7.0f) r = 7.0f;", 0),
]


def _mutate(text, old, new, which):
    pos = -1
    for _ in range(which + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, f"not in the oracle source: {old!r}"
    return text[:pos] + new + text[pos + len(old):]


def _pins_pass(src_text, tmp, tag):
    """Compile src_text like the oracle and run the pin tests against it;
    True when every pin passes."""
    d = os.path.join(tmp, tag)
    os.makedirs(d)
    c = os.path.join(d, "kvq_oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    lib = os.path.join(d, "libkvq_oracle.so")
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", lib,
                    c, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, KVQ_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode in (0, 1), r.stdout[-2000:] + r.stderr[-2000:]
    return r.returncode == 0


def test_every_planted_mistake_fails_a_pin():
    text = open(SRC).read()
    sources = [("unmodified", text)] + [
        (name, _mutate(text, old, new, which)) for name, old, new, which in MUTANTS]
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(4, (os.cpu_count() or 1) // 2))) as ex:
            passed = list(ex.map(lambda it: _pins_pass(it[1][1], tmp, f"m{it[0]}"),
                                 enumerate(sources)))
    assert passed[0], "the unmodified oracle, built the same way, fails its pins"
    survivors = [name for (name, _), ok in zip(sources[1:], passed[1:]) if ok]
    assert not survivors, f"mistakes no pin catches: {survivors}"
