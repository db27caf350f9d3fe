"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of ``oracle/oracle.c`` (a
dropped term, a wrong index, sign, scale or base, a doubled magnitude),
compiles it with gcc into a temporary library and runs the pins of
``test_oracle_pins.py`` against it in a child process.  The case passes when
at least one pin fails, i.e. when the mistake cannot slip through.  Every
replacement must match the oracle's source exactly once, so a change to the
oracle that moves a mutation site fails here loudly rather than silently
testing nothing.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name -> (text in oracle.c, its planted replacement)
MUTANTS = {
    "exchange reads the local head index":
        ("+ source_head(heads, P, rank, h)) * row;", "+ h) * row;"),
    "inverse exchange writes head slot h, not rank*hl + h":
        ("* heads) + rank * hl + h) * row;", "* heads) + h) * row;"),
    "causal mask drops the diagonal":
        ("*hi = a->causal ? i + 1 : doc_end(a, i);", "*hi = a->causal ? i : doc_end(a, i);"),
    "document start ignored":
        ("*lo = doc_start(a, i);", "*lo = 0;"),
    "query range ignores causality":
        ("*lo = a->causal ? j : doc_start(a, j);", "*lo = doc_start(a, j);"),
    "GQA maps q head h to kv head h % hkv":
        ("return h / (a->hq / a->hkv);", "return h % a->hkv;"),
    "LSE in log base 2":
        ("const double lse = m + log(l);", "const double lse = m + log2(l);"),
    "score without the softmax scale":
        ("return a->scale * acc;", "return acc;"),
    "O magnitude doubled":
        ("if (o_mag) o_mag[e] += p * fabs(", "if (o_mag) o_mag[e] += 2 * p * fabs("),
    "dQ drops D":
        ("out[e] += ds * qv(&a, k, hkv, j, b, kh, e);",
         "out[e] += p * dp * qv(&a, k, hkv, j, b, kh, e);"),
    "dQ without the softmax scale":
        ("for (int e = 0; e < hd; ++e) out[e] *= scale;", ";"),
    "dK without the softmax scale":
        ("for (int e = 0; e < hd; ++e) okk[e] *= scale;", ";"),
    "dK uses dO in place of Q":
        ("okk[e] += ds * qv(&a, q, hq, i, b, h, e);", "okk[e] += ds * qv(&a, dout, hq, i, b, h, e);"),
    "dV sums only the first head of the group":
        ("ovv[e] += p * qv(&a, dout, hq, i, b, h, e);",
         "if (h == kh * g) ovv[e] += p * qv(&a, dout, hq, i, b, h, e);"),
    "D from O with the wrong sign":
        ("d += qv(&a, dout, hq, i, b, h, e) * oe;", "d -= qv(&a, dout, hq, i, b, h, e) * oe;"),
    "dQ magnitude doubled":
        ("if (mag) mag[e] += fabs(ds) * fabs(", "if (mag) mag[e] += 2 * fabs(ds) * fabs("),
    "dK magnitude doubled":
        ("if (mk) mk[e] += fabs(ds) * fabs(", "if (mk) mk[e] += 2 * fabs(ds) * fabs("),
    "dV magnitude doubled":
        ("if (mv) mv[e] += p * fabs(", "if (mv) mv[e] += 2 * p * fabs("),
    "dQ sensitivity to D doubled":
        ("if (dmag) dmag[e] += p * A[idx] * fabs(", "if (dmag) dmag[e] += 2 * p * A[idx] * fabs("),
    "dK sensitivity to D doubled":
        ("if (dmk) dmk[e] += p * A[idx] * fabs(", "if (dmk) dmk[e] += 2 * p * A[idx] * fabs("),
    "merge drops the max shift":
        ("L = m + log(exp(la - m) + exp(lb - m));", "L = log(exp(la - m) + exp(lb - m));"),
    "merge weights swapped":
        ("if (la != -INFINITY) x += wa * o_a[row + e];", "if (la != -INFINITY) x += wb * o_a[row + e];"),
    "loss gradient with the wrong sign on the label":
        ("- (v == labels[i] ? 1.0 : 0.0));", "+ (v == labels[i] ? 1.0 : 0.0));"),
    "loss keeps ignored tokens' gradient rows":
        ("for (int64_t v = 0; v < V; ++v) z[v] = 0.0;\n      continue;", "continue;"),
    "loss logit magnitude doubled":
        ("if (zmag) zmag[i] = zm;", "if (zmag) zmag[i] = 2 * zm;"),
    "loss dh magnitude doubled":
        ("if (dh_mag) dh_mag[i * d + k] = mag;", "if (dh_mag) dh_mag[i * d + k] = 2 * mag;"),
    "loss dW magnitude doubled":
        ("if (dw_mag) dw_mag[v * d + k] = mag;", "if (dw_mag) dw_mag[v * d + k] = 2 * mag;"),
    "silu derivative drops its second term":
        ("* u * s * (1.0 + g * (1.0 - s));", "* u * s;"),
    "du without silu":
        ("du[(size_t)i * I + j] = da * g * s;", "du[(size_t)i * I + j] = da * g;"),
    "MLP y magnitude doubled":
        ("if (y_mag) y_mag[i * d + k] = mag;", "if (y_mag) y_mag[i * d + k] = 2 * mag;"),
    "MLP dx magnitude doubled":
        ("if (dx_mag) dx_mag[i * d + k] = mag;", "if (dx_mag) dx_mag[i * d + k] = 2 * mag;"),
    "MLP dWg magnitude doubled":
        ("if (dwg_mag) dwg_mag[j * d + k] = mg;", "if (dwg_mag) dwg_mag[j * d + k] = 2 * mg;"),
    "MLP dWu magnitude doubled":
        ("if (dwu_mag) dwu_mag[j * d + k] = mu;", "if (dwu_mag) dwu_mag[j * d + k] = 2 * mu;"),
    "MLP dWd magnitude doubled":
        ("if (dwd_mag) dwd_mag[k * I + j] = mag;", "if (dwd_mag) dwd_mag[k * I + j] = 2 * mag;"),
}


def _run_mutant(name, old, new, tmp):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation site of '{name}' matches {src.count(old)} times"
    idx = sorted(MUTANTS).index(name)
    c_path = os.path.join(tmp, f"m{idx}.c")
    so_path = os.path.join(tmp, f"m{idx}.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", c_path, "-o", so_path,
                    "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ULYSSES_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            futs = {n: ex.submit(_run_mutant, n, o, w, tmp) for n, (o, w) in MUTANTS.items()}
            return {n: f.result() for n, f in futs.items()}


def test_unmutated_oracle_passes_its_pins(tmp_path):
    """Control: the same machinery on the unchanged source passes."""
    so_path = str(tmp_path / "same.so")
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", ORACLE_SRC, "-o",
                    so_path, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ULYSSES_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_results):
    code, out = mutant_results[name]
    # 1: some pin failed.  Anything else (0: all passed; 2-5: the run broke
    # before judging) means the mistake was not caught by a pin.
    assert code == 1, f"planted mistake '{name}' not caught (pytest exit {code}):\n{out}"
