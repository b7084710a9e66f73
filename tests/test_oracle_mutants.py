"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below plants one mistake in a temporary copy of the oracle
(``oracle/oracle.cpp`` or ``oracle/oracle.py``): a dropped term, a flipped
sign, a wrong index or order, a transposed operand, a wrong constant. The
pin tests (tests/test_oracle_*.py, this file excluded) then run against the
copy in a subprocess; every mutant must make at least one of them fail, and
the unmodified copy must pass them all. Nothing here touches the real oracle
or its library.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f != "test_oracle_mutants.py")

# (name, file, text, replacement): `text` must occur exactly once.
MUTANTS = [
    ("int4 unsigned instead of two's complement", "oracle.cpp",
     "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("int4 high nibble first", "oracle.cpp",
     "(word >> (4 * (i % 8))) & 15u", "(word >> (4 * (7 - i % 8))) & 15u"),
    ("int4 first group's scale for every input", "oracle.cpp",
     "s[static_cast<int64_t>(o) * (cols / group) + i / group]",
     "s[static_cast<int64_t>(o) * (cols / group)]"),
    ("fp16 decode: exponent bias off by one", "oracle.cpp",
     "1024 + mant), expo - 25)", "1024 + mant), expo - 24)"),
    ("silu with the wrong sign", "oracle.cpp",
     "double silu(double z) { return z / (1.0 + std::exp(-z)); }",
     "double silu(double z) { return z / (1.0 + std::exp(z)); }"),
    ("erf GELU without the 1/sqrt(2)", "oracle.cpp",
     "std::erf(z / std::sqrt(2.0))", "std::erf(z)"),
    ("RMSNorm over the sum instead of the mean", "oracle.cpp",
     "1.0 / std::sqrt(ss / d + eps)", "1.0 / std::sqrt(ss + eps)"),
    ("top-K ties to the higher id", "oracle.cpp",
     "score[e] > score[best]", "score[e] >= score[best]"),
    ("softmax-top-K weights not renormalised", "oracle.cpp",
     "w[k] = norm ? g[idx[k]] / sel : g[idx[k]];", "w[k] = g[idx[k]];"),
    ("sigmoid-group weights on the biased score", "oracle.cpp",
     "w[k] = scale * sig[idx[k]] / (sum + 1e-20);", "w[k] = scale * sel[idx[k]] / (sum + 1e-20);"),
    ("sigmoid-group score from the top-1 only", "oracle.cpp",
     "gscore[g] = sel[g * per + top2[0]] + sel[g * per + top2[1]];",
     "gscore[g] = sel[g * per + top2[0]];"),
    ("routed expert with gate and up swapped", "oracle.cpp",
     "q4_matvec(up_q, up_s, I, d, group, x, u.data());\n  for (int i = 0; i < I; ++i) h[i] = silu(g[i]) * u[i];",
     "q4_matvec(up_q, up_s, I, d, group, x, u.data());\n  for (int i = 0; i < I; ++i) h[i] = silu(u[i]) * g[i];"),
    ("LoRA with B transposed", "oracle.cpp",
     "f16_to_f64(B[static_cast<int64_t>(o) * r + j])", "f16_to_f64(B[static_cast<int64_t>(j) * out + o])"),
    ("LoRA scale alpha instead of alpha / r", "oracle.cpp",
     "const double c = r > 0 ? alpha / r : 0.0;", "const double c = r > 0 ? alpha : 0.0;"),
    ("shared expert without its down LoRA", "oracle.cpp",
     "if (a_down && b_down) orc_lora_delta(a_down, b_down, Is, d, r, c, h.data(), y);", ""),
    ("head without the previous-set one-hot (gathered form)", "oracle.cpp",
     "        acc += f16_to_f64(row[d + cur[k]]);\n        if (prev) acc += f16_to_f64(row[d + E + prev[k]]);\n      }\n      z[p] = acc;",
     "        acc += f16_to_f64(row[d + cur[k]]);\n      }\n      z[p] = acc;"),
    ("head without GELU", "oracle.cpp",
     "for (int p = 0; p < P; ++p) a[p] = gelu_erf(z[p]);", "for (int p = 0; p < P; ++p) a[p] = z[p];"),
    ("layer step without the residual", "oracle.cpp",
     "for (int i = 0; i < d; ++i) h_out[i] = ha[i] + y[i];", "for (int i = 0; i < d; ++i) h_out[i] = y[i];"),
    ("slot policy takes free slots in descending order", "oracle.cpp",
     "int s = free_slots[j], e = misses[j];", "int s = free_slots[free_slots.size() - 1 - j], e = misses[j];"),
    ("slot policy evicts the running token's experts", "oracle.cpp",
     "      keep[in_use[k]] = 1;\n", ""),
    ("hot cache evicts the most recently staged first", "oracle.py",
     "free.sort(key=lambda c: (int(stamp[c]), c))", "free.sort(key=lambda c: (-int(stamp[c]), c))"),
    ("hot cache takes the running token's entries", "oracle.py",
     "stamp[c] < tick - 1]", "stamp[c] < tick]"),
    ("affine codec without the bias", "oracle.py",
     "return s[:, g] * nib + b[:, g]", "return s[:, g] * nib"),
    ("bf16 decode: exponent bias off by one", "oracle.py",
     "(expo - 134)", "(expo - 133)"),
    ("affine layer step without the residual", "oracle.py",
     'out["h_out"] = ha + moe_decode_affine(', 'out["h_out"] = 0.0 * ha + moe_decode_affine('),
]


def _run_pins(mutant):
    """Returns (name, pytest return code, tail of its output)."""
    name, fname, text, repl = mutant
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        dst = os.path.join(tmp, "oracle")
        shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                        ignore=shutil.ignore_patterns("liboracle.so*", "__pycache__"))
        if fname is not None:
            path = os.path.join(dst, fname)
            src = open(path).read()
            assert src.count(text) == 1, f"{name}: mutation site not unique ({src.count(text)})"
            open(path, "w").write(src.replace(text, repl))
        # run from the copy's directory: `python -m` puts the working
        # directory first on sys.path, so `import oracle` finds the copy
        env = dict(os.environ, PYTHONPATH=os.pathsep.join([tmp, ROOT]), PYTHONDONTWRITEBYTECODE="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-rf", "-p",
                            "no:cacheprovider", "--rootdir", ROOT, *PIN_FILES], cwd=tmp, env=env,
                           capture_output=True, text=True, timeout=600)
        probe = subprocess.run([sys.executable, "-c", "import oracle, os; print(os.path.dirname("
                                "os.path.abspath(oracle.__file__)))"], cwd=tmp, env=env,
                               capture_output=True, text=True, timeout=120)
        assert probe.stdout.strip() == dst, f"{name}: the copy is not the oracle imported"
        out = r.stdout + r.stderr
        # the pin that caught it: pytest's short summary line "FAILED <id> - ..."
        caught = [l.split()[1] for l in out.splitlines() if l.startswith("FAILED ")]
        errors = [l for l in out.splitlines() if l.startswith("ERROR ")]
        return name, r.returncode, caught, errors, out[-1500:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.timeout(900)
def test_every_mutant_is_caught_and_the_copy_passes():
    jobs = [("unmodified copy", None, None, None)] + MUTANTS
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run_pins, jobs))
    name, rc, caught, errors, out = results[0]
    assert rc == 0, f"the unmodified oracle copy fails its pins:\n{out}"
    # caught = a pin test failed (not an error in building or collecting)
    survived = [(n, o) for n, rc, caught, errors, o in results[1:]
                if rc != 1 or not caught or errors]
    assert not survived, "mutants not caught by any pin: " + ", ".join(n for n, _ in survived) + \
        "\n" + "\n".join(o for _, o in survived)
    for n, rc, caught, errors, o in results[1:]:
        print(f"{n}: caught by {caught[0].split('/')[-1]}")
