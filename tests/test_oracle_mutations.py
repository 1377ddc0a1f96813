"""Pin strength: plausible mistakes planted in a copy of the oracle (on the CPU)
must each make the pin suite fail.

Every mutant is a textual edit of oracle/mhc_oracle.c compiled into a temporary
directory; the pin suite then runs against it in a subprocess (the oracle
loader honours MHC_ORACLE_TEST_LIB for exactly this).  The real oracle build is
never touched.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mhc_oracle.c")


def _sinkhorn_body(src):
    a = src.index("static void sinkhorn(")
    b = src.index("static void token_gates(")
    return a, b


def _swap_pass_order(src):
    a, b = _sinkhorn_body(src)
    return src[:a] + src[a:b].replace("c[j * S + k]", "c[k * S + j]") + src[b:]


MUTANTS = {
    "eps dropped from the RMS root": lambda s: s.replace(
        "sqrt(ss / (double)n + eps)", "sqrt(ss / (double)n)"),
    "mean over hidden instead of the slab": lambda s: s.replace(
        "sqrt(ss / (double)n + eps)", "sqrt(ss / (double)H + eps)"),
    "weight read column-major": lambda s: s.replace(
        "acc += (double)w[i] * (double)xt[i];",
        "acc += (double)fn_w[i * R + r] * (double)xt[i];"),
    "post gate without the factor 2": lambda s: s.replace(
        "post[k] = 2.0 / (1.0 + exp(-z[S + k]));", "post[k] = 1.0 / (1.0 + exp(-z[S + k]));"),
    "sigmoid sign flipped": lambda s: s.replace(
        "pre[c] = 1.0 / (1.0 + exp(-z[c]));", "pre[c] = 1.0 / (1.0 + exp(z[c]));"),
    "post rows take the comb scale": lambda s: s.replace(
        "if (r < 2 * S) return 1;", "if (r < 2 * S) return 2;"),
    "comb block transposed in the split": lambda s: s.replace(
        "comb[j * S + k] = exp(z[2 * S + j * S + k]);",
        "comb[k * S + j] = exp(z[2 * S + j * S + k]);"),
    "comb block offset by one row": lambda s: s.replace(
        "exp(z[2 * S + j * S + k])", "exp(z[2 * S - 1 + j * S + k])"),
    "one Sinkhorn round too many": lambda s: s.replace(
        "for (int it = 0; it < iters; ++it)", "for (int it = 0; it <= iters; ++it)"),
    "eps missing from the row pass": lambda s: s.replace(
        "for (int k = 0; k < S; ++k) c[j * S + k] = c[j * S + k] / (s + eps);",
        "for (int k = 0; k < S; ++k) c[j * S + k] = c[j * S + k] / s;"),
    "column pass before row pass": _swap_pass_order,
    "collapse reads a stream-interleaved layout": lambda s: s.replace(
        "acc += pre[c] * (double)xt[(long)c * H + i];", "acc += pre[c] * (double)xt[(long)i * S + c];"),
    "post mix with comb transposed": lambda s: s.replace(
        "acc += (double)comb[j * S + k] * (double)xt[(long)j * H + i];",
        "acc += (double)comb[k * S + j] * (double)xt[(long)j * H + i];"),
    "post mix drops the branch term": lambda s: s.replace(
        "double acc = (double)post[k] * (double)ft[i];", "double acc = 0.0;"),
    "norm mean over H + 1": lambda s: s.replace(
        "sqrt(ss / (double)H + norm_eps)", "sqrt(ss / (double)(H + 1) + norm_eps)"),
    "norm eps dropped": lambda s: s.replace(
        "sqrt(ss / (double)H + norm_eps)", "sqrt(ss / (double)H)"),
    "norm weight ignored": lambda s: s.replace(
        "z[t * H + i] = (double)yt[i] * r * (double)nw[i];", "z[t * H + i] = (double)yt[i] * r;"),
    "q8 scale over 128": lambda s: s.replace("amax / 127.0f", "amax / 128.0f"),
    "q8 ties to even": lambda s: s.replace("(signed char)roundf(v)", "(signed char)rintf(v)"),
    "q8 truncates": lambda s: s.replace("(signed char)roundf(v)", "(signed char)v"),
    "q8 blocks of 16": lambda s: s.replace("const float *zb = z + t * H + b * 32;",
                                           "const float *zb = z + t * H + b * 16;"),
    "expand fills only the first stream": lambda s: s.replace(
        "x[(t * S + k) * H + i] = e[t * H + i];",
        "x[(t * S + k) * H + i] = k == 0 ? e[t * H + i] : 0.0f;"),
    "mean divides by S + 1": lambda s: s.replace(
        "y[t * H + i] = acc / (double)S;", "y[t * H + i] = acc / (double)(S + 1);"),
    "mean skips the last stream": lambda s: s.replace(
        "for (int k = 0; k < S; ++k) acc += (double)x[(t * S + k) * H + i];",
        "for (int k = 0; k < S - 1; ++k) acc += (double)x[(t * S + k) * H + i];"),
    "head gate without the RMS rescale": lambda s: s.replace(
        "(double)scale_h[0] * (rinv * acc) + (double)base_h[c];",
        "(double)scale_h[0] * acc + (double)base_h[c];"),
    "head scale multiplies the bias too": lambda s: s.replace(
        "(double)scale_h[0] * (rinv * acc) + (double)base_h[c];",
        "(double)scale_h[0] * ((rinv * acc) + (double)base_h[c]);"),
    "head sigmoid sign flipped": lambda s: s.replace(
        "g[c] = 1.0 / (1.0 + exp(-z));", "g[c] = 1.0 / (1.0 + exp(z));"),
    "head weight rows offset by one": lambda s: s.replace(
        "const float *w = fn_h + (long)c * n;", "const float *w = fn_h + (long)(c + 1) % S * n;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, f"mutation '{name}' did not apply; the oracle source changed"
    cfile = tmp_path / "mutant.c"
    lib = tmp_path / "libmutant.so"
    cfile.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), str(cfile), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, MHC_ORACLE_TEST_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught the planted mistake '{name}':\n{r.stdout[-2000:]}"
