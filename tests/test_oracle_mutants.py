"""The oracle's pins must catch plausible mistakes (no GPU).

Each case below plants one mistake in a COPY of the oracle's C source, builds it
into a temporary library and runs the pin suites (four streams and other stream
counts) against it; the suites must fail.
Nothing here touches the HIP library.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hc_oracle.c")

MUTANTS = {
    "rms over d instead of hc*d": ("sumsq / (double)D", "sumsq / (double)d"),
    "projection not scaled by r": ("(float)(dot * r)", "(float)(dot)"),
    "norm_eps replaced": ("+ norm_eps);", "+ 1e-6);"),
    "flatten order channel-major": ("row[c] = load_elem(x, dtype, t * D + c);",
                                    "row[c] = load_elem(x, dtype, t * D + (c % hc) * d + c / hc);"),
    "pre without eps": ("+ hc_base[j]) + eps);", "+ hc_base[j]));"),
    "post without factor 2": ("(float)(2.0 * sigmoid(", "(float)(1.0 * sigmoid("),
    "pre uses comb scale": ("sigmoid(s0 * m[j]", "sigmoid(s2 * m[j]"),
    "comb logits transposed": ("int i = 2 * hc + j * hc + k;", "int i = 2 * hc + k * hc + j;"),
    "softmax without max shift": ("exp(C[j * hc + k] - mx)", "exp(C[j * hc + k])"),
    "no eps after softmax": ("C[j * hc + k] / s + eps;", "C[j * hc + k] / s;"),
    "one round too few": ("for (int it = 1; it < sinkhorn_iters; ++it)",
                          "for (int it = 2; it < sinkhorn_iters; ++it)"),
    "column step before row step": (
        "        normalise_rows(C, hc, eps);\n            normalise_cols(C, hc, eps);",
        "        normalise_cols(C, hc, eps);\n            normalise_rows(C, hc, eps);"),
    "row normalisation without eps": ("C[j * hc + k] /= (s + eps);", "C[j * hc + k] /= s;"),
    "collapse uses wrong stream": ("load_elem(x, dtype, (t * hc + j) * d + e)",
                                   "load_elem(x, dtype, (t * hc + (hc - 1 - j)) * d + e)"),
    "post sums over comb's second index": ("(double)comb[(t * hc + j) * hc + k]",
                                           "(double)comb[(t * hc + k) * hc + j]"),
    "post drops f": ("(double)post[t * hc + k] * load_elem(f, dtype, t * d + e)", "0.0"),
    "bf16 truncation instead of rounding": ("nearbyint(ldexp(m, 8))", "floor(ldexp(m, 8))"),
    "bf16 subnormal grid 2^-134": ("nearbyint(ldexp(a, 133)), -133)", "nearbyint(ldexp(a, 134)), -134)"),
    "bf16 subnormal truncated": ("ldexp(nearbyint(ldexp(a, 133)), -133)", "ldexp(floor(ldexp(a, 133)), -133)"),
    "bf16 overflow saturates": ("q >= ldexp(1.0, 128) ? INFINITY : (float)q",
                                "q >= ldexp(1.0, 128) ? 0x1.fep127f : (float)q"),
    "rmsnorm mean over d - 1": ("sqrt(ss / (double)d + eps)", "sqrt(ss / (double)(d - 1) + eps)"),
    "rmsnorm gain dropped": ("* r * (double)gain[e]", "* r"),
    "rmsnorm eps replaced": ("sqrt(ss / (double)d + eps)", "sqrt(ss / (double)d + 1e-6)"),
    "mxfp8 no 1e-4 floor": ("(a > 1e-4 ? a : 1e-4)", "(a > 0.0 ? a : 1e-30)"),
    "mxfp8 scale rounded down": ("return m == 0.5 ? e - 1 : e;", "return e - 1;"),
    "mxfp8 divide by 256": ("/ 448.0);", "/ 256.0);"),
    "e4m3 mantissa truncated": ("nearbyint((2.0 * m - 1.0) * 8.0)", "floor((2.0 * m - 1.0) * 8.0)"),
    "e4m3 subnormal step 2^-10": ("nearbyint(ldexp(a, 9))", "nearbyint(ldexp(a, 10))"),
    "e4m3 sign dropped": ("signbit(v) ? 0x80 : 0x00", "0x00"),
    "e4m3 exponent bias 8": ("(((exp + 7) << 3)", "(((exp + 8) << 3)"),
    # mistakes invisible at four streams
    "comb offset fixed at 8": ("int i = 2 * hc + j * hc + k;", "int i = 8 + j * hc + k;"),
    "post offset fixed at 4": ("sigmoid(s1 * m[hc + j] + hc_base[hc + j])", "sigmoid(s1 * m[4 + j] + hc_base[4 + j])"),
    "column sums over 4 rows": ("        for (int j = 0; j < hc; ++j)\n            s += C[j * hc + k];",
                                "        for (int j = 0; j < hc && j < 4; ++j)\n            s += C[j * hc + k];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))
    lib = oracle.build(src=str(src), out=str(tmp_path / "libmutant.so"), werror=False)
    env = dict(os.environ, HC_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_generic_hc.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant '{name}':\n{r.stdout[-2000:]}"
