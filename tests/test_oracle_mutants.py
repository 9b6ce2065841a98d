"""Every plausible mistake planted in a copy of the oracle must fail some pin.

The mistakes are planted in the oracle's C source on the CPU (text substitution
into a temporary copy, compiled with gcc); the real oracle is untouched.  This is
what makes the pins in ``pins.py`` evidence: a dropped term, a wrong sign, index
or operand anywhere in the oracle is caught by at least one of them.
"""
import pytest

import oracle
from pins import ALL_PINS

# (name, original text, replacement, occurrence index or None for all)
MUTANTS = [
    ("drop-skip", "double out = acc + skip * xr[t];", "double out = acc;", None),
    ("skip-uses-wrong-x", "double out = acc + skip * xr[t];", "double out = acc + skip * xr[t > 0 ? t - 1 : 0];", None),
    ("sign-of-A", "const double abar = exp(delta * a);", "const double abar = exp(-delta * a);", 0),
    ("A-indexed-by-batch", "const double a = A[d * dstate + n];", "const double a = A[b * dstate + n];", 0),
    ("A-transposed", "const double a = A[d * dstate + n];", "const double a = A[n * dim + d];", 0),
    ("B-transposed", "const double bt = B[(b * dstate + n) * seqlen + t];",
     "const double bt = B[(b * seqlen + t) * dstate + n];", None),
    ("C-transposed", "const double ct = C[(b * dstate + n) * seqlen + t];",
     "const double ct = C[(b * seqlen + t) * dstate + n];", None),
    ("B-C-swapped", "const double ct = C[(b * dstate + n) * seqlen + t];",
     "const double ct = B[(b * dstate + n) * seqlen + t];", None),
    ("B-time-shift", "const double bt = B[(b * dstate + n) * seqlen + t];",
     "const double bt = B[(b * dstate + n) * seqlen + (t > 0 ? t - 1 : 0)];", None),
    ("readout-before-update",
     "        h[n] = abar * h[n] + bbar_x(delta, a, abar, bt, xr[t], zoh);\n        acc += ct * h[n];",
     "        acc += ct * h[n];\n        h[n] = abar * h[n] + bbar_x(delta, a, abar, bt, xr[t], zoh);", None),
    ("softplus-branch", "return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));", "return (v > 0.0 ? v : 0.0) + log1p(exp(-v));", None),
    ("softplus-as-exp", "return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));", "return exp(v);", None),
    ("bias-dropped", "softplus(dtr[t] + bias)", "softplus(dtr[t])", None),
    ("bias-outside", "softplus(dtr[t] + bias)", "(softplus(dtr[t]) + bias)", None),
    ("gate-sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));", None),
    ("gate-on-readout-only", "double out = acc + skip * xr[t];\n      if (zr) out *= silu(zr[t]);",
     "double out = acc;\n      if (zr) out *= silu(zr[t]);\n      out += skip * xr[t];", None),
    ("h0-ignored", "h[n] = h0 ? h0[ch * dstate + n] : 0.0;", "h[n] = 0.0;", None),
    ("euler-missing-delta", "if (!zoh) return delta * b * x;", "if (!zoh) return b * x;", None),
    ("zoh-times-A", "return expm1(delta * a) / a * b * x;", "return expm1(delta * a) * a * b * x;", None),
    ("zoh-no-expm1", "return expm1(delta * a) / a * b * x;", "return exp(delta * a) / a * b * x;", None),
    ("final-state-row", "h_final[ch * dstate + n] = h[n];", "h_final[ch * dstate + n] = h[dstate - 1 - n];", None),
    ("last-token-dropped", "for (int64_t t = 0; t < seqlen; ++t) {", "for (int64_t t = 0; t < seqlen; ++t) { if (t == seqlen - 1 && seqlen > 1) { yr[t] = yr[t - 1]; break; }", None),
    ("decode-no-input", "s[n] = abar * s[n] + in;", "s[n] = abar * s[n];", None),
    ("decode-readout-old-state", "      s[n] = abar * s[n] + in;\n      acc += C[b * dstate + n] * s[n];",
     "      acc += C[b * dstate + n] * s[n];\n      s[n] = abar * s[n] + in;", None),
    ("decode-bias-dropped", "const double v = dt[ch] + (dt_bias ? dt_bias[d] : 0.0);", "const double v = dt[ch];", None),
    ("decode-skip-dropped", "double out = acc + (Dskip ? Dskip[d] : 0.0) * x[ch];", "double out = acc;", None),
    ("decode-B-by-channel", "in = delta * B[b * dstate + n] * x[ch];", "in = delta * B[(d % batch) * dstate + n] * x[ch];", None),
    ("decode-gate-sign", "if (z) out *= z[ch] / (1.0 + exp(-z[ch]));", "if (z) out *= z[ch] / (1.0 + exp(z[ch]));", None),
]


def _mutate(src: str, old: str, new: str, occurrence):
    count = src.count(old)
    assert count >= 1, "mutant pattern not found: %r" % old
    if occurrence is None:
        return src.replace(old, new)
    i = -1
    for _ in range(occurrence + 1):
        i = src.index(old, i + 1)
    return src[:i] + new + src[i + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    src = oracle.SRC.read_text()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    csrc = tmp_path / ("mut_%s.c" % name)
    csrc.write_text(mutated)
    lib = tmp_path / ("mut_%s.so" % name)
    oracle.compile_oracle(csrc, lib)
    o = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
            caught.append((pin.__name__, str(e)[:80]))
            break
    assert caught, "planted mistake %r passed every pin" % name
