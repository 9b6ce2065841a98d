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
    # backward pass
    ("bwd-adjoint-not-decayed", "          lam[n] *= abar;\n", "", None),
    ("bwd-dC-previous-state", "pdC[n * L + t] += dr * hs[(t + 1) * N + n];", "pdC[n * L + t] += dr * hs[t * N + n];", None),
    ("bwd-dAbar-new-state", "const double dabar = lam[n] * hs[t * N + n];",
     "const double dabar = lam[n] * hs[(t + 1) * N + n];", None),
    ("bwd-dDelta-no-input-term", "ddelta += dabar * abar * a + lam[n] * bt * xr[t] * dcd;", "ddelta += dabar * abar * a;", None),
    ("bwd-dDelta-no-decay-term", "ddelta += dabar * abar * a + lam[n] * bt * xr[t] * dcd;",
     "ddelta += lam[n] * bt * xr[t] * dcd;", None),
    ("bwd-dA-missing-delta", "dA[d * N + n] += dabar * abar * delta + lam[n] * bt * xr[t] * dca;",
     "dA[d * N + n] += dabar * abar + lam[n] * bt * xr[t] * dca;", None),
    ("bwd-dA-no-zoh-term", "dA[d * N + n] += dabar * abar * delta + lam[n] * bt * xr[t] * dca;",
     "dA[d * N + n] += dabar * abar * delta;", None),
    ("bwd-dB-missing-x", "pdB[n * L + t] += lam[n] * c * xr[t];", "pdB[n * L + t] += lam[n] * c;", None),
    ("bwd-dx-missing-skip", "double dxv = dr * skip;", "double dxv = 0.0;", None),
    ("bwd-dx-missing-B", "dxv += lam[n] * c * bt;", "dxv += lam[n] * c;", None),
    ("bwd-dz-sigmoid", "dz[ch * L + t] = dy[ch * L + t] * rr[t] * dsilu(zr[t]);",
     "dz[ch * L + t] = dy[ch * L + t] * rr[t] * sigmoid(zr[t]);", None),
    ("bwd-dr-ungated", "const double dr = dy[ch * L + t] * g;", "const double dr = dy[ch * L + t];", None),
    ("bwd-softplus-derivative-no-bias", "const double dv = ddelta * sigmoid(dtr[t] + bias);",
     "const double dv = ddelta * sigmoid(dtr[t]);", None),
    ("bwd-dbias-dropped", "        ddt_bias[d] += dv;\n", "", None),
    ("bwd-dDskip-ungated", "dDskip[d] += dr * xr[t];", "dDskip[d] += dy[ch * L + t] * xr[t];", None),
    ("bwd-dB-one-row", "dB[b * N * L + i] += wk[i];", "dB[i] += wk[i];", None),
    ("bwd-dh-final-ignored", "lam[n] = dh_final ? dh_final[ch * N + n] : 0.0;", "lam[n] = 0.0;", None),
    ("bwd-readout-skip-missing", "rr[t] = acc + skip * xr[t];", "rr[t] = acc;", None),
    ("bwd-psi-series", "0.5 + u * (1.0 / 3.0 + u * (1.0 / 8.0 + u * (1.0 / 30.0)))",
     "0.5 + u * (1.0 / 6.0 + u * (1.0 / 8.0 + u * (1.0 / 30.0)))", None),
    ("bwd-psi-closed-form", "psi = (u * eu - expm1(u)) / (u * u);", "psi = (u * eu + expm1(u)) / (u * u);", None),
    ("bwd-zoh-dc-ddelta", "*dc_ddelta = eu;", "*dc_ddelta = 1.0;", None),
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
