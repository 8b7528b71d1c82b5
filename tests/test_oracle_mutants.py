"""Planted mistakes: each mutant below is one plausible slip in the oracle
(a dropped term, a wrong sign, index or operand), planted in a copy of the
oracle on the CPU, and every one must fail at least one pin of
``test_oracle_pins.py``.  That is what makes the pins evidence for the
oracle: a slip that no pin notices could sit in the oracle unseen.

A C mutant is compiled the way the oracle is (gcc, IEEE double, no FMA
contraction) into a temporary library that the oracle module loads in place
of its own; a Python mutant runs as a fresh module that the pins see in
place of the oracle.  Nothing here touches the HIP library.  CPU only.
"""
import os
import subprocess
import time
import types

import pytest

import oracle
from tests import test_oracle_pins as pins

C, PY = "gdn_oracle.c", "__init__.py"

# (name, file, text in the oracle, the slip that replaces it)
MUTANTS = [
    # one gated delta-rule step
    ("gate sign", C, "const double a = exp(g);", "const double a = exp(-g);"),
    ("state read with q", C, "rk += row[i] * k[i];", "rk += row[i] * q[i];"),
    ("output read with k", C, "rq += row[i] * q[i];", "rq += row[i] * k[i];"),
    ("delta without the decay", C, "const double e = beta * (v[j] - a * Sk[j]);",
     "const double e = beta * (v[j] - Sk[j]);"),
    ("delta without beta", C, "const double e = beta * (v[j] - a * Sk[j]);", "const double e = (v[j] - a * Sk[j]);"),
    ("delta sign", C, "const double e = beta * (v[j] - a * Sk[j]);", "const double e = beta * (v[j] + a * Sk[j]);"),
    ("state not decayed", C, "row[i] = a * row[i] + e * k[i];", "row[i] = row[i] + e * k[i];"),
    ("state written with q", C, "row[i] = a * row[i] + e * k[i];", "row[i] = a * row[i] + e * q[i];"),
    ("output not decayed", C, "y[j] = a * Sq[j] + kq * e;", "y[j] = Sq[j] + kq * e;"),
    ("output from the old state", C, "y[j] = a * Sq[j] + kq * e;", "y[j] = a * Sq[j];"),
    ("output without k.q", C, "y[j] = a * Sq[j] + kq * e;", "y[j] = a * Sq[j] + e;"),
    ("k.q taken as k.k", C, "for (int i = 0; i < Dk; ++i) kq += k[i] * q[i];",
     "for (int i = 0; i < Dk; ++i) kq += k[i] * k[i];"),
    ("decode heads interleaved", C, "      const int hk = hv / group;\n      const size_t n",
     "      const int hk = hv % Hk;\n      const size_t n"),
    # prefill over a pool
    ("prefill heads interleaved", C, "      const int hk = hv / group;\n      double* S = pool",
     "      const int hk = hv % Hk;\n      double* S = pool"),
    ("L2 norm without the root", C, "const double r = 1.0 / sqrt(ss + eps);", "const double r = 1.0 / (ss + eps);"),
    ("L2 norm eps outside the root", C, "const double r = 1.0 / sqrt(ss + eps);",
     "const double r = 1.0 / (sqrt(ss) + eps);"),
    ("q not scaled", C, "for (int i = 0; i < Dk; ++i) qn[i] *= scale;", ""),
    ("q not normalised", C, "          l2_normalise(qt, qn, Dk, eps);", "          memcpy(qn, qt, sizeof(double) * Dk);"),
    ("k not normalised", C, "          l2_normalise(kt, kn, Dk, eps);", "          memcpy(kn, kt, sizeof(double) * Dk);"),
    ("slot from the sequence number", C, "double* S = pool + ((size_t)slot * Hv + hv) * (size_t)Dv * Dk;",
     "double* S = pool + ((size_t)s * Hv + hv) * (size_t)Dv * Dk;"),
    ("beta of head 0", C, "g[th], beta[th], y + th * Dv", "g[th], beta[(size_t)t * Hv], y + th * Dv"),
    ("gate of head 0", C, "g[th], beta[th], y + th * Dv", "g[(size_t)t * Hv], beta[th], y + th * Dv"),
    ("last token dropped", C, "for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {",
     "for (int64_t t = cu_seqlens[s]; t + 1 < cu_seqlens[s + 1]; ++t) {"),
    # Comba step
    ("Comba read with k", C, "Stp[j] += pi * row[j];", "Stp[j] += kh[i] * row[j];"),
    ("Comba write with p", C, "row[j] = a * row[j] + kh[i] * Stp[j];", "row[j] = a * row[j] + ph[i] * Stp[j];"),
    ("Comba u without the decay", C, "const double u = beta[n] * (vh[j] - a * Stp[j]);",
     "const double u = beta[n] * (vh[j] - Stp[j]);"),
    ("Comba u without beta", C, "const double u = beta[n] * (vh[j] - a * Stp[j]);",
     "const double u = (vh[j] - a * Stp[j]);"),
    ("Comba output from the old state", C, "o[n * V + j] = a * Stq[j] + kq * u;", "o[n * V + j] = a * Stq[j];"),
    ("Comba output not decayed", C, "o[n * V + j] = a * Stq[j] + kq * u;", "o[n * V + j] = Stq[j] + kq * u;"),
    ("Comba k.q unscaled", C, "for (int i = 0; i < K; ++i) kq += kh[i] * (scale * qh[i]);",
     "for (int i = 0; i < K; ++i) kq += kh[i] * qh[i];"),
    ("Comba q unscaled", C, "const double pi = ph[i], qi = scale * qh[i];", "const double pi = ph[i], qi = qh[i];"),
    ("Comba state not decayed", C, "row[j] = a * row[j] + kh[i] * Stp[j];", "row[j] = row[j] + kh[i] * Stp[j];"),
    # gates
    ("gate without exp(A_log)", C, "g[n] = -exp(A_log[h]) * sp;", "g[n] = -A_log[h] * sp;"),
    ("gate sign (log space)", C, "g[n] = -exp(A_log[h]) * sp;", "g[n] = exp(A_log[h]) * sp;"),
    ("gate without dt_bias", C, "const double x = a[n] + dt_bias[h];", "const double x = a[n];"),
    ("softplus tail for negative x", C, "log1p(exp(-fabs(x)))", "log1p(exp(-x))"),
    ("softplus without max(x, 0)", C, "const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));",
     "const double sp = log1p(exp(-fabs(x)));"),
    ("beta sign", C, "beta[n] = 1.0 / (1.0 + exp(-b[n]));", "beta[n] = 1.0 / (1.0 + exp(b[n]));"),
    # conv + SiLU
    ("history read newest first", C, "double win[4] = {h[0], h[1], h[2], 0.0};",
     "double win[4] = {h[2], h[1], h[0], 0.0};"),
    ("taps reversed", C, "pre += win[m] * W[(size_t)c * 4 + m];", "pre += win[m] * W[(size_t)c * 4 + 3 - m];"),
    ("history shifted by one", C, "      h[0] = win[0];\n      h[1] = win[1];\n      h[2] = win[2];",
     "      h[0] = win[1];\n      h[1] = win[2];\n      h[2] = win[3];"),
    ("history not written", C, "      h[0] = win[0];\n      h[1] = win[1];\n      h[2] = win[2];", ""),
    ("SiLU sign", C, "out[(size_t)t * C + c] = pre / (1.0 + exp(-pre));",
     "out[(size_t)t * C + c] = pre / (1.0 + exp(pre));"),
    ("no SiLU", C, "out[(size_t)t * C + c] = pre / (1.0 + exp(-pre));", "out[(size_t)t * C + c] = pre;"),
    # gated RMS norm
    ("sum of squares for the mean", C, "const double r = 1.0 / sqrt(ss / Dv + eps);",
     "const double r = 1.0 / sqrt(ss + eps);"),
    ("RMS eps outside the root", C, "const double r = 1.0 / sqrt(ss / Dv + eps);",
     "const double r = 1.0 / (sqrt(ss / Dv) + eps);"),
    ("no gamma", C, "y[base + j] = o[base + j] * r * gamma[j] * (1.0 / (1.0 + exp(-z[base + j])));",
     "y[base + j] = o[base + j] * r * (1.0 / (1.0 + exp(-z[base + j])));"),
    ("gate sigmoid sign", C, "y[base + j] = o[base + j] * r * gamma[j] * (1.0 / (1.0 + exp(-z[base + j])));",
     "y[base + j] = o[base + j] * r * gamma[j] * (1.0 / (1.0 + exp(z[base + j])));"),
    ("SiLU gate instead of sigmoid", C,
     "y[base + j] = o[base + j] * r * gamma[j] * (1.0 / (1.0 + exp(-z[base + j])));",
     "y[base + j] = o[base + j] * r * gamma[j] * (z[base + j] / (1.0 + exp(-z[base + j])));"),
    # decode windows and Comba prefill (Python)
    ("window commits one token late", PY, "if t + 1 == commit:", "if t == commit:"),
    ("window keeps the last state", PY, "return kept, np.stack(ys, axis=1)", "return S, np.stack(ys, axis=1)"),
    ("Comba slot from the sequence number", PY, "S = P[ci[s]][None].copy()", "S = P[s][None].copy()"),
    ("Comba state not written back", PY, "        P[ci[s]] = S[0]\n", ""),
    ("Comba default scale of one", PY, "g[t][None], scale=scale, inplace=True)",
     "g[t][None], scale=1.0 if scale is None else scale, inplace=True)"),
]


def _calls(fn):
    """fn's parameter sets from its parametrize marks (cartesian product)."""
    sets = [{}]
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names = [n.strip() for n in m.args[0].split(",")]
        new = []
        for base in sets:
            for val in m.args[1]:
                d = dict(base)
                d.update(zip(names, val if len(names) > 1 else (val,)))
                new.append(d)
        sets = new
    return sets


@pytest.fixture(scope="module")
def pin_calls():
    """Every pin call, fastest first (timed on the real oracle, which must
    pass them all), so that a mutant's first failure comes early."""
    calls = []
    for name in sorted(n for n in dir(pins) if n.startswith("test_")):
        fn = getattr(pins, name)
        for kw in _calls(fn):
            t = time.perf_counter()
            fn(**kw)
            calls.append((time.perf_counter() - t, name, fn, kw))
    calls.sort(key=lambda c: c[0])
    return [(name, fn, kw) for _, name, fn, kw in calls]


def _first_failure(calls):
    for name, fn, kw in calls:
        try:
            fn(**kw)
        except Exception as e:  # an assertion, or the oracle refusing its input
            return f"{name}{kw or ''}: {type(e).__name__}"
    return None


@pytest.mark.parametrize("name,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(name, fname, old, new, pin_calls, tmp_path, monkeypatch):
    path = os.path.join(os.path.dirname(oracle.__file__), fname)
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"the text of mutant {name!r} is not in {fname} exactly once"
    mutated = src.replace(old, new)
    if fname == C:
        c_file, so = tmp_path / "mutant.c", tmp_path / "libmutant.so"
        c_file.write_text(mutated)
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", str(so), str(c_file), "-lm"])
        monkeypatch.setattr(oracle, "_LIB", str(so))
        monkeypatch.setattr(oracle, "_lib", None)
    else:
        mod = types.ModuleType("oracle")
        mod.__file__ = oracle.__file__
        exec(compile(mutated, oracle.__file__, "exec"), mod.__dict__)
        monkeypatch.setattr(pins, "oracle", mod)
    caught = _first_failure(pin_calls)
    assert caught is not None, f"mutant {name!r} passes every pin"
