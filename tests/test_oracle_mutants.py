"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
every one of them fails at least one pin -- evidence that the pins constrain
each function of the oracle, not only its happy path."""
import re
import shutil

import pytest

import oracle
from tests import pins

# (function, text in its body, replacement, what the slip is)
MUTANTS = [
    ("oracle_fwd", "S[e * M + m] += (double)k[i * E + e]", "S[e * M + m] += (double)q[i * E + e]",
     "state built from q"),
    ("oracle_fwd", "acc += (double)q[i * E + e] * S[e * M + m]", "acc += (double)k[i * E + e] * S[e * M + m]",
     "state read with k instead of q"),
    ("oracle_fwd", "* (double)v[i * M + m];", "* (double)v[(i > 0 ? i - 1 : 0) * M + m];",
     "off-by-one row of v"),
    ("oracle_fwd", "S[e * M + m] += (double)k", "S[e * M + m] -= (double)k", "sign of the update"),
    ("oracle_fwd_brute", "j <= i", "j < i", "exclusive prefix"),
    ("oracle_fwd_brute", "a * (double)v[j * M + m]", "a * (double)v[i * M + m]", "wrong row of v"),
    ("oracle_linattn", "double den = eps;", "double den = 0.0;", "dropped eps"),
    ("oracle_linattn", "z[e] += fk[e];", "z[e] += fq[e];", "normaliser from q"),
    ("phi", "x + 1.0", "x", "elu without the +1"),
    ("phi", "exp(x)", "x", "identity on the negative branch"),
    ("oracle_linattn_brute", "den += a;", "den += 1.0;", "uniform normaliser"),
    ("oracle_bwd", "for (int64_t i = L - 1; i >= 0; --i)", "for (int64_t i = 0; i < L; ++i)",
     "reverse sweep run forwards"),
    ("oracle_bwd", "acc += R[e * M + m] * (double)v[i * M + m]", "acc += R[e * M + m] * (double)go[i * M + m]",
     "dk from dO"),
    ("oracle_bwd", "acc += R[e * M + m] * (double)k[i * E + e]", "acc += R[e * M + m] * (double)q[i * E + e]",
     "dv from q"),
    ("oracle_bwd", "acc += S[e * M + m] * (double)go[i * M + m]", "acc += S[e * M + m] * (double)v[i * M + m]",
     "dq from v"),
    ("oracle_bwd_brute", "dk[j * E + e] += gv * (double)q[i * E + e]", "dk[j * E + e] += gv * (double)q[j * E + e]",
     "dk with the wrong row of q"),
    ("oracle_bwd_brute", "j <= i", "j < i", "exclusive backward"),
    ("oracle_bwd_brute", "dv[j * M + m] += qk * (double)go[i * M + m]", "dv[j * M + m] += qk * (double)go[j * M + m]",
     "dv with the wrong row of dO"),
    ("oracle_state", "(double)v[j * M + m]", "(double)v[(L - 1 - j) * M + m]", "state with reversed v"),
    ("oracle_fwd", "S[x] = (double)S0[s * E * M + x];", "S[x] = 0.0;", "initial state ignored"),
    ("oracle_fwd", "if (Sfin) memcpy(Sfin + s * E * M, S,", "if (Sfin) memcpy(Sfin + s * E * M, S + 1,",
     "final state shifted by one"),
    ("oracle_fwd_brute", "c += (double)q[i * E + e] * (double)S0", "c += (double)k[i * E + e] * (double)S0",
     "carried state read with k"),
    ("oracle_linattn", "z[e] = (double)z0[s * E + e];", "z[e] = 0.0;", "carried z ignored"),
    ("oracle_linattn_brute", "if (z0) den += c * (double)z0[s * E + e];", "if (z0) den += (double)z0[s * E + e];",
     "carried z not weighted by phi(q)"),
    ("oracle_bwd", "S[x] = (double)S0[s * E * M + x];", "S[x] = (double)S0[s * E * M + (x % E) * M + x / E];",
     "initial state transposed in dq"),
    ("oracle_bwd_brute", "g0[e * M + m] += (double)q[i * E + e]", "g0[e * M + m] += (double)k[i * E + e]",
     "gradient of the initial state from k"),
    ("oracle_linattn_bwd", "dd[i] = -gn / (den * den);", "dd[i] = gn / (den * den);", "sign of the denominator term"),
    ("oracle_linattn_bwd", "double acc = dd[i] * z[e];", "double acc = 0.0;", "denominator term of dq dropped"),
    ("oracle_linattn_bwd", "r[e] += dd[i] * c[i * E + e];", "r[e] += dd[i] * f[i * E + e];", "dk's denominator sum from k"),
    ("oracle_linattn_bwd", "dq[i * E + e] = acc * (feature_map ? dphi((double)q[i * E + e]) : 1.0);",
     "dq[i * E + e] = acc;", "chain rule through phi dropped for q"),
    ("dphi", "exp(x)", "1.0", "phi' = 1 on the negative branch"),
    ("oracle_linattn_bwd", "acc += R[e * M + m] * f[i * E + e];", "acc += R[e * M + m] * (double)k[i * E + e];",
     "dv from the raw k"),
]


def mutate(src: str, func: str, old: str, new: str) -> str:
    """Replace the first ``old`` inside the definition of C function ``func``."""
    m = re.search(rf"^(?:static )?(?:void|double|int) {func}\(", src, re.M)
    assert m, func
    pos = src.index(old, m.end())
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("func,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, func, old, new, what):
    with open(oracle.SRC) as f:
        src = f.read()
    o = oracle.build_variant(mutate(src, func, old, new), str(tmp_path))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {what}"
