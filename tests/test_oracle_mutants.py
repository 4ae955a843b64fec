"""Plant plausible mistakes in the oracle (on the CPU) and require the pins
to catch every one of them.

Each mutant is a text edit of ``oracle/osm_oracle.c`` compiled into a
temporary library; the edit must apply (so this list tracks the source), and
at least one pin must fail against the result.  The list includes the pages'
own warnings: forgetting to rescale when the maximum grows, letting padded
keys into the sum, and the merge that forgets to rescale.
"""
import os

import pytest

import oracle
import pins

MUTANTS = [
    # softmax
    ("numerator without max", "y[j] = exp(s[j] - m) / l;", "y[j] = exp(s[j]) / l;"),
    ("normalizer wrong sign", "l += exp(s[j] - m);", "l += exp(m - s[j]);"),
    ("no divide", "y[j] = exp(s[j] - m) / l;", "y[j] = exp(s[j] - m);"),
    ("max misses last entry", "for (int64_t j = 0; j < n; ++j)            /* pass 1",
     "for (int64_t j = 0; j + 1 < n; ++j)            /* pass 1"),
    ("masked row not zero", "for (int64_t j = 0; j < n; ++j) y[j] = 0.0;",
     "for (int64_t j = 0; j < n; ++j) y[j] = 1.0 / (double)n;"),
    ("row stride ignored", "const float *xr = x + r * ld;", "const float *xr = x + r;"),
    # the recurrence
    ("recurrence forgets to rescale", "l = l * alpha + term;", "l = l + term;"),
    ("recurrence rescale wrong sign",
     "double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);",
     "double alpha = (m == -INFINITY) ? 0.0 : exp(m_new - m);"),
    ("recurrence no -inf guard",
     "double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);",
     "double alpha = exp(m - m_new);"),
    # summary and merge
    ("summary unshifted weights", "double w = exp(s[i] - m);", "double w = exp(s[i]);"),
    ("merge forgets to rescale", "double wa = exp(*ma - m), wb = exp(mb - m);",
     "double wa = 1.0, wb = 1.0;"),
    ("merge keeps the smaller max", "double m = *ma > mb ? *ma : mb;",
     "double m = *ma < mb ? *ma : mb;"),
    ("merge rescales only one side", "double wa = exp(*ma - m), wb = exp(mb - m);",
     "double wa = exp(*ma - m), wb = 1.0;"),
    ("merge multiplies identity in", "if (mb == -INFINITY) return;               /* B",
     "if (0) return;               /* B"),
    ("merge no final divide", "for (int64_t k = 0; k < d; ++k) acc[k] /= l;",
     "for (int64_t k = 0; k < d; ++k) acc[k] /= 1.0;"),
    ("merge lse drops m", "lse[r] = m + log(l);", "lse[r] = log(l);"),
    # attention
    ("scale dropped", "s[j] = scale * dot;", "s[j] = dot;"),
    ("scale squared", "s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    ("lse drops m", "lse[t] = m + log(l);", "lse[t] = log(l);"),
    ("causal strict", "if (causal && n_vis > i + 1) n_vis = i + 1;",
     "if (causal && n_vis > i) n_vis = i;"),
    ("causal ignored", "if (causal && n_vis > i + 1) n_vis = i + 1;", "if (0) n_vis = i + 1;"),
    ("padded queries attend", "int64_t n_vis = (i < Lq) ? Lk : 0;", "int64_t n_vis = Lk;"),
    ("padded keys enter the sum", "int64_t Lk = clamp_len(seqlens_k, b, Nk);",
     "int64_t Lk = Nk;"),
    ("kv head interleaved", "int64_t g = h / group;", "int64_t g = h % Hkv;"),
    ("values from keys", "orow[c] += y[j] * (double)vh[j * d + c];",
     "orow[c] += y[j] * (double)kh[j * d + c];"),
    ("value row index off", "orow[c] += y[j] * (double)vh[j * d + c];",
     "orow[c] += y[j] * (double)vh[(n_vis - 1 - j) * d + c];"),
    ("query row index off", "const float *qr = q + ((b * Hq + h) * Nq + i) * d;",
     "const float *qr = q + ((b * Hq + h) * Nq + (Nq - 1 - i)) * d;"),
    ("dot product drops first dim", "for (int64_t c = 0; c < d; ++c)\n                        dot +=",
     "for (int64_t c = 1; c < d; ++c)\n                        dot +="),
    ("batch index from heads", "int64_t b = row / (Nq * Hq);", "int64_t b = 0;"),
    # lse-form merge
    ("lse merge unweighted", "double wa = exp(la - L), wb = exp(lb - L);",
     "double wa = 0.5, wb = 0.5;"),
    ("lse merge plain max", "double L = mx + log(exp(la - mx) + exp(lb - mx));",
     "double L = mx;"),
    # backward
    ("bwd drops the row term", "double ds = y[j] * (gy[j] - yg);", "double ds = y[j] * gy[j];"),
    ("bwd row term wrong sign", "double ds = y[j] * (gy[j] - yg);",
     "double ds = y[j] * (gy[j] + yg);"),
    ("bwd dk unscaled", "dkh[j * d + c] += scale * ds * (double)qr[c];",
     "dkh[j * d + c] += ds * (double)qr[c];"),
    ("bwd dq from values", "dqr[c] += scale * ds * (double)kh[j * d + c];",
     "dqr[c] += scale * ds * (double)vh[j * d + c];"),
    ("bwd dv weighted by score gradient", "dvh[j * d + c] += y[j] * (double)dor[c];",
     "dvh[j * d + c] += ds * (double)dor[c];"),
    ("bwd dL/dy from keys", "dot += (double)dor[c] * (double)vh[j * d + c];",
     "dot += (double)dor[c] * (double)kh[j * d + c];"),
    ("bwd causal ignored",
     "                        if (causal && n_vis > i + 1) n_vis = i + 1;\n"
     "                        if (n_vis == 0) continue;",
     "                        if (n_vis == 0) continue;"),
    ("bwd first head of the group only", "for (int64_t h = g * group; h < (g + 1) * group; ++h)",
     "for (int64_t h = g * group; h < g * group + 1; ++h)"),
    ("bwd padded keys enter",
     "int64_t Lk = clamp_len(seqlens_k, b, Nk);\n                const float *kh",
     "int64_t Lk = Nk;\n                const float *kh"),
    ("bwd padded queries enter",
     "                        int64_t n_vis = (i < Lq) ? Lk : 0;\n"
     "                        if (causal",
     "                        int64_t n_vis = Lk;\n"
     "                        if (causal"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) >= 1, f"mutant '{name}' no longer applies"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new, 1))
    lib = tmp_path / f"libmutant_{abs(hash(name))}.so"
    oracle.compile_oracle(str(src), str(lib))
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant '{name}'"
