"""Planted mistakes in the CPU reference must fail at least one pin.

Each mutant is a copy of oracle.c with one plausible mistake (a dropped term,
a wrong sign, index or operand), compiled on the CPU into a temporary
library. The pin battery runs against it and at least one pin must fail.
The real source is never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("no_scale", "prow[j] = scale * dot;", "prow[j] = dot;"),
    ("causal_strict", "if (causal && j > i)", "if (causal && j >= i)"),
    ("causal_upper", "if (causal && j > i)", "if (causal && j < i)"),
    ("mask_transposed", "mask[(i / blk) * nb + (j / blk)]", "mask[(j / blk) * nb + (i / blk)]"),
    ("mask_ignored", "if (mask && mask[(i / blk) * nb + (j / blk)] == 0)", "if (0)"),
    ("qk_index", "dot += q[i * d + c] * k[j * d + c];", "dot += q[i * d + c] * k[i * d + c];"),
    ("no_max_shift_in_lse", "*lse = m + log(l);", "*lse = log(l);"),
    ("lse_log2", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("no_normalise", "prow[j] /= l;", "prow[j] /= 1.0;"),
    ("pv_operand", "orow[c] += prow[j] * v[j * d + c];", "orow[c] += prow[j] * v[i * d + c];"),
    ("D_uses_v", "Di += dout[i * d + c] * o[i * d + c];", "Di += dout[i * d + c] * v[i * d + c];"),
    ("D_dropped", "dS[i * N + j] = pij * (dp - Di);", "dS[i * N + j] = pij * dp;"),
    ("dS_sign", "dS[i * N + j] = pij * (dp - Di);", "dS[i * N + j] = pij * (Di - dp);"),
    ("dP_operand", "dp += dout[i * d + c] * v[j * d + c];", "dp += dout[i * d + c] * k[j * d + c];"),
    ("dQ_operand", "dq[i * d + c] += s * k[j * d + c];", "dq[i * d + c] += s * q[j * d + c];"),
    ("dQ_no_scale", "dq[i * d + c] *= scale;", "dq[i * d + c] *= 1.0;"),
    ("dK_operand", "dk[j * d + c] += s * q[i * d + c];", "dk[j * d + c] += s * k[i * d + c];"),
    ("dK_no_scale", "dk[j * d + c] *= scale;", "dk[j * d + c] *= 1.0;"),
    ("dV_uses_dS", "dv[j * d + c] += pij * dout[i * d + c];", "dv[j * d + c] += s * dout[i * d + c];"),
    ("kv_top_left", "const long last = Nk - Nq + i;", "const long last = i;"),
    ("kv_no_normalise", "const double p = srow[j] / l;", "const double p = srow[j];"),
    ("kv_lse_no_max", "*lse = log(l) + m;", "*lse = log(l);"),
    ("kv_qk_index", "dot += q[c] * k[j * d + c];", "dot += q[c] * k[c];"),
    ("kv_pv_operand", "orow[c] += p * v[j * d + c];", "orow[c] += p * v[c];"),
    ("kv_no_scale", "srow[j] = scale * dot;", "srow[j] = dot;"),
    ("philox_multiplier", "0xD2511F53u", "0xD2511F55u"),
    ("philox_weyl", "k0 += 0x9E3779B9u;", "k0 += 0x9E3779BBu;"),
    ("drop_counter_swap",
     "const unsigned int ctr[4] = {(unsigned int)(j / 4), (unsigned int)i, (unsigned int)bh, 0u};",
     "const unsigned int ctr[4] = {(unsigned int)i, (unsigned int)(j / 4), (unsigned int)bh, 0u};"),
    ("drop_keep_flipped", "return w[j % 4] >= drop_threshold(p_drop);",
     "return w[j % 4] < drop_threshold(p_drop);"),
    ("drop_O_no_rescale", "const double pt = P[i * N + j] * Z[i * N + j] * inv_keep;",
     "const double pt = P[i * N + j] * Z[i * N + j];"),
    ("drop_dV_no_mask", "const double pt = inv_keep * Z[i * N + j] * P[i * N + j];",
     "const double pt = inv_keep * P[i * N + j];"),
    ("drop_dS_no_mask", "g = pij * (Z[i * N + j] * dp * inv_keep - D[i]);",
     "g = pij * (dp * inv_keep - D[i]);"),
    ("dV_transposed", "double pij = P[i * N + j];\n                if (s != 0.0)",
     "double pij = P[j * N + i];\n                if (s != 0.0)"),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    mutated = src.replace(old, new)
    d = tmp_path / name
    d.mkdir()
    (d / "oracle.c").write_text(mutated)
    (d / "oracle.h").write_text(open(os.path.join(os.path.dirname(SRC), "oracle.h")).read())
    lib = d / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    str(d / "oracle.c"), "-o", str(lib), "-lm"], check=True)
    return oracle.Oracle(str(lib))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = _build(tmp_path, name, old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
