"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.  This shows the pins constrain each part of
the oracle: the scale, the maximum subtraction, the normaliser, the key/value
strides, the K/V head of each query head, the mask alignment, the LSE, the
backward's terms, and the packed-sequence and sampled-row entry points."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins


def _read(path):
    with open(path) as f:
        return f.read()


SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_scale": ("s_buf[j] = scale * dot;", "s_buf[j] = dot;"),
    "sum_without_max": ("l += exp(s_buf[j] - m);", "l += exp(s_buf[j]);"),
    "no_normalise": ("double p = exp(s_buf[j] - m) / l;", "double p = exp(s_buf[j] - m);"),
    "key_stride_d": ("const double *kj = k + j * stride;", "const double *kj = k + j * d;"),
    "values_from_keys": ("const double *vj = v + j * stride;", "const double *vj = k + j * stride;"),
    "causal_off_by_one": ("return last + 1;", "return last;"),
    "top_left_alignment": ("int64_t last = i + Nk - Nq;", "int64_t last = i;"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "empty_row_lse_zero": ("*lse = -INFINITY;", "*lse = 0.0;"),
    "key_head_offset_dropped": ("const double *kb = k + (b * Nk * Hkv + h / group) * d;",
                                "const double *kb = k + (b * Nk * Hkv) * d;"),
    "kv_head_modulo": ("const double *kb = k + (b * Nk * Hkv + h / group) * d;\n"
                       "                const double *vb = v + (b * Nk * Hkv + h / group) * d;",
                       "const double *kb = k + (b * Nk * Hkv + h % Hkv) * d;\n"
                       "                const double *vb = v + (b * Nk * Hkv + h % Hkv) * d;"),
    "kv_stride_query_heads": ("const int64_t stride = Hkv * d;     /* between consecutive keys */",
                              "const int64_t stride = H * d;     /* between consecutive keys */"),
    "bwd_dq_without_scale": ("dqi[c] += scale * ds * k[j * kstride + c];", "dqi[c] += ds * k[j * kstride + c];"),
    "bwd_no_row_term": ("const double ds = p_buf[j] * (dp_buf[j] - D);", "const double ds = p_buf[j] * dp_buf[j];"),
    "bwd_dv_from_ds": ("dv[j * kstride + c] += p_buf[j] * doi[c];", "dv[j * kstride + c] += ds * doi[c];"),
    "bwd_dk_from_dq_side": ("dk[j * kstride + c] += scale * ds * qi[c];", "dk[j * kstride + c] += scale * ds * doi[c];"),
    "bwd_kv_head_modulo": ("for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h)\n                    bwd_head(q + (b * Nq * H + h) * d",
                           "for (int64_t h = kvh; h < H; h += Hkv)\n                    bwd_head(q + (b * Nq * H + h) * d"),
    "bwd_rows_dk_from_dout": ("ok[c] += scale * ds * qi[c];", "ok[c] += scale * ds * doi[c];"),
    "bwd_rows_row_term_unweighted": ("D += exp(s_buf[j] - L) * dot;", "D += dot;"),
    "lse_wrong_slot": ("lse + (b * H + h) * Nq + i);", "lse + (h * B + b) * Nq + i);"),
    # packed sequences and the sampled-rows entry point
    "varlen_lse_token_major": ("lse + h * T + t);", "lse + t * H + h);"),
    "varlen_keys_from_token_zero": ("attention_row(q + (t * H + h) * d, k + (start * Hkv + h / group) * d,",
                                    "attention_row(q + (t * H + h) * d, k + (h / group) * d,"),
    "rows_packed_query_ignores_start": ("qi = q + ((start + i) * H + h) * d;", "qi = q + (i * H + h) * d;"),
    "rows_fixed_batch_dropped": ("                    qi = q + ((b * Nq + i) * H + h) * d;\n"
                                 "                    kb = k + (b * Nk * Hkv + h / group) * d;",
                                 "                    qi = q + (i * H + h) * d;\n"
                                 "                    kb = k + (b * Nk * Hkv + h / group) * d;"),
    "rows_alignment_from_nk": ("                    vb = v + (b * Nk * Hkv + h / group) * d;\n"
                               "                    nvalid = valid_keys(i, Nq, Nk, causal);",
                               "                    vb = v + (b * Nk * Hkv + h / group) * d;\n"
                               "                    nvalid = valid_keys(i, Nk, Nk, causal);"),
    "bwd_varlen_keys_from_token_zero": ("bwd_head(q + (start * H + h) * d, k + (start * Hkv + kvh) * d,",
                                        "bwd_head(q + (start * H + h) * d, k + (kvh) * d,"),
}


def _run_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as exc:  # a crash or NaN counts as caught
            failed.append((pin.__name__, type(exc).__name__))
    return failed


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # mutants may produce NaN or inf
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = _read(SRC)
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"liboracle_{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(path), "-lm"],
                   check=True)
    failed = _run_pins(oracle.Oracle(str(so)))
    assert failed, f"mutant {name} passed every pin"
