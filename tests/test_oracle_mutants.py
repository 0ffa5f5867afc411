"""Plant plausible mistakes in copies of the oracle source and check that the
pins catch each one.  Runs on the CPU only; the real oracle is untouched."""

import pathlib
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "no_scale_on_beacon_scores": ("s[j] = p->scale * acc;", "s[j] = acc;"),
    "rope_sign_flipped": ("qr[i] = x1 * c - x2 * sn;\n      qr[i + half] = x2 * c + x1 * sn;",
                          "qr[i] = x1 * c + x2 * sn;\n      qr[i + half] = x2 * c - x1 * sn;"),
    "rope_adjacent_pairs": (
        "double x1 = widen(q, dt, q0 + i), x2 = widen(q, dt, q0 + i + half);\n"
        "      qr[i] = x1 * c - x2 * sn;\n      qr[i + half] = x2 * c + x1 * sn;",
        "double x1 = widen(q, dt, q0 + 2 * i), x2 = widen(q, dt, q0 + 2 * i + 1);\n"
        "      qr[2 * i] = x1 * c - x2 * sn;\n      qr[2 * i + 1] = x2 * c + x1 * sn;"),
    "rope_frequency_exponent": ("-2.0 * (double)i / (double)d", "-1.0 * (double)i / (double)d"),
    "u_k_transposed": ("widen(U_K, dt, uk0 + (size_t)i * rk + k)",
                       "widen(U_K, dt, uk0 + (size_t)k * d + i)"),
    "u_v_transposed": ("widen(U_V, dt, uv0 + (size_t)i * rv + k)",
                       "widen(U_V, dt, uv0 + (size_t)k * d + i)"),
    "beacon_only_normaliser": ("      l += s[j];", "      if (j < (size_t)nb || nb == 0) l += s[j];"),
    "gqa_strided_mapping": ("const int hq = h * G + g;", "const int hq = g * p->num_kv_heads + h;"),
    "lse_without_max": ("lse[(size_t)b * p->num_q_heads + hq] = m + log(l);",
                        "lse[(size_t)b * p->num_q_heads + hq] = log(l);"),
    "raw_value_row_shift": ("oraw[i] += s[nb + t] * widen(V_raw",
                            "oraw[i] += s[nb + (t + 1) % w] * widen(V_raw"),
    "raw_values_dropped": ("out[q0 + i] = acc + oraw[i];", "out[q0 + i] = acc;"),
    "no_scale_on_raw_scores": ("s[nb + t] = p->scale * acc;", "s[nb + t] = acc;"),
    "new_key_unrotated": ("ka[i] = narrow(x1 * c - x2 * sn, dt);\n      ka[i + half] = narrow(x2 * c + x1 * sn, dt);",
                          "ka[i] = narrow(x1, dt);\n      ka[i + half] = narrow(x2, dt);"),
    "new_key_one_position_back": ("double ang = (double)q_pos[b] * inv_freq;\n      double c = cos(ang), sn = sin(ang);\n      double x1 = widen(k_new",
                                  "double ang = (double)(q_pos[b] - 1) * inv_freq;\n      double c = cos(ang), sn = sin(ang);\n      double x1 = widen(k_new"),
    "new_value_dropped": ("oraw[i] += s[nb + w] * widen(v_new", "oraw[i] += 0.0 * widen(v_new"),
    "raw_rows_strided_by_live_length": ("const size_t kr0 = unit * (size_t)wcap * d;",
                                        "const size_t kr0 = unit * (size_t)w * d;"),
    "beacon_rows_not_clamped": ("nb = nb < 0 ? 0 : (nb > ncap ? ncap : nb);", "nb = nb < 0 ? 0 : nb;"),
    "bf16_rounding_truncates": ("nearbyint(ldexp(m, 8))", "trunc(ldexp(m, 8))"),
    "beacon_key_unrotated": ("acc += qr[i] * (kb[i] * c - kb[i + half] * sn) + qr[i + half] * (kb[i + half] * c + kb[i] * sn);",
                             "acc += qr[i] * kb[i] + qr[i + half] * kb[i + half];"),
    "beacon_key_rotated_backwards": ("acc += qr[i] * (kb[i] * c - kb[i + half] * sn) + qr[i + half] * (kb[i + half] * c + kb[i] * sn);",
                                     "acc += qr[i] * (kb[i] * c + kb[i + half] * sn) + qr[i + half] * (kb[i + half] * c - kb[i] * sn);"),
    "beacon_key_at_query_position": ("double ang = (double)bpos[j] * inv_freq;", "double ang = (double)q_pos[b] * inv_freq;"),
    "chunk_query_position_ignored": ("const double qpos = (double)q_pos[b] + (double)t;",
                                     "const double qpos = (double)q_pos[b];"),
    "chunk_keys_at_first_position": ("const double tpos = (double)q_pos[b] + (double)u;",
                                     "const double tpos = (double)q_pos[b];"),
    "chunk_future_tokens_visible": ("const int seen = app ? t + 1 : 0;",
                                    "const int seen = app ? ntok : 0;"),
    "chunk_token_excludes_itself": ("const int seen = app ? t + 1 : 0;",
                                    "const int seen = app ? t : 0;"),
    "chunk_values_of_first_token": ("const size_t v0 = (((size_t)b * ntok + u) * H + h) * d;",
                                    "const size_t v0 = (((size_t)b * ntok + 0) * H + h) * d;"),
    "chunk_rows_head_major": ("const size_t row = ((size_t)b * ntok + t) * Hq + hq;",
                              "const size_t row = ((size_t)b * Hq + hq) * ntok + t;"),
    "alibi_bias_sign_flipped": ("s[j] = p->scale * acc - m_h * (qp - (double)bpos[j]);",
                                "s[j] = p->scale * acc + m_h * (qp - (double)bpos[j]);"),
    "alibi_bias_scaled": ("s[nb + t] = p->scale * acc - m_h * (qp - kpos);",
                          "s[nb + t] = p->scale * (acc - m_h * (qp - kpos));"),
    "alibi_raw_position_off_by_one": ("const double kpos = qp - (double)w + 1.0 + (double)t;",
                                      "const double kpos = qp - (double)w + (double)t;"),
    "alibi_slope_of_kv_head": ("const double m_h = slope[hq];", "const double m_h = slope[h];"),
    "alibi_beacons_unbiased": ("s[j] = p->scale * acc - m_h * (qp - (double)bpos[j]);",
                               "s[j] = p->scale * acc;"),
    "fp32_storage_not_rounded": ("if (dtype == ORACLE_F32) return (double)(float)x;",
                                 "if (dtype == ORACLE_F32) return x;"),
    "fp32_storage_rounded_through_bf16": (
        "if (dtype == ORACLE_F32) return (double)(float)x;",
        "if (dtype == ORACLE_F32) dtype = ORACLE_BF16;"),
    "alibi_step_raw_rows_ignore_new_tokens": ("const double raw0 = qp0 - (double)w + (app ? 0.0 : 1.0);",
                                              "const double raw0 = qp0 - (double)w + 1.0;"),
    "alibi_step_token_one_position_late": ("m_h * (qpos - (qp0 + (double)u))",
                                           "m_h * (qpos - (qp0 + (double)u + 1.0))"),
    "alibi_step_query_position_fixed": ("    const double qpos = qp0 + (double)t;\n    const int seen",
                                        "    const double qpos = qp0;\n    const int seen"),
    "alibi_step_beacons_unbiased": ("sc[j] = p->scale * acc - m_h * (qpos - (double)bpos[j]);",
                                    "sc[j] = p->scale * acc;"),
    "alibi_step_token_value_of_first": ("vr[i] += sc[nb + w + u] * widen(v_new, dt, v0 + i);\n      }\n      for (int i = 0; i < d; ++i) {\n        double acc = 0.0;\n        for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * vl[k];\n        out[q0 + i] = acc + vr[i];\n      }\n      if (lse) lse[row] = mx + log(den);\n    }\n  }\n}\n\n/*\n * ALiBi counterpart",
                                        "vr[i] += sc[nb + w + u] * widen(v_new, dt, v0 - (size_t)u * H * d + i);\n      }\n      for (int i = 0; i < d; ++i) {\n        double acc = 0.0;\n        for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * vl[k];\n        out[q0 + i] = acc + vr[i];\n      }\n      if (lse) lse[row] = mx + log(den);\n    }\n  }\n}\n\n/*\n * ALiBi counterpart"),
    "empty_sequence_uniform": ("for (int i = 0; i < d; ++i) out[q0 + i] = 0.0;",
                               "for (int i = 0; i < d; ++i) out[q0 + i] = 1.0 / d;"),
}


_RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
from oracle_pins import ALL_PINS
failed = []
for pin in ALL_PINS:
    try:
        pin({lib!r})
    except (AssertionError, ValueError, FloatingPointError):
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path: pathlib.Path):
    src = oracle.SOURCE.read_text()
    old, new = MUTANTS[name]
    # an anchor that occurs more than once (the rotation of the query and of
    # a new token's key) is mutated everywhere
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(source=mutant_src, target=tmp_path / "libmutant.so")
    here = pathlib.Path(__file__).resolve().parent
    code = _RUNNER.format(root=str(here.parent), tests=str(here), lib=str(lib))
    # A mutant that dies on a signal (a planted index error) counts as caught;
    # any other non-zero exit is a broken harness and fails the test.
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    if res.returncode < 0:
        return
    assert res.returncode == 0, res.stderr[-3000:]
    line = [x for x in res.stdout.splitlines() if x.startswith("FAILED_PINS")][-1]
    assert line.split(" ", 1)[1].strip(), f"mutant {name} passed every pin"
