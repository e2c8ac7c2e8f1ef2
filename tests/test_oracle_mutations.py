"""Planted mistakes in the oracle, on the CPU: every plausible slip must fail a pin.

Each case copies ``oracle/hfa_ref.cpp``, applies one textual mistake (a dropped
term, a wrong sign, a wrong index, a missing rescale), builds the copy into a
temporary library and runs the pins against it.  The case passes when at least
one pin rejects the mutated oracle.  Nothing here touches a GPU.
"""

import pytest

import oracle
from oracle.build import SOURCE, build
import oracle_checks as C

MUTATIONS = {
    "no_max_subtraction": ("S[j] = std::exp(S[j] - m);", "S[j] = std::exp(S[j]);"),
    "wrong_sign_exponent": ("S[j] = std::exp(S[j] - m);", "S[j] = std::exp(m - S[j]);"),
    "dropped_scale": ("S[j] = scale * dot;", "S[j] = dot;"),
    "no_normalisation": ("out[c] = num / l;", "out[c] = num;"),
    "lse_without_max": ("*lse_out = m + std::log(l);", "*lse_out = std::log(l);"),
    "value_column_index": ("num += S[j] * V[j * d + c];", "num += S[j] * V[j * d + (d - 1 - c)];"),
    "key_column_index": ("dot += qrow[c] * K[j * d + c];", "dot += qrow[c] * K[j * d + (d - 1 - c)];"),
    "dropped_first_term": ("    l += S[j];", "    if (j > 0) l += S[j];"),
    "online_no_denominator_rescale": ("l = l * alpha + tile_sum;", "l = l + tile_sum;"),
    "online_no_accumulator_rescale": ("for (int64_t c = 0; c < d; ++c) acc[c] *= alpha;", ""),
    "online_alpha_sign": ("std::exp(m_old - m_new);", "std::exp(m_new - m_old);"),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "sampled_row_index": ("(h * P.N + i) * P.d + c", "(h * P.N + r) * P.d + c"),
    "keys_as_queries": ("qrow[c] = widen(P.q,", "qrow[c] = widen(P.k,"),
    "softmax_no_max": ("y[j] = std::exp(static_cast<double>(x[j]) - m);", "y[j] = std::exp(static_cast<double>(x[j]));"),
    "softmax_no_normalisation": ("for (int64_t j = 0; j < C; ++j) y[j] /= l;", ""),
    "softmax_dropped_first_term": ("    l += y[j];", "    if (j > 0) l += y[j];"),
    "softmax_online_no_rescale": ("l = (l == 0.0 ? 0.0 : l * std::exp(m - m_new)) + cs;", "l = l + cs;"),
    "softmax_online_rescale_sign": ("l * std::exp(m - m_new)", "l * std::exp(m_new - m)"),
    "softmax_sampled_row_index": ("const float* row = x + (rows ? rows[i] : i) * C;\n      if (chunk == 0)",
                                  "const float* row = x + i * C;\n      if (chunk == 0)"),
    "rms_no_mean": ("std::sqrt(sq / static_cast<double>(C) + eps)", "std::sqrt(sq + eps)"),
    "rms_eps_outside_root": ("std::sqrt(sq / static_cast<double>(C) + eps)",
                             "(std::sqrt(sq / static_cast<double>(C)) + eps)"),
    "rms_no_root": ("std::sqrt(sq / static_cast<double>(C) + eps)", "(sq / static_cast<double>(C) + eps)"),
    "rms_abs_not_square": ("sq += s[j] * s[j];", "sq += std::fabs(s[j]);"),
    "rms_dropped_first_square": ("sq += s[j] * s[j];", "if (j > 0) sq += s[j] * s[j];"),
    "rms_weight_reversed": ("s[j] / denom * widen(w, dtype, j)", "s[j] / denom * widen(w, dtype, C - 1 - j)"),
    "rms_residual_dropped": ("const float sum = a + b;", "const float sum = a;"),
    "rms_residual_sign": ("const float sum = a + b;", "const float sum = a - b;"),
    "rms_residual_in_fp64": ("const float sum = a + b;\n  return static_cast<double>(sum);",
                             "return static_cast<double>(a) + static_cast<double>(b);"),
    "rms_sampled_row_index": ("rmsnorm_row(x, r, w, dtype, rows ? rows[i] : i,", "rmsnorm_row(x, r, w, dtype, i,"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    text = SOURCE.read_text()
    assert text.count(before) == 1, f"mutation anchor for {name} not unique in the oracle source"
    src = tmp_path / "hfa_ref_mut.cpp"
    src.write_text(text.replace(before, after))
    lib = build(src=src, out=tmp_path / "libhfa_ref_mut.so")
    orc = oracle.OracleLib(lib)
    failed = []
    for check in C.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(getattr(check, "__name__", "check"))
    assert failed, f"no pin rejects the planted mistake {name}"
