"""Each plausible slip in the oracle must be caught by at least one pin.

The oracle source is copied, one textual change is applied (a dropped term, a
wrong sign, a wrong operand or index, an off-by-one in a mask), the copy is
compiled with the oracle's own gcc flags into a temporary directory, and every
pin in oracle_pin_checks.py is run against it.  A mutant that passes every pin
means the pins leave that part of the oracle unchecked.  Only mutations that
keep every memory access in bounds are used.
"""
import os

import pytest

import oracle
from tests import oracle_pin_checks as pins

MUTANTS = {
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "exp_sign_flipped": ("p[j] = exp(s[j] - m);", "p[j] = exp(m - s[j]);"),
    "exp2_for_exp": ("p[j] = exp(s[j] - m);", "p[j] = exp2(s[j] - m);"),
    "no_normalisation": ("for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;", ""),
    "causal_strict": ("if (causal && pos + 1 < n_vis) n_vis = pos + 1 > 0 ? pos + 1 : 0;",
                      "if (causal && pos < n_vis) n_vis = pos > 0 ? pos : 0;"),
    "causal_ignored": ("if (causal && pos + 1 < n_vis) n_vis = pos + 1 > 0 ? pos + 1 : 0;", ""),
    "causal_top_left": ("int64_t pos = i + (Nk - Nq);", "int64_t pos = i;"),
    "causal_offset_sign": ("int64_t pos = i + (Nk - Nq);", "int64_t pos = i + (Nq - Nk);"),
    "kv_head_interleaved": ("int64_t hk = h / group;", "int64_t hk = h % Hkv;"),
    "query_head_from_kv_head": ("const float *q  = Q + ((b * H + h) * Nq + i) * d;",
                                "const float *q  = Q + ((b * H + hk) * Nq + i) * d;"),
    "key_len_ignored": ("L = key_len[b];", "L = Nk;"),
    "mask_ignored": ("if (mrow != NULL) s[j] += (double)mrow[j];", ""),
    "mask_scaled": ("if (mrow != NULL) s[j] += (double)mrow[j];",
                    "if (mrow != NULL) s[j] += scale * (double)mrow[j];"),
    "mask_sign": ("if (mrow != NULL) s[j] += (double)mrow[j];",
                  "if (mrow != NULL) s[j] -= (double)mrow[j];"),
    "mask_first_row_only": ("+ h * mask_sh + i * Nk;", "+ h * mask_sh + 0 * Nk;"),
    "mask_batch_ignored": ("mask + b * mask_sb + h * mask_sh", "mask + h * mask_sh"),
    "mask_head_ignored": ("mask + b * mask_sb + h * mask_sh", "mask + b * mask_sb"),
    "masked_row_not_empty": ("if (m == -INFINITY) {  /* every visible key masked out by -inf */",
                             "if (0) {"),
    "key_operand_for_query": ("dot += (double)q[c] * (double)kb[j * d + c];",
                              "dot += (double)kb[j * d + c] * (double)kb[j * d + c];"),
    "key_operand_for_value": ("o[c] += p[j] * (double)vb[j * d + c];",
                              "o[c] += p[j] * (double)kb[j * d + c];"),
    "weight_dropped": ("o[c] += p[j] * (double)vb[j * d + c];",
                       "o[c] += (double)vb[j * d + c];"),
    "lse_without_max": ("LSE[t] = m + log(l);", "LSE[t] = log(l);"),
    "lse_log2": ("LSE[t] = m + log(l);", "LSE[t] = m + log2(l);"),
    "min_for_max": ("if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    "dot_offset": ("double dot = 0.0;", "double dot = 1.0;"),
    "empty_row_lse_zero": ("if (n_vis == 0) {\n                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;\n                LSE[t] = -INFINITY;",
                           "if (n_vis == 0) {\n                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;\n                LSE[t] = 0.0;"),
    "value_row_skipped": ("for (int64_t j = 0; j < n_vis; ++j)\n                for (int64_t c = 0; c < d; ++c)\n                    o[c] +=",
                          "for (int64_t j = 1; j < n_vis; ++j)\n                for (int64_t c = 0; c < d; ++c)\n                    o[c] +="),
    "query_row_off_by_one": ("const float *q  = Q + ((b * H + h) * Nq + i) * d;",
                             "const float *q  = Q + ((b * H + h) * Nq + (i > 0 ? i - 1 : 0)) * d;"),
    # the output index t taken for the tensor row: equal only when the
    # selection lists every row in order
    "query_row_from_output_index": ("const float *q  = Q + ((b * H + h) * Nq + i) * d;",
                                    "const float *q  = Q + t * d;"),
    "causal_position_from_output_index": ("int64_t pos = i + (Nk - Nq);",
                                          "int64_t pos = (t % Nq) + (Nk - Nq);"),
    "mask_row_from_output_index": ("+ h * mask_sh + i * Nk;", "+ h * mask_sh + (t % Nq) * Nk;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    oracle.build(src=str(mutated), out=so)
    lib = oracle.load(so, build_if_missing=False)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passes every pin"
