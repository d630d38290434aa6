"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant is a one-line textual change to a copy of `oracle/hils_oracle.c`,
built on the host; the pins of `test_oracle_pins.py` then run against it.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_backward as bwd
import test_oracle_bsa as bsa
import test_oracle_pins as pins
import test_oracle_qcal as qc

SRC = os.path.join(os.path.dirname(oracle.__file__), "hils_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("drop entropy bias in score", "scale * acc + bsum[((int64_t)b * Hq + h) * ks_NC + c]",
     "scale * acc + 0.0 * bsum[((int64_t)b * Hq + h) * ks_NC + c]"),
    ("entropy sign", "round_to(L - ps, ORND_F32)", "round_to(ps - L, ORND_F32)"),
    ("mean key instead of weighted", "acc += p[j] * ld(k, k_dt, koff + (int64_t)j * d + e);",
     "acc += ld(k, k_dt, koff + (int64_t)j * d + e) / S;"),
    ("tie to higher index", "return (x->c < y->c) ? -1 : (x->c > y->c);",
     "return (x->c > y->c) ? -1 : (x->c < y->c);"),
    ("window off by one", "(int64_t)S * floor_div(i - (int64_t)W + 1, S)",
     "(int64_t)S * floor_div(i - (int64_t)W, S)"),
    ("q_hat in token logits", "for (int e = 0; e < d; ++e) qv[e] = ld(q, q_dt, qo + e);",
     "for (int e = 0; e < d; ++e) qv[e] = ld(qh, q_dt, qo + e);"),
    ("window left out of normaliser", "const double Lhat = lse(ws, nsel + 1);",
     "const double Lhat = nsel ? lse(ws, nsel) : logZw;"),
    ("GQA without per-head normalisation", "const double x = sh[hh * nc + c] - L[hh];",
     "const double x = sh[hh * nc + c];"),
    ("GQA sum instead of max", "if (x > r) r = x;", "r = (r == -INFINITY ? 0.0 : r) + x;"),
    ("scale missing in summary", "            s[j] = scale * acc;\n        }\n        const double L",
     "            s[j] = acc;\n        }\n        const double L"),
    ("scale missing in token logits", "        s[j] = scale * acc;\n    }\n    const double logZ",
     "        s[j] = acc;\n    }\n    const double logZ"),
    ("fused weight uses window mass for chunks", "const double w = exp(ws[sidx] - Lhat);",
     "const double w = exp(logZw - Lhat);"),
    ("forced selection ignored", "sel[s] = forced_idx[t * topk + s];", "sel[s] = 0;"),
    ("forced selection shifted", "sel[s] = forced_idx[t * topk + s];",
     "sel[s] = forced_idx[t * topk + s] > 0 ? forced_idx[t * topk + s] - 1 : 0;"),
    ("backward: window gradient drops dlse", "const double dsj = aj * (gvj - Dd + gl);",
     "const double dsj = aj * (gvj - Dd);"),
    ("backward: chunk logits centred on D", "const double dsj = wc * pj * (gvj - Dc);",
     "const double dsj = wc * pj * (gvj - Dd);"),
    ("backward: s_hat gradient drops dlse", "const double dsh = wc * (Dc - Dd + gl);",
     "const double dsh = wc * (Dc - Dd);"),
    ("backward: entropy term sign", "ej[j] = acc - dbc * sj[j];", "ej[j] = acc + dbc * sj[j];"),
    ("backward: k' path to the keys missing", "dk[kvb + (c * S + j) * d + e] += pp[j] * dkc[e] + scale * dsj",
     "dk[kvb + (c * S + j) * d + e] += 0.0 * dkc[e] + scale * dsj"),
    ("BSA: chunk mass misses its last token", "lz[hh * nc + c] = lse(s, S);",
     "lz[hh * nc + c] = lse(s, S - 1);"),
    ("BSA: mean logit instead of log-mass", "lz[hh * nc + c] = lse(s, S);",
     "lz[hh * nc + c] = lse(s, S) - log((double)S);"),
    ("BSA: GQA without per-head normalisation", "best = fmax(best, lz[hh * nc + c] - L[hh]);",
     "best = fmax(best, lz[hh * nc + c]);"),
    ("Q-Cal: residual query dropped", "out[o] = round_to(ld(q, dt, o) + acc, round_mode);",
     "out[o] = round_to(acc, round_mode);"),
    ("Q-Cal: down-projection transposed",
     "acc += ld(w_down, dt, (int64_t)j * dm + m) * ld(h, dt, bt * dm + m);",
     "acc += ld(w_down, dt, (int64_t)m * r + j) * ld(h, dt, bt * dm + m);"),
    ("Q-Cal: up-projection of head 0 for every head",
     "acc += ld(w_up, dt, ((int64_t)hd * d + e) * r + j) * z[j];",
     "acc += ld(w_up, dt, ((int64_t)0 * d + e) * r + j) * z[j];"),
    ("Q-Cal: rounding skipped", "out[o] = round_to(ld(q, dt, o) + acc, round_mode);",
     "out[o] = ld(q, dt, o) + acc;"),
    ("BSA: logits of the next chunk", "const int64_t off = kvb + (c * S + j) * d;",
     "const int64_t off = kvb + ((c + 1) * S + j) * d;"),
]

PIN_TESTS = [
    lambda g: pins.test_golden_hand_example(g),
    lambda g: pins.test_golden_gqa_rule(g),
    lambda g: pins.test_window_and_candidates(),
    lambda g: pins.test_p1_taylor_exact_at_landmark(),
    lambda g: pins.test_p1_through_rows(),
    lambda g: pins.test_p7_mean_pool_special_case(),
    lambda g: pins.test_p8_entropy_regimes(),
    lambda g: pins.test_p3_fused_weights_sum_to_one(),
    lambda g: pins.test_p4_chunk_size_one_is_dense(3),
    lambda g: pins.test_p5_single_query_exact_any_chunk_size(),
    lambda g: pins.test_p6_short_prefix_and_window_only(),
    lambda g: pins.test_p9_brute_force_matrix_form(dict(B=1, Hq=4, Hkv=2, T=28, d=6, S=4, W=6, k=1)),
    lambda g: pins.test_p9_brute_force_matrix_form(dict(B=1, Hq=1, Hkv=1, T=32, d=4, S=2, W=4, k=3)),
    lambda g: pins.test_psel_exact_ties_lower_index_wins(1, 1),
    lambda g: pins.test_p11_gqa_identical_heads_equals_mha(),
    lambda g: pins.test_golden_forced_selection(g),
    lambda g: pins.test_forced_own_selection_is_identical(4, 2),
    lambda g: bwd.test_backward_matches_finite_differences(2),
    lambda g: bwd.test_backward_chunk_size_one_is_dense_attention_backward(),
    lambda g: bwd.test_backward_values_of_ones(),
    lambda g: bsa.test_bsa_matches_numpy_route(1),
    lambda g: bsa.test_bsa_matches_numpy_route(2),
    lambda g: bsa.test_bsa_chunk_size_one_is_top_logits(),
    lambda g: bsa.test_bsa_identical_keys_per_chunk(),
    lambda g: bsa.test_hils_equals_bsa_at_the_landmark_query(4),
    lambda g: qc.test_zero_up_projection_or_hidden_state_is_identity(),
    lambda g: qc.test_rank_one_one_hot_closed_form(),
    lambda g: qc.test_correction_is_linear_in_h(),
    lambda g: qc.test_stored_query_rounds_to_nearest_even(),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, mut, tmp_path, golden):
    src = open(SRC).read()
    assert src.count(orig) == 1, "mutation anchor not found: " + name
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(orig, mut))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-std=c11", "-shared", "-fPIC", str(mpath),
                           "-o", str(so), "-lm"])
    oracle.use_library(str(so))
    caught = []
    try:
        for k, t in enumerate(PIN_TESTS):
            try:
                t(golden)
            except (AssertionError, RuntimeError):
                caught.append(k)
    finally:
        oracle.use_library(None)
    assert caught, "planted mistake '%s' passed every pin" % name
