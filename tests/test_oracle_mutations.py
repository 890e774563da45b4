"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of lsh_oracle.c (on the CPU,
in a temporary directory), builds it, and checks that at least one pin fails.
"""
import pytest

import oracle

import test_oracle_backward as bpins
import test_oracle_ffn as fpins
import test_oracle_pins as pins
import test_oracle_variants as vpins

# (name, original text, planted mistake); a list replaces several places at once.
# Every planted mistake keeps all memory accesses in bounds.
MUTATIONS = [
    ("scale dropped", "logit[n] = dot * scale;", "logit[n] = dot;"),
    ("R transposed", "Rr[t * half + k]", "Rr[k * d + t]"),
    ("negated half dropped", "z[k + half] = -p;", "z[k + half] = p;"),
    ("ties to highest index", "if (z[k] > z[best]) best = k;", "if (z[k] >= z[best]) best = k;"),
    ("margin not a difference", "margin[out_idx] = z[best] - second;",
     "margin[out_idx] = z[best];"),
    ("no look-back", "const int64_t first = (chunk > 0 ? chunk - 1 : chunk) * m;",
     "const int64_t first = chunk * m;"),
    ("look-ahead instead of look-back",
     "const int64_t first = (chunk > 0 ? chunk - 1 : chunk) * m;\n  int64_t last = (chunk + 1) * m;",
     "const int64_t first = chunk * m;\n"
     "  int64_t last = (chunk + 2) * m < c->seq_len ? (chunk + 2) * m : c->seq_len;"),
    ("keys not normalised", "khat[t] = (nrm > 0.0) ? k[t] / nrm : 0.0;", "khat[t] = k[t];"),
    ("causal reversed", "if (c->causal && j > i) continue;", "if (c->causal && j < i) continue;"),
    ("self not masked", "if (j == i) continue;", "if (0) continue;"),
    ("self-only lse zero", "return LSH_ORACLE_SELF_LOGIT;", "return 0.0;"),
    ("lse without max", "const double lse = mx + log(sum);", "const double lse = log(sum);"),
    ("rounds averaged", "const double w = exp(lse_r0[r * lse_stride] - mx) / sum;",
     "const double w = 1.0 / (double)R;"),
    ("unstable sort", "for (int64_t i = 0; i < L; ++i) pm[start[bk[i]]++] = (int32_t)i;",
     "for (int64_t i = L - 1; i >= 0; --i) pm[start[bk[i]]++] = (int32_t)i;"),
    ("buckets in descending order",
     ["start[bk[i] + 1] += 1;", "pm[start[bk[i]]++] = (int32_t)i;"],
     ["start[nb - bk[i]] += 1;", "pm[start[nb - 1 - bk[i]]++] = (int32_t)i;"]),
    # backward
    ("bwd: logsumexp term dropped", "const double ds = pj[a] * (dp[a] - dsum) + pj[a] * dlse;",
     "const double ds = pj[a] * (dp[a] - dsum);"),
    ("bwd: key normalisation Jacobian dropped",
     "dqk[(bh * L + j) * d + u] += (dk[u] - (k[u] / nrm) * proj) / nrm;",
     "dqk[(bh * L + j) * d + u] += dk[u] / nrm;"),
    ("bwd: self-only value gradient dropped",
     "for (int64_t u = 0; u < d; ++u) dv[(bh * L + i) * d + u] += dor[u];",
     "for (int64_t u = 0; u < d; ++u) dv[(bh * L + i) * d + u] += 0.0 * dor[u];"),
    ("bwd: round weight missing", "dor[u] = w * drow[u];", "dor[u] = drow[u];"),
    ("bwd: logsumexp gradient against the round row only",
     "g += (orow[u] - outrow[u]) * drow[u];", "g += orow[u] * drow[u];"),
    ("bwd: key gradient from the key instead of the query",
     "dkhat[(bh * L + j) * d + u] += ds * q[u] * scale;",
     "dkhat[(bh * L + j) * d + u] += ds * khat[u] * scale;"),
    ("bwd: unit-query gradient outside the normalisation Jacobian",
     "double* dqi = nq ? dkhat + (bh * L + i) * d : dqk + (bh * L + i) * d;",
     "double* dqi = dqk + (bh * L + i) * d;"),
    ("bwd: key gradient from the raw query with unit queries",
     "          const double* q = nq ? qhat : qk_bh + i * d;\n          const double scale",
     "          const double* q = qk_bh + i * d;\n          const double scale"),
    ("bwd: dedup count ignored",
     "              logit[a] -= log((double)rounds_sharing(c, inv + bh * R * L,\n"
     "                                                     buckets",
     "              logit[a] -= 0.0 * log((double)rounds_sharing(c, inv + bh * R * L,\n"
     "                                                     buckets"),
    # variants
    ("look-ahead chunk missing", "&& last < L) last += m;", "&& last < L) last += 0;"),
    ("same-bucket mask against itself", "bk[j] != bk[i]) continue;", "bk[j] != bk[j]) continue;"),
    ("queries not normalised", "unit_key(q, d, qhat);\n    q = qhat;", "unit_key(q, d, qhat);"),
    ("dedup count ignored",
     "logit[a] -= log((double)rounds_sharing(c, inv_bh, bk_bh, i, key[a]));",
     "logit[a] -= 0.0 * log((double)rounds_sharing(c, inv_bh, bk_bh, i, key[a]));"),
    ("union not de-duplicated", "if (stamp[key[a]] == mark) continue;", "if (0) continue;"),
    ("shared rounds without the look-ahead chunk", "in = in || cj == ci + 1;", "in = in;"),
    # projections
    ("value weights for the keys", "sq += xr[k] * wq[k];", "sq += xr[k] * wv[k];"),
    ("head offset of the weights dropped",
     "const double* wq = w_qk + (h * d + e) * model_dim;",
     "const double* wq = w_qk + e * model_dim;"),
    # chunked feed-forward
    ("ffn: ReLU dropped", "h[r * d_ff + j] = s > 0.0 ? s : 0.0;", "h[r * d_ff + j] = s;"),
    ("ffn: ReLU as absolute value", "h[r * d_ff + j] = s > 0.0 ? s : 0.0;",
     "h[r * d_ff + j] = s > 0.0 ? s : -s;"),
    ("ffn: first bias dropped", "s += b1[j];", "s += 0.0 * b1[j];"),
    ("ffn: second bias dropped", "s += b2[e];", "s += 0.0 * b2[e];"),
    ("ffn: second weight transposed", "for (int64_t j = 0; j < d_ff; ++j) s += hr[j] * we[j];",
     "for (int64_t j = 0; j < d_ff; ++j) s += hr[j] * w2[j * d_model + e];"),
    ("ffn: chunk offset dropped from the input", "const double* yr = y1 + (c0 + r) * d_model;",
     "const double* yr = y1 + r * d_model;"),
    ("ffn: residual dropped", "if (x2) s += x2[(c0 + r) * d_model + e];",
     "if (0) s += x2[(c0 + r) * d_model + e];"),
]


def _pin_calls():
    o = oracle
    return [
        lambda: pins.test_hash_hand_worked_examples(o),
        lambda: pins.test_hash_signed_permutation_closed_form(o),
        lambda: pins.test_hash_rescale_invariance(o),
        lambda: pins.test_hash_antipodal(o),
        lambda: pins.test_sort_is_the_stable_bucket_order(o, 4, False),
        lambda: pins.test_sort_is_the_stable_bucket_order(o, 64, True),
        lambda: pins.test_windows_hand_enumerated(o, False),
        lambda: pins.test_windows_hand_enumerated(o, True),
        lambda: pins.test_single_chunk_equals_full_attention(o, 1, 1, True),
        lambda: pins.test_single_chunk_equals_full_attention(o, 8, 3, False),
        lambda: pins.test_dense_mask_and_multiset_union(o, True),
        lambda: pins.test_identical_rounds_collapse(o),
        lambda: pins.test_self_only_rows_return_their_value(o),
        lambda: bpins.test_backward_matches_finite_differences(o, False),
        lambda: bpins.test_backward_matches_finite_differences(o, True),
        lambda: bpins.test_backward_single_chunk_equals_dense_autograd(o, 3, True),
        lambda: bpins.test_variant_backward_matches_finite_differences(o, bpins.NQ, False),
        lambda: bpins.test_variant_backward_matches_finite_differences(o, bpins.DD, True),
        lambda: bpins.test_variant_backward_matches_finite_differences(
            o, bpins.LA | bpins.SB | bpins.NQ | bpins.DD, True),
        lambda: bpins.test_unit_query_backward_single_chunk_equals_dense_autograd(o, True),
        lambda: bpins.test_dedup_backward_of_identical_rounds_equals_one_round(o),
        lambda: vpins.test_variant_equals_dense_definition(o, vpins.LA, True),
        lambda: vpins.test_variant_equals_dense_definition(o, vpins.SB, False),
        lambda: vpins.test_variant_equals_dense_definition(o, vpins.NQ, False),
        lambda: vpins.test_variant_equals_dense_definition(o, vpins.DD, True),
        lambda: vpins.test_variant_equals_dense_definition(o, vpins.LA | vpins.DD, False),
        lambda: vpins.test_look_ahead_over_two_chunks_is_full_attention(o),
        lambda: vpins.test_dedup_with_identical_rounds_is_one_round(o),
        lambda: pins.test_projection_equals_library_matmul(o),
        lambda: pins.test_projection_with_selection_weights_copies_the_input(o),
        lambda: fpins.test_ffn_split_identity_returns_the_input(o),
        lambda: fpins.test_ffn_half_of_the_split_is_the_positive_part(o),
        lambda: fpins.test_ffn_biases_through_selection_weights(o),
        lambda: fpins.test_ffn_residual_is_added(o),
        lambda: fpins.test_ffn_chunking_changes_nothing(o, 3),
    ]


@pytest.mark.parametrize("name,orig,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, bad):
    src = oracle.source_text()
    origs = orig if isinstance(orig, list) else [orig]
    bads = bad if isinstance(bad, list) else [bad]
    for o, b in zip(origs, bads):
        assert src.count(o) == 1, f"mutation anchor not found once: {o!r}"
        src = src.replace(o, b)
    lib = oracle.compile_source(src, str(tmp_path / "liblsh_oracle_mut.so"))
    oracle.use_library(lib)
    failures = 0
    try:
        for call in _pin_calls():
            try:
                call()
            except (AssertionError, ValueError, IndexError):
                failures += 1
    finally:
        oracle.use_library(None)
    assert failures > 0, f"no pin caught: {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = oracle.compile_source(oracle.source_text(), str(tmp_path / "liblsh_oracle_copy.so"))
    oracle.use_library(lib)
    try:
        for call in _pin_calls():
            call()
    finally:
        oracle.use_library(None)
