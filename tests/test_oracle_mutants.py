"""Planted mistakes in the oracle must each fail a pin (CPU only).

Each mutant is a copy of oracle/rmm_oracle.c with one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, a reversed tie rule,
an off-by-one bound ...).  It is compiled to a temporary library and the whole
pin battery of tests/pins.py is run against it in a child process (so a mutant
that crashes cannot take pytest down; a crash also counts as caught).  The test
passes when the battery fails.  The snippets must occur in the oracle source,
so the list breaks loudly if the oracle is edited.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rmm_oracle.c")

# (name, function the edit is made in, [(old, new), ...])
MUTANTS = [
    ("rownorm_no_sqrt", "void oracle_rownorms", [("b[k] = sqrt(s);", "b[k] = s;")]),
    ("colnorm_abs_not_square", "void oracle_colnorms", [("s += v * v;", "s += fabs(v);")]),
    ("colnorm_drops_last_row", "void oracle_colnorms", [("m < rows;", "m < rows - 1;")]),
    ("group_offset", "void oracle_scores", [("int64_t r0 = g * group_rows;", "int64_t r0 = g * group_rows + (g > 0);")]),
    ("ragged_group_rows", "void oracle_scores", [("M - r0 < group_rows ? M - r0 : group_rows", "group_rows - 1")]),
    ("activation_only_zero", "void oracle_scores", [("(b ? b[k] : 1.0)", "(b ? b[k] : 0.0)")]),
    ("score_sum_not_product", "void oracle_scores", [("a[k] * (b ? b[k] : 1.0)", "a[k] + (b ? b[k] : 1.0)")]),
    ("ties_to_higher_index", "static int by_rank", [("return (i > j) - (i < j);", "return (i < j) - (i > j);")]),
    ("keeps_smallest", "static int by_rank", [("if (si > sj)\n        return -1;\n    if (si < sj)\n        return 1;",
                                               "if (si < sj)\n        return -1;\n    if (si > sj)\n        return 1;")]),
    ("topk_unsorted_output", "int oracle_topk", [("qsort(idx, (size_t)kk, sizeof(int32_t), by_index);", "")]),
    ("kk_floor", "int64_t oracle_kk", [("kk = (int64_t)ceil(x);", "kk = (int64_t)floor(x);")]),
    ("kk_no_snap", "int64_t oracle_kk", [("if (fabs(x - n) <= 1e-9 * (double)K)", "if (0)")]),
    ("kk_no_floor_clamp", "int64_t oracle_kk", [("if (kk < 1)\n        kk = 1;", "")]),
    ("reduced_drops_last", "void oracle_reduced", [("j < kk;", "j < kk - 1;")]),
    ("reduced_sign", "void oracle_reduced", [("y[n] += a * brow[n];", "y[n] -= a * brow[n];")]),
    ("reduced_group0_only", "void oracle_reduced", [("idx + (m / group_rows) * ldidx", "idx")]),
    ("reduced_transposed_B", "void oracle_reduced", [("y[n] += a * brow[n];", "y[n] += a * B[(n % ldb) * ldb + (k % ldb)];")]),
    ("entries_wrong_row", "void oracle_reduced_entries", [("A[m * lda + k]", "A[(m / group_rows) * group_rows * lda + k]")]),
    ("bound_sums_kept", "double oracle_bound", [("if (!kept[k])", "if (kept[k])")]),
    ("thresh_is_max", "float oracle_thresh", [("if (s32[idx[j]] < t)", "if (s32[idx[j]] > t)")]),
    ("thresh_first_kept", "float oracle_thresh", [("j < kk; ++j)", "j < 1; ++j)")]),
    ("near_absolute_band", "int64_t oracle_near_ties", [("<= rel * fabs(t)", "<= rel")]),
    ("near_one_sided", "int64_t oracle_near_ties", [("fabs(s64[k] - t)", "(s64[k] - t)")]),
    ("near_band_around_max", "int64_t oracle_near_ties",
     [("if (s32[i] < s32[last] || (s32[i] == s32[last] && i > last))", "if (s32[i] > s32[last])")]),
    ("near_lowest_index_of_tie", "int64_t oracle_near_ties", [("&& i > last))", "&& i < last))")]),
    ("near_centred_on_key", "int64_t oracle_near_ties", [("double t = s64[last];", "double t = (double)s32[last];")]),
    ("pv_prefix_off_by_block", "int64_t oracle_pv_prefix", [("qblock * (g + 1)", "qblock * (g + 2)")]),
    ("pv_mass_drops_last_query", "void oracle_pv_scores", [("for (int64_t i = 0; i < nq; ++i)\n            mass", "for (int64_t i = 0; i < nq - 1; ++i)\n            mass")]),
    ("pv_score_without_vnorm", "void oracle_pv_scores", [("double s = mass * sqrt(vv);", "double s = mass;")]),
    ("pv_block_transposed_P", "void oracle_pv_block", [("double p = Ptb[k * ldp + i];", "double p = Ptb[(i % nq) * ldp + (k % nq)];")]),
    ("pv_bound_mass_not_l2", "double oracle_pv_bound", [("pp += p * p;", "pp += p;")]),
    ("q8_floor", "void oracle_quantize_q8", [("rintf(B[k * ldb + n] / s)", "floorf(B[k * ldb + n] / s)")]),
    ("q8_ties_away", "void oracle_quantize_q8", [("rintf(B[k * ldb + n] / s)", "roundf(B[k * ldb + n] / s)")]),
    ("q8_scale_sum", "void oracle_quantize_q8", [("if (a > amax)\n                amax = a;", "amax += a;")]),
    ("q8_scale_128", "void oracle_quantize_q8", [("amax / 127.0f", "amax / 128.0f")]),
    ("q8_dequant_row_scale", "void oracle_dequant_q8", [("(double)scale[n]", "(double)scale[k % N]")]),
    ("q8_rownorm_no_scale", "void oracle_rownorms_q8", [("(double)scale[n] * (double)q", "(double)q")]),
    ("qk_key_norm_from_queries", "void oracle_qk_scores", [("double v = K[k * D + j];", "double v = Q[k * D + j];")]),
    ("qk_query_norm_drops_last", "void oracle_qk_scores", [("i < nq; ++i)", "i < nq - 1; ++i)")]),
    ("qk_key_norm_no_sqrt", "void oracle_qk_scores", [("kn = sqrt(kq);", "kn = kq;")]),
    ("qk_activation_only_ignored", "void oracle_qk_scores", [("if (use_k) {", "if (1) {")]),
    ("qk_sum_not_product", "void oracle_qk_scores", [("double s = sqrt(qq) * kn;", "double s = sqrt(qq) + kn;")]),
    ("probs_no_scale", "void oracle_attn_probs", [("S[k] = dot / sqrt((double)D);", "S[k] = dot;")]),
    ("probs_scale_by_kept", "void oracle_attn_probs", [("S[k] = dot / sqrt((double)D);", "S[k] = dot / sqrt((double)nf);")]),
    ("probs_mask_excludes_diagonal", "void oracle_attn_probs", [("causal ? q + 1 : L", "causal ? (q > 0 ? q : 1) : L")]),
    ("probs_first_features", "void oracle_attn_probs", [("int64_t f = idx ? idx[j] : j;", "int64_t f = j;")]),
    ("probs_unnormalised", "void oracle_attn_probs", [("p[k] /= sum;", "p[k] /= 1.0;")]),
    ("probs_transposed_K", "void oracle_attn_probs", [("Q[q * D + f] * K[k * D + f]", "Q[q * D + f] * K[(f % L) * D + (k % D)]")]),
]


def _mutate(src, anchor, edits):
    start = src.index(anchor)
    end = src.find("\n}\n", start)
    body = src[start:end]
    for old, new in edits:
        assert body.count(old) >= 1, f"snippet not found in {anchor}: {old!r}"
        body = body.replace(old, new, 1)
    return src[:start] + body + src[end:]


CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle as O
import pins
lib = O.load({lib!r})
failed = []
for pin in pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:   # AssertionError or an error the mistake provokes
        failed.append(pin.__name__)
print("FAILED_PINS", failed)
sys.exit(1 if failed else 0)
"""


@pytest.mark.parametrize("name,anchor,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, anchor, edits, tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import build as obuild  # oracle/build.py
    src = open(SRC).read()
    mutated = _mutate(src, anchor, edits)
    assert mutated != src
    csrc = tmp_path / f"{name}.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / f"lib{name}.so")
    obuild.build(src=str(csrc), out=lib, extra=["-Wno-unused-variable", "-Wno-unused-parameter",
                                                "-Wno-unused-function", "-Wno-error"])
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    # caught = some pin failed (exit 1) or the mistake crashed the process
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout}\n{proc.stderr}"
