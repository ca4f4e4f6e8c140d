"""Plant plausible mistakes in copies of the oracle's C source and check
that the pins catch every one.  The planted copies are built in a temporary
directory and used only inside this test; the oracle itself is untouched."""
import os

import pytest

import oracle
from tests import pin_battery as B

SRC = os.path.join(os.path.dirname(oracle.__file__), "frn_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("drop_eps", "float v = ms + eps;", "float v = ms;"),
    ("mean_over_H_minus_1", "(float)(ss / (double)H)", "(float)(ss / (double)(H - 1))"),
    ("one_plus_gamma", "float o = n * gamma[i];", "float o = n * (1.0f + gamma[i]);"),
    ("drop_residual", "h[i] = s[i] + oracle_bf16_to_f32(x[i]);", "h[i] = s[i];"),
    ("gamma2_in_first_norm", "a[i] = n * g1[i];", "a[i] = n * g2[i];"),
    ("sandwich_second_norm_gamma1", "float o = n * g2[i];", "float o = n * g1[i];"),
    ("skip_last_rank", "for (int32_t r = 1; r < R; ++r)", "for (int32_t r = 1; r < R - 1; ++r)"),
    ("drop_shared_expert", "if (shared_row) acc = acc + oracle_bf16_to_f32(shared_row[i]);", ""),
    ("finalize_sign", "acc = acc + prod;", "acc = acc - prod;"),
    ("finalize_weight_index", "float prod = w[j] * e;", "float prod = w[k - 1 - j] * e;"),
    ("finalize_fma", "float prod = w[j] * e;\n            acc = acc + prod;",
     "acc = fmaf(w[j], e, acc);"),
    ("sandwich_fma", "float n = s[i] * r1;\n        a[i] = n * g1[i];\n        h[i] = a[i] + oracle_bf16_to_f32(x[i]);",
     "float n = s[i] * r1;\n        a[i] = n * g1[i];\n        h[i] = fmaf(n, g1[i], oracle_bf16_to_f32(x[i]));"),
    ("sqrt_not_inverse", "return 1.0f / d;", "return d;"),
    ("no_rsqrt_root", "float d = sqrtf(v);", "float d = v;"),
    ("bf16_truncate", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))", "if (0)"),
    ("bf16_ties_away", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))",
     "if (lower >= 0x8000u)"),
    ("second_norm_reads_bf16_h", "        xout[i] = oracle_f32_to_bf16(h[i]);\n    }\n    float r = oracle_inv_rms",
     "        xout[i] = oracle_f32_to_bf16(h[i]);\n        h[i] = oracle_bf16_to_f32(xout[i]);\n    }\n    float r = oracle_inv_rms"),
    ("split_skips_rounding", "for (int64_t i = 0; i < H; ++i) u[i] = oracle_f32_to_bf16(s[i]);",
     "for (int64_t i = 0; i < H; ++i) u[i] = oracle_f32_to_bf16(s[i]);\n            if (J->epilogue != ORACLE_EPI_NONE) goto no_split;"),
    ("fp32_sum_of_squares", "double ss = 0.0;", "float ss = 0.0f;"),
    ("invalid_index_clamped", "e = NAN;", "e = 0.0f;"),
    # expert-parallel finalize
    ("ep_foreign_slot_reads_nan", "if (idx[j] < 0) continue; /* another rank's expert */",
     "if (idx[j] < 0) { acc = acc + (float)NAN; continue; }"),
    ("ep_foreign_slot_reads_row0", "if (idx[j] < 0) continue; /* another rank's expert */",
     "if (idx[j] < 0) { if (num_rows > 0) acc = acc + w[j] * oracle_bf16_to_f32(rows[i]); continue; }"),
    ("ep_rank0_indices", "J->idx_r[r] + t * J->k", "J->idx_r[0] + t * J->k"),
    ("ep_rank0_row_count", "finalize_row_ep(J->src[r], J->num_rows_r[r],",
     "finalize_row_ep(J->src[r], J->num_rows_r[0],"),
    ("ep_shared_on_every_rank", "J->shared && J->shared[r] ? J->shared[r] + t * H : NULL",
     "J->shared && J->shared[0] ? J->shared[0] + t * H : NULL"),
    ("ep_drop_shared", "if (shared_row != NULL) acc = acc + oracle_bf16_to_f32(shared_row[i]);", ""),
    ("ep_weight_index", "float term = w[j] * e;", "float term = w[k - 1 - j] * e;"),
    ("ep_fma", "float term = w[j] * e;\n            acc = acc + term;", "acc = fmaf(w[j], e, acc);"),
    ("ep_shared_first", "float acc = 0.0f;\n        for (int32_t j = 0; j < k; ++j) {\n            if (idx[j] < 0) continue;",
     "float acc = shared_row != NULL ? oracle_bf16_to_f32(shared_row[i]) : 0.0f;\n        shared_row = NULL;\n        for (int32_t j = 0; j < k; ++j) {\n            if (idx[j] < 0) continue;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    text = source.replace(old, new)
    if name == "split_skips_rounding":
        # jump past the R=1 restart so the epilogue runs on the FP32 sum
        text = text.replace("            const bf16_t* one[1] = {u};\n            reduce_row(one, 1, H, s);",
                            "            const bf16_t* one[1] = {u};\n            reduce_row(one, 1, H, s);\n        }\n        if (0) {\n        no_split:;")
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text)
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle.compile_source(str(src), so, werror=False)
    with oracle.use_library(so):
        fails = B.all_pins(quick=False)
    assert fails, f"planted mistake '{name}' passed every pin"
