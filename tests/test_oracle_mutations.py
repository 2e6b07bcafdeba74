"""The oracle pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index or
operand order, a wrong tie rule) in a copy of the oracle's C source, builds
it with gcc into a temporary directory, and runs the pin suite against it
in a subprocess.  The suite must fail for every mutant.  This runs on the
CPU only and never touches the GPU library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hhr_oracle.c")

MUTANTS = {
    "dropped_first_term": ("for (int d = 0; d < n; ++d) acc = fmaf", "for (int d = 1; d < n; ++d) acc = fmaf"),
    "bit_on_zero": ("if (y > 0.0f) code", "if (y >= 0.0f) code"),
    "msb_first_bits": ("(uint64_t)1 << (j % 64)", "(uint64_t)1 << (63 - j % 64)"),
    "transposed_rotation": ("xrot[r] = dot_canon(R + (int64_t)r * D, x, D)",
                            "{ float t_[512]; for (int c_ = 0; c_ < D; ++c_) t_[c_] = R[(int64_t)c_ * D + r]; "
                            "xrot[r] = dot_canon(t_, x, D); }"),
    "bound_min_not_max": ("U += a > c ? a : c;", "U += a < c ? a : c;"),
    "bound_always_kmax": ("U += a > c ? a : c;", "U += a;"),
    "group_min_not_max": ("(dm->page_group ? U < S : U > S)", "(dm->page_group ? U < S : U < S)"),
    "group_min_mode_is_max": ("(dm->page_group ? U < S : U > S)", "(dm->page_group ? U > S : U > S)"),
    "mean_query_first_head": ("for (int i = 0; i < G; ++i) acc += q[i * D + d];", "for (int i = 0; i < 1; ++i) acc += q[i * D + d];"),
    "page_ties_high_first": ("return (x->p > y->p) - (x->p < y->p);", "return (x->p < y->p) - (x->p > y->p);"),
    "hamming_and": ("__builtin_popcountll(cq[i * NW + w] ^ codes", "__builtin_popcountll(cq[i * NW + w] & codes"),
    "hamming_first_head_only": ("for (int i = 0; i < G; ++i)\n                            for (int w = 0; w < NW; ++w)",
                                "for (int i = 0; i < 1; ++i)\n                        for (int w = 0; w < NW; ++w)"),
    "key_ties_high_first": ("return (x->t > y->t) - (x->t < y->t);", "return (x->t < y->t) - (x->t > y->t);"),
    "scale_without_sqrt": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "meta_from_start_not_page_start": ("const int64_t lo = p * P,", "const int64_t lo = p * P < s ? s : p * P,"),
    "candidates_past_length": ("? L - dm->local_window : s_end;", "? T - dm->local_window : s_end;"),
    "keep_not_clamped_to_one": ("if (keep < 1) keep = 1;", ""),
    "topk_group_min_not_max": ("if (i == 0 || s > z) z = s;", "if (i == 0 || s < z) z = s;"),
    "topk_logit_from_value_rows": ("double s = 0.0;\n                    for (int d = 0; d < D; ++d) s += (double)q[i * D + d] * (double)elem(K",
                                   "double s = 0.0;\n                    for (int d = 0; d < D; ++d) s += (double)q[i * D + d] * (double)elem(V"),
    "topk_first_head_only": ("double z = 0.0;\n                for (int i = 0; i < G; ++i) {",
                             "double z = 0.0;\n                for (int i = 0; i < 1; ++i) {"),
    "forced_keys_compete": ("if (t >= L || t < s_end || t >= w_start) continue;", "if (t >= L) continue;"),
    "window_one_short": ("for (int64_t t = w_start; t < L; ++t) sel[", "for (int64_t t = w_start + 1; t < L; ++t) sel["),
    "value_from_key_rows": ("o[d] += wgt * (double)elem(V, row + d, bf);", "o[d] += wgt * (double)elem(K, row + d, bf);"),
    "mean_query_first_head_only": ("for (int i = 0; i < G; ++i) acc += q[i * D + d];",
                                   "for (int i = 0; i < 1; ++i) acc += q[i * D + d];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    sys.path.insert(0, ROOT)
    import oracle
    oracle.compile_source(str(mut), str(lib))
    env = dict(os.environ, HHR_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
