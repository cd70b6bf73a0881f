"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a plausible slip in ``oracle/oracle.c`` (a dropped term, a
wrong sign, a wrong index or stride, a transposed operand).  The copy is
compiled on the CPU into a temporary library and the pins of
``test_oracle.py``, ``test_oracle_append.py``, ``test_oracle_chunk.py`` and
``test_oracle_backward.py`` run against it in a child process (a mutant may read out of
bounds and crash, which also counts as caught).  The real oracle is never
modified.
"""

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("drop_scale", "scores[j] = scale * dot;", "scores[j] = dot;"),
    ("exp_sign", "double w = exp(scores[j] - m);", "double w = exp(m - scores[j]);"),
    ("lse_without_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("no_final_divide", "out[c] /= l;", "out[c] /= 1.0;"),
    ("max_reversed", "if (scores[j] > m)", "if (scores[j] < m && scores[j] > -INFINITY)"),
    ("causal_off_by_one", "(causal ? pos + 1 : len)", "(causal ? pos : len)"),
    ("causal_ignored", "(causal ? pos + 1 : len)", "(len)"),
    ("chunk_top_left", "int64_t pos = len - qlen + t;", "int64_t pos = t;"),
    ("chunk_query_rows", "n_keys = t < qlen ?", "n_keys = t < len ?"),
    ("gqa_interleaved", "int kvh = h / g;", "int kvh = h % Hkv;"),
    ("v_offset_dropped", "vrow[j] = (const uint16_t *)(pool + off + v_offset_bytes(&s));",
     "vrow[j] = (const uint16_t *)(pool + off);"),
    ("k_as_v_operand", "dot += qd[c] * bf16_to_double(krow[j][c]);",
     "dot += qd[c] * bf16_to_double(vrow[j][c]);"),
    ("layer_stride", "(int64_t)s->layer * s->mbps", "(int64_t)s->layer * s->n_layers"),
    ("slot_stride", "(int64_t)slot * s->n_layers * s->mbps", "(int64_t)slot * s->mbps"),
    ("token_in_page", "(p % ORACLE_PAGE_TOKENS) * row", "(p / ORACLE_PAGE_TOKENS) * row"),
    ("head_stride", "(int64_t)h * s->head_dim * 2;", "(int64_t)h * 2;"),
    ("decode_drops_newest", "ctx_lens[b] > 0 ? ctx_lens[b] : 0", "ctx_lens[b] > 0 ? ctx_lens[b] - 1 : 0"),
    ("v_offset_half", "return (int64_t)ORACLE_PAGE_TOKENS * s->n_kv_heads * s->head_dim * 2;",
     "return (int64_t)ORACLE_PAGE_TOKENS * s->n_kv_heads * s->head_dim;"),
    ("q_row_stride", "q + (((int64_t)b * T + t) * Hq + h) * d;", "q + (((int64_t)t * B + b) * Hq + h) * d;"),
    ("bf16_widen", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    # decode append: rounding, RoPE, allocation, release
    ("round_precision", "int qexp = (e > -125 ? e : -125) - 8;", "int qexp = (e > -125 ? e : -125) - 7;"),
    ("round_ties_away", "ldexp(nearbyint(ldexp(x, -qexp)), qexp)", "ldexp(round(ldexp(x, -qexp)), qexp)"),
    ("rope_sign", "y[i] = x1 * c - x2 * s;", "y[i] = x1 * c + x2 * s;"),
    ("rope_cos_sin_swapped", "double c = (double)cos_row[i], s = (double)sin_row[i];",
     "double c = (double)sin_row[i], s = (double)cos_row[i];"),
    ("rope_adjacent_pairs", "double x1 = bf16_to_double(x[i]), x2 = bf16_to_double(x[i + half]);",
     "double x1 = bf16_to_double(x[i]), x2 = bf16_to_double(x[(i + 1) % d]);"),
    ("rope_table_stride", "cos_t + (int64_t)pos * (d / 2)", "cos_t + (int64_t)pos * d"),
    ("pop_from_front", "page = free_pages[*top - 1];", "page = free_pages[0];"),
    ("alloc_when_unassigned", "if (pos % ORACLE_PAGE_TOKENS == 0) {", "if (*entry == -1) {"),
    ("append_v_rotated", "uint16_t vb = v[b * row_elems + (int64_t)h * d + c];",
     "uint16_t vb = double_to_bf16(y[c]);"),
    ("release_descending", "for (int blk = 0; blk < mbps; ++blk) {", "for (int blk = mbps - 1; blk >= 0; --blk) {"),
    ("release_keeps_entry", "                *entry = -1;\n", "\n"),
    # backward
    ("bwd_drop_D", "double ds = p * (dp[j] - D);", "double ds = p * dp[j];"),
    ("bwd_dq_no_scale", "dq[c] += scale * ds * kc;", "dq[c] += ds * kc;"),
    ("bwd_dv_uses_ds", "dV[kvo + c] += p * od[c];", "dV[kvo + c] += ds * od[c];"),
    ("bwd_dk_uses_p", "dK[kvo + c] += scale * ds * qd[c];", "dK[kvo + c] += scale * p * qd[c];"),
    ("bwd_causal_off_by_one", "int n = causal ? i + 1 : T;", "int n = causal ? i : T;"),
    ("bwd_dp_uses_k", "dv += od[c] * bf16_to_double(vr[c]);", "dv += od[c] * bf16_to_double(kr[c]);"),
    ("bwd_gqa_interleaved", "for (int h = kvh * g; h < (kvh + 1) * g; ++h) {",
     "for (int h = kvh; h < Hq; h += Hkv) {"),
]

RUNNER = textwrap.dedent("""
    import sys, traceback
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, test_oracle as T, test_oracle_append as A, test_oracle_chunk as C
    import test_oracle_backward as G
    import inspect
    failed = []
    pins = [
        (T.test_worked_example_matches_printed_numbers, {{}}),
        (T.test_worked_example_block_one_is_causal_row_one, {{}}),
        (T.test_stress_tied_row_is_uniform, {{}}),
        (T.test_zero_query_gives_causal_running_mean, {{}}),
        (T.test_zero_query_decode_is_context_mean, {{}}),
        (T.test_gqa_uses_consecutive_groups, {{}}),
        (T.test_prefill_matches_brute_force, dict(Hq=32, Hkv=8, causal=True)),
        (T.test_dense_matches_brute_force, dict(d=64, H=4, causal=True)),
        (T.test_decode_matches_brute_force, {{}}),
        (T.test_scatter_places_rows_at_page_addresses, dict(Hkv=8, d=64)),
        (T.test_page_geometry_matches_printed_constants, {{}}),
        (A.test_round_bf16_brute_force, {{}}),
        (A.test_round_bf16_matches_torch_on_fp32_values, {{}}),
        (A.test_rope_is_complex_rotation, dict(d=64)),
        (A.test_rope_special_angles, {{}}),
        (A.test_rope_relative_position, {{}}),
        (A.test_append_pop_order_by_hand, {{}}),
        (A.test_append_equals_rope_then_scatter, {{}}),
        (A.test_append_runs_out_of_pages, {{}}),
        (A.test_append_flags, {{}}),
        (A.test_release_push_order_by_hand, {{}}),
        (A.test_release_stack_full_and_bad_slot, {{}}),
        (A.test_append_release_round_trip, {{}}),
        (C.test_chunk_rows_equal_whole_prompt_rows, dict(causal=True)),
        (C.test_chunk_single_row_is_decode, {{}}),
        (C.test_chunk_zero_query_closed_form, {{}}),
        (C.test_chunk_matches_numpy_direct, dict(causal=True)),
        (G.test_backward_matches_autograd, dict(Hq=4, Hkv=1, d=64, causal=True)),
        (G.test_backward_matches_autograd, dict(Hq=8, Hkv=2, d=128, causal=False)),
        (G.test_backward_single_key, {{}}),
        (G.test_backward_zero_query_dv_closed_form, {{}}),
        (G.test_backward_key_gradients_sum_to_zero, dict(causal=True)),
    ]
    for fn, kw in pins:
        try:
            fn(oracle, **kw)
        except Exception:
            failed.append(fn.__name__)
    print("FAILED_PINS", len(failed), " ".join(failed))
""")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", str(mutant), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    script = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=300)
    if r.returncode != 0:        # crashed on a wild read: caught
        return
    line = [x for x in r.stdout.splitlines() if x.startswith("FAILED_PINS")][-1]
    assert int(line.split()[1]) > 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    """Control: the same runner on an unmodified copy reports no failing pin."""
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", SRC, "-o", str(lib),
                    "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    script = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    line = [x for x in r.stdout.splitlines() if x.startswith("FAILED_PINS")][-1]
    assert int(line.split()[1]) == 0, r.stdout
