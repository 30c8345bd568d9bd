"""Strength of the oracle's pins: plant plausible mistakes in copies of the
oracle's C source (built on the CPU with gcc into a temporary directory) and
require that at least one pin fails for every planted mistake."""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_commit as commit_pins
from tests import test_oracle_dfs as dfs_pins
from tests import test_oracle_pins as pins
from tests import test_oracle_tree as tree_pins

# (description, exact text in tree_attn_oracle.c, replacement).  Mutants run in
# this process, so none may remove a bounds check (an out-of-bounds write
# would corrupt the test process itself).
MUTANTS = [
    ("node does not see itself",
     "for (int32_t j = i; j != -1; j = J->parent[off + j]) {\n        if (j < 0",
     "for (int32_t j = J->parent[off + i]; j != -1; j = J->parent[off + j]) {\n        if (j < 0"),
    ("siblings and other branches leak in",
     "for (int32_t j = i; j != -1; j = J->parent[off + j]) {\n        if (j < 0",
     "for (int32_t j = i; j != -1; j = (j > 0 ? j - 1 : -1)) {\n        if (j < 0"),
    ("wrong GQA head map", "int32_t c = h / G;", "int32_t c = h % J->Hkv;"),
    ("first prefix token dropped", "for (int32_t t = 0; t < L; ++t) {", "for (int32_t t = 1; t < L; ++t) {"),
    ("wrong slot inside a page", "int64_t slot = (int64_t)page * J->page_size + t % J->page_size;",
     "int64_t slot = (int64_t)page * J->page_size + (t + 1) % J->page_size;"),
    ("LSE in base 2", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("prefix scores unscaled", "score[n] = J->scale * dot(qrow, krow, D);\n        vrow[n] = J->v_cache",
     "score[n] = dot(qrow, krow, D);\n        vrow[n] = J->v_cache"),
    ("tree value of the wrong node", "vrow[n] = J->v_tree + ((int64_t)(off + j) * J->Hkv + c) * D;",
     "vrow[n] = J->v_tree + ((int64_t)(off + i) * J->Hkv + c) * D;"),
    ("max not subtracted in the weights", "double w = exp(score[k] - m) / l;", "double w = exp(score[k]) / l;"),
    ("position id off by one", "pos_id[off + i] = prefix_len[b] + d - 1;", "pos_id[off + i] = prefix_len[b] + d;"),
    ("mask bit shifted", "|= (uint64_t)1 << (j % 64);", "|= (uint64_t)1 << ((j + 1) % 64);"),
    ("status index not one-based", "status[b] = first_bad + 1;\n            continue;\n        }\n        for (int32_t i = 0; i < T; ++i) {\n            int32_t d = 0;",
     "status[b] = first_bad;\n            continue;\n        }\n        for (int32_t i = 0; i < T; ++i) {\n            int32_t d = 0;"),
    ("dfs: status index not one-based", "status[b] = first_bad + 1;\n            continue;\n        }\n        /* Depth-first walk.",
     "status[b] = first_bad;\n            continue;\n        }\n        /* Depth-first walk."),
    ("q row of the wrong head", "const double *qrow = J->q + ((int64_t)node * J->Hq + h) * D;",
     "const double *qrow = J->q + ((int64_t)node * J->Hq + (h + 1) % J->Hq) * D;"),
    ("commit: path written leaf first", "const int32_t node = path[depth - d];", "const int32_t node = path[d - 1];"),
    ("commit: position off by one", "const int64_t t = (int64_t)L + d - 1;\n            const int32_t page",
     "const int64_t t = (int64_t)L + d;\n            const int32_t page"),
    ("commit: accepted node itself left out", "path[depth++] = i;\n            i = p;",
     "if (i != a) path[depth++] = i;\n            i = p;"),
    ("commit: V not copied", "memcpy((char *)v_cache + dst_row * row_bytes", "if (0) memcpy((char *)v_cache + dst_row * row_bytes"),
    ("commit: new length not advanced", "new_prefix_len[b] = L + depth;", "new_prefix_len[b] = L;"),
    ("tree: ties go to the later push", "return a->push < b->push;", "return a->push > b->push;"),
    ("tree: child score drops the parent's", "volatile float s = c.score + lp[(int64_t)c.depth * K + k];",
     "volatile float s = lp[(int64_t)c.depth * K + k];"),
    ("tree: child uses the parent's depth logits", "volatile float s = c.score + lp[(int64_t)c.depth * K + k];",
     "volatile float s = c.score + lp[(int64_t)(c.depth - 1) * K + k];"),
    ("tree: depth limit off by one", "if (c.depth < Dmax) {", "if (c.depth < Dmax - 1) {"),
    ("tree: push numbers per parent collide", "cand_t ch = {s, (int64_t)K + (int64_t)K * i + k, i, c.depth + 1, k};",
     "cand_t ch = {s, (int64_t)K + k, i, c.depth + 1, k};"),
    ("commit: missing page reported as a bad accepted node", "status[b] = ORACLE_COMMIT_BAD_PAGE;",
     "status[b] = ORACLE_COMMIT_BAD_ACCEPTED;"),
    ("dfs: children taken in decreasing index", "for (int32_t c = T - 1; c > v; --c)\n                if (parent[off + c] == v)",
     "for (int32_t c = v + 1; c < T; ++c)\n                if (parent[off + c] == v)"),
    ("dfs: roots taken in decreasing index", "for (int32_t i = T - 1; i >= 0; --i)\n            if (parent[off + i] == -1)",
     "for (int32_t i = 0; i < T; ++i)\n            if (parent[off + i] == -1)"),
    ("dfs: parents left in the old labelling", "parent_new[inv[off + i]] = (p == -1) ? -1 : inv[off + p] - off;",
     "parent_new[inv[off + i]] = p;"),
    ("dfs: breadth-first instead of depth-first", "int32_t v = stack[--top];",
     "int32_t v = stack[0]; for (int32_t q = 1; q < top; ++q) stack[q - 1] = stack[q]; --top;"),
]

PIN_CALLS = [
    pins.test_plan_hand_fixture,
    lambda: pins.test_plan_chain_closed_form(65),
    pins.test_plan_recurrence_and_popcount,
    pins.test_plan_error_statuses,
    pins.test_attn_hand_fixture,
    lambda: pins.test_chain_equals_causal_sdpa(45, 16, 16),
    lambda: pins.test_path_as_flat_sequence(2, 4),
    pins.test_zero_keys_closed_form,
    pins.test_one_visible_key,
    pins.test_non_ancestors_do_not_leak,
    commit_pins.test_chain_commits_nodes_in_order,
    lambda: commit_pins.test_rows_are_the_accepted_nodes_ancestors_by_depth(__import__("torch").bfloat16, 16),
    commit_pins.test_nothing_accepted_changes_nothing,
    commit_pins.test_two_commits_equal_one_flat_append,
    commit_pins.test_error_statuses_write_nothing_for_that_request,
    lambda: tree_pins.test_equal_candidates_give_breadth_first_order(3, 12),
    lambda: tree_pins.test_equal_candidates_give_breadth_first_order(8, 100),
    tree_pins.test_dominant_candidate_gives_a_chain,
    lambda: tree_pins.test_top_t_by_brute_force(0),
    tree_pins.test_structure_invariants,
    lambda: dfs_pins.test_permutation_is_the_lexicographic_order_of_paths(0),
    dfs_pins.test_hand_written_preorder,
    lambda: dfs_pins.test_bad_trees_report_the_plan_status([-1, 0, 2, 1], 3),
    lambda: dfs_pins.test_relabelled_tree_is_topological_with_contiguous_subtrees(1),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new, tmp_path, monkeypatch):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site not unique/present: {desc}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-w", "-o", str(so),
                           str(mpath), "-lm", "-lpthread"])
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(so)))
    caught = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {desc}"
