"""Planted mistakes in the oracle, on the CPU: each pin must catch the mistake it names.

Every case copies ``oracle/attn_oracle.c``, replaces one statement by a
plausible mistake (a dropped or off-by-one mask term, an ignored offset, a
transposed or misplaced output write), builds the copy with gcc, points the
``oracle`` module at it and runs the pins that should fail.  The pins pass
on the real oracle in their own test files.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_mask_pins as MP
from tests import test_oracle_pins as OP
from tests import test_relproj_oracle_pins as RP

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# name -> (anchor the statement follows, statement, mistake, pins that must fail)
MUTANTS = {
    "causal test drops the query itself": (
        None, "if ((int64_t)j > gi) return 0;", "if ((int64_t)j >= gi) return 0;",
        [MP.test_mask_counts_closed_forms, MP.test_full_mask_equals_bruteforce_matrix_and_counts]),
    "window keeps one key more": (
        None, "!(p_i - k_j < window)", "!(p_i - k_j <= window)",
        [MP.test_mask_counts_closed_forms, MP.test_full_mask_equals_bruteforce_matrix_and_counts,
         MP.test_full_mask_of_query_slice_equals_bruteforce_rows]),
    "document test left out": (
        None, "if (gi - p_i != (int64_t)j - k_j) return 0;", ";",
        [MP.test_mask_counts_closed_forms, MP.test_full_mask_equals_bruteforce_matrix_and_counts,
         MP.test_full_mask_of_query_slice_equals_bruteforce_rows]),
    "key validity ignored": (
        None, "if (!key_valid[(size_t)b * Sk + j]) return 0;", ";",
        [MP.test_full_mask_equals_bruteforce_matrix_and_counts]),
    "query offset ignored": (
        None, "int64_t gi = query_offset + i;", "int64_t gi = i;",
        [MP.test_mask_query_slice_counts_are_rows_of_full_run, MP.test_full_mask_of_query_slice_equals_bruteforce_rows,
         OP.test_query_slice_with_offset_equals_rows_of_full_run]),
    "mask matrix written in reverse key order": (
        "int attn_oracle_mask(", "mask[(size_t)row * Sk + j] = (uint8_t)a;",
        "mask[(size_t)row * Sk + (Sk - 1 - j)] = (uint8_t)a;",
        [MP.test_full_mask_equals_bruteforce_matrix_and_counts, MP.test_full_mask_of_query_slice_equals_bruteforce_rows]),
    "flex row subset written to the neighbouring slot": (
        "int flex_oracle_fwd(", "double* o = out + ((size_t)t * Hq + h) * D;",
        "double* o = out + ((size_t)(rows ? (t + 1) % n_rows : t) * Hq + h) * D;",
        [MP.test_flex_rows_equal_rows_of_full_run]),
    "forward row subset written to the neighbouring slot": (
        "int attn_oracle_fwd(", "double* o = out + ((size_t)t * Hq + h) * D;",
        "double* o = out + ((size_t)(rows ? (t + 1) % n_rows : t) * Hq + h) * D;",
        [OP.test_row_subset_matches_full_run]),
    "distance taken key minus query": (
        "int attn_oracle_fwd(", "int64_t r = p_i - (int64_t)key_positions[(size_t)b * Sk + j];",
        "int64_t r = (int64_t)key_positions[(size_t)b * Sk + j] - p_i;",
        [OP.test_index_probe_decodes_key_exactly, functools.partial(OP.test_bruteforce_agrees, OP.CASES[3])]),
    "K/V head taken as h % Hkv": (
        "int attn_oracle_fwd(", "int g = h / G;", "int g = h % Hkv;",
        [OP.test_gqa_equals_repeated_kv_heads, OP.test_index_probe_decodes_key_exactly]),
    "sink left out of the denominator": (
        "int attn_oracle_fwd(", "double L = exp(sigma - M);", "double L = 0.0;",
        [OP.test_sink_rescales_output_and_adds_to_lse, functools.partial(OP.test_bruteforce_agrees, OP.CASES[0])]),
    "logit scale left out": (
        "int attn_oracle_fwd(", "z[j] = scale * dot + bias;", "z[j] = dot + bias;",
        [functools.partial(OP.test_reduces_to_causal_sdpa, 2), OP.test_first_token_of_each_document_closed_form]),
    "bias added beyond the extent as the last entry": (
        "int attn_oracle_fwd(", "if (r >= 0 && r < E)", "if (r >= 0 && (r = r < E ? r : E - 1) >= 0)",
        [functools.partial(OP.test_bruteforce_agrees, OP.CASES[0])]),
    "relative table read transposed": (
        "int attn_oracle_relproj_profiles(", "t[(size_t)r * d_rel + c]", "t[(size_t)c * E + r]",
        [RP.test_one_hot_table_reproduces_features]),
    "per-head table slice ignored": (
        "int attn_oracle_relproj_profiles(", "(table_heads == 1 ? 0 : h)", "(table_heads == 1 ? 0 : 0)",
        [RP.test_per_head_table_scales_by_head]),
    "features of head 0 for every head": (
        "int attn_oracle_relproj_profiles(", "(((size_t)b * Sq + i) * Hq + h) * (size_t)d_rel",
        "(((size_t)b * Sq + i) * Hq + 0) * (size_t)d_rel",
        [RP.test_one_hot_table_reproduces_features]),
}


def _mutant_source(anchor, stmt, mistake):
    src = open(SRC).read()
    start = src.index(anchor) if anchor else 0
    at = src.index(stmt, start)
    return src[:at] + mistake + src[at + len(stmt):]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    anchor, stmt, mistake, pins = MUTANTS[name]
    c = tmp_path / "mutant.c"
    c.write_text(_mutant_source(anchor, stmt, mistake))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so), str(c), "-lm"],
                   check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._configure(ctypes.CDLL(str(so))))
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
