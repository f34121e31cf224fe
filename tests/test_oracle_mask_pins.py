"""Pins of the oracle's mask helper and of the flex oracle's row-subset path.

``oracle.mask`` (allowed-key counts, and for small shapes the whole
visibility matrix) is the reference of the GPU count and tile checks; the
mask follows the forward's parameters ``valid``, ``key_valid``, ``positions``,
``key_positions`` and ``query_offset`` (page "nemo_automodel.components.models.
inkling2.flex_attention", Inkling2FlexAttention.forward) and the window of the
sliding-window mask mod (page "nemo_automodel.components.attention.
flex_attention").  It is pinned here against:

* closed forms of the counts: i + 1 (causal), min(i + 1, W) (window),
  i - start + 1 (packed documents), 0 at tokens that are not real, and the
  rows of the full run for a query slice with ``query_offset``;
* the independent brute-force matrix of ``tests/bruteforce.py`` (documents by
  reset scan, window on the column distance), element by element;
* the forward oracle's own per-row counts.

The flex oracle's ``rows=`` compaction is pinned against the rows of the full
run (bit for bit).  ``tests/test_oracle_mutants.py`` plants a mistake in each
path and checks that these pins catch it.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests import bruteforce
from transformer_attention_03_amd import workloads as W


def _x(seed, S=61, B=1, window=None, structure="single", **kw):
    return W.custom(B=B, S=S, Hq=2, Hkv=1, D=8, E=5, window=window, seed=seed, structure=structure, **kw)


def _doc_start(starts, i):
    return max(s for s in starts if s <= i)


def test_mask_counts_closed_forms():
    S = 61
    x = _x(41, S=S)
    assert np.array_equal(oracle.mask(x["valid"], positions=x["positions"])[0], np.arange(1, S + 1))
    for W_ in (1, 3, 16, S, S + 9):
        cnt = oracle.mask(x["valid"], positions=x["positions"], window=W_)
        assert np.array_equal(cnt[0], np.minimum(np.arange(1, S + 1), W_)), W_
    x = _x(42, S=S, B=2, structure="tail_pad", max_tail_pad=20)
    cnt = oracle.mask(x["valid"], positions=x["positions"])
    for b in range(2):
        nv = int(x["valid"][b].sum())
        expect = np.where(np.arange(S) < nv, np.arange(1, S + 1), 0)
        assert np.array_equal(cnt[b], expect)
    x = _x(43, S=S, structure="packed", doc_min=3, doc_max=14, invalid_tail=6)
    starts = x["doc_starts"][0]
    for W_ in (None, 4):
        cnt = oracle.mask(x["valid"], positions=x["positions"], window=W_)
        expect = np.array([i - _doc_start(starts, i) + 1 for i in range(S)])
        if W_:
            expect = np.minimum(expect, W_)
        expect[S - 6:] = 0
        assert np.array_equal(cnt[0], expect), W_


def test_mask_query_slice_counts_are_rows_of_full_run():
    S, a, n = 70, 23, 31
    x = _x(44, S=S, structure="packed", doc_min=4, doc_max=25, invalid_tail=3)
    full = oracle.mask(x["valid"], positions=x["positions"], window=9)
    sl = oracle.mask(x["valid"][:, a:a + n], key_valid=x["valid"], positions=x["positions"][:, a:a + n],
                     key_positions=x["positions"], window=9, query_offset=a)
    assert np.array_equal(sl, full[:, a:a + n])


def test_full_mask_equals_bruteforce_matrix_and_counts():
    cases = [dict(seed=45), dict(seed=46, window=5), dict(seed=47, structure="tail_pad", max_tail_pad=11, B=2),
             dict(seed=48, structure="packed", doc_min=1, doc_max=9, invalid_tail=4, window=3),
             dict(seed=49, structure="packed", doc_min=5, doc_max=30, B=2)]
    for c in cases:
        x = _x(S=57, **c)
        if c["seed"] == 49:
            # tokens that are not real between real ones (keys before real queries)
            x["valid"][:, 3::7] = False
        cnt, m = oracle.mask(x["valid"], positions=x["positions"], window=x["window"], full=True)
        ref = bruteforce.mask(x["valid"], x["positions"], x["window"])
        assert np.array_equal(m.astype(bool), ref), c
        assert np.array_equal(cnt, m.sum(axis=-1)), c


def test_full_mask_of_query_slice_equals_bruteforce_rows():
    S, a, n = 66, 17, 29
    x = _x(50, S=S, structure="packed", doc_min=3, doc_max=20, invalid_tail=2)
    ref = bruteforce.mask(x["valid"], x["positions"], 7)[:, a:a + n]
    cnt, m = oracle.mask(x["valid"][:, a:a + n], key_valid=x["valid"], positions=x["positions"][:, a:a + n],
                         key_positions=x["positions"], window=7, query_offset=a, full=True)
    assert np.array_equal(m.astype(bool), ref)
    assert np.array_equal(cnt, ref.sum(axis=-1))


def test_mask_counts_equal_forward_counts():
    for c in (dict(seed=51, window=6), dict(seed=52, structure="packed", doc_min=2, doc_max=12, invalid_tail=5)):
        x = _x(S=45, **c)
        _, _, fcnt = oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"],
                                     positions=x["positions"], window=x["window"])
        assert np.array_equal(oracle.mask(x["valid"], positions=x["positions"], window=x["window"]), fcnt)


def test_flex_rows_equal_rows_of_full_run():
    B, Hq, Hkv, S, D = 2, 4, 2, 53, 16
    g = torch.Generator().manual_seed(53)
    q = torch.randn(B, Hq, S, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, D, generator=g).to(torch.bfloat16)
    sw = torch.randn(Hq, generator=g)
    tokens = torch.randint(0, 6, (B, S), generator=g, dtype=torch.int32)
    for kw in (dict(sink_weights=sw, tokens=tokens, eos_id=0), dict(fixed_block_size=8, sliding_window=5),
               dict(tokens=tokens, eos_id=3, scale=0.3)):
        o, l, c = oracle.flex_fwd(q, k, v, **kw)
        rows = torch.tensor([0, 1, 17, 52, 53, 54, 99, 105], dtype=torch.int64)
        o1, l1, c1 = oracle.flex_fwd(q, k, v, rows=rows, **kw)
        r = rows.numpy()
        bb, ii = r // S, r % S
        assert np.array_equal(o1, o.transpose(0, 2, 1, 3)[bb, ii]), kw
        assert np.array_equal(l1, l.transpose(0, 2, 1)[bb, ii]), kw
        assert np.array_equal(c1, c[bb, ii]), kw
