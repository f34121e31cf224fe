"""Pins of the generic flex-attention oracle (``oracle.flex_fwd``), CPU only.

Each check ties the oracle to something other than itself, following the page
"nemo_automodel.components.attention.flex_attention" (FlexAttention: the
"causal" / "block_causal" mask types, fixed_block_size, and forward's scale,
sink_weights and sliding_window):

* causal with no sink = ``torch.nn.functional.scaled_dot_product_attention``
  (float64, repeated K/V heads), with the default and with a given scale;
* block_causal = the blocks run as separate sequences and concatenated;
* fixed_block_size = the fixed chunks run as separate sequences;
* a window at least S long = no window;
* a per-head sink rescales the output by 1 / (1 + e^(s - lse)) and adds to lse;
* brute force on tiny inputs over a materialised mask built from the page's
  words by a different route (token scan), with an explicit sink column;
* allowed-key counts against closed forms.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_03_amd import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore")


def _f64(t):
    return t.to(torch.float64)


def _sdpa(q, k, v, scale=None):
    """Textbook causal attention in float64 (head-major layouts, K/V heads repeated)."""
    G = q.shape[1] // k.shape[1]
    kk = _f64(k).repeat_interleave(G, dim=1)
    vv = _f64(v).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(_f64(q), kk, vv, is_causal=True, scale=scale).numpy()


@pytest.mark.parametrize("G", [1, 4])
def test_causal_is_textbook_sdpa(G):
    x = W.flex_custom(2, 37, 4 * G, 4, 64, seed=11, sinks=False)
    out, lse, _ = oracle.flex_fwd(x["q"], x["k"], x["v"])
    np.testing.assert_allclose(out, _sdpa(x["q"], x["k"], x["v"]), atol=1e-12, rtol=0)


def test_given_scale_applies_without_sinks():
    x = W.flex_custom(1, 29, 4, 2, 64, seed=12, sinks=False)
    out, _, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], scale=0.3)
    np.testing.assert_allclose(out, _sdpa(x["q"], x["k"], x["v"], scale=0.3), atol=1e-12, rtol=0)


def test_scale_is_ignored_with_sinks():
    x = W.flex_custom(1, 23, 4, 2, 64, seed=13)
    a = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], scale=0.3)
    b = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"])
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_block_causal_is_separate_runs():
    x = W.flex_custom(1, 60, 4, 2, 64, mask="block_causal", doc_min=4, doc_max=15, seed=14)
    tok = x["tokens"]
    out, lse, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], tok, W.EOS_ID)
    ends = x["doc_ends"][0]
    starts = [0] + [e + 1 for e in ends]
    bounds = [(s, e) for s, e in zip(starts, [e + 1 for e in ends] + [60]) if e > s]
    assert len(bounds) >= 3
    for s, e in bounds:
        o, l, _ = oracle.flex_fwd(x["q"][:, :, s:e], x["k"][:, :, s:e], x["v"][:, :, s:e], x["sink_weights"])
        np.testing.assert_allclose(out[:, :, s:e], o, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[:, :, s:e], l, atol=1e-13, rtol=0)


def test_fixed_blocks_are_separate_runs():
    x = W.flex_custom(2, 50, 4, 1, 64, seed=15)
    F = 16
    out, lse, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], fixed_block_size=F)
    for s in range(0, 50, F):
        e = min(50, s + F)
        o, l, _ = oracle.flex_fwd(x["q"][:, :, s:e], x["k"][:, :, s:e], x["v"][:, :, s:e], x["sink_weights"])
        np.testing.assert_allclose(out[:, :, s:e], o, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[:, :, s:e], l, atol=1e-13, rtol=0)


def test_window_at_least_S_is_no_window():
    x = W.flex_custom(1, 33, 4, 2, 64, mask="block_causal", doc_min=5, doc_max=20, seed=16)
    a = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], x["tokens"], W.EOS_ID, sliding_window=33)
    b = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], x["tokens"], W.EOS_ID)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_per_head_sink_rescales():
    x = W.flex_custom(1, 31, 8, 2, 64, mask="block_causal", doc_min=4, doc_max=12, seed=17)
    o0, l0, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], None, x["tokens"], W.EOS_ID)
    o1, l1, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], x["tokens"], W.EOS_ID)
    s = x["sink_weights"].numpy().astype(np.float64)[None, :, None]
    np.testing.assert_allclose(o1, o0 / (1.0 + np.exp(s - l0))[..., None], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l1, np.logaddexp(l0, s), atol=1e-13, rtol=0)


def _brute(q, k, v, sink, tokens, eos, F, W_, scale):
    """Materialised scores with an explicit sink column; blocks from a token scan."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qd, kd, vd = _f64(q).numpy(), _f64(k).numpy(), _f64(v).numpy()
    out = np.zeros((B, Hq, S, D))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        block = np.zeros(S, dtype=np.int64)
        cur = 0
        for t in range(S):                 # EOS closes its block: the next token opens a new one
            block[t] = cur
            if tokens is not None and int(tokens[b, t]) == eos:
                cur += 1
        for h in range(Hq):
            for i in range(S):
                ok = [j for j in range(S) if j <= i and block[j] == block[i]
                      and (F <= 0 or i // F == j // F) and (W_ <= 0 or i - j < W_)]
                sc = scale if (sink is None and scale) else 1.0 / math.sqrt(D)
                z = [sc * float(qd[b, h, i] @ kd[b, h // G, j]) for j in ok]
                cols = z + ([float(sink[h])] if sink is not None else [])
                if not cols:
                    lse[b, h, i] = -math.inf
                    continue
                m = max(cols)
                w = np.exp(np.array(cols) - m)
                lse[b, h, i] = m + math.log(w.sum())
                for n, j in enumerate(ok):
                    out[b, h, i] += w[n] * vd[b, h // G, j]
                out[b, h, i] /= w.sum()
    return out, lse


@pytest.mark.parametrize("case", [
    dict(mask="block_causal", doc_min=2, doc_max=6, F=0, W=0, scale=None, sinks=True),
    dict(mask="block_causal", doc_min=3, doc_max=9, F=5, W=4, scale=None, sinks=True),
    dict(mask="causal", F=4, W=0, scale=0.7, sinks=False),
    dict(mask="causal", F=0, W=3, scale=None, sinks=True),
])
def test_bruteforce_agrees(case):
    kw = {k: case[k] for k in ("doc_min", "doc_max") if k in case}
    x = W.flex_custom(1, 19, 4, 2, 64, mask=case["mask"], seed=18, sinks=case["sinks"], **kw)
    sink = x["sink_weights"]
    out, lse, _ = oracle.flex_fwd(x["q"], x["k"], x["v"], sink, x["tokens"], W.EOS_ID, case["F"], case["W"],
                                  case["scale"])
    bo, bl = _brute(x["q"], x["k"], x["v"], None if sink is None else sink.numpy(), x["tokens"], W.EOS_ID,
                    case["F"], case["W"], case["scale"])
    np.testing.assert_allclose(out, bo, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, bl, atol=1e-12, rtol=0)


def test_counts_closed_form():
    """n_allowed = i - start(i) + 1 clipped by the window, start = max(block start, fixed start)."""
    S, F, Wn = 200, 48, 30
    x = W.flex_custom(2, S, 4, 2, 64, mask="block_causal", doc_min=7, doc_max=40, seed=19)
    _, _, cnt = oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], x["tokens"], W.EOS_ID, F, Wn)
    for b in range(2):
        ends = set(x["doc_ends"][b])
        start = 0
        for i in range(S):
            st = max(start, (i // F) * F, i - Wn + 1)
            assert cnt[b, i] == i - st + 1
            if i in ends:
                start = i + 1
