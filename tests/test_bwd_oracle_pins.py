"""Pins of the fp64 backward oracle (``oracle.attn_bwd``), CPU only.

The page "nemo_automodel.components.models.inkling2.flex_attention" makes the
per-query sinks differentiable and lets gradients reach the relative profiles
and flow in through the returned log-sum-exp.  The oracle's gradients are
hand-derived; each pin below ties them to something that is not that
derivation:

* torch autograd through a dense fp64 formulation (materialised scores, an
  explicit sink column, documents from a reset scan, bias gathered by fancy
  indexing) -- every gradient, every feature (catches a dropped term, a wrong
  sign, a transposed operand, a wrong GQA head or a wrong distance index);
* central finite differences with Richardson extrapolation of the *forward*
  oracle (already pinned on its own) at single entries of q, k, v, profiles
  and sink, moved by exactly representable steps;
* invariants: adding one constant to every logit and to the sink moves lse by
  that constant and leaves out unchanged, so the profile gradients of a row
  plus its sink gradient sum to dlse when every allowed key lies within the
  profile extent; the value gradients of a key/value head sum to the
  non-sink probability mass times dout; a row with no allowed key passes
  dlse to the sink and nothing elsewhere.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce
from transformer_attention_03_amd import workloads as W


def _upstream(x, seed, with_dlse=True):
    g = torch.Generator().manual_seed(seed)
    B, S, Hq, D = x["q"].shape
    dout = torch.randn(B, S, Hq, D, generator=g, dtype=torch.float64)
    dlse = torch.randn(B, S, Hq, generator=g, dtype=torch.float64) if with_dlse else None
    return dout, dlse


def _dense_autograd(x, dout, dlse):
    """fp64 forward with autograd; documents by reset scan, explicit sink column."""
    q = x["q"].to(torch.float64).requires_grad_()
    k = x["k"].to(torch.float64).requires_grad_()
    v = x["v"].to(torch.float64).requires_grad_()
    prof = x["profiles"].to(torch.float64).requires_grad_()
    sink = x["sink"].to(torch.float64).requires_grad_()
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    E = prof.shape[-1]
    G = Hq // Hkv
    pos = x["positions"].numpy().astype(np.int64)
    valid = x["valid"].numpy().astype(bool)
    doc = bruteforce.doc_ids_by_reset_scan(pos)
    window = x.get("window")
    ii, jj = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    outs, lses = [], []
    for b in range(B):
        m = (jj <= ii) & valid[b][:, None] & valid[b][None, :] & (doc[b][:, None] == doc[b][None, :])
        if window is not None and window > 0:
            m &= (ii - jj) < window
        rel = pos[b][:, None] - pos[b][None, :]
        inside = torch.from_numpy((rel >= 0) & (rel < E))
        relc = torch.from_numpy(np.clip(rel, 0, E - 1))
        mask = torch.from_numpy(m)
        kk = k[b].repeat_interleave(G, dim=1)                   # [S, Hq, D]
        vv = v[b].repeat_interleave(G, dim=1)
        content = torch.einsum("ihd,jhd->hij", q[b], kk) / np.sqrt(D)
        bias = torch.gather(prof[b], 2, relc.unsqueeze(0).expand(Hq, S, S))
        bias = torch.where(inside.unsqueeze(0), bias, torch.zeros((), dtype=torch.float64))
        scores = torch.where(mask.unsqueeze(0), content + bias, torch.tensor(-np.inf, dtype=torch.float64))
        full = torch.cat([sink[b].t().unsqueeze(-1), scores], dim=-1)      # [Hq, S, 1+S]
        lse = torch.logsumexp(full, dim=-1)                                 # [Hq, S]
        p = torch.exp(full - lse.unsqueeze(-1))[..., 1:]
        outs.append(torch.einsum("hij,jhd->ihd", p, vv))
        lses.append(lse.t())
    out = torch.stack(outs)
    lse = torch.stack(lses)
    loss = (out * dout).sum()
    if dlse is not None:
        loss = loss + (lse * dlse).sum()
    loss.backward()
    return [t.grad.numpy() for t in (q, k, v, prof, sink)]


def _bwd(x, dout, dlse):
    return oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                           positions=x["positions"], window=x.get("window"))


def small(seed, B=2, S=29, Hq=4, Hkv=2, D=8, E=6, window=None, structure="single", **kw):
    return W.custom(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, E=E, window=window, seed=seed, structure=structure, **kw)


CASES = [
    dict(seed=31),
    dict(seed=32, window=5),
    dict(seed=33, structure="tail_pad", max_tail_pad=7),
    dict(seed=34, structure="packed", doc_min=2, doc_max=9, invalid_tail=3),
    dict(seed=35, structure="packed", doc_min=3, doc_max=10, window=4, Hq=8, Hkv=1, E=3),
    dict(seed=36, E=40, Hq=3, Hkv=3, D=16),
    dict(seed=37, profiles_dtype=torch.bfloat16, sink_std=2.0),
    dict(seed=38, structure="packed", doc_min=1, doc_max=4, E=1, window=2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c['seed']}" for c in CASES])
@pytest.mark.parametrize("with_dlse", [True, False])
def test_autograd_agrees(case, with_dlse):
    x = small(**case)
    dout, dlse = _upstream(x, case["seed"] + 100, with_dlse)
    got = _bwd(x, dout, dlse)
    ref = _dense_autograd(x, dout, dlse)
    for name, a, r in zip(("dq", "dk", "dv", "dprofiles", "dsink"), got, ref):
        np.testing.assert_allclose(a, r, atol=1e-12, rtol=1e-10, err_msg=name)


def _loss(x, dout, dlse):
    out, lse, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"],
                                  positions=x["positions"], window=x.get("window"))
    return float((out * dout.numpy()).sum() + (lse * dlse.numpy()).sum())


def _fd(x, dout, dlse, name, idx, x0, h):
    """Richardson-extrapolated central difference at entry ``idx`` of input ``name``."""
    def at(val):
        y = dict(x)
        t = x[name].clone()
        t[idx] = val
        y[name] = t
        return _loss(y, dout, dlse)

    d1 = (at(x0 + h) - at(x0 - h)) / (2 * h)
    d2 = (at(x0 + 2 * h) - at(x0 - 2 * h)) / (4 * h)
    return (4 * d1 - d2) / 3


@pytest.mark.parametrize("name,idx,x0,h", [
    ("q", (1, 9, 3, 2), 0.5, 2.0 ** -6),
    ("q", (0, 20, 0, 7), -0.75, 2.0 ** -6),
    ("k", (1, 4, 1, 5), 0.25, 2.0 ** -6),
    ("v", (0, 11, 0, 0), 1.0, 2.0 ** -5),
    ("profiles", (1, 2, 14, 3), 0.25, 2.0 ** -8),
    ("profiles", (0, 3, 25, 0), -0.5, 2.0 ** -8),
    ("sink", (0, 17, 2), 0.125, 2.0 ** -8),
    ("sink", (1, 0, 1), -1.0, 2.0 ** -8),
])
def test_finite_differences_of_forward(name, idx, x0, h):
    x = small(41, window=9)
    dout, dlse = _upstream(x, 141)
    t = x[name].clone()
    t[idx] = x0                       # exact value: every step below is exact in the input dtype
    x[name] = t
    grads = dict(zip(("q", "k", "v", "profiles", "sink"), _bwd(x, dout, dlse)))
    fd = _fd(x, dout, dlse, name, idx, x0, h)
    assert abs(grads[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (grads[name][idx], fd)


def test_shift_invariance_profile_and_sink_grads_sum_to_dlse():
    """E >= S and one document: every allowed key has its distance inside the extent."""
    x = small(42, S=23, E=23)
    dout, dlse = _upstream(x, 142)
    _, _, _, dp, ds = _bwd(x, dout, dlse)
    total = dp.sum(axis=-1).transpose(0, 2, 1) + ds          # [B, S, Hq]
    np.testing.assert_allclose(total, dlse.numpy(), atol=1e-12, rtol=0)


def test_value_grads_sum_to_non_sink_mass():
    x = small(43, structure="packed", doc_min=3, doc_max=8, Hq=6, Hkv=2)
    dout, dlse = _upstream(x, 143)
    _, _, dv, _, _ = _bwd(x, dout, dlse)
    out, lse, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"],
                                  positions=x["positions"])
    mass = 1.0 - np.exp(x["sink"].numpy().astype(np.float64) - lse)      # [B, S, Hq]
    G = 3
    want = (mass[..., None] * dout.numpy()).reshape(2, 29, 2, G, 8).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, atol=1e-11, rtol=0)


def test_row_without_keys_feeds_only_the_sink():
    x = small(44, structure="tail_pad", max_tail_pad=0, invalid_tail=0)
    x["valid"][1, 10] = False                                # that query sees no key at all
    dout, dlse = _upstream(x, 144)
    dq, _, _, dp, ds = _bwd(x, dout, dlse)
    assert np.all(dq[1, 10] == 0) and np.all(dp[1, :, 10] == 0)
    np.testing.assert_array_equal(ds[1, 10], dlse.numpy()[1, 10])


def test_row_range_keeps_later_rows_and_keys():
    x = small(45, structure="packed", doc_min=3, doc_max=9)
    dout, dlse = _upstream(x, 145)
    full = _bwd(x, dout, dlse)
    part = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                           positions=x["positions"], row_lo=17)
    np.testing.assert_array_equal(part[0][:, 17:], full[0][:, 17:])
    np.testing.assert_array_equal(part[3][:, :, 17:], full[3][:, :, 17:])
    np.testing.assert_array_equal(part[4][:, 17:], full[4][:, 17:])
    np.testing.assert_allclose(part[1][:, 17:], full[1][:, 17:], atol=1e-14, rtol=0)
    np.testing.assert_allclose(part[2][:, 17:], full[2][:, 17:], atol=1e-14, rtol=0)
    assert np.all(part[0][:, :17] == 0)


def test_row_window_range_keeps_its_rows_and_keys():
    """Rows lo..hi-1 under a window w: their dq / dprofiles / dsink are the whole run's, and dk / dv
    of the keys j with lo <= j and j + w - 1 < hi (no row outside the range sees them) too."""
    w = 6
    x = small(47, window=w, structure="single")
    dout, dlse = _upstream(x, 147)
    full = _bwd(x, dout, dlse)
    lo, hi = 9, 27
    part = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                           positions=x["positions"], window=w, row_lo=lo, row_hi=hi)
    np.testing.assert_array_equal(part[0][:, lo:hi], full[0][:, lo:hi])
    np.testing.assert_array_equal(part[3][:, :, lo:hi], full[3][:, :, lo:hi])
    np.testing.assert_array_equal(part[4][:, lo:hi], full[4][:, lo:hi])
    kl, kh = lo, hi - w + 1
    np.testing.assert_allclose(part[1][:, kl:kh], full[1][:, kl:kh], atol=1e-14, rtol=0)
    np.testing.assert_allclose(part[2][:, kl:kh], full[2][:, kl:kh], atol=1e-14, rtol=0)
    # rows outside the range leave nothing, and keys seen from outside differ from the whole run
    assert np.all(part[0][:, :lo] == 0) and np.all(part[0][:, hi:] == 0)
    assert np.all(part[3][:, :, hi:] == 0) and np.all(part[4][:, :lo] == 0)
    assert not np.allclose(part[1][:, kh:hi], full[1][:, kh:hi])


def test_thread_count_does_not_change_the_gradients():
    x = small(48, structure="packed", doc_min=3, doc_max=9)
    dout, dlse = _upstream(x, 148)
    one = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                          positions=x["positions"], n_threads=1)
    many = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                           positions=x["positions"], n_threads=5)
    for a, b in zip(one, many):
        np.testing.assert_array_equal(a, b)


def test_magnitudes_bound_the_gradients():
    x = small(46, window=7)
    dout, dlse = _upstream(x, 146)
    g = _bwd(x, dout, dlse)
    m = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                        positions=x["positions"], window=7, magnitudes=True)
    for a, b in zip(g, m):
        assert np.all(np.abs(a) <= b * (1 + 1e-12) + 1e-300)
    # with dout >= 0 every dv contribution is non-negative: the magnitude is the value
    dpos = dout.abs()
    gv = _bwd(x, dpos, dlse)[2]
    mv = oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dpos, dlse,
                         positions=x["positions"], window=7, magnitudes=True)[2]
    np.testing.assert_allclose(gv, mv, rtol=1e-12, atol=0)
