"""Materialised fp64 brute force for tiny shapes (tests only).

An independent formulation of the forward used to pin the C oracle:

* the score matrix is built whole, ``[Sq, 1 + Sk]`` per (batch, head), with an
  explicit sink column in front and a zero value row for it;
* documents are found by a reset scan of the positions (a document starts
  where the position is 0 or does not continue the previous token's position),
  not by the oracle's start-column comparison;
* the window is applied to the column distance ``i - j``;
* the relative bias is gathered with numpy fancy indexing;
* the softmax is numpy's ``exp`` / ``sum`` over the whole row.

Only queries and keys that are the same tokens (``Sk == Sq``, no offset) are
supported, which is all the brute-force pins need.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def doc_ids_by_reset_scan(positions: np.ndarray) -> np.ndarray:
    """Document index per token: a new document begins where positions restart."""
    B, S = positions.shape
    ids = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        cur = 0
        for i in range(S):
            if i > 0 and not (positions[b, i] == positions[b, i - 1] + 1):
                cur += 1
            ids[b, i] = cur
    return ids


def forward(q, k, v, profiles, sink, valid, positions, window=None):
    q, k, v = _f64(q), _f64(k), _f64(v)
    prof, sink = _f64(profiles), _f64(sink)
    valid = valid.cpu().numpy().astype(bool)
    pos = positions.cpu().numpy().astype(np.int64)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    E = prof.shape[-1]
    G = Hq // Hkv
    doc = doc_ids_by_reset_scan(pos)
    out = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, S, Hq))
    ii, jj = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    for b in range(B):
        mask = (jj <= ii) & valid[b][:, None] & valid[b][None, :] & (doc[b][:, None] == doc[b][None, :])
        if window is not None and window > 0:
            mask &= (ii - jj) < window
        rel = pos[b][:, None] - pos[b][None, :]
        inside = (rel >= 0) & (rel < E)
        for h in range(Hq):
            g = h // G
            content = (q[b, :, h, :] @ k[b, :, g, :].T) / np.sqrt(D)
            bias = np.where(inside, prof[b, h][ii, np.clip(rel, 0, E - 1)], 0.0)
            scores = np.where(mask, content + bias, -np.inf)
            full = np.concatenate([sink[b, :, h][:, None], scores], axis=1)  # sink column first
            vals = np.concatenate([np.zeros((1, D)), v[b, :, g, :]], axis=0)  # zero value for sink
            m = np.max(full, axis=1, keepdims=True)
            m_safe = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(full - m_safe)
            den = e.sum(axis=1, keepdims=True)
            with np.errstate(invalid="ignore", divide="ignore"):
                o = (e @ vals) / den
                l = (m_safe + np.log(den))[:, 0]
            o = np.where(den > 0, o, 0.0)
            out[b, :, h, :] = o
            lse[b, :, h] = l
    return out, lse


def mask(valid, positions, window=None):
    """Whole visibility matrix ``[B, S, S]`` (bool) of queries and keys that are the
    same tokens: both real, key not after the query, same document by reset scan,
    column distance below the window."""
    valid = valid.cpu().numpy().astype(bool)
    pos = positions.cpu().numpy().astype(np.int64)
    B, S = valid.shape
    doc = doc_ids_by_reset_scan(pos)
    ii, jj = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    out = np.zeros((B, S, S), dtype=bool)
    for b in range(B):
        m = (jj <= ii) & valid[b][:, None] & valid[b][None, :] & (doc[b][:, None] == doc[b][None, :])
        if window is not None and window > 0:
            m &= (ii - jj) < window
        out[b] = m
    return out
