"""Helpers shared by the GPU parity tests: device copies, the HIP call, oracle comparison.

Acceptance bar (fixed for the forward): masks and indexing exact; output
max-abs error <= 2e-3; lse max-abs error <= 1e-3 over finite entries, with -inf
exactly where the oracle has -inf; rows without an allowed key have out == 0.
"""
from __future__ import annotations

import math
import sys
from typing import Optional

import numpy as np
import torch

import oracle
from transformer_attention_03_amd import binding

OUT_ATOL = 2e-3
LSE_ATOL = 1e-3

TENSORS = ("q", "k", "v", "profiles", "sink", "valid", "key_valid", "positions", "key_positions")


def announce(msg: str) -> None:
    """Name the case on stderr, unbuffered, before a GPU step runs."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def to_device(x: dict, device: str = "cuda") -> dict:
    return {k: (x[k].to(device) if isinstance(x.get(k), torch.Tensor) else None) for k in TENSORS}


def run_hip(x: dict, d: Optional[dict] = None, **kw):
    """Forward through the C-ABI on the GPU; returns host (out, lse) as float64 numpy."""
    d = d if d is not None else to_device(x)
    args = dict(window=x.get("window"), query_offset=x.get("query_offset", 0))
    args.update(kw)
    out, lse = binding.attn_fwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"],
                                d["key_valid"], d["positions"], d["key_positions"], **args)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def run_oracle(x: dict, rows=None, **kw):
    args = dict(key_valid=x.get("key_valid"), positions=x.get("positions"),
                key_positions=x.get("key_positions"), window=x.get("window"),
                query_offset=x.get("query_offset", 0), rows=rows)
    args.update(kw)
    return oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], **args)


def assert_close(out, lse, ref_out, ref_lse, ref_cnt, what: str):
    """The acceptance bar, element by element (arrays of equal shape)."""
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape, what
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref_out)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= OUT_ATOL, \
        f"{what}: out max-abs {err.max():.3e} at {worst} (gpu {out[worst]:.6f} ref {ref_out[worst]:.6f})"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(ninf, np.isneginf(lse)), f"{what}: -inf pattern of lse differs"
    assert not np.any(np.isnan(lse)), f"{what}: NaN in lse"
    fin = ~ninf
    if fin.any():
        lerr = np.abs(lse[fin] - ref_lse[fin])
        assert lerr.max() <= LSE_ATOL, f"{what}: lse max-abs {lerr.max():.3e}"
    empty = (ref_cnt == 0)
    if empty.any():
        assert np.all(out[empty] == 0.0), f"{what}: rows without keys must be exactly 0"


def check_full(x: dict, what: str, **kw):
    """Whole-output comparison (small shapes)."""
    announce(f"{what}: attn_fwd full compare, shape q={tuple(x['q'].shape)} E={x['profiles'].shape[-1]} "
             f"window={kw.get('window', x.get('window'))}")
    out, lse = run_hip(x, **kw)
    ref_out, ref_lse, ref_cnt = run_oracle(x, **kw)
    assert_close(out, lse, ref_out, ref_lse, ref_cnt, what)
    return out, lse, ref_cnt


def check_rows(x: dict, rows: torch.Tensor, what: str, d: Optional[dict] = None):
    """Compare sampled rows (flattened b*Sq + i) of a full-size run with the oracle."""
    announce(f"{what}: attn_fwd sampled rows ({rows.numel()}), shape q={tuple(x['q'].shape)}")
    out, lse = run_hip(x, d=d)
    B, Sq, Hq, D = x["q"].shape
    ref_out, ref_lse, ref_cnt = run_oracle(x, rows=rows)
    r = rows.numpy()
    assert_close(out.reshape(B * Sq, Hq, D)[r], lse.reshape(B * Sq, Hq)[r], ref_out, ref_lse,
                 np.repeat(ref_cnt[:, None], Hq, axis=1), what)
    return out, lse


def count_probe_inputs(x: dict) -> dict:
    """q = k = 0, profiles = 0, sink = -inf: every allowed key weighs 1, so lse = ln(n_allowed)."""
    y = dict(x)
    y["q"] = torch.zeros_like(x["q"])
    y["k"] = torch.zeros_like(x["k"])
    y["profiles"] = torch.zeros_like(x["profiles"])
    y["sink"] = torch.full_like(x["sink"], -math.inf)
    return y


def counts_from_lse(lse: np.ndarray) -> np.ndarray:
    """Decode n_allowed from a count-probe lse (exact for n below 2^24)."""
    with np.errstate(over="ignore"):
        n = np.where(np.isneginf(lse), 0.0, np.exp(lse))
    return np.rint(n).astype(np.int64)
