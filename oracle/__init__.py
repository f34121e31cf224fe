"""fp64 CPU oracle of the learned-relative GQA attention forward (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its Python
binding) never does, and this package imports nothing from the product path.

The arithmetic lives in ``attn_oracle.c`` (plain sequential fp64 loops, OpenMP
over query rows only).  This wrapper applies the defaults of the forward's
optional arguments, as the page "nemo_automodel.components.models.inkling2.
flex_attention" (Inkling2FlexAttention.forward, parameters key_valid,
positions, key_positions) describes them, read as follows:

* ``key_valid`` defaults to ``valid`` (single context-parallel rank);
* ``positions`` defaults to the global column ``query_offset + i`` (one
  document);
* ``key_positions`` defaults to ``positions`` when keys and queries are the same
  tokens (``Sk == Sq`` and ``query_offset == 0``), otherwise to the key column.

Parity is pinned by the tests in ``tests/test_oracle_pins.py`` (brute force,
textbook causal attention, closed forms, invariants); see that file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import time
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "libattn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O3, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    lib.attn_oracle_fwd.restype = ctypes.c_int
    lib.attn_oracle_fwd.argtypes = [
        P, P, P, P, ctypes.c_int, P, P, P, P, P,
        ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int,
        P, ctypes.c_int64, P, P, P, ctypes.c_int]
    lib.flex_oracle_fwd.restype = ctypes.c_int
    lib.flex_oracle_fwd.argtypes = [
        P, P, P, P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        P, ctypes.c_int64, P, P, P, ctypes.c_int]
    lib.attn_oracle_bwd.restype = ctypes.c_int
    lib.attn_oracle_bwd.argtypes = [
        P, P, P, P, ctypes.c_int, P, P, P, P, P, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int]
    lib.attn_oracle_relproj_profiles.restype = ctypes.c_int
    lib.attn_oracle_relproj_profiles.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, P]
    lib.attn_oracle_max_threads.restype = ctypes.c_int
    lib.attn_oracle_mask.restype = ctypes.c_int
    lib.attn_oracle_mask.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P,
                                     ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _as_np(t, dtype):
    """Host numpy view/copy of a tensor or array in the exact storage dtype."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.bool:
                return t.numpy().astype(np.uint8)
            t = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(t), dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().attn_oracle_max_threads())


def _mask_inputs(valid, key_valid, positions, key_positions, query_offset, B, Sq, Sk):
    """Host arrays of the mask inputs, with the optional ones defaulted."""
    valid_n = _as_np(valid, np.uint8)
    if key_valid is None:
        if Sk != Sq or query_offset != 0:
            raise ValueError("key_valid is required when keys are not the query tokens")
        kvalid_n = valid_n
    else:
        kvalid_n = _as_np(key_valid, np.uint8)
    if positions is None:
        pos_n = np.broadcast_to(np.arange(query_offset, query_offset + Sq, dtype=np.int32),
                                (B, Sq)).copy()
    else:
        pos_n = _as_np(positions, np.int32)
    if key_positions is None:
        if Sk == Sq and query_offset == 0:
            kpos_n = pos_n
        else:
            kpos_n = np.broadcast_to(np.arange(Sk, dtype=np.int32), (B, Sk)).copy()
    else:
        kpos_n = _as_np(key_positions, np.int32)
    return valid_n, kvalid_n, pos_n, kpos_n


def mask(valid, key_valid=None, positions=None, key_positions=None, window=None,
         query_offset: int = 0, Sk=None, full: bool = False, n_threads: int = 0):
    """Allowed-key counts [B, Sq] (and the [B, Sq, Sk] mask when ``full``)."""
    B, Sq = (int(x) for x in valid.shape)
    if Sk is None:
        Sk = int(key_valid.shape[1]) if key_valid is not None else Sq
    valid_n, kvalid_n, pos_n, kpos_n = _mask_inputs(valid, key_valid, positions, key_positions,
                                                    query_offset, B, Sq, Sk)
    cnt = np.empty((B, Sq), dtype=np.int32)
    m = np.empty((B, Sq, Sk), dtype=np.uint8) if full else None
    rc = _load().attn_oracle_mask(_ptr(valid_n), _ptr(kvalid_n), _ptr(pos_n), _ptr(kpos_n),
                                  0 if window is None else int(window), int(query_offset), B, Sq, Sk,
                                  _ptr(cnt), None if m is None else _ptr(m), int(n_threads))
    if rc != 0:
        raise RuntimeError("attn_oracle_mask failed")
    return (cnt, m) if full else cnt


def attn_fwd(q, k, v, profiles, sink, valid, key_valid=None, positions=None,
             key_positions=None, window: Optional[int] = None, query_offset: int = 0,
             rows=None, n_threads: int = 0, profiles_bf16: Optional[bool] = None):
    """fp64 forward.  Returns ``(out, lse, n_allowed)`` as numpy arrays.

    ``q``/``k``/``v`` are bf16 (torch tensors, or uint16 bit arrays); ``profiles``
    fp32 or bf16.  With ``rows`` (flattened ``b*Sq + i``) only those rows are
    computed and the outputs are compact: ``out [n, Hq, D]``, ``lse [n, Hq]``,
    ``n_allowed [n]``; otherwise ``out [B, Sq, Hq, D]``, ``lse [B, Sq, Hq]``,
    ``n_allowed [B, Sq]``.
    """
    import torch

    B, Sq, Hq, D = (int(x) for x in q.shape)
    Sk, Hkv = int(k.shape[1]), int(k.shape[2])
    E = int(profiles.shape[-1])
    if profiles_bf16 is None:
        profiles_bf16 = isinstance(profiles, torch.Tensor) and profiles.dtype == torch.bfloat16
    # fp64 profiles (relproj_profiles) are read as they are
    prof64 = (isinstance(profiles, np.ndarray) and profiles.dtype == np.float64) or \
        (isinstance(profiles, torch.Tensor) and profiles.dtype == torch.float64)
    qn = _as_np(q, np.uint16)
    kn = _as_np(k, np.uint16)
    vn = _as_np(v, np.uint16)
    pn = _as_np(profiles, np.float64 if prof64 else np.uint16 if profiles_bf16 else np.float32)
    pdt = 2 if prof64 else int(bool(profiles_bf16))
    sn = _as_np(sink, np.float32)
    valid_n, kvalid_n, pos_n, kpos_n = _mask_inputs(valid, key_valid, positions, key_positions,
                                                    query_offset, B, Sq, Sk)
    for name, a, shape in (("q", qn, (B, Sq, Hq, D)), ("k", kn, (B, Sk, Hkv, D)),
                           ("v", vn, (B, Sk, Hkv, D)), ("profiles", pn, (B, Hq, Sq, E)),
                           ("sink", sn, (B, Sq, Hq)), ("valid", valid_n, (B, Sq)),
                           ("key_valid", kvalid_n, (B, Sk)), ("positions", pos_n, (B, Sq)),
                           ("key_positions", kpos_n, (B, Sk))):
        if tuple(a.shape) != shape:
            raise ValueError(f"{name}: shape {tuple(a.shape)} != {shape}")
    if rows is None:
        rows_n = None
        n = B * Sq
    else:
        rows_n = _as_np(rows, np.int64).reshape(-1)
        n = int(rows_n.shape[0])
    out = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    cnt = np.empty((n,), dtype=np.int32)
    w = 0 if window is None else int(window)
    rc = _load().attn_oracle_fwd(
        _ptr(qn), _ptr(kn), _ptr(vn), _ptr(pn), pdt, _ptr(sn),
        _ptr(valid_n), _ptr(kvalid_n), _ptr(pos_n), _ptr(kpos_n), w, int(query_offset),
        B, Sq, Sk, Hq, Hkv, D, E,
        None if rows_n is None else _ptr(rows_n), n, _ptr(out), _ptr(lse), _ptr(cnt),
        int(n_threads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_fwd failed ({rc})")
    if rows is None:
        return out.reshape(B, Sq, Hq, D), lse.reshape(B, Sq, Hq), cnt.reshape(B, Sq)
    return out, lse, cnt


def attn_bwd(q, k, v, profiles, sink, valid, dout, dlse=None, key_valid=None, positions=None,
             key_positions=None, window: Optional[int] = None, query_offset: int = 0,
             profiles_bf16: Optional[bool] = None, row_lo: int = 0, row_hi: int = 0,
             magnitudes: bool = False, n_threads: int = 0):
    """fp64 gradients of the forward for upstream gradients ``dout [B,Sq,Hq,D]`` and ``dlse
    [B,Sq,Hq]`` (None: zero).  Returns ``(dq, dk, dv, dprofiles, dsink)`` as fp64 numpy arrays.

    Only the query rows ``row_lo <= i < row_hi`` take part (``row_hi`` 0: up to Sq); dk / dv
    then hold only those rows' contributions.  ``magnitudes`` returns the sums of absolute
    contributions instead.  The work runs on ``n_threads`` threads (0: OpenMP's default)
    split by (batch row, K/V head); the result does not depend on the count."""
    import torch

    B, Sq, Hq, D = (int(x) for x in q.shape)
    Sk, Hkv = int(k.shape[1]), int(k.shape[2])
    E = int(profiles.shape[-1])
    if profiles_bf16 is None:
        profiles_bf16 = isinstance(profiles, torch.Tensor) and profiles.dtype == torch.bfloat16
    qn, kn, vn = _as_np(q, np.uint16), _as_np(k, np.uint16), _as_np(v, np.uint16)
    pn = _as_np(profiles, np.uint16 if profiles_bf16 else np.float32)
    sn = _as_np(sink, np.float32)
    don = np.ascontiguousarray(_as_np(dout, np.float64) if not isinstance(dout, torch.Tensor)
                               else dout.to(torch.float64).numpy())
    dln = None
    if dlse is not None:
        dln = np.ascontiguousarray(dlse.to(torch.float64).numpy() if isinstance(dlse, torch.Tensor)
                                   else np.asarray(dlse, dtype=np.float64))
    valid_n, kvalid_n, pos_n, kpos_n = _mask_inputs(valid, key_valid, positions, key_positions,
                                                    query_offset, B, Sq, Sk)
    dq = np.empty((B, Sq, Hq, D)); dk = np.empty((B, Sk, Hkv, D)); dv = np.empty((B, Sk, Hkv, D))
    dp = np.empty((B, Hq, Sq, E)); ds = np.empty((B, Sq, Hq))
    w = 0 if window is None else int(window)
    rc = _load().attn_oracle_bwd(
        _ptr(qn), _ptr(kn), _ptr(vn), _ptr(pn), int(bool(profiles_bf16)), _ptr(sn),
        _ptr(valid_n), _ptr(kvalid_n), _ptr(pos_n), _ptr(kpos_n), w, int(query_offset),
        B, Sq, Sk, Hq, Hkv, D, E, _ptr(don), None if dln is None else _ptr(dln), int(row_lo),
        int(row_hi), int(bool(magnitudes)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dp), _ptr(ds),
        int(n_threads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_bwd failed ({rc})")
    return dq, dk, dv, dp, ds


def flex_fwd(q, k, v, sink_weights=None, tokens=None, eos_id: int = 0, fixed_block_size=None,
             sliding_window: int = 0, scale=None, rows=None, n_threads: int = 0):
    """fp64 generic flex-attention forward (no relative term), head-major layouts.

    ``q [B,Hq,Sq,D]``, ``k``/``v [B,Hkv,Sk,D]`` bf16; ``sink_weights [Hq]`` or None;
    ``tokens [B,Sq]`` or None.  Returns ``(out [B,Hq,Sq,D], lse [B,Hq,Sq], n_allowed [B,Sq])``,
    or with ``rows`` (flattened ``b*Sq + i``) the compact ``out [n,Hq,D]``, ``lse [n,Hq]``,
    ``n_allowed [n]``.
    """
    B, Hq, Sq, D = (int(x) for x in q.shape)
    Hkv, Sk = int(k.shape[1]), int(k.shape[2])
    qn = _as_np(q, np.uint16)
    kn = _as_np(k, np.uint16)
    vn = _as_np(v, np.uint16)
    sn = None if sink_weights is None else _as_np(sink_weights, np.float32)
    tn = None if tokens is None else _as_np(tokens, np.int32)
    for name, a, shape in (("q", qn, (B, Hq, Sq, D)), ("k", kn, (B, Hkv, Sk, D)), ("v", vn, (B, Hkv, Sk, D)),
                           ("sink_weights", sn, (Hq,)), ("tokens", tn, (B, Sq))):
        if a is not None and tuple(a.shape) != shape:
            raise ValueError(f"{name}: shape {tuple(a.shape)} != {shape}")
    if rows is None:
        rows_n, n = None, B * Sq
    else:
        rows_n = _as_np(rows, np.int64).reshape(-1)
        n = int(rows_n.shape[0])
    out = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    cnt = np.empty((n,), dtype=np.int32)
    rc = _load().flex_oracle_fwd(
        _ptr(qn), _ptr(kn), _ptr(vn), None if sn is None else _ptr(sn), None if tn is None else _ptr(tn),
        int(eos_id), int(fixed_block_size or 0), int(sliding_window or 0),
        float(scale) if scale is not None else 0.0, B, Sq, Sk, Hq, Hkv, D,
        None if rows_n is None else _ptr(rows_n), n, _ptr(out), _ptr(lse), _ptr(cnt), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"flex_oracle_fwd failed ({rc})")
    if rows is None:
        return (out.reshape(B, Sq, Hq, D).transpose(0, 2, 1, 3).copy(), lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy(),
                cnt.reshape(B, Sq))
    return out, lse, cnt


def relproj_profiles(rfeat, table, E: Optional[int] = None):
    """Relative logits from relative features, fp64 ``[B, Hq, Sq, E]`` (reading stated in
    ``attn_oracle.c``): ``profiles[b,h,i,r] = sum_c rfeat[b,i,h,c] * table[t,r,c]``.

    ``rfeat [B,Sq,Hq,d_rel]`` bf16; ``table [T,E,d_rel]`` bf16 with T = 1 (shared) or Hq."""
    B, Sq, Hq, d_rel = (int(x) for x in rfeat.shape)
    T, Et, dt = (int(x) for x in table.shape)
    if dt != d_rel or T not in (1, Hq):
        raise ValueError(f"table {tuple(table.shape)} does not match rfeat {tuple(rfeat.shape)}")
    E = Et if E is None else int(E)
    rn = _as_np(rfeat, np.uint16)
    tn = _as_np(table, np.uint16)
    out = np.empty((B, Hq, Sq, E), dtype=np.float64)
    if _load().attn_oracle_relproj_profiles(_ptr(rn), _ptr(tn), T, B, Sq, Hq, d_rel, E, _ptr(out)) != 0:
        raise RuntimeError("attn_oracle_relproj_profiles failed")
    return out


def timed_fwd(inputs: dict, rows, n_threads: int = 0):
    """Run the oracle on ``rows`` of a generated workload; returns (seconds, result)."""
    t0 = time.perf_counter()
    res = attn_fwd(inputs["q"], inputs["k"], inputs["v"], inputs["profiles"], inputs["sink"],
                   inputs["valid"], inputs.get("key_valid"), inputs.get("positions"),
                   inputs.get("key_positions"), inputs.get("window"),
                   inputs.get("query_offset", 0), rows=rows, n_threads=n_threads)
    return time.perf_counter() - t0, res
