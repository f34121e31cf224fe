"""Seeded synthetic inputs for the learned-relative GQA attention forward.

This module only draws random numbers and lays out structure (padding spans,
document boundaries, positions).  It holds none of the attention arithmetic, so
that both the fp64 oracle and the HIP path can consume the same inputs without
sharing any code of the method.

Shapes follow the forward of ``Inkling2FlexAttention`` (page
"nemo_automodel.components.models.inkling2.flex_attention", section API,
``forward`` parameters):

* q ``[B, S, Hq, D]``, k / v ``[B, Sk, Hkv, D]`` -- bf16
* profiles ``[B, Hq, S, E]`` -- fp32 or bf16
* sink ``[B, S, Hq]`` -- fp32
* valid ``[B, S]`` / key_valid ``[B, Sk]`` -- bool
* positions ``[B, S]`` / key_positions ``[B, Sk]`` -- int32, restarting at 0
  at every document start.

Every tensor is generated on the CPU with ``torch.Generator().manual_seed``;
the draw order is fixed: structure first, then q, k, v, profiles, sink.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic attention workload."""

    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    E: int
    window: Optional[int]           # None: no sliding window
    structure: str                  # "single", "tail_pad", "packed"
    invalid_tail: int = 0           # fixed number of invalid trailing tokens
    max_tail_pad: int = 0           # tail_pad: per-row padding drawn in U{0..max}
    doc_min: int = 0                # packed: document length range (inclusive)
    doc_max: int = 0
    profiles_dtype: torch.dtype = torch.float32
    profile_std: float = 0.5
    sink_std: float = 1.0
    qkv_std: float = 1.0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads the pages' method is exercised on, plus the full-causal
# variant of the local-layer shape (same sizes, window removed).
WORKLOADS = {
    "tiny": Workload("tiny", B=1, S=128, Hq=4, Hkv=1, D=64, E=32, window=None,
                     structure="single", invalid_tail=8, seed=1001),
    "causal_gqa": Workload("causal_gqa", B=2, S=2048, Hq=16, Hkv=4, D=128, E=128,
                           window=None, structure="tail_pad", max_tail_pad=256, seed=1002),
    "local": Workload("local", B=1, S=8192, Hq=32, Hkv=8, D=128, E=1024, window=1024,
                      structure="single", seed=1003),
    "full_causal_8k": Workload("full_causal_8k", B=1, S=8192, Hq=32, Hkv=8, D=128, E=1024,
                               window=None, structure="single", seed=1013),
    "packed": Workload("packed", B=1, S=16384, Hq=32, Hkv=8, D=128, E=256, window=None,
                       structure="packed", doc_min=256, doc_max=4096, invalid_tail=100,
                       seed=1004),
    "long": Workload("long", B=1, S=32768, Hq=64, Hkv=8, D=128, E=512, window=None,
                     structure="single", profiles_dtype=torch.bfloat16, sink_std=2.0,
                     seed=1005),
}


def _structure(w: Workload, gen: torch.Generator):
    """valid [B,S] bool and positions [B,S] int32 for the workload's structure."""
    B, S = w.B, w.S
    valid = torch.zeros(B, S, dtype=torch.bool)
    positions = torch.empty(B, S, dtype=torch.int32)
    cols = torch.arange(S, dtype=torch.int32)
    doc_starts = []
    for b in range(B):
        if w.structure == "single":
            positions[b] = cols
            starts = [0]
        elif w.structure == "tail_pad":
            positions[b] = cols
            starts = [0]
        elif w.structure == "packed":
            starts = []
            c = 0
            while c < S:
                starts.append(c)
                length = int(torch.randint(w.doc_min, w.doc_max + 1, (1,), generator=gen))
                end = min(S, c + length)
                positions[b, c:end] = torch.arange(end - c, dtype=torch.int32)
                c = end
        else:
            raise ValueError(f"unknown structure {w.structure!r}")
        n_valid = S - w.invalid_tail
        if w.structure == "tail_pad":
            pad = int(torch.randint(0, w.max_tail_pad + 1, (1,), generator=gen))
            n_valid = S - pad
        valid[b, :max(0, n_valid)] = True
        doc_starts.append(starts)
    return valid, positions, doc_starts


def _randn(shape, std: float, gen: torch.Generator, dtype: torch.dtype) -> torch.Tensor:
    """Normal draw of the given standard deviation, rounded (RNE) to ``dtype``.

    Large tensors are drawn in slabs along the first axis so that the fp32
    staging buffer stays bounded; the slab size does not change the values.
    """
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    n = flat.numel()
    slab = 1 << 26
    for s in range(0, n, slab):
        e = min(n, s + slab)
        x = torch.randn(e - s, generator=gen, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[s:e] = x.to(dtype)
    return out


def generate(w: Workload, seed: Optional[int] = None) -> dict:
    """Host tensors for workload ``w``; deterministic in (w, seed)."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    valid, positions, doc_starts = _structure(w, gen)
    q = _randn((w.B, w.S, w.Hq, w.D), w.qkv_std, gen, torch.bfloat16)
    k = _randn((w.B, w.S, w.Hkv, w.D), w.qkv_std, gen, torch.bfloat16)
    v = _randn((w.B, w.S, w.Hkv, w.D), w.qkv_std, gen, torch.bfloat16)
    profiles = _randn((w.B, w.Hq, w.S, w.E), w.profile_std, gen, w.profiles_dtype)
    sink = _randn((w.B, w.S, w.Hq), w.sink_std, gen, torch.float32)
    return dict(q=q, k=k, v=v, profiles=profiles, sink=sink, valid=valid,
                positions=positions, key_valid=None, key_positions=None,
                window=w.window, query_offset=0, doc_starts=doc_starts, workload=w)


def custom(B: int, S: int, Hq: int, Hkv: int, D: int, E: int, window: Optional[int] = None,
           seed: int = 0, structure: str = "single", invalid_tail: int = 0,
           max_tail_pad: int = 0, doc_min: int = 0, doc_max: int = 0,
           profiles_dtype: torch.dtype = torch.float32, sink_std: float = 1.0,
           profile_std: float = 0.5) -> dict:
    """Inputs for an ad-hoc shape with the same value recipe as the named workloads."""
    w = Workload("custom", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, E=E, window=window,
                 structure=structure, invalid_tail=invalid_tail, max_tail_pad=max_tail_pad,
                 doc_min=doc_min, doc_max=doc_max, profiles_dtype=profiles_dtype,
                 profile_std=profile_std, sink_std=sink_std, seed=seed)
    return generate(w)


def sample_rows(B: int, S: int, n: int, seed: int, must: tuple = ()) -> torch.Tensor:
    """Deterministic sample of flattened query rows ``b*S + i`` (sorted, unique).

    ``must`` lists (b, i) rows that are always included (e.g. the first and last
    rows, document starts).
    """
    gen = torch.Generator().manual_seed(seed)
    picks = torch.randint(0, B * S, (n,), generator=gen, dtype=torch.int64)
    extra = torch.tensor([b * S + i for (b, i) in must], dtype=torch.int64)
    rows = torch.unique(torch.cat([picks, extra]))
    return rows[(rows >= 0) & (rows < B * S)]


# ----------------------------------------------------------------------------
# Generic flex-attention inputs (page "nemo_automodel.components.attention.
# flex_attention", FlexAttention.forward): head-major q [B,Hq,S,D], k / v
# [B,Hkv,S,D] bf16, per-head sink weights [Hq] fp32, and token ids [B,S] int32
# whose EOS tokens end the documents of "block_causal".
# ----------------------------------------------------------------------------
EOS_ID = 2


@dataclasses.dataclass(frozen=True)
class FlexWorkload:
    """Shape and value recipe of one synthetic generic flex-attention workload."""

    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    mask: str                       # "causal" or "block_causal"
    doc_min: int = 0                # block_causal: document lengths U{doc_min..doc_max}
    doc_max: int = 0
    fixed_block_size: Optional[int] = None
    sliding_window: int = 0
    sinks: bool = True
    sink_std: float = 1.0
    scale: Optional[float] = None
    Sk: Optional[int] = None        # key length (default S; only for "causal" without fixed blocks)
    seed: int = 0


FLEX_WORKLOADS = {
    # the S = 8192 GQA shape of the local / full-causal workloads, as a generic
    # block-causal layer: EOS-delimited documents, per-head sinks, bf16 output
    "flex_block_causal": FlexWorkload("flex_block_causal", B=1, S=8192, Hq=32, Hkv=8, D=128,
                                      mask="block_causal", doc_min=256, doc_max=4096, seed=1101),
}


def generate_flex(w: FlexWorkload, seed: Optional[int] = None) -> dict:
    """Host tensors for a generic flex workload; deterministic in (w, seed)."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    B, S = w.B, w.S
    Sk = S if w.Sk is None else w.Sk
    tokens = None
    doc_ends = []
    if w.mask == "block_causal":
        # token ids in [3, 1000); an EOS closes each document (the last one may run to the end)
        tokens = torch.randint(3, 1000, (B, S), generator=gen, dtype=torch.int32)
        for b in range(B):
            ends = []
            c = 0
            while True:
                length = int(torch.randint(w.doc_min, w.doc_max + 1, (1,), generator=gen))
                if c + length > S:
                    break
                tokens[b, c + length - 1] = EOS_ID
                ends.append(c + length - 1)
                c += length
            doc_ends.append(ends)
    q = _randn((B, w.Hq, S, w.D), 1.0, gen, torch.bfloat16)
    k = _randn((B, w.Hkv, Sk, w.D), 1.0, gen, torch.bfloat16)
    v = _randn((B, w.Hkv, Sk, w.D), 1.0, gen, torch.bfloat16)
    sink_weights = _randn((w.Hq,), w.sink_std, gen, torch.float32) if w.sinks else None
    return dict(q=q, k=k, v=v, sink_weights=sink_weights, tokens=tokens, eos_id=EOS_ID,
                fixed_block_size=w.fixed_block_size, sliding_window=w.sliding_window, scale=w.scale,
                doc_ends=doc_ends, workload=w)


def flex_custom(B: int, S: int, Hq: int, Hkv: int, D: int, mask: str = "causal", seed: int = 0,
                **kw) -> dict:
    """Inputs for an ad-hoc generic flex shape with the same value recipe."""
    return generate_flex(FlexWorkload("custom", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mask=mask, seed=seed, **kw))


# ----------------------------------------------------------------------------
# Relative features instead of profiles (the in-kernel profile rows of
# attn_fwd_relproj): per (token, query head) d_rel features rfeat
# [B,S,Hq,d_rel] and a relative table [T,E,d_rel] (T = 1 shared, or Hq), both
# bf16.  rfeat ~ N(0, 1) and table ~ N(0, 0.5 / sqrt(d_rel)), so that the
# profile entries they form have the standard deviation 0.5 of the profiles
# of the workloads above.  Drawn after the workload's own tensors, from the
# same generator.
# ----------------------------------------------------------------------------
RELPROJ_WORKLOADS = {
    # the local (sliding-window) layer with its profiles formed in-kernel
    "local_relproj": (WORKLOADS["local"], 32, 1),
}


def add_relative_features(x: dict, d_rel: int, table_heads: int, seed: int) -> dict:
    """Adds ``rfeat`` and ``table`` (and ``d_rel``) to the inputs ``x`` of a workload; the
    profiles tensor is dropped (the kernel forms its rows)."""
    w = x["workload"]
    gen = torch.Generator().manual_seed(seed)
    B, S, Hq = x["q"].shape[0], x["q"].shape[1], x["q"].shape[2]
    E = x["profiles"].shape[-1]
    T = 1 if table_heads == 1 else Hq
    y = dict(x)
    y["rfeat"] = _randn((B, S, Hq, d_rel), 1.0, gen, torch.bfloat16)
    y["table"] = _randn((T, E, d_rel), 0.5 / d_rel ** 0.5, gen, torch.bfloat16)
    y["d_rel"] = d_rel
    y["E"] = E
    y["profiles"] = None
    del w
    return y


def generate_relproj(name: str) -> dict:
    """Inputs of a named relative-feature workload (deterministic)."""
    w, d_rel, table_heads = RELPROJ_WORKLOADS[name]
    x = generate(w)
    y = add_relative_features(x, d_rel, table_heads, seed=w.seed + 500)
    y["relproj_name"] = name
    return y
