"""attn_fwd_noalloc, the forward entry point that allocates nothing (its workspace is the
library's per-GPU scratch), against attn_fwd with a workspace of its own: bit for bit, on
calls in a row whose second input is smaller than the first (the scratch keeps the first
call's contents), and within the oracle's acceptance bar on the small case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_util import announce, assert_close, run_oracle, to_device
from transformer_attention_03_amd import binding
from transformer_attention_03_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield


def _both(x, name):
    d = to_device(x)
    B, S, Hq, D = x["q"].shape
    Hkv = x["k"].shape[2]
    need = binding.attn_fwd_workspace_size(B, S, S, Hkv, D)
    assert need <= binding.NOALLOC_SCRATCH_BYTES
    announce(f"no-alloc: attn_fwd reference on {name} (workspace {need} bytes)")
    ref_out, ref_lse = binding.attn_fwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"],
                                        positions=d["positions"], window=x["window"])
    out = torch.full((B, S, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, S, Hq), float("nan"), device="cuda")
    torch.cuda.synchronize()
    announce(f"no-alloc: attn_fwd_noalloc on {name}")
    binding.attn_fwd_noalloc(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"], positions=d["positions"],
                             window=x["window"], out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), name
    assert torch.equal(lse, ref_lse), name
    return out, lse


def test_noalloc_equals_attn_fwd_on_two_calls_in_a_row_second_smaller():
    # first: the long-context workload, whose workspace (64.2 MiB) is near the scratch's size
    _both(W.generate(W.WORKLOADS["long"]), "long")
    # second: a smaller input with a window, documents and invalid tokens (stale scratch behind it)
    x = W.custom(B=2, S=333, Hq=8, Hkv=2, D=64, E=70, window=90, seed=401, structure="packed", doc_min=20,
                 doc_max=160, invalid_tail=9)
    out, lse = _both(x, "packed_window_small")
    ref_out, ref_lse, ref_cnt = run_oracle(x)
    assert_close(out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_out, ref_lse, ref_cnt,
                 "noalloc small vs oracle")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    x = W.custom(B=1, S=64, Hq=4, Hkv=2, D=128, E=8, seed=402)
    d = to_device(x)
    # one batch row of 40000 keys x 8 heads needs more than the scratch: rejected before any launch
    q = torch.zeros(1, 40000, 8, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 40000, 8, 128, dtype=torch.bfloat16, device="cuda")
    prof = torch.zeros(1, 8, 40000, 1, device="cuda")
    sink = torch.zeros(1, 40000, 8, device="cuda")
    valid = torch.ones(1, 40000, dtype=torch.bool, device="cuda")
    announce("no-alloc: size beyond the scratch is rejected")
    with pytest.raises(binding.InkAttnError, match="no-allocation scratch") as e:
        binding.attn_fwd_noalloc(q, kv, kv, prof, sink, valid)
    assert e.value.status == 5
    # and the entry point still works afterwards
    _both(x, "tiny_after_rejection")
