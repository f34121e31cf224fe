"""CPU-side checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any launch (no GPU needed).

Fake device addresses are used only in calls that must fail validation; no
call here reaches a kernel launch.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from transformer_attention_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "inkattn.h")

A = 1 << 20          # a 16-byte aligned fake address (never dereferenced)
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:flex_)?attn_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = binding.load()
    names = declared_functions()
    assert names == sorted(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_sizes():
    assert binding.attn_status_string(0) == "ok"
    assert "NULL" in binding.attn_status_string(1)
    assert binding.attn_query_block() == 32 and binding.attn_key_tile() == 64
    # tile summaries (16 B per query block / key tile) + key start columns (4 B per key),
    # each rounded up to 256 B, then the fp16 values
    # and one flag byte per staged value tile (rounded up to 256 B)
    assert binding.attn_fwd_workspace_size(1, 128, 128, 2, 64) == 256 + 512 + 128 * 2 * 64 * 2 + 256
    # values are staged in whole 64-key tiles: 65 keys take two
    assert binding.attn_fwd_workspace_size(2, 33, 65, 1, 128) == 256 + 1024 + 2 * 128 * 128 * 2 + 256
    assert binding.attn_fwd_workspace_size(40, 64, 64, 1, 64) == 2048 + 40 * 64 * 4 + 40 * 64 * 64 * 2 + 256
    assert binding.attn_fwd_workspace_size(1, 64, 64 * 300, 1, 64) == (4864 + 64 * 300 * 4 + 64 * 300 * 64 * 2
                                                                       + 512)
    assert binding.attn_fwd_workspace_size(0, 10, 10, 1, 64) == 0


def call(**over):
    a = dict(q=A, k=A, v=A, profiles=A, pdt=0, sink=A, valid=A, key_valid=None, positions=None,
             key_positions=None, window=0, qoff=0, B=1, Sq=64, Sk=64, Hq=4, Hkv=2, D=128, E=16,
             out=A, lse=A, ws=A, wsb=1 << 20, stream=None)
    a.update(over)
    lib = binding.load()
    return lib.attn_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["profiles"]), a["pdt"], P(a["sink"]),
                        P(a["valid"]), P(a["key_valid"]), P(a["positions"]), P(a["key_positions"]),
                        a["window"], a["qoff"], a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"],
                        a["E"], P(a["out"]), P(a["lse"]), P(a["ws"]), a["wsb"], P(a["stream"]))


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(sink=None), 1), (dict(out=None), 1), (dict(valid=None), 1),
    (dict(k=None), 1),
    (dict(Sk=100), 1),                      # Sk != Sq needs key_valid
    (dict(qoff=5), 1),                      # query_offset != 0 needs key_valid
    (dict(Hq=6, Hkv=4), 2), (dict(Hkv=0), 2), (dict(E=0), 2), (dict(Sq=-1), 2),
    (dict(Sq=1 << 30, Sk=1 << 30), 2), (dict(qoff=-1, key_valid=A), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(pdt=7), 3),
    (dict(q=A + 8), 4), (dict(out=A + 4), 4), (dict(profiles=A + 2), 4), (dict(positions=A + 2), 4),
    (dict(ws=None), 5), (dict(wsb=16), 5), (dict(wsb=256 + 256 + 64 * 2 * 128 * 2), 5), (dict(ws=A + 8), 4),
    (dict(wsb=256 + 256 + 64 * 2 * 128 * 2 + 255), 5),
    (dict(Sq=1 << 20, Sk=1 << 20, Hkv=16, Hq=16, key_valid=A), 2),   # one k/v row of 4 GiB
])
def test_host_validation_rejects_before_launch(over, status):
    assert call(**over) == status
    assert binding.attn_last_error() != ""


def test_bf16_profiles_need_only_2_byte_alignment_and_empty_rows_return_ok():
    # B*Sq == 0 returns OK without touching memory
    assert call(Sq=0, Sk=0, B=1) == 0
    assert call(B=0) == 0
    # bf16 profiles at a 2-byte offset pass the alignment check; a too-small
    # workspace is what stops the call (still before any launch)
    assert call(pdt=1, profiles=A + 2, wsb=8) == 5


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.attn_fwd(x, x, x, torch.zeros(1, 2, 4, 8), torch.zeros(1, 4, 2),
                         torch.ones(1, 4, dtype=torch.bool))


def test_product_path_does_not_reach_the_oracle():
    """The package and the HIP source never name the oracle."""
    pkg = os.path.join(ROOT, "transformer_attention_03_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "attn_oracle" not in text, f


def flex_call(**over):
    a = dict(q=A, k=A, v=A, sink=None, tokens=None, eos=0, fixed=0, window=0, scale=0.0,
             B=1, Sq=64, Sk=64, Hq=4, Hkv=2, D=128, out=A, lse=None, ws=A, wsb=1 << 20, stream=None)
    a.update(over)
    lib = binding.load()
    return lib.flex_attn_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["sink"]), P(a["tokens"]), a["eos"],
                             a["fixed"], a["window"], a["scale"], a["B"], a["Sq"], a["Sk"], a["Hq"],
                             a["Hkv"], a["D"], P(a["out"]), P(a["lse"]), P(a["ws"]), a["wsb"],
                             P(a["stream"]))


@pytest.mark.parametrize("over,status", [
    (dict(Hq=3, Hkv=2), 2), (dict(D=96), 3), (dict(q=None), 1), (dict(out=None), 1), (dict(k=None), 1),
    (dict(q=A + 8), 4), (dict(out=A + 4), 4), (dict(sink=A + 2), 4), (dict(tokens=A, Sk=65), 2),
    (dict(fixed=16, Sk=65), 2), (dict(ws=None), 5), (dict(wsb=100), 5), (dict(B=-1), 2),
])
def test_flex_host_validation(over, status):
    assert flex_call(**over) == status
    assert binding.attn_last_error() != ""


def test_flex_workspace_size():
    # the attention workspace, then positions (4 B per query) and validity (1 B per token), each rounded to 256 B
    assert binding.flex_attn_workspace_size(1, 64, 64, 2, 128) == (binding.attn_fwd_workspace_size(1, 64, 64, 2, 128)
                                                                   + 256 + 256)
    assert binding.flex_attn_workspace_size(2, 100, 300, 1, 64) == (binding.attn_fwd_workspace_size(2, 100, 300, 1, 64)
                                                                     + 1024 + 768)
    assert binding.flex_attn_workspace_size(0, 64, 64, 2, 128) == 0


def bwd_call(**over):
    a = dict(q=A, k=A, v=A, profiles=A, pdt=0, sink=A, valid=A, key_valid=None, positions=None,
             key_positions=None, window=0, qoff=0, B=1, Sq=64, Sk=64, Hq=4, Hkv=2, D=128, E=16,
             out=A, lse=A, dout=A, dlse=None, dq=A, dk=A, dv=A, dprof=A, dsink=A, ws=A, wsb=1 << 20,
             stream=None)
    a.update(over)
    lib = binding.load()
    return lib.attn_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["profiles"]), a["pdt"], P(a["sink"]),
                        P(a["valid"]), P(a["key_valid"]), P(a["positions"]), P(a["key_positions"]),
                        a["window"], a["qoff"], a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"], a["E"],
                        P(a["out"]), P(a["lse"]), P(a["dout"]), P(a["dlse"]), P(a["dq"]), P(a["dk"]),
                        P(a["dv"]), P(a["dprof"]), P(a["dsink"]), P(a["ws"]), a["wsb"], P(a["stream"]))


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(dq=None), 1), (dict(dk=None), 1), (dict(dprof=None), 1),
    (dict(dsink=None), 1), (dict(lse=None), 1), (dict(valid=None), 1), (dict(Sk=100), 1),
    (dict(Hq=6, Hkv=4), 2), (dict(E=0), 2), (dict(Sq=-1), 2), (dict(D=96), 3), (dict(pdt=5), 3),
    (dict(dout=A + 8), 4), (dict(dk=A + 4), 4), (dict(dprof=A + 2), 4), (dict(dsink=A + 2), 4),
    (dict(ws=None), 5), (dict(wsb=68607), 5),
])
def test_bwd_host_validation(over, status):
    assert bwd_call(**over) == status
    assert binding.attn_last_error() != ""


def test_bwd_workspace_size():
    # summaries 256 + 256; per query 8 B; per row 8 B; bf16 dout; each rounded up to 256 B
    assert binding.attn_bwd_workspace_size(1, 64, 64, 4, 2, 128) == 512 + 512 + 2048 + 65536
    assert bwd_call(wsb=68608, ws=None) == 5
    assert binding.attn_bwd_workspace_size(0, 64, 64, 4, 2, 128) == 0
    # bf16 profile gradients need only 2-byte alignment: the workspace check is what stops this call
    assert bwd_call(pdt=1, profiles=A + 2, dprof=A + 2, wsb=8) == 5


def test_late_size_checks_run_before_any_launch():
    """A call whose tile count overflows the pre-pass grid is rejected by its checks alone: the
    status is the shape error, not a launch error (this container has no GPU, so an attempted
    launch would fail with INKATTN_ERR_LAUNCH)."""
    big = dict(B=4096, Sq=1, Sk=(1 << 25) - 64, Hq=1, Hkv=1, D=64, wsb=1 << 62)
    assert flex_call(**big) == 2
    assert "too many tiles" in binding.attn_last_error()
    assert call(E=1, key_valid=A, **big) == 2
    assert "too many tiles" in binding.attn_last_error()


def debug_mask_call(**over):
    a = dict(valid=A, key_valid=None, positions=None, key_positions=None, window=0, qoff=0, B=1, Sq=64, Sk=64,
             mask=A, stream=None)
    a.update(over)
    return binding.load().attn_debug_mask(P(a["valid"]), P(a["key_valid"]), P(a["positions"]),
                                          P(a["key_positions"]), a["window"], a["qoff"], a["B"], a["Sq"],
                                          a["Sk"], P(a["mask"]), P(a["stream"]))


@pytest.mark.parametrize("over,status", [
    (dict(mask=None), 1), (dict(valid=None), 1), (dict(Sk=10), 1), (dict(B=-1), 2),
    (dict(B=2, Sq=1 << 16, Sk=1 << 16, key_valid=A), 2), (dict(positions=A + 1), 4),
])
def test_debug_mask_validation(over, status):
    assert debug_mask_call(**over) == status
    assert binding.attn_last_error() != ""


def test_debug_mask_empty_is_ok():
    assert debug_mask_call(B=0) == 0 and debug_mask_call(Sq=0, Sk=0) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 1 << 20, 1, 64, 64, 2, 128), 5), ((A, 16, 1, 64, 64, 2, 128), 5), ((A, 1 << 20, 1, 64, 64, 2, 96), 3),
    ((A + 8, 1 << 20, 1, 64, 64, 2, 128), 4), ((A, 1 << 20, -1, 64, 64, 2, 128), 2),
])
def test_check_values_validation(args, status):
    ws, wsb, B, Sq, Sk, Hkv, D = args
    assert binding.load().attn_check_values(P(ws), wsb, B, Sq, Sk, Hkv, D, None) == status
    assert binding.attn_last_error() != ""


def test_check_values_without_tiles_is_ok():
    assert binding.load().attn_check_values(None, 0, 0, 64, 64, 2, 128, None) == 0
    assert binding.load().attn_check_values(None, 0, 1, 64, 0, 2, 128, None) == 0
    assert binding.attn_status_string(7) == "a value outside the supported range"


def test_int64_positions_and_tokens_are_range_checked_before_narrowing():
    import torch
    ok = binding._narrow_int64(torch.tensor([0, 5, (1 << 30) - 1]), "positions", 0, binding.POS_LIMIT)
    assert ok.dtype == torch.int32 and ok.tolist() == [0, 5, (1 << 30) - 1]
    for bad in ([0, 1 << 30], [-1, 3], [1 << 40]):
        with pytest.raises(ValueError, match="positions"):
            binding._narrow_int64(torch.tensor(bad), "positions", 0, binding.POS_LIMIT)
    with pytest.raises(ValueError, match="tokens"):
        binding._narrow_int64(torch.tensor([1 << 31]), "tokens", -(1 << 31), 1 << 31)
    assert binding._narrow_int64(torch.tensor([-(1 << 31), 7]), "tokens", -(1 << 31), 1 << 31).tolist() == [
        -(1 << 31), 7]


def test_noalloc_rejects_sizes_beyond_the_scratch_before_touching_the_device():
    lib = binding.load()
    # B=1, Sq=Sk=40000, Hkv=8, D=128: the fp16 value copy alone is 82 MB, above the 72 MiB scratch
    rc = lib.attn_fwd_noalloc(P(A), P(A), P(A), P(A), 0, P(A), P(A), None, None, None, 0, 0,
                              1, 40000, 40000, 8, 8, 128, 1, P(A), P(A), None)
    assert rc == 5
    assert "no-allocation scratch" in binding.attn_last_error()
    assert binding.attn_fwd_workspace_size(1, 40000, 40000, 8, 128) > binding.NOALLOC_SCRATCH_BYTES
    # the long-context workload (B=1, S=32768, Hkv=8, D=128) fits
    assert binding.attn_fwd_workspace_size(1, 32768, 32768, 8, 128) <= binding.NOALLOC_SCRATCH_BYTES
