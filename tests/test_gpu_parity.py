"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes are compared element by element (every output, several tiles
and ragged tails).  The full-size workloads, in the launch configuration the
benchmark times, are compared element by element over every row, except the
long-context one (S = 32768, 64 heads), which is compared on its first 1024
rows, every row with a dominating sink and 1024 random rows; exact properties
hold at every size (allowed-key counts of every row, count probe, index probe,
determinism).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (announce, assert_close, check_full, check_rows, count_probe_inputs,
                            counts_from_lse, run_hip, run_oracle, to_device)
from transformer_attention_03_amd import binding
from transformer_attention_03_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()   # fails loudly when the HIP library is missing
    yield


# ------------------------------------------------------------------------------------------
# small shapes, whole output
# ------------------------------------------------------------------------------------------
SMALL = {
    "tiny": lambda: W.generate(W.WORKLOADS["tiny"]),
    "tailpad_G4_D128": lambda: W.custom(B=2, S=300, Hq=8, Hkv=2, D=128, E=64, seed=101,
                                        structure="tail_pad", max_tail_pad=40),
    "window_G4_D64": lambda: W.custom(B=1, S=517, Hq=4, Hkv=1, D=64, E=100, window=70, seed=102),
    "packed_G2_D128": lambda: W.custom(B=1, S=700, Hq=8, Hkv=4, D=128, E=48, seed=103, structure="packed",
                                       doc_min=20, doc_max=200, invalid_tail=13),
    "packed_window": lambda: W.custom(B=2, S=400, Hq=4, Hkv=2, D=128, E=30, window=45, seed=104,
                                      structure="packed", doc_min=5, doc_max=90, invalid_tail=7),
    "bf16_profiles_sink2": lambda: W.custom(B=1, S=333, Hq=16, Hkv=2, D=128, E=77, seed=105,
                                            profiles_dtype=torch.bfloat16, sink_std=2.0),
    "bf16_profiles_D64": lambda: W.custom(B=2, S=290, Hq=8, Hkv=2, D=64, E=150, seed=113,
                                          profiles_dtype=torch.bfloat16, structure="tail_pad", max_tail_pad=30),
    "bf16_profiles_D64_window": lambda: W.custom(B=1, S=400, Hq=4, Hkv=1, D=64, E=64, window=64, seed=114,
                                                 profiles_dtype=torch.bfloat16),
    "G1": lambda: W.custom(B=1, S=260, Hq=3, Hkv=3, D=128, E=16, seed=106),
    "G3_hpw3": lambda: W.custom(B=1, S=190, Hq=6, Hkv=2, D=64, E=200, seed=107, window=33),
    "G16_two_chunks": lambda: W.custom(B=1, S=150, Hq=16, Hkv=1, D=128, E=40, seed=108,
                                       structure="packed", doc_min=10, doc_max=60),
    "E1_window1": lambda: W.custom(B=1, S=100, Hq=4, Hkv=2, D=64, E=1, window=1, seed=109),
    "E_beyond_S": lambda: W.custom(B=1, S=97, Hq=4, Hkv=1, D=128, E=300, seed=110),
    "S1": lambda: W.custom(B=3, S=1, Hq=4, Hkv=2, D=128, E=5, seed=111),
    "wide_sink": lambda: W.custom(B=1, S=200, Hq=8, Hkv=2, D=128, E=64, seed=112, sink_std=8.0,
                                  profile_std=3.0),
    # strip runs that reach past the end of a (batch row, head) profile block: the last row
    # (E 100), and with E below a run's entry count several rows before it (E 5, bf16 E 3)
    "E100_block_end": lambda: W.custom(B=1, S=333, Hq=4, Hkv=2, D=128, E=100, seed=115),
    "E5_rows_near_end": lambda: W.custom(B=1, S=100, Hq=4, Hkv=2, D=64, E=5, seed=116),
    "bf16_E3_rows_near_end": lambda: W.custom(B=1, S=129, Hq=4, Hkv=1, D=128, E=3, seed=117,
                                              profiles_dtype=torch.bfloat16),
    # more workgroups than two per CU: 531 (59 batch rows x 9 heads, not a multiple of the
    # 8 XCDs) and 544 (17 batch rows x 8 K/V heads x 4 query groups, G = 4, documents, window)
    "items_531_G1_D64": lambda: W.custom(B=59, S=256, Hq=9, Hkv=9, D=64, E=40, seed=118,
                                         structure="tail_pad", max_tail_pad=60),
    "items_544_G4_D128": lambda: W.custom(B=17, S=256, Hq=32, Hkv=8, D=128, E=100, seed=119, window=150,
                                          structure="packed", doc_min=20, doc_max=120, invalid_tail=9),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    x = SMALL[name]()
    check_full(x, name)


def test_determinism_bitwise():
    x = SMALL["packed_G2_D128"]()
    d = to_device(x)
    announce("determinism: attn_fwd x3 on packed_G2_D128")
    runs = [run_hip(x, d=d) for _ in range(3)]
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])


def test_marshal_once_launchers_equal_the_calls():
    """planned_forward_launchers (the bench's timed path) gives attn_fwd's bits, launch after launch."""
    x = SMALL["packed_G2_D128"]()
    d = to_device(x)
    announce("marshal-once launchers: plan / stage_values / attention on packed_G2_D128, twice")
    ref_out, ref_lse = run_hip(x, d=d)
    ws = torch.empty(binding.attn_fwd_workspace_size(*d["q"].shape[:2], d["k"].shape[1], d["k"].shape[2],
                                                     d["q"].shape[3]), dtype=torch.uint8, device="cuda")
    plan, stage_values, attention, out, lse = binding.planned_forward_launchers(
        d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"], d["key_valid"], d["positions"],
        d["key_positions"], window=x.get("window"), workspace=ws)
    for _ in range(2):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        plan()
        stage_values()
        attention()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().double().numpy(), ref_out)
        assert np.array_equal(lse.cpu().double().numpy(), ref_lse)


def test_count_probe_small():
    """Mask inside the hot path: lse = ln(n_allowed) exactly decodes the oracle's counts."""
    for name in ("packed_window", "tailpad_G4_D128", "window_G4_D64"):
        x = count_probe_inputs(SMALL[name]())
        announce(f"count probe: attn_fwd on {name}")
        _, lse = run_hip(x)
        cnt = oracle.mask(x["valid"], positions=x["positions"], window=x["window"])
        got = counts_from_lse(lse)
        for h in range(got.shape[-1]):
            assert np.array_equal(got[..., h], cnt), f"{name} head {h}"


INDEX_PROBES = [
    # (E, D, profiles dtype, S, structure): E >= 128 reaches the row-by-row strip copy (every
    # distance of a wave's 32 rows x 64 keys inside [0, E)); E = 70 only the per-lane paths
    (70, 128, torch.float32, 300, "packed"),
    (128, 128, torch.float32, 600, "single"),
    (160, 64, torch.float32, 600, "single"),
    (128, 128, torch.bfloat16, 600, "single"),
    (200, 64, torch.bfloat16, 520, "packed"),
]


@pytest.mark.parametrize("E,D,pdt,S,structure", INDEX_PROBES,
                         ids=[f"E{c[0]}_D{c[1]}_{str(c[2])[6:]}" for c in INDEX_PROBES])
def test_index_probe_decodes_key(E, D, pdt, S, structure):
    """Profile gather indexing: only distance r*(h,i) carries weight; v encodes the key."""
    B, Hq, Hkv = 1, 8, 2
    x = W.custom(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, E=E, seed=120, structure=structure, doc_min=150, doc_max=400,
                 profiles_dtype=pdt)
    pos = x["positions"].numpy()
    x["q"].zero_()
    x["k"].zero_()
    x["sink"].fill_(-math.inf)
    h_idx = torch.arange(Hq)[:, None]
    i_idx = torch.arange(S)[None, :]
    n_i = torch.from_numpy(pos[0]).long()[None, :] + 1
    rstar = (7 * h_idx + i_idx) % torch.clamp(n_i, max=E)
    prof = torch.full((B, Hq, S, E), -30000.0)
    prof[0].scatter_(2, rstar[..., None], 40.0)
    x["profiles"] = prof.to(pdt)
    v = torch.zeros(B, S, Hkv, D)
    j = torch.arange(S, dtype=torch.float32)
    v[0, :, :, 0] = (j % 256)[:, None]
    v[0, :, :, 1] = (j // 256)[:, None]
    v[0, :, :, 2] = torch.arange(Hkv, dtype=torch.float32)[None, :]
    x["v"] = v.to(torch.bfloat16)
    announce(f"index probe: attn_fwd E={E} D={D} profiles={pdt} S={S}")
    out, _ = run_hip(x)
    dec = np.rint(out[0, :, :, 0]) + 256 * np.rint(out[0, :, :, 1])
    expect = (np.arange(S)[:, None] - rstar.numpy().T)
    assert np.array_equal(dec, expect)
    assert np.array_equal(np.rint(out[0, :, :, 2]), np.repeat((np.arange(Hq) // (Hq // Hkv))[None, :], S, 0))


@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("E,S", [(128, 400), (100, 333)])
def test_index_probe_at_the_extent_edge(E, S, pdt):
    """The peak at distances E-1 .. E-3 (by head) for every row that reaches them, the last row
    of each (batch row, head) profile block included: the entries next to the block's end and
    to the next row's, where a 16-byte run of the strip reaches past the row."""
    B, Hq, Hkv, D = 1, 6, 2, 128
    x = W.custom(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, E=E, seed=130, profiles_dtype=pdt)
    x["q"].zero_()
    x["k"].zero_()
    x["sink"].fill_(-math.inf)
    n_i = torch.arange(S)[None, :] + 1
    h_idx = torch.arange(Hq)[:, None]
    rstar = torch.clamp(torch.minimum(n_i, torch.tensor(E)) - 1 - (h_idx % 3), min=0)
    prof = torch.full((B, Hq, S, E), -30000.0)
    prof[0].scatter_(2, rstar[..., None], 40.0)
    x["profiles"] = prof.to(pdt)
    v = torch.zeros(B, S, Hkv, D)
    j = torch.arange(S, dtype=torch.float32)
    v[0, :, :, 0] = (j % 256)[:, None]
    v[0, :, :, 1] = (j // 256)[:, None]
    x["v"] = v.to(torch.bfloat16)
    announce(f"index probe at the extent edge: E={E} S={S} profiles={pdt}")
    out, _ = run_hip(x)
    dec = np.rint(out[0, :, :, 0]) + 256 * np.rint(out[0, :, :, 1])
    assert np.array_equal(dec, np.arange(S)[:, None] - rstar.numpy().T)


def test_garbage_at_invalid_tokens():
    x = W.custom(B=2, S=260, Hq=8, Hkv=2, D=128, E=50, seed=121, structure="tail_pad", max_tail_pad=60,
                 window=100)
    inv = ~x["valid"]
    g = torch.Generator().manual_seed(9)
    for name in ("q", "k", "v"):
        t = x[name]
        t[inv] = ((torch.rand(t[inv].shape, generator=g) - 0.5) * 2e4).to(t.dtype)
    x["profiles"].permute(0, 2, 1, 3)[inv] = 1e4
    x["sink"][inv] = 5e3
    out, lse, _ = check_full(x, "garbage_invalid")
    np.testing.assert_array_equal(lse[inv.numpy()], x["sink"].double().numpy()[inv.numpy()])


@pytest.mark.parametrize("sink", [-math.inf, 30.0, -30.0])
def test_sink_extremes(sink):
    x = W.custom(B=1, S=257, Hq=4, Hkv=1, D=128, E=64, seed=122, structure="tail_pad", max_tail_pad=20)
    x["sink"].fill_(sink)
    check_full(x, f"sink={sink}")


@pytest.mark.parametrize("growth,sink,D,pdt", [(6.0, None, 128, torch.float32), (6.0, -math.inf, 128, torch.float32),
                                               (-0.8, None, 128, torch.float32), (10.0, 3.0, 128, torch.float32),
                                               (8.0, -math.inf, 64, torch.bfloat16)],
                         ids=["rising", "rising_no_sink", "falling", "steep_sink3", "rising_no_sink_D64_bf16"])
def test_softmax_frame_moves_within_rows(growth, sink, D, pdt):
    # Logit scale that changes along the keys: the fp16 weights of later tiles
    # leave the range of the frame set by earlier ones (rising), or fall far
    # below it (falling), so the frame has to move in the middle of rows.
    x = W.custom(B=2, S=700, Hq=8, Hkv=2, D=D, E=90, seed=125, structure="tail_pad", max_tail_pad=50,
                 window=500 if growth > 9 else None, profiles_dtype=pdt)
    S = x["k"].shape[1]
    f = 1.0 + growth * torch.arange(S, dtype=torch.float32) / S
    x["k"] = (x["k"].float() * f[None, :, None, None]).to(torch.bfloat16)
    if sink is not None:
        x["sink"].fill_(sink)
    check_full(x, f"frame growth={growth} sink={sink}")


def test_all_invalid_and_empty_keys():
    x = W.custom(B=1, S=130, Hq=4, Hkv=2, D=64, E=8, seed=123)
    x["valid"].zero_()
    out, lse, _ = check_full(x, "all_invalid")
    assert np.all(out == 0)
    # no keys at all (context-parallel call with an empty key range)
    y = dict(x)
    y["valid"] = torch.ones_like(x["valid"])
    y["k"] = x["k"][:, :0].contiguous()
    y["v"] = x["v"][:, :0].contiguous()
    y["key_valid"] = torch.ones(1, 0, dtype=torch.bool)
    y["key_positions"] = torch.zeros(1, 0, dtype=torch.int32)
    y["query_offset"] = 64
    announce("empty key range: attn_fwd Sk=0")
    out, lse = run_hip(y)
    assert np.all(out == 0)
    np.testing.assert_allclose(lse, y["sink"].double().numpy(), atol=1e-5, rtol=0)


def test_zero_rows_is_a_no_op():
    x = W.custom(B=1, S=4, Hq=4, Hkv=2, D=128, E=8, seed=124)
    d = to_device(x)
    q = d["q"][:, :0].contiguous()
    announce("B*Sq == 0: attn_fwd")
    out, lse = binding.attn_fwd(q, d["k"], d["v"], d["profiles"][:, :, :0].contiguous(), d["sink"][:, :0].contiguous(),
                                d["valid"][:, :0].contiguous(), key_valid=d["valid"], key_positions=d["positions"],
                                query_offset=4)
    torch.cuda.synchronize()
    assert out.numel() == 0 and lse.numel() == 0


def test_query_slice_with_offset():
    """Context-parallel contract on one GPU: local queries [a, a+n) against global keys."""
    x = W.custom(B=2, S=500, Hq=8, Hkv=2, D=128, E=90, seed=125, structure="packed", doc_min=40,
                 doc_max=220, invalid_tail=9, window=150)
    full_out, full_lse, _ = check_full(x, "cp_full")
    a, n = 161, 211
    y = dict(q=x["q"][:, a:a + n].contiguous(), k=x["k"], v=x["v"],
             profiles=x["profiles"][:, :, a:a + n].contiguous(), sink=x["sink"][:, a:a + n].contiguous(),
             valid=x["valid"][:, a:a + n].contiguous(), key_valid=x["valid"],
             positions=x["positions"][:, a:a + n].contiguous(), key_positions=x["positions"],
             window=150, query_offset=a)
    out, lse, _ = check_full(y, "cp_slice")
    np.testing.assert_allclose(out, full_out[:, a:a + n], atol=1e-6, rtol=0)
    np.testing.assert_allclose(lse, full_lse[:, a:a + n], atol=1e-6, rtol=0)


@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("a", [31, 63, 95, 130])
def test_query_slice_first_rows_bias(a, pdt):
    """A query slice starting just past a key tile: the first local rows read
    profile runs that start at distance 0..3 of their row, in the first row of
    the profile block."""
    n = 70
    x = W.custom(B=1, S=a + n, Hq=4, Hkv=1, D=128, E=200, seed=126, profiles_dtype=pdt)
    y = dict(q=x["q"][:, a:].contiguous(), k=x["k"], v=x["v"],
             profiles=x["profiles"][:, :, a:].contiguous(), sink=x["sink"][:, a:].contiguous(),
             valid=x["valid"][:, a:].contiguous(), key_valid=x["valid"],
             positions=x["positions"][:, a:].contiguous(), key_positions=x["positions"],
             window=None, query_offset=a)
    check_full(y, f"cp_first_rows_{a}")


def test_debug_counts_and_tiles_match_oracle_mask():
    for name in ("packed_window", "tailpad_G4_D128", "G16_two_chunks", "window_G4_D64"):
        x = SMALL[name]()
        d = to_device(x)
        announce(f"debug counts/tiles: {name}")
        cnt = binding.attn_debug_counts(d["valid"], positions=d["positions"], window=x["window"]).cpu().numpy()
        tiles = binding.attn_debug_tiles(d["valid"], positions=d["positions"], window=x["window"]).cpu().numpy()
        torch.cuda.synchronize()
        ref_cnt, ref_mask = oracle.mask(x["valid"], positions=x["positions"], window=x["window"], full=True)
        assert np.array_equal(cnt, ref_cnt), name
        bm, bn = binding.attn_query_block(), binding.attn_key_tile()
        B, S = x["valid"].shape
        for b in range(B):
            for qb in range(tiles.shape[1]):
                for kt in range(tiles.shape[2]):
                    blk = ref_mask[b, qb * bm:(qb + 1) * bm, kt * bn:(kt + 1) * bn]
                    c = tiles[b, qb, kt]
                    if c == 0:
                        assert not blk.any(), f"{name}: skipped tile ({b},{qb},{kt}) holds allowed pairs"
                    if c == 2:
                        assert blk.shape == (bm, bn) and blk.all(), f"{name}: full tile ({b},{qb},{kt}) masked"


# ------------------------------------------------------------------------------------------
# full-size workloads (the benchmark's launch configuration)
# ------------------------------------------------------------------------------------------
WHOLE = ["causal_gqa", "local", "full_causal_8k", "packed"]


@pytest.mark.parametrize("name", WHOLE)
def test_full_size_whole_output_and_counts(name):
    """Every element of out and lse at full size against the oracle over all rows."""
    x = W.generate(W.WORKLOADS[name])
    d = to_device(x)
    announce(f"{name}: attn_fwd full size, whole output against the oracle")
    out, lse = run_hip(x, d=d)
    ref_out, ref_lse, ref_cnt = run_oracle(x)
    assert_close(out, lse, ref_out, ref_lse, ref_cnt, name)
    del out, ref_out
    announce(f"{name}: attn_debug_counts all rows")
    cnt = binding.attn_debug_counts(d["valid"], positions=d["positions"], window=x["window"]).cpu().numpy()
    assert np.array_equal(cnt, ref_cnt)


def test_long_rows_with_every_sink_dominated_row():
    """long (S = 32768, 64 heads, bf16 profiles, sink std 2): the first 1024 rows, every row where
    some head's sink weight is at least the content's (e^s >= sum e^z, read off the GPU's lse),
    and 1024 random rows beyond, against the oracle."""
    x = W.generate(W.WORKLOADS["long"])
    w = x["workload"]
    d = to_device(x)
    announce("long: attn_fwd full size")
    out, lse = run_hip(x, d=d)
    sig = x["sink"].double().numpy()[0]
    dominated = np.nonzero(np.any(sig >= lse[0] - math.log(2.0) - 1e-3, axis=1))[0]
    g = np.random.default_rng(5)
    rest = g.choice(np.arange(1024, w.S), size=1024, replace=False)
    rows = np.unique(np.concatenate([np.arange(1024), dominated, rest, [w.S - 1]]))
    assert rows.size >= 2048
    announce(f"long: oracle on {rows.size} rows ({dominated.size} with a dominating sink)")
    ref_out, ref_lse, ref_cnt = run_oracle(x, rows=torch.from_numpy(rows))
    assert_close(out[0, rows], lse[0, rows], ref_out, ref_lse, np.repeat(ref_cnt[:, None], w.Hq, axis=1), "long")
    # the sample holds sink-dominated entries by the oracle's own lse, and the GPU flagged all of them
    ref_dom = sig[rows] >= ref_lse - math.log(2.0)
    assert ref_dom.sum() > 100
    assert np.all(np.isin(rows[np.any(ref_dom, axis=1)], dominated))


def test_key_tiles_beyond_one_schedule_round():
    """More than 512 key tiles: the workgroup's tile schedule is built in
    several rounds; rows near the end read tiles of both."""
    S = 33000
    x = W.custom(B=1, S=S, Hq=8, Hkv=1, D=64, E=48, seed=127)
    rows = W.sample_rows(1, S, 20, 127, must=((0, 0), (0, 32767), (0, 32768), (0, 32831), (0, S - 1)))
    check_rows(x, rows, "two_schedule_rounds")
    y = count_probe_inputs(x)
    out, lse = run_hip(y)
    cnt = counts_from_lse(lse)
    assert np.array_equal(cnt[0, :, 0], np.arange(1, S + 1))


@pytest.mark.parametrize("name", ["local", "packed", "causal_gqa", "full_causal_8k", "long"])
def test_full_size_count_probe(name):
    """lse = ln(n_allowed) for every row and head at full size: the hot path's mask is exact."""
    x = count_probe_inputs(W.generate(W.WORKLOADS[name]))
    announce(f"{name}: count probe attn_fwd full size")
    _, lse = run_hip(x)
    ref = oracle.mask(x["valid"], positions=x["positions"], window=x["window"])
    got = counts_from_lse(lse)
    assert np.array_equal(got, np.repeat(ref[..., None], got.shape[-1], axis=-1))
