"""GPU parity of the backward (``attn_bwd``) against the fp64 oracle (``oracle.attn_bwd``).

Tolerance, derived from the arithmetic of the HIP path: the products run in bf16
MFMA with fp32 accumulation, and dout, P and dz are rounded to bf16 (relative
error <= 2^-9 each) before they enter a product.  Each gradient entry is a sum
of terms that carry at most two such roundings, so its error is at most about
2^-8 times the sum of the absolute values of its terms; fp32 accumulation adds
at most n 2^-24 of the same sum (n <= 2^15 terms here).  The bar is therefore

    |gpu - oracle| <= 2^-7 * M

with M the oracle's magnitude of that entry (``magnitudes=True``: the sum of
absolute contributions).  bf16 profile gradients add half a bf16 unit in the
last place of the value (the output rounding).  Masks are exact: the oracle's
exact zeros of dprofiles (no key at that distance), of dq at rows that are not
real and of dk / dv at keys that are not real must be exact zeros.

The backward is given the oracle's out and lse (rounded to fp32), which isolates
it; one case feeds it the GPU forward's instead.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import announce
from transformer_attention_03_amd import binding
from transformer_attention_03_amd import workloads as W

pytestmark = pytest.mark.gpu

REL = 2.0 ** -7
NAMES = ("dq", "dk", "dv", "dprofiles", "dsink")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.load()
    yield


def _upstream(x, seed, with_dlse=True, Sq=None):
    g = torch.Generator().manual_seed(seed)
    B, S, Hq, D = x["q"].shape
    dout = torch.randn(B, S, Hq, D, generator=g, dtype=torch.float32)
    dlse = torch.randn(B, S, Hq, generator=g, dtype=torch.float32) if with_dlse else None
    return dout, dlse


def _okw(x):
    return dict(key_valid=x.get("key_valid"), positions=x.get("positions"), key_positions=x.get("key_positions"),
                window=x.get("window"), query_offset=x.get("query_offset", 0))


def _dev(t):
    return None if t is None else t.cuda()


def run_gpu_bwd(x, out, lse, dout, dlse):
    kw = _okw(x)
    g = binding.attn_bwd(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["profiles"].cuda(), x["sink"].cuda(),
                         x["valid"].cuda(), out.cuda(), lse.cuda(), dout.cuda(), _dev(dlse),
                         key_valid=_dev(kw["key_valid"]), positions=_dev(kw["positions"]),
                         key_positions=_dev(kw["key_positions"]), window=kw["window"],
                         query_offset=kw["query_offset"])
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in g]


def oracle_bwd(x, dout, dlse, row_lo=0, row_hi=0, magnitudes=False):
    return oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout.double(),
                           None if dlse is None else dlse.double(), row_lo=row_lo, row_hi=row_hi,
                           magnitudes=magnitudes, **_okw(x))


def oracle_fwd(x):
    out, lse, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], **_okw(x))
    return torch.from_numpy(out).float(), torch.from_numpy(lse).float()


def assert_grads_close(got, ref, mag, what, bf16_prof=False, sel=None):
    for n, a, r, m in zip(NAMES, got, ref, mag):
        if sel is not None and sel.get(n) is not None:
            a, r, m = a[sel[n]], r[sel[n]], m[sel[n]]
        bound = REL * m + 1e-30          # (+ fp32 underflow of weights below 2^-126)
        if n == "dprofiles" and bf16_prof:
            bound = bound + np.abs(r) * 2.0 ** -9
        err = np.abs(a - r)
        bad = ~(err <= bound)
        assert not bad.any(), (f"{what} {n}: {int(bad.sum())} entries off, first {np.argwhere(bad)[:3].tolist()}, "
                               f"max err {np.nanmax(err):.3g}, max err/M {np.nanmax(err / np.maximum(m, 1e-300)):.3g}")
        zero = (r == 0) & (m == 0)
        assert np.all(a[zero] == 0), f"{what} {n}: nonzero where no term exists"


SMALL = {
    "single_G4_D128": dict(B=1, S=300, Hq=8, Hkv=2, D=128, E=48, structure="single", seed=301),
    "packed_window_invalid": dict(B=2, S=260, Hq=8, Hkv=2, D=128, E=40, window=50, structure="packed",
                                  doc_min=20, doc_max=120, invalid_tail=9, seed=302),
    "window_G8": dict(B=1, S=200, Hq=16, Hkv=2, D=128, E=64, window=70, structure="single", seed=303),
    "tailpad_G1_D64": dict(B=2, S=170, Hq=3, Hkv=3, D=64, E=30, structure="tail_pad", max_tail_pad=40, seed=304),
    "bf16_profiles": dict(B=1, S=230, Hq=8, Hkv=2, D=128, E=100, structure="packed", doc_min=30, doc_max=150,
                          profiles_dtype=torch.bfloat16, sink_std=2.0, seed=305),
    "extent_1": dict(B=1, S=140, Hq=4, Hkv=1, D=128, E=1, structure="single", seed=306),
    "extent_beyond_S": dict(B=1, S=150, Hq=4, Hkv=2, D=64, E=400, structure="packed", doc_min=10, doc_max=90,
                            seed=307),
    "G2_D64_window": dict(B=1, S=333, Hq=4, Hkv=2, D=64, E=64, window=100, structure="single", seed=308),
    # 16 heads per K/V head: four head chunks per group in the dQ grid; G = 3:
    # one head per dQ unit, four query blocks per workgroup
    "G16_chunks": dict(B=1, S=180, Hq=16, Hkv=1, D=128, E=70, structure="single", seed=309),
    "G3_D64": dict(B=2, S=150, Hq=6, Hkv=2, D=64, E=40, window=60, structure="tail_pad", max_tail_pad=30,
                   seed=310),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_small_parity(name):
    c = dict(SMALL[name])
    x = W.custom(**c)
    dout, dlse = _upstream(x, c["seed"] + 1000, with_dlse=(name != "extent_1"))
    announce(f"bwd {name}: q={tuple(x['q'].shape)} E={c['E']}")
    out, lse = oracle_fwd(x)
    got = run_gpu_bwd(x, out, lse, dout, dlse)
    ref = oracle_bwd(x, dout, dlse)
    mag = oracle_bwd(x, dout, dlse, magnitudes=True)
    assert_grads_close(got, ref, mag, name, bf16_prof=x["profiles"].dtype == torch.bfloat16)


def test_bwd_garbage_at_invalid_tokens_stays_out():
    """Large finite garbage in q / k / v and NaN in dout at tokens that are not real reach no
    output (as for the forward, q / k / v at such tokens must be finite)."""
    c = dict(SMALL["packed_window_invalid"])
    x = W.custom(**c)
    dout, dlse = _upstream(x, 2302)
    out, lse = oracle_fwd(x)
    ref = oracle_bwd(x, dout, dlse)
    mag = oracle_bwd(x, dout, dlse, magnitudes=True)
    bad = ~x["valid"]
    y = dict(x)
    g = torch.Generator().manual_seed(2303)
    for n in ("q", "k", "v"):
        t = x[n].clone()
        t[bad] = (torch.randn(t[bad].shape, generator=g) * 3e4).to(t.dtype)
        y[n] = t
    dn = dout.clone()
    dn[bad] = float("nan")
    announce("bwd NaN at invalid tokens")
    got = run_gpu_bwd(y, out, lse, dn, dlse)
    assert_grads_close(got, ref, mag, "nan_invalid")


def test_bwd_query_slice_with_offset():
    """Queries are a slice [a, a + n) of the sequence (query_offset = a), keys the whole sequence."""
    c = dict(B=1, S=320, Hq=8, Hkv=2, D=128, E=64, structure="packed", doc_min=40, doc_max=200, seed=309)
    x = W.custom(**c)
    a, n = 97, 130
    y = dict(x)
    y["q"] = x["q"][:, a:a + n].contiguous()
    y["profiles"] = x["profiles"][:, :, a:a + n].contiguous()
    y["sink"] = x["sink"][:, a:a + n].contiguous()
    y["valid"] = x["valid"][:, a:a + n].contiguous()
    y["positions"] = x["positions"][:, a:a + n].contiguous()
    y["key_valid"] = x["valid"]
    y["key_positions"] = x["positions"]
    y["query_offset"] = a
    dout, dlse = _upstream(y, 2309)
    announce(f"bwd query slice a={a} n={n}")
    out, lse = oracle_fwd(y)
    got = run_gpu_bwd(y, out, lse, dout, dlse)
    ref = oracle_bwd(y, dout, dlse)
    mag = oracle_bwd(y, dout, dlse, magnitudes=True)
    assert_grads_close(got, ref, mag, "query_slice")


def test_bwd_fed_by_gpu_forward():
    c = dict(SMALL["single_G4_D128"])
    x = W.custom(**c)
    dout, dlse = _upstream(x, 2310)
    announce("bwd after the GPU forward")
    out, lse = binding.attn_fwd(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), x["profiles"].cuda(),
                                x["sink"].cuda(), x["valid"].cuda(), positions=x["positions"].cuda())
    got = run_gpu_bwd(x, out.cpu(), lse.cpu(), dout, dlse)
    ref = oracle_bwd(x, dout, dlse)
    mag = oracle_bwd(x, dout, dlse, magnitudes=True)
    assert_grads_close(got, ref, mag, "after_gpu_forward")


def test_bwd_no_keys_and_no_queries():
    """Sk = 0 keys: dq = 0, dprofiles = 0, dsink = dlse; B * Sq = 0: dk = dv = 0."""
    x = W.custom(B=1, S=40, Hq=4, Hkv=2, D=64, E=8, seed=310)
    dout, dlse = _upstream(x, 2311)
    q, sink, valid = x["q"].cuda(), x["sink"].cuda(), x["valid"].cuda()
    kz = torch.empty(1, 0, 2, 64, dtype=torch.bfloat16, device="cuda")
    kvz = torch.empty(1, 0, dtype=torch.bool, device="cuda")
    out = torch.zeros(1, 40, 4, 64, device="cuda")
    lse = sink.clone()
    announce("bwd Sk = 0")
    dq, dk, dv, dp, ds = binding.attn_bwd(q, kz, kz, x["profiles"].cuda(), sink, valid, out, lse, dout.cuda(),
                                          dlse.cuda(), key_valid=kvz, positions=x["positions"].cuda(),
                                          key_positions=torch.empty(1, 0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(dp == 0)
    torch.testing.assert_close(ds.cpu(), dlse, rtol=0, atol=0)
    announce("bwd Sq = 0")
    qz = torch.empty(1, 0, 4, 64, dtype=torch.bfloat16, device="cuda")
    k, v = x["k"].cuda(), x["v"].cuda()
    dk = torch.full((1, 40, 2, 64), 7.0, device="cuda")
    dv = torch.full((1, 40, 2, 64), 7.0, device="cuda")
    empty = torch.empty(1, 0, 4, device="cuda")
    binding.attn_bwd(qz, k, v, torch.empty(1, 4, 0, 8, device="cuda"), empty, torch.empty(1, 0, dtype=torch.bool,
                     device="cuda"), torch.empty(1, 0, 4, 64, device="cuda"), empty, torch.empty(1, 0, 4, 64,
                     device="cuda"), None, key_valid=valid, key_positions=x["positions"].cuda(),
                     grads=(torch.empty(1, 0, 4, 64, device="cuda"), dk, dv, torch.empty(1, 4, 0, 8, device="cuda"),
                            torch.empty(1, 0, 4, device="cuda")))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def _full_size_ranges(name):
    """Query-row ranges (lo, hi) of a full-size workload, each with the key range (klo, khi) whose
    keys no row outside [lo, hi) can see (None: rows only).  Within a range the oracle's dq,
    dprofiles and dsink are exact; dk and dv are exact on the key range."""
    w = W.WORKLOADS[name]
    S = w.S
    if name == "full_causal_8k":
        return w, [(0, 512, None), (S - 48, S, (S - 48, S))]
    if name == "local":
        # key j is seen by rows j .. j + window - 1
        lo, hi = 4000, 5100
        return w, [(0, 256, None), (lo, hi, (lo, hi - w.window + 1)), (S - 48, S, (S - 48, S))]
    if name == "long":
        return w, [(0, 256, None), (S - 16, S, (S - 16, S))]
    if name == "causal_gqa":
        return w, [(0, S, (0, S))]
    raise KeyError(name)


def _check_full_size(x, w, ranges, seed):
    S = w.S
    dout, dlse = _upstream(x, seed)
    d = {k: (x[k].cuda() if isinstance(x.get(k), torch.Tensor) else None) for k in ("q", "k", "v", "profiles",
                                                                                   "sink", "valid", "positions")}
    announce(f"bwd full size {w.name}: forward")
    out, lse = binding.attn_fwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"],
                                positions=d["positions"], window=w.window)
    # the tested rows take the oracle's out / lse, which isolates the backward
    for lo, hi, _ in ranges:
        rows = (torch.arange(w.B)[:, None] * S + torch.arange(lo, hi)[None, :]).reshape(-1)
        o_r, l_r, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"],
                                      positions=x["positions"], window=w.window, rows=rows)
        out[:, lo:hi] = torch.from_numpy(o_r).float().reshape(w.B, hi - lo, w.Hq, w.D).cuda()
        lse[:, lo:hi] = torch.from_numpy(l_r).float().reshape(w.B, hi - lo, w.Hq).cuda()
    announce(f"bwd full size {w.name}: backward")
    g = binding.attn_bwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"], out, lse, dout.cuda(),
                         dlse.cuda(), positions=d["positions"], window=w.window)
    torch.cuda.synchronize()
    bf16_prof = x["profiles"].dtype == torch.bfloat16
    for lo, hi, keys in ranges:
        announce(f"bwd full size {w.name}: oracle rows {lo}..{hi - 1}, keys {keys}")
        sl = {"dq": (slice(None), slice(lo, hi)), "dprofiles": (slice(None), slice(None), slice(lo, hi)),
              "dsink": (slice(None), slice(lo, hi))}
        if keys is not None:
            sl["dk"] = sl["dv"] = (slice(None), slice(keys[0], keys[1]))
        names = [n for n in NAMES if n in sl]
        pick = lambda arrs: [arrs[NAMES.index(n)][sl[n]] for n in names]     # noqa: E731
        got = [g[NAMES.index(n)][sl[n]].float().cpu().numpy().astype(np.float64) for n in names]
        ref = pick(oracle_bwd(x, dout, dlse, row_lo=lo, row_hi=hi))
        mag = pick(oracle_bwd(x, dout, dlse, row_lo=lo, row_hi=hi, magnitudes=True))
        for n, a, r, m in zip(names, got, ref, mag):
            bound = REL * m + 1e-30
            if n == "dprofiles" and bf16_prof:
                bound = bound + np.abs(r) * 2.0 ** -9
            err = np.abs(a - r)
            bad = ~(err <= bound)
            assert not bad.any(), (f"{w.name} rows {lo}..{hi - 1} {n}: {int(bad.sum())} entries off, first "
                                   f"{np.argwhere(bad)[:3].tolist()}, max err/M "
                                   f"{np.nanmax(err / np.maximum(m, 1e-300)):.3g}")
            zero = (r == 0) & (m == 0)
            assert np.all(a[zero] == 0), f"{w.name} rows {lo}..{hi - 1} {n}: nonzero where no term exists"
        del ref, mag


@pytest.mark.parametrize("name", ["full_causal_8k", "local", "long", "causal_gqa"])
def test_bwd_full_size_row_ranges(name):
    """The full-size workloads in the launch configuration the backward bench times: row ranges
    at the start, inside and at the end of the sequence (dq, dprofiles, dsink of every row in a
    range; dk, dv of the keys only that range's rows see) against the oracle.  causal_gqa is
    compared whole (both batch rows, every row and key)."""
    w, ranges = _full_size_ranges(name)
    x = W.generate(w)
    _check_full_size(x, w, ranges, 2400 + len(name))


def test_bwd_full_size_packed_documents():
    """Packed documents (S = 16384, positions reset per document, last 100 tokens not real): two
    short documents whole (every row and every key of each, which only its own rows see) and the
    last 160 rows and keys (across the tail that is not real)."""
    w = W.WORKLOADS["packed"]
    x = W.generate(w)
    st = list(x["doc_starts"][0]) + [w.S]
    docs = sorted(((st[n + 1] - st[n], st[n], st[n + 1]) for n in range(len(st) - 1)))[:2]
    ranges = [(a, b, (a, b)) for _, a, b in docs] + [(w.S - 160, w.S, (w.S - 160, w.S))]
    _check_full_size(x, w, ranges, 2500)
