"""GPU parity of spec_verify_attn against the CPU oracle (fp64).

Gate (per output row r = (b,t,h)): max_c |o - o_ref| / max_c |o_ref|
  <= 1e-3 for fp32 KV, <= 2e-2 for bf16 and E4M3 KV (E4M3 against the
  dequantised oracle).
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verify_attn_amd as sv
import workloads as W
from .gpu_helpers import TOL, oracle_attn, row_rel_err, run_attn, sample_rows, unit_rows, upload_attn

pytestmark = pytest.mark.gpu

SMALL = [
    # (seed, B, T, Hq, Hkv, d, lens, kv)
    (1, 1, 5, 4, 1, 64, [256], "f32"),
    (2, 3, 6, 32, 8, 128, [37, 400, 16], "bf16"),
    (3, 2, 5, 64, 8, 128, [1000, 77], "bf16"),          # T*G = 40 (three row tiles)
    (4, 2, 7, 64, 8, 128, [517, 7], "bf16"),            # T*G = 56, L_b = T
    (5, 2, 8, 32, 8, 128, [300, 129], "bf16"),          # T*G = 32
    (6, 3, 2, 8, 8, 64, [33, 64, 190], "bf16"),         # MHA (G=1), d=64
    (7, 2, 4, 64, 4, 64, [250, 31], "bf16"),            # T*G = 64 (maximum)
    (8, 2, 7, 64, 8, 128, [700, 45], "fp8"),
    (9, 2, 3, 16, 2, 64, [129, 100], "fp8"),
    (10, 2, 5, 8, 2, 64, [90, 300], "f32"),
    (11, 1, 1, 4, 4, 128, [1], "bf16"),                 # single query row, single key
    (12, 3, 6, 64, 8, 128, [333, 6, 1100], "fp8"),      # E4M3, T*G = 48: row halves of two and one tiles
    (13, 2, 16, 16, 4, 64, [500, 260], "fp8"),          # E4M3, d=64, T*G = 64
    (14, 2, 5, 64, 8, 128, [2100, 47], "fp8"),          # E4M3, T*G = 40: the second half's last tile is padding
    (15, 2, 4, 64, 8, 128, [613, 4], "fp8"),            # E4M3, T*G = 32: two row tiles, one wave per page
    # more than 64 rows per KV head (more than four row tiles): two waves per
    # page, each owning half the row tiles; with four tiles per wave the Q
    # operands wait in LDS
    (16, 2, 9, 64, 8, 128, [600, 40], "bf16"),          # T*G = 72: five row tiles
    (17, 2, 16, 64, 8, 128, [700, 30], "bf16"),         # T*G = 128: eight row tiles, Q in LDS
    (18, 3, 12, 64, 8, 128, [900, 12, 301], "bf16"),    # T*G = 96: six row tiles
    (19, 2, 14, 64, 8, 128, [513, 77], "fp8"),          # E4M3, T*G = 112: seven tiles (32x32 PV, Q in LDS)
    (20, 2, 16, 32, 4, 64, [400, 16], "bf16"),          # d=64, T*G = 128
    (21, 2, 10, 64, 8, 128, [1300, 90], "fp8"),         # E4M3, T*G = 80: five tiles (16x16 PV)
    (22, 2, 16, 64, 8, 128, [800, 100], "fp8"),         # E4M3, T*G = 128
    (23, 2, 11, 32, 4, 64, [333, 11], "fp8"),           # E4M3, d=64, T*G = 88
    (24, 2, 13, 64, 8, 128, [250, 140], "f32"),         # fp32 (vector ALU), T*G = 104
    # E4M3, d = 128, four row tiles (shared pages, 32x32 PV)
    (25, 3, 8, 16, 2, 128, [5000, 17, 1200], "fp8"),    # two KV heads, T*G = 64, ragged
    (26, 2, 7, 24, 3, 128, [900, 30], "fp8"),           # odd Hkv, T*G = 56
    (27, 1, 7, 64, 8, 128, [7], "fp8"),                 # one page: most page streams get none
]


# E4M3 with four row tiles under forced fixed splits: more splits than the
# merge requests at once, a split of one page per stream, and splits past
# the end of the short sequence, over a garbage-filled workspace.
@pytest.mark.parametrize("bps", [4, 8, 64])
def test_e4m3_four_tiles_forced_splits(bps):
    a = W.make_attn_from_lens(28, 2, 7, 64, 8, 128, [2600, 50], kv="fp8", extra_blocks=2)
    t = upload_attn(a)
    ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, bps),
                            torch.device("cuda", 0))
    ws.fill_(0xFF)
    out = run_attn(a, t, blocks_per_split=bps, ws=ws)
    err = _check(a, out)
    print("bps %d: max row rel err %.3e" % (bps, err))
    assert err <= TOL[a.kv_dtype]


def _check(a, out, rows=None):
    ref = oracle_attn(a, rows=rows)
    got = out.cpu().numpy().reshape(-1, a.d)
    if rows is not None:
        got = got[rows]
    err = row_rel_err(got, ref)
    bad = np.nonzero(~np.all(np.isfinite(got), axis=1))[0]
    assert bad.size == 0, "non-finite output rows %s" % bad[:8]
    return float(err.max())


@pytest.mark.parametrize("case", SMALL, ids=[str(c[0]) for c in SMALL])
def test_small_shapes_auto(case):
    seed, B, T, Hq, Hkv, d, lens, kv = case
    a = W.make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=3)
    out = run_attn(a)
    err = _check(a, out)
    print("case %d max row rel err %.3e" % (seed, err))
    assert err <= TOL[a.kv_dtype]


@pytest.mark.parametrize("case", [c for c in SMALL if c[7] != "f32"], ids=lambda c: str(c[0]))
def test_small_shapes_valu(case):
    seed, B, T, Hq, Hkv, d, lens, kv = case
    a = W.make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=1)
    out = run_attn(a, algo=sv.SV_ATTN_VALU)
    err = _check(a, out)
    assert err <= TOL[a.kv_dtype]


@pytest.mark.parametrize("bps", [8, 16, 24, 64])
def test_forced_splits_merge(bps):
    a = W.make_attn_from_lens(21, 3, 6, 32, 8, 128, [1500, 80, 999], kv="bf16")
    out = run_attn(a, blocks_per_split=bps)
    assert _check(a, out) <= TOL[a.kv_dtype]
    out_v = run_attn(a, algo=sv.SV_ATTN_VALU, blocks_per_split=bps)
    assert _check(a, out_v) <= TOL[a.kv_dtype]


# Many fixed splits: the merge variants that prefetch 16 or 32 splits' rows.
# bps=4 over 313 pages gives 79 splits (more than the 32 requested at once,
# and more than one statistic per lane); bps=16 gives 20 (the 32-split
# prefetch, partly empty).  The short sequence has 2 splits, so most of its
# prefetched slots are discarded (never written in this call: the workspace
# starts filled with 0xAB).  Every row is compared, for both kernels.
@pytest.mark.parametrize("bps", [4, 16])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_forced_many_splits_merge(bps, kv):
    a = W.make_attn_from_lens(24, 3, 6, 32, 8, 128, [5000, 80, 1500], kv=kv)
    t = upload_attn(a)
    for algo in (sv.SV_ATTN_AUTO, sv.SV_ATTN_VALU):
        ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, bps),
                                t["q"].device)
        ws.fill_(0xAB)
        out = run_attn(a, t, algo=algo, blocks_per_split=bps, ws=ws)
        err = _check(a, out)
        print("bps %d %s algo %d: max row rel err %.3e" % (bps, kv, algo, err))
        assert err <= TOL[a.kv_dtype]


def test_deterministic_and_workspace_reusable():
    # a workspace full of garbage must not matter: nothing in it is read before written
    a = W.make_attn_from_lens(22, 4, 5, 64, 8, 128, [2000, 33, 700, 1024], kv="bf16")
    t = upload_attn(a)
    ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, 16), t["q"].device)
    ws.fill_(0xAB)
    o1 = run_attn(a, t, blocks_per_split=16, ws=ws).clone()
    for _ in range(5):
        o2 = run_attn(a, t, blocks_per_split=16, ws=ws)
        assert torch.equal(o1, o2)


def test_physical_placement_is_invisible():
    a1 = W.make_attn_from_lens(23, 2, 5, 32, 8, 128, [300, 517], kv="bf16", identity_table=True)
    o1 = run_attn(a1).cpu()
    a2 = W.make_attn_from_lens(23, 2, 5, 32, 8, 128, [300, 517], kv="bf16", identity_table=True)
    rng = np.random.default_rng(1)
    perm = rng.permutation(a2.num_blocks)
    k2 = np.empty_like(a2.k_cache)
    v2 = np.empty_like(a2.v_cache)
    k2[perm] = a2.k_cache
    v2[perm] = a2.v_cache
    a2.k_cache, a2.v_cache = k2, v2
    a2.block_table = perm[a2.block_table].astype(np.int32)
    o2 = run_attn(a2).cpu()
    assert torch.equal(o1, o2)


def test_split_calls_back_to_back():
    """One workspace, filled with garbage first, serves calls with different
    split counts (and hence different partial-slot layouts) back to back,
    with and without waiting in between; every call must match the oracle and
    repeat bit for bit."""
    cases = [(41, [2000, 33, 700, 1024], 16), (42, [1500, 1499, 17], 24), (43, [900, 6, 300, 880], 8),
             (44, [4096] * 3, 0)]
    ins = [W.make_attn_from_lens(seed, len(lens), 6, 32, 8, 128, lens, kv="bf16") for seed, lens, _ in cases]
    ts = [upload_attn(a) for a in ins]
    need = max(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, bps) for a, (_, _, bps) in zip(ins, cases))
    ws = sv.alloc_workspace(need, ts[0]["q"].device)
    ws.fill_(0xAB)
    outs = []
    for rep in range(2):
        cur = []
        for a, t, (_, _, bps) in zip(ins, ts, cases):
            out = torch.full((a.B, a.T, a.Hq, a.d), float("nan"), dtype=torch.float32, device=t["q"].device)
            sv.spec_verify_attn(t["q"], t["k"], t["v"], t["table"], t["lens"], out, ws, kv_dtype=a.kv_dtype,
                                blocks_per_split=bps)
            cur.append(out)
            if rep == 1:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        outs.append(cur)
    for a, o0, o1 in zip(ins, outs[0], outs[1]):
        assert _check(a, o0) <= TOL[a.kv_dtype]
        assert torch.equal(o0, o1)


# E4M3 over long runs: runs of 512 pages give every page stream of 4 (or 8)
# waves 128 (64) pages, each with its own K and V page scales; shared pages
# (three row tiles) and own pages (one and two row tiles), both head sizes,
# a forced fixed split and balanced shares.
LONG_E4M3 = [(5, 64, 8, 128), (4, 32, 8, 128), (2, 16, 8, 128), (4, 32, 4, 64)]


@pytest.mark.parametrize("T,Hq,Hkv,d", LONG_E4M3, ids=["T%d-Hq%d-Hkv%d-d%d" % c for c in LONG_E4M3])
def test_e4m3_long_runs(T, Hq, Hkv, d):
    a = W.make_attn_from_lens(51, 2, T, Hq, Hkv, d, [9000, 8200], kv="fp8", extra_blocks=2)
    t = upload_attn(a)
    for bps in (512, -1):
        out = run_attn(a, t, blocks_per_split=bps)
        assert _check(a, out) <= TOL[a.kv_dtype], "blocks_per_split %d" % bps


# Every row count from four to eight row tiles per KV head (shared pages:
# for four tiles under balanced shares only; Q operands in LDS at seven and
# eight) for both head sizes and both low-precision storages, under balanced
# shares, a forced fixed split and the planner's choice.  Regression: under register pressure the compiler
# reloaded a spilled copy offset into an SGPR one instruction before the
# inline-assembly LDS copy that reads it, which needs five wait states in
# between; the copy then fetched the wrong key's V bytes (all rows wrong at
# d = 64 with eight tiles and at d = 128 E4M3 with five and six).
WIDE = [(kv, d, T) for kv in ("bf16", "fp8") for d in (64, 128) for T in (7, 8, 10, 12, 14, 16)]


@pytest.mark.parametrize("kv,d,T", WIDE, ids=["%s-d%d-T%d" % c for c in WIDE])
def test_wide_rows_every_split_mode(kv, d, T):
    Hq, Hkv = (32, 4) if d == 64 else (64, 8)
    a = W.make_attn_from_lens(20, 2, T, Hq, Hkv, d, [400, 16], kv=kv, extra_blocks=2)
    t = upload_attn(a)
    for bps in (-1, 4, 0):
        out = run_attn(a, t, blocks_per_split=bps)
        assert _check(a, out) <= TOL[a.kv_dtype], "blocks_per_split %d" % bps


# Full-size configurations in the launch configuration bench.py times (the
# planner's split).  c1, c2, c5a and c5b: every output row.  c3 and c4 (whose
# balanced shares cut units at arbitrary pages): at least one row of every
# (sequence, KV head) unit plus 384 sampled rows, and the covered units are
# asserted to be all of them.
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5a", "c5b"])
def test_config_full_size(name):
    a = W.make_attn(name, seed=0)
    out = run_attn(a)
    if name in ("c3", "c4"):
        rows, units = unit_rows(a, seed=1)
        assert len(units) == a.B * a.Hkv
        rows = np.union1d(rows, sample_rows(a, 384, seed=2))
    else:
        rows = None
    err = _check(a, out, rows)
    print("%s max row rel err %.3e over %s rows" % (name, err, "all" if rows is None else len(rows)))
    assert err <= TOL[a.kv_dtype]
    assert torch.isfinite(out).all()


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.integers(1, 17))
        if T * G > 64:
            continue
        B = int(rng.integers(1, 6))
        kv = str(rng.choice(["f32", "bf16", "fp8"]))
        lens = [int(rng.integers(T, 900)) for _ in range(B)]
        bps = int(rng.choice([0, 4, 8, 32]))
        out.append((len(out), B, T, Hkv * G, Hkv, d, lens, kv, bps))
    return out


RANDOM = _random_shapes(24, 2024)


def _random_wide_shapes(n, seed):
    """As _random_shapes, with 64 < T*G <= 128 (five to eight row tiles)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([8, 16]))
        T = int(rng.integers(1, 17))
        if not 64 < T * G <= 128:
            continue
        B = int(rng.integers(1, 5))
        kv = str(rng.choice(["f32", "bf16", "fp8"]))
        lens = [int(rng.integers(T, 900)) for _ in range(B)]
        bps = int(rng.choice([0, 4, 8, 32, -1])) if kv != "f32" else int(rng.choice([0, 8]))
        out.append((len(out), B, T, Hkv * G, Hkv, d, lens, kv, bps))
    return out


RANDOM_WIDE = _random_wide_shapes(12, 2026)


@pytest.mark.parametrize("case", RANDOM_WIDE, ids=[str(c[0]) for c in RANDOM_WIDE])
def test_random_wide_shapes(case):
    i, B, T, Hq, Hkv, d, lens, kv, bps = case
    a = W.make_attn_from_lens(900 + i, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    out = run_attn(a, blocks_per_split=bps)
    err = _check(a, out)
    assert err <= TOL[a.kv_dtype], (case, err)


@pytest.mark.parametrize("case", RANDOM, ids=[str(c[0]) for c in RANDOM])
def test_random_shapes(case):
    """Seeded random shapes: every GQA ratio and head count, 1 to 16 verify
    rows, ragged lengths, all storage types, forced context splits, both
    kernels (bf16/E4M3 also through the vector-ALU kernel)."""
    i, B, T, Hq, Hkv, d, lens, kv, bps = case
    a = W.make_attn_from_lens(500 + i, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    algos = [sv.SV_ATTN_AUTO] + ([sv.SV_ATTN_VALU] if kv != "f32" else [])
    for algo in algos:
        out = run_attn(a, algo=algo, blocks_per_split=bps)
        err = _check(a, out)
        assert err <= TOL[a.kv_dtype], (case, algo, err)


@pytest.mark.parametrize("case", [c for c in SMALL if c[7] != "f32"], ids=lambda c: str(c[0]))
def test_small_shapes_balanced(case):
    """Balanced shares (blocks_per_split = -1): the batch's (unit, page)
    pairs cut into equal runs, here of 4 pages, so units are split across
    many workgroups and workgroups span several units."""
    seed, B, T, Hq, Hkv, d, lens, kv = case
    a = W.make_attn_from_lens(seed, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    out = run_attn(a, blocks_per_split=-1)
    err = _check(a, out)
    assert err <= TOL[a.kv_dtype], (case, err)


@pytest.mark.parametrize("lens", [
    [5000, 16, 17, 5, 700, 9, 6, 33, 1200, 64, 65, 300],   # ragged: runs cross unit and sequence ends
    [4096] * 5,                                            # uniform: shares of whole splits
    [8, 3000, 8, 8, 8, 8, 8, 2500],                        # many one-page units inside one share
])
def test_balanced_shares_ragged(lens):
    a = W.make_attn_from_lens(31, len(lens), 5, 32, 8, 128, lens, kv="bf16", extra_blocks=2)
    out = run_attn(a, blocks_per_split=-1)
    err = _check(a, out)
    print("balanced lens %s: max row rel err %.3e" % (lens[:4], err))
    assert err <= TOL[a.kv_dtype]
    out_f = run_attn(a, blocks_per_split=16)
    assert _check(a, out_f) <= TOL[a.kv_dtype]


def test_balanced_shares_skip_empty_sequences():
    """A sequence without context holds no pairs: the shares skip it and the
    other sequences' rows are unaffected (its own rows are not written)."""
    lens = [300, 0, 900, 0, 0, 45]
    a = W.make_attn_from_lens(32, len(lens), 5, 32, 8, 128, [max(L, 5) for L in lens], kv="bf16", extra_blocks=2)
    keep = np.array([L > 0 for L in lens])
    ref_rows = np.arange(a.B * a.T * a.Hq).reshape(a.B, -1)[keep].ravel()
    t = upload_attn(a)
    t["lens"].copy_(torch.tensor(lens, dtype=torch.int32))
    out = run_attn(a, t, blocks_per_split=-1)
    err = _check(a, out, rows=ref_rows)
    assert err <= TOL[a.kv_dtype]


def test_balanced_shares_deterministic_with_garbage_workspace():
    a = W.make_attn_from_lens(33, 6, 6, 32, 8, 128, [2000, 33, 700, 1024, 6, 4000], kv="bf16")
    t = upload_attn(a)
    ws = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, -1), t["q"].device)
    ws.fill_(0xAB)
    o1 = run_attn(a, t, blocks_per_split=-1, ws=ws).clone()
    assert _check(a, o1) <= TOL[a.kv_dtype]
    for _ in range(3):
        o2 = run_attn(a, t, blocks_per_split=-1, ws=ws)
        assert torch.equal(o1, o2)


@pytest.mark.parametrize("B,T,Hq,d,kv", [(1000, 5, 16, 64, "bf16"), (1024, 5, 16, 64, "bf16"),
                                         (1024, 7, 64, 128, "fp8")])
def test_balanced_shares_many_sequences(B, T, Hq, d, kv):
    """Up to the 1024 sequences the balanced prefix sums hold: every thread
    of the workgroup carries four (8-wave E4M3 workgroups: two) sequences'
    page counts."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(T, 200, size=B)]
    a = W.make_attn_from_lens(34, B, T, Hq, 8, d, lens, kv=kv, extra_blocks=2)
    out = run_attn(a, blocks_per_split=-1)
    rows = sample_rows(a, 2048, seed=3)
    err = _check(a, out, rows)
    assert err <= TOL[a.kv_dtype]
    assert torch.isfinite(out).all()


def test_balanced_shares_capped_more_than_one_round():
    """More (sequence, KV head, page) pairs than 256 shares of the largest
    run an 8-wave workgroup holds (2048 pages): the shares are capped, the
    grid exceeds the compute units, and every unit (960 here, 2.4 GB of KV)
    is still covered once.  15 KV heads: no head groups (an odd head count
    runs one head per workgroup), so the pairs are (unit, page) pairs."""
    rng = np.random.default_rng(7)
    B, T, Hq, Hkv, d = 64, 2, 15, 15, 64
    lens = [int(x) for x in rng.integers(8000, 11000, size=B)]
    a = W.make_attn_from_lens(7, B, T, Hq, Hkv, d, lens, kv="bf16", extra_blocks=2)
    assert Hkv * sum((L + 15) // 16 for L in lens) > 256 * 2048
    t = upload_attn(a)
    rows, units = unit_rows(a, seed=3)
    assert len(units) == B * Hkv
    for bps in (-1, 0):
        out = run_attn(a, t, blocks_per_split=bps)
        assert _check(a, out, rows) <= TOL[a.kv_dtype], "blocks_per_split %d" % bps


# Head groups under balanced shares (at most two row tiles per KV head: the
# workgroup runs two heads side by side, a share cuts (group, page) pairs and
# a cut group's partials sit two slots apart).  Ragged lengths, so shares
# start and end inside groups; odd group counts (6 heads: 3 groups).
HGROUPS = [(2, 4, 8, 128, "bf16"), (4, 2, 8, 64, "fp8"), (6, 2, 16, 128, "bf16"), (8, 4, 8, 128, "bf16"),
           (8, 4, 8, 128, "fp8"), (12, 1, 7, 64, "bf16"), (16, 2, 5, 128, "fp8"), (8, 1, 1, 64, "bf16")]


@pytest.mark.parametrize("Hkv,G,T,d,kv", HGROUPS, ids=["Hkv%d-G%d-T%d-d%d-%s" % c for c in HGROUPS])
def test_head_groups_ragged(Hkv, G, T, d, kv):
    rng = np.random.default_rng(Hkv * 100 + G * 10 + T)
    B = 24
    lens = [int(x) for x in rng.integers(T, 2500, size=B - 3)] + [T, 16, 17]
    a = W.make_attn_from_lens(50 + Hkv, B, T, Hkv * G, Hkv, d, lens, kv=kv, extra_blocks=2)
    t = upload_attn(a)
    rows, units = unit_rows(a, seed=4)
    assert len(units) == B * Hkv
    for bps in (-1, 0):
        out = run_attn(a, t, blocks_per_split=bps)
        assert torch.isfinite(out).all()
        assert _check(a, out, rows) <= TOL[a.kv_dtype], "blocks_per_split %d" % bps


RANDOM_BAL = [c for c in _random_shapes(40, 2025) if c[7] != "f32"][:12]


@pytest.mark.parametrize("case", RANDOM_BAL, ids=[str(c[0]) for c in RANDOM_BAL])
def test_random_shapes_balanced(case):
    i, B, T, Hq, Hkv, d, lens, kv, _ = case
    a = W.make_attn_from_lens(700 + i, B, T, Hq, Hkv, d, lens, kv=kv, extra_blocks=2)
    out = run_attn(a, blocks_per_split=-1)
    err = _check(a, out)
    assert err <= TOL[a.kv_dtype], (case, err)
