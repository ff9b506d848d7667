"""Pins of the plan mirror (oracle/plan_mirror.py) against facts other than
itself: plans worked by hand (one projection; two projections sharing the
input; rows given as per-token ids), split-K factors worked by hand, and
invariants every correct plan has, over seeded random layers with one to
four projections.  Each pin takes the mirror module, so a copy with a
planted mistake can be run through the same pins."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _expect(p, g):
    for k, v in g["expect"].items():
        got = p[k]
        if isinstance(got, np.ndarray):
            assert np.array_equal(got, np.asarray(v, dtype=got.dtype).reshape(got.shape)), (k, got, v)
        else:
            assert got == v, (k, got, v)


def check_invariants(m, offsets, ranks, opts, p, widths=None):
    """Properties every correct plan has, over (adapter, projection) pairs
    v = i P + q (P = 1: the adapters).  ``ranks`` is [n] or, with widths,
    [n][P]."""
    o = [int(x) for x in offsets]
    n = len(o) - 1
    P = 1 if widths is None else len(widths)
    wd = [1] if widths is None else [int(x) for x in widths]
    rk = [int(r) for r in ranks] if widths is None else [int(ranks[i][q]) for i in range(n) for q in range(P)]
    nv = n * P
    T = o[-1]
    rpad = p["rpad"]
    assert len(rpad) == nv
    for v, r in enumerate(rk):
        assert rpad[v] >= max(32, r) and (rpad[v] & (rpad[v] - 1)) == 0 and rpad[v] < 2 * max(32, r)
    g = p["group_first_adapter"]
    assert g[0] == 0 and g[-1] == n and all(g[k] <= g[k + 1] for k in range(len(g) - 1))
    assert p["n_groups"] == min(opts.n_streams, n)
    # groups: boundary s is the first adapter starting at or after ceil(s T / S')
    S = p["n_groups"]
    for s in range(1, S):
        target = -(-(s * T) // S)
        first = next((j for j in range(n) if o[j] >= target), n)
        assert g[s] == max(g[s - 1], first)
    # nano-batches: per projection every row exactly once; each pair's rows in
    # order, in pieces of exactly NB rows but the last
    cover = np.zeros((P, T), dtype=np.int64)
    per_pair = {}
    NB = opts.nano_rows or p["nano_rows"]
    assert p["nano_rows"] == NB
    for (v, r0, mm) in p["nb"]:
        i = v // P
        assert 1 <= mm <= NB and o[i] <= r0 and r0 + mm <= o[i + 1]
        cover[v % P, r0:r0 + mm] += 1
        per_pair.setdefault(int(v), []).append((int(r0), int(mm)))
    assert np.all(cover == 1)
    for v, pieces in per_pair.items():
        pos = o[v // P]
        for k, (r0, mm) in enumerate(pieces):
            assert r0 == pos and (mm == NB or k == len(pieces) - 1)
            pos += mm
    for s in range(S):
        seen = [int(v) for (v, _, _) in p["nb"][p["nb_start"][s]:p["nb_start"][s + 1]]]
        for v in seen:
            assert g[s] <= v // P < g[s + 1]
        # bucket order inside a group: r_pad descending, then projection, then adapter
        keys = [(-int(rpad[v]), v % P, v // P) for v in seen]
        assert keys == sorted(keys)
    # chunks partition each pair's rows in pieces of exactly KC but the last,
    # consecutive per pair, pairs in the nano-batch walk order
    order = []
    for v in range(nv):
        i = v // P
        f, c = p["adapter_chunk_first"][v], p["adapter_chunk_count"][v]
        assert all(a == v for (a, _, _) in p["chunks"][f:f + c])
        pos = o[i]
        kc = min(opts.chunk_max, max(opts.chunk_min, opts.chunk_per_rank * int(rpad[v])))
        for k, (_, r0, mm) in enumerate(p["chunks"][f:f + c]):
            assert r0 == pos and (mm == kc or (k == c - 1 and 1 <= mm <= kc))
            pos += mm
        assert pos == o[i + 1]
    walk = []
    for (v, _, _) in p["chunks"]:
        if not walk or walk[-1] != int(v):
            walk.append(int(v))
    assert walk == [v for v in dict.fromkeys(int(x) for (x, _, _) in p["nb"])]
    cp = cb = 0
    for k, (v, _, _) in enumerate(p["chunks"]):
        assert p["chunk_rpref"][k] == cp and p["chunk_boff"][k] == cb
        cp += int(rpad[v])
        cb += int(rpad[v]) * wd[v % P]
    assert cp == p["partial_rows"] and cb == p["partial_b_elems"]
    # tiles: BM-row tiles from row 0 over every row, in order; group s takes
    # a contiguous run whose rows all belong to groups <= s, each boundary the
    # largest multiple of G tiles (16 with at least 32 tiles per group, else
    # 1) ending at or before the next group's first row, never below the
    # previous boundary
    BM = opts.gemm_rows
    M = -(-T // BM)
    assert [tuple(int(x) for x in t) for t in p["tiles"]] == [(k * BM, min(BM, T - k * BM)) for k in range(M)]
    ts = [int(x) for x in p["tile_start"]]
    assert len(ts) == S + 1 and ts[0] == 0 and ts[S] == M
    G = 16 if M >= 32 * S else 1
    for s in range(1, S):
        fits = [k for k in range(0, M + 1, G) if k * BM <= o[g[s]]]
        assert ts[s] == max(ts[s - 1], max(fits))
        assert ts[s] * BM <= o[g[s]]
    # extension entries per (tile, projection) are exactly the pairs of that
    # projection meeting the tile, adapters ascending, k0 = 0, 32, .. < r_pad
    es = p["tile_ext_start"]
    assert len(es) == len(p["tiles"]) * P + 1
    for t, (r0, mm) in enumerate(p["tiles"]):
        for q in range(P):
            want = []
            for j in range(n):
                lo, hi = max(o[j], r0), min(o[j + 1], r0 + mm)
                if lo < hi:
                    want += [(j * P + q, lo, hi, k0) for k0 in range(0, int(rpad[j * P + q]), 32)]
            got = [tuple(int(x) for x in e) for e in p["ext"][es[t * P + q]:es[t * P + q + 1]]]
            assert got == want
    # offsets into Z' and the rank-padded concatenations, pairs in index order
    z = rr = 0
    for v in range(nv):
        assert p["zoff"][v] == z and p["roff"][v] == rr and p["seg_start"][v] == o[v // P]
        z += (o[v // P + 1] - o[v // P]) * int(rpad[v])
        rr += int(rpad[v])
    assert z == p["z_elems"] and rr == p["rpad_total"]


def pin_hand_single(m):
    """One projection, two groups, an empty adapter (tests/golden/plan_hand.json)."""
    g = _load("plan_hand.json")
    p = m.build_plan(g["offsets"], g["ranks"], m.PlanOpts(**g["opts"]))
    _expect(p, g)


def pin_hand_multi(m):
    """Two projections sharing the input (tests/golden/plan_multi_hand.json)."""
    g = _load("plan_multi_hand.json")
    p = m.build_plan(g["offsets"], g["ranks"], m.PlanOpts(**g["opts"]), widths=g["widths"],
                     dims=(g["d_in"], sum(g["widths"]), g["dtype"]))
    _expect(p, g)


def pin_hand_ids(m):
    """Rows as per-token ids: counting sort and permutation (tests/golden/plan_ids_hand.json)."""
    g = _load("plan_ids_hand.json")
    p = m.build_plan_from_ids(g["ids"], g["ranks"], m.PlanOpts(**g["opts"]),
                              dims=(g["d_in"], g["d_out"], g["dtype"]))
    _expect(p, g)


def pin_group_tiles_by_hand(m):
    """Rule 7's group boundaries on layers worked by hand."""
    # 65536 rows, four groups: 256 tiles >= 32 x 4, so boundaries are multiples
    # of 16 tiles.  Groups start at adapters 1, 2, 3 (rows 20000, 40000,
    # 50000 >= 16384, 32768, 49152); floor(row / 256) = 78, 156, 195, rounded
    # down to 64, 144, 192.
    p = m.build_plan([0, 20000, 40000, 50000, 65536], [8, 16, 32, 64], m.PlanOpts(n_streams=4))
    assert p["tile_start"].tolist() == [0, 64, 144, 192, 256]
    assert p["tiles"][78].tolist() == [19968, 256] and p["tiles"][255].tolist() == [65280, 256]
    # tile 78 (group 1's run) holds adapter 0's last 32 rows and adapter 1's first 224
    e0, e1 = p["tile_ext_start"][78], p["tile_ext_start"][79]
    assert p["ext"][e0:e1].tolist() == [[0, 19968, 20000, 0], [1, 20000, 20224, 0]]
    # 1000 rows, two groups: 4 tiles < 64, boundaries not rounded; group 1 starts
    # at row 600, floor(600 / 256) = 2, so tile 2 (rows 512..767, both adapters) is group 1's
    p = m.build_plan([0, 600, 1000], [8, 8], m.PlanOpts(n_streams=2))
    assert p["tile_start"].tolist() == [0, 2, 4]
    assert p["tiles"].tolist() == [[0, 256], [256, 256], [512, 256], [768, 232]]
    e0, e1 = p["tile_ext_start"][2], p["tile_ext_start"][3]
    assert p["ext"][e0:e1].tolist() == [[0, 512, 600, 0], [1, 600, 768, 0]]
    # the threshold: 16384 rows make 64 tiles = 32 x 2 (rounded: floor(9000 / 256) = 35 -> 32);
    # 16128 rows make 63 (not rounded: 35)
    assert m.build_plan([0, 9000, 16384], [8, 8], m.PlanOpts(n_streams=2))["tile_start"].tolist() == [0, 32, 64]
    assert m.build_plan([0, 9000, 16128], [8, 8], m.PlanOpts(n_streams=2))["tile_start"].tolist() == [0, 35, 63]


def pin_ids_definition(m):
    """A plan from ids groups each adapter's rows in the caller's order: perm
    is a permutation, grouped rows of adapter i are rows with id i, ascending."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        n = int(rng.integers(1, 9))
        ids = rng.integers(0, n, size=int(rng.integers(0, 300)))
        p = m.build_plan_from_ids(ids, [8] * n, m.PlanOpts())
        o, perm = p["offsets"], p["perm"]
        assert sorted(perm.tolist()) == list(range(len(ids)))
        for i in range(n):
            rows = perm[o[i]:o[i + 1]]
            assert len(rows) == int(np.sum(ids == i))
            assert np.all(ids[rows] == i) and np.all(np.diff(rows) > 0)


def pin_default_nano_rows_by_hand(m):
    """Rule 5's default nano-batch size, at the thresholds, worked by hand."""
    for T, want in ((65536, 128), (65535, 64), (32768, 64), (32767, 32), (7680, 32), (0, 32)):
        p = m.build_plan([0, T // 2, T], [8, 16], m.PlanOpts())
        assert p["nano_rows"] == want, (T, p["nano_rows"], want)
    # three projections over 22000 rows cover 66000 rows of pairs: 128; two over 16384 rows: 64 (32768)
    p = m.build_plan([0, 11000, 22000], [[8, 8, 8], [16, 16, 16]], m.PlanOpts(), widths=[256, 256, 256])
    assert p["nano_rows"] == 128
    p = m.build_plan([0, 8192, 16384], [[8, 8], [16, 16]], m.PlanOpts(), widths=[256, 256])
    assert p["nano_rows"] == 64
    # the 70B MLP pair's 65536 rows: 128-row pieces, the last of each adapter partial
    p = m.build_plan([0, 300, 65536], [64, 128], m.PlanOpts())
    assert [tuple(x) for x in p["nb"][:3]] == [(1, 300, 128), (1, 428, 128), (1, 556, 128)]
    assert tuple(p["nb"][-1]) == (0, 256, 44)
    # an explicit size overrides the default
    assert m.build_plan([0, 300, 65536], [64, 128], m.PlanOpts(nano_rows=32))["nano_rows"] == 32


def pin_split_k_by_hand(m):
    """Rule 9 on launches worked by hand."""
    # 16 tiles, 64 K-steps: min(16, 8, 16) = 8, kper 8 -> 8
    assert m.split_k(16, 64) == 8
    # 10 tiles, 130 K-steps: min(25, 16, 16) = 16, kper = ceil(130/16) = 9 -> ceil(130/9) = 15
    assert m.split_k(10, 130) == 15
    # 17 tiles, 80 K-steps: min(15, 10, 16) = 10, kper 8 -> 10
    assert m.split_k(17, 80) == 10
    # 64 tiles, 16 K-steps: min(4, 2, 16) = 2
    assert m.split_k(64, 16) == 2
    # 128 tiles or more, or fewer than 16 K-steps: no split
    assert m.split_k(128, 512) == 1 and m.split_k(4, 15) == 1
    # 112 tiles, 112 K-steps: min(2, 14, 16) = 2
    assert m.split_k(112, 112) == 2


def pin_invariants_random(m):
    """Invariants over seeded random layers: one projection and one to four
    projections, empty adapters, one to five stream groups."""
    rng = np.random.default_rng(11)
    for case in range(60):
        n = int(rng.integers(1, 14))
        P = int(rng.integers(1, 5)) if case % 2 else 1
        toks = rng.integers(0, 600, size=n) * (rng.random(n) > 0.15)
        off = np.concatenate([[0], np.cumsum(toks)]).tolist()
        opts = m.PlanOpts(nano_rows=int(rng.choice([0, 16, 32, 64])), gemm_rows=int(rng.choice([128, 256])),
                          n_streams=int(rng.integers(1, 6)), chunk_min=int(rng.choice([16, 64, 256])),
                          chunk_max=0, chunk_per_rank=int(rng.choice([1, 8])))
        opts.chunk_max = opts.chunk_min * int(rng.choice([1, 4, 8]))
        if P == 1:
            ranks = rng.integers(1, 257, size=n).tolist()
            p = m.build_plan(off, ranks, opts)
            check_invariants(m, off, ranks, opts, p)
        else:
            ranks = rng.integers(1, 257, size=(n, P)).tolist()
            widths = rng.choice([256, 512, 768], size=P).tolist()
            p = m.build_plan(off, ranks, opts, widths=widths)
            check_invariants(m, off, ranks, opts, p, widths=widths)
    # layers large enough that the group boundaries round to 16 tiles
    for case in range(12):
        n = int(rng.integers(2, 20))
        toks = rng.integers(0, 12000, size=n)
        off = np.concatenate([[0], np.cumsum(toks)]).tolist()
        opts = m.PlanOpts(n_streams=int(rng.integers(2, 5)))
        ranks = rng.integers(1, 257, size=n).tolist()
        check_invariants(m, off, ranks, opts, m.build_plan(off, ranks, opts))


ALL_PINS = [pin_hand_single, pin_hand_multi, pin_hand_ids, pin_group_tiles_by_hand, pin_ids_definition,
            pin_split_k_by_hand, pin_default_nano_rows_by_hand, pin_invariants_random]
