"""The plan mirror against a hand-worked plan and against invariants any
correct plan must satisfy (every row covered once, chunks partition each
adapter, extension steps cover exactly the adapters meeting each tile)."""
import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.plan_mirror import build_plan, PlanOpts

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_hand_worked_plan():
    with open(os.path.join(GOLDEN, "plan_hand.json")) as f:
        g = json.load(f)
    p = build_plan(g["offsets"], g["ranks"], PlanOpts(**g["opts"]))
    for k, v in g["expect"].items():
        got = p[k]
        if isinstance(got, np.ndarray):
            assert np.array_equal(got, np.asarray(v, dtype=got.dtype).reshape(got.shape)), (k, got, v)
        else:
            assert got == v, (k, got, v)


def check_invariants(offsets, ranks, opts, p):
    o = [int(x) for x in offsets]
    n = len(ranks)
    T = o[-1]
    rpad = p["rpad"]
    for i, r in enumerate(ranks):
        assert rpad[i] >= max(32, r) and (rpad[i] & (rpad[i] - 1)) == 0 and rpad[i] < 2 * max(32, r)
    g = p["group_first_adapter"]
    assert g[0] == 0 and g[-1] == n and all(g[k] <= g[k + 1] for k in range(len(g) - 1))
    # nano-batches: each row of each adapter exactly once, pieces <= NB, within a group
    cover = np.zeros(T, dtype=np.int64)
    for (a, r0, m) in p["nb"]:
        assert 1 <= m <= opts.nano_rows and o[a] <= r0 and r0 + m <= o[a + 1]
        cover[r0:r0 + m] += 1
    assert np.all(cover == 1)
    for s in range(p["n_groups"]):
        for (a, _, _) in p["nb"][p["nb_start"][s]:p["nb_start"][s + 1]]:
            assert g[s] <= a < g[s + 1]
    # chunks partition each adapter, in row order, consecutive per adapter
    for i in range(n):
        f, c = p["adapter_chunk_first"][i], p["adapter_chunk_count"][i]
        rows = [(r0, m) for (a, r0, m) in p["chunks"][f:f + c]]
        assert all(a == i for (a, _, _) in p["chunks"][f:f + c])
        pos = o[i]
        for r0, m in rows:
            assert r0 == pos and m >= 1
            pos += m
        assert pos == o[i + 1]
    cp = 0
    for k, (a, _, _) in enumerate(p["chunks"]):
        assert p["chunk_rpref"][k] == cp
        cp += rpad[a]
    assert cp == p["partial_rows"]
    # tiles cover [0, T) once; extension entries = adapters meeting the tile
    cover = np.zeros(T, dtype=np.int64)
    for t, (r0, m) in enumerate(p["tiles"]):
        assert 1 <= m <= opts.gemm_rows
        cover[r0:r0 + m] += 1
        want = []
        for j in range(n):
            lo, hi = max(o[j], r0), min(o[j + 1], r0 + m)
            if lo < hi:
                want += [(j, lo, hi, k0) for k0 in range(0, int(rpad[j]), 32)]
        got = [tuple(e) for e in p["ext"][p["tile_ext_start"][t]:p["tile_ext_start"][t + 1]]]
        assert got == want
    assert np.all(cover == 1)
    # offsets
    z = 0
    for i in range(n):
        assert p["zoff"][i] == z
        z += (o[i + 1] - o[i]) * rpad[i]
    assert z == p["z_elems"]


@st.composite
def plan_inputs(draw):
    n = draw(st.integers(1, 24))
    toks = draw(st.lists(st.integers(0, 700), min_size=n, max_size=n))
    ranks = draw(st.lists(st.integers(1, 256), min_size=n, max_size=n))
    nb = draw(st.sampled_from([16, 32, 64]))
    bm = draw(st.sampled_from([128, 256]))
    S = draw(st.integers(1, 5))
    off = [0]
    for t in toks:
        off.append(off[-1] + t)
    return off, ranks, PlanOpts(nano_rows=nb, gemm_rows=bm, n_streams=S)


@settings(max_examples=150, deadline=None)
@given(plan_inputs())
def test_plan_invariants(args):
    off, ranks, opts = args
    p = build_plan(off, ranks, opts)
    check_invariants(off, ranks, opts, p)
