"""Independent mirror of the plan rule -- TEST INFRASTRUCTURE ONLY.

The pages fix no plan: the tLoRA page (tLoRA: Efficient Multi-LoRA Training
with Elastic Shared Super-Models, abstract) says only that the fused kernel
re-forms low-rank tiles and schedules rank-aware nano-batches, and the PLoRA
page (§9.2) that adapters are concatenated and work is tiled along the token
and hidden axes, never along the rank.  The rule below is this library's own;
it is written down once (the library header states the same rule) and
re-implemented here in plain Python so the C++ builder can be checked bit for
bit.

Rule (all integers; counts and indexes int32, offsets into tensors int64):
 1. r_pad(i) = max(32, smallest power of two >= r_i); 1 <= r_i <= 256.
 2. zoff(i) = sum_{j<i} n_j r_pad(j);  roff(i) = sum_{j<i} r_pad(j).
 3. Stream groups: S' = min(S, n); g_0 = 0, g_S' = n; for 1 <= s < S',
    g_s = max(g_{s-1}, first adapter a with o_a >= ceil(s T / S'), else n).
 4. Within each group, adapters are visited by r_pad descending, then index
    ascending ("bucket order").
 5. Nano-batches: in bucket order, each adapter's rows cut into consecutive
    pieces of NB rows (last one partial; none when n_i = 0).  Entry
    (adapter, first row, rows).  NB given as 0 (the default) is chosen from
    the rows the nano-batches cover, T P (P projections): 128 when
    T P >= 65536, 64 when T P >= 32768, else 32.
 6. Reduction chunks: the same walk with KC_i = min(chunk_max, max(chunk_min,
    chunk_per_rank * r_pad(i))) rows per piece.  Entry (adapter, first row,
    rows); cpref(c) = sum of r_pad over earlier chunks.  Each adapter's chunks
    are consecutive: first(i), count(i) (first = total chunks before it in the
    walk order when count is 0 is still defined as the walk position).
 7. GEMM row tiles: rows [0, T) cut into tiles of BM rows from row 0 (the
    last one partial), M = ceil(T / BM) of them.  Group s takes tiles
    [a_s, a_{s+1}): a_0 = 0, a_S' = M, and for 1 <= s < S'
    a_s = max(a_{s-1}, G floor(floor(o_{g_s} / BM) / G)) with G = 16 when
    M >= 32 S', else 1.  For each tile, its extension steps: for every
    adapter j (ascending, whatever its group) whose rows meet the tile, for
    k0 = 0, 32, ... < r_pad(j): entry (j, lo, hi, k0) with [lo, hi) the rows
    of j inside the tile.
 8. Optimizer blocks: for every adapter i ascending, its trained tensors A_i
    (tensor 2i, d_in r_i elements) then B_i (tensor 2i+1, r_i d_out
    elements), each cut into consecutive pieces of OPT_BLOCK elements (last
    one partial).  Entry (tensor, piece).

 9. Split-K (bf16 only): a group's GEMM with t = (its row tiles) x ceil(N/256)
    output tiles and nk = K/32 K-steps (forward N = d_out, K = d_in; dX
    N = d_in, K = d_out) splits K into S parts when t < 128 and nk >= 16:
    S = min(floor(256/t), floor(nk/8), 16); then kper = ceil(nk/S) and
    S = ceil(nk/kper); S < 2 means 1.  Entry per group: (S_forward, S_dX).

Several projections sharing the input (widths d_0 .. d_{P-1}, ranks [n][P]):
every (adapter i, projection q) pair v = i P + q is planned as a unit over
adapter i's rows.  Rules 1, 2, 5, 6 and 8 run over pairs (B_v has d_q
columns); rule 3 stays over adapters; rule 4 orders a group's pairs by
r_pad descending, then projection, then adapter; rule 7 lists each tile's
steps projection by projection (tile_ext_start has n_tiles P + 1 entries),
pairs of one projection by adapter.  A chunk's dB partial sits at element
offset chunk_boff(c) = sum over earlier chunks of r_pad(v) d_q(v).  P = 1 is
the single-projection plan (v = i).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KSTEP = 32
OPT_BLOCK = 2048


@dataclass
class PlanOpts:
    nano_rows: int = 0
    gemm_rows: int = 256
    n_streams: int = 1
    chunk_min: int = 256
    chunk_max: int = 2048
    chunk_per_rank: int = 8


def _pow2_at_least(r: int) -> int:
    p = 1
    while p < r:
        p *= 2
    return p


def split_k(tiles, nk):
    """Rule 9 for one GEMM launch."""
    if tiles <= 0 or tiles >= 128 or nk < 16:
        return 1
    sp = min(256 // tiles, nk // 8, 16)
    if sp < 2:
        return 1
    kper = -(-nk // sp)
    return -(-nk // kper)


def build_plan(offsets, ranks, opts: PlanOpts | None = None, widths=None, dims=None) -> dict:
    """The plan tables.  ``widths``: output widths of projections sharing the
    input (then ``ranks`` is [n][P]); None is one projection (its width only
    enters chunk_boff, reported as chunk_rpref * d_out by the caller)."""
    opts = opts or PlanOpts()
    o = [int(v) for v in offsets]
    n = len(o) - 1
    if widths is None:
        P, wd = 1, [1]
        rk = [int(v) for v in ranks]
    else:
        P, wd = len(widths), [int(v) for v in widths]
        rk = [int(ranks[i][q]) for i in range(n) for q in range(P)]
    nv = n * P
    assert len(rk) == nv and o[0] == 0
    assert all(o[i] <= o[i + 1] for i in range(n))
    assert all(1 <= r <= 256 for r in rk)
    T = o[n]
    cnt = [o[i + 1] - o[i] for i in range(n)]
    rpad = [max(32, _pow2_at_least(r)) for r in rk]

    zoff, roff, seg_start = [], [], []
    z = rr = 0
    for v in range(nv):
        zoff.append(z)
        roff.append(rr)
        seg_start.append(o[v // P])
        z += cnt[v // P] * rpad[v]
        rr += rpad[v]

    S = min(opts.n_streams, n)
    g = [0] * (S + 1)
    g[S] = n
    for s in range(1, S):
        target = -(-(s * T) // S)  # ceil
        a = n
        for j in range(n):
            if o[j] >= target:
                a = j
                break
        g[s] = max(g[s - 1], a)

    def bucket_order(s):
        idx = list(range(g[s] * P, g[s + 1] * P))
        return sorted(idx, key=lambda v: (-rpad[v], v % P, v // P))

    NB = opts.nano_rows
    if NB == 0:
        NB = 128 if T * P >= 65536 else (64 if T * P >= 32768 else 32)
    nb, nb_start = [], []
    ch, ch_start, cpref, cboff = [], [], [], []
    ch_first = [0] * nv
    ch_count = [0] * nv
    cp = cb = 0
    for s in range(S):
        nb_start.append(len(nb))
        ch_start.append(len(ch))
        for v in bucket_order(s):
            lo, hi = o[v // P], o[v // P + 1]
            r0 = lo
            while r0 < hi:
                nb.append((v, r0, min(NB, hi - r0)))
                r0 += NB
            kc = min(opts.chunk_max, max(opts.chunk_min, opts.chunk_per_rank * rpad[v]))
            ch_first[v] = len(ch)
            r0 = lo
            while r0 < hi:
                ch.append((v, r0, min(kc, hi - r0)))
                cpref.append(cp)
                cboff.append(cb)
                cp += rpad[v]
                cb += rpad[v] * wd[v % P]
                ch_count[v] += 1
                r0 += kc
    nb_start.append(len(nb))
    ch_start.append(len(ch))

    tiles, tile_start, ext, ext_start = [], [], [], []
    BM = opts.gemm_rows
    ntile = -(-T // BM)
    G = 16 if ntile >= 32 * S else 1
    a = [0] * (S + 1)
    a[S] = ntile
    for s in range(1, S):
        a[s] = max(a[s - 1], G * ((o[g[s]] // BM) // G))
    for s in range(S):
        tile_start.append(len(tiles))
        for t in range(a[s], a[s + 1]):
            t0 = t * BM
            rows = min(BM, T - t0)
            for q in range(P):
                ext_start.append(len(ext))
                for j in range(n):
                    lo, hi = max(o[j], t0), min(o[j + 1], t0 + rows)
                    if lo < hi:
                        v = j * P + q
                        for k0 in range(0, rpad[v], KSTEP):
                            ext.append((v, lo, hi, k0))
            tiles.append((t0, rows))
    tile_start.append(len(tiles))
    ext_start.append(len(ext))

    ksplit = []
    if dims is not None:
        d_in, d_out, dtype = dims
        for s in range(S):
            nm = tile_start[s + 1] - tile_start[s]
            if dtype == "bf16":
                ksplit.append((split_k(nm * -(-d_out // 256), d_in // 32),
                               split_k(nm * -(-d_in // 256), d_out // 32)))
            else:
                ksplit.append((1, 1))

    def a32(x, cols=None):
        a = np.asarray(x, dtype=np.int32)
        if cols is not None:
            a = a.reshape(-1, cols)
        return a

    return {
        "T": T,
        "n": n,
        "n_groups": S,
        "z_elems": z,
        "rpad_total": rr,
        "partial_rows": cp,
        "rpad": a32(rpad),
        "zoff": np.asarray(zoff, dtype=np.int64),
        "roff": a32(roff),
        "group_first_adapter": a32(g),
        "nb": a32(nb, 3),
        "nb_start": a32(nb_start),
        "chunks": a32(ch, 3),
        "chunk_start": a32(ch_start),
        "chunk_rpref": a32(cpref),
        "adapter_chunk_first": a32(ch_first),
        "adapter_chunk_count": a32(ch_count),
        "tiles": a32(tiles, 2),
        "tile_start": a32(tile_start),
        "ext": a32(ext, 4),
        "tile_ext_start": a32(ext_start),
        "seg_start": np.asarray(seg_start, dtype=np.int64),
        "chunk_boff": np.asarray(cboff, dtype=np.int64),
        "proj_cols": a32(np.concatenate([[0], np.cumsum(wd)]) if widths is not None else [0]),
        "partial_b_elems": cb,
        "nano_rows": NB,
        "ksplit": a32(ksplit, 2) if dims is not None else None,
    }


def build_plan_from_ids(token_adapter, ranks, opts: PlanOpts | None = None, widths=None, dims=None) -> dict:
    """The plan for rows in the caller's order with per-token adapter ids:
    rows grouped by adapter with a stable counting sort (counts, exclusive
    prefix sums, then every row placed at its adapter's next free position,
    in row order); "perm" lists the caller's row of each grouped row, and the
    grouped segments get the plan of build_plan."""
    ids = [int(v) for v in token_adapter]
    n = len(ranks)
    assert all(0 <= a < n for a in ids)
    off = [0] * (n + 1)
    for a in ids:
        off[a + 1] += 1
    for a in range(n):
        off[a + 1] += off[a]
    nxt = off[:n]
    perm = [0] * len(ids)
    for t, a in enumerate(ids):
        perm[nxt[a]] = t
        nxt[a] += 1
    plan = build_plan(off, ranks, opts, widths=widths, dims=dims)
    plan["perm"] = np.asarray(perm, dtype=np.int32)
    plan["offsets"] = np.asarray(off, dtype=np.int64)
    return plan


def optimizer_blocks(ranks, d_in, d_out, widths=None) -> np.ndarray:
    """Rule 8: the (tensor, piece) work items of the per-adapter optimizer
    step.  With ``widths``, ranks is [n][P] and pair v = i P + q has B of
    widths[q] columns."""
    if widths is None:
        pairs = [(int(r), int(d_out)) for r in ranks]
    else:
        pairs = [(int(ranks[i][q]), int(widths[q])) for i in range(len(ranks)) for q in range(len(widths))]
    out = []
    for i, (r, w) in enumerate(pairs):
        for t, numel in ((2 * i, d_in * r), (2 * i + 1, r * w)):
            for piece in range(-(-numel // OPT_BLOCK)):
                out.append((t, piece))
    return np.asarray(out, dtype=np.int32).reshape(-1, 2)


def optimizer_first(ranks, d_in, d_out, widths=None) -> np.ndarray:
    """Rule 8's index of pair v's first work item (nv + 1 entries, the last
    the item count): the items of a pair are contiguous, A's then B's."""
    blocks = optimizer_blocks(ranks, d_in, d_out, widths)
    nv = len(ranks) if widths is None else len(ranks) * len(widths)
    pair = blocks[:, 0] // 2
    return np.searchsorted(pair, np.arange(nv + 1), side="left").astype(np.int32)
