"""Host-side checks of libmlora.so without a GPU: it loads, exports every
symbol include/mlora.h declares, builds plans bit-identical to the
independent Python mirror, and rejects malformed arguments with the
documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from adapter_lora_segments_amd import _lib
from adapter_lora_segments_amd.binding import Plan
from adapter_lora_segments_amd._lib import MloraError
from oracle.plan_mirror import build_plan, optimizer_blocks, optimizer_first, PlanOpts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "mlora.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"\b(mlora_[a-z_]+)\s*\(", hdr))
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert L.mlora_version().decode().startswith("mlora")
    assert L.mlora_status_string(-4).decode() == "MLORA_ERR_WORKSPACE"


def test_probe_library_exports_every_declared_symbol():
    """libmlora_probes.so (the measured ceilings) exports what
    include/mlora_probes.h declares, and refuses malformed calls before any
    HIP call (hipErrorInvalidValue = 1)."""
    with open(os.path.join(ROOT, "include", "mlora_probes.h")) as f:
        hdr = f.read()
    declared = set(re.findall(r"\b(mlora_probe_[a-z0-9_]+)\s*\(", hdr))
    assert declared == {"mlora_probe_mfma", "mlora_probe_mfma8", "mlora_probe_copy", "mlora_probe_read",
                        "mlora_probe_l2_to_lds"}, declared
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libmlora_probes.so")
    L = ctypes.CDLL(path)
    for name in declared:
        assert hasattr(L, name), name
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f = L.mlora_probe_l2_to_lds
    f.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
    f.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(64)
    ok = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    assert f(3, 1, 2, vp(ok), vp(ok), None) == 1            # no such path
    assert f(0, 0, 2, vp(ok), vp(ok), None) == 1            # no workgroup
    assert f(0, 1, 1, vp(ok), vp(ok), None) == 1            # fewer than two passes
    assert f(0, 1, 2, vp(ok + 4), vp(ok), None) == 1        # misaligned source
    assert f(0, 1, 2, None, vp(ok), None) == 1
    g = L.mlora_probe_copy
    g.argtypes = [vp, vp, i64, vp]
    g.restype = ctypes.c_int
    assert g(vp(ok), vp(ok), 16, None) == 1                  # overlapping


def _mirror_vs_library(off, ranks, d_in, d_out, dtype, opts):
    p = Plan(off, ranks, d_in, d_out, dtype, nano_rows=opts.nano_rows, gemm_rows=opts.gemm_rows,
             n_streams=opts.n_streams, chunk_min=opts.chunk_min, chunk_max=opts.chunk_max,
             chunk_per_rank=opts.chunk_per_rank)
    m = build_plan(off, ranks, opts, dims=(d_in, d_out, dtype))
    for name in ["rpad", "zoff", "roff", "group_first_adapter", "nb", "nb_start", "chunks",
                 "chunk_start", "chunk_rpref", "adapter_chunk_first", "adapter_chunk_count",
                 "tiles", "tile_start", "ext", "tile_ext_start", "ksplit"]:
        got = p.export(name)
        want = m[name]
        if want.size == 0:
            assert got.size == 0, name
        else:
            assert np.array_equal(got, want.reshape(got.shape)) and got.dtype == want.dtype, name
    assert p.info["z_elems"] == m["z_elems"]
    assert p.info["partial_rows"] == m["partial_rows"]
    assert p.info["rpad_total"] == m["rpad_total"]
    assert p.info["n_groups"] == m["n_groups"]
    assert np.array_equal(p.export("offsets"), np.asarray(off, dtype=np.int64))
    ob = optimizer_blocks(ranks, d_in, d_out)
    assert np.array_equal(p.export("opt_blocks"), ob) and p.info["n_opt_blocks"] == ob.shape[0]
    assert np.array_equal(p.export("opt_first"), optimizer_first(ranks, d_in, d_out))
    # one projection: pairs are the adapters, dB partials of d_out columns per rank row
    assert np.array_equal(p.export("seg_start"), np.asarray(off[:-1], dtype=np.int64))
    assert np.array_equal(p.export("chunk_boff"), m["chunk_rpref"].astype(np.int64) * d_out)
    assert np.array_equal(p.export("proj_cols"), np.asarray([0, d_out], dtype=np.int32))
    assert p.info["n_proj"] == 1


@st.composite
def plan_cases(draw):
    n = draw(st.integers(1, 40))
    toks = draw(st.lists(st.one_of(st.just(0), st.just(1), st.integers(0, 900)), min_size=n, max_size=n))
    ranks = draw(st.lists(st.one_of(st.sampled_from([1, 4, 8, 16, 31, 32, 33, 64, 65, 128, 129, 255, 256]),
                                    st.integers(1, 256)), min_size=n, max_size=n))
    nb = draw(st.sampled_from([32, 64, 96, 256]))
    S = draw(st.integers(1, 4))
    cmin = draw(st.sampled_from([16, 64, 256]))
    cmax = cmin * draw(st.sampled_from([1, 4, 8]))
    cpr = draw(st.sampled_from([1, 8, 16]))
    off = [0]
    for t in toks:
        off.append(off[-1] + t)
    return off, ranks, PlanOpts(nano_rows=nb, gemm_rows=256, n_streams=S, chunk_min=cmin,
                                chunk_max=cmax, chunk_per_rank=cpr)


@settings(max_examples=200, deadline=None)
@given(plan_cases())
def test_plan_bit_exact_against_mirror(case):
    off, ranks, opts = case
    _mirror_vs_library(off, ranks, 128, 192, "bf16", opts)


@pytest.mark.parametrize("name,seed", [(w, s) for w in ["tiny_fp32", "llama7b_proj", "llama3_8b_layer",
                                                          "nano_stress", "mlp70b_pair"] for s in (0, 1, 2)])
def test_plan_bit_exact_on_workloads(name, seed):
    from workloads import load_workload
    w = load_workload(name, seed)
    for p in w.projections:
        _mirror_vs_library(w.seg_offsets(), w.ranks, p.d_in, p.d_out, w.dtype,
                           PlanOpts(n_streams=w.n_streams))


@st.composite
def ids_cases(draw):
    n = draw(st.integers(1, 24))
    T = draw(st.integers(0, 1500))
    ids = draw(st.lists(st.integers(0, n - 1), min_size=T, max_size=T))
    ranks = draw(st.lists(st.sampled_from([1, 8, 16, 33, 64, 128, 256]), min_size=n, max_size=n))
    S = draw(st.integers(1, 4))
    return ids, ranks, PlanOpts(nano_rows=draw(st.sampled_from([32, 64, 256])), gemm_rows=256, n_streams=S)


@settings(max_examples=120, deadline=None)
@given(ids_cases())
def test_plan_from_ids_bit_exact_against_mirror(case):
    """mlora_plan_from_ids: the grouping permutation and every table equal the
    mirror's (an independent counting sort, then the segment rule)."""
    from oracle.plan_mirror import build_plan_from_ids
    ids, ranks, opts = case
    p = Plan.from_ids(ids, ranks, 128, 192, "bf16", nano_rows=opts.nano_rows, n_streams=opts.n_streams)
    m = build_plan_from_ids(ids, ranks, opts)
    assert np.array_equal(p.export("perm"), m["perm"]) and p.export("perm").dtype == np.int32
    assert np.array_equal(p.export("offsets"), m["offsets"])
    for name in ["rpad", "zoff", "roff", "group_first_adapter", "nb", "nb_start", "chunks",
                 "chunk_start", "chunk_rpref", "adapter_chunk_first", "adapter_chunk_count",
                 "tiles", "tile_start", "ext", "tile_ext_start"]:
        got, want = p.export(name), m[name]
        assert (got.size == 0 and want.size == 0) or np.array_equal(got, want.reshape(got.shape)), name


def test_plan_from_ids_errors_and_segment_plans_have_no_perm():
    assert _status(lambda: Plan.from_ids([0, 2, 1], [4, 8], 128, 64)) == -1   # id 2 >= n
    assert _status(lambda: Plan.from_ids([0, -1], [4, 8], 128, 64)) == -1     # negative id
    assert _status(lambda: Plan.from_ids([0, 1], [4, 0], 128, 64)) == -1      # rank 0
    p = Plan.from_ids([], [4, 8], 128, 64)                                      # no rows at all
    assert p.info["T"] == 0 and p.export("perm").size == 0
    assert Plan([0, 5, 9], [4, 8], 128, 64).export("perm").size == 0


def _status(fn):
    with pytest.raises(MloraError) as e:
        fn()
    return e.value.status


def test_plan_argument_errors():
    ok = dict(seg_offsets=[0, 5, 9], ranks=[4, 8], d_in=128, d_out=64)
    Plan(**ok)  # valid
    assert _status(lambda: Plan([1, 5, 9], [4, 8], 128, 64)) == -1          # offsets[0] != 0
    assert _status(lambda: Plan([0, 5, 3], [4, 8], 128, 64)) == -1          # decreasing
    assert _status(lambda: Plan([0, 5, 9], [0, 8], 128, 64)) == -1          # rank 0
    assert _status(lambda: Plan([0, 5, 9], [4, 257], 128, 64)) == -2        # rank > 256
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 100, 64)) == -2          # d_in % 64
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 0)) == -1           # d_out <= 0
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 64, nano_rows=8)) == -1
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 64, n_streams=5)) == -1
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 64, gemm_rows=128)) == -2  # bf16 needs 256
    Plan([0, 5, 9], [4, 8], 128, 64, "fp32", gemm_rows=128)
    L = _lib.lib()
    h = ctypes.c_void_p()
    off = (ctypes.c_int64 * 1)(0)
    rk = (ctypes.c_int32 * 1)(4)
    assert L.mlora_plan(0, off, rk, 64, 64, 1, None, ctypes.byref(h)) == -1  # n = 0
    assert L.mlora_plan(1, None, rk, 64, 64, 1, None, ctypes.byref(h)) == -1
    assert L.mlora_plan(1, off, rk, 64, 64, 1, None, None) == -1
    assert "out" in L.mlora_last_error().decode()
    assert not h.value  # untouched on error


def test_forward_rejects_bad_arguments_without_launching():
    """Errors found on the host return before any HIP call (no GPU here)."""
    L = _lib.lib()
    p = Plan([0, 5, 9], [4, 8], 128, 64)
    vp = ctypes.c_void_p
    dummy = vp(4096)
    # NULL X
    assert L.mlora_forward(p.handle, None, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 30, None) == -1
    # misaligned pointer
    assert L.mlora_forward(p.handle, vp(4097), dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 30, None) == -1
    # workspace too small
    assert L.mlora_forward(p.handle, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 16, None) == -4
    # workspace never uploaded
    assert L.mlora_forward(p.handle, dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 30, None) == -4
    assert L.mlora_backward(p.handle, dummy, dummy, dummy, dummy, dummy, dummy, None, None, None,
                            dummy, dummy, 1 << 30, None) == -1
    # unknown table id / small buffer
    n = ctypes.c_size_t(0)
    assert L.mlora_plan_export(p.handle, 99, None, ctypes.byref(n)) == -1
    assert L.mlora_plan_export(p.handle, 0, None, ctypes.byref(n)) == 0 and n.value == 8
    small = ctypes.c_size_t(4)
    buf = (ctypes.c_int32 * 1)()
    assert L.mlora_plan_export(p.handle, 0, buf, ctypes.byref(small)) == -1 and small.value == 8


def test_plan_info_sizes():
    p = Plan([0, 40, 40, 200, 300], [8, 64, 100, 16], 256, 512)
    i = p.info
    assert i["T"] == 300 and i["n"] == 4 and i["z_elems"] == 24960 and i["z_bytes"] == 2 * 24960
    assert i["workspace_bytes"] >= i["table_bytes"] + 2 * i["z_elems"] + 4 * i["partial_rows"] * (256 + 512)


def test_optimizer_blocks_cover_every_element_once():
    """Rule 8 read back from the library: the pieces of each tensor tile its
    elements exactly once, adapters ascending, A before B."""
    ranks = [1, 7, 64, 256, 3]
    d_in, d_out = 192, 4096
    p = Plan([0, 3, 3, 10, 11, 20], ranks, d_in, d_out)
    ob = p.export("opt_blocks")
    assert ob.dtype == np.int32 and ob.shape == (p.info["n_opt_blocks"], 2)
    tensors = ob[:, 0]
    assert np.all(np.diff(tensors) >= 0)
    for t in range(2 * len(ranks)):
        r = ranks[t // 2]
        numel = r * (d_out if t % 2 else d_in)
        pieces = ob[tensors == t, 1]
        assert np.array_equal(pieces, np.arange(-(-numel // 2048))), t


def test_adamw_rejects_bad_arguments_without_launching():
    L = _lib.lib()
    vp = ctypes.c_void_p
    d = vp(4096)
    ok = [d] * 9                      # hparams, A, B, dA, dB, mA, vA, mB, vB
    bf = Plan([0, 5, 9], [4, 8], 128, 64)
    f32 = Plan([0, 5, 9], [4, 8], 128, 64, "fp32")
    assert L.mlora_adamw_step(None, *ok, None, None, 0, d, 1 << 30, None) == -1
    for k in range(9):                # each required array NULL, then misaligned
        args = list(ok)
        args[k] = None
        assert L.mlora_adamw_step(bf.handle, *args, None, None, 0, d, 1 << 30, None) == -1, k
        args[k] = vp(4100)
        assert L.mlora_adamw_step(bf.handle, *args, None, None, 0, d, 1 << 30, None) == -1, k
    assert L.mlora_adamw_step(bf.handle, *ok, d, None, 0, d, 1 << 30, None) == -1      # one copy only
    assert L.mlora_adamw_step(f32.handle, *ok, d, d, 0, d, 1 << 30, None) == -1        # fp32 takes none
    assert "fp32" in L.mlora_last_error().decode()
    assert L.mlora_adamw_step(bf.handle, *ok, d, d, 0, d, 16, None) == -4              # workspace small
    assert L.mlora_adamw_step(bf.handle, *ok, None, None, 0, d, 1 << 30, None) == -4   # not uploaded
    assert L.mlora_adamw_step(bf.handle, *ok, d, d, 2, d, 1 << 30, None) == -1      # clip_grads not 0/1
    assert _lib.KERNELS[7:] == ["adamw", "dequant", "grad_norm", "quant_act"] and len(_lib.KERNELS) == 11


def test_adamw_hparams_layout():
    """The ctypes mirror of mlora_adamw_hparams: five floats, the step, then
    max_grad_norm."""
    assert ctypes.sizeof(_lib.AdamwHparams) == 28
    h = _lib.AdamwHparams(1e-4, 0.9, 0.999, 1e-8, 0.01, 3, 0.5)
    raw = np.frombuffer(bytes(h), dtype=np.uint8)
    assert np.array_equal(raw[:20].view(np.float32), np.float32([1e-4, 0.9, 0.999, 1e-8, 0.01]))
    assert raw[20:24].view(np.int32)[0] == 3
    assert raw[24:].view(np.float32)[0] == np.float32(0.5)


TABLES_ALL = ["rpad", "zoff", "roff", "group_first_adapter", "nb", "nb_start", "chunks", "chunk_start",
              "chunk_rpref", "adapter_chunk_first", "adapter_chunk_count", "tiles", "tile_start", "ext",
              "tile_ext_start", "seg_start", "chunk_boff", "proj_cols"]


@st.composite
def multi_cases(draw):
    n = draw(st.integers(1, 12))
    P = draw(st.integers(1, 4))
    dtype = draw(st.sampled_from(["bf16", "fp32"]))
    unit = 256 if dtype == "bf16" else 64
    widths = [unit * draw(st.integers(1, 6)) for _ in range(P)]
    toks = draw(st.lists(st.one_of(st.just(0), st.integers(0, 700)), min_size=n, max_size=n))
    ranks = [draw(st.lists(st.sampled_from([1, 8, 16, 33, 64, 100, 128, 256]), min_size=P, max_size=P))
             for _ in range(n)]
    S = draw(st.integers(1, 4))
    nb = draw(st.sampled_from([32, 64, 256]))
    off = [0]
    for t in toks:
        off.append(off[-1] + t)
    return off, ranks, widths, dtype, PlanOpts(nano_rows=nb, gemm_rows=256 if dtype == "bf16" else 64,
                                                n_streams=S)


@settings(max_examples=150, deadline=None)
@given(multi_cases())
def test_plan_multi_bit_exact_against_mirror(case):
    """mlora_plan_multi: every table equals the mirror's rule over
    (adapter, projection) pairs."""
    off, ranks, widths, dtype, opts = case
    d_in = 192
    p = Plan.multi(off, ranks, d_in, widths, dtype, nano_rows=opts.nano_rows, n_streams=opts.n_streams,
                   gemm_rows=opts.gemm_rows)
    m = build_plan(off, ranks, opts, widths=widths, dims=(d_in, sum(widths), dtype))
    for name in TABLES_ALL + ["ksplit"]:
        got, want = p.export(name), m[name]
        assert (got.size == 0 and want.size == 0) or (
            np.array_equal(got, want.reshape(got.shape)) and got.dtype == want.dtype), name
    assert np.array_equal(p.export("ranks"), np.asarray(ranks, dtype=np.int32).reshape(-1))
    assert np.array_equal(p.export("offsets"), np.asarray(off, dtype=np.int64))
    ob = optimizer_blocks(ranks, d_in, None, widths=widths)
    assert np.array_equal(p.export("opt_blocks"), ob)
    assert np.array_equal(p.export("opt_first"), optimizer_first(ranks, d_in, None, widths=widths))
    i = p.info
    assert i["n_proj"] == len(widths) and i["d_out"] == sum(widths) and i["n"] == len(ranks)
    assert i["z_elems"] == m["z_elems"] and i["partial_rows"] == m["partial_rows"]
    assert i["rpad_total"] == m["rpad_total"]
    if dtype == "bf16":  # the fp32 path keeps no chunk partials
        assert i["workspace_bytes"] >= i["table_bytes"] + 4 * m["partial_b_elems"]


def test_plan_multi_errors():
    ok = dict(seg_offsets=[0, 5, 9], ranks=[[4, 8], [2, 2]], d_in=128, widths=[256, 512])
    Plan.multi(**ok)
    assert _status(lambda: Plan.multi([0, 5, 9], [[4, 8], [2, 2]], 128, [256, 320])) == -2   # width % 256 (bf16)
    Plan.multi([0, 5, 9], [[4, 8], [2, 2]], 128, [64, 320], "fp32")                        # fp32: % 64
    assert _status(lambda: Plan.multi([0, 5, 9], [[4, 8], [2, 2]], 128, [64, 96], "fp32")) == -2
    assert _status(lambda: Plan.multi([0, 5, 9], [[4, 0], [2, 2]], 128, [256, 256])) == -1   # rank 0
    assert _status(lambda: Plan.multi([0, 5, 9], [[4, 300], [2, 2]], 128, [256, 256])) == -2  # rank > 256
    assert _status(lambda: Plan.multi([0, 5, 9], [[1] * 9] * 2, 128, [256] * 9)) == -1       # n_proj > 8
    L = _lib.lib()
    h = ctypes.c_void_p()
    off = (ctypes.c_int64 * 3)(0, 5, 9)
    rk = (ctypes.c_int32 * 4)(4, 8, 2, 2)
    w = (ctypes.c_int64 * 2)(256, 256)
    assert L.mlora_plan_multi(2, off, 0, w, rk, 128, 1, None, ctypes.byref(h)) == -1          # n_proj 0
    assert L.mlora_plan_multi(2, off, 2, None, rk, 128, 1, None, ctypes.byref(h)) == -1       # no widths
    assert L.mlora_plan_multi(40000, off, 2, w, rk, 128, 1, None, ctypes.byref(h)) == -1      # n * n_proj too big
    assert not h.value
    p1 = Plan.multi([0, 5, 9], [[4], [8]], 128, [320])                                         # one projection
    p0 = Plan([0, 5, 9], [4, 8], 128, 320)
    for name in TABLES_ALL + ["opt_blocks"]:
        assert np.array_equal(p1.export(name), p0.export(name)), name


def test_split_k_rule():
    """Rule 9 read back from the library on hand-worked launches."""
    from oracle.plan_mirror import split_k
    # 7680 rows, 4096 x 4096: 30 x 16 = 480 tiles -> no split
    p = Plan([0, 7680], [16], 4096, 4096)
    assert p.export("ksplit").tolist() == [[1, 1]]
    # 512 rows, 2048 x 2048: 2 x 8 = 16 tiles, 64 K-steps: S = min(256 // 16, 64 // 8, 16) = 8
    p = Plan([0, 512], [16], 2048, 2048)
    assert p.export("ksplit").tolist() == [[8, 8]]
    # 300 rows, d_in 512, d_out 8192: forward 2 x 32 = 64 tiles, 16 K-steps -> S = min(4, 2, 16) = 2;
    # dX 2 x 2 = 4 tiles, 256 K-steps -> S = 16
    p = Plan([0, 300], [8], 512, 8192)
    assert p.export("ksplit").tolist() == [[2, 16]]
    # K below 16 steps never splits; fp32 never splits
    assert Plan([0, 100], [8], 256, 256).export("ksplit").tolist() == [[1, 1]]
    assert Plan([0, 512], [16], 2048, 2048, "fp32").export("ksplit").tolist() == [[1, 1]]
    # 2048 rows, 3584 x 3584: 8 x 14 = 112 tiles -> S = 256 // 112 = 2 (224 workgroups, one round)
    assert Plan([0, 2048], [64], 3584, 3584).export("ksplit").tolist() == [[2, 2]]
    # every part non-empty: (S - 1) * ceil(nk / S) < nk over a range of shapes
    for tiles in range(1, 130):
        for nk in range(1, 700, 7):
            S = split_k(tiles, nk)
            kper = -(-nk // S)
            assert 1 <= S <= 16 and (S - 1) * kper < nk and (S == 1 or S * tiles <= 256), (tiles, nk, S)


def test_mxfp8_plan_options():
    """An MXFP8 base needs a bf16 plan; its decoded weight is counted in the
    workspace; the binding expects codes then scales in one uint8 buffer."""
    from adapter_lora_segments_amd.binding import _w0_shape
    p_bf = Plan([0, 5, 9], [4, 8], 128, 192)
    p_mx = Plan([0, 5, 9], [4, 8], 128, 192, w0_format="mxfp8")
    assert p_mx.info["workspace_bytes"] >= p_bf.info["workspace_bytes"] + 2 * 128 * 192 - 256  # an empty region still takes 256
    assert _w0_shape(p_mx) == (128 * 192 + 192 * 4,)
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 192, "fp32", w0_format="mxfp8")) == -2
    for name in ["rpad", "zoff", "nb", "chunks", "tiles", "ext", "ksplit", "opt_blocks"]:
        assert np.array_equal(p_mx.export(name), p_bf.export(name)), name


def test_mxfp4_plan_options():
    """An MXFP4 base needs a bf16 plan, counts the same decoded copy in the
    workspace as MXFP8, and takes half a byte per code then the scales."""
    from adapter_lora_segments_amd.binding import _w0_shape, _w0_dtype
    p8 = Plan([0, 5, 9], [4, 8], 128, 192, w0_format="mxfp8")
    p4 = Plan([0, 5, 9], [4, 8], 128, 192, w0_format="mxfp4", w0_layout="nk")
    assert p4.info["workspace_bytes"] == p8.info["workspace_bytes"]
    assert _w0_shape(p4) == (128 * 192 // 2 + 192 * 4,)
    import torch
    assert _w0_dtype(p4) == torch.uint8
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 192, "fp32", w0_format="mxfp4")) == -2
    o = _lib.PlanOpts()
    o.w0_format = 3
    L = _lib.lib()
    h = ctypes.c_void_p()
    off = (ctypes.c_int64 * 3)(0, 5, 9)
    rk = (ctypes.c_int32 * 2)(4, 8)
    assert L.mlora_plan(2, off, rk, 128, 192, 0, ctypes.byref(o), ctypes.byref(h)) == -1
    assert "MXFP4" in L.mlora_last_error().decode()


def test_two_layout_base_options():
    """MLORA_W0_BOTH: accepted for bf16 and fp32 plans, refused with a
    microscaled base; the binding expects both layouts in one flat buffer;
    the transpose entry point checks its arguments before launching."""
    from adapter_lora_segments_amd.binding import _w0_shape
    for dt in ("bf16", "fp32"):
        p2 = Plan([0, 5, 9], [4, 8], 128, 192, dt, w0_layout="both")
        p1 = Plan([0, 5, 9], [4, 8], 128, 192, dt)
        assert _w0_shape(p2) == (2 * 128 * 192,)
        assert p2.info["workspace_bytes"] == p1.info["workspace_bytes"]
        for name in ["rpad", "zoff", "nb", "chunks", "tiles", "ext", "ksplit"]:
            assert np.array_equal(p2.export(name), p1.export(name)), name
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 128, 192, w0_layout="both", w0_format="mxfp4")) == -2
    L = _lib.lib()
    vp = ctypes.c_void_p
    a, b = vp(1 << 20), vp(1 << 24)
    assert L.mlora_base_transpose(None, b, 64, 64, 0, None) == -1
    assert L.mlora_base_transpose(a, vp((1 << 24) + 8), 64, 64, 0, None) == -1          # misaligned
    assert L.mlora_base_transpose(a, b, 64, 96, 0, None) == -1                          # not a multiple of 64
    assert L.mlora_base_transpose(a, b, 0, 64, 0, None) == -1
    assert L.mlora_base_transpose(a, b, 64, 64, 7, None) == -1                          # dtype
    assert L.mlora_base_transpose(a, vp((1 << 20) + 4096), 64, 64, 0, None) == -1       # overlap
    assert "overlap" in L.mlora_last_error().decode()
    import torch
    from adapter_lora_segments_amd import PackedLoRALinear
    p2 = Plan([0, 5, 9], [4, 8], 128, 192, w0_layout="both")
    with pytest.raises(ValueError, match="d_in"):
        PackedLoRALinear(p2, torch.zeros((192, 128), dtype=torch.bfloat16), [None, None], [None, None], [1.0, 1.0],
                         device="cpu")


def test_mx4_quantizer_round_trip():
    """The MXFP4 input quantizer against the oracle's decoder: every weight
    decodes to the nearest E2M1 value of its scaled magnitude (ties low), with
    the weight's sign, and no block overflows."""
    from oracle import mx as omx
    from workloads.mx import quantize_mx4, E2M1_MAGNITUDES
    rng = np.random.default_rng(1)
    w = rng.standard_normal((128, 64)) * 0.02
    w[7, 2] = 0.0
    mags = np.asarray(E2M1_MAGNITUDES)
    for layout in ("kn", "nk"):
        codes, scales = quantize_mx4(w, layout)
        rows, cols = (128, 64) if layout == "kn" else (64, 128)
        assert codes.shape == (rows, cols // 2) and scales.shape == (64, 4)
        dec = omx.decode_e2m1(omx.unpack_e2m1(codes, rows, cols))
        if layout == "nk":
            dec = dec.T
        sc = omx.decode_e8m0(scales).T.repeat(32, axis=0)
        q = w / sc
        assert np.all(np.abs(q) <= 6.0 + 1e-12)
        want = mags[np.argmin(np.abs(np.abs(q)[..., None] - mags), axis=-1)] * np.sign(q)
        assert np.array_equal(dec, want)


def test_mx_quantizer_round_trip():
    """The input quantizer (workloads/mx.py) against the oracle's decoder:
    every decoded weight is within half an E4M3 step of the float weight, and
    no block overflows."""
    from oracle import mx as omx
    from workloads.mx import quantize_mx
    rng = np.random.default_rng(0)
    w = rng.standard_normal((128, 64)) * 0.02
    w[5, 3] = 0.0
    for layout in ("kn", "nk"):
        codes, scales = quantize_mx(w, layout)
        assert codes.dtype == np.uint8 and scales.shape == (64, 4)
        dec = omx.decode_e4m3(codes).reshape(codes.shape)
        if layout == "nk":
            dec = dec.T
        sc = omx.decode_e8m0(scales).T.repeat(32, axis=0)
        assert np.all(np.isfinite(dec)) and np.all(np.abs(dec) <= 448)
        err = np.abs(dec * sc - w)
        assert np.all(err <= sc * 2.0 ** -3 * np.maximum(np.abs(dec), 2.0 ** -6) + 1e-300)


@st.composite
def multi_ids_cases(draw):
    n = draw(st.integers(1, 10))
    P = draw(st.integers(1, 3))
    T = draw(st.integers(0, 1200))
    ids = draw(st.lists(st.integers(0, n - 1), min_size=T, max_size=T))
    ranks = [draw(st.lists(st.sampled_from([1, 8, 33, 64, 128, 256]), min_size=P, max_size=P)) for _ in range(n)]
    widths = [256 * draw(st.integers(1, 4)) for _ in range(P)]
    S = draw(st.integers(1, 4))
    return ids, ranks, widths, PlanOpts(nano_rows=32, gemm_rows=256, n_streams=S)


@settings(max_examples=100, deadline=None)
@given(multi_ids_cases())
def test_plan_multi_from_ids_bit_exact_against_mirror(case):
    """mlora_plan_multi_from_ids: the permutation and every table equal the
    mirror's counting sort followed by its multi-projection rule."""
    from oracle.plan_mirror import build_plan_from_ids
    ids, ranks, widths, opts = case
    d_in = 320
    p = Plan.multi_from_ids(ids, ranks, d_in, widths, "bf16", n_streams=opts.n_streams)
    m = build_plan_from_ids(ids, ranks, opts, widths=widths, dims=(d_in, sum(widths), "bf16"))
    assert np.array_equal(p.export("perm"), m["perm"]) and np.array_equal(p.export("offsets"), m["offsets"])
    for name in TABLES_ALL + ["ksplit"]:
        got, want = p.export(name), m[name]
        assert (got.size == 0 and want.size == 0) or np.array_equal(got, want.reshape(got.shape)), name
    assert _status(lambda: Plan.multi_from_ids([0, 3], [[4, 4], [8, 8]], 128, [256, 256])) == -1  # id 3 >= n


def test_packed_layer_checks_adapter_tensors_before_any_device_call():
    """PackedLoRALinear refuses adapter tensors the kernels would misread
    through their raw pointers (wrong shape, dtype, layout or device),
    before it allocates anything on a device."""
    import torch
    from adapter_lora_segments_amd.binding import PackedLoRALinear
    ranks, d_in, d_out = [8, 33], 128, 192
    plan = Plan([0, 5, 9], ranks, d_in, d_out, "bf16")
    good_A = [torch.zeros((d_in, r), dtype=torch.bfloat16) for r in ranks]
    good_B = [torch.zeros((r, d_out), dtype=torch.bfloat16) for r in ranks]

    def refuse(A, B, scales=(1.0, 1.0), match=""):
        with pytest.raises(ValueError, match=match):
            PackedLoRALinear(plan, None, A, B, list(scales))

    refuse(good_A, good_B, match="device tensor")                    # host tensors
    refuse([good_A[0], torch.zeros((d_in, 32), dtype=torch.bfloat16)], good_B, match=r"A\[1\].*shape")
    refuse(good_A, [good_B[0], torch.zeros((33, d_out - 64), dtype=torch.bfloat16)], match=r"B\[1\].*shape")
    refuse([good_A[0], good_A[1].float()], good_B, match=r"A\[1\].*bfloat16")
    refuse(good_A, [good_B[0], torch.zeros((d_out, 33), dtype=torch.bfloat16).t()], match="contiguous")
    refuse(good_A[:1], good_B, match="adapter tensors")
    refuse(good_A, good_B, scales=(1.0,), match="scales")
    # a multi-projection plan: B of pair (i, q) is [r][width of q]
    mp = Plan.multi([0, 4, 9], [[8, 16], [4, 32]], d_in, [256, 512], "bf16")
    A = [torch.zeros((d_in, r), dtype=torch.bfloat16) for r in (8, 16, 4, 32)]
    B = [torch.zeros((r, w), dtype=torch.bfloat16) for r, w in ((8, 256), (16, 512), (4, 256), (32, 256))]
    with pytest.raises(ValueError, match=r"B\[3\].*shape"):
        PackedLoRALinear(mp, None, A, B, [1.0] * 4)


def _lib_tables_match(p, expect, skip=()):
    """Library export of every table named in a hand-worked golden."""
    info_keys = {"T", "n_groups", "z_elems", "rpad_total", "partial_rows"}
    for k, v in expect.items():
        if k in skip:
            continue
        if k in info_keys:
            assert p.info[k] == v, (k, p.info[k], v)
            continue
        got = p.export(k)
        want = np.asarray(v).reshape(got.shape) if got.size else np.asarray(v)
        assert np.array_equal(got, want), (k, got, v)


def test_library_plans_match_hand_worked_goldens():
    """The C++ plan builder against the plans worked by hand (the same
    goldens that pin the Python mirror): one projection, two projections
    sharing the input, and rows as per-token ids."""
    import json
    gdir = os.path.join(ROOT, "tests", "golden")
    g = json.load(open(os.path.join(gdir, "plan_hand.json")))
    o = g["opts"]
    p = Plan(g["offsets"], g["ranks"], 256, 256, "fp32", nano_rows=o["nano_rows"], gemm_rows=o["gemm_rows"],
             n_streams=o["n_streams"], chunk_min=o["chunk_min"], chunk_max=o["chunk_max"],
             chunk_per_rank=o["chunk_per_rank"])
    _lib_tables_match(p, g["expect"])

    g = json.load(open(os.path.join(gdir, "plan_multi_hand.json")))
    o = g["opts"]
    p = Plan.multi(g["offsets"], g["ranks"], g["d_in"], g["widths"], g["dtype"], nano_rows=o["nano_rows"],
                   gemm_rows=o["gemm_rows"], n_streams=o["n_streams"], chunk_min=o["chunk_min"],
                   chunk_max=o["chunk_max"], chunk_per_rank=o["chunk_per_rank"])
    # partial_b_elems is the mirror's running total, not a library table
    _lib_tables_match(p, g["expect"], skip=("partial_b_elems",))

    g = json.load(open(os.path.join(gdir, "plan_ids_hand.json")))
    o = g["opts"]
    p = Plan.from_ids(g["ids"], g["ranks"], g["d_in"], g["d_out"], g["dtype"], nano_rows=o["nano_rows"],
                      gemm_rows=o["gemm_rows"], n_streams=o["n_streams"], chunk_min=o["chunk_min"],
                      chunk_max=o["chunk_max"], chunk_per_rank=o["chunk_per_rank"])
    _lib_tables_match(p, g["expect"])
    # rule 9 rebalanced by hand: 10 forward tiles over 130 K-steps -> 15 parts,
    # 17 dX tiles over 80 K-steps -> 10 parts
    assert Plan([0, 256], [8], 4160, 2560).export("ksplit").tolist() == [[15, 10]]


def test_weight_gradient_placement_rule():
    """wg_overlap: AUTO puts a bf16 plan's weight gradients beside the dX
    GEMMs while those (all stream groups together) have at most 16 rounds of
    256 output tiles (4096 tiles), after them otherwise; SIDE and AFTER force
    the choice; fp32 plans run them on the caller's stream; other values are
    refused."""
    # 4096 tiles exactly: 256 row tiles x 16 column tiles (T = 65536, d_in = 4096)
    assert Plan([0, 65536], [8], 4096, 256).info["wg_side"] == 1
    # one more column tile: 256 x 17
    assert Plan([0, 65536], [8], 4352, 256).info["wg_side"] == 0
    assert Plan([0, 65536], [8], 4352, 256, wg_overlap="side").info["wg_side"] == 1
    assert Plan([0, 100], [8], 256, 256, wg_overlap="after").info["wg_side"] == 0
    assert Plan([0, 100], [8], 256, 256).info["wg_side"] == 1
    assert Plan([0, 65536, 70000], [8, 16], 4352, 256, n_streams=2).info["wg_side"] == 0
    assert Plan([0, 30000, 65536], [8, 16], 4096, 256, n_streams=2).info["wg_side"] == 1
    assert Plan([0, 30000, 65536], [8, 16], 4096, 256, n_streams=2, wg_overlap="after").info["wg_side"] == 0
    assert Plan([0, 100], [8], 256, 256, "fp32", wg_overlap="side").info["wg_side"] == 0
    o = _lib.PlanOpts()
    o.wg_overlap = 3
    L = _lib.lib()
    h = ctypes.c_void_p()
    off = (ctypes.c_int64 * 2)(0, 100)
    rk = (ctypes.c_int32 * 1)(8)
    assert L.mlora_plan(1, off, rk, 256, 256, 0, ctypes.byref(o), ctypes.byref(h)) == -1
    assert "wg_overlap" in L.mlora_last_error().decode()


def test_grad_accumulate_option():
    """grad_accumulate: 0 and 1 are accepted (the plan's tables do not depend
    on it); any other value is refused with a message."""
    a = Plan([0, 100, 300], [8, 16], 256, 256)
    b = Plan([0, 100, 300], [8, 16], 256, 256, grad_accumulate=True)
    for name in ("nb", "chunks", "tiles", "ext"):
        assert np.array_equal(a.export(name), b.export(name)), name
    assert a.info["workspace_bytes"] == b.info["workspace_bytes"]
    L = _lib.lib()
    off = (ctypes.c_int64 * 2)(0, 100)
    rk = (ctypes.c_int32 * 1)(8)
    for bad in (-1, 2):
        o = _lib.PlanOpts()
        o.grad_accumulate = bad
        h = ctypes.c_void_p()
        assert L.mlora_plan(1, off, rk, 256, 256, 0, ctypes.byref(o), ctypes.byref(h)) == -1
        assert "grad_accumulate" in L.mlora_last_error().decode()


def test_mxfp8_activation_plan_options():
    """MXFP8 activations: accepted with an MXFP8 or MXFP4 base held as
    [d_out][d_in] and d_in a multiple of 128; refused otherwise, with a
    message; the workspace then holds the activations' codes and scales."""
    for fmt in ("mxfp8", "mxfp4"):
        p = Plan([0, 5, 9], [4, 8], 256, 192, w0_format=fmt, w0_layout="nk", act_format="mxfp8")
        q = Plan([0, 5, 9], [4, 8], 256, 192, w0_format=fmt, w0_layout="nk")
        assert p.info["act_offset"] >= 0 and q.info["act_offset"] == -1
        assert p.info["workspace_bytes"] >= q.info["workspace_bytes"] - 2 * 256 * 192 + 9 * 256 * 33 // 32
        assert _status(lambda: Plan([0, 5, 9], [4, 8], 256, 192, w0_format=fmt, act_format="mxfp8")) == -2
        assert _status(lambda: Plan([0, 5, 9], [4, 8], 192, 192, w0_format=fmt, w0_layout="nk",
                                    act_format="mxfp8")) == -2
    assert _status(lambda: Plan([0, 5, 9], [4, 8], 256, 192, w0_layout="nk", act_format="mxfp8")) == -2
    assert "MXFP4" in _lib.lib().mlora_last_error().decode()
