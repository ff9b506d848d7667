"""The plan mirror against plans worked by hand (one projection, two
projections sharing the input, rows as per-token ids), split-K factors
worked by hand, and invariants any correct plan must satisfy (every row
covered once per projection, chunks partition each pair, extension steps
cover exactly the pairs meeting each tile), seeded and under hypothesis."""
import pytest
from hypothesis import given, settings, strategies as st

from oracle import plan_mirror
from oracle.plan_mirror import build_plan, PlanOpts
from tests import pins_plan


@pytest.mark.parametrize("pin", pins_plan.ALL_PINS, ids=lambda f: f.__name__)
def test_plan_pin(pin):
    pin(plan_mirror)


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
    pins_plan.check_invariants(plan_mirror, off, ranks, opts, p)


@st.composite
def multi_inputs(draw):
    n = draw(st.integers(1, 12))
    P = draw(st.integers(1, 4))
    toks = draw(st.lists(st.integers(0, 500), min_size=n, max_size=n))
    ranks = [draw(st.lists(st.integers(1, 256), min_size=P, max_size=P)) for _ in range(n)]
    widths = draw(st.lists(st.sampled_from([256, 512, 768]), min_size=P, max_size=P))
    nb = draw(st.sampled_from([16, 32, 64]))
    S = draw(st.integers(1, 5))
    cmin = draw(st.sampled_from([16, 64, 256]))
    cmax = cmin * draw(st.sampled_from([1, 4]))
    off = [0]
    for t in toks:
        off.append(off[-1] + t)
    return off, ranks, widths, PlanOpts(nano_rows=nb, gemm_rows=256, n_streams=S, chunk_min=cmin,
                                         chunk_max=cmax, chunk_per_rank=draw(st.sampled_from([1, 8])))


@settings(max_examples=150, deadline=None)
@given(multi_inputs())
def test_plan_invariants_several_projections(args):
    off, ranks, widths, opts = args
    p = build_plan(off, ranks, opts, widths=widths)
    pins_plan.check_invariants(plan_mirror, off, ranks, opts, p, widths=widths)
