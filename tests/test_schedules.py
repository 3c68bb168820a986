"""The IC sampler schedules: the oracle's table pinned to the pages' numbers and
to closed forms, and the package's host-side schedules equal to the oracle's."""
import math
import os

import pytest

import oracle
from few_step_diffusion_amd import schedules

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ic_sampler.txt")


def golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *rest = line.split()
            vals[key] = rest
    return vals


def test_table_hits_the_printed_up4_start():
    g = golden()
    steps = int(g["table_steps"][0])
    shift = float(g["video_shift"][0])
    table = oracle.shifted_table(steps, shift)
    # t = 1/2 is k = steps/2; the pages print 0.923 for the up4 start
    assert round(table[steps // 2], 3) == float(g["up4_start"][0])
    assert table[steps // 2] == pytest.approx(12.0 / 13.0, abs=1e-15)


def test_table_end_points_and_order():
    table = oracle.shifted_table()
    assert table[0] == 1.0 and table[-1] == 0.0
    assert all(a > b for a, b in zip(table, table[1:]))


def test_shift_one_is_the_linear_table():
    assert oracle.shifted_table(8, 1.0) == pytest.approx([1 - k / 8 for k in range(9)], abs=1e-15)


def test_routes_follow_the_pages():
    g = golden()
    for name in ("up3", "up4", "hf8"):
        start, _, steps = g[f"{name}_start"]
        r = oracle.ic_route(name)
        assert r[0] == float(start)
        assert len(r) == int(steps) + 1 and r[-1] == 0.0
        assert all(a > b for a, b in zip(r, r[1:]))
    # hf8 is the whole table; up4 shares its last four targets
    assert oracle.ic_route("hf8") == oracle.shifted_table()
    assert oracle.ic_route("up4")[1:] == oracle.shifted_table()[-4:]
    assert oracle.REFERENCE_ROW_SIGMA == float(g["reference_row_sigma"][0])


def test_package_schedules_equal_the_oracles():
    assert schedules.shifted_table() == pytest.approx(oracle.shifted_table(), abs=1e-15)
    for name in ("up3", "up4", "hf8"):
        assert schedules.route(name) == pytest.approx(oracle.ic_route(name), abs=1e-15)
    assert schedules.REFERENCE_ROW_SIGMA == oracle.REFERENCE_ROW_SIGMA
    assert tuple(schedules.REFINE) == tuple(oracle.SIGMAS)
    with pytest.raises(ValueError):
        schedules.route("up5")


def test_up3_start_is_not_a_table_point():
    """The pages' up3 start 0.835 does not lie on the shift-12 table (whose last-three
    start is 0.878): the route mixes to the printed value instead."""
    table = oracle.shifted_table()
    assert all(abs(x - 0.835) > 0.03 for x in table)
    assert round(table[5], 3) == 0.878
