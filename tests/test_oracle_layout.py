"""Pins for the oracle's layout algebra (oracle/layout_ref.py).

Each check is fixed by something other than the oracle itself: values the
Tylo.jl pages print (tests/golden/layout_pages.json), the pages' closed form for
128-byte swizzled rows, and brute-force properties that any correct
implementation of the stated semantics must have.

Parity unpinned: the element offsets of the 64-byte and 32-byte swizzle rows
(SharedTilePlan with row_bytes 64 or 32, i.e. Swizzle{2,M,3} and Swizzle{1,M,3}).
No page prints an offset for them, so only invariants check them here
(bijection onto the tile, involution, the low M bits kept, 16-byte chunks kept
whole); the planner's C++ copy of the plan is compared with this oracle, not
with the pages.
"""
import random

import pytest

from golden_cases import layout_cases, tup
from oracle import layout_ref as L

CASES = layout_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_page_values(case):
    k = case["kind"]
    if k == "eval":
        assert L.Layout(tup(case["shape"]), tup(case["stride"]))(tup(case["coord"])) == case["expect"]
    elif k == "tile_eq":
        l = L.Layout(tup(case["shape"]), tup(case["stride"]))
        t = L.tile(l, tup(case["tile"]))
        assert t(tup(case["tiled_coord"])) == l(tup(case["flat_coord"]))
    elif k == "permute_eq":
        l = L.Layout(tup(case["shape"]), tup(case["stride"]))
        assert L.permutedims(l)(tup(case["permuted_coord"])) == l(tup(case["coord"]))
    elif k == "swizzle_window_eq":
        l = L.compose(L.Swizzle(*case["swizzle"]), L.Layout(tup(case["shape"]), tup(case["stride"])))
        w = L.window(l, tup(case["origin"]), tup(case["wshape"]))
        assert w(tup(case["wcoord"])) == l(tup(case["coord"]))
    elif k == "tile_plan":
        p = L.SharedTilePlan(case["elem_bytes"], tup(case["shape"]), case["inner_axis"], case["row_bytes"])
        if "transfer_bytes" in case:
            assert p.transfer_bytes() == case["transfer_bytes"]
        if "probe" in case:
            assert p.shared_layout()(tup(case["probe"])) == case["probe_offset"]
        if "swizzle_bytes" in case:
            assert p.swizzle_bytes() == case["swizzle_bytes"]
        if "size" in case:
            assert p.size() == tup(case["size"])
    elif k == "closed_form_128B":
        rows, cols = case["rows"], case["cols"]
        for r0 in range(0, rows, 64):
            plan = L.SharedTilePlan(2, (64, cols), 2, 128)
            f = plan.shared_layout()
            for r in range(64):
                for kk in range(cols):
                    rr = r0 + r
                    # a taller tile continues the same map; evaluate through the base row
                    expect = 64 * rr + (kk ^ (8 * (rr % 8)))
                    assert f((r, kk)) + 64 * r0 == expect
    else:
        raise AssertionError(k)


def test_integer_coordinate_is_first_mode_fastest():
    # Brute force: walk a nested-loop enumeration with the FIRST mode innermost;
    # its running counter must equal the integer coordinate.
    shape, stride = ((3, 4), 5), ((7, 1), 40)
    l = L.Layout(shape, stride)
    i = 0
    for c1 in range(5):
        for b in range(4):
            for a in range(3):
                assert l(i) == l(((a, b), c1)) == a * 7 + b * 1 + c1 * 40
                i += 1
    # the flat 2-D pin: index 3 + 16*7 is coordinate (3, 7) of a 16x32 layout
    assert L.Layout((16, 32), (32, 1))(3 + 16 * 7) == 103


def test_tile_roundtrip_bruteforce():
    rng = random.Random(7)
    for _ in range(20):
        s0, s1 = rng.choice([4, 8, 12, 16]), rng.choice([6, 8, 16, 24])
        d0, d1 = rng.randint(1, 50), rng.randint(1, 50)
        t0 = rng.choice([t for t in (1, 2, 4) if s0 % t == 0])
        t1 = rng.choice([t for t in (1, 2, 3) if s1 % t == 0])
        l = L.Layout((s0, s1), (d0, d1))
        t = L.tile(l, (t0, t1))
        for i0 in range(s0):
            for i1 in range(s1):
                assert t(((i0 % t0, i0 // t0), (i1 % t1, i1 // t1))) == l((i0, i1))
    with pytest.raises(ValueError):
        L.tile(L.Layout((6, 8), (8, 1)), (4, 4))


def test_coalesce_preserves_function():
    rng = random.Random(11)
    for _ in range(200):
        rank = rng.randint(1, 4)
        shape = tuple(rng.choice([1, 1, 2, 3, 4]) for _ in range(rank))
        stride = []
        run = 1
        for s in shape:
            stride.append(run if rng.random() < 0.6 else rng.randint(0, 30))
            run = stride[-1] * s
        l = L.Layout(shape, tuple(stride))
        c = L.coalesce(l)
        assert c.size() == l.size()
        for i in range(l.size()):
            assert c(i) == l(i)
        assert all(s != 1 for s in L.leaves(c.shape)) or c.shape == 1
    assert repr(L.coalesce(L.Layout((2, (1, 6)), (1, (7, 2))))) == "12:1"


def test_swizzle_bijective_involution_and_low_bits():
    for B, M, S in [(3, 3, 3), (2, 3, 2), (2, 4, 3), (1, 2, 4), (0, 3, 3), (3, 0, 5)]:
        sw = L.Swizzle(B, M, S)
        period = sw.period()
        image = [sw(o) for o in range(4 * period)]
        assert sorted(image) == list(range(4 * period))          # bijection
        assert all(sw(sw(o)) == o for o in range(4 * period))    # involution
        low = (1 << M) - 1
        assert all((sw(o) & low) == (o & low) for o in range(4 * period))
    for bad in [(3, 3, 2), (2, 0, 1), (-1, 3, 3)]:
        with pytest.raises(ValueError):
            L.Swizzle(*bad)


def test_windows_keep_parent_offsets_and_nest():
    l = L.compose(L.Swizzle(3, 3, 3), L.Layout((64, 64), (64, 1)))
    w = L.window(l, (8, 16), (32, 32))
    ww = L.window(w, (4, 8), (8, 8))
    for r in range(8):
        for c in range(8):
            assert ww((r, c)) == w((4 + r, 8 + c)) == l((12 + r, 24 + c))
    # restarting the swizzle at the window's first offset describes other storage
    base = l((8, 16))
    restarted = L.compose(L.Swizzle(3, 3, 3), L.Layout((32, 32), (64, 1)))
    assert any(w((r, c)) != base + restarted((r, c)) for r in range(32) for c in range(32))
    with pytest.raises(IndexError):
        L.window(l, (40, 0), (32, 8))


def test_cosize_closed_form_matches_enumeration():
    # affine layouts with non-negative strides: 1 + sum (s-1)*d
    rng = random.Random(3)
    for _ in range(100):
        shape = tuple(rng.randint(1, 5) for _ in range(3))
        stride = tuple(rng.randint(0, 20) for _ in range(3))
        l = L.Layout(shape, stride)
        assert L.cosize(l) == 1 + sum((s - 1) * d for s, d in zip(shape, stride))
    # a window counts the parent's prefix
    l = L.Layout((16, 16), (16, 1))
    assert L.cosize(L.window(l, (4, 4), (4, 4))) == 1 + 7 * 16 + 7
