"""Host-side tests of the C ABI library (no GPU needed, no kernel launched).

* the library loads and exports every symbol the headers in include/ declare;
* the planner's layout algebra reproduces the pages' printed values and
  agrees with the oracle's independent Python layout reference;
* plans for every workload build and describe themselves; invalid requests
  are rejected with the documented status before anything is launched.
"""
import ctypes
import os
import random
import re

import pytest

import layout_algebra_amd as la
from golden_cases import layout_cases, tup
from oracle import layout_ref as L
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    text = ""
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            with open(os.path.join(ROOT, "include", name)) as f:
                text += f.read()
    declared = set(re.findall(r"^\s*(?:gemm_status|void|const char\*)\s+(\w+)\s*\(", text, re.M))
    assert declared, "no declarations parsed"
    lib = la.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(la.EXPORTED_SYMBOLS)


@pytest.mark.parametrize("case", [c for c in layout_cases() if c["kind"] in ("eval", "tile_plan", "closed_form_128B")],
                         ids=lambda c: c["id"])
def test_page_values_through_the_c_abi(case):
    if case["kind"] == "eval":
        shape, stride, coord = tup(case["shape"]), tup(case["stride"]), tup(case["coord"])
        # the pages' notation, nested as printed (no flattening)
        assert la.la_layout_eval_str((shape, stride), coord) == case["expect"]
        if any(isinstance(s, tuple) for s in shape):
            # and through the flat-array entry point: ((8,4),5) -> (8,4,5)
            fs, fd, fc = L.leaves(shape), L.leaves(stride), L.leaves(coord)
            assert la.la_layout_eval(fs, fd, fc) == case["expect"]
        else:
            assert la.la_layout_eval(shape, stride, coord) == case["expect"]
    elif case["kind"] == "tile_plan":
        if "probe" in case:
            off, tb = la.la_tile_plan_offset(case["elem_bytes"], case["shape"], case["inner_axis"],
                                             case["row_bytes"], case["probe"])
            assert off == case["probe_offset"]
            assert tb == case["transfer_bytes"]
        else:
            off, tb = la.la_tile_plan_offset(case["elem_bytes"], case["shape"], case["inner_axis"],
                                             case["row_bytes"], (0, 0))
            assert tb == case["shape"][0] * case["shape"][1] * case["elem_bytes"]
    else:
        for r in range(64):
            for k in range(64):
                off, _ = la.la_tile_plan_offset(2, (64, 64), 2, 128, (r, k))
                assert off == 64 * r + (k ^ (8 * (r % 8)))


def test_swizzle_matches_reference_and_rejects_overlap():
    rng = random.Random(5)
    for B, M, S in [(3, 3, 3), (2, 3, 2), (2, 4, 3), (1, 2, 4), (0, 3, 3), (3, 0, 5)]:
        ref = L.Swizzle(B, M, S)
        for _ in range(500):
            o = rng.randrange(0, 1 << 20)
            assert la.la_swizzle_apply(B, M, S, o) == ref(o)
    with pytest.raises(la.GemmError) as e:
        la.la_swizzle_apply(3, 3, 2, 1)
    assert e.value.name == "GEMM_ERR_INVALID_ARG"


def test_layout_eval_matches_reference_on_random_layouts():
    rng = random.Random(9)
    for _ in range(200):
        rank = rng.randint(1, 4)
        shape = [rng.randint(1, 6) for _ in range(rank)]
        stride = [rng.randint(0, 40) for _ in range(rank)]
        ref = L.Layout(tuple(shape), tuple(stride))
        for _ in range(10):
            idx = rng.randrange(0, ref.size())
            coord = L.split_index(idx, tuple(shape))
            assert la.la_layout_eval_index(shape, stride, idx) == ref(idx)
            assert la.la_layout_eval(shape, stride, list(coord)) == ref(idx)
    with pytest.raises(la.GemmError):
        la.la_layout_eval([4, 4], [4, 1], [4, 0])


@pytest.mark.parametrize("case", [c for c in layout_cases() if c["kind"] in ("tile_eq", "permute_eq", "swizzle_window_eq")],
                         ids=lambda c: c["id"])
def test_page_equalities_through_the_c_abi(case):
    """tile(), permutedims and a swizzled window, as the pages print them, through the C ABI."""
    lay = (tup(case["shape"]), tup(case["stride"]))
    if case["kind"] == "tile_eq":
        tiled = la.la_layout_tile_str(lay, tup(case["tile"]))
        got = la.la_layout_eval_str(tiled, tup(case["tiled_coord"]))
        assert got == la.la_layout_eval_str(lay, tup(case["flat_coord"])) == 375
    elif case["kind"] == "permute_eq":
        perm = la.la_layout_permute_str(lay)
        assert la.la_layout_eval_str(perm, tup(case["permuted_coord"])) == la.la_layout_eval_str(lay, tup(case["coord"]))
    else:
        sw, ext = tup(case["swizzle"]), L.Layout(*lay).top_extents()
        w = la.la_view_window_eval(sw, lay, tup(case["origin"]), tup(case["wshape"]), tup(case["wcoord"]))
        whole = la.la_view_window_eval(sw, lay, (0,) * len(ext), ext, tup(case["coord"]))
        assert w == whole == 115


def _random_tree(rng, depth=0):
    if depth >= 2 or rng.random() < 0.6:
        return rng.randint(1, 5)
    return tuple(_random_tree(rng, depth + 1) for _ in range(rng.randint(2, 3)))


def _strides_like(rng, shape):
    if isinstance(shape, int):
        return rng.randint(0, 60)
    return tuple(_strides_like(rng, s) for s in shape)


def _as_text(x):
    return "(" + ",".join(_as_text(v) for v in x) + ")" if isinstance(x, tuple) else str(x)


def _map_of(text_layout, n):
    return [la.la_layout_eval_str(text_layout, str(i)) for i in range(n)]


def test_nested_algebra_matches_the_reference():
    """Random nested layouts: evaluation (natural coordinates and integer indices), tile(),
    coalesce(), permutedims and cosize through the C ABI against the oracle's enumeration."""
    rng = random.Random(23)
    for _ in range(150):
        rank = rng.randint(1, 3)
        shape = tuple(_random_tree(rng) for _ in range(rank)) if rank > 1 else _random_tree(rng)
        stride = _strides_like(rng, shape)
        ref = L.Layout(shape, stride)
        text = _as_text(shape) + ":" + _as_text(stride)
        n = ref.size()
        if n > 300:
            continue
        for i in range(n):
            assert la.la_layout_eval_str(text, str(i)) == ref(i)
            assert la.la_layout_eval_str(text, _as_text(L.split_index(i, shape))) == ref(i)
        # coalesce: the same map on [0, size), and the oracle's reduced modes
        co = la.la_layout_coalesce_str(text)
        rco = L.coalesce(ref)
        assert co == _as_text(rco.shape) + ":" + _as_text(rco.stride)
        assert _map_of(co, n) == [ref(i) for i in range(n)]
        # permutedims: a coordinate with its top-level modes reversed maps to the same offset
        if rank > 1:
            pe = la.la_layout_permute_str(text)
            rp = L.permutedims(ref)
            assert pe == _as_text(rp.shape) + ":" + _as_text(rp.stride)
        assert la.la_layout_cosize_str(text) == L.cosize(ref)
    # tile(): flat modes, divisors
    for _ in range(100):
        rank = rng.randint(1, 3)
        tiles = [rng.choice([1, 2, 3, 4]) for _ in range(rank)]
        shape = tuple(t * rng.randint(1, 4) for t in tiles)
        stride = tuple(rng.randint(0, 50) for _ in range(rank))
        ref = L.tile(L.Layout(shape if rank > 1 else shape[0], stride if rank > 1 else stride[0]), tiles)
        got = la.la_layout_tile_str(_as_text(shape) + ":" + _as_text(stride), tiles)
        assert got == _as_text(ref.shape) + ":" + _as_text(ref.stride)
    with pytest.raises(la.GemmError):
        la.la_layout_tile_str("(6,4):(4,1)", [4, 2])           # 4 does not divide 6
    with pytest.raises(la.GemmError):
        la.la_layout_eval_str("((8,4),5):((1,8),128)", "((8,0),0)")   # outside the mode
    with pytest.raises(la.GemmError):
        la.la_layout_eval_str("(8,4):(1,8", "(0,0)")           # malformed text
    with pytest.raises(la.GemmError):
        la.la_view_window_eval((2, 3, 2), "(32,32):(32,1)", (20, 0), (16, 16), (0, 0))   # window leaves the parent


@pytest.mark.parametrize("name", ["square4096", "gate_up", "ragged", "skinny", "square256"])
def test_plans_describe_global_views_copies_and_stores(name):
    """Each plan tiles its operands' global views, checks and coalesces the copy of one wave
    instruction, and checks its store plan on every class of tile."""
    w = synth.WORKLOADS[name]
    code = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}
    d = la.gemm_plan(w.M, w.N, w.K, code[w.in_kind], code[w.out_kind], gate_up=w.gate_up).describe()
    bm, bn, bk = d["tile"]
    # the tiled global view of A: ((BM, M/BM), (BK, K/BK)) : ((lda, BM lda), (1, BK)) over the covering extents
    ga = L.Layout(*_split_layout(d["global_a"]))
    tm, tk = min(1, d["tiles"][0] - 1), min(1, (w.K + bk - 1) // bk - 1)
    assert ga(((3, tm), (5, tk))) == (3 + tm * bm) * d["lda"] + 5 + tk * bk
    # copy runs: a wave instruction reads whole rows of the block (coalesced)
    for op in ("A", "B"):
        c = d["copy"][op]
        assert c["run_bytes"] >= 64 and c["instrs_per_block"] >= 1
    assert d["store"]["tile_classes_checked"] >= (1 if d["tiles"] == [1, 1] else 2)
    assert d["store"]["run_bytes"] >= 64


def _split_layout(text):
    """"shape:stride" text -> (shape, stride) as ints / nested tuples."""
    import ast
    depth = 0
    for i, ch in enumerate(text):
        depth += ch == "("
        depth -= ch == ")"
        if ch == ":" and depth == 0:
            return ast.literal_eval(text[:i]), ast.literal_eval(text[i + 1:])
    raise ValueError(text)


def test_tile_plan_rejects_what_the_page_forbids():
    for args in [(3, (64, 64), 2, 128), (2, (64, 32), 2, 128), (2, (12, 64), 2, 128),
                 (2, (512, 64), 2, 128), (2, (64, 64), 2, 96)]:
        with pytest.raises(la.GemmError):
            la.la_tile_plan_offset(args[0], args[1], args[2], args[3], (0, 0))


CODES = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32, "f8e4m3": la.F8E4M3, "f8e5m2": la.F8E5M2}


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_plans_build(name):
    w = synth.WORKLOADS[name]
    p = la.gemm_plan(w.M, w.N, w.K, CODES[w.in_kind], CODES[w.out_kind], gate_up=w.gate_up, b_kmajor=w.b_kmajor)
    d = p.describe()
    assert d["m"] == w.M and d["n"] == w.N and d["k"] == w.K
    assert d["lds_bytes"] <= 163840
    assert d["grid"] >= 1


@pytest.mark.parametrize("shape", [(4096, 4096, 4096, False), (1000, 1537, 999, False), (4096, 11008, 4096, True)],
                         ids=["fast", "tiled", "fast_gate_up"])
def test_planner_lds_map_agrees_with_reference(shape):
    m, n, k, gu = shape
    p = la.gemm_plan(m, n, k, la.BF16, la.BF16, gate_up=gu)
    d = p.describe()
    bm, bn, bk = d["tile"]
    a_ref = L.compose(L.Swizzle(*d["swizzle_a"]), L.Layout((bm, bk), (bk, 1)))
    if d["lds_b"] == "(%d,%d):(1,%d)" % (bk, bn, bk):          # K-contiguous B block
        b_ref = L.compose(L.Swizzle(*d["swizzle_b"]), L.Layout((bk, bn), (1, bk)))
    else:                                                      # N-contiguous B block
        assert d["lds_b"] == "(%d,%d):(%d,1)" % (bk, bn, bn)
        b_ref = L.compose(L.Swizzle(*d["swizzle_b"]), L.Layout((bk, bn), (bn, 1)))
    seen = set()
    for r in range(bm):
        for c in range(bk):
            o = la.gemm_plan_lds_offset(p, 0, r, c)
            assert o == a_ref((r, c))
            seen.add(o)
    for operand in ([1, 2] if gu else [1]):
        base = bm * bk + (operand - 1) * bk * bn
        for r in range(bk):
            for c in range(bn):
                o = la.gemm_plan_lds_offset(p, operand, r, c)
                assert o == base + b_ref((r, c))
                seen.add(o)
    assert len(seen) == d["stage_elems"]


def test_invalid_requests_are_rejected():
    bad = [dict(m=-1, n=4, k=4), dict(m=4, n=4, k=4, lda=3), dict(m=4, n=4, k=4, ldb=2),
           dict(m=4, n=4, k=4, ldc=1)]
    for kw in bad:
        with pytest.raises(la.GemmError) as e:
            la.gemm_plan(**kw)
        assert e.value.name == "GEMM_ERR_INVALID_ARG"
    # binary32 inputs: plain GEMMs only, and never mixed with 16-bit inputs
    with pytest.raises(la.GemmError, match="plain GEMMs only") as e:
        la.gemm_plan(4, 4, 4, la.F32, la.F32, gate_up=True)
    assert e.value.name == "GEMM_ERR_UNSUPPORTED"
    lib = la._lib
    for a_t, b_t in ((la.BF16, la.F32), (la.F32, la.F16), (la.BF16, la.F16)):
        d = lib._Desc(4, 4, 4, a_t, b_t, la.F32, 4, 4, 4, 0, 1, 16, 16, 16)
        h = ctypes.c_void_p()
        assert lib.load().gemm_plan(ctypes.byref(d), ctypes.byref(h)) == 3, (a_t, b_t)   # GEMM_ERR_UNSUPPORTED
        assert not h.value
    # a grid of more than 2^32 work-items along x does not fit one launch (8,388,608 tiles of
    # 256 x 256 at 512 threads each is exactly 2^32); a tile row fewer plans
    with pytest.raises(la.GemmError, match="too many tiles") as e:
        la.gemm_plan(256 * 4096, 256 * 2048, 64, la.BF16, la.BF16)
    assert e.value.name == "GEMM_ERR_UNSUPPORTED"
    assert la.gemm_plan_describe(la.gemm_plan(256 * 4096, 256 * 2047, 64, la.BF16, la.BF16))["kernel"].startswith("fast")


def test_skinny_rows_and_grid_guard():
    """M <= 32 always streams B through the skinny kernel; 33 <= M <= 128 only on grids of at
    least 128 column strips (64-column strips for B stored [N, K] up to 64 rows, else 128)."""
    def kern(m, n, k, km=False, t=la.BF16):
        return la.gemm_plan(m, n, k, t, la.F32, b_kmajor=km).describe()["kernel"]
    assert kern(32, 4096, 14336).startswith("skinny_32x128x")
    assert kern(32, 4096, 14336, True).startswith("skinny_bkmajor_32x64x")
    assert kern(64, 4096, 14336).startswith("tiled_64x64")
    assert kern(64, 4096, 14336, True).startswith("tiled_64x64")
    assert kern(64, 8192, 4096, True).startswith("skinny_bkmajor_64x64x")    # 128 strips
    assert kern(64, 8192, 4096).startswith("tiled_64x64")                   # 64 strips
    assert kern(64, 16384, 4096).startswith("skinny_64x128x")
    assert kern(65, 28672, 8192).startswith("skinny_128x128x64")
    assert kern(128, 28672, 8192, True).startswith("skinny_bkmajor_128x128x64")
    assert kern(128, 28672, 8192, True, la.F8E4M3).startswith("skinny_f8_128x128x128")
    assert kern(129, 28672, 8192).startswith("tiled_64x64")
    assert kern(128, 28672, 8160).startswith("tiled_")                      # K not a multiple of 64


def test_split_form_workspace_bound():
    """Every split form the planner makes fits the 64 MiB array of gemm_run_split_noalloc:
    workspace = split * m * n * 4 with at most 256 workgroups of at most 128 x 256 outputs (skinny
    strips x split at most 256, 512 for 16 rows; 128-row tiles x split at most 256)."""
    worst = 0
    kinds = set()
    for m in (1, 16, 17, 32, 33, 64, 65, 100, 128, 129, 192, 256, 300, 512, 1000, 1024, 2048):
        for n in (64, 1024, 4096, 8128, 8192, 11008, 16320):
            for k in (1024, 4096, 14336, 65536):
                for km in (False, True):
                    try:
                        d = la.gemm_plan(m, n, k, la.BF16, la.F32, b_kmajor=km).describe()
                    except la.GemmError:
                        continue
                    assert d["workspace_bytes"] == (d["split_k"] * m * n * 4 if d["split_k"] > 1 else 0), d
                    if d["split_k"] > 1:
                        sk = d["split_kernel"]
                        kinds.add(sk.split("_")[0])
                        wgs = d["split_grid"][0] * d["split_grid"][1]
                        if sk.startswith("skinny"):
                            assert m <= 128 and wgs <= (512 if sk.startswith(("skinny_bkmajor_16x", "skinny_f8_16x")) else 256), d
                        else:
                            assert sk.startswith(("fast_128x256", "fast_bkmajor_128x256")) and wgs <= 256, d
                            assert d["split_k"] <= 8 and k % (32 * d["split_k"]) == 0 and n % 8 == 0, d
                            assert k // d["split_k"] >= 1024 and k % (d["split_k"] * int(sk.rsplit("x", 1)[1])) == 0, d
                    worst = max(worst, d["workspace_bytes"])
    assert kinds == {"skinny", "fast"}
    assert 0 < worst <= 64 << 20


def test_fast_split_form_and_padding_rule():
    """The 256-wide kernel's split form on grids of at most 64 tiles; edge tiles padded up to 4/3
    kept on the 256-wide kernel from 80 tiles on; 128-row tiles for grids of at most 128 tiles."""
    def plan(m, n, k, km=False):
        return la.gemm_plan(m, n, k, la.BF16, la.BF16, b_kmajor=km).describe()
    d = plan(512, 4096, 14336, True)
    assert d["kernel"] == "fast_bkmajor_128x256x64" and d["split_k"] == 4 and d["split_grid"] == [64, 4]
    assert d["split_kernel"] == "fast_bkmajor_128x256x64"
    d = plan(256, 4096, 14336)
    assert d["kernel"].startswith("tiled_64x64") and d["split_k"] == 8 and d["split_kernel"] == "fast_128x256x64"
    d = plan(300, 520, 2048)                                                     # ranges of 1024
    assert d["split_k"] == 2 and d["split_kernel"] == "fast_128x256x64" and d["split_grid"] == [9, 2]
    d = plan(300, 520, 2112)                                                     # ranges of 33 blocks of 32
    assert d["split_k"] == 2 and d["split_kernel"] == "fast_128x256x32"
    d = plan(1024, 4096, 14336)
    assert d["split_k"] == 2 and d["split_grid"] == [128, 2]
    assert plan(512, 11008, 4096)["split_k"] == 1                               # 172 tiles of 128 rows
    assert plan(4096, 4096, 4096)["split_k"] == 1
    assert plan(512, 4096, 512)["split_k"] == 1                                 # ranges under 1024
    assert plan(384, 28672, 8192)["kernel"].startswith("fast_256x256")          # 224 tiles, padding 4/3
    assert plan(384, 11008, 4096)["kernel"].startswith("fast_128x256")          # 86 tiles of 256 rows
    assert plan(192, 11008, 4096)["kernel"].startswith("tiled_64x64")           # 43 tiles
    assert plan(320, 28672, 8192)["kernel"].startswith("tiled_64x64")           # padding 1.6
    d = la.gemm_plan(512, 4096, 14336, la.F8E4M3, la.BF16, b_kmajor=True).describe()
    assert d["kernel"] == "fast_f8_128x256x128" and d["split_k"] == 4 and d["split_kernel"] == "fast_f8_128x256x128"
    assert plan(192, 28672, 8192)["kernel"] == "fast_128x256x64"                 # 112 tiles of 256 rows
    f8 = lambda m, n, k: la.gemm_plan(m, n, k, la.F8E4M3, la.BF16, b_kmajor=True).describe()["kernel"]
    assert f8(1024, 4096, 2048) == "fast_f8_128x256x128" and f8(1024, 4096, 1040) == "fast_f8_128x256x64" and f8(4096, 4096, 4096) == "fast_f8_256x256x64"
    assert f8(256, 256, 64) == "fast_f8_256x256x64"                             # small grid: no one-byte general kernel
    assert plan(1000, 4096, 1000, True)["kernel"] == "fast_bkmajor_128x256x32"  # K not a multiple of 64
    assert plan(2048, 4096, 4096, True)["kernel"] == "fast_bkmajor_128x256x64"   # 128 tiles
    assert plan(1024, 11008, 4096)["kernel"] == "fast_256x256x32"                # 172 tiles
    assert plan(4096, 4096, 4096)["kernel"] == "fast_256x256x32"
    d = la.gemm_plan(2048, 1024, 512, la.BF16, la.BF16, large_tiles=True).describe()
    assert d["kernel"] == "fast_256x256x32"                                      # pinned: the largest tile
    assert la.gemm_plan(256, 256, 256, la.BF16, la.BF16, batch=64).describe()["kernel"] == "fast_128x256x64"


def test_small_grids_take_64x64_tiles_unless_pinned():
    """Kernel choice by grid size: a grid that would leave most of the 256 CUs idle moves to
    64 x 64 tiles of the general kernel; GEMM_FLAG_LARGE_TILES keeps the largest tile."""
    def kern(m, n, k, t=la.BF16, **kw):
        return la.gemm_plan(m, n, k, t, la.F32, **kw).describe()
    # full tiles: below 32 workgroups of 256 x 256 (256^3: 1, 1024 x 1536: 24), from 32 on kept
    for shape in ((256, 256, 256), (1024, 1536, 1024)):
        assert kern(*shape)["kernel"].startswith("tiled_64x64"), shape
        assert kern(*shape, large_tiles=True)["kernel"].startswith("fast_256x256"), shape
    assert kern(2048, 1024, 512)["kernel"].startswith("fast_128x256")          # 32 workgroups (128-row tiles)
    assert kern(256, 256, 256, batch=32)["kernel"].startswith("fast_128x256")  # batch counts
    assert kern(512, 512, 128, gate_up=True)["kernel"].startswith("tiled_64x64")
    # edge tiles on the full-tile kernel: M and N inside a tile, K ending inside a K block from
    # K = 256 on, padding within 1.3x and at least 64 workgroups
    assert kern(4000, 4000, 1000)["kernel"].startswith("fast_256x256")       # 256 tiles
    assert kern(4000, 4000, 200)["kernel"].startswith("tiled_64x64")          # short K with a tail
    assert kern(1088, 1920, 512)["kernel"].startswith("tiled_64x64")         # 40 edge tiles
    assert kern(1088, 1920, 512, large_tiles=True)["kernel"].startswith("fast_256x256")
    assert kern(300, 520, 96)["kernel"].startswith("tiled_")                 # 2.5x padding
    assert kern(300, 520, 96, large_tiles=True)["kernel"].startswith("fast_256x256")
    assert kern(4000, 4004, 1024)["kernel"].startswith("tiled_")             # B rows cut inside a chunk
    assert kern(4000, 4004, 1024, b_kmajor=True, ldc=4008)["kernel"].startswith("fast_bkmajor")  # C rows on 16 bytes
    # general kernel with 16-byte loads: 64 x 64 at any grid
    d = kern(4000, 4000, 200)
    assert d["kernel"].startswith("tiled_64x64") and d["vec_elems"] == 8
    assert kern(4000, 4000, 200, large_tiles=True)["kernel"].startswith("tiled_128x128")
    # rows on 16 bytes with whole chunks: aligned 16-byte loads
    assert kern(1000, 1536, 1024)["vec_elems"] == 8 and kern(1000, 1536, 1024)["align_bytes"] == 16
    # ragged shapes keep 16-byte loads at 2-byte alignment (a chunk cut by an edge loads the 8
    # elements ending at its last valid one)
    for shape in ((2000, 3074, 999), (1536, 1537, 999), (512, 512, 1001), (512, 516, 1000)):
        d = kern(*shape, la.F16)
        assert d["kernel"].startswith("tiled_64x64") and d["vec_elems"] == 2 and d["align_bytes"] == 2, shape
    # rows of at most 8 elements that are not whole chunks take 2-byte loads: 128 x 128 from 384 of its
    # workgroups on (4000 x 4000: 1024), 64 x 64 below
    d = kern(4000, 4000, 7)
    assert d["kernel"].startswith("tiled_128x128") and d["vec_elems"] == 1
    assert kern(1000, 1537, 7)["kernel"].startswith("tiled_64x64")
    assert kern(512, 6, 1000)["vec_elems"] == 1
    assert kern(512, 6, 1000, b_kmajor=True)["vec_elems"] == 8          # K-major B: chunks run along K
    assert kern(512, 512, 8)["vec_elems"] == 8 and kern(512, 512, 9)["vec_elems"] == 2
    # the flag is a known bit
    assert la.FLAG_LARGE_TILES == 0x4


def test_batch_descriptor_is_validated():
    """Batch count and strides: a batch of independent matrices, each addressed by a
    third origin coordinate (Tylo.jl, "TMA and Hopper WGMMA", section "The same
    storage contract on both sides")."""
    bad = [dict(batch=0), dict(batch=65536), dict(batch=2, stride_a=-8),
           dict(batch=2, stride_c=64 * 64 - 1)]          # matrix 1 of C would overlap matrix 0
    for kw in bad:
        with pytest.raises(la.GemmError) as e:
            la.gemm_plan(64, 64, 64, la.BF16, la.F32, **kw)
        assert e.value.name == "GEMM_ERR_INVALID_ARG", kw
    # inputs may alias: stride 0 broadcasts one B to every matrix of the batch
    d = la.gemm_plan(4096, 4096, 4096, la.BF16, la.BF16, batch=3, stride_b=0).describe()
    assert d["batch"] == 3 and d["kernel"].startswith("fast_") and d["align_bytes"] == 16
    # a stride that is not a multiple of 8 elements leaves the 16-byte class
    d = la.gemm_plan(256, 256, 256, la.BF16, la.BF16, batch=2, stride_a=256 * 256 + 4).describe()
    assert d["kernel"].startswith("tiled") and d["align_bytes"] == 2
    # the same stride is ignored for a single matrix
    d = la.gemm_plan(256, 256, 256, la.BF16, la.BF16, batch=1, stride_a=256 * 256 + 4, large_tiles=True).describe()
    assert d["kernel"].startswith("fast_")
    d = la.gemm_plan(256, 256, 256, la.BF16, la.BF16, batch=2, stride_c=256 * 256 + 4).describe()
    assert d["kernel"].startswith("tiled") and d["align_bytes"] == 16 and d["out_align_bytes"] == 2


def test_run_argument_errors_are_caught_before_launch():
    lib = la.load()
    p = la.gemm_plan(64, 64, 64, la.BF16, la.F32)
    vp = ctypes.c_void_p
    # misaligned A for the full-tile kernel's 16-byte alignment class: rejected on the host
    pf = la.gemm_plan(256, 256, 64, la.BF16, la.F32, large_tiles=True)
    assert pf.describe()["align_bytes"] == 16
    rc = lib.gemm_run(pf.handle, vp(0x1002), vp(0x2000), vp(0x3000), 1.0, 0.0, vp(0))
    assert la._lib.STATUS[rc] == "GEMM_ERR_ALIGNMENT"
    # with 2-byte aligned rows the general kernel takes any element-aligned pointer, but not an odd
    # byte address
    p2 = la.gemm_plan(64, 64, 63, la.BF16, la.F32)
    assert p2.describe()["align_bytes"] == 2
    rc = lib.gemm_run(p2.handle, vp(0x1001), vp(0x2000), vp(0x3000), 1.0, 0.0, vp(0))
    assert la._lib.STATUS[rc] == "GEMM_ERR_ALIGNMENT"
    rc = lib.gemm_run(p.handle, vp(0x1000), vp(0), vp(0x3000), 1.0, 0.0, vp(0))
    assert la._lib.STATUS[rc] == "GEMM_ERR_NULL"
    rc = lib.gemm_gate_up_run(p.handle, vp(0x1000), vp(0x1000), vp(0x1000), vp(0x1000), vp(0x1000), vp(0))
    assert la._lib.STATUS[rc] == "GEMM_ERR_INVALID_ARG"
    # m == 0 is a no-op success that never touches the pointers
    p0 = la.gemm_plan(0, 64, 64, la.BF16, la.F32)
    assert lib.gemm_run(p0.handle, vp(0), vp(0), vp(0), 1.0, 0.0, vp(0)) == 0
    # tile index outside the grid for the debug image
    rc = lib.gemm_debug_lds_image(p.handle, vp(0x1000), vp(0x1000), vp(0), 5, 0, vp(0x1000), vp(0))
    assert la._lib.STATUS[rc] == "GEMM_ERR_INVALID_ARG"


def test_rms_norm_argument_errors_are_caught_before_launch():
    lib = la.load()
    vp = ctypes.c_void_p
    st = la._lib.STATUS

    def call(m=8, d=256, xt=la.F32, yt=la.F32, X=0x10000, ldx=256, G=0x80000, Y=0x40000, ldy=256, eps=1e-6):
        return st[lib.la_rms_norm_run(m, d, xt, yt, vp(X), ldx, vp(G), vp(Y), ldy, eps, vp(0))]

    assert call(xt=7) == "GEMM_ERR_INVALID_ARG"
    assert call(m=-1) == "GEMM_ERR_INVALID_ARG"
    assert call(ldx=255) == "GEMM_ERR_INVALID_ARG"
    assert call(ldy=0) == "GEMM_ERR_INVALID_ARG"
    assert call(eps=-1.0) == "GEMM_ERR_INVALID_ARG"
    assert call(eps=float("nan")) == "GEMM_ERR_INVALID_ARG"
    assert call(eps=float("inf")) == "GEMM_ERR_INVALID_ARG"
    assert call(d=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1) == "GEMM_ERR_UNSUPPORTED"
    assert call(G=0) == "GEMM_ERR_NULL"
    assert call(X=0x10002) == "GEMM_ERR_ALIGNMENT"                  # f32 X on a 2-byte boundary
    assert call(Y=0x10000 + 1024) == "GEMM_ERR_INVALID_ARG"         # Y overlaps X, shifted by one row
    assert call(Y=0x10000, ldy=512) == "GEMM_ERR_INVALID_ARG"       # same start, other rows
    assert call(Y=0x10000, yt=la.BF16) == "GEMM_ERR_INVALID_ARG"    # same start, other element size
    assert call(G=0x40000 + 64) == "GEMM_ERR_INVALID_ARG"           # Y overlaps G
    # nothing to do: no launch, pointers never touched
    assert call(m=0, X=0, G=0, Y=0) == "GEMM_OK"
    assert call(d=0, ldx=1, ldy=1, X=0, G=0, Y=0) == "GEMM_OK"


def test_attention_argument_errors_are_caught_before_launch():
    lib = la.load()
    vp = ctypes.c_void_p
    st = la._lib.STATUS

    def call(**kw):
        f = dict(batch=2, sq=256, sk=300, d=128, in_type=la.BF16, out_type=la.BF16, ld_q=128, ld_k=128, ld_v=128,
                 ld_o=128, stride_q=256 * 128, stride_k=300 * 128, stride_v=300 * 128, stride_o=256 * 128, scale=0.088)
        ptrs = dict(Q=0x1000000, K=0x2000000, V=0x3000000, O=0x4000000)
        for k in list(kw):
            if k in ptrs:
                ptrs[k] = kw.pop(k)
        f.update(kw)
        desc = la._lib._AttnDesc(*[f[n] for n, _ in la._lib._AttnDesc._fields_])
        return st[lib.la_attention_run(ctypes.byref(desc), vp(ptrs["Q"]), vp(ptrs["K"]), vp(ptrs["V"]), vp(ptrs["O"]),
                                       vp(0))]

    assert call(d=96) == "GEMM_ERR_UNSUPPORTED"
    assert call(in_type=la.F32) == "GEMM_ERR_INVALID_ARG"
    assert call(out_type=9) == "GEMM_ERR_INVALID_ARG"
    assert call(scale=float("nan")) == "GEMM_ERR_INVALID_ARG"
    assert call(ld_k=100) == "GEMM_ERR_INVALID_ARG"
    assert call(ld_k=132) == "GEMM_ERR_ALIGNMENT"
    assert call(sk=0) == "GEMM_ERR_INVALID_ARG"
    assert call(V=0) == "GEMM_ERR_NULL"
    assert call(Q=0x1000008) == "GEMM_ERR_ALIGNMENT"
    assert call(stride_o=128) == "GEMM_ERR_INVALID_ARG"            # batch entries of O overlap
    assert call(O=0x3000000 + 4096) == "GEMM_ERR_INVALID_ARG"      # O overlaps V
    assert call(ld_k=1 << 25, stride_k=0) == "GEMM_ERR_UNSUPPORTED"
    # 2^24 query tiles of 256 threads are 2^32 work-items: more than one launch carries
    big = dict(batch=1 << 24, sq=128, stride_q=128 * 128, stride_o=128 * 128, stride_k=0, stride_v=0)
    assert call(**big) == "GEMM_ERR_UNSUPPORTED"
    assert "too many query tiles" in lib.gemm_last_error().decode()
    assert call(batch=0, Q=0, K=0, V=0, O=0) == "GEMM_OK"            # nothing to do, nothing touched
    assert call(sq=0, sk=0, Q=0, K=0, V=0, O=0) == "GEMM_OK"


def test_mfma_probe_argument_errors_are_caught_before_launch():
    lib = la.load()
    vp = ctypes.c_void_p
    st = la._lib.STATUS

    def call(ops=0x1000000, nbytes=1 << 20, sink=0x2000000, wg=256, n=4096, t=la.BF16):
        return st[lib.la_probe_mfma(vp(ops), nbytes, vp(sink), wg, n, t, vp(0))]

    assert call(t=la.F8E5M2) == "GEMM_ERR_INVALID_ARG" and call(t=-1) == "GEMM_ERR_INVALID_ARG"
    assert call(nbytes=0) == "GEMM_ERR_INVALID_ARG"
    assert call(nbytes=24) == "GEMM_ERR_INVALID_ARG"
    assert call(wg=0) == "GEMM_ERR_INVALID_ARG"
    assert call(wg=(1 << 20) + 1) == "GEMM_ERR_INVALID_ARG"
    assert call(n=0) == "GEMM_ERR_INVALID_ARG"
    assert call(n=24) == "GEMM_ERR_INVALID_ARG"
    assert call(n=(1 << 24) + 16) == "GEMM_ERR_INVALID_ARG"
    assert call(ops=0) == "GEMM_ERR_NULL"
    assert call(sink=0) == "GEMM_ERR_NULL"
    assert call(ops=0x1000008) == "GEMM_ERR_ALIGNMENT"
    assert call(sink=0x2000002) == "GEMM_ERR_ALIGNMENT"


def test_missing_library_raises_instead_of_falling_back(monkeypatch):
    # Without the built HIP library every entry point raises: there is no CPU path to fall back to.
    from layout_algebra_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_LIB_PATH", os.path.join(ROOT, "no_such_dir", "liblagemm.so"))
    for call in (lambda: la.gemm_plan(256, 256, 256),
                 lambda: la.la_swizzle_apply(3, 3, 4, 0),
                 lambda: la.la_layout_eval((4, 8), (8, 1), (1, 2))):
        with pytest.raises(RuntimeError, match="no fallback"):
            call()


def test_prefetch_depth_follows_the_grid():
    """The general kernel's 64 x 64 tiles keep three K blocks in flight on grids of 257 to 512
    workgroups (plain GEMM, 16-byte loads), two on other grids, one with element loads or gate/up."""
    def depth(m, n, k, **kw):
        d = la.gemm_plan(m, n, k, la.F16, la.F32, **kw).describe()
        return d["kernel"], d["grid"] * d["batch"], d["prefetch_blocks"]
    assert depth(1000, 1537, 999) == ("tiled_64x64x64", 400, 3)
    assert depth(1024, 1088, 64) == ("tiled_64x64x64", 272, 3)
    assert depth(1024, 1024, 64)[1:] == (256, 2)
    assert depth(1536, 1537, 999)[1:] == (600, 2)
    assert depth(1088, 1920, 64)[1:] == (510, 3)
    assert depth(1088, 2048, 64)[1:] == (544, 2)
    assert depth(200, 300, 5)[2] == 1                                  # element loads
    assert depth(1000, 1537, 999, gate_up=True)[2] == 1                 # gate/up keeps one set
    assert depth(300, 300, 64, batch=12)[1:] == (300, 3)                # batch entries count as workgroups


def _slots_256(offsets_words):
    """16-byte slots (mod 256 bytes, i.e. of gfx950's 64 four-byte banks) that a set of 16-byte reads at
    these word offsets touches."""
    return {(o * 4 // 16) % 16 for o in offsets_words}


def test_binary32_plan_maps_and_64_byte_rows():
    """The binary32 kernel's A block: two sub-blocks of 16 values per M row, i.e. 64-byte rows of the
    page's 64-byte fp32 plan, with the XOR taken from row bits 2-3 (Swizzle{2,2,4}) instead of 1-2
    (the page's Swizzle{2,2,3}); every map checked element by element against the XOR written out."""
    p = la.gemm_plan(1000, 1537, 999, la.F32, la.F32)
    d = p.describe()
    assert d["kernel"] == "tiled_f32_128x128x32" and d["in"] == "f32" and d["in_bytes"] == 4 and d["k_sub"] == 16
    assert d["mfma"] == "32x32x2" and d["tile"] == [128, 128, 32] and d["stages"] == 2
    assert d["lds_a"] == "(128,(16,2)):(16,(1,2048))" and d["swizzle_a"] == [2, 2, 4]
    assert d["lds_b"] == "(32,128):(128,1)" and d["swizzle_b"] == [1, 5, 5]
    assert d["lds_bytes"] == 2 * 8192 * 4 and la.gemm_plan_lds_stage_bytes(p) == 8192 * 4
    assert (d["vec_elems"], d["align_bytes"]) == (1, 4)
    for m in range(128):
        for k in range(32):
            want = 2048 * (k // 16) + 16 * m + ((k % 16) ^ (4 * ((m >> 2) & 3)))
            assert la.gemm_plan_lds_offset(p, 0, m, k) == want
    for k in range(32):
        for n in range(128):
            assert la.gemm_plan_lds_offset(p, 1, k, n) == 8192 // 2 + 128 * k + (n ^ (32 * ((k >> 3) & 1)))
    # the page's 64-byte fp32 plan over the same 16 x 128 sub-block (inner axis 1 = K)
    page = {(k, m): la.la_tile_plan_offset(4, (16, 128), 1, 64, (k, m))[0] for k in range(16) for m in range(128)}
    assert all(page[(k, m)] == 16 * m + (k ^ (4 * ((m >> 1) & 3))) for (k, m) in page)
    # 16-byte fragment reads of 16 consecutive rows at one K chunk: all 16 slots of the 256-byte
    # bank window under the kernel's map, only 8 under the page's
    for r0 in range(0, 128, 16):
        for kc in range(0, 16, 4):
            ours = [la.gemm_plan_lds_offset(p, 0, r0 + i, kc) for i in range(16)]
            theirs = [page[(kc, r0 + i)] for i in range(16)]
            assert len(_slots_256(ours)) == 16 and len(_slots_256(theirs)) == 8
    # 4-byte reads of the N-contiguous B block: lanes 0-31 read row k, lanes 32-63 row k + 8, 32
    # consecutive columns each: all 64 banks
    for k in range(8):
        for c0 in range(0, 128, 32):
            offs = [la.gemm_plan_lds_offset(p, 1, k + 8 * (l // 32), c0 + l % 32) for l in range(64)]
            assert len({o % 64 for o in offs}) == 64


def test_binary32_storage_orders_and_staging_width():
    def plan(m, n, k, **kw):
        return la.gemm_plan(m, n, k, la.F32, la.F32, **kw).describe()
    d = plan(4096, 4096, 4096)
    assert (d["vec_elems"], d["align_bytes"], d["grid"]) == (4, 16, 1024)
    assert d["copy"]["A"]["run_bytes"] == 128 and d["copy"]["B"]["run_bytes"] == 512
    d = plan(300, 260, 200, a_transposed=True, b_kmajor=True)
    assert d["a_order"] == "km" and d["b_order"] == "nk" and d["vec_elems"] == 4
    assert d["lds_a"] == "(128,32):(1,128)" and d["swizzle_a"] == [1, 5, 5]
    assert d["lds_b"] == "((16,2),128):((1,2048),16)" and d["swizzle_b"] == [2, 2, 4]
    # a row stride that is not a multiple of 4 elements, or a contiguous extent cut by a chunk: 4-byte loads
    assert plan(256, 256, 64, lda=66)["vec_elems"] == 1
    assert plan(256, 256, 62)["vec_elems"] == 1
    assert plan(256, 254, 64)["vec_elems"] == 1
    assert plan(254, 256, 64, a_transposed=True)["vec_elems"] == 1
    assert plan(254, 256, 64)["vec_elems"] == 4


def _swz(off, b, m, s):
    """Swizzle{B,M,S} written out: bits [M+S, M+S+B) XORed into bits [M, M+B)."""
    return off ^ (((off >> (m + s)) & ((1 << b) - 1)) << m)


@pytest.mark.parametrize("fa,fb", [(la.F8E4M3, la.F8E4M3), (la.F8E4M3, la.F8E5M2), (la.F8E5M2, la.F8E5M2)])
def test_one_byte_plans_describe_64_byte_rows(fa, fb):
    """One-byte inputs: the K-major full-tile kernel on byte pairs, described in codes: K blocks of
    64 codes (64-byte rows) under Swizzle{2,4,4}, one 32x32x64 product per block; every LDS offset
    the library reports is the written-out swizzle of m*64 + k (A) and n*64 + k (B)."""
    p = la.gemm_plan(4096, 4096, 4096, fa, la.BF16, b_kmajor=True, b_type=fb)
    d = p.describe()
    names = {la.F8E4M3: "f8e4m3", la.F8E5M2: "f8e5m2"}
    assert d["kernel"] == "fast_f8_256x256x64" and d["in"] == names[fa] and d["in_b"] == names[fb]
    assert d["tile"] == [256, 256, 64] and d["mfma"] == "32x32x64" and d["in_bytes"] == 1
    assert d["swizzle_a"] == [2, 4, 4] and d["swizzle_b"] == [2, 4, 4]
    assert d["lds_a"] == "(256,64):(64,1)" and d["lds_b"] == "(64,256):(1,64)"
    assert d["stage_elems"] == 2 * 256 * 64 and d["lds_bytes"] == 4 * 2 * 256 * 64
    assert d["copy"]["A"]["run_bytes"] == 64 and d["copy"]["A"]["instrs_per_block"] == 16
    assert la.gemm_plan_lds_stage_bytes(p) == 2 * 256 * 64
    for (r, k) in [(0, 0), (1, 17), (4, 16), (7, 63), (255, 40), (130, 33)]:
        assert la.gemm_plan_lds_offset(p, 0, r, k) == _swz(r * 64 + k, 2, 4, 4)
        assert la.gemm_plan_lds_offset(p, 1, k, r) == 256 * 64 + _swz(r * 64 + k, 2, 4, 4)
    # 16-lane groups of a 16-byte read: rows r..r+15 at one K chunk hit distinct 16-byte slots of
    # each 256-byte window (the bank rule the 16-bit swizzles were chosen by)
    for k0 in (0, 16, 32, 48):
        slots = [(_swz(r * 64 + k0, 2, 4, 4) % 256) // 16 for r in range(4)]
        assert len(set(slots)) == 4


def test_one_byte_plans_shapes_and_rejections():
    def plan(m, n, k, **kw):
        kw.setdefault("b_kmajor", True)
        return la.gemm_plan(m, n, k, la.F8E4M3, la.F32, ldc=max(8, (n + 7) // 8 * 8),
                            lda=max(16, (k + 15) // 16 * 16), ldb=max(16, (k + 15) // 16 * 16), **kw)
    # edges in M and N, a K tail of 16 / 48 codes from k = 512 on, small grids: all on the one kernel
    for m, n, k in [(300, 520, 512), (777, 1000, 1040), (513, 64, 1008), (64, 64, 64), (1, 1, 64)]:
        assert plan(m, n, k).describe()["kernel"] == "fast_f8_256x256x64", (m, n, k)
    # k = 0 reads neither operand (C = beta * C on the general kernel); m = 0 launches nothing
    assert plan(100, 100, 0).describe()["k"] == 0
    for m, n, k, kw in [(256, 256, 96, {}),                      # k % 64 below 512
                        (256, 256, 520, {}),                     # k % 16
                        (256, 256, 256, {"b_kmajor": False}),    # B stored [K, N]
                        (256, 256, 256, {"a_transposed": True})]:
        with pytest.raises(la.GemmError) as e:
            plan(m, n, k, **kw)
        assert "GEMM_ERR_UNSUPPORTED" in str(e.value)
    with pytest.raises(la.GemmError):      # rows not on 16 bytes
        la.gemm_plan(256, 256, 256, la.F8E4M3, la.F32, b_kmajor=True, lda=264)
    with pytest.raises(la.GemmError):      # one-byte A with a 16-bit B
        la.gemm_plan(256, 256, 256, la.F8E4M3, la.F32, b_kmajor=True, b_type=la.BF16)
    with pytest.raises(la.GemmError):      # not an output type
        la.gemm_plan(256, 256, 256, la.BF16, la.F8E4M3)


def test_one_byte_gate_up_plans():
    """Gate/up on one-byte X and weights: the waves-split-by-weight kernel on byte pairs, W_up's
    block after W_gate's in each stage, every offset the written-out swizzle of n*64 + k."""
    p = la.gemm_plan(4096, 11008, 4096, la.F8E4M3, la.BF16, gate_up=True, b_kmajor=True)
    d = p.describe()
    assert d["kernel"] == "fast_gate_up_f8_256x128x64" and d["tile"] == [256, 128, 64] and d["gate_up"]
    assert d["waves_split_by_weight"] and d["in_bytes"] == 1 and d["mfma"] == "32x32x64"
    assert d["lds_b"] == "(64,128):(1,64)"
    for (n, k) in [(0, 0), (5, 17), (127, 63), (64, 32)]:
        assert la.gemm_plan_lds_offset(p, 1, k, n) == 256 * 64 + _swz(n * 64 + k, 2, 4, 4)
        assert la.gemm_plan_lds_offset(p, 2, k, n) == 256 * 64 + 128 * 64 + _swz(n * 64 + k, 2, 4, 4)
    with pytest.raises(la.GemmError):      # weights stored [K, N]
        la.gemm_plan(256, 256, 256, la.F8E4M3, la.BF16, gate_up=True)
