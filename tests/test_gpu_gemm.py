"""GPU parity tests: the HIP path (through the C ABI) against the FP64 oracle.

Every test calls the library through its Python binding, which only marshals
pointers and the current stream.  Inputs come from the seeded generators in
`synth`; the oracle sees the same 16-bit patterns.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import synth
from parity import assert_close, band_rows, oracle_gemm, sample_rows, swiglu_bound
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def run_gemm(a, b, out_kind, alpha=1.0, beta=0.0, c=None, b_kmajor=False, expect=None, large_tiles=False):
    """a [M,K], b [K,N] CPU tensors (b is handed to the GPU as [N,K] when b_kmajor);
    returns the GPU result on the CPU.  large_tiles pins the largest tile (GEMM_FLAG_LARGE_TILES)."""
    M, K = a.shape
    N = b.shape[1]
    in_kind = "bf16" if a.dtype == torch.bfloat16 else "f16"
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], b_kmajor=b_kmajor, large_tiles=large_tiles)
    if expect is not None:
        assert plan.describe()["kernel"].startswith(expect), plan.describe()["kernel"]
    A = a.to(DEV)
    B = b.t().contiguous().to(DEV) if b_kmajor else b.to(DEV)
    if c is None:
        C = torch.full((M, N), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    else:
        C = c.to(DEV).clone()
    la.gemm_run(plan, A, B, C, alpha, beta)
    torch.cuda.synchronize()
    return C.cpu()


def test_library_is_the_native_one():
    import os
    assert os.path.exists(la.lib_path())
    la.load()


@pytest.mark.parametrize("name", ["square256", "ragged"])
def test_workload_full_parity(name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    print("case", name, flush=True)
    got = run_gemm(x["A"], x["B"], w.out_kind, w.alpha, w.beta, x.get("C"))
    ref = oracle_gemm(x["A"], x["B"], w.in_kind, w.alpha, w.beta, x.get("C"))
    assert_close(got, ref, w.K, x["A"], x["B"], w.out_kind, name, beta=w.beta)


def test_square4096_sampled_rows():
    w = synth.WORKLOADS["square4096"]
    x = synth.make_inputs(w)
    got = run_gemm(x["A"], x["B"], w.out_kind)
    rows = band_rows(w.M, seed=2003)                  # every 256-row tile band, each wave's first and last row
    ref = oracle_gemm(x["A"], x["B"], w.in_kind, rows=rows)
    assert_close(got[rows], ref, w.K, x["A"], x["B"], w.out_kind, "square4096")


def test_skinny_full():
    w = synth.WORKLOADS["skinny"]
    x = synth.make_inputs(w)
    got = run_gemm(x["A"], x["B"], w.out_kind)
    ref = oracle_gemm(x["A"], x["B"], w.in_kind)
    assert_close(got, ref, w.K, x["A"], x["B"], w.out_kind, "skinny")


def test_gate_up_sampled_rows():
    w = synth.WORKLOADS["gate_up"]
    x = synth.make_inputs(w)
    plan = la.gemm_plan(w.M, w.N, w.K, la.BF16, la.BF16, gate_up=True)
    X, Wg, Wu = x["A"].to(DEV), x["Wg"].to(DEV), x["Wu"].to(DEV)
    G = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=DEV)
    U = torch.empty_like(G)
    la.gemm_gate_up_run(plan, X, Wg, Wu, G, U)
    torch.cuda.synchronize()
    rows = band_rows(w.M, seed=4004)                  # every 256-row tile band, each wave's first and last row
    assert len(rows) >= 2 * (w.M // 256)
    for name, W, out in (("G", x["Wg"], G), ("U", x["Wu"], U)):
        ref = oracle_gemm(x["A"], W, "bf16", rows=rows)
        assert_close(out.cpu()[rows], ref, w.K, x["A"], W, "bf16", "gate_up " + name)


SHAPES = [(1, 1, 1), (1, 7, 3), (33, 65, 17), (64, 64, 64), (127, 129, 65), (129, 257, 130),
          (200, 72, 1000), (300, 300, 8), (5, 1000, 333), (257, 31, 64), (200, 300, 5), (300, 6, 200)]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_shapes_and_types(shape, in_kind, out_kind):
    M, N, K = shape
    seed = M * 7 + N * 13 + K
    a = synth.uniform((M, K), seed, in_kind)
    b = synth.uniform((K, N), seed + 1, in_kind)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    alpha, beta = 0.75, 1.25
    got = run_gemm(a, b, out_kind, alpha, beta, c)
    ref = oracle_gemm(a, b, in_kind, alpha, beta, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "shape %s" % (shape,), beta=beta)


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
def test_general_kernel_both_tile_sizes(in_kind, out_kind):
    """Both tile sizes of the general kernel on ragged shapes: 64 x 64 as planned for 1000 x 1537
    (400 workgroups), 128 x 128 pinned with GEMM_FLAG_LARGE_TILES for 1536 x 1537 (156); alpha,
    beta and an existing C, every element against the oracle."""
    for (M, N, K), kernel, large in (((1000, 1537, 999), "tiled_64x64", False),
                                     ((1536, 1537, 999), "tiled_128x128", True)):
        seed = M + N + K
        a = synth.uniform((M, K), seed, in_kind)
        b = synth.uniform((K, N), seed + 1, in_kind)
        c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
        got = run_gemm(a, b, out_kind, 1.5, -0.5, c, expect=kernel, large_tiles=large)
        ref = oracle_gemm(a, b, in_kind, 1.5, -0.5, c.to(torch.float32))
        assert_close(got, ref, K, a, b, out_kind, "%s %dx%dx%d" % (kernel, M, N, K), beta=-0.5)


LONG_K = [((70, 100, 65536), False, "tiled_64x64"), ((256, 256, 65536), True, "fast_256x256"),
          ((16, 128, 65536), False, "skinny_")]


@pytest.mark.parametrize("case", LONG_K, ids=[c[2] for c in LONG_K])
def test_long_k_accumulation(case):
    """K = 65536 (the longest accumulation chains and K loops of the tests) through each kernel
    family, zero-mean inputs as in the workloads; the oracle on all rows, or sampled rows of the
    full-tile case."""
    (M, N, K), large, kernel = case
    a = synth.uniform((M, K), 1234 + M, "bf16")
    b = synth.uniform((K, N), 4321 + N, "bf16")
    got = run_gemm(a, b, "f32", expect=kernel, large_tiles=large)
    rows = sample_rows(M, 6, 99) if M > 100 else list(range(M))
    ref = oracle_gemm(a, b, "bf16", rows=rows)
    assert_close(got[rows], ref, K, a, b, "f32", "long K %s" % ((M, N, K),))


def _view(t_cpu, ld, offset, dev_dtype):
    """t_cpu [r, c] placed on the GPU as a row-major view with leading dimension ld that starts
    `offset` elements into a NaN-filled buffer (so its base pointer has only element alignment)."""
    r, c = t_cpu.shape
    flat = torch.full((offset + max(r - 1, 0) * ld + c + 5,), float("nan"), dtype=dev_dtype, device=DEV)
    v = flat.as_strided((r, c), (ld, 1), offset)
    v.copy_(t_cpu.to(DEV))
    return v


@pytest.mark.parametrize("case", range(24))
def test_general_kernel_random_layouts(case):
    """Seeded random shapes (1..300), leading dimensions padded by 0..9 elements, operands starting
    at element (not 16-byte) offsets inside larger buffers, both B storages, alpha and beta: the
    general kernel's element-aligned 16-byte staging, cut chunks at K and N edges included; every
    element against the oracle."""
    g = torch.Generator().manual_seed(777 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    M, N, K = ri(1, 300), ri(1, 300), ri(1, 300)
    km = case % 3 == 2
    in_kind = "bf16" if case % 2 == 0 else "f16"
    out_kind = ("f32", "bf16", "f32", "f16")[case % 4]
    lda, ldb, ldc = K + ri(0, 9), (K if km else N) + ri(0, 9), N + ri(0, 9)
    a = synth.uniform((M, K), 900 + case, in_kind)
    b = synth.uniform((K, N), 1900 + case, in_kind)
    c = synth.uniform((M, N), 2900 + case, "f32").to(synth.torch_dtype(out_kind))
    alpha, beta = 0.5 + ri(0, 3) * 0.25, (0.0, -0.5, 1.0)[case % 3]
    dt = synth.torch_dtype(in_kind)
    A = _view(a, lda, ri(0, 7), dt)
    B = _view(b.t().contiguous() if km else b, ldb, ri(0, 7), dt)
    C = _view(c, ldc, ri(0, 7), synth.torch_dtype(out_kind))
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], lda=lda, ldb=ldb, ldc=ldc, b_kmajor=km)
    d = plan.describe()
    print("case", case, (M, N, K), (lda, ldb, ldc), km, in_kind, out_kind, d["kernel"], d["vec_elems"], flush=True)
    la.gemm_run(plan, A, B, C, alpha, beta)
    torch.cuda.synchronize()
    ref = oracle_gemm(a, b, in_kind, alpha, beta, c.to(torch.float32))
    assert_close(C.cpu(), ref, K, a, b, out_kind, "random layout case %d" % case, beta=beta)


PREFETCH_SHAPES = [(200, 136, 64), (130, 72, 128), (64, 64, 192), (100, 200, 1000), (96, 96, 8), (65, 130, 320),
                   (70, 90, 999), (129, 67, 257)]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", PREFETCH_SHAPES, ids=[str(s) for s in PREFETCH_SHAPES])
def test_general_kernel_prefetch_depths(shape, out_kind):
    """64 x 64 tiles of the general kernel (two register sets, 16-byte loads) over 1 to 16 K blocks,
    even and odd counts, ragged M and N edges and K tails, so that chunks cut by the K or N edge
    load the 8 elements ending at their last valid one and shift into place; every element
    against the oracle."""
    M, N, K = shape
    seed = 3 * M + 5 * N + K
    a = synth.uniform((M, K), seed, "bf16")
    b = synth.uniform((K, N), seed + 1, "bf16")
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    d = la.gemm_plan(M, N, K, la.BF16, CODE[out_kind]).describe()
    assert d["kernel"].startswith("tiled_64x64"), d["kernel"]
    assert d["vec_elems"] == (8 if K % 8 == 0 and N % 8 == 0 else 2)
    got = run_gemm(a, b, out_kind, -0.75, 1.5, c, expect="tiled_64x64")
    ref = oracle_gemm(a, b, "bf16", -0.75, 1.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "prefetch %s" % (shape,), beta=1.5)


DEEP_SHAPES = [(1088, 1088, 64, False), (1088, 1088, 128, False), (1088, 1088, 192, False), (1000, 1100, 130, False),
               (1030, 1037, 320, False), (1000, 1537, 999, False), (1088, 1030, 456, True), (1030, 1088, 999, True)]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", DEEP_SHAPES, ids=[str(s) for s in DEEP_SHAPES])
def test_general_kernel_three_blocks_in_flight(shape, out_kind):
    """Grids of 257 to 512 workgroups of 64 x 64 tiles (plain GEMM, 16-byte loads) keep three K
    blocks in flight: 1 to 16 blocks, block counts of every residue mod 3, K tails and N edges
    cutting chunks, both B storages; every element against the oracle."""
    M, N, K, km = shape
    seed = 7 * M + 3 * N + K + km
    print("case", shape, out_kind, flush=True)
    a = synth.uniform((M, K), seed, "f16")
    b = synth.uniform((K, N), seed + 1, "f16")
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    d = la.gemm_plan(M, N, K, la.F16, CODE[out_kind], b_kmajor=km).describe()
    assert d["kernel"].startswith("tiled_64x64") and 256 < d["grid"] <= 512, d
    assert d["prefetch_blocks"] == 3
    got = run_gemm(a, b, out_kind, 1.25, -0.5, c, b_kmajor=km, expect="tiled_64x64")
    ref = oracle_gemm(a, b, "f16", 1.25, -0.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "three blocks in flight %s" % (shape,), beta=-0.5)


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
def test_identity_and_permutation_B_are_exact(in_kind):
    K, M = 256, 192
    a = synth.uniform((M, K), 17, in_kind)
    eye = torch.eye(K, dtype=synth.torch_dtype(in_kind))
    got = run_gemm(a, eye, "f32")
    assert torch.equal(got, a.to(torch.float32))
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(18))
    P = torch.zeros((K, K), dtype=synth.torch_dtype(in_kind))
    P[perm, torch.arange(K)] = 1
    got = run_gemm(a, P, "f32")
    assert torch.equal(got, a.to(torch.float32)[:, perm])
    got16 = run_gemm(a, P, in_kind)          # 16-bit output of an exact value is exact
    assert torch.equal(got16, a[:, perm])


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
def test_ones_times_ones_is_K(in_kind):
    for (M, N, K) in [(100, 300, 4096), (130, 70, 999)]:
        a = torch.ones((M, K), dtype=synth.torch_dtype(in_kind))
        b = torch.ones((K, N), dtype=synth.torch_dtype(in_kind))
        got = run_gemm(a, b, "f32")
        assert torch.all(got == K)


def test_beta_zero_never_reads_C():
    M, N, K = 150, 170, 90
    a = synth.uniform((M, K), 1, "bf16")
    b = synth.uniform((K, N), 2, "bf16")
    c = torch.full((M, N), float("nan"))
    got = run_gemm(a, b, "f32", 1.0, 0.0, c)
    assert torch.isfinite(got).all()
    ref = oracle_gemm(a, b, "bf16")
    assert_close(got, ref, K, a, b, "f32", "beta=0")


def test_k_zero_and_empty_outputs():
    M, N = 70, 90
    c = synth.uniform((M, N), 3, "f32")
    a = torch.zeros((M, 0), dtype=torch.bfloat16)
    b = torch.zeros((0, N), dtype=torch.bfloat16)
    got = run_gemm(a, b, "f32", 3.0, -0.5, c)
    assert torch.equal(got, c * -0.5)
    for (m, n, k) in [(0, 5, 7), (5, 0, 7), (0, 0, 0)]:
        plan = la.gemm_plan(m, n, k, la.BF16, la.F32)
        A = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
        B = torch.zeros((k, n), dtype=torch.bfloat16, device=DEV)
        C = torch.zeros((m, n), dtype=torch.float32, device=DEV)
        la.gemm_run(plan, A, B, C)
    torch.cuda.synchronize()


def test_ragged_never_writes_outside_C():
    """C is a window of a bigger buffer: padding columns and rows stay untouched."""
    w = synth.WORKLOADS["ragged"]
    x = synth.make_inputs(w)
    M, N, K, ldc = w.M, w.N, w.K, w.N + 63
    big = torch.full((M + 5, ldc), 12345.0, dtype=torch.float32, device=DEV)
    C = big[:M, :N]
    C.copy_(x["C"].to(DEV))
    plan = la.gemm_plan(M, N, K, la.F16, la.F32, ldc=ldc)
    la.gemm_run(plan, x["A"].to(DEV), x["B"].to(DEV), C, w.alpha, w.beta)
    torch.cuda.synchronize()
    big = big.cpu()
    assert torch.all(big[:M, N:] == 12345.0)
    assert torch.all(big[M:, :] == 12345.0)
    ref = oracle_gemm(x["A"], x["B"], "f16", w.alpha, w.beta, x["C"])
    assert_close(big[:M, :N], ref, K, x["A"], x["B"], "f32", "ragged window", beta=w.beta)


def test_deterministic_and_plan_reuse():
    M, N, K = 512, 384, 700
    a = synth.normal((M, K), 5, "bf16")
    b = synth.normal((K, N), 6, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32)
    A, B = a.to(DEV), b.to(DEV)
    C1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    C2 = torch.empty_like(C1)
    la.gemm_run(plan, A, B, C1)
    la.gemm_run(plan, A, B, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    # same plan, modified input values
    a2 = synth.normal((M, K), 7, "bf16")
    A.copy_(a2.to(DEV))
    la.gemm_run(plan, A, B, C2)
    torch.cuda.synchronize()
    ref = oracle_gemm(a2, b, "bf16")
    assert_close(C2.cpu(), ref, K, a2, b, "f32", "reuse")


def test_one_plan_on_concurrent_streams():
    """A plan is immutable host data: the same plan runs on two streams at once
    (and a second plan beside it) with the same results as one after another."""
    M, N, K = 1024, 1024, 512
    a = synth.normal((M, K), 11, "bf16")
    b = synth.normal((K, N), 12, "bf16")
    b2 = synth.normal((K, N), 13, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    plan2 = la.gemm_plan(M - 1, N, K, la.BF16, la.F32, lda=K)     # a second plan (general kernel)
    A, B, B2 = a.to(DEV), b.to(DEV), b2.to(DEV)
    ref1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ref2 = torch.empty_like(ref1)
    ref3 = torch.empty((M - 1, N), dtype=torch.float32, device=DEV)
    la.gemm_run(plan, A, B, ref1)
    la.gemm_run(plan, A, B2, ref2)
    la.gemm_run(plan2, A[:M - 1], B, ref3)
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for it in range(3):
        C1, C2 = torch.empty_like(ref1), torch.empty_like(ref2)
        C3 = torch.empty_like(ref3)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            la.gemm_run(plan, A, B, C1)
        with torch.cuda.stream(s2):
            la.gemm_run(plan, A, B2, C2)
        with torch.cuda.stream(s3):
            la.gemm_run(plan2, A[:M - 1], B, C3)
        torch.cuda.synchronize()
        assert torch.equal(C1, ref1) and torch.equal(C2, ref2) and torch.equal(C3, ref3), "iteration %d" % it


def test_graph_capture_replay():
    M, N, K = 384, 512, 320
    a = synth.normal((M, K), 8, "bf16")
    b = synth.normal((K, N), 9, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    A, B = a.to(DEV), b.to(DEV)
    C = torch.zeros((M, N), dtype=torch.bfloat16, device=DEV)
    eager = torch.empty_like(C)
    la.gemm_run(plan, A, B, eager)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.gemm_run(plan, A, B, C)       # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.gemm_run(plan, A, B, C)
    for it in range(4):
        C.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), "replay %d" % it
        A.add_(0)                        # unrelated eager work between replays


def _lds_image(plan, A, B, B2, tm, tn):
    nbytes = la.gemm_plan_lds_stage_bytes(plan)
    out = torch.zeros(nbytes // 2, dtype=torch.int16, device=DEV)
    la.gemm_debug_lds_image(plan, A, B, B2, tm, tn, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def _expected_image(plan, ops, tm, tn):
    """Build the predicted stage from the planner's offsets and the host operands."""
    d = la.gemm_plan_describe(plan)
    bm, bn, bk = d["tile"]
    img = np.full(d["stage_elems"], 0xDEAD, dtype=np.uint32)
    for operand, (mat, rows, cols, r0, c0) in enumerate(ops):
        bits = synth.bits(mat)
        for r in range(rows):
            for c in range(cols):
                gr, gc = r0 + r, c0 + c
                v = bits[gr, gc] if gr < bits.shape[0] and gc < bits.shape[1] else 0
                img[la.gemm_plan_lds_offset(plan, operand, r, c)] = v
    return img, (bm, bn, bk)


LDS_CASES = {
    # name: (M, N, K, kind, gate_up, tile_m, tile_n, expected kernel prefix)
    "fast_bf16": (512, 512, 256, "bf16", False, 1, 1, "fast_"),
    "fast_f16_last_tile": (768, 512, 128, "f16", False, 2, 1, "fast_"),
    "tiled_bf16_interior": (384, 384, 200, "bf16", False, 1, 1, "tiled_"),
    "tiled64_f16_ragged_edge": (1000, 1537, 999, "f16", False, 15, 24, "tiled_64x64"),
    "tiled128_f16_ragged_edge": (1536, 1537, 999, "f16", False, 11, 12, "tiled_128x128"),
    "fast_gate_up": (512, 256, 128, "bf16", True, 1, 1, "fast_gate_up_"),
    "tiled_gate_up_edge": (300, 200, 100, "bf16", True, 2, 1, "tiled_"),
    "skinny_bf16": (16, 512, 256, "bf16", False, 0, 2, "skinny_"),
    "skinny_bkmajor_f16": (16, 512, 256, "f16", False, 0, 3, "skinny_bkmajor_", True),
    "skinny_64_bf16": (64, 16384, 256, "bf16", False, 0, 2, "skinny_64x"),
    "skinny_128_bf16": (128, 16384, 256, "bf16", False, 0, 7, "skinny_128x"),
    "skinny_bkmajor_128_f16": (128, 16384, 256, "f16", False, 0, 9, "skinny_bkmajor_128x", True),
    "skinny_bkmajor_32_f16": (32, 512, 256, "f16", False, 0, 5, "skinny_bkmajor_32x", True),
    "fast_bkmajor": (512, 512, 256, "bf16", False, 1, 1, "fast_bkmajor_", True),
    "fast_gate_up_bkmajor": (512, 256, 128, "f16", True, 1, 1, "fast_gate_up_bkmajor_", True),
    "tiled_bkmajor_edge": (300, 200, 100, "bf16", False, 2, 1, "tiled_", True),
}


@pytest.mark.parametrize("case", list(LDS_CASES))
def test_lds_image_matches_planner(case):
    M, N, K, kind, gu, tm, tn, prefix = LDS_CASES[case][:8]
    km = len(LDS_CASES[case]) > 8 and LDS_CASES[case][8]
    a = synth.uniform((M, K), 21, kind)
    b = synth.uniform((K, N), 22, kind)
    b2 = synth.uniform((K, N), 23, kind) if gu else None
    # the full-tile and 128 x 128 cases are small grids: pin their kernels with the large-tile flag
    plan = la.gemm_plan(M, N, K, CODE[kind], la.F32, gate_up=gu, b_kmajor=km, large_tiles=not prefix.startswith("tiled_64"))
    d = la.gemm_plan_describe(plan)
    assert d["kernel"].startswith(prefix), d["kernel"]
    bm, bn, bk = d["tile"]
    ops = [(a, bm, bk, tm * bm, 0), (b, bk, bn, 0, tn * bn)]
    if gu:
        ops.append((b2, bk, bn, 0, tn * bn))
    want, _ = _expected_image(plan, ops, tm, tn)
    dev_b = (lambda t: t.t().contiguous().to(DEV)) if km else (lambda t: t.to(DEV))
    got = _lds_image(plan, a.to(DEV), dev_b(b), dev_b(b2) if gu else None, tm, tn)
    assert not np.any(want == 0xDEAD), "planner map does not cover the stage"
    assert np.array_equal(got.astype(np.uint32), want)


FAST_SHAPES = [(256, 256, 64), (512, 768, 320), (768, 512, 1024), (256, 1024, 4096)]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", FAST_SHAPES, ids=[str(s) for s in FAST_SHAPES])
def test_fast_kernel_shapes(shape, in_kind, out_kind):
    M, N, K = shape
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast_")
    seed = M + 3 * N + 7 * K
    a = synth.normal((M, K), seed, in_kind)
    b = synth.normal((K, N), seed + 1, in_kind, 0.5)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got = run_gemm(a, b, out_kind, -1.25, 0.5, c, expect="fast_", large_tiles=True)
    ref = oracle_gemm(a, b, in_kind, -1.25, 0.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "fast %s" % (shape,), beta=0.5)


@pytest.mark.parametrize("large", [True, False], ids=["large_tiles", "planned"])
@pytest.mark.parametrize("shape", [(512, 256, 192), (300, 200, 100), (256, 384, 64)],
                         ids=["fast", "tiled_edges", "fast_min_k"])
def test_gate_up_small(shape, large):
    """Pinned to the largest tiles (full-tile gate/up kernel, general 128 x 128) and as planned
    (64 x 64 tiles for these small grids)."""
    M, N, K = shape
    x = synth.normal((M, K), 31, "bf16")
    wg = synth.normal((K, N), 32, "bf16", 0.3)
    wu = synth.normal((K, N), 33, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, large_tiles=large)
    want = ("fast_gate_up_" if M % 256 == 0 else "tiled_128x128") if large else "tiled_64x64"
    assert plan.describe()["kernel"].startswith(want), plan.describe()["kernel"]
    G = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    U = torch.full_like(G, float("nan"))
    la.gemm_gate_up_run(plan, x.to(DEV), wg.to(DEV), wu.to(DEV), G, U)
    torch.cuda.synchronize()
    for name, w, out in (("G", wg, G), ("U", wu, U)):
        assert_close(out.cpu(), oracle_gemm(x, w, "bf16"), K, x, w, "bf16", "gate_up %s %s" % (name, shape))


def test_fast_kernel_identity_is_exact():
    K = 512
    a = synth.uniform((256, K), 41, "bf16")
    eye = torch.eye(K, dtype=torch.bfloat16)
    plan = la.gemm_plan(256, K, K, la.BF16, la.F32, large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast_")
    got = run_gemm(a, eye, "f32", expect="fast_", large_tiles=True)
    assert torch.equal(got, a.to(torch.float32))
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(42))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[perm, torch.arange(K)] = 1
    assert torch.equal(run_gemm(a, P, "bf16", expect="fast_", large_tiles=True), a[:, perm])


SKINNY_SHAPES = [(16, 128, 128), (1, 256, 256), (7, 384, 1024), (16, 1024, 2048), (13, 128, 8192)]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SKINNY_SHAPES, ids=[str(s) for s in SKINNY_SHAPES])
def test_skinny_kernel_shapes(shape, in_kind, out_kind):
    M, N, K = shape
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind])
    assert plan.describe()["kernel"].startswith("skinny_")
    seed = 11 * M + N + K
    a = synth.normal((M, K), seed, in_kind)
    b = synth.normal((K, N), seed + 1, in_kind, 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got = run_gemm(a, b, out_kind, 0.5, -2.0, c)
    ref = oracle_gemm(a, b, in_kind, 0.5, -2.0, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "skinny %s" % (shape,), beta=-2.0)


SKINNY_KM_SHAPES = [(16, 64, 256), (1, 256, 256), (7, 384, 1024), (16, 1024, 2048), (13, 192, 8192)]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SKINNY_KM_SHAPES, ids=[str(s) for s in SKINNY_KM_SHAPES])
def test_skinny_kernel_kmajor_b(shape, in_kind, out_kind):
    """B stored [N, K] (a linear layer's weight): strips of 64 K-contiguous B rows."""
    M, N, K = shape
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], b_kmajor=True)
    assert plan.describe()["kernel"].startswith("skinny_bkmajor_"), plan.describe()["kernel"]
    seed = 13 * M + N + 3 * K
    a = synth.normal((M, K), seed, in_kind)
    b = synth.normal((K, N), seed + 1, in_kind, 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got = run_gemm(a, b, out_kind, -0.75, 1.5, c, b_kmajor=True)
    ref = oracle_gemm(a, b, in_kind, -0.75, 1.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "skinny kmajor %s" % (shape,), beta=1.5)


# more than 32 rows of A plan the skinny kernel on grids of at least 128 column strips only
SKINNY_MID_SHAPES = [(17, 256, 256), (32, 384, 1024), (32, 4096, 2048), (33, 16384, 512), (48, 16384, 1024),
                     (64, 16384, 256), (65, 16384, 512), (100, 16384, 256), (128, 16384, 1024)]


@pytest.mark.parametrize("km", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SKINNY_MID_SHAPES, ids=[str(s) for s in SKINNY_MID_SHAPES])
def test_skinny_kernel_32_to_128_rows(shape, out_kind, km):
    """17 <= M <= 128: the skinny kernel with 32, 64 or 128 rows of A (rows past M read row M - 1
    and are not stored), both storages of B."""
    M, N, K = shape
    plan = la.gemm_plan(M, N, K, la.BF16, CODE[out_kind], b_kmajor=km)
    want = "skinny_%s%dx" % ("bkmajor_" if km else "", 32 if M <= 32 else 64 if M <= 64 else 128)
    assert plan.describe()["kernel"].startswith(want), plan.describe()["kernel"]
    seed = 19 * M + N + 5 * K
    a = synth.normal((M, K), seed, "bf16")
    b = synth.normal((K, N), seed + 1, "bf16", 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got = run_gemm(a, b, out_kind, 1.5, -0.25, c, b_kmajor=km)
    ref = oracle_gemm(a, b, "bf16", 1.5, -0.25, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "skinny %s %s" % (shape, km), beta=-0.25)


def test_skinny_kmajor_permutation_is_exact():
    K = 512
    a = synth.uniform((9, K), 52, "bf16")
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(53))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[perm, torch.arange(K)] = 1
    plan = la.gemm_plan(9, K, K, la.BF16, la.F32, b_kmajor=True)
    assert plan.describe()["kernel"].startswith("skinny_bkmajor_")
    assert torch.equal(run_gemm(a, P, "f32", b_kmajor=True), a.to(torch.float32)[:, perm])


def test_skinny_identity_is_exact():
    K = 256
    a = synth.uniform((16, K), 51, "bf16")
    eye = torch.eye(K, dtype=torch.bfloat16)
    plan = la.gemm_plan(16, K, K, la.BF16, la.F32)
    assert plan.describe()["kernel"].startswith("skinny_")
    assert torch.equal(run_gemm(a, eye, "f32"), a.to(torch.float32))


@pytest.mark.parametrize("shape", [(512, 256, 192), (300, 200, 100), (4096, 11008, 4096)],
                         ids=["fast", "tiled_edges", "gate_up_workload"])
def test_gate_up_swiglu(shape):
    M, N, K = shape
    if (M, N, K) == (4096, 11008, 4096):
        w = synth.WORKLOADS["gate_up"]
        inp = synth.make_inputs(w)
        x, wg, wu = inp["A"], inp["Wg"], inp["Wu"]
        rows = sample_rows(M, 16, 4005)
    else:
        x = synth.normal((M, K), 71, "bf16")
        wg = synth.normal((K, N), 72, "bf16", 0.3)
        wu = synth.normal((K, N), 73, "bf16", 0.3)
        rows = list(range(M))
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, large_tiles=(M, N, K) == (512, 256, 192))
    H = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.gemm_gate_up_swiglu_run(plan, x.to(DEV), wg.to(DEV), wu.to(DEV), H)
    torch.cuda.synchronize()
    h_ref, g_ref, u_ref = oracle.gate_up_swiglu_f64(synth.bits(x[rows]), synth.bits(wg), synth.bits(wu), "bf16")
    got = H.cpu()[rows].to(torch.float64).numpy()
    tol = swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16")
    err = np.abs(got - h_ref)
    assert np.all(err <= tol), "max err %g at %s" % (err.max(), np.unravel_index(np.argmax(err - tol), err.shape))


KM_SHAPES = [((256, 256, 64), "fast_bkmajor_"), ((512, 768, 320), "fast_bkmajor_"), ((33, 65, 17), "tiled_"),
             ((1000, 1537, 999), "tiled_"), ((65, 1024, 2048), "tiled_"), ((256, 1024, 4096), "fast_bkmajor_")]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("case", KM_SHAPES, ids=[str(c[0]) for c in KM_SHAPES])
def test_bkmajor_shapes(case, in_kind, out_kind):
    (M, N, K), expect = case
    seed = 5 * M + 3 * N + K
    a = synth.normal((M, K), seed, in_kind)
    b = synth.normal((K, N), seed + 1, in_kind, 0.5)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got = run_gemm(a, b, out_kind, 0.5, 1.5, c, b_kmajor=True, expect=expect, large_tiles=expect.startswith("fast"))
    ref = oracle_gemm(a, b, in_kind, 0.5, 1.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "K-major B %s" % ((M, N, K),), beta=1.5)


def test_bkmajor_permutation_is_exact():
    K = 512
    a = synth.uniform((256, K), 81, "bf16")
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(82))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[perm, torch.arange(K)] = 1
    got = run_gemm(a, P, "bf16", b_kmajor=True, expect="fast_bkmajor_", large_tiles=True)
    assert torch.equal(got, a[:, perm])


@pytest.mark.parametrize("shape", [(512, 256, 192), (300, 200, 100)], ids=["fast", "tiled_edges"])
def test_gate_up_swiglu_bkmajor(shape):
    M, N, K = shape
    x = synth.normal((M, K), 97, "bf16")
    wg = synth.normal((K, N), 98, "bf16", 0.3)
    wu = synth.normal((K, N), 99, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, b_kmajor=True, large_tiles=(M, N, K) == (512, 256, 192))
    H = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.gemm_gate_up_swiglu_run(plan, x.to(DEV), wg.t().contiguous().to(DEV), wu.t().contiguous().to(DEV), H)
    torch.cuda.synchronize()
    h_ref, g_ref, u_ref = oracle.gate_up_swiglu_f64(synth.bits(x), synth.bits(wg), synth.bits(wu), "bf16")
    err = np.abs(H.cpu().to(torch.float64).numpy() - h_ref)
    assert np.all(err <= swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16"))


@pytest.mark.parametrize("shape", [(512, 256, 192), (300, 200, 100)], ids=["fast", "tiled_edges"])
def test_gate_up_bkmajor(shape):
    M, N, K = shape
    x = synth.normal((M, K), 91, "bf16")
    wg = synth.normal((K, N), 92, "bf16", 0.3)
    wu = synth.normal((K, N), 93, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, b_kmajor=True, large_tiles=(M, N, K) == (512, 256, 192))
    G = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    U = torch.full_like(G, float("nan"))
    la.gemm_gate_up_run(plan, x.to(DEV), wg.t().contiguous().to(DEV), wu.t().contiguous().to(DEV), G, U)
    torch.cuda.synchronize()
    for name, w, out in (("G", wg, G), ("U", wu, U)):
        assert_close(out.cpu(), oracle_gemm(x, w, "bf16"), K, x, w, "bf16", "gate_up K-major %s %s" % (name, shape))
