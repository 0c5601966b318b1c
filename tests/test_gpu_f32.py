"""GPU parity of the GEMM with binary32 inputs (v_mfma_f32_32x32x2_f32), through the
C ABI, against the binary64 oracle on the same 32-bit words.

The plan stages K-contiguous operands through 64-byte rows of 16 binary32 values
(the 64-byte plan of Tylo.jl "TMA and Hopper WGMMA", section "The same storage
contract on both sides") and M/N-contiguous ones as rows of 128 values; covered:
all four storage orders (A [M, K] or [K, M], B [K, N] or [N, K]), 16-byte and
4-byte staging, ragged edges on every side, alpha / beta with an existing C,
fp32 / bf16 / fp16 outputs, padded leading dimensions, batched runs, the row
reductions, exact identity / permutation / ones products, empty and K = 0
shapes, a 2048^3 run sampled on rows that cover every tile row, and the LDS
image of each storage order against the planner's map.

Bound: the same elementwise bound as the 16-bit inputs,
2^-20 K max|A| max|B| (+ the output's rounding).  Binary32 products are not
exact in FP32 (16-bit products are); each product's rounding adds at most
2^-24 |a b| <= 2^-24 max|A| max|B| per term, one sixteenth of the allowance.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, band_rows, oracle_gemm
from test_gpu_reduce import red_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def to_dev(t, transposed, ld=None):
    """t [r, c] (mathematical) -> device storage: [r, c] or its transpose [c, r], row stride ld."""
    s = t.t() if transposed else t
    rows, cols = s.shape
    ld = ld or max(1, cols)
    buf = torch.full((rows, ld), float("nan"), dtype=t.dtype, device=DEV)
    buf[:, :cols] = s.to(DEV)
    return buf[:, :cols]


def run(a, b, out_kind, alpha=1.0, beta=0.0, c=None, at=False, bk=False, lda=None, ldb=None, expect_vec=None):
    M, K = a.shape
    N = b.shape[1]
    A = to_dev(a, at, lda)
    B = to_dev(b, bk, ldb)
    plan = la.gemm_plan(M, N, K, la.F32, CODE[out_kind], lda=A.stride(0) if A.dim() == 2 and A.shape[0] > 0 else None,
                        ldb=B.stride(0) if B.shape[0] > 0 else None, a_transposed=at, b_kmajor=bk)
    d = plan.describe()
    assert d["kernel"] == "tiled_f32_128x128x32" and d["in"] == "f32", d["kernel"]
    if expect_vec is not None:
        assert d["vec_elems"] == expect_vec, d["vec_elems"]
    C = torch.full((M, N), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV) if c is None \
        else c.to(DEV).clone()
    la.gemm_run(plan, A, B, C, alpha, beta)
    torch.cuda.synchronize()
    return C.cpu(), d


ORDERS = [(False, False), (True, False), (False, True), (True, True)]
ORDER_IDS = ["mk_kn", "km_kn", "mk_nk", "km_nk"]

SHAPES = [
    # (M, N, K, expected staging width for A [M,K], B [K,N])
    (256, 256, 64, 4),
    (512, 768, 320, 4),
    (1000, 1537, 999, 1),      # ragged on every side, 4-byte staging
    (1003, 512, 257, 1),
    (129, 257, 130, 1),
    (9, 64, 64, 4),
    (200, 72, 1000, 4),
    (300, 300, 1, 1),
    (1, 1, 1, 1),
    (128, 128, 32, 4),         # exactly one tile and one K block
]


@pytest.mark.parametrize("order", ORDERS, ids=ORDER_IDS)
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:3]) for s in SHAPES])
def test_f32_shapes(shape, out_kind, order):
    M, N, K, vec = shape
    at, bk = order
    print("f32", shape, out_kind, order, flush=True)
    seed = 7 * M + 13 * N + K
    a = synth.uniform((M, K), seed, "f32")
    b = synth.uniform((K, N), seed + 1, "f32")
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    whole = (M if at else K) % 4 == 0 and (K if bk else N) % 4 == 0
    got, _ = run(a, b, out_kind, 1.5, -0.5, c, at=at, bk=bk, expect_vec=4 if whole else 1)
    ref = oracle_gemm(a, b, "f32", 1.5, -0.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "f32 %s %s" % (shape, order), beta=-0.5)


@pytest.mark.parametrize("order", ORDERS, ids=ORDER_IDS)
def test_f32_beta_zero_never_reads_c(order):
    M, N, K = 300, 200, 100
    a = synth.normal((M, K), 41, "f32")
    b = synth.normal((K, N), 42, "f32", 0.5)
    got, _ = run(a, b, "f32", at=order[0], bk=order[1])      # C starts as NaN
    assert_close(got, oracle_gemm(a, b, "f32"), K, a, b, "f32", "beta 0")


def test_f32_fp16_output():
    M, N, K = 257, 130, 77
    a = synth.uniform((M, K), 51, "f32")
    b = synth.uniform((K, N), 52, "f32")
    got, _ = run(a, b, "f16")
    assert_close(got, oracle_gemm(a, b, "f32"), K, a, b, "f16", "f16 out")


def test_f32_large_sampled_rows():
    """2048^3 (256 tiles, 64 K blocks): rows covering every 128-row band (both waves' halves)."""
    M = N = K = 2048
    a = synth.normal((M, K), 61, "f32", 1.0 / 45.25)
    b = synth.normal((K, N), 62, "f32", 1.0 / 45.25)
    got, d = run(a, b, "f32", expect_vec=4)
    assert d["grid"] == 256
    rows = band_rows(M, band=128, wave_rows=64, extra=1, seed=63)
    ref = oracle_gemm(a, b, "f32", rows=rows)
    assert_close(got[rows], ref, K, a, b, "f32", "2048^3 rows")


@pytest.mark.parametrize("order", ORDERS, ids=ORDER_IDS)
def test_f32_padded_leading_dimensions(order):
    """Padded rows: a multiple of 4 keeps 16-byte staging, any other pad takes 4-byte loads."""
    at, bk = order
    M, N, K = 300, 260, 200
    a = synth.normal((M, K), 71, "f32")
    b = synth.normal((K, N), 72, "f32", 0.5)
    for pad, vec in ((8, 4), (3, 1)):
        lda = (M if at else K) + pad
        ldb = (K if bk else N) + pad
        got, d = run(a, b, "f32", at=at, bk=bk, lda=lda, ldb=ldb, expect_vec=vec)
        assert d["lda"] == lda and d["ldb"] == ldb
        assert_close(got, oracle_gemm(a, b, "f32"), K, a, b, "f32", "lda %d ldb %d" % (lda, ldb))


@pytest.mark.parametrize("order", ORDERS, ids=ORDER_IDS)
def test_f32_identity_permutation_and_ones_are_exact(order):
    at, bk = order
    K, M = 160, 200
    a = synth.uniform((M, K), 17, "f32")
    eye = torch.eye(K, dtype=torch.float32)
    got, _ = run(a, eye, "f32", at=at, bk=bk)
    assert torch.equal(got, a)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(18))
    P = torch.zeros((K, K), dtype=torch.float32)
    P[perm, torch.arange(K)] = 1
    got, _ = run(a, P, "f32", at=at, bk=bk)
    assert torch.equal(got, a[:, perm])
    ones_a = torch.ones((33, 999), dtype=torch.float32)
    ones_b = torch.ones((999, 65), dtype=torch.float32)
    got, _ = run(ones_a, ones_b, "f32", at=at, bk=bk)
    assert torch.all(got == 999.0)


def test_f32_empty_and_k_zero():
    c = synth.uniform((70, 40), 5, "f32")
    got, _ = run(torch.zeros((70, 0)), torch.zeros((0, 40)), "f32", 2.0, -0.5, c)
    assert torch.equal(got, (-0.5 * c.double()).float())
    plan = la.gemm_plan(0, 40, 10, la.F32, la.F32)
    C = torch.full((0, 40), float("nan"), device=DEV)
    la.gemm_run(plan, torch.zeros((0, 10), device=DEV), torch.zeros((10, 40), device=DEV), C)
    torch.cuda.synchronize()


def test_f32_batched():
    batch, M, N, K = 5, 100, 70, 45
    a = synth.normal((batch, M, K), 81, "f32")
    b = synth.normal((batch, K, N), 82, "f32", 0.5)
    sa, sc = M * K + 11, M * N + 5
    Af = torch.full((batch * sa,), float("nan"), device=DEV)
    A = Af.as_strided((batch, M, K), (sa, K, 1))
    A.copy_(a.to(DEV))
    Cf = torch.full((batch * sc,), float("nan"), device=DEV)
    C = Cf.as_strided((batch, M, N), (sc, N, 1))
    plan = la.gemm_plan(M, N, K, la.F32, la.F32, batch=batch, stride_a=sa, stride_b=K * N, stride_c=sc)
    assert plan.describe()["vec_elems"] == 1      # the batch stride sa is odd
    la.gemm_run(plan, A, b.to(DEV), C)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        assert_close(got[z], oracle_gemm(a[z], b[z], "f32"), K, a[z], b[z], "f32", "batch %d" % z)
    mask = torch.ones(batch * sc, dtype=torch.bool)
    for z in range(batch):
        mask[z * sc:z * sc + M * N] = False
    assert torch.isnan(Cf.cpu()[mask]).all()


@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_f32_row_reduce(op):
    M, N, K = 300, 257, 99
    a = synth.uniform((M, K), 91, "f32")
    b = synth.uniform((K, N), 92, "f32")
    c = synth.uniform((M, N), 93, "f32")
    plan = la.gemm_plan(M, N, K, la.F32, la.F32)
    C = c.to(DEV).clone()
    R = torch.full((M,), 12345.0, dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, a.to(DEV), b.to(DEV), C, 1.25, 0.5, op, R)
    torch.cuda.synchronize()
    out, r = oracle.gemm_row_reduce_f64(synth.bits(a), "f32", synth.bits(b), "f32", op, 1.25, 0.5, c.numpy())
    assert_close(C.cpu(), out, K, a, b, "f32", "reduce C", beta=0.5)
    err = np.abs(R.cpu().double().numpy() - r)
    assert np.all(err <= red_bound(op, K, a, b, out))


LDS_CASES = {
    # name: (M, N, K, A stored [K, M], B stored [N, K], tile_m, tile_n)
    "mk_kn_interior": (384, 384, 200, False, False, 1, 1),
    "mk_kn_ragged_corner": (1000, 1537, 999, False, False, 7, 12),
    "km_kn_edges": (300, 260, 70, True, False, 2, 2),
    "mk_nk_edges": (300, 260, 70, False, True, 2, 2),
    "km_nk_interior": (512, 512, 64, True, True, 1, 2),
}


@pytest.mark.parametrize("case", list(LDS_CASES))
def test_f32_lds_image_matches_planner(case):
    M, N, K, at, bk, tm, tn = LDS_CASES[case]
    a = synth.uniform((M, K), 21, "f32")
    b = synth.uniform((K, N), 22, "f32")
    A, B = to_dev(a, at), to_dev(b, bk)
    plan = la.gemm_plan(M, N, K, la.F32, la.F32, a_transposed=at, b_kmajor=bk)
    d = plan.describe()
    bm, bn, bk_ = d["tile"]
    img = np.full(d["stage_elems"], 0xDEADBEEF, dtype=np.uint64)
    for operand, (mat, rows, cols, r0, c0) in enumerate([(a, bm, bk_, tm * bm, 0), (b, bk_, bn, 0, tn * bn)]):
        bits = synth.bits(mat)
        for r in range(rows):
            for c in range(cols):
                gr, gc = r0 + r, c0 + c
                v = bits[gr, gc] if gr < bits.shape[0] and gc < bits.shape[1] else 0
                img[la.gemm_plan_lds_offset(plan, operand, r, c)] = v
    assert not np.any(img == 0xDEADBEEF), "planner map does not cover the stage"
    nbytes = la.gemm_plan_lds_stage_bytes(plan)
    assert nbytes == 4 * d["stage_elems"]
    out = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    la.gemm_debug_lds_image(plan, A, B, None, tm, tn, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).astype(np.uint64)
    assert np.array_equal(got, img)
