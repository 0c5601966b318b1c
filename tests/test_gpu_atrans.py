"""GPU parity of A stored [K, M] (M contiguous, GEMM_FLAG_A_TRANSPOSED): either
major order is the same matrix (Tylo.jl "Layouts, storage and ownership",
section "A layout is a function": permutedims swaps the modes).

The GPU receives A^T's storage ([K, M], a.t().contiguous()); the oracle reads
the same values as A[i, k] by index, with its arithmetic unchanged.  Covered:
the full-tile kernels (plain and gate/up), the general kernel with 16-byte
staging (aligned and 2-byte aligned with chunks cut at M's edge), 64 x 64 and
128 x 128 tiles, padded leading dimensions, gate/up and SwiGLU, batched runs,
the LDS image of each kernel family against the planner's map, and exact
identity / permutation products.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import synth
from parity import assert_close, oracle_gemm, swiglu_bound
from test_gpu_gemm import _expected_image, _lds_image

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def run_at(a, b, out_kind, alpha=1.0, beta=0.0, c=None, expect=None, large_tiles=False, lda=None):
    """a [M,K], b [K,N] CPU tensors; A goes to the GPU as its transpose [K, M] (row stride lda)."""
    M, K = a.shape
    N = b.shape[1]
    in_kind = "bf16" if a.dtype == torch.bfloat16 else "f16"
    lda = lda or max(1, M)
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], lda=lda, large_tiles=large_tiles, a_transposed=True)
    d = plan.describe()
    assert d["a_order"] == "km"
    if expect is not None:
        assert d["kernel"].startswith(expect), d["kernel"]
    At = torch.full((K, lda), float("nan"), dtype=a.dtype, device=DEV)
    At[:, :M] = a.t().to(DEV)
    A = At[:, :M]
    C = torch.full((M, N), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV) if c is None else c.to(DEV).clone()
    la.gemm_run(plan, A, b.to(DEV), C, alpha, beta)
    torch.cuda.synchronize()
    return C.cpu(), d


SHAPES = [
    # (M, N, K, large_tiles, expected kernel)
    (256, 256, 64, True, "fast_atrans_"),
    (512, 768, 320, True, "fast_atrans_"),
    (2048, 1024, 512, False, "fast_atrans_"),        # 32 full tiles: planned on the full-tile kernel
    (1000, 1537, 999, False, "tiled_64x64"),        # chunks cut at N's edge; M whole
    (1003, 512, 257, False, "tiled_64x64"),         # chunks cut at M's edge
    (1536, 1537, 999, True, "tiled_128x128"),
    (9, 64, 64, False, "tiled_64x64"),              # one whole M chunk and one of a single element
    (200, 72, 1000, False, "tiled_64x64"),
    (129, 257, 130, False, "tiled_64x64"),
    (64, 64, 64, False, "tiled_64x64"),
    (300, 300, 1, False, "tiled_64x64"),
]


@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s[:3]) for s in SHAPES])
def test_atrans_shapes(shape, in_kind, out_kind):
    M, N, K, large, expect = shape
    print("atrans", shape, in_kind, out_kind, flush=True)
    seed = 5 * M + 11 * N + K
    a = synth.uniform((M, K), seed, in_kind)
    b = synth.uniform((K, N), seed + 1, in_kind)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got, _ = run_at(a, b, out_kind, 1.5, -0.5, c, expect=expect, large_tiles=large)
    ref = oracle_gemm(a, b, in_kind, 1.5, -0.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "A^T %s" % (shape,), beta=-0.5)


@pytest.mark.parametrize("shape", [(512, 512, 256, 520), (1000, 1537, 999, 1003), (300, 200, 100, 307)],
                         ids=["fast_pad8", "tiled_pad3", "tiled_small_pad7"])
def test_atrans_padded_leading_dimension(shape):
    M, N, K, lda = shape
    a = synth.normal((M, K), 71, "bf16")
    b = synth.normal((K, N), 72, "bf16", 0.5)
    got, d = run_at(a, b, "f32", lda=lda, large_tiles=M % 256 == 0)
    assert d["lda"] == lda
    assert_close(got, oracle_gemm(a, b, "bf16"), K, a, b, "f32", "A^T lda %d" % lda)


@pytest.mark.parametrize("kind", ["fast", "tiled"])
def test_atrans_identity_and_permutation_are_exact(kind):
    K, M = 256, 256 if kind == "fast" else 200
    a = synth.uniform((M, K), 17, "bf16")
    eye = torch.eye(K, dtype=torch.bfloat16)
    got, d = run_at(a, eye, "f32", large_tiles=kind == "fast")
    assert d["kernel"].startswith("fast_atrans" if kind == "fast" else "tiled_")
    assert torch.equal(got, a.to(torch.float32))
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(18))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[perm, torch.arange(K)] = 1
    got, _ = run_at(a, P, "bf16", large_tiles=kind == "fast")
    assert torch.equal(got, a[:, perm])


@pytest.mark.parametrize("shape", [(512, 256, 192, True), (300, 200, 100, False), (256, 384, 64, True)],
                         ids=["fast", "tiled_edges", "fast_min_k"])
def test_atrans_gate_up_and_swiglu(shape):
    M, N, K, large = shape
    x = synth.normal((M, K), 31, "bf16")
    wg = synth.normal((K, N), 32, "bf16", 0.3)
    wu = synth.normal((K, N), 33, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, large_tiles=large, a_transposed=True)
    want = "fast_gate_up_atrans_" if M % 256 == 0 and large else "tiled_"
    assert plan.describe()["kernel"].startswith(want), plan.describe()["kernel"]
    Xt = x.t().contiguous().to(DEV)
    G = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    U = torch.full_like(G, float("nan"))
    la.gemm_gate_up_run(plan, Xt, wg.to(DEV), wu.to(DEV), G, U)
    H = torch.full_like(G, float("nan"))
    la.gemm_gate_up_swiglu_run(plan, Xt, wg.to(DEV), wu.to(DEV), H)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle_gemm(x, wg, "bf16"), oracle_gemm(x, wu, "bf16")
    assert_close(G.cpu(), g_ref, K, x, wg, "bf16", "A^T gate")
    assert_close(U.cpu(), u_ref, K, x, wu, "bf16", "A^T up")
    with np.errstate(over="ignore"):
        h_ref = g_ref / (1.0 + np.exp(-g_ref)) * u_ref
    err = np.abs(H.cpu().double().numpy() - h_ref)
    assert np.all(err <= swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16"))


def test_atrans_batched():
    """Batch of A^T matrices with padded batch strides; the gaps between outputs stay NaN."""
    batch, M, N, K = 5, 100, 70, 45
    a = synth.normal((batch, M, K), 81, "f16")
    b = synth.normal((batch, K, N), 82, "f16", 0.5)
    sa, sc = K * M + 11, M * N + 5
    At = torch.full((batch * sa,), float("nan"), dtype=torch.float16, device=DEV)
    A = At.as_strided((batch, K, M), (sa, M, 1))
    A.copy_(a.transpose(1, 2).to(DEV))
    Cf = torch.full((batch * sc,), float("nan"), dtype=torch.float32, device=DEV)
    C = Cf.as_strided((batch, M, N), (sc, N, 1))
    plan = la.gemm_plan(M, N, K, la.F16, la.F32, batch=batch, stride_a=sa, stride_b=K * N, stride_c=sc,
                        a_transposed=True)
    la.gemm_run(plan, A, b.to(DEV), C)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        assert_close(got[z], oracle_gemm(a[z], b[z], "f16"), K, a[z], b[z], "f32", "A^T batch %d" % z)
    mask = torch.ones(batch * sc, dtype=torch.bool)
    for z in range(batch):
        mask[z * sc:z * sc + M * N] = False
    assert torch.isnan(Cf.cpu()[mask]).all()


LDS_CASES = {
    # name: (M, N, K, kind, gate_up, tile_m, tile_n, expected kernel prefix, large tiles)
    "fast_atrans": (512, 512, 256, "bf16", False, 1, 1, "fast_atrans_", True),
    "fast_gate_up_atrans": (512, 256, 128, "f16", True, 1, 0, "fast_gate_up_atrans_", True),
    "tiled64_atrans_m_edge": (1003, 512, 257, "bf16", False, 15, 3, "tiled_64x64", False),
    "tiled128_atrans_edges": (1536, 1537, 999, "f16", False, 11, 12, "tiled_128x128", True),
    "tiled64_atrans_aligned": (512, 512, 200, "bf16", False, 2, 1, "tiled_64x64", False),
}


@pytest.mark.parametrize("case", list(LDS_CASES))
def test_atrans_lds_image_matches_planner(case):
    M, N, K, kind, gu, tm, tn, prefix, large = LDS_CASES[case]
    a = synth.uniform((M, K), 21, kind)
    b = synth.uniform((K, N), 22, kind)
    b2 = synth.uniform((K, N), 23, kind) if gu else None
    plan = la.gemm_plan(M, N, K, CODE[kind], la.F32, gate_up=gu, large_tiles=large, a_transposed=True)
    d = la.gemm_plan_describe(plan)
    assert d["kernel"].startswith(prefix), d["kernel"]
    bm, bn, bk = d["tile"]
    ops = [(a, bm, bk, tm * bm, 0), (b, bk, bn, 0, tn * bn)]
    if gu:
        ops.append((b2, bk, bn, 0, tn * bn))
    want, _ = _expected_image(plan, ops, tm, tn)
    got = _lds_image(plan, a.t().contiguous().to(DEV), b.to(DEV), b2.to(DEV) if gu else None, tm, tn)
    assert not np.any(want == 0xDEAD), "planner map does not cover the stage"
    assert np.array_equal(got.astype(np.uint32), want)
