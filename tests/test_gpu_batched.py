"""GPU parity of batched runs: one launch over `batch` independent matrices,
matrix b of each operand starting b * stride elements after matrix 0 (the batch
coordinate of the Tylo.jl page "TMA and Hopper WGMMA", section "The same
storage contract on both sides").  Each matrix is checked against the FP64
oracle on its own; the gaps between output matrices must stay untouched.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, oracle_gemm, swiglu_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def strided(t3, pad):
    """Place the CPU tensor t3 [batch, r, c] on the GPU with batch stride r*c + pad;
    the gaps hold NaN so that any read of them shows up in the result."""
    batch, r, c = t3.shape
    stride = r * c + pad
    flat = torch.full((batch * stride,), float("nan"), dtype=t3.dtype, device=DEV)
    view = flat.as_strided((batch, r, c), (stride, c, 1))
    view.copy_(t3.to(DEV))
    return flat, view, stride


def gaps_untouched(flat, batch, rows, cols, stride):
    mask = torch.ones(flat.numel(), dtype=torch.bool)
    for z in range(batch):
        mask[z * stride:z * stride + rows * cols] = False
    return bool(torch.isnan(flat.cpu()[mask].float()).all())


CASES = [
    # (batch, M, N, K, in, out, pads (A, B, C), kernel prefix)
    (3, 256, 512, 128, "bf16", "bf16", (64, 8, 128), "fast_"),
    (4, 100, 70, 45, "f16", "f32", (3, 5, 7), "tiled_"),
    (3, 8, 256, 256, "bf16", "f32", (8, 16, 24), "skinny_"),
    (64, 32, 40, 24, "bf16", "bf16", (0, 0, 0), "tiled_"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1] + str(c[:4]) for c in CASES])
def test_batched_gemm(case):
    batch, M, N, K, ik, ok, (pa, pb, pc), expect = case
    print("batched", case, flush=True)
    seed = 11 * M + 7 * N + K + batch
    a = synth.normal((batch, M, K), seed, ik)
    b = synth.normal((batch, K, N), seed + 1, ik, 0.5)
    c = synth.uniform((batch, M, N), seed + 2, "f32").to(synth.torch_dtype(ok))
    fa, A, sa = strided(a, pa)
    fb, B, sb = strided(b, pb)
    fc, C, sc = strided(c, pc)
    plan = la.gemm_plan(M, N, K, CODE[ik], CODE[ok], batch=batch, stride_a=sa, stride_b=sb, stride_c=sc,
                        large_tiles=expect.startswith("fast"))
    assert plan.describe()["kernel"].startswith(expect), plan.describe()["kernel"]
    la.gemm_run(plan, A, B, C, 0.5, 1.5)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        ref = oracle_gemm(a[z], b[z], ik, 0.5, 1.5, c[z].to(torch.float32))
        assert_close(got[z], ref, K, a[z], b[z], ok, "matrix %d of %s" % (z, case), beta=1.5)
    assert gaps_untouched(fc, batch, M, N, sc)


P3_CASES = [
    # (batch, M, N, K, in, out, pads (A, B, C), staging width): 257 to 512 workgroups of 64 x 64
    # tiles over the whole batch, where the planner keeps three K blocks in flight
    (100, 128, 128, 256, "bf16", "bf16", (8, 16, 24), 8),    # 400 workgroups, 16-byte aligned rows
    (80, 100, 70, 45, "f16", "f32", (3, 5, 7), 2),            # 320 workgroups, 2-byte aligned rows
]


@pytest.mark.parametrize("case", P3_CASES, ids=["vec%d" % c[-1] for c in P3_CASES])
def test_batched_three_blocks_in_flight(case):
    batch, M, N, K, ik, ok, (pa, pb, pc), vec = case
    print("batched three blocks", case, flush=True)
    seed = 5 * M + 3 * N + K + batch
    a = synth.normal((batch, M, K), seed, ik)
    b = synth.normal((batch, K, N), seed + 1, ik, 0.5)
    c = synth.uniform((batch, M, N), seed + 2, "f32").to(synth.torch_dtype(ok))
    fa, A, sa = strided(a, pa)
    fb, B, sb = strided(b, pb)
    fc, C, sc = strided(c, pc)
    plan = la.gemm_plan(M, N, K, CODE[ik], CODE[ok], batch=batch, stride_a=sa, stride_b=sb, stride_c=sc)
    d = plan.describe()
    assert d["kernel"] == "tiled_64x64x64" and d["prefetch_blocks"] == 3 and d["vec_elems"] == vec, d
    assert 256 < d["grid"] * batch <= 512
    la.gemm_run(plan, A, B, C, 0.5, 1.5)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        ref = oracle_gemm(a[z], b[z], ik, 0.5, 1.5, c[z].to(torch.float32))
        assert_close(got[z], ref, K, a[z], b[z], ok, "matrix %d of %s" % (z, case), beta=1.5)
    assert gaps_untouched(fc, batch, M, N, sc)


@pytest.mark.parametrize("shape", [(256, 256, 256), (96, 130, 70)], ids=["fast", "tiled"])
def test_batched_broadcast_B(shape):
    """stride_b = 0: every matrix of A multiplies the same B."""
    M, N, K = shape
    batch = 5
    a = synth.normal((batch, M, K), 301, "bf16")
    b = synth.normal((K, N), 302, "bf16", 0.5)
    A = a.to(DEV)
    B = b.to(DEV).unsqueeze(0).expand(batch, K, N)
    C = torch.full((batch, M, N), float("nan"), dtype=torch.float32, device=DEV)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, batch=batch, stride_b=0, large_tiles=M == 256)
    la.gemm_run(plan, A, B, C, 1.0, 0.0)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        assert_close(got[z], oracle_gemm(a[z], b, "bf16"), K, a[z], b, "f32", "broadcast B, matrix %d" % z)


def test_batched_bkmajor():
    batch, M, N, K = 3, 256, 256, 64
    a = synth.normal((batch, M, K), 311, "bf16")
    b = synth.normal((batch, K, N), 312, "bf16", 0.5)
    bt = b.transpose(1, 2).contiguous()
    fb, B, sb = strided(bt, 24)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, b_kmajor=True, batch=batch, stride_b=sb, large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast_bkmajor_")
    C = torch.full((batch, M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, a.to(DEV), B, C, 1.0, 0.0)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        assert_close(got[z], oracle_gemm(a[z], b[z], "bf16"), K, a[z], b[z], "bf16", "K-major matrix %d" % z)


@pytest.mark.parametrize("shape", [(256, 256, 64), (100, 70, 45)], ids=["fast", "tiled"])
def test_batched_gate_up_and_swiglu(shape):
    M, N, K = shape
    batch = 2
    x = synth.normal((batch, M, K), 321, "bf16")
    wg = synth.normal((batch, K, N), 322, "bf16", 0.3)
    wu = synth.normal((batch, K, N), 323, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, batch=batch, large_tiles=M == 256)
    X, Wg, Wu = x.to(DEV), wg.to(DEV), wu.to(DEV)
    G = torch.full((batch, M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    U = torch.full_like(G, float("nan"))
    H = torch.full_like(G, float("nan"))
    la.gemm_gate_up_run(plan, X, Wg, Wu, G, U)
    la.gemm_gate_up_swiglu_run(plan, X, Wg, Wu, H)
    torch.cuda.synchronize()
    for z in range(batch):
        for name, w, out in (("G", wg[z], G), ("U", wu[z], U)):
            assert_close(out.cpu()[z], oracle_gemm(x[z], w, "bf16"), K, x[z], w, "bf16",
                         "gate_up %s matrix %d" % (name, z))
        h_ref, g_ref, u_ref = oracle.gate_up_swiglu_f64(synth.bits(x[z]), synth.bits(wg[z]), synth.bits(wu[z]),
                                                        "bf16")
        err = np.abs(H.cpu()[z].to(torch.float64).numpy() - h_ref)
        assert np.all(err <= swiglu_bound(K, x[z], wg[z], wu[z], g_ref, u_ref, h_ref, "bf16")), z
