"""GPU parity of the GEMM with a row reduction of its FP32 outputs (sum, maximum,
minimum along every output row; Tylo.jl "TMA and Hopper WGMMA", section "WGMMA
values and ownership"), through the C ABI, against the binary64 oracle.

Bounds: the GPU folds the FP32 values v[i, j] = alpha * acc + beta * C_old,
each within e[i, j] = 2^-20 K max|A| max|B| + 2^-22 |out| of the oracle's
out[i, j].  Maximum and minimum move by at most max_j e[i, j]; a sum by at
most sum_j e[i, j] plus the FP32 rounding of an N-term sum,
(N + 8) 2^-24 sum_j |out[i, j]|.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, max_abs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def red_bound(op, K, a, b, out):
    e = 2.0 ** -20 * K * max_abs(a) * max_abs(b) + 2.0 ** -22 * np.abs(out)
    if op == "sum":
        return e.sum(axis=1) + (out.shape[1] + 8) * 2.0 ** -24 * np.abs(out).sum(axis=1)
    return e.max(axis=1)


def run_reduce(a, b, out_kind, op, alpha=1.0, beta=0.0, c=None, b_kmajor=False, expect=None):
    M, K = a.shape
    N = b.shape[1]
    in_kind = "bf16" if a.dtype == torch.bfloat16 else "f16"
    # full-tile cases are small grids: pin their kernel with the large-tile flag
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], b_kmajor=b_kmajor,
                        large_tiles=expect is not None and expect.startswith("fast"))
    if expect is not None:
        assert plan.describe()["kernel"].startswith(expect), plan.describe()["kernel"]
    A = a.to(DEV)
    B = b.t().contiguous().to(DEV) if b_kmajor else b.to(DEV)
    C = torch.full((M, N), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV) if c is None \
        else c.to(DEV).clone()
    R = torch.full((M,), 12345.0, dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, A, B, C, alpha, beta, op, R)
    torch.cuda.synchronize()
    return C.cpu(), R.cpu().double().numpy()


def check(op, a, b, in_kind, out_kind, alpha, beta, c, got_c, got_r, what):
    K = a.shape[1]
    cin = None if c is None else c.to(torch.float32).numpy()
    out, r = oracle.gemm_row_reduce_f64(synth.bits(a), in_kind, synth.bits(b), in_kind, op, alpha, beta, cin)
    assert_close(got_c, out, K, a, b, out_kind, what + " C", beta=beta)
    tol = red_bound(op, K, a, b, out)
    err = np.abs(got_r - r)
    bad = ~(err <= tol)
    assert not bad.any(), "%s %s: %d rows out of tolerance, first %d: gpu=%r oracle=%r tol=%r" % (
        what, op, int(bad.sum()), int(np.argmax(bad)), got_r[np.argmax(bad)], r[np.argmax(bad)], tol[np.argmax(bad)])


CASES = [
    # (M, N, K, in, out, alpha, beta, b_kmajor, kernel)
    (512, 512, 256, "bf16", "bf16", 1.0, 0.0, False, "fast_"),
    (256, 768, 128, "f16", "f32", 0.5, 1.5, False, "fast_"),
    (512, 256, 64, "bf16", "f32", 1.0, 0.0, True, "fast_bkmajor_"),
    (1000, 1537, 999, "f16", "f32", 1.5, -0.5, False, "tiled_"),
    (77, 45, 33, "bf16", "bf16", 1.0, 0.0, False, "tiled_"),
    (16, 1024, 512, "bf16", "f32", 1.0, 0.0, False, "skinny_"),
    (5, 384, 256, "f16", "f32", 2.0, 0.25, False, "skinny_"),
]


@pytest.mark.parametrize("op", ["sum", "max", "min"])
@pytest.mark.parametrize("case", CASES, ids=[c[-1] + str(c[:3]) for c in CASES])
def test_row_reduce(case, op):
    M, N, K, ik, ok, alpha, beta, bkm, expect = case
    print("reduce", case, op, flush=True)
    seed = 3 * M + 5 * N + K
    a = synth.normal((M, K), seed, ik)
    b = synth.normal((K, N), seed + 1, ik, 0.5)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(ok)) if beta != 0.0 else None
    got_c, got_r = run_reduce(a, b, ok, op, alpha, beta, c, bkm, expect)
    check(op, a, b, ik, ok, alpha, beta, c, got_c, got_r, str(case))


@pytest.mark.parametrize("shape", [(256, 512, 512), (100, 300, 200)], ids=["fast", "tiled"])
def test_exact_cases(shape):
    """Permutation B: rows of the output are permuted rows of A, so max and min are
    A's, bit for bit; all-ones operands: every row sums to N * K exactly."""
    M, N, K = shape
    a = synth.normal((M, K), 51, "bf16")
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(52))[:N] if N <= K else None
    if perm is not None:
        P = torch.zeros((K, N), dtype=torch.bfloat16)
        P[perm, torch.arange(N)] = 1
        want = a.float()[:, perm]
        for op, f in (("max", torch.amax), ("min", torch.amin)):
            _, r = run_reduce(a, P, "f32", op)
            assert np.array_equal(r, f(want, dim=1).double().numpy()), op
    ones_a = torch.ones((M, K), dtype=torch.bfloat16)
    ones_b = torch.ones((K, N), dtype=torch.bfloat16)
    _, r = run_reduce(ones_a, ones_b, "f32", "sum")
    assert np.all(r == float(N * K))


def test_batched_reduce_and_empty_rows():
    batch, M, N, K = 3, 256, 256, 64
    a = synth.normal((batch, M, K), 61, "bf16")
    b = synth.normal((batch, K, N), 62, "bf16", 0.5)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, batch=batch)
    C = torch.empty((batch, M, N), dtype=torch.float32, device=DEV)
    R = torch.empty((batch, M), dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, a.to(DEV), b.to(DEV), C, 1.0, 0.0, "max", R)
    torch.cuda.synchronize()
    for z in range(batch):
        check("max", a[z], b[z], "bf16", "f32", 1.0, 0.0, None, C.cpu()[z], R.cpu()[z].double().numpy(),
              "batch %d" % z)
    # N == 0: nothing to reduce, R holds the identity of each operation
    p0 = la.gemm_plan(8, 0, 16, la.BF16, la.F32)
    A0 = torch.zeros((8, 16), dtype=torch.bfloat16, device=DEV)
    B0 = torch.zeros((16, 0), dtype=torch.bfloat16, device=DEV)
    C0 = torch.zeros((8, 0), dtype=torch.float32, device=DEV)
    for op, ident in (("sum", 0.0), ("max", -np.inf), ("min", np.inf)):
        R0 = torch.full((8,), 7.0, device=DEV)
        la.gemm_run_reduce(p0, A0, B0, C0, 1.0, 0.0, op, R0)
        torch.cuda.synchronize()
        assert np.all(R0.cpu().numpy() == ident), op


def test_reduce_graph_replay():
    """The fill kernel and the GEMM replay from a HIP graph with the eager result each time."""
    M, N, K = 512, 512, 128
    a = synth.normal((M, K), 71, "bf16")
    b = synth.normal((K, N), 72, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    A, B = a.to(DEV), b.to(DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    R = torch.empty((M,), dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, A, B, C, 1.0, 0.0, "max", R)
    torch.cuda.synchronize()
    eager_c, eager_r = C.clone(), R.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.gemm_run_reduce(plan, A, B, C, 1.0, 0.0, "max", R)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.gemm_run_reduce(plan, A, B, C, 1.0, 0.0, "max", R)
    for it in range(4):
        C.zero_()
        R.fill_(123.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager_c) and torch.equal(R, eager_r), "replay %d" % it
        A.add_(0)
