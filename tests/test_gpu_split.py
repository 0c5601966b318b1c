"""GPU parity of gemm_run_split: the skinny shapes with K cut into ranges.

The plan's split form writes each K range's FP32 partial product into a
caller-owned workspace (one launch, ranges along the grid's y dimension) and a
second kernel sums the ranges in order with alpha, beta and the rounding.  Only
the order of the FP32 additions differs from a single pass, so the bound is the
plain GEMM's (tests/parity.py).  Cases: the skinny kernel's split form for 1 to
128 rows of A and the full-tile kernel's on 128-row tiles (M and N edges, K blocks of
64 and 32, one-byte inputs, a 512 x 4096 x 14336 prefill shape on sampled rows), both storages of B,
bf16 / fp16 inputs with fp32 / bf16 / fp16 outputs, alpha and beta with C in
padded rows that must stay untouched, one-byte inputs, the skinny_split workload
(32 x 4096 x 14336, B stored [N, K]) in full, determinism, the workspace
checks of the C ABI, plans without a split form, and graph replays.
"""
import ctypes

import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import synth
from parity import assert_close, band_rows, oracle_gemm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32, "f8e4m3": la.F8E4M3, "f8e5m2": la.F8E5M2}


def run_split(a, b, in_kind, out_kind, km, alpha=1.0, beta=0.0, c=None, b_kind=None, workspace=None):
    """a [M,K], b [K,N] CPU tensors; C lives in rows padded by 8 NaN columns.  Returns (C, plan description)."""
    M, K = a.shape
    N = b.shape[1]
    ld = N + 8
    Cbuf = torch.full((M, ld), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    C = Cbuf[:, :N]
    if c is not None:
        C.copy_(c.to(DEV))
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], ldc=ld, b_kmajor=km,
                        b_type=CODE[b_kind or in_kind])
    d = plan.describe()
    B = b.t().contiguous().to(DEV) if km else b.to(DEV)
    la.gemm_run_split(plan, a.to(DEV), B, C, alpha, beta, workspace)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf[:, N:].cpu().float()).all(), "a store landed in C's row padding"
    return C.cpu(), d


SHAPES = [
    # (M, N, K, B stored [N, K])
    (1, 4096, 4096, False),
    (1, 4096, 4096, True),
    (16, 1024, 2048, True),
    (13, 2048, 4096, False),
    (32, 2048, 4096, False),
    (27, 1024, 8192, True),
    (48, 1024, 4096, True),
    (64, 2048, 2048, False),
    (100, 1024, 2048, False),
    (128, 2048, 1024, True),
]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("case", SHAPES, ids=[str(c) for c in SHAPES])
def test_split_shapes(case, out_kind):
    M, N, K, km = case
    print("split", case, out_kind, flush=True)
    seed = 23 * M + N + 7 * K + km
    a = synth.normal((M, K), seed, "bf16")
    b = synth.normal((K, N), seed + 1, "bf16", 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got, d = run_split(a, b, "bf16", out_kind, km, 0.75, -1.25, c)
    assert d["split_k"] > 1 and d["split_kernel"].startswith("skinny_"), d
    assert d["workspace_bytes"] == d["split_k"] * M * N * 4
    ref = oracle_gemm(a, b, "bf16", 0.75, -1.25, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "split %s" % (case,), beta=-1.25)


FAST = [
    # (M, N, K, B stored [N, K]): the 256-wide kernel's split form (at most 64 tiles)
    (256, 1024, 4096, False),
    (300, 520, 2048, False),      # M and N edges
    (300, 520, 2112, True),       # ranges of 1056: K blocks of 32
    (129, 4096, 2048, True),      # one row past the skinny range, M edge
    (1000, 1024, 4096, True),
    (512, 2048, 8192, False),
]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("case", FAST, ids=[str(c) for c in FAST])
def test_fast_split_shapes(case, out_kind):
    M, N, K, km = case
    print("fast split", case, out_kind, flush=True)
    seed = 29 * M + N + 3 * K + km
    a = synth.normal((M, K), seed, "bf16")
    b = synth.normal((K, N), seed + 1, "bf16", 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got, d = run_split(a, b, "bf16", out_kind, km, 1.5, 0.5, c)
    assert d["split_k"] > 1 and d["split_kernel"].startswith("fast_"), d
    ref = oracle_gemm(a, b, "bf16", 1.5, 0.5, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "fast split %s" % (case,), beta=0.5)


def test_fast_split_prefill_shape_sampled_rows():
    """512 x 4096 x 14336, B stored [N, K] (4 ranges over 32 tiles), on rows covering both tile bands."""
    M, N, K = 512, 4096, 14336
    a = synth.normal((M, K), 551, "bf16")
    b = synth.normal((K, N), 552, "bf16", 0.02)
    got, d = run_split(a, b, "bf16", "bf16", True)
    assert d["split_k"] == 4 and d["split_grid"] == [64, 4] and d["split_kernel"] == "fast_bkmajor_128x256x64", d
    rows = band_rows(M, seed=553)
    ref = oracle_gemm(a, b, "bf16", rows=rows)
    assert_close(got[rows], ref, K, a, b, "bf16", "fast split prefill shape")


@pytest.mark.parametrize("K,blk", [(4096, 128), (4224, 64)], ids=["blocks128", "blocks64"])
def test_fast_split_one_byte(K, blk):
    """One-byte split forms on 128-row tiles: ranges of 1024 pairs (blocks of 128 codes) and of 1056
    pairs (blocks of 64 codes)."""
    M, N = 512, 2048
    a = synth.normal((M, K), 561, "f8e4m3", 1.0)
    b = synth.normal((K, N), 562, "f8e5m2", 0.5)
    got, d = run_split(a, b, "f8e4m3", "bf16", True, b_kind="f8e5m2")
    assert d["split_k"] == 2 and d["split_kernel"] == "fast_f8_128x256x%d" % blk, d
    ref = oracle_gemm(a, b, "f8e4m3", b_kind="f8e5m2")
    assert_close(got, ref, K, a, b, "bf16", "fast split f8")


@pytest.mark.parametrize("case", [(16, 2048, 4096, True), (64, 1024, 2048, False)], ids=["nk", "kn"])
def test_split_f16_in_f16_out_beta_zero_nan_c(case):
    """beta = 0: C is not read (NaN there stays out of the result)."""
    M, N, K, km = case
    a = synth.normal((M, K), 301, "f16")
    b = synth.normal((K, N), 302, "f16", 0.05)
    got, d = run_split(a, b, "f16", "f16", km)
    assert d["split_k"] > 1
    ref = oracle_gemm(a, b, "f16")
    assert_close(got, ref, K, a, b, "f16", "split f16 %s" % (case,))


F8 = [
    (16, 2048, 8192, "f8e4m3", "f8e4m3"),
    (20, 1024, 4096, "f8e4m3", "f8e5m2"),
    (64, 1024, 4096, "f8e5m2", "f8e4m3"),
    (128, 2048, 2048, "f8e5m2", "f8e5m2"),
]


@pytest.mark.parametrize("case", F8, ids=[str(c) for c in F8])
def test_split_one_byte(case):
    M, N, K, ka, kb = case
    print("split f8", case, flush=True)
    a = synth.normal((M, K), 401 + M, ka, 1.0)
    b = synth.normal((K, N), 402 + M, kb, 0.5)
    c = synth.uniform((M, N), 403 + M, "f32").to(torch.bfloat16)
    got, d = run_split(a, b, ka, "bf16", True, 1.0, 0.5, c, b_kind=kb)
    assert d["split_k"] > 1 and d["split_kernel"].startswith("skinny_f8_"), d
    ref = oracle_gemm(a, b, ka, 1.0, 0.5, c.to(torch.float32), b_kind=kb)
    assert_close(got, ref, K, a, b, "bf16", "split f8 %s" % (case,), beta=0.5)


def test_split_decode_shape_full():
    """The skinny_split workload (32 x 4096 x 14336, B stored [N, K]: a down projection at a decode
    batch of 32) in full, in the launch configuration the bench times (plan, workspace, entry point)."""
    w = synth.WORKLOADS["skinny_split"]
    x = synth.make_inputs(w)
    plan = la.gemm_plan(w.M, w.N, w.K, la.BF16, la.F32, b_kmajor=True)
    d = plan.describe()
    assert d["split_k"] == 4 and d["split_grid"] == [64, 4], d
    ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device=DEV)
    la.gemm_run_split(plan, x["A"].to(DEV), x["B"].t().contiguous().to(DEV), C, w.alpha, w.beta, ws)
    torch.cuda.synchronize()
    ref = oracle_gemm(x["A"], x["B"], "bf16")
    assert_close(C.cpu(), ref, w.K, x["A"], x["B"], "f32", "skinny_split workload")


def test_split_is_deterministic_and_matches_single_pass_within_rounding():
    M, N, K = 32, 2048, 4096
    a = synth.normal((M, K), 601, "bf16")
    b = synth.normal((K, N), 602, "bf16", 0.05)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, b_kmajor=True)
    A, B = a.to(DEV), b.t().contiguous().to(DEV)
    ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        ws.fill_(0xFF)                                   # workspace contents on entry do not matter
        la.gemm_run_split(plan, A, B, C, workspace=ws)
        torch.cuda.synchronize()
        outs.append(C.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    single = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    la.gemm_run(plan, A, B, single)
    torch.cuda.synchronize()
    ref = oracle_gemm(a, b, "bf16")
    assert_close(outs[0], ref, K, a, b, "f32", "split")
    assert_close(single.cpu(), ref, K, a, b, "f32", "single pass")


def test_split_workspace_checks():
    """A missing, short or misaligned workspace is an error and nothing is written."""
    M, N, K = 16, 1024, 2048
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, b_kmajor=True)
    need = la.gemm_plan_workspace_bytes(plan)
    assert need == plan.describe()["split_k"] * M * N * 4 > 0
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    lib = la.load()
    ws = torch.empty(need + 16, dtype=torch.uint8, device=DEV)
    vp = ctypes.c_void_p

    def call(w, nbytes):
        return lib.gemm_run_split(plan.handle, vp(A.data_ptr()), vp(B.data_ptr()), vp(C.data_ptr()),
                                  ctypes.c_float(1.0), ctypes.c_float(0.0), w, ctypes.c_int64(nbytes), vp(0))
    assert call(vp(0), need) == 1                                  # GEMM_ERR_NULL
    assert call(vp(ws.data_ptr()), need - 4) == 2                  # GEMM_ERR_INVALID_ARG
    assert call(vp(ws.data_ptr() + 4), need) == 4                  # GEMM_ERR_ALIGNMENT
    torch.cuda.synchronize()
    assert torch.isnan(C.cpu()).all()
    with pytest.raises(la.GemmError):
        la.gemm_run_split(plan, A, B, C, workspace=ws[: need - 16])
    assert call(vp(ws.data_ptr()), need) == 0
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), torch.zeros((M, N)))


def test_plan_without_split_form_runs_as_gemm_run():
    M, N, K = 16, 28672, 1024
    a = synth.normal((M, K), 701, "bf16")
    b = synth.normal((K, N), 702, "bf16", 0.05)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    assert plan.describe()["split_k"] == 1 and la.gemm_plan_workspace_bytes(plan) == 0
    A, B = a.to(DEV), b.to(DEV)
    C1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    C2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, A, B, C1)
    assert la.gemm_run_split(plan, A, B, C2) is None              # no workspace needed, none allocated
    torch.cuda.synchronize()
    assert torch.equal(C1.cpu(), C2.cpu())


def test_split_graph_replays():
    """Both launches captured in a HIP graph; each replay (eager work and synchronisations between
    them) must equal the eager result bit for bit."""
    M, N, K = 64, 2048, 4096
    a = synth.normal((M, K), 801, "bf16")
    b = synth.normal((K, N), 802, "bf16", 0.05)
    c = synth.uniform((M, N), 803, "f32").to(torch.bfloat16)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, b_kmajor=True)
    assert plan.describe()["split_k"] > 1
    A, B, C0 = a.to(DEV), b.t().contiguous().to(DEV), c.to(DEV)
    ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    eager = C0.clone()
    la.gemm_run_split(plan, A, B, eager, 1.0, 0.5, ws)
    torch.cuda.synchronize()
    C = C0.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            la.gemm_run_split(plan, A, B, C, 1.0, 0.5, ws)
    torch.cuda.synchronize()
    for i in range(4):
        C.copy_(C0)
        ws.fill_(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.cpu(), eager.cpu()), "replay %d" % i
    ref = oracle_gemm(a, b, "bf16", 1.0, 0.5, c.to(torch.float32))
    assert_close(eager.cpu(), ref, K, a, b, "bf16", "split graph", beta=0.5)
