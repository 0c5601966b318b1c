"""GPU parity of the 256-wide kernel with 128-row tiles (8 waves of 64 x 64), which the planner takes
for plain GEMMs whose grid of 256 x 256 tiles would hold at most 128 of them (K blocks of 64 when
K is a multiple of 64, else of 32).

Cases, each planned without flags (the planner's own choice is asserted): whole tiles, M and N
ending inside a tile, a K tail, B stored [K, N] and [N, K], bf16 and fp16 inputs, fp32 / bf16 /
fp16 outputs with alpha, beta and C in NaN-padded rows, a batch, the three row reductions, the
staged LDS image of an edge tile against the planner's map, one-byte inputs (the K-major
configuration on byte pairs) with edges and a K tail, and the prefill_384 workload in full as the
bench runs it.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, band_rows, max_abs, oracle_gemm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}

SHAPES = [
    # (M, N, K, B stored [N, K]) -- all planned on 128-row tiles
    (2048, 1024, 512, False),     # 32 tiles of 256: whole
    (1024, 4096, 2048, True),     # 64 tiles
    (384, 11008, 1024, False),    # 43 columns, M = 3 x 128 (256-row tiles would pad it to 512)
    (1000, 4096, 1000, True),     # M edge and a K tail of 8
    (200, 28672, 512, False),     # one 128-row tile and one of 72 rows, 112 columns
]


def _plan(M, N, K, km, in_kind, out_kind, ldc):
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], b_kmajor=km, ldc=ldc)
    d = plan.describe()
    bk = 64 if K % 64 == 0 else 32      # K blocks of 64 when K allows
    assert d["kernel"] == ("fast_bkmajor_128x256x%d" if km else "fast_128x256x%d") % bk, d["kernel"]
    return plan


@pytest.mark.parametrize("io", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16")], ids=["bf16", "bf16_f32", "f16"])
@pytest.mark.parametrize("case", SHAPES, ids=[str(c) for c in SHAPES])
def test_fast128_shapes(case, io):
    M, N, K, km = case
    in_kind, out_kind = io
    print("fast128", case, io, flush=True)
    seed = 31 * M + N + K + km
    a = synth.normal((M, K), seed, in_kind, 1.0 / 8)
    b = synth.normal((K, N), seed + 1, in_kind, 1.0 / 8)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    ld = N + 8
    plan = _plan(M, N, K, km, in_kind, out_kind, ld)
    Cbuf = torch.full((M, ld), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    C = Cbuf[:, :N]
    C.copy_(c.to(DEV))
    B = b.t().contiguous().to(DEV) if km else b.to(DEV)
    la.gemm_run(plan, a.to(DEV), B, C, 0.75, -0.5)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf[:, N:].cpu().float()).all(), "a store landed in C's row padding"
    rows = band_rows(M, band=128, wave_rows=64, seed=seed) if M > 512 else list(range(M))
    ref = oracle_gemm(a, b, in_kind, 0.75, -0.5, c.to(torch.float32), rows=rows)
    assert_close(C.cpu()[rows], ref, K, a, b, out_kind, "fast128 %s %s" % (case, io), beta=-0.5)


def test_fast128_batch():
    """64 batch entries of 256 x 256 x 256 (64 tiles of 256, so 128-row tiles), B broadcast."""
    Z, M, N, K = 64, 256, 256, 256
    a = synth.normal((Z, M, K), 71, "bf16", 0.25)
    b = synth.normal((K, N), 72, "bf16", 0.25)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, batch=Z, stride_b=0)
    assert plan.describe()["kernel"] == "fast_128x256x64"
    C = torch.full((Z, M, N), float("nan"), dtype=torch.float32, device=DEV)
    Bb = torch.as_strided(b.to(DEV), (Z, K, N), (0, N, 1))
    la.gemm_run(plan, a.to(DEV), Bb, C)
    torch.cuda.synchronize()
    for z in (0, 17, 63):
        ref = oracle_gemm(a[z], b, "bf16")
        assert_close(C[z].cpu(), ref, K, a[z], b, "f32", "fast128 batch %d" % z)


@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_fast128_row_reductions(op):
    M, N, K = 1024, 4096, 512
    a = synth.normal((M, K), 81, "bf16", 0.25)
    b = synth.normal((K, N), 82, "bf16", 0.25)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32)
    assert plan.describe()["kernel"] == "fast_128x256x64"
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    R = torch.full((M,), 12345.0, dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, a.to(DEV), b.to(DEV), C, 1.0, 0.0, op, R)
    torch.cuda.synchronize()
    rows = band_rows(M, band=128, wave_rows=64, seed=83)
    out, r = oracle.gemm_row_reduce_f64(synth.bits(a[rows]), "bf16", synth.bits(b), "bf16", op, 1.0, 0.0, None)
    assert_close(C.cpu()[rows], out, K, a, b, "f32", "fast128 reduce C")
    e = 2.0 ** -20 * K * max_abs(a) * max_abs(b) + 2.0 ** -22 * np.abs(out)
    tol = e.sum(axis=1) + (N + 8) * 2.0 ** -24 * np.abs(out).sum(axis=1) if op == "sum" else e.max(axis=1)
    err = np.abs(R.cpu().double().numpy()[rows] - r)
    assert np.all(err <= tol), "%s: max err %g" % (op, err.max())


def test_fast128_lds_image_of_an_edge_tile():
    """Stage 0 of the last tile (M and N edges) of 1000 x 4000 x 1024 (B [N, K]) as the kernel stages it."""
    M, N, K = 1000, 4000, 1024
    a = synth.uniform((M, K), 91, "bf16")
    b = synth.uniform((K, N), 92, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, b_kmajor=True)
    d = plan.describe()
    assert d["kernel"] == "fast_bkmajor_128x256x64" and d["tile"] == [128, 256, 64], d
    bk = 64
    tm, tn = (M + 127) // 128 - 1, (N + 255) // 256 - 1
    img = torch.zeros(la.gemm_plan_lds_stage_bytes(plan) // 2, dtype=torch.int16, device=DEV)
    la.gemm_debug_lds_image(plan, a.to(DEV), b.t().contiguous().to(DEV), None, tm, tn, img)
    torch.cuda.synchronize()
    got = img.cpu().numpy().view(np.uint16)
    abits, bbits = synth.bits(a), synth.bits(b)
    checked = 0
    for r in range(128):
        for k in range(bk):
            if tm * 128 + r < M:
                assert got[la.gemm_plan_lds_offset(plan, 0, r, k)] == abits[tm * 128 + r, k], (r, k)
                checked += 1
    for k in range(bk):
        for n in range(256):
            if tn * 256 + n < N:
                assert got[la.gemm_plan_lds_offset(plan, 1, k, n)] == bbits[k, tn * 256 + n], (k, n)
                checked += 1
    assert checked == (M - tm * 128) * bk + bk * (N - tn * 256)


F8_SHAPES = [
    # (M, N, K, A format, B format): one-byte inputs on 128-row tiles (B stored [N, K])
    (1024, 4096, 2048, "f8e4m3", "f8e4m3"),
    (1024, 4096, 1040, "f8e4m3", "f8e5m2"),  # a K tail of 16 codes
    (1000, 4104, 1024, "f8e5m2", "f8e4m3"),  # M and N edges
]


@pytest.mark.parametrize("out_kind", ["bf16", "f32"])
@pytest.mark.parametrize("case", F8_SHAPES, ids=[str(c) for c in F8_SHAPES])
def test_fast128_one_byte(case, out_kind):
    M, N, K, ka, kb = case
    print("fast128 f8", case, out_kind, flush=True)
    a = synth.normal((M, K), 101 + M, ka, 1.0)
    b = synth.normal((K, N), 102 + N, kb, 0.5)
    c = synth.uniform((M, N), 103 + K, "f32").to(synth.torch_dtype(out_kind))
    ld = N + 8
    plan = la.gemm_plan(M, N, K, la.F8E4M3 if ka == "f8e4m3" else la.F8E5M2, CODE[out_kind], ldc=ld, b_kmajor=True,
                        b_type=la.F8E4M3 if kb == "f8e4m3" else la.F8E5M2)
    # K blocks of 128 codes when K is a multiple of 128, else of 64
    assert plan.describe()["kernel"] == "fast_f8_128x256x%d" % (128 if K % 128 == 0 else 64), plan.describe()["kernel"]
    Cbuf = torch.full((M, ld), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    C = Cbuf[:, :N]
    C.copy_(c.to(DEV))
    la.gemm_run(plan, a.to(DEV), b.t().contiguous().to(DEV), C, 1.0, 0.5)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf[:, N:].cpu().float()).all(), "a store landed in C's row padding"
    rows = band_rows(M, band=128, wave_rows=64, seed=M + N)
    ref = oracle_gemm(a, b, ka, 1.0, 0.5, c.to(torch.float32), rows=rows, b_kind=kb)
    assert_close(C.cpu()[rows], ref, K, a, b, out_kind, "fast128 f8 %s" % (case,), beta=0.5)


def test_prefill_workload_full():
    """The prefill_384 workload (384 x 11008 x 4096 bf16) in full, planned as the bench plans it."""
    w = synth.WORKLOADS["prefill_384"]
    x = synth.make_inputs(w)
    plan = la.gemm_plan(w.M, w.N, w.K, la.BF16, la.BF16)
    assert plan.describe()["kernel"] == "fast_128x256x64" and plan.describe()["grid"] == 129
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, x["A"].to(DEV), x["B"].to(DEV), C)
    torch.cuda.synchronize()
    ref = oracle_gemm(x["A"], x["B"], "bf16")
    assert_close(C.cpu(), ref, w.K, x["A"], x["B"], "bf16", "prefill_384 workload")
