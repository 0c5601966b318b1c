"""GPU parity of one-byte inputs (OCP E4M3 / E5M2, A and B each either) against the oracle.

The plans run the K-major full-tile kernel on byte pairs with one 32x32x64
product per K block of 64 codes (A [M, K], B stored [N, K]).  Cases cover every
format pair and output type, whole tiles, M and N ending inside a tile, a K
tail (16 and 48 codes past the last whole block, from K = 512 on), beta != 0
on padded C rows whose padding must stay untouched, batches, the row
reductions, the staged LDS image against the plan's one-byte map, the
4096^3 workload on rows covering every tile band, and the fused gate/up with
its SwiGLU epilogue (X and weights one-byte, the formats mixed).  The agreement bound's
accumulation term is 2^-14 K max|A| max|B| (the matrix core's measured
precision on 64-deep one-byte products; see tests/parity.py).
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, band_rows, oracle_gemm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"f8e4m3": la.F8E4M3, "f8e5m2": la.F8E5M2, "bf16": la.BF16, "f16": la.F16, "f32": la.F32}
PAIRS = [("f8e4m3", "f8e4m3"), ("f8e4m3", "f8e5m2"), ("f8e5m2", "f8e4m3"), ("f8e5m2", "f8e5m2")]


def inputs(M, N, K, ka, kb, seed):
    a = synth.normal((M, K), seed, ka, 1.0)
    b = synth.normal((K, N), seed + 1, kb, 0.5)
    return a, b


def run_f8(a, b, ka, kb, out_kind, alpha=1.0, beta=0.0, c=None, batch_dims=None):
    M, K = a.shape
    N = b.shape[1]
    ld = (N + 7) // 8 * 8 + 8
    Cbuf = torch.full((M, ld), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    C = Cbuf[:, :N]
    if c is not None:
        C.copy_(c.to(DEV))
    plan = la.gemm_plan(M, N, K, CODE[ka], CODE[out_kind], ldc=ld, b_kmajor=True, b_type=CODE[kb])
    d = plan.describe()
    la.gemm_run(plan, a.to(DEV), b.t().contiguous().to(DEV), C, alpha, beta)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf[:, N:].cpu().float()).all(), "a store landed in C's row padding"
    return C.cpu(), d


CASES = [
    # (M, N, K)
    (256, 256, 64),       # one tile, one K block
    (512, 768, 1024),     # whole tiles
    (300, 520, 512),      # M and N edges
    (777, 1000, 1040),    # edges and a K tail of 16 codes
    (513, 264, 1008),     # a K tail of 48 codes (one full 32-code step and a half step)
    (64, 64, 640),        # a single edge tile
]


@pytest.mark.parametrize("ka,kb", PAIRS, ids=["%s-%s" % p for p in PAIRS])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_one_byte_gemm_f32_out_with_beta(case, ka, kb):
    M, N, K = case
    print("f8", case, ka, kb, flush=True)
    a, b = inputs(M, N, K, ka, kb, 3 * M + 5 * N + K)
    c = synth.uniform((M, N), M + N, "f32")
    got, d = run_f8(a, b, ka, kb, "f32", 0.75, -1.25, c)
    assert d["kernel"] == "fast_f8_256x256x64"
    ref = oracle_gemm(a, b, ka, 0.75, -1.25, c, b_kind=kb)
    assert_close(got, ref, K, a, b, "f32", "f8 %s %s %s" % (case, ka, kb), beta=-1.25)


@pytest.mark.parametrize("out_kind", ["bf16", "f16"])
@pytest.mark.parametrize("case", [(512, 768, 1024), (777, 1000, 1040)], ids=["whole", "edges_tail"])
def test_one_byte_gemm_16bit_out(case, out_kind):
    M, N, K = case
    print("f8 out", case, out_kind, flush=True)
    a, b = inputs(M, N, K, "f8e4m3", "f8e4m3", 11 * M + N)
    a = (a.to(torch.float32) / 8).to(torch.float8_e4m3fn)     # keep f16 outputs far from overflow
    got, _ = run_f8(a, b, "f8e4m3", "f8e4m3", out_kind)
    ref = oracle_gemm(a, b, "f8e4m3")
    assert_close(got, ref, K, a, b, out_kind, "f8 out %s %s" % (case, out_kind))


def test_one_byte_exact_small_integers():
    """Integers below 16 are exact in both formats and every partial sum below 2^11 is exact in
    any accumulation of at least 12 bits: the products must come back bit for bit."""
    M, N, K = 300, 260, 1040
    g = torch.Generator().manual_seed(5)
    a = torch.randint(-3, 4, (M, K), generator=g).to(torch.float32).to(torch.float8_e4m3fn)
    b = torch.randint(-3, 4, (K, N), generator=g).to(torch.float32).to(torch.float8_e5m2)
    got, _ = run_f8(a, b, "f8e4m3", "f8e5m2", "f32")
    ref = oracle_gemm(a, b, "f8e4m3", b_kind="f8e5m2")
    assert np.abs(ref).max() < 2 ** 11
    assert np.array_equal(got.double().numpy(), ref)


def test_one_byte_batched_and_reduced():
    M, N, K, batch = 300, 264, 576, 3
    print("f8 batch", flush=True)
    a = synth.normal((batch, M, K), 21, "f8e4m3")
    b = synth.normal((batch, K, N), 22, "f8e5m2", 0.5)
    plan = la.gemm_plan(M, N, K, la.F8E4M3, la.F32, b_kmajor=True, b_type=la.F8E5M2, batch=batch)
    C = torch.empty((batch, M, N), dtype=torch.float32, device=DEV)
    R = torch.empty((batch, M), dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, a.to(DEV), b.transpose(1, 2).contiguous().to(DEV), C, op="max", R=R)
    torch.cuda.synchronize()
    for z in range(batch):
        ref = oracle_gemm(a[z], b[z], "f8e4m3", b_kind="f8e5m2")
        assert_close(C[z].cpu(), ref, K, a[z], b[z], "f32", "f8 batch %d" % z)
        # the row maxima are maxima of the FP32 outputs the kernel stored
        assert torch.equal(R[z].cpu(), C[z].cpu().max(dim=1).values)


def test_one_byte_lds_image_matches_the_plan():
    """K block 0 of tile (1, 2) staged by the kernel's own copy code: byte lds_offset(A, r, k) holds
    A[256 + r, k] and byte lds_offset(B, k, n) holds B[k, 512 + n] (edge rows and columns clamped)."""
    M, N, K = 600, 700, 512
    a, b = inputs(M, N, K, "f8e4m3", "f8e5m2", 7)
    plan = la.gemm_plan(M, N, K, la.F8E4M3, la.F32, b_kmajor=True, b_type=la.F8E5M2, ldc=704)
    nbytes = la.gemm_plan_lds_stage_bytes(plan)
    out = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    la.gemm_debug_lds_image(plan, a.to(DEV), b.t().contiguous().to(DEV), None, 1, 2, out)
    torch.cuda.synchronize()
    img = out.cpu().numpy()
    ab, bb = synth.bits(a), synth.bits(b)
    for r in range(256):
        row = min(256 + r, M - 1)
        for k in range(64):
            assert img[la.gemm_plan_lds_offset(plan, 0, r, k)] == ab[row, k], (r, k)
    for n in range(0, 256, 3):
        col = min(512 + n, N - 1)
        for k in range(64):
            assert img[la.gemm_plan_lds_offset(plan, 1, k, n)] == bb[k, col], (k, n)


def test_square4096_f8_workload_rows():
    w = synth.WORKLOADS["square4096_f8"]
    x = synth.make_inputs(w)
    print("f8 4096", flush=True)
    plan = la.gemm_plan(w.M, w.N, w.K, la.F8E4M3, la.BF16, b_kmajor=True)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, x["A"].to(DEV), x["B"].t().contiguous().to(DEV), C)
    torch.cuda.synchronize()
    rows = band_rows(w.M, band=256, wave_rows=128, extra=1, seed=44)
    ref = oracle_gemm(x["A"], x["B"], w.in_kind, rows=rows)
    assert_close(C.cpu()[rows], ref, w.K, x["A"], x["B"], "bf16", "square4096_f8 rows")


GU_CASES = [
    # (M, N, K, x format, weight format)
    (512, 1024, 1024, "f8e4m3", "f8e4m3"),     # whole tiles
    (300, 520, 1040, "f8e4m3", "f8e5m2"),      # M and N edges, a K tail of 16 codes
    (777, 261, 512, "f8e5m2", "f8e4m3"),       # odd N (weights are K-major: any N)
]


@pytest.mark.parametrize("case", GU_CASES, ids=[str(c) for c in GU_CASES])
def test_one_byte_gate_up_and_swiglu(case):
    """Fused gate/up on one-byte X and weights (both K-contiguous): G, U and silu(G) * U, bf16 out,
    in padded rows whose padding must stay untouched."""
    from parity import swiglu_bound
    M, N, K, kx, kw = case
    print("f8 gate/up", case, flush=True)
    x = synth.normal((M, K), 61 + M, kx, 1.0)
    wg = synth.normal((K, N), 62 + N, kw, 0.25)
    wu = synth.normal((K, N), 63 + K, kw, 0.25)
    ld = (N + 7) // 8 * 8 + 8
    bufs = [torch.full((M, ld), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    G, U, H = (b[:, :N] for b in bufs)
    plan = la.gemm_plan(M, N, K, CODE[kx], la.BF16, ldc=ld, gate_up=True, b_kmajor=True, b_type=CODE[kw])
    assert plan.describe()["kernel"] == "fast_gate_up_f8_256x128x64", plan.describe()["kernel"]
    X, Wg, Wu = x.to(DEV), wg.t().contiguous().to(DEV), wu.t().contiguous().to(DEV)
    la.gemm_gate_up_run(plan, X, Wg, Wu, G, U)
    la.gemm_gate_up_swiglu_run(plan, X, Wg, Wu, H)
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.isnan(b[:, N:].float().cpu()).all(), "a store landed in the row padding"
    h_ref, g_ref, u_ref = oracle.gate_up_swiglu_f64(synth.bits(x), synth.bits(wg), synth.bits(wu), kx, w_kind=kw)
    assert_close(G.cpu(), g_ref, K, x, wg, "bf16", "f8 gate %s" % (case,))
    assert_close(U.cpu(), u_ref, K, x, wu, "bf16", "f8 up %s" % (case,))
    err = np.abs(H.cpu().double().numpy() - h_ref)
    assert np.all(err <= swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16")), float(err.max())


def test_one_byte_k_zero_and_broadcast_batch():
    """K = 0 reads neither operand (C = beta * C); a batch with B broadcast (stride 0)."""
    M, N = 300, 264
    c = synth.uniform((M, N), 77, "f32")
    plan = la.gemm_plan(M, N, 0, la.F8E4M3, la.F32, b_kmajor=True, lda=16, ldb=16)
    C = c.clone().to(DEV)
    dummy = torch.zeros((M, 0), dtype=torch.float8_e4m3fn, device=DEV)
    la.gemm_run(plan, dummy, torch.zeros((N, 0), dtype=torch.float8_e4m3fn, device=DEV), C, 2.0, -0.5)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), (-0.5 * c.double()).float())
    K, batch = 1024, 3
    a = synth.normal((batch, M, K), 78, "f8e4m3")
    b = synth.normal((K, N), 79, "f8e4m3", 0.5)
    plan = la.gemm_plan(M, N, K, la.F8E4M3, la.BF16, b_kmajor=True, batch=batch, stride_b=0)
    Cb = torch.empty((batch, M, N), dtype=torch.bfloat16, device=DEV)
    Bt = b.t().contiguous().to(DEV)
    la.gemm_run(plan, a.to(DEV), Bt.expand(batch, N, K), Cb)
    torch.cuda.synchronize()
    for z in range(batch):
        ref = oracle_gemm(a[z], b, "f8e4m3")
        assert_close(Cb[z].cpu(), ref, K, a[z], b, "bf16", "f8 broadcast %d" % z)


def test_one_byte_gate_up_lds_image():
    """Stage 0 of a gate/up tile: byte lds_offset(W_up, k, n) holds W_up[k, 128 + n] of tile column 1."""
    M, N, K = 300, 300, 512
    x = synth.normal((M, K), 81, "f8e4m3")
    wg = synth.normal((K, N), 82, "f8e4m3")
    wu = synth.normal((K, N), 83, "f8e4m3")
    plan = la.gemm_plan(M, N, K, la.F8E4M3, la.BF16, gate_up=True, b_kmajor=True, ldc=304)
    out = torch.zeros(la.gemm_plan_lds_stage_bytes(plan), dtype=torch.uint8, device=DEV)
    la.gemm_debug_lds_image(plan, x.to(DEV), wg.t().contiguous().to(DEV), wu.t().contiguous().to(DEV), 1, 1, out)
    torch.cuda.synchronize()
    img = out.cpu().numpy()
    xb, gb, ub = synth.bits(x), synth.bits(wg), synth.bits(wu)
    for r in range(0, 256, 5):
        for k in range(64):
            assert img[la.gemm_plan_lds_offset(plan, 0, r, k)] == xb[min(256 + r, M - 1), k]
    for n in range(128):
        col = min(128 + n, N - 1)
        for k in range(64):
            assert img[la.gemm_plan_lds_offset(plan, 1, k, n)] == gb[k, col]
            assert img[la.gemm_plan_lds_offset(plan, 2, k, n)] == ub[k, col]


def _random_f8_cases(n, seed):
    """Seeded one-byte shapes: M, N in 1..1100, K a multiple of 64 from 64 to 1024 or of 16 from
    512 to 1600, formats, output type and beta drawn."""
    g = torch.Generator().manual_seed(seed)
    draw = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    out = []
    for _ in range(n):
        M, N = draw(1, 1100), draw(1, 1100)
        K = draw(1, 16) * 64 if draw(0, 1) else draw(32, 100) * 16
        ka, kb = PAIRS[draw(0, 3)]
        out.append((M, N, K, ka, kb, ["f32", "bf16", "f16"][draw(0, 2)], [0.0, 0.5][draw(0, 1)]))
    return out


RANDOM_F8 = _random_f8_cases(16, 808)


@pytest.mark.parametrize("case", RANDOM_F8, ids=[str(c) for c in RANDOM_F8])
def test_one_byte_random_shapes(case):
    M, N, K, ka, kb, out_kind, beta = case
    print("f8 random", case, flush=True)
    a, b = inputs(M, N, K, ka, kb, 5 * M + 3 * N + K)
    a = (a.to(torch.float32) / 4).to(synth.torch_dtype(ka))          # f16 outputs stay far from overflow
    c = synth.uniform((M, N), M * N, "f32").to(synth.torch_dtype(out_kind)) if beta else None
    got, d = run_f8(a, b, ka, kb, out_kind, 1.0, beta, c)
    assert d["kernel"] == "fast_f8_256x256x64"
    ref = oracle_gemm(a, b, ka, 1.0, beta, c.to(torch.float32) if c is not None else None, b_kind=kb)
    assert_close(got, ref, K, a, b, out_kind, "f8 random %s" % (case,), beta=beta)


SKINNY_F8 = [
    # (M, N, K, A format, B format)
    (16, 64, 512, "f8e4m3", "f8e4m3"),
    (1, 384, 1024, "f8e4m3", "f8e5m2"),
    (7, 1024, 2048, "f8e5m2", "f8e4m3"),
    (13, 192, 8192, "f8e5m2", "f8e5m2"),
    (20, 128, 512, "f8e4m3", "f8e4m3"),     # 32 rows of A
    (40, 8192, 1024, "f8e4m3", "f8e5m2"),   # 64 rows of A (from 33 rows on: 128 strips or more)
    (64, 8192, 256, "f8e5m2", "f8e4m3"),
    (100, 16384, 512, "f8e4m3", "f8e4m3"),  # 128 rows of A
]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("case", SKINNY_F8, ids=[str(c) for c in SKINNY_F8])
def test_one_byte_skinny(case, out_kind):
    """M <= 128 with one-byte A and B stored [N, K]: the K-major skinny kernel on byte pairs, one
    16x16x128 product per two 32-unit steps."""
    M, N, K, ka, kb = case
    print("f8 skinny", case, out_kind, flush=True)
    a, b = inputs(M, N, K, ka, kb, 17 * M + N + K)
    c = synth.uniform((M, N), M + 2 * N, "f32").to(synth.torch_dtype(out_kind))
    got, d = run_f8(a, b, ka, kb, out_kind, 1.25, -0.5, c)
    assert d["kernel"].startswith(("skinny_f8_%dx64x" % (16 if M <= 16 else 32 if M <= 32 else 64)) if M <= 64
                                  else "skinny_f8_128x128x"), d["kernel"]
    ref = oracle_gemm(a, b, ka, 1.25, -0.5, c.to(torch.float32), b_kind=kb)
    assert_close(got, ref, K, a, b, out_kind, "f8 skinny %s" % (case,), beta=-0.5)


def test_one_byte_skinny_workload_and_lds_image():
    w = synth.WORKLOADS["skinny_f8"]
    x = synth.make_inputs(w)
    print("f8 skinny workload", flush=True)
    plan = la.gemm_plan(w.M, w.N, w.K, la.F8E4M3, la.F32, b_kmajor=True)
    assert plan.describe()["kernel"] == "skinny_f8_16x64x512"
    A, Bt = x["A"].to(DEV), x["B"].t().contiguous().to(DEV)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    la.gemm_run(plan, A, Bt, C)
    torch.cuda.synchronize()
    ref = oracle_gemm(x["A"], x["B"], "f8e4m3")
    assert_close(C.cpu(), ref, w.K, x["A"], x["B"], "f32", "skinny_f8 workload")
    # stage 0 of column strip 5: byte lds_offset(B, k, n) holds B[k, 320 + n], A's rows likewise
    out = torch.zeros(la.gemm_plan_lds_stage_bytes(plan), dtype=torch.uint8, device=DEV)
    la.gemm_debug_lds_image(plan, A, Bt, None, 0, 5, out)
    torch.cuda.synchronize()
    img, ab, bb = out.cpu().numpy(), synth.bits(x["A"]), synth.bits(x["B"])
    for r in range(16):
        for k in range(0, 512, 7):
            assert img[la.gemm_plan_lds_offset(plan, 0, r, k)] == ab[r, k]
    for n in range(0, 64, 3):
        for k in range(512):
            assert img[la.gemm_plan_lds_offset(plan, 1, k, n)] == bb[k, 320 + n]
