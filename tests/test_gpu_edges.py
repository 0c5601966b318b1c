"""GPU parity of the full-tile kernels on edge tiles: M and N ending inside a tile.

The full-tile (direct-load, ping-pong) kernels take any M and N once K is a
multiple of their 32-deep K block and rows start on 16 bytes: an edge tile loads
clamped source rows and columns (every address stays inside the operand; the
values only reach rows and columns of C that are not stored, since C[i, j]
depends on row i of A and column j of B alone) and stores only inside C.
Covered: M and N edges separately and together, one row or column past a tile
boundary, K-major B with N not a multiple of 8 (the last 8-column segment of a
row is stored element by element), A stored [K, M], gate/up and SwiGLU, beta with
C_old inside a padded buffer whose padding must stay untouched, fp32 / bf16 / fp16
outputs, row reductions, a batch with NaN gaps, 4000^3 as planned (sampled rows
covering every tile band), and the LDS image of an edge tile on its valid
positions.  Bounds as in the other GEMM tests.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import assert_close, band_rows, oracle_gemm, swiglu_bound
from test_gpu_reduce import red_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"bf16": la.BF16, "f16": la.F16, "f32": la.F32}


def padded(rows, cols, dtype, fill=float("nan")):
    """A [rows, cols] view into a [rows, ld] buffer with ld = cols rounded up to 8, plus 8 (16-byte rows)."""
    ld = (cols + 7) // 8 * 8 + 8
    buf = torch.full((rows, ld), fill, dtype=dtype, device=DEV)
    return buf, buf[:, :cols]


def run_edge(a, b, out_kind, alpha, beta, c, b_kmajor=False, a_trans=False, large=True):
    M, K = a.shape
    N = b.shape[1]
    in_kind = "bf16" if a.dtype == torch.bfloat16 else "f16"
    Cbuf, C = padded(M, N, synth.torch_dtype(out_kind))
    if c is not None:
        C.copy_(c.to(DEV))
    plan = la.gemm_plan(M, N, K, CODE[in_kind], CODE[out_kind], ldc=Cbuf.shape[1], b_kmajor=b_kmajor,
                        a_transposed=a_trans, large_tiles=large)
    d = plan.describe()
    A = a.t().contiguous().to(DEV) if a_trans else a.to(DEV)
    B = b.t().contiguous().to(DEV) if b_kmajor else b.to(DEV)
    la.gemm_run(plan, A, B, C, alpha, beta)
    torch.cuda.synchronize()
    pad = Cbuf[:, N:].cpu()
    assert torch.isnan(pad.float()).all(), "a store landed in C's row padding"
    return C.cpu(), d


EDGE = [
    # (M, N, K, B stored [N, K], A stored [K, M])
    (300, 520, 96, False, False),    # 44 rows and 8 columns in the last tile row / column
    (513, 256, 64, False, False),    # one row past a tile boundary
    (256, 264, 32, False, False),    # N edge only, one K block
    (700, 300, 160, True, False),    # K-major B, N % 8 = 4: element-wise tail stores
    (300, 299, 64, True, False),     # K-major B, odd N
    (264, 520, 64, False, True),     # A stored [K, M] with an M edge
    (777, 1000, 128, True, False),   # K-major B, both edges, 4 x 4 tiles
]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("in_kind", ["bf16", "f16"])
@pytest.mark.parametrize("case", EDGE, ids=[str(c) for c in EDGE])
def test_full_tile_kernel_edges(case, in_kind, out_kind):
    M, N, K, km, at = case
    print("edges", case, in_kind, out_kind, flush=True)
    seed = 3 * M + 5 * N + K
    a = synth.uniform((M, K), seed, in_kind)
    b = synth.uniform((K, N), seed + 1, in_kind)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got, d = run_edge(a, b, out_kind, 1.25, -0.75, c, b_kmajor=km, a_trans=at)
    assert d["kernel"].startswith("fast"), d["kernel"]
    ref = oracle_gemm(a, b, in_kind, 1.25, -0.75, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "edges %s" % (case,), beta=-0.75)


def test_full_tile_kernel_edges_beta_zero_and_f16_out():
    M, N, K = 300, 520, 96
    a = synth.normal((M, K), 1, "bf16")
    b = synth.normal((K, N), 2, "bf16", 0.5)
    got, d = run_edge(a, b, "f16", 1.0, 0.0, None)
    assert d["kernel"].startswith("fast")
    assert_close(got, oracle_gemm(a, b, "bf16"), K, a, b, "f16", "edges f16")


def test_planned_4000_cube_takes_the_full_tile_kernel():
    """4000^3 as planned (no flag): 16 x 16 tiles of 256 with edges; rows covering every tile band."""
    M = N = K = 4000
    a = synth.normal((M, K), 41, "bf16", 1.0 / 64)
    b = synth.normal((K, N), 42, "bf16", 1.0 / 64)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    d = plan.describe()
    assert d["kernel"].startswith("fast_256x256") and d["grid"] == 256, d["kernel"]
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, a.to(DEV), b.to(DEV), C)
    torch.cuda.synchronize()
    rows = band_rows(M, band=256, wave_rows=128, extra=1, seed=43)
    ref = oracle_gemm(a, b, "bf16", rows=rows)
    assert_close(C.cpu()[rows], ref, K, a, b, "bf16", "4000^3 rows")


@pytest.mark.parametrize("km", [False, True], ids=["kn", "nk"])
def test_gate_up_and_swiglu_edges(km):
    M, N, K = 300, 264 if not km else 261, 64
    x = synth.normal((M, K), 51, "bf16")
    wg = synth.normal((K, N), 52, "bf16", 0.3)
    wu = synth.normal((K, N), 53, "bf16", 0.3)
    Gbuf, G = padded(M, N, torch.bfloat16)
    Ubuf, U = padded(M, N, torch.bfloat16)
    Hbuf, H = padded(M, N, torch.bfloat16)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, ldc=Gbuf.shape[1], gate_up=True, b_kmajor=km, large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast_gate_up"), plan.describe()["kernel"]
    dev_w = (lambda t: t.t().contiguous().to(DEV)) if km else (lambda t: t.to(DEV))
    la.gemm_gate_up_run(plan, x.to(DEV), dev_w(wg), dev_w(wu), G, U)
    la.gemm_gate_up_swiglu_run(plan, x.to(DEV), dev_w(wg), dev_w(wu), H)
    torch.cuda.synchronize()
    for buf in (Gbuf, Ubuf, Hbuf):
        assert torch.isnan(buf[:, N:].float()).all().item(), "a store landed in the row padding"
    g_ref, u_ref = oracle_gemm(x, wg, "bf16"), oracle_gemm(x, wu, "bf16")
    assert_close(G.cpu(), g_ref, K, x, wg, "bf16", "gate edges")
    assert_close(U.cpu(), u_ref, K, x, wu, "bf16", "up edges")
    with np.errstate(over="ignore"):
        h_ref = g_ref / (1.0 + np.exp(-g_ref)) * u_ref
    err = np.abs(H.cpu().double().numpy() - h_ref)
    assert np.all(err <= swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16"))


@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_row_reduce_on_edge_tiles(op):
    M, N, K = 300, 520, 96
    a = synth.uniform((M, K), 61, "bf16")
    b = synth.uniform((K, N), 62, "bf16")
    c = synth.uniform((M, N), 63, "f32")
    Cbuf, C = padded(M, N, torch.float32)
    C.copy_(c.to(DEV))
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, ldc=Cbuf.shape[1], large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast"), plan.describe()["kernel"]
    R = torch.full((M,), 12345.0, dtype=torch.float32, device=DEV)
    la.gemm_run_reduce(plan, a.to(DEV), b.to(DEV), C, 0.5, 1.5, op, R)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf[:, N:]).all().item()
    out, r = oracle.gemm_row_reduce_f64(synth.bits(a), "bf16", synth.bits(b), "bf16", op, 0.5, 1.5, c.numpy())
    assert_close(C.cpu(), out, K, a, b, "f32", "reduce C", beta=1.5)
    err = np.abs(R.cpu().double().numpy() - r)
    assert np.all(err <= red_bound(op, K, a, b, out))


def test_batched_edges():
    batch, M, N, K = 3, 300, 264, 64
    a = synth.normal((batch, M, K), 71, "f16")
    b = synth.normal((batch, K, N), 72, "f16", 0.5)
    sc = M * N + 8 * 5
    Cf = torch.full((batch * sc,), float("nan"), dtype=torch.float32, device=DEV)
    C = Cf.as_strided((batch, M, N), (sc, N, 1))
    plan = la.gemm_plan(M, N, K, la.F16, la.F32, batch=batch, stride_c=sc, large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast"), plan.describe()["kernel"]
    la.gemm_run(plan, a.to(DEV), b.to(DEV), C)
    torch.cuda.synchronize()
    got = C.cpu()
    for z in range(batch):
        assert_close(got[z], oracle_gemm(a[z], b[z], "f16"), K, a[z], b[z], "f32", "batch %d" % z)
    mask = torch.ones(batch * sc, dtype=torch.bool)
    for z in range(batch):
        mask[z * sc:z * sc + M * N] = False
    assert torch.isnan(Cf.cpu()[mask]).all()


@pytest.mark.parametrize("case", [(300, 520, 96, 1, 2, False), (700, 300, 64, 2, 1, True)],
                         ids=["corner_kn", "corner_nk"])
def test_edge_tile_lds_image_on_valid_positions(case):
    """The staged stage of an edge tile equals the planner's map on every position whose element lies
    inside the operand (the others hold clamped source rows or columns, which no stored output reads)."""
    M, N, K, tm, tn, km = case
    a = synth.uniform((M, K), 81, "bf16")
    b = synth.uniform((K, N), 82, "bf16")
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32, ldc=(N + 7) // 8 * 8, b_kmajor=km, large_tiles=True)
    d = plan.describe()
    assert d["kernel"].startswith("fast"), d["kernel"]
    bm, bn, bk = d["tile"]
    img = np.full(d["stage_elems"], 0xDEAD, dtype=np.uint32)
    valid = np.zeros(d["stage_elems"], dtype=bool)
    for operand, (mat, rows, cols, r0, c0) in enumerate([(a, bm, bk, tm * bm, 0), (b, bk, bn, 0, tn * bn)]):
        bits = synth.bits(mat)
        for r in range(rows):
            for c in range(cols):
                o = la.gemm_plan_lds_offset(plan, operand, r, c)
                gr, gc = r0 + r, c0 + c
                if gr < bits.shape[0] and gc < bits.shape[1]:
                    img[o] = bits[gr, gc]
                    valid[o] = True
    nbytes = la.gemm_plan_lds_stage_bytes(plan)
    out = torch.zeros(nbytes // 2, dtype=torch.int16, device=DEV)
    B = b.t().contiguous().to(DEV) if km else b.to(DEV)
    la.gemm_debug_lds_image(plan, a.to(DEV), B, None, tm, tn, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).astype(np.uint32)
    assert valid.sum() > 0 and not valid.all()
    assert np.array_equal(got[valid], img[valid])


K_TAIL = [
    # (M, N, K, B stored [N, K], A stored [K, M]): K % 32 = 8 (one half step) or 24 (a step and a half)
    (300, 520, 264, False, False),
    (300, 520, 280, False, False),
    (512, 512, 1000, False, False),    # whole tiles in M and N, K tail only
    (700, 300, 296, True, False),      # K-major B: contiguous tail loads for both operands
    (264, 520, 280, False, True),      # A stored [K, M]: strided tail loads for both operands
]


@pytest.mark.parametrize("out_kind", ["f32", "bf16"])
@pytest.mark.parametrize("case", K_TAIL, ids=[str(c) for c in K_TAIL])
def test_full_tile_kernel_k_tail(case, out_kind):
    """K ending inside a 32-deep K block: the last K % 32 values are added after the main loop."""
    M, N, K, km, at = case
    print("k tail", case, out_kind, flush=True)
    seed = 11 * M + 3 * N + K
    a = synth.uniform((M, K), seed, "bf16")
    b = synth.uniform((K, N), seed + 1, "bf16")
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    got, d = run_edge(a, b, out_kind, 0.5, 2.0, c, b_kmajor=km, a_trans=at)
    assert d["kernel"].startswith("fast"), d["kernel"]
    ref = oracle_gemm(a, b, "bf16", 0.5, 2.0, c.to(torch.float32))
    assert_close(got, ref, K, a, b, out_kind, "k tail %s" % (case,), beta=2.0)


def test_k_tail_identity_is_exact():
    """With K = 264 the identity's last 8 columns sit in the tail: the product must still equal A."""
    M, K = 512, 264
    a = synth.uniform((M, K), 91, "bf16")
    eye = torch.eye(K, dtype=torch.bfloat16)
    got, d = run_edge(a, eye, "f32", 1.0, 0.0, None)
    assert d["kernel"].startswith("fast"), d["kernel"]
    assert torch.equal(got, a.to(torch.float32))


def test_gate_up_swiglu_k_tail():
    M, N, K = 512, 384, 296
    x = synth.normal((M, K), 95, "bf16")
    wg = synth.normal((K, N), 96, "bf16", 0.3)
    wu = synth.normal((K, N), 97, "bf16", 0.3)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16, gate_up=True, large_tiles=True)
    assert plan.describe()["kernel"].startswith("fast_gate_up"), plan.describe()["kernel"]
    G = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    U = torch.full_like(G, float("nan"))
    H = torch.full_like(G, float("nan"))
    la.gemm_gate_up_run(plan, x.to(DEV), wg.to(DEV), wu.to(DEV), G, U)
    la.gemm_gate_up_swiglu_run(plan, x.to(DEV), wg.to(DEV), wu.to(DEV), H)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle_gemm(x, wg, "bf16"), oracle_gemm(x, wu, "bf16")
    assert_close(G.cpu(), g_ref, K, x, wg, "bf16", "gate k tail")
    assert_close(U.cpu(), u_ref, K, x, wu, "bf16", "up k tail")
    with np.errstate(over="ignore"):
        h_ref = g_ref / (1.0 + np.exp(-g_ref)) * u_ref
    err = np.abs(H.cpu().double().numpy() - h_ref)
    assert np.all(err <= swiglu_bound(K, x, wg, wu, g_ref, u_ref, h_ref, "bf16"))


def test_planned_4000_by_1000_with_k_tail():
    """4000 x 4000 x 1000 as planned: edge tiles in M and N and a K tail of 8; rows covering every band."""
    M = N = 4000
    K = 1000
    a = synth.normal((M, K), 98, "bf16", 1.0 / 32)
    b = synth.normal((K, N), 99, "bf16", 1.0 / 32)
    plan = la.gemm_plan(M, N, K, la.BF16, la.F32)
    assert plan.describe()["kernel"].startswith("fast_256x256"), plan.describe()["kernel"]
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    la.gemm_run(plan, a.to(DEV), b.to(DEV), C)
    torch.cuda.synchronize()
    rows = band_rows(M, band=256, wave_rows=128, extra=1, seed=100)
    ref = oracle_gemm(a, b, "bf16", rows=rows)
    assert_close(C.cpu()[rows], ref, K, a, b, "f32", "4000x4000x1000 rows")


def _random_edge_cases(n, seed):
    """Seeded shapes for the full-tile kernels: M, N anywhere in 1..1100 (M % 8 for A stored [K, M],
    N % 8 for B stored [K, N]), K a multiple of 8 from 32 to 1200 (a multiple of 32 below 256)."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for i in range(n):
        km = bool(torch.randint(0, 2, (1,), generator=g))
        at = (not km) and bool(torch.randint(0, 3, (1,), generator=g) == 0)
        M = int(torch.randint(1, 1101, (1,), generator=g))
        N = int(torch.randint(1, 1101, (1,), generator=g))
        if at:
            M = max(8, M // 8 * 8)
        if not km:
            N = max(8, N // 8 * 8)
        K = int(torch.randint(4, 151, (1,), generator=g)) * 8
        if K < 256:
            K = max(32, K // 32 * 32)
        out.append((M, N, K, km, at))
    return out


RANDOM_EDGE = _random_edge_cases(24, 2027)


@pytest.mark.parametrize("case", RANDOM_EDGE, ids=[str(c) for c in RANDOM_EDGE])
def test_full_tile_kernel_random_shapes(case):
    M, N, K, km, at = case
    print("random edges", case, flush=True)
    seed = 13 * M + 7 * N + K
    a = synth.normal((M, K), seed, "f16")
    b = synth.normal((K, N), seed + 1, "f16", 0.5)
    c = synth.uniform((M, N), seed + 2, "f32")
    got, d = run_edge(a, b, "f32", -0.5, 0.25, c, b_kmajor=km, a_trans=at)
    assert d["kernel"].startswith("fast"), d["kernel"]
    ref = oracle_gemm(a, b, "f16", -0.5, 0.25, c)
    assert_close(got, ref, K, a, b, "f32", "random edges %s" % (case,), beta=0.25)
