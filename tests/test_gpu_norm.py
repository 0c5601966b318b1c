"""GPU parity of the row normalisation (Phobos page "Tiles and shared memory",
section "A complete kernel") against the binary64 oracle, through the C ABI.
"""
import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import exact_values, norm_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_norm(x, g, out_kind, eps, pad_x=0, pad_y=0):
    """x [M, D], g [D] CPU tensors; rows padded by pad_* elements on the GPU (the
    padding is NaN and must stay NaN).  Returns Y on the CPU."""
    M, D = x.shape
    Xb = torch.full((M, D + pad_x), float("nan"), dtype=x.dtype, device=DEV)
    Xb[:, :D] = x.to(DEV)
    Yb = torch.full((M, D + pad_y), float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    la.la_rms_norm_run(Xb[:, :D], g.to(DEV), Yb[:, :D], eps)
    torch.cuda.synchronize()
    Yb = Yb.cpu()
    if pad_y:
        assert torch.isnan(Yb[:, D:].float()).all(), "row padding of Y was written"
    return Yb[:, :D]


def check(got, x, g, eps, out_kind, what):
    y_ref, _ = oracle.rms_norm_f64(exact_values(x), exact_values(g), eps)
    y = got.to(torch.float64).numpy()
    tol = norm_bound(x.shape[1], y_ref, out_kind)
    bad = ~(np.abs(y - y_ref) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d elements out of tolerance; first at %s: gpu=%r oracle=%r tol=%r"
                             % (what, int(bad.sum()), i, y[i], y_ref[i], tol[i]))


# (M, D, in, out, pads): every register-path variant, the streaming path, the
# element-wise path and ragged last chunks and row groups
CASES = [
    (1001, 256, "f32", "f32", (0, 0)),     # the page's rows, four rows per wave, short last group
    (300, 4096, "bf16", "bf16", (0, 0)),   # eight 16-byte chunks per lane
    (257, 1000, "f16", "f32", (0, 0)),     # two chunks, the second one partial
    (33, 8200, "bf16", "bf16", (0, 0)),    # streaming path (two passes), partial last chunk
    (65, 77, "f32", "bf16", (0, 0)),       # rows not 16-byte aligned: element-wise path
    (40, 2048, "f32", "f16", (0, 0)),      # eight chunks of f32
    (9, 4096, "f32", "f32", (0, 0)),       # streaming path for f32
    (100, 512, "bf16", "f32", (16, 8)),    # padded rows (16-byte aligned strides)
    (100, 300, "f16", "f16", (3, 5)),      # padded rows, odd strides: element-wise path
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:4]) for c in CASES])
def test_rms_norm_shapes(case):
    M, D, ik, ok, (px, py) = case
    print("rms_norm", case, flush=True)
    seed = 7 * M + D
    x = synth.normal((M, D), seed, ik)
    g = synth.uniform((D,), seed + 1, ik, 0.5, 1.5)
    got = run_norm(x, g, ok, 1e-6, px, py)
    check(got, x, g, 1e-6, ok, str(case))


@pytest.mark.parametrize("name", ["rms_norm", "rms_norm_bf16"])
def test_rms_norm_workloads_sampled_rows(name):
    """Full-size workloads in the bench's launch configuration; the oracle checks sampled rows."""
    w = synth.NORM_WORKLOADS[name]
    inp = synth.make_norm_inputs(w)
    x, g = inp["X"], inp["G"]
    X = x.to(DEV)
    Y = torch.empty((w.M, w.D), dtype=synth.torch_dtype(w.out_kind), device=DEV)
    la.la_rms_norm_run(X, g.to(DEV), Y, w.eps)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(77)
    rows = sorted(set(torch.randperm(w.M, generator=gen)[:48].tolist()) | {0, w.M - 1})
    check(Y.cpu()[rows], x[rows], g, w.eps, w.out_kind, name)


def test_constant_rows_are_exact():
    """x = +-2^e on a row, g = 1, eps = 0: every step is exact, so y = +-1 bit for bit."""
    D = 1024
    vals = torch.tensor([2.0, -0.25, 64.0, -1.0, 2.0 ** -10], dtype=torch.float32)
    x = vals[:, None].expand(5, D).contiguous()
    g = torch.ones(D)
    got = run_norm(x, g, "f32", 0.0)
    assert torch.equal(got, torch.sign(vals)[:, None].expand(5, D))


def test_in_place_and_zero_rows():
    D = 512
    x = synth.normal((64, D), 91, "bf16")
    x[5] = 0.0
    g = synth.uniform((D,), 92, "bf16", 0.5, 1.5)
    X = x.to(DEV)
    la.la_rms_norm_run(X, g.to(DEV), X, 1e-6)
    torch.cuda.synchronize()
    got = X.cpu()
    check(got, x, g, 1e-6, "bf16", "in place")
    assert torch.all(got[5] == 0)


def test_deterministic_and_empty():
    x = synth.normal((128, 4096), 93, "f32")
    g = synth.uniform((4096,), 94, "f32", 0.5, 1.5)
    a = run_norm(x, g, "f32", 1e-6)
    b = run_norm(x, g, "f32", 1e-6)
    assert torch.equal(a, b)
    e = torch.empty((0, 64), device=DEV)
    la.la_rms_norm_run(e, torch.ones(64, device=DEV), torch.empty((0, 64), device=DEV))
    torch.cuda.synchronize()


def test_graph_replay():
    """Captured in a HIP graph, the normalisation replays to the eager result each time."""
    x = synth.normal((512, 1024), 95, "bf16")
    g = synth.uniform((1024,), 96, "bf16", 0.5, 1.5)
    X, G = x.to(DEV), g.to(DEV)
    Y = torch.empty_like(X)
    la.la_rms_norm_run(X, G, Y, 1e-6)
    torch.cuda.synchronize()
    eager = Y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.la_rms_norm_run(X, G, Y, 1e-6)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.la_rms_norm_run(X, G, Y, 1e-6)
    for it in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), "replay %d" % it
