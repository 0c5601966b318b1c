"""gemm_run_split_noalloc (the split form on the library's per-GPU workspace array) against
gemm_run_split (the same kernels on a caller workspace): bit-identical outputs, and both within the
GEMM bound of the oracle, on two calls in a row, the second with a smaller input.  Also run in a
fresh process on its own."""
import ctypes

import pytest
import torch

import layout_algebra_amd as la
import synth
from parity import assert_close, oracle_gemm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(M, N, K, km, out_type, out_kind, seed):
    a = synth.normal((M, K), seed, "bf16")
    b = synth.normal((K, N), seed + 1, "bf16", 0.05)
    c = synth.uniform((M, N), seed + 2, "f32").to(synth.torch_dtype(out_kind))
    plan = la.gemm_plan(M, N, K, la.BF16, out_type, b_kmajor=km)
    d = plan.describe()
    assert d["split_k"] > 1, d
    A = a.to(DEV)
    B = b.t().contiguous().to(DEV) if km else b.to(DEV)
    return a, b, c, plan, A, B


@pytest.mark.parametrize("first,second", [
    ((128, 2048, 4096, True, "bf16"), (16, 1024, 2048, True, "bf16")),
    ((64, 4096, 14336, False, "f32"), (1, 4096, 4096, False, "f32")),
    ((512, 4096, 8192, True, "bf16"), (300, 520, 2048, False, "bf16")),   # the 256-wide kernel's split form
], ids=["nk", "kn", "tiles"])
def test_noalloc_matches_split_on_two_calls(first, second):
    lib = la.load()
    vp = ctypes.c_void_p
    for i, (M, N, K, km, out_kind) in enumerate((first, second)):
        print("noalloc call", i, (M, N, K, km, out_kind), flush=True)
        out_type = la.BF16 if out_kind == "bf16" else la.F32
        a, b, c, plan, A, B = _case(M, N, K, km, out_type, out_kind, 900 + 10 * i + M)
        C0 = c.to(DEV)
        want = C0.clone()
        ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
        la.gemm_run_split(plan, A, B, want, 0.5, 1.5, ws)
        got = C0.clone()
        st = lib.gemm_run_split_noalloc(plan.handle, vp(A.data_ptr()), vp(B.data_ptr()), vp(got.data_ptr()),
                                        ctypes.c_float(0.5), ctypes.c_float(1.5),
                                        vp(torch.cuda.current_stream().cuda_stream))
        assert st == 0, la.load().gemm_last_error()
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want.cpu()), "call %d differs from gemm_run_split" % i
        ref = oracle_gemm(a, b, "bf16", 0.5, 1.5, c.to(torch.float32))
        assert_close(got.cpu(), ref, K, a, b, out_kind, "noalloc call %d" % i, beta=1.5)


def test_noalloc_without_split_form_runs_as_gemm_run():
    M, N, K = 16, 28672, 1024
    a = synth.normal((M, K), 951, "bf16")
    b = synth.normal((K, N), 952, "bf16", 0.05)
    plan = la.gemm_plan(M, N, K, la.BF16, la.BF16)
    assert plan.describe()["split_k"] == 1
    A, B = a.to(DEV), b.to(DEV)
    C1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    C2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    la.gemm_run(plan, A, B, C1)
    la.gemm_run_split_noalloc(plan, A, B, C2)
    torch.cuda.synchronize()
    assert torch.equal(C1.cpu(), C2.cpu())


def test_noalloc_under_graph_capture():
    """The call this entry point is for: captured into a HIP graph (torch's capture forbids allocating
    calls on the capturing thread), replayed four times with eager work between the replays, each
    replay equal bit for bit to an eager gemm_run_split of the same inputs."""
    M, N, K = 16, 2048, 4096
    a, b, c, plan, A, B = _case(M, N, K, True, la.BF16, "bf16", 971)
    C0 = c.to(DEV)
    want = C0.clone()
    ws = torch.empty(la.gemm_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    la.gemm_run_split(plan, A, B, want, 1.0, 0.5, ws)
    C = C0.clone()
    la.gemm_run_split_noalloc(plan, A, B, C, 1.0, 0.5)       # first call on this device: address lookup
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), want.cpu())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            la.gemm_run_split_noalloc(plan, A, B, C, 1.0, 0.5, stream=s)
    torch.cuda.synchronize()
    for i in range(4):
        C.copy_(C0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.cpu(), want.cpu()), "replay %d" % i
