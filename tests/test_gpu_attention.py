"""GPU parity of the streaming softmax attention (Phobos page "Tiles and shared
memory", section "How long a tile lives") against the binary64 oracle, through
the C ABI.

The bound is computed row by row from the oracle's own softmax weights
(oracle.tolerance.attention_bound): the rounding of P to the input type and
the FP32 score error move each weight by a relative eta, which moves the
output by at most eta times the weighted spread of the row's values around it;
then the FP32 accumulation and the output's own rounding.  On the benchmarked
length (4096 keys) it is tight enough that dropping any one 64-key tile breaks
it on the rows the workload test checks (tests/test_attention_bound.py).
"""
import math

import numpy as np
import pytest
import torch

import layout_algebra_amd as la
import oracle
import synth
from parity import attention_bound, attention_workload_rows, exact_values, max_abs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def check(got, q, k, v, scale, in_kind, out_kind, what):
    ref, tol = attention_bound(exact_values(q), exact_values(k), exact_values(v), scale, in_kind, out_kind)
    g = got.to(torch.float64).numpy()
    bad = ~(np.abs(g - ref) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d elements out of tolerance; first at %s: gpu=%r oracle=%r tol=%r"
                             % (what, int(bad.sum()), i, g[i], ref[i], tol[i]))


def run(q, k, v, out_kind, scale):
    O = torch.full(q.shape, float("nan"), dtype=synth.torch_dtype(out_kind), device=DEV)
    la.la_attention_run(q.to(DEV), k.to(DEV), v.to(DEV), O, scale)
    torch.cuda.synchronize()
    return O.cpu()


CASES = [
    # (batch, sq, sk, d, in, out, scale)
    (2, 200, 333, 128, "bf16", "bf16", None),     # ragged query tile and key tile
    (3, 128, 64, 64, "f16", "f32", None),         # one tile each
    (1, 1, 1, 128, "bf16", "f32", None),          # one query, one key
    (2, 77, 1000, 64, "bf16", "f16", 0.5),        # many key tiles, larger scale
    (4, 300, 129, 128, "f16", "bf16", None),      # key count one past two tiles
    (1, 50, 70, 64, "bf16", "f32", 0.0),          # zero scale: uniform weights over the valid keys
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:6]) for c in CASES])
def test_attention_shapes(case):
    b, sq, sk, d, ik, ok, scale = case
    print("attention", case, flush=True)
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    seed = 13 * sq + 7 * sk + d
    q = synth.normal((b, sq, d), seed, ik)
    k = synth.normal((b, sk, d), seed + 1, ik)
    v = synth.normal((b, sk, d), seed + 2, ik)
    check(run(q, k, v, ok, scale), q, k, v, scale, ik, ok, str(case))


def test_peaked_softmax_needs_the_running_maximum():
    """Scores in the hundreds: exp would overflow without subtracting the running maximum."""
    q = synth.normal((2, 130, 128), 31, "bf16", 3.0)
    k = synth.normal((2, 500, 128), 32, "bf16", 3.0)
    v = synth.normal((2, 500, 128), 33, "bf16")
    got = run(q, k, v, "f32", 1.0)
    assert torch.isfinite(got).all()
    check(got, q, k, v, 1.0, "bf16", "f32", "peaked")


def test_single_key_returns_v_exactly():
    q = synth.normal((3, 50, 128), 41, "bf16")
    k = synth.normal((3, 1, 128), 42, "bf16")
    v = synth.normal((3, 1, 128), 43, "bf16")
    got = run(q, k, v, "bf16", 0.1)
    assert torch.equal(got, v.expand(3, 50, 128))


def test_equal_keys_average_the_values():
    q = synth.normal((1, 64, 64), 51, "f16")
    k = synth.normal((1, 1, 64), 52, "f16").expand(1, 200, 64).contiguous()
    v = synth.normal((1, 200, 64), 53, "f16")
    got = run(q, k, v, "f32", 0.125).double().numpy()
    mean = v.double().numpy().mean(axis=1, keepdims=True)
    assert np.allclose(got, np.broadcast_to(mean, got.shape), rtol=0, atol=2.0 ** -10 * max_abs(v))


def test_interleaved_heads_layout():
    """Heads interleaved in one [seq, heads, d] tensor: batch stride d, row stride heads * d."""
    H, S, D = 4, 150, 128
    qs = synth.normal((S, H, D), 61, "bf16")
    ks = synth.normal((S, H, D), 62, "bf16")
    vs = synth.normal((S, H, D), 63, "bf16")
    Qd, Kd, Vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    Ob = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    la.la_attention_run(Qd.permute(1, 0, 2), Kd.permute(1, 0, 2), Vd.permute(1, 0, 2), Ob.permute(1, 0, 2))
    torch.cuda.synchronize()
    got = Ob.cpu().permute(1, 0, 2)
    q, k, v = (t.permute(1, 0, 2).contiguous() for t in (qs, ks, vs))
    check(got, q, k, v, 1.0 / math.sqrt(D), "bf16", "bf16", "interleaved heads")


def test_workload_sampled_rows():
    """The benchmarked workload in its launch configuration; the oracle checks sampled queries."""
    w = synth.ATTN_WORKLOADS["attention"]
    x = synth.make_attn_inputs(w)
    O = torch.empty((w.batch, w.sq, w.d), dtype=synth.torch_dtype(w.out_kind), device=DEV)
    la.la_attention_run(x["Q"].to(DEV), x["K"].to(DEV), x["V"].to(DEV), O, w.scale)
    torch.cuda.synchronize()
    got = O.cpu()
    for z, rows in attention_workload_rows(w):
        check(got[z, rows], x["Q"][z, rows], x["K"][z], x["V"][z], w.scale, w.in_kind, w.out_kind, "entry %d" % z)


def test_deterministic():
    q = synth.normal((2, 256, 128), 71, "bf16")
    k = synth.normal((2, 512, 128), 72, "bf16")
    v = synth.normal((2, 512, 128), 73, "bf16")
    assert torch.equal(run(q, k, v, "f32", 0.09), run(q, k, v, "f32", 0.09))


def test_graph_replay():
    """Captured in a HIP graph, attention replays to the eager result each time."""
    q = synth.normal((2, 300, 128), 81, "bf16")
    k = synth.normal((2, 700, 128), 82, "bf16")
    v = synth.normal((2, 700, 128), 83, "bf16")
    Q, K, V = q.to(DEV), k.to(DEV), v.to(DEV)
    O = torch.empty_like(Q)
    la.la_attention_run(Q, K, V, O)
    torch.cuda.synchronize()
    eager = O.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.la_attention_run(Q, K, V, O)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.la_attention_run(Q, K, V, O)
    for it in range(3):
        O.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, eager), "replay %d" % it
