"""The attention parity bound can fail, and legitimate rounding stays inside it.

On the benchmarked workload (64 entries x 4096 queries x 4096 keys, d = 128,
bf16), on exactly the rows tests/test_gpu_attention.py::test_workload_sampled_rows
checks:

* planted mistakes: the oracle's output with one 64-key tile left out (the
  first, an interior and the last tile), rounded to bf16 as the kernel's output
  would be, must break the per-row bound somewhere;
* a model of the kernel's own arithmetic (FP32 scores and exponentials,
  P rounded to bf16 in numerator and denominator alike, FP32 sums, bf16
  output) must stay inside it everywhere.

CPU only: the oracle and a numpy/torch model, no GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import attention_bound, attention_workload_rows, exact_values

W = synth.ATTN_WORKLOADS["attention"]
TILE = 64


@pytest.fixture(scope="module")
def workload():
    x = synth.make_attn_inputs(W)
    cases = []
    for z, rows in attention_workload_rows(W):
        q = exact_values(x["Q"][z, rows])
        k = exact_values(x["K"][z])
        v = exact_values(x["V"][z])
        ref, tol = attention_bound(q, k, v, W.scale, W.in_kind, W.out_kind)
        cases.append((z, rows, q, k, v, ref, tol))
    return cases


def as_output(o):
    """Round binary64 values to the workload's output type, as the kernel's store would."""
    return torch.from_numpy(np.ascontiguousarray(o)).to(synth.torch_dtype(W.out_kind)).double().numpy()


@pytest.mark.parametrize("tile", [0, 32, TILE - 1])
def test_dropping_one_key_tile_breaks_the_bound(workload, tile):
    broken = 0
    for z, rows, q, k, v, ref, tol in workload:
        keep = np.r_[0:tile * TILE, (tile + 1) * TILE:W.sk]
        bad = as_output(oracle.attention_f64(q, k[keep], v[keep], W.scale))
        broken += int(np.sum(np.abs(bad - ref) > tol))
    assert broken >= 1, "key tile %d left out still passes the bound" % tile


def test_model_of_the_kernel_arithmetic_stays_inside(workload):
    for z, rows, q, k, v, ref, tol in workload:
        qf, kf, vf = (torch.from_numpy(t).float() for t in (q, k, v))
        c = np.float32(W.scale * np.log2(np.e))
        s = qf @ kf.T                                           # FP32 scores
        m = (s * c).max(dim=-1, keepdim=True).values
        p = torch.exp2(s * c - m).to(torch.bfloat16).float()    # P rounded once to the input type
        o = (p @ vf) / p.sum(dim=-1, keepdim=True)             # same rounded weights in both sums
        got = as_output(o.double().numpy())
        err = np.abs(got - ref)
        assert np.all(err <= tol), "entry %d: max err %g, min tol %g" % (z, err.max(), tol.min())
        # the bound is not loose to the point of blindness: well under the output's scale
        assert np.median(tol) < 0.01 * np.abs(v).max()
