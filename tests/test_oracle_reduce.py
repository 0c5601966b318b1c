"""Pins for the row-reduction oracle (the sum / max / min of every output row of
the GEMM; Tylo.jl "TMA and Hopper WGMMA", section "WGMMA values and
ownership").

The pins come from other routes to the same numbers: the row sums equal A times
the row sums of B (plus beta times the row sums of C), which multiplies in the
other order; a permutation B makes the rows of the output permuted rows of A,
whose maximum and minimum are read off A directly; a hand-worked 2 x 2 case;
empty rows give the identity of the operation.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_hand_worked():
    # A = [[1, 2], [3, -4]], B = [[1, 0.5], [-1, 2]] -> out = [[-1, 4.5], [7, -6.5]]
    a = torch.tensor([[1.0, 2.0], [3.0, -4.0]], dtype=torch.bfloat16)
    b = torch.tensor([[1.0, 0.5], [-1.0, 2.0]], dtype=torch.bfloat16)
    for op, want in (("sum", [3.5, 0.5]), ("max", [4.5, 7.0]), ("min", [-1.0, -6.5])):
        _, r = oracle.gemm_row_reduce_f64(synth.bits(a), "bf16", synth.bits(b), "bf16", op)
        assert list(r) == want, (op, r)


def test_row_sums_through_rowsums_of_B():
    M, N, K = 9, 70, 33
    a = synth.uniform((M, K), 31, "f16")
    b = synth.uniform((K, N), 32, "f16")
    c = synth.uniform((M, N), 33, "f32")
    _, r = oracle.gemm_row_reduce_f64(synth.bits(a), "f16", synth.bits(b), "f16", "sum", 1.5, -0.5, c.numpy())
    av = a.double().numpy()
    want = 1.5 * (av @ b.double().numpy().sum(axis=1)) - 0.5 * c.double().numpy().sum(axis=1)
    assert np.allclose(r, want, rtol=1e-12, atol=1e-12)


def test_permutation_B_max_min_are_those_of_A():
    K = 40
    a = synth.normal((7, K), 41, "bf16")
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(42))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[perm, torch.arange(K)] = 1
    av = a.double().numpy()
    for op, f in (("max", np.max), ("min", np.min)):
        _, r = oracle.gemm_row_reduce_f64(synth.bits(a), "bf16", synth.bits(P), "bf16", op)
        assert np.array_equal(r, f(av, axis=1))


def test_empty_rows_give_the_identity():
    a = np.zeros((3, 4), dtype=np.uint16)
    b = np.zeros((4, 0), dtype=np.uint16)
    for op, ident in (("sum", 0.0), ("max", -np.inf), ("min", np.inf)):
        out, r = oracle.gemm_row_reduce_f64(a, "bf16", b, "bf16", op)
        assert out.shape == (3, 0) and np.all(r == ident)
    with pytest.raises(ValueError):
        oracle.gemm_row_reduce_f64(a, "bf16", b, "bf16", "mean")
