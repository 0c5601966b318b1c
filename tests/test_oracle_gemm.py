"""Pins for the FP64 oracle GEMM (oracle/gemm_f64.c).

The oracle is checked against things it does not compute itself:
  * torch's and numpy's own bf16/fp16 decoding, for all 65,536 patterns,
    numpy's binary32 decoding on every exponent with edge and random fractions,
    and torch's E4M3 / E5M2 decoding for all 256 codes of each;
  * exact rational arithmetic (fractions) on tiny shapes;
  * closed forms: ones x ones = K, identity and permutation B, alpha = 0;
  * numpy's float64 matmul (a library routine) on moderate shapes.
A dropped term, a transposed operand, a wrong stride or a wrong sign in the
epilogue fails at least one of these.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _bits_all():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_decode_bf16_exhaustive():
    b = _bits_all()
    mine = oracle.decode(b, "bf16")
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_decode_f16_exhaustive():
    b = _bits_all()
    mine = oracle.decode(b, "f16")
    ref = b.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def _f32_patterns():
    """Every sign and exponent with the edge fractions (0, 1, 2, all ones, the top bit, one below it)
    and 64 drawn fractions each, plus a million random words."""
    rng = np.random.default_rng(32)
    fr = np.concatenate([np.array([0, 1, 2, 0x7FFFFF, 0x400000, 0x3FFFFF], dtype=np.uint32),
                         rng.integers(0, 1 << 23, 64, dtype=np.uint32)])
    se = np.arange(512, dtype=np.uint32) << 23          # sign and exponent fields
    grid = (se[:, None] | fr[None, :]).ravel()
    return np.concatenate([grid, rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)])


def test_decode_f32_against_numpy():
    b = _f32_patterns()
    mine = oracle.decode(b, "f32")
    with np.errstate(invalid="ignore"):      # signalling NaN patterns
        ref = b.view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    # hand values from the format's definition
    assert oracle.decode(np.array([0x3F800000, 0x00000001, 0x007FFFFF, 0x7F7FFFFF, 0xC0490FDB], dtype=np.uint32),
                         "f32").tolist() == [1.0, 2.0 ** -149, (2.0 ** 23 - 1) * 2.0 ** -149,
                                             (2.0 - 2.0 ** -23) * 2.0 ** 127, -3.1415927410125732]


_E4M3_HAND = [  # code -> value from the format's definition (bias 7, 3 fraction bits, subnormals 2^-9)
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x3C, 1.5),
    (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x77, 240.0), (0x78, 256.0)]
_E5M2_HAND = [  # bias 15, 2 fraction bits, subnormals 2^-16
    (0x00, 0.0), (0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16), (0x04, 2.0 ** -14), (0x3C, 1.0), (0x3E, 1.5),
    (0x40, 2.0), (0x7B, 57344.0), (0xFB, -57344.0), (0x7C, np.inf), (0xFC, -np.inf), (0xBC, -1.0)]


@pytest.mark.parametrize("kind,hand,tdt", [("f8e4m3", _E4M3_HAND, torch.float8_e4m3fn),
                                           ("f8e5m2", _E5M2_HAND, torch.float8_e5m2)])
def test_decode_f8_against_torch_and_hand_values(kind, hand, tdt):
    b = np.arange(256, dtype=np.uint8)
    mine = oracle.decode(b, kind)
    ref = torch.from_numpy(b.copy()).view(tdt).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    codes = np.array([c for c, _ in hand], dtype=np.uint8)
    assert oracle.decode(codes, kind).tolist() == [v for _, v in hand]
    nan_codes = [0x7F, 0xFF] if kind == "f8e4m3" else [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert np.isnan(oracle.decode(np.array(nan_codes, dtype=np.uint8), kind)).all()
    assert int(np.isnan(mine).sum()) == len(nan_codes)


def test_e5m2_is_the_upper_byte_of_binary16():
    """E5M2 shares binary16's sign, exponent field and bias: code c is the binary16 pattern c << 8."""
    c = np.arange(256, dtype=np.uint16)
    a = oracle.decode(c.astype(np.uint8), "f8e5m2")
    h = oracle.decode((c << 8).astype(np.uint16), "f16")
    assert np.array_equal(np.isnan(a), np.isnan(h))
    assert np.array_equal(a[~np.isnan(a)], h[~np.isnan(h)])


def test_mixed_element_widths_are_rejected():
    a = synth.uniform((2, 3), 1, "f32")
    b = synth.uniform((3, 2), 2, "bf16")
    with pytest.raises(ValueError):
        oracle.gemm_f64(synth.bits(a), "f32", synth.bits(b), "bf16")
    with pytest.raises(TypeError):
        oracle.gemm_f64(synth.bits(b.t().contiguous()), "f32", synth.bits(a.t().contiguous()), "f32")
    f8 = synth.uniform((3, 2), 3, "f8e4m3")
    with pytest.raises(ValueError):
        oracle.gemm_f64(synth.bits(synth.uniform((2, 3), 4, "bf16")), "bf16", synth.bits(f8), "f8e4m3")


def test_mixed_byte_formats_match_numpy_float64_matmul():
    """A in E4M3 and B in E5M2 (the two 8-bit formats may differ per operand)."""
    a = synth.normal((33, 70), 11, "f8e4m3", 2.0)
    b = synth.normal((70, 29), 12, "f8e5m2", 0.5)
    got = oracle.gemm_f64(synth.bits(a), "f8e4m3", synth.bits(b), "f8e5m2", -1.5)
    ref = -1.5 * (a.to(torch.float64).numpy() @ b.to(torch.float64).numpy())
    scale = 1.5 * (np.abs(a.to(torch.float64).numpy()) @ np.abs(b.to(torch.float64).numpy()))
    assert np.all(np.abs(got - ref) <= scale * 1e-13)
    # the same values stored as binary32 words give the same result (the decoders agree)
    got32 = oracle.gemm_f64(synth.bits(a.to(torch.float32)), "f32", synth.bits(b.to(torch.float32)), "f32", -1.5)
    assert np.array_equal(got, got32)


def _exact(a_t, b_t, alpha, beta, c):
    """Exact rational alpha*A@B + beta*C from torch's decoding."""
    A = [[Fraction(float(v)) for v in row] for row in a_t.to(torch.float64).tolist()]
    B = [[Fraction(float(v)) for v in row] for row in b_t.to(torch.float64).tolist()]
    M, K, N = len(A), len(B), len(B[0]) if B else 0
    al, be = Fraction(float(alpha)), Fraction(float(beta))
    out, mag = [], []
    for i in range(M):
        row, mrow = [], []
        for j in range(N):
            s = sum((A[i][k] * B[k][j] for k in range(K)), Fraction(0))
            m = sum((abs(A[i][k] * B[k][j]) for k in range(K)), Fraction(0))
            v = al * s
            mm = abs(al) * m
            if beta != 0:
                cv = Fraction(float(c[i, j]))
                v += be * cv
                mm += abs(be * cv)
            row.append(v)
            mrow.append(mm)
        out.append(row)
        mag.append(mrow)
    return out, mag


@pytest.mark.parametrize("kind", ["bf16", "f16", "f32", "f8e4m3", "f8e5m2"])
def test_exact_rational_tiny_shapes(kind):
    seed = 100
    for M in range(1, 5):
        for N in range(1, 5):
            for K in range(1, 5):
                seed += 1
                a = synth.uniform((M, K), seed, kind, -2.0, 2.0)
                b = synth.uniform((K, N), seed + 5000, kind, -2.0, 2.0)
                c = synth.uniform((M, N), seed + 9000, "f32")
                alpha = float(np.float32(1.0 + 0.37 * (seed % 5)))
                beta = float(np.float32(-0.5 + 0.25 * (seed % 3)))
                got = oracle.gemm_f64(synth.bits(a), kind, synth.bits(b), kind, alpha, beta, c.numpy())
                exact, mag = _exact(a, b, alpha, beta, c.numpy())
                for i in range(M):
                    for j in range(N):
                        bound = float(mag[i][j]) * (K + 3) * 2.0 ** -53
                        assert abs(got[i, j] - float(exact[i][j])) <= bound, (M, N, K, i, j)


def test_exact_rational_odd_shapes_with_beta_zero():
    for (M, N, K) in [(3, 7, 5), (7, 3, 9), (1, 9, 17)]:
        a = synth.uniform((M, K), M * 100 + K, "bf16")
        b = synth.uniform((K, N), N * 100 + K, "bf16")
        got = oracle.gemm_f64(synth.bits(a), "bf16", synth.bits(b), "bf16", 1.0, 0.0)
        exact, mag = _exact(a, b, 1.0, 0.0, None)
        for i in range(M):
            for j in range(N):
                assert abs(got[i, j] - float(exact[i][j])) <= float(mag[i][j]) * (K + 3) * 2.0 ** -53


@pytest.mark.parametrize("kind", ["bf16", "f16", "f32", "f8e4m3", "f8e5m2"])
def test_ones_times_ones_is_K(kind):
    for (M, N, K) in [(5, 7, 13), (3, 4, 4096)]:
        a = torch.ones((M, K), dtype=synth.torch_dtype(kind))
        b = torch.ones((K, N), dtype=synth.torch_dtype(kind))
        got = oracle.gemm_f64(synth.bits(a), kind, synth.bits(b), kind)
        assert np.all(got == K)


def test_ones_A_gives_column_sums():
    b = synth.uniform((33, 10), 77, "bf16")
    a = torch.ones((4, 33), dtype=torch.bfloat16)
    got = oracle.gemm_f64(synth.bits(a), "bf16", synth.bits(b), "bf16")
    colsum = b.to(torch.float64).sum(dim=0).numpy()
    np.testing.assert_allclose(got, np.broadcast_to(colsum, got.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["bf16", "f16", "f32", "f8e4m3", "f8e5m2"])
def test_identity_and_permutation_B(kind):
    K, M = 48, 20
    a = synth.uniform((M, K), 5, kind)
    eye = torch.eye(K, dtype=synth.torch_dtype(kind))
    got = oracle.gemm_f64(synth.bits(a), kind, synth.bits(eye), kind)
    assert np.array_equal(got, a.to(torch.float64).numpy())
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(9))
    P = torch.zeros((K, K), dtype=synth.torch_dtype(kind))
    P[perm, torch.arange(K)] = 1          # column j of A@P is column perm[j] of A
    got = oracle.gemm_f64(synth.bits(a), kind, synth.bits(P), kind)
    assert np.array_equal(got, a.to(torch.float64).numpy()[:, perm.numpy()])


def test_alpha_beta_special_cases():
    M, N, K = 9, 11, 13
    a = synth.uniform((M, K), 1, "f16")
    b = synth.uniform((K, N), 2, "f16")
    c = synth.uniform((M, N), 3, "f32").numpy()
    got = oracle.gemm_f64(synth.bits(a), "f16", synth.bits(b), "f16", 0.0, 1.0, c)
    assert np.array_equal(got, c.astype(np.float64))
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    got = oracle.gemm_f64(synth.bits(a), "f16", synth.bits(b), "f16", 1.0, 0.0, nan_c)
    assert np.all(np.isfinite(got))
    # K = 0: the sum is empty
    a0 = torch.zeros((M, 0), dtype=torch.float16)
    b0 = torch.zeros((0, N), dtype=torch.float16)
    got = oracle.gemm_f64(synth.bits(a0), "f16", synth.bits(b0), "f16", 2.0, -0.5, c)
    assert np.array_equal(got, -0.5 * c.astype(np.float64))
    # M = 0 / N = 0 are empty results
    assert oracle.gemm_f64(synth.bits(a[:0]), "f16", synth.bits(b), "f16").shape == (0, N)


@pytest.mark.parametrize("kind", ["bf16", "f16", "f32", "f8e4m3", "f8e5m2"])
def test_matches_numpy_float64_matmul(kind):
    for (M, N, K), seed in [((37, 53, 129), 1), ((64, 80, 257), 2), ((5, 300, 64), 3)]:
        a = synth.normal((M, K), seed, kind)
        b = synth.normal((K, N), seed + 50, kind, 0.5)
        c = synth.uniform((M, N), seed + 99, "f32").numpy()
        got = oracle.gemm_f64(synth.bits(a), kind, synth.bits(b), kind, 1.5, -0.25, c)
        ref = 1.5 * (a.to(torch.float64).numpy() @ b.to(torch.float64).numpy()) - 0.25 * c.astype(np.float64)
        scale = 1.5 * (np.abs(a.to(torch.float64).numpy()) @ np.abs(b.to(torch.float64).numpy())) + 0.25 * np.abs(c)
        assert np.all(np.abs(got - ref) <= scale * 1e-13)


def test_thread_count_does_not_change_bits():
    a = synth.normal((70, 300), 4, "bf16")
    b = synth.normal((300, 90), 5, "bf16")
    r1 = oracle.gemm_f64(synth.bits(a), "bf16", synth.bits(b), "bf16", nthreads=1)
    r4 = oracle.gemm_f64(synth.bits(a), "bf16", synth.bits(b), "bf16", nthreads=4)
    assert np.array_equal(r1, r4)


def test_swiglu_oracle_against_hand_values():
    """X = identity picks rows of the weights, so G and U are the weight values
    themselves and H = w_g / (1 + e^-w_g) * w_u can be written out by hand."""
    import math
    K = N = 8
    x = torch.eye(K, dtype=torch.bfloat16)
    wg_vals = [-20.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0, 20.0]
    wg = torch.tensor([wg_vals] * K, dtype=torch.bfloat16)
    wu = synth.uniform((K, N), 61, "bf16", -3.0, 3.0)
    h, g, u = oracle.gate_up_swiglu_f64(synth.bits(x), synth.bits(wg), synth.bits(wu), "bf16")
    for i in range(K):
        for j in range(N):
            gv = float(wg[i, j]); uv = float(wu[i, j])
            want = gv / (1.0 + math.exp(-gv)) * uv
            assert abs(h[i, j] - want) <= 1e-15 * max(1.0, abs(want))
    assert abs(h[0, 1] / float(wu[0, 1]) - (-0.2689414213699951)) < 1e-15     # silu(-1)
    assert abs(h[0, 5] / float(wu[0, 5]) - 0.7310585786300049) < 1e-15       # silu(1)
    assert h[0, 3] == 0.0                                                     # silu(0)
