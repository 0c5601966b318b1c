"""Pins for the row-normalisation oracle (Phobos page "Tiles and shared memory",
section "A complete kernel": sum of squares per row, inverse root of its mean
plus eps, row scaled by it and by the gain vector).

Each pin comes from outside the oracle's own formula: a value worked out by
hand, closed forms (constant rows, unit mean square, scale invariance, a zero
row), and torch's own rms_norm routine in float64.  Planted mistakes (sum for
mean, D-1 for D, a dropped eps, a dropped or transposed gain) each fail at
least one of them; test_planted_mistakes_fail checks that.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_hand_worked_row():
    # x = (3, 4), eps = 0: mean square 12.5, root 3.5355339059327378
    y, inv = oracle.rms_norm_f64([[3.0, 4.0]], [1.0, 1.0], 0.0)
    assert abs(inv[0] - 0.28284271247461906) < 1e-16
    assert abs(y[0, 0] - 0.848528137423857) < 1e-15
    assert abs(y[0, 1] - 1.131370849898476) < 1e-15
    # gains scale the columns: (2, -0.5)
    y, _ = oracle.rms_norm_f64([[3.0, 4.0]], [2.0, -0.5], 0.0)
    assert abs(y[0, 0] - 1.697056274847714) < 1e-15
    assert abs(y[0, 1] + 0.565685424949238) < 1e-15


def test_constant_rows_give_sign_times_gain():
    D = 256
    g = synth.uniform((D,), 7, "f32", 0.5, 1.5).double().numpy()
    x = np.array([[c] * D for c in (2.0, -0.125, 1e-3, 300.0)])
    y, _ = oracle.rms_norm_f64(x, g, 0.0)
    for i, c in enumerate((2.0, -0.125, 1e-3, 300.0)):
        assert np.allclose(y[i], np.sign(c) * g, rtol=1e-15, atol=0)


def test_unit_mean_square_and_scale_invariance():
    x = synth.normal((6, 1000), 11, "f32").double().numpy()
    ones = np.ones(1000)
    y, _ = oracle.rms_norm_f64(x, ones, 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13, atol=0)
    y2, _ = oracle.rms_norm_f64(7.5 * x, ones, 0.0)
    assert np.allclose(y2, y, rtol=1e-14, atol=1e-15)


def test_zero_row_and_eps():
    y, inv = oracle.rms_norm_f64(np.zeros((2, 64)), np.ones(64), 1e-6)
    assert np.all(y == 0.0)
    assert abs(inv[0] - 1000.0) < 1e-9          # 1 / sqrt(1e-6)
    # eps enters under the root: x = (1, 1, 1, 1), eps = 3 -> 1 / sqrt(1 + 3) = 0.5
    y, inv = oracle.rms_norm_f64([[1.0, 1.0, 1.0, 1.0]], np.ones(4), 3.0)
    assert inv[0] == 0.5 and np.all(y == 0.5)


def test_matches_torch_rms_norm_in_float64():
    for (m, d, eps, seed) in [(5, 256, 1e-6, 21), (3, 4096, 1e-5, 22), (7, 77, 0.1, 23)]:
        x = synth.normal((m, d), seed, "f32").double()
        g = synth.uniform((d,), seed + 1, "f32", -2.0, 2.0).double()
        want = torch.nn.functional.rms_norm(x, (d,), weight=g, eps=eps).numpy()
        got, _ = oracle.rms_norm_f64(x.numpy(), g.numpy(), eps)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14)


def test_empty_shapes():
    y, inv = oracle.rms_norm_f64(np.zeros((0, 8)), np.ones(8), 1e-6)
    assert y.shape == (0, 8) and inv.shape == (0,)
    y, inv = oracle.rms_norm_f64(np.zeros((3, 0)), np.ones(0), 1e-6)
    assert y.shape == (3, 0)


def _wrong(kind):
    def f(x, g, eps):
        x = np.asarray(x, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        D = x.shape[1]
        ss = np.sum(x * x, axis=1)
        if kind == "sum":
            inv = 1.0 / np.sqrt(ss + eps)
        elif kind == "d-1":
            inv = 1.0 / np.sqrt(ss / (D - 1) + eps)
        elif kind == "no-eps":
            inv = 1.0 / np.sqrt(ss / D)
        else:
            inv = 1.0 / np.sqrt(ss / D + eps)
        y = x * inv[:, None]
        if kind == "reversed-gain":
            y = y * g[::-1][None, :]
        elif kind != "no-gain":
            y = y * g[None, :]
        return y, inv
    return f


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("kind", ["sum", "d-1", "no-eps", "no-gain", "reversed-gain"])
def test_planted_mistakes_fail(kind, monkeypatch):
    monkeypatch.setattr(oracle, "rms_norm_f64", _wrong(kind))
    pins = [test_hand_worked_row, test_constant_rows_give_sign_times_gain, test_unit_mean_square_and_scale_invariance,
            test_zero_row_and_eps, test_matches_torch_rms_norm_in_float64]
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ZeroDivisionError, FloatingPointError):
            failed += 1
    assert failed >= 1, kind
