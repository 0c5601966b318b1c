"""Pins for the attention oracle (softmax(scale * Q K^T) V, the computation the
Phobos page "Tiles and shared memory" streams over key tiles in section "How
long a tile lives").

Pins from other routes: equal keys give equal weights (the output is the mean
of V's rows); one dominant key selects its V row; one key returns V itself; a
hand-worked two-key case; torch's scaled_dot_product_attention in float64;
shift invariance of the softmax.  Planted mistakes (no max subtraction in a way
that changes the result, a transposed product, a missing normalisation, the
scale applied twice) each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_hand_worked_two_keys():
    # q = (1, 0), keys (1, 0) and (0, 1), scale 1: weights e/(e+1), 1/(e+1)
    o = oracle.attention_f64([[1.0, 0.0]], [[1.0, 0.0], [0.0, 1.0]], [[2.0, 0.0], [0.0, 4.0]], 1.0)
    w0 = math.e / (math.e + 1.0)
    assert abs(o[0, 0] - 2.0 * w0) < 1e-15 and abs(o[0, 1] - 4.0 * (1.0 - w0)) < 1e-15
    assert abs(o[0, 0] - 1.4621171572600098) < 1e-15      # 2e / (e + 1)


def test_equal_keys_average_the_values():
    q = synth.normal((5, 64), 1, "f32").double().numpy()
    k = np.tile(synth.normal((1, 64), 2, "f32").double().numpy(), (37, 1))
    v = synth.normal((37, 64), 3, "f32").double().numpy()
    o = oracle.attention_f64(q, k, v, 0.125)
    assert np.allclose(o, np.tile(v.mean(axis=0), (5, 1)), rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value_row():
    D, Sk = 32, 20
    k = np.zeros((Sk, D))
    k[np.arange(Sk), np.arange(Sk)] = 1.0
    q = np.zeros((Sk, D))
    q[np.arange(Sk), np.arange(Sk)] = 1.0
    v = synth.normal((Sk, D), 4, "f32").double().numpy()
    o = oracle.attention_f64(q, k, v, 200.0)        # weights exp(-200) off the matching key
    assert np.allclose(o, v, rtol=0, atol=1e-80 + 1e-12 * np.abs(v).max())


def test_single_key_returns_v():
    v = synth.normal((1, 64), 5, "f32").double().numpy()
    q = synth.normal((9, 64), 6, "f32").double().numpy()
    k = synth.normal((1, 64), 7, "f32").double().numpy()
    assert np.array_equal(oracle.attention_f64(q, k, v, 0.1), np.tile(v, (9, 1)))


def test_matches_torch_sdpa_in_float64():
    for (b, sq, sk, d, seed) in [(2, 17, 33, 64, 11), (3, 64, 100, 128, 12)]:
        q = synth.normal((b, sq, d), seed, "f32").double()
        k = synth.normal((b, sk, d), seed + 1, "f32").double()
        v = synth.normal((b, sk, d), seed + 2, "f32").double()
        scale = 1.0 / math.sqrt(d)
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale).numpy()
        got = oracle.attention_f64(q.numpy(), k.numpy(), v.numpy(), scale)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_shift_invariance_and_zero_keys():
    q = synth.normal((4, 16), 21, "f32").double().numpy()
    k = synth.normal((8, 16), 22, "f32").double().numpy()
    v = synth.normal((8, 16), 23, "f32").double().numpy()
    # adding the same vector c to every key adds q.c to every score of a row: no change
    c = synth.normal((1, 16), 24, "f32").double().numpy()
    assert np.allclose(oracle.attention_f64(q, k + c, v, 0.5), oracle.attention_f64(q, k, v, 0.5), rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.attention_f64(q, k[:0], v[:0], 0.5)


def _wrong(kind):
    def f(q, k, v, scale):
        q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
        sc = scale * scale if kind == "double-scale" else scale
        s = sc * (np.matmul(k, np.swapaxes(q, -1, -2)).swapaxes(-1, -2) if kind != "transposed" else
                  np.matmul(q, np.swapaxes(k, -1, -2)).swapaxes(-1, -2))
        p = np.exp(s - np.max(s, axis=-1, keepdims=True))
        o = np.matmul(p, v)
        return o if kind == "unnormalised" else o / np.sum(p, axis=-1, keepdims=True)
    return f


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("kind", ["double-scale", "transposed", "unnormalised"])
def test_planted_mistakes_fail(kind, monkeypatch):
    monkeypatch.setattr(oracle, "attention_f64", _wrong(kind))
    pins = [test_hand_worked_two_keys, test_equal_keys_average_the_values, test_dominant_key_selects_its_value_row,
            test_single_key_returns_v, test_matches_torch_sdpa_in_float64]
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1, kind


# ---- the normalised weights (used by the per-row parity bound of the GPU tests) ----

def test_weights_hand_worked_two_keys():
    w = oracle.attention_weights_f64([[1.0, 0.0]], [[1.0, 0.0], [0.0, 1.0]], 1.0)
    e = math.e
    assert abs(w[0, 0] - e / (e + 1.0)) < 1e-15 and abs(w[0, 1] - 1.0 / (e + 1.0)) < 1e-15


def test_weights_equal_keys_are_uniform():
    q = synth.normal((3, 32), 91, "f32").double().numpy()
    k = np.tile(synth.normal((1, 32), 92, "f32").double().numpy(), (25, 1))
    assert np.allclose(oracle.attention_weights_f64(q, k, 0.3), 1.0 / 25, rtol=1e-13, atol=0)


def test_weights_match_torch_softmax_and_give_the_output():
    q = synth.normal((2, 9, 64), 93, "f32").double()
    k = synth.normal((2, 40, 64), 94, "f32").double()
    v = synth.normal((2, 40, 64), 95, "f32").double()
    w = oracle.attention_weights_f64(q.numpy(), k.numpy(), 0.125)
    want = torch.softmax(0.125 * (q @ k.transpose(-1, -2)), dim=-1).numpy()
    assert np.allclose(w, want, rtol=1e-13, atol=1e-16)
    assert np.allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-14) and (w >= 0).all()
    assert np.allclose(w @ v.numpy(), oracle.attention_f64(q.numpy(), k.numpy(), v.numpy(), 0.125), rtol=1e-12,
                       atol=1e-14)
