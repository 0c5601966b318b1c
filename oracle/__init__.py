"""Oracle: plain CPU reference implementations of the tiled GEMM and of the
layout algebra that describes its operand storage.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and never imports it; the two meet only through
the seeded inputs the callers pass to both.

* ``gemm_f64``  -- FP64 triple loop (C, OpenMP over rows), see ``gemm_f64.c``;
  inputs are 16-bit bf16/fp16 patterns, 32-bit binary32 words or 8-bit
  E4M3 / E5M2 codes.
* ``gate_up_swiglu_f64`` -- the gate/up products with the SwiGLU activation.
* ``rms_norm_f64`` -- the row normalisation, numpy in binary64.
* ``gemm_row_reduce_f64`` -- the GEMM with a sum / max / min of every output row.
* ``attention_f64`` -- softmax attention, numpy in binary64.
* ``attention_weights_f64`` -- the normalised softmax weights of the same rows.
* ``layout_ref`` -- the layout algebra written out by enumeration in Python.
"""
import ctypes
import os

import numpy as np

from . import layout_ref  # noqa: F401  (re-exported for the tests)

BF16 = 0
F16 = 1
F32 = 2
F8E4M3 = 3
F8E5M2 = 4
_CODES = {"bf16": BF16, "f16": F16, "f32": F32, "f8e4m3": F8E4M3, "f8e5m2": F8E5M2}
_WIDTH = {"bf16": 2, "f16": 2, "f32": 4, "f8e4m3": 1, "f8e5m2": 1}
_STORE = {1: np.uint8, 2: np.uint16, 4: np.uint32}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    from .build import LIB, build
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, ctypes.c_int, i64, vp, ctypes.c_int, i64,
                                    vp, i64, ctypes.c_double, ctypes.c_double, vp, i64, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [vp, ctypes.c_int, i64, vp]
    lib.oracle_decode.restype = None
    lib.oracle_decode32.argtypes = [vp, i64, vp]
    lib.oracle_decode32.restype = None
    lib.oracle_decode8.argtypes = [vp, ctypes.c_int, i64, vp]
    lib.oracle_decode8.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _type_code(kind: str) -> int:
    if kind not in _CODES:
        raise ValueError("oracle inputs are patterns of kind %s, got %r" % (", ".join(map(repr, _CODES)), kind))
    return _CODES[kind]


def _as_bits(x, kind: str) -> np.ndarray:
    a = np.ascontiguousarray(x)
    want = _STORE[_WIDTH[kind]] if kind in _WIDTH else None
    if want is None:
        _type_code(kind)
    if a.dtype != want:
        raise TypeError("pass raw %s patterns as a %s array, got %s" % (kind, np.dtype(want).name, a.dtype))
    return a


def decode(bits, kind: str) -> np.ndarray:
    """Exact float64 values of 16-bit (bf16, f16), 32-bit (f32) or 8-bit (f8e4m3, f8e5m2) patterns."""
    b = _as_bits(bits, kind)
    out = np.empty(b.shape, dtype=np.float64)
    if kind == "f32":
        _load().oracle_decode32(b.ctypes.data, b.size, out.ctypes.data)
    elif _WIDTH[kind] == 1:
        _load().oracle_decode8(b.ctypes.data, _type_code(kind), b.size, out.ctypes.data)
    else:
        _load().oracle_decode(b.ctypes.data, _type_code(kind), b.size, out.ctypes.data)
    return out


def gemm_f64(a_bits, a_kind, b_bits, b_kind, alpha=1.0, beta=0.0, c=None, nthreads=0):
    """out = alpha * A @ B + beta * C in FP64 (k ascending), from input patterns.

    ``a_bits`` is (M, K), ``b_bits`` is (K, N) (N contiguous): uint16 patterns
    of kind 'bf16' / 'f16', uint32 words of kind 'f32' (both operands then), or
    uint8 codes of kind 'f8e4m3' / 'f8e5m2' (each operand either);
    ``c`` is (M, N) float32 or None (only read when beta != 0).
    Returns an (M, N) float64 array.
    """
    _type_code(a_kind), _type_code(b_kind)
    if _WIDTH[a_kind] != _WIDTH[b_kind]:
        raise ValueError("A and B must have the same element width (16-bit patterns, 'f32' words or 8-bit codes)")
    a = _as_bits(a_bits, a_kind)
    b = _as_bits(b_bits, b_kind)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("shape mismatch: A %s, B %s" % (a.shape, b.shape))
    M, K = a.shape
    N = b.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    cptr, ldc = None, max(N, 1)
    if beta != 0.0:
        if c is None:
            raise ValueError("beta != 0 needs the existing C")
        cc = np.ascontiguousarray(c, dtype=np.float32)
        if cc.shape != (M, N):
            raise ValueError("C shape %s, expected %s" % (cc.shape, (M, N)))
        cptr = cc.ctypes.data
    rc = _load().oracle_gemm_f64(M, N, K, a.ctypes.data, _type_code(a_kind), max(K, 1),
                                 b.ctypes.data, _type_code(b_kind), max(N, 1),
                                 cptr, ldc, float(alpha), float(beta),
                                 out.ctypes.data, max(N, 1), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64 failed (rc=%d)" % rc)
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gate_up_swiglu_f64(x_bits, w_gate_bits, w_up_bits, kind, nthreads=0, w_kind=None):
    """H = silu(X @ W_gate) * (X @ W_up) with silu(g) = g / (1 + exp(-g)), all in binary64.

    The activation composed into the gate/up epilogue (Tylo.jl "Layouts, storage
    and ownership", section "Plans describe work, callers establish readiness":
    scaling and activation become part of the epilogue).  G and U are the
    oracle's own FP64 products; the activation is applied elementwise.
    ``w_kind`` (default ``kind``) is the weights' format when it differs from X's.
    Returns (H, G, U) as float64 arrays.
    """
    wk = w_kind or kind
    g = gemm_f64(x_bits, kind, w_gate_bits, wk, nthreads=nthreads)
    u = gemm_f64(x_bits, kind, w_up_bits, wk, nthreads=nthreads)
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return h, g, u


def rms_norm_f64(x, g, eps):
    """Row normalisation in binary64, the kernel of the Phobos page "Tiles and
    shared memory" (section "A complete kernel"): for every row i,
    ss[i] = sum_j x[i, j]^2, inv[i] = 1 / sqrt(ss[i] / D + eps), and
    y[i, j] = x[i, j] * inv[i] * g[j].

    ``x`` is an (M, D) array of the exact input values, ``g`` the D gains.
    Returns (y, inv) as float64 arrays; with D == 0 there is nothing to
    normalise and inv is NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    if x.ndim != 2 or g.shape[0] != x.shape[1]:
        raise ValueError("x must be (M, D) and g (D,), got %s and %s" % (x.shape, g.shape))
    M, D = x.shape
    if D == 0:
        return np.empty((M, 0)), np.full(M, np.nan)
    ss = np.sum(x * x, axis=1)
    inv = 1.0 / np.sqrt(ss / D + float(eps))
    y = x * inv[:, None] * g[None, :]
    return y, inv


REDUCE_OPS = ("sum", "max", "min")


def gemm_row_reduce_f64(a_bits, a_kind, b_bits, b_kind, op, alpha=1.0, beta=0.0, c=None, nthreads=0):
    """out = alpha * A @ B + beta * C (the FP64 loop above) and, for every row i,
    r[i] = sum, maximum or minimum over j of out[i, j], in binary64.

    Reductions of a finished accumulator along its second axis (Tylo.jl "TMA and
    Hopper WGMMA", section "WGMMA values and ownership": sum, maximum and
    minimum along axis 2 of the finished fragment), taken here over whole
    output rows.  Returns (out, r).
    """
    if op not in REDUCE_OPS:
        raise ValueError("op must be one of %s, got %r" % (REDUCE_OPS, op))
    out = gemm_f64(a_bits, a_kind, b_bits, b_kind, alpha, beta, c, nthreads)
    if out.shape[1] == 0:
        ident = {"sum": 0.0, "max": -np.inf, "min": np.inf}[op]
        return out, np.full(out.shape[0], ident)
    r = {"sum": np.sum, "max": np.max, "min": np.min}[op](out, axis=1)
    return out, r


def attention_f64(q, k, v, scale):
    """Softmax attention in binary64, the computation the Phobos page "Tiles and
    shared memory" streams over key tiles (section "How long a tile lives": a
    query tile, a running maximum and a running sum live through the key loop,
    s = dot_t(q, k), and the accumulator is divided by the sum at the end):

        s[i, j] = scale * sum_d q[i, d] k[j, d]
        p[i, j] = exp(s[i, j] - max_j s[i, j])
        o[i, :] = sum_j p[i, j] v[j, :] / sum_j p[i, j]

    The whole row is formed at once (the exact value the streamed form reaches).
    q: (..., Sq, D), k and v: (..., Sk, D) float64 values; returns o (..., Sq, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[-2] == 0:
        raise ValueError("attention over zero keys is undefined")
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    p = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return np.matmul(p, v) / np.sum(p, axis=-1, keepdims=True)


def attention_weights_f64(q, k, scale):
    """The normalised softmax weights of attention_f64, in binary64:

        w[i, j] = p[i, j] / sum_j p[i, j],   p[i, j] = exp(s[i, j] - max_j s[i, j]),
        s[i, j] = scale * sum_d q[i, d] k[j, d]

    (the weights the Phobos page "Tiles and shared memory" accumulates through
    the key loop, section "How long a tile lives", normalised as the sum at the
    end of that loop does).  attention_f64's output is w @ v.
    q: (..., Sq, D), k: (..., Sk, D); returns w (..., Sq, Sk).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if k.shape[-2] == 0:
        raise ValueError("attention over zero keys is undefined")
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    p = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return p / np.sum(p, axis=-1, keepdims=True)
