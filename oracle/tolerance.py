"""Agreement bounds between the HIP path and the oracle.

TEST INFRASTRUCTURE ONLY (like the rest of this package): used by the test
suite and by the CPU-baseline leg of bench.py to decide whether a GPU result
matches the oracle's binary64 value.

Softmax attention (the computation the Phobos page "Tiles and shared memory"
streams over key tiles, section "How long a tile lives").  The GPU forms, for
query row i and column e,

    O~[i,e] = sum_j p~[i,j] v[j,e] / sum_j p~[i,j]

with weights p~ that differ from the exact p = exp(s - max s) by a relative
error of at most eta (the rounding of P to the input type, u_in, and the FP32
score error Delta in the exponent: 1 + eta = (1 + u_in) e^Delta) plus, for
fp16 inputs, an absolute error a_in from fp16's subnormal spacing.  Because
the same rounded weights enter numerator and denominator,

    O~ - O = sum_j (p~_j - p_j) (v_j - O) / sum_j p~_j,

so |O~ - O| <= (eta S1 + a_in T) / (1 - eta - sk a_in) with
S1 = sum_j w_j |v_j - O| (w the normalised weights) and T = sum_j |v_j - O|
(the largest p is at least 1 in the kernel's frame, so sum_j p_j >= 1).  The
FP32 accumulation of numerator and denominator adds 2^-20 of the sum of the
terms' magnitudes each (the statistical allowance the GEMM bound uses,
16 units of 2^-24), i.e. at most 2^-19 S2 with S2 = sum_j w_j |v_j|, plus
2^-22 S2 for the final division and rescales; the output's own rounding adds
r_out |O|.  Delta = scale 2^-19 d max|Q| max|K| + 2^-22: the dot product's
accumulation allowance 2^-20 d max|Q| max|K|, the same again for the FP32
fused multiply-add that scales and shifts the exponent argument (at most the
largest score in size), and exp2's own relative error.

Unlike a bound through max|V| alone, this one scales with the spread of each
row's values under its own weights, so dropping one key tile of a long row
moves the output beyond it.
"""
import numpy as np

from . import attention_weights_f64

IN_UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}          # unit roundoff of P's rounding
IN_ABS = {"bf16": 0.0, "f16": 2.0 ** -25}                # half the fp16 subnormal spacing
OUT_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -22}
OUT_ABS = {"bf16": 0.0, "f16": 2.0 ** -25, "f32": 0.0}


def attention_bound(q, k, v, scale, in_kind, out_kind):
    """Oracle output and per-element agreement bound for softmax attention.

    q (..., Sq, D), k and v (..., Sk, D): exact binary64 values of the inputs.
    Returns (o_ref, tol), both (..., Sq, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d, sk = q.shape[-1], k.shape[-2]
    w = attention_weights_f64(q, k, scale)
    o = np.matmul(w, v)
    mq = float(np.abs(q).max()) if q.size else 0.0
    mk = float(np.abs(k).max()) if k.size else 0.0
    delta = abs(float(scale)) * 2.0 ** -19 * d * mq * mk + 2.0 ** -22
    eta = (1.0 + IN_UNIT[in_kind]) * np.exp(delta) - 1.0
    a_in = IN_ABS[in_kind]
    denom = 1.0 - eta - sk * a_in
    if denom <= 0:
        raise ValueError("attention bound undefined: weight error %g too large" % eta)
    lead = o.shape[:-2]
    sq = o.shape[-2]
    wf = w.reshape((-1, sq, sk))
    vf = v.reshape((-1, sk, d))
    of = o.reshape((-1, sq, d))
    chunk = max(1, (1 << 22) // max(1, sk * d))      # rows per pass: at most 2^22 deviations in memory
    s1 = np.empty_like(of)
    t = np.empty_like(of)
    for b in range(of.shape[0]):
        for i0 in range(0, sq, chunk):
            dev = np.abs(vf[b][None, :, :] - of[b, i0:i0 + chunk][:, None, :])     # (rows, sk, d)
            s1[b, i0:i0 + chunk] = np.einsum("rj,rje->re", wf[b, i0:i0 + chunk], dev)
            t[b, i0:i0 + chunk] = dev.sum(axis=1)
    s2 = np.matmul(wf, np.abs(vf))
    tol = (eta * s1 + a_in * t) / denom + (2.0 ** -19 + 2.0 ** -22) * s2 + OUT_REL[out_kind] * np.abs(of) + \
        OUT_ABS[out_kind]
    return o, tol.reshape(lead + (sq, d))
