"""Helpers shared by the GPU parity tests: running the HIP path, running the
oracle on the same 16-bit patterns, and the agreement bound.

Agreement bound (elementwise):
    |gpu - oracle| <= 2^-20 * K * max|A| * max|B|  +  r * |oracle|
with r = 2^-8 for bf16 outputs (the output's own rounding) and 2^-11 for fp16
outputs.  The first term is the FP32 accumulation allowance.  FP32 outputs add
a rounding term (r = 2^-22) only where the result carries beta * C_old
(beta != 0) or K = 0: there the final FP32 rounding of the beta * C_old term
is not part of any accumulation (with K = 1 and beta = 1.25 it exceeds the
first term).  With beta = 0 and K > 0 the final FP32 rounding (at most
2^-24 |out|) must sit well inside the first term, which bound() checks instead
of silently widening the tolerance.

One-byte inputs (E4M3 / E5M2) replace the first term by 2^-14 * K * max|A| * max|B|:
the gfx950 matrix core adds the 64 products of one v_mfma_f32_32x32x64_f8f6f4 with
less than binary32 precision (an in-bounds check of the instruction on the box:
over 5000+ random 32x32x64 blocks of every format pair the error stayed within
8.1e-4 of the block's largest product, i.e. 1.3e-5 * 64 * max|a| * max|b| per
instruction, and a dot product of one 2^12 product and 63 products of 2^-6
returns 4096.875 against 4096.984).  2^-14 = 6.1e-5 per unit of K covers the
worst instruction measured 4.9 times with every instruction's error adding up.
"""
import numpy as np
import torch

import oracle
import synth
from oracle.tolerance import attention_bound  # noqa: F401  (re-exported for the tests)

REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -22}
ACC_EXP = {"bf16": -20, "f16": -20, "f32": -20, "f8e4m3": -14, "f8e5m2": -14}


def max_abs(t):
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        t = t.to(torch.float32)
    return float(t.abs().max()) if t.numel() else 0.0


def kind_of(t):
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32",
            torch.float8_e4m3fn: "f8e4m3", torch.float8_e5m2: "f8e5m2"}[t.dtype]


def bound(K, a, b, ref, out_kind, beta=0.0):
    acc = 2.0 ** ACC_EXP[kind_of(a)] * K * max_abs(a) * max_abs(b)
    if out_kind == "f32":
        if beta != 0.0 or K == 0:
            return acc + REL["f32"] * np.abs(ref)
        peak = float(np.abs(ref).max()) if np.size(ref) else 0.0
        if 2.0 ** -22 * peak > acc:
            raise ValueError("fp32 output: the final rounding (2^-24 of %g) is not covered by the accumulation "
                             "term %g; these inputs need an output rounding term" % (peak, acc))
        return np.full(np.shape(ref), acc)
    return acc + REL[out_kind] * np.abs(ref)


def assert_close(gpu, ref, K, a, b, out_kind, what="", beta=0.0):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    tol = bound(K, a, b, ref, out_kind, beta)
    err = np.abs(g - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance; first at %s: gpu=%r oracle=%r tol=%r"
                             % (what, int(bad.sum()), tuple(i), g[tuple(i)], ref[tuple(i)], tol[tuple(i)]))
    return float(err.max()) if err.size else 0.0, float(tol.min()) if np.size(tol) else 0.0


def oracle_gemm(a_cpu, b_cpu, in_kind, alpha=1.0, beta=0.0, c_cpu=None, rows=None, b_kind=None):
    """Oracle on CPU tensors; `rows` restricts to a subset of output rows; b_kind defaults to in_kind."""
    a = a_cpu if rows is None else a_cpu[rows]
    c = None
    if c_cpu is not None:
        c = (c_cpu if rows is None else c_cpu[rows]).numpy()
    return oracle.gemm_f64(synth.bits(a), in_kind, synth.bits(b_cpu), b_kind or in_kind, alpha, beta, c)


def band_rows(M, band=256, wave_rows=128, extra=1, seed=0):
    """Rows that cover every band of `band` output rows (one row-tile of the full-tile kernels):
    the first and last row of each wave's block of `wave_rows` rows in it, plus `extra` drawn rows
    per band."""
    g = torch.Generator().manual_seed(seed)
    rows = set()
    for b0 in range(0, M, band):
        hi = min(M, b0 + band)
        for w0 in range(b0, hi, wave_rows):
            rows |= {w0, min(hi, w0 + wave_rows) - 1}
        rows |= set((b0 + torch.randint(0, hi - b0, (extra,), generator=g)).tolist())
    return sorted(rows)


def sample_rows(M, n, seed):
    g = torch.Generator().manual_seed(seed)
    pick = torch.randperm(M, generator=g)[:n].tolist()
    return sorted(set(pick) | {0, M - 1})


def swiglu_bound(K, x, w_gate, w_up, g_ref, u_ref, h_ref, out_kind):
    """Agreement bound for silu(G) * U: each accumulator may be off by
    e = 2^-20 K max|X| max|W| (2^-14 for one-byte inputs); |d silu / dg| <= 1.1, so
    |dH| <= 1.1 |U| e + |silu(G)| e, plus the FP32 evaluation of the
    activation (2^-20 |H|) and the output rounding (REL |H|)."""
    e = 2.0 ** ACC_EXP[kind_of(x)]
    e_g = e * K * max_abs(x) * max_abs(w_gate)
    e_u = e * K * max_abs(x) * max_abs(w_up)
    with np.errstate(over="ignore"):
        silu = g_ref / (1.0 + np.exp(-g_ref))
    return 1.1 * np.abs(u_ref) * e_g + np.abs(silu) * e_u + (2.0 ** -20 + REL[out_kind]) * np.abs(h_ref)


def exact_values(t):
    """Exact float64 values of a CPU tensor of f32 / bf16 / f16 elements."""
    if t.dtype == torch.float32:
        return t.double().numpy()
    return oracle.decode(synth.bits(t), "bf16" if t.dtype == torch.bfloat16 else "f16")


def norm_bound(D, y_ref, out_kind):
    """Agreement bound for the row normalisation: the FP32 sum of D squares is off
    by at most (D-1) units of 2^-24 relatively (all terms are non-negative), the
    divide, add, root and reciprocal by one unit each, the half-power of the root
    halves the sum's share, and the two products add two units; 8 units cover the
    fixed steps.  Then the output's own rounding, and for f16 outputs half its
    smallest subnormal."""
    r = np.abs(y_ref)
    absolute = 2.0 ** -25 if out_kind == "f16" else 0.0
    return (D + 8) * 2.0 ** -24 * r + REL[out_kind] * r + absolute


def attention_workload_rows(w):
    """(batch entry, query rows) pairs the workload parity test checks: the first and last entry
    plus up to four drawn ones, each with its first and last query plus up to 24 drawn ones."""
    g = torch.Generator().manual_seed(99)
    out = []
    for z in sorted(set(torch.randint(0, w.batch, (4,), generator=g).tolist()) | {0, w.batch - 1}):
        rows = sorted(set(torch.randint(0, w.sq, (24,), generator=g).tolist()) | {0, w.sq - 1})
        out.append((z, rows))
    return out
