"""ctypes marshalling for liblagemm.so (see include/la_gemm.h for contracts)."""
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liblagemm.so")

BF16, F16, F32, F8E4M3, F8E5M2 = 0, 1, 2, 3, 4
FLAG_GATE_UP = 0x1
FLAG_B_KMAJOR = 0x2
FLAG_LARGE_TILES = 0x4
FLAG_A_TRANSPOSED = 0x8

EXPORTED_SYMBOLS = (
    "gemm_plan", "gemm_plan_destroy", "gemm_run", "gemm_plan_workspace_bytes", "gemm_run_split", "gemm_run_split_noalloc", "gemm_run_reduce", "gemm_gate_up_run", "gemm_gate_up_swiglu_run", "gemm_plan_describe",
    "la_rms_norm_run", "la_attention_run", "la_probe_mfma", "gemm_plan_lds_offset", "gemm_debug_lds_image", "gemm_plan_lds_stage_bytes",
    "la_layout_eval", "la_layout_eval_index", "la_swizzle_apply", "la_tile_plan_offset",
    "la_layout_eval_str", "la_layout_tile_str", "la_layout_coalesce_str", "la_layout_permute_str",
    "la_layout_cosize_str", "la_view_window_eval",
    "gemm_status_string", "gemm_last_error",
)

STATUS = {0: "GEMM_OK", 1: "GEMM_ERR_NULL", 2: "GEMM_ERR_INVALID_ARG", 3: "GEMM_ERR_UNSUPPORTED",
          4: "GEMM_ERR_ALIGNMENT", 5: "GEMM_ERR_RESOURCE", 6: "GEMM_ERR_HIP"}


class GemmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status
        self.name = STATUS.get(status, str(status))


class _AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("sq", ctypes.c_int64), ("sk", ctypes.c_int64), ("d", ctypes.c_int64),
                ("in_type", ctypes.c_int32), ("out_type", ctypes.c_int32),
                ("ld_q", ctypes.c_int64), ("ld_k", ctypes.c_int64), ("ld_v", ctypes.c_int64), ("ld_o", ctypes.c_int64),
                ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64), ("stride_v", ctypes.c_int64),
                ("stride_o", ctypes.c_int64), ("scale", ctypes.c_float)]


class _Desc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32), ("c_type", ctypes.c_int32),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("batch", ctypes.c_int64),
                ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64), ("stride_c", ctypes.c_int64)]


_lib = None


def lib_path():
    return _LIB_PATH


def load():
    """Load liblagemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("liblagemm.so is not built (run __graft_entry__.build() or "
                           "python layout_algebra_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    p64 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "gemm_plan": ([ctypes.POINTER(_Desc), ctypes.POINTER(vp)], i32),
        "gemm_plan_destroy": ([vp], None),
        "gemm_run": ([vp, vp, vp, vp, f32, f32, vp], i32),
        "gemm_run_reduce": ([vp, vp, vp, vp, f32, f32, i32, vp, vp], i32),
        "gemm_plan_workspace_bytes": ([vp, p64], i32),
        "gemm_run_split": ([vp, vp, vp, vp, f32, f32, vp, i64, vp], i32),
        "gemm_run_split_noalloc": ([vp, vp, vp, vp, f32, f32, vp], i32),
        "gemm_gate_up_run": ([vp, vp, vp, vp, vp, vp, vp], i32),
        "gemm_gate_up_swiglu_run": ([vp, vp, vp, vp, vp, vp], i32),
        "la_rms_norm_run": ([i64, i64, i32, i32, vp, i64, vp, vp, i64, f32, vp], i32),
        "la_attention_run": ([ctypes.POINTER(_AttnDesc), vp, vp, vp, vp, vp], i32),
        "la_probe_mfma": ([vp, i64, vp, i64, i64, i32, vp], i32),
        "gemm_plan_describe": ([vp, ctypes.c_char_p, ctypes.c_size_t], i32),
        "gemm_plan_lds_offset": ([vp, i32, i64, i64, p64], i32),
        "gemm_plan_lds_stage_bytes": ([vp, p64], i32),
        "gemm_debug_lds_image": ([vp, vp, vp, vp, i64, i64, vp, vp], i32),
        "la_layout_eval": ([p64, p64, i32, p64, p64], i32),
        "la_layout_eval_index": ([p64, p64, i32, i64, p64], i32),
        "la_swizzle_apply": ([i32, i32, i32, i64, p64], i32),
        "la_tile_plan_offset": ([i32, i64, i64, i32, i32, i64, i64, p64, p64], i32),
        "la_layout_eval_str": ([ctypes.c_char_p, ctypes.c_char_p, p64], i32),
        "la_layout_tile_str": ([ctypes.c_char_p, p64, i32, ctypes.c_char_p, ctypes.c_size_t], i32),
        "la_layout_coalesce_str": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_size_t], i32),
        "la_layout_permute_str": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_size_t], i32),
        "la_layout_cosize_str": ([ctypes.c_char_p, p64], i32),
        "la_view_window_eval": ([i32, i32, i32, ctypes.c_char_p, p64, p64, i32, p64, p64], i32),
        "gemm_status_string": ([i32], ctypes.c_char_p),
        "gemm_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise GemmError(rc, load().gemm_last_error().decode())


def _i64s(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


# ------------------------------------------------------------------ plans
class Plan:
    """Owns a gemm_plan_t.  Immutable; reusable for any number of runs."""

    def __init__(self, handle, desc):
        self._h = ctypes.c_void_p(handle)
        self.desc = desc

    @property
    def handle(self):
        return self._h

    def describe(self):
        return gemm_plan_describe(self)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.gemm_plan_destroy(h)
            self._h = ctypes.c_void_p(0)


def gemm_plan(m, n, k, in_type=BF16, c_type=F32, lda=None, ldb=None, ldc=None, gate_up=False, b_kmajor=False,
              batch=1, stride_a=None, stride_b=None, stride_c=None, large_tiles=False, a_transposed=False, b_type=None):
    """Plan C[m,n] = A @ B.  A is an [m,k] tensor, or with a_transposed=True a [k,m] tensor (A transposed);
    B is a [k,n] tensor, or with b_kmajor=True a [n,k] tensor (B transposed).
    in_type is A's element type and B's unless b_type is given (the two one-byte formats may differ).
    batch > 1: tensors gain a leading batch dimension with the given element strides (default: packed).
    large_tiles=True keeps the largest tile the shape allows (GEMM_FLAG_LARGE_TILES)."""
    lda = int(lda if lda is not None else max(1, m if a_transposed else k))
    ldb = int(ldb if ldb is not None else max(1, k if b_kmajor else n))
    ldc = int(ldc if ldc is not None else max(1, n))
    d = _Desc(int(m), int(n), int(k), int(in_type), int(in_type if b_type is None else b_type), int(c_type), lda, ldb, ldc,
              (FLAG_GATE_UP if gate_up else 0) | (FLAG_B_KMAJOR if b_kmajor else 0) |
              (FLAG_LARGE_TILES if large_tiles else 0) | (FLAG_A_TRANSPOSED if a_transposed else 0), int(batch),
              int(stride_a if stride_a is not None else (k if a_transposed else m) * lda),
              int(stride_b if stride_b is not None else (n if b_kmajor else k) * ldb),
              int(stride_c if stride_c is not None else m * ldc))
    h = ctypes.c_void_p()
    _check(load().gemm_plan(ctypes.byref(d), ctypes.byref(h)))
    return Plan(h.value, d)


def gemm_plan_describe(plan):
    buf = ctypes.create_string_buffer(16384)
    _check(load().gemm_plan_describe(plan.handle, buf, len(buf)))
    return json.loads(buf.value.decode())


def gemm_plan_lds_offset(plan, operand, row, col):
    out = ctypes.c_int64()
    _check(load().gemm_plan_lds_offset(plan.handle, int(operand), int(row), int(col), ctypes.byref(out)))
    return out.value


def gemm_plan_lds_stage_bytes(plan):
    out = ctypes.c_int64()
    _check(load().gemm_plan_lds_stage_bytes(plan.handle, ctypes.byref(out)))
    return out.value


# ------------------------------------------------------------------ runs (torch tensors)
_KIND = {}


def _torch():
    import torch
    if not _KIND:
        _KIND.update({torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32,
                      torch.float8_e4m3fn: F8E4M3, torch.float8_e5m2: F8E5M2})
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_matrix(t, name, rows, cols, ld, kind, batch=1, bstride=0):
    """2-D [rows, cols] tensor, or for batch > 1 a 3-D [batch, rows, cols] tensor with batch stride bstride."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a tensor on the GPU" % name)
    if _KIND.get(t.dtype) != kind:
        raise ValueError("%s has dtype %s, plan expects type code %d" % (name, t.dtype, kind))
    want = (rows, cols) if batch == 1 else (batch, rows, cols)
    if tuple(t.shape) != want:
        raise ValueError("%s must have shape %s, got %s" % (name, want, tuple(t.shape)))
    if rows > 0 and cols > 0:
        if t.stride(-1) != 1 or (rows > 1 and t.stride(-2) != ld):
            raise ValueError("%s must be row-major with leading dimension %d (strides %s)" % (name, ld, t.stride()))
        if batch > 1 and t.stride(0) != bstride:
            raise ValueError("%s must have batch stride %d (strides %s)" % (name, bstride, t.stride()))


def _check_a(t, name, d):
    if d.flags & FLAG_A_TRANSPOSED:
        _check_matrix(t, name + " ([k,m], A transposed)", d.k, d.m, d.lda, d.a_type, d.batch, d.stride_a)
    else:
        _check_matrix(t, name, d.m, d.k, d.lda, d.a_type, d.batch, d.stride_a)


def _check_b(t, name, d):
    if d.flags & FLAG_B_KMAJOR:
        _check_matrix(t, name + " ([n,k], K-major)", d.n, d.k, d.ldb, d.b_type, d.batch, d.stride_b)
    else:
        _check_matrix(t, name, d.k, d.n, d.ldb, d.b_type, d.batch, d.stride_b)


def gemm_run(plan, A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C = alpha * A @ B + beta * C, enqueued on `stream` (default: current)."""
    d = plan.desc
    _check_a(A, "A", d)
    _check_b(B, "B", d)
    _check_matrix(C, "C", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    _check(load().gemm_run(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                           ctypes.c_void_p(C.data_ptr()), float(alpha), float(beta), _stream_ptr(stream)))


def gemm_plan_workspace_bytes(plan):
    """Bytes of workspace gemm_run_split needs for `plan` (0: no split form)."""
    out = ctypes.c_int64(0)
    _check(load().gemm_plan_workspace_bytes(plan.handle, ctypes.byref(out)))
    return out.value


def gemm_run_split(plan, A, B, C, alpha=1.0, beta=0.0, workspace=None, stream=None):
    """gemm_run with K split into the plan's ranges (partial products in `workspace`, a GPU tensor
    of at least gemm_plan_workspace_bytes(plan) bytes; allocated here when None)."""
    torch = _torch()
    d = plan.desc
    _check_a(A, "A", d)
    _check_b(B, "B", d)
    _check_matrix(C, "C", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    need = gemm_plan_workspace_bytes(plan)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=C.device) if need else None
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda"
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    wp = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().gemm_run_split(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                 ctypes.c_void_p(C.data_ptr()), float(alpha), float(beta), wp, wb, _stream_ptr(stream)))
    return workspace


def gemm_run_split_noalloc(plan, A, B, C, alpha=1.0, beta=0.0, stream=None):
    """gemm_run_split with the library's per-GPU workspace array: allocates nothing (calls that
    overlap on one GPU race on that array)."""
    d = plan.desc
    _check_a(A, "A", d)
    _check_b(B, "B", d)
    _check_matrix(C, "C", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    _check(load().gemm_run_split_noalloc(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                         ctypes.c_void_p(C.data_ptr()), float(alpha), float(beta), _stream_ptr(stream)))


REDUCE_OPS = {"sum": 1, "max": 2, "min": 3}


def gemm_run_reduce(plan, A, B, C, alpha=1.0, beta=0.0, op="sum", R=None, stream=None):
    """gemm_run plus R[i] = op over j of the FP32 output row i (R: float32 [m], or [batch, m])."""
    torch = _torch()
    d = plan.desc
    if op not in REDUCE_OPS:
        raise ValueError("op must be one of %s" % sorted(REDUCE_OPS))
    _check_a(A, "A", d)
    _check_b(B, "B", d)
    _check_matrix(C, "C", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    want = (d.m,) if d.batch == 1 else (d.batch, d.m)
    if not isinstance(R, torch.Tensor) or R.device.type != "cuda" or R.dtype != torch.float32 or \
            tuple(R.shape) != want or not R.is_contiguous():
        raise ValueError("R must be a contiguous float32 GPU tensor of shape %s" % (want,))
    _check(load().gemm_run_reduce(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                  ctypes.c_void_p(C.data_ptr()), float(alpha), float(beta), REDUCE_OPS[op],
                                  ctypes.c_void_p(R.data_ptr()), _stream_ptr(stream)))


def gemm_gate_up_run(plan, X, W_gate, W_up, G, U, stream=None):
    """G = X @ W_gate and U = X @ W_up in one launch."""
    d = plan.desc
    _check_a(X, "X", d)
    _check_b(W_gate, "W_gate", d)
    _check_b(W_up, "W_up", d)
    _check_matrix(G, "G", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    _check_matrix(U, "U", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    _check(load().gemm_gate_up_run(plan.handle, *[ctypes.c_void_p(t.data_ptr()) for t in (X, W_gate, W_up, G, U)],
                                   _stream_ptr(stream)))


def gemm_gate_up_swiglu_run(plan, X, W_gate, W_up, H, stream=None):
    """H = silu(X @ W_gate) * (X @ W_up) in one launch (activation fused into the epilogue)."""
    d = plan.desc
    _check_a(X, "X", d)
    _check_b(W_gate, "W_gate", d)
    _check_b(W_up, "W_up", d)
    _check_matrix(H, "H", d.m, d.n, d.ldc, d.c_type, d.batch, d.stride_c)
    _check(load().gemm_gate_up_swiglu_run(plan.handle, *[ctypes.c_void_p(t.data_ptr()) for t in (X, W_gate, W_up, H)],
                                          _stream_ptr(stream)))


def la_rms_norm_run(X, G, Y, eps=1e-6, stream=None):
    """Y = X * (1 / sqrt(mean(X^2 along a row) + eps)) * G for an [m, d] X (rows may be padded:
    stride(0) >= d, stride(1) == 1), a contiguous [d] G of X's dtype and an [m, d] Y (may be X itself)."""
    torch = _torch()
    for name, t in (("X", X), ("G", G), ("Y", Y)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype not in _KIND:
            raise ValueError("%s must be an f32/bf16/f16 tensor on the GPU" % name)
    if X.dim() != 2 or Y.dim() != 2 or tuple(Y.shape) != tuple(X.shape):
        raise ValueError("X and Y must be [m, d] tensors of the same shape, got %s and %s" % (tuple(X.shape), tuple(Y.shape)))
    m, d = X.shape
    if G.dim() != 1 or G.shape[0] != d or G.dtype != X.dtype or (d > 1 and G.stride(0) != 1):
        raise ValueError("G must be a contiguous [%d] tensor of X's dtype" % d)
    for name, t in (("X", X), ("Y", Y)):
        if m > 0 and d > 0 and (t.stride(1) != 1 or (m > 1 and t.stride(0) < d)):
            raise ValueError("%s rows must be contiguous with stride(0) >= d (strides %s)" % (name, t.stride()))
    ldx = X.stride(0) if m > 1 else max(1, d)
    ldy = Y.stride(0) if m > 1 else max(1, d)
    _check(load().la_rms_norm_run(int(m), int(d), _KIND[X.dtype], _KIND[Y.dtype], ctypes.c_void_p(X.data_ptr()), int(ldx),
                                  ctypes.c_void_p(G.data_ptr()), ctypes.c_void_p(Y.data_ptr()), int(ldy), float(eps),
                                  _stream_ptr(stream)))


def la_attention_run(Q, K, V, O, scale=None, stream=None):
    """O = softmax(scale * Q K^T) V per batch entry.  Q [batch, sq, d], K and V [batch, sk, d], O [batch, sq, d]
    (2-D tensors are one batch entry); rows may be padded (stride(-2) >= d, stride(-1) == 1).
    scale defaults to 1/sqrt(d)."""
    torch = _torch()
    ts = {"Q": Q, "K": K, "V": V, "O": O}
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype not in _KIND:
            raise ValueError("%s must be a bf16/f16/f32 tensor on the GPU" % name)
        if t.dim() not in (2, 3):
            raise ValueError("%s must be [batch, seq, d] or [seq, d]" % name)
    if not (Q.dim() == K.dim() == V.dim() == O.dim()):
        raise ValueError("Q, K, V and O must all be 2-D or all 3-D")
    v3 = {n: (t if t.dim() == 3 else t.unsqueeze(0)) for n, t in ts.items()}
    b, sq, d = v3["Q"].shape
    sk = v3["K"].shape[1]
    if tuple(v3["K"].shape) != (b, sk, d) or tuple(v3["V"].shape) != (b, sk, d) or tuple(v3["O"].shape) != (b, sq, d):
        raise ValueError("shapes: Q %s, K %s, V %s, O %s" % tuple(tuple(t.shape) for t in ts.values()))
    if Q.dtype != K.dtype or Q.dtype != V.dtype or Q.dtype == torch.float32:
        raise ValueError("Q, K and V must share one 16-bit dtype")
    for n, t in v3.items():
        if t.shape[1] > 0 and d > 0 and t.stride(2) != 1:
            raise ValueError("%s rows must be contiguous (stride(-1) == 1)" % n)
    ld = {n: (t.stride(1) if t.shape[1] > 1 else d) for n, t in v3.items()}
    st = {n: (t.stride(0) if t.shape[0] > 1 else 0) for n, t in v3.items()}
    desc = _AttnDesc(int(b), int(sq), int(sk), int(d), _KIND[Q.dtype], _KIND[O.dtype],
                     int(ld["Q"]), int(ld["K"]), int(ld["V"]), int(ld["O"]),
                     int(st["Q"]), int(st["K"]), int(st["V"]), int(st["O"]),
                     float(scale if scale is not None else 1.0 / (d ** 0.5)))
    _check(load().la_attention_run(ctypes.byref(desc), *[ctypes.c_void_p(t.data_ptr()) for t in (Q, K, V, O)],
                                   _stream_ptr(stream)))


def la_probe_mfma(operands, sink, workgroups, mfma_per_wave, stream=None):
    """Matrix-core rate probe: `workgroups` x 4 waves, each issuing mfma_per_wave MFMAs on 16-byte fragments
    taken from `operands` (a contiguous bf16/f16/f32/E4M3 tensor on the GPU, its dtype selects the instruction);
    `sink` is a float32 GPU tensor of at least workgroups * 256 elements."""
    torch = _torch()
    if not isinstance(operands, torch.Tensor) or operands.device.type != "cuda" or \
            operands.dtype not in (torch.bfloat16, torch.float16, torch.float32, torch.float8_e4m3fn):
        raise ValueError("operands must be a bf16/f16/f32/float8_e4m3fn tensor on the GPU")
    if not operands.is_contiguous():
        raise ValueError("operands must be contiguous")
    if not isinstance(sink, torch.Tensor) or sink.device.type != "cuda" or sink.dtype != torch.float32 or \
            not sink.is_contiguous() or sink.numel() < int(workgroups) * 256:
        raise ValueError("sink must be a contiguous float32 GPU tensor of at least workgroups * 256 elements")
    nbytes = (operands.numel() * operands.element_size()) // 16 * 16
    _check(load().la_probe_mfma(ctypes.c_void_p(operands.data_ptr()), int(nbytes), ctypes.c_void_p(sink.data_ptr()),
                                int(workgroups), int(mfma_per_wave), _KIND[operands.dtype], _stream_ptr(stream)))


def gemm_debug_lds_image(plan, A, B, B2, tile_m, tile_n, out, stream=None):
    """Copy the kernel's LDS stage for K block 0 of tile (tile_m, tile_n) into `out` (uint8/int16 tensor)."""
    _check(load().gemm_debug_lds_image(plan.handle, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                       ctypes.c_void_p(B2.data_ptr() if B2 is not None else 0),
                                       int(tile_m), int(tile_n), ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))


# ------------------------------------------------------------------ layout algebra (host)
def la_layout_eval(shape, stride, coord):
    out = ctypes.c_int64()
    _check(load().la_layout_eval(_i64s(shape), _i64s(stride), len(shape), _i64s(coord), ctypes.byref(out)))
    return out.value


def la_layout_eval_index(shape, stride, idx):
    out = ctypes.c_int64()
    _check(load().la_layout_eval_index(_i64s(shape), _i64s(stride), len(shape), int(idx), ctypes.byref(out)))
    return out.value


def la_swizzle_apply(b, m, s, offset):
    out = ctypes.c_int64()
    _check(load().la_swizzle_apply(int(b), int(m), int(s), int(offset), ctypes.byref(out)))
    return out.value


def la_tile_plan_offset(elem_bytes, shape, inner_axis, row_bytes, coord):
    off, tb = ctypes.c_int64(), ctypes.c_int64()
    _check(load().la_tile_plan_offset(int(elem_bytes), int(shape[0]), int(shape[1]), int(inner_axis), int(row_bytes),
                                      int(coord[0]), int(coord[1]), ctypes.byref(off), ctypes.byref(tb)))
    return off.value, tb.value


# layouts in the pages' notation ("shape:stride", nested tuples)
def _nested(x):
    """A Python int or nested tuple/list -> the pages' tuple text."""
    if isinstance(x, (list, tuple)):
        return "(" + ",".join(_nested(v) for v in x) + ")"
    return str(int(x))


def _layout_text(layout):
    """A "shape:stride" string, or a (shape, stride) pair of ints / nested tuples."""
    if isinstance(layout, str):
        return layout
    shape, stride = layout
    return _nested(shape) + ":" + _nested(stride)


def _text_out(fn, *args):
    buf = ctypes.create_string_buffer(4096)
    _check(fn(*args, buf, len(buf)))
    return buf.value.decode()


def la_layout_eval_str(layout, coord):
    out = ctypes.c_int64()
    c = coord if isinstance(coord, str) else _nested(coord)
    _check(load().la_layout_eval_str(_layout_text(layout).encode(), c.encode(), ctypes.byref(out)))
    return out.value


def la_layout_tile_str(layout, tile):
    return _text_out(load().la_layout_tile_str, _layout_text(layout).encode(), _i64s(tile), len(tile))


def la_layout_coalesce_str(layout):
    return _text_out(load().la_layout_coalesce_str, _layout_text(layout).encode())


def la_layout_permute_str(layout):
    return _text_out(load().la_layout_permute_str, _layout_text(layout).encode())


def la_layout_cosize_str(layout):
    out = ctypes.c_int64()
    _check(load().la_layout_cosize_str(_layout_text(layout).encode(), ctypes.byref(out)))
    return out.value


def la_view_window_eval(swizzle, layout, origin, extent, coord):
    out = ctypes.c_int64()
    b, m, s = swizzle
    _check(load().la_view_window_eval(int(b), int(m), int(s), _layout_text(layout).encode(), _i64s(origin),
                                      _i64s(extent), len(origin), _i64s(coord), ctypes.byref(out)))
    return out.value
