// extern "C" boundary of the GEMM library (declarations and contracts in
// include/la_gemm.h; the measurement aid in include/la_probe.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/la_gemm.h"
#include "../../include/la_probe.h"
#include "attention.hpp"
#include "kernel_table.hpp"
#include "launch.hpp"
#include "layout.hpp"
#include "norm.hpp"
#include "planner.hpp"

namespace {

thread_local std::string g_last_error;

gemm_status set_err(gemm_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % uintptr_t(bytes)) == 0; }

lak::TiledArgs base_args(const gemm_plan_s& p) {
  lak::TiledArgs a{};
  a.M = p.kd.m;
  a.N = p.kd.n;
  a.K = p.kd.k;
  a.lda = p.kd.lda;
  a.ldb = p.kd.ldb;
  a.ldc = p.kd.ldc;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.group_m = p.group_m;
  a.sa = p.kd.stride_a;
  a.sb = p.kd.stride_b;
  a.sc = p.kd.stride_c;
  a.out_bytes = p.out_bytes;
  return a;
}

gemm_status launch(const gemm_plan_s& p, const lak::TiledArgs& a, void* stream, bool image) {
  const dim3 grid(static_cast<unsigned>(p.grid), image ? 1u : static_cast<unsigned>(p.d.batch));
  const hipError_t e = lak::launch_kernel(p.kid, p.in_kind, p.out_kind, p.vec, p.gate_up, p.b_kmajor, p.a_trans, a, grid,
                                         static_cast<hipStream_t>(stream), image);
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

// The checks gemm_run makes before anything is enqueued.
gemm_status check_run(const gemm_plan_s& p, const void* A, const void* B, const void* C) {
  if (!C) return set_err(GEMM_ERR_NULL, "C is NULL");
  if (p.d.k > 0 && (!A || !B)) return set_err(GEMM_ERR_NULL, "A or B is NULL");
  if (!aligned(A, p.align_bytes) || !aligned(B, p.align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "A and B must be " + std::to_string(p.align_bytes) + "-byte aligned for this plan");
  if (!aligned(C, p.out_align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "C must be " + std::to_string(p.out_align_bytes) + "-byte aligned for this plan");
  return GEMM_OK;
}

// The split form of a plan (p.split > 1, inputs checked): S partial products into the workspace
// W (S slices of m x n FP32 values), one launch of the skinny or 256-wide kernel with the K ranges
// along y, then their sum in range order with alpha, beta and the rounding into C.
gemm_status run_split(const gemm_plan_s& p, const void* A, const void* B, void* C, float alpha, float beta, void* W,
                      void* stream) {
  lak::TiledArgs a = base_args(p);
  const int64_t ks = p.kd.k / p.split;     // K per range, in the kernel's units (byte pairs for one-byte codes)
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.K = ks;
  a.sa = ks;                                // range z starts ks units further along A's rows
  a.sb = p.b_kmajor ? ks : ks * p.kd.ldb;   // ... and along B's rows ([N, K]) or down its rows ([K, N])
  a.C = W;
  a.ldc = p.d.n;
  a.sc = p.d.m * p.d.n;
  a.out_bytes = 4;
  a.alpha = 1.0f;
  a.beta = 0.0f;
  a.tiles_m = p.split_tiles_m;
  a.tiles_n = p.split_tiles_n;
  a.group_m = 8;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned tiles = static_cast<unsigned>(p.split_tiles_m) * static_cast<unsigned>(p.split_tiles_n);
  hipError_t e = lak::launch_kernel(p.split_kid, p.in_kind, lak::OUT_F32, p.vec, false, p.b_kmajor, false, a,
                                    dim3(tiles, static_cast<unsigned>(p.split)), s, false);
  if (e == hipSuccess)
    e = lak::launch_split_sum(static_cast<const float*>(W), p.split, p.d.m, p.d.n, C, p.d.ldc, p.out_kind, alpha, beta, s);
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

}  // namespace

extern "C" {

const char* gemm_status_string(gemm_status s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_NULL: return "GEMM_ERR_NULL";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_ALIGNMENT: return "GEMM_ERR_ALIGNMENT";
    case GEMM_ERR_RESOURCE: return "GEMM_ERR_RESOURCE";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
  }
  return "GEMM_ERR_UNKNOWN";
}

const char* gemm_last_error(void) { return g_last_error.c_str(); }

gemm_status gemm_plan(const gemm_desc* desc, gemm_plan_t* out_plan) {
  if (!desc || !out_plan) return set_err(GEMM_ERR_NULL, "desc and out_plan must not be NULL");
  *out_plan = nullptr;
  gemm_plan_s* p = new (std::nothrow) gemm_plan_s();
  if (!p) return set_err(GEMM_ERR_RESOURCE, "out of host memory");
  std::string err;
  const gemm_status s = plan::build(*desc, *p, &err);
  if (s != GEMM_OK) {
    delete p;
    return set_err(s, err);
  }
  *out_plan = p;
  return GEMM_OK;
}

void gemm_plan_destroy(gemm_plan_t plan) { delete plan; }

gemm_status gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha, float beta, void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (p.gate_up) return set_err(GEMM_ERR_INVALID_ARG, "plan was made for gemm_gate_up_run");
  if (p.d.m == 0 || p.d.n == 0) return GEMM_OK;
  if (!C) return set_err(GEMM_ERR_NULL, "C is NULL");
  if (p.d.k > 0 && (!A || !B)) return set_err(GEMM_ERR_NULL, "A or B is NULL");
  if (!aligned(A, p.align_bytes) || !aligned(B, p.align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "A and B must be " + std::to_string(p.align_bytes) + "-byte aligned for this plan");
  if (!aligned(C, p.out_align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "C must be " + std::to_string(p.out_align_bytes) + "-byte aligned for this plan");
  lak::TiledArgs a = base_args(p);
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.C = C;
  a.alpha = alpha;
  a.beta = beta;
  return launch(p, a, stream, false);
}

gemm_status gemm_plan_workspace_bytes(gemm_plan_t plan, int64_t* out_bytes) {
  if (!plan || !out_bytes) return set_err(GEMM_ERR_NULL, "plan and out_bytes must not be NULL");
  *out_bytes = plan->ws_bytes;
  return GEMM_OK;
}

gemm_status gemm_run_split(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha, float beta,
                           void* workspace, int64_t workspace_bytes, void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (p.split <= 1) return gemm_run(plan, A, B, C, alpha, beta, stream);
  const gemm_status st = check_run(p, A, B, C);
  if (st != GEMM_OK) return st;
  if (!workspace) return set_err(GEMM_ERR_NULL, "workspace is NULL (this plan needs " + std::to_string(p.ws_bytes) + " bytes)");
  if (workspace_bytes < p.ws_bytes)
    return set_err(GEMM_ERR_INVALID_ARG, "workspace of " + std::to_string(workspace_bytes) + " bytes; this plan needs " +
                                             std::to_string(p.ws_bytes));
  if (!aligned(workspace, 16)) return set_err(GEMM_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  return run_split(p, A, B, C, alpha, beta, workspace, stream);
}

gemm_status gemm_run_split_noalloc(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha, float beta,
                                   void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (p.split <= 1) return gemm_run(plan, A, B, C, alpha, beta, stream);
  const gemm_status st = check_run(p, A, B, C);
  if (st != GEMM_OK) return st;
  if (p.ws_bytes > lak::kSplitScratchBytes)
    return set_err(GEMM_ERR_RESOURCE, "this plan's workspace of " + std::to_string(p.ws_bytes) + " bytes exceeds the " +
                                          std::to_string(lak::kSplitScratchBytes) + "-byte scratch of gemm_run_split_noalloc");
  void* W = nullptr;
  const hipError_t e = lak::split_scratch(&W);
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("scratch lookup failed: ") + hipGetErrorString(e));
  return run_split(p, A, B, C, alpha, beta, W, stream);
}

gemm_status gemm_run_reduce(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha, float beta,
                            int32_t op, float* R, void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (op != GEMM_REDUCE_SUM && op != GEMM_REDUCE_MAX && op != GEMM_REDUCE_MIN)
    return set_err(GEMM_ERR_INVALID_ARG, "op must be GEMM_REDUCE_SUM, GEMM_REDUCE_MAX or GEMM_REDUCE_MIN");
  if (p.gate_up) return set_err(GEMM_ERR_INVALID_ARG, "row reductions need a plan without GEMM_FLAG_GATE_UP");
  if (p.d.m == 0) return GEMM_OK;
  if (!R) return set_err(GEMM_ERR_NULL, "R is NULL");
  if (!aligned(R, 4)) return set_err(GEMM_ERR_ALIGNMENT, "R must be 4-byte aligned");
  const int red = op == GEMM_REDUCE_SUM ? lak::RED_SUM : op == GEMM_REDUCE_MAX ? lak::RED_MAX : lak::RED_MIN;
  if (p.d.n > 0) {
    // validate before anything is enqueued: on an error nothing runs and nothing is written
    if (!C) return set_err(GEMM_ERR_NULL, "C is NULL");
    if (p.d.k > 0 && (!A || !B)) return set_err(GEMM_ERR_NULL, "A or B is NULL");
    if (!aligned(A, p.align_bytes) || !aligned(B, p.align_bytes))
      return set_err(GEMM_ERR_ALIGNMENT, "A and B must be " + std::to_string(p.align_bytes) + "-byte aligned for this plan");
    if (!aligned(C, p.out_align_bytes))
      return set_err(GEMM_ERR_ALIGNMENT, "C must be " + std::to_string(p.out_align_bytes) + "-byte aligned for this plan");
  }
  const hipError_t e = lak::launch_reduce_init(R, p.d.m * p.d.batch, red, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (p.d.n == 0) return GEMM_OK;     // empty rows: R holds the identity
  lak::TiledArgs a = base_args(p);
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.C = C;
  a.alpha = alpha;
  a.beta = beta;
  a.red = red;
  a.R = R;
  return launch(p, a, stream, false);
}

gemm_status gemm_gate_up_run(gemm_plan_t plan, const void* X, const void* W_gate, const void* W_up, void* G, void* U,
                             void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (!p.gate_up) return set_err(GEMM_ERR_INVALID_ARG, "plan was not made with GEMM_FLAG_GATE_UP");
  if (p.d.m == 0 || p.d.n == 0) return GEMM_OK;
  if (!G || !U) return set_err(GEMM_ERR_NULL, "G or U is NULL");
  if (p.d.k > 0 && (!X || !W_gate || !W_up)) return set_err(GEMM_ERR_NULL, "X, W_gate or W_up is NULL");
  if (!aligned(X, p.align_bytes) || !aligned(W_gate, p.align_bytes) || !aligned(W_up, p.align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "X, W_gate and W_up must be " + std::to_string(p.align_bytes) + "-byte aligned for this plan");
  if (!aligned(G, p.out_align_bytes) || !aligned(U, p.out_align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "G and U must be " + std::to_string(p.out_align_bytes) + "-byte aligned for this plan");
  lak::TiledArgs a = base_args(p);
  a.A = static_cast<const uint16_t*>(X);
  a.B = static_cast<const uint16_t*>(W_gate);
  a.B2 = static_cast<const uint16_t*>(W_up);
  a.C = G;
  a.C2 = U;
  a.alpha = 1.0f;
  a.beta = 0.0f;
  return launch(p, a, stream, false);
}

gemm_status gemm_gate_up_swiglu_run(gemm_plan_t plan, const void* X, const void* W_gate, const void* W_up, void* H,
                                    void* stream) {
  if (!plan) return set_err(GEMM_ERR_NULL, "plan is NULL");
  const gemm_plan_s& p = *plan;
  if (!p.gate_up) return set_err(GEMM_ERR_INVALID_ARG, "plan was not made with GEMM_FLAG_GATE_UP");
  if (p.d.m == 0 || p.d.n == 0) return GEMM_OK;
  if (!H) return set_err(GEMM_ERR_NULL, "H is NULL");
  if (p.d.k > 0 && (!X || !W_gate || !W_up)) return set_err(GEMM_ERR_NULL, "X, W_gate or W_up is NULL");
  if (!aligned(X, p.align_bytes) || !aligned(W_gate, p.align_bytes) || !aligned(W_up, p.align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "X, W_gate and W_up must be " + std::to_string(p.align_bytes) + "-byte aligned for this plan");
  if (!aligned(H, p.out_align_bytes))
    return set_err(GEMM_ERR_ALIGNMENT, "H must be " + std::to_string(p.out_align_bytes) + "-byte aligned for this plan");
  lak::TiledArgs a = base_args(p);
  a.A = static_cast<const uint16_t*>(X);
  a.B = static_cast<const uint16_t*>(W_gate);
  a.B2 = static_cast<const uint16_t*>(W_up);
  a.C = H;
  a.C2 = nullptr;
  a.alpha = 1.0f;
  a.beta = 0.0f;
  a.act = 1;
  return launch(p, a, stream, false);
}

gemm_status la_rms_norm_run(int64_t m, int64_t d, int32_t x_type, int32_t y_type, const void* X, int64_t ldx,
                            const void* G, void* Y, int64_t ldy, float eps, void* stream) {
  auto kind = [](int32_t t) {
    return t == GEMM_F32 ? lak::OUT_F32 : t == GEMM_BF16 ? lak::OUT_BF16 : t == GEMM_F16 ? lak::OUT_F16 : -1;
  };
  const int xk = kind(x_type), yk = kind(y_type);
  if (xk < 0 || yk < 0) return set_err(GEMM_ERR_INVALID_ARG, "x_type and y_type must be GEMM_F32, GEMM_BF16 or GEMM_F16");
  if (m < 0 || d < 0) return set_err(GEMM_ERR_INVALID_ARG, "m and d must be >= 0");
  if (ldx < std::max<int64_t>(1, d) || ldy < std::max<int64_t>(1, d))
    return set_err(GEMM_ERR_INVALID_ARG, "ldx and ldy must be >= max(1, d)");
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return set_err(GEMM_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (m > (int64_t{1} << 40) || d > (int64_t{1} << 24) || ldx > (int64_t{1} << 40) || ldy > (int64_t{1} << 40))
    return set_err(GEMM_ERR_UNSUPPORTED, "d must be <= 2^24 (exact as FP32), m, ldx and ldy <= 2^40");
  if (m == 0 || d == 0) return GEMM_OK;
  if (!X || !G || !Y) return set_err(GEMM_ERR_NULL, "X, G and Y must not be NULL");
  const int xs = x_type == GEMM_F32 ? 4 : 2, ys = y_type == GEMM_F32 ? 4 : 2;
  if (!aligned(X, xs) || !aligned(G, xs) || !aligned(Y, ys))
    return set_err(GEMM_ERR_ALIGNMENT, "X, G and Y must be aligned to their element size");
  // Byte ranges: Y may be X itself (same rows, same element size); no other overlap.
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), y0 = reinterpret_cast<uintptr_t>(Y);
  const uintptr_t g0 = reinterpret_cast<uintptr_t>(G);
  const __int128 xb = (__int128(m - 1) * ldx + d) * xs, yb = (__int128(m - 1) * ldy + d) * ys;
  if (xb > (__int128(1) << 56) || yb > (__int128(1) << 56)) return set_err(GEMM_ERR_UNSUPPORTED, "X or Y spans more than 2^56 bytes");
  const uintptr_t x1 = x0 + uintptr_t(xb), y1 = y0 + uintptr_t(yb);
  const uintptr_t g1 = g0 + uintptr_t(d * xs);
  const bool in_place = x0 == y0 && ldx == ldy && xs == ys;
  if (!in_place && x0 < y1 && y0 < x1) return set_err(GEMM_ERR_INVALID_ARG, "Y overlaps X without being X itself");
  if (g0 < y1 && y0 < g1) return set_err(GEMM_ERR_INVALID_ARG, "Y overlaps G");
  const int v = lak::rms_norm_vec_elems(xk);
  const bool vec = aligned(X, 16) && aligned(G, 16) && aligned(Y, 16) && ldx % v == 0 && ldy % v == 0;
  lak::NormArgs a{X, G, Y, m, d, ldx, ldy, eps};
  const hipError_t e = lak::launch_rms_norm(a, xk, yk, vec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status la_probe_mfma(const void* operands, int64_t operand_bytes, float* sink, int64_t workgroups,
                          int64_t mfma_per_wave, int32_t in_type, void* stream) {
  if (in_type != GEMM_BF16 && in_type != GEMM_F16 && in_type != GEMM_F32 && in_type != GEMM_F8E4M3)
    return set_err(GEMM_ERR_INVALID_ARG, "in_type must be GEMM_BF16, GEMM_F16, GEMM_F32 or GEMM_F8E4M3");
  if (operand_bytes < 16 || operand_bytes % 16) return set_err(GEMM_ERR_INVALID_ARG, "operand_bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > (int64_t{1} << 20)) return set_err(GEMM_ERR_INVALID_ARG, "workgroups must be in 1..2^20");
  if (mfma_per_wave < 16 || mfma_per_wave % 16 || mfma_per_wave > (int64_t{1} << 24))
    return set_err(GEMM_ERR_INVALID_ARG, "mfma_per_wave must be a positive multiple of 16, at most 2^24");
  if (!operands || !sink) return set_err(GEMM_ERR_NULL, "operands and sink must not be NULL");
  if (!aligned(operands, 16) || !aligned(sink, 4)) return set_err(GEMM_ERR_ALIGNMENT, "operands must be 16-byte aligned, sink 4-byte aligned");
  const hipError_t e = lak::launch_mfma_probe(operands, operand_bytes / 16, sink, workgroups, mfma_per_wave,
                                              in_type == GEMM_BF16 ? lak::IN_BF16 : in_type == GEMM_F16 ? lak::IN_F16
                                              : in_type == GEMM_F32 ? lak::IN_F32 : lak::IN_F8,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status la_attention_run(const attn_desc* desc, const void* Q, const void* K, const void* V, void* O,
                             void* stream) {
  if (!desc) return set_err(GEMM_ERR_NULL, "desc is NULL");
  const attn_desc& d = *desc;
  if (d.batch < 0 || d.sq < 0 || d.sk < 0) return set_err(GEMM_ERR_INVALID_ARG, "batch, sq and sk must be >= 0");
  if (d.d != 64 && d.d != 128) return set_err(GEMM_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if (d.in_type != GEMM_BF16 && d.in_type != GEMM_F16) return set_err(GEMM_ERR_INVALID_ARG, "in_type must be GEMM_BF16 or GEMM_F16");
  if (d.out_type != GEMM_F32 && d.out_type != GEMM_BF16 && d.out_type != GEMM_F16)
    return set_err(GEMM_ERR_INVALID_ARG, "out_type must be GEMM_F32, GEMM_BF16 or GEMM_F16");
  if (!(d.scale == d.scale) || d.scale == __builtin_inff() || d.scale == -__builtin_inff())
    return set_err(GEMM_ERR_INVALID_ARG, "scale must be finite");
  if (d.scale < 0.0f) return set_err(GEMM_ERR_UNSUPPORTED, "scale must be >= 0");
  const int64_t lds[4] = {d.ld_q, d.ld_k, d.ld_v, d.ld_o};
  const int64_t strides[4] = {d.stride_q, d.stride_k, d.stride_v, d.stride_o};
  if (d.batch > (int64_t{1} << 31) || d.sq > (int64_t{1} << 31) || d.sk > (int64_t{1} << 31))
    return set_err(GEMM_ERR_UNSUPPORTED, "batch, sq and sk must be <= 2^31");
  for (int i = 0; i < 4; ++i) {
    if (lds[i] < d.d || strides[i] < 0) return set_err(GEMM_ERR_INVALID_ARG, "row strides must be >= d and batch strides >= 0");
    if (lds[i] > (int64_t{1} << 40) || strides[i] > (int64_t{1} << 40))
      return set_err(GEMM_ERR_UNSUPPORTED, "row and batch strides must be <= 2^40 elements");
    if (lds[i] % 8 || strides[i] % 8) return set_err(GEMM_ERR_ALIGNMENT, "row and batch strides must be multiples of 8 elements");
  }
  if (d.batch * d.sq == 0) return GEMM_OK;
  if (d.sk == 0) return set_err(GEMM_ERR_INVALID_ARG, "attention over zero keys is undefined (sk must be >= 1)");
  if (!Q || !K || !V || !O) return set_err(GEMM_ERR_NULL, "Q, K, V and O must not be NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return set_err(GEMM_ERR_ALIGNMENT, "Q, K, V and O must be 16-byte aligned");
  if (128 * d.ld_k >= (int64_t{1} << 32) || 128 * d.ld_v >= (int64_t{1} << 32))
    return set_err(GEMM_ERR_UNSUPPORTED, "K and V row strides must keep 64 rows below 4 GiB");
  const int64_t q_tiles = (d.sq + 127) / 128;
  // one launch: the grid's work-items along x (query tiles x threads per tile) must fit in 32 bits
  if (d.batch > int64_t(UINT32_MAX) / (q_tiles * lak::ATTN_THREADS))
    return set_err(GEMM_ERR_UNSUPPORTED, "too many query tiles for one launch");
  const int osz = d.out_type == GEMM_F32 ? 4 : 2;
  // batch entries of O: disjoint blocks, or rows interleaved with disjoint segments
  const bool o_blocks = __int128(d.stride_o) >= __int128(d.sq - 1) * d.ld_o + d.d;
  const bool o_interleaved = d.stride_o >= d.d && __int128(d.ld_o) >= __int128(d.batch - 1) * d.stride_o + d.d;
  if (d.batch > 1 && !o_blocks && !o_interleaved)
    return set_err(GEMM_ERR_INVALID_ARG, "batch entries of O overlap");
  // O must not overlap any input (byte ranges of everything each pointer may touch)
  auto span = [&](const void* p, int64_t stride, int64_t rows, int64_t ld, int esz) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    const __int128 bytes = (__int128(d.batch - 1) * stride + __int128(rows - 1) * ld + d.d) * esz;
    return std::pair<uintptr_t, uintptr_t>(b, b + uintptr_t(bytes < (__int128(1) << 62) ? bytes : (__int128(1) << 62)));
  };
  const auto o = span(O, d.stride_o, d.sq, d.ld_o, osz);
  const std::pair<uintptr_t, uintptr_t> ins[3] = {span(Q, d.stride_q, d.sq, d.ld_q, 2), span(K, d.stride_k, d.sk, d.ld_k, 2),
                                                  span(V, d.stride_v, d.sk, d.ld_v, 2)};
  for (const auto& r : ins)
    if (o.first < r.second && r.first < o.second) return set_err(GEMM_ERR_INVALID_ARG, "O overlaps Q, K or V");
  lak::AttnArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = O;
  a.batch = d.batch;
  a.sq = d.sq;
  a.sk = d.sk;
  a.ldq = d.ld_q; a.ldk = d.ld_k; a.ldv = d.ld_v; a.ldo = d.ld_o;
  a.bq = d.stride_q; a.bk = d.stride_k; a.bv = d.stride_v; a.bo = d.stride_o;
  // the kernel needs a positive factor to push masked keys to -inf; a zero scale
  // (uniform weights) becomes the smallest normal float, for which every valid
  // score still gives probability exactly 1
  a.scale_log2 = d.scale > 0.0f ? d.scale * 1.4426950408889634f : 1.17549435e-38f;
  a.q_tiles = static_cast<int>(q_tiles);
  const hipError_t e = lak::launch_attention(a, static_cast<int>(d.d), d.in_type == GEMM_BF16 ? lak::IN_BF16 : lak::IN_F16,
                                             d.out_type == GEMM_F32 ? lak::OUT_F32 : d.out_type == GEMM_BF16 ? lak::OUT_BF16 : lak::OUT_F16,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_err(GEMM_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GEMM_OK;
}

gemm_status gemm_plan_describe(gemm_plan_t plan, char* buf, size_t len) {
  if (!plan || !buf) return set_err(GEMM_ERR_NULL, "plan and buf must not be NULL");
  if (plan->json.size() + 1 > len) return set_err(GEMM_ERR_RESOURCE, "buffer too small for the plan description");
  std::memcpy(buf, plan->json.c_str(), plan->json.size() + 1);
  return GEMM_OK;
}

gemm_status gemm_plan_lds_offset(gemm_plan_t plan, int operand, int64_t row, int64_t col, int64_t* out_elem_offset) {
  if (!plan || !out_elem_offset) return set_err(GEMM_ERR_NULL, "plan and out_elem_offset must not be NULL");
  std::string err;
  const gemm_status s = plan::lds_offset(*plan, operand, row, col, out_elem_offset, &err);
  return s == GEMM_OK ? s : set_err(s, err);
}

gemm_status gemm_plan_lds_stage_bytes(gemm_plan_t plan, int64_t* out_bytes) {
  if (!plan || !out_bytes) return set_err(GEMM_ERR_NULL, "plan and out_bytes must not be NULL");
  *out_bytes = plan->stage_elems * plan->in_bytes;
  return GEMM_OK;
}

gemm_status gemm_debug_lds_image(gemm_plan_t plan, const void* A, const void* B, const void* B2, int64_t tile_m,
                                 int64_t tile_n, void* out, void* stream) {
  if (!plan || !out || !A || !B) return set_err(GEMM_ERR_NULL, "plan, A, B and out must not be NULL");
  const gemm_plan_s& p = *plan;
  if (p.gate_up && !B2) return set_err(GEMM_ERR_NULL, "gate/up plans need B2");
  if (tile_m < 0 || tile_m >= p.tiles_m || tile_n < 0 || tile_n >= p.tiles_n)
    return set_err(GEMM_ERR_INVALID_ARG, "tile index outside the plan's tile grid");
  if (!aligned(A, p.align_bytes) || !aligned(B, p.align_bytes) || (B2 && !aligned(B2, p.align_bytes)))
    return set_err(GEMM_ERR_ALIGNMENT, "operands break the plan's alignment class");
  if (!aligned(out, 16)) return set_err(GEMM_ERR_ALIGNMENT, "out must be 16-byte aligned");
  lak::TiledArgs a = base_args(p);
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.B2 = static_cast<const uint16_t*>(B2);
  a.dbg_tm = static_cast<int>(tile_m);
  a.dbg_tn = static_cast<int>(tile_n);
  a.dbg_out = static_cast<uint16_t*>(out);
  return launch(p, a, stream, true);
}

// ---- layout algebra entry points (host only) ----

gemm_status la_layout_eval(const int64_t* shape, const int64_t* stride, int rank, const int64_t* coord,
                           int64_t* out_offset) {
  if (!shape || !stride || !coord || !out_offset) return set_err(GEMM_ERR_NULL, "NULL argument");
  if (rank <= 0 || rank > 16) return set_err(GEMM_ERR_INVALID_ARG, "rank must be 1..16");
  try {
    const la::Layout l = la::Layout::flat(std::vector<int64_t>(shape, shape + rank), std::vector<int64_t>(stride, stride + rank));
    *out_offset = l.at(std::vector<int64_t>(coord, coord + rank));
  } catch (const la::LayoutError& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

gemm_status la_layout_eval_index(const int64_t* shape, const int64_t* stride, int rank, int64_t idx,
                                 int64_t* out_offset) {
  if (!shape || !stride || !out_offset) return set_err(GEMM_ERR_NULL, "NULL argument");
  if (rank <= 0 || rank > 16) return set_err(GEMM_ERR_INVALID_ARG, "rank must be 1..16");
  try {
    const la::Layout l = la::Layout::flat(std::vector<int64_t>(shape, shape + rank), std::vector<int64_t>(stride, stride + rank));
    *out_offset = l(idx);
  } catch (const la::LayoutError& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

gemm_status la_swizzle_apply(int b, int m, int s, int64_t offset, int64_t* out_offset) {
  if (!out_offset) return set_err(GEMM_ERR_NULL, "NULL argument");
  if (!la::Swizzle::valid(b, m, s) || offset < 0 || b > 16 || m > 30 || s > 30)
    return set_err(GEMM_ERR_INVALID_ARG, "Swizzle fields overlap, a parameter is out of range or the offset is negative");
  *out_offset = la::Swizzle(b, m, s)(offset);
  return GEMM_OK;
}

gemm_status la_tile_plan_offset(int elem_bytes, int64_t d1, int64_t d2, int inner_axis, int row_bytes, int64_t c1,
                                int64_t c2, int64_t* out_offset, int64_t* out_transfer_bytes) {
  if (!out_offset || !out_transfer_bytes) return set_err(GEMM_ERR_NULL, "NULL argument");
  try {
    const la::SharedTilePlan tp(elem_bytes, d1, d2, inner_axis, row_bytes);
    *out_offset = tp.layout.at({c1, c2});
    *out_transfer_bytes = tp.transfer_bytes();
  } catch (const la::LayoutError& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

namespace {
gemm_status copy_out(const std::string& text, char* out, size_t len) {
  if (text.size() + 1 > len) return set_err(GEMM_ERR_RESOURCE, "output buffer of " + std::to_string(len) + " bytes is too small");
  std::memcpy(out, text.c_str(), text.size() + 1);
  return GEMM_OK;
}
}  // namespace

gemm_status la_layout_eval_str(const char* layout, const char* coord, int64_t* out_offset) {
  if (!layout || !coord || !out_offset) return set_err(GEMM_ERR_NULL, "NULL argument");
  try {
    *out_offset = la::parse_layout(layout)(la::parse_tree(coord));
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

gemm_status la_layout_tile_str(const char* layout, const int64_t* tile, int32_t rank, char* out, size_t len) {
  if (!layout || !tile || !out) return set_err(GEMM_ERR_NULL, "NULL argument");
  if (rank <= 0 || rank > 16) return set_err(GEMM_ERR_INVALID_ARG, "rank must be 1..16");
  try {
    return copy_out(la::tile(la::parse_layout(layout), std::vector<int64_t>(tile, tile + rank)).str(), out, len);
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
}

gemm_status la_layout_coalesce_str(const char* layout, char* out, size_t len) {
  if (!layout || !out) return set_err(GEMM_ERR_NULL, "NULL argument");
  try {
    return copy_out(la::coalesce(la::parse_layout(layout)).str(), out, len);
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
}

gemm_status la_layout_permute_str(const char* layout, char* out, size_t len) {
  if (!layout || !out) return set_err(GEMM_ERR_NULL, "NULL argument");
  try {
    return copy_out(la::permute(la::parse_layout(layout)).str(), out, len);
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
}

gemm_status la_layout_cosize_str(const char* layout, int64_t* out_cosize) {
  if (!layout || !out_cosize) return set_err(GEMM_ERR_NULL, "NULL argument");
  try {
    *out_cosize = la::cosize(la::parse_layout(layout));
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

gemm_status la_view_window_eval(int32_t b, int32_t m, int32_t s, const char* layout, const int64_t* origin,
                                const int64_t* extent, int32_t rank, const int64_t* coord, int64_t* out_offset) {
  if (!layout || !origin || !extent || !coord || !out_offset) return set_err(GEMM_ERR_NULL, "NULL argument");
  if (rank <= 0 || rank > 16) return set_err(GEMM_ERR_INVALID_ARG, "rank must be 1..16");
  if (!la::Swizzle::valid(b, m, s) || b > 16 || m > 30 || s > 30)
    return set_err(GEMM_ERR_INVALID_ARG, "Swizzle fields overlap or a parameter is out of range");
  try {
    const la::View parent(la::Swizzle(b, m, s), la::parse_layout(layout));
    const la::View w = parent.window(std::vector<int64_t>(origin, origin + rank), std::vector<int64_t>(extent, extent + rank));
    *out_offset = w.at(std::vector<int64_t>(coord, coord + rank));
  } catch (const std::exception& e) {
    return set_err(GEMM_ERR_INVALID_ARG, e.what());
  }
  return GEMM_OK;
}

}  // extern "C"
