/*
 * la_gemm.h -- C ABI of the MI355X (gfx950) tiled GEMM library.
 *
 * One operation: C = alpha * A * B + beta * C with bf16 or fp16 inputs and
 * FP32 accumulation, plus a fused gate/up variant that multiplies one
 * activation matrix by two weight matrices.  The epilogue form follows the
 * Phobos page "Tiles and shared memory" (section "var and let": new C is
 * alpha times the accumulator plus beta times the old C) and the Tylo.jl page
 * "Layouts, storage and ownership" (section "Plans describe work, callers
 * establish readiness": scaling is composed into the epilogue, no separate
 * kernel).  The fused gate/up projection is the consumer named on the Tylo.jl
 * page "TMA and Hopper WGMMA" (opening paragraph and section "Worked
 * consumers and current validation").
 *
 * Storage (all row-major, element strides, zero-based, as on the Tylo.jl page
 * "Layouts, storage and ownership", section "A layout is a function"):
 *   A  [M, K]  element (i, k) at A[i * lda + k]          (K contiguous; or, with
 *              GEMM_FLAG_A_TRANSPOSED, at A[k * lda + i], M contiguous)
 *   B  [K, N]  element (k, j) at B[k * ldb + j]          (N contiguous; or, with
 *              GEMM_FLAG_B_KMAJOR, at B[j * ldb + k], K contiguous)
 *   C  [M, N]  element (i, j) at C[i * ldc + j]
 * B is addressed in its mathematical (K, N) coordinates throughout.
 *
 * Ownership and lifetime (Tylo.jl "TMEM tiles and transfers", section
 * "Completion and validation"; "Layouts, storage and ownership", section
 * "Plans describe work, callers establish readiness"): the caller owns every
 * buffer, its size, its lifetime and its reuse.  A plan is an immutable host
 * object describing the work; it never touches device memory.  Device
 * pointers are passed per run, so one plan serves any number of runs with
 * changed values or other buffers of the same shape.
 *
 * Errors: every entry point returns a gemm_status.  On an error nothing is
 * launched and nothing is written.  Requests the kernels do not support are
 * rejected, never silently routed elsewhere (Tylo.jl "TMEM tiles and
 * transfers", section "Storage units": no silent substitution of another
 * instruction).  gemm_last_error() gives a thread-local description of the
 * most recent failure.  Device faults surface at the caller's next
 * synchronisation, as with any asynchronous launch.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Runs are asynchronous, never allocate, never synchronise and
 * never read device memory on the host, so they may be captured in a HIP
 * graph.
 */
#ifndef LA_GEMM_H
#define LA_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_NULL = 1,          /* a required pointer argument is NULL */
  GEMM_ERR_INVALID_ARG = 2,   /* negative size, leading dimension too small, bad enum */
  GEMM_ERR_UNSUPPORTED = 3,   /* a well-formed request no kernel implements */
  GEMM_ERR_ALIGNMENT = 4,     /* a pointer breaks the plan's alignment class */
  GEMM_ERR_RESOURCE = 5,      /* a layout or tile would not fit (e.g. LDS) */
  GEMM_ERR_HIP = 6            /* the HIP runtime reported an error */
} gemm_status;

typedef enum {
  GEMM_BF16 = 0,
  GEMM_F16 = 1,
  GEMM_F32 = 2,
  GEMM_F8E4M3 = 3,   /* OCP 8-bit E4M3 (bias 7, no infinities, largest 448): inputs only */
  GEMM_F8E5M2 = 4    /* OCP 8-bit E5M2 (bias 15, binary16's upper byte): inputs only */
} gemm_dtype;

/* Flags for gemm_desc.flags. */
#define GEMM_FLAG_GATE_UP 0x1u   /* plan is for gemm_gate_up_run / gemm_gate_up_swiglu_run */
#define GEMM_FLAG_B_KMAJOR 0x2u  /* B (and W_gate, W_up) stored [N, K]: element (k, n) at
                                    B[n * ldb + k], ldb >= max(1, k) -- the K-contiguous operand
                                    storage of the Tylo.jl page "TMA and Hopper WGMMA" (section
                                    "The same storage contract on both sides") */
#define GEMM_FLAG_A_TRANSPOSED 0x8u  /* A (and X) stored [K, M]: element (i, k) at A[k * lda + i],
                                    lda >= max(1, m) -- a layout is a function and either major order
                                    is the same matrix (Tylo.jl "Layouts, storage and ownership",
                                    section "A layout is a function": permutedims swaps the modes).
                                    With 16-bit inputs: not combined with GEMM_FLAG_B_KMAJOR, and m
                                    a multiple of 8 or larger than 8 (16-byte staging along M); never
                                    the skinny kernel.  Otherwise rejected with GEMM_ERR_UNSUPPORTED.
                                    Binary32 inputs take every combination */
#define GEMM_FLAG_LARGE_TILES 0x4u  /* keep the largest tile the shape allows.  Without it the
                                    planner moves a GEMM whose grid would leave most of the 256
                                    CUs idle to 64 x 64 tiles (fewer than 32 workgroups of the
                                    256-wide full-tile kernels, 64 when M or N ends inside a tile;
                                    for the general kernel, always with 16-byte loads and below
                                    384 workgroups of 128 x 128 with 2-byte loads), and keeps
                                    shapes whose 256-wide tiles would pad M x N by more than 1.3x
                                    on the general kernel.  For callers that run many small GEMMs
                                    on concurrent streams, where one GEMM need not fill the chip. */

typedef struct {
  int64_t m, n, k;             /* problem sizes, each >= 0 */
  int32_t a_type, b_type;      /* gemm_dtype; equal: BF16, F16, or F32 (binary32 inputs: plain GEMMs
                                  and row reductions only, any shape and storage order, staged
                                  through 64-byte rows of 16 values -- the 64-byte fp32 plan of the
                                  Tylo.jl page "TMA and Hopper WGMMA", section "The same storage
                                  contract on both sides" -- and multiplied on the FP32 matrix cores;
                                  gate/up plans and mixed widths are GEMM_ERR_UNSUPPORTED); or each
                                  of F8E4M3 / F8E5M2 (one-byte codes, the formats may differ: plain
                                  GEMMs, row reductions and gate/up with A (X) stored [M, K] and B
                                  (the weights) stored [N, K] (GEMM_FLAG_B_KMAJOR), lda, ldb and the
                                  A / B batch strides
                                  multiples of 16, ldc and stride_c multiples of 8, k a multiple of
                                  64 below 512 and of 16 from 512 on; staged through the same
                                  page's 64-byte rows (64 codes) and multiplied 64 deep per matrix
                                  instruction, which adds its 64 products with less than binary32
                                  precision; anything else is GEMM_ERR_UNSUPPORTED) */
  int32_t c_type;              /* gemm_dtype of C (and of G, U): F32, BF16 or F16 */
  int64_t lda, ldb, ldc;       /* element strides: lda >= max(1,k) (max(1,m) for A stored [K,M]),
                                  ldb >= max(1,n) (max(1,k) for K-major B), ldc >= max(1,n) */
  uint32_t flags;              /* GEMM_FLAG_* */
  int64_t batch;               /* >= 1: independent GEMMs per run (1..65535); matrix b of each operand
                                  starts stride_* elements after matrix b-1 (a batch coordinate, as the
                                  Tylo.jl page "TMA and Hopper WGMMA" binds a batch of matrices with a
                                  third origin coordinate, section "The same storage contract on both
                                  sides") */
  int64_t stride_a, stride_b, stride_c;  /* element strides between matrices, >= 0, read only when
                                  batch > 1; inputs may alias (0 broadcasts one matrix), outputs may
                                  not: stride_c >= (m-1)*ldc + n (blocks), or stride_c >= n and
                                  ldc >= (batch-1)*stride_c + n (interleaved rows).  They join
                                  lda/ldb/ldc in the alignment class (16-byte vectors need
                                  multiples of 8 elements, 4 for binary32) */
} gemm_desc;

typedef struct gemm_plan_s* gemm_plan_t;   /* opaque, immutable, host-only */

/* Validate `desc`, choose a kernel configuration and build its layouts.
 * On success *out_plan owns a new plan (free with gemm_plan_destroy). */
gemm_status gemm_plan(const gemm_desc* desc, gemm_plan_t* out_plan);

/* Release a plan.  NULL is ignored.  Runs already enqueued are unaffected. */
void gemm_plan_destroy(gemm_plan_t plan);

/* C = alpha * A * B + beta * C on `stream`.
 * A, B, C are device pointers laid out as described above; A and B must be
 * aligned to the plan's alignment class (see gemm_plan_describe); C may be
 * read (beta != 0) and written only inside [0,m) x [0,n).  When beta == 0, C
 * is not read (NaN there does not propagate).  k == 0 gives C = beta * C.
 * m == 0 or n == 0 launches nothing.  Outputs are rounded to nearest even.
 * With batch > 1 the pointers address matrix 0 and matrix b sits at
 * b * stride_* elements further on; all matrices run in one launch. */
gemm_status gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C,
                     float alpha, float beta, void* stream);

/* Bytes of device workspace gemm_run_split needs for this plan: split * m * n * 4
 * (the FP32 partial products), 0 when the plan has no split form. */
gemm_status gemm_plan_workspace_bytes(gemm_plan_t plan, int64_t* out_bytes);

/* gemm_run with the sum over k cut into `split` equal ranges (gemm_plan_describe:
 * "split_k", "split_kernel", "split_grid", "workspace_bytes").  The result is the
 * same C = alpha * A * B + beta * C (the epilogue of the Phobos page "Tiles
 * and shared memory", section "var and let") with the sum over k grouped by
 * range: the accumulator is built from K slices of A and B (section "Making a
 * tile", slices A[r :+ 64, kt :+ 16]), the ranges are runs of whole K slices,
 * and their FP32 partial sums are added in range order, so only the order of
 * the FP32 additions differs from gemm_run (deterministic: the same inputs
 * give the same bits).  The planner gives a plan a split form where a single
 * matrix's grid leaves most CUs idle: the skinny shapes (m <= 128, B streamed
 * once) on few column strips, and other shapes with at most 128 tiles of the
 * 256-wide kernel, split on 128-row tiles (n a multiple of 8, K cut into
 * ranges of whole K blocks, at least 1024 deep).  One launch writes the ranges'
 * products into `workspace` (split slices of m x n FP32 values), a second sums
 * them into C with alpha, beta and the rounding.
 * `workspace` is a device buffer of at least gemm_plan_workspace_bytes bytes,
 * 16-byte aligned, owned by the caller, overlapping no operand; its contents on
 * entry do not matter and are overwritten.  Runs that share a workspace must be
 * ordered (same stream, or synchronised).  A plan without a split form runs as
 * gemm_run (workspace may be NULL).  Errors as gemm_run, plus GEMM_ERR_NULL /
 * GEMM_ERR_INVALID_ARG / GEMM_ERR_ALIGNMENT for a missing, short or misaligned
 * workspace; nothing is enqueued then.  Allocates nothing; capturable. */
gemm_status gemm_run_split(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha,
                           float beta, void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_run_split for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * partial products go to a workspace array the library holds on each GPU for
 * the life of the process (64 MiB, enough for every split form the planner
 * makes), instead of a caller-provided buffer.  The array of the current
 * device is used; its address is looked up on the first call on that device.
 * Calls that overlap on one GPU (concurrent streams, or two threads) share the
 * array and race: order them (one stream, or synchronise between them).  The
 * array needs no clearing (each run overwrites what it reads).  Same results
 * (bit for bit) and errors as gemm_run_split; a plan whose workspace would
 * exceed the array is GEMM_ERR_RESOURCE, nothing enqueued.  A plan without a
 * split form runs as gemm_run.  Calls no allocating routine. */
gemm_status gemm_run_split_noalloc(gemm_plan_t plan, const void* A, const void* B, void* C,
                                   float alpha, float beta, void* stream);

/* Row reductions for gemm_run_reduce. */
typedef enum { GEMM_REDUCE_SUM = 1, GEMM_REDUCE_MAX = 2, GEMM_REDUCE_MIN = 3 } gemm_reduce_op;

/* gemm_run that also reduces every output row: R[b*m + i] = sum, maximum or
 * minimum over j < n of out[i, j] of matrix b, where out is the FP32 value
 * alpha * acc + beta * C_old before it is rounded to C's type -- the sum /
 * maximum / minimum along the second axis of a finished accumulator of the
 * Tylo.jl page "TMA and Hopper WGMMA" (section "WGMMA values and ownership"),
 * taken over whole rows.  R is a device array of m * batch floats, written
 * whole (n == 0 leaves the identity: 0, -inf, +inf).  Each workgroup folds
 * its rows' partial results into R with atomics, so sums may differ in the
 * last bits from run to run; maximum and minimum are exact (NaN outputs give
 * an unspecified result).  A plan with GEMM_FLAG_GATE_UP is rejected.
 * R must not overlap A, B or C.  Same stream, graph and error rules as
 * gemm_run (a fill kernel prepares R on the stream first). */
gemm_status gemm_run_reduce(gemm_plan_t plan, const void* A, const void* B, void* C, float alpha,
                            float beta, int32_t op, float* R, void* stream);

/* G = X * W_gate and U = X * W_up (alpha = 1, beta = 0) in one launch that
 * stages each X tile once for both products.  Needs a plan made with
 * GEMM_FLAG_GATE_UP; X is [m, k] (lda), W_gate and W_up are [k, n] (ldb),
 * G and U are [m, n] (ldc). */
gemm_status gemm_gate_up_run(gemm_plan_t plan, const void* X, const void* W_gate,
                             const void* W_up, void* G, void* U, void* stream);

/* H = silu(X * W_gate) (.) (X * W_up), silu(g) = g / (1 + e^-g), evaluated
 * in FP32 on the two accumulators of each element and rounded once to H's
 * type: the activation composed into the gate/up epilogue (Tylo.jl "Layouts,
 * storage and ownership", section "Plans describe work, callers establish
 * readiness": scaling and activation fuse into the epilogue).  Same plan and
 * operands as gemm_gate_up_run; H is [m, n] (ldc). */
gemm_status gemm_gate_up_swiglu_run(gemm_plan_t plan, const void* X, const void* W_gate,
                                    const void* W_up, void* H, void* stream);

/* Row normalisation, the kernel of the Phobos page "Tiles and shared memory"
 * (section "A complete kernel"): for each row i < m,
 *   inv[i] = 1 / sqrt((sum_j X[i,j]^2) / d + eps),   Y[i,j] = X[i,j] * inv[i] * G[j].
 * X is [m, d] row-major with row stride ldx >= max(1, d), G is [d] (same type
 * as X), Y is [m, d] with row stride ldy >= max(1, d); x_type, y_type are
 * GEMM_F32, GEMM_BF16 or GEMM_F16 (device pointers, caller-owned, aligned to
 * their element size; 16-byte aligned rows take the vector path).  The sum,
 * the root and the scaling run in FP32 (squares summed with fused
 * multiply-adds), Y is rounded once to nearest even.  eps must be finite and
 * >= 0.  Y may be X itself (same ld, same element size: in place); any other
 * overlap of Y with X or G is rejected.  m == 0 or d == 0 launches nothing;
 * d <= 2^24.  Asynchronous on `stream`, allocates nothing. */
gemm_status la_rms_norm_run(int64_t m, int64_t d, int32_t x_type, int32_t y_type, const void* X,
                            int64_t ldx, const void* G, void* Y, int64_t ldy, float eps, void* stream);

/* Softmax attention over a batch of (query, key, value) sets -- the
 * computation the Phobos page "Tiles and shared memory" streams over key tiles
 * (section "How long a tile lives": the query tile, its accumulator and the
 * running maximum and sum live through the key loop) -- with the batch of
 * matrices addressed by a third coordinate as on the Tylo.jl page "TMA and
 * Hopper WGMMA" (section "The same storage contract on both sides"):
 *   O[b,i,:] = sum_j p[b,i,j] V[b,j,:] / sum_j p[b,i,j],
 *   p[b,i,j] = exp(scale * Q[b,i,:].K[b,j,:] - max_j(...)).
 * Element (b, i, e) of X lives at X[b * stride_x + i * ld_x + e]. */
typedef struct {
  int64_t batch;               /* >= 0 */
  int64_t sq, sk;              /* query and key counts; sk >= 1 unless batch * sq == 0 */
  int64_t d;                   /* head dimension: 64 or 128 */
  int32_t in_type;             /* GEMM_BF16 or GEMM_F16 (Q, K, V) */
  int32_t out_type;            /* GEMM_F32, GEMM_BF16 or GEMM_F16 (O) */
  int64_t ld_q, ld_k, ld_v, ld_o;                  /* row strides, >= d, multiples of 8 */
  int64_t stride_q, stride_k, stride_v, stride_o;  /* batch strides, >= 0, multiples of 8; entries of O
                                                      are disjoint blocks (stride_o >= (sq-1)*ld_o + d)
                                                      or interleaved rows (stride_o >= d,
                                                      ld_o >= (batch-1)*stride_o + d) */
  float scale;                 /* finite, >= 0; 1/sqrt(d) is the usual choice */
} attn_desc;

/* O for every batch entry and query, on `stream`.  Scores and the softmax run
 * in FP32 (exp through exp2 with scale*log2(e) folded in), P is rounded once
 * to the input type and both the product with V and the running sum use the
 * rounded values, O is rounded once to out_type.  Q, K, V, O are device pointers, 16-byte
 * aligned; O must not overlap Q, K or V, and batch entries of O must not
 * overlap each other (see stride_o).  Row strides times 128 bytes must stay below 2^32.
 * batch * sq == 0 launches nothing. */
gemm_status la_attention_run(const attn_desc* desc, const void* Q, const void* K, const void* V, void* O,
                             void* stream);

/* JSON description of the plan (kernel, tile sizes, grid, LDS layouts and
 * swizzle, alignment class).  Writes at most len bytes including the NUL;
 * returns GEMM_ERR_RESOURCE if it did not fit. */
gemm_status gemm_plan_describe(gemm_plan_t plan, char* buf, size_t len);

/* Element offset, inside one LDS pipeline stage, at which the plan's kernel
 * stores operand element (row, col) of a tile.  operand 0 = A with (row, col)
 * = (m, k) inside the tile; operand 1 = B (and W_gate) with (row, col) = (k, n);
 * operand 2 = W_up.  Host-only; used to check the kernel's LDS image. */
gemm_status gemm_plan_lds_offset(gemm_plan_t plan, int operand, int64_t row, int64_t col,
                                 int64_t* out_elem_offset);

/* Debug: copy tile (tile_m, tile_n) of stage 0 -- the first K block -- of the
 * plan's kernel LDS image to `out` (device memory of at least
 * gemm_plan_lds_stage_bytes bytes), using the kernel's own staging code.
 * A, B (and B2 for gate/up plans, else NULL) are as for a run. */
gemm_status gemm_debug_lds_image(gemm_plan_t plan, const void* A, const void* B, const void* B2,
                                 int64_t tile_m, int64_t tile_n, void* out, void* stream);
gemm_status gemm_plan_lds_stage_bytes(gemm_plan_t plan, int64_t* out_bytes);

/* ---- layout algebra, host only (Tylo.jl "Layouts, storage and ownership") ----
 * Shapes and strides are flat arrays of `rank` int64 values (one mode each).
 * la_layout_eval: offset of the zero-based coordinate `coord` (rank values),
 *   "A layout is a function".
 * la_layout_eval_index: offset of integer index `idx`, split first mode
 *   fastest over the flat modes.
 * la_swizzle_apply: Swizzle{B,M,S} of an element offset, section "Swizzle phase
 *   belongs to the allocation"; GEMM_ERR_INVALID_ARG if the fields overlap.
 * la_tile_plan_offset: shared-tile plan of the Tylo.jl page "TMA and Hopper
 *   WGMMA" (section "The same storage contract on both sides"): element size
 *   1/2/4 bytes, tile (d1, d2), inner axis 1 or 2, swizzle row 128/64/32 bytes;
 *   returns the swizzled element offset of (c1, c2) and the transfer bytes. */
gemm_status la_layout_eval(const int64_t* shape, const int64_t* stride, int rank,
                           const int64_t* coord, int64_t* out_offset);
gemm_status la_layout_eval_index(const int64_t* shape, const int64_t* stride, int rank,
                                 int64_t idx, int64_t* out_offset);
gemm_status la_swizzle_apply(int b, int m, int s, int64_t offset, int64_t* out_offset);
gemm_status la_tile_plan_offset(int elem_bytes, int64_t d1, int64_t d2, int inner_axis,
                                int row_bytes, int64_t c1, int64_t c2,
                                int64_t* out_offset, int64_t* out_transfer_bytes);

/* ---- the same algebra on the pages' own notation, host only ----
 * A layout is written as the Tylo.jl page "Layouts, storage and ownership"
 * writes it: "shape:stride" with nested tuples, e.g. "(16,32):(32,1)" or
 * "((8,4),5):((1,8),128)" (section "Static layout notation").  A coordinate is a
 * nested tuple congruent to the shape, an integer per mode, or one integer
 * index split first mode fastest (section "A layout is a function").  Strings
 * are NUL-terminated; results are written to `out` (at most len bytes with the
 * NUL; GEMM_ERR_RESOURCE if they do not fit).  Malformed text, coordinates
 * outside the domain and tiles that do not divide their mode return
 * GEMM_ERR_INVALID_ARG with a description in gemm_last_error().
 * la_layout_eval_str: offset of `coord`.
 * la_layout_tile_str: tile() with one extent per flat top-level mode: mode i
 *   of extent s and stride d becomes (tile[i], s / tile[i]) : (d, tile[i] * d).
 * la_layout_coalesce_str: coalesce(): unit modes dropped, (s0:d0)(s1:d1)
 *   merged when d1 = s0 * d0, the same map on the linear domain.
 * la_layout_permute_str: permutedims: the top-level modes reversed.
 * la_layout_cosize_str: 1 + the largest offset (non-negative strides).
 * la_view_window_eval: Swizzle{b,m,s} o layout, windowed at `origin` with
 *   `extent` (rank values, one per top-level mode, inside the parent's domain;
 *   section "Swizzle phase belongs to the allocation": the window keeps the
 *   parent's map and origin), evaluated at `coord` (rank values). */
gemm_status la_layout_eval_str(const char* layout, const char* coord, int64_t* out_offset);
gemm_status la_layout_tile_str(const char* layout, const int64_t* tile, int32_t rank, char* out, size_t len);
gemm_status la_layout_coalesce_str(const char* layout, char* out, size_t len);
gemm_status la_layout_permute_str(const char* layout, char* out, size_t len);
gemm_status la_layout_cosize_str(const char* layout, int64_t* out_cosize);
gemm_status la_view_window_eval(int32_t b, int32_t m, int32_t s, const char* layout, const int64_t* origin,
                                const int64_t* extent, int32_t rank, const int64_t* coord, int64_t* out_offset);

const char* gemm_status_string(gemm_status s);
const char* gemm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LA_GEMM_H */
