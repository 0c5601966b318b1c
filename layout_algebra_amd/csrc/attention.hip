// Streaming softmax attention for gfx950, O = softmax(scale * Q K^T) V per
// batch entry, the computation the Phobos page "Tiles and shared memory" uses
// to illustrate tile lifetimes (section "How long a tile lives"): a query tile,
// its accumulator and the running maximum and sum live through the whole key
// loop; key and value tiles live for one iteration; the accumulator is divided
// by the running sum at the end.
//
// MI355X mapping (one workgroup = 4 waves = 128 queries, 2 workgroups per CU):
//  * Each wave owns 32 queries.  Their Q^T fragments stay in registers for the
//    whole key loop (global -> registers once).
//  * Key and value tiles of 64 rows are staged global -> LDS with direct loads
//    (global_load_lds_dwordx4, 1 KB per wave instruction, swizzle applied on
//    the source side as in the GEMM), two stages, one barrier per tile.
//  * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16): in the
//    32x32 result layout a lane holds 16 keys of ONE query, so the row maximum
//    and sum are in-lane reductions plus one swap with the other half-wave,
//    and the rescaling of the output accumulator (also kept transposed,
//    O^T = V^T P^T) is a per-lane multiply.
//  * P^T feeds the second product straight from registers: the key order of
//    the 32x32 result layout is used as the MFMA k order, and the V^T
//    fragments are read in that same key order with transposing LDS reads
//    (ds_read_b64_tr_b16: 4 consecutive keys of one head-dimension column per
//    lane), so no shuffle or LDS round trip is needed for P.
//  * exp goes through exp2 with scale * log2(e) folded into one fused
//    multiply-add per score (scale >= 0); the probabilities are rounded once
//    to the input type, and both the product with V and the running sum use
//    those rounded values (the sum through packed dot products).  The reference maximum is updated lazily (only when a tile
//    exceeds it by more than 8 in log2 units, a factor 256), which skips the
//    rescaling of the output accumulator on most tiles; the result acc / sum
//    does not depend on the reference.
//  * Keys past the end of the sequence read the last valid key and value row
//    (no out-of-bounds access), are left out of the maximum and get
//    probability 0; queries past the end compute on zeros and are not stored.
//  * Workgroups are numbered so that each XCD takes a contiguous run of
//    (batch entry, query tile) pairs: the query tiles of one batch entry
//    share its K and V through one L2.
// LDS bank conflicts: K tiles use Swizzle{4,3,4} (D = 128) / {3,3,4} (D = 64)
// for 16-byte fragment reads of 16 consecutive keys; V tiles use
// Swizzle{2,5,2} for the transposing reads of 4 keys x 16 columns.
#include "attention.hpp"
#include "kernel_common.hpp"

namespace lak {
namespace {

#define AT_LDS __attribute__((address_space(3)))
typedef short i16x4_a __attribute__((ext_vector_type(4)));

template <int D>
struct AttnCfg;
template <>
struct AttnCfg<128> {
  static constexpr int KB = 4, KM = 3, KS = 4;
  static constexpr int VB = 2, VM = 5, VS = 2;
};
template <>
struct AttnCfg<64> {
  static constexpr int KB = 3, KM = 3, KS = 4;
  static constexpr int VB = 2, VM = 5, VS = 2;
};

constexpr int BR = 128, BC = 64, NW = 4, NTHREADS = NW * 64;
static_assert(NTHREADS == ATTN_THREADS, "the launch checks size the grid with ATTN_THREADS");

// One direct load: 64 lanes x 16 bytes from base + voff (bytes) into the KB of
// LDS at lds_addr (wave-uniform, through M0).  Inline assembly keeps the
// compiler's wait-count pass from stalling later LDS reads on it; completion
// is waited for explicitly before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(const uint16_t* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const AT_LDS uint16_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ void barrier_after_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct loads have landed
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __bf16 bf16x2_a __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_a __attribute__((ext_vector_type(2)));

// Two FP32 values rounded to nearest even and packed (one conversion instruction for bf16).
template <class TI>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<InBF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_a{static_cast<__bf16>(lo), static_cast<__bf16>(hi)});
}
template <>
__device__ __forceinline__ uint32_t pack2<InF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2_a{static_cast<_Float16>(lo), static_cast<_Float16>(hi)});
}

// c + x.lo + x.hi for a packed pair of the input type (one dot-product instruction).
template <class TI>
__device__ __forceinline__ float dot2_ones(uint32_t x, float c);
template <>
__device__ __forceinline__ float dot2_ones<InBF16>(uint32_t x, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_a, x), bf16x2_a{(__bf16)1.0f, (__bf16)1.0f}, c, false);
}
template <>
__device__ __forceinline__ float dot2_ones<InF16>(uint32_t x, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_a, x), f16x2_a{(_Float16)1.0f, (_Float16)1.0f}, c, false);
}

// Combine every lane with its partner in the other half-wave (lane l ^ 32) without LDS:
// v_permlane32_swap with the same register on both sides returns lanes 0-31 twice in one
// result and lanes 32-63 twice in the other, so f(first, second) is f(x[l], x[l ^ 32]) up to
// the order of the operands (exact for the maximum and for a two-term sum).
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class TO>
__device__ __forceinline__ void store4(void* O, int64_t off, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<OutF32>(void* O, int64_t off, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(static_cast<float*>(O) + off) = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<OutBF16>(void* O, int64_t off, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + off) = u32x2{pack2<InBF16>(a, b), pack2<InBF16>(c, d)};
}
template <>
__device__ __forceinline__ void store4<OutF16>(void* O, int64_t off, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + off) = u32x2{pack2<InF16>(a, b), pack2<InF16>(c, d)};
}

template <class TI, class TO, int D>
__global__ void __launch_bounds__(NTHREADS, 2) attn_fwd_kernel(const AttnArgs a) {
  using Cfg = AttnCfg<D>;
  constexpr int KE = BC * D;                   // elements of one K (or V) tile
  constexpr int STAGE = 2 * KE;
  constexpr int CHUNKS = KE / 512 / NW;        // 1 KB direct loads per wave per tile and operand
  constexpr int DS = D / 16;                   // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;                   // 32-row blocks of O^T
  static_assert(CHUNKS * 512 * NW == KE, "tile must split into whole KB per wave");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[2 * STAGE];
  AT_LDS uint16_t* lds = (AT_LDS uint16_t*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;
  const int id = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t z = id / a.q_tiles;
  const int64_t q0 = int64_t(id % a.q_tiles) * BR + wave * 32;
  const uint16_t* Qz = a.Q + z * a.bq;
  const uint16_t* Kz = a.K + z * a.bk;
  const uint16_t* Vz = a.V + z * a.bv;

  // Q^T fragments of this wave's 32 queries: lane (c, h) holds query q0 + c,
  // head-dimension elements 16 s + 8 h .. + 7 for every k-step s.
  u32x4 qf[DS];
  {
    const int64_t q = q0 + c;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[s] = q < a.sq ? *reinterpret_cast<const u32x4*>(Qz + q * a.ldq + 16 * s + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }

  // Direct loads: the lane that fills physical element P of a tile fetches
  // logical element Sw(P) = key * D + d.  A full tile uses the byte offsets
  // computed here once; the last tile, when partial, recomputes them with rows
  // past the end clamped to the last key / value row.  Offsets stay 32-bit:
  // the host guarantees 128 * ld < 2^32.
  uint32_t ofk[CHUNKS], ofv[CHUNKS];
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int P = (wave * CHUNKS + i) * 512 + lane * 8;
    const int Lk = swz<Cfg::KB, Cfg::KM, Cfg::KS>(P);
    const int Lv = swz<Cfg::VB, Cfg::VM, Cfg::VS>(P);
    ofk[i] = uint32_t(Lk / D) * uint32_t(a.ldk) * 2u + uint32_t(Lk % D) * 2u;
    ofv[i] = uint32_t(Lv / D) * uint32_t(a.ldv) * 2u + uint32_t(Lv % D) * 2u;
  }
  auto issue = [&](int t, int st) {
    const int64_t kbase = int64_t(t) * BC;
    const uint16_t* kb = Kz + kbase * a.ldk;
    const uint16_t* vb = Vz + kbase * a.ldv;
    AT_LDS uint16_t* dst = lds + st * STAGE + wave * CHUNKS * 512;
    if (kbase + BC <= a.sk) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) dma16(kb, ofk[i], lds_address(dst + i * 512));
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) dma16(vb, ofv[i], lds_address(dst + KE + i * 512));
      return;
    }
    const int last = int(a.sk - 1 - kbase);     // rows past the end repeat the last key / value
    const uint32_t ldk2 = uint32_t(a.ldk) * 2u, ldv2 = uint32_t(a.ldv) * 2u;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int P = (wave * CHUNKS + i) * 512 + lane * 8;
      const int Lk = swz<Cfg::KB, Cfg::KM, Cfg::KS>(P);
      const int rk = Lk / D < last ? Lk / D : last;
      dma16(kb, uint32_t(rk) * ldk2 + uint32_t(Lk % D) * 2u, lds_address(dst + i * 512));
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int P = (wave * CHUNKS + i) * 512 + lane * 8;
      const int Lv = swz<Cfg::VB, Cfg::VM, Cfg::VS>(P);
      const int rv = Lv / D < last ? Lv / D : last;
      dma16(vb, uint32_t(rv) * ldv2 + uint32_t(Lv % D) * 2u, lds_address(dst + KE + i * 512));
    }
  };

  // LDS fragment addresses (bytes within a tile).  The XOR swizzles of both
  // tiles take their source bits from the key row and only flip bits that
  // the k-step (K tile) or the 32-column block (V tile) occupies, so
  //   K: Sw(row D + 16 s + 8 h) = Sw(row D + 8 h) ^ (16 s),  row = 32 kb + c
  //   V: Sw(key D + 32 b + x)   = Sw(key0 D + x) ^ (32 b) + (key - key0) D
  // with key0 = 4 h + e the lane's first key: one base per lane and operand,
  // the rest is an XOR and an immediate offset per read.
  const uint32_t kaddr0 = uint32_t(swz<Cfg::KB, Cfg::KM, Cfg::KS>(c * D + 8 * h)) * 2u;
  const int e4 = (lane >> 2) & 3;
  const uint32_t vaddr0 = uint32_t(swz<Cfg::VB, Cfg::VM, Cfg::VS>((4 * h + e4) * D + 16 * ((lane >> 4) & 1) + 4 * (lane & 3))) * 2u;

  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
  float m = -__builtin_inff(), l = 0.0f;

  const int nt = int((a.sk + BC - 1) / BC);
  issue(0, 0);
  for (int t = 0; t < nt; ++t) {
    barrier_after_loads();                     // tile t is in LDS; every wave is done with tile t - 1
    if (t + 1 < nt) issue(t + 1, (t + 1) & 1);
    const AT_LDS uint16_t* ks = lds + (t & 1) * STAGE;
    const AT_LDS uint16_t* vs = ks + KE;
    const AT_LDS char* ksb = reinterpret_cast<const AT_LDS char*>(ks);
    const AT_LDS char* vsb = reinterpret_cast<const AT_LDS char*>(vs);
    uint32_t ka = kaddr0, va = vaddr0;
    asm volatile("" : "+v"(ka), "+v"(va));     // per-read addresses are formed here, not kept live

    // S^T = K Q^T: two 32-key blocks x 32 queries.  All K fragments of the tile
    // are requested before the first MFMA, so LDS latency is paid once per tile.
    u32x4 kf[DS][2];
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[s][kb] = *reinterpret_cast<const AT_LDS u32x4*>(ksb + (ka ^ uint32_t(32 * s)) + kb * 32 * D * 2);
    __builtin_amdgcn_sched_barrier(0);         // keep the reads ahead of the MFMAs (the scheduler would sink them)
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma_32x32x16<TI>(kf[s][kb], qf[s], sacc[kb]);
    }

    // Online softmax for query c: register r of block kb is key
    // kb * 32 + 8 (r / 4) + 4 h + r % 4 of this tile; the other half-wave holds the rest.
    // Scores stay raw; with c = scale * log2(e) >= 0, max(c s) = c max(s) and
    // p = exp2(c s - m) is one fused multiply-add and one exp2 per score.
    // Keys past the end (only in the last tile) score -inf: they drop out of the
    // maximum and exp2(k * -inf - m) = 0 (k > 0; a zero scale is passed as the
    // smallest normal float, which leaves every valid probability at exactly 1).
    const int64_t remaining = a.sk - int64_t(t) * BC;
    if (remaining < BC) {
      asm volatile("" ::: "memory");           // a real branch: full tiles skip the selects below
      const int rem = int(remaining);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= rem) sacc[kb][r] = -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = halves_max(mx);
    // Lazy reference maximum (log2 units): it moves only when the tile's maximum
    // exceeds it by more than 8, so probabilities stay <= 2^8 and the rescaling
    // of the accumulator and the running sum is skipped for most tiles; the
    // quotient acc / l does not depend on the reference.
    const float m_tile = mx * a.scale_log2;
    if (__any(m_tile > m + 8.0f)) {
      const float m_new = m_tile > m + 8.0f ? m_tile : m;
      const float corr = __builtin_amdgcn_exp2f(m - m_new);   // 0 on the first tile (m = -inf)
      l *= corr;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] *= corr;
      m = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], a.scale_log2, -m));
    // P^T as MFMA B operands (16-key step u: score registers 8 (u % 2) .. + 7 of
    // block u / 2), rounded to the input type; the running sum adds the same
    // rounded values, two per dot-product instruction, so numerator and
    // denominator see identical weights.
    u32x4 pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x16& sp = sacc[u >> 1];
      const int rr = (u & 1) * 8;
      pf[u] = u32x4{pack2<TI>(sp[rr + 0], sp[rr + 1]), pack2<TI>(sp[rr + 2], sp[rr + 3]),
                    pack2<TI>(sp[rr + 4], sp[rr + 5]), pack2<TI>(sp[rr + 6], sp[rr + 7])};
    }
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) sum = dot2_ones<TI>(pf[u][w2], sum);
    l += halves_sum(sum);

    // O^T += V^T P^T over four 16-key steps; slot e of the lane's 8 k values is
    // key 16 u + 8 (e / 4) + 4 h + e % 4, the order of the score registers.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const AT_LDS char* vp = vsb + (va ^ uint32_t(64 * b)) + 16 * u * D * 2;
        const i16x4_a lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AT_LDS i16x4_a*)(vp));
        const i16x4_a hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AT_LDS i16x4_a*)(vp + 8 * D * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        acc[b] = mfma_32x32x16<TI>(u32x4{l2.x, l2.y, h2.x, h2.y}, pf[u], acc[b]);
      }
    }
  }

  // O[q, d] = acc / l: register r of block b is d = 32 b + 8 (r / 4) + 4 h + r % 4.
  const int64_t q = q0 + c;
  if (q < a.sq) {
    const float inv = 1.0f / l;
    const int64_t row = z * a.bo + q * a.ldo;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * b + 8 * g4 + 4 * h;
        store4<TO>(a.O, row + d0, acc[b][4 * g4] * inv, acc[b][4 * g4 + 1] * inv, acc[b][4 * g4 + 2] * inv,
                   acc[b][4 * g4 + 3] * inv);
      }
  }
}

template <class TI, class TO, int D>
hipError_t go(const AttnArgs& a, hipStream_t s) {
  const int64_t blocks = a.batch * a.q_tiles;
  hipLaunchKernelGGL((attn_fwd_kernel<TI, TO, D>), dim3(static_cast<unsigned>(blocks)), dim3(NTHREADS), 0, s, a);
  return hipGetLastError();
}

template <class TI, int D>
hipError_t by_out(const AttnArgs& a, int out_kind, hipStream_t s) {
  switch (out_kind) {
    case OUT_F32: return go<TI, OutF32, D>(a, s);
    case OUT_BF16: return go<TI, OutBF16, D>(a, s);
    case OUT_F16: return go<TI, OutF16, D>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <class TI>
hipError_t by_d(const AttnArgs& a, int d, int out_kind, hipStream_t s) {
  if (d == 128) return by_out<TI, 128>(a, out_kind, s);
  if (d == 64) return by_out<TI, 64>(a, out_kind, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int d, int in_kind, int out_kind, hipStream_t stream) {
  if (a.batch * a.q_tiles == 0) return hipSuccess;
  return in_kind == IN_BF16 ? by_d<InBF16>(a, d, out_kind, stream) : by_d<InF16>(a, d, out_kind, stream);
}

}  // namespace lak
