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
//    the source side as in the GEMM), each in a ring of two slots, one barrier
//    per tile.
//  * Software pipeline across key tiles: while tile t's probabilities are
//    formed (vector ALU), the scores of tile t+1 run on the matrix cores, and
//    tile t+1's maximum is taken after tile t's product with V.  K(t+1) and
//    V(t) are resident together, so K and V have rings of their own: after the
//    barrier that opens tile t, V(t+1) goes into the slot V(t-1) left and
//    K(t+2) into the slot K(t) left (both read completely before that
//    barrier).  The arithmetic and its order are those of the plain loop
//    (scores, lazy reference update, probabilities, sum, product per tile), so
//    the result is the same bit for bit; the overlap took the 4096-key
//    workload from 570-605 to 490-530 us on the boxes measured.
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
#include <type_traits>

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
  constexpr int KE = BC * D;
  constexpr int CHUNKS = KE / 512 / NW;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_raw[4 * KE];
  AT_LDS uint16_t* lds = (AT_LDS uint16_t*)lds_raw;      // K slots 0, 1, then V slots 0, 1

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

  u32x4 qf[DS];
  {
    const int64_t q = q0 + c;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[s] = q < a.sq ? *reinterpret_cast<const u32x4*>(Qz + q * a.ldq + 16 * s + 8 * h) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t ofk[CHUNKS], ofv[CHUNKS];
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int P = (wave * CHUNKS + i) * 512 + lane * 8;
    const int Lk = swz<Cfg::KB, Cfg::KM, Cfg::KS>(P);
    const int Lv = swz<Cfg::VB, Cfg::VM, Cfg::VS>(P);
    ofk[i] = uint32_t(Lk / D) * uint32_t(a.ldk) * 2u + uint32_t(Lk % D) * 2u;
    ofv[i] = uint32_t(Lv / D) * uint32_t(a.ldv) * 2u + uint32_t(Lv % D) * 2u;
  }
  // one operand tile (K: kv = 0, V: kv = 1) of key tile t into its slot
  auto issue1 = [&](int kv, int t, int slot) {
    const int64_t kbase = int64_t(t) * BC;
    const int64_t ld = kv ? a.ldv : a.ldk;
    const uint16_t* src = (kv ? Vz : Kz) + kbase * ld;
    AT_LDS uint16_t* dst = lds + (2 * kv + slot) * KE + wave * CHUNKS * 512;
    if (kbase + BC <= a.sk) {
#pragma unroll
      for (int i = 0; i < CHUNKS; ++i) dma16(src, kv ? ofv[i] : ofk[i], lds_address(dst + i * 512));
      return;
    }
    const int last = int(a.sk - 1 - kbase);
    const uint32_t ld2 = uint32_t(ld) * 2u;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int P = (wave * CHUNKS + i) * 512 + lane * 8;
      const int L = kv ? swz<Cfg::VB, Cfg::VM, Cfg::VS>(P) : swz<Cfg::KB, Cfg::KM, Cfg::KS>(P);
      const int r = L / D < last ? L / D : last;
      dma16(src, uint32_t(r) * ld2 + uint32_t(L % D) * 2u, lds_address(dst + i * 512));
    }
  };

  const uint32_t kaddr0 = uint32_t(swz<Cfg::KB, Cfg::KM, Cfg::KS>(c * D + 8 * h)) * 2u;
  const int e4 = (lane >> 2) & 3;
  const uint32_t vaddr0 = uint32_t(swz<Cfg::VB, Cfg::VM, Cfg::VS>((4 * h + e4) * D + 16 * ((lane >> 4) & 1) + 4 * (lane & 3))) * 2u;

  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
  float m = -__builtin_inff(), l = 0.0f;

  // S^T = K Q^T of the tile in K slot `slot`
  auto scores = [&](int slot, f32x16 (&s)[2]) {
    const AT_LDS char* ksb = reinterpret_cast<const AT_LDS char*>(lds + slot * KE);
    uint32_t ka = kaddr0;
    asm volatile("" : "+v"(ka));
    u32x4 kf[DS][2];
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[st][kb] = *reinterpret_cast<const AT_LDS u32x4*>(ksb + (ka ^ uint32_t(32 * st)) + kb * 32 * D * 2);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_32x32x16<TI>(kf[st][kb], qf[st], s[kb]);
  };
  // keys past the end of tile t score -inf
  auto mask = [&](int t, f32x16 (&s)[2]) {
    const int64_t remaining = a.sk - int64_t(t) * BC;
    if (remaining < BC) {
      asm volatile("" ::: "memory");
      const int rem = int(remaining);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3) >= rem) s[kb][r] = -__builtin_inff();
    }
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return halves_max(mx) * a.scale_log2;
  };
  // lazy reference maximum: rescale acc and l only when the tile's maximum exceeds m by more than 8
  auto update_ref = [&](float m_tile) {
    if (__any(m_tile > m + 8.0f)) {
      const float m_new = m_tile > m + 8.0f ? m_tile : m;
      const float corr = __builtin_amdgcn_exp2f(m - m_new);
      l *= corr;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] *= corr;
      m = m_new;
    }
  };
  // probabilities of one 32-key block, packed as the MFMA operands of two 16-key steps; returns their sum
  auto probs = [&](f32x16& sb, u32x4& p0, u32x4& p1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[r], a.scale_log2, -m));
    p0 = u32x4{pack2<TI>(sb[0], sb[1]), pack2<TI>(sb[2], sb[3]), pack2<TI>(sb[4], sb[5]), pack2<TI>(sb[6], sb[7])};
    p1 = u32x4{pack2<TI>(sb[8], sb[9]), pack2<TI>(sb[10], sb[11]), pack2<TI>(sb[12], sb[13]), pack2<TI>(sb[14], sb[15])};
    float sum = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) sum = dot2_ones<TI>(p0[w2], sum);
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) sum = dot2_ones<TI>(p1[w2], sum);
    return sum;
  };
  // O^T += V^T P^T over the 16-key steps u0, u0 + 1 of the tile in V slot `slot`
  auto pv = [&](int slot, int u0, const u32x4& p0, const u32x4& p1) {
    const AT_LDS char* vsb = reinterpret_cast<const AT_LDS char*>(lds + (2 + slot) * KE);
    uint32_t va = vaddr0;
    asm volatile("" : "+v"(va));
#pragma unroll
    for (int du = 0; du < 2; ++du) {
      const int u = u0 + du;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const AT_LDS char* vp = vsb + (va ^ uint32_t(64 * b)) + 16 * u * D * 2;
        const i16x4_a lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AT_LDS i16x4_a*)(vp));
        const i16x4_a hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((AT_LDS i16x4_a*)(vp + 8 * D * 2));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        acc[b] = mfma_32x32x16<TI>(u32x4{l2.x, l2.y, h2.x, h2.y}, du ? p1 : p0, acc[b]);
      }
    }
  };

  // prologue: K(0), V(0), K(1) in flight; wait for K(0) only, then tile 0's scores and reference
  const int nt = int((a.sk + BC - 1) / BC);
  issue1(0, 0, 0);
  issue1(1, 0, 0);
  if (nt > 1) {
    issue1(0, 1, 1);
    __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | ((2 * CHUNKS) & 0xF) | (((2 * CHUNKS) >> 4) << 14));  // K(0) landed
  } else {
    __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | (CHUNKS & 0xF) | ((CHUNKS >> 4) << 14));
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  f32x16 sA[2], sB[2];
  scores(0, sA);
  mask(0, sA);
  update_ref(tile_max(sA));

  // One key tile t: s holds its scores (reference already updated); with a next tile, sn receives
  // tile t+1's scores, computed while tile t's first half of probabilities is formed.  Whether a
  // next tile exists is a compile-time property of each call (the last tile is peeled), so the
  // scores and the probabilities sit in one basic block, where the compiler interleaves them.
  auto step = [&](int t, f32x16 (&s)[2], f32x16 (&sn)[2], auto has_next) {
    constexpr bool NEXT = decltype(has_next)::value;
    barrier_after_loads();                    // V(t) and K(t+1) in LDS; tile t-1 and S(t) fully read
    if constexpr (NEXT) {
      issue1(1, t + 1, (t + 1) & 1);
      if (t + 2 < nt) issue1(0, t + 2, t & 1);
    }
    u32x4 p0, p1, p2, p3;
    float sum;
    if constexpr (NEXT) scores((t + 1) & 1, sn);
    sum = probs(s[0], p0, p1);
    pv(t & 1, 0, p0, p1);
    sum = sum + probs(s[1], p2, p3);
    l += halves_sum(sum);
    pv(t & 1, 2, p2, p3);
    if constexpr (NEXT) {
      mask(t + 1, sn);
      update_ref(tile_max(sn));
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  // unrolled by two so that the score registers of tiles t and t+1 trade roles without copies
  int t = 0;
  for (; t + 2 < nt; t += 2) {
    step(t, sA, sB, yes{});
    step(t + 1, sB, sA, yes{});
  }
  if (t + 1 < nt) {
    step(t, sA, sB, yes{});
    step(t + 1, sB, sA, no{});
  } else {
    step(t, sA, sB, no{});
  }

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
