// Attention launch interface (see attention.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace lak {

struct AttnArgs {
  const uint16_t* Q;     // [batch][sq][d], row stride ldq, batch stride bq (elements)
  const uint16_t* K;     // [batch][sk][d]
  const uint16_t* V;     // [batch][sk][d]
  void* O;               // [batch][sq][d] in the output type
  int64_t batch, sq, sk;
  int64_t ldq, ldk, ldv, ldo;
  int64_t bq, bk, bv, bo;
  float scale_log2;      // scale * log2(e): scores go through exp2
  int q_tiles;           // ceil(sq / 128)
};

// Threads per workgroup; one workgroup per 128 queries of one batch entry.
constexpr int ATTN_THREADS = 256;

// in_kind: IN_BF16 or IN_F16; out_kind: OUT_F32, OUT_BF16 or OUT_F16; d: 64 or 128.
// Rows of Q, K, V, O start on 16 bytes (checked by the caller).
hipError_t launch_attention(const AttnArgs& a, int d, int in_kind, int out_kind, hipStream_t stream);

}  // namespace lak
