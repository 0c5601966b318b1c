// GEMM planner.  Host only; touches no device memory.
//
// Steps, in order (constructors check domains before anything is launched, as
// the Tylo.jl page "Layouts, storage and ownership" requires in section "Swizzle
// phase belongs to the allocation"):
//   1. validate the descriptor (sizes, leading dimensions, dtypes, flags);
//   2. derive the alignment class, which the run checks pointers against:
//      16 bytes when every row start is 16-byte aligned, else the element
//      (Tylo.jl, section "Three representations, three addressing rules":
//      accesses follow the declared alignment of pointer and strides).  The
//      general kernel still moves 16 bytes per load for element-aligned rows
//      longer than 8 elements, since gfx950 executes unaligned vector loads;
//      only shorter rows fall back to element loads;
//   3. choose a kernel and its tile grid;
//   4. build each operand's LDS map as Swizzle o Layout in the operand's own
//      mathematical coordinates (B in (K, N), section "Three representations,
//      three addressing rules") and check it: injective, cosize inside its
//      block, block bases on the swizzle period (the allocation fixes the
//      phase), total LDS within the 160 KiB a gfx950 workgroup may use;
//   5. check the copy plans (every 16-byte LDS vector written exactly once,
//      contiguous and aligned; section "Plans describe work, callers establish
//      readiness") and the MFMA ownership (every C element of the tile owned by
//      exactly one (wave, lane, register));
//   6. build each operand's global view with tile() (section "A layout is a
//      function": tile splits a mode into (within-tile, tile-index)), derive the
//      global elements one wave instruction of the copy plan reads, check them
//      against the kernel's per-lane chunk map, and reduce that copy layout with
//      coalesce() (coalescing is host-side planning) to its contiguous runs;
//   7. model each operand's LDS ring as one allocation and every stage as a
//      window of it (section "Swizzle phase belongs to the allocation": a window
//      keeps the parent's map and origin), checking that each stage sees the same
//      swizzled map as the block plan;
//   8. check the epilogue's store plan on every class of tile (interior, last
//      row of tiles, last column, corner): every element of C inside [0,M)x[0,N)
//      written exactly once, nothing outside it; and reduce one store
//      instruction to its contiguous runs.
#include "planner.hpp"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <sstream>
#include <vector>

namespace plan {
namespace {

constexpr int64_t kMaxLdsBytes = 163840;   // gfx950 per-workgroup LDS

// K blocks a workgroup keeps loading ahead of the one it multiplies: the
// general kernel's register sets, or the direct-load kernels' LDS ring less
// the stage being read.
int prefetch_blocks(const gemm_plan_s& p) {
  switch (p.kid) {
    case lak::KID_TILED_64_P3: return 3;
    case lak::KID_TILED_64: return p.vec != 1 && !p.gate_up ? 2 : 1;
    case lak::KID_TILED_128:
    case lak::KID_TILED_F32: return 1;
    default: return p.shape.stages - 1;
  }
}

bool fail(std::string* err, const std::string& msg);

// The kernel's copy of one block of an operand: for wave instruction `ins`, the
// tile coordinates (row, col) of the chunk each lane moves (8 16-bit or 4
// binary32 elements, running along the operand's contiguous direction).
struct CopyChunk { int64_t row, col; };

bool fast_kid(int kid) {
  return kid == lak::KID_FAST_256 || kid == lak::KID_FAST_GU || kid == lak::KID_FAST_256_KM || kid == lak::KID_FAST_GU_KM ||
         kid == lak::KID_FAST_256_AT || kid == lak::KID_FAST_GU_AT || kid == lak::KID_FAST_F8 || kid == lak::KID_FAST_GU_F8 ||
         kid == lak::KID_FAST_128 || kid == lak::KID_FAST_128_KM || kid == lak::KID_FAST_F8_128 ||
         kid == lak::KID_FAST_128_KM64 || kid == lak::KID_FAST_128_K64 || kid == lak::KID_FAST_F8_128_K64;
}

bool skinny_kid(int kid) {
  return kid == lak::KID_SKINNY_16 || kid == lak::KID_SKINNY_32 || kid == lak::KID_SKINNY_64 ||
         kid == lak::KID_SKINNY_16_KM || kid == lak::KID_SKINNY_32_KM || kid == lak::KID_SKINNY_64_KM ||
         kid == lak::KID_SKINNY_F8 || kid == lak::KID_SKINNY_F8_32 || kid == lak::KID_SKINNY_F8_64 ||
         kid == lak::KID_SKINNY_128 || kid == lak::KID_SKINNY_128_KM || kid == lak::KID_SKINNY_F8_128;
}

bool fail(std::string* err, const std::string& msg) {
  if (err) *err = msg;
  return false;
}

// 16-byte copy plan of an A block: thread t, slot j covers (row, 8-element chunk).
bool check_copy_a(const gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  const int chunks = s.bm * s.bk / 8;
  if (chunks % s.threads) return fail(err, "A block does not split evenly into 16-byte vectors per thread");
  std::vector<int> hits(static_cast<size_t>(s.bm) * s.bk, 0);
  for (int t = 0; t < s.threads; ++t) {
    for (int j = 0; j < chunks / s.threads; ++j) {
      const int idx = t + s.threads * j;
      const int row = idx / (s.bk / 8), ch = idx % (s.bk / 8);
      const int64_t o0 = p.lds_a.at({row, ch * 8});
      if (o0 % 8) return fail(err, "A copy destination is not 16-byte aligned");
      for (int e = 0; e < 8; ++e) {
        const int64_t o = p.lds_a.at({row, ch * 8 + e});
        if (o != o0 + e) return fail(err, "A copy destination is not contiguous");
        if (hits[o]++) return fail(err, "A copy plan writes an LDS element twice");
      }
    }
  }
  for (int h : hits)
    if (h != 1) return fail(err, "A copy plan leaves an LDS element unwritten");
  return true;
}

// A stored [K, M] in the general kernel: thread t, slot j covers (row k,
// 8-element M chunk), written as one 16-byte vector (like N-contiguous B).
bool check_copy_a_t(const gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  const int chunks = s.bk * s.bm / 8;
  if (chunks % s.threads) return fail(err, "A block does not split evenly into 16-byte vectors per thread");
  std::vector<int> hits(static_cast<size_t>(s.bm) * s.bk, 0);
  for (int t = 0; t < s.threads; ++t) {
    for (int j = 0; j < chunks / s.threads; ++j) {
      const int idx = t + s.threads * j;
      const int k = idx / (s.bm / 8), mc = idx % (s.bm / 8);
      const int64_t o0 = p.lds_a.at({mc * 8, k});
      if (o0 % 8) return fail(err, "A copy destination is not 16-byte aligned");
      for (int e = 0; e < 8; ++e) {
        const int64_t o = p.lds_a.at({mc * 8 + e, k});
        if (o != o0 + e) return fail(err, "A copy destination is not contiguous along M");
        if (hits[o]++) return fail(err, "A copy plan writes an LDS element twice");
      }
    }
  }
  for (int h : hits)
    if (h != 1) return fail(err, "A copy plan leaves an LDS element unwritten");
  return true;
}

// N-contiguous B in the general kernel: thread t, slot j covers (row k,
// 8-element N chunk), written as one 16-byte vector.
bool check_copy_b(const gemm_plan_s& p, const la::View& v, std::string* err) {
  const auto& s = p.shape;
  const int chunks = s.bk * s.bn / 8;
  if (chunks % s.threads) return fail(err, "B block does not split evenly into 16-byte vectors per thread");
  std::vector<int> hits(static_cast<size_t>(s.bn) * s.bk, 0);
  for (int t = 0; t < s.threads; ++t) {
    for (int j = 0; j < chunks / s.threads; ++j) {
      const int idx = t + s.threads * j;
      const int k = idx / (s.bn / 8), nc = idx % (s.bn / 8);
      const int64_t o0 = v.at({k, nc * 8});
      if (o0 % 8) return fail(err, "B copy destination is not 16-byte aligned");
      for (int e = 0; e < 8; ++e) {
        const int64_t o = v.at({k, nc * 8 + e});
        if (o != o0 + e) return fail(err, "B copy destination is not contiguous along N");
        if (hits[o]++) return fail(err, "B copy plan writes an LDS element twice");
      }
    }
  }
  for (int h : hits)
    if (h != 1) return fail(err, "B copy plan leaves an LDS element unwritten");
  return true;
}

// K-major B in the general kernel: like A, thread t, slot j covers
// (column n, 8-element K chunk), written as one 16-byte vector.
bool check_copy_b_rows(const gemm_plan_s& p, const la::View& v, std::string* err) {
  const auto& s = p.shape;
  const int chunks = s.bn * s.bk / 8;
  if (chunks % s.threads) return fail(err, "B block does not split evenly into 16-byte vectors per thread");
  std::vector<int> hits(static_cast<size_t>(s.bn) * s.bk, 0);
  for (int t = 0; t < s.threads; ++t) {
    for (int j = 0; j < chunks / s.threads; ++j) {
      const int idx = t + s.threads * j;
      const int n = idx / (s.bk / 8), ch = idx % (s.bk / 8);
      const int64_t o0 = v.at({ch * 8, n});
      if (o0 % 8) return fail(err, "B copy destination is not 16-byte aligned");
      for (int e = 0; e < 8; ++e) {
        const int64_t o = v.at({ch * 8 + e, n});
        if (o != o0 + e) return fail(err, "B copy destination is not contiguous along K");
        if (hits[o]++) return fail(err, "B copy plan writes an LDS element twice");
      }
    }
  }
  for (int h : hits)
    if (h != 1) return fail(err, "B copy plan leaves an LDS element unwritten");
  return true;
}

// Direct global -> LDS copy: wave instruction `blk` writes the contiguous
// kilobyte [512 blk, 512 blk + 512) (elements) with lane l at 8 l.  The lane's
// 8 elements must be 8 consecutive elements of one row of the operand as it
// sits in global memory (K for A, N for B), so one 16-byte load feeds them.
bool check_copy_direct(const la::View& v, int64_t rows, int64_t cols, bool contiguous_in_cols, const char* name,
                       std::string* err) {
  const int64_t n = rows * cols;
  if (n % 512) return fail(err, std::string(name) + " block is not a whole number of kilobytes");
  std::vector<int64_t> inv(n, -1);   // physical offset -> row * cols + col
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const int64_t o = v.at({r, c});
      if (o < 0 || o >= n || inv[o] != -1) return fail(err, std::string(name) + " LDS map is not a bijection onto its block");
      inv[o] = r * cols + c;
    }
  for (int64_t p = 0; p < n; p += 8) {
    const int64_t r0 = inv[p] / cols, c0 = inv[p] % cols;
    for (int e = 1; e < 8; ++e) {
      const int64_t r = inv[p + e] / cols, c = inv[p + e] % cols;
      const bool ok = contiguous_in_cols ? (r == r0 && c == c0 + e) : (c == c0 && r == r0 + e);
      if (!ok) return fail(err, std::string(name) + " direct copy: a 16-byte LDS chunk is not 8 contiguous source elements");
    }
  }
  return true;
}

// Staging chunks of the binary32 kernel (4 elements, 16 bytes): slot j of
// thread t moves chunk idx = t + threads * j, and a wave instruction moves 64
// consecutive chunks.  Returned in storage coordinates (row of the operand as
// it sits in memory, first element along that row).  K-contiguous block (rows
// of bk values): instruction idx / 64 covers 8 rows; within it lane l stages
// row 4 (l / 32) + (l % 16) / 4, sub-block (l / 16) % 2, chunk l % 4, so each
// 16-lane group writes 4 whole 64-byte rows of one sub-block.  M/N-contiguous
// block (rows of `row_len` values per k): row idx / (row_len / 4), chunk
// idx % (row_len / 4).
CopyChunk f32_chunk(const lak::KernelShape& s, bool kcontig, int64_t row_len, int64_t idx) {
  if (kcontig) {
    const int64_t l = idx % 64, q = l / 16, w = l % 16;
    return CopyChunk{(idx / 64) * 8 + (q / 2) * 4 + w / 4, (q % 2) * s.k_sub + (w % 4) * 4};
  }
  return CopyChunk{idx / (row_len / 4), (idx % (row_len / 4)) * 4};
}

// Binary32 copy plan of one operand block: every 16-byte LDS vector written
// once, by a chunk of 4 consecutive elements of one storage row.  `v` maps
// the operand's mathematical (row, col) coordinates; `rows_are_math_rows`:
// a storage row is a mathematical row (A [M, K], and B [K, N] in (k, n)).
bool check_copy_f32(const gemm_plan_s& p, const la::View& v, int64_t srows, int64_t scols, bool kcontig,
                    bool rows_are_math_rows, const char* name, std::string* err) {
  const auto& s = p.shape;
  const int64_t chunks = srows * scols / 4;
  if (chunks % s.threads) return fail(err, std::string(name) + " block does not split evenly into 16-byte vectors per thread");
  std::vector<int> hits(static_cast<size_t>(srows * scols), 0);
  for (int64_t idx = 0; idx < chunks; ++idx) {
    const CopyChunk c = f32_chunk(s, kcontig, scols, idx);
    if (c.row >= srows || c.col + 4 > scols) return fail(err, std::string(name) + " copy chunk outside its block");
    auto at = [&](int64_t e) { return rows_are_math_rows ? v.at({c.row, c.col + e}) : v.at({c.col + e, c.row}); };
    const int64_t o0 = at(0);
    if (o0 % 4) return fail(err, std::string(name) + " copy destination is not 16-byte aligned");
    for (int e = 0; e < 4; ++e) {
      const int64_t o = at(e);
      if (o != o0 + e) return fail(err, std::string(name) + " copy destination is not contiguous");
      if (o < 0 || o >= srows * scols || hits[o]++) return fail(err, std::string(name) + " copy plan writes an LDS word twice");
    }
  }
  for (int h : hits)
    if (h != 1) return fail(err, std::string(name) + " copy plan leaves an LDS word unwritten");
  return true;
}

// LDS -> register reads of the binary32 kernel: a K-contiguous block is read
// 4 K values (16 bytes) per lane, which must be contiguous and aligned; an
// M/N-contiguous block one value per lane (nothing to check beyond the map's
// injectivity).  `v` in mathematical coordinates, K the second (A) or first (B) mode.
bool check_fragment_reads_f32(const la::View& v, int64_t others, int64_t bk, bool k_second, const char* name,
                              std::string* err) {
  for (int64_t r = 0; r < others; ++r)
    for (int64_t k = 0; k < bk; k += 4) {
      auto at = [&](int64_t kk) { return k_second ? v.at({r, kk}) : v.at({kk, r}); };
      const int64_t o = at(k);
      if (o % 4) return fail(err, std::string(name) + " fragment read is not 16-byte aligned");
      for (int e = 1; e < 4; ++e)
        if (at(k + e) != o + e) return fail(err, std::string(name) + " fragment read is not contiguous");
    }
  return true;
}

// LDS -> register reads of the fast kernels.  A: lane l of fragment row block
// reads 8 consecutive K values of row l % 32 as one 16-byte chunk.  B:
// transposing reads, where lanes 4e..4e+3 of each 16-lane group address 4
// consecutive N values (8 bytes) of K row e.  Both need those runs to be
// contiguous and aligned in the LDS map.
bool check_fragment_reads(const gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  if (s.a_trans) {
    // M-contiguous A: transposing reads of 4 consecutive M values of one K row
    for (int64_t k = 0; k < s.bk; ++k)
      for (int64_t m = 0; m < s.bm; m += 4) {
        const int64_t o = p.lds_a.at({m, k});
        if (o % 4) return fail(err, "A transposing read is not 8-byte aligned");
        for (int e = 1; e < 4; ++e)
          if (p.lds_a.at({m + e, k}) != o + e) return fail(err, "A transposing read is not contiguous");
      }
  } else {
    for (int64_t r = 0; r < s.bm; ++r)
      for (int64_t k = 0; k < s.bk; k += 8) {
        const int64_t o = p.lds_a.at({r, k});
        if (o % 8) return fail(err, "A fragment read is not 16-byte aligned");
        for (int e = 1; e < 8; ++e)
          if (p.lds_a.at({r, k + e}) != o + e) return fail(err, "A fragment read is not contiguous");
      }
  }
  if (!s.b_kmajor) {
    for (int64_t k = 0; k < s.bk; ++k)
      for (int64_t n = 0; n < s.bn; n += 4) {
        const int64_t o = p.lds_b.at({k, n});
        if (o % 4) return fail(err, "B transposing read is not 8-byte aligned");
        for (int e = 1; e < 4; ++e)
          if (p.lds_b.at({k, n + e}) != o + e) return fail(err, "B transposing read is not contiguous");
      }
  } else {
    for (int64_t n = 0; n < s.bn; ++n)
      for (int64_t k = 0; k < s.bk; k += 8) {
        const int64_t o = p.lds_b.at({k, n});
        if (o % 8) return fail(err, "B fragment read is not 16-byte aligned");
        for (int e = 1; e < 8; ++e)
          if (p.lds_b.at({k + e, n}) != o + e) return fail(err, "B fragment read is not contiguous");
      }
  }
  return true;
}

// MFMA result ownership.  32x32 blocks: register r of lane l of fragment
// (i, j) of wave (wm, wn) holds tile element
//   (wm*TM + 32 i + 8 (r/4) + 4 (l/32) + r%4,  wn*TN + 32 j + l%32);
// 16x16 blocks: (wm*TM + 16 i + 4 (l/16) + r,  wn*TN + 16 j + l%16).
bool check_ownership(const gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  const int mm = s.mfma_m;
  // waves split by weight: the tile is [W_gate block | W_up block], nb * bn columns
  const int cols = s.wave_split ? s.nb * s.bn : s.bn;
  const int tm = s.bm / s.waves_m, tn = cols / s.waves_n;
  if (tm % mm || tn % mm) return fail(err, "wave tile is not a multiple of the MFMA block");
  if (s.wave_split && s.bn % tn) return fail(err, "a wave's slice straddles the two weights");
  const int regs = mm == 32 ? 16 : 4;
  std::vector<int> hits(static_cast<size_t>(s.bm) * cols, 0);
  for (int w = 0; w < s.waves_m * s.waves_n; ++w) {
    const int wm = w % s.waves_m, wn = w / s.waves_m;
    for (int i = 0; i < tm / mm; ++i)
      for (int j = 0; j < tn / mm; ++j)
        for (int l = 0; l < 64; ++l)
          for (int r = 0; r < regs; ++r) {
            const int row = mm == 32 ? wm * tm + 32 * i + 8 * (r / 4) + 4 * (l / 32) + r % 4
                                     : wm * tm + 16 * i + 4 * (l / 16) + r;
            const int col = mm == 32 ? wn * tn + 32 * j + l % 32 : wn * tn + 16 * j + l % 16;
            ++hits[static_cast<size_t>(row) * cols + col];
          }
  }
  for (int h : hits)
    if (h != 1) return fail(err, "MFMA ownership does not cover the C tile exactly once");
  return true;
}

bool check_block(const la::View& v, int64_t base, int64_t block_elems, const char* name, std::string* err) {
  if (!la::injective(v)) return fail(err, std::string(name) + " LDS map is not injective");
  if (la::cosize(v) > block_elems) return fail(err, std::string(name) + " LDS map overruns its block");
  if (base % v.swizzle().period()) return fail(err, std::string(name) + " block base breaks the swizzle phase");
  return true;
}

// ---- step 6: global views and coalesced copy plans ----

// Elements one wave instruction reads, as a layout whose first mode is the
// contiguous run: `rows` rows of `cols` elements, row stride `ld`, columns
// fastest (first mode fastest), reduced by coalesce().
la::Layout copy_instr_layout(int64_t rows, int64_t cols, int64_t ld) {
  return la::coalesce(la::permute(la::Layout::row_major(rows, cols, ld)));
}

// Contiguous run of a coalesced copy layout, in elements (its first mode when
// that mode has stride 1).
int64_t run_elems(const la::Layout& c) {
  std::vector<int64_t> sh, st;
  la::leaves(c.shape(), sh);
  la::leaves(c.stride(), st);
  return st.empty() || st[0] != 1 ? 1 : sh[0];
}


// The set of global elements (relative to the tile origin, through the tiled
// global view's within-tile mode) that wave instruction `ins` reads must equal
// the image of its copy layout placed at its first row.  `along_cols`: the
// chunk is ce consecutive columns of (rows, cols) (else ce consecutive rows).
bool check_instr_reads(const la::Layout& glob, const std::vector<CopyChunk>& chunks, bool along_cols,
                       const la::Layout& instr, int ce, std::string* err, const char* name) {
  std::vector<int64_t> got;
  int64_t r0 = INT64_MAX, c0 = INT64_MAX;
  for (const CopyChunk& ch : chunks) {
    r0 = std::min(r0, ch.row);
    c0 = std::min(c0, ch.col);
    for (int e = 0; e < ce; ++e) {
      const int64_t r = along_cols ? ch.row : ch.row + e, c = along_cols ? ch.col + e : ch.col;
      got.push_back(glob.at({r, c}));
    }
  }
  const int64_t base = glob.at({r0, c0});
  std::vector<int64_t> want;
  for (int64_t i = 0; i < instr.size(); ++i) want.push_back(base + instr(i));
  std::sort(got.begin(), got.end());
  std::sort(want.begin(), want.end());
  if (got != want) return fail(err, std::string(name) + " copy: a wave instruction does not read its planned rows");
  return true;
}

// Inverse of an LDS block map: physical element -> (row, col) of the block.
std::vector<CopyChunk> lds_inverse(const la::View& v, int64_t rows, int64_t cols) {
  std::vector<CopyChunk> inv(static_cast<size_t>(rows * cols));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) inv[v.at({r, c})] = CopyChunk{r, c};
  return inv;
}

// Within-tile mode of a tiled global view (coordinate (r, c) of tile (0, 0)).
struct TileView {
  la::Layout tiled;
  int64_t at(int64_t r, int64_t c) const { return tiled.at({r, c}); }
};

bool plan_copies(gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  const gemm_desc& d = p.d;
  const int eb = s.in_bytes, ce = 16 / eb;   // bytes per element, elements per 16-byte chunk
  // covering extents: tile() needs whole tiles; coordinates past M, N or K are
  // the edges the general kernel masks
  const int64_t Mc = std::max<int64_t>(1, p.tiles_m) * s.bm, Nc = std::max<int64_t>(1, p.tiles_n) * s.bn;
  const int64_t Kc = std::max<int64_t>(1, (d.k + s.bk - 1) / s.bk) * s.bk;
  p.glob_a = s.a_trans ? la::tile(la::Layout::col_major(Mc, Kc, d.lda), {s.bm, s.bk})
                       : la::tile(la::Layout::row_major(Mc, Kc, d.lda), {s.bm, s.bk});
  p.glob_b = p.b_kmajor ? la::tile(la::Layout::col_major(Kc, Nc, d.ldb), {s.bk, s.bn})
                        : la::tile(la::Layout::row_major(Kc, Nc, d.ldb), {s.bk, s.bn});
  p.glob_c = la::tile(la::Layout::row_major(Mc, Nc, d.ldc), {s.bm, s.bn});
  // within-tile maps of tile (0, 0): coordinate ((r, 0), (c, 0)) of the tiled view
  auto inner = [](const la::Layout& t, int64_t r, int64_t c) {
    return t(la::Tree::T({la::Tree::T({la::Tree::L(r), la::Tree::L(0)}), la::Tree::T({la::Tree::L(c), la::Tree::L(0)})}));
  };
  const la::Layout ga = la::Layout::flat({s.bm, s.bk}, {inner(p.glob_a, 1, 0), inner(p.glob_a, 0, 1)});
  // B in (k, n) coordinates of the block
  const la::Layout gb = la::Layout::flat({s.bk, s.bn}, {inner(p.glob_b, 1, 0), inner(p.glob_b, 0, 1)});

  // Per-instruction copy layouts: a wave instruction moves 64 x 16 bytes.
  // Rows of an operand block as stored in memory: A rows of BK along K;
  // B rows of BN along N ([K, N]) or of BK along K ([N, K]).
  const int64_t a_cols = s.a_trans ? s.bm : s.bk, b_cols = s.b_kmajor ? s.bk : s.bn;
  const int64_t b_ld = d.ldb;
  const int64_t per_instr = 64 * ce;
  if (per_instr % a_cols || per_instr % b_cols) return fail(err, "a copy instruction does not cover whole rows");
  const la::Layout ca = copy_instr_layout(per_instr / a_cols, a_cols, d.lda);
  const la::Layout cb = copy_instr_layout(per_instr / b_cols, b_cols, b_ld);
  const int64_t na = int64_t(s.bm) * s.bk / per_instr, nbk = int64_t(s.bk) * s.bn / per_instr;

  std::vector<std::vector<CopyChunk>> ia(na), ib(nbk);
  if (eb == 4) {
    // binary32 kernel: storage coordinates -> block coordinates (A (m, k), B (k, n))
    for (int64_t ins = 0; ins < na; ++ins)
      for (int l = 0; l < 64; ++l) {
        const CopyChunk c = f32_chunk(s, !s.a_trans, a_cols, ins * 64 + l);
        ia[ins].push_back(s.a_trans ? CopyChunk{c.col, c.row} : c);
      }
    for (int64_t ins = 0; ins < nbk; ++ins)
      for (int l = 0; l < 64; ++l) {
        const CopyChunk c = f32_chunk(s, s.b_kmajor, b_cols, ins * 64 + l);
        ib[ins].push_back(s.b_kmajor ? CopyChunk{c.col, c.row} : c);
      }
  } else if (s.direct) {
    // lane l of instruction `ins` fills physical elements [512 ins + 8 l, +8)
    const std::vector<CopyChunk> inva = lds_inverse(p.lds_a, s.bm, s.bk);
    const std::vector<CopyChunk> invb = lds_inverse(p.lds_b, s.bk, s.bn);
    for (int64_t ins = 0; ins < na; ++ins)
      for (int l = 0; l < 64; ++l) ia[ins].push_back(inva[per_instr * ins + 8 * l]);
    for (int64_t ins = 0; ins < nbk; ++ins)
      for (int l = 0; l < 64; ++l) ib[ins].push_back(invb[per_instr * ins + 8 * l]);
  } else {
    // register-staged: slot j of thread t moves chunk t + threads * j (row-major over chunks);
    // a wave instruction is one slot of 64 consecutive threads
    const int T = s.threads;
    for (int64_t ins = 0; ins < na; ++ins) {
      const int64_t j = ins / (T / 64), w = ins % (T / 64);
      for (int l = 0; l < 64; ++l) {
        const int64_t idx = w * 64 + l + T * j;
        if (s.a_trans) ia[ins].push_back(CopyChunk{(idx % (s.bm / 8)) * 8, idx / (s.bm / 8)});
        else ia[ins].push_back(CopyChunk{idx / (s.bk / 8), (idx % (s.bk / 8)) * 8});
      }
    }
    for (int64_t ins = 0; ins < nbk; ++ins) {
      const int64_t j = ins / (T / 64), w = ins % (T / 64);
      for (int l = 0; l < 64; ++l) {
        const int64_t idx = w * 64 + l + T * j;
        if (s.b_kmajor) ib[ins].push_back(CopyChunk{(idx % (s.bk / 8)) * 8, idx / (s.bk / 8)});
        else ib[ins].push_back(CopyChunk{idx / (s.bn / 8), (idx % (s.bn / 8)) * 8});
      }
    }
  }
  for (const auto& ch : ia)
    if (!check_instr_reads(ga, ch, !s.a_trans, ca, ce, err, "A")) return false;
  for (const auto& ch : ib)
    if (!check_instr_reads(gb, ch, !s.b_kmajor, cb, ce, err, "B")) return false;
  std::ostringstream js;
  js << "{\"A\":{\"instr\":\"" << ca.str() << "\",\"run_bytes\":" << run_elems(ca) * eb << ",\"instrs_per_block\":" << na << "}"
     << ",\"B\":{\"instr\":\"" << cb.str() << "\",\"run_bytes\":" << run_elems(cb) * eb << ",\"instrs_per_block\":" << nbk << "}}";
  p.copy_json = js.str();
  return true;
}

// ---- step 7: the LDS ring as one allocation, stages as windows ----

// Ring of `stages` blocks of (rows, cols), block base `base` inside a stage of
// `stage` elements.  The allocation map is Swizzle o ((rows, cols, stages) :
// (ld_r, ld_c, stage)) applied to offsets relative to the block base (the row
// and column modes as the block map has them, nested or flat); stage s
// is the window at origin (0, 0, s).  Every window must give stage * s plus the
// block map: the stage bases sit on the swizzle period, so the phase is the
// allocation's.
bool check_ring(const la::View& block, int64_t rows, int64_t cols, int64_t stage, int stages, const char* name,
                std::string* err) {
  const la::Layout& bl = block.base();
  const la::View ring(block.swizzle(),
                      la::Layout(la::Tree::T({bl.shape().mode(0), bl.shape().mode(1), la::Tree::L(stages)}),
                                 la::Tree::T({bl.stride().mode(0), bl.stride().mode(1), la::Tree::L(stage)})));
  for (int sidx = 0; sidx < stages; ++sidx) {
    const la::View w = ring.window({0, 0, sidx}, {rows, cols, 1});
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t c = 0; c < cols; ++c)
        if (w.at({r, c, 0}) != int64_t(sidx) * stage + block.at({r, c}))
          return fail(err, std::string(name) + " ring: a stage window does not keep the allocation's swizzle phase");
  }
  return true;
}

// ---- step 8: store plans ----

// One store of the epilogue: lane `lane` of store instruction `ins` writes
// `n` consecutive elements of row `row` starting at column `col` (tile
// coordinates), guarded by the kernel's mask.
struct Store { int64_t ins; int lane; int64_t row, col; int n; };

std::vector<Store> store_plan(const gemm_plan_s& p) {
  const auto& s = p.shape;
  std::vector<Store> out;
  // waves split by weight: columns of [W_gate block | W_up block]; column c is column c mod bn of output c / bn
  const int tm = s.bm / s.waves_m, tn = (s.wave_split ? s.nb * s.bn : s.bn) / s.waves_n;
  int64_t ins = 0;
  const bool fast = fast_kid(p.kid);
  for (int w = 0; w < s.waves_m * s.waves_n; ++w) {
    const int wm = w % s.waves_m, wn = w / s.waves_m;
    if (fast) {
      // rows of 8 consecutive outputs per lane, read back from the wave's LDS window
      const int ch = tn / 8, rpp = 64 / ch;
      for (int i = 0; i < tm / 32; ++i)
        for (int q = 0; q < 32 / rpp; ++q, ++ins)
          for (int l = 0; l < 64; ++l) out.push_back(Store{ins, l, wm * tm + 32 * i + q * rpp + l / ch, wn * tn + (l % ch) * 8, 8});
    } else if (s.mfma_m == 32) {
      // straight from the 32 x 32 accumulator lane map, one element per lane and register
      for (int i = 0; i < tm / 32; ++i)
        for (int j = 0; j < tn / 32; ++j)
          for (int e = 0; e < 16; ++e, ++ins)
            for (int l = 0; l < 64; ++l)
              out.push_back(Store{ins, l, wm * tm + 32 * i + 4 * (l / 32) + 8 * (e / 4) + e % 4, wn * tn + 32 * j + l % 32, 1});
    } else {
      // 16 x 16 accumulator lane map, 16-row blocks i of the wave's rows
      for (int j = 0; j < tn / 16; ++j)
        for (int i = 0; i < tm / 16; ++i)
          for (int r = 0; r < 4; ++r, ++ins)
            for (int l = 0; l < 64; ++l)
              out.push_back(Store{ins, l, wm * tm + 16 * i + 4 * (l / 16) + r, wn * tn + 16 * j + l % 16, 1});
    }
  }
  return out;
}

bool plan_stores(gemm_plan_s& p, std::string* err) {
  const auto& s = p.shape;
  const gemm_desc& d = p.d;
  const std::vector<Store> plan = store_plan(p);
  // the kernels' store mask: element (row, col) of tile (tm, tn) is written
  // when it lies inside C (all kernels mask their stores at M and N)
  const int64_t wcols = s.wave_split ? int64_t(s.nb) * s.bn : s.bn;   // store-plan columns per tile
  auto check_tile = [&](int64_t tm, int64_t tn) {
    const int64_t rows = std::min<int64_t>(s.bm, d.m - tm * s.bm), cols = std::min<int64_t>(s.bn, d.n - tn * s.bn);
    std::vector<int> hits(static_cast<size_t>(s.bm) * wcols, 0);
    for (const Store& st : plan)
      for (int e = 0; e < st.n; ++e) {
        const int64_t r = st.row, c = st.col + e;
        if (r < 0 || r >= s.bm || c < 0 || c >= wcols) return fail(err, "store plan leaves its tile");
        if (r < rows && c % s.bn < cols) ++hits[r * wcols + c];
      }
    for (int64_t r = 0; r < s.bm; ++r)
      for (int64_t c = 0; c < wcols; ++c) {
        const int h = hits[r * wcols + c];
        if (r < rows && c % s.bn < cols ? h != 1 : h != 0)
          return fail(err, "store plan does not write every element of C inside its tile exactly once");
      }
    return true;
  };
  int classes = 0;
  if (d.m > 0 && d.n > 0) {
    const int64_t lm = p.tiles_m - 1, ln = p.tiles_n - 1;
    const int64_t cls[4][2] = {{0, 0}, {lm, 0}, {0, ln}, {lm, ln}};
    for (int c = 0; c < 4; ++c) {
      bool seen = false;
      for (int c2 = 0; c2 < c; ++c2) seen |= cls[c2][0] == cls[c][0] && cls[c2][1] == cls[c][1];
      if (seen) continue;
      if (!check_tile(cls[c][0], cls[c][1])) return false;
      ++classes;
    }
  }
  // one store instruction reduced to its contiguous runs
  std::vector<int64_t> offs;
  for (const Store& st : plan)
    if (st.ins == 0)
      for (int e = 0; e < st.n; ++e) offs.push_back(p.glob_c.at({st.row, (st.col + e) % s.bn}));
  std::sort(offs.begin(), offs.end());
  int64_t runs = offs.empty() ? 0 : 1, longest = offs.empty() ? 0 : 1, cur = 1;
  for (size_t i = 1; i < offs.size(); ++i) {
    if (offs[i] == offs[i - 1] + 1) { ++cur; } else { ++runs; cur = 1; }
    longest = std::max(longest, cur);
  }
  const bool fast = fast_kid(p.kid);
  std::ostringstream js;
  js << "{\"style\":\"" << (fast ? "lds_rows" : s.mfma_m == 32 ? "mfma32" : "mfma16") << "\",\"elems_per_lane\":"
     << (fast ? 8 : 1) << ",\"runs_per_instr\":" << runs << ",\"run_bytes\":" << longest * p.out_bytes
     << ",\"tile_classes_checked\":" << classes << "}";
  p.store_json = js.str();
  return true;
}

const char* dtype_name(int t) {
  switch (t) {
    case GEMM_BF16: return "bf16";
    case GEMM_F16: return "f16";
    case GEMM_F32: return "f32";
    case GEMM_F8E4M3: return "f8e4m3";
    case GEMM_F8E5M2: return "f8e5m2";
    default: return "?";
  }
}

// The plan as JSON (gemm_plan_describe): sizes, kernel, tile, layouts, copy and store plans.
std::string describe(const gemm_plan_s& p) {
  const gemm_desc& d = p.d;
  const auto& s = p.shape;
  std::ostringstream js;
  static const char* const kNames[] = {"tiled", "fast", "fast_gate_up", "skinny", "fast_bkmajor", "fast_gate_up_bkmajor", "tiled",
                                      "tiled", "fast_atrans", "fast_gate_up_atrans", "tiled_f32", "fast_f8",
                                      "fast_gate_up_f8", "skinny_bkmajor", "skinny_f8", "skinny", "skinny",
                                      "skinny_bkmajor", "skinny_bkmajor", "skinny_f8", "skinny_f8", "skinny",
                                      "skinny_bkmajor", "skinny_f8", "fast", "fast_bkmajor", "fast_f8",
                                      "fast_bkmajor", "fast", "fast_f8"};
  static_assert(sizeof(kNames) / sizeof(kNames[0]) == lak::KID_COUNT, "one name per kernel id");
  js << "{\"kernel\":\"" << kNames[p.kid] << "_" << s.bm << "x" << s.bn << "x" << s.bk << "\""
     << ",\"m\":" << d.m << ",\"n\":" << d.n << ",\"k\":" << d.k
     << ",\"lda\":" << d.lda << ",\"ldb\":" << d.ldb << ",\"ldc\":" << d.ldc
     << ",\"in\":\"" << dtype_name(d.a_type) << "\",\"in_b\":\"" << dtype_name(d.b_type) << "\""
     << ",\"out\":\"" << dtype_name(d.c_type) << "\""
     << ",\"gate_up\":" << (p.gate_up ? "true" : "false")
     << ",\"a_order\":\"" << (p.a_trans ? "km" : "mk") << "\""
     << ",\"b_order\":\"" << (p.b_kmajor ? "nk" : "kn") << "\""
     << ",\"batch\":" << d.batch
     << ",\"tile\":[" << s.bm << "," << s.bn << "," << s.bk << "]"
     << ",\"waves\":[" << s.waves_m << "," << s.waves_n << "],\"threads\":" << s.threads
     << ",\"mfma\":\"" << s.mfma_m << "x" << s.mfma_n << "x" << s.mfma_k << "\""
     << ",\"tiles\":[" << p.tiles_m << "," << p.tiles_n << "],\"grid\":" << p.grid << ",\"group_m\":" << p.group_m
     << ",\"stages\":" << s.stages << ",\"stage_elems\":" << p.stage_elems << ",\"lds_bytes\":" << p.lds_bytes
     << ",\"swizzle_a\":[" << s.sw_a[0] << "," << s.sw_a[1] << "," << s.sw_a[2] << "]"
     << ",\"swizzle_b\":[" << s.sw_b[0] << "," << s.sw_b[1] << "," << s.sw_b[2] << "]"
     << ",\"direct_loads\":" << (s.direct ? "true" : "false")
     << ",\"waves_split_by_weight\":" << (s.wave_split ? "true" : "false")
     << ",\"lds_a\":\"" << p.lds_a.base().str() << "\",\"lds_b\":\"" << p.lds_b.base().str() << "\""
     << ",\"prefetch_blocks\":" << prefetch_blocks(p)
     << ",\"global_a\":\"" << p.glob_a.str() << "\",\"global_b\":\"" << p.glob_b.str() << "\",\"global_c\":\""
     << p.glob_c.str() << "\""
     << ",\"copy\":" << p.copy_json << ",\"store\":" << p.store_json
     << ",\"in_bytes\":" << s.in_bytes << ",\"k_sub\":" << s.k_sub
     << ",\"vec_elems\":" << p.vec << ",\"align_bytes\":" << p.align_bytes
     << ",\"out_align_bytes\":" << p.out_align_bytes
     << ",\"split_k\":" << p.split;
  if (p.split > 1) {
    const lak::KernelShape ss = lak::kernel_shape(p.split_kid);
    js << ",\"split_kernel\":\"" << kNames[p.split_kid] << "_" << ss.bm << "x" << ss.bn << "x" << ss.bk << "\""
       << ",\"split_grid\":[" << int64_t(p.split_tiles_m) * p.split_tiles_n << "," << p.split << "]";
  }
  js << ",\"workspace_bytes\":" << p.ws_bytes << "}";
  return js.str();
}

bool is_f8(int32_t t) { return t == GEMM_F8E4M3 || t == GEMM_F8E5M2; }

}  // namespace

// One-byte inputs (OCP E4M3 / E5M2, A and B each either; plain GEMMs, row
// reductions and gate/up): both operands K-contiguous (A [M, K], B and the
// gate/up weights [N, K]), every row on 16 bytes.  Copies and
// fragment reads move whole 16-byte chunks, so the kernel addresses a row of
// codes as 16-bit units holding byte pairs: the plan is the K-major 16-bit
// full-tile plan of the pair view (K, lda, ldb and the A / B batch strides
// halved), checked by the same steps, then described in one-byte elements
// after checking that every byte's LDS offset is its pair's offset doubled
// plus its position in the pair.  The 64-code rows of a K block are the
// 64-byte swizzle rows of the Tylo.jl page "TMA and Hopper WGMMA" (section
// "The same storage contract on both sides"), Swizzle{2,4,4}.
static gemm_status build_f8(const gemm_desc& d, gemm_plan_s& p, std::string* err) {
  auto unsupported = [&](const char* m) { fail(err, m); return GEMM_ERR_UNSUPPORTED; };
  if (!is_f8(d.a_type) || !is_f8(d.b_type))
    return unsupported("A and B must both be one-byte (E4M3 or E5M2) or both be wider");
  if (!(d.flags & GEMM_FLAG_B_KMAJOR) || (d.flags & GEMM_FLAG_A_TRANSPOSED))
    return unsupported("one-byte inputs need A stored [M, K] and B stored [N, K] (GEMM_FLAG_B_KMAJOR): both K-contiguous");
  const bool many = d.batch > 1;
  if (d.lda % 16 || d.ldb % 16 || (many && (d.stride_a % 16 || d.stride_b % 16)))
    return unsupported("one-byte inputs need lda, ldb (and the A and B batch strides) to be multiples of 16");
  if (d.ldc % 8 || (many && d.stride_c % 8))
    return unsupported("one-byte inputs need ldc (and stride_c) to be multiples of 8: C rows on 16 bytes");
  if (d.k % 16) return unsupported("one-byte inputs need k to be a multiple of 16");
  if (d.k % 64 && d.k < 512)
    return unsupported("one-byte inputs need k to be a multiple of 64 below 512 (from 512 on the last k % 64 are added "
                       "after the main loop)");
  gemm_desc v = d;
  v.k = d.k / 2;
  v.lda = d.lda / 2;
  v.ldb = d.ldb / 2;
  v.stride_a = d.stride_a / 2;
  v.stride_b = d.stride_b / 2;
  v.a_type = v.b_type = GEMM_BF16;
  // The pair view's own choice where it has a one-byte form (the K-major 256-wide kernel, its
  // 128-row tiles, the skinny kernels), else the full-tile kernel at every grid size.
  auto has_f8_form = [](int kid) {
    return kid == lak::KID_FAST_256_KM || kid == lak::KID_FAST_GU_KM || kid == lak::KID_FAST_128_KM ||
           kid == lak::KID_FAST_128_KM64 ||
           kid == lak::KID_SKINNY_16_KM || kid == lak::KID_SKINNY_32_KM || kid == lak::KID_SKINNY_64_KM ||
           kid == lak::KID_SKINNY_128_KM;
  };
  gemm_status st = build(v, p, err);
  if (st != GEMM_OK || !has_f8_form(p.kid)) {
    v.flags |= GEMM_FLAG_LARGE_TILES;
    st = build(v, p, err);
  }
  if (st != GEMM_OK) return st;
  const bool runs = d.m > 0 && d.n > 0 && d.k > 0;
  // the pair view's kernel and its one-byte counterpart
  int pair_kid = p.gate_up ? lak::KID_FAST_GU_KM : lak::KID_FAST_256_KM;
  int kid8 = p.gate_up ? lak::KID_FAST_GU_F8 : lak::KID_FAST_F8;
  if (p.kid == lak::KID_FAST_128_KM) pair_kid = p.kid, kid8 = lak::KID_FAST_F8_128;
  if (p.kid == lak::KID_FAST_128_KM64) pair_kid = p.kid, kid8 = lak::KID_FAST_F8_128_K64;
  if (p.kid == lak::KID_SKINNY_16_KM) pair_kid = p.kid, kid8 = lak::KID_SKINNY_F8;
  if (p.kid == lak::KID_SKINNY_32_KM) pair_kid = p.kid, kid8 = lak::KID_SKINNY_F8_32;
  if (p.kid == lak::KID_SKINNY_64_KM) pair_kid = p.kid, kid8 = lak::KID_SKINNY_F8_64;
  if (p.kid == lak::KID_SKINNY_128_KM) pair_kid = p.kid, kid8 = lak::KID_SKINNY_F8_128;
  if (runs && p.kid != pair_kid)
    return unsupported("one-byte inputs: operand rows too far apart for the kernel's 32-bit byte offsets");
  // the split form's partial products on byte pairs (the ranges cut K in pairs, an even count of codes)
  if (p.split > 1) {
    const int sk = p.split_kid;
    p.split_kid = sk == lak::KID_SKINNY_16_KM ? lak::KID_SKINNY_F8
                : sk == lak::KID_FAST_256_KM ? lak::KID_FAST_F8
                : sk == lak::KID_FAST_128_KM ? lak::KID_FAST_F8_128
                : sk == lak::KID_FAST_128_KM64 ? lak::KID_FAST_F8_128_K64
                : sk == lak::KID_SKINNY_32_KM ? lak::KID_SKINNY_F8_32
                : sk == lak::KID_SKINNY_64_KM ? lak::KID_SKINNY_F8_64
                : sk == lak::KID_SKINNY_128_KM ? lak::KID_SKINNY_F8_128 : -1;
    if (p.split_kid < 0) {
      fail(err, "one-byte split form without a one-byte kernel");
      return GEMM_ERR_RESOURCE;
    }
  }
  p.d = d;
  p.kd = v;
  if (p.kid == pair_kid) {
    p.in_bytes = 1;
    const lak::KernelShape s8 = lak::kernel_shape(kid8);
    try {
      using la::Tree;
      const la::Swizzle swa(s8.sw_a[0], s8.sw_a[1], s8.sw_a[2]), swb(s8.sw_b[0], s8.sw_b[1], s8.sw_b[2]);
      const la::View a8(swa, la::Layout(Tree::T({Tree::L(s8.bm), Tree::L(s8.bk)}), Tree::T({Tree::L(s8.bk), Tree::L(1)})));
      const la::View b8(swb, la::Layout(Tree::T({Tree::L(s8.bk), Tree::L(s8.bn)}), Tree::T({Tree::L(1), Tree::L(s8.bk)})));
      for (int64_t r = 0; r < s8.bm; ++r)
        for (int64_t k = 0; k < s8.bk; ++k)
          if (a8.at({r, k}) != 2 * p.lds_a.at({r, k / 2}) + k % 2) {
            fail(err, "one-byte A map differs from its byte-pair map at (" + std::to_string(r) + ", " + std::to_string(k) + ")");
            return GEMM_ERR_RESOURCE;
          }
      for (int64_t k = 0; k < s8.bk; ++k)
        for (int64_t n = 0; n < s8.bn; ++n)
          if (b8.at({k, n}) != 2 * p.lds_b.at({k / 2, n}) + k % 2) {
            fail(err, "one-byte B map differs from its byte-pair map at (" + std::to_string(k) + ", " + std::to_string(n) + ")");
            return GEMM_ERR_RESOURCE;
          }
      if (!check_block(a8, 0, int64_t(s8.bm) * s8.bk, "A", err) || !check_block(b8, 0, int64_t(s8.bn) * s8.bk, "B", err))
        return GEMM_ERR_RESOURCE;
      // the W_up block follows W_gate's in each stage, as in the pair view
      if (p.gate_up && 2 * (p.base_b2 - p.base_b) != int64_t(s8.bn) * s8.bk) {
        fail(err, "one-byte W_up block does not follow W_gate's");
        return GEMM_ERR_RESOURCE;
      }
      p.lds_a = a8;
      p.lds_b = p.lds_b2 = b8;
      p.base_b = int64_t(s8.bm) * s8.bk;
      p.base_b2 = p.base_b + int64_t(s8.bn) * s8.bk;
      p.stage_elems *= 2;
      const int64_t Mc = int64_t(p.tiles_m) * s8.bm, Nc = int64_t(p.tiles_n) * s8.bn;
      const int64_t Kc = (d.k + s8.bk - 1) / s8.bk * s8.bk;
      p.glob_a = la::tile(la::Layout::row_major(Mc, Kc, d.lda), {s8.bm, s8.bk});
      p.glob_b = la::tile(la::Layout::col_major(Kc, Nc, d.ldb), {s8.bk, s8.bn});
      // a wave instruction moves 1 KiB: 1024 / bk rows of one K block row each
      const la::Layout ca = copy_instr_layout(1024 / s8.bk, s8.bk, d.lda), cb = copy_instr_layout(1024 / s8.bk, s8.bk, d.ldb);
      const int64_t per_a = int64_t(s8.bm) * s8.bk / 1024, per_b = int64_t(s8.bn) * s8.bk / 1024;
      std::ostringstream js;
      js << "{\"A\":{\"instr\":\"" << ca.str() << "\",\"run_bytes\":" << s8.bk << ",\"instrs_per_block\":" << per_a << "}"
         << ",\"B\":{\"instr\":\"" << cb.str() << "\",\"run_bytes\":" << s8.bk << ",\"instrs_per_block\":" << per_b << "}}";
      p.copy_json = js.str();
    } catch (const la::LayoutError& e) {
      fail(err, e.what());
      return GEMM_ERR_RESOURCE;
    }
    p.kid = kid8;
    p.shape = s8;
    p.vec = 16;
    p.in_kind = lak::IN_F8 + 2 * (d.a_type == GEMM_F8E5M2 ? 1 : 0) + (d.b_type == GEMM_F8E5M2 ? 1 : 0);
  }
  // (k == 0, or nothing to compute: the pair view's plan, maps and all, which reads no element of A or B)
  p.json = describe(p);
  return GEMM_OK;
}

gemm_status build(const gemm_desc& d, gemm_plan_s& p, std::string* err) {
  p = gemm_plan_s{};
  p.d = d;
  p.kd = d;
  if (d.m < 0 || d.n < 0 || d.k < 0) { fail(err, "m, n and k must be >= 0"); return GEMM_ERR_INVALID_ARG; }
  const bool kmajor = (d.flags & GEMM_FLAG_B_KMAJOR) != 0;
  const bool atrans = (d.flags & GEMM_FLAG_A_TRANSPOSED) != 0;
  if (!atrans && d.lda < std::max<int64_t>(1, d.k)) { fail(err, "lda must be >= max(1, k)"); return GEMM_ERR_INVALID_ARG; }
  if (atrans && d.lda < std::max<int64_t>(1, d.m)) { fail(err, "lda must be >= max(1, m) for A stored [K, M]"); return GEMM_ERR_INVALID_ARG; }
  if (!kmajor && d.ldb < std::max<int64_t>(1, d.n)) { fail(err, "ldb must be >= max(1, n)"); return GEMM_ERR_INVALID_ARG; }
  if (kmajor && d.ldb < std::max<int64_t>(1, d.k)) { fail(err, "ldb must be >= max(1, k) for K-major B"); return GEMM_ERR_INVALID_ARG; }
  if (d.ldc < std::max<int64_t>(1, d.n)) { fail(err, "ldc must be >= max(1, n)"); return GEMM_ERR_INVALID_ARG; }
  // element offsets are 64-bit: keep every stride far below the point where row * ld could wrap
  constexpr int64_t kMaxStride = int64_t{1} << 40;
  if (d.lda > kMaxStride || d.ldb > kMaxStride || d.ldc > kMaxStride || d.stride_a > kMaxStride ||
      d.stride_b > kMaxStride || d.stride_c > kMaxStride) {
    fail(err, "leading dimensions and batch strides must be <= 2^40 elements");
    return GEMM_ERR_UNSUPPORTED;
  }
  auto in_type = [](int32_t t) { return t >= GEMM_BF16 && t <= GEMM_F8E5M2; };
  if (!in_type(d.a_type) || !in_type(d.b_type) ||
      (d.c_type != GEMM_BF16 && d.c_type != GEMM_F16 && d.c_type != GEMM_F32)) {
    fail(err, "unknown dtype");
    return GEMM_ERR_INVALID_ARG;
  }
  if (d.flags & ~(GEMM_FLAG_GATE_UP | GEMM_FLAG_B_KMAJOR | GEMM_FLAG_LARGE_TILES | GEMM_FLAG_A_TRANSPOSED)) {
    fail(err, "unknown flag bits");
    return GEMM_ERR_INVALID_ARG;
  }
  if (is_f8(d.a_type) || is_f8(d.b_type)) return build_f8(d, p, err);
  const bool in32 = d.a_type == GEMM_F32 && d.b_type == GEMM_F32;
  if (atrans && kmajor && !in32) {
    fail(err, "A stored [K, M] together with B stored [N, K] is implemented for binary32 inputs only");
    return GEMM_ERR_UNSUPPORTED;
  }
  if (d.batch < 1 || d.batch > 65535) { fail(err, "batch must be in 1..65535"); return GEMM_ERR_INVALID_ARG; }
  if (d.stride_a < 0 || d.stride_b < 0 || d.stride_c < 0) { fail(err, "batch strides must be >= 0"); return GEMM_ERR_INVALID_ARG; }
  if (d.batch > 1 && d.m > 0 && d.n > 0) {
    // disjoint blocks, or rows of the matrices interleaved with disjoint segments
    const bool blocks = __int128(d.stride_c) >= __int128(d.m - 1) * d.ldc + d.n;
    const bool interleaved = d.stride_c >= d.n && __int128(d.ldc) >= __int128(d.batch - 1) * d.stride_c + d.n;
    if (!blocks && !interleaved) {
      fail(err, "batched outputs would overlap: use stride_c >= (m-1)*ldc + n, or interleaved rows with "
                "stride_c >= n and ldc >= (batch-1)*stride_c + n");
      return GEMM_ERR_INVALID_ARG;
    }
  }
  if (d.a_type != d.b_type) {
    fail(err, "A and B must both be bf16, both be f16 or both be f32");
    return GEMM_ERR_UNSUPPORTED;
  }
  if (in32 && (d.flags & GEMM_FLAG_GATE_UP)) {
    fail(err, "binary32 inputs are planned for plain GEMMs only (no gate/up)");
    return GEMM_ERR_UNSUPPORTED;
  }
  // 32-bit tile ids and in-tile offsets; global offsets are 64-bit.
  if (d.m > (int64_t{1} << 31) - 256 || d.n > (int64_t{1} << 31) - 256 || d.k > (int64_t{1} << 31) - 256) {
    fail(err, "dimension too large");
    return GEMM_ERR_UNSUPPORTED;
  }

  p.gate_up = (d.flags & GEMM_FLAG_GATE_UP) != 0;
  p.b_kmajor = kmajor;
  p.a_trans = atrans;
  p.in_kind = d.a_type == GEMM_BF16 ? lak::IN_BF16 : d.a_type == GEMM_F16 ? lak::IN_F16 : lak::IN_F32;
  p.in_bytes = in32 ? 4 : 2;
  p.out_kind = d.c_type == GEMM_F32 ? lak::OUT_F32 : d.c_type == GEMM_BF16 ? lak::OUT_BF16 : lak::OUT_F16;
  p.out_bytes = d.c_type == GEMM_F32 ? 4 : 2;
  // Batch strides move every row start of matrix b by b*stride, so with more
  // than one matrix they join the leading dimensions in the alignment class.
  const bool many = d.batch > 1;
  const bool in16 = d.lda % 8 == 0 && d.ldb % 8 == 0 && (!many || (d.stride_a % 8 == 0 && d.stride_b % 8 == 0));
  const bool out16 = d.ldc % 8 == 0 && (!many || d.stride_c % 8 == 0);
  if (in32) {
    // Binary32 inputs: one kernel for every shape and storage order, staging
    // 4-element chunks along each operand's contiguous direction: one 16-byte
    // load each when every row starts on 16 bytes and no chunk is cut by an
    // edge (vec 4), else four 4-byte loads (vec 1).
    const bool rows16 = d.lda % 4 == 0 && d.ldb % 4 == 0 && (!many || (d.stride_a % 4 == 0 && d.stride_b % 4 == 0));
    const bool whole = (atrans ? d.m : d.k) % 4 == 0 && (kmajor ? d.k : d.n) % 4 == 0;
    p.vec = rows16 && whole ? 4 : 1;
    p.align_bytes = p.vec == 4 ? 16 : 4;
    p.kid = lak::KID_TILED_F32;
  }
  // The general kernel stages 8-element chunks along K (A, K-major B) or N
  // (N-contiguous B), one 16-byte load each: aligned (vec 8) when rows start
  // on 16 bytes and no chunk is cut by an edge; else at 2-byte alignment
  // (vec 2), a chunk cut by an edge loading the 8 elements that end at its
  // last valid one, which stay inside the row only when the row holds more
  // than 8 elements.  Shorter rows that are not whole chunks take 2-byte
  // loads (vec 1).
  // (A stored [K, M] is staged in chunks along M instead of K.)
  const int64_t a_row = atrans ? d.m : d.k;
  if (!in32) {
  const bool chunks_whole = a_row % 8 == 0 && (kmajor || d.n % 8 == 0);
  const bool rows_fit = (a_row % 8 == 0 || a_row > 8) && (kmajor || d.n % 8 == 0 || d.n > 8);
  p.vec = in16 && chunks_whole ? 8 : rows_fit ? 2 : 1;
  p.align_bytes = p.vec == 8 ? 16 : 2;
  if (atrans && p.vec == 1) {
    fail(err, "A stored [K, M] needs m to be a multiple of 8 or larger than 8 (and n likewise)");
    return GEMM_ERR_UNSUPPORTED;
  }

  // Kernel choice: the full-tile direct-load kernels when every row starts on
  // 16 bytes; M and N may end inside a tile (edge tiles read clamped source
  // rows and columns and store only inside C), as long as the rows of the
  // operand read in 16-byte chunks along M or N hold whole chunks (N % 8 for B
  // stored [K, N], M % 8 for A stored [K, M]: no chunk reaches past a row's
  // last element) and the tiles' padding stays small; K may end inside a K
  // block from K = 256 on.  Otherwise the general kernel, which masks edges
  // and stages with the width chosen above.
  p.kid = lak::KID_TILED_128;
  {
    const int fk = p.gate_up ? (kmajor ? lak::KID_FAST_GU_KM : atrans ? lak::KID_FAST_GU_AT : lak::KID_FAST_GU)
                             : (kmajor ? lak::KID_FAST_256_KM : atrans ? lak::KID_FAST_256_AT : lak::KID_FAST_256);
    const lak::KernelShape fs = lak::kernel_shape(fk);
    const bool whole = d.m > 0 && d.n > 0 && d.k > 0 && d.m % fs.bm == 0 && d.n % fs.bn == 0 && d.k % fs.bk == 0;
    const bool rows16 = in16 && out16;
    // per-lane source offsets of the direct loads are 32-bit byte offsets
    const int64_t b_rows = kmajor ? fs.bn : fs.bk;   // rows of B one block spans in memory
    const int64_t a_rows = atrans ? fs.bk : fs.bm;   // rows of A one block spans in memory
    const bool off32 = 2 * a_rows * d.lda < (int64_t{1} << 32) && 2 * b_rows * d.ldb < (int64_t{1} << 32);
    const bool large = (d.flags & GEMM_FLAG_LARGE_TILES) != 0;
    const int64_t ftm = (d.m + fs.bm - 1) / fs.bm, ftn = (d.n + fs.bn - 1) / fs.bn;
    // K ending inside a K block: the kernels add the last K % 32 values after the main loop from
    // global memory (one short pass per tile), taken only where that pass is a small part of K
    const bool k_ok = d.k > 0 && (d.k % fs.bk == 0 || d.k >= 256);
    const bool edges = d.m > 0 && d.n > 0 && k_ok && (kmajor || d.n % 8 == 0) && (!atrans || d.m % 8 == 0);
    // padded tile area within 1.3x of M x N (4000^2: 1.05x; 1000 rows: 1.02x), unless the
    // caller keeps the largest tile
    // (up to 4/3 on grids of 80 tiles or more: M = 192 or 384 against 256-row tiles measured ahead on
    // the 256-wide kernel from 86 tiles on, e.g. 384 x 28672 x 8192 217 against 343 us, 384 x 11008 x
    // 4096 74 against 80; behind at 43 tiles, 192 x 11008 x 4096 73 against 50)
    const __int128 padded = __int128(ftm * fs.bm) * (ftn * fs.bn), area = __int128(d.m) * d.n;
    const bool little_padding = 10 * padded <= 13 * area || (ftm * ftn >= 80 && 3 * padded <= 4 * area);
    if ((whole || (edges && (little_padding || large))) && rows16 && off32) p.kid = fk;
    // Fewer than 32 full-tile workgroups leave most CUs idle: 64 x 64 tiles of
    // the general kernel give 16 times as many and finish sooner (measured at
    // 1 to 24 workgroups; from 64 on the full-tile kernel is faster).  With
    // edge tiles the bar is 64 workgroups (measured: 40 edge tiles 11.1 us on
    // the general kernel against 15.0; 96 tiles 16.9 against 12.1).
    if (!large && p.kid == fk && ftm * ftn * d.batch < (whole ? 32 : 64)) p.kid = lak::KID_TILED_64;
    // Up to 128 tiles of 256 x 256 (plain GEMMs, A stored [M, K]): 128-row tiles, twice as many
    // workgroups on the otherwise idle CUs.  Measured on one box (bf16 -> bf16, 256-row -> 128-row
    // tiles, us): 192 x 28672 x 8192 188.9 -> 148.6 (B [N, K] 193.3 -> 165.4); 256 x 28672 x 8192
    // 210.3 -> 161.3; 384 x 11008 x 4096 69.9 -> 56.6; 512 x 11008 x 4096 70.1 -> 62.0;
    // 1024 x 4096 x 14336 224.0 -> 173.6 (278.8 -> 215.7); 2048 x 4096 x 4096 79.3 -> 73.2; from
    // 172 tiles on slower (1024 x 11008 x 4096 88.5 -> 117.3, 384 x 28672 x 8192 209.7 -> 265.9,
    // 4096^3 109.4 -> 136.5).
    if (!large && (p.kid == lak::KID_FAST_256 || p.kid == lak::KID_FAST_256_KM) && ftm * ftn * d.batch <= 128)
      p.kid = kmajor ? lak::KID_FAST_128_KM : lak::KID_FAST_128;
    // with K a multiple of 64, K blocks of 64 (longer row segments per block; for the one-byte pair
    // view 64 pairs, 128 codes)
    if (d.k % 64 == 0 && (p.kid == lak::KID_FAST_128 || p.kid == lak::KID_FAST_128_KM))
      p.kid = kmajor ? lak::KID_FAST_128_KM64 : lak::KID_FAST_128_K64;
    // M <= 128: stream B once through the skinny kernel with 16, 32, 64 or 128 rows of A
    // (HBM-bound shapes); B stored [N, K] streams strips of K-contiguous rows.  With more than 32
    // rows only on grids of at least 128 strips: measured ahead of the general kernel on 28672 x
    // 8192 operands (224 or 448 strips), level with or behind it on 4096 x 14336 (32 or 64 strips),
    // where a strip's K loop is long and most CUs idle; with 32 rows ahead on both.
    const int sk = d.m <= 16 ? (kmajor ? lak::KID_SKINNY_16_KM : lak::KID_SKINNY_16)
                 : d.m <= 32 ? (kmajor ? lak::KID_SKINNY_32_KM : lak::KID_SKINNY_32)
                 : d.m <= 64 ? (kmajor ? lak::KID_SKINNY_64_KM : lak::KID_SKINNY_64)
                             : (kmajor ? lak::KID_SKINNY_128_KM : lak::KID_SKINNY_128);
    const lak::KernelShape ks = lak::kernel_shape(sk);
    const bool wide = d.m <= 32 || (d.n / ks.bn) * d.batch >= 128;
    const bool skinny_fit = !p.gate_up && !atrans && wide && d.m >= 1 && d.m <= ks.bm && d.n % ks.bn == 0 && d.k > 0 &&
                            d.k % ks.bk == 0 && in16 &&
                            2 * int64_t(ks.bm) * d.lda < (int64_t{1} << 32) &&
                            2 * int64_t(kmajor ? ks.bn : ks.bk) * d.ldb < (int64_t{1} << 32);
    if (skinny_fit) p.kid = sk;
    // Split K for the skinny shapes on grids that leave CUs idle (a single matrix): workgroups
    // = strips x split doubled while they fit one per CU (two per CU for the 16-row K-major
    // configuration, whose 80 KiB of stages seat two), each range keeping at least 4 K blocks.
    // Measured on one box (bf16, B stored [N, K] unless noted), 4096 x 14336: 16 rows 512
    // workgroups 21.5 us against 256 24.0; 32 rows 256 workgroups 24.4 against 512 26.1; 128 rows
    // 256 workgroups 37.3 against 128 48.9; B [K, N], 64 rows 256 workgroups 32.7 against 512
    // 36.6; 11008 x 4096: 16 rows 344 workgroups 20.8 against 688 21.5; B [K, N], 64 rows 172
    // workgroups 27.4 against 344 33.4.  (Against the rule: 64 rows, 4096 x 14336, 512 workgroups
    // 31.4 us, 256 36.3.)
    const bool skinny_shape_fit = !p.gate_up && !atrans && d.batch == 1 && d.m >= 1 && d.m <= ks.bm && d.n > 0 &&
                                  d.n % ks.bn == 0 && d.k > 0 && d.k % ks.bk == 0 && in16 &&
                                  2 * int64_t(ks.bm) * d.lda < (int64_t{1} << 32) &&
                                  2 * int64_t(kmajor ? ks.bn : ks.bk) * d.ldb < (int64_t{1} << 32);
    if (skinny_shape_fit) {
      const int64_t strips = d.n / ks.bn, nk = d.k / ks.bk;
      const int64_t lds = 2 * int64_t(ks.stages) * lak::stage_elems(ks, false);
      const int64_t slots = 256 * (ks.bm == 16 && lds <= 80 * 1024 ? 2 : 1);
      int split = 1;
      while (strips * split * 2 <= slots && nk % (2 * split) == 0 && nk / (2 * split) >= 4 && split < 16) split *= 2;
      if (split > 1) {
        p.split = split;
        p.split_kid = sk;
        p.split_tiles_n = static_cast<int>(strips);
        p.ws_bytes = int64_t(split) * d.m * d.n * 4;
      }
    }
    // Split K for the full-tile kernel on grids of at most 128 tiles of 256 x 256 (a single matrix
    // the skinny kernel does not take), on 128-row tiles: the largest power-of-two split count (at
    // most 8) that keeps 128-row tiles x split within 256 workgroups and gives each range at least
    // 1024 of K in whole K blocks (of 64 when K allows, else of 32); FP32 partials in rows of n values (n % 8
    // == 0: the kernel's 8-value row chunks).  Measured on one box (bf16, partials + a library sum
    // against the 256-row split, us, B [N, K] / [K, N]): 512 x 4096 x 14336 4 ranges 71.6 + 8 /
    // 72.9 + 8 against 88.0 / 83.5; 1024 x 4096 x 14336 2 ranges 120.5 + 8 against 147.7;
    // 256 x 11008 x 4096 2 ranges 40.2 + 8 against 51.3; 256 x 4096 x 14336 8 ranges 47.2 + 8
    // against 55.7.  Earlier, on 256-row tiles: 512 x 4096 x 14336 240 (single pass) -> 91 against
    // torch.matmul 85; grids of 86 tiles of 256 and more gained nothing (512 x 11008 x 4096 77 ->
    // 83), where 128-row tiles x 2 exceed 256 workgroups anyway.
    const int64_t ftiles = ftm * ftn, htm = (d.m + 127) / 128;
    if (p.split == 1 && !p.gate_up && !atrans && d.batch == 1 && (whole || edges) && in16 && off32 &&
        d.n % 8 == 0 && ftiles <= 128) {
      int split = 1;
      while (split < 8 && htm * ftn * split * 2 <= 256) split *= 2;
      // the largest such count whose ranges are whole K blocks (of 64 first) and at least 1024 deep
      // (shorter ranges do not repay the partial sums' traffic and second launch)
      bool k64 = false;
      for (; split > 1; split /= 2) {
        if (d.k / split < 1024) continue;
        if (d.k % (int64_t(64) * split) == 0) { k64 = true; break; }
        if (d.k % (int64_t(32) * split) == 0) break;
      }
      if (split > 1) {
        p.split = split;
        p.split_kid = kmajor ? (k64 ? lak::KID_FAST_128_KM64 : lak::KID_FAST_128_KM)
                             : (k64 ? lak::KID_FAST_128_K64 : lak::KID_FAST_128);
        p.split_tiles_m = static_cast<int>(htm);
        p.split_tiles_n = static_cast<int>(ftn);
        p.ws_bytes = int64_t(split) * d.m * d.n * 4;
      }
    }
    // The general kernel: 64 x 64 tiles (two register sets of prefetch with
    // 16-byte loads) measured faster than 128 x 128 at every size with 16-byte
    // loads but 4000 x 4000 x 1000 (3 % slower), and with 2-byte loads up to
    // grids of about 400 workgroups of 128 x 128 (e.g. 104 at 1000 x 1537).
    if (!large && p.kid == lak::KID_TILED_128) {
      const int64_t wg128 = ((d.m + 127) / 128) * ((d.n + 127) / 128) * d.batch;
      if (p.vec != 1 || wg128 < 384) p.kid = lak::KID_TILED_64;
    }
  }
  }  // 16-bit inputs
  p.shape = lak::kernel_shape(p.kid);
  if (p.shape.b_follows_storage && !kmajor) {
    // general kernel, B stored N-contiguous: the B block stays N-contiguous in LDS
    p.shape.b_kmajor = 0;
    for (int i = 0; i < 3; ++i) p.shape.sw_b[i] = p.shape.sw_bn[i];
  }
  if (p.shape.a_follows_storage && atrans) {
    // general kernel, A stored [K, M]: the A block stays M-contiguous in LDS
    p.shape.a_trans = 1;
    for (int i = 0; i < 3; ++i) p.shape.sw_a[i] = p.shape.sw_am[i];
  }
  const auto& s = p.shape;
  // The fast kernels write C with 16-byte vectors, so C rows start on 16 bytes.
  const bool fast = fast_kid(p.kid);
  p.out_align_bytes = fast ? 16 : p.out_bytes;
  // The direct-load kernels need 16-byte rows (their planning checked in16 above).
  if (fast || skinny_kid(p.kid)) p.align_bytes = 16;
  p.tiles_m = static_cast<int>((d.m + s.bm - 1) / s.bm);
  p.tiles_n = static_cast<int>((d.n + s.bn - 1) / s.bn);
  // one launch: the grid's work-items along x (tiles x threads per tile) must fit in 32 bits
  if (int64_t(p.tiles_m) * p.tiles_n * s.threads > int64_t(UINT32_MAX)) {
    fail(err, "too many tiles for one launch");
    return GEMM_ERR_UNSUPPORTED;
  }
  p.grid = p.tiles_m * p.tiles_n;
  // 64 x 64 tiles of a plain GEMM with 16-byte loads on grids of one to two
  // workgroups per CU (257 to 512 of them): three K blocks in flight instead
  // of two (measured 6-9 % faster there: the deeper prefetch needs 240
  // registers, one wave per SIMD, which still seats two workgroups of two
  // waves per CU; at 256 and fewer it measured no gain, above 512 the second
  // workgroup per SIMD is worth more)
  const int64_t wgs = int64_t(p.grid) * d.batch;
  if (p.kid == lak::KID_TILED_64 && p.vec != 1 && !p.gate_up && !atrans && wgs > 256 && wgs <= 512) p.kid = lak::KID_TILED_64_P3;
  p.group_m = 8;

  try {
    const la::Swizzle swa(s.sw_a[0], s.sw_a[1], s.sw_a[2]);
    const la::Swizzle swb(s.sw_b[0], s.sw_b[1], s.sw_b[2]);
    using la::Tree;
    // K-contiguous block of `rows` rows: one row of bk values, or bk / k_sub sub-blocks of k_sub
    // values per row ((rows, (k_sub, bk/k_sub)) : (k_sub, (1, rows*k_sub)), the K mode nested)
    auto kmode = [&](int64_t rows, Tree& sh, Tree& st) {
      if (s.k_sub) {
        sh = Tree::T({Tree::L(s.k_sub), Tree::L(s.bk / s.k_sub)});
        st = Tree::T({Tree::L(1), Tree::L(rows * s.k_sub)});
      } else {
        sh = Tree::L(s.bk);
        st = Tree::L(1);
      }
    };
    const int64_t krow = s.k_sub ? s.k_sub : s.bk;   // stride between rows of a K-contiguous block
    Tree ksh, kst;
    kmode(s.bm, ksh, kst);
    p.lds_a = s.a_trans ? la::View(swa, la::Layout::col_major(s.bm, s.bk, s.bm))   // (m, k) -> k*BM + m
                        : la::View(swa, la::Layout(Tree::T({Tree::L(s.bm), ksh}), Tree::T({Tree::L(krow), kst})));  // (m, k) -> m*BK + k
    kmode(s.bn, ksh, kst);
    p.lds_b = s.b_kmajor ? la::View(swb, la::Layout(Tree::T({ksh, Tree::L(s.bn)}), Tree::T({kst, Tree::L(krow)})))  // (k, n) -> n*BK + k
                         : la::View(swb, la::Layout::row_major(s.bk, s.bn, s.bn));  // (k, n) -> k*BN + n
    p.lds_b2 = p.lds_b;
    p.base_a = 0;
    p.base_b = int64_t(s.bm) * s.bk;
    p.base_b2 = p.base_b + int64_t(s.bn) * s.bk;
    p.stage_elems = lak::stage_elems(s, p.gate_up);
    p.lds_bytes = int64_t(s.stages) * p.stage_elems * s.in_bytes;
    if (s.wave_split) {
      // the SwiGLU epilogue of waves split by weight exchanges FP32 bands through two regions of
      // 4 waves x (tn / 32) blocks x 64 lanes x 16 floats, plus a 32 x (tn + 8) float window per wave
      const int64_t tn = int64_t(s.nb) * s.bn / s.waves_n, nw = int64_t(s.waves_m) * s.waves_n;
      p.lds_bytes = std::max(p.lds_bytes, (2 * 4 * (tn / 32) * 64 * 16 + nw * 32 * (tn + 8)) * 4);
    }
    if (p.lds_bytes > kMaxLdsBytes) { fail(err, "LDS footprint exceeds 160 KiB"); return GEMM_ERR_RESOURCE; }
    if (!check_block(p.lds_a, p.base_a, int64_t(s.bm) * s.bk, "A", err) ||
        !check_block(p.lds_b, p.base_b, int64_t(s.bn) * s.bk, "B", err) ||
        (p.gate_up && !check_block(p.lds_b2, p.base_b2, int64_t(s.bn) * s.bk, "W_up", err)))
      return GEMM_ERR_RESOURCE;
    if (s.in_bytes == 4) {
      if (!(s.a_trans ? check_copy_f32(p, p.lds_a, s.bk, s.bm, false, false, "A", err)
                      : check_copy_f32(p, p.lds_a, s.bm, s.bk, true, true, "A", err)) ||
          !(s.b_kmajor ? check_copy_f32(p, p.lds_b, s.bn, s.bk, true, false, "B", err)
                       : check_copy_f32(p, p.lds_b, s.bk, s.bn, false, true, "B", err)))
        return GEMM_ERR_RESOURCE;
    } else if (s.direct) {
      if (!check_copy_direct(p.lds_a, s.bm, s.bk, !s.a_trans, "A", err) ||
          !check_copy_direct(p.lds_b, s.bk, s.bn, !s.b_kmajor, "B", err))
        return GEMM_ERR_RESOURCE;
    } else if (!(s.a_trans ? check_copy_a_t(p, err) : check_copy_a(p, err)) ||
               !(p.b_kmajor ? check_copy_b_rows(p, p.lds_b, err) : check_copy_b(p, p.lds_b, err))) {
      return GEMM_ERR_RESOURCE;
    }
    if (s.in_bytes == 4) {
      if ((!s.a_trans && !check_fragment_reads_f32(p.lds_a, s.bm, s.bk, true, "A", err)) ||
          (s.b_kmajor && !check_fragment_reads_f32(p.lds_b, s.bn, s.bk, false, "B", err)))
        return GEMM_ERR_RESOURCE;
    } else if (!check_fragment_reads(p, err)) {
      return GEMM_ERR_RESOURCE;
    }
    if (!check_ownership(p, err)) return GEMM_ERR_RESOURCE;
    if (!plan_copies(p, err)) return GEMM_ERR_RESOURCE;
    // rings in storage order: (k, m) for A stored [K, M], (n, k) for B stored [N, K] (permute()
    // reverses the block map's modes)
    if (!(s.a_trans ? check_ring(la::View(p.lds_a.swizzle(), la::permute(p.lds_a.base())), s.bk, s.bm,
                                 p.stage_elems, s.stages, "A", err)
                    : check_ring(p.lds_a, s.bm, s.bk, p.stage_elems, s.stages, "A", err)) ||
        !(s.b_kmajor ? check_ring(la::View(p.lds_b.swizzle(), la::permute(p.lds_b.base())), s.bn, s.bk,
                                  p.stage_elems, s.stages, "B", err)
                     : check_ring(p.lds_b, s.bk, s.bn, p.stage_elems, s.stages, "B", err)))
      return GEMM_ERR_RESOURCE;
    if (!plan_stores(p, err)) return GEMM_ERR_RESOURCE;
  } catch (const la::LayoutError& e) {
    fail(err, e.what());
    return GEMM_ERR_RESOURCE;
  }

  p.json = describe(p);
  return GEMM_OK;
}

gemm_status lds_offset(const gemm_plan_s& p, int operand, int64_t row, int64_t col, int64_t* out, std::string* err) {
  const la::View* v = nullptr;
  int64_t base = 0;
  if (operand == 0) { v = &p.lds_a; base = p.base_a; }
  else if (operand == 1) { v = &p.lds_b; base = p.base_b; }
  else if (operand == 2 && p.gate_up) { v = &p.lds_b2; base = p.base_b2; }
  else { fail(err, "operand must be 0 (A), 1 (B) or 2 (W_up of a gate/up plan)"); return GEMM_ERR_INVALID_ARG; }
  try {
    *out = base + v->at({row, col});
  } catch (const la::LayoutError& e) {
    fail(err, e.what());
    return GEMM_ERR_INVALID_ARG;
  }
  return GEMM_OK;
}

}  // namespace plan

namespace plan {
bool is_fast(int kid) { return fast_kid(kid); }
}  // namespace plan
