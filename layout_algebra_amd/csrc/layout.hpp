// Host-side layout algebra for planning LDS tiles and copies.
//
// Follows the Tylo.jl page "Layouts, storage and ownership":
//  * section "A layout is a function": a layout maps zero-based coordinates to
//    offsets (sum of coordinate x stride over the leaves of possibly nested
//    shape/stride trees); an integer coordinate splits first mode fastest;
//    tile() factors flat modes into (within-tile, tile-index); coalesce()
//    removes unit modes and merges contiguous ones; permute() reverses the
//    top-level modes; composition applies an offset map after a layout.
//  * section "Swizzle phase belongs to the allocation": Swizzle{B,M,S} XORs two
//    disjoint bit fields and keeps the low M bits; a window keeps the parent's
//    map and origin; cosize counts storage through the largest offset (by
//    enumeration for nonlinear maps); constructors and windows check domains.
// Everything here runs on the host before a launch; kernels use the plan's
// results (compile-time tile shapes and swizzle parameters).
#pragma once

#include <cstdint>
#include <stdexcept>
#include <string>
#include <vector>

namespace la {

// A node of a shape or stride tree: a leaf integer or a tuple of nodes.
struct Tree {
  bool leaf = true;
  int64_t value = 0;
  std::vector<Tree> kids;

  static Tree L(int64_t v) { Tree t; t.leaf = true; t.value = v; return t; }
  static Tree T(std::vector<Tree> k) { Tree t; t.leaf = false; t.kids = std::move(k); return t; }
  static Tree flat(const std::vector<int64_t>& v);

  int rank() const { return leaf ? 1 : static_cast<int>(kids.size()); }
  const Tree& mode(int i) const { return leaf ? *this : kids.at(i); }
  std::string str() const;
};

int64_t size_of(const Tree& shape);
bool congruent(const Tree& a, const Tree& b);
void leaves(const Tree& t, std::vector<int64_t>& out);

struct LayoutError : std::runtime_error {
  using std::runtime_error::runtime_error;
};

class Layout {
 public:
  Layout() = default;
  Layout(Tree shape, Tree stride);
  static Layout flat(const std::vector<int64_t>& shape, const std::vector<int64_t>& stride);
  static Layout row_major(int64_t rows, int64_t cols, int64_t ld);   // (rows, cols):(ld, 1)
  static Layout col_major(int64_t rows, int64_t cols, int64_t ld);   // (rows, cols):(1, ld)

  const Tree& shape() const { return shape_; }
  const Tree& stride() const { return stride_; }
  int rank() const { return shape_.rank(); }
  int64_t size() const { return size_of(shape_); }
  int64_t mode_size(int i) const { return size_of(shape_.mode(i)); }

  // Natural coordinate (tree congruent to the shape, or ints per mode).
  int64_t operator()(const Tree& coord) const;
  // Integer index, split first mode fastest.
  int64_t operator()(int64_t idx) const;
  // One integer per top-level mode (each split first mode fastest inside its mode).
  int64_t at(const std::vector<int64_t>& top) const;

  std::string str() const { return shape_.str() + ":" + stride_.str(); }

 private:
  Tree shape_, stride_;
};

// The pages' notation: "shape:stride" with nested tuples, e.g. "((8,4),5):((1,8),128)";
// a coordinate is a nested tuple or an integer ("((3,2),1)", "(3,7)", "5").
Tree parse_tree(const std::string& text);
Layout parse_layout(const std::string& text);

Layout permute(const Layout& l);                              // reverse top-level modes
Layout tile(const Layout& l, const std::vector<int64_t>& t);  // per flat top-level mode
Layout coalesce(const Layout& l);

struct Swizzle {
  int b = 0, m = 0, s = 0;
  Swizzle() = default;
  Swizzle(int b_, int m_, int s_);   // throws LayoutError on overlapping/negative fields
  static bool valid(int b, int m, int s) { return b >= 0 && m >= 0 && s >= 0 && (b == 0 || s >= b); }
  int64_t operator()(int64_t off) const {
    const int64_t low = ((int64_t{1} << b) - 1) << m;
    return off ^ ((off >> s) & low);
  }
  int64_t period() const { return int64_t{1} << (m + s + b); }
  bool identity() const { return b == 0; }
};

// Swizzle o Layout, optionally windowed: f(c) = sw(base(origin + c)).
// Origins and extents are per top-level mode.  Nested windows add origins and
// keep the base (and therefore the swizzle phase of the allocation).
class View {
 public:
  View() = default;
  View(Swizzle sw, Layout base);
  View window(const std::vector<int64_t>& origin, const std::vector<int64_t>& extent) const;

  int64_t at(const std::vector<int64_t>& c) const;   // top-level coordinate
  int64_t operator()(int64_t idx) const;             // first-mode-fastest over the extents
  int64_t size() const;
  int rank() const { return static_cast<int>(extent_.size()); }
  const std::vector<int64_t>& extent() const { return extent_; }
  const std::vector<int64_t>& origin() const { return origin_; }
  const Swizzle& swizzle() const { return sw_; }
  const Layout& base() const { return base_; }

 private:
  Swizzle sw_;
  Layout base_;
  std::vector<int64_t> origin_, extent_;
};

int64_t cosize(const Layout& l);   // closed form for non-negative strides
int64_t cosize(const View& v);     // by enumeration (nonlinear)
bool injective(const View& v);     // by enumeration

// Shared tile plan of the Tylo.jl page "TMA and Hopper WGMMA" (section "The
// same storage contract on both sides"): a 2-D tile whose inner axis is one
// swizzle row of 128/64/32 bytes, stored as Swizzle{B,M,3} over packed rows,
// M = log2(elements per 16-byte chunk), 2^B chunks per row.
struct SharedTilePlan {
  int elem_bytes = 2;
  int64_t d1 = 0, d2 = 0;
  int inner_axis = 2;   // 1 or 2 (1-based, as the page writes it)
  int row_bytes = 128;
  View layout;

  SharedTilePlan(int elem_bytes, int64_t d1, int64_t d2, int inner_axis, int row_bytes);
  int64_t transfer_bytes() const { return d1 * d2 * elem_bytes; }
};

}  // namespace la
