// Host-side layout algebra (see layout.hpp for the semantics and sources).
#include "layout.hpp"

#include <algorithm>
#include <sstream>

namespace la {

Tree Tree::flat(const std::vector<int64_t>& v) {
  if (v.size() == 1) return L(v[0]);
  std::vector<Tree> k;
  k.reserve(v.size());
  for (int64_t x : v) k.push_back(L(x));
  return T(std::move(k));
}

std::string Tree::str() const {
  if (leaf) return std::to_string(value);
  std::ostringstream os;
  os << "(";
  for (size_t i = 0; i < kids.size(); ++i) os << (i ? "," : "") << kids[i].str();
  os << ")";
  return os.str();
}

int64_t size_of(const Tree& shape) {
  if (shape.leaf) return shape.value;
  int64_t n = 1;
  for (const Tree& k : shape.kids) n *= size_of(k);
  return n;
}

bool congruent(const Tree& a, const Tree& b) {
  if (a.leaf || b.leaf) return a.leaf && b.leaf;
  if (a.kids.size() != b.kids.size()) return false;
  for (size_t i = 0; i < a.kids.size(); ++i)
    if (!congruent(a.kids[i], b.kids[i])) return false;
  return true;
}

void leaves(const Tree& t, std::vector<int64_t>& out) {
  if (t.leaf) { out.push_back(t.value); return; }
  for (const Tree& k : t.kids) leaves(k, out);
}

namespace {

// Offset of an integer index inside a (sub)mode, first mode fastest.
int64_t index_offset(int64_t idx, const Tree& shape, const Tree& stride) {
  if (shape.leaf) return idx * stride.value;
  int64_t off = 0;
  for (size_t i = 0; i < shape.kids.size(); ++i) {
    const int64_t n = size_of(shape.kids[i]);
    off += index_offset(idx % n, shape.kids[i], stride.kids[i]);
    idx /= n;
  }
  return off;
}

int64_t coord_offset(const Tree& c, const Tree& shape, const Tree& stride) {
  if (c.leaf) {
    if (c.value < 0 || c.value >= size_of(shape))
      throw LayoutError("coordinate " + std::to_string(c.value) + " outside mode " + shape.str());
    return index_offset(c.value, shape, stride);
  }
  if (shape.leaf || c.kids.size() != shape.kids.size())
    throw LayoutError("coordinate " + c.str() + " does not match shape " + shape.str());
  int64_t off = 0;
  for (size_t i = 0; i < c.kids.size(); ++i) off += coord_offset(c.kids[i], shape.kids[i], stride.kids[i]);
  return off;
}

}  // namespace

Layout::Layout(Tree shape, Tree stride) : shape_(std::move(shape)), stride_(std::move(stride)) {
  if (!congruent(shape_, stride_)) throw LayoutError("shape " + shape_.str() + " and stride " + stride_.str() + " are not congruent");
  std::vector<int64_t> s;
  leaves(shape_, s);
  for (int64_t v : s)
    if (v <= 0) throw LayoutError("extents must be positive: " + shape_.str());
}

Layout Layout::flat(const std::vector<int64_t>& shape, const std::vector<int64_t>& stride) {
  if (shape.empty() || shape.size() != stride.size()) throw LayoutError("flat layout needs equal, non-zero ranks");
  return Layout(Tree::flat(shape), Tree::flat(stride));
}
Layout Layout::row_major(int64_t rows, int64_t cols, int64_t ld) { return flat({rows, cols}, {ld, 1}); }
Layout Layout::col_major(int64_t rows, int64_t cols, int64_t ld) { return flat({rows, cols}, {1, ld}); }

int64_t Layout::operator()(const Tree& coord) const { return coord_offset(coord, shape_, stride_); }

int64_t Layout::operator()(int64_t idx) const {
  if (idx < 0 || idx >= size()) throw LayoutError("index " + std::to_string(idx) + " outside layout of size " + std::to_string(size()));
  return index_offset(idx, shape_, stride_);
}

int64_t Layout::at(const std::vector<int64_t>& top) const {
  if (static_cast<int>(top.size()) != rank()) throw LayoutError("coordinate rank mismatch");
  int64_t off = 0;
  for (int i = 0; i < rank(); ++i) {
    const Tree& s = shape_.mode(i);
    if (top[i] < 0 || top[i] >= size_of(s)) throw LayoutError("coordinate outside mode " + s.str());
    off += index_offset(top[i], s, stride_.mode(i));
  }
  return off;
}

namespace {

void skip_spaces(const std::string& t, size_t& i) {
  while (i < t.size() && (t[i] == ' ' || t[i] == '\t')) ++i;
}

Tree parse_node(const std::string& t, size_t& i, int depth) {
  if (depth > 64) throw LayoutError("nesting too deep in '" + t + "'");
  skip_spaces(t, i);
  if (i < t.size() && t[i] == '(') {
    ++i;
    std::vector<Tree> kids;
    for (;;) {
      kids.push_back(parse_node(t, i, depth + 1));
      skip_spaces(t, i);
      if (i < t.size() && t[i] == ',') { ++i; continue; }
      if (i < t.size() && t[i] == ')') { ++i; break; }
      throw LayoutError("expected ',' or ')' at position " + std::to_string(i) + " of '" + t + "'");
    }
    // a one-element tuple is that element (as the pages write (n,) for a single mode)
    return kids.size() == 1 ? kids[0] : Tree::T(std::move(kids));
  }
  size_t j = i;
  if (j < t.size() && t[j] == '-') ++j;
  const size_t digits = j;
  while (j < t.size() && t[j] >= '0' && t[j] <= '9') ++j;
  if (j == digits || j - digits > 18) throw LayoutError("expected an integer at position " + std::to_string(i) + " of '" + t + "'");
  const int64_t v = std::stoll(t.substr(i, j - i));
  i = j;
  return Tree::L(v);
}

}  // namespace

Tree parse_tree(const std::string& text) {
  size_t i = 0;
  Tree r = parse_node(text, i, 0);
  skip_spaces(text, i);
  if (i != text.size()) throw LayoutError("trailing characters in '" + text + "'");
  return r;
}

Layout parse_layout(const std::string& text) {
  // the colon that separates shape and stride sits outside every parenthesis
  int depth = 0;
  size_t colon = std::string::npos;
  for (size_t i = 0; i < text.size(); ++i) {
    if (text[i] == '(') ++depth;
    else if (text[i] == ')') --depth;
    else if (text[i] == ':' && depth == 0) {
      if (colon != std::string::npos) throw LayoutError("more than one ':' in '" + text + "'");
      colon = i;
    }
  }
  if (colon == std::string::npos) throw LayoutError("a layout is written shape:stride, got '" + text + "'");
  return Layout(parse_tree(text.substr(0, colon)), parse_tree(text.substr(colon + 1)));
}

Layout permute(const Layout& l) {
  if (l.shape().leaf) return l;
  std::vector<Tree> s(l.shape().kids.rbegin(), l.shape().kids.rend());
  std::vector<Tree> d(l.stride().kids.rbegin(), l.stride().kids.rend());
  return Layout(Tree::T(std::move(s)), Tree::T(std::move(d)));
}

Layout tile(const Layout& l, const std::vector<int64_t>& t) {
  if (static_cast<int>(t.size()) != l.rank()) throw LayoutError("tile needs one extent per top-level mode");
  std::vector<Tree> s, d;
  for (int i = 0; i < l.rank(); ++i) {
    const Tree& si = l.shape().mode(i);
    const Tree& di = l.stride().mode(i);
    if (!si.leaf) throw LayoutError("tile needs flat modes");
    if (t[i] <= 0 || si.value % t[i] != 0)
      throw LayoutError("tile extent " + std::to_string(t[i]) + " does not divide " + std::to_string(si.value));
    s.push_back(Tree::T({Tree::L(t[i]), Tree::L(si.value / t[i])}));
    d.push_back(Tree::T({Tree::L(di.value), Tree::L(t[i] * di.value)}));
  }
  return Layout(Tree::T(std::move(s)), Tree::T(std::move(d)));
}

Layout coalesce(const Layout& l) {
  std::vector<int64_t> s, d;
  leaves(l.shape(), s);
  leaves(l.stride(), d);
  std::vector<int64_t> ms, md;
  for (size_t i = 0; i < s.size(); ++i) {
    if (s[i] == 1) continue;
    if (!ms.empty() && d[i] == ms.back() * md.back()) {
      ms.back() *= s[i];
    } else {
      ms.push_back(s[i]);
      md.push_back(d[i]);
    }
  }
  if (ms.empty()) return Layout(Tree::L(1), Tree::L(0));
  return Layout::flat(ms, md);
}

Swizzle::Swizzle(int b_, int m_, int s_) : b(b_), m(m_), s(s_) {
  if (!valid(b, m, s))
    throw LayoutError("Swizzle{" + std::to_string(b) + "," + std::to_string(m) + "," + std::to_string(s) +
                      "}: bit fields overlap or a parameter is negative");
}

View::View(Swizzle sw, Layout base) : sw_(sw), base_(std::move(base)) {
  origin_.assign(base_.rank(), 0);
  for (int i = 0; i < base_.rank(); ++i) extent_.push_back(base_.mode_size(i));
}

View View::window(const std::vector<int64_t>& origin, const std::vector<int64_t>& extent) const {
  if (origin.size() != extent_.size() || extent.size() != extent_.size())
    throw LayoutError("window rank must match the parent's top-level rank");
  View w = *this;
  for (size_t i = 0; i < extent_.size(); ++i) {
    if (origin[i] < 0 || extent[i] <= 0 || origin[i] + extent[i] > extent_[i])
      throw LayoutError("window outside its parent's domain");
    w.origin_[i] = origin_[i] + origin[i];
    w.extent_[i] = extent[i];
  }
  return w;
}

int64_t View::at(const std::vector<int64_t>& c) const {
  if (c.size() != extent_.size()) throw LayoutError("coordinate rank mismatch");
  std::vector<int64_t> p(c.size());
  for (size_t i = 0; i < c.size(); ++i) {
    if (c[i] < 0 || c[i] >= extent_[i]) throw LayoutError("coordinate outside window");
    p[i] = origin_[i] + c[i];
  }
  return sw_(base_.at(p));
}

int64_t View::size() const {
  int64_t n = 1;
  for (int64_t e : extent_) n *= e;
  return n;
}

int64_t View::operator()(int64_t idx) const {
  std::vector<int64_t> c(extent_.size());
  for (size_t i = 0; i < extent_.size(); ++i) {
    c[i] = idx % extent_[i];
    idx /= extent_[i];
  }
  return at(c);
}

int64_t cosize(const Layout& l) {
  std::vector<int64_t> s, d;
  leaves(l.shape(), s);
  leaves(l.stride(), d);
  int64_t hi = 0;
  for (size_t i = 0; i < s.size(); ++i) {
    if (d[i] < 0) throw LayoutError("closed-form cosize needs non-negative strides");
    hi += (s[i] - 1) * d[i];
  }
  return hi + 1;
}

int64_t cosize(const View& v) {
  int64_t hi = -1;
  const int64_t n = v.size();
  for (int64_t i = 0; i < n; ++i) hi = std::max(hi, v(i));
  return hi + 1;
}

bool injective(const View& v) {
  std::vector<int64_t> offs;
  offs.reserve(v.size());
  for (int64_t i = 0; i < v.size(); ++i) offs.push_back(v(i));
  std::sort(offs.begin(), offs.end());
  return std::adjacent_find(offs.begin(), offs.end()) == offs.end();
}

namespace {
int log2_exact(int64_t v) {
  int r = 0;
  while ((int64_t{1} << r) < v) ++r;
  if ((int64_t{1} << r) != v) throw LayoutError("not a power of two: " + std::to_string(v));
  return r;
}
}  // namespace

SharedTilePlan::SharedTilePlan(int eb, int64_t a, int64_t b, int inner, int rb)
    : elem_bytes(eb), d1(a), d2(b), inner_axis(inner), row_bytes(rb) {
  if (eb != 1 && eb != 2 && eb != 4) throw LayoutError("element size must be 1, 2 or 4 bytes");
  if (rb != 128 && rb != 64 && rb != 32) throw LayoutError("swizzle row must be 128, 64 or 32 bytes");
  if (inner != 1 && inner != 2) throw LayoutError("inner axis must be 1 or 2");
  const int64_t inner_ext = inner == 1 ? d1 : d2;
  const int64_t outer_ext = inner == 1 ? d2 : d1;
  if (inner_ext * eb != rb) throw LayoutError("inner extent must be exactly one swizzle row");
  if (outer_ext <= 0 || outer_ext % 8 != 0 || outer_ext > 256)
    throw LayoutError("outer extent must be a positive multiple of 8, at most 256");
  const int m_bits = log2_exact(16 / eb);
  const int b_bits = log2_exact(rb / 16);
  const Layout base = inner == 2 ? Layout::row_major(d1, d2, d2) : Layout::col_major(d1, d2, d1);
  layout = View(Swizzle(b_bits, m_bits, 3), base);
}

}  // namespace la
