"""Layout algebra written out by enumeration (test infrastructure only).

A plain Python statement of the coordinate maps the Tylo.jl page "Layouts,
storage and ownership" describes, used to pin the C++ planner bit-exactly.
Shapes and strides are ints or nested tuples of ints.  Everything here is
direct evaluation or brute-force enumeration; nothing is optimised.

Facts followed (page and section):
  * "A layout is a function": a layout maps zero-based coordinates to offsets
    as the sum of coordinate*stride over the leaves; shapes and strides may
    nest; an integer coordinate is split first-mode-fastest; tile() splits each
    flat mode into (within-tile, tile-index); coalesce() drops unit modes and
    merges contiguous ones without changing the map on the linear domain;
    permutedims() reverses the top-level modes; compose(f, l) is f(l(c)).
  * "Swizzle phase belongs to the allocation": Swizzle{B,M,S} XORs two
    disjoint bit fields and keeps the low M bits; a window keeps its parent's
    map and origin; nested windows add origins; cosize counts storage up to the
    largest offset, holes and the window's prefix included; constructors and
    windows check their domains.
  * Tylo.jl "TMA and Hopper WGMMA", section "The same storage contract on both
    sides": a shared tile plan uses Swizzle{B,M,3} over packed rows, with M the
    16-byte-chunk bits and 2^B chunks per row of 128, 64 or 32 bytes.

Readings where the pages leave a point open:
  * Swizzle bit positions: the field of B bits starting at bit M+S is XORed
    into the field of B bits starting at bit M; the fields are disjoint iff
    S >= B (B = 0 is the identity).  Negative parameters are rejected.
  * tile() needs each tile extent to divide its mode and each tiled mode to be
    flat.
  * A window's origin and extent are given per top-level mode; it must lie
    inside the parent's domain.
"""
from itertools import product


# ---------------------------------------------------------------- int tuples
def is_int(x):
    return isinstance(x, int) and not isinstance(x, bool)


def size(shape):
    if is_int(shape):
        return shape
    n = 1
    for s in shape:
        n *= size(s)
    return n


def leaves(t):
    if is_int(t):
        return [t]
    out = []
    for x in t:
        out.extend(leaves(x))
    return out


def congruent(a, b):
    if is_int(a) or is_int(b):
        return is_int(a) and is_int(b)
    return len(a) == len(b) and all(congruent(x, y) for x, y in zip(a, b))


def split_index(i, shape):
    """Integer index -> natural coordinate of `shape`, first mode fastest."""
    if is_int(shape):
        return i
    coord = []
    for s in shape:
        n = size(s)
        coord.append(split_index(i % n, s))
        i //= n
    return tuple(coord)


def _offset(coord, shape, stride):
    if is_int(shape):
        if not is_int(coord):
            raise ValueError("coordinate %r does not fit leaf mode %r" % (coord, shape))
        if not 0 <= coord < shape:
            raise IndexError("coordinate %d outside mode of extent %d" % (coord, shape))
        return coord * stride
    if is_int(coord):
        if not 0 <= coord < size(shape):
            raise IndexError("coordinate %d outside mode of size %d" % (coord, size(shape)))
        coord = split_index(coord, shape)
    if len(coord) != len(shape):
        raise ValueError("coordinate %r has the wrong rank for shape %r" % (coord, shape))
    return sum(_offset(c, s, d) for c, s, d in zip(coord, shape, stride))


# ---------------------------------------------------------------- layouts
class Layout:
    def __init__(self, shape, stride):
        if not congruent(shape, stride):
            raise ValueError("shape %r and stride %r are not congruent" % (shape, stride))
        if any(s <= 0 for s in leaves(shape)):
            raise ValueError("extents must be positive: %r" % (shape,))
        self.shape = shape
        self.stride = stride

    def __call__(self, coord):
        return _offset(coord, self.shape, self.stride)

    def size(self):
        return size(self.shape)

    def top_extents(self):
        return (self.shape,) if is_int(self.shape) else tuple(size(s) for s in self.shape)

    def __repr__(self):
        return "%r:%r" % (self.shape, self.stride)


def permutedims(layout):
    """Reverse the top-level modes of shape and stride together."""
    if is_int(layout.shape):
        return Layout(layout.shape, layout.stride)
    return Layout(tuple(reversed(layout.shape)), tuple(reversed(layout.stride)))


def tile(layout, tiles):
    """Split flat top-level mode i into (tiles[i], extent/tiles[i])."""
    shape = (layout.shape,) if is_int(layout.shape) else layout.shape
    stride = (layout.stride,) if is_int(layout.stride) else layout.stride
    if len(tiles) != len(shape):
        raise ValueError("one tile extent per top-level mode")
    new_shape, new_stride = [], []
    for s, d, t in zip(shape, stride, tiles):
        if not is_int(s):
            raise ValueError("tile() needs flat modes")
        if t <= 0 or s % t:
            raise ValueError("tile extent %d does not divide %d" % (t, s))
        new_shape.append((t, s // t))
        new_stride.append((d, t * d))
    return Layout(tuple(new_shape), tuple(new_stride))


def coalesce(layout):
    """Drop unit modes, merge (s0:d0)(s1:d1) with d1 == s0*d0; first-mode-fastest order."""
    pairs = [(s, d) for s, d in zip(leaves(layout.shape), leaves(layout.stride)) if s != 1]
    merged = []
    for s, d in pairs:
        if merged and d == merged[-1][0] * merged[-1][1]:
            merged[-1] = (merged[-1][0] * s, merged[-1][1])
        else:
            merged.append((s, d))
    if not merged:
        return Layout(1, 0)
    if len(merged) == 1:
        return Layout(merged[0][0], merged[0][1])
    return Layout(tuple(s for s, _ in merged), tuple(d for _, d in merged))


class Swizzle:
    """Offset permutation: XOR the B bits at [M+S, M+S+B) into [M, M+B)."""

    def __init__(self, B, M, S):
        if B < 0 or M < 0 or S < 0:
            raise ValueError("negative swizzle parameter")
        if B > 0 and S < B:
            raise ValueError("Swizzle{%d,%d,%d}: overlapping bit fields" % (B, M, S))
        self.B, self.M, self.S = B, M, S

    def __call__(self, offset):
        low_mask = ((1 << self.B) - 1) << self.M
        return offset ^ ((offset >> self.S) & low_mask)

    def period(self):
        """Offsets repeat their XOR pattern every 2^(M+S+B) elements."""
        return 1 << (self.M + self.S + self.B)


class Composed:
    """f(inner(c)) for an offset function f over a layout-like inner."""

    def __init__(self, f, inner):
        self.f = f
        self.inner = inner
        self.shape = inner.shape

    def __call__(self, coord):
        return self.f(self.inner(coord))

    def size(self):
        return self.inner.size()

    def top_extents(self):
        return self.inner.top_extents()


def compose(f, layout):
    return Composed(f, layout)


class Window:
    """A sub-box of a parent map that keeps the parent's offsets (and swizzle phase)."""

    def __init__(self, parent, origin, shape):
        ext = parent.top_extents()
        if len(origin) != len(ext) or len(shape) != len(ext):
            raise ValueError("window origin/shape rank must match the parent's top-level rank")
        for o, s, e in zip(origin, shape, ext):
            if o < 0 or s <= 0 or o + s > e:
                raise IndexError("window [%d, %d) outside mode of extent %d" % (o, o + s, e))
        self.parent = parent
        self.origin = tuple(origin)
        self.shape = tuple(shape)

    def __call__(self, coord):
        if is_int(coord):
            coord = split_index(coord, self.shape)
        if len(coord) != len(self.shape):
            raise ValueError("window coordinate rank mismatch")
        for c, s in zip(coord, self.shape):
            if not 0 <= c < s:
                raise IndexError("coordinate outside window")
        return self.parent(tuple(o + c for o, c in zip(self.origin, coord)))

    def size(self):
        return size(self.shape)

    def top_extents(self):
        return self.shape


def window(parent, origin, shape):
    return Window(parent, origin, shape)


def cosize(f):
    """1 + the largest offset over the whole domain (by enumeration)."""
    return 1 + max(f(i) for i in range(f.size()))


def all_coords(extents):
    """Every top-level coordinate tuple, first mode fastest."""
    for rev in product(*[range(e) for e in reversed(extents)]):
        yield tuple(reversed(rev))


# ---------------------------------------------------------------- shared tile plan
class SharedTilePlan:
    """A 2-D shared-memory tile whose inner axis is one swizzle row.

    elem_bytes in {1, 2, 4}; shape = (d1, d2); inner_axis in {1, 2} (1-based,
    as the page writes it); row_bytes in {128, 64, 32}.  The inner extent must
    be exactly one row; the outer extent a multiple of 8, at most 256.
    """

    def __init__(self, elem_bytes, shape, inner_axis, row_bytes=128):
        if elem_bytes not in (1, 2, 4):
            raise ValueError("element size must be 1, 2 or 4 bytes")
        if row_bytes not in (32, 64, 128):
            raise ValueError("swizzle row must be 128, 64 or 32 bytes")
        if inner_axis not in (1, 2):
            raise ValueError("inner axis is 1 or 2")
        d1, d2 = shape
        inner = d1 if inner_axis == 1 else d2
        outer = d2 if inner_axis == 1 else d1
        if inner * elem_bytes != row_bytes:
            raise ValueError("inner extent must be one %d-byte row" % row_bytes)
        if outer % 8 or not 0 < outer <= 256:
            raise ValueError("outer extent must be a multiple of 8, at most 256")
        self.elem_bytes = elem_bytes
        self.shape = (d1, d2)
        self.inner_axis = inner_axis
        self.row_bytes = row_bytes
        m_bits = (16 // elem_bytes).bit_length() - 1      # elements per 16-byte chunk
        b_bits = (row_bytes // 16).bit_length() - 1       # chunks per row
        self.swizzle = Swizzle(b_bits, m_bits, 3)
        if inner_axis == 2:
            base = Layout((d1, d2), (d2, 1))
        else:
            base = Layout((d1, d2), (1, d1))
        self.layout = compose(self.swizzle, base)

    def transfer_bytes(self):
        return self.shape[0] * self.shape[1] * self.elem_bytes

    def swizzle_bytes(self):
        return self.row_bytes

    def size(self):
        return self.shape

    def shared_layout(self):
        return self.layout
