"""Descriptor encode, plan search and partition synthesis (oracle).

Sources
-------
* "copy_async -> tma", "What it accepts": a legal descriptor has rank <= 5,
  innermost stride 1, and an innermost box that fits the shared swizzle atom;
  otherwise the plan search shrinks or declines.
* "copy_async -> tma", "Algorithm" step 2: canonicalize (L1), cut each
  contiguous chain into box segments (L2), stack into a descriptor and
  validate, shrinking and retrying on failure (L3); adjacent fully-boxed
  contiguous dims merge; a box over 256 may promote the element type.
* "copy_async -> tma", "How inputs change the algorithm": a 128-byte swizzle
  on a 2-D tile yields a rank-3 descriptor (the inner axis splits into
  swizzle atoms); box > 256 triggers promotion 1 -> 2 -> 4 -> 8 bytes; and the
  final paragraph: the variant declines when no legal descriptor exists.
* "copy_async -> tma", "Generated TIRx IR": the worked 8x256 float16 example
  (rank 3, dims 64/8/4 innermost-first, byte strides 512/128, box 64/8/4).
* "Add TMA support for circular buffering pass", "Lowering Details": each box
  dimension is limited to 256, so a larger tile takes several loads.
* "elementwise -> smem", "Algorithm" step 2, and "copy_async -> ldgsts",
  "Algorithm" step 1 and "How inputs change the algorithm": the
  ``[outer, threads, vec]`` partition, the vector width as the widest legal
  aligned width, and the table of vec / cp_size / outer for 4096 elements over
  128 threads.

Readings where the pages are silent:
* The atom axis produced by the swizzle split is the OUTERMOST descriptor
  dimension: that is the only order that reproduces the worked example's
  strides (512 then 128 bytes innermost-first).
* Merging needs the inner dim fully boxed and contiguous with its outer
  neighbour, a merged box <= 256 (or, for copies of the innermost pair, one
  that promotion brings to <= 256), and under swizzle an innermost box of at
  most 128 bytes.  Atom axes never merge.
* A box > 256 that promotion cannot fix is cut into equal segments: the
  largest divisor <= 256 (for the innermost dim, one whose bytes are a
  multiple of 16 if possible, else of 4, else any).  The quotient becomes an
  issue axis.
* Under a swizzle, an innermost box wider than one atom that is not a whole
  number of atoms (or over a tensor row that is not) is shrunk the same
  way: cut into equal segments, the largest divisor whose bytes fit the atom
  and are a whole number of 16-byte chunks, the quotient an issue axis.  An
  innermost box within one atom may merge with whole rows (up to the atom);
  the plan declines when the final innermost box is no whole number of
  16-byte chunks.
* A merge joins whole boxes, and a merged dim is never cut into several
  loads again.
* "Shrinking the chain prefix": while the descriptor has more than 5 dims,
  the outermost dim leaves the descriptor and its box becomes issue axes.
  Under this reading the shrink always reaches rank <= 5, so the page's
  "rank > 5 after shrinking" decline cannot occur; the pages set no limit on
  the number of loads per tile.
* The stage's LDS image is issue-major, then box-dense row-major over the
  descriptor dims (each load writes one dense box), then swizzled.
* The element-count rule of the ldgsts page is read as: threads * vec must
  divide the region's element count (narrower vec otherwise).
* Vector widths: the ldgsts page's candidates are {16, 8, 4} bytes; the
  gfx950 direct-to-LDS loads have {16, 4} (no 8-byte form).  Both sets are
  supported through ``vec_candidates``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import swizzle as _swz

MAX_RANK = 5            # descriptor rank limit
MAX_BOX = 256           # per-dimension box limit
MAX_INPUT_RANK = 8      # rank of the tensor handed to the encoder
SWIZZLE_NONE = 0
SWIZZLE_32B = 1
SWIZZLE_64B = 2
SWIZZLE_128B = 3        # mode number of the worked example
ATOM_BYTES = 128        # the 128-byte mode's atom (16 << mode bytes in general)

ESIZE = {"u8": 1, "u16": 2, "u32": 4, "u64": 8, "f16": 2, "f32": 4}
GFX950_VEC_BYTES = (16, 4)
PAGE_VEC_BYTES = (16, 8, 4)


class Declined(Exception):
    """No legal plan (the variant declines); ``args[0]`` is the reason."""


class Invalid(Exception):
    """Malformed request (not a question of legality)."""


@dataclass
class Axis:
    """One axis of the LDS image: ``count`` indices along tensor dim ``dim``,
    each advancing that dim's coordinate by ``step`` elements."""
    count: int
    dim: int
    step: int


@dataclass
class DescDim:
    extent: int          # elements of the descriptor element type
    stride: int          # bytes
    box: int             # elements of the descriptor element type
    parts: list          # image axes of one box along this dim, row-major
    atom: bool = False
    seg_issue: Axis | None = None


@dataclass
class Plan:
    esize: int
    desc_esize: int
    shape: tuple
    strides: tuple       # elements, outermost-first
    box: tuple
    swizzle: int
    dims: list           # DescDim, outermost-first (the descriptor)
    issue_axes: list     # Axis, outermost-first
    promoted: bool = False
    threads: int = 0
    vec_bytes: int = 0
    vec: int = 0
    outer: int = 0

    @property
    def rank(self) -> int:
        return len(self.dims)

    @property
    def image_axes(self) -> list:
        """Axes of the LDS image, outermost-first (issue axes, then the box
        parts of each descriptor dim).  Axes of count 1 change nothing and are
        left out, except the innermost, which is always kept."""
        axes = list(self.issue_axes)
        for d in self.dims:
            axes.extend(d.parts)
        return [a for a in axes[:-1] if a.count > 1] + axes[-1:]

    @property
    def issues(self) -> int:
        n = 1
        for a in self.issue_axes:
            n *= a.count
        return n

    @property
    def tile_elems(self) -> int:
        n = 1
        for a in self.image_axes:
            n *= a.count
        return n

    @property
    def tile_bytes(self) -> int:
        return self.tile_elems * self.esize

    def encode_args(self):
        """The descriptor in the order of the host encode call of the pages:
        (rank, dims innermost-first, byte strides innermost-first without the
        innermost, box innermost-first, element strides, interleave, swizzle
        mode, L2 promotion, OOB fill)."""
        dims = [d.extent for d in reversed(self.dims)]
        strides = [d.stride for d in reversed(self.dims)][1:]
        box = [d.box for d in reversed(self.dims)]
        return (self.rank, dims, strides, box, [1] * self.rank, 0, self.swizzle, 2, 0)


def _largest_divisor_at_most(n: int, cap: int, ok=lambda s: True) -> int:
    best = 0
    for s in range(1, min(n, cap) + 1):
        if n % s == 0 and ok(s):
            best = s
    return best


def _promotion(inner: DescDim, others: list, desc_esize: int, base_addr: int):
    """Smallest wider element type that brings the inner box to <= 256."""
    for wide in (2, 4, 8):
        if wide <= desc_esize:
            continue
        f = wide // desc_esize
        if inner.box % f or inner.extent % f:
            continue
        if any(d.stride % wide for d in others) or base_addr % wide:
            continue
        if inner.box // f <= MAX_BOX:
            return wide
    return None


def plan_box(esize: int, shape, strides, box, swizzle: int = SWIZZLE_NONE,
             copy_only: bool = True, base_addr: int = 0) -> Plan:
    """Plan the descriptor for tiles of ``box`` over a tensor (L1 -> L2 -> L3).

    ``shape``, ``strides`` (elements) and ``box`` are outermost-first.
    Raises ``Invalid`` for malformed input and ``Declined`` when no legal
    descriptor exists.
    """
    shape = tuple(int(s) for s in shape)
    strides = tuple(int(s) for s in strides)
    box = tuple(int(b) for b in box)
    r = len(shape)
    if not (1 <= r <= MAX_INPUT_RANK) or len(strides) != r or len(box) != r:
        raise Invalid("rank must be 1..8 with matching shape/strides/box")
    if any(s < 0 for s in shape) or any(b < 1 for b in box) or any(s < 1 for s in strides):
        raise Invalid("extents must be >= 0 (0: an empty tensor), strides and box >= 1")
    if esize not in (1, 2, 4, 8):
        raise Invalid("element size must be 1, 2, 4 or 8 bytes")
    if swizzle not in (SWIZZLE_NONE, SWIZZLE_32B, SWIZZLE_64B, SWIZZLE_128B):
        raise Invalid("swizzle must be none, 32-, 64- or 128-byte")
    atom_bytes = _swz.span_bytes(swizzle)

    # L1: canonicalize.  The innermost dim must have stride 1; dims of
    # extent 1 with box 1 carry no information and are dropped.
    if strides[-1] != 1:
        raise Declined("innermost stride must be 1")
    dims = []
    for d in range(r):
        if shape[d] == 1 and box[d] == 1 and d != r - 1:
            continue
        dims.append(DescDim(extent=shape[d], stride=strides[d] * esize, box=box[d],
                            parts=[Axis(box[d], d, 1)]))

    # L2: a swizzle splits an inner box wider than one atom (16 << mode
    # bytes) into atoms; the atom axis becomes the outermost descriptor dim.
    # An inner box that is no whole number of atoms is shrunk into equal
    # segments that fit one atom (issue axis).
    if swizzle != SWIZZLE_NONE:
        inner = dims[-1]
        inner_bytes = inner.box * esize
        if inner_bytes > atom_bytes and inner_bytes % 16:
            raise Declined("innermost box is not a whole number of 16-byte swizzle chunks")
        if inner_bytes > atom_bytes and (inner_bytes % atom_bytes or (inner.extent * esize) % atom_bytes):
            seg = _largest_divisor_at_most(inner.box, atom_bytes // esize, lambda s: (s * esize) % 16 == 0)
            part = inner.parts[0]
            inner.seg_issue = Axis(inner.box // seg, part.dim, part.step * seg)
            inner.parts = [Axis(seg, part.dim, part.step)]
            inner.box = seg
        elif inner_bytes > atom_bytes:
            w = atom_bytes // esize
            d_in = inner.parts[0].dim
            atom = DescDim(extent=inner.extent // w, stride=atom_bytes, box=inner.box // w,
                           parts=[Axis(inner.box // w, d_in, w)], atom=True)
            dims[-1] = DescDim(extent=w, stride=esize, box=w, parts=[Axis(w, d_in, 1)])
            dims.insert(0, atom)

    desc_esize = esize

    # L3 (merge): adjacent fully-boxed contiguous dims collapse into one.
    changed = True
    while changed:
        changed = False
        for k in range(len(dims) - 1, 0, -1):
            o, i = dims[k - 1], dims[k]
            if o.atom or i.atom or o.seg_issue is not None or i.seg_issue is not None:
                continue
            if i.box != i.extent or o.stride != i.extent * i.stride:
                continue
            mb = o.box * i.extent
            merged = DescDim(extent=o.extent * i.extent, stride=i.stride, box=mb,
                             parts=o.parts + i.parts)
            innermost = (k == len(dims) - 1)
            if innermost and swizzle != SWIZZLE_NONE and mb * desc_esize > atom_bytes:
                continue
            if mb > MAX_BOX:
                if not (innermost and copy_only and
                        _promotion(merged, dims[:k - 1], desc_esize, base_addr)):
                    continue
            dims[k - 1:k + 1] = [merged]
            changed = True
            break

    # Under a swizzle the innermost box (merged rows included) must be a whole
    # number of 16-byte chunks.
    if swizzle != SWIZZLE_NONE and (dims[-1].box * desc_esize) % 16:
        raise Declined("innermost box is not a whole number of 16-byte swizzle chunks")

    # Promotion of the innermost dim (copies only): box > 256 -> wider element.
    promoted = False
    inner = dims[-1]
    if copy_only and inner.box > MAX_BOX:
        wide = _promotion(inner, dims[:-1], desc_esize, base_addr)
        if wide:
            f = wide // desc_esize
            dims[-1] = DescDim(extent=inner.extent // f, stride=wide, box=inner.box // f,
                               parts=inner.parts, atom=inner.atom)
            desc_esize = wide
            promoted = True

    # L2 (segments): a box > 256 is cut into equal segments issued separately.
    for k, d in enumerate(dims):
        if d.box <= MAX_BOX:
            continue
        if len(d.parts) != 1:
            raise Declined("merged dim exceeds the box limit")
        part = d.parts[0]
        if k == len(dims) - 1:
            seg = _largest_divisor_at_most(d.box, MAX_BOX, lambda s: (s * desc_esize) % 16 == 0)
            if not seg:
                seg = _largest_divisor_at_most(d.box, MAX_BOX, lambda s: (s * desc_esize) % 4 == 0)
            if not seg:
                seg = _largest_divisor_at_most(d.box, MAX_BOX)
        else:
            seg = _largest_divisor_at_most(d.box, MAX_BOX)
        d.seg_issue = Axis(d.box // seg, part.dim, part.step * seg)
        d.parts = [Axis(seg, part.dim, part.step)]
        d.box = seg

    # L3 (shrink): too many descriptor dims -> the outermost leaves the
    # descriptor and becomes issue axes.
    shrunk = []
    while len(dims) > MAX_RANK:
        shrunk.append(dims.pop(0))
    issue_axes = []
    for d in shrunk:
        if d.seg_issue is not None:
            issue_axes.append(d.seg_issue)
        issue_axes.extend(d.parts)
    for d in dims:
        if d.seg_issue is not None:
            issue_axes.append(d.seg_issue)

    return Plan(esize=esize, desc_esize=desc_esize, shape=shape, strides=strides, box=box,
                swizzle=swizzle, dims=dims, issue_axes=issue_axes, promoted=promoted)


def partition(p: Plan, threads: int, vec_candidates=GFX950_VEC_BYTES, base_addr: int = 0) -> Plan:
    """Synthesize ``[outer, threads, vec]`` for one tile of plan ``p``.

    The vector width is the widest candidate that divides the innermost LDS
    run, the tensor's inner extent and every stride (in bytes), that the base
    address honours, and for which threads * vec divides the tile.
    """
    if threads < 64 or threads > 1024 or threads % 64:
        raise Invalid("threads must be a multiple of 64 in 64..1024")
    inner_run = p.image_axes[-1].count * p.esize
    inner_extent = p.shape[-1] * p.esize
    outer_strides = [s * p.esize for s in p.strides[:-1]]
    for v in vec_candidates:
        if inner_run % v or inner_extent % v or base_addr % v:
            continue
        if any(s % v for s in outer_strides):
            continue
        if p.tile_bytes % (threads * v):
            continue
        p.threads = threads
        p.vec_bytes = v
        p.vec = v // p.esize
        p.outer = p.tile_bytes // (threads * v)
        return p
    raise Declined("no legal vector width of at least 4 bytes")


def plan(dtype: str, shape, strides, box, swizzle=SWIZZLE_NONE, threads=0,
         copy_only=True, vec_candidates=GFX950_VEC_BYTES, base_addr=0) -> Plan:
    p = plan_box(ESIZE[dtype], shape, strides, box, swizzle, copy_only, base_addr)
    if threads:
        partition(p, threads, vec_candidates, base_addr)
    return p


def tile_grid(shape, box):
    """Tiles per dim (ceil division), outermost-first."""
    return tuple(-(-int(n) // int(b)) for n, b in zip(shape, box))


def tile_origin(shape, box, tile_index: int):
    """Element coordinates of the first element of tile ``tile_index`` (row-major)."""
    grid = tile_grid(shape, box)
    coords = []
    rem = int(tile_index)
    for g, b in zip(reversed(grid), reversed(box)):
        coords.append((rem % g) * b)
        rem //= g
    if rem:
        raise Invalid("tile index out of range")
    return tuple(reversed(coords))


def image_coords(p: Plan):
    """For each element of the LDS image (row-major over the image axes), its
    coordinate offset within the tile, as a tuple over the tensor dims."""
    axes = p.image_axes
    r = len(p.shape)
    out = []

    def rec(k, acc):
        if k == len(axes):
            out.append(tuple(acc))
            return
        a = axes[k]
        for idx in range(a.count):
            nxt = list(acc)
            nxt[a.dim] += idx * a.step
            rec(k + 1, nxt)

    rec(0, [0] * r)
    return out


def lds_offset(p: Plan, logical_byte: int) -> int:
    """Physical LDS byte offset of a logical image byte."""
    return _swz.swizzle(logical_byte, p.swizzle)
