"""Brute-force pin of the oracle planner's accept / decline decision.

Every way of describing the tiles of a small tensor with one descriptor and a
set of loads per tile is enumerated here directly, without any step of the
oracle planner.  A candidate is:

* an element size: the tensor's own, or for copies a wider one (2, 4 or 8
  bytes; "copy_async -> tma", "How inputs change the algorithm": box > 256
  may promote the element type);
* for every tensor dim, the number of loads along it and the box of each
  load (equal pieces of the tile's box along that dim);
* optionally the innermost box written as two descriptor dims (an outer dim
  whose stride is the width of the inner one: the form the swizzle-atom
  split of the worked example takes);
* optionally dropping dims of extent 1, and merging adjacent descriptor
  dims that each load takes whole and whose inner one is fully boxed
  (reading adopted: a merge joins whole boxes, and a merged dim is not cut
  into several loads again).

Its legality is judged on its numbers by the rules of "copy_async -> tma",
"What it accepts" (rank <= 5, innermost stride one element, innermost box
inside the swizzle atom and a whole number of 16-byte chunks) and "Add TMA
support for circular buffering pass", "Lowering Details" (box <= 256 per
dim), and on its behaviour: every load of every tile is simulated the way a
descriptor-driven copy walks it (per-dim coordinates, clipped against the
descriptor's extents), and the elements it reads must be exactly the tile's
in-bounds elements, each once.  The planner must accept exactly when some
candidate is legal ("copy_async -> tma", last paragraph of "How inputs
change the algorithm": the variant declines when no legal descriptor
exists).
"""
import itertools
import random

import pytest

from oracle import plan as P


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


class _Dim:
    """One descriptor dim of a candidate: extent, byte stride and box, plus
    how a load's start coordinate along it follows from the load's start in
    tensor coordinates (``coord``: tensor start coords -> this dim's
    coordinate, or None when the load cannot be expressed)."""

    def __init__(self, extent, stride, box, coord, whole):
        self.extent, self.stride, self.box, self.coord = extent, stride, box, coord
        self.whole = whole            # every load takes the tile's whole box along it


def _candidates(es, shape, strides, box, copy_only, base):
    """Yield (element size, [_Dim] outermost-first, per-dim load counts) for
    every candidate, cheapest checks first."""
    r = len(shape)
    widths = [es] + ([w for w in (2, 4, 8) if w > es] if copy_only else [])
    for ep in widths:
        f = ep // es
        if f > 1:
            # a wider element is a valid reinterpretation only when every
            # promoted element is aligned and no row ends inside one
            if base % ep or (shape[-1] * es) % ep or any((s * es) % ep for s in strides[:-1]):
                continue
            if box[-1] % f:
                continue
        # pieces of the innermost box (in promoted elements)
        bi = box[-1] // f
        for c_in in _divisors(bi):
            q_in = bi // c_in
            for w in _divisors(c_in):
                # w == c_in: one innermost descriptor dim; else two (split)
                yield from _outer(ep, f, es, shape, strides, box, copy_only, c_in, q_in, w)


def _outer(ep, f, es, shape, strides, box, copy_only, c_in, q_in, w):
    r = len(shape)
    ext_in = -(-shape[-1] // f)           # promoted inner extent (whole by the check above)
    stride_in = strides[-1] * es * f      # bytes between promoted inner elements

    def inner_dims():
        if w == c_in:
            return [_Dim(ext_in, stride_in, c_in,
                         lambda s: s[-1] // f if s[-1] % f == 0 else None, q_in == 1)]
        return [_Dim(-(-ext_in // w), stride_in * w, c_in // w,
                     lambda s: (s[-1] // f) // w if s[-1] % (f * w) == 0 else None, q_in == 1),
                _Dim(w, stride_in, w, lambda s: 0, q_in == 1)]

    per_dim = [[(q, box[d] // q) for q in _divisors(box[d])] for d in range(r - 1)]
    for choice in itertools.product(*per_dim):
        for drop in itertools.product(*[([False, True] if shape[d] == 1 else [False]) for d in range(r - 1)]):
            dims = []
            for d in range(r - 1):
                if drop[d]:
                    continue
                q, c = choice[d]
                dims.append(_Dim(shape[d], strides[d] * es, c, (lambda dd: lambda s: s[dd])(d), q == 1))
            dims.extend(inner_dims())
            loads = [q for q, _ in choice] + [q_in]
            pieces = [c for _, c in choice] + [c_in * f]
            dropped = [d for d in range(r - 1) if drop[d]]
            for merged in _merges(dims):
                yield ep, merged, loads, pieces, dropped


def _merges(dims):
    """The dim list itself and every list obtained by merging adjacent dims
    taken whole by every load whose inner one is fully boxed (merged
    coordinate = outer * extent + inner)."""
    yield dims
    for k in range(len(dims) - 1):
        o, i = dims[k], dims[k + 1]
        if i.box != i.extent or not (o.whole and i.whole):
            continue

        def coord(s, o=o, i=i):
            a, b = o.coord(s), i.coord(s)
            return None if a is None or b is None else a * i.extent + b

        m = _Dim(o.extent * i.extent, i.stride, o.box * i.extent, coord, True)
        yield from _merges(dims[:k] + [m] + dims[k + 2:])


def _rules_ok(ep, dims, swizzle):
    if len(dims) > P.MAX_RANK:
        return False
    if any(d.box > P.MAX_BOX or d.box < 1 for d in dims):
        return False
    if dims[-1].stride != ep:
        return False
    if swizzle:
        ib = dims[-1].box * ep
        if ib > (16 << swizzle) or ib % 16:
            return False
    return True


def _tile_elements(shape, strides, box, origin):
    out = []
    for rel in itertools.product(*[range(b) for b in box]):
        c = [o + x for o, x in zip(origin, rel)]
        if all(v < n for v, n in zip(c, shape)):
            out.append(sum(v * s for v, s in zip(c, strides)))
    return sorted(out)


def _simulate(es, ep, dims, shape, strides, box, loads, pieces, dropped, origin):
    """Element offsets read by the candidate's loads for the tile at
    ``origin``, or None when a load's start cannot be expressed."""
    f = ep // es
    got = []
    for k in itertools.product(*[range(q) for q in loads]):
        start = [o + ki * c for o, ki, c in zip(origin, k, pieces)]
        if any(start[d] != 0 for d in dropped):
            return None               # a dropped dim has no coordinate to move
        xs = [d.coord(start) for d in dims]
        if any(x is None for x in xs):
            return None
        for rel in itertools.product(*[range(d.box) for d in dims]):
            pos = [x + i for x, i in zip(xs, rel)]
            if any(p >= d.extent for p, d in zip(pos, dims)):
                continue              # clipped: out of the descriptor's bounds
            byte = sum(p * d.stride for p, d in zip(pos, dims))
            if byte % es:
                return None
            got.extend(byte // es + j for j in range(f))
    return sorted(got)


def legal_candidate_exists(es, shape, strides, box, swizzle, copy_only, base=0):
    shape, strides, box = list(shape), list(strides), list(box)
    if any(n == 0 for n in shape):
        return True                   # no tiles: nothing to describe
    grid = [-(-n // b) for n, b in zip(shape, box)]
    origins = [[g * b for g, b in zip(t, box)] for t in itertools.product(*[range(g) for g in grid])]
    want = [_tile_elements(shape, strides, box, o) for o in origins]
    for ep, dims, loads, pieces, dropped in _candidates(es, shape, strides, box, copy_only, base):
        if not _rules_ok(ep, dims, swizzle):
            continue
        if all(_simulate(es, ep, dims, shape, strides, box, loads, pieces, dropped, o) == w
               for o, w in zip(origins, want)):
            return True
    return False


def _planner_accepts(dt, shape, strides, box, swz, copy_only):
    try:
        P.plan_box(P.ESIZE[dt], shape, strides, box, swz, copy_only)
        return True
    except P.Declined:
        return False


def _random_case(rng):
    r = rng.randint(1, 3)
    dt = rng.choice(["u8", "f16", "f32", "u64"])
    shape = [rng.randint(1, 8) for _ in range(r)]
    big = rng.randrange(r)
    shape[big] = rng.choice([8, 12, 24, 40, 48, 64, 96, 100, 128, 192, 200, 257, 300])
    box = [rng.randint(1, s) for s in shape]
    if rng.random() < 0.5:
        box[big] = rng.choice(_divisors(shape[big]))
    if rng.random() < 0.1:
        box[rng.randrange(r)] += rng.randint(1, 3)      # a box past the tensor's extent
    pad = rng.choice([0, 0, 1, 4, 16])
    strides, st = [], 1
    for k, ext in enumerate(reversed(shape)):
        strides.append(st)
        st *= ext + (pad if k == 0 else 0)
    strides = list(reversed(strides))
    if rng.random() < 0.05:
        strides[-1] = rng.choice([2, 3])
    swz = rng.choice([0, 0, 1, 2, 3])
    copy_only = rng.random() < 0.5
    return dt, shape, strides, box, swz, copy_only


def test_enumerator_pins_itself_on_hand_cases():
    # the worked example: legal (one rank-3 descriptor)
    assert legal_candidate_exists(2, (8, 256), (256, 1), (8, 256), 3, True)
    # innermost stride 2: nothing is legal
    assert not legal_candidate_exists(2, (8, 256), (1, 8), (8, 256), 0, True)
    # 24-byte inner box under a swizzle: no whole 16-byte chunks, and the
    # whole 8-row box merged is 192 bytes, wider than the atom
    assert not legal_candidate_exists(2, (8, 12), (12, 1), (8, 12), 3, True)
    # ... but 4 rows merge into 96 bytes: whole chunks inside the atom
    assert legal_candidate_exists(2, (8, 12), (12, 1), (4, 12), 3, True)
    # 192-byte inner box under the 128-byte swizzle: two loads of 96 bytes
    assert legal_candidate_exists(2, (8, 96), (96, 1), (8, 96), 3, False)
    # f16 box of 257 (prime) without swizzle: 257 loads of one element
    assert legal_candidate_exists(2, (2, 257), (257, 1), (2, 257), 0, False)
    # a 4-byte promoted element may not straddle a row of odd length
    assert legal_candidate_exists(1, (3, 300), (301, 1), (3, 300), 0, True)


@pytest.mark.parametrize("seed", range(4))
def test_planner_accepts_iff_a_legal_candidate_exists(seed):
    rng = random.Random(1000 + seed)
    n_acc = n_dec = 0
    for _ in range(150):
        dt, shape, strides, box, swz, copy_only = _random_case(rng)
        es = P.ESIZE[dt]
        want = legal_candidate_exists(es, shape, strides, box, swz, copy_only)
        got = _planner_accepts(dt, shape, strides, box, swz, copy_only)
        assert got == want, (dt, shape, strides, box, swz, copy_only)
        n_acc += got
        n_dec += not got
    assert n_acc > 50 and n_dec > 3


def test_planner_accepts_iff_legal_on_swizzle_edges():
    # inner boxes around the atom widths of every mode, rows of several
    # lengths (atom-aligned and not), both element sizes that matter
    for swz in (1, 2, 3):
        for es, dt in ((2, "f16"), (4, "f32")):
            for inner in (4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64, 80, 96):
                for ext in (inner, inner + 8, 2 * inner):
                    for copy_only in (False, True):
                        shape, strides, box = (3, ext), (ext, 1), (2, inner)
                        want = legal_candidate_exists(es, shape, strides, box, swz, copy_only)
                        assert _planner_accepts(dt, shape, strides, box, swz, copy_only) == want, \
                            (dt, shape, box, swz, copy_only)
