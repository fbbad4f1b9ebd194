"""Pins of the oracle planner: the pages' worked examples, the decline rules,
and brute force over small shapes."""
import itertools
import os
import random

import pytest

from oracle import plan as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(path):
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_golden_tma_descriptor():
    g = _read_kv(os.path.join(GOLDEN, "tma_descriptor_8x256_f16_swizzle128.txt"))
    dt, shape, strides, box, swz = [s.strip() for s in g["request"].split("|")]
    p = P.plan(dt, [int(x) for x in shape.split()], [int(x) for x in strides.split()],
               [int(x) for x in box.split()], int(swz))
    rank, dims, bstrides, pbox, estr, inter, swz_mode, l2, oob = p.encode_args()
    ints = lambda s: [int(x) for x in s.split()]
    assert rank == int(g["rank"])
    assert dims == ints(g["dims"])
    assert bstrides == ints(g["strides"])
    assert pbox == ints(g["box"])
    assert estr == ints(g["element_strides"])
    assert inter == int(g["interleave"])
    assert swz_mode == int(g["swizzle"])
    assert l2 == int(g["l2_promotion"])
    assert oob == int(g["oob_fill"])
    assert p.issues == 1          # "a single issue" for the whole tile


def _partition_rows():
    with open(os.path.join(GOLDEN, "partitions.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split("|")]


@pytest.mark.parametrize("row", list(_partition_rows()), ids=lambda r: r[0])
def test_golden_partitions(row):
    name, dt, rc, threads, align, vset, vec, vb, outer = row
    rows, cols = (int(x) for x in rc.split())
    cands = P.PAGE_VEC_BYTES if vset == "page" else P.GFX950_VEC_BYTES
    base = int(align) if int(align) else 0
    if vec == "-":
        with pytest.raises(P.Declined):
            P.plan(dt, (rows, cols), (cols, 1), (rows, cols), threads=int(threads),
                   vec_candidates=cands, base_addr=base)
        return
    p = P.plan(dt, (rows, cols), (cols, 1), (rows, cols), threads=int(threads),
               vec_candidates=cands, base_addr=base)
    assert (p.vec, p.vec_bytes, p.outer) == (int(vec), int(vb), int(outer))


def test_swizzled_2d_tile_gives_rank3():
    # "How inputs change the algorithm": a 128-B swizzle on a 2-D tile yields rank 3.
    for rows, cols, dt in ((8, 256, "f16"), (16, 128, "f32"), (4, 512, "u8")):
        p = P.plan(dt, (rows, cols), (cols, 1), (rows, cols), P.SWIZZLE_128B)
        assert p.rank == 3
        assert p.dims[-1].box * P.ESIZE[dt] == 128


def test_narrow_swizzle_modes_split_into_their_atoms():
    # 32- and 64-byte modes: the inner axis splits into 32- / 64-byte atoms,
    # the atom axis outermost (same construction as the 128-byte example)
    p = P.plan("f16", (8, 256), (256, 1), (8, 256), P.SWIZZLE_32B)
    assert p.rank == 3
    assert [d.extent for d in reversed(p.dims)] == [16, 8, 16]     # 16 f16 = 32 B, 8 rows, 16 atoms of 512 B
    assert [d.stride for d in reversed(p.dims)] == [2, 512, 32]
    p = P.plan("f32", (4, 64), (64, 1), (4, 64), P.SWIZZLE_64B)
    assert [d.box for d in reversed(p.dims)] == [16, 4, 4]
    # a 48-byte inner box fits the 64-byte atom; under the 32-byte mode it is
    # no whole number of atoms and is shrunk into three 16-byte loads
    P.plan("f16", (8, 24), (24, 1), (8, 24), P.SWIZZLE_64B)
    p = P.plan("f16", (8, 24), (24, 1), (8, 24), P.SWIZZLE_32B)
    assert p.issues == 3 and p.dims[-1].box == 8
    with pytest.raises(P.Invalid):
        P.plan("f16", (8, 24), (24, 1), (8, 24), 4)


def test_declines():
    with pytest.raises(P.Declined, match="innermost stride"):
        P.plan("f16", (8, 256), (1, 8), (8, 256))
    # 24-byte inner box under swizzle is not whole 16-byte chunks, and the
    # eight rows merged (192 bytes) overflow the atom
    with pytest.raises(P.Declined, match="16-byte"):
        P.plan("f16", (8, 12), (12, 1), (8, 12), P.SWIZZLE_128B)
    # four such rows merge into 96 bytes: whole chunks within the atom
    p = P.plan("f16", (8, 12), (12, 1), (4, 12), P.SWIZZLE_128B)
    assert p.rank == 1 and p.dims[0].box == 48
    # 192-byte inner box, no whole number of 128-byte atoms: shrunk into two
    # 96-byte loads
    p = P.plan("f16", (8, 96), (96, 1), (8, 96), P.SWIZZLE_128B)
    assert p.issues == 2 and p.dims[-1].box == 48
    # 2-byte aligned base: no vector width >= 4 bytes
    with pytest.raises(P.Declined, match="vector width"):
        P.plan("f16", (128, 32), (32, 1), (128, 32), threads=128, base_addr=2)
    # rank 8 tensor whose 8 dims cannot merge: the shrink moves the three
    # outermost into issue axes (343 loads); the pages set no limit on loads
    shape = (7, 7, 7, 7, 7, 7, 7, 64)
    strides = []
    s = 1
    for ext in reversed(shape):
        strides.append(s)
        s *= ext + 1   # padded: never contiguous, so nothing merges
    strides = tuple(reversed(strides))
    p = P.plan("f32", shape, strides, shape)
    assert p.rank == 5 and p.issues == 343


def test_invalid_requests():
    with pytest.raises(P.Invalid):
        P.plan("f16", (8, 256), (256, 1), (8, 256), threads=96)
    with pytest.raises(P.Invalid):
        P.plan("f16", (8, -1), (256, 1), (8, 256))
    # extent 0 is an empty tensor: a valid plan that covers no tiles
    p = P.plan("f16", (0, 256), (256, 1), (8, 256))
    assert P.tile_grid(p.shape, p.box) == (0, 1)
    with pytest.raises(P.Invalid):
        P.plan("f16", (8,) * 9, (1,) * 9, (1,) * 9)


def test_merge_and_promotion():
    # (4, 64) uint8 fully boxed and contiguous: merges into one dim of 256.
    p = P.plan("u8", (4, 64), (64, 1), (4, 64))
    assert p.rank == 1 and p.dims[0].box == 256
    # (8, 128) uint8 merges to 1024 > 256 and promotes 1 -> 4 bytes (box 256).
    p = P.plan("u8", (8, 128), (128, 1), (8, 128))
    assert p.rank == 1 and p.promoted and p.desc_esize == 4 and p.dims[0].box == 256
    # an elementwise plan never promotes: 1024 float32 stay two dims
    p = P.plan("f32", (32, 32), (32, 1), (32, 32), copy_only=False)
    assert p.rank == 2 and not p.promoted


def test_box_over_256_takes_several_loads():
    # "Lowering Details": box dims <= 256, larger tiles need several loads.
    p = P.plan("f32", (128, 500, 1024), (512000, 1024, 1), (1, 4, 1024), copy_only=False)
    assert p.issues == 4 and max(d.box for d in p.dims) <= 256
    p = P.plan("f16", (600, 64), (64, 1), (600, 64), copy_only=False)
    assert p.issues == 3 and p.dims[0].box == 200


def _box_address_walk(p):
    """Byte offsets of a tile's elements as a descriptor walk would visit them:
    issue offsets outermost, then the box of each descriptor dim in its own
    coordinates and byte strides.  Independent of the image-axis coordinates."""
    es = p.esize
    r = len(p.shape)
    # Issue offsets: each issue axis advances one tensor dim.
    issue_ranges = [range(a.count) for a in p.issue_axes]
    offsets = []
    for iidx in itertools.product(*issue_ranges):
        ioff = sum(i * a.step * p.strides[a.dim] * es for i, a in zip(iidx, p.issue_axes))
        box_ranges = [range(d.box) for d in p.dims]
        for bidx in itertools.product(*box_ranges):
            base = ioff + sum(b * d.stride for b, d in zip(bidx, p.dims))
            # a promoted element covers desc_esize / esize original elements
            offsets.extend(base + k * es for k in range(p.desc_esize // es))
    return offsets


def _image_address_walk(p):
    es = p.esize
    return [sum(c * s for c, s in zip(rel, p.strides)) * es for rel in P.image_coords(p)]


def test_bruteforce_small_plans_cover_box_exactly_once():
    rng = random.Random(7)
    accepted = 0
    for _ in range(400):
        r = rng.randint(1, 3)
        dt = rng.choice(["u8", "f16", "f32"])
        es = P.ESIZE[dt]
        shape = [rng.randint(1, 8) for _ in range(r)]
        shape[-1] = rng.choice([8, 16, 32, 64, 96, 128, 300, 512])
        box = [rng.randint(1, s) for s in shape]
        box[-1] = rng.choice([d for d in range(1, shape[-1] + 1) if shape[-1] % d == 0])
        pad = rng.choice([0, 0, 4, 16])
        strides = []
        st = 1
        for ext in reversed(shape):
            strides.append(st)
            st *= ext + (pad if st == 1 else 0)
        strides = list(reversed(strides))
        swz = rng.choice([P.SWIZZLE_NONE, P.SWIZZLE_32B, P.SWIZZLE_64B, P.SWIZZLE_128B])
        copy_only = rng.random() < 0.5
        try:
            p = P.plan(dt, shape, strides, box, swz, copy_only=copy_only)
        except P.Declined:
            continue
        accepted += 1
        # legality of the descriptor
        assert p.rank <= 5
        assert all(d.box <= 256 for d in p.dims)
        assert p.dims[-1].stride == p.desc_esize
        if swz:
            ib = p.dims[-1].box * p.desc_esize
            assert ib <= 16 << swz and ib % 16 == 0
        # the image axes enumerate every box element exactly once
        coords = P.image_coords(p)
        assert len(coords) == len(set(coords))
        assert set(coords) == set(itertools.product(*[range(b) for b in box]))
        # ... in the same order and at the same addresses as the descriptor walk
        assert _image_address_walk(p) == _box_address_walk(p)
    assert accepted > 100


def test_partition_covers_every_chunk_once():
    for threads in (64, 128, 256, 512):
        p = P.plan("f16", (64, 256), (256, 1), (64, 256), threads=threads)
        seen = set()
        for f in range(p.outer):
            for t in range(threads):
                for v in range(p.vec):
                    seen.add((f * threads + t) * p.vec + v)
        assert seen == set(range(p.tile_elems))
