// Plan search and partition synthesis for acp tile descriptors.
//
// Rules ("copy_async -> tma": "What it accepts", "Algorithm" step 2, "How
// inputs change the algorithm"; "Add TMA support for circular buffering
// pass": "Lowering Details"; "copy_async -> ldgsts": "Algorithm" step 1 and
// its vec / cp_size / outer table; "elementwise -> smem": "Algorithm" step 2):
//
//  L1  The innermost stride must be 1.  Dims of extent 1 and box 1 carry no
//      information and are dropped.
//  L2  Under a swizzle an innermost box wider than the mode's atom (16 << mode
//      bytes: 32, 64 or 128) is split into atoms; the atom axis becomes the
//      outermost descriptor dim (the only order that gives the worked 8x256
//      float16 example's byte strides 512, 128).  When that box, or the
//      tensor row, is no whole number of atoms, the box is shrunk instead:
//      cut into equal segments (the largest divisor whose bytes fit the atom
//      and are a whole number of 16-byte chunks), the quotient an issue axis.
//  L3  Adjacent dims merge when the inner one is fully boxed and contiguous
//      with the outer one and the merged box stays <= 256 (copies may merge
//      the innermost pair beyond 256 when promotion then fixes it; under the
//      swizzle the innermost box stays within one atom; atom axes never merge).
//      A merge joins whole boxes; a merged dim is not cut again.  Under a
//      swizzle the innermost box must now be a whole number of 16-byte
//      chunks, else the plan declines.  A copy's innermost box over 256
//      promotes the element 1 -> 2 -> 4 -> 8 bytes.  Any box still over 256
//      is cut into equal segments (largest divisor <= 256; for the innermost
//      dim preferably a 16-byte multiple, else a 4-byte one, else any); the
//      quotient is an issue axis (several loads).  While the descriptor is
//      deeper than 5, its outermost dim leaves it and becomes issue axes, so
//      the shrink always succeeds.  More than 256 loads per tile, or more
//      than 12 image axes, exceed what the kernels index: Unsupported (not
//      a decline: a legal descriptor exists).
//  Partition: vec_bytes is the widest of {16, 4} (the gfx950 direct-to-LDS
//      sizes; the page's 8-byte form does not exist there) that divides the
//      innermost LDS run, the tensor's inner extent and every stride (bytes),
//      that the base address honours, and with threads * vec_bytes dividing
//      the tile's bytes.  outer = tile bytes / (threads * vec_bytes).
#include "acp_plan.hpp"

#include <algorithm>

namespace acp {

int dtype_size(int dtype) {
  switch (dtype) {
    case 0: return 1;  // u8
    case 1: return 2;  // u16
    case 2: return 4;  // u32
    case 3: return 8;  // u64
    case 4: return 2;  // f16
    case 5: return 4;  // f32
    default: return -1;
  }
}

std::vector<Axis> Plan::image_axes() const {
  std::vector<Axis> all(issue_axes);
  for (const DescDim& d : dims) all.insert(all.end(), d.parts.begin(), d.parts.end());
  std::vector<Axis> out;
  for (size_t k = 0; k < all.size(); ++k)
    if (all[k].count > 1 || k + 1 == all.size()) out.push_back(all[k]);
  return out;
}

int64_t Plan::issues() const {
  int64_t n = 1;
  for (const Axis& a : issue_axes) n *= a.count;
  return n;
}

int64_t Plan::tile_elems() const {
  int64_t n = 1;
  for (const Axis& a : image_axes()) n *= a.count;
  return n;
}

int64_t Plan::n_tiles() const {
  int64_t n = 1;
  for (int d = 0; d < rank_t; ++d) n *= (shape[d] + box[d] - 1) / box[d];
  return n;
}

namespace {

PlanStatus fail(std::string* reason, PlanStatus s, const char* why) {
  if (reason) *reason = why;
  return s;
}

// Widest legal element for a copy's innermost dim so that its box drops to
// <= 256; 0 if none.
int promotion_width(const DescDim& inner, const std::vector<DescDim>& others, int desc_esize,
                    uint64_t base) {
  for (int wide = 2; wide <= 8; wide *= 2) {
    if (wide <= desc_esize) continue;
    const int64_t f = wide / desc_esize;
    if (inner.box % f != 0 || inner.extent % f != 0) continue;
    bool aligned = (base % static_cast<uint64_t>(wide)) == 0;
    for (const DescDim& o : others) aligned = aligned && (o.stride % wide == 0);
    if (!aligned) continue;
    if (inner.box / f <= kMaxBox) return wide;
  }
  return 0;
}

int64_t largest_divisor_upto(int64_t n, int64_t cap, int64_t bytes_per, int64_t multiple) {
  for (int64_t s = std::min(n, cap); s >= 1; --s)
    if (n % s == 0 && (s * bytes_per) % multiple == 0) return s;
  return 0;
}

}  // namespace

PlanStatus plan_box_with(const DescData& dd, const int32_t* boxp, bool copy_only, Plan* out,
                         std::string* reason) {
  const int r = dd.rank;
  const int es = dd.esize;
  if (r < 1 || r > kMaxInputRank) return fail(reason, PlanStatus::Invalid, "rank must be 1..8");
  if (es != 1 && es != 2 && es != 4 && es != 8)
    return fail(reason, PlanStatus::Invalid, "element size must be 1, 2, 4 or 8 bytes");
  if (dd.swizzle > 3) return fail(reason, PlanStatus::Invalid, "swizzle must be none, 32-, 64- or 128-byte");
  const int64_t atom_bytes = dd.swizzle ? (int64_t(16) << dd.swizzle) : 0;
  for (int d = 0; d < r; ++d)
    if (dd.shape[d] < 0 || dd.strides[d] < 1 || boxp[d] < 1)
      return fail(reason, PlanStatus::Invalid, "extents must be >= 0 (0: an empty tensor), strides and box >= 1");

  Plan p;
  p.esize = es;
  p.desc_esize = es;
  p.swizzle = dd.swizzle;
  p.rank_t = r;
  for (int d = 0; d < r; ++d) {
    p.shape[d] = dd.shape[d];
    p.strides[d] = dd.strides[d];
    p.box[d] = boxp[d];
  }

  // L1
  if (dd.strides[r - 1] != 1) return fail(reason, PlanStatus::Declined, "innermost stride must be 1");
  std::vector<DescDim> dims;
  for (int d = 0; d < r; ++d) {
    if (d != r - 1 && dd.shape[d] == 1 && boxp[d] == 1) continue;
    DescDim dim;
    dim.extent = dd.shape[d];
    dim.stride = dd.strides[d] * es;
    dim.box = boxp[d];
    dim.parts.push_back(Axis{boxp[d], d, 1});
    dims.push_back(dim);
  }

  // L2: swizzle atoms (16 << mode bytes)
  if (dd.swizzle != 0) {
    DescDim inner = dims.back();
    const int64_t ib = inner.box * es;
    if (ib > atom_bytes && ib % 16 != 0) {
      return fail(reason, PlanStatus::Declined, "innermost box is not a whole number of 16-byte swizzle chunks");
    } else if (ib > atom_bytes && (ib % atom_bytes != 0 || (inner.extent * es) % atom_bytes != 0)) {
      // shrink: equal segments within one atom, the quotient an issue axis
      const int64_t seg = largest_divisor_upto(inner.box, atom_bytes / es, es, 16);
      DescDim& d = dims.back();
      const Axis part = d.parts[0];
      d.segmented = true;
      d.seg = Axis{d.box / seg, part.dim, part.step * seg};
      d.parts[0] = Axis{seg, part.dim, part.step};
      d.box = seg;
    } else if (ib > atom_bytes) {
      const int64_t w = atom_bytes / es;
      const int dim = inner.parts[0].dim;
      DescDim atom;
      atom.extent = inner.extent / w;
      atom.stride = atom_bytes;
      atom.box = inner.box / w;
      atom.parts.push_back(Axis{inner.box / w, dim, w});
      atom.atom = true;
      DescDim in2;
      in2.extent = w;
      in2.stride = es;
      in2.box = w;
      in2.parts.push_back(Axis{w, dim, 1});
      dims.back() = in2;
      dims.insert(dims.begin(), atom);
    }
  }

  // L3: merge
  for (bool changed = true; changed;) {
    changed = false;
    for (size_t k = dims.size() - 1; k >= 1; --k) {
      const DescDim& o = dims[k - 1];
      const DescDim& i = dims[k];
      if (o.atom || i.atom || o.segmented || i.segmented) continue;
      if (i.box != i.extent || o.stride != i.extent * i.stride) continue;
      DescDim m;
      m.extent = o.extent * i.extent;
      m.stride = i.stride;
      m.box = o.box * i.extent;
      m.parts = o.parts;
      m.parts.insert(m.parts.end(), i.parts.begin(), i.parts.end());
      const bool innermost = (k == dims.size() - 1);
      if (innermost && dd.swizzle != 0 && m.box * p.desc_esize > atom_bytes) continue;
      if (m.box > kMaxBox) {
        std::vector<DescDim> rest(dims.begin(), dims.begin() + (k - 1));
        if (!(innermost && copy_only && promotion_width(m, rest, p.desc_esize, dd.gbase))) continue;
      }
      dims[k - 1] = m;
      dims.erase(dims.begin() + k);
      changed = true;
      break;
    }
  }

  // under a swizzle the innermost box (merged rows included) is whole chunks
  if (dd.swizzle != 0 && (dims.back().box * p.desc_esize) % 16 != 0)
    return fail(reason, PlanStatus::Declined, "innermost box is not a whole number of 16-byte swizzle chunks");

  // promotion of a copy's innermost box
  if (copy_only && dims.back().box > kMaxBox) {
    std::vector<DescDim> rest(dims.begin(), dims.end() - 1);
    const int wide = promotion_width(dims.back(), rest, p.desc_esize, dd.gbase);
    if (wide) {
      const int64_t f = wide / p.desc_esize;
      dims.back().extent /= f;
      dims.back().box /= f;
      dims.back().stride = wide;
      p.desc_esize = wide;
      p.promoted = true;
    }
  }

  // L3: segments for boxes over 256 (issue axes)
  for (size_t k = 0; k < dims.size(); ++k) {
    DescDim& d = dims[k];
    if (d.box <= kMaxBox) continue;
    if (d.parts.size() != 1) return fail(reason, PlanStatus::Declined, "merged dim exceeds the box limit");
    int64_t seg;
    if (k + 1 == dims.size()) {
      seg = largest_divisor_upto(d.box, kMaxBox, p.desc_esize, 16);
      if (!seg) seg = largest_divisor_upto(d.box, kMaxBox, p.desc_esize, 4);
      if (!seg) seg = largest_divisor_upto(d.box, kMaxBox, 1, 1);
    } else {
      seg = largest_divisor_upto(d.box, kMaxBox, 1, 1);
    }
    const Axis part = d.parts[0];
    d.segmented = true;
    d.seg = Axis{d.box / seg, part.dim, part.step * seg};
    d.parts[0] = Axis{seg, part.dim, part.step};
    d.box = seg;
  }

  // L3: shrink
  std::vector<DescDim> shrunk;
  while (static_cast<int>(dims.size()) > kMaxRank) {
    shrunk.push_back(dims.front());
    dims.erase(dims.begin());
  }
  for (const DescDim& d : shrunk) {
    if (d.segmented) p.issue_axes.push_back(d.seg);
    p.issue_axes.insert(p.issue_axes.end(), d.parts.begin(), d.parts.end());
  }
  for (const DescDim& d : dims)
    if (d.segmented) p.issue_axes.push_back(d.seg);
  p.dims = dims;
  if (p.issues() > kMaxIssues || static_cast<int>(p.image_axes().size()) > kMaxImageAxes)
    return fail(reason, PlanStatus::Unsupported,
                "the shrunk plan needs more than 256 loads per tile or 12 image axes (kernel limits)");
  *out = p;
  return PlanStatus::Ok;
}

PlanStatus plan_box(const DescData& d, bool copy_only, Plan* out, std::string* reason) {
  return plan_box_with(d, d.box, copy_only, out, reason);
}

PlanStatus plan_partition(Plan* p, int threads, uint64_t base, std::string* reason) {
  if (threads < 64 || threads > 1024 || threads % 64 != 0)
    return fail(reason, PlanStatus::Invalid, "threads must be a multiple of 64 in 64..1024");
  const std::vector<Axis> axes = p->image_axes();
  const int64_t inner_run = axes.back().count * p->esize;
  const int64_t inner_extent = p->shape[p->rank_t - 1] * p->esize;
  const int64_t tile = p->tile_bytes();
  static const int kVec[] = {16, 4};
  for (int v : kVec) {
    if (inner_run % v || inner_extent % v || base % static_cast<uint64_t>(v)) continue;
    bool ok = true;
    for (int d = 0; d + 1 < p->rank_t; ++d) ok = ok && ((p->strides[d] * p->esize) % v == 0);
    if (!ok || tile % (static_cast<int64_t>(threads) * v) != 0) continue;
    p->threads = threads;
    p->vec_bytes = v;
    p->vec = v / p->esize;
    p->outer = static_cast<int>(tile / (static_cast<int64_t>(threads) * v));
    return PlanStatus::Ok;
  }
  return fail(reason, PlanStatus::Declined, "no legal vector width of at least 4 bytes");
}

}  // namespace acp
