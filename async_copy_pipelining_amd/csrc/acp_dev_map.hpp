// Per-lane maps from LDS image chunks to tensor offsets, launch values held
// in registers, trip geometry and the store helpers shared by the kernels.
#pragma once

#include "acp_dev_ops.hpp"

namespace acp {
namespace dev {

// ---------------------------------------------------------------------------
// Per-lane map of the rounds f < outer: physical chunk (f * waves + wave) *
// 64 + lane of a slot, its logical position through the swizzle, and from the
// image axes its offsets inside the stage.  Computed once per workgroup.

struct LaneMap {
  uint32_t xoff[kMaxOuter];   // input byte offset from the stage origin
  uint32_t ooff[kMaxOuter];   // output byte offset from the stage origin
  uint32_t oobm[kMaxOuter];   // partial slots along which the chunk lies past the edge
  uint32_t lpos[kMaxOuter];   // logical byte offset of the chunk in the image
  uint32_t abo[kMaxOuter];    // LDS offset of the chunk's row scalar (row ops)
};

// Offsets of the staged byte at physical LDS position pb of the image: the
// logical byte lb (through the swizzle), its input and output byte offsets
// from the stage origin, its stage row (row ops) and the partial slots along
// which it lies past the edge.
struct ByteMap {
  uint32_t lb, xo, oo, row, ob, col;  // col: coordinate along the innermost dim (elements)
};

__device__ __forceinline__ ByteMap map_byte(CArgs* A, uint32_t pb, int n_axes, int swz_mask, int es_log2) {
  ByteMap r;
  r.lb = swz(pb, static_cast<uint32_t>(swz_mask));
  const uint32_t sub_byte = r.lb & ((1u << es_log2) - 1u);  // copies of elements wider than the chunk
  uint32_t e = r.lb >> es_log2;
  r.xo = sub_byte;
  r.oo = sub_byte;
  r.row = 0;
  r.col = 0;
  const uint32_t inner = A->ax_inner_mask;
  uint32_t rel[kPartial] = {0, 0, 0, 0};
#pragma nounroll
  for (int k = n_axes - 1; k >= 0; --k) {
    const uint32_t q = mdiv(e, A->ax_mag[k], A->ax_sh[k]);
    const uint32_t idx = e - q * A->ax_count[k];
    e = q;
    r.xo += idx * A->ax_xs[k];
    r.oo += idx * A->ax_os[k];
    r.row += idx * A->ax_rs[k];
    if ((inner >> k) & 1u) r.col += idx * A->ax_step[k];
    const int ps = A->ax_pslot[k];
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2)
      if (ps == s2) rel[s2] += idx * A->ax_step[k];
  }
  r.ob = 0;
#pragma unroll
  for (int s2 = 0; s2 < kPartial; ++s2)
    if (rel[s2] >= A->prem[s2]) r.ob |= 1u << s2;
  return r;
}

template <int VB>
__device__ __forceinline__ void build_map(CArgs* A, int wave, int lane, LaneMap& m) {
  const int outer = A->outer, waves = A->waves, n_axes = A->n_axes;
  const int swz_mask = A->swizzle, es_log2 = A->esize_log2;
#pragma unroll
  for (int g = 0; g < kMaxOuter; ++g) m.xoff[g] = m.ooff[g] = m.oobm[g] = m.lpos[g] = m.abo[g] = 0;
#pragma nounroll
  for (int f = 0; f < outer; ++f) {
    const ByteMap b = map_byte(A, ((f * waves + wave) * 64u + lane) * VB, n_axes, swz_mask, es_log2);
    const uint32_t abo = (b.row >> 5) * 256u + (b.row & 31u) * 4u;
#pragma unroll
    for (int g = 0; g < kMaxOuter; ++g)
      if (g == f) {
        m.xoff[g] = b.xo;
        m.ooff[g] = b.oo;
        m.oobm[g] = b.ob;
        m.lpos[g] = b.lb;
        m.abo[g] = abo;
      }
  }
}

// The same map for a round count known at compile time (the linear
// kernels): the axes run in the outer loop and the rounds in the inner one,
// so each axis' parameters are read once rather than once per round.  The
// fields equal build_map's: map_byte's walk, round by round.
template <int VB, int OUTER>
__device__ __forceinline__ void build_map_c(CArgs* A, int wave, int lane, LaneMap& m) {
  static_assert(OUTER >= 1 && OUTER <= kMaxOuter, "round count");
  const int waves = A->waves, n_axes = A->n_axes;
  const uint32_t swz_mask = static_cast<uint32_t>(A->swizzle);
  const int es_log2 = A->esize_log2;
#pragma unroll
  for (int g = 0; g < kMaxOuter; ++g) m.xoff[g] = m.ooff[g] = m.oobm[g] = m.lpos[g] = m.abo[g] = 0;
  uint32_t e[OUTER], row[OUTER], rel[OUTER][kPartial];
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    const uint32_t lb = swz(((static_cast<uint32_t>(f) * waves + wave) * 64u + lane) * VB, swz_mask);
    const uint32_t sub_byte = lb & ((1u << es_log2) - 1u);
    e[f] = lb >> es_log2;
    m.lpos[f] = lb;
    m.xoff[f] = sub_byte;
    m.ooff[f] = sub_byte;
    row[f] = 0;
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2) rel[f][s2] = 0;
  }
#pragma nounroll
  for (int k = n_axes - 1; k >= 0; --k) {
    const uint32_t mag = A->ax_mag[k], sh = A->ax_sh[k], cnt = A->ax_count[k];
    const uint32_t xs = A->ax_xs[k], os = A->ax_os[k], rs = A->ax_rs[k], step = A->ax_step[k];
    const int ps = A->ax_pslot[k];
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const uint32_t q = mdiv(e[f], mag, sh);
      const uint32_t idx = e[f] - q * cnt;
      e[f] = q;
      m.xoff[f] += idx * xs;
      m.ooff[f] += idx * os;
      row[f] += idx * rs;
#pragma unroll
      for (int s2 = 0; s2 < kPartial; ++s2)
        if (ps == s2) rel[f][s2] += idx * step;
    }
  }
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    uint32_t ob = 0;
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2)
      if (rel[f][s2] >= A->prem[s2]) ob |= 1u << s2;
    m.oobm[f] = ob;
    m.abo[f] = (row[f] >> 5) * 256u + (row[f] & 31u) * 4u;
  }
}

// Consumer pieces of a widening op: every 16-byte round of a wave (1 KiB of
// LDS) is consumed as two halves of 512 B, lane l taking the 8 bytes at
// 8 * l of each half.  Eight input bytes widen to 16 output bytes, so every
// store instruction writes 1 KiB of whole output rows instead of 16-byte
// pieces 32 bytes apart.  Piece 2 * f + h: output offset, partial slots and
// logical image byte.
template <int N>
__device__ __forceinline__ void build_pieces(CArgs* A, int wave, int lane, int outer, uint32_t (&oo)[N],
                                             uint32_t (&ob)[N], uint32_t (&lp)[N]) {
  const int waves = A->waves, n_axes = A->n_axes;
  const int swz_mask = A->swizzle, es_log2 = A->esize_log2;
#pragma unroll
  for (int g = 0; g < N; ++g) oo[g] = ob[g] = lp[g] = 0;
#pragma nounroll
  for (int q = 0; q < 2 * outer; ++q) {
    const uint32_t f = q >> 1, h = q & 1;
    const ByteMap b = map_byte(A, (f * waves + wave) * 1024u + h * 512u + lane * 8u, n_axes, swz_mask, es_log2);
#pragma unroll
    for (int g = 0; g < N; ++g)
      if (g == q) {
        oo[g] = b.oo;
        ob[g] = b.ob;
        lp[g] = b.lb;
      }
  }
}

// build_pieces for a piece count known at compile time (N = 2 * rounds): the
// axes in the outer loop, as in build_map_c.
template <int N>
__device__ __forceinline__ void build_pieces_c(CArgs* A, int wave, int lane, uint32_t (&oo)[N], uint32_t (&ob)[N],
                                               uint32_t (&lp)[N]) {
  const int waves = A->waves, n_axes = A->n_axes;
  const uint32_t swz_mask = static_cast<uint32_t>(A->swizzle);
  const int es_log2 = A->esize_log2;
  uint32_t e[N], rel[N][kPartial];
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const uint32_t f = static_cast<uint32_t>(q) >> 1, h = static_cast<uint32_t>(q) & 1u;
    const uint32_t lb = swz((f * waves + wave) * 1024u + h * 512u + lane * 8u, swz_mask);
    const uint32_t sub_byte = lb & ((1u << es_log2) - 1u);
    e[q] = lb >> es_log2;
    lp[q] = lb;
    oo[q] = sub_byte;
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2) rel[q][s2] = 0;
  }
#pragma nounroll
  for (int k = n_axes - 1; k >= 0; --k) {
    const uint32_t mag = A->ax_mag[k], sh = A->ax_sh[k], cnt = A->ax_count[k];
    const uint32_t os = A->ax_os[k], step = A->ax_step[k];
    const int ps = A->ax_pslot[k];
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const uint32_t d = mdiv(e[q], mag, sh);
      const uint32_t idx = e[q] - d * cnt;
      e[q] = d;
      oo[q] += idx * os;
#pragma unroll
      for (int s2 = 0; s2 < kPartial; ++s2)
        if (ps == s2) rel[q][s2] += idx * step;
    }
  }
#pragma unroll
  for (int q = 0; q < N; ++q) {
    uint32_t b = 0;
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2)
      if (rel[q][s2] >= A->prem[s2]) b |= 1u << s2;
    ob[q] = b;
  }
}

// Launch values the ring touches every trip, read from the argument block
// once: they then live in registers across the asm statements (whose memory
// clobbers would otherwise force a reload of every argument per trip).
struct Loc {
  const char* in[3];
  char* out;
  uint64_t in_span, out_span, total_rows;
  int64_t lin_x, lin_o, lin_r;
  int lin, load_nt, store_nt;
  int outer, waves, n_in, row_ops, ab_instr;
  uint32_t in_image_bytes, slot_bytes, ab_off, ab_wave_bytes, out_image_off, subs, tile0;
};

__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  return (static_cast<uint64_t>(uni(static_cast<uint32_t>(v >> 32))) << 32) | uni(static_cast<uint32_t>(v));
}
template <typename P> __device__ __forceinline__ P* unip(P* p) {
  return reinterpret_cast<P*>(uni64(reinterpret_cast<uint64_t>(p)));
}

// Every value passes through readfirstlane: the result is a register value
// the compiler cannot re-derive by reloading the argument block inside the
// ring (a reload would also cost an lgkmcnt wait that drains the LDS reads).
__device__ __forceinline__ Loc load_loc(CArgs* A) {
  Loc L;
  for (int k = 0; k < 3; ++k) L.in[k] = unip(A->in[k]);
  L.out = unip(A->out);
  L.in_span = uni64(A->in_span);
  L.out_span = uni64(A->out_span);
  L.total_rows = uni64(A->total_rows);
  L.lin_x = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_x)));
  L.lin_o = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_o)));
  L.lin_r = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_r)));
  L.lin = uni(A->lin);
  L.load_nt = uni(A->load_nt);
  L.store_nt = uni(A->store_nt);
  L.outer = uni(A->outer);
  L.waves = uni(A->waves);
  L.n_in = uni(A->n_in);
  L.row_ops = uni(A->row_ops);
  L.ab_instr = uni(A->ab_instr);
  L.in_image_bytes = uni(A->in_image_bytes);
  L.slot_bytes = uni(A->slot_bytes);
  L.ab_off = uni(A->ab_off);
  L.ab_wave_bytes = uni(A->ab_wave_bytes);
  L.out_image_off = uni(A->out_image_off);
  L.subs = uni(A->subs);
  L.tile0 = uni(A->tile0);
  return L;
}

struct Trip {
  uint64_t xbase, obase, rbase;
  uint32_t last;   // partial slots along which this stage is the cut last one
  bool beyond;     // stage lies entirely past the tensor
};

__device__ __forceinline__ Trip trip_geometry(CArgs* A, const Loc& L, uint32_t wg, uint32_t grid, int j) {
  Trip t{0, 0, 0, 0u, false};
  if (L.lin) {
    // one stage per tile, exact tiling, row-major contiguous grid
    const uint64_t s = static_cast<uint64_t>(L.tile0) + wg + static_cast<uint64_t>(j) * grid;
    t.xbase = s * static_cast<uint64_t>(L.lin_x);
    t.obase = s * static_cast<uint64_t>(L.lin_o);
    t.rbase = s * static_cast<uint64_t>(L.lin_r);
    return t;
  }
  const uint32_t tl = mdiv(static_cast<uint32_t>(j), A->subs_mag, A->subs_sh);
  uint32_t sub = static_cast<uint32_t>(j) - tl * L.subs;
  uint32_t tile = L.tile0 + wg + tl * grid;
#pragma nounroll
  for (int d = A->rank - 1; d >= 0; --d) {
    const uint32_t qt = mdiv(tile, A->tg_mag[d], A->tg_sh[d]);
    const uint32_t tc = tile - qt * A->tgrid[d];
    tile = qt;
    const uint32_t qs = mdiv(sub, A->sub_mag[d], A->sub_sh[d]);
    const uint32_t scs = sub - qs * A->sub[d];
    sub = qs;
    const uint32_t sc = tc * A->sub[d] + scs;
    if (sc >= A->nst[d]) t.beyond = true;
    const int ps = A->pslot_of_dim[d];
    if (ps >= 0 && sc + 1 == A->nst[d]) t.last |= 1u << ps;
    t.xbase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->xstep[d]);
    t.obase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->ostep[d]);
    t.rbase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->rstep[d]);
  }
  if (t.beyond) t.xbase = t.obase = t.rbase = 0;
  return t;
}

// Per-lane row-scalar sources: lane l < 32 loads a[row], l >= 32 loads b[row]
// for stage rows q * 32 + (l & 31).  row_ptr[0] is the lane's array,
// row_ptr[1 + q] the row's byte offset from the stage's first row, row_bad[q]
// the partial slots along which the row lies past the edge (all bits when
// the stage has no such row).
__device__ __forceinline__ void build_rows(CArgs* A, int lane, uint64_t* row_ptr, uint32_t* row_bad) {
  // both pointers are read as scalars first: a lane-dependent address into
  // the argument block would become a vector load whose wait lands in the ring
  const uint64_t pa = reinterpret_cast<uint64_t>(A->row_a), pb = reinterpret_cast<uint64_t>(A->row_b);
  const uint64_t ua = (static_cast<uint64_t>(uni(static_cast<uint32_t>(pa >> 32))) << 32) | uni(static_cast<uint32_t>(pa));
  const uint64_t ub = (static_cast<uint64_t>(uni(static_cast<uint32_t>(pb >> 32))) << 32) | uni(static_cast<uint32_t>(pb));
  row_ptr[0] = lane < 32 ? ua : ub;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    row_ptr[1 + q] = 0;
    row_bad[q] = ~0u;
    if (!A->row_ops || q >= A->ab_instr) continue;
    uint32_t r = q * 32u + (lane & 31);
    if (r >= static_cast<uint32_t>(A->n_rows)) continue;
    uint64_t off = 0;
    uint32_t bad = 0;
    for (int d = A->rank - 2; d >= 0; --d) {
      const uint32_t sb = A->sbox[d];
      const uint32_t rel = r % sb;
      r /= sb;
      off += static_cast<uint64_t>(rel) * static_cast<uint64_t>(A->rstep[d] / sb);
      const int ps = A->pslot_of_dim[d];
      if (ps >= 0 && rel >= A->prem[ps]) bad |= 1u << ps;
    }
    row_ptr[1 + q] = off * 4u;
    row_bad[q] = bad;
  }
}

template <int OB, int CP>
__device__ __forceinline__ void store_chunk_cp(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const uint32_t* w) {
  if constexpr (OB == 32) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rs, voff, 0, CP);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[4], w[5], w[6], w[7]}, rs, voff + 16u, 0, CP);
  } else if constexpr (OB == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rs, voff, 0, CP);
  } else if constexpr (OB == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rs, voff, 0, CP);
  } else if constexpr (OB == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, voff, 0, CP);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[0]), rs, voff, 0, CP);
  }
}

// Stores go out non-temporal (cache policy bit NT) unless disabled: the
// output is written once and never read back by the kernel.
template <int OB>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const uint32_t* w, bool nt) {
  if (nt)
    store_chunk_cp<OB, 2>(rs, voff, w);
  else
    store_chunk_cp<OB, 0>(rs, voff, w);
}

template <class OP, int VB>
struct ChunkShape {
  static constexpr int EI = sizeof(typename OP::TI);
  static constexpr int EO = sizeof(typename OP::TO);
  static constexpr int NE = VB / EI;            // elements per chunk
  static constexpr int OB = NE * EO;            // output bytes per chunk
  static constexpr int ST = OB == 32 ? 2 : 1;   // stores per chunk
};


// Rounds consumed together: the largest power of two dividing `total` (a
// power of two) whose staged operands (ns each) stay within `cap` registers'
// worth of chunks.
constexpr int round_group(int total, int ns, int cap) {
  int g = total;
  while (g > 1 && g * (ns > 0 ? ns : 1) > cap) g /= 2;
  return g;
}

}  // namespace dev
}  // namespace acp
