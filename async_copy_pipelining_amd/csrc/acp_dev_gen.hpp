// The general lean kernel: any stage grid, trip geometry in VGPR lanes.
#pragma once

#include "acp_dev_lin.hpp"

namespace acp {
namespace dev {

// ---------------------------------------------------------------------------
// General lean kernel: any stage grid (partial and out-of-range stages,
// sub-stages inside a workgroup tile, persistent grids), 16-byte rounds,
// OUTER rounds per thread known at compile time.  Trip geometry lives in a
// table in VGPR lanes: lane l of every wave computes trip (batch * 64 + l)
// with vector arithmetic, and each trip reads its row with v_readlane.  Two
// table sets alternate so that the load cursor (up to S-1 trips ahead) can
// enter the next batch while the consume cursor finishes the current one.

struct TripRow {
  uint32_t xlo, xhi, olo, ohi, rlo, flags;  // flags: bits 0..3 last-stage slots, bit 8 out of range
};

__device__ __forceinline__ TripRow trip_lane(CArgs* A, uint32_t wg, uint32_t grid, uint32_t tile0, uint32_t subs,
                                             uint32_t subs_mag, uint32_t subs_sh, int rank, uint32_t tpt_log2,
                                             uint32_t j) {
  const uint32_t tl = mdiv(j, subs_mag, subs_sh);
  uint32_t sub = j - tl * subs;
  const uint32_t per_wg = A->per_wg;
  uint32_t tile = per_wg ? tile0 + wg * per_wg + tl
                         : tile0 + (((wg + (tl >> tpt_log2) * grid) << tpt_log2) | (tl & ((1u << tpt_log2) - 1u)));
  uint64_t xb = 0, ob = 0, rb = 0;
  uint32_t flags = 0;
  // rolled: the per-dim parameters are read on each refill (once per 64
  // trips) rather than held in scalar registers across the ring
#pragma nounroll
  for (int d = rank - 1; d >= 0; --d) {
    const uint32_t qt = mdiv(tile, A->tg_mag[d], A->tg_sh[d]);
    const uint32_t tc = tile - qt * A->tgrid[d];
    tile = qt;
    const uint32_t qs = mdiv(sub, A->sub_mag[d], A->sub_sh[d]);
    const uint32_t scs = sub - qs * A->sub[d];
    sub = qs;
    const uint32_t sc = tc * A->sub[d] + scs;
    const uint32_t nst = A->nst[d];
    if (sc >= nst) flags |= 0x100u;
    const int ps = A->pslot_of_dim[d];
    if (ps >= 0 && sc + 1 == nst) flags |= 1u << ps;
    xb += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->xstep[d]);
    ob += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->ostep[d]);
    rb += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->rstep[d]);
  }
  if (tile != 0) flags |= 0x100u;  // past the last tile
  if (flags & 0x100u) xb = ob = rb = 0;
  return TripRow{static_cast<uint32_t>(xb), static_cast<uint32_t>(xb >> 32), static_cast<uint32_t>(ob),
                 static_cast<uint32_t>(ob >> 32), static_cast<uint32_t>(rb), flags};
}

__device__ __forceinline__ uint32_t rdl(uint32_t v, uint32_t lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), static_cast<int>(lane)));
}

template <class OP, int MODE, int OUTER, bool SROW, int ZSET = 0, bool GROUP = false, bool NT = false>
struct GenPolicy {
  static constexpr bool STAGE_OUT = (MODE == 1);
  // staged operands: every input of a tile op or of a two-tensor stream op;
  // streams with per-row scalars stage x only
  static constexpr int NS = (MODE == 0 || OP::ROW) ? 1 : OP::NIN;
  // ZSET: the last staged operand is loaded synchronously (registers, wait,
  // LDS store) into its image instead of by a direct-to-LDS load
  static constexpr int NDMA = ZSET ? NS - 1 : NS;
  // widening ops (16 input bytes -> 32 output bytes) consume 8-byte pieces
  // (tile ops up to 4 rounds: beyond, the piece maps no longer fit in registers)
  static constexpr bool SPLIT = (MODE == 2 || (MODE == 1 && OUTER <= 4)) && ChunkShape<OP, 16>::OB == 32;
  static constexpr int NP = SPLIT ? 2 * OUTER : 1;
  uint32_t pooff[NP], poobm[NP], plpos[NP];
  CArgs* A;
  unsigned char* lds;
  const char* in[3];
  char* out;
  uint64_t in_span, out_span, total_rows;
  uint32_t lds0, slot_bytes, in_image_bytes, out_image_off, ab_base, waves_kb, wg, grid, tile0, subs, subs_mag, subs_sh;
  uint32_t tpt_log2, tile_lds;  // tiles per trip (log2) and LDS bytes of one tile's images in a slot
  // row reduction (MODE 4): each round's partial-sum index (row * row_chunks
  // + chunk of the row), and the reduction geometry
  uint32_t pidx[OUTER];
  uint32_t row_chunks, red_rows, part_off, part_bytes, waves;
  uint32_t red_off, red_bad;  // lane k: packed-row offset and cut-edge slots of the wave's k-th row
  // store with reduce-add over batch dims: trips per destination tile, the
  // trips summed so far and the lane's running sums
  uint32_t red_group, rcount;
  typename AccOf<OP, MODE>::T racc[GROUP ? OUTER : 1];
  // wave-local rows: lane k holds the wave's k-th distinct row (in round
  // order; ~0 for none), its packed-row offset and cut-edge slots
  bool red_local;
  bool one_row;      // wave-local: all of the wave's blocks lie in one row
  uint32_t lrow, loff, lbad;
  int wave, lane, rank, ab_instr, swizzle, esize_log2;
  bool load_nt, store_nt;  // NT: both known to be set
  uint32_t xoff[OUTER], ooff[OUTER], oobm[OUTER], lpos[OUTER], abo[OUTER];
  // two table sets as separate members: a dynamically indexed array would
  // live in scratch memory, whose loads share the wave's vmcnt with the ring
  TripRow tab0, tab1;
  uint64_t row_ptr[3];   // [0] lane's array, [1 + q] row byte offset in the stage
  uint32_t row_bad[2];   // partial slots along which the lane's row q lies past the edge
  // SROW: this wave's row (relative to the stage) of each round, and the
  // scalars of the trip being consumed, read through the scalar cache
  const float __attribute__((address_space(4)))* ca;
  const float __attribute__((address_space(4)))* cb;
  uint32_t row_of[OUTER];
  float sa[OUTER], sb[OUTER];

  __device__ __forceinline__ void fill(int set, uint32_t j0) {
    const TripRow r =
        trip_lane(A, wg, grid, tile0, subs, subs_mag, subs_sh, rank, tpt_log2, j0 + static_cast<uint32_t>(lane));
    // field-wise selects: a conditional store of the whole row would be
    // merged into one store through a selected address, i.e. into memory
    const bool lo = set == 0;
    tab0 = TripRow{lo ? r.xlo : tab0.xlo, lo ? r.xhi : tab0.xhi, lo ? r.olo : tab0.olo,
                   lo ? r.ohi : tab0.ohi, lo ? r.rlo : tab0.rlo, lo ? r.flags : tab0.flags};
    tab1 = TripRow{lo ? tab1.xlo : r.xlo, lo ? tab1.xhi : r.xhi, lo ? tab1.olo : r.olo,
                   lo ? tab1.ohi : r.ohi, lo ? tab1.rlo : r.rlo, lo ? tab1.flags : r.flags};
  }
  struct T {
    uint64_t xb, ob, rb;
    uint32_t flags;
  };
  __device__ __forceinline__ T row(int j) const {
    const uint32_t l = static_cast<uint32_t>(j) & 63u;
    const bool hi = ((j >> 6) & 1) != 0;
    T t;
    t.xb = (static_cast<uint64_t>(rdl(hi ? tab1.xhi : tab0.xhi, l)) << 32) | rdl(hi ? tab1.xlo : tab0.xlo, l);
    t.ob = (static_cast<uint64_t>(rdl(hi ? tab1.ohi : tab0.ohi, l)) << 32) | rdl(hi ? tab1.olo : tab0.olo, l);
    t.rb = rdl(hi ? tab1.rlo : tab0.rlo, l);
    t.flags = rdl(hi ? tab1.flags : tab0.flags, l);
    return t;
  }

  // Table entry e is the workgroup's e-th tile (tile ops) or stage; ring
  // trip j holds entries j * 2^tpt_log2 ... (a batch boundary of the table
  // always falls on the first entry of a trip).
  __device__ __forceinline__ void load(int j, int slot) {
    const int e0 = j << tpt_log2;
    if (e0 > 0 && (e0 & 63) == 0) fill((e0 >> 6) & 1, static_cast<uint32_t>(e0));
#pragma nounroll
    for (int u = 0; u < (1 << tpt_log2); ++u) load_entry(e0 + u, slot * slot_bytes + u * tile_lds);
  }

  __device__ __forceinline__ void load_entry(int j, uint32_t sl) {
    const T t = row(j);
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    const uint32_t sbase = lds0 + sl + wave * 1024u;
#pragma unroll
    for (int k = 0; k < NDMA; ++k) {
      const v4i rs = rsrc_v4(in[k] + t.xb, range_from(in_span, t.xb));
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const bool ok = !beyond && (oobm[f] & last) == 0;
        dma_b128(rs, ok ? xoff[f] : kOobOffset, sbase + k * in_image_bytes + f * waves_kb, NT || load_nt);
      }
    }
    if constexpr (ZSET) {
      // synchronous staging: the data must reach registers before it can be
      // stored to LDS, so the wave waits for all its outstanding loads here
      const __amdgpu_buffer_rsrc_t rz = rsrc_store(const_cast<char*>(in[NDMA]) + t.xb, range_from(in_span, t.xb));
      u32x4 zv[OUTER];
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const bool ok = !beyond && (oobm[f] & last) == 0;
        zv[f] = __builtin_amdgcn_raw_buffer_load_b128(rz, ok ? xoff[f] : kOobOffset, 0, 0);
      }
      wait_vmcnt(0);
#pragma unroll
      for (int f = 0; f < OUTER; ++f)
        *reinterpret_cast<u32x4*>(__builtin_assume_aligned(
            lds + sl + NDMA * in_image_bytes + f * waves_kb + wave * 1024u + lane * 16u, 16)) = zv[f];
    }
    if constexpr (OP::ROW && !SROW) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= ab_instr) continue;
        const bool ok = !beyond && (row_bad[q] & last) == 0;
        uint64_t r = ok ? t.rb + row_ptr[1 + q] / 4u : 0u;
        if (r >= total_rows) r = 0;
        dma_global_b32(reinterpret_cast<const void*>(row_ptr[0] + r * 4u), lds0 + sl + ab_base + q * 256u);
      }
    }
  }

  __device__ __forceinline__ void pre_wait(int i, int, int) {
    if constexpr (OP::ROW && SROW) {
      // rows of a cut stage may lie past the tensor: their results are
      // never stored, and they read row 0 instead of memory past the arrays
      const T t = row(i);
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        uint64_t r = t.rb + row_of[f];
        if (r >= total_rows) r = 0;
        sa[f] = ca[r];
        sb[f] = cb[r];
      }
    }
  }

  // Widening ops: 8 input bytes per lane and piece, 16 output bytes.
  __device__ __forceinline__ void consume_pieces(__amdgpu_buffer_rsrc_t rs, uint32_t sl, bool beyond, uint32_t last) {
    typedef typename OP::TI TI;
    typedef typename OP::TO TO;
    constexpr int NE = 8 / sizeof(TI);
    constexpr int GRP = round_group(NP, NS, 32);
    static_assert(NP % GRP == 0, "piece groups must tile the pieces");
#pragma unroll
    for (int g0 = 0; g0 < NP; g0 += GRP) {
      u32x2 v[NS > 0 ? NS : 1][GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = g0 + u, f = q >> 1, h = q & 1;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          v[k][u] = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(
              lds + sl + k * in_image_bytes + f * waves_kb + wave * 1024u + h * 512u + lane * 8u, 8));
        if constexpr (NS == 0) v[0][u] = u32x2{0, 0};
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = g0 + u;
        TI in0[NE], in1[NE], in2[NE];
        __builtin_memcpy(in0, &v[0][u], 8);
        __builtin_memcpy(in1, &v[NS > 1 ? 1 : 0][u], 8);
        __builtin_memcpy(in2, &v[NS > 2 ? 2 : 0][u], 8);
        TO res[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) res[e] = OP::f(in0[e], in1[e], in2[e], 0.f, 0.f);
        uint32_t words[4];
        __builtin_memcpy(words, res, 16);
        if constexpr (STAGE_OUT) {
          const uint32_t lo = (plpos[q] >> esize_log2) * sizeof(TO);
          __builtin_memcpy(lds + out_image_off + swz(lo, swizzle), words, 16);
          asm volatile("" ::: "memory");
          __builtin_memcpy(words, lds + out_image_off + swz(lo, swizzle), 16);
        }
        const bool ok = !beyond && (poobm[q] & last) == 0;
        store_chunk<16>(rs, ok ? pooff[q] : kOobOffset, words, NT || store_nt);
      }
    }
  }

  // Row reduction of one staged trip.  Each lane sums its chunks and puts
  // the partials into LDS at (row, chunk of the row); after a workgroup
  // barrier each wave reduces whole rows: lane-strided sums over the row's
  // chunks, then a DPP sum across the 64 lanes, in a fixed order.  Lane 0
  // stores the row's sum.  Partials alternate between two buffers, so the
  // next trip's writes never meet this trip's reads (every wave passes the
  // next barrier only after finishing them).
  // Rows that a single wave holds entirely (each 1 KiB wave block inside one
  // row): the wave sums each block (chunk sums, then a DPP sum over the 64
  // lanes); lane k accumulates the blocks of the wave's k-th row in round
  // order, and one store instruction writes every row total of the trip.
  // No other wave is involved, so there is no barrier.
  __device__ __forceinline__ void reduce_rows_local(uint32_t sl, const T& t, __amdgpu_buffer_rsrc_t rs) {
    float part[OUTER];
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
      part[f] = OP::chunk(v);
    }
    float acc = 0.f;
    if (one_row) {
      // every block of the wave lies in one row: each lane adds its chunk
      // partials in round order, then one cross-lane sum
      float p = part[0];
#pragma unroll
      for (int f = 1; f < OUTER; ++f) p += part[f];
      acc = wave_sum(p);
    } else {
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const float s = wave_sum(part[f]);
        acc += (lrow == row_of[f]) ? s : 0.f;
      }
    }
    const bool ok = (t.flags & 0x100u) == 0 && lrow != ~0u && (lbad & t.flags & 0xFFu) == 0;
    const uint64_t g = t.rb + loff;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), rs,
                                          ok ? static_cast<uint32_t>(g * 4u) : kOobOffset, 0, 0);
  }

  __device__ __forceinline__ void reduce_rows_trip(int i, uint32_t sl, const T& t, __amdgpu_buffer_rsrc_t rs) {
    if (red_local) {
      reduce_rows_local(sl, t, rs);
      return;
    }
    const uint32_t buf = part_off + (static_cast<uint32_t>(i) & 1u) * part_bytes;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
      *reinterpret_cast<float*>(lds + buf + pidx[f] * 4u) = OP::chunk(v);
    }
    // only LDS traffic is waited for: the ring's loads stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    uint32_t k = 0;
#pragma nounroll
    for (uint32_t r = static_cast<uint32_t>(wave); r < red_rows; r += waves, ++k) {
      float acc = 0.f;
      for (uint32_t c = static_cast<uint32_t>(lane); c < row_chunks; c += 64u)
        acc += *reinterpret_cast<const float*>(lds + buf + (r * row_chunks + c) * 4u);
      acc = wave_sum(acc);
      // the row's place in the tensor and the cut edges it lies past (lane k
      // of the wave holds them for the wave's k-th row)
      const uint32_t roff = rdl(red_off, k), rbad = rdl(red_bad, k);
      const bool ok = !beyond && (rbad & last) == 0;
      const uint64_t g = t.rb + roff;
      if (lane == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), rs,
                                              ok ? static_cast<uint32_t>(g * 4u) : kOobOffset, 0, 0);
    }
  }

  __device__ __forceinline__ void consume(int i, int slot) {
    const int e0 = i << tpt_log2;
#pragma nounroll
    for (int u = 0; u < (1 << tpt_log2); ++u) consume_entry(e0 + u, slot * slot_bytes + u * tile_lds);
  }

  __device__ __forceinline__ void consume_entry(int i, uint32_t sl) {
    typedef ChunkShape<OP, 16> CS;
    typedef typename OP::TI TI;
    typedef typename OP::TO TO;
    const T t = row(i);
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    const __amdgpu_buffer_rsrc_t rs = rsrc_store(out + t.ob, range_from(out_span, t.ob));
    if constexpr (SPLIT) {
      consume_pieces(rs, sl, beyond, last);
      return;
    }
    if constexpr (MODE == 4) {
      reduce_rows_trip(i, sl, t, rs);
      return;
    }
    if constexpr (MODE == 3) {
      if constexpr (GROUP) {
        // sum the group's contributions in registers; the group's last trip
        // adds the sums into the destination (past-the-end chunks were
        // staged as zeros and add nothing)
#pragma unroll
        for (int f = 0; f < OUTER; ++f) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(
              __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
          racc[f] = OP::accumulate(racc[f], v);
        }
        if (++rcount == red_group) {
          rcount = 0;
#pragma unroll
          for (int f = 0; f < OUTER; ++f) {
            const bool ok = !beyond && (oobm[f] & last) == 0;
            const uint32_t o = ok ? ooff[f] : kOobOffset;
            const u32x4 w = OP::finish(racc[f]);
            OP::add(rs, o, w.x);
            OP::add(rs, o + 4u, w.y);
            OP::add(rs, o + 8u, w.z);
            OP::add(rs, o + 12u, w.w);
            racc[f] = OP::zero_acc();
          }
        }
        return;
      }
      // store with reduce-add: four 4-byte atomics per staged chunk
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
        const bool ok = !beyond && (oobm[f] & last) == 0;
        const uint32_t o = ok ? ooff[f] : kOobOffset;
        OP::add(rs, o, v.x);
        OP::add(rs, o + 4u, v.y);
        OP::add(rs, o + 8u, v.z);
        OP::add(rs, o + 12u, v.w);
      }
      return;
    }
    // rounds in groups whose staged operands fit in registers together
    constexpr int GRP = round_group(OUTER, NS, 16);
    static_assert(OUTER % GRP == 0, "round groups must tile the rounds");
#pragma unroll
    for (int g0 = 0; g0 < OUTER; g0 += GRP) {
      u32x4 v[NS > 0 ? NS : 1][GRP];
      float ra[GRP], rb[GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int f = g0 + u;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          v[k][u] = *reinterpret_cast<const u32x4*>(
              __builtin_assume_aligned(lds + sl + k * in_image_bytes + f * waves_kb + wave * 1024u + lane * 16u, 16));
        if constexpr (NS == 0) v[0][u] = u32x4{0, 0, 0, 0};
        if constexpr (OP::ROW && SROW) {
          ra[u] = sa[f];
          rb[u] = sb[f];
        } else if constexpr (OP::ROW) {
          ra[u] = *reinterpret_cast<const float*>(lds + sl + ab_base + abo[f]);
          rb[u] = *reinterpret_cast<const float*>(lds + sl + ab_base + abo[f] + 128u);
        } else {
          ra[u] = rb[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int f = g0 + u;
        TI in0[CS::NE], in1[CS::NE], in2[CS::NE];
        __builtin_memcpy(in0, &v[0][u], 16);
        __builtin_memcpy(in1, &v[NS > 1 ? 1 : 0][u], 16);
        __builtin_memcpy(in2, &v[NS > 2 ? 2 : 0][u], 16);
        TO res[CS::NE];
#pragma unroll
        for (int e = 0; e < CS::NE; ++e) res[e] = OP::f(in0[e], in1[e], in2[e], ra[u], rb[u]);
        uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        __builtin_memcpy(words, res, CS::OB);
        if constexpr (STAGE_OUT) {
          // the output tile is LDS-resident ("elementwise -> smem") and is copied out from there
          const uint32_t lo = (lpos[f] >> esize_log2) * CS::EO;
          constexpr int P = (CS::OB + 15) / 16;
          constexpr int PB = CS::OB < 16 ? CS::OB : 16;
#pragma unroll
          for (int piece = 0; piece < P; ++piece) {
            const uint32_t lp = lo + piece * 16;
            __builtin_memcpy(lds + out_image_off + swz(lp, swizzle), words + piece * 4, PB);
          }
          asm volatile("" ::: "memory");
#pragma unroll
          for (int piece = 0; piece < P; ++piece) {
            const uint32_t lp = lo + piece * 16;
            __builtin_memcpy(words + piece * 4, lds + out_image_off + swz(lp, swizzle), PB);
          }
        }
        const bool ok = !beyond && (oobm[f] & last) == 0;
        store_chunk<CS::OB>(rs, ok ? ooff[f] : kOobOffset, words, NT || store_nt);
      }
    }
  }
};

template <class OP, int MODE, int OUTER, bool SROW, int ZSET, bool GROUP, bool NT>
__device__ __forceinline__ void gen_body(CArgs* A, unsigned char* lds, uint32_t warm) {
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t tpt_log2 = uni(A->tpt_log2);
  const uint32_t groups = (A->n_tiles + (1u << tpt_log2) - 1u) >> tpt_log2;
  const uint32_t per_wg = uni(A->per_wg);
  const uint32_t first = wg * per_wg;
  const uint32_t mine = per_wg ? (first < A->n_tiles ? min(per_wg, A->n_tiles - first) : 0u)
                               : (wg < groups ? (groups - wg + grid - 1) / grid : 0);
  const int n = static_cast<int>(mine * A->subs);  // ring trips
  if (n == 0) {
    karg_warm_done(warm);
    return;
  }
  LaneMap m;
  // the lane map with the axes outside the rounds (store with reduce-add
  // keeps the per-round walk: measured 1.6 % faster there)
  if constexpr (MODE == 3)
    build_map<16>(A, wave, lane, m);
  else
    build_map_c<16, OUTER>(A, wave, lane, m);
  uint64_t row_ptr[3] = {0, 0, 0};
  uint32_t row_bad[2] = {~0u, ~0u};
  if constexpr (OP::ROW && !SROW) build_rows(A, lane, row_ptr, row_bad);
  const Loc L = load_loc(A);
  GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP, NT> p;
  p.tpt_log2 = tpt_log2;
  p.tile_lds = L.slot_bytes >> tpt_log2;
  p.A = A;
  p.lds = lds;
  for (int k = 0; k < 3; ++k) p.in[k] = L.in[k];
  p.out = L.out;
  p.in_span = L.in_span;
  p.out_span = L.out_span;
  p.total_rows = L.total_rows;
  p.lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  p.slot_bytes = L.slot_bytes;
  p.in_image_bytes = L.in_image_bytes;
  p.out_image_off = L.out_image_off;
  p.ab_base = L.ab_off + wave * L.ab_wave_bytes;
  p.waves_kb = static_cast<uint32_t>(L.waves) * 1024u;
  p.wg = wg;
  p.grid = grid;
  p.tile0 = L.tile0;
  p.subs = L.subs;
  p.subs_mag = uni(A->subs_mag);
  p.subs_sh = uni(A->subs_sh);
  p.wave = wave;
  p.lane = lane;
  p.rank = uni(A->rank);
  p.ab_instr = L.ab_instr;
  p.swizzle = uni(A->swizzle);
  p.esize_log2 = uni(A->esize_log2);
  p.load_nt = L.load_nt != 0;
  p.store_nt = L.store_nt != 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) p.row_ptr[q] = row_ptr[q];
#pragma unroll
  for (int q = 0; q < 2; ++q) p.row_bad[q] = row_bad[q];
  p.ca = (const float __attribute__((address_space(4)))*)(unip(A->row_a));
  p.cb = (const float __attribute__((address_space(4)))*)(unip(A->row_b));
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    p.xoff[f] = m.xoff[f];
    p.ooff[f] = m.ooff[f];
    p.oobm[f] = m.oobm[f];
    p.lpos[f] = m.lpos[f];
    p.abo[f] = m.abo[f];
    const uint32_t abo = uni(m.abo[f]);
    p.row_of[f] = (abo >> 8) * 32u + (abo & 255u) / 4u;
    p.sa[f] = p.sb[f] = 0.f;
  }
  if constexpr (GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP, NT>::SPLIT) {
    // the piece map with the axes outside the pieces, up to 8 pieces (above
    // that the per-piece walk keeps the register count down)
    if constexpr (2 * OUTER <= 8 && GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP, NT>::NP == 2 * OUTER)
      build_pieces_c(A, wave, lane, p.pooff, p.poobm, p.plpos);
    else
      build_pieces(A, wave, lane, OUTER, p.pooff, p.poobm, p.plpos);
  }
  if constexpr (GROUP) {
    p.red_group = uni(A->red_group);
    p.rcount = 0;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) p.racc[f] = OP::zero_acc();
  }
  int red_stores = 0;  // row reduction: rows this wave stores per trip
  if constexpr (MODE == 4) {
    p.row_chunks = uni(A->row_chunks);
    p.red_rows = uni(A->red_rows);
    p.part_off = uni(A->part_off);
    p.part_bytes = uni(A->part_bytes);
    p.waves = static_cast<uint32_t>(L.waves);
    const int n_axes = uni(A->n_axes), swz_mask = uni(A->swizzle), es_log2 = uni(A->esize_log2);
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const ByteMap b = map_byte(A, ((f * L.waves + wave) * 64u + lane) * 16u, n_axes, swz_mask, es_log2);
      p.pidx[f] = b.row * p.row_chunks + ((b.col << es_log2) >> 4);
    }
    red_stores = static_cast<uint32_t>(wave) < p.red_rows
                     ? static_cast<int>((p.red_rows - wave + p.waves - 1) / p.waves) : 0;
    // lane k: the wave's k-th row r = wave + k * waves of a stage (at most
    // 64 per wave): its packed-row offset from the stage's first row and the
    // partial slots along which it lies past the edge of a cut stage
    const uint32_t r = static_cast<uint32_t>(wave) + static_cast<uint32_t>(lane) * p.waves;
    uint32_t rr = r < p.red_rows ? r : 0u, off = 0, bad = 0;
    for (int dd = p.rank - 2; dd >= 0; --dd) {
      const uint32_t sb = A->sbox[dd];
      const uint32_t rel = rr % sb;
      rr /= sb;
      off += rel * A->rowstr[dd];
      const int ps = A->pslot_of_dim[dd];
      if (ps >= 0 && rel >= A->prem[ps]) bad |= 1u << ps;
    }
    p.red_off = off;
    p.red_bad = bad;
    p.red_local = uni(A->red_local) != 0;
    p.one_row = true;
#pragma unroll
    for (int f = 1; f < OUTER; ++f) p.one_row = p.one_row && p.row_of[f] == p.row_of[0];
    p.lrow = ~0u;
    p.loff = p.lbad = 0;
    if (p.red_local) {
      // the wave's distinct block rows in round order; lane k takes the k-th
      uint32_t n_local = 0;
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        bool seen = false;
#pragma unroll
        for (int g = 0; g < f; ++g) seen = seen || (p.row_of[g] == p.row_of[f]);
        if (!seen) {
          if (static_cast<uint32_t>(lane) == n_local) p.lrow = p.row_of[f];
          ++n_local;
        }
      }
      uint32_t rr2 = p.lrow != ~0u ? p.lrow : 0u, off2 = 0, bad2 = 0;
      for (int dd = p.rank - 2; dd >= 0; --dd) {
        const uint32_t sb = A->sbox[dd];
        const uint32_t rel = rr2 % sb;
        rr2 /= sb;
        off2 += rel * A->rowstr[dd];
        const int ps = A->pslot_of_dim[dd];
        if (ps >= 0 && rel >= A->prem[ps]) bad2 |= 1u << ps;
      }
      p.loff = off2;
      p.lbad = bad2;
      red_stores = 1;  // one store instruction per trip
    }
  }
  p.tab1 = TripRow{0, 0, 0, 0, 0, 0};
  p.fill(0, 0u);
  karg_warm_done(warm);
  typedef ChunkShape<OP, 16> CS;
  constexpr int NS = GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP, NT>::NS;
  // copies and streams with one tile per trip take the ring whose waits are
  // compile-time counts (the per-trip counts are known here)
  if constexpr ((MODE == 0 || MODE == 2) && !(OP::ROW && !SROW)) {
    if (tpt_log2 == 0) {
      run_ring_fixed<NS * OUTER, OUTER * CS::ST>(p, n, uni(A->stages));
      return;
    }
  }
  // grouped reduce-add: atomics only on a group's last trip, counted as none
  // per trip (the waits are then only stronger), one tile per trip
  if constexpr (MODE == 3 && GROUP) {
    if (tpt_log2 == 0) {
      run_ring_fixed<NS * OUTER, 0>(p, n, uni(A->stages));
      return;
    }
  }
  const int d = (NS * OUTER + ((OP::ROW && !SROW) ? L.ab_instr : 0)) << tpt_log2;
  // grouped reduce-add stores only on a group's last trip: counting none
  // per trip only makes the waits stronger
  const int st = MODE == 4 ? red_stores : (MODE == 3 ? (GROUP ? 0 : OUTER * 4) : OUTER * CS::ST);
  run_ring(p, n, uni(A->stages), d, st << tpt_log2);
}

// Copies and grouped reduce-adds with non-temporal loads and stores get a
// body with the cache policy fixed at compile time, so no load or store of a
// trip branches on it.
template <class OP, int MODE, int OUTER, bool SROW, int ZSET = 0, bool GROUP = false>
__global__ __launch_bounds__(1024) void gen_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  const uint32_t warm = prefetch_kargs();
  CArgs* A = kargs();
  if constexpr (MODE == 0 || (MODE == 3 && GROUP)) {
    if (A->load_nt && A->store_nt) {
      gen_body<OP, MODE, OUTER, SROW, ZSET, GROUP, true>(A, lds, warm);
      return;
    }
  }
  gen_body<OP, MODE, OUTER, SROW, ZSET, GROUP, false>(A, lds, warm);
}

}  // namespace dev
}  // namespace acp
