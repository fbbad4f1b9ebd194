// C ABI of acp: argument validation, planning and kernel launch.
//
// Every entry point returns an acp_status and records a reason string for
// acp_last_error() (the pages' dispatch predicates return an (ok, reason)
// pair: "copy_async -> tma", "What it accepts"; "elementwise -> smem",
// "What it accepts").  Planning is pure host code; compute calls enqueue one
// kernel on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <string>

#include "acp.h"
#include "acp_engine.hpp"
#include "acp_plan.hpp"

namespace {

thread_local std::string g_last_error;
thread_local std::string g_last_kernel;

acp_status ret(acp_status s, const std::string& why = std::string()) {
  g_last_error = (s == ACP_OK) ? std::string() : why;
  return s;
}

acp_status from_plan(acp::PlanStatus s, const std::string& why) {
  if (s == acp::PlanStatus::Invalid) return ret(ACP_ERR_INVALID, why);
  if (s == acp::PlanStatus::Declined) return ret(ACP_ERR_DECLINED, why);
  if (s == acp::PlanStatus::Unsupported) return ret(ACP_ERR_UNSUPPORTED, why);
  return ACP_OK;
}

bool load_desc(const acp_tile_desc* d, acp::DescData* out) {
  if (!d) return false;
  std::memcpy(out, d->opaque, sizeof(acp::DescData));
  return out->magic == acp::kDescMagic;
}

bool same_geometry(const acp::DescData& a, const acp::DescData& b, bool strides) {
  if (a.rank != b.rank) return false;
  for (int d = 0; d < a.rank; ++d) {
    if (a.shape[d] != b.shape[d] || a.box[d] != b.box[d]) return false;
    if (strides && a.strides[d] != b.strides[d]) return false;
  }
  return true;
}

// bytes from a tensor's base to one past its last element (0 when empty)
uint64_t tensor_span(const acp::DescData& t) {
  uint64_t last = 0;
  for (int d = 0; d < t.rank; ++d) {
    if (t.shape[d] == 0) return 0;
    last += static_cast<uint64_t>(t.shape[d] - 1) * static_cast<uint64_t>(t.strides[d]) * t.esize;
  }
  return last + t.esize;
}

// Whether [a, a + na) and [b, b + nb) share a byte.  The kernels read and
// write different tensors from different workgroups with no ordering
// between them, so a written tensor must not share memory with another
// operand (strided layouts interleaved in one buffer included).
bool overlap(uint64_t a, uint64_t na, uint64_t b, uint64_t nb) { return na && nb && a < b + nb && b < a + na; }

bool overlap(const acp::DescData& a, const acp::DescData& b) {
  return overlap(a.gbase, tensor_span(a), b.gbase, tensor_span(b));
}

// the same elements at the same addresses: an elementwise op may write its
// result over its operand, since each element is loaded before the same
// lane stores it and no other trip touches it
bool same_elements(const acp::DescData& a, const acp::DescData& b) {
  return a.gbase == b.gbase && a.esize == b.esize && same_geometry(a, b, true);
}

int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Device attributes, read from the runtime once per device and kept.
constexpr int kMaxDevices = 64;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

int device_attr(hipDeviceAttribute_t attr, std::atomic<int>* cache, int dflt) {
  const int dev = current_device();
  if (dev < 0) return dflt;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) return dflt;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

std::atomic<int> g_lds_limit[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];

int device_lds_limit() { return device_attr(hipDeviceAttributeMaxSharedMemoryPerBlock, g_lds_limit, 65536); }

// ACP_TILE_STAGES (1..4): ring slots of persistent tile grids; 0 when unset.
int tile_stages_env() {
  static const int v = [] {
    const char* e = std::getenv("ACP_TILE_STAGES");
    return (e && std::atoi(e) > 0 && std::atoi(e) <= 4) ? std::atoi(e) : 0;
  }();
  return v;
}

// Launch knobs read once from the environment (measurement aids; the
// defaults are the measured best on MI355X):
//   ACP_XCD_REMAP=0  keep blockIdx order for persistent grids (default: tiles
//                    of consecutive workgroups stay on one XCD, except for
//                    copies of whole 128-byte lines on a 2-D tile walk); =2
//                    remap those too
//   ACP_STORE_NT=0   cached stores (default: non-temporal)
//   ACP_LOAD_NT=0|1  cached / non-temporal direct-to-LDS loads (default:
//                    non-temporal for contiguous stages on a linear grid and
//                    for copies of whole line-aligned 128-byte rows)
// Non-temporal on both sides measured 6.2 TB/s against 5.8 TB/s cached for
// the 262 MB fp32 stream (the staged data is touched once); cached loads
// measured 3.6 against 3.1 TB/s for 128x32 float16 tiles, whose 64-byte rows
// share each cache line with the neighbouring tile.
//   ACP_FAST_PATH=0  no linear-grid streaming kernel
//   ACP_LIN_TILE=0   no linear-grid kernel for tile ewise
//   ACP_LIN_ROWS=0   no linear-grid kernel for wave-local row sums
//   ACP_GEN_PATH=0   no general lean kernel (the rolled engine runs instead)
//   ACP_SCALAR_ROWS=0  stage per-row scalars in LDS even when rows are uniform per wave block
//   ACP_REDUCE_LOCAL=0, ACP_REDUCE_GROUPED=0  row sums through LDS partials only; reduce-add over
//                    batch dims with one atomic per staged element
//   ACP_BLOCKED_COPY=0  whole-line tile copies on persistent grids walk every
//                    G-th tile instead of a blocked run of consecutive tiles
bool env_flag(const char* name, bool dflt) {
  const char* e = std::getenv(name);
  if (!e || !e[0]) return dflt;
  return e[0] != '0';
}

// 0: never remap, 1: the default rule, 2: remap every eligible grid
int xcd_remap_mode() {
  static const int mode = [] {
    const char* e = std::getenv("ACP_XCD_REMAP");
    if (!e || !e[0]) return 1;
    return e[0] == '0' ? 0 : (e[0] == '2' ? 2 : 1);
  }();
  return mode;
}

// Everything one launch of the engine needs.
struct Launch {
  acp::EngineArgs args;
  acp::KernelKey key;
  unsigned grid = 0, block = 0, lds = 0;
  int64_t n_tiles = 0;
  const void* kernel = nullptr;  // resolved from `key` when the launch is cached
  std::string desc;              // acp_last_kernel text of this launch
};

struct EngineRequest {
  int op;                      // acp_op
  int mode;                    // 0 copy, 1 tile ewise, 2 stream, 3 store with reduce-add, 4 row reduction
  const acp::DescData* x;      // layout of every staged operand
  const acp::DescData* out;
  const void* in_ptrs[3];
  int n_in;
  const int32_t* stage_box;    // per dim of x
  int stages, threads, workgroups;
  const float* row_a;
  const float* row_b;
  bool row_ops;
  bool copy_only;
  int tiles_per_trip = 1;      // tile ops on a persistent grid: 1, 2 or 4
  int binary = 0;              // stream of two tensors: 1 both on the ring, 2 the second one "Set"
  int64_t red_group = 0;       // reduce-add over batch dims: contributions per destination tile
  int64_t red_per_wg = 0;      // ... and tiles per workgroup (a multiple of red_group)
};

acp_status prepare(const EngineRequest& q, Launch* L) {
  const acp::DescData& x = *q.x;
  const acp::DescData& o = *q.out;
  const int r = x.rank;
  std::string why;
  acp::Plan p;
  acp::PlanStatus ps = acp::plan_box_with(x, q.stage_box, q.copy_only, &p, &why);
  if (ps != acp::PlanStatus::Ok) return from_plan(ps, why);

  uint64_t align = 0;
  for (int k = 0; k < q.n_in; ++k) align |= reinterpret_cast<uint64_t>(q.in_ptrs[k]);
  if (q.mode == 1 && q.n_in == 0) align |= x.gbase;
  ps = acp::plan_partition(&p, q.threads, align, &why);
  if (ps != acp::PlanStatus::Ok) return from_plan(ps, why);

  const int ei = x.esize, eo = o.esize;
  // The output side stores vec * eo bytes per round: its base and strides
  // must honour that width (capped at 16), else fall back to 4-byte rounds.
  auto out_ok = [&](int vb) {
    const int64_t ob = static_cast<int64_t>(vb) / ei * eo;
    const int64_t need = ob >= 16 ? 16 : ob;
    if (o.gbase % static_cast<uint64_t>(need)) return false;
    for (int d = 0; d + 1 < r; ++d)
      if ((o.strides[d] * eo) % need) return false;
    if ((o.shape[r - 1] * eo) % need) return false;
    return true;
  };
  if (!out_ok(p.vec_bytes)) {
    if (p.vec_bytes == 16 && (p.tile_bytes() % (static_cast<int64_t>(q.threads) * 4)) == 0 && out_ok(4)) {
      p.vec_bytes = 4;
      p.vec = 4 / ei;
      p.outer = static_cast<int>(p.tile_bytes() / (static_cast<int64_t>(q.threads) * 4));
    } else {
      return ret(ACP_ERR_DECLINED, "output base or strides are not aligned to the chosen vector width");
    }
  }
  if (q.mode != 0 && p.vec_bytes < ei) return ret(ACP_ERR_DECLINED, "vector narrower than one element");
  if (q.mode != 0 && (p.vec_bytes / ei) * eo < 2) return ret(ACP_ERR_UNSUPPORTED, "output chunk below 2 bytes");
  if (p.outer > acp::kMaxOuter)
    return ret(ACP_ERR_UNSUPPORTED, "staged tile needs more than 8 rounds per thread; use more threads or a smaller box");
  if (p.tile_bytes() >= (int64_t(1) << 31)) return ret(ACP_ERR_UNSUPPORTED, "staged tile too large");

  acp::EngineArgs& A = L->args;
  std::memset(&A, 0, sizeof(A));
  for (int k = 0; k < q.n_in; ++k) A.in[k] = static_cast<const char*>(q.in_ptrs[k]);
  A.out = reinterpret_cast<char*>(o.gbase);
  A.row_a = q.row_a ? q.row_a : q.row_b;
  A.row_b = q.row_b ? q.row_b : q.row_a;
  A.rank = r;

  // packed strides of the row array (shape[:-1]) and of a stage's rows
  int64_t rowstride[acp::kDims] = {};
  int64_t srow[acp::kDims] = {};
  int64_t rs = 1, n_rows = 1;
  for (int d = r - 2; d >= 0; --d) {
    rowstride[d] = rs;
    rs *= x.shape[d];
    srow[d] = n_rows;
    n_rows *= q.stage_box[d];
  }

  int64_t n_tiles = 1, subs = 1, max_x = 0, max_o = 0;
  int64_t xstride[acp::kDims] = {}, ostride[acp::kDims] = {};
  int n_partial = 0;
  for (int d = 0; d < acp::kDims; ++d) A.pslot_of_dim[d] = -1;
  for (int s = 0; s < acp::kPartial; ++s) A.prem[s] = 0xFFFFFFFFu;
  for (int d = 0; d < r; ++d) {
    const int64_t sb = q.stage_box[d];
    if (x.box[d] % sb != 0) return ret(ACP_ERR_INVALID, "stage box must divide the descriptor box in every dim");
    const int64_t nst = (x.shape[d] + sb - 1) / sb;
    const int64_t sub = x.box[d] / sb;
    const int64_t tg = (nst + sub - 1) / sub;
    xstride[d] = x.strides[d] * ei;
    // a reduce-add destination of extent 1 along a dim the source spans:
    // every source stage along it adds into the same destination elements
    ostride[d] = (q.mode == 3 && o.shape[d] == 1 && x.shape[d] > 1) ? 0 : o.strides[d] * eo;
    if (q.mode == 4) ostride[d] = 0;  // row sums are addressed by row index, not by the stage grid
    A.sbox[d] = static_cast<uint32_t>(sb);
    A.nst[d] = static_cast<uint32_t>(nst);
    const int64_t rem = nst ? x.shape[d] - (nst - 1) * sb : sb;
    if (rem < sb) {
      if (n_partial == acp::kPartial)
        return ret(ACP_ERR_UNSUPPORTED, "more than 4 dims end in a partial stage");
      A.pslot_of_dim[d] = n_partial;
      A.prem[n_partial] = static_cast<uint32_t>(rem);
      ++n_partial;
    }
    A.sub[d] = static_cast<uint32_t>(sub);
    acp::magic_for(A.sub[d], &A.sub_mag[d], &A.sub_sh[d]);
    A.tgrid[d] = static_cast<uint32_t>(tg ? tg : 1);
    acp::magic_for(A.tgrid[d], &A.tg_mag[d], &A.tg_sh[d]);
    A.xstep[d] = sb * xstride[d];
    A.ostep[d] = sb * ostride[d];
    A.rstep[d] = d < r - 1 ? sb * rowstride[d] : 0;
    max_x += (sb - 1) * xstride[d];
    max_o += (sb - 1) * ostride[d];
    n_tiles *= tg;
    subs *= sub;
  }
  A.in_span = tensor_span(x);
  A.out_span = tensor_span(o);
  A.total_rows = static_cast<uint64_t>(rs);
  if (max_x + 16 >= (int64_t(1) << 31) || max_o + 32 >= (int64_t(1) << 31))
    return ret(ACP_ERR_UNSUPPORTED, "a stage spans more than 2 GiB");

  // Linear stage grid: with one stage per tile and no partial stage, stage t
  // of a row-major contiguous grid (over the dims with more than one stage)
  // starts at t times the innermost such dim's step.
  {
    int prev = -1;
    bool lin = (subs == 1 && n_partial == 0);
    int64_t lx = 0, lo = 0, lr = 0;
    int prev_r = -1;
    for (int d = 0; d < r && lin; ++d) {
      if (A.nst[d] <= 1) continue;
      if (prev >= 0 && (A.xstep[prev] != A.nst[d] * A.xstep[d] || A.ostep[prev] != A.nst[d] * A.ostep[d]))
        lin = false;
      prev = d;
      lx = A.xstep[d];
      lo = A.ostep[d];
      if (q.row_ops || q.mode == 4) {
        if (d == r - 1) {
          lin = false;  // stages split rows: the row index is not linear in t
        } else {
          if (prev_r >= 0 && A.rstep[prev_r] != A.nst[d] * A.rstep[d]) lin = false;
          prev_r = d;
          lr = A.rstep[d];
        }
      }
    }
    A.lin = lin ? 1 : 0;
    A.lin_x = lin ? lx : 0;
    A.lin_o = lin ? lo : 0;
    A.lin_r = lin ? lr : 0;
  }
  // Loads go out non-temporal only where no two stages share a cache line:
  // a linear grid of contiguous stages (each input byte is read once), and
  // copies whose staged rows are whole 128-byte lines at line-aligned
  // addresses (paired 128x32 float16 tiles over [128,500,1024]: 1.5 % faster
  // than cached).  Elsewhere (2-D tiles whose rows are shorter than a line,
  // padded rows) the neighbouring stage reads the rest of the line from L2.
  static const bool store_nt = env_flag("ACP_STORE_NT", true);
  static const int load_nt_env = [] {
    const char* e = std::getenv("ACP_LOAD_NT");
    return (!e || !e[0]) ? -1 : (e[0] != '0' ? 1 : 0);
  }();
  const bool contiguous_stages = A.lin && A.lin_x == p.tile_bytes() && A.lin_x % 128 == 0;
  bool line_rows = q.mode == 0 && (static_cast<int64_t>(q.stage_box[r - 1]) * ei) % 128 == 0 && x.gbase % 128 == 0;
  for (int d = 0; d + 1 < r; ++d) line_rows = line_rows && (x.strides[d] * ei) % 128 == 0;
  A.store_nt = store_nt ? 1 : 0;
  A.load_nt = load_nt_env >= 0 ? load_nt_env : ((contiguous_stages || line_rows) ? 1 : 0);
  if (n_tiles * subs >= (int64_t(1) << 31)) return ret(ACP_ERR_UNSUPPORTED, "more than 2^31 stages");
  A.n_tiles = static_cast<uint32_t>(n_tiles);
  A.subs = static_cast<uint32_t>(subs);
  acp::magic_for(A.subs, &A.subs_mag, &A.subs_sh);
  L->n_tiles = n_tiles;

  const std::vector<acp::Axis> axes = p.image_axes();
  A.n_axes = static_cast<int>(axes.size());
  for (size_t k = 0; k < axes.size(); ++k) {
    const int d = axes[k].dim;
    A.ax_count[k] = static_cast<uint32_t>(axes[k].count);
    acp::magic_for(A.ax_count[k], &A.ax_mag[k], &A.ax_sh[k]);
    A.ax_step[k] = static_cast<uint32_t>(axes[k].step);
    A.ax_xs[k] = static_cast<uint32_t>(axes[k].step * xstride[d]);
    A.ax_os[k] = static_cast<uint32_t>(axes[k].step * ostride[d]);
    A.ax_rs[k] = d < r - 1 ? static_cast<uint32_t>(axes[k].step * srow[d]) : 0u;
    A.ax_pslot[k] = A.pslot_of_dim[d];
    if (d == r - 1) A.ax_inner_mask |= 1u << k;
  }
  A.esize_log2 = log2i(ei);
  A.outer = p.outer;
  A.waves = q.threads / 64;
  A.swizzle = (1 << x.swizzle) - 1;  // the mask of row bits XORed into the chunk index
  A.n_in = q.n_in;

  // every 1 KiB wave block inside one row: the innermost image run holds a
  // whole number of such blocks and nothing permutes it
  // The scalar-cache path indexes the row arrays with the stage's first row
  // plus the row's packed position inside the stage, so it also needs the
  // stage's rows to be consecutive in the packed row array: along every row
  // dim the stage spans, the stage covers all of each inner row dim.
  bool rows_consecutive = true;
  for (int d = 0; d + 1 < r; ++d)
    if (q.stage_box[d] > 1 && srow[d] != rowstride[d]) rows_consecutive = false;
  A.row_uniform = (q.row_ops && rows_consecutive && A.swizzle == 0 &&
                   (axes.back().count * ei) % (64 * p.vec_bytes) == 0) ? 1 : 0;
  if (q.mode == 4) {
    const int64_t row_bytes = x.shape[r - 1] * ei;
    // Wave-local reduction when every 1 KiB wave block lies in one row and
    // every row's blocks belong to one wave (block b goes to wave b % waves).
    auto row_of = [&](int64_t e) {  // stage-packed row of image element e
      int64_t row = 0;
      for (size_t k = axes.size(); k-- > 0;) {
        const int64_t idx = e % axes[k].count;
        e /= axes[k].count;
        if (axes[k].dim < r - 1) row += idx * axes[k].step * srow[axes[k].dim];
      }
      return row;
    };
    bool local = row_bytes % 1024 == 0;
    std::vector<int> wave_of_row(static_cast<size_t>(n_rows), -1);
    const int64_t blocks = p.tile_bytes() / 1024;
    for (int64_t b = 0; local && b < blocks; ++b) {
      const int64_t r0 = row_of(b * 1024 / ei);
      for (int c = 1; c < 64 && local; ++c) local = row_of((b * 1024 + c * 16) / ei) == r0;
      const int w = static_cast<int>(b % A.waves);
      if (!local || r0 >= n_rows) break;
      if (wave_of_row[r0] < 0) wave_of_row[r0] = w;
      else if (wave_of_row[r0] != w) local = false;
    }
    static const bool local_ok = env_flag("ACP_REDUCE_LOCAL", true);
    A.red_local = (local && local_ok) ? 1 : 0;
  }
  L->key = acp::KernelKey{q.op, q.mode == 0 ? ACP_U32 : static_cast<int>(x.dtype),
                          q.mode == 0 ? ACP_U32 : (q.mode == 4 ? ACP_F32 : static_cast<int>(o.dtype)), p.vec_bytes,
                          q.mode, 0, 0};
  // streaming on a linear grid with 16-byte rounds: the lean kernel; a
  // tile copy whose tiles form a linear grid (a single tile among them) is
  // the same stream with the copy op, and its smaller argument block and
  // set-up shorten a latency-bound launch
  static const bool fast_ok = env_flag("ACP_FAST_PATH", true);
  bool fast = false;
  // (two tensors: with both on the direct-to-LDS ring)
  if (fast_ok && (q.mode == 2 || q.mode == 0) && A.lin && p.vec_bytes == 16 && (q.n_in == 1 || q.binary == 1) &&
      (p.outer == 1 || p.outer == 2 || p.outer == 4 || p.outer == 8)) {
    acp::KernelKey fk = L->key;
    fk.mode = 3;
    fk.outer = p.outer;
    fk.variant = q.binary;
    static const bool srow_ok = env_flag("ACP_SCALAR_ROWS", true);
    fk.srow = (q.mode == 2 && A.row_uniform && srow_ok) ? 1 : 0;
    if (acp::engine_kernel(fk)) {
      L->key = fk;
      fast = true;
    }
  }
  // tile ewise on a linear tile grid with 16-byte rounds: the linear kernel
  // with the output staged in LDS, the tiles of one ring trip (1, 2 or 4,
  // dividing the tile count) forming one stage
  static const bool lin_tile_ok = env_flag("ACP_LIN_TILE", true);
  int lin_tiles = 0;
  if (lin_tile_ok && !fast && q.mode == 1 && A.lin && p.vec_bytes == 16 && q.n_in >= 1) {
    int t = 1;
    if (q.workgroups > 0)
      while (2 * t <= q.tiles_per_trip && 2 * t <= 4 && n_tiles % (2 * t) == 0 && 2 * t * p.outer <= acp::kMaxOuter)
        t *= 2;
    const int rounds = t * p.outer;
    const bool fits = (t - 1) * A.lin_x + max_x + 16 < (int64_t(1) << 31) &&
                      (t - 1) * A.lin_o + max_o + 32 < (int64_t(1) << 31);
    if (fits && (rounds == 1 || rounds == 2 || rounds == 4 || rounds == 8)) {
      acp::KernelKey tk = L->key;
      tk.mode = 9;
      tk.outer = rounds;
      if (acp::engine_kernel(tk)) {
        L->key = tk;
        fast = true;
        lin_tiles = t;
        A.outer = rounds;
        A.tile_rounds_log2 = static_cast<uint32_t>(log2i(p.outer));
        A.tile_x = A.lin_x;
        A.tile_o = A.lin_o;
        A.lin_x *= t;
        A.lin_o *= t;
        A.n_tiles = static_cast<uint32_t>(n_tiles / t);
      }
    }
  }
  // wave-local row reduction on a linear stage grid with 16-byte rounds
  static const bool lin_rows_ok = env_flag("ACP_LIN_ROWS", true);
  if (lin_rows_ok && !fast && q.mode == 4 && A.lin && A.red_local && p.vec_bytes == 16 &&
      (p.outer == 1 || p.outer == 2 || p.outer == 4 || p.outer == 8)) {
    acp::KernelKey rk = L->key;
    rk.mode = 10;
    rk.outer = p.outer;
    if (acp::engine_kernel(rk)) {
      L->key = rk;
      fast = true;
    }
  }
  // any other grid with 16-byte rounds: the general lean kernel
  static const bool gen_ok = env_flag("ACP_GEN_PATH", true);
  if (gen_ok && !fast && p.vec_bytes == 16 &&
      (p.outer == 1 || p.outer == 2 || p.outer == 4 || p.outer == 8)) {
    acp::KernelKey gk = L->key;
    gk.mode = q.mode + 4;
    gk.outer = p.outer;
    static const bool srow_ok = env_flag("ACP_SCALAR_ROWS", true);
    gk.srow = (q.mode == 2 && A.row_uniform && srow_ok) ? 1 : 0;
    gk.variant = q.mode == 3 ? (q.red_group > 0 ? 1 : 0) : q.binary;
    if (acp::engine_kernel(gk)) L->key = gk;
  }
  if (q.binary && L->key.variant != q.binary) {
    return ret(ACP_ERR_UNSUPPORTED,
               "two-tensor streams need 16-byte rounds and 1, 2, 4 or 8 rounds per thread");
  }
  // tile ops in the general kernel on a persistent grid: tiles per ring trip
  int tpt_log2 = 0;
  if ((L->key.mode == 4 || L->key.mode == 5 || L->key.mode == 7) && q.workgroups > 0 && subs == 1)
    while ((2 << tpt_log2) <= q.tiles_per_trip && tpt_log2 < 2) ++tpt_log2;
  if (lin_tiles) tpt_log2 = log2i(lin_tiles);
  // the linear kernel's stage already spans the trip's tiles
  A.tpt_log2 = static_cast<uint32_t>(lin_tiles ? 0 : tpt_log2);

  const int64_t in_img = align_up(p.tile_bytes(), 1024);
  // linear kernel: each operand's image holds the trip's tiles back to
  // back, and so does the output image
  const int64_t out_img =
      q.mode == 1 ? align_up(p.tile_elems() * eo * (lin_tiles ? lin_tiles : 1), 1024) : 0;
  A.in_image_bytes = static_cast<uint32_t>(lin_tiles ? in_img * lin_tiles : in_img);
  A.ab_off = static_cast<uint32_t>(q.n_in * in_img);
  A.row_ops = q.row_ops ? 1 : 0;
  if (q.row_ops) {
    if (n_rows > 64) return ret(ACP_ERR_UNSUPPORTED, "per-row scalars need at most 64 rows per stage");
    A.n_rows = static_cast<int32_t>(n_rows);
    A.ab_instr = static_cast<int32_t>((n_rows + 31) / 32);
    A.ab_wave_bytes = static_cast<uint32_t>(A.ab_instr * 256);
  }
  const int64_t slot = align_up(A.ab_off + (q.row_ops ? A.waves * A.ab_wave_bytes : 0), 1024) << tpt_log2;
  A.slot_bytes = static_cast<uint32_t>(slot);

  const int64_t groups = (n_tiles + (int64_t(1) << tpt_log2) - 1) >> tpt_log2;
  const int64_t trips_max = subs * ((q.workgroups > 0 && q.workgroups < groups)
                                        ? (groups + q.workgroups - 1) / q.workgroups : 1);
  // Copies whose staged rows are whole 128-byte lines, on a persistent grid
  // of the general kernel, walk blocked runs of consecutive tiles (workgroup
  // w: tiles w * per, ..., (w + 1) * per - 1) instead of every G-th tile, so
  // the trips a workgroup has in flight cover neighbouring pieces of the
  // same rows (128x32 float16 tiles in pairs over [128,500,1024]: 4.88-4.90
  // TB/s against 4.70-4.80 on the cyclic walk, with cached loads).  Tiles of
  // half lines keep the cyclic walk with the XCD remap (3.83 against 3.77
  // TB/s).  ACP_BLOCKED_COPY=0 keeps the cyclic walk everywhere.
  static const bool blocked_ok = env_flag("ACP_BLOCKED_COPY", true);
  const bool whole_lines =
      q.mode == 0 && !A.lin && (static_cast<int64_t>(q.stage_box[r - 1]) * ei) % 128 == 0;
  const bool blocked = blocked_ok && whole_lines && L->key.mode == 4 && q.workgroups > 0 && tpt_log2 == 0 &&
                       n_tiles > q.workgroups;
  const int slots = static_cast<int>(q.stages < trips_max ? q.stages : trips_max);
  A.stages = slots < 1 ? 1 : slots;
  // The staged output image lies after the ring, one per workgroup: each
  // lane writes its chunks there and reads the same bytes back before its
  // store, so trips can share it and it costs no ring slot.
  A.out_image_off = static_cast<uint32_t>(slot * A.stages);
  int64_t lds = slot * A.stages + out_img;
  if (q.mode == 4) {
    // row reduction: whole rows per stage, partial sums double-buffered after the ring
    const int64_t row_bytes = x.shape[r - 1] * ei;
    A.row_chunks = static_cast<uint32_t>(row_bytes / 16);
    A.red_rows = static_cast<uint32_t>(n_rows);
    A.part_bytes = static_cast<uint32_t>(n_rows * (row_bytes / 16) * 4);
    A.part_off = static_cast<uint32_t>(lds);
    if (!A.red_local) lds += 2 * static_cast<int64_t>(A.part_bytes);  // the wave-local path needs none
    for (int d = 0; d + 1 < r; ++d) A.rowstr[d] = static_cast<uint32_t>(rowstride[d]);
  }
  const int limit = device_lds_limit();
  if (lds > limit)
    return ret(ACP_ERR_LDS, "ring needs " + std::to_string(lds) + " bytes of LDS, device allows " +
                                std::to_string(limit));

  if (q.mode == 3 && q.red_group > 0) {
    // List the summed dims last (fastest) in the per-dim tile arrays, so
    // that consecutive tiles are the contributions to one destination tile;
    // workgroups take contiguous runs of whole groups.
    int order[acp::kDims], n = 0;
    for (int d = 0; d < r; ++d)
      if (!(o.shape[d] == 1 && x.shape[d] > 1)) order[n++] = d;
    for (int d = 0; d < r; ++d)
      if (o.shape[d] == 1 && x.shape[d] > 1) order[n++] = d;
    const acp::EngineArgs B = A;
    for (int k = 0; k < r; ++k) {
      const int d = order[k];
      A.tgrid[k] = B.tgrid[d];
      A.tg_mag[k] = B.tg_mag[d];
      A.tg_sh[k] = B.tg_sh[d];
      A.sub[k] = B.sub[d];
      A.sub_mag[k] = B.sub_mag[d];
      A.sub_sh[k] = B.sub_sh[d];
      A.nst[k] = B.nst[d];
      A.pslot_of_dim[k] = B.pslot_of_dim[d];
      A.xstep[k] = B.xstep[d];
      A.ostep[k] = B.ostep[d];
      A.rstep[k] = B.rstep[d];
    }
    A.red_group = static_cast<uint32_t>(q.red_group);
    A.per_wg = static_cast<uint32_t>(q.red_per_wg);
  }
  unsigned grid = static_cast<unsigned>(n_tiles);
  if (q.workgroups > 0) grid = static_cast<unsigned>(q.workgroups);
  if (blocked) A.per_wg = static_cast<uint32_t>((n_tiles + grid - 1) / grid);
  // consecutive tiles (which often share cache lines at their edges) run on
  // one XCD and hence one L2: blockIdx b -> (b % 8) * (G / 8) + b / 8.
  // Copies walking a 2-D tile grid whose staged rows are whole 128-byte
  // lines share no line with their neighbours and go without it (128x32
  // float16 tiles in pairs over [128,500,1024]: 4.79 TB/s against 4.60 on
  // the cyclic walk, equal on the blocked one); copies of contiguous tiles
  // on a linear grid keep it (8 KiB tiles: 6.25-6.27 TB/s against 6.19).
  const int remap = xcd_remap_mode();
  A.xcd_remap = (grid % 8 == 0 && grid >= 16 && remap != 0 && (!whole_lines || remap == 2)) ? 1 : 0;
  L->grid = grid;
  L->block = static_cast<unsigned>(q.threads);
  L->lds = static_cast<unsigned>(lds);
  return ACP_OK;
}

std::string describe(const Launch& L) {
  static const char* const kinds[] = {"engine copy",        "engine tile ewise",  "engine stream",
                                      "stream linear grid", "general copy",       "general tile ewise",
                                      "general stream",     "general reduce-add", "general row reduction",
                                      "tile linear grid",   "row reduction linear grid"};
  const int m = L.key.mode;
  const bool lin_copy = m == 3 && L.key.op == ACP_OP_COPY;
  return std::string(lin_copy ? "copy linear grid" : (m >= 0 && m <= 10 ? kinds[m] : "?")) + " vec " +
         std::to_string(L.key.vec_bytes) +
         " rounds " + std::to_string(L.args.outer) + " srow " + std::to_string(L.key.srow) + " variant " +
         std::to_string(L.key.variant) + " grid " + std::to_string(L.grid) + " threads " +
         std::to_string(L.block) + " slots " + std::to_string(L.args.stages) + " lds " + std::to_string(L.lds) +
         (L.key.mode == 4 && L.args.per_wg ? " blocked-walk" : "") + (L.args.xcd_remap ? " xcd-remap" : "") +
         (m == 8 || m == 10 ? std::string(L.args.red_local ? " wave-local" : " lds partials") : std::string());
}

// Resolve the kernel and the description of a prepared launch (done once,
// when the launch enters the cache).
acp_status finalize(Launch* L) {
  if (L->n_tiles == 0) return ACP_OK;
  L->kernel = acp::engine_kernel(L->key);
  if (!L->kernel) return ret(ACP_ERR_UNSUPPORTED, "op / dtype combination is not in the registry");
  L->desc = describe(*L);
  return ACP_OK;
}

acp_status launch(const Launch& L, void* stream) {
  g_last_kernel = "none";
  if (L.n_tiles == 0) return ret(ACP_OK);
  const hipError_t e = acp::engine_launch(L.kernel, L.args, L.grid, L.block, L.lds, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  g_last_kernel = L.desc;
  return ret(ACP_OK);
}

// Prepared launches, per thread: the host plan and the kernel arguments of a
// call depend only on its arguments (descriptors by value, scalars, device
// addresses) and on the device, so a repeated call reuses them ("copy_async
// -> tma", "Algorithm" step 3: the host descriptor is emitted once, keyed by
// a cache).  A key is those bytes; a small round-robin table of recent keys
// per thread.
struct CallKey {
  unsigned char b[4 * sizeof(acp::DescData) + 256];
  size_t n = 0;
  bool ok = true;
  explicit CallKey(int entry) {
    add(&entry, sizeof(entry));
    const int dev = current_device();
    add(&dev, sizeof(dev));
  }
  void add(const void* p, size_t k) {
    if (n + k > sizeof(b)) { ok = false; return; }
    std::memcpy(b + n, p, k);
    n += k;
  }
  template <class T>
  void val(const T& v) { add(&v, sizeof(v)); }
  void desc(const acp_tile_desc* d) {
    if (!d) { val(-1); return; }
    add(d->opaque, sizeof(acp::DescData));
  }
  void ints(const int32_t* v, int k) {
    if (!v) { val(-1); return; }
    add(v, sizeof(int32_t) * static_cast<size_t>(k));
  }
};

// rank of an encoded descriptor (0 if it is not one): the length of the
// stage box a call passes
int desc_rank(const acp_tile_desc* d) {
  acp::DescData dd;
  return load_desc(d, &dd) ? dd.rank : 0;
}

constexpr int kCacheEntries = 16;
struct CacheEntry {
  std::string key;
  Launch L;
};
thread_local CacheEntry g_cache[kCacheEntries];
thread_local int g_cache_next = 0;

const Launch* cache_find(const CallKey& k) {
  if (!k.ok) return nullptr;
  for (const CacheEntry& e : g_cache)
    if (e.key.size() == k.n && std::memcmp(e.key.data(), k.b, k.n) == 0) return &e.L;
  return nullptr;
}

const Launch* cache_put(const CallKey& k, const Launch& L) {
  if (!k.ok) return nullptr;
  CacheEntry& e = g_cache[g_cache_next];
  g_cache_next = (g_cache_next + 1) % kCacheEntries;
  e.key.assign(reinterpret_cast<const char*>(k.b), k.n);
  e.L = L;
  return &e.L;
}

// Launch the cached launch for `k`, or build, finalize, cache and launch it.
template <class Build>
acp_status run_cached(const CallKey& k, Build&& build, void* stream) {
  if (const Launch* c = cache_find(k)) return launch(*c, stream);
  Launch L;
  acp_status st = build(&L);
  if (st != ACP_OK) return st;
  st = finalize(&L);
  if (st != ACP_OK) return st;
  const Launch* c = cache_put(k, L);
  return launch(c ? *c : L, stream);
}

bool is_float(int dt) { return dt == ACP_F16 || dt == ACP_F32; }

int device_cu_count() { return device_attr(hipDeviceAttributeMultiprocessorCount, g_cu_count, 256); }

// Tile copy and tile elementwise: the result of a tile does not depend on
// which workgroup moves it, so large tile counts run on a persistent grid
// that walks tile groups w, w+G, ... (whole-line copies: a blocked run of
// consecutive groups, see prepare) through a ring of ACP_TILE_STAGES slots
// (default 2); a group (one ring trip) is 1, 2 or 4 consecutive tiles.
// Defaults, the best measured on MI355X (the environment overrides them):
// * copy: one tile per trip and one workgroup per CU (fewer concurrent
//   streams keep DRAM pages open; 128x32 float16 tiles, one per trip, ran
//   3.9 TB/s at one workgroup per CU against 3.4 TB/s at 2 or 4);
// * elementwise: trips of about 16 KiB (ACP_TILES_PER_TRIP: 1, 2, 4) and
//   about 32 KiB of loads in flight per CU (ACP_TILE_WG_PER_CU), within 32
//   waves per CU and the LDS (32x32 float32 sqrt: 6.1 TB/s with 4 tiles per
//   trip against 5.7 with two and 4.2 with one).
int tile_wg_per_cu_env() {
  static const int v = [] {
    const char* e = std::getenv("ACP_TILE_WG_PER_CU");
    return (e && std::atoi(e) > 0) ? std::atoi(e) : 0;
  }();
  return v;
}

void tile_schedule(const acp::Plan& p, int n_in, int threads, int64_t out_image, int* workgroups, int* stages,
                   int* tiles_per_trip) {
  const int env_per_cu = tile_wg_per_cu_env();
  const int slots = tile_stages_env() ? tile_stages_env() : 2;
  static const int env_tpt = [] {
    const char* e = std::getenv("ACP_TILES_PER_TRIP");
    const int v = e ? std::atoi(e) : 0;
    return (v == 1 || v == 2 || v == 4) ? v : 0;
  }();
  const int64_t n_tiles = p.n_tiles();
  const int64_t img = align_up(p.tile_bytes(), 1024);
  const int64_t ops = std::max(1, n_in);
  const bool copy = out_image == 0;
  int tpt = env_tpt;
  if (tpt == 0) {
    tpt = 1;
    while (!copy && tpt < 4 && 2 * tpt * ops * p.tile_bytes() <= 16384) tpt *= 2;
  }
  int64_t per_cu = env_per_cu;
  if (per_cu == 0) {
    const int64_t lds_wg = slots * tpt * ops * img + align_up(out_image, 1024);
    per_cu = copy ? 1 : std::max<int64_t>(1, 32768 / (tpt * ops * p.tile_bytes()));
    per_cu = std::min<int64_t>(per_cu, std::max(1, 32 / std::max(1, threads / 64)));
    per_cu = std::min<int64_t>(per_cu, std::max<int64_t>(1, device_lds_limit() / lds_wg));
  }
  const int64_t g = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (n_tiles > g) {
    *workgroups = static_cast<int>(g);
    *stages = slots;
    *tiles_per_trip = tpt;
  } else {
    *workgroups = 0;  // one workgroup per tile, one trip each
    *stages = 1;
    *tiles_per_trip = 1;
  }
}

// The compute entry points, without the launch: validate and prepare (no
// HIP calls besides device attributes).  The exported functions cache the
// result and launch it.
acp_status keep(Launch* res, Launch& L) {
  *res = std::move(L);
  return ACP_OK;
}

acp_status build_tile_copy(const acp_tile_desc* src, const acp_tile_desc* dst, int threads, Launch* res) {
  acp::DescData s, d;
  if (!load_desc(src, &s) || !load_desc(dst, &d)) return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  // validate_copy_op: both sides laid out, equal dtype, equal extents
  if (s.dtype != d.dtype) return ret(ACP_ERR_INVALID, "not a valid copy op: dtypes differ");
  if (!same_geometry(s, d, false)) return ret(ACP_ERR_INVALID, "not a valid copy op: shapes or boxes differ");
  if (overlap(s, d)) return ret(ACP_ERR_INVALID, "source and destination share memory");
  EngineRequest q{};
  q.op = ACP_OP_COPY;
  q.mode = 0;
  q.x = &s;
  q.out = &d;
  q.in_ptrs[0] = reinterpret_cast<const void*>(s.gbase);
  q.n_in = 1;
  q.stage_box = s.box;
  q.threads = threads;
  q.copy_only = true;
  acp::Plan p;
  std::string why;
  const bool planned = acp::plan_box(s, true, &p, &why) == acp::PlanStatus::Ok;
  if (planned) tile_schedule(p, 1, threads, 0, &q.workgroups, &q.stages, &q.tiles_per_trip);
  else q.stages = 1;
  // Tiles whose rows are narrower than a 128-byte cache line: on a
  // persistent grid each trip stages k neighbouring tiles along the
  // innermost dim side by side (their union, k * box wide), so every wave
  // instruction reads and writes whole lines instead of line pieces; each
  // tile still moves in its own rounds of the partition.  A copy's result
  // does not depend on how tiles are grouped into trips.  128x32 float16
  // tiles over [128,500,1024]: 4.6-4.8 TB/s paired against 3.9 alone.
  // ACP_TILE_MERGE=0 keeps one tile per trip.
  static const bool merge_ok = env_flag("ACP_TILE_MERGE", true);
  const int r = s.rank;
  const int64_t row_bytes = static_cast<int64_t>(s.box[r - 1]) * s.esize;
  const int64_t inner_tiles = s.shape[r - 1] > 0 ? (s.shape[r - 1] + s.box[r - 1] - 1) / s.box[r - 1] : 0;
  int k = 1;
  if (merge_ok && planned && q.workgroups > 0)
    while (2 * k * row_bytes <= 128 && 2 * k <= inner_tiles) k *= 2;
  for (; k > 1; k /= 2) {
    acp::DescData s2 = s, d2 = d;
    s2.box[r - 1] *= k;
    d2.box[r - 1] *= k;
    acp::Plan p2;
    if (acp::plan_box(s2, true, &p2, &why) != acp::PlanStatus::Ok) continue;
    EngineRequest q2 = q;
    q2.x = &s2;
    q2.out = &d2;
    q2.stage_box = s2.box;
    int unused_w = 0, unused_tpt = 0;
    tile_schedule(p2, 1, threads, 0, &unused_w, &q2.stages, &unused_tpt);
    q2.tiles_per_trip = 1;
    Launch L2;
    if (prepare(q2, &L2) == ACP_OK && (L2.key.mode == 4 || L2.key.mode == 3)) return keep(res, L2);
  }
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  return keep(res, L);
}

acp_status build_tile_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* const* in, int n_in,
                          int threads, Launch* res) {
  acp::DescData o;
  if (!load_desc(out, &o)) return ret(ACP_ERR_INVALID, "not an encoded output descriptor");
  int need = -1;
  switch (op) {
    case ACP_OP_ZERO: need = n_in <= 1 ? n_in : -1; break;
    case ACP_OP_SQRT: case ACP_OP_EXP: need = 1; break;
    case ACP_OP_ADD: case ACP_OP_MUL: need = 2; break;
    case ACP_OP_FMA: need = 3; break;
    default: return ret(ACP_ERR_INVALID, "unknown op for tile_ewise");
  }
  if (need != n_in) return ret(ACP_ERR_INVALID, "wrong number of operands for the op");
  if (n_in > 0 && !in) return ret(ACP_ERR_INVALID, "null operand list");
  acp::DescData ins[3];
  for (int k = 0; k < n_in; ++k) {
    if (!load_desc(in[k], &ins[k])) return ret(ACP_ERR_INVALID, "not an encoded operand descriptor");
    if (!same_geometry(ins[k], ins[0], true) || ins[k].dtype != ins[0].dtype || ins[k].swizzle != ins[0].swizzle)
      return ret(ACP_ERR_INVALID, "operands must share one layout (dtype, shape, strides, box, swizzle)");
  }
  const acp::DescData& anchor = n_in ? ins[0] : o;
  if (!same_geometry(anchor, o, false)) return ret(ACP_ERR_INVALID, "output shape or box differs from the operands");
  const int ti = anchor.dtype, to = o.dtype;
  if (!is_float(ti) || !is_float(to)) return ret(ACP_ERR_UNSUPPORTED, "elementwise ops take float16 or float32");
  if ((op == ACP_OP_ADD || op == ACP_OP_MUL || op == ACP_OP_FMA || op == ACP_OP_ZERO) && ti != to)
    return ret(ACP_ERR_UNSUPPORTED, "this op keeps the operand type");
  for (int k = 0; k < n_in; ++k)
    if (overlap(ins[k], o) && !same_elements(ins[k], o))
      return ret(ACP_ERR_INVALID, "the output shares memory with an operand other than element for element");
  EngineRequest q{};
  q.op = op;
  q.mode = 1;
  q.x = &anchor;
  q.out = &o;
  for (int k = 0; k < n_in; ++k) q.in_ptrs[k] = reinterpret_cast<const void*>(ins[k].gbase);
  q.n_in = n_in;
  q.stage_box = anchor.box;
  q.threads = threads;
  q.copy_only = false;
  {
    acp::Plan p;
    std::string why;
    if (acp::plan_box(anchor, false, &p, &why) == acp::PlanStatus::Ok)
      tile_schedule(p, n_in, threads, p.tile_elems() * o.esize, &q.workgroups, &q.stages, &q.tiles_per_trip);
    else q.stages = 1;
  }
  Launch L;
  acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  // The linear tile kernel streams best with one workgroup per CU (32x32
  // float32 sqrt: 6.13 against 5.98 TB/s with two); the general
  // kernel keeps the schedule's count, whose extra waves cover the LDS round
  // trip of its output image.
  const int cus = device_cu_count();
  if (L.key.mode == 9 && tile_wg_per_cu_env() == 0 && q.workgroups > cus) {
    q.workgroups = cus;
    st = prepare(q, &L);
    if (st != ACP_OK) return st;
  }
  return keep(res, L);
}

acp_status build_stream_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x, const float* row_a,
                            const float* row_b, const int32_t* stage_box, int stages, int threads, int workgroups,
                            Launch* res) {
  acp::DescData xd, od;
  if (!load_desc(x, &xd) || !load_desc(out, &od)) return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  if (!stage_box) return ret(ACP_ERR_INVALID, "null stage box");
  if (stages < 2 || stages > 4) return ret(ACP_ERR_INVALID, "stages must be 2, 3 or 4");
  if (workgroups < 0) return ret(ACP_ERR_INVALID, "workgroups must be >= 0");
  if (!same_geometry(xd, od, false)) return ret(ACP_ERR_INVALID, "output shape or box differs from x");
  if (overlap(xd, od)) return ret(ACP_ERR_INVALID, "x and the output share memory");
  for (int d = 0; d < xd.rank; ++d)
    if (stage_box[d] < 1) return ret(ACP_ERR_INVALID, "stage box must be >= 1");
  bool row_ops = false;
  switch (op) {
    case ACP_OP_ZERO: case ACP_OP_SQRT: case ACP_OP_EXP:
      if (!is_float(xd.dtype) || !is_float(od.dtype))
        return ret(ACP_ERR_UNSUPPORTED, "elementwise ops take float16 or float32");
      if (op == ACP_OP_ZERO && xd.dtype != od.dtype) return ret(ACP_ERR_UNSUPPORTED, "zero keeps the type");
      break;
    case ACP_OP_ADD: case ACP_OP_MUL: case ACP_OP_FMA:
      if (xd.dtype != ACP_F32 || od.dtype != ACP_F32)
        return ret(ACP_ERR_UNSUPPORTED, "per-row ops take float32 x and output");
      if ((op != ACP_OP_ADD && !row_a) || (op != ACP_OP_MUL && !row_b))
        return ret(ACP_ERR_INVALID, "missing per-row scalar array");
      row_ops = true;
      break;
    default: return ret(ACP_ERR_INVALID, "unknown op for stream_ewise");
  }
  if (xd.rank < 2 && row_ops) return ret(ACP_ERR_INVALID, "per-row scalars need rank >= 2");
  if (row_ops) {
    uint64_t rows = 1;
    for (int d = 0; d + 1 < xd.rank; ++d) rows *= static_cast<uint64_t>(xd.shape[d]);
    const uint64_t ob = od.gbase, on = tensor_span(od);
    if ((row_a && overlap(reinterpret_cast<uint64_t>(row_a), rows * 4, ob, on)) ||
        (row_b && overlap(reinterpret_cast<uint64_t>(row_b), rows * 4, ob, on)))
      return ret(ACP_ERR_INVALID, "a per-row scalar array shares memory with the output");
  }
  EngineRequest q{};
  q.op = op;
  q.mode = 2;
  q.x = &xd;
  q.out = &od;
  q.in_ptrs[0] = reinterpret_cast<const void*>(xd.gbase);
  q.n_in = 1;
  q.stage_box = stage_box;
  q.stages = stages;
  q.threads = threads;
  q.workgroups = workgroups;
  q.row_a = row_a;
  q.row_b = row_b;
  q.row_ops = row_ops;
  q.copy_only = false;
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  return keep(res, L);
}

acp_status build_tile_reduce(acp_op op, const acp_tile_desc* dst, const acp_tile_desc* src, int threads,
                           Launch* res) {
  acp::DescData s, d;
  if (!load_desc(src, &s) || !load_desc(dst, &d)) return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  if (op != ACP_OP_ADD) return ret(ACP_ERR_INVALID, "the store reduces with add");
  if (s.dtype != d.dtype) return ret(ACP_ERR_INVALID, "source and destination dtypes differ");
  if (s.dtype != ACP_U32 && s.dtype != ACP_F32 && s.dtype != ACP_F16)
    return ret(ACP_ERR_UNSUPPORTED, "reduce-add takes u32, f32 or f16");
  if (s.rank != d.rank) return ret(ACP_ERR_INVALID, "source and destination ranks differ");
  for (int k = 0; k < s.rank; ++k) {
    if (s.box[k] != d.box[k]) return ret(ACP_ERR_INVALID, "source and destination boxes differ");
    if (d.shape[k] == s.shape[k]) continue;
    if (d.shape[k] != 1 || s.box[k] != 1)
      return ret(ACP_ERR_INVALID, "a destination extent must equal the source's, or be 1 where the box is 1");
  }
  if (overlap(s, d)) return ret(ACP_ERR_INVALID, "source and destination share memory");
  bool one_each = true;  // every destination element receives one contribution
  for (int k = 0; k < s.rank; ++k) one_each = one_each && d.shape[k] == s.shape[k] && d.strides[k] == s.strides[k];
  if (one_each && s.dtype != ACP_U32) {
    // No two source elements meet in one destination element: dst' = src + dst
    // needs no atomics.  Both tensors ride the ring and the sum is stored in
    // place; every element is staged before the same lane stores it, and no
    // other trip touches it.
    EngineRequest q{};
    q.op = ACP_OP_ADD;
    q.mode = 2;
    q.x = &s;
    q.out = &d;
    q.in_ptrs[0] = reinterpret_cast<const void*>(s.gbase);
    q.in_ptrs[1] = reinterpret_cast<const void*>(d.gbase);
    q.n_in = 2;
    q.stage_box = s.box;
    q.threads = threads;
    q.copy_only = false;
    q.binary = 1;
    int tpt = 1;
    acp::Plan p;
    std::string why;
    if (acp::plan_box(s, false, &p, &why) == acp::PlanStatus::Ok)
      tile_schedule(p, 2, threads, 0, &q.workgroups, &q.stages, &tpt);
    q.stages = q.workgroups > 0 ? q.stages : 2;
    Launch L;
    const acp_status st = prepare(q, &L);
    if (st == ACP_OK && L.key.variant == 1) return keep(res, L);
    if (st != ACP_OK && st != ACP_ERR_UNSUPPORTED) return st;
    // otherwise: the atomic path below
  }
  EngineRequest q{};
  q.op = ACP_OP_ADD;
  q.mode = 3;
  q.x = &s;
  q.out = &d;
  q.in_ptrs[0] = reinterpret_cast<const void*>(s.gbase);
  q.n_in = 1;
  q.stage_box = s.box;
  q.threads = threads;
  q.copy_only = false;
  {
    acp::Plan p;
    std::string why;
    if (acp::plan_box(s, false, &p, &why) == acp::PlanStatus::Ok) {
      tile_schedule(p, 1, threads, 0, &q.workgroups, &q.stages, &q.tiles_per_trip);
      // Sums over batch dims: each workgroup owns whole destination tiles,
      // sums their contributions in registers and adds once per element.
      int64_t group = 1;
      for (int k = 0; k < s.rank; ++k)
        if (d.shape[k] == 1 && s.shape[k] > 1) group *= s.shape[k];
      static const bool grouped_ok = env_flag("ACP_REDUCE_GROUPED", true);
      const int64_t n_tiles = p.n_tiles();
      if (grouped_ok && group > 1 && n_tiles > 0) {
        const int64_t dst_tiles = n_tiles / group;
        static const int env_wg_per_cu = [] {
          const char* e = std::getenv("ACP_REDUCE_WG_PER_CU");
          return (e && std::atoi(e) > 0) ? std::atoi(e) : 0;
        }();
        static const int env_slots = [] {
          const char* e = std::getenv("ACP_REDUCE_STAGES");
          return (e && std::atoi(e) >= 2 && std::atoi(e) <= 4) ? std::atoi(e) : 3;
        }();
        const int64_t per_cu = env_wg_per_cu ? env_wg_per_cu : std::max<int64_t>(1, 16384 / p.tile_bytes());
        const int64_t want = static_cast<int64_t>(device_cu_count()) * per_cu;
        // About 16 KiB of tiles per CU in flight per ring step and 3 ring
        // slots (ACP_REDUCE_WG_PER_CU, ACP_REDUCE_STAGES): the best of 2-8
        // workgroups per CU x 2-4 slots x 4 or 8 KiB tiles measured on 128
        // float32 contributions per element of [500,1024] (8 KiB tiles, two
        // per CU: 5.1 TB/s).  Few destination tiles: split each one's
        // contributions over k workgroups (k atomic adds per element instead
        // of one).
        int64_t k = 1;
        while (dst_tiles * k * 2 <= want && group % (k * 2) == 0) k *= 2;
        const int64_t sub = group / k;                 // contributions summed per workgroup group
        const int64_t groups = dst_tiles * k;
        const int64_t g = std::min<int64_t>(groups, want);
        const int64_t per = (groups + g - 1) / g;      // groups per workgroup
        q.red_group = sub;
        q.red_per_wg = per * sub;
        q.workgroups = static_cast<int>((groups + per - 1) / per);
        q.stages = env_slots;
        q.tiles_per_trip = 1;
      }
    } else {
      q.stages = 1;
    }
  }
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  if (L.key.mode != 7) return ret(ACP_ERR_UNSUPPORTED, "reduce-add needs 16-byte rounds and 1, 2, 4 or 8 rounds per thread");
  return keep(res, L);
}

acp_status build_stream_reduce_rows(acp_op op, float* out, const acp_tile_desc* x, const int32_t* stage_box, int stages,
                                  int threads, int workgroups, Launch* res) {
  acp::DescData xd;
  if (!load_desc(x, &xd)) return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  if (op != ACP_OP_ADD) return ret(ACP_ERR_INVALID, "rows reduce with add");
  if (!out) return ret(ACP_ERR_INVALID, "null output");
  if (!stage_box) return ret(ACP_ERR_INVALID, "null stage box");
  if (stages < 2 || stages > 4) return ret(ACP_ERR_INVALID, "stages must be 2, 3 or 4");
  if (workgroups < 0) return ret(ACP_ERR_INVALID, "workgroups must be >= 0");
  if (xd.dtype != ACP_F32 && xd.dtype != ACP_F16) return ret(ACP_ERR_UNSUPPORTED, "row reduction takes f16 or f32");
  const int r = xd.rank;
  if (r < 2) return ret(ACP_ERR_INVALID, "row reduction needs rank >= 2");
  for (int d = 0; d < r; ++d)
    if (stage_box[d] < 1) return ret(ACP_ERR_INVALID, "stage box must be >= 1");
  if (xd.box[r - 1] != xd.shape[r - 1] || stage_box[r - 1] != xd.shape[r - 1])
    return ret(ACP_ERR_INVALID, "tiles and stages must hold whole rows (innermost box = innermost extent)");
  int64_t rows = 1;
  for (int d = 0; d + 1 < r; ++d) rows *= xd.shape[d];
  if (rows >= (int64_t(1) << 29)) return ret(ACP_ERR_UNSUPPORTED, "too many rows");
  if (reinterpret_cast<uint64_t>(out) % 4) return ret(ACP_ERR_INVALID, "output not 4-byte aligned");
  if (overlap(reinterpret_cast<uint64_t>(out), static_cast<uint64_t>(rows) * 4, xd.gbase, tensor_span(xd)))
    return ret(ACP_ERR_INVALID, "the output shares memory with x");
  EngineRequest q{};
  q.op = ACP_OP_ADD;
  q.mode = 4;
  q.x = &xd;
  q.out = &xd;  // same shape; the output is the packed row array `out`
  q.in_ptrs[0] = reinterpret_cast<const void*>(xd.gbase);
  q.n_in = 1;
  q.stage_box = stage_box;
  q.stages = stages;
  q.threads = threads;
  q.workgroups = workgroups;
  q.copy_only = false;
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  if (L.key.mode != 8 && L.key.mode != 10)
    return ret(ACP_ERR_UNSUPPORTED, "row reduction needs 16-byte rounds and 1, 2, 4 or 8 rounds per thread");
  if (L.args.red_rows > 64u * static_cast<uint32_t>(L.args.waves))
    return ret(ACP_ERR_UNSUPPORTED, "row reduction stages hold at most 64 rows per wave");
  L.args.out = reinterpret_cast<char*>(out);
  L.args.out_span = static_cast<uint64_t>(rows) * 4u;
  return keep(res, L);
}

acp_status build_stream_binary(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x, const acp_tile_desc* z,
                             const int32_t* stage_box, int stages, int threads, int workgroups, acp_staging z_staging,
                             Launch* res) {
  acp::DescData xd, zd, od;
  if (!load_desc(x, &xd) || !load_desc(z, &zd) || !load_desc(out, &od))
    return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  if (op != ACP_OP_ADD && op != ACP_OP_MUL) return ret(ACP_ERR_INVALID, "two-tensor streams are add or mul");
  if (z_staging != ACP_STAGE_RING && z_staging != ACP_STAGE_SET) return ret(ACP_ERR_INVALID, "unknown staging");
  if (!stage_box) return ret(ACP_ERR_INVALID, "null stage box");
  if (stages < 2 || stages > 4) return ret(ACP_ERR_INVALID, "stages must be 2, 3 or 4");
  if (workgroups < 0) return ret(ACP_ERR_INVALID, "workgroups must be >= 0");
  if (!same_geometry(zd, xd, true) || zd.dtype != xd.dtype || zd.swizzle != xd.swizzle)
    return ret(ACP_ERR_INVALID, "x and z must share one layout (dtype, shape, strides, box, swizzle)");
  if (!same_geometry(xd, od, false) || od.dtype != xd.dtype)
    return ret(ACP_ERR_INVALID, "output dtype, shape or box differs from x");
  if (!is_float(xd.dtype)) return ret(ACP_ERR_UNSUPPORTED, "two-tensor streams take float16 or float32");
  if (overlap(xd, od) || overlap(zd, od)) return ret(ACP_ERR_INVALID, "the output shares memory with x or z");
  for (int d = 0; d < xd.rank; ++d)
    if (stage_box[d] < 1) return ret(ACP_ERR_INVALID, "stage box must be >= 1");
  EngineRequest q{};
  q.op = op;
  q.mode = 2;
  q.x = &xd;
  q.out = &od;
  q.in_ptrs[0] = reinterpret_cast<const void*>(xd.gbase);
  q.in_ptrs[1] = reinterpret_cast<const void*>(zd.gbase);
  q.n_in = 2;
  q.stage_box = stage_box;
  q.stages = stages;
  q.threads = threads;
  q.workgroups = workgroups;
  q.copy_only = false;
  q.binary = z_staging == ACP_STAGE_SET ? 2 : 1;
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  return keep(res, L);
}

}  // namespace

extern "C" {

int acp_abi_version(void) { return ACP_ABI_VERSION; }

const char* acp_last_error(void) { return g_last_error.c_str(); }

const char* acp_last_kernel(void) { return g_last_kernel.c_str(); }

acp_status acp_encode_tiled(acp_tile_desc* out, acp_dtype dtype, int rank, const void* gbase,
                            const int64_t* shape, const int64_t* strides, const int32_t* box,
                            acp_swizzle swizzle, acp_oob oob) {
  if (!out || !shape || !strides || !box) return ret(ACP_ERR_INVALID, "null argument");
  if (!gbase) return ret(ACP_ERR_INVALID, "null tensor address");
  const int es = acp::dtype_size(dtype);
  if (es < 0) return ret(ACP_ERR_INVALID, "unknown dtype");
  if (rank < 1 || rank > ACP_MAX_INPUT_RANK) return ret(ACP_ERR_INVALID, "rank must be 1..8");
  if (swizzle != ACP_SWIZZLE_NONE && swizzle != ACP_SWIZZLE_32B && swizzle != ACP_SWIZZLE_64B &&
      swizzle != ACP_SWIZZLE_128B)
    return ret(ACP_ERR_INVALID, "unknown swizzle");
  if (oob != ACP_OOB_ZERO) return ret(ACP_ERR_INVALID, "unknown out-of-bounds fill");
  acp::DescData d;
  std::memset(&d, 0, sizeof(d));
  d.magic = acp::kDescMagic;
  d.dtype = static_cast<uint8_t>(dtype);
  d.esize = static_cast<uint8_t>(es);
  d.rank = static_cast<uint8_t>(rank);
  d.swizzle = static_cast<uint8_t>(swizzle);
  d.oob = static_cast<uint8_t>(oob);
  d.gbase = reinterpret_cast<uint64_t>(gbase);
  for (int k = 0; k < rank; ++k) {
    if (shape[k] < 0 || strides[k] < 1 || box[k] < 1)
      return ret(ACP_ERR_INVALID, "extents must be >= 0, strides and box >= 1");
    d.shape[k] = shape[k];
    d.strides[k] = strides[k];
    d.box[k] = box[k];
  }
  acp::Plan p;
  std::string why;
  const acp::PlanStatus ps = acp::plan_box(d, true, &p, &why);
  if (ps != acp::PlanStatus::Ok) return from_plan(ps, why);
  std::memset(out->opaque, 0, sizeof(out->opaque));
  std::memcpy(out->opaque, &d, sizeof(d));
  return ret(ACP_OK);
}

acp_status acp_plan_query(const acp_tile_desc* desc, int threads, int copy_only, acp_plan_info* out) {
  acp::DescData d;
  if (!out || !load_desc(desc, &d)) return ret(ACP_ERR_INVALID, "not an encoded descriptor");
  acp::Plan p;
  std::string why;
  acp::PlanStatus ps = acp::plan_box(d, copy_only != 0, &p, &why);
  if (ps != acp::PlanStatus::Ok) return from_plan(ps, why);
  if (threads) {
    ps = acp::plan_partition(&p, threads, d.gbase, &why);
    if (ps != acp::PlanStatus::Ok) return from_plan(ps, why);
  }
  std::memset(out, 0, sizeof(*out));
  out->rank = static_cast<int32_t>(p.dims.size());
  out->desc_elem_bytes = p.desc_esize;
  for (int k = 0; k < out->rank; ++k) {
    const acp::DescDim& dd = p.dims[p.dims.size() - 1 - k];
    out->dims[k] = dd.extent;
    out->strides[k] = dd.stride;
    out->box[k] = static_cast<int32_t>(dd.box);
  }
  out->issues = static_cast<int32_t>(p.issues());
  out->n_issue_axes = static_cast<int32_t>(p.issue_axes.size());
  out->n_image_axes = static_cast<int32_t>(p.image_axes().size());
  out->swizzle = p.swizzle;
  out->promoted = p.promoted ? 1 : 0;
  out->threads = p.threads;
  out->vec = p.vec;
  out->vec_bytes = p.vec_bytes;
  out->outer = p.outer;
  out->tile_bytes = p.tile_bytes();
  out->n_tiles = p.n_tiles();
  return ret(ACP_OK);
}

acp_status acp_tile_copy(const acp_tile_desc* src, const acp_tile_desc* dst, int threads, void* hip_stream) {
  CallKey k(1);
  k.desc(src);
  k.desc(dst);
  k.val(threads);
  return run_cached(k, [&](Launch* L) { return build_tile_copy(src, dst, threads, L); }, hip_stream);
}

acp_status acp_tile_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* const* in, int n_in,
                          int threads, void* hip_stream) {
  CallKey k(2);
  k.val(op);
  k.desc(out);
  k.val(n_in);
  if (n_in < 0 || n_in > 3 || (n_in > 0 && !in)) k.ok = false;
  for (int i = 0; k.ok && i < n_in; ++i) k.desc(in[i]);
  k.val(threads);
  return run_cached(k, [&](Launch* L) { return build_tile_ewise(op, out, in, n_in, threads, L); }, hip_stream);
}

acp_status acp_stream_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x, const float* row_a,
                            const float* row_b, const int32_t* stage_box, int stages, int threads, int workgroups,
                            void* hip_stream) {
  CallKey k(3);
  k.val(op);
  k.desc(out);
  k.desc(x);
  k.val(row_a);
  k.val(row_b);
  k.ints(stage_box, desc_rank(x));
  k.val(stages);
  k.val(threads);
  k.val(workgroups);
  return run_cached(k, [&](Launch* L) {
    return build_stream_ewise(op, out, x, row_a, row_b, stage_box, stages, threads, workgroups, L);
  }, hip_stream);
}

acp_status acp_tile_reduce(acp_op op, const acp_tile_desc* dst, const acp_tile_desc* src, int threads,
                           void* hip_stream) {
  CallKey k(4);
  k.val(op);
  k.desc(dst);
  k.desc(src);
  k.val(threads);
  return run_cached(k, [&](Launch* L) { return build_tile_reduce(op, dst, src, threads, L); }, hip_stream);
}

acp_status acp_stream_reduce_rows(acp_op op, float* out, const acp_tile_desc* x, const int32_t* stage_box, int stages,
                                  int threads, int workgroups, void* hip_stream) {
  CallKey k(5);
  k.val(op);
  k.val(out);
  k.desc(x);
  k.ints(stage_box, desc_rank(x));
  k.val(stages);
  k.val(threads);
  k.val(workgroups);
  return run_cached(k, [&](Launch* L) {
    return build_stream_reduce_rows(op, out, x, stage_box, stages, threads, workgroups, L);
  }, hip_stream);
}

acp_status acp_stream_binary(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x, const acp_tile_desc* z,
                             const int32_t* stage_box, int stages, int threads, int workgroups, acp_staging z_staging,
                             void* hip_stream) {
  CallKey k(6);
  k.val(op);
  k.desc(out);
  k.desc(x);
  k.desc(z);
  k.ints(stage_box, desc_rank(x));
  k.val(stages);
  k.val(threads);
  k.val(workgroups);
  k.val(z_staging);
  return run_cached(k, [&](Launch* L) {
    return build_stream_binary(op, out, x, z, stage_box, stages, threads, workgroups, z_staging, L);
  }, hip_stream);
}

acp_status acp_debug_lds_image(const acp_tile_desc* src, int64_t tile_index, int threads, void* out_bytes,
                               void* hip_stream) {
  acp::DescData s;
  if (!load_desc(src, &s) || !out_bytes) return ret(ACP_ERR_INVALID, "bad descriptor or output");
  EngineRequest q{};
  q.op = ACP_OP_COPY;
  q.mode = 0;
  q.x = &s;
  q.out = &s;
  q.in_ptrs[0] = reinterpret_cast<const void*>(s.gbase);
  q.n_in = 1;
  q.stage_box = s.box;
  q.stages = 1;
  q.threads = threads;
  q.copy_only = true;
  Launch L;
  const acp_status st = prepare(q, &L);
  if (st != ACP_OK) return st;
  if (tile_index < 0 || tile_index >= L.n_tiles) return ret(ACP_ERR_INVALID, "tile index out of range");
  L.args.tile0 = static_cast<uint32_t>(tile_index);
  acp::Plan p;
  std::string why;
  acp::plan_box(s, true, &p, &why);
  const hipError_t e = acp::lds_image_launch(acp::lds_image_kernel(L.key.vec_bytes), L.args, L.block, L.lds,
                                             out_bytes, static_cast<uint32_t>(p.tile_bytes()),
                                             static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_ring_trace(int n_iters, int stages, int loads, int stores, int32_t* out_events,
                                void* hip_stream) {
  if (!out_events || n_iters < 0 || stages < 1 || stages > 4 || loads < 0 || stores < 0)
    return ret(ACP_ERR_INVALID, "bad ring trace arguments");
  if (n_iters == 0) return ret(ACP_OK);
  const hipError_t e = acp::ring_trace_launch(n_iters, stages, loads, stores, out_events,
                                              static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_stream_copy(void* dst, const void* src, int64_t bytes, int workgroups, void* hip_stream) {
  if (!dst || !src || bytes < 0 || workgroups < 0) return ret(ACP_ERR_INVALID, "bad stream copy arguments");
  if (bytes % 16 != 0) return ret(ACP_ERR_INVALID, "stream copy moves whole 16-byte units");
  if (bytes >= (int64_t(1) << 40)) return ret(ACP_ERR_INVALID, "stream copy size out of range");
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return ret(ACP_ERR_INVALID, "source and destination overlap");
  if (bytes == 0) return ret(ACP_OK);
  const int64_t blocks = (bytes + 16383) / 16384;
  int64_t grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid > blocks) grid = blocks;
  const hipError_t e = acp::stream_copy_launch(src, dst, static_cast<uint64_t>(bytes), static_cast<unsigned>(grid),
                                               static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_stream_copy_shape(void* dst, const void* src, int64_t bytes, int workgroups, int threads,
                                       int unroll, int load_nt, int store_nt, void* hip_stream) {
  if (!dst || !src || bytes < 0 || workgroups < 0) return ret(ACP_ERR_INVALID, "bad stream copy arguments");
  if ((load_nt != 0 && load_nt != 1) || (store_nt != 0 && store_nt != 1))
    return ret(ACP_ERR_INVALID, "cache policies are 0 (default) or 1 (non-temporal)");
  if (bytes % 16 != 0) return ret(ACP_ERR_INVALID, "stream copy moves whole 16-byte units");
  if (bytes >= (int64_t(1) << 40)) return ret(ACP_ERR_INVALID, "stream copy size out of range");
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return ret(ACP_ERR_INVALID, "source and destination overlap");
  const void* kernel = acp::copy_shape_kernel_for(threads, unroll, load_nt, store_nt);
  if (!kernel) return ret(ACP_ERR_UNSUPPORTED, "no reference copy kernel of that shape is built");
  if (bytes == 0) return ret(ACP_OK);
  const int64_t block = static_cast<int64_t>(threads) * unroll * 16;
  const int64_t blocks = (bytes + block - 1) / block;
  int64_t grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid > blocks) grid = blocks;
  const hipError_t e = acp::copy_shape_launch(kernel, src, dst, static_cast<uint64_t>(bytes),
                                              static_cast<unsigned>(grid), static_cast<unsigned>(threads),
                                              static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_copy_tiles(void* dst, const void* src, int esize, const int64_t* shape,
                                const int64_t* src_strides, const int32_t* box, int tiles_per_trip, int threads,
                                int workgroups, void* hip_stream) {
  if (!dst || !src || !shape || !src_strides || !box || workgroups < 0) return ret(ACP_ERR_INVALID, "null argument");
  if (esize != 1 && esize != 2 && esize != 4 && esize != 8) return ret(ACP_ERR_INVALID, "element size 1, 2, 4 or 8");
  if (tiles_per_trip != 1 && tiles_per_trip != 2 && tiles_per_trip != 4)
    return ret(ACP_ERR_INVALID, "tiles per trip 1, 2 or 4");
  if (threads != 128 && threads != 256) return ret(ACP_ERR_INVALID, "threads 128 or 256");
  for (int d = 0; d < 3; ++d)
    if (shape[d] < 1 || src_strides[d] < 1 || box[d] < 1)
      return ret(ACP_ERR_INVALID, "extents, strides and boxes must be >= 1");
  if (src_strides[2] != 1) return ret(ACP_ERR_INVALID, "innermost source stride must be 1");
  if (box[0] != 1) return ret(ACP_ERR_INVALID, "a tile spans one index of dim 0");
  const int64_t row_bytes = shape[2] * esize;
  const int64_t group_bytes = static_cast<int64_t>(tiles_per_trip) * box[2] * esize;
  if (row_bytes % 16 != 0 || group_bytes % 16 != 0)
    return ret(ACP_ERR_INVALID, "rows and tile groups must be whole 16-byte chunks");
  if (static_cast<int64_t>(box[1]) * (group_bytes / 16) > 8 * static_cast<int64_t>(threads))
    return ret(ACP_ERR_INVALID, "a tile group holds at most 8 chunks of 16 bytes per lane");
  const int64_t in_b[2] = {src_strides[0] * esize, src_strides[1] * esize};
  const int64_t out_b[2] = {shape[1] * row_bytes, row_bytes};
  if (in_b[0] % 16 != 0 || in_b[1] % 16 != 0) return ret(ACP_ERR_INVALID, "source strides must be 16-byte multiples");
  if (reinterpret_cast<uint64_t>(src) % 16 != 0 || reinterpret_cast<uint64_t>(dst) % 16 != 0)
    return ret(ACP_ERR_INVALID, "source and destination must be 16-byte aligned");
  if ((box[1] - 1) * std::max(in_b[1], out_b[1]) + group_bytes >= (int64_t(1) << 31) || row_bytes >= (int64_t(1) << 31))
    return ret(ACP_ERR_INVALID, "a tile group spans 2 GiB or more");
  const int64_t tiles_1 = (shape[1] + box[1] - 1) / box[1];
  const int64_t groups_2 = (row_bytes + group_bytes - 1) / group_bytes;
  const int64_t n_groups = shape[0] * tiles_1 * groups_2;
  if (n_groups >= (int64_t(1) << 31) || shape[1] >= (int64_t(1) << 31)) return ret(ACP_ERR_INVALID, "too many tiles");
  const int64_t span_in = (shape[0] - 1) * in_b[0] + (shape[1] - 1) * in_b[1] + row_bytes;
  const int64_t span_out = shape[0] * out_b[0];
  const char* s = static_cast<const char*>(src);
  const char* o = static_cast<const char*>(dst);
  if (s < o + span_out && o < s + span_in) return ret(ACP_ERR_INVALID, "source and destination overlap");
  int64_t grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid > n_groups) grid = n_groups;
  const hipError_t e = acp::copy_tiles_launch(
      src, dst, in_b, out_b, static_cast<uint32_t>(shape[1]), static_cast<uint32_t>(row_bytes),
      static_cast<uint32_t>(box[1]), static_cast<uint32_t>(group_bytes), static_cast<uint32_t>(tiles_1),
      static_cast<uint32_t>(groups_2), static_cast<uint32_t>(n_groups), static_cast<unsigned>(threads),
      static_cast<unsigned>(grid), static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

// grid of a reference stream: `workgroups` (0: one per compute unit), at
// most one per 16 KiB block
unsigned ref_grid(int64_t bytes, int workgroups) {
  const int64_t blocks = (bytes + 16383) / 16384;
  int64_t grid = workgroups > 0 ? workgroups : device_cu_count();
  return static_cast<unsigned>(grid > blocks ? blocks : grid);
}

acp_status acp_debug_stream_read(const void* src, int64_t bytes, void* sums, int workgroups, void* hip_stream) {
  if (!src || !sums || bytes < 0 || workgroups < 0) return ret(ACP_ERR_INVALID, "bad stream read arguments");
  if (bytes % 16 != 0) return ret(ACP_ERR_INVALID, "stream read moves whole 16-byte units");
  if (bytes >= (int64_t(1) << 40)) return ret(ACP_ERR_INVALID, "stream read size out of range");
  if (bytes == 0) return ret(ACP_OK);
  const unsigned grid = ref_grid(bytes, workgroups);
  const char* s = static_cast<const char*>(src);
  const char* o = static_cast<const char*>(sums);
  if (o < s + bytes && s < o + 16 * static_cast<int64_t>(grid)) return ret(ACP_ERR_INVALID, "sums overlap the source");
  const hipError_t e = acp::stream_read_launch(src, static_cast<uint64_t>(bytes), sums, grid,
                                               static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_stream_fill(void* dst, int64_t bytes, uint32_t pattern, int workgroups, void* hip_stream) {
  if (!dst || bytes < 0 || workgroups < 0) return ret(ACP_ERR_INVALID, "bad stream fill arguments");
  if (bytes % 16 != 0) return ret(ACP_ERR_INVALID, "stream fill writes whole 16-byte units");
  if (bytes >= (int64_t(1) << 40)) return ret(ACP_ERR_INVALID, "stream fill size out of range");
  if (bytes == 0) return ret(ACP_OK);
  const hipError_t e = acp::stream_fill_launch(dst, static_cast<uint64_t>(bytes), pattern, ref_grid(bytes, workgroups),
                                               static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_stream_widen(float* dst, const void* src, int64_t elements, int workgroups, void* hip_stream) {
  if (!dst || !src || elements < 0 || workgroups < 0) return ret(ACP_ERR_INVALID, "bad stream widen arguments");
  if (elements % 8 != 0) return ret(ACP_ERR_INVALID, "stream widen converts whole groups of 8 elements");
  if (elements >= (int64_t(1) << 38)) return ret(ACP_ERR_INVALID, "stream widen size out of range");
  const int64_t in_bytes = elements * 2;
  const char* s = static_cast<const char*>(src);
  const char* d = reinterpret_cast<const char*>(dst);
  if (s < d + 2 * in_bytes && d < s + in_bytes) return ret(ACP_ERR_INVALID, "source and destination overlap");
  if (elements == 0) return ret(ACP_OK);
  const int64_t blocks = (in_bytes + 8191) / 8192;
  int64_t grid = workgroups > 0 ? workgroups : device_cu_count();
  if (grid > blocks) grid = blocks;
  const hipError_t e = acp::stream_widen_launch(src, dst, static_cast<uint64_t>(in_bytes), static_cast<unsigned>(grid),
                                                static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

acp_status acp_debug_widen_tiles(float* dst, const void* src, const int64_t* shape, const int64_t* src_strides,
                                 const int32_t* box, const int32_t* stage_box, void* hip_stream) {
  if (!dst || !src || !shape || !src_strides || !box || !stage_box) return ret(ACP_ERR_INVALID, "null argument");
  if (src_strides[4] != 1) return ret(ACP_ERR_INVALID, "innermost source stride must be 1");
  int64_t in_b[5], out_b[5], span_in = 2, n_tiles = 1, st = 4;
  uint32_t tgrid[5], bx[5], sb[5];
  for (int d = 4; d >= 0; --d) {
    if (shape[d] < 1 || box[d] < 1 || stage_box[d] < 1 || src_strides[d] < 1)
      return ret(ACP_ERR_INVALID, "extents, strides and boxes must be >= 1");
    if (shape[d] % box[d] != 0 || box[d] % stage_box[d] != 0)
      return ret(ACP_ERR_INVALID, "tiles and stages must be whole");
    if (d < 3 && stage_box[d] != 1) return ret(ACP_ERR_INVALID, "a stage spans the two innermost dims only");
    in_b[d] = src_strides[d] * 2;
    out_b[d] = st;
    st *= shape[d];
    span_in += (shape[d] - 1) * in_b[d];
    tgrid[d] = static_cast<uint32_t>(shape[d] / box[d]);
    bx[d] = static_cast<uint32_t>(box[d]);
    sb[d] = static_cast<uint32_t>(stage_box[d]);
    n_tiles *= shape[d] / box[d];
  }
  if (stage_box[4] % 4 != 0 || static_cast<int64_t>(stage_box[3]) * stage_box[4] / 4 > 2048)
    return ret(ACP_ERR_INVALID, "a stage row must hold whole 4-element pieces, at most 2048 per stage");
  for (int d = 0; d < 4; ++d)
    if (in_b[d] % 8 != 0) return ret(ACP_ERR_INVALID, "source strides must be 8-byte multiples");
  if (reinterpret_cast<uint64_t>(src) % 8 != 0 || reinterpret_cast<uint64_t>(dst) % 16 != 0)
    return ret(ACP_ERR_INVALID, "source must be 8-byte and destination 16-byte aligned");
  if (n_tiles >= (int64_t(1) << 31)) return ret(ACP_ERR_INVALID, "too many tiles");
  const char* s = static_cast<const char*>(src);
  const char* o = reinterpret_cast<const char*>(dst);
  if (s < o + st && o < s + span_in) return ret(ACP_ERR_INVALID, "source and destination overlap");
  const hipError_t e = acp::widen_tiles_launch(src, dst, in_b, out_b, tgrid, bx, sb, static_cast<uint32_t>(n_tiles),
                                               static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return ret(ACP_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return ret(ACP_OK);
}

}  // extern "C"
