// Host-only robustness check of the planner: random descriptors (ranks 1-8,
// every dtype and swizzle mode, unaligned bases, padded strides, empty dims,
// boxes past the tensor) through plan_box, plan_partition and the plan
// queries, built with the address and undefined-behaviour sanitizers; any
// finding aborts.  Prints the status counts.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include "acp_plan.hpp"
int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  std::mt19937_64 rng(12345);
  auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long ok = 0, declined = 0, unsup = 0, invalid = 0;
  for (long it = 0; it < iters; ++it) {
    acp::DescData d{};
    d.magic = acp::kDescMagic;
    const int esz[] = {1, 2, 4, 8, 2, 4};
    d.dtype = static_cast<uint8_t>(U(0, 5));
    d.esize = static_cast<uint8_t>(esz[d.dtype]);
    d.rank = static_cast<uint8_t>(U(1, 8));
    d.swizzle = static_cast<uint8_t>(U(0, 4) == 0 ? U(1, 3) : 0);
    d.gbase = static_cast<uint64_t>(U(0, 3)) * 16 + (U(0, 9) == 0 ? U(0, 15) : 0);
    int64_t st = U(0, 50) == 0 ? 1 + U(0, 3) : 1;
    for (int k = d.rank - 1; k >= 0; --k) {
      d.shape[k] = U(0, 20) == 0 ? 0 : U(1, k == d.rank - 1 ? 700 : 40);
      d.strides[k] = st;
      d.box[k] = U(0,2) ? U(1, k == d.rank - 1 ? 600 : 40) : (d.shape[k] > 0 ? int(d.shape[k]) : 1);
      st = st * (d.shape[k] > 0 ? d.shape[k] : 1) + (U(0, 4) == 0 ? U(1, 9) : 0);
    }
    acp::Plan p;
    std::string why;
    const bool copy_only = U(0, 1);
    auto s = acp::plan_box(d, copy_only, &p, &why);
    if (s == acp::PlanStatus::Ok) {
      const int threads = 64 * U(1, 16);
      s = acp::plan_partition(&p, threads, d.gbase, &why);
      if (s == acp::PlanStatus::Ok) {
        (void)p.image_axes(); (void)p.issues(); (void)p.tile_bytes(); (void)p.n_tiles();
        ++ok;
        continue;
      }
    }
    if (s == acp::PlanStatus::Declined) ++declined;
    else if (s == acp::PlanStatus::Unsupported) ++unsup;
    else ++invalid;
  }
  printf("ok %ld declined %ld unsupported %ld invalid %ld\n", ok, declined, unsup, invalid);
  return 0;
}
