/* A plain C99 client of the C ABI (no C++ in the header it includes):
 * encode the 8x256 float16 swizzled tile of the TMA worked example, query
 * its plan, and see a declined request with its reason.  Host code only. */
#include <stdio.h>
#include "acp.h"
int main(void) {
  acp_tile_desc d;
  const int64_t shape[2] = {8, 256}, strides[2] = {256, 1};
  const int32_t box[2] = {8, 256};
  acp_status s = acp_encode_tiled(&d, ACP_F16, 2, (const void*)(uintptr_t)(1u << 20), shape, strides, box,
                                  ACP_SWIZZLE_128B, ACP_OOB_ZERO);
  if (s != ACP_OK) { printf("encode failed %d %s\n", (int)s, acp_last_error()); return 1; }
  acp_plan_info p;
  s = acp_plan_query(&d, 64, 1, &p);
  if (s != ACP_OK) { printf("query failed %d\n", (int)s); return 1; }
  printf("rank %d dims %lld %lld %lld strides %lld %lld %lld box %d %d %d vec %d vec_bytes %d outer %d\n", p.rank,
         (long long)p.dims[0], (long long)p.dims[1], (long long)p.dims[2], (long long)p.strides[0],
         (long long)p.strides[1], (long long)p.strides[2], p.box[0], p.box[1], p.box[2], p.vec, p.vec_bytes, p.outer);
  const int64_t bad_strides[2] = {1, 8};
  s = acp_encode_tiled(&d, ACP_F16, 2, (const void*)(uintptr_t)(1u << 20), shape, bad_strides, box, ACP_SWIZZLE_NONE,
                       ACP_OOB_ZERO);
  printf("declined %d %s\n", (int)(s == ACP_ERR_DECLINED), acp_last_error());
  printf("abi %d\n", acp_abi_version());
  return 0;
}
