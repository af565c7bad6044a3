// Group index maps, written by the same geometry functions the attention
// kernels use to address rows (s2a_geom.h), so a bit-exact comparison of
// these maps with an independent reference checks the kernels' grouping.
#include "s2a_device.h"
#include "s2a_kernels.h"

namespace {

__global__ __launch_bounds__(256) void s2a_map_kernel(S2AGeom g, int *gid,
                                                      int *slot, int *src) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= g.N) return;
#pragma unroll
  for (int cls = 0; cls < 2; ++cls) {
    int gi, sl;
    s2a_locate(g, cls, x, gi, sl);
    gid[cls * g.N + x] = gi;
    slot[cls * g.N + x] = sl;
    int gr, j, len;
    S2ARun run;
    s2a_row_locate(g, cls, x, gr, j);  // x read as a row of the layout
    s2a_group(g, cls, gr, run, len);
    src[cls * g.N + x] = run.pos(j);
  }
}

}  // namespace

hipError_t s2a_launch_map(const S2AGeom &g, int *gid, int *slot, int *src,
                          hipStream_t st) {
  dim3 grid((unsigned)((g.N + 255) / 256)), block(256);
  S2AGeom gg = g;
  void *args[] = {(void *)&gg, (void *)&gid, (void *)&slot, (void *)&src};
  return hipLaunchKernel((const void *)s2a_map_kernel, grid, block, args, 0,
                         st);
}
