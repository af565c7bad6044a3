// Launch entry points of the kernels (host side of the library).
#pragma once
#include <hip/hip_runtime.h>

#include "s2a_geom.h"

struct S2AParams;

int s2a_fwd_tile_rows(int D);  // query rows per forward workgroup

hipError_t s2a_launch_fwd(const void *q, const void *k, const void *v,
                          void *o, bool o_f32, float *lse, int D,
                          const S2AParams &p, hipStream_t st);

hipError_t s2a_launch_bwd(const void *q, const void *k, const void *v,
                          const void *o, bool o_f32, const float *lse,
                          const void *dout, float *dq, float *dk, float *dv,
                          float *delta, int D, const S2AParams &p,
                          hipStream_t st);

hipError_t s2a_launch_bwd_pre(const void *o, bool o_f32, const void *dout,
                              float *delta, int B, int N, int H, int D,
                              hipStream_t st);

hipError_t s2a_launch_bwd_dkdv(const void *q, const void *k, const void *v,
                               const void *dout, const float *lse,
                               const float *delta, float *dk, float *dv,
                               int D, const S2AParams &p, hipStream_t st);

hipError_t s2a_launch_bwd_dq(const void *q, const void *k, const void *v,
                             const void *dout, const float *lse,
                             const float *delta, float *dq, int D,
                             const S2AParams &p, hipStream_t st);

// Bytes of the dS workspace for the launch geometry p (long double: the
// caller checks the range before it forms a size_t).
long double s2a_ds_workspace_bytes(const S2AParams &p);

hipError_t s2a_launch_map(const S2AGeom &g, int *gid, int *slot, int *src,
                          hipStream_t st);

hipError_t s2a_launch_rope(const void *x, void *y, bool f32, bool inverse,
                           int B, int N, int H, int D, const int *pos,
                           float base, float pscale, bool half,
                           hipStream_t st);
