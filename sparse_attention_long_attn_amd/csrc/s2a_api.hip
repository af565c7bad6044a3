// C ABI of the shifted sparse attention engine: argument checks, launch
// geometry and error reporting.  See include/s2attn.h for the contract.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "s2attn.h"
#include "s2a_device.h"
#include "s2a_kernels.h"

namespace {

thread_local char g_err[512];

s2a_status fail(s2a_status st, const char *fmt, long long a = 0,
                long long b = 0) {
  snprintf(g_err, sizeof g_err, fmt, a, b);
  return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// Launch-time checks of the group shape: H % 2 == 0, G % 2 == 0 and
// N % G == 0 after padding, the valid length inside [1, N], and only the
// shifts 0 and G/2 (PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调",
// §1, paragraph on asserting the divisibility conditions at launch).
s2a_status check_shape(int B, int N, int H, int D, int G, int shift,
                       int boundary, int valid_len) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0 || G <= 0)
    return fail(S2A_EINVAL, "sizes must be positive");
  if (H % 2) return fail(S2A_EINVAL, "H=%lld must be even", H);
  if (G % 2) return fail(S2A_EINVAL, "G=%lld must be even", G);
  if (N % G)
    return fail(S2A_EINVAL, "padded N=%lld is not a multiple of G=%lld", N, G);
  if (valid_len < 1 || valid_len > N)
    return fail(S2A_EINVAL, "valid_len=%lld outside [1, N=%lld]", valid_len, N);
  if (shift != 0 && shift != G / 2)
    return fail(S2A_EINVAL, "shift=%lld must be 0 or G/2=%lld", shift, G / 2);
  if (boundary != S2A_WRAP && boundary != S2A_SPLIT && boundary != S2A_CYCLIC)
    return fail(S2A_EINVAL, "boundary=%lld is not WRAP, SPLIT or CYCLIC",
                boundary);
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(S2A_EUNSUPPORTED, "head width D=%lld not in {16,32,64,128}", D);
  // Offsets of a row are formed in 64 bits; positions and grid sizes in 32;
  // offsets inside one 128-row tile in 32 (128 * H * D * 2 bytes < 2^32).
  const long long units = (long long)B * H * (N / G + 1);
  if ((long long)B * N > (1ll << 31) || units * (G / 16 + 1) > (1ll << 31))
    return fail(S2A_EINVAL, "problem too large for one launch");
  if ((long long)H * D >= (1ll << 24))
    return fail(S2A_EUNSUPPORTED, "H*D=%lld is 2^24 or more", (long long)H * D);
  return S2A_OK;
}

S2AGeom make_geom(int N, int G, int shift, int boundary, int L) {
  S2AGeom g;
  g.N = N;
  g.G = G;
  g.M = N / G;
  g.s = (g.M == 1) ? 0 : shift;  // a single group has nothing to shift across
  g.boundary = boundary;
  g.L = L;
  g.hl = 0;
  g.hw = 0;
  return g;
}

// Halo of the shard [row0, row0 + T) (see s2a_geom.h): exactly the rows
// outside it that its valid queries read.  The left halo holds global
// rows [left0, left0 + hl), the wrap halo rows [0, hw).  Under WRAP the
// first shard's left halo is the end of the sequence, N-s .. N-1, of which
// only the rows below L are kept (padding never enters a softmax, and
// dropping it keeps the valid halo rows next to row 0).  A shard without
// valid queries (L <= row0) reads nothing; the wrap halo is read only by
// valid queries among the last s rows.
void shard_halo(int N, int row0, int T, int G, int shift, int boundary,
                int L, int &left0, int &hl, int &hw) {
  const int s = (N / G == 1) ? 0 : shift;
  left0 = row0;
  hl = 0;
  hw = 0;
  if (s == 0 || L <= row0) return;
  if (row0 > 0) {
    left0 = row0 - s;
    hl = s;
  } else if (boundary == S2A_WRAP) {
    left0 = N - s;
    hl = L - left0 < 0 ? 0 : (L - left0 > s ? s : L - left0);
  }
  if (boundary == S2A_CYCLIC && row0 + T == N && L > N - s) hw = s;
}

S2AGeom make_shard_geom(int N, int row0, int T, int G, int shift,
                        int boundary, int L) {
  S2AGeom g;
  g.N = T;
  g.G = G;
  g.M = T / G;
  g.s = (N / G == 1) ? 0 : shift;
  g.boundary = S2A_BOUNDARY_SHARD;
  g.L = L - row0 < T ? L - row0 : T;  // positions are counted from row0
  int left0;
  shard_halo(N, row0, T, G, shift, boundary, L, left0, g.hl, g.hw);
  return g;
}

S2AParams make_params_g(const S2AGeom &g, int B, int H, float scale,
                        int tile_rows, const int *doc) {
  S2AParams p;
  p.doc = doc;
  p.dsws = nullptr;
  p.g = g;
  p.B = B;
  p.H = H;
  p.ngmax = s2a_max_groups(p.g);
  p.tiles = (g.G + tile_rows - 1) / tile_rows;
  p.units = B * H * p.ngmax;
  p.scale = scale;
  p.scale_log2 = scale * S2A_LOG2E;
  return p;
}

S2AParams make_params(int B, int N, int H, int G, int shift, int boundary,
                      int L, float scale, int tile_rows, const int *doc) {
  return make_params_g(make_geom(N, G, shift, boundary, L), B, H, scale,
                       tile_rows, doc);
}

s2a_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return S2A_OK;
  snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
  return S2A_EHIP;
}

// Shared checks of the two gradient stages.
s2a_status check_grad_stage(const void *q, const void *k, const void *v,
                            const float *lse, const float *delta_ws,
                            const void *dout, const void *o1, const void *o2,
                            int B, int N, int H, int D, int G, int shift,
                            int boundary, int valid_len, float scale) {
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!q || !k || !v || !lse || !delta_ws || !dout || !o1 || !o2)
    return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) ||
      !aligned16(delta_ws) || !aligned16(dout) || !aligned16(o1) ||
      !aligned16(o2))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  return S2A_OK;
}

}  // namespace

extern "C" {

s2a_status s2attn_fwd(const void *q, const void *k, const void *v, void *o,
                      int o_dtype, float *lse, int B, int N, int H, int D,
                      int G, int shift, int boundary, int valid_len,
                      const int *doc_ids, float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!aligned4(doc_ids))
    return fail(S2A_EINVAL, "doc_ids must be 4-byte aligned");
  if (!q || !k || !v || !o || !lse)
    return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (o_dtype != S2A_BF16 && o_dtype != S2A_F32)
    return fail(S2A_EINVAL, "o_dtype=%lld is neither BF16 nor F32", o_dtype);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  const S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len,
                                  scale, s2a_fwd_tile_rows(D), doc_ids);
  return hip_status(s2a_launch_fwd(q, k, v, o, o_dtype == S2A_F32, lse, D, p,
                                   (hipStream_t)stream),
                    "forward launch");
}

namespace {

// Everything s2attn_bwd and s2attn_bwd_noalloc check before launching; the
// delta workspace is checked by the caller.
s2a_status check_bwd(const void *q, const void *k, const void *v,
                     const void *o, int o_dtype, const float *lse,
                     const void *dout, float *dq, float *dk, float *dv, int B,
                     int N, int H, int D, int G, int shift, int boundary,
                     int valid_len, const int *doc_ids, float scale) {
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!aligned4(doc_ids))
    return fail(S2A_EINVAL, "doc_ids must be 4-byte aligned");
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (o_dtype != S2A_BF16 && o_dtype != S2A_F32)
    return fail(S2A_EINVAL, "o_dtype=%lld is neither BF16 nor F32", o_dtype);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  return S2A_OK;
}

// The delta workspace of s2attn_bwd_noalloc: a device array of the library
// (one copy per GPU, held until the process ends), never allocated at run
// time.  Host code uses it only through the per-device address that
// hipGetSymbolAddress returns; the name itself is not a device address.
constexpr size_t NOALLOC_DELTA_FLOATS = (size_t)S2A_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[NOALLOC_DELTA_FLOATS];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
float *g_scratch[MAX_DEVICES];  // address of scratch on each device

// Address of scratch on the current device, looked up on the first call on
// that device (with it current) and kept.
s2a_status scratch_of_current_device(float **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(g_err, sizeof g_err, "hipGetDevice: %s", hipGetErrorString(e));
    return S2A_EHIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(S2A_EUNSUPPORTED, "device %lld: at most %lld devices", dev,
                MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      snprintf(g_err, sizeof g_err, "hipGetSymbolAddress(scratch): %s",
               hipGetErrorString(e));
      return S2A_EHIP;
    }
    g_scratch[dev] = (float *)ptr;
  }
  *out = g_scratch[dev];
  return S2A_OK;
}

}  // namespace

s2a_status s2attn_bwd(const void *q, const void *k, const void *v,
                      const void *o, int o_dtype, const float *lse,
                      const void *dout, float *dq, float *dk, float *dv,
                      float *delta_ws, int B, int N, int H, int D, int G,
                      int shift, int boundary, int valid_len,
                      const int *doc_ids, float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_bwd(q, k, v, o, o_dtype, lse, dout, dq, dk, dv, B, N,
                            H, D, G, shift, boundary, valid_len, doc_ids,
                            scale);
  if (st != S2A_OK) return st;
  if (!delta_ws) return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(delta_ws))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  const S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len,
                                  scale, 1, doc_ids);
  return hip_status(s2a_launch_bwd(q, k, v, o, o_dtype == S2A_F32, lse, dout,
                                   dq, dk, dv, delta_ws, D, p,
                                   (hipStream_t)stream),
                    "backward launch");
}

s2a_status s2attn_bwd_noalloc(const void *q, const void *k, const void *v,
                              const void *o, int o_dtype, const float *lse,
                              const void *dout, float *dq, float *dk,
                              float *dv, int B, int N, int H, int D, int G,
                              int shift, int boundary, int valid_len,
                              const int *doc_ids, float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_bwd(q, k, v, o, o_dtype, lse, dout, dq, dk, dv, B, N,
                            H, D, G, shift, boundary, valid_len, doc_ids,
                            scale);
  if (st != S2A_OK) return st;
  const long long rows = (long long)B * H * N;
  if (rows > (long long)NOALLOC_DELTA_FLOATS)
    return fail(S2A_EINVAL,
                "B*H*N=%lld rows exceed the %lld of the no-allocation "
                "workspace (use s2attn_bwd with a workspace)",
                rows, (long long)NOALLOC_DELTA_FLOATS);
  float *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != S2A_OK) return st;
  // The preprocess kernel writes all B*H*N entries of delta before the
  // gradient kernels read any, so nothing needs clearing.
  const S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len,
                                  scale, 1, doc_ids);
  return hip_status(s2a_launch_bwd(q, k, v, o, o_dtype == S2A_F32, lse, dout,
                                   dq, dk, dv, ws, D, p, (hipStream_t)stream),
                    "backward launch");
}

s2a_status s2attn_bwd_preprocess(const void *o, int o_dtype,
                                 const void *dout, float *delta_ws, int B,
                                 int N, int H, int D, void *stream) {
  g_err[0] = 0;
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0)
    return fail(S2A_EINVAL, "sizes must be positive");
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(S2A_EUNSUPPORTED, "head width D=%lld not in {16,32,64,128}", D);
  if (!o || !dout || !delta_ws) return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta_ws))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (o_dtype != S2A_BF16 && o_dtype != S2A_F32)
    return fail(S2A_EINVAL, "o_dtype=%lld is neither BF16 nor F32", o_dtype);
  return hip_status(s2a_launch_bwd_pre(o, o_dtype == S2A_F32, dout, delta_ws,
                                       B, N, H, D, (hipStream_t)stream),
                    "backward preprocess launch");
}

s2a_status s2attn_bwd_dkdv(const void *q, const void *k, const void *v,
                           const float *lse, const float *delta_ws,
                           const void *dout, float *dk, float *dv, int B,
                           int N, int H, int D, int G, int shift,
                           int boundary, int valid_len, const int *doc_ids,
                           float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_grad_stage(q, k, v, lse, delta_ws, dout, dk, dv, B, N,
                                   H, D, G, shift, boundary, valid_len, scale);
  if (st != S2A_OK) return st;
  if (!aligned4(doc_ids))
    return fail(S2A_EINVAL, "doc_ids must be 4-byte aligned");
  const S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len,
                                  scale, 1, doc_ids);
  return hip_status(s2a_launch_bwd_dkdv(q, k, v, dout, lse, delta_ws, dk, dv,
                                        D, p, (hipStream_t)stream),
                    "dK/dV launch");
}

s2a_status s2attn_bwd_dq(const void *q, const void *k, const void *v,
                         const float *lse, const float *delta_ws,
                         const void *dout, float *dq, int B, int N, int H,
                         int D, int G, int shift, int boundary,
                         int valid_len, const int *doc_ids, float scale,
                         void *stream) {
  g_err[0] = 0;
  s2a_status st = check_grad_stage(q, k, v, lse, delta_ws, dout, dq, dq, B, N,
                                   H, D, G, shift, boundary, valid_len, scale);
  if (st != S2A_OK) return st;
  if (!aligned4(doc_ids))
    return fail(S2A_EINVAL, "doc_ids must be 4-byte aligned");
  const S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len,
                                  scale, 1, doc_ids);
  return hip_status(s2a_launch_bwd_dq(q, k, v, dout, lse, delta_ws, dq, D, p,
                                      (hipStream_t)stream),
                    "dQ launch");
}

}  // extern "C"

namespace {

// Checks of the stored-dS variant: D in {64, 128}, a workspace of at least
// s2attn_bwd_ds_workspace bytes, 16-byte aligned.  Sets p.dsws.
s2a_status check_ds(int D, void *ds_ws, size_t ds_ws_bytes, S2AParams &p) {
  if (D != 64 && D != 128)
    return fail(S2A_EUNSUPPORTED,
                "the stored-dS backward needs D in {64,128}, not %lld", D);
  const long double need = s2a_ds_workspace_bytes(p);
  if (need > 4.0e18L)
    return fail(S2A_EINVAL, "dS workspace too large for one launch");
  if (!ds_ws) return fail(S2A_EINVAL, "NULL dS workspace");
  if (!aligned16(ds_ws))
    return fail(S2A_EINVAL, "dS workspace must be 16-byte aligned");
  if ((long double)ds_ws_bytes < need)
    return fail(S2A_EINVAL, "dS workspace of %lld bytes, %lld needed",
                (long long)ds_ws_bytes, (long long)need);
  p.dsws = ds_ws;
  return S2A_OK;
}

}  // namespace

extern "C" {

s2a_status s2attn_bwd_ds_workspace(int B, int N, int H, int D, int G,
                                   int shift, int boundary, size_t *bytes) {
  g_err[0] = 0;
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, N);
  if (st != S2A_OK) return st;
  if (!bytes) return fail(S2A_EINVAL, "NULL result pointer");
  if (D != 64 && D != 128)
    return fail(S2A_EUNSUPPORTED,
                "the stored-dS backward needs D in {64,128}, not %lld", D);
  const S2AParams p = make_params(B, N, H, G, shift, boundary, N, 1.f, 1,
                                  nullptr);
  const long double need = s2a_ds_workspace_bytes(p);
  if (need > 4.0e18L)
    return fail(S2A_EINVAL, "dS workspace too large for one launch");
  *bytes = (size_t)need;
  return S2A_OK;
}

s2a_status s2attn_bwd_ds(const void *q, const void *k, const void *v,
                         const void *o, int o_dtype, const float *lse,
                         const void *dout, float *dq, float *dk, float *dv,
                         float *delta_ws, void *ds_ws, size_t ds_ws_bytes,
                         int B, int N, int H, int D, int G, int shift,
                         int boundary, int valid_len, float scale,
                         void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta_ws)
    return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(delta_ws))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (o_dtype != S2A_BF16 && o_dtype != S2A_F32)
    return fail(S2A_EINVAL, "o_dtype=%lld is neither BF16 nor F32", o_dtype);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len, scale, 1,
                            nullptr);
  st = check_ds(D, ds_ws, ds_ws_bytes, p);
  if (st != S2A_OK) return st;
  return hip_status(s2a_launch_bwd(q, k, v, o, o_dtype == S2A_F32, lse, dout,
                                   dq, dk, dv, delta_ws, D, p,
                                   (hipStream_t)stream),
                    "backward launch");
}

s2a_status s2attn_bwd_dkdv_ds(const void *q, const void *k, const void *v,
                              const float *lse, const float *delta_ws,
                              const void *dout, float *dk, float *dv,
                              void *ds_ws, size_t ds_ws_bytes, int B, int N,
                              int H, int D, int G, int shift, int boundary,
                              int valid_len, float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_grad_stage(q, k, v, lse, delta_ws, dout, dk, dv, B, N,
                                   H, D, G, shift, boundary, valid_len, scale);
  if (st != S2A_OK) return st;
  S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len, scale, 1,
                            nullptr);
  st = check_ds(D, ds_ws, ds_ws_bytes, p);
  if (st != S2A_OK) return st;
  return hip_status(s2a_launch_bwd_dkdv(q, k, v, dout, lse, delta_ws, dk, dv,
                                        D, p, (hipStream_t)stream),
                    "dK/dV launch");
}

s2a_status s2attn_bwd_dq_ds(const void *k, const void *ds_ws,
                            size_t ds_ws_bytes, float *dq, int B, int N, int H,
                            int D, int G, int shift, int boundary,
                            int valid_len, float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shape(B, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!k || !dq) return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(k) || !aligned16(dq))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  S2AParams p = make_params(B, N, H, G, shift, boundary, valid_len, scale, 1,
                            nullptr);
  st = check_ds(D, const_cast<void *>(ds_ws), ds_ws_bytes, p);
  if (st != S2A_OK) return st;
  return hip_status(s2a_launch_bwd_dq(nullptr, k, nullptr, nullptr, nullptr,
                                      nullptr, dq, D, p, (hipStream_t)stream),
                    "dQ launch");
}

namespace {

// Shape checks of a shard: those of the whole sequence (one batch row),
// and a slice [row0, row0 + T) of whole groups inside it.
s2a_status check_shard(int N, int row0, int T, int H, int D, int G,
                       int shift, int boundary, int valid_len) {
  s2a_status st = check_shape(1, N, H, D, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (row0 < 0 || T <= 0 || row0 % G || T % G)
    return fail(S2A_EINVAL, "row0=%lld and T=%lld must be multiples of G, "
                "T > 0", row0, T);
  if ((long long)row0 + T > N)
    return fail(S2A_EINVAL, "row0 + T = %lld exceeds N=%lld",
                (long long)row0 + T, N);
  return S2A_OK;
}

s2a_status check_ptrs(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (!p) return fail(S2A_EINVAL, "NULL tensor pointer");
  for (const void *p : ps)
    if (!aligned16(p))
      return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  return S2A_OK;
}

s2a_status check_common(const int *doc_ids, int o_dtype, float scale) {
  if (!aligned4(doc_ids))
    return fail(S2A_EINVAL, "doc_ids must be 4-byte aligned");
  if (o_dtype != S2A_BF16 && o_dtype != S2A_F32)
    return fail(S2A_EINVAL, "o_dtype=%lld is neither BF16 nor F32", o_dtype);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(S2A_EINVAL, "scale must be positive and finite");
  return S2A_OK;
}

}  // namespace

s2a_status s2attn_shard_halo(int N, int row0, int T, int G, int shift,
                             int boundary, int valid_len, int *left_first,
                             int *left_rows, int *wrap_rows) {
  g_err[0] = 0;
  s2a_status st = check_shard(N, row0, T, 2, 16, G, shift, boundary,
                              valid_len);
  if (st != S2A_OK) return st;
  if (!left_first || !left_rows || !wrap_rows)
    return fail(S2A_EINVAL, "NULL output pointer");
  shard_halo(N, row0, T, G, shift, boundary, valid_len, *left_first,
             *left_rows, *wrap_rows);
  return S2A_OK;
}

s2a_status s2attn_fwd_shard(const void *q, const void *k, const void *v,
                            void *o, int o_dtype, float *lse, int N, int row0,
                            int T, int H, int D, int G, int shift,
                            int boundary, int valid_len, const int *doc_ids,
                            float scale, void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shard(N, row0, T, H, D, G, shift, boundary,
                              valid_len);
  if (st == S2A_OK) st = check_ptrs({q, k, v, o, lse});
  if (st == S2A_OK) st = check_common(doc_ids, o_dtype, scale);
  if (st != S2A_OK) return st;
  const S2AGeom g = make_shard_geom(N, row0, T, G, shift, boundary,
                                    valid_len);
  const S2AParams p = make_params_g(g, 1, H, scale, s2a_fwd_tile_rows(D),
                                    doc_ids);
  return hip_status(s2a_launch_fwd(q, k, v, o, o_dtype == S2A_F32, lse, D, p,
                                   (hipStream_t)stream),
                    "shard forward launch");
}

s2a_status s2attn_bwd_shard(const void *q, const void *k, const void *v,
                            const void *o, int o_dtype, const float *lse,
                            const void *dout, float *dq, float *dk, float *dv,
                            float *delta_ws, int N, int row0, int T, int H,
                            int D, int G, int shift, int boundary,
                            int valid_len, const int *doc_ids, float scale,
                            void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shard(N, row0, T, H, D, G, shift, boundary,
                              valid_len);
  if (st == S2A_OK)
    st = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv, delta_ws});
  if (st == S2A_OK) st = check_common(doc_ids, o_dtype, scale);
  if (st != S2A_OK) return st;
  const S2AGeom g = make_shard_geom(N, row0, T, G, shift, boundary,
                                    valid_len);
  const S2AParams p = make_params_g(g, 1, H, scale, 1, doc_ids);
  return hip_status(s2a_launch_bwd(q, k, v, o, o_dtype == S2A_F32, lse, dout,
                                   dq, dk, dv, delta_ws, D, p,
                                   (hipStream_t)stream),
                    "shard backward launch");
}

namespace {

s2a_status rope_common(const void *x, void *y, int B, int N, int H, int D,
                       const int *pos_ids, float base, float pos_scale,
                       int pairing) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0)
    return fail(S2A_EINVAL, "sizes must be positive");
  if (D != 16 && D != 32 && D != 64 && D != 128)
    return fail(S2A_EUNSUPPORTED, "head width D=%lld not in {16,32,64,128}", D);
  if ((long long)B * N > (1ll << 31))
    return fail(S2A_EINVAL, "B*N=%lld too large for one launch",
                (long long)B * N);
  if (!x || !y) return fail(S2A_EINVAL, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(y))
    return fail(S2A_EINVAL, "tensor pointers must be 16-byte aligned");
  if (!aligned4(pos_ids))
    return fail(S2A_EINVAL, "pos_ids must be 4-byte aligned");
  if (!(base > 0.f) || !isfinite(base))
    return fail(S2A_EINVAL, "base must be positive and finite");
  if (!(pos_scale > 0.f) || !isfinite(pos_scale))
    return fail(S2A_EINVAL, "pos_scale must be positive and finite");
  if (pairing != S2A_ROPE_HALF && pairing != S2A_ROPE_INTERLEAVED)
    return fail(S2A_EINVAL, "pairing=%lld is neither HALF nor INTERLEAVED",
                pairing);
  return S2A_OK;
}

}  // namespace

s2a_status s2attn_rope(const void *x, void *y, int B, int N, int H, int D,
                       const int *pos_ids, float base, float pos_scale,
                       int pairing, void *stream) {
  g_err[0] = 0;
  s2a_status st = rope_common(x, y, B, N, H, D, pos_ids, base, pos_scale,
                              pairing);
  if (st != S2A_OK) return st;
  return hip_status(s2a_launch_rope(x, y, false, false, B, N, H, D, pos_ids,
                                    base, pos_scale,
                                    pairing == S2A_ROPE_HALF,
                                    (hipStream_t)stream),
                    "rope launch");
}

s2a_status s2attn_rope_bwd(const float *gy, float *gx, int B, int N, int H,
                           int D, const int *pos_ids, float base,
                           float pos_scale, int pairing, void *stream) {
  g_err[0] = 0;
  s2a_status st = rope_common(gy, gx, B, N, H, D, pos_ids, base, pos_scale,
                              pairing);
  if (st != S2A_OK) return st;
  return hip_status(s2a_launch_rope(gy, gx, true, true, B, N, H, D, pos_ids,
                                    base, pos_scale,
                                    pairing == S2A_ROPE_HALF,
                                    (hipStream_t)stream),
                    "rope backward launch");
}

s2a_status s2attn_group_map(int N, int G, int shift, int boundary,
                            int valid_len, int *gid, int *slot, int *src,
                            void *stream) {
  g_err[0] = 0;
  s2a_status st = check_shape(1, N, 2, 16, G, shift, boundary, valid_len);
  if (st != S2A_OK) return st;
  if (!gid || !slot || !src) return fail(S2A_EINVAL, "NULL map pointer");
  if (!aligned16(gid) || !aligned16(slot) || !aligned16(src))
    return fail(S2A_EINVAL, "map pointers must be 16-byte aligned");
  const S2AGeom g = make_geom(N, G, shift, boundary, valid_len);
  return hip_status(s2a_launch_map(g, gid, slot, src, (hipStream_t)stream),
                    "group map launch");
}

const char *s2attn_strerror(int status) {
  switch (status) {
    case S2A_OK: return "ok";
    case S2A_EINVAL: return "invalid argument";
    case S2A_EUNSUPPORTED: return "unsupported head width";
    case S2A_EHIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char *s2attn_last_error(void) { return g_err; }

const char *s2attn_version(void) { return "s2attn 0.1.0 gfx950"; }

}  // extern "C"
