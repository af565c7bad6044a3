// Rotary position embedding at global positions, the prologue of the path.
//
// For one pair of channels RoPE at position m applies the plane rotation
// R(m, w) = [[cos mw, -sin mw], [sin mw, cos mw]] (PaperTrace "4.1.2 ·
// LongLoRA: 用S²-Attn完成长上下文微调", §3.1).  The position is the token's
// original (global) position ID, never its offset inside a group, and
// linear position interpolation maps p to p * L0/L1 before the angle is
// formed (§1.1, the paragraphs on RoPE and position interpolation).  Pair i
// of a head of width D turns at w_i = base^(-2i/D); it is channels
// (i, i + D/2) ("half" pairing) or (2i, 2i + 1) ("interleaved").
//
// One workgroup per token (b, n): the D/2 angles are formed once, in double
// precision (m * w reaches 1e5 rad, where a float product would already be
// off by up to 4e-3 rad), and every head of the token is rotated with them.
// The kernel streams the tensor once (HBM bound): per token it reads and
// writes H*D elements.  The forward map rounds once to bf16; the inverse map
// (R^T, the gradient of the rotation) runs on fp32 gradients.
#include "s2a_device.h"
#include "s2a_kernels.h"

namespace {

constexpr int ROPE_THREADS = 256;

// 8 pairs of one head per work item.
template <int D, bool F32>
struct RopeIO;

template <int D>
struct RopeIO<D, false> {  // bf16
  static __device__ void load8(const void *p, size_t off, float (&x)[8]) {
    const bf16x8 v = __builtin_bit_cast(
        bf16x8, *(const u32x4 *)((const bf16_t *)p + off));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  }
  static __device__ void store8(void *p, size_t off, const float (&x)[8]) {
    *(bf16x8 *)((bf16_t *)p + off) =
        to_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
  }
};

template <int D>
struct RopeIO<D, true> {  // fp32
  static __device__ void load8(const void *p, size_t off, float (&x)[8]) {
    const f32x4 a = *(const f32x4 *)((const float *)p + off);
    const f32x4 b = *(const f32x4 *)((const float *)p + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[e + 4] = b[e];
    }
  }
  static __device__ void store8(void *p, size_t off, const float (&x)[8]) {
    const f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
    *(f32x4 *)((float *)p + off) = a;
    *(f32x4 *)((float *)p + off + 4) = b;
  }
};

template <int D, bool F32, bool HALFPAIR, bool INV>
__global__ __launch_bounds__(ROPE_THREADS) void s2a_rope_kernel(
    const void *x, void *y, int N, int H, const int *__restrict__ pos,
    double base, double pscale) {
  // (x and y may be the same buffer: every element is read and written by
  // one thread, read first)
  static_assert(D % 16 == 0, "8 pairs per work item");
  using IO = RopeIO<D, F32>;
  __shared__ float cs[D / 2], sn[D / 2];
  const int row = blockIdx.x;  // b * N + n
  const int tid = threadIdx.x;
  if (tid < D / 2) {
    const double m = (double)(pos ? pos[row] : row % N) * pscale;
    const double w = pow(base, -2.0 * tid / D);
    double s, c;
    sincos(m * w, &s, &c);
    cs[tid] = (float)c;
    sn[tid] = INV ? -(float)s : (float)s;
  }
  __syncthreads();

  constexpr int IPH = D / 16;  // items per head
  const int items = H * IPH;
  const size_t rbase = (size_t)row * H * D;
  for (int j = tid; j < items; j += ROPE_THREADS) {
    const int h = j / IPH, c = j - h * IPH;
    const size_t hb = rbase + (size_t)h * D;
    float a[8], b[8];  // first and second channel of pairs 8c .. 8c+7
    if (HALFPAIR) {
      IO::load8(x, hb + 8 * c, a);
      IO::load8(x, hb + D / 2 + 8 * c, b);
    } else {
      float u[8], v[8];
      IO::load8(x, hb + 16 * c, u);
      IO::load8(x, hb + 16 * c + 8, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = u[2 * e];
        b[e] = u[2 * e + 1];
        a[e + 4] = v[2 * e];
        b[e + 4] = v[2 * e + 1];
      }
    }
    float ya[8], yb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float co = cs[8 * c + e], si = sn[8 * c + e];
      ya[e] = fmaf(co, a[e], -si * b[e]);
      yb[e] = fmaf(si, a[e], co * b[e]);
    }
    if (HALFPAIR) {
      IO::store8(y, hb + 8 * c, ya);
      IO::store8(y, hb + D / 2 + 8 * c, yb);
    } else {
      float u[8], v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[2 * e] = ya[e];
        u[2 * e + 1] = yb[e];
        v[2 * e] = ya[e + 4];
        v[2 * e + 1] = yb[e + 4];
      }
      IO::store8(y, hb + 16 * c, u);
      IO::store8(y, hb + 16 * c + 8, v);
    }
  }
}

template <int D, bool F32>
hipError_t launch_rope_t(const void *x, void *y, bool inverse, int B, int N,
                         int H, const int *pos, float base, float pscale,
                         bool half, hipStream_t st) {
  double b = base, ps = pscale;
  void *args[] = {(void *)&x, (void *)&y,  (void *)&N, (void *)&H,
                  (void *)&pos, (void *)&b, (void *)&ps};
  const void *fn;
  if (half)
    fn = inverse ? (const void *)s2a_rope_kernel<D, F32, true, true>
                 : (const void *)s2a_rope_kernel<D, F32, true, false>;
  else
    fn = inverse ? (const void *)s2a_rope_kernel<D, F32, false, true>
                 : (const void *)s2a_rope_kernel<D, F32, false, false>;
  return hipLaunchKernel(fn, dim3((unsigned)B * (unsigned)N),
                         dim3(ROPE_THREADS), args, 0, st);
}

}  // namespace

hipError_t s2a_launch_rope(const void *x, void *y, bool f32, bool inverse,
                           int B, int N, int H, int D, const int *pos,
                           float base, float pscale, bool half,
                           hipStream_t st) {
  switch (D) {
#define S2A_CASE(DD)                                                        \
  case DD:                                                                  \
    return f32 ? launch_rope_t<DD, true>(x, y, inverse, B, N, H, pos, base, \
                                         pscale, half, st)                  \
               : launch_rope_t<DD, false>(x, y, inverse, B, N, H, pos, base,\
                                          pscale, half, st);
    S2A_CASE(16)
    S2A_CASE(32)
    S2A_CASE(64)
    S2A_CASE(128)
#undef S2A_CASE
    default: return hipErrorInvalidValue;
  }
}
