// Device-side vector types and CDNA4 (gfx950) helpers used by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "s2a_geom.h"

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define S2A_LOG2E 1.4426950408889634f
#define S2A_LN2 0.6931471805599453f

// Launch parameters shared by the attention kernels.
struct S2AParams {
  S2AGeom g;
  int B, H;
  int ngmax;      // groups per head, laid out for both classes
  int tiles;      // row tiles per group (query tiles fwd, key tiles bwd)
  int units;      // B * H * ngmax; unit gi * (B*H) + (b*H + h)
  float scale;    // softmax scale
  float scale_log2;  // scale * log2(e)
  const int *doc; // document IDs [B, N] (nullptr: no document mask)
  // dS workspace of the backward (nullptr: the dQ kernel recomputes S and
  // dP; otherwise dK/dV stores bf16 dS blocks there and dQ reads them)
  void *dsws;
};

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (checked on
// gfx950): lane l holds A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32];
// accumulator element i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b,
                                         const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulate-only form of mfma32 whose accumulator stays in AGPRs (the
// compiler otherwise shuffles long-lived accumulators between register
// files under pressure).  The leading s_nop covers the wait states a VALU
// write of a or b needs before an MFMA reads it.  Back-to-back chaining on
// the same accumulator needs none; before the accumulator is read by
// anything but this form, call mfma_agpr_drain().
__device__ __forceinline__ void mfma32_agpr(f32x16 &acc, const bf16x8 &a,
                                            const bf16x8 &b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
      : "+a"(acc)
      : "v"(a), "v"(b));
}

// Wait states between the last mfma32_agpr and a read of its accumulator
// (a 16-pass MFMA needs 18).
__device__ __forceinline__ void mfma_agpr_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// LDS transposing read: within each group of 16 lanes, lanes 4r..4r+3 each
// name 4 consecutive 16-bit elements that together form row r (r = 0..3);
// lane i of the group receives column i of those four rows.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16_t *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4 &lo, const bf16x4 &hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2,
                                            float a3, float a4, float a5,
                                            float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2,
                                            float a3) {
  f32x4 f = {a0, a1, a2, a3};
  return __builtin_convertvector(f, bf16x4);
}

// max / sum of x over lanes l and l^32, with v_permlane32_swap (a VALU
// cross-half swap: both registers start as x; afterwards lane l holds x of
// lanes l and l^32 between them).  Written as asm because the builtin's
// second result is not returned correctly by this compiler.
__device__ __forceinline__ float wave_max_x32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
// Minimum and maximum of an int over the 64 lanes of a wave, returned
// wave-uniform.
__device__ __forceinline__ void wave_minmax(int &mn, int &mx) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, __shfl_xor(mn, o, 64));
    mx = max(mx, __shfl_xor(mx, o, 64));
  }
  mn = __builtin_amdgcn_readfirstlane(mn);
  mx = __builtin_amdgcn_readfirstlane(mx);
}

__device__ __forceinline__ float wave_sum_x32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

