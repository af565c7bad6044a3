// Group geometry of shifted sparse attention, shared by every kernel of the
// library and by its host-side launch code.
//
// A head of class 0 groups the original positions as [kG, (k+1)G).  A head
// of class 1 (the second half of the heads) groups them after a shift of
// s = G/2 (PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调", §1: the
// group functions b(i) = floor(i/G) and b'(i) = floor((i - G/2)/G), and the
// cyclic-shift paragraph for the two boundary variants).
//
// Every group is described by (base, len): its slot j (0 <= j < len) holds
// the original position base + j, reduced mod N.  The reduction only
// matters for the wrapped group of the WRAP variant, whose slots run over
// N-s .. N-1 and then 0 .. s-1; everywhere else base + j < N.  The kernels
// never build a rolled copy of Q/K/V: a row's address is computed from its
// slot with slot_pos().
#pragma once

#ifndef __HIPCC__
#define __host__
#define __device__
#endif

#define S2A_BOUNDARY_WRAP 0
#define S2A_BOUNDARY_SPLIT 1

struct S2AGeom {
  int N;         // padded length
  int G;         // group length
  int s;         // effective shift (0 if shift == 0 or N == G)
  int M;         // N / G
  int boundary;  // S2A_BOUNDARY_WRAP or S2A_BOUNDARY_SPLIT
  int L;         // valid length
};

// Number of groups of head class cls.
__host__ __device__ inline int s2a_num_groups(const S2AGeom &g, int cls) {
  return (cls == 1 && g.s > 0 && g.boundary == S2A_BOUNDARY_SPLIT) ? g.M + 1
                                                                     : g.M;
}

// Groups of a class laid end to end; the largest count over both classes.
__host__ __device__ inline int s2a_max_groups(const S2AGeom &g) {
  return s2a_num_groups(g, 1);
}

// (base, len) of group gi of class cls; returns false if gi is past the
// last group of that class.
__host__ __device__ inline bool s2a_group(const S2AGeom &g, int cls, int gi,
                                          int &base, int &len) {
  if (gi < 0 || gi >= s2a_num_groups(g, cls)) return false;
  if (cls == 0 || g.s == 0) {
    base = gi * g.G;
    len = g.G;
  } else if (g.boundary == S2A_BOUNDARY_WRAP) {
    base = gi * g.G + g.s;  // rolled left by s: slot j of group gi holds
    len = g.G;              // position (gi*G + s + j) mod N
  } else {
    base = gi == 0 ? 0 : g.s + (gi - 1) * g.G;
    len = (gi == 0 || gi == g.M) ? g.s : g.G;
  }
  return true;
}

// Original position of slot j of a group with the given base.
__host__ __device__ inline int s2a_slot_pos(int base, int j, int N) {
  int p = base + j;
  return p >= N ? p - N : p;
}

// Inverse map: group and slot of original position x in class cls.
__host__ __device__ inline void s2a_locate(const S2AGeom &g, int cls, int x,
                                           int &gi, int &slot) {
  if (cls == 0 || g.s == 0) {
    gi = x / g.G;
    slot = x - gi * g.G;
  } else if (g.boundary == S2A_BOUNDARY_WRAP) {
    int p = x - g.s;
    if (p < 0) p += g.N;
    gi = p / g.G;
    slot = p - gi * g.G;
  } else if (x < g.s) {
    gi = 0;
    slot = x;
  } else {
    gi = (x - g.s) / g.G + 1;
    slot = x - (g.s + (gi - 1) * g.G);
  }
}

// Row r of the regrouped layout (the groups of a class laid end to end in
// group order): its group gi and slot j.  For the WRAP variant the rows are
// the rolled layout; for SPLIT and for class 0 they are the original order.
__host__ __device__ inline void s2a_row_locate(const S2AGeom &g, int cls,
                                               int r, int &gi, int &j) {
  if (cls == 1 && g.s > 0 && g.boundary == S2A_BOUNDARY_SPLIT) {
    if (r < g.s) {
      gi = 0;
      j = r;
    } else {
      gi = (r - g.s) / g.G + 1;
      j = r - (g.s + (gi - 1) * g.G);
    }
  } else {
    gi = r / g.G;
    j = r - gi * g.G;
  }
}
