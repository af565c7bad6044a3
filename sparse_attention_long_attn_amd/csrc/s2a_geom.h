// Group geometry of shifted sparse attention, shared by every kernel of the
// library and by its host-side launch code.
//
// A head of class 0 groups the original positions as [kG, (k+1)G).  A head
// of class 1 (the second half of the heads) groups them after a shift of
// s = G/2 (PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调", §1: the
// group functions b(i) = floor(i/G) and b'(i) = floor((i - G/2)/G), and the
// cyclic-shift paragraph for the two boundary variants; §2.2 for the third).
// The boundary variant decides the shifted class's groups and their order:
//   WRAP    the original roll: groups [s + kG, s + (k+1)G) mod N; the last
//           one holds N-s .. N-1 and then 0 .. s-1, in that order (the
//           causal triangle is taken in this rolled order);
//   SPLIT   strict causal: [0, s), [s + kG, s + (k+1)G), [N-s, N);
//   CYCLIC  the cyclic partition of WRAP with causality on original
//           positions (§2.2's teaching graph): the last group is ordered
//           0 .. s-1, then N-s .. N-1, so its tail reads its head.
//
// A group is a run of slots j = 0 .. len-1 (S2ARun) whose original
// positions form at most two increasing runs: slot j holds
// base + j - (j >= cut ? jump : 0).  The kernels never build a rolled copy
// of Q/K/V: a row's address is computed from its slot with pos().
//
// A shard (sequence parallelism, PaperTrace LongLoRA §1.1, the paragraphs
// on distributed boundaries) is the slice [row0, row0 + T) of the rows,
// with row0 and T multiples of G, so that only the shifted class has
// groups that cross its edges.  Its geometry (S2A_BOUNDARY_SHARD) numbers
// positions from row0: the slice holds 0 .. T-1, and the rows it reads
// from other slices sit at negative positions, in front of row 0 of the
// same buffers:
//   left halo  -hl .. -1    the hl rows that precede the slice in the
//                            shifted class's group order (rows row0-s ..
//                            row0-1, or the valid part of N-s .. N-1 for
//                            the first slice under WRAP);
//   wrap halo  -2s .. -s-1  rows 0 .. s-1 (the last slice under CYCLIC,
//                            whose last group starts with them).
// Its groups: class 0 [kG, (k+1)G); class 1 first {left halo, 0 .. s-1},
// then [kG - s, (k+1)G - s), and last {wrap halo if any, T-s .. T-1}.
// Halo rows are keys only: a query counts when its position is >= 0,
// which every position of the unsharded geometries is.
#pragma once

#ifndef __HIPCC__
#define __host__
#define __device__
#endif

#define S2A_BOUNDARY_WRAP 0
#define S2A_BOUNDARY_SPLIT 1
#define S2A_BOUNDARY_CYCLIC 2
#define S2A_BOUNDARY_SHARD 3  // internal: one slice of the rows (see above)

struct S2AGeom {
  int N;         // padded length (a shard: its row count T)
  int G;         // group length
  int s;         // effective shift (0 if shift == 0 or N == G)
  int M;         // N / G
  int boundary;  // S2A_BOUNDARY_WRAP, _SPLIT, _CYCLIC or _SHARD
  int L;         // valid length (a shard: positions below L are valid;
                 // it may be <= 0 or, for halo rows, cover negatives)
  int hl;        // shard: rows of the left halo (0 .. s)
  int hw;        // shard: rows of the wrap halo (0 or s)
};

// Slot -> original position of one group (see the file comment).
struct S2ARun {
  int base;  // position of slot 0
  int cut;   // first slot of the second run (len if there is none)
  int jump;  // subtracted from base + j from slot cut on
  __host__ __device__ int pos(int j) const {
    return base + j - (j >= cut ? jump : 0);
  }
};

// Number of groups of head class cls.
__host__ __device__ inline int s2a_num_groups(const S2AGeom &g, int cls) {
  return (cls == 1 && g.s > 0 && (g.boundary == S2A_BOUNDARY_SPLIT ||
                                  g.boundary == S2A_BOUNDARY_SHARD))
             ? g.M + 1
             : g.M;
}

// Groups of a class laid end to end; the largest count over both classes.
__host__ __device__ inline int s2a_max_groups(const S2AGeom &g) {
  return s2a_num_groups(g, 1);
}

// Run and length of group gi of class cls; returns false if gi is past the
// last group of that class.
__host__ __device__ inline bool s2a_group(const S2AGeom &g, int cls, int gi,
                                          S2ARun &run, int &len) {
  if (gi < 0 || gi >= s2a_num_groups(g, cls)) return false;
  if (cls == 0 || g.s == 0) {
    run = {gi * g.G, g.G, 0};
    len = g.G;
  } else if (g.boundary == S2A_BOUNDARY_SHARD) {
    if (gi == 0) {  // left halo, then 0 .. s-1
      len = g.hl + g.s;
      run = {-g.hl, len, 0};
    } else if (gi < g.M) {
      run = {gi * g.G - g.s, g.G, 0};
      len = g.G;
    } else if (g.hw > 0) {  // wrap halo (-2s .. -s-1), then T-s .. T-1
      len = g.hw + g.s;
      run = {-2 * g.s, g.hw, -g.N - g.s + g.hw};
    } else {  // T-s .. T-1 (the rest of the group is on the next slice)
      run = {g.N - g.s, g.s, 0};
      len = g.s;
    }
  } else if (g.boundary == S2A_BOUNDARY_SPLIT) {
    const int base = gi == 0 ? 0 : g.s + (gi - 1) * g.G;
    len = (gi == 0 || gi == g.M) ? g.s : g.G;
    run = {base, len, 0};
  } else if (gi < g.M - 1) {  // WRAP and CYCLIC agree away from the wrap
    run = {gi * g.G + g.s, g.G, 0};
    len = g.G;
  } else if (g.boundary == S2A_BOUNDARY_WRAP) {
    run = {g.N - g.s, g.s, g.N};  // N-s .. N-1, then 0 .. s-1
    len = g.G;
  } else {
    run = {0, g.s, 2 * g.s - g.N};  // 0 .. s-1, then N-s .. N-1
    len = g.G;
  }
  return true;
}

// First slot of a group whose position is >= 0 (holds a query of the
// slice); 0 outside shards.  Used to skip query tiles of halo rows.
__host__ __device__ inline int s2a_first_query_slot(const S2ARun &run,
                                                    int len) {
  if (run.base >= 0) return 0;
  if (run.base + run.cut > 0) return -run.base;  // inside the first run
  return run.cut < len ? run.cut : len;
}

// True if a slot of [j0, j1) (j0 < j1) holds a position >= L.  The largest
// position of the range is the last slot of one of its runs.
__host__ __device__ inline bool s2a_range_has_padding(const S2ARun &run,
                                                      int j0, int j1, int N,
                                                      int L) {
  if (L >= N) return false;
  int mx = run.pos(j1 - 1);
  if (j0 < run.cut && j1 > run.cut) {
    const int m1 = run.pos(run.cut - 1);
    mx = m1 > mx ? m1 : mx;
  }
  return mx >= L;
}

// Inverse map: group and slot of original position x in class cls.
__host__ __device__ inline void s2a_locate(const S2AGeom &g, int cls, int x,
                                           int &gi, int &slot) {
  if (cls == 0 || g.s == 0) {
    gi = x / g.G;
    slot = x - gi * g.G;
  } else if (g.boundary == S2A_BOUNDARY_SPLIT) {
    if (x < g.s) {
      gi = 0;
      slot = x;
    } else {
      gi = (x - g.s) / g.G + 1;
      slot = x - (g.s + (gi - 1) * g.G);
    }
  } else {
    int p = x - g.s;  // rolled index
    if (p < 0) p += g.N;
    gi = p / g.G;
    slot = p - gi * g.G;
    if (g.boundary == S2A_BOUNDARY_CYCLIC && gi == g.M - 1)
      slot = x < g.s ? x : x - (g.N - g.s) + g.s;  // position order
  }
}

// Row r of the regrouped layout (the groups of a class laid end to end in
// group order): its group gi and slot j.  For WRAP the rows are the rolled
// layout (CYCLIC: the same, with the last group in position order); for
// SPLIT and for class 0 they are the original order.
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
