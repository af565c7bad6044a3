// Row tiles of Q/K/V/dO in LDS for head widths D in {64, 128}.
//
// A tile holds ROWS consecutive slots of one group as ROWS x D bf16, rows
// back to back (no padding), filled straight from global memory with
// global_load_lds_dwordx4: one wave instruction copies 64 chunks of 16
// bytes, lane i landing at byte 16*i past the wave's LDS base.  Bank
// conflicts are avoided by permuting the 16-byte chunks inside each row:
// logical chunk c of row r sits at physical chunk c ^ swz(r).  The lane
// that fills physical chunk p of row r therefore reads logical chunk
// p ^ swz(r) from global memory.
//
// swz(r) (see SwTile below) is chosen so that both read patterns of the
// kernels touch every LDS bank once per pass: 16-byte operand reads (32
// lanes on 32 consecutive rows, same logical chunk) and ds_read_b64_tr_b16
// (16 lanes on 4 consecutive rows, chunks 4j .. 4j+3).  An unpermuted
// layout serialises both on a few banks.
#pragma once
#include <limits.h>
#include <stdint.h>

#include "s2a_device.h"

template <int D>
struct SwTile {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int ROWB = D * 2;        // bytes per row
  // Logical chunk c of row r sits at physical chunk c ^ swz(r).  The LDS
  // has 64 banks of 4 bytes (256 bytes per sweep); a 16-byte read is served
  // 16 lanes at a time and an 8-byte (transposing) read 32 lanes at a time.
  // The operand reads (lane l: row l % 32, one chunk) need the 16 rows of a
  // pass in distinct bank groups; the transposing reads (32 lanes: rows
  // 4k .. 4k+3, chunks 4j .. 4j+3) need those four rows in distinct aligned
  // groups of four chunks.  D = 128 (one row per sweep): swz is the 4x4
  // transpose of r's low four bits.  D = 64 (two rows per sweep): rows of
  // one parity take distinct chunks, rows 4k and 4k+2 different halves.
  // Period 16 in r.
  __device__ static constexpr int swz(int r) {
    if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (((r & 7) << 1) | ((r >> 3) & 1)) & (CPR - 1);
  }
  // byte offset of logical chunk c of row r
  __device__ static constexpr int off(int r, int c) {
    return r * ROWB + ((c ^ swz(r)) << 4);
  }
};

// Direct global -> LDS copy of 16 bytes per lane.  lds_wave must be the
// same for every lane of the wave (it is kept in M0).
//
// Written as inline asm on purpose: the compiler counts these loads as
// outstanding LDS operations too, and then waits for every LDS read in
// flight (lgkmcnt(0)) wherever a read result is used, instead of only for
// the oldest.  Hidden from it, the loads are waited for explicitly: every
// kernel ends each tile with s_waitcnt vmcnt(0) and a barrier before the
// buffer is read.  No VGPR is written (the data goes to LDS), and "memory"
// keeps the loads in program order with the barriers and LDS accesses.
__device__ __forceinline__ void g2lds16(const void *gptr, void *lds_wave) {
  const unsigned m0 = (unsigned)(uintptr_t)lds_wave;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(m0)
               : "memory", "m0");
}

// The same with a wave-uniform base address and a 32-bit per-lane byte
// offset (the scalar-base form of the instruction).
__device__ __forceinline__ void g2lds16_s(const void *gbase, unsigned off,
                                          void *lds_wave) {
  // (both are wave-uniform; readfirstlane tells the compiler so, which the
  // scalar operands need)
  const unsigned m0 =
      (unsigned)__builtin_amdgcn_readfirstlane((int)(uintptr_t)lds_wave);
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint64_t gu =
      ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(g >> 32)) << 32) |
      (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)g);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(gu), "s"(m0)
               : "memory", "m0");
}

// The same, streaming (nt): for data read once, so that it does not
// displace lines that later loads of the kernel read again.
__device__ __forceinline__ void g2lds16_snt(const void *gbase, unsigned off,
                                          void *lds_wave) {
  // (both are wave-uniform; readfirstlane tells the compiler so, which the
  // scalar operands need)
  const unsigned m0 =
      (unsigned)__builtin_amdgcn_readfirstlane((int)(uintptr_t)lds_wave);
  const uint64_t g = (uint64_t)(uintptr_t)gbase;
  const uint64_t gu =
      ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(g >> 32)) << 32) |
      (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)g);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(off), "s"(gu), "s"(m0)
               : "memory", "m0");
}

// Direct global -> LDS copy of 4 bytes per lane (lane i lands at byte 4*i
// past lds_wave, which must be the same for every lane of the wave).  Inline
// asm for the reason given at g2lds16.
__device__ __forceinline__ void g2lds4(const void *gptr, void *lds_wave) {
  const unsigned m0 = (unsigned)(uintptr_t)lds_wave;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(m0)
               : "memory", "m0");
}

// Loader of one ROWS-row tile of a [B,N,H,D] tensor by NWAVES waves.  Each
// wave issues IPW instructions; instruction i of wave w fills tile chunks
// [(w*IPW + i)*64, +64).  Per lane it keeps the tile row it fills and the
// element offset of its logical chunk inside that row.
template <int D, int ROWS, int NWAVES>
struct TileLoader {
  using T = SwTile<D>;
  static constexpr int CHUNKS = ROWS * T::CPR;
  static constexpr int IPW = CHUNKS / (64 * NWAVES);
  static_assert(CHUNKS % (64 * NWAVES) == 0, "tile must split into waves");
  int w, lane;         // this lane's wave and lane
  unsigned boff[IPW];  // byte offset of its chunk of instruction i from the
                       // tile's first row when rows are rs elements apart
                       // (see init_rs)

  // tile row filled by this lane in instruction i, and the element offset
  // of its logical chunk within the row
  __device__ void chunk(int i, int &r, int &co) const {
    const int c = (w * IPW + i) * 64 + lane;
    r = c / T::CPR;
    co = ((c % T::CPR) ^ T::swz(r)) * 8;
  }
  // wave's LDS byte offset of instruction i (uniform)
  __device__ static constexpr int ldsb(int w, int i) {
    return (w * IPW + i) * 64 * 16;
  }

  __device__ void init(int w_, int lane_) {
    w = w_;
    lane = lane_;
#pragma unroll
    for (int i = 0; i < IPW; ++i) boff[i] = 0;
  }
  // Precompute the byte offsets used by fast_s(): row < ROWS <= 128 and
  // rs = H*D, so they fit in 32 bits while H*D stays below 2^24.
  __device__ void init_rs(size_t rs) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      int r, co;
      chunk(i, r, co);
      boff[i] = (unsigned)(r * rs + co) * 2u;
    }
  }

  // Rows are slots s0 + row of a group, all valid and contiguous from the
  // wave-uniform row pointer g0 (slot s0's row, head h): global_load_lds
  // with a scalar base and a 32-bit per-lane offset, so no per-lane 64-bit
  // addresses stay live across a loop.
  __device__ void fast_s(const bf16_t *g0, char *lds) const {
#pragma unroll
    for (int i = 0; i < IPW; ++i) g2lds16_s(g0, boff[i], lds + ldsb(w, i));
  }

  // General rows: slot s0 + row of the group (run, glen); rows outside
  // the group, at positions >= L or below lo read position 0 of the same
  // (b, h) instead (finite data that the kernels mask out).  Query tiles
  // pass lo = 0: a shard's halo rows are keys only.
  __device__ void general(const bf16_t *gbh, size_t rs, const S2ARun &run,
                          int glen, int s0, int L, char *lds,
                          int lo = INT_MIN) const {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      int r, co;
      chunk(i, r, co);
      // opaque copies keep the compiler from hoisting per-lane 64-bit
      // addresses of this (rare) path out of the caller's loop
      asm volatile("" : "+v"(r), "+v"(co));
      const int s = s0 + r;
      int pos = 0;
      if (s < glen) {
        pos = run.pos(s);
        if (pos >= L || pos < lo) pos = 0;
      }
      g2lds16(gbh + (size_t)pos * rs + co, lds + ldsb(w, i));
    }
  }
};

// The tile [s0, s0 + rows) of a group is "plain" when every slot is inside
// the group, inside one run, and at a position in [lo, L): then its rows
// are contiguous in memory from slot s0's position.
__device__ __forceinline__ bool tile_plain(const S2ARun &run, int glen,
                                           int s0, int rows, int L,
                                           int lo = INT_MIN) {
  if (s0 + rows > glen) return false;
  if (s0 < run.cut && s0 + rows > run.cut) return false;
  const int p0 = run.pos(s0);
  return p0 + rows <= L && p0 >= lo;
}

__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0);
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) |
                             (15 << 8));
}


// ---------------------------------------------------------------------------
// Document-mask tile lists.  A kernel that walks the 64-slot tiles
// t0, t0 + 64, ... of a group needs only the tiles whose document IDs can
// meet those of its own rows.  doc_tiles() marks, one bit per tile in the
// LDS words live[], every tile j with a valid slot (inside the group, at a
// position below L) whose ID lies in [lo, hi] (the range of the caller's
// own IDs, so a tile left unmarked shares no document with them); with
// hot != nullptr it also marks tiles holding a "hot" valid slot s: s < 64,
// or an ID different from that of slot s - 64 (a row that sees few keys).
// Tiles past DOC_MAXT are all marked live (and hot): correct, not skipped.
// Every thread of the workgroup calls it; it ends with a barrier.
constexpr int DOC_MAXT = 1024;            // tiles tracked (groups <= 64K)
constexpr int DOC_WORDS = DOC_MAXT / 32;

template <int NW>
__device__ void doc_tiles(const int *docb, const S2ARun &run, int glen, int L,
                          int t0, int ntiles, int lo, int hi, unsigned *live,
                          unsigned *hot, int w, int lane) {
  const int nw = (min(ntiles, DOC_MAXT) + 31) / 32;
  for (int k = w; k < DOC_WORDS; k += NW) {
    unsigned lbits = ~0u, hbits = ~0u;  // beyond the tracked tiles: walk all
    if (k < nw) {
      // Word k covers tiles 32k .. 32k+31.  Load e of a lane reads slot
      // lane of tile 32k + e, so each load instruction reads one tile's 64
      // consecutive slots (coalesced) and a ballot per tile gives its bits.
      // Padded slots are read at their own position too: the hot test
      // compares with the slot one tile earlier whatever it holds.
      const int sb = t0 + 64 * 32 * k + lane;
      lbits = hbits = 0u;
      int prev = 0;  // ID of slot sb - 64 (hot test of the word's first tile)
      if (hot != nullptr && sb >= 64) prev = docb[run.pos(sb - 64)];
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        int d[16];
        bool vv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int s = sb + 64 * (16 * part + e);
          const bool in = s < glen;
          const int pos = in ? run.pos(s) : 0;
          vv[e] = in && pos < L;
          d[e] = docb[pos];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = 16 * part + e;
          const int s = sb + 64 * j;
          if (__any(vv[e] && d[e] >= lo && d[e] <= hi)) lbits |= 1u << j;
          if (hot != nullptr) {
            if (__any(vv[e] && (s < 64 || d[e] != prev))) hbits |= 1u << j;
            prev = d[e];
          }
        }
      }
    }
    if (lane == 0) {
      live[k] = lbits;
      if (hot != nullptr) hot[k] = hbits;
    }
  }
  __syncthreads();
}

// First tile >= j whose bit is set in words[] (ntiles if none); tiles past
// DOC_MAXT count as set.  Wave-uniform.
__device__ __forceinline__ int next_tile(const unsigned *words, int j,
                                         int ntiles) {
  while (j < ntiles && j < DOC_MAXT) {
    // (every lane reads the same word: made uniform for the compiler)
    const unsigned b =
        (unsigned)__builtin_amdgcn_readfirstlane((int)words[j >> 5]) >> (j & 31);
    if (b) return j + __builtin_ctz(b);
    j = (j | 31) + 1;
  }
  return min(j, ntiles);
}

// Whether tile j is set in words[] (tiles past DOC_MAXT count as set).
__device__ __forceinline__ bool tile_bit(const unsigned *words, int j) {
  if (j >= DOC_MAXT) return true;
  const unsigned w = (unsigned)__builtin_amdgcn_readfirstlane((int)words[j >> 5]);
  return (w >> (j & 31)) & 1u;
}

// [min, max] of (mn, mx) over the workgroup's waves, through 2*NW ints of
// LDS scratch; every thread gets the result.  Contains barriers.
template <int NW>
__device__ void wg_range(int &mn, int &mx, int *scratch, int w, int lane) {
  wave_minmax(mn, mx);
  if (lane == 0) {
    scratch[2 * w] = mn;
    scratch[2 * w + 1] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mn = min(mn, scratch[2 * i]);
    mx = max(mx, scratch[2 * i + 1]);
  }
  __syncthreads();
}
