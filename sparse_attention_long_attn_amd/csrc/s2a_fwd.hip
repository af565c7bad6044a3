// Forward of shifted sparse attention on gfx950.
//
// One workgroup (4 waves) computes 128 query rows of one group of one
// (batch, head): every query's visible set is the keys of its own group at
// or before it in group order whose position is below the valid length
// (PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调", §1, visible sets
// N_0(i), N_1(i) and the cyclic-shift paragraph).  Only the key tiles of
// that group up to the diagonal are visited, so the work is proportional
// to the allowed pairs, not to N^2 (§1.1, last paragraph).
//
// Per key tile of 32 keys (D >= 64 without a document mask; 64 keys
// otherwise):
//   S^T = K Q^T           bf16 MFMA 32x32x16, fp32 accumulate; each lane
//                         owns one query column, so the row max needs a
//                         single cross-lane exchange (lane l <-> l^32)
//   online softmax        fp32, base 2 with log2(e) folded into the scale
//   O^T += V^T P^T        bf16 MFMA; V^T operands come straight from the
//                         row-major V tile in LDS through ds_read_tr16_b64,
//                         P^T from the S^T accumulators (same key order)
// and the epilogue writes O and the natural-log LSE at the rows' original
// positions (the inverse shift costs nothing: addresses come from
// the group's S2ARun).
#include <type_traits>

#include "s2a_device.h"
#include "s2a_kernels.h"
#include "s2a_tile.h"

namespace {

constexpr int FWD_BQ = 128;  // query rows per workgroup, 32 per wave
constexpr int FWD_BK = 64;   // keys per LDS tile (D < 64) and per document-list tile
constexpr int FWD_THREADS = FWD_BQ / 32 * 64;
// two waves per SIMD: 256-thread groups two per CU, 512-thread groups one
constexpr int FWD_MINBLOCKS = 512 / FWD_THREADS;

template <int D>
struct FwdDims {
  static constexpr int DP = D < 32 ? 32 : D;  // width in LDS (32-blocks)
  static constexpr int KP = DP + 16;          // LDS row pitch, elements
  static constexpr int KSTEPS = D / 16;       // 16-wide steps over d
  static constexpr int DB = DP / 32;          // 32-wide blocks over d
  static constexpr int CPR = DP / 8;          // 16-byte chunks per row
};

template <int D, bool OF32, bool DOC>
__global__ __launch_bounds__(FWD_THREADS, FWD_MINBLOCKS) void s2a_fwd_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, void *__restrict__ o,
    float *__restrict__ lse, S2AParams p) {
  using Dm = FwdDims<D>;
  constexpr int KP = Dm::KP;
  constexpr int TILE = FWD_BK * KP;                       // elements per buffer
  constexpr int TCH = FWD_BK * Dm::CPR;                  // chunks per tile
  constexpr int NCH = (TCH + FWD_THREADS - 1) / FWD_THREADS;    // chunks per thread
  // Two K and two V buffers: tile t+1 is written while tile t is read.
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2 * TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2 * TILE];
  __shared__ __attribute__((aligned(16))) int kdoc[2][FWD_BK];  // DOC only

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // Workgroup -> (unit, query tile).  Consecutive workgroup ids go to the
  // 8 XCDs in turn, so ids equal mod 8 share an XCD and its L2: all tiles
  // of one (batch, head, group) unit run there, heaviest (last) tile first.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, jj = bid >> 3;
  const int lu = jj / p.tiles;
  const int tile = p.tiles - 1 - (jj - lu * p.tiles);
  const int u = lu * 8 + xcd;
  if (u >= p.units) return;
  // unit u = gi * (B*H) + (b*H + h): the units of one XCD (equal mod 8)
  // are spread over the groups instead of sharing one group index, so the
  // XCDs get equal work even when groups do not (under a document mask)
  const int bh = u % (p.B * p.H);
  const int gi = u / (p.B * p.H);
  const int h = bh % p.H, b = bh / p.H;
  const int cls = h >= (p.H >> 1);
  S2ARun run;
  int glen;
  if (!s2a_group(p.g, cls, gi, run, glen)) return;
  const int q0 = tile * FWD_BQ;
  if (q0 >= glen) return;
  if (run.pos(min(q0 + FWD_BQ, glen) - 1) < 0) return;  // halo rows only
  const int N = p.g.N, L = p.g.L;
  const size_t rs = (size_t)p.H * D;  // elements between consecutive positions
  const size_t boff = (size_t)b * N * rs + (size_t)h * D;

  // This lane's query (one column of S^T).
  const int qslot = q0 + 32 * w + l32;
  // (a shard's halo rows sit at negative positions and are keys only)
  const int qp0 = qslot < glen ? run.pos(qslot) : -1;
  const bool qin = qp0 >= 0;
  const int qpos = qin ? qp0 : 0;
  const bool qvalid = qin && qpos < L;
  const int qdoc = DOC ? p.doc[(size_t)b * N + qpos] : 0;

  bf16x8 qreg[Dm::KSTEPS];
  {
    const bf16_t *qrow = q + boff + (size_t)qpos * rs;
#pragma unroll
    for (int t = 0; t < Dm::KSTEPS; ++t) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qin) raw = *(const u32x4 *)(qrow + 16 * t + 8 * hf);
      qreg[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Staging of one K/V tile through registers: chunk c of the tile is row
  // c / CPR, 16-byte column c % CPR.  Rows outside the group or at padded
  // positions are zero.
  u32x4 kst[NCH], vst[NCH];
  int kdst = 0;  // document ID of key k0 + tid (DOC, tid < FWD_BK)
  auto fetch = [&](int k0) {
    if (DOC && tid < FWD_BK) {
      const int ks = k0 + tid;
      kdst = p.doc[(size_t)b * N + (ks < glen ? run.pos(ks) : 0)];
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * FWD_THREADS;
      const int r = c / Dm::CPR, ch = c - r * Dm::CPR;
      const int ks = k0 + r;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (c < TCH && ks < glen && ch * 8 < D) {
        const int kp = run.pos(ks);
        if (kp < L) {
          const size_t off = boff + (size_t)kp * rs + ch * 8;
          kv = *(const u32x4 *)(k + off);
          vv = *(const u32x4 *)(v + off);
        }
      }
      kst[i] = kv;
      vst[i] = vv;
    }
  };
  auto stage = [&](int buf) {
    if (DOC && tid < FWD_BK) kdoc[buf][tid] = kdst;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * FWD_THREADS;
      if (c >= TCH) continue;
      const int r = c / Dm::CPR, ch = c - r * Dm::CPR;
      *(u32x4 *)(Ks + buf * TILE + r * KP + ch * 8) = kst[i];
      *(u32x4 *)(Vs + buf * TILE + r * KP + ch * 8) = vst[i];
    }
  };

  f32x16 oacc[Dm::DB];
#pragma unroll
  for (int db = 0; db < Dm::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  // Running reference max (base 2) and this lane's partial row sum.  The
  // reference only moves when a tile's max exceeds it by more than
  // 2^RESCALE, so P <= 2^RESCALE and the O rescale is rarely needed.
  constexpr float RESCALE = 8.f;
  float m_ref = -INFINITY, l_run = 0.f;

  const int kend = min(glen, q0 + FWD_BQ);
  const int ntiles = (kend + FWD_BK - 1) / FWD_BK;
  const int wq_lo = q0 + 32 * w;
  const int wq_hi = wq_lo + 31;
  const float c2 = p.scale_log2;
  const int grp = lane >> 4;
  const int trow = 4 * hf + ((lane & 15) >> 2);
  const int tcol = 16 * (grp & 1) + 4 * (lane & 3);

  fetch(0);
  stage(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * FWD_BK;
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) fetch(k0 + FWD_BK);  // in flight during this tile's math

    if (k0 <= wq_hi) {  // else every query of this wave precedes the tile
      const bf16_t *Kb = Ks + buf * TILE;
      const bf16_t *Vb = Vs + buf * TILE;
      // S^T = K Q^T for 64 keys x 32 queries.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
        for (int t = 0; t < Dm::KSTEPS; ++t) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8,
              *(const u32x4 *)(Kb + (32 * kb + l32) * KP + 16 * t + 8 * hf));
          sacc[kb] = mfma32(a, qreg[t], sacc[kb]);
        }
      }

      // Mask where the tile crosses the diagonal, the group end or padding
      // (and everywhere under a document mask).
      const int kstop = min(k0 + FWD_BK, glen);
      const bool edge = DOC || (k0 + FWD_BK - 1 > wq_lo) ||
                        (k0 + FWD_BK > glen) ||
                        s2a_range_has_padding(run, k0, kstop, N, L);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            i32x4 kd = {0, 0, 0, 0};
            if (DOC) kd = *(const i32x4 *)&kdoc[buf][32 * kb + 8 * g4 + 4 * hf];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * g4 + j;
              const int ks = k0 + 32 * kb + 8 * g4 + 4 * hf + j;
              bool ok = (ks <= qslot) & (ks < glen) & (run.pos(ks) < L);
              if (DOC) ok &= kd[j] == qdoc;
              sacc[kb][i] = ok ? sacc[kb][i] : -INFINITY;
            }
          }
      }

      // Online softmax (base 2) with a lazily moved reference max.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = wave_max_x32(mx) * c2;
      if (__any(mx > m_ref + RESCALE)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha =
            m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < Dm::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_ref = m_new;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e =
              __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c2, -m_use));
          sacc[kb][i] = e;
          ls += e;
        }
      l_run += ls;

      // O^T += V^T P^T, 16 keys per MFMA.  Key order inside a step: element
      // j of half hf is key 16*ks + 8*(j/4) + 4*hf + j%4 on both operands.
#pragma unroll
      for (int ks = 0; ks < FWD_BK / 16; ++ks) {
        const f32x16 &sp = sacc[ks >> 1];
        const int e0 = 8 * (ks & 1);
        const bf16x8 pb = to_bf16x8(sp[e0 + 0], sp[e0 + 1], sp[e0 + 2],
                                    sp[e0 + 3], sp[e0 + 4], sp[e0 + 5],
                                    sp[e0 + 6], sp[e0 + 7]);
        const bf16_t *vr = Vb + (16 * ks + trow) * KP + tcol;
#pragma unroll
        for (int db = 0; db < Dm::DB; ++db) {
          const bf16x4 lo = lds_read_tr(vr + 32 * db);
          const bf16x4 hi = lds_read_tr(vr + 8 * KP + 32 * db);
          oacc[db] = mfma32(cat4(lo, hi), pb, oacc[db]);
        }
      }
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: normalise, write O and LSE at the original position.
  const float lt = wave_sum_x32(l_run);
  if (qin) {
    const float inv = qvalid ? 1.f / lt : 0.f;
    const size_t orow = boff + (size_t)qpos * rs;
#pragma unroll
    for (int db = 0; db < Dm::DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * hf;
        if (d < D) {
          float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
          if (qvalid) {
            r0 = oacc[db][4 * i4 + 0] * inv;
            r1 = oacc[db][4 * i4 + 1] * inv;
            r2 = oacc[db][4 * i4 + 2] * inv;
            r3 = oacc[db][4 * i4 + 3] * inv;
          }
          if (OF32) {
            f32x4 val = {r0, r1, r2, r3};
            *(f32x4 *)((float *)o + orow + d) = val;
          } else {
            *(bf16x4 *)((bf16_t *)o + orow + d) = to_bf16x4(r0, r1, r2, r3);
          }
        }
      }
    if (hf == 0)
      lse[((size_t)b * p.H + h) * N + qpos] =
          qvalid ? (m_ref + __builtin_amdgcn_logf(lt)) * S2A_LN2 : -INFINITY;
  }
}

// Forward for D in {64, 128}: same math as s2a_fwd_kernel, with K/V tiles
// of BK keys in the swizzled unpadded layout of s2a_tile.h filled by
// direct global -> LDS loads (no staging registers, addresses
// precomputed).  Without a document mask the tiles are 32 keys: 32 KiB of
// LDS and 162 VGPRs, so three workgroups (three waves per SIMD) share a
// CU, 4-5 % faster at 32K than 64-key tiles with two.  Under a document
// mask the tiles are 64 keys, the granularity of the document lists: the
// mask's registers (177 VGPRs with 32-key tiles) leave two workgroups per
// CU either way, and there 64-key tiles are 7-14 % faster.
template <int D, bool OF32, bool DOC, int BK>
__global__ __launch_bounds__(FWD_THREADS, BK == 32 ? 3 : FWD_MINBLOCKS) void s2a_fwd_sw_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, void *__restrict__ o,
    float *__restrict__ lse, S2AParams p) {
  static_assert(BK == 32 || BK == 64, "32- or 64-key tiles");
  static_assert(!DOC || BK == FWD_BK, "document lists mark 64-key tiles");
  using T = SwTile<D>;
  using LD = TileLoader<D, BK, FWD_THREADS / 64>;
  constexpr int KSTEPS = D / 16, DB = D / 32, NKB = BK / 32;
  constexpr int TILEB = BK * T::ROWB;  // bytes per tile buffer
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];
  __shared__ __attribute__((aligned(16))) int kdoc[2][FWD_BK];  // DOC only
  __shared__ unsigned klive[DOC_WORDS];                          // DOC only
  __shared__ int rng[2 * (FWD_THREADS / 64)];                    // DOC only
  char *const Ks = smem;              // two K buffers
  char *const Vs = smem + 2 * TILEB;  // two V buffers

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;

  const int bid = blockIdx.x;
  const int xcd = bid & 7, jj = bid >> 3;
  const int lu = jj / p.tiles;
  const int tile = p.tiles - 1 - (jj - lu * p.tiles);
  const int u = lu * 8 + xcd;
  if (u >= p.units) return;
  // unit u = gi * (B*H) + (b*H + h): the units of one XCD (equal mod 8)
  // are spread over the groups instead of sharing one group index, so the
  // XCDs get equal work even when groups do not (under a document mask)
  const int bh = u % (p.B * p.H);
  const int gi = u / (p.B * p.H);
  const int h = bh % p.H, b = bh / p.H;
  const int cls = h >= (p.H >> 1);
  S2ARun run;
  int glen;
  if (!s2a_group(p.g, cls, gi, run, glen)) return;
  const int q0 = tile * FWD_BQ;
  if (q0 >= glen) return;
  if (run.pos(min(q0 + FWD_BQ, glen) - 1) < 0) return;  // halo rows only
  const int N = p.g.N, L = p.g.L;
  const size_t rs = (size_t)p.H * D;
  const size_t boff = (size_t)b * N * rs + (size_t)h * D;
  const bf16_t *kbh = k + boff, *vbh = v + boff;

  const int qslot = q0 + 32 * w + l32;
  // (a shard's halo rows sit at negative positions and are keys only)
  const int qp0 = qslot < glen ? run.pos(qslot) : -1;
  const bool qin = qp0 >= 0;
  const int qpos = qin ? qp0 : 0;
  const bool qvalid = qin && qpos < L;
  const int qdoc = DOC ? p.doc[(size_t)b * N + qpos] : 0;
  // Document IDs the wave's valid queries span: a key tile whose IDs all
  // lie outside [qdmn, qdmx] shares no document with them and is skipped.
  int qdmn = qvalid ? qdoc : INT_MAX, qdmx = qvalid ? qdoc : INT_MIN;
  if (DOC) wave_minmax(qdmn, qdmx);

  bf16x8 qreg[KSTEPS];
  {
    const bf16_t *qrow = q + boff + (size_t)qpos * rs;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qin) raw = *(const u32x4 *)(qrow + 16 * t + 8 * hf);
      qreg[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  LD ld;
  ld.init(w, lane);
  ld.init_rs(rs);
  auto issue = [&](int k0, int buf) {
    char *kd = Ks + buf * TILEB, *vd = Vs + buf * TILEB;
    if (tile_plain(run, glen, k0, BK, L)) {
      const size_t r0 = (size_t)run.pos(k0) * rs;
      ld.fast_s(kbh + r0, kd);
      ld.fast_s(vbh + r0, vd);
    } else {
      ld.general(kbh, rs, run, glen, k0, L, kd);
      ld.general(vbh, rs, run, glen, k0, L, vd);
    }
    if (DOC && w == 0) {  // the tile's 64 document IDs
      const int ks = k0 + lane;
      g2lds4(p.doc + (size_t)b * N + (ks < glen ? run.pos(ks) : 0),
             &kdoc[buf][0]);
    }
  };

  // Per-lane byte offsets of the MFMA operand reads.
  //   K (A of S^T): row 32*kb + l32, logical chunk 2t + hf
  //   V^T (A of O^T, transposing read): row 16*ks + trow (+8), element
  //   column 32*db + tcol, i.e. logical chunk 4db + 2*(grp&1) + (lane&3)/2
  const int grp = lane >> 4;
  const int trow = 4 * hf + ((lane & 15) >> 2);
  // (rows trow and trow + 8 of a 16-key step have different swizzles)
  int koff[KSTEPS], voff[DB], voff8[DB];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) koff[t] = T::off(l32, 2 * t + hf);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int c = 4 * db + 2 * (grp & 1) + ((lane & 3) >> 1);
    voff[db] = T::off(trow, c) + (lane & 1) * 8;
    voff8[db] = T::off(trow + 8, c) + (lane & 1) * 8;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  constexpr float RESCALE = 8.f;
  float m_ref = -INFINITY, l_run = 0.f;

  const int kend = min(glen, q0 + FWD_BQ);
  const int ntiles = (kend + BK - 1) / BK;
  const int wq_lo = q0 + 32 * w;
  const int wq_hi = wq_lo + 31;
  const float c2 = p.scale_log2;

  // Under a document mask the workgroup walks only the key tiles whose IDs
  // can meet its queries' (the rest would be masked out entirely).
  if (DOC) {
    int mn = qdmn, mx = qdmx;
    wg_range<FWD_THREADS / 64>(mn, mx, rng, w, lane);
    doc_tiles<FWD_THREADS / 64>(p.doc + (size_t)b * N, run, glen, L, 0,
                                ntiles, mn, mx, klive, nullptr, w, lane);
  }
  // first walked tile >= i (ntiles if none)
  auto next_walk = [&](int i) { return next_tile(klive, i, ntiles); };
  int it = DOC ? next_walk(0) : 0;
  if (it < ntiles) issue(it * BK, 0);
  wait_vm_all();
  __syncthreads();

  // One walk step on the tile in buffer buf (a compile-time constant: the
  // loop below alternates two copies, so every LDS address of a step is a
  // register plus an immediate offset, with no per-step address arithmetic).
  auto step = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int k0 = it * BK;
    const int nx = DOC ? next_walk(it + 1) : it + 1;
    const bool more = nx < ntiles;
    if (more) issue(nx * BK, buf ^ 1);  // lands during this tile's math

    // (docedge: the tile's keys and the wave's queries are not all of one
    // document, so the document mask must be applied)
    bool live = k0 <= wq_hi, docedge = false;
    if (DOC && live) {
      // one key ID per lane; ballots rather than a cross-lane min/max,
      // whose dependent shuffles would stall every tile
      const int kd = kdoc[buf][lane & (BK - 1)];
      live = __any(kd >= qdmn && kd <= qdmx);
      docedge = !(qdmn == qdmx && __all(kd == qdmn));
    }
    if (live) {
      const char *Kb = Ks + buf * TILEB;
      const char *Vb = Vs + buf * TILEB;
      // S^T = K Q^T, NKB * KSTEPS MFMAs over (kb, t); each operand read runs PIPE
      // steps ahead of its MFMA (the fences keep the compiler from waiting
      // on every read right before its use)
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      constexpr int PIPE = 3, NS = NKB * KSTEPS;
      bf16x8 a[NS];
      auto opload = [&](int st) {
        a[st] = *(const bf16x8 *)(Kb + (st / KSTEPS) * 32 * T::ROWB +
                                  koff[st % KSTEPS]);
      };
#pragma unroll
      for (int st = 0; st < PIPE; ++st) opload(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        if (st + PIPE < NS) opload(st + PIPE);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = st / KSTEPS, t = st % KSTEPS;
        sacc[kb] = mfma32(a[st], qreg[t], sacc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }

      const bool edge = docedge || (k0 + BK - 1 > wq_lo) ||
                        !tile_plain(run, glen, k0, BK, L);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            i32x4 kd = {0, 0, 0, 0};
            if (DOC) kd = *(const i32x4 *)&kdoc[buf][32 * kb + 8 * g4 + 4 * hf];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * g4 + j;
              const int ks = k0 + 32 * kb + 8 * g4 + 4 * hf + j;
              bool ok = (ks <= qslot) & (ks < glen) & (run.pos(ks) < L);
              if (DOC) ok &= kd[j] == qdoc;
              sacc[kb][i] = ok ? sacc[kb][i] : -INFINITY;
            }
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = wave_max_x32(mx) * c2;
      if (__any(mx > m_ref + RESCALE)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha =
            m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_ref = m_new;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e =
              __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c2, -m_use));
          sacc[kb][i] = e;
          ls += e;
        }
      l_run += ls;

      // Two waves (of two workgroups) share a SIMD: while one issues this
      // PV cluster it takes issue priority over the other's element work
      // (3 % faster at 32K; the same around the S cluster gains nothing)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const f32x16 &sp = sacc[ks >> 1];
        const int e0 = 8 * (ks & 1);
        const bf16x8 pb = to_bf16x8(sp[e0 + 0], sp[e0 + 1], sp[e0 + 2],
                                    sp[e0 + 3], sp[e0 + 4], sp[e0 + 5],
                                    sp[e0 + 6], sp[e0 + 7]);
        const char *vr = Vb + 16 * ks * T::ROWB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = lds_read_tr((const bf16_t *)(vr + voff[db]));
          const bf16x4 hi = lds_read_tr((const bf16_t *)(vr + voff8[db]));
          oacc[db] = mfma32(cat4(lo, hi), pb, oacc[db]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    wait_vm_all();
    __syncthreads();
    it = nx;
  };
  while (it < ntiles) {
    step(std::integral_constant<int, 0>{});
    if (it >= ntiles) break;
    step(std::integral_constant<int, 1>{});
  }

  const float lt = wave_sum_x32(l_run);
  if (qin) {
    const float inv = qvalid ? 1.f / lt : 0.f;
    const size_t orow = boff + (size_t)qpos * rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * hf;
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        if (qvalid) {
          r0 = oacc[db][4 * i4 + 0] * inv;
          r1 = oacc[db][4 * i4 + 1] * inv;
          r2 = oacc[db][4 * i4 + 2] * inv;
          r3 = oacc[db][4 * i4 + 3] * inv;
        }
        if (OF32) {
          f32x4 val = {r0, r1, r2, r3};
          *(f32x4 *)((float *)o + orow + d) = val;
        } else {
          *(bf16x4 *)((bf16_t *)o + orow + d) = to_bf16x4(r0, r1, r2, r3);
        }
      }
    if (hf == 0)
      lse[((size_t)b * p.H + h) * N + qpos] =
          qvalid ? (m_ref + __builtin_amdgcn_logf(lt)) * S2A_LN2 : -INFINITY;
  }
}

template <int D, bool OF32, bool DOC>
hipError_t launch_fwd_d(const void *q, const void *k, const void *v, void *o,
                        float *lse, const S2AParams &p, hipStream_t st) {
  const int units_pad = (p.units + 7) / 8 * 8;
  const bf16_t *qq = (const bf16_t *)q, *kk = (const bf16_t *)k,
               *vv = (const bf16_t *)v;
  S2AParams pp = p;
  void *args[] = {(void *)&qq, (void *)&kk, (void *)&vv, (void *)&o,
                  (void *)&lse, (void *)&pp};
  dim3 grid((unsigned)units_pad * (unsigned)p.tiles);
  const void *fn;
  if constexpr (D >= 64)
    fn = (const void *)s2a_fwd_sw_kernel<D, OF32, DOC, DOC ? FWD_BK : 32>;
  else
    fn = (const void *)s2a_fwd_kernel<D, OF32, DOC>;
  return hipLaunchKernel(fn, grid, dim3(FWD_THREADS), args, 0, st);
}

template <int D, bool OF32>
hipError_t launch_fwd_t(const void *q, const void *k, const void *v, void *o,
                        float *lse, const S2AParams &p, hipStream_t st) {
  return p.doc ? launch_fwd_d<D, OF32, true>(q, k, v, o, lse, p, st)
               : launch_fwd_d<D, OF32, false>(q, k, v, o, lse, p, st);
}

}  // namespace

int s2a_fwd_tile_rows(int) { return FWD_BQ; }

hipError_t s2a_launch_fwd(const void *q, const void *k, const void *v,
                          void *o, bool o_f32, float *lse, int D,
                          const S2AParams &p, hipStream_t st) {
  switch (D) {
    case 16: return o_f32 ? launch_fwd_t<16, true>(q, k, v, o, lse, p, st)
                          : launch_fwd_t<16, false>(q, k, v, o, lse, p, st);
    case 32: return o_f32 ? launch_fwd_t<32, true>(q, k, v, o, lse, p, st)
                          : launch_fwd_t<32, false>(q, k, v, o, lse, p, st);
    case 64: return o_f32 ? launch_fwd_t<64, true>(q, k, v, o, lse, p, st)
                          : launch_fwd_t<64, false>(q, k, v, o, lse, p, st);
    case 128: return o_f32 ? launch_fwd_t<128, true>(q, k, v, o, lse, p, st)
                           : launch_fwd_t<128, false>(q, k, v, o, lse, p, st);
    default: return hipErrorInvalidValue;
  }
}
