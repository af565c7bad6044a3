// Backward of shifted sparse attention on gfx950.
//
// Gradients follow the logit gradient dL/dz = a * g.(v_j - o_i) (PaperTrace
// "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调", §3) and stay inside each
// group: no out-of-group pair is ever visited (§1.1, "反向传播确实保持稀疏").
//
// s2a_bwd_pre_kernel    delta_x = dO_x . O_x per (batch, head, row), and
//                       dQ cleared (it is accumulated with atomics)
// s2a_bwd_kernel        one workgroup owns 128 keys of one group and walks
//                       the group's query tiles at or after them:
//                         S  = Q K^T,  dP = dO V^T      (MFMA, K/V in regs)
//                         P  = exp(S - lse),  dS = P (dP - delta)
//                         dV^T += dO^T P,  dK^T += Q^T dS  (MFMA, registers)
//                         dQ += dS K  -> fp32 atomics at the rows' original
//                                        positions
//                       dK and dV are stored once at the end.
#include "s2a_device.h"
#include "s2a_kernels.h"

namespace {

constexpr int BWD_BK = 128;  // keys per workgroup, 32 per wave
constexpr int BWD_BQ = 64;   // queries per inner tile
constexpr int BWD_THREADS = 256;

template <int D>
struct BwdDims {
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int KP = DP + 16;      // LDS row pitch of K, Q, dO tiles
  static constexpr int SP = BWD_BQ + 8;   // LDS row pitch of dS^T
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = DP / 32;
  static constexpr int CPR = DP / 8;
};

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O), dQ = 0
// ---------------------------------------------------------------------------
template <int D, bool OF32>
__global__ __launch_bounds__(256) void s2a_bwd_pre_kernel(
    const void *__restrict__ o, const bf16_t *__restrict__ dout,
    float *__restrict__ delta, float *__restrict__ dq, int B, int N, int H) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const size_t rows = (size_t)B * N * H;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = row * D + c * 8;
    const bf16x8 g = __builtin_bit_cast(bf16x8, *(const u32x4 *)(dout + off));
    float ov[8];
    if (OF32) {
      const f32x4 a = *(const f32x4 *)((const float *)o + off);
      const f32x4 b2 = *(const f32x4 *)((const float *)o + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = a[e];
        ov[e + 4] = b2[e];
      }
    } else {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *(const u32x4 *)((const bf16_t *)o + off));
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = (float)a[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)g[e], ov[e], acc);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4 *)(dq + off) = z;
    *(f32x4 *)(dq + off + 4) = z;
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && c == 0) {
    const int hh = (int)(row % H);
    const size_t bx = row / H;
    const int x = (int)(bx % N);
    const int b = (int)(bx / N);
    delta[((size_t)b * H + hh) * N + x] = acc;
  }
}

// ---------------------------------------------------------------------------
// main backward
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(BWD_THREADS, 1) void s2a_bwd_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
    const bf16_t *__restrict__ v, const bf16_t *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ delta,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv,
    S2AParams p) {
  using Dm = BwdDims<D>;
  constexpr int KP = Dm::KP, SP = Dm::SP;
  constexpr int QT = BWD_BQ * KP;                        // elements per buffer
  constexpr int NCH = BWD_BQ * Dm::CPR / BWD_THREADS;    // chunks per thread
  static_assert(BWD_BQ * Dm::CPR % BWD_THREADS == 0, "tile split");
  __shared__ __attribute__((aligned(16))) bf16_t Ksm[BWD_BK * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2 * QT];
  __shared__ __attribute__((aligned(16))) bf16_t dOs[2 * QT];
  __shared__ __attribute__((aligned(16))) bf16_t dSt[BWD_BK * SP];
  __shared__ __attribute__((aligned(16))) float lse2s[2 * BWD_BQ];
  __shared__ __attribute__((aligned(16))) float dlts[2 * BWD_BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int grp = lane >> 4;
  const int trow = 4 * hf + ((lane & 15) >> 2);   // tr-read row in a 16-step
  const int tcol = 16 * (grp & 1) + 4 * (lane & 3);  // tr-read column

  // Workgroup -> (unit, key tile); all key tiles of a unit on one XCD,
  // first key tile (longest query walk) first.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, jj = bid >> 3;
  const int lu = jj / p.tiles;
  const int tile = jj - lu * p.tiles;
  const int u = lu * 8 + xcd;
  if (u >= p.units) return;
  const int gi = u % p.ngmax;
  const int bh = u / p.ngmax;
  const int h = bh % p.H, b = bh / p.H;
  const int cls = h >= (p.H >> 1);
  int base, glen;
  if (!s2a_group(p.g, cls, gi, base, glen)) return;
  const int k0 = tile * BWD_BK;
  if (k0 >= glen) return;
  const int N = p.g.N, L = p.g.L;
  const size_t rs = (size_t)p.H * D;
  const size_t boff = (size_t)b * N * rs + (size_t)h * D;
  const size_t lrow = ((size_t)b * p.H + h) * N;
  const float c2 = p.scale_log2;

  // This lane's key (one column of S) and the wave's key range.
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;
  const bool kin = key < glen;
  const int kpos = kin ? s2a_slot_pos(base, key, N) : 0;
  const bool kvalid = kin && kpos < L;
  const bool wave_keys_valid = __all(kvalid);

  bf16x8 kreg[Dm::KSTEPS], vreg[Dm::KSTEPS];
  {
    const size_t off = boff + (size_t)kpos * rs;
#pragma unroll
    for (int t = 0; t < Dm::KSTEPS; ++t) {
      u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
      if (kvalid) {
        a = *(const u32x4 *)(k + off + 16 * t + 8 * hf);
        c = *(const u32x4 *)(v + off + 16 * t + 8 * hf);
      }
      kreg[t] = __builtin_bit_cast(bf16x8, a);
      vreg[t] = __builtin_bit_cast(bf16x8, c);
    }
  }
  // K tile in LDS (B operand of dQ = dS K).
  for (int c = tid; c < BWD_BK * Dm::CPR; c += BWD_THREADS) {
    const int r = c / Dm::CPR, ch = c - r * Dm::CPR;
    const int ks = k0 + r;
    u32x4 kv = {0u, 0u, 0u, 0u};
    if (ks < glen && ch * 8 < D) {
      const int kp = s2a_slot_pos(base, ks, N);
      if (kp < L) kv = *(const u32x4 *)(k + boff + (size_t)kp * rs + ch * 8);
    }
    *(u32x4 *)(Ksm + r * KP + ch * 8) = kv;
  }

  // Query-tile staging through registers.  Rows outside the group or padded
  // get q = dO = 0, lse = +inf (so P = 0) and delta = 0 (so dS = 0).
  u32x4 qst[NCH], gst[NCH];
  float l2st = INFINITY, dlst = 0.f;
  auto fetch = [&](int q0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * BWD_THREADS;
      const int r = c / Dm::CPR, ch = c - r * Dm::CPR;
      const int qsl = q0 + r;
      u32x4 qv = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
      if (qsl < glen && ch * 8 < D) {
        const int qp = s2a_slot_pos(base, qsl, N);
        if (qp < L) {
          const size_t off = boff + (size_t)qp * rs + ch * 8;
          qv = *(const u32x4 *)(q + off);
          gv = *(const u32x4 *)(dout + off);
        }
      }
      qst[i] = qv;
      gst[i] = gv;
    }
    if (tid < BWD_BQ) {
      const int qsl = q0 + tid;
      l2st = INFINITY;
      dlst = 0.f;
      if (qsl < glen) {
        const int qp = s2a_slot_pos(base, qsl, N);
        if (qp < L) {
          l2st = lse[lrow + qp] * S2A_LOG2E;
          dlst = delta[lrow + qp];
        }
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * BWD_THREADS;
      const int r = c / Dm::CPR, ch = c - r * Dm::CPR;
      *(u32x4 *)(Qs + buf * QT + r * KP + ch * 8) = qst[i];
      *(u32x4 *)(dOs + buf * QT + r * KP + ch * 8) = gst[i];
    }
    if (tid < BWD_BQ) {
      lse2s[buf * BWD_BQ + tid] = l2st;
      dlts[buf * BWD_BQ + tid] = dlst;
    }
  };

  f32x16 dkacc[Dm::DB], dvacc[Dm::DB];
#pragma unroll
  for (int db = 0; db < Dm::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[db][i] = 0.f;
      dvacc[db][i] = 0.f;
    }

  const int nq = (glen - k0 + BWD_BQ - 1) / BWD_BQ;  // query tiles from k0
  fetch(k0);
  stage(0);
  __syncthreads();

  for (int it = 0; it < nq; ++it) {
    const int q0 = k0 + it * BWD_BQ;
    const int buf = it & 1;
    const bool more = it + 1 < nq;
    if (more) fetch(q0 + BWD_BQ);  // in flight during this tile's math
    const bf16_t *Qb = Qs + buf * QT;
    const bf16_t *dOb = dOs + buf * QT;
    const float *l2b = lse2s + buf * BWD_BQ;
    const float *dlb = dlts + buf * BWD_BQ;

    const bool active = q0 + BWD_BQ - 1 >= kw0;
    if (active) {
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[qb][i] = 0.f;
          dpacc[qb][i] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < Dm::KSTEPS; ++t) {
          const int ro = (32 * qb + l32) * KP + 16 * t + 8 * hf;
          const bf16x8 aq = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Qb + ro));
          const bf16x8 ag = __builtin_bit_cast(bf16x8, *(const u32x4 *)(dOb + ro));
          sacc[qb] = mfma32(aq, kreg[t], sacc[qb]);
          dpacc[qb] = mfma32(ag, vreg[t], dpacc[qb]);
        }
      }
      // P and dS.  Element i of block qb is query q0 + 32qb + 8(i/4) + 4hf + i%4.
      const bool edge = (q0 < kw0 + 31) || !wave_keys_valid;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = 32 * qb + 8 * i4 + 4 * hf;
          const f32x4 l2 = *(const f32x4 *)(l2b + r0);
          const f32x4 dl = *(const f32x4 *)(dlb + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            float pp = __builtin_amdgcn_exp2f(fmaf(sacc[qb][i], c2, -l2[e]));
            if (edge && !(kvalid && key <= q0 + r0 + e)) pp = 0.f;
            dpacc[qb][i] = pp * (dpacc[qb][i] - dl[e]);
            sacc[qb][i] = pp;
          }
        }
      // dV^T += dO^T P and dK^T += Q^T dS over 64 queries (4 steps of 16).
#pragma unroll
      for (int qs = 0; qs < BWD_BQ / 16; ++qs) {
        const int e0 = 8 * (qs & 1);
        const f32x16 &sp = sacc[qs >> 1];
        const f32x16 &dp = dpacc[qs >> 1];
        const bf16x8 pb = to_bf16x8(sp[e0], sp[e0 + 1], sp[e0 + 2], sp[e0 + 3],
                                    sp[e0 + 4], sp[e0 + 5], sp[e0 + 6], sp[e0 + 7]);
        const bf16x8 sb = to_bf16x8(dp[e0], dp[e0 + 1], dp[e0 + 2], dp[e0 + 3],
                                    dp[e0 + 4], dp[e0 + 5], dp[e0 + 6], dp[e0 + 7]);
        const int ro = (16 * qs + trow) * KP + tcol;
#pragma unroll
        for (int db = 0; db < Dm::DB; ++db) {
          const bf16x8 ag = cat4(lds_read_tr(dOb + ro + 32 * db),
                                 lds_read_tr(dOb + ro + 8 * KP + 32 * db));
          dvacc[db] = mfma32(ag, pb, dvacc[db]);
          const bf16x8 aq = cat4(lds_read_tr(Qb + ro + 32 * db),
                                 lds_read_tr(Qb + ro + 8 * KP + 32 * db));
          dkacc[db] = mfma32(aq, sb, dkacc[db]);
        }
      }
      // dS^T tile (bf16) for the dQ product.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16 &dp = dpacc[qb];
          *(bf16x4 *)(dSt + (32 * w + l32) * SP + 32 * qb + 8 * i4 + 4 * hf) =
              to_bf16x4(dp[4 * i4], dp[4 * i4 + 1], dp[4 * i4 + 2], dp[4 * i4 + 3]);
        }
    } else {
      const bf16x4 z = to_bf16x4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *(bf16x4 *)(dSt + (32 * w + l32) * SP + 32 * qb + 8 * i4 + 4 * hf) = z;
    }
    __syncthreads();  // dS^T complete

    // dQ[q][d] += dS[q][key] K[key][d] over the workgroup's 128 keys.
    for (int blk = w; blk < 2 * Dm::DB; blk += 4) {
      const int qb = blk & 1, db = blk >> 1;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < BWD_BK / 16; ++ks) {
        const int r = 16 * ks + trow;
        const bf16x8 as = cat4(lds_read_tr(dSt + r * SP + 32 * qb + tcol),
                               lds_read_tr(dSt + (r + 8) * SP + 32 * qb + tcol));
        const bf16x8 bk = cat4(lds_read_tr(Ksm + r * KP + 32 * db + tcol),
                               lds_read_tr(Ksm + (r + 8) * KP + 32 * db + tcol));
        acc = mfma32(as, bk, acc);
      }
      const int d = 32 * db + l32;
      if (d < D) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qsl = q0 + 32 * qb + 8 * (i >> 2) + 4 * hf + (i & 3);
          if (qsl < glen) {
            const int qp = s2a_slot_pos(base, qsl, N);
            if (qp < L)
              unsafeAtomicAdd(dq + boff + (size_t)qp * rs + d, acc[i] * p.scale);
          }
        }
      }
    }
    if (more) stage(buf ^ 1);
    __syncthreads();  // next tile staged; dS^T reads done
  }

  // dK, dV rows of this lane's key (padded keys get their exact zeros).
  if (kin) {
    const size_t row = boff + (size_t)kpos * rs;
#pragma unroll
    for (int db = 0; db < Dm::DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * hf;
        if (d < D) {
          const f32x4 kk = {dkacc[db][4 * i4] * p.scale, dkacc[db][4 * i4 + 1] * p.scale,
                            dkacc[db][4 * i4 + 2] * p.scale, dkacc[db][4 * i4 + 3] * p.scale};
          const f32x4 vv = {dvacc[db][4 * i4], dvacc[db][4 * i4 + 1],
                            dvacc[db][4 * i4 + 2], dvacc[db][4 * i4 + 3]};
          *(f32x4 *)(dk + row + d) = kk;
          *(f32x4 *)(dv + row + d) = vv;
        }
      }
  }
}

template <int D, bool OF32>
hipError_t launch_pre_t(const void *o, const void *dout, float *delta,
                        float *dq, int B, int N, int H, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const size_t rows = (size_t)B * N * H;
  dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  const bf16_t *g = (const bf16_t *)dout;
  void *args[] = {(void *)&o, (void *)&g, (void *)&delta, (void *)&dq,
                  (void *)&B, (void *)&N, (void *)&H};
  return hipLaunchKernel((const void *)s2a_bwd_pre_kernel<D, OF32>, grid,
                         block, args, 0, st);
}

template <int D>
hipError_t launch_bwd_t(const void *q, const void *k, const void *v,
                        const void *dout, const float *lse, const float *delta,
                        float *dq, float *dk, float *dv, const S2AParams &p,
                        hipStream_t st) {
  const int units_pad = (p.units + 7) / 8 * 8;
  dim3 grid((unsigned)units_pad * (unsigned)p.tiles), block(BWD_THREADS);
  const bf16_t *qq = (const bf16_t *)q, *kk = (const bf16_t *)k,
               *vv = (const bf16_t *)v, *gg = (const bf16_t *)dout;
  S2AParams pp = p;
  void *args[] = {(void *)&qq,  (void *)&kk, (void *)&vv, (void *)&gg,
                  (void *)&lse, (void *)&delta, (void *)&dq, (void *)&dk,
                  (void *)&dv,  (void *)&pp};
  return hipLaunchKernel((const void *)s2a_bwd_kernel<D>, grid, block, args,
                         0, st);
}

}  // namespace

int s2a_bwd_tile_rows() { return BWD_BK; }

hipError_t s2a_launch_bwd_pre(const void *o, bool o_f32, const void *dout,
                              float *dq, float *delta, int B, int N, int H,
                              int D, hipStream_t st) {
  switch (D) {
#define S2A_CASE(DD)                                                       \
  case DD:                                                                 \
    return o_f32 ? launch_pre_t<DD, true>(o, dout, delta, dq, B, N, H, st)  \
                 : launch_pre_t<DD, false>(o, dout, delta, dq, B, N, H, st);
    S2A_CASE(16)
    S2A_CASE(32)
    S2A_CASE(64)
    S2A_CASE(128)
#undef S2A_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t s2a_launch_bwd_main(const void *q, const void *k, const void *v,
                               const float *lse, const float *delta,
                               const void *dout, float *dq, float *dk,
                               float *dv, int D, const S2AParams &p,
                               hipStream_t st) {
  switch (D) {
    case 16: return launch_bwd_t<16>(q, k, v, dout, lse, delta, dq, dk, dv, p, st);
    case 32: return launch_bwd_t<32>(q, k, v, dout, lse, delta, dq, dk, dv, p, st);
    case 64: return launch_bwd_t<64>(q, k, v, dout, lse, delta, dq, dk, dv, p, st);
    case 128: return launch_bwd_t<128>(q, k, v, dout, lse, delta, dq, dk, dv, p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t s2a_launch_bwd(const void *q, const void *k, const void *v,
                          const void *o, bool o_f32, const float *lse,
                          const void *dout, float *dq, float *dk, float *dv,
                          float *delta, int D, const S2AParams &p,
                          hipStream_t st) {
  const hipError_t e =
      s2a_launch_bwd_pre(o, o_f32, dout, dq, delta, p.B, p.g.N, p.H, D, st);
  if (e != hipSuccess) return e;
  return s2a_launch_bwd_main(q, k, v, lse, delta, dout, dq, dk, dv, D, p, st);
}
