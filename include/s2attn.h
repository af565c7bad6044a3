/*
 * s2attn.h -- C ABI of the MI355X (gfx950) shifted sparse attention engine.
 *
 * Shifted sparse attention (S²-Attn) as described on the PaperTrace page
 * "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调" (§1 "S²-Attn的计算图") and in
 * the study notes "精读笔记：LongLoRA" (§3.2): the sequence is cut into groups
 * of G tokens and each group runs causal attention on its own.  Heads
 * [0, H/2) group on the original boundaries; heads [H/2, H) group after a
 * shift of s = G/2 tokens and their outputs land back on the original
 * positions.  Three boundary variants of the shifted heads exist:
 *
 *   S2A_WRAP   -- the original roll: the rolled layout is cut into N/G
 *                 groups, so the last group holds positions
 *                 [N-s .. N-1, 0 .. s-1] with the causal triangle taken in
 *                 that order (queries 0..s-1 read keys N-s..N-1);
 *   S2A_SPLIT  -- the strict-causal variant: groups [0, s),
 *                 [s+kG, s+(k+1)G) for k = 0..N/G-2, and [N-s, N);
 *   S2A_CYCLIC -- the cyclic partition of WRAP with the causal order taken
 *                 on original positions: the last group is
 *                 [0 .. s-1, N-s .. N-1] in that order, so queries
 *                 N-s..N-1 read keys 0..s-1 and nothing reads a later
 *                 position.
 *
 * The first two come from §1's paragraph on cyclic shifts (Figure 1, right
 * and left), the third from §2.2 ("平移分组究竟改变了怎样的信息图"), the
 * mask M^(s) with j <= i and floor(((i+s) mod N)/G) equal for i and j.
 * A padded tail is masked inside every softmax: keys at positions >= the
 * valid length never contribute (§1, paragraph on padding to whole groups).
 * If N/G == 1 the shift has no effect (both head classes are plain causal
 * attention over the whole sequence).
 *
 * Layouts (all tensors dense, row-major, on the device):
 *   q, k, v, dout      bf16  [B, N, H, D]   N = padded length
 *   o                  bf16 or f32 [B, N, H, D]
 *   lse, delta         f32   [B, H, N]      natural log-sum-exp of the
 *                                           scaled logits of each row
 *   dq, dk, dv         f32   [B, N, H, D]
 *   gid, slot, src     int32 [2, N]         index maps, class 0 then 1
 *
 * Ownership and streams: the caller owns every buffer.  The library never
 * allocates, frees or synchronises; work is enqueued on `stream` (a
 * hipStream_t; NULL = the null stream) and is complete when that stream
 * reaches it.  Inputs must not alias outputs.
 *
 * Errors: every argument is checked before anything is enqueued; on an
 * error nothing is written and nothing is launched.  Status codes are
 * returned, never thrown; s2attn_last_error() gives a thread-local
 * description of the last failure on the calling thread.
 */
#ifndef S2ATTN_H
#define S2ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  S2A_OK = 0,
  S2A_EINVAL = 1,       /* bad size, shift, valid length, pointer, scale */
  S2A_EUNSUPPORTED = 2, /* head width D not in {16, 32, 64, 128}          */
  S2A_EHIP = 3          /* a HIP launch failed                            */
} s2a_status;

typedef enum { S2A_WRAP = 0, S2A_SPLIT = 1, S2A_CYCLIC = 2 } s2a_boundary;
typedef enum { S2A_BF16 = 0, S2A_F32 = 1 } s2a_dtype;

/*
 * Forward.  For every head h, group and query x < valid_len with visible
 * set S_x (same group, at or before x in group order, key position <
 * valid_len, and -- if doc_ids is given -- the same document as x):
 *   o[x]   = sum_{y in S_x} softmax_y(scale * q[x].k[y]) v[y]
 *   lse[x] = ln sum_{y in S_x} exp(scale * q[x].k[y])
 * (PaperTrace LongLoRA §3, the equation for o_i^s; the per-row
 * log-sum-exp of §1.1 is kept in place of the probabilities).
 * Rows x >= valid_len get o = 0 and lse = -inf.
 *
 * Arguments: q, k, v bf16 [B,N,H,D]; o of dtype o_dtype [B,N,H,D];
 * lse f32 [B,H,N]; N the padded length; shift 0 (plain grouping) or G/2;
 * valid_len in [1, N]; scale > 0 and finite (1/sqrt(D) in the method).
 * doc_ids: NULL, or int32 [B, N] document IDs of a packed sequence (any
 * values; two positions are in one document iff their IDs are equal): a
 * query then reads only keys of its own document, with the same rule for
 * both head classes (PaperTrace LongLoRA §1.1, paragraph on causal masks
 * and sample packing).  Every valid query still sees itself.
 * Checks (PaperTrace LongLoRA §1, launch-time asserts): H % 2 == 0,
 * G % 2 == 0, N % G == 0, all sizes > 0, tensor pointers non-NULL and
 * 16-byte aligned, doc_ids 4-byte aligned.  Returns S2A_EINVAL /
 * S2A_EUNSUPPORTED / S2A_EHIP / S2A_OK.
 */
s2a_status s2attn_fwd(const void *q, const void *k, const void *v, void *o,
                      int o_dtype, float *lse, int B, int N, int H, int D,
                      int G, int shift, int boundary, int valid_len,
                      const int *doc_ids, float scale, void *stream);

/*
 * Backward.  Given dout = dL/do and the o, lse produced by s2attn_fwd with
 * the same arguments, writes (overwriting) the gradients of L:
 *   a_xy  = exp(scale * q[x].k[y] - lse[x]),  delta_x = dout[x].o[x]
 *   dz_xy = a_xy * (dout[x].v[y] - delta_x)
 *   dq[x] = scale * sum_y dz_xy k[y],  dk[y] = scale * sum_x dz_xy q[x],
 *   dv[y] = sum_x a_xy dout[x]
 * summed over allowed pairs only (PaperTrace LongLoRA §3, the gradient of a
 * logit; §1.1, the backward stays inside the groups).  Rows >= valid_len
 * of dq, dk and dv are exactly 0.
 *
 * delta_ws: caller-provided f32 workspace of B*H*N floats; on return it
 * holds delta_x.  doc_ids: as for s2attn_fwd (the same array).  Every
 * output element is written exactly once (no atomics), so results are
 * bitwise repeatable.
 */
s2a_status s2attn_bwd(const void *q, const void *k, const void *v,
                      const void *o, int o_dtype, const float *lse,
                      const void *dout, float *dq, float *dk, float *dv,
                      float *delta_ws, int B, int N, int H, int D, int G,
                      int shift, int boundary, int valid_len,
                      const int *doc_ids, float scale, void *stream);

/*
 * The backward without any workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, checks and
 * results as s2attn_bwd, bit for bit, minus delta_ws: delta lives in a
 * static device array of the library (one per GPU, held until the process
 * ends) of S2A_NOALLOC_MAX_ROWS floats, so B*H*N must not exceed
 * S2A_NOALLOC_MAX_ROWS (else S2A_EINVAL, nothing enqueued).  Calls no
 * allocating routine.  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (on different streams) race and must be ordered
 * by the caller.
 */
#define S2A_NOALLOC_MAX_ROWS (1 << 22) /* 16 MiB of float */
s2a_status s2attn_bwd_noalloc(const void *q, const void *k, const void *v,
                              const void *o, int o_dtype, const float *lse,
                              const void *dout, float *dq, float *dk,
                              float *dv, int B, int N, int H, int D, int G,
                              int shift, int boundary, int valid_len,
                              const int *doc_ids, float scale, void *stream);

/*
 * The three stages of s2attn_bwd, for callers that schedule or time them
 * separately.  Calling them in this order on one stream equals s2attn_bwd;
 * the last two only read delta_ws and may run in either order or
 * concurrently once it is written.
 *   s2attn_bwd_preprocess  delta_ws[b,h,x] = dout[x].o[x]
 *   s2attn_bwd_dkdv        writes dk and dv (every row)
 *   s2attn_bwd_dq          writes dq (every row)
 * Arguments, layouts and checks are those of s2attn_bwd.
 */
s2a_status s2attn_bwd_preprocess(const void *o, int o_dtype,
                                 const void *dout, float *delta_ws, int B,
                                 int N, int H, int D, void *stream);

s2a_status s2attn_bwd_dkdv(const void *q, const void *k, const void *v,
                           const float *lse, const float *delta_ws,
                           const void *dout, float *dk, float *dv, int B,
                           int N, int H, int D, int G, int shift,
                           int boundary, int valid_len, const int *doc_ids,
                           float scale, void *stream);

s2a_status s2attn_bwd_dq(const void *q, const void *k, const void *v,
                         const float *lse, const float *delta_ws,
                         const void *dout, float *dq, int B, int N, int H,
                         int D, int G, int shift, int boundary,
                         int valid_len, const int *doc_ids, float scale,
                         void *stream);

/*
 * The backward with dS stored instead of recomputed.  Same gradients as
 * s2attn_bwd, to the same tolerance (not bitwise: dQ sums in another
 * order); D in {64, 128} and no document mask.  The dK/dV stage keeps
 * dz_xy (above) in bf16, as its dK product uses it, for every allowed pair
 * in a caller-provided workspace, and the dQ stage forms
 * dq[x] = scale * sum_y dz_xy k[y] from it, so S and dP are computed once
 * (PaperTrace LongLoRA §3: the gradient of a logit is the only term dq
 * needs).  The queries that see fewest keys (the first 128 slots of each
 * group) also keep the bf16 rounding residual of their dz.
 *
 * ds_ws: device workspace of at least s2attn_bwd_ds_workspace() bytes,
 * 16-byte aligned, owned by the caller; its contents are scratch (written
 * by the dK/dV stage, read by the dQ stage; neither zeroes it first, and
 * no output depends on bytes the dK/dV stage did not write).  Calls that
 * may run at the same time (other streams) need workspaces of their own.
 * About 2 bytes per allowed pair: 8.7 GB for B=1, N=32768, H=32, G=8192.
 * Other arguments as for s2attn_bwd.  Errors: S2A_EUNSUPPORTED for other
 * D, S2A_EINVAL for a missing, misaligned or short workspace, as well as
 * every check of s2attn_bwd.
 */
s2a_status s2attn_bwd_ds_workspace(int B, int N, int H, int D, int G,
                                   int shift, int boundary, size_t *bytes);

s2a_status s2attn_bwd_ds(const void *q, const void *k, const void *v,
                         const void *o, int o_dtype, const float *lse,
                         const void *dout, float *dq, float *dk, float *dv,
                         float *delta_ws, void *ds_ws, size_t ds_ws_bytes,
                         int B, int N, int H, int D, int G, int shift,
                         int boundary, int valid_len, float scale,
                         void *stream);

/*
 * The stages of s2attn_bwd_ds after s2attn_bwd_preprocess, for callers
 * that time them separately: s2attn_bwd_dkdv_ds writes dk, dv and fills
 * ds_ws; s2attn_bwd_dq_ds then writes dq (every row) from ds_ws and k
 * alone.  They must run in this order, with the same geometry.
 */
s2a_status s2attn_bwd_dkdv_ds(const void *q, const void *k, const void *v,
                              const float *lse, const float *delta_ws,
                              const void *dout, float *dk, float *dv,
                              void *ds_ws, size_t ds_ws_bytes, int B, int N,
                              int H, int D, int G, int shift, int boundary,
                              int valid_len, float scale, void *stream);

s2a_status s2attn_bwd_dq_ds(const void *k, const void *ds_ws,
                            size_t ds_ws_bytes, float *dq, int B, int N, int H,
                            int D, int G, int shift, int boundary,
                            int valid_len, float scale, void *stream);

/*
 * Group index maps, computed on the device by the same group geometry the
 * attention kernels use (PaperTrace "4.1.2 · LongLoRA", §1: the group
 * functions b(i) = floor(i/G) of the unshifted heads and
 * b'(i) = floor((i - G/2)/G) of the shifted ones, the N=8, G=4 worked
 * example, and the cyclic-shift paragraph for the boundary variants; §2.2
 * for the cyclic-causal partition).  For head class c (0: heads < H/2,
 * 1: the rest) and original position x:
 *   gid[c*N + x]  = group of x,   slot[c*N + x] = rank of x in its group,
 * and for row r of the regrouped layout (groups laid end to end in order):
 *   src[c*N + r]  = original position held at row r.
 * Class 0 groups are [kG, (k+1)G).  Class 1 follows `boundary` (WRAP:
 * N/G groups of the layout rolled left by s; SPLIT: N/G + 1 groups, the
 * first and last of length s; CYCLIC: the groups of WRAP, the last one in
 * position order, so its slots hold 0..s-1 and then N-s..N-1).  The maps do
 * not depend on valid_len (pad first, then shift), which is only
 * validated.
 */
s2a_status s2attn_group_map(int N, int G, int shift, int boundary,
                            int valid_len, int *gid, int *slot, int *src,
                            void *stream);

/*
 * Sequence-parallel shards: the attention of one slice of the sequence,
 * as one of several devices holding consecutive slices would run it.
 * PaperTrace LongLoRA §1.1 (the paragraphs on sequence-parallel
 * communication): when rank boundaries fall on the unshifted groups'
 * boundaries, only the shifted heads' groups cross them, and each slice
 * needs the s = G/2 preceding tokens' K and V from its neighbour (a halo);
 * the backward sends the gradients of those keys back.  Exchanging the
 * halo is the caller's (a point-to-point send/receive per layer); these
 * calls compute everything else.
 *
 * The slice is rows [row0, row0 + T) of a sequence of padded length N
 * (one batch row), with row0 and T multiples of G.  Within it, heads are
 * grouped exactly as by s2attn_fwd over the whole sequence, so the slices
 * together give the same results (bit for bit wherever no halo partial
 * sum is involved).
 *
 * s2attn_shard_halo (host only, no device work) names the halo rows:
 *   left halo  global rows [*left_first, *left_first + *left_rows): the
 *              rows before the slice in the shifted heads' group order
 *              (row0-s .. row0-1; for the first slice under WRAP the valid
 *              rows of N-s .. N-1; none for the first slice otherwise);
 *   wrap halo  global rows [0, *wrap_rows): only the last slice under
 *              CYCLIC (whose last shifted group starts with rows 0..s-1).
 * Layouts (B = 1):
 *   q, dout, o, dq    [T, H, D]  the slice's rows
 *   k, v              point at the slice's row 0, [T, H, D] from there;
 *                     the left halo must sit in the *left_rows rows just
 *                     before it (k - left_rows*H*D ..), the wrap halo in
 *                     rows [-2s, -2s + wrap_rows) relative to it
 *   dk, dv            f32, the same layout as k: rows [0, T) get this
 *                     slice's gradients; the halo rows of the shifted heads
 *                     get the partial gradients this slice's queries give
 *                     the neighbours' keys, to be sent back and added to
 *                     their rows; other halo rows are not written
 *   doc_ids           NULL, or int32 in k's layout (the halo rows' IDs
 *                     included)
 *   lse, delta_ws     f32 [H, T]
 * Rows of the slice and of the halos must hold finite values (padded rows
 * included).  valid_len is that of the whole sequence; rows at or past it
 * are masked and zeroed as in s2attn_fwd / s2attn_bwd.  The shifted heads'
 * dk, dv rows [T-s, T) of every slice but the last (under WRAP the last
 * one's too) and, under CYCLIC, rows [0, s) of the first are partial
 * until the halo partials that other slices computed for them are added.
 * Checks: those of s2attn_fwd with B = 1, plus 0 <= row0, T > 0, row0 and
 * T multiples of G, row0 + T <= N.
 */
s2a_status s2attn_shard_halo(int N, int row0, int T, int G, int shift,
                             int boundary, int valid_len, int *left_first,
                             int *left_rows, int *wrap_rows);

s2a_status s2attn_fwd_shard(const void *q, const void *k, const void *v,
                            void *o, int o_dtype, float *lse, int N, int row0,
                            int T, int H, int D, int G, int shift,
                            int boundary, int valid_len, const int *doc_ids,
                            float scale, void *stream);

s2a_status s2attn_bwd_shard(const void *q, const void *k, const void *v,
                            const void *o, int o_dtype, const float *lse,
                            const void *dout, float *dq, float *dk, float *dv,
                            float *delta_ws, int N, int row0, int T, int H,
                            int D, int G, int shift, int boundary,
                            int valid_len, const int *doc_ids, float scale,
                            void *stream);

/*
 * Rotary position embedding (RoPE) at global positions: the prologue that
 * turns projected q and k into the rotated q and k the attention calls
 * take.  For pair i of every head (i = 0 .. D/2-1) at token (b, n):
 *   m      = pos_scale * (pos_ids ? pos_ids[b*N + n] : n)
 *   w_i    = base^(-2i/D)
 *   (y_a, y_b) = (cos(m w_i) x_a - sin(m w_i) x_b,
 *                 sin(m w_i) x_a + cos(m w_i) x_b)
 * with channels (a, b) = (i, i + D/2) for S2A_ROPE_HALF (the Llama layout)
 * or (2i, 2i + 1) for S2A_ROPE_INTERLEAVED.  The rotation is the R(m, w) of
 * PaperTrace LongLoRA §3.1; m is the token's original position ID -- the
 * shift of the grouped heads only permutes tensors -- and linear position
 * interpolation is pos_scale = L0 / L1 (§1.1, the paragraphs on RoPE and
 * position interpolation).  The frequency schedule and the pairing are not
 * fixed by the pages; these are the conventions of the Llama models the
 * pages fine-tune.
 *
 * s2attn_rope:      x, y bf16 [B, N, H, D]; y = R x, angles formed in
 *                   double precision, the rotation in fp32, rounded once.
 * s2attn_rope_bwd:  gy, gx f32 [B, N, H, D]; gx = R^T gy (the gradient of
 *                   s2attn_rope with respect to x, given that of y).
 * pos_ids: NULL or int32 [B, N] (4-byte aligned); y may equal x and gx may
 * equal gy (in place).  Checks: sizes > 0, D in {16, 32, 64, 128}
 * (S2A_EUNSUPPORTED otherwise), pointers non-NULL and 16-byte aligned,
 * base and pos_scale positive and finite, pairing one of the two values.
 */
typedef enum { S2A_ROPE_HALF = 0, S2A_ROPE_INTERLEAVED = 1 } s2a_rope_pairing;

s2a_status s2attn_rope(const void *x, void *y, int B, int N, int H, int D,
                       const int *pos_ids, float base, float pos_scale,
                       int pairing, void *stream);

s2a_status s2attn_rope_bwd(const float *gy, float *gx, int B, int N, int H,
                           int D, const int *pos_ids, float base,
                           float pos_scale, int pairing, void *stream);

/* Static description of a status code. */
const char *s2attn_strerror(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char *s2attn_last_error(void);

/* Library version string. */
const char *s2attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* S2ATTN_H */
