/*
 * attn.h -- C ABI of libattn.so: causal grouped-query flash attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes softmax attention without ever writing a score or
 * probability matrix to device memory.  The softmax maximum and its two sums
 * are folded into one streaming reduction over keys that carries three running
 * values per query row (running max, running sum, running weighted sum of
 * values) -- the rewrite described in "tang -- differentiable computing in
 * Rust", section "How tang works", part 3 "Optimizations are derived, not
 * written" (equations (5) and (6)); the combine is associative, which is what
 * lets the keys be tiled and split.  The gradient is the gradient of the same
 * reduction, recomputed tile by tile (same part 3, and the compiler article
 * "A compiler that derives GPU kernels matches hand-tuned code", paragraph on
 * views and comprehensions).  Shapes follow the grouped-query statement of the
 * problem in the "RustingBrain" docs ("What is in the box"; "A language model
 * in twenty lines": query heads, key/value heads, head dim).
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, owned by the caller.  The library
 *    allocates no device memory, creates no streams or events and keeps no
 *    state between calls (save the device address of attn_bwd_noalloc's
 *    array, resolved once per device): every call is re-entrant and may be
 *    captured into a HIP graph (including the first call of a process).
 *  - Layouts are contiguous row-major with the head dimension fastest:
 *        q, dout, o, dq      [B][Hq][N][d]
 *        k, v, dk, dv        [B][Hkv][N][d]
 *        lse                 [B][Hq][N]
 *  - Input dtype (q, k, v, dout, caches) is ATTN_F32 (IEEE float) or ATTN_BF16
 *    (bfloat16, stored as 16-bit words).  Every output (o, lse, dq, dk, dv,
 *    decode partials) is float32 for both input dtypes.
 *  - Grouped-query head map: query head h reads key/value head h / (Hq/Hkv)
 *    (contiguous groups).  Hq must be a multiple of Hkv.
 *  - Causal mask: key j is visible to query i iff j <= i.
 *  - lse is the natural-log log-sum-exp of the row's scaled scores.
 *  - scale multiplies q.k (normally 1/sqrt(d)); it must be finite.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns at once.  ATTN_OK means the work was enqueued; results
 *    are valid after the caller synchronises the stream.
 *  - Errors are fail-closed: every argument is checked on the host before any
 *    launch, and an invalid call launches nothing and leaves every output
 *    untouched.  There is no host fallback: the work runs on the GPU or the call
 *    returns an error.  No C++ exception crosses this boundary.
 *  - Pointers must be non-null and 16-byte aligned.
 *  - Supported head dims: 16, 32, 64, 128.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,  /* a dim <= 0, Hq % Hkv != 0, null or misaligned pointer,
                                  non-finite scale, n_splits < 1, bad dtype code */
    ATTN_ERR_UNSUPPORTED = 2,  /* head dim outside {16,32,64,128}, or a size beyond the
                                  documented limits (see each entry point) */
    ATTN_ERR_WORKSPACE = 3,    /* workspace null or smaller than attn_bwd_workspace_bytes */
    ATTN_ERR_HIP = 4           /* a HIP launch reported an error */
} attn_status;

typedef enum {
    ATTN_F32 = 0,
    ATTN_BF16 = 1
} attn_dtype;

/*
 * attn_fwd -- causal (or full) grouped-query attention forward.
 *   Per query row: o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the
 *   visible keys, and lse_i = log sum_j exp(scale * q_i . k_j).
 *   Source: "How tang works" part 3 (the streaming softmax reduction); the
 *   causal fused kernel of the RustingBrain docs ("What is in the box").
 *   q [B][Hq][N][d], k/v [B][Hkv][N][d] of dtype dt -> o [B][Hq][N][d] f32,
 *   lse [B][Hq][N] f32.  causal: nonzero for the causal mask.
 */
attn_status attn_fwd(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     const void *q, const void *k, const void *v,
                     float *o, float *lse, void *stream);

/*
 * attn_fwd_kv -- the forward for Nq queries against Nk >= Nq keys, the queries
 *   being the last Nq positions: query row i sits at key position
 *   i + (Nk - Nq), and with causal it sees keys 0 .. i + (Nk - Nq).  This is
 *   a chunk of new tokens prefilled against a cache that already holds the
 *   first Nk - Nq ("RustingBrain" docs, "Generating text": only the new tokens
 *   are computed, the cache supplies the rest).  Nq = Nk is attn_fwd; Nq = 1
 *   is one decode row.
 *   q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] of dtype dt -> o [B][Hq][Nq][d] f32,
 *   lse [B][Hq][Nq] f32.  Nq <= 0 or Nk < Nq: ATTN_ERR_INVALID_ARG; other
 *   checks as attn_fwd.  Buffers caller-owned; one launch on `stream`.
 */
attn_status attn_fwd_kv(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, const void *q, const void *k, const void *v, float *o,
                        float *lse, void *stream);

/*
 * attn_bwd_workspace_bytes -- device workspace attn_bwd needs, in bytes:
 *   one f32 per query row, D_i = dout_i . o_i, rounded up to 256 bytes.
 *   Returns 0 for invalid shapes.
 */
size_t attn_bwd_workspace_bytes(attn_dtype dt, int B, int Hq, int Hkv, int N, int d);

/*
 * attn_bwd -- gradient of attn_fwd's o with respect to q, k and v, given the
 *   upstream gradient dout of o (the upstream gradient of lse is taken as 0).
 *   With P the softmax probabilities (recomputed tile by tile from q, k and
 *   lse, never stored), D_i = dout_i . o_i, dP_ij = dout_i . v_j and
 *   dS_ij = P_ij (dP_ij - D_i):
 *     dq_i = scale sum_j dS_ij k_j
 *     dk_j = scale sum_{h in group} sum_i dS_ij q_i
 *     dv_j = sum_{h in group} sum_i P_ij dout_i
 *   Source: "How tang works" part 3 (gradients of the reduction are
 *   reductions too) and the compiler article's paragraph on comprehensions.
 *   o and lse must be the outputs of attn_fwd for the same q, k, v, causal,
 *   scale.  dq [B][Hq][N][d], dk/dv [B][Hkv][N][d] are f32 and overwritten.
 *   dq is bitwise deterministic.  When the key tiles alone are too few to fill
 *   the GPU, dk and dv sum the query heads of a group with f32 atomics and may
 *   then differ from run to run in the last bits.
 *   workspace: device memory of at least attn_bwd_workspace_bytes(...) bytes,
 *   owned by the caller; its contents on entry do not matter.
 *   Launches, all on `stream`: for bf16 inputs at d = 128 (f32 o) the dq
 *   kernel computes delta itself (into the workspace) and the dk/dv kernel
 *   follows it.  Otherwise the preprocess runs, then the gradients as
 *   described at attn_bwd_grads.
 */
attn_status attn_bwd(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     const void *q, const void *k, const void *v,
                     const float *o, const float *lse, const void *dout,
                     float *dq, float *dk, float *dv,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 *   or pass a workspace (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid allocation).  The row terms D_i live in a device
 *   array of the library instead of a caller workspace: 4 MiB per device,
 *   held for the life of the process, so B * Hq * N may be at most 2^20
 *   (larger shapes return ATTN_ERR_WORKSPACE and launch nothing).  The
 *   array's device address is resolved on the first call on each device
 *   (ATTN_ERR_HIP if it cannot be); no call allocates or frees anything.
 *   Every call on a device shares that device's array: calls that overlap
 *   on one device (on different streams, or from several threads) race and
 *   give wrong results; calls in stream order are safe (the array needs no
 *   clearing: each call writes every D_i before reading it).  Arguments,
 *   outputs, launches and every other check as attn_bwd.
 */
attn_status attn_bwd_noalloc(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                             float scale, const void *q, const void *k, const void *v,
                             const float *o, const float *lse, const void *dout,
                             float *dq, float *dk, float *dv, void *stream);

/*
 * attn_bwd_dlse -- attn_bwd with an upstream gradient of lse as well:
 *   dlse [B][Hq][N] f32 (device, 16-byte aligned, read only).  Since
 *   d lse_i / d s_ij = P_ij, it enters as dS_ij = P_ij (dP_ij - D_i + dlse_i),
 *   i.e. the preprocess writes D_i - dlse_i into the workspace and the
 *   gradient stage is unchanged.  Needed wherever lse itself is consumed, e.g.
 *   when partial attention outputs are merged by their log-sum-exp (split-KV,
 *   ring attention: "How tang works" part 3, the associative combine).
 *   Everything else as attn_bwd.
 */
attn_status attn_bwd_dlse(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, const void *q, const void *k, const void *v,
                          const float *o, const float *lse, const void *dout, const float *dlse,
                          float *dq, float *dk, float *dv, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * attn_bwd_kv -- the backward of attn_fwd_kv: Nq query rows against Nk >= Nq
 *   keys, query row i at key position i + (Nk - Nq) (under causal it sees keys
 *   0 .. i + (Nk - Nq), so key j receives gradient from query rows
 *   i >= j - (Nk - Nq)).  Same sums as attn_bwd over the visible pairs; this
 *   is the gradient of a prefill chunk against a cache, and of one block pair
 *   of ring attention ("How tang works" part 3: the reduction over keys and
 *   its gradient do not depend on where the keys sit).
 *   q, dout [B][Hq][Nq][d] and k, v [B][Hkv][Nk][d] of dtype dt; o, lse from
 *   attn_fwd_kv with the same arguments; dlse [B][Hq][Nq] f32 or NULL (no
 *   upstream gradient of lse; otherwise as attn_bwd_dlse).  dq [B][Hq][Nq][d],
 *   dk/dv [B][Hkv][Nk][d] f32, overwritten.  workspace: at least
 *   attn_bwd_workspace_bytes(dt, B, Hq, Hkv, Nq, d) bytes.  Nq <= 0 or
 *   Nk < Nq: ATTN_ERR_INVALID_ARG; Nq = Nk is attn_bwd (or attn_bwd_dlse).
 *   Streams, determinism and every other check as attn_bwd.
 */
attn_status attn_bwd_kv(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, const void *q, const void *k, const void *v,
                        const float *o, const float *lse, const void *dout, const float *dlse,
                        float *dq, float *dk, float *dv, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * attn_fwd_ex -- the general forward: attn_fwd_kv (Nq <= Nk, bottom-right
 *   causal) with the output dtype chosen by o_dt: ATTN_F32 (as attn_fwd_kv),
 *   or ATTN_BF16 (o rounded to nearest even, half the bytes written and read
 *   back by the backward; lse stays f32).  o [B][Hq][Nq][d] of dtype o_dt.
 *   o_dt other than these two: ATTN_ERR_INVALID_ARG; other checks as
 *   attn_fwd_kv.  One launch on `stream`.
 */
attn_status attn_fwd_ex(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                        int d, int causal, float scale, const void *q, const void *k,
                        const void *v, void *o, float *lse, void *stream);

/*
 * attn_bwd_ex -- the general backward: attn_bwd_kv taking o in dtype o_dt
 *   (the output of attn_fwd_ex with the same o_dt); dlse may be NULL.
 *   Gradients stay f32.  Other arguments and checks as attn_bwd_kv.
 */
attn_status attn_bwd_ex(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                        int d, int causal, float scale, const void *q, const void *k,
                        const void *v, const void *o, const float *lse, const void *dout,
                        const float *dlse, float *dq, float *dk, float *dv, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * attn_bwd_bf16grad_workspace_bytes -- device workspace attn_bwd_bf16grad
 *   needs, in bytes: the row terms of attn_bwd_ex, then f32 copies of dq, dk
 *   and dv (each section rounded up to 256 bytes).  Returns 0 for invalid
 *   shapes (as attn_bwd_ex would refuse them).
 */
size_t attn_bwd_bf16grad_workspace_bytes(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk,
                                         int d);

/*
 * attn_bwd_bf16grad -- attn_bwd_ex with the gradients written in bf16: dq
 *   [B][Hq][Nq][d], dk/dv [B][Hkv][Nk][d], each the f32 gradient of attn_bwd_ex
 *   (same formulas: "How tang works" part 3) rounded to nearest even.  The
 *   pages fix no output precision; the gradients are accumulated in f32 and
 *   rounded once.  The f32 gradients are computed into the workspace (at least
 *   attn_bwd_bf16grad_workspace_bytes(...) bytes, caller-owned, contents on
 *   entry irrelevant; dq, dk, dv must not overlap it) and then rounded by one
 *   more launch on `stream`, so the call moves the f32 gradients through HBM
 *   twice more than attn_bwd_ex.  dq, dk, dv 16-byte aligned.  Other
 *   arguments, checks and error codes as attn_bwd_ex; a short workspace gives
 *   ATTN_ERR_WORKSPACE.
 */
attn_status attn_bwd_bf16grad(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                              int d, int causal, float scale, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, const void *dout,
                              const float *dlse, void *dq, void *dk, void *dv, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Strides of a 4-D tensor [B][H][N][d] whose head dim is contiguous, in
 * elements: element (b, h, n, c) sits at b*batch + h*head + n*row + c.  The
 * contiguous layout is {H*N*d, N*d, d}; interleaved heads ([B][N][H][d], as
 * a fused projection writes them) are {N*H*d, d, H*d}.  Every stride must be
 * positive, row >= d and at most 2^31 - 1, and each a multiple of 16 bytes of
 * the tensor's element size (so every row starts 16-byte aligned).  Tensors
 * the call writes must not overlap one another or the inputs.
 */
typedef struct {
    long long batch;
    long long head;
    long long row;
} attn_layout;

/*
 * attn_fwd_strided -- attn_fwd_ex over tensors of any strides: each of q, k,
 *   v, o comes with its attn_layout (NULL: contiguous).  lse stays contiguous
 *   [B][Hq][Nq] f32.  The matrix-core kernels read the strided rows directly
 *   (one buffer resource per head, its row stride in the tile copies), as
 *   long as each bf16 head spans less than 2^31 bytes; otherwise the generic
 *   kernels run.  A layout that breaks the rules above: ATTN_ERR_INVALID_ARG.
 *   "RustingBrain" docs, "Generating text": caches and activations are read
 *   where the caller keeps them.  Other arguments, checks and launches as
 *   attn_fwd_ex.
 */
attn_status attn_fwd_strided(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, float scale, const void *q, const attn_layout *lq,
                             const void *k, const attn_layout *lk, const void *v,
                             const attn_layout *lv, void *o, const attn_layout *lo, float *lse,
                             void *stream);

/*
 * attn_bwd_strided -- attn_bwd_ex over tensors of any strides: q, k, v, o,
 *   dout, dq, dk, dv each with its attn_layout (NULL: contiguous); lse, dlse
 *   and the workspace stay contiguous.  dk and dv are written with plain
 *   stores (the query heads of a group are never split over workgroups, which
 *   would need a zero-fill that follows their strides).  Other arguments,
 *   checks and launches as attn_bwd_ex.
 */
attn_status attn_bwd_strided(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, float scale, const void *q, const attn_layout *lq,
                             const void *k, const attn_layout *lk, const void *v,
                             const attn_layout *lv, const void *o, const attn_layout *lo,
                             const float *lse, const void *dout, const attn_layout *ldout,
                             const float *dlse, float *dq, const attn_layout *ldq, float *dk,
                             const attn_layout *ldk, float *dv, const attn_layout *ldv,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_rope -- rotary positions on rows: x, y [B][H][N][d] of dtype dt, row n
 *   of each head at position pos0 + n.  For pair i in [0, d/2),
 *   theta_i = base^(-2i/d), a = position * theta_i:
 *     y_i = x_i cos a - x_{i+d/2} sin a,   y_{i+d/2} = x_i sin a + x_{i+d/2} cos a;
 *   inverse != 0 applies the transposed rotation (angle -a), which carries a
 *   gradient with respect to y back to x.  The pages list rotary positions
 *   beside grouped-query attention ("tang": the "A transformer" panel;
 *   RustingBrain docs, "What is in the box") without a formula; this is the
 *   usual rotation on paired halves of the head dimension.  Angles are reduced
 *   in double precision before f32 sine and cosine.  x and y may be the same
 *   buffer (device, 16-byte aligned).  base > 0 and finite, |pos0| <= 2^40,
 *   d in {16, 32, 64, 128}; otherwise ATTN_ERR_INVALID_ARG / ATTN_ERR_UNSUPPORTED.
 *   One launch on `stream`.
 */
attn_status attn_rope(attn_dtype dt, int B, int H, int N, int d, long long pos0, double base,
                      int inverse, const void *x, void *y, void *stream);

/*
 * attn_fwd_rope -- attn_fwd_kv over rotated queries and keys: q_rot =
 *   rope(q) with query row i at position i + (Nk - Nq), k_rot = rope(k) with
 *   key j at position j (so scores depend on the positions' difference), then
 *   the forward on (q_rot, k_rot, v).  q_rot [B][Hq][Nq][d] and k_rot
 *   [B][Hkv][Nk][d] (dtype dt, caller-owned, may alias q and k) receive the
 *   rotated inputs: attn_bwd_rope takes them, and k_rot is what a key cache
 *   holds.  Two launches on `stream`.  On the bf16 matrix-core path (q_rot
 *   not aliasing q): one pass rotates k, and the forward rotates each query
 *   row as it loads it (hardware sine and cosine of the angle reduced in
 *   double, about 1e-6, rounded to bf16: q_rot is within one bf16 unit in the
 *   last place of attn_rope's) and writes q_rot.  Otherwise one pass rotates
 *   q and k (as attn_rope) before the forward.  Other arguments and checks as
 *   attn_fwd_kv and attn_rope.
 */
attn_status attn_fwd_rope(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, double base, const void *q, const void *k, const void *v,
                          void *q_rot, void *k_rot, float *o, float *lse, void *stream);

/*
 * attn_bwd_rope -- the backward of attn_fwd_rope: attn_bwd_kv at the rotated
 *   inputs q_rot, k_rot (from attn_fwd_rope), with dq and dk carried back to
 *   the unrotated q and k by the transposed rotations: in the gradient
 *   kernels' epilogues on the bf16 matrix-core path (hardware sine and cosine
 *   of the angle reduced in double, about 1e-6), else by one more launch.  dq, dk, dv
 *   are the gradients with respect to q, k, v.  dlse may be NULL.  Arguments,
 *   workspace, streams and checks as attn_bwd_kv and attn_rope.
 */
attn_status attn_bwd_rope(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, double base, const void *q_rot, const void *k_rot,
                          const void *v, const float *o, const float *lse, const void *dout,
                          const float *dlse, float *dq, float *dk, float *dv, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * The three stages attn_bwd runs, callable one by one (for example to put the
 * dK/dV stage and the dQ stage on two streams once delta is ready, or to time
 * them).  Arguments mean the same as in attn_bwd; delta [B][Hq][N] f32 is
 * caller-owned device memory holding D_i = dout_i . o_i.
 *
 * attn_bwd_preprocess -- writes delta from o (f32) and dout (dtype dt).
 * attn_bwd_dkdv       -- writes dk and dv; reads q, k, v, lse, dout, delta.
 * attn_bwd_dq         -- writes dq; reads q, k, v, lse, dout, delta.
 * attn_bwd_grads      -- writes dq, dk and dv from a given delta: on the bf16
 *                        matrix-core path at d = 64 ONE kernel launch whose
 *                        grid holds both the dk/dv and the dq work items (after
 *                        a zero-fill launch of dk and dv when they are
 *                        accumulated with atomics), as attn_bwd runs it after
 *                        its preprocess (see attn_bwd_grads_plan); otherwise
 *                        the dq kernel, then the dk/dv kernel, on `stream`.
 * dkdv and dq do not depend on each other; all need the preprocess first.
 */
attn_status attn_bwd_preprocess(attn_dtype dt, int B, int Hq, int N, int d,
                                const float *o, const void *dout, float *delta, void *stream);
attn_status attn_bwd_dkdv(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, const void *q, const void *k, const void *v,
                          const float *lse, const void *dout, const float *delta,
                          float *dk, float *dv, void *stream);
attn_status attn_bwd_dq(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                        float scale, const void *q, const void *k, const void *v,
                        const float *lse, const void *dout, const float *delta,
                        float *dq, void *stream);
attn_status attn_bwd_grads(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                           float scale, const void *q, const void *k, const void *v,
                           const float *lse, const void *dout, const float *delta,
                           float *dq, float *dk, float *dv, void *stream);

/*
 * attn_bwd_grads_plan -- 1 when attn_bwd_grads (and the gradient part of
 *   attn_bwd / attn_bwd_kv) runs dq, dk and dv as ONE kernel for this shape,
 *   else 0 (also 0 for arguments attn_bwd_kv would refuse).  The one kernel
 *   orders its blocks by a host-side plan of at most 48 block groups, passed
 *   as a kernel argument; a shape whose plan cannot be made to fit (the group
 *   caps shrink until it does) runs the two gradient kernels instead.  When
 *   groups / blocks are non-null they receive the plan's group count and grid
 *   size (0 when the result is 0).  Nq == Nk for attn_bwd.  No device work.
 */
int attn_bwd_grads_plan(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, int *groups, int *blocks);

/*
 * attn_decode -- split-KV attention of one new query token per (b, query head)
 *   against a cache of L keys, all of which are visible to it (the token sits
 *   after the cache).  Source: RustingBrain docs, "Generating text" (after the
 *   prefill each token costs one row of attention against the cache); the
 *   split is legal because the softmax combine is associative ("How tang
 *   works" part 3).
 *   The keys are cut into n_splits contiguous chunks of C = ceil(L / n_splits)
 *   keys; chunk s covers [s*C, min((s+1)*C, L)).  For each chunk the call
 *   writes the chunk's normalised output and log-sum-exp:
 *     part_o[b][h][s][:]  = sum_{j in chunk} softmax_j(scale q . k_j) v_j
 *     part_lse[b][h][s]   = log sum_{j in chunk} exp(scale q . k_j)
 *   An empty chunk (possible when n_splits > L) gets part_o = 0 and
 *   part_lse = -inf.
 *   q [B][Hq][d], k_cache/v_cache [B][Hkv][L][d] of dtype dt;
 *   part_o [B][Hq][n_splits][d] f32, part_lse [B][Hq][n_splits] f32.
 *   Combine the partials with attn_lse_merge.
 *   Limits: Hq/Hkv <= 16.
 */
attn_status attn_decode(attn_dtype dt, int B, int Hq, int Hkv, int L, int d, float scale,
                        int n_splits, const void *q, const void *k_cache, const void *v_cache,
                        float *part_o, float *part_lse, void *stream);

/*
 * attn_lse_merge -- associative merge of split partials by their log-sum-exp:
 *     M = max_s lse_s,  w_s = exp(lse_s - M),
 *     o = sum_s w_s o_s / sum_s w_s,   lse = M + log sum_s w_s.
 *   If every chunk is empty (M = -inf) the result is o = 0, lse = -inf.
 *   Source: "How tang works" part 3 (the combine is associative, so it tiles
 *   and parallelises like a sum).
 *   part_o [B][Hq][n_splits][d], part_lse [B][Hq][n_splits] f32
 *   -> o [B][Hq][d] f32, lse [B][Hq] f32.
 */
attn_status attn_lse_merge(int B, int Hq, int n_splits, int d,
                           const float *part_o, const float *part_lse,
                           float *o, float *lse, void *stream);

/*
 * attn_decode_merged -- attn_decode followed by attn_lse_merge, enqueued by
 *   one call (two launches on `stream`).  part_o and part_lse are written as by
 *   attn_decode, o [B][Hq][d] and lse [B][Hq] as by attn_lse_merge; argument
 *   checks are those of both calls and an invalid call launches nothing.
 *   (A single-launch form, in which the last workgroup of each (batch, kv
 *   head) merges after a device-scope release, measured slower on MI355X:
 *   the release writes back and invalidates L2.)
 */
attn_status attn_decode_merged(attn_dtype dt, int B, int Hq, int Hkv, int L, int d, float scale,
                               int n_splits, const void *q, const void *k_cache,
                               const void *v_cache, float *part_o, float *part_lse, float *o,
                               float *lse, void *stream);

/*
 * attn_decode_append -- one decode step of B sequences of their own lengths
 *   against caches that grow by one token per step.  Source: RustingBrain
 *   docs, "Generating text" (after the prefill each new token's key and value
 *   join the cache, and the token costs one row of attention over it); the
 *   split and merge are those of attn_decode / attn_lse_merge.
 *   For sequence b with n = seq_lens[b] tokens already cached:
 *     1. k_new[b][g] and v_new[b][g] are written to cache row n of every kv
 *        head g (the caller then counts the sequence as n + 1 long);
 *     2. every query head h of the group attends over the n + 1 keys 0..n
 *        (all visible: the token sits after the cache), split into n_splits
 *        chunks of ceil((n + 1) / n_splits) keys, then merged:
 *        o[b][h] = softmax(scale q.K^T) V, lse[b][h] = log-sum-exp.
 *   q [B][Hq][d], k_new / v_new [B][Hkv][d]: dtype dt (bf16 only; d 64 or 128,
 *   Hq/Hkv <= 16, scale != 0, L_cap * d * 2 + 65536 < 2^31; anything else
 *   returns ATTN_ERR_UNSUPPORTED).
 *   k_cache / v_cache [B][Hkv][L_cap][d] dt: read at rows < n, written at row
 *   n only.  seq_lens [B] int32 device memory, read only (4-byte aligned).
 *   part_o [B][Hq][n_splits][d], part_lse [B][Hq][n_splits] f32 scratch as in
 *   attn_decode (chunks past n hold (0, -inf)); o [B][Hq][d], lse [B][Hq] f32.
 *   All buffers caller-owned device memory; the call enqueues two launches on
 *   `stream` (the decode kernel, then the merge) and allocates nothing.
 *   A length outside [0, L_cap) is not an error the host can see: that
 *   sequence's cache is left untouched and its o and lse come out NaN.
 */
attn_status attn_decode_append(attn_dtype dt, int B, int Hq, int Hkv, int L_cap, int d,
                               float scale, int n_splits, const void *q, const void *k_new,
                               const void *v_new, void *k_cache, void *v_cache,
                               const int *seq_lens, float *part_o, float *part_lse, float *o,
                               float *lse, void *stream);

/*
 * attn_read_probe -- a reference, not part of attention: reads `bytes` bytes at
 *   src once (16-byte loads, many in flight on every compute unit) and writes
 *   nothing but, practically never, a sentinel word to *out.  A decode step is
 *   bound by reading the cache once (RustingBrain docs, "Generating text"), so
 *   the time of this call over the same bytes is the decode kernels' measured
 *   floor.  src: device, 16-byte aligned; bytes: a positive multiple of 16,
 *   at most 2^40; out: device, 4-byte aligned.  One launch on `stream`.
 */
attn_status attn_read_probe(const void *src, size_t bytes, unsigned *out, void *stream);

/* Human-readable name of a status code (a static string). */
const char *attn_status_str(attn_status s);

/* Version of this ABI; bumped on any incompatible change. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
