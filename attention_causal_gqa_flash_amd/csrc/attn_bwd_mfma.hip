// attn_bwd_mfma.hip -- causal grouped-query attention backward on gfx950
// matrix cores (bf16 operands, f32 accumulation).
//
// The gradient of the streaming softmax reduction is itself a reduction
// ("tang -- differentiable computing in Rust", "How tang works" part 3; the
// compiler article "A compiler that derives GPU kernels matches hand-tuned
// code", paragraph on views and comprehensions): with P recomputed tile by tile
// from q, k and the forward's log-sum-exp,
//     D_i = dO_i . O_i,   dP = dO V^T,   dS = P o (dP - D),
//     dV = P^T dO,        dK = scale dS^T Q,   dQ = scale dS K,
// and no P or dS tile ever reaches device memory.
//
// Two kernels:
//   * dkdv: key-stationary.  A workgroup owns 64 keys of one key/value head and
//     keeps their dK^T and dV^T accumulators in registers while it streams the
//     query tiles of every query head of the group past them.  4 waves = 2 key
//     blocks x 2 query halves, each wave a 32x32 (query x key) tile per step;
//     scores are laid out S = Q K^T (lane = key column), so P and dS feed the
//     dV and dK MFMAs straight from registers, and Q^T, dO^T come from the
//     row-major Q and dO tiles through the transposed LDS read.  The two query
//     halves' partials are summed through LDS at the end.  When the key tiles
//     alone are too few to fill the GPU, the group's query heads are split
//     over several workgroups whose partial dK/dV are added with f32 atomics
//     (so dK/dV are then order-dependent in the last bits).
//   * dq (deterministic): query-stationary, the forward's layout (lane = query row, S^T = K Q^T)
//     with dQ^T = K^T dS^T accumulated in registers; P and dP are recomputed,
//     K^T is read from the row-major K tile through the transposed LDS read.
// Both double-buffer their LDS tiles (row-major, 16-byte chunks XOR-swizzled by
// row), filled by direct global->LDS loads with the next step's loads in
// flight during the current step's MFMAs, one barrier per step.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#include <vector>

namespace attn {

// Block order of the one-launch backward: plan.n groups of blocks; group i
// starts at block first[i] and holds consecutive levels of one kind (0: dK/dV
// key tiles, lev0 first and ascending; 1: dQ query tiles, lev0 first and
// descending), each level padded to a multiple of kXcds blocks.  A dK/dV
// group's key tiles split each query-head group over hs[i] work items.
struct BwdPlan {
    static constexpr int kMax = 48;
    int n;
    int first[kMax + 1];
    int lev0[kMax];
    int kind[kMax];
    int hs[kMax];
};

namespace {

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kKvBN = 64;   // keys per workgroup
constexpr int kKvBM = 64;   // queries per sub-step (the two query halves of the waves)
constexpr int kKvSub = 2;   // sub-steps per step: one LDS buffer holds 128 query rows

// One (64-query sub-step, 32x32 block) of the dK/dV kernel for one wave, in
// three phases: S = Q K^T and dP = dO V^T (lane = key column); P = 2^(c2 s -
// lse log2 e) and dS = P (dP - D); then dV^T += dO^T P and dK^T += Q^T dS
// over the block's 32 queries.  With `mask` (wave-uniform: causal diagonal
// blocks) keys after the query get P = 0.  Query rows past Nq need no mask:
// their Q and dO rows and their lse and D read as zero, so P = 1 there and
// every product they feed (dV += P^T dO, dK += dS^T Q with dS = P (dP - D) =
// 0) adds exact zeros.
constexpr int kAhead = 8;    // operand reads issued ahead of the score MFMAs
constexpr int kAheadT = 8;   // ... and of the dV/dK MFMAs
// (measured on the 32/8-head N = 4096 dK/dV kernel: 4 ahead 374 us, 8 ahead
// 354 us, 12 or 16 ahead slower again)

template <int D>
__device__ __forceinline__ void dkdv_scores(const uint16_t *qt, const uint16_t *dt,
                                            const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                            f32x16 &sacc, f32x16 &pacc, int qh, int lane)
{
    constexpr int KS = D / 16;
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 aq = tile_row_operand<D>(qt, 32 * qh + l32, 2 * ks + hf);
        const bf16x8 ad = tile_row_operand<D>(dt, 32 * qh + l32, 2 * ks + hf);
        sacc = mfma32x32x16(aq, kf[ks], sacc);
        pacc = mfma32x32x16(ad, vf[ks], pacc);
    }
}

// The row terms of the block's rows as the initial S and dP accumulators
// (register r: local row 32qh + 8(r/4) + 4hf + r%4): the LDS row arrays hold
// -lse_i / |scale| and -D_i, so the MFMAs leave q.k - lse_i / |scale| and
// dP - D_i, and P = 2^(c2 (q.k - lse_i / |scale|)) = e^(scale q.k - lse_i)
// takes one multiply and one exponential per score.
__device__ __forceinline__ void dkdv_rows(const float *lt, const float *ddt, int qh, int lane,
                                          f32x16 &sacc, f32x16 &pacc)
{
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int rr = 32 * qh + 8 * a + 4 * (lane >> 5);
        const float4 l = *(const float4 *)&lt[rr];
        const float4 d = *(const float4 *)&ddt[rr];
        sacc[4 * a + 0] = l.x; sacc[4 * a + 1] = l.y; sacc[4 * a + 2] = l.z; sacc[4 * a + 3] = l.w;
        pacc[4 * a + 0] = d.x; pacc[4 * a + 1] = d.y; pacc[4 * a + 2] = d.z; pacc[4 * a + 3] = d.w;
    }
}

__device__ __forceinline__ void dkdv_probs(f32x16 &sacc, f32x16 &pacc, float c2, bool mask, int t)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = exp2_fast(sacc[r] * c2);
    // Register r holds query row q0 + 32qh + 4hf + c, c = 8(r/4) + r%4 (a
    // constant): the causal mask keeps c >= t = kj - off - (q0 + 32qh + 4hf)
    // (key kj is visible to query rows at or after kj - off), one compare and
    // one select per score.
    if (mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = 8 * (r >> 2) + (r & 3);
            sacc[r] = c >= t ? sacc[r] : 0.f;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] *= sacc[r];
}

// dV^T += dO^T P,  dK^T += Q^T dS   (contraction over the wave's 32 queries)
template <int D>
__device__ __forceinline__ void dkdv_grads(const uint16_t *qt, const uint16_t *dt, const f32x16 &sacc,
                                           const f32x16 &pacc, f32x16 (&dka)[D / 32],
                                           f32x16 (&dva)[D / 32], int qh, int lane)
{
    constexpr int DB = D / 32;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 pb = tt ? pack_operand<8>(sacc) : pack_operand<0>(sacc);
        const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const bf16x8 ado = tr_operand<D>(dt, 32 * qh + 16 * tt, db * 32, lane);
            const bf16x8 aqt = tr_operand<D>(qt, 32 * qh + 16 * tt, db * 32, lane);
            dva[db] = mfma32x32x16(ado, pb, dva[db]);
            dka[db] = mfma32x32x16(aqt, sb, dka[db]);
        }
    }
}

// One sub-step, the three phases in sequence (the block's row terms are read
// first: they are the score accumulators' initial values).  kq = kj - off: the
// first query row that sees this lane's key.
template <int D>
__device__ __forceinline__ void dkdv_block(const uint16_t *qt, const uint16_t *dt, const float *lt,
                                           const float *ddt, const bf16x8 (&kf)[D / 16],
                                           const bf16x8 (&vf)[D / 16], f32x16 (&dka)[D / 32],
                                           f32x16 (&dva)[D / 32], float c2, int qh, int q0, int kq,
                                           bool mask, int lane)
{
    constexpr int KS = D / 16, DB = D / 32;
    f32x16 sacc, pacc;
    dkdv_rows(lt, ddt, qh, lane, sacc, pacc);
    dkdv_scores<D>(qt, dt, kf, vf, sacc, pacc, qh, lane);
    sched_pipeline<2 * KS + 8, 2 * KS, kAhead + 8, 1>();
    dkdv_probs(sacc, pacc, c2, mask, kq - (q0 + 32 * qh + 4 * (lane >> 5)));
    dkdv_grads<D>(qt, dt, sacc, pacc, dka, dva, qh, lane);
    sched_pipeline<8 * DB, 4 * DB, kAheadT, 2>();
}

// The LDS of the dK/dV work: double-buffered Q, dO, lse and D tiles of
// kKvSub * kKvBM query rows, each buffer an array of its own (see Buf).  The
// dQ work uses the first kQBN rows of the Q and dO arrays as its
// double-buffered K and V tiles.
template <int D>
struct BwdLds {
    static constexpr int SR = kKvSub * kKvBM;   // query rows per dK/dV step
    uint16_t *q0s, *q1s, *d0s, *d1s;
    float *l0s, *l1s, *e0s, *e1s;
};

#define ATTN_BWD_LDS(D_, name)                                                                    \
    __shared__ __attribute__((aligned(16))) uint16_t name##q0[BwdLds<D_>::SR * D_],                \
        name##q1[BwdLds<D_>::SR * D_], name##d0[BwdLds<D_>::SR * D_], name##d1[BwdLds<D_>::SR * D_]; \
    __shared__ __attribute__((aligned(16))) float name##l0[BwdLds<D_>::SR], name##l1[BwdLds<D_>::SR], \
        name##e0[BwdLds<D_>::SR], name##e1[BwdLds<D_>::SR];                                       \
    const BwdLds<D_> name{name##q0, name##q1, name##d0, name##d1, name##l0, name##l1, name##e0, name##e1}

// dK/dV of key tile kt for work item `item` = (batch, kv head, head subset),
// Nq query rows against Nk >= Nq keys, query row i at key position i + Nk - Nq
// (so under the causal mask key j is seen by query rows i >= j - (Nk - Nq)):
// the G query heads of a group are split into hs subsets of Gs heads; with
// hs > 1 the subsets' partial dK/dV are summed with atomics into zero-filled
// outputs.  The copy of step s+1 has the two sub-steps of step s to land; at
// the end the four tile arrays hold the dK^T / dV^T partials of the two query
// halves.  XL = false compiles the square case (Nk taken equal to Nq).
template <int D, bool XL, bool STR = false>
__device__ __forceinline__ void dkdv_body(
    int kt, int item, const BwdLds<D> &lds, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int hs,
    double rope_lb, const Layouts &L = Layouts{})
{
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int SR = BwdLds<D>::SR;
    if constexpr (!XL) Nk = Nq;
    // XL = false: a literal 0, folded before the compiler shapes the loop's branches
    // (Nk - Nq with Nk = Nq was folded too late and cost 2% in the loop)
    const int off = XL ? Nk - Nq : 0;
    uint16_t *const q0s = lds.q0s, *const q1s = lds.q1s, *const d0s = lds.d0s, *const d1s = lds.d1s;
    float *const l0s = lds.l0s, *const l1s = lds.l1s, *const e0s = lds.e0s, *const e1s = lds.e1s;

    const int grp = item / hs, hsub = item % hs;
    const int b = grp / Hkv, g = grp % Hkv;
    const int G = Hq / Hkv, Gs = G / hs;
    const int k0 = kt * kKvBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l32 = lane & 31, hf = lane >> 5;
    const int kb = wave & 1, qh = wave >> 1;
    const int kj = k0 + 32 * kb + l32;       // this lane's key column

    const uint32_t ksign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    // strides of the 4-D tensors (STR: the caller's; else contiguous [B][H][N][D])
    const TL lq = STR ? L.q : contiguous_tl(Hq, Nq, D), ldo = STR ? L.dout : contiguous_tl(Hq, Nq, D);
    const TL lk = STR ? L.k : contiguous_tl(Hkv, Nk, D), lv = STR ? L.v : contiguous_tl(Hkv, Nk, D);
    const TL ldk = STR ? L.dk : contiguous_tl(Hkv, Nk, D), ldv = STR ? L.dv : contiguous_tl(Hkv, Nk, D);
    const uint16_t *Kg = K + b * lk.b + g * lk.h;
    const uint16_t *Vg = V + b * lv.b + g * lv.h;

    // K^T and V^T operands, resident: lane holds row kj, dims 16ks + 8hf .. +7.
    // The key tile's K and V rows move global -> LDS directly (whole rows,
    // rows past Nk read as zero and are never stored), into the second Q and
    // dO buffers, which step 1's copy fills only after step 0 has read them.
    bf16x8 kf[KS], vf[KS];
    {
        const TileCopy<D, kKvBN, 4> kcopy(wave, lane, lk.n), vcopy(wave, lane, lv.n);
        kcopy(q1s, make_rsrc(Kg, head_bytes(Nk, lk.n, D, 2)), k0, wave);
        vcopy(d1s, make_rsrc(Vg, head_bytes(Nk, lv.n, D, 2)), k0, wave);
    }
    auto read_kv = [&] {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 uk = *(const uint4 *)tile_chunk<D>(q1s, 32 * kb + l32, 2 * ks + hf);
            const uint4 uv = *(const uint4 *)tile_chunk<D>(d1s, 32 * kb + l32, 2 * ks + hf);
            uk.x ^= ksign; uk.y ^= ksign; uk.z ^= ksign; uk.w ^= ksign;
            kf[ks] = as_bf16x8(uk);
            vf[ks] = as_bf16x8(uv);
        }
    };

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dva[db][r] = 0.f; dka[db][r] = 0.f; }

    const int nqt = (Nq + SR - 1) / SR;
    const int qt0 = causal ? (XL ? max(k0 - off, 0) : k0) / SR : 0;
    const int nq = nqt - qt0;
    const int steps = Gs * nq;               // (query head, query tile) pairs

    // Step s covers query head g*G + hsub*Gs + s/nq, query rows (qt0 + s%nq)*SR
    // .. +SR-1.  Its Q and dO tiles move global -> LDS directly; its lse and
    // D rows go through a register of waves 0/1 (the two halves of lse) and
    // 2/3 (those of D), which store them as -lse / |scale| and -D at the top
    // of the step.  Rows past Nq read as zero and are masked in the step's
    // arithmetic.
    const uint32_t q_bytes = head_bytes(Nq, lq.n, D, 2), do_bytes = head_bytes(Nq, ldo.n, D, 2);
    const uint32_t row_bytes = (uint32_t)Nq * 4;
    const TileCopy<D, SR, 4> copy(wave, lane, lq.n), dcopy(wave, lane, ldo.n);
    const float row_mul = wave < 2 ? -1.f / fabsf(scale) : -1.f;
    float row_v = 0.f;                       // this lane's row term of the next step
    auto load_step = [&](int s_, uint16_t *qd, uint16_t *dd) {
        const int hq = g * G + hsub * Gs + s_ / nq;
        const size_t hrow = ((size_t)b * Hq + hq) * Nq;
        const int q0_ = (qt0 + s_ % nq) * SR;
        copy(qd, make_rsrc(Q + b * lq.b + hq * lq.h, q_bytes), q0_, wave);
        dcopy(dd, make_rsrc(dO + b * ldo.b + hq * ldo.h, do_bytes), q0_, wave);
        const int half = wave & 1;
        row_v = row_load(make_rsrc((wave < 2 ? LSE : Dws) + hrow, row_bytes), q0_ + 64 * half, lane);
    };
    if (steps > 0) load_step(0, q0s, d0s);
    // The resident K and V operands as soon as their copies have landed (they
    // were issued before step 0's copies and its row load, and loads complete
    // in order), while step 0's copies are still in flight; step 0's barrier
    // then also tells every wave that buffer 1 is free for step 1's copies.
    if (steps > 0) wait_vmcnt<2 * decltype(copy)::PER_WAVE + 1>();
    else wait_vmcnt<0>();
    lds_barrier();
    read_kv();

    auto run_step = [&](auto bufc, int s) {
        constexpr int BI = decltype(bufc)::value;
        const uint16_t *qc = BI ? q1s : q0s, *dc = BI ? d1s : d0s;
        float *lc = BI ? l1s : l0s, *ec = BI ? e1s : e0s;
        wait_vmcnt<0>();                    // this wave's copies of step s have landed
        (wave < 2 ? lc : ec)[64 * (wave & 1) + lane] = row_v * row_mul;
        __syncthreads();                    // ... and every wave's; buffer s+1 is free
        if (s + 1 < steps) {
            if (BI) load_step(s + 1, q0s, d0s);
            else load_step(s + 1, q1s, d1s);
        }
        const int qs = (qt0 + s % nq) * SR;  // first query row of the step
#pragma unroll
        for (int sub = 0; sub < kKvSub; ++sub) {
            const int q0 = qs + sub * kKvBM;
            const int qb0 = q0 + 32 * qh;   // first query row of this wave's block
            if (qb0 < Nq && k0 + 32 * kb < Nk && (!causal || qb0 + 31 + off >= k0 + 32 * kb)) {
                const bool mask = causal && qb0 + off < k0 + 32 * kb + 32;
                dkdv_block<D>(qc + sub * kKvBM * D, dc + sub * kKvBM * D, lc + sub * kKvBM,
                              ec + sub * kKvBM, kf, vf, dka, dva, c2, qh, q0, kj - off, mask, lane);
            }
        }
        sched_fence();
    };
    for (int s = 0; s < steps; s += 2) {
        run_step(Buf<0>{}, s);
        if (s + 1 < steps) run_step(Buf<1>{}, s + 1);
    }

    // Sum the two query halves and write dK = scale (dK^T)^T and dV.
    // Accumulator layout: lane = key column kj, register r of block db = dim
    // db*32 + 8(r/4) + 4hf + (r&3): registers 4a..4a+3 are four consecutive
    // dims.  The query-half-1 waves park their partials in the tile arrays
    // (one array per (key block, dK or dV)) transposed to [key][dim], four
    // dims per 16-byte write, the half-0 waves add theirs in place, so that
    // the final stores (or atomics) run along the dim with consecutive lanes.
    // Key row r keeps its 16-byte chunk c at c ^ (r mod NC): the XOR spreads
    // the rows written by one instruction over the banks and keeps each row a
    // permutation of its chunks.
    static_assert(32 * D * sizeof(float) <= SR * D * sizeof(uint16_t), "transposed partial fits");
    constexpr int NC = D / 4;                                      // 16-byte chunks per row
    auto pidx = [](int row, int dim) { return row * D + 4 * ((dim >> 2) ^ (row & (NC - 1))) + (dim & 3); };
    float *redk = reinterpret_cast<float *>(kb ? q1s : q0s);
    float *redv = reinterpret_cast<float *>(kb ? d1s : d0s);
    wait_vmcnt<0>();                         // (no step: the K/V copies have landed)
    __syncthreads();                         // the last step's reads are done
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int at = pidx(l32, db * 32 + 8 * a + 4 * hf);
                *(float4 *)&redk[at] = make_float4(dka[db][4 * a], dka[db][4 * a + 1], dka[db][4 * a + 2],
                                                   dka[db][4 * a + 3]);
                *(float4 *)&redv[at] = make_float4(dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2],
                                                   dva[db][4 * a + 3]);
            }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int at = pidx(l32, db * 32 + 8 * a + 4 * hf);
                const float4 pk = *(const float4 *)&redk[at];
                const float4 pv = *(const float4 *)&redv[at];
                *(float4 *)&redk[at] = make_float4((pk.x + dka[db][4 * a]) * scale, (pk.y + dka[db][4 * a + 1]) * scale,
                                                   (pk.z + dka[db][4 * a + 2]) * scale,
                                                   (pk.w + dka[db][4 * a + 3]) * scale);
                *(float4 *)&redv[at] = make_float4(pv.x + dva[db][4 * a], pv.y + dva[db][4 * a + 1],
                                                   pv.z + dva[db][4 * a + 2], pv.w + dva[db][4 * a + 3]);
            }
    }
    __syncthreads();
    // all 4 waves write: wave w takes key rows w, w+4, ... of the 64-key tile,
    // lanes along the dim; every LDS read is issued before the first store
    constexpr int RPW = kKvBN / 4, CPR = D / 64;   // rows per wave, 64-dim chunks per row
    float vk[RPW * CPR], vv[RPW * CPR];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int kr = wave + 4 * i;
        const float *sk = reinterpret_cast<const float *>((kr >> 5) ? q1s : q0s);
        const float *sv = reinterpret_cast<const float *>((kr >> 5) ? d1s : d0s);
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const int src = pidx(kr & 31, 64 * c + lane);
            vk[i * CPR + c] = sk[src];
            vv[i * CPR + c] = sv[src];
        }
    }
    // rope_lb != 0: dK was taken at rotated keys; the transposed rotation of
    // key `key` carries it back (dim and its partner dim ^ D/2 of the same row)
    if (rope_lb != 0.0) {
        // every value of this lane is dim 64c + lane: one pair index, one frequency
        const double th = rope_theta(lane & (D / 2 - 1), D, rope_lb);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int kr = wave + 4 * i;
            const float *sk = reinterpret_cast<const float *>((kr >> 5) ? q1s : q0s);
            float sn, cs;
            rope_sincos_hw((double)(k0 + kr) * th, sn, cs);
#pragma unroll
            for (int c = 0; c < CPR; ++c) {
                const int dim = 64 * c + lane;
                const float partner = sk[pidx(kr & 31, dim ^ (D / 2))];
                vk[i * CPR + c] = vk[i * CPR + c] * cs + (dim < D / 2 ? sn : -sn) * partner;
            }
        }
    }
    float *dKg = dK + b * ldk.b + g * ldk.h;
    float *dVg = dV + b * ldv.b + g * ldv.h;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int key = k0 + wave + 4 * i;
        if (key < Nk) {
#pragma unroll
            for (int c = 0; c < CPR; ++c) {
                const size_t atk = (size_t)key * ldk.n + 64 * c + lane;
                const size_t atv = (size_t)key * ldv.n + 64 * c + lane;
                if (hs == 1) {
                    dKg[atk] = vk[i * CPR + c];
                    dVg[atv] = vv[i * CPR + c];
                } else {
                    atomicAdd(dKg + atk, vk[i * CPR + c]);
                    atomicAdd(dVg + atv, vv[i * CPR + c]);
                }
            }
        }
    }
}

// d = 128 needs more than the 256 registers of two waves per SIMD (K, V
// operands 64 + dK, dV accumulators 128 + scores 32 + operands in flight):
// it runs one wave per SIMD with up to 512.
template <int D, bool XL, bool STR = false>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int hs,
    double rope_lb, Layouts L)
{
    ATTN_BWD_LDS(D, lds);
    if constexpr (!XL) Nk = Nq;
    // XCD-aware (see xcd_work_item): a group's Q and dO rows stay in one L2,
    // the heaviest key tiles (causal: the lowest) first.
    const int nkt = (Nk + kKvBN - 1) / kKvBN;
    WorkItem w;
    if (!xcd_work_item(blockIdx.x, B * Hkv, nkt, hs, w)) return;
    dkdv_body<D, XL, STR>(nkt - 1 - w.tile, w.group * hs + w.head, lds, Q, K, V, LSE, dO, Dws, dK, dV, B,
                          Hq, Hkv, Nq, Nk, scale, causal, hs, rope_lb, L);
}

// ---------------------------------------------------------------------------
// dK, dV with paired roles (d = 128): two waves per SIMD
// ---------------------------------------------------------------------------
// The kernel above holds, per wave, the K and V operands of its 32 keys and
// both the dK and the dV accumulators (about 356 registers at d = 128), so it
// runs one wave per SIMD: while that wave waits on LDS reads or works through
// the softmax, the matrix core idles.  Here the work of a (32-query, 32-key)
// block is split between two waves of the same SIMD:
//   * role P (waves 0-3): K operand resident; S = Q K^T, P = e^(scale S - lse)
//     (masked), P handed over through LDS, then dV^T += dO^T P;
//   * role G (waves 4-7): V operand resident; dP = dO V^T, then, with P from
//     LDS, dS = P (dP - D) and dK^T += Q^T dS.
// Each wave keeps one operand (32 registers) and one accumulator set (64),
// about 200 registers in all, so eight waves fit a CU (two per SIMD; a wave
// and its partner, w and w + 4, share a SIMD) and one wave's MFMAs overlap
// the other's softmax and LDS waits.  P crosses as bf16 (the precision it has
// as an MFMA operand anyway) in a per-lane slot of LDS, double-buffered by
// sub-step; one barrier per sub-step orders the hand-over.  Work items, the
// step loop over query heads and 128-row query tiles, and the epilogue are
// those of the kernel above.
constexpr int kPairWaves = 8;

template <int D>
struct BwdPairLds {
    static constexpr int SR = kKvSub * kKvBM;   // query rows per step
    uint16_t *q0s, *q1s, *d0s, *d1s;
    float *l0s, *l1s, *e0s, *e1s;
    uint4 *pbuf;                                // [sub][pair][2][64 lanes]
};

template <int D, bool XL, bool STR = false>
__device__ __forceinline__ void dkdv_pair_body(
    int kt, int item, const BwdPairLds<D> &lds, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int hs,
    double rope_lb, const Layouts &L = Layouts{})
{
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int SR = BwdPairLds<D>::SR;
    if constexpr (!XL) Nk = Nq;
    const int off = XL ? Nk - Nq : 0;
    uint16_t *const q0s = lds.q0s, *const q1s = lds.q1s, *const d0s = lds.d0s, *const d1s = lds.d1s;
    float *const l0s = lds.l0s, *const l1s = lds.l1s, *const e0s = lds.e0s, *const e1s = lds.e1s;

    const int grp = item / hs, hsub = item % hs;
    const int b = grp / Hkv, g = grp % Hkv;
    const int G = Hq / Hkv, Gs = G / hs;
    const int k0 = kt * kKvBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l32 = lane & 31, hf = lane >> 5;
    const bool role_p = wave < 4;            // P and dV; else dP and dK
    const int pair = wave & 3;
    const int kb = wave & 1, qh = (wave >> 1) & 1;
    const int kj = k0 + 32 * kb + l32;       // this lane's key column

    const uint32_t ksign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    // strides of the 4-D tensors (STR: the caller's; else contiguous [B][H][N][D])
    const TL lq = STR ? L.q : contiguous_tl(Hq, Nq, D), ldo = STR ? L.dout : contiguous_tl(Hq, Nq, D);
    const TL lk = STR ? L.k : contiguous_tl(Hkv, Nk, D), lv = STR ? L.v : contiguous_tl(Hkv, Nk, D);
    const TL ldk = STR ? L.dk : contiguous_tl(Hkv, Nk, D), ldv = STR ? L.dv : contiguous_tl(Hkv, Nk, D);
    const uint16_t *Kg = K + b * lk.b + g * lk.h;
    const uint16_t *Vg = V + b * lv.b + g * lv.h;

    // the resident operand: K^T (role P) or V^T (role G), rows of the key
    // tile copied global -> LDS whole into the second Q / dO buffers first
    bf16x8 opf[KS];
    {
        const TileCopy<D, kKvBN, kPairWaves> kcopy(wave, lane, lk.n), vcopy(wave, lane, lv.n);
        kcopy(q1s, make_rsrc(Kg, head_bytes(Nk, lk.n, D, 2)), k0, wave);
        vcopy(d1s, make_rsrc(Vg, head_bytes(Nk, lv.n, D, 2)), k0, wave);
    }
    auto read_op = [&] {
        const uint16_t *src = role_p ? q1s : d1s;
        const uint32_t sign = role_p ? ksign : 0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = *(const uint4 *)tile_chunk<D>(src, 32 * kb + l32, 2 * ks + hf);
            u.x ^= sign; u.y ^= sign; u.z ^= sign; u.w ^= sign;
            opf[ks] = as_bf16x8(u);
        }
    };

    f32x16 acc[DB];                          // dV^T (role P) or dK^T (role G)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const int nqt = (Nq + SR - 1) / SR;
    const int qt0 = causal ? (XL ? max(k0 - off, 0) : k0) / SR : 0;
    const int nq = nqt - qt0;
    const int steps = Gs * nq;

    const uint32_t q_bytes = head_bytes(Nq, lq.n, D, 2), do_bytes = head_bytes(Nq, ldo.n, D, 2);
    const uint32_t row_bytes = (uint32_t)Nq * 4;
    const TileCopy<D, SR, kPairWaves> copy(wave, lane, lq.n), dcopy(wave, lane, ldo.n);
    // row terms: waves 0/1 load the two halves of lse, 2/3 those of D
    const float row_mul = wave < 2 ? -1.f / fabsf(scale) : -1.f;
    float row_v = 0.f;
    auto load_step = [&](int s_, uint16_t *qd, uint16_t *dd) {
        const int hq = g * G + hsub * Gs + s_ / nq;
        const size_t hrow = ((size_t)b * Hq + hq) * Nq;
        const int q0_ = (qt0 + s_ % nq) * SR;
        copy(qd, make_rsrc(Q + b * lq.b + hq * lq.h, q_bytes), q0_, wave);
        dcopy(dd, make_rsrc(dO + b * ldo.b + hq * ldo.h, do_bytes), q0_, wave);
        if (wave < 4)
            row_v = row_load(make_rsrc((wave < 2 ? LSE : Dws) + hrow, row_bytes), q0_ + 64 * (wave & 1), lane);
    };
    if (steps > 0) load_step(0, q0s, d0s);

    auto run_step = [&](auto bufc, int s) {
        constexpr int BI = decltype(bufc)::value;
        const uint16_t *qc = BI ? q1s : q0s, *dc = BI ? d1s : d0s;
        float *lc = BI ? l1s : l0s, *ec = BI ? e1s : e0s;
        wait_vmcnt<0>();                    // this wave's copies of step s have landed
        if (wave < 4) (wave < 2 ? lc : ec)[64 * (wave & 1) + lane] = row_v * row_mul;
        __syncthreads();                    // ... and every wave's; buffer s+1 is free
        if constexpr (BI == 0) {
            if (s == 0) {                   // the resident operand, then buffer 1 is free
                read_op();
                __syncthreads();
            }
        }
        if (s + 1 < steps) {
            if (BI) load_step(s + 1, q0s, d0s);
            else load_step(s + 1, q1s, d1s);
        }
        const int qs = (qt0 + s % nq) * SR;
        // Phase 1 of both sub-steps, then one barrier, then phase 2 of both:
        // while role P works through a sub-step's softmax, role G (on the
        // same SIMD) issues the score MFMAs of the next one, and role G's dS
        // arithmetic overlaps role P's dV MFMAs.
        bool active[kKvSub];
        f32x16 acc1[kKvSub];                 // role G: dP - D of each sub-step
        bf16x8 pk[kKvSub][2];                // role P: P of each sub-step as bf16 operands
#pragma unroll
        for (int sub = 0; sub < kKvSub; ++sub) {
            const int q0 = qs + sub * kKvBM;
            const int qb0 = q0 + 32 * qh;
            active[sub] = qb0 < Nq && k0 + 32 * kb < Nk && (!causal || qb0 + 31 + off >= k0 + 32 * kb);
            const bool mask = causal && qb0 + off < k0 + 32 * kb + 32;
            const uint16_t *qt = qc + sub * kKvBM * D, *dt = dc + sub * kKvBM * D;
            uint4 *pb = lds.pbuf + (sub * 4 + pair) * 128;
            if (active[sub]) {
                // phase 1: S (role P) or dP (role G) from the row term up
                f32x16 sacc;
                const float *rt = role_p ? lc + sub * kKvBM : ec + sub * kKvBM;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 t = *(const float4 *)&rt[32 * qh + 8 * a + 4 * hf];
                    sacc[4 * a + 0] = t.x; sacc[4 * a + 1] = t.y;
                    sacc[4 * a + 2] = t.z; sacc[4 * a + 3] = t.w;
                }
                const uint16_t *src = role_p ? qt : dt;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sacc = mfma32x32x16(tile_row_operand<D>(src, 32 * qh + l32, 2 * ks + hf), opf[ks], sacc);
                sched_pipeline<KS + 4, KS, 8, 1>();
                if (role_p) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[r] = exp2_fast(sacc[r] * c2);
                    if (mask) {
                        const int t = kj - off - (q0 + 32 * qh + 4 * hf);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int c = 8 * (r >> 2) + (r & 3);
                            sacc[r] = c >= t ? sacc[r] : 0.f;
                        }
                    }
                    pk[sub][0] = pack_operand<0>(sacc);
                    pk[sub][1] = pack_operand<8>(sacc);
                    pb[lane] = __builtin_bit_cast(uint4, pk[sub][0]);
                    pb[64 + lane] = __builtin_bit_cast(uint4, pk[sub][1]);
                } else {
                    acc1[sub] = sacc;
                }
            }
        }
        __syncthreads();                    // every P of the step is in LDS
#pragma unroll
        for (int sub = 0; sub < kKvSub; ++sub) {
            if (!active[sub]) continue;
            const uint16_t *qt = qc + sub * kKvBM * D, *dt = dc + sub * kKvBM * D;
            const uint4 *pb = lds.pbuf + (sub * 4 + pair) * 128;
            bf16x8 op0, op1;
            if (role_p) {
                op0 = pk[sub][0];
                op1 = pk[sub][1];
            } else {
                // dS = P (dP - D): P from the partner, in this lane's layout
                const uint4 p0 = pb[lane], p1 = pb[64 + lane];
                const f32x16 &dp = acc1[sub];
                f32x16 ds;
                ds[0] = bf16lo(p0.x) * dp[0]; ds[1] = bf16hi(p0.x) * dp[1];
                ds[2] = bf16lo(p0.y) * dp[2]; ds[3] = bf16hi(p0.y) * dp[3];
                ds[4] = bf16lo(p0.z) * dp[4]; ds[5] = bf16hi(p0.z) * dp[5];
                ds[6] = bf16lo(p0.w) * dp[6]; ds[7] = bf16hi(p0.w) * dp[7];
                ds[8] = bf16lo(p1.x) * dp[8]; ds[9] = bf16hi(p1.x) * dp[9];
                ds[10] = bf16lo(p1.y) * dp[10]; ds[11] = bf16hi(p1.y) * dp[11];
                ds[12] = bf16lo(p1.z) * dp[12]; ds[13] = bf16hi(p1.z) * dp[13];
                ds[14] = bf16lo(p1.w) * dp[14]; ds[15] = bf16hi(p1.w) * dp[15];
                op0 = pack_operand<0>(ds);
                op1 = pack_operand<8>(ds);
            }
            // phase 2: dV^T += dO^T P (role P) or dK^T += Q^T dS (role G)
            const uint16_t *src = role_p ? dt : qt;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = mfma32x32x16(tr_operand<D>(src, 32 * qh + 16 * tt, db * 32, lane),
                                           tt ? op1 : op0, acc[db]);
            sched_pipeline<4 * DB, 2 * DB, 8, 2>();
        }
        sched_fence();
    };
    for (int s = 0; s < steps; s += 2) {
        run_step(Buf<0>{}, s);
        if (s + 1 < steps) run_step(Buf<1>{}, s + 1);
    }

    // Sum the two query halves: the half-1 waves park their partials in the
    // tile arrays transposed to [key][dim] (dV of key block kb in the Q
    // arrays, dK in the dO arrays), the half-0 waves add theirs in place, then
    // all eight waves store (or add atomically) along the dim.  Key row r
    // keeps its 16-byte chunk c at c ^ (r mod NC).
    static_assert(32 * D * sizeof(float) <= SR * D * sizeof(uint16_t), "transposed partial fits");
    constexpr int NC = D / 4;
    auto pidx = [](int row, int dim) { return row * D + 4 * ((dim >> 2) ^ (row & (NC - 1))); };
    float *red = reinterpret_cast<float *>(role_p ? (kb ? q1s : q0s) : (kb ? d1s : d0s));
    const float amul = role_p ? 1.f : scale;
    wait_vmcnt<0>();
    __syncthreads();
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(float4 *)&red[pidx(l32, db * 32 + 8 * a + 4 * hf)] =
                    make_float4(acc[db][4 * a], acc[db][4 * a + 1], acc[db][4 * a + 2], acc[db][4 * a + 3]);
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int at = pidx(l32, db * 32 + 8 * a + 4 * hf);
                const float4 pv = *(const float4 *)&red[at];
                *(float4 *)&red[at] = make_float4((pv.x + acc[db][4 * a]) * amul, (pv.y + acc[db][4 * a + 1]) * amul,
                                                  (pv.z + acc[db][4 * a + 2]) * amul,
                                                  (pv.w + acc[db][4 * a + 3]) * amul);
            }
    }
    __syncthreads();
    // wave w takes key rows w, w + 8, ... of the tile, lanes along the dim
    constexpr int RPW = kKvBN / kPairWaves, CPR = D / 64;
    float vk[RPW * CPR], vv[RPW * CPR];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int kr = wave + kPairWaves * i;
        const float *sk = reinterpret_cast<const float *>((kr >> 5) ? d1s : d0s);
        const float *sv = reinterpret_cast<const float *>((kr >> 5) ? q1s : q0s);
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const int dim = 64 * c + lane;
            const int src = pidx(kr & 31, dim) + (dim & 3);
            vk[i * CPR + c] = sk[src];
            vv[i * CPR + c] = sv[src];
        }
    }
    if (rope_lb != 0.0) {
        const double th = rope_theta(lane & (D / 2 - 1), D, rope_lb);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int kr = wave + kPairWaves * i;
            const float *sk = reinterpret_cast<const float *>((kr >> 5) ? d1s : d0s);
            float sn, cs;
            rope_sincos_hw((double)(k0 + kr) * th, sn, cs);
#pragma unroll
            for (int c = 0; c < CPR; ++c) {
                const int dim = 64 * c + lane;
                const int pd = dim ^ (D / 2);
                const float partner = sk[pidx(kr & 31, pd) + (pd & 3)];
                vk[i * CPR + c] = vk[i * CPR + c] * cs + (dim < D / 2 ? sn : -sn) * partner;
            }
        }
    }
    float *dKg = dK + b * ldk.b + g * ldk.h;
    float *dVg = dV + b * ldv.b + g * ldv.h;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int key = k0 + wave + kPairWaves * i;
        if (key < Nk) {
#pragma unroll
            for (int c = 0; c < CPR; ++c) {
                const size_t atk = (size_t)key * ldk.n + 64 * c + lane;
                const size_t atv = (size_t)key * ldv.n + 64 * c + lane;
                if (hs == 1) {
                    dKg[atk] = vk[i * CPR + c];
                    dVg[atv] = vv[i * CPR + c];
                } else {
                    atomicAdd(dKg + atk, vk[i * CPR + c]);
                    atomicAdd(dVg + atv, vv[i * CPR + c]);
                }
            }
        }
    }
}

template <int D, bool XL, bool STR = false>
__global__ __launch_bounds__(64 * kPairWaves, 1) void bwd_dkdv_pair_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int hs,
    double rope_lb, Layouts L)
{
    constexpr int SR = BwdPairLds<D>::SR;
    __shared__ __attribute__((aligned(16))) uint16_t q0[SR * D], q1[SR * D], d0[SR * D], d1[SR * D];
    __shared__ __attribute__((aligned(16))) float l0[SR], l1[SR], e0[SR], e1[SR];
    __shared__ __attribute__((aligned(16))) uint4 pbuf[kKvSub * 4 * 2 * 64];
    const BwdPairLds<D> lds{q0, q1, d0, d1, l0, l1, e0, e1, pbuf};
    if constexpr (!XL) Nk = Nq;
    const int nkt = (Nk + kKvBN - 1) / kKvBN;
    WorkItem w;
    if (!xcd_work_item(blockIdx.x, B * Hkv, nkt, hs, w)) return;
    dkdv_pair_body<D, XL, STR>(nkt - 1 - w.tile, w.group * hs + w.head, lds, Q, K, V, LSE, dO, Dws, dK,
                               dV, B, Hq, Hkv, Nq, Nk, scale, causal, hs, rope_lb, L);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kQBM = 128;   // queries per workgroup (32 per wave)
constexpr int kQBN = 64;    // keys per tile

// One 64-key tile of the dQ kernel for one wave (lane = query row): S^T = K Q^T
// and dP^T = V dO^T per 32-key block, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// `prefetch` issues NV direct copies (the next tile), interleaved with the
// first block's MFMAs.  qk: the lane's query row as a key position (the last
// key it sees under the causal mask).
template <int D, int NV, class Prefetch>
__device__ __forceinline__ void dq_tile(const uint16_t *skb, const uint16_t *svb, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&dof)[D / 16], f32x16 (&dqa)[D / 32], float c2,
                                        float lse2, const f32x16 &negD, int kv0, int qk, int Nk, int causal,
                                        bool mask, int lane, const Prefetch &prefetch)
{
    constexpr int KS = D / 16, DB = D / 32;
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb == 0) prefetch();
        // dP^T starts from -D_i (the lane's row): the MFMAs leave dP^T - D_i
        f32x16 sacc, pacc = negD;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ak = tile_row_operand<D>(skb, kb * 32 + l32, 2 * ks + hf);
            const bf16x8 av = tile_row_operand<D>(svb, kb * 32 + l32, 2 * ks + hf);
            sacc = mfma32x32x16(ak, qf[ks], sacc);
            pacc = mfma32x32x16(av, dof[ks], pacc);
        }
        if (kb == 0) sched_pipeline<2 * KS, 2 * KS, 4, 1, NV>();
        else sched_pipeline<2 * KS, 2 * KS, 4, 1>();
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = exp2_fast(fmaf(sacc[r], c2, -lse2));
        if (mask) {   // keys kv0 + 32kb + 4hf + c (c constant) kept iff c < lim
            const int lim = (causal ? min(qk + 1, Nk) : Nk) - (kv0 + kb * 32 + 4 * hf);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = 8 * (r >> 2) + (r & 3);
                sacc[r] = c < lim ? sacc[r] : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * pacc[r];
        // dQ^T += K^T dS^T over this block's 32 keys (two 16-key steps)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dqa[db] = mfma32x32x16(tr_operand<D>(skb, kb * 32 + 16 * tt, db * 32, lane), sb, dqa[db]);
        }
        sched_pipeline<4 * DB, 2 * DB, 4, 2>();
    }
}

// dQ of query tile qt for work item `item` = (batch, query head), Nq query
// rows against Nk >= Nq keys (query row i at key position i + Nk - Nq; XL =
// false compiles the square case).  K and V tiles, row-major with swizzled
// 16-byte chunks, double-buffered in the first kQBN rows of the Q and dO
// arrays of `lds`.  STAGE (arrays of kQBM rows or more): the tile's Q and dO
// rows for the resident operands go global -> LDS directly (whole rows) into
// the second arrays, which tile 1's copy fills only after tile 0 read them.
// PRE (not with STAGE): the rows' D_i = dO_i . O_i - dlse_i is computed here,
// from O (f32) and the dO operands the lane holds, and written to Dws for a
// dK/dV kernel that runs afterwards.
template <int D, bool XL, bool STAGE, bool PRE = false, bool STR = false>
__device__ __forceinline__ void dq_body(
    int qt, int item, const BwdLds<D> &lds, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dQ, int B,
    int Hq, int Hkv, int Nq, int Nk, float scale, int causal, double rope_lb,
    const float *__restrict__ O = nullptr, const float *__restrict__ dlse = nullptr,
    float *__restrict__ Dout = nullptr, const Layouts &L = Layouts{})
{
    static_assert(!(PRE && STAGE), "the row terms come from the lane's own dO operands");
    constexpr int KS = D / 16, DB = D / 32;
    if constexpr (!XL) Nk = Nq;
    // XL = false: a literal 0, folded before the compiler shapes the loop's branches
    // (Nk - Nq with Nk = Nq was folded too late and cost 2% in the loop)
    const int off = XL ? Nk - Nq : 0;
    uint16_t *const sk0 = lds.q0s, *const sk1 = lds.q1s, *const sv0 = lds.d0s, *const sv1 = lds.d1s;

    const int G = Hq / Hkv;
    const int grp = item / G;
    const int b = grp / Hkv, g = grp % Hkv;
    const int h = g * G + item % G;
    const int q0 = qt * kQBM;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l32 = lane & 31, hf = lane >> 5;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + l32;

    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    const size_t qrow0 = ((size_t)b * Hq + h) * Nq;      // rows of lse, D, dlse
    // strides of the 4-D tensors (STR: the caller's; else contiguous [B][H][N][D])
    const TL lq = STR ? L.q : contiguous_tl(Hq, Nq, D), ldo = STR ? L.dout : contiguous_tl(Hq, Nq, D);
    const TL lo = STR ? L.o : contiguous_tl(Hq, Nq, D), ldq = STR ? L.dq : contiguous_tl(Hq, Nq, D);
    const TL lk = STR ? L.k : contiguous_tl(Hkv, Nk, D), lv = STR ? L.v : contiguous_tl(Hkv, Nk, D);
    const uint16_t *Qh = Q + b * lq.b + h * lq.h, *dOh = dO + b * ldo.b + h * ldo.h;
    const uint16_t *Kg = K + b * lk.b + g * lk.h;
    const uint16_t *Vg = V + b * lv.b + g * lv.h;

    bf16x8 qf[KS], dof[KS];
    if constexpr (STAGE) {
        const TileCopy<D, kQBM, 4> qcopy(wave, lane, lq.n), dcopy(wave, lane, ldo.n);
        qcopy(sk1, make_rsrc(Qh, head_bytes(Nq, lq.n, D, 2)), q0, wave);
        dcopy(sv1, make_rsrc(dOh, head_bytes(Nq, ldo.n, D, 2)), q0, wave);
    } else {
        const int qr = min(qi, Nq - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 uq = *(const uint4 *)(Qh + (size_t)qr * lq.n + 16 * ks + 8 * hf);
            const uint4 ud = *(const uint4 *)(dOh + (size_t)qr * ldo.n + 16 * ks + 8 * hf);
            uq.x ^= qsign; uq.y ^= qsign; uq.z ^= qsign; uq.w ^= qsign;
            qf[ks] = as_bf16x8(uq);
            dof[ks] = as_bf16x8(ud);
        }
    }
    // Every load of the prologue before tile 0's copies, and none behind a
    // branch (rows clamped, values selected), so that nothing waits for them
    // before those copies are issued: the row terms, and with PRE the O
    // elements matching the lane's dO operands (and dlse).
    const int qcl = min(qi, Nq - 1);
    const float lse_raw = LSE[qrow0 + qcl];
    float dr = 0.f, dl = 0.f;
    float4 oa[KS], oc[KS];
    if constexpr (PRE) {
        const float *orow = O + b * lo.b + h * lo.h + (size_t)qcl * lo.n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            oa[ks] = *(const float4 *)(orow + 16 * ks + 8 * hf);
            oc[ks] = *(const float4 *)(orow + 16 * ks + 8 * hf + 4);
        }
        if (dlse) dl = dlse[qrow0 + qcl];
    } else {
        dr = Dws[qrow0 + qcl];
    }

    const int kv_end = causal ? min(Nk, q0 + kQBM + off) : Nk;
    const int ntiles = (kv_end + kQBN - 1) / kQBN;

    // Tiles move global -> LDS directly; rows past Nk read as zero and are masked.
    const uint32_t k_bytes = head_bytes(Nk, lk.n, D, 2), v_bytes = head_bytes(Nk, lv.n, D, 2);
    using Copy = TileCopy<D, kQBN, 4>;
    const Copy copy(wave, lane, lk.n), copyv(wave, lane, lv.n);
    copy(sk0, make_rsrc(Kg, k_bytes), 0, wave);
    copyv(sv0, make_rsrc(Vg, v_bytes), 0, wave);
    if constexpr (STAGE) {
        // the resident Q and dO rows as soon as their copies have landed (issued
        // before the row-term loads and tile 0's copies; loads complete in
        // order), while tile 0's copies are still in flight; tile 0's barrier
        // then also frees buffer 1 for tile 1's copies
        wait_vmcnt<2 * Copy::PER_WAVE>();
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 uq = *(const uint4 *)tile_chunk<D>(sk1, wave * 32 + l32, 2 * ks + hf);
            const uint4 ud = *(const uint4 *)tile_chunk<D>(sv1, wave * 32 + l32, 2 * ks + hf);
            uq.x ^= qsign; uq.y ^= qsign; uq.z ^= qsign; uq.w ^= qsign;
            qf[ks] = as_bf16x8(uq);
            dof[ks] = as_bf16x8(ud);
        }
    }

    // the row terms, while tile 0's copies are in flight
    const float lse2 = qi < Nq ? lse_raw * kLog2e : INFINITY;
    float Di;
    if constexpr (PRE) {
        // the lane holds dO[qi][16ks + 8hf .. +7] and the matching O elements;
        // the two halves of the row summed across the lane pair
        float sm = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 a = oa[ks], c = oc[ks];
            const uint4 u = __builtin_bit_cast(uint4, dof[ks]);
            sm = fmaf(bf16lo(u.x), a.x, sm); sm = fmaf(bf16hi(u.x), a.y, sm);
            sm = fmaf(bf16lo(u.y), a.z, sm); sm = fmaf(bf16hi(u.y), a.w, sm);
            sm = fmaf(bf16lo(u.z), c.x, sm); sm = fmaf(bf16hi(u.z), c.y, sm);
            sm = fmaf(bf16lo(u.w), c.z, sm); sm = fmaf(bf16hi(u.w), c.w, sm);
        }
        Di = pair32_sum(sm) - dl;
        if (qi < Nq && hf == 0) Dout[qrow0 + qi] = Di;
        Di = qi < Nq ? Di : 0.f;
    } else {
        Di = qi < Nq ? dr : 0.f;
    }
    f32x16 negD;
#pragma unroll
    for (int r = 0; r < 16; ++r) negD[r] = -Di;

    f32x16 dqa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

    auto run_tile = [&](auto bufc, int t) {
        constexpr int BI = decltype(bufc)::value;
        const uint16_t *skc = BI ? sk1 : sk0, *svc = BI ? sv1 : sv0;
        uint16_t *skn = BI ? sk0 : sk1, *svn = BI ? sv0 : sv1;
        wait_vmcnt<0>();                    // this wave's copies of tile t have landed
        __syncthreads();                    // ... and every wave's; buffer t+1 is free
        // copies of tile t+1 (branch-free, so they can interleave with MFMAs);
        // past the last tile they read nothing (zero-byte resources)
        const bool more = t + 1 < ntiles;
        const __amdgpu_buffer_rsrc_t rkn = make_rsrc(Kg, more ? k_bytes : 0u),
                                     rvn = make_rsrc(Vg, more ? v_bytes : 0u);
        auto prefetch = [&] {
            copy(skn, rkn, (t + 1) * kQBN, wave);
            copyv(svn, rvn, (t + 1) * kQBN, wave);
        };
        // No branch on whether the wave has work in this tile (a branch would
        // duplicate the interleaved copies and spill registers): a wave whose
        // rows all precede the tile runs it fully masked, and rows past Nq have
        // lse = +inf, so both add exact zeros.
        const int kv0 = t * kQBN;
        const bool mask = (causal && kv0 + kQBN - 1 > qw0 + off) || kv0 + kQBN > Nk;
        dq_tile<D, 2 * Copy::PER_WAVE>(skc, svc, qf, dof, dqa, c2, lse2, negD, kv0, qi + off, Nk, causal,
                                       mask, lane, prefetch);
        sched_fence();
    };
    for (int t = 0; t < ntiles; t += 2) {
        run_tile(Buf<0>{}, t);
        if (t + 1 < ntiles) run_tile(Buf<1>{}, t + 1);
    }

    // rope_lb != 0: dQ was taken at rotated queries; the transposed rotation of
    // position qi + off carries it back (dims i and i + D/2 sit in blocks db
    // and db + DB/2 of the same lane and register)
    if (rope_lb != 0.0) {
        // pair i = 32db + 8(r/4) + 4hf + r%4 has frequency q^i, q = base^(-2/D):
        // q^(4hf + r%4) once, then steps of q^8 and q^32
        const double pos = (double)(qi + off);
        const double q1 = rope_theta(1, D, rope_lb), q8 = rope_theta(8, D, rope_lb);
        const double q32 = rope_theta(32, D, rope_lb);
        double t0[4];
        t0[0] = rope_theta(4 * hf, D, rope_lb);
        t0[1] = t0[0] * q1; t0[2] = t0[1] * q1; t0[3] = t0[2] * q1;
        double tdb = 1.0;
#pragma unroll
        for (int db = 0; db < DB / 2; ++db, tdb *= q32) {
            double ta = tdb;
#pragma unroll
            for (int a = 0; a < 4; ++a, ta *= q8)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    float sn, cs;
                    rope_sincos_hw(pos * (t0[e] * ta), sn, cs);
                    const float x0 = dqa[db][r], x1 = dqa[db + DB / 2][r];
                    dqa[db][r] = x0 * cs + x1 * sn;
                    dqa[db + DB / 2][r] = x1 * cs - x0 * sn;
                }
        }
    }
    // dQ = scale (dQ^T)^T through LDS: each wave parks its 32 rows as [row][dim]
    // (four dims per 16-byte write, chunk c of row r at c ^ (r mod NC)) in a
    // tile array of its own, reads them back along the dim and stores whole
    // rows (consecutive lanes, consecutive addresses) instead of 32-byte
    // pieces of 32 rows.
    constexpr int NC = D / 4, RPI = 64 / NC;    // 16-byte chunks per row, rows per read
    static_assert(32 * D * sizeof(float) <= kQBN * D * sizeof(uint16_t), "a wave's dQ rows fit");
    float *pk = reinterpret_cast<float *>(wave == 0 ? sk0 : wave == 1 ? sk1 : wave == 2 ? sv0 : sv1);
    __syncthreads();                         // the last tile's reads are done
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int c = 8 * db + 2 * a + hf;
            *(float4 *)&pk[l32 * D + 4 * (c ^ (l32 & (NC - 1)))] =
                make_float4(dqa[db][4 * a + 0] * scale, dqa[db][4 * a + 1] * scale, dqa[db][4 * a + 2] * scale,
                            dqa[db][4 * a + 3] * scale);
        }
    float4 vq[32 / RPI];
    const int rl = lane / NC, cl = lane % NC;  // this lane's row within a read, its chunk
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int r = RPI * i + rl;
        vq[i] = *(const float4 *)&pk[r * D + 4 * (cl ^ (r & (NC - 1)))];
    }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int qr = qw0 + RPI * i + rl;
        if (qr < Nq) *(float4 *)(dQ + b * ldq.b + h * ldq.h + (size_t)qr * ldq.n + 4 * cl) = vq[i];
    }
}

template <int D, bool XL, bool PRE, bool STR = false>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dQ, int B,
    int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int nqt, double rope_lb,
    const float *__restrict__ O, const float *__restrict__ dlse, float *__restrict__ Dout, Layouts L,
    float *__restrict__ zf_a = nullptr, float *__restrict__ zf_b = nullptr, long zf_n = 0)
{
    __shared__ __attribute__((aligned(16))) uint16_t sk0[kQBN * D], sk1[kQBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t sv0[kQBN * D], sv1[kQBN * D];
    const BwdLds<D> lds{sk0, sk1, sv0, sv1, nullptr, nullptr, nullptr, nullptr};
    // work item (query tile, batch, query head), XCD-aware (see xcd_work_item)
    const int G = Hq / Hkv;
    WorkItem w;
    if (xcd_work_item(blockIdx.x, B * Hkv, nqt, G, w))
        dq_body<D, XL, false, PRE, STR>(w.tile, w.group * G + w.head, lds, Q, K, V, LSE, dO, Dws, dQ, B,
                                        Hq, Hkv, Nq, Nk, scale, causal, rope_lb, O, dlse, Dout, L);
    // zf_n > 0: the dK/dV kernel that follows adds its head subsets into zf_a
    // and zf_b (zf_n floats each, a multiple of 4) atomically; every block
    // (padding ones too) zeroes a slice of both after its own work, which
    // saves a launch of its own
    if (zf_n > 0) {
        const long per = ((zf_n + gridDim.x - 1) / gridDim.x + 3) & ~3L;
        const long end = min(zf_n, (long)(blockIdx.x + 1) * per);
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        for (long i = (long)blockIdx.x * per + 4 * threadIdx.x; i < end; i += 4 * 256) {
            *(float4 *)(zf_a + i) = z;
            *(float4 *)(zf_b + i) = z;
        }
    }
}

// Both gradients in one launch, ordered by a plan (see BwdPlan): groups of
// blocks, each group one or more levels of one kind -- dK/dV key tiles or dQ
// query tiles -- with the heaviest levels first over both kinds, so that the
// hardware's in-order dispatch of blocks to free CU slots packs the two kinds
// together.  Within a level, the block's XCD picks a contiguous range of its
// work items (a group's rows stay in one L2).
template <int D, bool XL, bool STR = false>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void bwd_fused_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dQ,
    float *__restrict__ dK, float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk,
    float scale, int causal, int hs, BwdPlan plan, double rope_lb, Layouts L)
{
    static_assert(kQBN <= BwdLds<D>::SR && kQBM <= BwdLds<D>::SR, "dQ's K/V tiles and Q/dO rows fit the Q/dO arrays");
    ATTN_BWD_LDS(D, lds);
    const int blk = blockIdx.x;
    int i = 0;
    while (i + 1 < plan.n && blk >= plan.first[i + 1]) ++i;
    const int kind = plan.kind[i];
    const int hsi = plan.hs[i];
    const int per_level = kind == 0 ? B * Hkv * hsi : B * Hq;
    const int per_xcd = (per_level + kXcds - 1) / kXcds;
    const int rel = blk - plan.first[i];
    const int k = rel / kXcds;
    const int level = kind == 0 ? plan.lev0[i] + k / per_xcd : plan.lev0[i] - k / per_xcd;
    const int item = (rel % kXcds) * per_xcd + k % per_xcd;
    if (item >= per_level) return;
    if (kind == 0)
        dkdv_body<D, XL, STR>(level, item, lds, Q, K, V, LSE, dO, Dws, dK, dV, B, Hq, Hkv, Nq, Nk, scale,
                              causal, hsi, rope_lb, L);
    else
        dq_body<D, XL, true, false, STR>(level, item, lds, Q, K, V, LSE, dO, Dws, dQ, B, Hq, Hkv, Nq, Nk,
                                         scale, causal, rope_lb, nullptr, nullptr, nullptr, L);
}

// Runs f(D, XL, STR) (as integral constants) for head dim d, the
// cross-length flag xl and the strided-layout flag str; the square
// instantiations keep Nk == Nq known to the compiler.
template <class F>
hipError_t bwd_variant(int d, bool xl, bool str, F &&f)
{
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using T = std::true_type;
    using Fa = std::false_type;
    auto with_str = [&](auto dc, auto xc) { str ? f(dc, xc, T{}) : f(dc, xc, Fa{}); };
    if (d == 128) xl ? with_str(I128{}, T{}) : with_str(I128{}, Fa{});
    else if (d == 64) xl ? with_str(I64{}, T{}) : with_str(I64{}, Fa{});
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int device_cus()
{
    // the current device's compute-unit count, queried per call (each device
    // of a process may differ); 256 (MI355X) when no device answers
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        return n;
    return 256;
}

// The d = 128 dK/dV work goes to the 128-key kernel (attn_bwd_dkdv128.hip)
// unless its key tiles number fewer than a quarter of the CUs: smaller grids
// take this file's 64-key kernel, which has twice as many items.  Measured
// on MI355X, attn_bwd at 32/8 heads, causal: N = 256 / 512 27.8 / 39.2 us
// (64 keys) vs 32.0 / 41.5 us (128 keys); N = 1024 / 4096 80.8 / 482.8 vs
// 65.4 / 455.3 us.  (ATTN_DKDV_KV64: always the 64-key kernel;
// ATTN_DKDV_KV128: always the 128-key one.)
bool dkdv_use128(int B, int Hkv, int Nk, int d)
{
#if defined(ATTN_DKDV_KV64)
    return false;
#elif defined(ATTN_DKDV_KV128)
    return d == 128;
#else
    return d == 128 && 4L * dkdv128_tiles(Nk) * B * Hkv >= device_cus();
#endif
}

int dkdv_head_split(int B, int Hq, int Hkv, int Nk, int d)
{
    // Split each group's query heads over workgroups until there are about two
    // work items per CU.  The split workgroups add their partial dK/dV with
    // f32 atomics (coalesced along the head dim); measured on MI355X: 4 x 1024
    // x 64 grouped-query workload 46.5 -> 39.6 us with the 3 heads split, while
    // splitting further than two items per CU (32/8 heads at N = 4096) only
    // adds atomic traffic.
    const int cus = device_cus();
    const int G = Hq / Hkv;
    const long tiles = dkdv_use128(B, Hkv, Nk, d) ? dkdv128_tiles(Nk) : (Nk + kKvBN - 1) / kKvBN;
    const long base = tiles * B * Hkv;
    int hs = 1;
    for (int c = 1; c <= G; ++c)
        if (G % c == 0) {
            hs = c;
            if (base * c >= 2L * cus) break;
        }
    return hs;
}

hipError_t bwd_dkdv_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         const void *q, const void *k, const void *v, const float *lse,
                         const void *dout, const float *Dws, float *dk, float *dv, int hs,
                         hipStream_t st, double rope_lb, const Layouts *L)
{
    if (dkdv_use128(B, Hkv, Nk, d))
        return bwd_dkdv128_mfma(B, Hq, Hkv, Nq, Nk, causal, scale, q, k, v, lse, dout, Dws, dk, dv, hs, st,
                                rope_lb, L);
    const int nkt = (Nk + kKvBN - 1) / kKvBN;
    const dim3 grid((unsigned)(nkt * B * Hkv * hs));
    const Layouts lay = L ? *L : Layouts{};
    return bwd_variant(d, Nq != Nk, L != nullptr, [&](auto dc, auto xc, auto sc) {
        constexpr int DD = decltype(dc)::value;
        constexpr bool XX = decltype(xc)::value, SS = decltype(sc)::value;
#ifndef ATTN_DKDV_ONE_WAVE_PER_SIMD
        if constexpr (DD == 128) {
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<128, XX, SS>), grid, dim3(64 * kPairWaves), 0, st,
                               (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, lse,
                               (const uint16_t *)dout, Dws, dk, dv, B, Hq, Hkv, Nq, Nk, scale, causal,
                               hs, rope_lb, lay);
            return;
        }
#endif
        hipLaunchKernelGGL((bwd_dkdv_kernel<DD, XX, SS>), grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout, Dws,
                           dk, dv, B, Hq, Hkv, Nq, Nk, scale, causal, hs, rope_lb, lay);
    });
}

hipError_t bwd_dq_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       const void *q, const void *k, const void *v, const float *lse,
                       const void *dout, const float *Dws, float *dq, hipStream_t st,
                       double rope_lb, const Layouts *L)
{
    const int nqt = (Nq + kQBM - 1) / kQBM;
    const dim3 grid((unsigned)((nqt * B * Hq + kXcds - 1) / kXcds * kXcds));
    const Layouts lay = L ? *L : Layouts{};
    return bwd_variant(d, Nq != Nk, L != nullptr, [&](auto dc, auto xc, auto sc) {
        hipLaunchKernelGGL((bwd_dq_kernel<decltype(dc)::value, decltype(xc)::value, false,
                                          decltype(sc)::value>),
                           grid, dim3(256), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                           (const uint16_t *)v, lse, (const uint16_t *)dout, Dws, dq, B, Hq, Hkv,
                           Nq, Nk, scale, causal, nqt, rope_lb, nullptr, nullptr, nullptr, lay);
    });
}

hipError_t bwd_dq_pre_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           const void *q, const void *k, const void *v, const float *lse,
                           const void *dout, const float *o, const float *dlse, float *Dws,
                           float *dq, hipStream_t st, double rope_lb, const Layouts *L, float *zf_a,
                           float *zf_b, long zf_n)
{
    if (zf_n % 4 != 0 || (zf_n > 0 && (((uintptr_t)zf_a | (uintptr_t)zf_b) & 15) != 0))
        return hipErrorInvalidValue;
    if (d != 128) return hipErrorInvalidValue;
    const int nqt = (Nq + kQBM - 1) / kQBM;
    const dim3 grid((unsigned)((nqt * B * Hq + kXcds - 1) / kXcds * kXcds));
    const Layouts lay = L ? *L : Layouts{};
    return bwd_variant(d, Nq != Nk, L != nullptr, [&](auto, auto xc, auto sc) {
        hipLaunchKernelGGL((bwd_dq_kernel<128, decltype(xc)::value, true, decltype(sc)::value>), grid,
                           dim3(256), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                           (const uint16_t *)v, lse, (const uint16_t *)dout, nullptr, dq, B, Hq, Hkv, Nq,
                           Nk, scale, causal, nqt, rope_lb, o, dlse, Dws, lay, zf_a, zf_b, zf_n);
    });
}

namespace {

// Estimated time of one work item of each kind (arbitrary units, fitted to
// per-workgroup timelines measured on MI355X at d = 64: about 1.9 per 128-query
// dK/dV step and 0.8 per 64-key dQ tile on top of a fixed part for loading the
// item's resident operands and storing its result), for ordering only.
double dkdv_cost(int steps, int d) { return 7.0 + 1.9 * steps * (d / 64); }
double dq_cost(int tiles, int d) { return 6.0 + 0.8 * tiles * (d / 64); }

struct PlanLevel {
    int kind, lev, nlev, hs;
    double cost;
};

// Level groups of one kind, heaviest first, coarsened to at most `cap` groups
// (a group never mixes head splits).
void plan_levels(int kind, int nlev, int cap, const double *cost, const int *lev, const int *hs,
                 std::vector<PlanLevel> &out)
{
    const int chunk = (nlev + cap - 1) / cap;
    for (int i = 0; i < nlev;) {
        int n = 1;
        while (n < chunk && i + n < nlev && hs[i + n] == hs[i]) ++n;
        double c = 0;
        for (int j = 0; j < n; ++j) c += cost[i + j];
        out.push_back({kind, lev[i], n, hs[i], c / n});
        i += n;
    }
}

}  // namespace

// The one-launch plan of a shape, or false when its level groups do not fit
// BwdPlan (the caller then runs the two gradient kernels instead).  The dK/dV
// side splits a group wherever the key tiles' head split changes, so it can
// hold more groups than its cap: the caps shrink (dK/dV first) until both
// sides fit together.
bool bwd_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int hs, BwdPlan &p,
              int *grid)
{
    const int off = Nk - Nq;
    const int nkt = (Nk + kKvBN - 1) / kKvBN, nqkv = (Nq + kKvSub * kKvBM - 1) / (kKvSub * kKvBM);
    const int nqt = (Nq + kQBM - 1) / kQBM;
    const int G = Hq / Hkv;
    // Key tiles whose query range is short take fewer head subsets: the
    // fewest (a divisor of G) whose chain of steps stays within the longest
    // chain under the split hs (fewer work items and, at one subset, plain
    // stores instead of atomics).
    const int max_chain = (G / hs) * nqkv;
    std::vector<double> ck(nkt), cq(nqt);
    std::vector<int> lk(nkt), lq(nqt), hk(nkt), hq(nqt, 1);
    for (int kt = 0; kt < nkt; ++kt) {
        const int nq = nqkv - (causal ? std::max(kt * kKvBN - off, 0) / (kKvSub * kKvBM) : 0);
        int c = hs;
        for (int e = 1; e <= hs; ++e)
            if (G % e == 0 && hs % e == 0 && (G / e) * nq <= max_chain) { c = e; break; }
        lk[kt] = kt;
        hk[kt] = c;
        ck[kt] = dkdv_cost((G / c) * nq, d);
    }
    for (int j = 0; j < nqt; ++j) {
        const int qt = nqt - 1 - j;
        const int kv_end = causal ? std::min(Nk, (qt + 1) * kQBM + off) : Nk;
        lq[j] = qt;
        cq[j] = dq_cost((kv_end + kQBN - 1) / kQBN, d);
    }
    std::vector<PlanLevel> a, q, m;
    int cap_a = BwdPlan::kMax / 2, cap_q = BwdPlan::kMax / 2;
    for (;;) {
        a.clear();
        q.clear();
        plan_levels(0, nkt, cap_a, ck.data(), lk.data(), hk.data(), a);
        plan_levels(1, nqt, cap_q, cq.data(), lq.data(), hq.data(), q);
        if (a.size() + q.size() <= (size_t)BwdPlan::kMax) break;
        if (cap_a > 1) --cap_a;
        else if (cap_q > 1) --cap_q;
        else return false;
    }
    // merge, heaviest first (ties: dK/dV first)
    size_t ia = 0, iq = 0;
    while (ia < a.size() || iq < q.size()) {
        if (iq == q.size() || (ia < a.size() && a[ia].cost >= q[iq].cost)) m.push_back(a[ia++]);
        else m.push_back(q[iq++]);
    }
    p = BwdPlan{};
    p.n = (int)m.size();
    long blk = 0;
    for (int i = 0; i < p.n; ++i) {
        const int per_level = m[i].kind == 0 ? B * Hkv * m[i].hs : B * Hq;
        const int per_xcd = (per_level + kXcds - 1) / kXcds;
        p.first[i] = (int)blk;
        p.lev0[i] = m[i].lev;
        p.kind[i] = m[i].kind;
        p.hs[i] = m[i].hs;
        blk += (long)m[i].nlev * per_xcd * kXcds;
        if (blk > 2147483647L) return false;
    }
    p.first[p.n] = (int)blk;
    *grid = (int)blk;
    return true;
}

bool bwd_fused_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int hs, int *groups,
                    int *blocks)
{
    BwdPlan p;
    int nblk = 0;
    if (!bwd_plan(B, Hq, Hkv, Nq, Nk, d, causal, hs, p, &nblk)) return false;
    if (groups) *groups = p.n;
    if (blocks) *blocks = nblk;
    return true;
}

hipError_t bwd_fused_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                          const void *q, const void *k, const void *v, const float *lse,
                          const void *dout, const float *Dws, float *dq, float *dk, float *dv,
                          int hs, hipStream_t st, double rope_lb, const Layouts *L)
{
    BwdPlan plan;
    int nblk = 0;
    if (!bwd_plan(B, Hq, Hkv, Nq, Nk, d, causal, hs, plan, &nblk)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk);
    const Layouts lay = L ? *L : Layouts{};
    return bwd_variant(d, Nq != Nk, L != nullptr, [&](auto dc, auto xc, auto sc) {
        hipLaunchKernelGGL((bwd_fused_kernel<decltype(dc)::value, decltype(xc)::value, decltype(sc)::value>),
                           grid, dim3(256), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                           (const uint16_t *)v, lse, (const uint16_t *)dout, Dws, dq, dk, dv, B,
                           Hq, Hkv, Nq, Nk, scale, causal, hs, plan, rope_lb, lay);
    });
}

}  // namespace attn
