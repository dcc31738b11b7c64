// attn_bwd_dkdv128.hip -- dK and dV of causal grouped-query attention at head
// dim 128 on gfx950 matrix cores (bf16 operands, f32 accumulation).
//
// The same gradient as the other key-stationary kernel (from P recomputed out
// of q, k and the forward's log-sum-exp: dV = P^T dO, dK = scale dS^T Q with
// dS = P o (dP - D), dP = dO V^T; "tang -- differentiable computing in Rust",
// "How tang works" part 3), laid out for d = 128:
//
//   * 128 keys per workgroup, so each query tile streamed through LDS feeds
//     twice the key rows (half the L2 -> LDS traffic of 64-key workgroups);
//   * 8 waves in pairs on one SIMD: wave kb (0..3) computes S = Q K^T and P
//     for keys 32 kb .. 32 kb + 31 against the 64 query rows of an iteration
//     and accumulates dV^T of those keys; wave 4 + kb computes dP = dO V^T for
//     the same keys and rows, takes P from its partner through LDS, and
//     accumulates dK^T.  Each wave owns its keys' accumulators outright (no
//     partial sums between waves);
//   * software-pipelined by one iteration, one barrier per iteration: in
//     iteration t the P waves issue the score MFMAs of query tile t and the
//     dV MFMAs of tile t - 1 in one stream (two independent score chains and
//     four accumulators), re-reading P of tile t - 1 from the exchange
//     buffer; the dP waves run tile t - 1 whole (dP, dS, dK), its P having
//     been published by the barrier before.  Query tiles live in a ring of
//     three LDS slots: tile t is read in iterations t and t + 1 while the
//     direct global->LDS copy of tile t + 1 fills the third slot.  The loop
//     body holds three iterations (one per slot, so that every LDS address
//     is a compile-time array: the copy in flight is then known not to alias
//     the reads);
//   * the LDS operand reads run a fixed distance ahead of the MFMAs
//     (scheduling-group hints), and the lane part of every operand address is
//     computed once and re-derived each iteration from an opaque zero, so
//     that the compiler neither waits on each read nor hoists one address per
//     slot and read out of the loop.
//
// Keys past Nk read as zero and their rows are never stored; query rows past
// Nq read as zero (Q, dO, lse and D), which makes their P . dO and dS terms
// zero.  Score tiles wholly above the causal diagonal are computed and masked
// to P = 0 rather than skipped, so that the MFMA stream has no branches (they
// occur only in the first two iterations of each query head).
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

#include <type_traits>

// LDS operand reads kept in flight ahead of the MFMAs that consume them (P
// waves / dP waves), beyond the 8 row-term reads that start an iteration.
#ifndef ATTN_K128_PAHEAD
#define ATTN_K128_PAHEAD 16
#endif
#ifndef ATTN_K128_GAHEAD
#define ATTN_K128_GAHEAD 16
#endif

namespace attn {

namespace {

constexpr int kBN = 128;     // keys per workgroup
constexpr int kBM = 64;      // query rows per iteration
constexpr int kWaves = 8;    // 4 P/dV waves + 4 dP/dK waves

// (Named members, selected with constants or conditionals: an array of LDS
// pointers indexed at run time would be kept in scratch memory.)
struct K128Lds {
    uint16_t *q0, *q1, *q2;  // ring slots: Q tiles [kBM][128], swizzled
    uint16_t *d0, *d1, *d2;  // ... and dO tiles
    float *rows;             // [3 slots][2][kBM]: -lse / |scale| and -D of each tile's rows
    uint4 *pbuf;             // [2][4 key blocks][2 query halves][2 operand halves][64 lanes]
};

// P of one wave's two 32x32 tiles, as its four bf16 MFMA operands.
struct POps {
    bf16x8 v[2][2];          // [query half][operand half]
};

// Byte offsets of this lane's MFMA operand reads within a swizzled [kBM][128]
// tile (the layout of tile_chunk): row[ks] for the operand of row l32, chunk
// 2 ks + hf (tile_row_operand; query half qh adds 32 rows), tr[db] for the
// first transposed read of tr_operand at row base 0 and column base 32 db
// (row bases that are multiples of 16 add 16 rows each).  They are kept in
// registers and re-derived at every iteration (opaque below): otherwise the
// compiler hoists the address of every (slot, read) pair of the 3-way
// unrolled loop out of it and runs out of registers.
struct LaneOffsets {
    int row[8];
    int tr[4];
};

// The second transposed read of tr_operand (8 rows down) differs from the
// first by a constant: rows 0..7 have swz < 8, so row + 8 flips bit 3 of the
// chunk, which is bit 1 of db.  (That holds for the default swizzle only.)
#ifdef ATTN_LDS_SWIZZLE_256
#error "the 128-key dK/dV kernel's operand offsets assume the default LDS swizzle"
#endif
constexpr int kTrHi[4] = {2 * (8 * 128 + 64), 2 * (8 * 128 + 64), 2 * (8 * 128 - 64), 2 * (8 * 128 - 64)};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane)
{
    constexpr int D = 128;
    LaneOffsets o;
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) o.row[ks] = 2 * (l32 * D + 8 * ((2 * ks + hf) ^ swz<D>(l32)));
    const int i = lane & 15, g16 = (lane >> 4) & 1;
    const int row = 4 * hf + (i >> 2), e = 4 * (i & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int c = 4 * db + 2 * g16 + ((i & 3) >> 1);
        o.tr[db] = 2 * (row * D + 8 * (c ^ swz<D>(row)) + e);
    }
    return o;
}

// The offsets plus a zero the compiler cannot see through (one scalar per
// iteration), so that the addresses are formed inside the loop.
__device__ __forceinline__ LaneOffsets opaque(const LaneOffsets &o)
{
    int z = 0;
    asm volatile("" : "+s"(z));
    LaneOffsets r;
#pragma unroll
    for (int k = 0; k < 8; ++k) r.row[k] = o.row[k] + z;
#pragma unroll
    for (int db = 0; db < 4; ++db) r.tr[db] = o.tr[db] + z;
    return r;
}

__device__ __forceinline__ bf16x8 row_read(const uint16_t *tile, int byte_off)
{
    return as_bf16x8(*(const uint4 *)((const char *)tile + byte_off));
}

__device__ __forceinline__ bf16x8 tr_read(const uint16_t *tile, int lo, int hi)
{
    const uint2 a = lds_read_tr16((const uint16_t *)((const char *)tile + lo));
    const uint2 b = lds_read_tr16((const uint16_t *)((const char *)tile + hi));
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

template <bool XL, bool STR>
__device__ __forceinline__ void dkdv128_body(
    int kt, int item, const K128Lds &lds, const uint16_t *__restrict__ Q,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, int hs,
    double rope_lb, const Layouts &L)
{
    constexpr int D = 128, KS = D / 16, DB = D / 32;
    // (the LDS pointers as locals: address-space inference then sees every
    // use as an LDS access)
    uint16_t *const Q0 = lds.q0, *const Q1 = lds.q1, *const Q2 = lds.q2;
    uint16_t *const D0 = lds.d0, *const D1 = lds.d1, *const D2 = lds.d2;
    float *const ROWS = lds.rows;
    uint4 *const PBUF = lds.pbuf;
    auto qsel = [&](int s) { return s == 0 ? Q0 : s == 1 ? Q1 : Q2; };
    auto dsel = [&](int s) { return s == 0 ? D0 : s == 1 ? D1 : D2; };
    if constexpr (!XL) Nk = Nq;
    const int off = XL ? Nk - Nq : 0;

    const int grp = item / hs, hsub = item % hs;
    const int b = grp / Hkv, g = grp % Hkv;
    const int G = Hq / Hkv, Gs = G / hs;
    const int k0 = kt * kBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const bool role_p = wave < 4;            // P and dV; else dP, dS and dK
    const int kb = wave & 3;                 // key block: keys k0 + 32 kb ..
    const int kj = k0 + 32 * kb + l32;       // this lane's key column

    const uint32_t ksign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    const TL lq = STR ? L.q : contiguous_tl(Hq, Nq, D), ldo = STR ? L.dout : contiguous_tl(Hq, Nq, D);
    const TL lk = STR ? L.k : contiguous_tl(Hkv, Nk, D), lv = STR ? L.v : contiguous_tl(Hkv, Nk, D);
    const TL ldk = STR ? L.dk : contiguous_tl(Hkv, Nk, D), ldv = STR ? L.dv : contiguous_tl(Hkv, Nk, D);

    // The resident operand, K^T (P waves, sign-flipped for a negative scale)
    // or V^T (dP waves): the 128 key rows of K go to slot 1 and those of V to
    // slot 2 (rows 0..63 in the Q array, 64..127 in the dO array) first.
    {
        const TileCopy<D, kBM, kWaves> kc(wave, lane, lk.n), vc(wave, lane, lv.n);
        const auto rk = make_rsrc(K + b * lk.b + g * lk.h, head_bytes(Nk, lk.n, D, 2));
        const auto rv = make_rsrc(V + b * lv.b + g * lv.h, head_bytes(Nk, lv.n, D, 2));
        kc(Q1, rk, k0, wave);
        kc(D1, rk, k0 + kBM, wave);
        vc(Q2, rv, k0, wave);
        vc(D2, rv, k0 + kBM, wave);
    }

    const int nqt = (Nq + kBM - 1) / kBM;
    const int qt0 = causal ? (XL ? max(k0 - off, 0) : k0) / kBM : 0;
    const int nq = nqt - qt0;
    const int T = Gs * nq;                   // iterations with a query tile (>= 1)

    const uint32_t q_bytes = head_bytes(Nq, lq.n, D, 2), do_bytes = head_bytes(Nq, ldo.n, D, 2);
    const uint32_t row_bytes = (uint32_t)Nq * 4;
    const TileCopy<D, kBM, kWaves> qcopy(wave, lane, lq.n), dcopy(wave, lane, ldo.n);
    // row terms: wave 0 loads the tile's lse, wave 1 its D, into a register
    // (stored to LDS, scaled, before the barrier that publishes the tile)
    const float row_mul = wave == 0 ? -1.f / fabsf(scale) : -1.f;
    float row_v = 0.f;
    auto tile_q0 = [&](int t) { return (qt0 + t % nq) * kBM; };
    // (The row load goes first: a wait for it -- or for a register reloaded
    // on its behalf -- then does not also wait for the tile copies.)
    auto load = [&](int t, uint16_t *qs, uint16_t *ds) {
        const int hq = g * G + hsub * Gs + t / nq;
        const int q0 = tile_q0(t);
        if (wave < 2)
            row_v = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(
                           make_rsrc((wave == 0 ? LSE : Dws) + ((size_t)b * Hq + hq) * Nq, row_bytes), lane * 4,
                           q0 * 4, 0));
        qcopy(qs, make_rsrc(Q + b * lq.b + hq * lq.h, q_bytes), q0, wave);
        dcopy(ds, make_rsrc(dO + b * ldo.b + hq * ldo.h, do_bytes), q0, wave);
    };
    auto store_rows = [&](int slot) {
        if (wave < 2) ROWS[(2 * slot + wave) * kBM + lane] = row_v * row_mul;
    };

    load(0, Q0, D0);
    wait_vmcnt<0>();
    store_rows(0);
    __syncthreads();

    bf16x8 opf[KS];
    {
        const int slot = role_p ? 1 : 2, r = 32 * kb + l32;
        const uint16_t *src = r < kBM ? qsel(slot) : dsel(slot);
        const uint32_t sign = role_p ? ksign : 0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = *(const uint4 *)tile_chunk<D>(src, r & (kBM - 1), 2 * ks + hf);
            u.x ^= sign; u.y ^= sign; u.z ^= sign; u.w ^= sign;
            opf[ks] = as_bf16x8(u);
        }
    }
    __syncthreads();                         // slots 1 and 2 are free for query tiles

    // Epilogue: each wave parks its 32 x 128 accumulator transposed to
    // [key][dim] f32 in a 16 KiB region of its own (the six tile arrays and
    // the two halves of the P buffer), row r keeping its 4-float chunk c at
    // c ^ (r mod 32), then stores (or adds atomically) one key row per step
    // with the lanes along the dim.
    auto epilogue = [&](const f32x16 (&acc)[DB]) {
        constexpr int NC = D / 4;
        auto pidx = [](int row, int dim) { return row * D + 4 * ((dim >> 2) ^ (row & (NC - 1))) + (dim & 3); };
        float *red = reinterpret_cast<float *>(wave < 6 ? (wave < 3 ? qsel(wave) : dsel(wave - 3))
                                                        : reinterpret_cast<uint16_t *>(PBUF + (wave - 6) * 1024));
        const float amul = role_p ? 1.f : scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(float4 *)&red[pidx(l32, db * 32 + 8 * a + 4 * hf)] =
                    make_float4(acc[db][4 * a] * amul, acc[db][4 * a + 1] * amul, acc[db][4 * a + 2] * amul,
                                acc[db][4 * a + 3] * amul);
        // (a wave reads back only what it wrote: no barrier)
        const bool rot = !role_p && rope_lb != 0.0;
        const double th = rot ? rope_theta(lane, D, rope_lb) : 0.0;
        float *dst = role_p ? dV + b * ldv.b + g * ldv.h : dK + b * ldk.b + g * ldk.h;
        const int ld = role_p ? ldv.n : ldk.n;
        for (int r = 0; r < 32; ++r) {
            const int key = k0 + 32 * kb + r;
            if (key >= Nk) break;
            float x0 = red[pidx(r, lane)], x1 = red[pidx(r, lane + 64)];
            if (rot) {
                float sn, cs;
                rope_sincos_hw((double)key * th, sn, cs);
                const float y0 = x0 * cs + x1 * sn, y1 = x1 * cs - x0 * sn;
                x0 = y0;
                x1 = y1;
            }
            float *row = dst + (size_t)key * ld;
            if (hs == 1) {
                row[lane] = x0;
                row[lane + 64] = x1;
            } else {
                atomicAdd(row + lane, x0);
                atomicAdd(row + lane + 64, x1);
            }
        }
    };

    // The main loop, compiled once per role (wave-uniform), so that every LDS
    // address is a lane offset plus a constant.  Iteration t (0 <= t <= T):
    //   P waves:  S and P of tile t (t < T), dV^T += dO^T P of tile t-1 (t >= 1);
    //   dP waves: dP, dS and dK^T += Q^T dS of tile t-1 (t >= 1), with P of
    //             tile t-1 from the partner's buffer (published at the end of
    //             iteration t-1).
    auto run = [&](auto rolec) {
        constexpr bool RP = decltype(rolec)::value;
        f32x16 acc[DB];                      // dV^T (P waves) or dK^T (dP waves) of the wave's keys
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
        const LaneOffsets lo0 = lane_offsets(lane);
        POps op2;                            // P waves: P of the previous tile (read back from LDS)

        // scores of one 64-row tile into sacc (from the row term up): rows of
        // src times the resident operand
        auto scores_init = [&](f32x16 (&sacc)[2], const float *rt) {
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 v = *(const float4 *)&rt[32 * qh + 8 * a + 4 * hf];
                    sacc[qh][4 * a + 0] = v.x; sacc[qh][4 * a + 1] = v.y;
                    sacc[qh][4 * a + 2] = v.z; sacc[qh][4 * a + 3] = v.w;
                }
        };
        auto score_mfma = [&](f32x16 (&sacc)[2], const uint16_t *src, int ks, const LaneOffsets &lo) {
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
                sacc[qh] = mfma32x32x16(row_read(src + 32 * qh * D, lo.row[ks]), opf[ks], sacc[qh]);
        };
        // one of the 16 MFMAs of acc^T += src^T op over a 64-row tile
        auto grad_mfma = [&](const uint16_t *src, const POps &op, int m, const LaneOffsets &lo) {
            const int qh = m >> 3, tt = (m >> 2) & 1, db = m & 3;
            const uint16_t *tb = src + (32 * qh + 16 * tt) * D;
            acc[db] = mfma32x32x16(tr_read(tb, lo.tr[db], lo.tr[db] + kTrHi[db]), op.v[qh][tt], acc[db]);
        };

        // qc, rc: tile t's Q slot and row terms; qp, dpv: tile t-1's Q and dO
        // slots; qn, dn, nslot: tile t+1's slots.
        auto iteration = [&](auto p1c, auto p2c, auto sidc, int t, const uint16_t *qc, const float *rc,
                             const uint16_t *qp, const uint16_t *dpv, uint16_t *qn, uint16_t *dn, int nslot) {
            constexpr bool P1 = decltype(p1c)::value, P2 = decltype(p2c)::value;
            constexpr int SID = decltype(sidc)::value;
            const LaneOffsets lo = opaque(lo0);
            if (P1 && t + 1 < T) load(t + 1, qn, dn);
            if constexpr (RP) {
                f32x16 sacc[2];
                if constexpr (P2) {
                    // P of tile t-1 back from the exchange buffer (not carried in registers)
                    const uint4 *pb = PBUF + (((t - 1) & 1) * 4 + kb) * 4 * 64;
#pragma unroll
                    for (int j = 0; j < 4; ++j) op2.v[j >> 1][j & 1] = as_bf16x8(pb[j * 64 + lane]);
                }
                if constexpr (P1) scores_init(sacc, rc);
                // per contraction step: the two score MFMAs, then two dV MFMAs
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if constexpr (P1) score_mfma(sacc, qc, ks, lo);
                    if constexpr (P2) {
                        grad_mfma(dpv, op2, 2 * ks, lo);
                        grad_mfma(dpv, op2, 2 * ks + 1, lo);
                    }
                }
                // reads: 8 row terms + 16 score operands (P1), 32 transposed (P2)
                if constexpr (P1 && P2) sched_lead<SID, 60, 32, 12 + ATTN_K128_PAHEAD, 3, 2>();
                else if constexpr (P1) sched_lead<SID, 24, 16, 8 + ATTN_K128_PAHEAD, 1, 1>();
                else sched_lead<SID, 36, 16, 4 + ATTN_K128_PAHEAD, 2, 1>();
                if constexpr (P1) {
                    const int q0 = tile_q0(t);
#pragma unroll
                    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[qh][r] = exp2_fast(sacc[qh][r] * c2);
                        if (causal && q0 + 32 * qh + off < k0 + 32 * kb + 32) {
                            const int th = kj - off - (q0 + 32 * qh + 4 * hf);
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int c = 8 * (r >> 2) + (r & 3);
                                sacc[qh][r] = c >= th ? sacc[qh][r] : 0.f;
                            }
                        }
                    }
                    uint4 *pb = PBUF + ((t & 1) * 4 + kb) * 4 * 64;
#pragma unroll
                    for (int qh = 0; qh < 2; ++qh) {
                        pb[(2 * qh) * 64 + lane] = __builtin_bit_cast(uint4, pack_operand<0>(sacc[qh]));
                        pb[(2 * qh + 1) * 64 + lane] = __builtin_bit_cast(uint4, pack_operand<8>(sacc[qh]));
                    }
                }
            } else if constexpr (P2) {
                // dP - D of tile t-1, then dS = P (dP - D), then dK^T += Q^T dS
                f32x16 sacc[2];
                scores_init(sacc, ROWS + 2 * kBM * ((t - 1) % 3) + kBM);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) score_mfma(sacc, dpv, ks, lo);
                const uint4 *pb = PBUF + (((t - 1) & 1) * 4 + kb) * 4 * 64;
                POps ds;
#pragma unroll
                for (int qh = 0; qh < 2; ++qh) {
                    const uint4 p0 = pb[(2 * qh) * 64 + lane], p1 = pb[(2 * qh + 1) * 64 + lane];
                    f32x16 &e = sacc[qh];
                    e[0] *= bf16lo(p0.x); e[1] *= bf16hi(p0.x); e[2] *= bf16lo(p0.y); e[3] *= bf16hi(p0.y);
                    e[4] *= bf16lo(p0.z); e[5] *= bf16hi(p0.z); e[6] *= bf16lo(p0.w); e[7] *= bf16hi(p0.w);
                    e[8] *= bf16lo(p1.x); e[9] *= bf16hi(p1.x); e[10] *= bf16lo(p1.y); e[11] *= bf16hi(p1.y);
                    e[12] *= bf16lo(p1.z); e[13] *= bf16hi(p1.z); e[14] *= bf16lo(p1.w); e[15] *= bf16hi(p1.w);
                    ds.v[qh][0] = pack_operand<0>(e);
                    ds.v[qh][1] = pack_operand<8>(e);
                }
#pragma unroll
                for (int m = 0; m < 16; ++m) grad_mfma(qp, ds, m, lo);
                // reads: 8 row terms + 16 score operands, 4 of P, 32 transposed
                sched_lead<SID + 8, 60, 32, 8 + ATTN_K128_GAHEAD, 13, 8>();
            }
            wait_vmcnt<0>();                 // this wave's copies of tile t+1 have landed
            if (P1 && t + 1 < T) store_rows(nslot);
            __syncthreads();                 // ... every wave's; tile t+1 and P of tile t are published
        };

        using T_ = std::integral_constant<bool, true>;
        using F_ = std::integral_constant<bool, false>;
        iteration(T_{}, F_{}, std::integral_constant<int, 0>{}, 0, Q0, ROWS, nullptr, nullptr, Q1, D1, 1);
        // Tiles 1 .. T-1 in groups of three (slots 1, 2, 0: no conditionals
        // inside the loop body, which keeps the accumulators in place), then
        // the one or two left over.
        int t = 1;
        for (const int tend = 1 + (T - 1) / 3 * 3; t < tend; t += 3) {
            iteration(T_{}, T_{}, std::integral_constant<int, 1>{}, t, Q1, ROWS + 2 * kBM, Q0, D0, Q2, D2, 2);
            iteration(T_{}, T_{}, std::integral_constant<int, 2>{}, t + 1, Q2, ROWS + 4 * kBM, Q1, D1, Q0, D0, 0);
            iteration(T_{}, T_{}, std::integral_constant<int, 3>{}, t + 2, Q0, ROWS, Q2, D2, Q1, D1, 1);
        }
        if (t < T) {
            iteration(T_{}, T_{}, std::integral_constant<int, 5>{}, t, Q1, ROWS + 2 * kBM, Q0, D0, Q2, D2, 2);
            if (++t < T) {
                iteration(T_{}, T_{}, std::integral_constant<int, 6>{}, t, Q2, ROWS + 4 * kBM, Q1, D1, Q0, D0, 0);
                ++t;
            }
        }
        {
            // tile T-1's gradients (no copy in flight: the slot may be chosen at run time)
            const int sp = (T - 1) % 3;
            iteration(F_{}, T_{}, std::integral_constant<int, 4>{}, T, nullptr, nullptr, qsel(sp), dsel(sp),
                      nullptr, nullptr, 0);
        }
        epilogue(acc);
    };

    if (role_p) run(std::integral_constant<bool, true>{});
    else run(std::integral_constant<bool, false>{});
}

template <bool XL, bool STR>
__global__ __launch_bounds__(64 * kWaves, 1) void bwd_dkdv128_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const float *__restrict__ LSE, const uint16_t *__restrict__ dO, const float *__restrict__ Dws,
    float *__restrict__ dK, float *__restrict__ dV, int B, int Hq, int Hkv, int Nq, int Nk, float scale,
    int causal, int hs, double rope_lb, Layouts L)
{
    constexpr int D = 128;
    __shared__ __attribute__((aligned(16))) uint16_t q0[kBM * D], q1[kBM * D], q2[kBM * D];
    __shared__ __attribute__((aligned(16))) uint16_t d0[kBM * D], d1[kBM * D], d2[kBM * D];
    __shared__ __attribute__((aligned(16))) float rows[3 * 2 * kBM];
    __shared__ __attribute__((aligned(16))) uint4 pbuf[2 * 4 * 4 * 64];
    K128Lds lds;                             // (assigned, not brace-initialised: a constant
    lds.q0 = q0; lds.q1 = q1; lds.q2 = q2;   //  aggregate of LDS addresses would become a
    lds.d0 = d0; lds.d1 = d1; lds.d2 = d2;   //  static initialiser the target cannot emit)
    lds.rows = rows;
    lds.pbuf = pbuf;
    if constexpr (!XL) Nk = Nq;
    const int nkt = (Nk + kBN - 1) / kBN;
    WorkItem w;
    if (!xcd_work_item(blockIdx.x, B * Hkv, nkt, hs, w)) return;
    dkdv128_body<XL, STR>(nkt - 1 - w.tile, w.group * hs + w.head, lds, Q, K, V, LSE, dO, Dws, dK, dV, Hq,
                          Hkv, Nq, Nk, scale, causal, hs, rope_lb, L);
}

}  // namespace

int dkdv128_tiles(int Nk) { return (Nk + kBN - 1) / kBN; }

hipError_t bwd_dkdv128_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int causal, float scale,
                            const void *q, const void *k, const void *v, const float *lse,
                            const void *dout, const float *Dws, float *dk, float *dv, int hs,
                            hipStream_t st, double rope_lb, const Layouts *L)
{
    const dim3 grid((unsigned)(dkdv128_tiles(Nk) * B * Hkv * hs));
    const Layouts lay = L ? *L : Layouts{};
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * kWaves), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                           (const uint16_t *)v, lse, (const uint16_t *)dout, Dws, dk, dv, B, Hq, Hkv, Nq, Nk,
                           scale, causal, hs, rope_lb, lay);
    };
    const bool xl = Nq != Nk;
    if (L) {
        if (xl) go(bwd_dkdv128_kernel<true, true>);
        else go(bwd_dkdv128_kernel<false, true>);
    } else {
        if (xl) go(bwd_dkdv128_kernel<true, false>);
        else go(bwd_dkdv128_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace attn
