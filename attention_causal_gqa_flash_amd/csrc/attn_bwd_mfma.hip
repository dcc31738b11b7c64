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

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kKvBN = 64;   // keys per workgroup
constexpr int kKvBM = 64;   // queries per step

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int N, float scale, int causal, int hs)
{
    constexpr int KS = D / 16, DB = D / 32;

    // One LDS block: double-buffered Q, dO, lse and D tiles during the loop,
    // then the reduction buffer for the two query halves' dK^T and dV^T.
    struct Smem {
        uint16_t q[2][kKvBM * D];                  // row-major, swizzled chunks
        uint16_t dO[2][kKvBM * D];
        float lse[2][kKvBM];
        float dd[2][kKvBM];
    };
    constexpr int RED = DB * 16 * 64;        // floats per (key block, dK or dV) partial
    static_assert(4 * RED * sizeof(float) <= sizeof(Smem), "reduction must fit in the staging LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(Smem)];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

    // Work item = (key tile, batch, kv head, head subset).  The G query heads of
    // a group are split into hs subsets of Gs heads; with hs > 1 the subsets'
    // partial dK/dV are summed with atomics into zero-filled outputs.
    const int BGH = B * Hkv * hs;
    const int kt = blockIdx.x / BGH;         // causal: low key tiles see the most queries
    const int rem = blockIdx.x % BGH;
    const int b = rem / (Hkv * hs), g = (rem / hs) % Hkv, hsub = rem % hs;
    const int G = Hq / Hkv, Gs = G / hs;
    const int k0 = kt * kKvBN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l32 = lane & 31, hf = lane >> 5;
    const int kb = wave & 1, qh = wave >> 1;
    const int kj = k0 + 32 * kb + l32;       // this lane's key column

    const uint32_t ksign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    const uint16_t *Kg = K + ((size_t)b * Hkv + g) * (size_t)N * D;
    const uint16_t *Vg = V + ((size_t)b * Hkv + g) * (size_t)N * D;

    // K^T and V^T operands, resident: lane holds row kj (clamped), dims 16ks + 8hf .. +7.
    bf16x8 kf[KS], vf[KS];
    {
        const int kr = min(kj, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 uk = *(const uint4 *)(Kg + (size_t)kr * D + 16 * ks + 8 * hf);
            const uint4 uv = *(const uint4 *)(Vg + (size_t)kr * D + 16 * ks + 8 * hf);
            uk.x ^= ksign; uk.y ^= ksign; uk.z ^= ksign; uk.w ^= ksign;
            kf[ks] = as_bf16x8(uk);
            vf[ks] = as_bf16x8(uv);
        }
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dva[db][r] = 0.f; dka[db][r] = 0.f; }

    const int nqt = (N + kKvBM - 1) / kKvBM;
    const int qt0 = causal ? k0 / kKvBM : 0;
    const int nq = nqt - qt0;
    const int steps = Gs * nq;               // (query head, query tile) pairs

// Step s covers query head g*G + hsub*Gs + s/nq, query tile qt0 + s%nq.  Its Q and dO
// tiles and its lse and D rows move global -> LDS directly (rows past N are
// clamped to N-1 and masked in the step's arithmetic).
#define ATTN_LOAD_STEP(s_, buf_)                                                                \
    {                                                                                           \
        const size_t hrow_ = ((size_t)b * Hq + g * G + hsub * Gs + (s_) / nq) * N;              \
        const int q0_ = (qt0 + (s_) % nq) * kKvBM;                                              \
        tile_load_lds<D, kKvBM>(sm.q[buf_], Q + hrow_ * D, q0_, N, wave, 4, lane);              \
        tile_load_lds<D, kKvBM>(sm.dO[buf_], dO + hrow_ * D, q0_, N, wave, 4, lane);            \
        const int row_ = min(q0_ + lane, N - 1);                                                \
        if (wave == 0)                                                                          \
            __builtin_amdgcn_global_load_lds((const void *)(LSE + hrow_ + row_),                \
                (__attribute__((address_space(3))) void *)&sm.lse[buf_][0], 4, 0, 0);           \
        else if (wave == 1)                                                                     \
            __builtin_amdgcn_global_load_lds((const void *)(Dws + hrow_ + row_),                \
                (__attribute__((address_space(3))) void *)&sm.dd[buf_][0], 4, 0, 0);            \
    }
    if (steps > 0) ATTN_LOAD_STEP(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        if (s + 1 < steps) ATTN_LOAD_STEP(s + 1, buf ^ 1);   // in flight during the MFMAs
        const int q0 = (qt0 + s % nq) * kKvBM;
        const int qb0 = q0 + 32 * qh;       // first query row of this wave's block
        const bool active = qb0 < N && k0 + 32 * kb < N && (!causal || qb0 + 31 >= k0 + 32 * kb);
        if (active) {
            f32x16 sacc, pacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
            bf16x8 aq[KS], ad[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                aq[ks] = tile_row_operand<D>(sm.q[buf], 32 * qh + l32, 2 * ks + hf);
                ad[ks] = tile_row_operand<D>(sm.dO[buf], 32 * qh + l32, 2 * ks + hf);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = mfma32x32x16(aq[ks], kf[ks], sacc);
                pacc = mfma32x32x16(ad[ks], vf[ks], pacc);
            }
            sched_pipeline<2 * KS, 2 * KS, 4, 1>();
            // P = exp(scale s - lse), dS = P (dP - D); rows are queries, lane = key.
            // Masked (only on diagonal and tail steps, a wave-uniform branch):
            // keys after the query (causal) and query rows past N.
            const bool masked = (causal && qb0 < k0 + 32 * kb + 32) || qb0 + 32 > N;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int rr = 32 * qh + 8 * a + 4 * hf;       // local query row of r = 4a
                const float4 l4 = *(const float4 *)&sm.lse[buf][rr];
                const float4 d4 = *(const float4 *)&sm.dd[buf][rr];
                const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    sacc[r] = exp2_fast(fmaf(sacc[r], c2, -lv[e]));
                    pacc[r] = pacc[r] - dv[e];
                }
                if (masked) {
                    const int qrow = q0 + rr;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool keep = (!causal || kj <= qrow + e) && qrow + e < N;
                        sacc[4 * a + e] = keep ? sacc[4 * a + e] : 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) pacc[4 * a + e] *= sacc[4 * a + e];
            }
            // dV^T += dO^T P,  dK^T += Q^T dS   (contraction over the wave's 32 queries)
            bf16x8 ado[2][DB], aqt[2][DB];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    ado[tt][db] = tr_operand<D>(sm.dO[buf], 32 * qh + 16 * tt, db * 32, lane);
                    aqt[tt][db] = tr_operand<D>(sm.q[buf], 32 * qh + 16 * tt, db * 32, lane);
                }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 pb = tt ? pack_operand<8>(sacc) : pack_operand<0>(sacc);
                const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dva[db] = mfma32x32x16(ado[tt][db], pb, dva[db]);
                    dka[db] = mfma32x32x16(aqt[tt][db], sb, dka[db]);
                }
            }
            sched_pipeline<8 * DB, 4 * DB, 4, 2>();
        }
        __builtin_amdgcn_s_waitcnt(0);      // this wave's prefetch has landed
        __syncthreads();
    }
#undef ATTN_LOAD_STEP

    // Sum the two query halves through LDS, then write dK = scale (dK^T)^T and
    // dV.  Accumulator layout: lane = key column kj, register r = dim
    // db*32 + 8(r/4) + 4hf + (r&3).
    float *red = reinterpret_cast<float *>(smem_raw);   // [key block][dK, dV][DB*16][64]
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[(kb * 2 + 0) * RED + (db * 16 + r) * 64 + lane] = dka[db][r];
                red[(kb * 2 + 1) * RED + (db * 16 + r) * 64 + lane] = dva[db][r];
            }
    }
    __syncthreads();
    if (qh == 0 && kj < N) {
        float *dkrow = dK + (((size_t)b * Hkv + g) * N + kj) * D;
        float *dvrow = dV + (((size_t)b * Hkv + g) * N + kj) * D;
        const float *rk = red + (kb * 2 + 0) * RED + lane;
        const float *rv = red + (kb * 2 + 1) * RED + lane;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = db * 32 + 8 * a + 4 * hf;
                const int r0 = db * 16 + 4 * a;
                float4 k4, v4;
                k4.x = (dka[db][4 * a + 0] + rk[(r0 + 0) * 64]) * scale;
                k4.y = (dka[db][4 * a + 1] + rk[(r0 + 1) * 64]) * scale;
                k4.z = (dka[db][4 * a + 2] + rk[(r0 + 2) * 64]) * scale;
                k4.w = (dka[db][4 * a + 3] + rk[(r0 + 3) * 64]) * scale;
                v4.x = dva[db][4 * a + 0] + rv[(r0 + 0) * 64];
                v4.y = dva[db][4 * a + 1] + rv[(r0 + 1) * 64];
                v4.z = dva[db][4 * a + 2] + rv[(r0 + 2) * 64];
                v4.w = dva[db][4 * a + 3] + rv[(r0 + 3) * 64];
                if (hs == 1) {
                    *(float4 *)(dkrow + d0) = k4;
                    *(float4 *)(dvrow + d0) = v4;
                } else {
                    atomicAdd(dkrow + d0 + 0, k4.x); atomicAdd(dkrow + d0 + 1, k4.y);
                    atomicAdd(dkrow + d0 + 2, k4.z); atomicAdd(dkrow + d0 + 3, k4.w);
                    atomicAdd(dvrow + d0 + 0, v4.x); atomicAdd(dvrow + d0 + 1, v4.y);
                    atomicAdd(dvrow + d0 + 2, v4.z); atomicAdd(dvrow + d0 + 3, v4.w);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kQBM = 128;   // queries per workgroup (32 per wave)
constexpr int kQBN = 64;    // keys per tile

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dQ, int B,
    int Hq, int Hkv, int N, float scale, int causal, int nqt)
{
    constexpr int KS = D / 16, DB = D / 32;

    // K and V tiles, row-major with swizzled 16-byte chunks, double-buffered
    __shared__ __attribute__((aligned(16))) uint16_t sk[2][kQBN * D];
    __shared__ __attribute__((aligned(16))) uint16_t sv[2][kQBN * D];

    const int BH = B * Hq;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // heaviest tiles first
    const int bh = blockIdx.x % BH;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);
    const int q0 = qt * kQBM;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l32 = lane & 31, hf = lane >> 5;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + l32;

    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    const size_t qrow0 = ((size_t)b * Hq + h) * N;
    const uint16_t *Kg = K + ((size_t)b * Hkv + g) * (size_t)N * D;
    const uint16_t *Vg = V + ((size_t)b * Hkv + g) * (size_t)N * D;

    bf16x8 qf[KS], dof[KS];
    {
        const int qr = min(qi, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 uq = *(const uint4 *)(Q + (qrow0 + qr) * D + 16 * ks + 8 * hf);
            const uint4 ud = *(const uint4 *)(dO + (qrow0 + qr) * D + 16 * ks + 8 * hf);
            uq.x ^= qsign; uq.y ^= qsign; uq.z ^= qsign; uq.w ^= qsign;
            qf[ks] = as_bf16x8(uq);
            dof[ks] = as_bf16x8(ud);
        }
    }
    const float lse2 = qi < N ? LSE[qrow0 + qi] * kLog2e : INFINITY;
    const float Di = qi < N ? Dws[qrow0 + qi] : 0.f;

    f32x16 dqa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

    const int kv_end = causal ? min(N, q0 + kQBM) : N;
    const int ntiles = (kv_end + kQBN - 1) / kQBN;

    // Tiles move global -> LDS directly; rows past N are clamped and masked.
    tile_load_lds<D, kQBN>(sk[0], Kg, 0, N, wave, 4, lane);
    tile_load_lds<D, kQBN>(sv[0], Vg, 0, N, wave, 4, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) {       // prefetch into the idle buffer, in flight during the MFMAs
            tile_load_lds<D, kQBN>(sk[buf ^ 1], Kg, (t + 1) * kQBN, N, wave, 4, lane);
            tile_load_lds<D, kQBN>(sv[buf ^ 1], Vg, (t + 1) * kQBN, N, wave, 4, lane);
        }
        const int kv0 = t * kQBN;
        const bool active = qw0 < N && (!causal || kv0 <= qw0 + 31);
        if (active) {
            const bool need_mask = (causal && kv0 + kQBN - 1 > qw0) || kv0 + kQBN > N;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sacc, pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
                bf16x8 ak[KS], av[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    ak[ks] = tile_row_operand<D>(sk[buf], kb * 32 + l32, 2 * ks + hf);
                    av[ks] = tile_row_operand<D>(sv[buf], kb * 32 + l32, 2 * ks + hf);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    sacc = mfma32x32x16(ak[ks], qf[ks], sacc);
                    pacc = mfma32x32x16(av[ks], dof[ks], pacc);
                }
                sched_pipeline<2 * KS, 2 * KS, 4, 1>();
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_fast(fmaf(sacc[r], c2, -lse2));
                    if (need_mask) {
                        const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if ((causal && key > qi) || key >= N) p = 0.f;
                    }
                    pacc[r] = p * (pacc[r] - Di);
                }
                // dQ^T += K^T dS^T over this block's 32 keys (two 16-key steps)
                bf16x8 kt_[2][DB];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        kt_[tt][db] = tr_operand<D>(sk[buf], kb * 32 + 16 * tt, db * 32, lane);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
                    for (int db = 0; db < DB; ++db) dqa[db] = mfma32x32x16(kt_[tt][db], sb, dqa[db]);
                }
                sched_pipeline<4 * DB, 2 * DB, 4, 2>();
            }
        }
        __builtin_amdgcn_s_waitcnt(0);      // this wave's prefetch has landed
        __syncthreads();
    }

    if (qi < N) {
        float *row = dQ + (qrow0 + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = db * 32 + 8 * a + 4 * hf;
                *(float4 *)(row + d0) = make_float4(dqa[db][4 * a + 0] * scale, dqa[db][4 * a + 1] * scale,
                                                    dqa[db][4 * a + 2] * scale, dqa[db][4 * a + 3] * scale);
            }
    }
}

}  // namespace

int dkdv_head_split(int B, int Hq, int Hkv, int N)
{
    // Split each group's query heads over enough workgroups to give every
    // workgroup slot (two per CU) about two causal-imbalanced work items.
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    // Measured on MI355X: f32 atomics into dK/dV cost far more than the load
    // imbalance they remove (4 x 1024 x 64 grouped-query workload: 66 -> 171 us;
    // 32/8 heads at N=4096: no gain), so the split is only taken when the key
    // tiles leave most of the GPU idle.
    const int G = Hq / Hkv;
    const long base = (long)((N + kKvBN - 1) / kKvBN) * B * Hkv;
    int hs = 1;
    for (int c = 1; c <= G; ++c)
        if (G % c == 0) {
            hs = c;
            if (base * c >= cus / 4) break;
        }
    return hs;
}

hipError_t bwd_dkdv_mfma(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         const void *q, const void *k, const void *v, const float *lse,
                         const void *dout, const float *Dws, float *dk, float *dv, int hs,
                         hipStream_t st)
{
    const int nkt = (N + kKvBN - 1) / kKvBN;
    dim3 grid((unsigned)(nkt * B * Hkv * hs));
    if (d == 128)
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dk, dv, B, Hq, Hkv, N, scale, causal, hs);
    else if (d == 64)
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dk, dv, B, Hq, Hkv, N, scale, causal, hs);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t bwd_dq_mfma(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       const void *q, const void *k, const void *v, const float *lse,
                       const void *dout, const float *Dws, float *dq, hipStream_t st)
{
    const int nqt = (N + kQBM - 1) / kQBM;
    dim3 grid((unsigned)(nqt * B * Hq));
    if (d == 128)
        hipLaunchKernelGGL(bwd_dq_kernel<128>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dq, B, Hq, Hkv, N, scale, causal, nqt);
    else if (d == 64)
        hipLaunchKernelGGL(bwd_dq_kernel<64>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dq, B, Hq, Hkv, N, scale, causal, nqt);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
