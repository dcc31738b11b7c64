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
// Two kernels, both deterministic (no atomics):
//   * dkdv: key-stationary.  A workgroup owns 64 keys of one key/value head and
//     keeps their dK^T and dV^T accumulators in registers while it streams the
//     query tiles of every query head of the group past them.  4 waves = 2 key
//     blocks x 2 query halves, each wave a 32x32 (query x key) tile per step;
//     scores are laid out S = Q K^T (lane = key column), so P and dS feed the
//     dV and dK MFMAs straight from registers, and Q^T, dO^T come from the
//     row-major Q and dO tiles through the transposed LDS read.  The two query
//     halves' partials are summed through LDS at the end.
//   * dq: query-stationary, the forward's layout (lane = query row, S^T = K Q^T)
//     with dQ^T = K^T dS^T accumulated in registers; P and dP are recomputed,
//     K^T is read from the row-major K tile through the transposed LDS read.
// Both double-buffer their LDS tiles with one barrier per step, the next
// step's global loads in flight during the current step's MFMAs.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kPad = 16;

// Global -> registers for one tile of 64 rows of two row-major tensors (rows
// past N clamped to N-1; the callers give such rows zero weight), and back to LDS.
template <int D, int CH_T>
__device__ __forceinline__ void load_tile2(uint4 (&a)[CH_T], uint4 (&b)[CH_T], const uint16_t *A,
                                           const uint16_t *Bm, int r0, int N, int tid)
{
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
        const int c = tid + 256 * i;
        const int row = min(r0 + c / (D / 8), N - 1), col = (c % (D / 8)) * 8;
        a[i] = *(const uint4 *)(A + (size_t)row * D + col);
        b[i] = *(const uint4 *)(Bm + (size_t)row * D + col);
    }
}

template <int D, int CH_T, int ROW>
__device__ __forceinline__ void store_tile2(uint16_t (*sa)[ROW], uint16_t (*sb)[ROW],
                                            const uint4 (&a)[CH_T], const uint4 (&b)[CH_T], int tid)
{
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
        const int c = tid + 256 * i;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *(uint4 *)&sa[row][col] = a[i];
        *(uint4 *)&sb[row][col] = b[i];
    }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kKvBN = 64;   // keys per workgroup
constexpr int kKvBM = 64;   // queries per step

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dK,
    float *__restrict__ dV, int B, int Hq, int Hkv, int N, float scale, int causal)
{
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int ROW = D + kPad;
    constexpr int CH_T = kKvBM * D / 8 / 256;      // 16-byte chunks per thread per tile
    static_assert(kKvBM * D / 8 % 256 == 0, "tile must split evenly over the workgroup");

    // One LDS block: double-buffered Q, dO, lse and D tiles during the loop,
    // then the reduction buffer for the two query halves' dK^T and dV^T.
    struct Smem {
        uint16_t q[2][kKvBM][ROW];
        uint16_t dO[2][kKvBM][ROW];
        float lse[2][kKvBM];
        float dd[2][kKvBM];
    };
    constexpr int RED = DB * 16 * 64;        // floats per (key block, dK or dV) partial
    static_assert(4 * RED * sizeof(float) <= sizeof(Smem), "reduction must fit in the staging LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(Smem)];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

    const int BG = B * Hkv;
    const int kt = blockIdx.x / BG;          // causal: low key tiles see the most queries
    const int bg = blockIdx.x % BG;
    const int b = bg / Hkv, g = bg % Hkv;
    const int G = Hq / Hkv;
    const int k0 = kt * kKvBN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
    const int steps = G * nq;                // (query head, query tile) pairs

    uint4 qst[CH_T], dst[CH_T];     // staging registers for one step
    float lst = 0.f, dstv = 0.f;

// step s covers query head g*G + s/nq, query tile qt0 + s%nq
#define ATTN_LOAD_STEP(s_)                                                                      \
    {                                                                                           \
        const size_t hrow_ = ((size_t)b * Hq + g * G + (s_) / nq) * N;                          \
        const int q0_ = (qt0 + (s_) % nq) * kKvBM;                                              \
        load_tile2<D, CH_T>(qst, dst, Q + hrow_ * D, dO + hrow_ * D, q0_, N, tid);              \
        if (tid < kKvBM) {                                                                      \
            const int row_ = q0_ + tid;                                                         \
            lst = row_ < N ? LSE[hrow_ + row_] * kLog2e : INFINITY; /* P = 0 on padded rows */  \
            dstv = row_ < N ? Dws[hrow_ + row_] : 0.f;                                          \
        }                                                                                       \
    }
#define ATTN_STORE_STEP(buf_)                                                                   \
    {                                                                                           \
        store_tile2<D, CH_T, ROW>(sm.q[buf_], sm.dO[buf_], qst, dst, tid);                      \
        if (tid < kKvBM) {                                                                      \
            sm.lse[buf_][tid] = lst;                                                            \
            sm.dd[buf_][tid] = dstv;                                                            \
        }                                                                                       \
    }
    if (steps > 0) {
        ATTN_LOAD_STEP(0);
        ATTN_STORE_STEP(0);
    }
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        // unconditional prefetch (see the dq loop); the last step re-reads itself
        ATTN_LOAD_STEP(min(s + 1, steps - 1));
        const int q0 = (qt0 + s % nq) * kKvBM;
        const int qb0 = q0 + 32 * qh;       // first query row of this wave's block
        const bool active = qb0 < N && k0 + 32 * kb < N && (!causal || qb0 + 31 >= k0 + 32 * kb);
        if (active) {
            f32x16 sacc, pacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 aq = as_bf16x8(*(const uint4 *)&sm.q[buf][32 * qh + l32][16 * ks + 8 * hf]);
                const bf16x8 ad = as_bf16x8(*(const uint4 *)&sm.dO[buf][32 * qh + l32][16 * ks + 8 * hf]);
                sacc = mfma32x32x16(aq, kf[ks], sacc);
                pacc = mfma32x32x16(ad, vf[ks], pacc);
            }
            // P = exp(scale s - lse), dS = P (dP - D); rows are queries, lane = key.
            const bool diag = causal && qb0 < k0 + 32 * kb + 32;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int rr = 32 * qh + 8 * a + 4 * hf;       // local query row of r = 4a
                const float4 l4 = *(const float4 *)&sm.lse[buf][rr];
                const float4 d4 = *(const float4 *)&sm.dd[buf][rr];
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    float p = exp2_fast(fmaf(sacc[r], c2, -lv[e]));
                    if (diag && kj > q0 + rr + e) p = 0.f;
                    sacc[r] = p;
                    pacc[r] = p * (pacc[r] - dv[e]);
                }
            }
            // dV^T += dO^T P,  dK^T += Q^T dS   (contraction over the wave's 32 queries)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const bf16x8 pb = tt ? pack_operand<8>(sacc) : pack_operand<0>(sacc);
                const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 ado = tr_operand(&sm.dO[buf][0][0], ROW, 32 * qh + 16 * tt, db * 32, lane);
                    const bf16x8 aqt = tr_operand(&sm.q[buf][0][0], ROW, 32 * qh + 16 * tt, db * 32, lane);
                    dva[db] = mfma32x32x16(ado, pb, dva[db]);
                    dka[db] = mfma32x32x16(aqt, sb, dka[db]);
                }
            }
        }
        ATTN_STORE_STEP(buf ^ 1);
        __syncthreads();
    }
#undef ATTN_LOAD_STEP
#undef ATTN_STORE_STEP

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
                *(float4 *)(dkrow + d0) = k4;
                *(float4 *)(dvrow + d0) = v4;
            }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kQBM = 128;   // queries per workgroup (32 per wave)
constexpr int kQBN = 64;    // keys per tile

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const float *__restrict__ LSE,
    const uint16_t *__restrict__ dO, const float *__restrict__ Dws, float *__restrict__ dQ, int B,
    int Hq, int Hkv, int N, float scale, int causal, int nqt)
{
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int ROW = D + kPad;
    constexpr int CH_T = kQBN * D / 8 / 256;
    static_assert(kQBN * D / 8 % 256 == 0, "tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) uint16_t sk[2][kQBN][ROW];
    __shared__ __attribute__((aligned(16))) uint16_t sv[2][kQBN][ROW];

    const int BH = B * Hq;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // heaviest tiles first
    const int bh = blockIdx.x % BH;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);
    const int q0 = qt * kQBM;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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

    uint4 kst[CH_T], vst[CH_T];     // staging registers for one tile

    load_tile2<D, CH_T>(kst, vst, Kg, Vg, 0, N, tid);
    store_tile2<D, CH_T, ROW>(sk[0], sv[0], kst, vst, tid);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        // Prefetch unconditionally (the last iteration re-reads its own tile into
        // the idle buffer): a conditional prefetch makes the compiler keep the
        // staging registers in scratch memory.
        load_tile2<D, CH_T>(kst, vst, Kg, Vg, min(t + 1, ntiles - 1) * kQBN, N, tid);
        const int kv0 = t * kQBN;
        const bool active = qw0 < N && (!causal || kv0 <= qw0 + 31);
        if (active) {
            const bool need_mask = (causal && kv0 + kQBN - 1 > qw0) || kv0 + kQBN > N;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sacc, pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 ak = as_bf16x8(*(const uint4 *)&sk[buf][kb * 32 + l32][16 * ks + 8 * hf]);
                    const bf16x8 av = as_bf16x8(*(const uint4 *)&sv[buf][kb * 32 + l32][16 * ks + 8 * hf]);
                    sacc = mfma32x32x16(ak, qf[ks], sacc);
                    pacc = mfma32x32x16(av, dof[ks], pacc);
                }
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
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const bf16x8 sb = tt ? pack_operand<8>(pacc) : pack_operand<0>(pacc);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a = tr_operand(&sk[buf][0][0], ROW, kb * 32 + 16 * tt, db * 32, lane);
                        dqa[db] = mfma32x32x16(a, sb, dqa[db]);
                    }
                }
            }
        }
        store_tile2<D, CH_T, ROW>(sk[buf ^ 1], sv[buf ^ 1], kst, vst, tid);
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

hipError_t bwd_dkdv_mfma(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         const void *q, const void *k, const void *v, const float *lse,
                         const void *dout, const float *Dws, float *dk, float *dv, hipStream_t st)
{
    const int nkt = (N + kKvBN - 1) / kKvBN;
    dim3 grid((unsigned)(nkt * B * Hkv));
    if (d == 128)
        hipLaunchKernelGGL(bwd_dkdv_kernel<128>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dk, dv, B, Hq, Hkv, N, scale, causal);
    else if (d == 64)
        hipLaunchKernelGGL(bwd_dkdv_kernel<64>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, lse, (const uint16_t *)dout,
                           Dws, dk, dv, B, Hq, Hkv, N, scale, causal);
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
