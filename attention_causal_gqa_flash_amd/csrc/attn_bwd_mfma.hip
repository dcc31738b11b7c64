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
//     dV and dK MFMAs straight from registers.  The two query-half partials are
//     summed through LDS at the end.
//   * dq: query-stationary, the forward's layout (lane = query row, S^T = K Q^T)
//     with dQ^T = K^T dS^T accumulated in registers; P and dP are recomputed.
// Staging: every tile is loaded as (4 rows x 8 columns) units, stored to LDS
// row-major and, where an MFMA needs the other operand order, also transposed
// (the 4x8 block is transposed in registers and written as 8-byte rows).
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kPad = 8;

// Transpose a 4-row x 8-column bf16 block held as 4 rows of uint4 and write it
// as 8 rows of 4 elements: dst(e, 0..3) = src(0..3, e); row stride in elements.
__device__ __forceinline__ void store_transposed_4x8(uint16_t *dst, int stride, const uint4 (&r)[4])
{
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
    const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
            lo = (w0[wd] >> 16) | (w1[wd] & 0xffff0000u);
            hi = (w2[wd] >> 16) | (w3[wd] & 0xffff0000u);
        } else {
            lo = (w0[wd] & 0xffffu) | (w1[wd] << 16);
            hi = (w2[wd] & 0xffffu) | (w3[wd] << 16);
        }
        *(uint2 *)(dst + (size_t)e * stride) = make_uint2(lo, hi);
    }
}

// 8 bf16 of an MFMA operand read from a key- or query-contiguous LDS row in the
// permuted order that matches the 32x32 accumulator layout: elements
// 0..3 = row[16t + 4hf + 0..3], elements 4..7 = row[16t + 8 + 4hf + 0..3].
__device__ __forceinline__ bf16x8 read_perm_operand(const uint16_t *row, int t, int hf)
{
    const uint2 lo = *(const uint2 *)(row + 16 * t + 4 * hf);
    const uint2 hi = *(const uint2 *)(row + 16 * t + 8 + 4 * hf);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Accumulator registers r0..r0+7 packed to a bf16 MFMA operand.
__device__ __forceinline__ bf16x8 pack_operand(const f32x16 &acc, int r0)
{
    return as_bf16x8(make_uint4(pack_bf16x2(acc[r0 + 0], acc[r0 + 1]), pack_bf16x2(acc[r0 + 2], acc[r0 + 3]),
                                pack_bf16x2(acc[r0 + 4], acc[r0 + 5]), pack_bf16x2(acc[r0 + 6], acc[r0 + 7])));
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
    constexpr int ROW = D + kPad;            // row-major tiles [64][ROW]
    constexpr int TROW = kKvBM + kPad;       // transposed tiles [D][TROW]
    constexpr int UNITS = (kKvBM / 4) * (D / 8);
    constexpr int UNITS_T = (UNITS + 255) / 256;

    // One LDS block: the staging tiles during the loop, then the reduction
    // buffer for the two query halves' partial dK^T and dV^T.
    struct Smem {
        uint16_t q[kKvBM][ROW];
        uint16_t dO[kKvBM][ROW];
        uint16_t qt[D][TROW];
        uint16_t dOt[D][TROW];
        float lse[kKvBM];
        float dd[kKvBM];
    };
    constexpr int RED = DB * 16 * 64;        // floats per (key block, dK or dV) partial
    static_assert(4 * RED * sizeof(float) <= sizeof(Smem), "reduction must fit in the staging LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[sizeof(Smem)];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
    auto &sq = sm.q;
    auto &sdo = sm.dO;
    auto &sqt = sm.qt;
    auto &sdot = sm.dOt;
    auto &slse = sm.lse;
    auto &sdd = sm.dd;

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

    // K^T and V^T operands, resident: lane holds row kj, dims 16ks + 8hf .. +7.
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 uk = make_uint4(0, 0, 0, 0), uv = make_uint4(0, 0, 0, 0);
        if (kj < N) {
            uk = *(const uint4 *)(Kg + (size_t)kj * D + 16 * ks + 8 * hf);
            uv = *(const uint4 *)(Vg + (size_t)kj * D + 16 * ks + 8 * hf);
        }
        uk.x ^= ksign; uk.y ^= ksign; uk.z ^= ksign; uk.w ^= ksign;
        kf[ks] = as_bf16x8(uk);
        vf[ks] = as_bf16x8(uv);
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dva[db][r] = 0.f; dka[db][r] = 0.f; }

    const int nqt = (N + kKvBM - 1) / kKvBM;
    const int qt0 = causal ? k0 / kKvBM : 0;

    uint4 qst[UNITS_T][4], dst[UNITS_T][4];
    float lst = 0.f, dstv = 0.f;

    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        const uint16_t *Qh = Q + ((size_t)b * Hq + h) * (size_t)N * D;
        const uint16_t *dOh = dO + ((size_t)b * Hq + h) * (size_t)N * D;
        const float *Lh = LSE + ((size_t)b * Hq + h) * N;
        const float *Dh = Dws + ((size_t)b * Hq + h) * N;
        for (int qt = qt0; qt < nqt; ++qt) {
            const int q0 = qt * kKvBM;
            // global -> registers
#pragma unroll
            for (int i = 0; i < UNITS_T; ++i) {
                const int u = tid + 256 * i;
                if (u < UNITS) {
                    const int rq = u / (D / 8), dc = u % (D / 8);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = q0 + 4 * rq + r;
                        qst[i][r] = make_uint4(0, 0, 0, 0);
                        dst[i][r] = make_uint4(0, 0, 0, 0);
                        if (row < N) {
                            qst[i][r] = *(const uint4 *)(Qh + (size_t)row * D + dc * 8);
                            dst[i][r] = *(const uint4 *)(dOh + (size_t)row * D + dc * 8);
                        }
                    }
                }
            }
            if (tid < kKvBM) {
                const int row = q0 + tid;
                lst = row < N ? Lh[row] * kLog2e : INFINITY;   // P = 0 on padded rows
                dstv = row < N ? Dh[row] : 0.f;
            }
            __syncthreads();   // previous step's readers are done with LDS
#pragma unroll
            for (int i = 0; i < UNITS_T; ++i) {
                const int u = tid + 256 * i;
                if (u < UNITS) {
                    const int rq = u / (D / 8), dc = u % (D / 8);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        *(uint4 *)&sq[4 * rq + r][dc * 8] = qst[i][r];
                        *(uint4 *)&sdo[4 * rq + r][dc * 8] = dst[i][r];
                    }
                    store_transposed_4x8(&sqt[dc * 8][4 * rq], TROW, qst[i]);
                    store_transposed_4x8(&sdot[dc * 8][4 * rq], TROW, dst[i]);
                }
            }
            if (tid < kKvBM) {
                slse[tid] = lst;
                sdd[tid] = dstv;
            }
            __syncthreads();

            const int qb0 = q0 + 32 * qh;    // first query row of this wave's block
            const bool active = qb0 < N && kj - l32 < N && (!causal || qb0 + 31 >= k0 + 32 * kb);
            if (active) {
                f32x16 sacc, pacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; pacc[r] = 0.f; }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 aq = as_bf16x8(*(const uint4 *)&sq[32 * qh + l32][16 * ks + 8 * hf]);
                    const bf16x8 ad = as_bf16x8(*(const uint4 *)&sdo[32 * qh + l32][16 * ks + 8 * hf]);
                    sacc = mfma32x32x16(aq, kf[ks], sacc);
                    pacc = mfma32x32x16(ad, vf[ks], pacc);
                }
                // P = exp(scale s - lse), dS = P (dP - D); rows are queries, lane = key.
                const bool diag = causal && qb0 < k0 + 32 * kb + 32;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int rr = 32 * qh + 8 * a + 4 * hf;       // local query row of r = 4a
                    const float4 l4 = *(const float4 *)&slse[rr];
                    const float4 d4 = *(const float4 *)&sdd[rr];
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
                // dV^T += dO^T P,  dK^T += Q^T dS   (k = the wave's 32 queries)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const bf16x8 pb = pack_operand(sacc, 8 * tt);
                    const bf16x8 sb = pack_operand(pacc, 8 * tt);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 ado = read_perm_operand(&sdot[db * 32 + l32][32 * qh], tt, hf);
                        const bf16x8 aqt = read_perm_operand(&sqt[db * 32 + l32][32 * qh], tt, hf);
                        dva[db] = mfma32x32x16(ado, pb, dva[db]);
                        dka[db] = mfma32x32x16(aqt, sb, dka[db]);
                    }
                }
            }
        }
    }

    // Sum the two query halves through LDS (reusing the staging buffers), then
    // write dK = scale dK^T^T and dV.  Accumulator layout: lane = key column kj,
    // register r = dim db*32 + 8(r/4) + 4hf + (r&3).
    __syncthreads();
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
        const float sgn_scale = scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = db * 32 + 8 * a + 4 * hf;
                float4 k4, v4;
                k4.x = (dka[db][4 * a + 0] + red[(kb * 2) * RED + (db * 16 + 4 * a + 0) * 64 + lane]) * sgn_scale;
                k4.y = (dka[db][4 * a + 1] + red[(kb * 2) * RED + (db * 16 + 4 * a + 1) * 64 + lane]) * sgn_scale;
                k4.z = (dka[db][4 * a + 2] + red[(kb * 2) * RED + (db * 16 + 4 * a + 2) * 64 + lane]) * sgn_scale;
                k4.w = (dka[db][4 * a + 3] + red[(kb * 2) * RED + (db * 16 + 4 * a + 3) * 64 + lane]) * sgn_scale;
                v4.x = dva[db][4 * a + 0] + red[(kb * 2 + 1) * RED + (db * 16 + 4 * a + 0) * 64 + lane];
                v4.y = dva[db][4 * a + 1] + red[(kb * 2 + 1) * RED + (db * 16 + 4 * a + 1) * 64 + lane];
                v4.z = dva[db][4 * a + 2] + red[(kb * 2 + 1) * RED + (db * 16 + 4 * a + 2) * 64 + lane];
                v4.w = dva[db][4 * a + 3] + red[(kb * 2 + 1) * RED + (db * 16 + 4 * a + 3) * 64 + lane];
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
    constexpr int TROW = kQBN + kPad;
    constexpr int UNITS = (kQBN / 4) * (D / 8);
    constexpr int UNITS_T = (UNITS + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint16_t sk[kQBN][ROW];
    __shared__ __attribute__((aligned(16))) uint16_t sv[kQBN][ROW];
    __shared__ __attribute__((aligned(16))) uint16_t skt[D][TROW];

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
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 uq = make_uint4(0, 0, 0, 0), ud = make_uint4(0, 0, 0, 0);
        if (qi < N) {
            uq = *(const uint4 *)(Q + (qrow0 + qi) * D + 16 * ks + 8 * hf);
            ud = *(const uint4 *)(dO + (qrow0 + qi) * D + 16 * ks + 8 * hf);
        }
        uq.x ^= qsign; uq.y ^= qsign; uq.z ^= qsign; uq.w ^= qsign;
        qf[ks] = as_bf16x8(uq);
        dof[ks] = as_bf16x8(ud);
    }
    const float lse2 = qi < N ? LSE[qrow0 + qi] * kLog2e : 0.f;
    const float Di = qi < N ? Dws[qrow0 + qi] : 0.f;

    f32x16 dqa[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

    const int kv_end = causal ? min(N, q0 + kQBM) : N;
    const int ntiles = (kv_end + kQBN - 1) / kQBN;
    uint4 kst[UNITS_T][4], vst[UNITS_T][4];

    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = t * kQBN;
#pragma unroll
        for (int i = 0; i < UNITS_T; ++i) {
            const int u = tid + 256 * i;
            if (u < UNITS) {
                const int rk = u / (D / 8), dc = u % (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kv0 + 4 * rk + r;
                    kst[i][r] = make_uint4(0, 0, 0, 0);
                    vst[i][r] = make_uint4(0, 0, 0, 0);
                    if (key < N) {
                        kst[i][r] = *(const uint4 *)(Kg + (size_t)key * D + dc * 8);
                        vst[i][r] = *(const uint4 *)(Vg + (size_t)key * D + dc * 8);
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < UNITS_T; ++i) {
            const int u = tid + 256 * i;
            if (u < UNITS) {
                const int rk = u / (D / 8), dc = u % (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *(uint4 *)&sk[4 * rk + r][dc * 8] = kst[i][r];
                    *(uint4 *)&sv[4 * rk + r][dc * 8] = vst[i][r];
                }
                store_transposed_4x8(&skt[dc * 8][4 * rk], TROW, kst[i]);
            }
        }
        __syncthreads();

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
                    const bf16x8 ak = as_bf16x8(*(const uint4 *)&sk[kb * 32 + l32][16 * ks + 8 * hf]);
                    const bf16x8 av = as_bf16x8(*(const uint4 *)&sv[kb * 32 + l32][16 * ks + 8 * hf]);
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
                    const bf16x8 sb = pack_operand(pacc, 8 * tt);
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a = read_perm_operand(&skt[db * 32 + l32][kb * 32], tt, hf);
                        dqa[db] = mfma32x32x16(a, sb, dqa[db]);
                    }
                }
            }
        }
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
