// attn_fwd_mfma.hip -- causal grouped-query attention forward on gfx950
// matrix cores (bf16 operands, f32 accumulation).
//
// Method: the softmax max and its two sums become one streaming reduction over
// keys that carries three running values per query row -- running max m,
// running sum l and running weighted sum of values acc -- so no score or
// probability ever leaves registers ("tang -- differentiable computing in
// Rust", "How tang works" part 3 "Optimizations are derived, not written",
// equations (5) and (6)).  Causal masking as in the fused causal kernel of the
// RustingBrain docs ("What is in the box"); grouped-query head sharing as in
// the same docs.
//
// Layout of the work (MI355X-first, not a translation of any other design):
//   * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//     each wave owns 32 query rows and every lane owns ONE query row, so the
//     softmax state (m, l) of a row lives in a single lane pair (l, l^32);
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the accumulator layout then gives each lane one query and 16 keys, the
//     row max needs one cross-lane exchange and the row sum none until the end;
//   * the output is accumulated transposed too, O^T = V^T P^T, so the per-row
//     rescale by alpha is a per-lane scalar and P^T feeds the next MFMA
//     straight from registers (the key order inside an MFMA step is permuted to
//     match the accumulator layout; V^T is read with the same permutation);
//   * K tiles are staged in LDS row-major, V tiles transposed (key-contiguous)
//     by a register 4x8 transpose on the way in, double-buffered with one
//     barrier per tile; the next tile's global loads are in flight during the
//     current tile's MFMAs;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA;
//   * the grid is ordered heaviest query tiles first (causal tiles near the end
//     of the sequence see the most keys).
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kPad = 8;    // bf16 padding per LDS row (keeps 16-byte alignment, spreads banks)

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE, int B, int Hq,
    int Hkv, int N, float scale, int causal, int nqt)
{
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int DB = D / 32;              // 32-row blocks of O^T
    constexpr int KROW = D + kPad;          // LDS row length of the K tile
    constexpr int VROW = kBN + kPad;        // LDS row length of the V^T tile
    constexpr int KCH = kBN * D / 8;        // 16-byte chunks per K tile
    constexpr int KCH_T = KCH / 256;
    constexpr int VUN = (kBN / 4) * (D / 8);   // 4-key x 8-dim transpose units per V tile
    constexpr int VUN_T = (VUN + 255) / 256;
    static_assert(KCH % 256 == 0, "K tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) uint16_t sk[2][kBN][KROW];
    __shared__ __attribute__((aligned(16))) uint16_t svt[2][D][VROW];

    const int BH = B * Hq;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // heaviest tiles first
    const int bh = blockIdx.x % BH;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);
    const int q0 = qt * kBM;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int qw0 = q0 + wave * 32;         // first query row of this wave
    const int qi = qw0 + l32;               // this lane's query row

    const uint16_t *Qh = Q + ((size_t)b * Hq + h) * (size_t)N * D;
    const uint16_t *Kg = K + ((size_t)b * Hkv + g) * (size_t)N * D;
    const uint16_t *Vg = V + ((size_t)b * Hkv + g) * (size_t)N * D;

    // The softmax is computed on x = q.k scaled by c = |scale| log2(e) > 0; a
    // negative scale is carried by negating q, which is exact in bf16.
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float cabs = fabsf(scale);
    const float c2 = cabs * kLog2e;

    // Q^T operand, resident for the whole loop: lane holds q[qi][16ks + 8hf .. +7].
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qi < N) u = *(const uint4 *)(Qh + (size_t)qi * D + 16 * ks + 8 * hf);
        u.x ^= qsign; u.y ^= qsign; u.z ^= qsign; u.w ^= qsign;
        qf[ks] = as_bf16x8(u);
    }

    const int kv_end = causal ? min(N, q0 + kBM) : N;
    const int ntiles = (kv_end + kBN - 1) / kBN;

    uint4 kst[KCH_T];
    uint4 vst[VUN_T][4];

    auto load_tile = [&](int t) {
        const int kv0 = t * kBN;
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            kst[i] = make_uint4(0, 0, 0, 0);
            if (kv0 + row < N) kst[i] = *(const uint4 *)(Kg + (size_t)(kv0 + row) * D + col);
        }
#pragma unroll
        for (int i = 0; i < VUN_T; ++i) {
            const int u = tid + 256 * i;
            if (u < VUN) {
                const int kq = u / (D / 8), dc = u % (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kv0 + 4 * kq + r;
                    vst[i][r] = make_uint4(0, 0, 0, 0);
                    if (key < N) vst[i][r] = *(const uint4 *)(Vg + (size_t)key * D + dc * 8);
                }
            }
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            *(uint4 *)&sk[buf][row][col] = kst[i];
        }
#pragma unroll
        for (int i = 0; i < VUN_T; ++i) {
            const int u = tid + 256 * i;
            if (u < VUN) {
                const int kq = u / (D / 8), dc = u % (D / 8);
                const uint32_t w0[4] = {vst[i][0].x, vst[i][0].y, vst[i][0].z, vst[i][0].w};
                const uint32_t w1[4] = {vst[i][1].x, vst[i][1].y, vst[i][1].z, vst[i][1].w};
                const uint32_t w2[4] = {vst[i][2].x, vst[i][2].y, vst[i][2].z, vst[i][2].w};
                const uint32_t w3[4] = {vst[i][3].x, vst[i][3].y, vst[i][3].z, vst[i][3].w};
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
                    *(uint2 *)&svt[buf][dc * 8 + e][4 * kq] = make_uint2(lo, hi);
                }
            }
        }
    };

    float m_run = -INFINITY;   // running max of x for this lane's row
    float l_run = 0.f;         // this lane's share of the running sum
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);
        const int kv0 = t * kBN;
        const bool active = qw0 < N && (!causal || kv0 <= qw0 + 31);
        if (active) {
            // S^T = K Q^T for the 64 keys of the tile, two 32-key blocks.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = as_bf16x8(*(const uint4 *)&sk[buf][kb * 32 + l32][16 * ks + 8 * hf]);
                    sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
                }
            }
            // Mask keys after the query (causal) and past the end of the sequence.
            if ((causal && kv0 + kBN - 1 > qw0) || kv0 + kBN > N) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if ((causal && key > qi) || key >= N) sacc[kb][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);          // finite: key 0 is seen first
            const float alpha = m_run == -INFINITY ? 0.f : exp2_fast((m_run - m_new) * c2);
            const float mc = m_new * c2;
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(fmaf(sacc[kb][r], c2, -mc));
                    sacc[kb][r] = p;
                    rs += p;
                }
            l_run = fmaf(l_run, alpha, rs);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;

            // O^T += V^T P^T, four 16-key steps.  Step tt consumes accumulator
            // registers (tt&1)*8 .. +7 of block tt>>1, i.e. keys
            // 16tt + 8(e/4) + 4hf + (e&3) for element e; V^T is read likewise.
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int kb = tt >> 1, r0 = (tt & 1) * 8;
                const uint4 pu = make_uint4(pack_bf16x2(sacc[kb][r0 + 0], sacc[kb][r0 + 1]),
                                            pack_bf16x2(sacc[kb][r0 + 2], sacc[kb][r0 + 3]),
                                            pack_bf16x2(sacc[kb][r0 + 4], sacc[kb][r0 + 5]),
                                            pack_bf16x2(sacc[kb][r0 + 6], sacc[kb][r0 + 7]));
                const bf16x8 pb = as_bf16x8(pu);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint2 lo = *(const uint2 *)&svt[buf][db * 32 + l32][16 * tt + 4 * hf];
                    const uint2 hi = *(const uint2 *)&svt[buf][db * 32 + l32][16 * tt + 8 + 4 * hf];
                    const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                    oacc[db] = mfma32x32x16(a, pb, oacc[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < N) {
        const float inv = 1.f / l_tot;
        float *orow = O + (((size_t)b * Hq + h) * N + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = db * 32 + 8 * a + 4 * hf;
                *(float4 *)(orow + d0) = make_float4(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv,
                                                     oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
            }
        if (hf == 0) LSE[((size_t)b * Hq + h) * N + qi] = m_run * cabs + logf(l_tot);
    }
}

}  // namespace

bool mfma_supported(int dt, int d) { return dt == kBF16 && (d == 64 || d == 128); }

hipError_t fwd_mfma(int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                    const void *q, const void *k, const void *v, float *o, float *lse,
                    hipStream_t st)
{
    const int nqt = (N + kBM - 1) / kBM;
    dim3 grid((unsigned)(nqt * B * Hq));
    if (d == 128)
        hipLaunchKernelGGL(fwd_mfma_kernel<128>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, o, lse, B, Hq, Hkv, N, scale,
                           causal, nqt);
    else if (d == 64)
        hipLaunchKernelGGL(fwd_mfma_kernel<64>, grid, dim3(256), 0, st, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, o, lse, B, Hq, Hkv, N, scale,
                           causal, nqt);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
