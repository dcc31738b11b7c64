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
// Layout of the work:
//   * one workgroup = 4 waves = 128 query rows of one (batch, query head);
//     each wave owns 32 query rows and every lane owns ONE query row, so the
//     softmax state (m, l) of a row lives in a single lane pair (l, l^32);
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     the accumulator layout then gives each lane one query and 16 keys per
//     32-key block, the row max needs one cross-lane exchange and the row sum
//     none until the end;
//   * the output is accumulated transposed too, O^T = V^T P^T: the per-row
//     rescale is a per-lane scalar and P^T feeds the next MFMA straight from
//     the score registers; V^T is read from the row-major V tile with the
//     gfx950 transposed LDS read, in the key order of the score accumulator;
//   * K and V tiles stay row-major in LDS, double-buffered, one barrier per
//     tile, the next tile's global loads in flight during the current MFMAs;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA, and the
//     running max is only raised when a row's tile max exceeds it by more than
//     kLazy (log2 units), so most tiles skip the rescale of O entirely
//     (probabilities then stay below 2^kLazy, well inside f32 and bf16 range);
//   * the grid is ordered heaviest query tiles first.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kPad = 16;      // bf16 padding per LDS row
constexpr float kLazy = 8.f;  // max growth tolerated before rescaling (log2 units)

// Global -> registers for one K/V tile of kBN rows (rows past N clamped to
// N-1: their scores are masked, so their finite values carry zero weight).
template <int D, int CH_T>
__device__ __forceinline__ void load_kv_tile(uint4 (&kst)[CH_T], uint4 (&vst)[CH_T],
                                             const uint16_t *Kg, const uint16_t *Vg, int kv0,
                                             int N, int tid)
{
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
        const int c = tid + 256 * i;
        const int row = min(kv0 + c / (D / 8), N - 1), col = (c % (D / 8)) * 8;
        kst[i] = *(const uint4 *)(Kg + (size_t)row * D + col);
        vst[i] = *(const uint4 *)(Vg + (size_t)row * D + col);
    }
}

template <int D, int CH_T, int ROW>
__device__ __forceinline__ void store_kv_tile(uint16_t (*sk)[ROW], uint16_t (*sv)[ROW],
                                              const uint4 (&kst)[CH_T], const uint4 (&vst)[CH_T],
                                              int tid)
{
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
        const int c = tid + 256 * i;
        const int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *(uint4 *)&sk[row][col] = kst[i];
        *(uint4 *)&sv[row][col] = vst[i];
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE, int B, int Hq,
    int Hkv, int N, float scale, int causal, int nqt)
{
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int DB = D / 32;              // 32-row blocks of O^T
    constexpr int ROW = D + kPad;           // LDS row length of the K and V tiles
    constexpr int CH = kBN * D / 8;         // 16-byte chunks per tile
    constexpr int CH_T = CH / 256;
    static_assert(CH % 256 == 0, "tile must split evenly over the workgroup");

    __shared__ __attribute__((aligned(16))) uint16_t sk[2][kBN][ROW];
    __shared__ __attribute__((aligned(16))) uint16_t sv[2][kBN][ROW];

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

    // Softmax on x = q.k scaled by c2 = |scale| log2(e) > 0; a negative scale
    // is carried by negating q, which is exact in bf16.
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float cabs = fabsf(scale);
    const float c2 = cabs * kLog2e;

    // Q^T operand, resident: lane holds q[qi][16ks + 8hf .. +7] (rows past N read row N-1).
    bf16x8 qf[KS];
    {
        const int qr = min(qi, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 u = *(const uint4 *)(Qh + (size_t)qr * D + 16 * ks + 8 * hf);
            u.x ^= qsign; u.y ^= qsign; u.z ^= qsign; u.w ^= qsign;
            qf[ks] = as_bf16x8(u);
        }
    }

    const int kv_end = causal ? min(N, q0 + kBM) : N;
    const int ntiles = (kv_end + kBN - 1) / kBN;

    uint4 kst[CH_T], vst[CH_T];     // staging registers for one tile

    float m_run = -INFINITY;   // running max of x * c2 for this lane's row
    float l_run = 0.f;         // this lane's share of the running sum
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

    load_kv_tile<D>(kst, vst, Kg, Vg, 0, N, tid);
    store_kv_tile<D, CH_T, ROW>(sk[0], sv[0], kst, vst, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        // Prefetch unconditionally (the last iteration re-reads its own tile into
        // the idle buffer): a conditional prefetch makes the compiler keep the
        // staging registers in scratch memory.
        load_kv_tile<D>(kst, vst, Kg, Vg, min(t + 1, ntiles - 1) * kBN, N, tid);
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
            // scale to log2 units; mask keys after the query and past the sequence end
            const bool need_mask = (causal && kv0 + kBN - 1 > qw0) || kv0 + kBN > N;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = sacc[kb][r] * c2;
                    if (need_mask) {
                        const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if ((causal && key > qi) || key >= N) x = -INFINITY;
                    }
                    sacc[kb][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // lazy rescale: raise the running max only when some row of the wave
            // grew past it by more than kLazy; the first tile always sets it.
            if (__any(mx > m_run + kLazy)) {
                const float m_new = fmaxf(m_run, mx);      // finite: key 0 is in the first tile
                const float alpha = m_run == -INFINITY ? 0.f : exp2_fast(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m_run = m_new;
            }
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(sacc[kb][r] - m_run);
                    sacc[kb][r] = p;
                    rs += p;
                }
            l_run += rs;

            // O^T += V^T P^T, four 16-key steps.  Step tt consumes accumulator
            // registers (tt&1)*8 .. +7 of block tt>>1, i.e. keys 16tt + 4hf + {0..3}
            // and 16tt + 8 + 4hf + {0..3}; tr_operand reads V^T in that order.
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 pb = (tt & 1) ? pack_operand<8>(sacc[tt >> 1]) : pack_operand<0>(sacc[tt >> 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = tr_operand(&sv[buf][0][0], ROW, 16 * tt, db * 32, lane);
                    oacc[db] = mfma32x32x16(a, pb, oacc[db]);
                }
            }
        }
        store_kv_tile<D, CH_T, ROW>(sk[buf ^ 1], sv[buf ^ 1], kst, vst, tid);
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
        // lse = ln(sum exp(scale q.k)) = (m + log2 l) * ln 2
        if (hf == 0) LSE[((size_t)b * Hq + h) * N + qi] = (m_run + __log2f(l_tot)) * kLn2;
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
