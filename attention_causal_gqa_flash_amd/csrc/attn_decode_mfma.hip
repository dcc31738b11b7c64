// attn_decode_mfma.hip -- split-KV decode on gfx950 matrix cores (bf16 caches).
//
// One new query token per query head attends to every cached key; the keys are
// cut into contiguous chunks, each chunk yields a normalised partial output and
// its log-sum-exp, and the partials combine associatively ("tang --
// differentiable computing in Rust", "How tang works" part 3: the combine is
// associative, so it tiles and parallelises like any sum; the decode workload
// is one row of attention per new token, "RustingBrain" docs, "Generating
// text").  Decoding reads every cached byte once, so the kernel is bound by HBM
// bandwidth ("Generating text": a decode step reads every active weight once).
//
// Layout of the work:
//   * one workgroup per (split, key/value head, batch) handles all G <= 16
//     query heads of the group, so each cached K/V byte is read from HBM once;
//   * 8 waves, each takes 32-key blocks of the chunk (block w, w+8, ...); for
//     the 4096-key, 16-split decode every wave has exactly one block, and all
//     of a workgroup's loads are in flight before any arithmetic;
//   * scores S^T = K q^T on v_mfma_f32_16x16x32_bf16 with K rows loaded from
//     HBM straight into operand registers (no LDS) and q^T resident;
//   * O = P V on the same instruction: P comes from the score registers (each
//     lane holds one head and 4+4 keys, exactly an A operand), V is staged in
//     the wave's own LDS slice and read back key-contiguous with
//     ds_read_b64_tr_b16;
//   * the 8 waves' running states (max, sum, output) merge through LDS with the
//     associative combine, and the workgroup writes (part_o, part_lse).
// The append form (one decode step of a batch of sequences of their own
// lengths, "Generating text": each new token's key and value join the cache)
// reads sequence b's length n from device memory, attends over the n + 1 keys
// 0..n -- key n is the new token's, taken straight from k_new / v_new -- and
// the split-0 workgroup of each (kv head, sequence) writes the new row into the
// cache; no workgroup reads cache row n, so the write races with no read.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kWaves = 8;
constexpr int kBlk = 32;        // keys per wave step

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool APPEND>
__global__ __launch_bounds__(512, APPEND ? 4 : 1) void decode_mfma_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
    float *__restrict__ part_o, float *__restrict__ part_lse, int Hq, int Hkv, int L, float scale,
    int n_splits, const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const int *__restrict__ seq_lens)
{
    constexpr int KS = D / 32;            // k-steps over the head dim (32 per MFMA)
    constexpr int DB = D / 16;            // 16-column blocks of the output
    constexpr int VROW = D + 8;           // padded LDS row of the V tile
    constexpr int VCH = kBlk * D / 8 / 64;   // 16-byte V chunks per lane per block

    // per-wave V tiles; reused afterwards for the cross-wave merge
    constexpr int VBYTES = kWaves * kBlk * VROW * 2;
    constexpr int MBYTES = kWaves * 16 * D * 4 + 2 * kWaves * 16 * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[VBYTES > MBYTES ? VBYTES : MBYTES];
    uint16_t(*sv)[kBlk][VROW] = reinterpret_cast<uint16_t(*)[kBlk][VROW]>(smem);

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l16 = lane & 15, grp = lane >> 4;

    // scores are x = q.k; the softmax runs on x * c2 in base 2 (c2 may be negative)
    const float c2 = scale * kLog2e;

    // keys attended: all L cached ones, or (append) the n + 1 of sequence b
    long Lk = L, nb = -1;
    const uint16_t *Kn = nullptr, *Vn = nullptr;
    if constexpr (APPEND) {
        nb = seq_lens[b];
        if (nb < 0 || nb >= L) {
            // invalid length: nothing is written to the cache; partials that the
            // merge turns into NaN (lse +inf makes every weight inf - inf)
            for (int t = tid; t < G * D; t += 512) {
                const size_t ob = ((size_t)b * Hq + g * G + t / D) * n_splits + s;
                part_o[ob * D + t % D] = NAN;
                if (t % D == 0) part_lse[ob] = INFINITY;
            }
            return;
        }
        Lk = nb + 1;
        Kn = k_new + ((size_t)b * Hkv + g) * D;
        Vn = v_new + ((size_t)b * Hkv + g) * D;
        if (s == 0 && wave == 0 && lane < 2 * (D / 8)) {
            // the new row into the cache, 16 bytes per lane (K: lanes 0..D/8-1)
            const int c = 8 * (lane % (D / 8));
            const uint16_t *src = lane < D / 8 ? Kn : Vn;
            uint16_t *dst = (lane < D / 8 ? kc : vc) + (((size_t)b * Hkv + g) * (size_t)L + nb) * D;
            *(uint4 *)(dst + c) = *(const uint4 *)(src + c);
        }
    }

    const long C = (Lk + n_splits - 1) / n_splits;
    const long j0 = (long)s * C;
    const long j1 = min(Lk, j0 + C);
    const uint16_t *Kg = kc + ((size_t)b * Hkv + g) * (size_t)L * D;
    const uint16_t *Vg = vc + ((size_t)b * Hkv + g) * (size_t)L * D;
    // row `key` of the keys attended (append: key n is the new token's)
    auto krow = [&](long key) { return (APPEND && key == nb) ? Kn : Kg + (size_t)key * D; };
    auto vrow = [&](long key) { return (APPEND && key == nb) ? Vn : Vg + (size_t)key * D; };

    // q^T operand: lane holds head l16 (rows past G read head G-1 and are never
    // written out), dims 32ks + 8grp .. +7.  Loaded without a branch and
    // consumed only by the first MFMA, so its latency overlaps the K/V loads.
    bf16x8 qf[KS];
    {
        const int hq = g * G + min(l16, G - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = as_bf16x8(*(const uint4 *)(q + ((size_t)b * Hq + hq) * D + 32 * ks + 8 * grp));
    }

    float m_run = -INFINITY;   // running max of x * c2 for head l16
    float l_run = 0.f;         // this lane's share of the running sum
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (long kb0 = j0 + (long)kBlk * wave; kb0 < j1; kb0 += (long)kBlk * kWaves) {
        // ---- issue every load of the block: K operands and the V tile ----
        // Rows past the chunk end are clamped to its last key: their scores are
        // masked to -inf below, so their (finite) values get zero weight.
        uint4 kraw[2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint16_t *kr = krow(min(kb0 + 16 * kb + l16, j1 - 1));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kraw[kb][ks] = *(const uint4 *)(kr + 32 * ks + 8 * grp);
        }
        uint4 vraw[VCH];
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            vraw[i] = *(const uint4 *)(vrow(min(kb0 + row, j1 - 1)) + col);
        }
        // ---- scores: S^T (16 keys x 16 heads) for the two 16-key halves ----
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[kb] = mfma16x16x32(as_bf16x8(kraw[kb][ks]), qf[ks], sacc[kb]);
        }
        // lane: head l16, keys kb0 + 16kb + 4grp + r
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = sacc[kb][r] * c2;
                if (kb0 + 16 * kb + 4 * grp + r >= j1) x = -INFINITY;
                sacc[kb][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = pair32_max(pair16_max(mx));
        const float m_new = fmaxf(m_run, mx);            // finite: the block's first key is valid
        const float alpha = m_run == -INFINITY ? 0.f : exp2_fast(m_run - m_new);
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_fast(sacc[kb][r] - m_new);
                sacc[kb][r] = p;
                rs += p;
            }
        l_run = fmaf(l_run, alpha, rs);
        m_run = m_new;
        // rescale the output rows (heads 4grp + r) by their heads' alpha
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db][r] *= ar;
        }
        // P operand: head l16, keys 4grp + 0..3 then 16 + 4grp + 0..3
        const bf16x8 pa = as_bf16x8(make_uint4(pack_bf16x2(sacc[0][0], sacc[0][1]), pack_bf16x2(sacc[0][2], sacc[0][3]),
                                               pack_bf16x2(sacc[1][0], sacc[1][1]), pack_bf16x2(sacc[1][2], sacc[1][3])));
        // ---- V tile to this wave's LDS slice, then O += P V ----
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = lane + 64 * i;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            *(uint4 *)&sv[wave][row][col] = vraw[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // source lane l16 of group grp addresses key (4grp + l16/4), dims 16db + 4(l16%4)
            const uint2 lo = lds_read_tr16(&sv[wave][4 * grp + (l16 >> 2)][16 * db + 4 * (l16 & 3)]);
            const uint2 hi = lds_read_tr16(&sv[wave][16 + 4 * grp + (l16 >> 2)][16 * db + 4 * (l16 & 3)]);
            const bf16x8 vb = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            oacc[db] = mfma16x16x32(pa, vb, oacc[db]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }

    // ---- per-wave state -> LDS, then combine the 8 waves ----
    l_run = pair32_sum(pair16_sum(l_run));
    __syncthreads();                                   // V slices are no longer read
    float *wo = reinterpret_cast<float *>(smem);       // [wave][head 16][D]
    float *wm = wo + kWaves * 16 * D;                  // [wave][16]
    float *wl = wm + kWaves * 16;                      // [wave][16]
    if (grp == 0) {
        wm[wave * 16 + l16] = m_run;
        wl[wave * 16 + l16] = l_run;
    }
    // output layout: lane holds column 16db + l16 of heads 4grp + r
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) wo[(wave * 16 + 4 * grp + r) * D + 16 * db + l16] = oacc[db][r];
    __syncthreads();
    for (int t = tid; t < G * D; t += 512) {
        const int hh = t / D, c = t % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * 16 + hh]);
        const size_t ob = ((size_t)b * Hq + g * G + hh) * n_splits + s;
        if (M == -INFINITY) {                          // empty chunk: the identity
            part_o[ob * D + c] = 0.f;
            if (c == 0) part_lse[ob] = -INFINITY;
            continue;
        }
        float lt = 0.f, at = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = wm[w * 16 + hh];
            if (mw == -INFINITY) continue;
            const float e = exp2_fast(mw - M);
            lt = fmaf(wl[w * 16 + hh], e, lt);
            at = fmaf(wo[(w * 16 + hh) * D + c], e, at);
        }
        part_o[ob * D + c] = at / lt;
        if (c == 0) part_lse[ob] = M * kLn2 + logf(lt);
    }
}

}  // namespace

bool decode_mfma_supported(int dt, int d, int G) { return dt == kBF16 && (d == 64 || d == 128) && G <= 16; }

hipError_t decode_split_mfma(int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                             const void *q, const void *kc, const void *vc, float *part_o,
                             float *part_lse, hipStream_t st)
{
    // the plain form never writes the caches
    uint16_t *k = const_cast<uint16_t *>((const uint16_t *)kc);
    uint16_t *v = const_cast<uint16_t *>((const uint16_t *)vc);
    dim3 grid(n_splits, Hkv, B);
    if (d == 128)
        hipLaunchKernelGGL((decode_mfma_kernel<128, false>), grid, dim3(512), 0, st, (const uint16_t *)q,
                           k, v, part_o, part_lse, Hq, Hkv, L, scale, n_splits, nullptr, nullptr,
                           nullptr);
    else if (d == 64)
        hipLaunchKernelGGL((decode_mfma_kernel<64, false>), grid, dim3(512), 0, st, (const uint16_t *)q,
                           k, v, part_o, part_lse, Hq, Hkv, L, scale, n_splits, nullptr, nullptr,
                           nullptr);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t decode_append_mfma(int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                              const void *q, const void *k_new, const void *v_new, void *kc,
                              void *vc, const int *seq_lens, float *part_o, float *part_lse,
                              hipStream_t st)
{
    dim3 grid(n_splits, Hkv, B);
    if (d == 128)
        hipLaunchKernelGGL((decode_mfma_kernel<128, true>), grid, dim3(512), 0, st, (const uint16_t *)q,
                           (uint16_t *)kc, (uint16_t *)vc, part_o, part_lse, Hq, Hkv, L, scale,
                           n_splits, (const uint16_t *)k_new, (const uint16_t *)v_new, seq_lens);
    else if (d == 64)
        hipLaunchKernelGGL((decode_mfma_kernel<64, true>), grid, dim3(512), 0, st, (const uint16_t *)q,
                           (uint16_t *)kc, (uint16_t *)vc, part_o, part_lse, Hq, Hkv, L, scale,
                           n_splits, (const uint16_t *)k_new, (const uint16_t *)v_new, seq_lens);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
