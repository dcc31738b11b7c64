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
//   * V goes straight from HBM into the wave's own LDS tile (buffer_load ...
//     lds: no registers, and the LDS writes happen while the loads arrive, not
//     after); K rows load into MFMA operand registers; both through buffer
//     resources whose rows past the keys attended read as zero, so no address
//     is clamped;
//   * scores S^T = K q^T on v_mfma_f32_16x16x32_bf16 with q^T resident; its 16
//     columns are the G heads, each repeated 16/G times (column n is head
//     n G / 16), so that at G = 4 every lane of the output holds a real head;
//   * O = P V on the same instruction: P comes from the score registers (each
//     lane holds one column and 4+4 keys, exactly an A operand), V is read
//     key-contiguous from the swizzled tile with ds_read_b64_tr_b16;
//   * the 8 waves' states (max, sum, output) merge through LDS with the
//     associative combine -- only one copy of each head's output row is
//     written -- and the workgroup writes (part_o, part_lse).
// The append form (one decode step of a batch of sequences of their own
// lengths, "Generating text": each new token's key and value join the cache)
// reads sequence b's length n from device memory, attends over the n + 1 keys
// 0..n -- key n is the new token's, taken straight from k_new / v_new -- and
// the split-0 workgroup of each (kv head, sequence) writes the new row into the
// cache; no workgroup reads cache row n (the resources end at row n), so the
// write races with no read.
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

// The per-wave V tile is [32 keys][D] bf16 with logical 16-byte chunk c of row
// r stored at chunk c ^ vswz(r).  One transposed read of the P V operand takes,
// in each half wave, 8 rows x one 32-byte chunk pair; vswz sends those 8 pairs
// to 8 distinct 32-byte bank groups of the 256-byte-wide LDS (one 256-byte row
// each at D = 128, two 128-byte rows per 256 bytes at D = 64).  The swizzle
// only flips bits 5.. of the byte offset within a row, so the address of
// column block db is the block-0 address XOR 32 db.
template <int D>
__device__ __forceinline__ int vswz(int r)
{
    return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// The per-wave K tile (same shape) uses chunk c ^ kswz(r): the score operand
// reads 16 consecutive rows at one logical chunk per 16 lanes, which kswz
// spreads over 16 distinct 16-byte bank groups.  The XOR only touches bits
// 4.. of the byte offset within a row, so the four k-steps of a lane are its
// k-step-0 address XOR 64 ks.
template <int D>
__device__ __forceinline__ int kswz(int r)
{
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
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
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int RPB = 64 / CPR;         // rows per 1 KiB direct copy
    constexpr int VBLK = kBlk / RPB;      // direct copies per V tile
    constexpr int NKV = D == 128 ? 4 : 2; // distinct K copy offsets (the K swizzle's period in blocks)
    // LDS: per-wave K and V tiles (the append form, two workgroups per compute
    // unit, keeps K in registers), per-wave (max, sum); the f32 output rows
    // [wave][16][D] (as large as one set of tiles) reuse the K tiles (append:
    // the V tiles) once every wave is past them.  Separate arrays, so that
    // reads of one tile set wait only for the copies into that set.
    __shared__ __attribute__((aligned(1024))) uint16_t sk[APPEND ? 8 : kWaves * kBlk * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sv[kWaves * kBlk * D];
    __shared__ __attribute__((aligned(16))) float wml[2 * kWaves * 16];
    float *const wo = reinterpret_cast<float *>(APPEND ? sv : sk);            // [wave][16][D]
    float *const wm = wml;                                                    // [head][wave]
    float *const wl = wml + kWaves * 16;                                      // [head][wave]
    static_assert(kWaves * 16 * D * 4 == kWaves * kBlk * D * 2, "output rows fit one tile set");

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int l16 = lane & 15, grp = lane >> 4;

    // scores are x = q.k; the softmax runs on x * c2 in base 2 (c2 may be negative)
    const float c2 = scale * kLog2e;

    const size_t hoff = ((size_t)b * Hkv + g) * (size_t)L * D;   // this (batch, kv head)'s cache

    // keys attended: all L cached ones, or (append) the n + 1 of sequence b,
    // of which the cache supplies rows 0..n-1
    int Lk = L, ncache = L, nb = -1;
    if constexpr (APPEND) {
        nb = __builtin_amdgcn_readfirstlane(seq_lens[b]);   // uniform: scalar offsets follow
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
        ncache = nb;
        if (s == 0 && wave == 0 && lane < 2 * CPR) {
            // the new row into the cache, 16 bytes per lane (K: lanes 0..CPR-1)
            const int c = 8 * (lane % CPR);
            const uint16_t *src = (lane < CPR ? k_new : v_new) + ((size_t)b * Hkv + g) * D;
            uint16_t *dst = (lane < CPR ? kc : vc) + hoff + (size_t)nb * D;
            *(uint4 *)(dst + c) = *(const uint4 *)(src + c);
        }
    }

    const int C = (Lk + n_splits - 1) / n_splits;
    const int j0 = s * C;                 // may exceed Lk: an empty chunk
    const int j1 = min(Lk, j0 + C);
    // cache rows of this (batch, kv head); rows at or past ncache read as zero
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + hoff, (uint32_t)ncache * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + hoff, (uint32_t)ncache * D * 2);

    // q^T operand: column l16 is head l16 * G / 16 of the group, dims
    // 32ks + 8grp .. +7.  Consumed only by the first MFMA, so its latency
    // overlaps the K/V loads.
    bf16x8 qf[KS];
    {
        const int hq = g * G + ((l16 * G) >> 4);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = as_bf16x8(*(const uint4 *)(q + ((size_t)b * Hq + hq) * D + 32 * ks + 8 * grp));
    }
    // append: the new token's K operand chunks (key n), loaded by every lane
    uint4 kn[KS];
    if constexpr (APPEND) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kn[ks] = *(const uint4 *)(k_new + ((size_t)b * Hkv + g) * D + 32 * ks + 8 * grp);
    }

    // byte offsets of this lane: the K operand rows, the direct V copies (block
    // i of the tile: rows i*RPB + lane / CPR, physical chunk lane % CPR; at
    // D = 128 the swizzle differs between even and odd blocks), the transposed
    // V reads (row 4grp + l16/4, column block 0)
    const int koff = (l16 * D + 8 * grp) * 2;             // K from memory into registers (append)
    int kvoff[4];                                          // K copies (plain; NKV used)
#pragma unroll
    for (int par = 0; par < NKV; ++par) {
        const int r = par * RPB + lane / CPR;
        kvoff[par] = ((lane / CPR) * D + 8 * ((lane % CPR) ^ kswz<D>(r))) * 2;
    }
    // K operand reads: row l16 (+16 for the second half), logical chunk
    // 4ks + grp; the k-step-0 address, XOR 64 ks for the others
    const int kr0 = l16 * D * 2 + 16 * ((grp) ^ kswz<D>(l16));
    int voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int r = par * RPB + lane / CPR;
        voff[par] = ((lane / CPR) * D + 8 * ((lane % CPR) ^ vswz<D>(r))) * 2;
    }
    const int trow = 4 * grp + (l16 >> 2);
    const int tr0 = trow * D * 2 + 16 * (vswz<D>(trow) >> 1) * 2 + 16 * ((l16 & 3) >> 1) + 8 * (l16 & 1);
    uint16_t *const tile = sv + wave * kBlk * D;
    uint16_t *const ktile = sk + (APPEND ? 0 : wave * kBlk * D);

    float m_run = -INFINITY;   // running max of x * c2 for column l16
    float l_run = 0.f;         // this lane's share of the running sum
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    bool first = true;
    for (int kb0 = j0 + kBlk * wave; kb0 < j1; kb0 += kBlk * kWaves) {
        // ---- issue every load of the block: the K tile copies (plain form),
        // the V tile copies, then (append form) K into registers ----
        if constexpr (!APPEND) {
#pragma unroll
            for (int i = 0; i < VBLK; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(ktile + 512 * i), 16, kvoff[i % NKV],
                                                         (kb0 + i * RPB) * D * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VBLK; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(tile + 512 * i), 16,
                                                     voff[D == 128 ? (i & 1) : 0],
                                                     (kb0 + i * RPB) * D * 2, 0, 0);
        sched_fence();   // every copy issued before the first wait for one
        uint4 kraw[2][KS];
        if constexpr (!APPEND) {
            // K operand: lane row l16 (+16), 16 bytes of logical chunk 4ks + grp
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kraw[kb][ks] = *reinterpret_cast<const uint4 *>(
                        reinterpret_cast<const unsigned char *>(ktile) + (kr0 ^ (64 * ks)) + kb * 16 * D * 2);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kraw[kb][ks] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * ks, (kb0 + 16 * kb) * D * 2, 0));
            // key n reads as zero from the cache resource; take the new token's
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bool isn = kb0 + 16 * kb + l16 == nb;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    // element-wise, so the arrays stay in registers
                    const uint4 a = kraw[kb][ks], k = kn[ks];
                    kraw[kb][ks] = make_uint4(isn ? k.x : a.x, isn ? k.y : a.y, isn ? k.z : a.z, isn ? k.w : a.w);
                }
            }
        }
        // ---- scores: S^T (16 keys x 16 columns) for the two 16-key halves ----
        f32x4 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[kb] = mfma16x16x32(as_bf16x8(kraw[kb][ks]), qf[ks], sacc[kb]);
        }
        // lane: column l16, keys kb0 + 16kb + 4grp + r; keys past the chunk get -inf
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
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_fast(sacc[kb][r] - m_new);
                sacc[kb][r] = p;
                rs += p;
            }
        if (first) {
            l_run = rs;
        } else {
            // rescale the running sum and the output rows (columns 4grp + r)
            const float alpha = exp2_fast(m_run - m_new);
            l_run = fmaf(l_run, alpha, rs);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db][r] *= ar;
            }
        }
        m_run = m_new;
        first = false;
        // P operand: column l16, keys 4grp + 0..3 then 16 + 4grp + 0..3
        const bf16x8 pa = as_bf16x8(make_uint4(pack_bf16x2(sacc[0][0], sacc[0][1]), pack_bf16x2(sacc[0][2], sacc[0][3]),
                                               pack_bf16x2(sacc[1][0], sacc[1][1]), pack_bf16x2(sacc[1][2], sacc[1][3])));
        if constexpr (APPEND) {
            // key n's row of the tile (zero from the copy) takes the new value
            // once the copies have landed
            if (nb >= kb0 && nb < kb0 + kBlk) {
                wait_vmcnt<0>();
                const int rr = nb - kb0;
                if (lane < CPR)
                    *(uint4 *)(tile + rr * D + 8 * (lane ^ vswz<D>(rr))) =
                        *(const uint4 *)(v_new + ((size_t)b * Hkv + g) * D + 8 * lane);
            }
        }
        // ---- O += P V, V read key-contiguous from the tile ----
        // source lane l16 of group grp addresses key (4grp + l16/4) (+16 for the
        // upper half), columns 16db + 4(l16%4) .. +3
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t *p0 = reinterpret_cast<const uint16_t *>(
                reinterpret_cast<const unsigned char *>(tile) + (tr0 ^ (32 * db)));
            const uint2 lo = lds_read_tr16(p0);
            const uint2 hi = lds_read_tr16(p0 + 16 * D);
            const bf16x8 vb = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            oacc[db] = mfma16x16x32(pa, vb, oacc[db]);
        }
        // the next block's copies overwrite the tile: its reads must be done
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    }

    // ---- per-wave state -> LDS, then combine the 8 waves ----
    l_run = pair32_sum(pair16_sum(l_run));
    {
        // [head][wave], from the head's first column
        const int h = (l16 * G) >> 4;
        if (grp == 0 && l16 * G < 16 * h + G) {
            wm[h * kWaves + wave] = m_run;
            wl[h * kWaves + wave] = l_run;
        }
    }
    // accumulator row 4grp + r is column n = 4grp + r, i.e. head n G / 16; the
    // first column of each head writes its row: lane l16 holds output column
    // 16db + l16, stored at column XOR 16 (h % 4) so that the rows of four
    // heads written at once fall in distinct banks.  Wave w's rows [16][D] f32
    // occupy exactly its own K tile (append: V tile), which only it has read,
    // and its reads precede these writes in its LDS queue: no barrier.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = 4 * grp + r, h = (n * G) >> 4;
        if (n * G < 16 * h + G) {                       // n == ceil(16 h / G)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                wo[(wave * 16 + h) * D + ((16 * db + l16) ^ (16 * (h & 3)))] = oacc[db][r];
        }
    }
    __syncthreads();
    for (int t = tid; t < G * D; t += 512) {
        const int hh = t / D, c = t % D;
        // every read issued at once: the 8 waves' (max, sum) of head hh and
        // their output at column c
        static_assert(kWaves == 8, "two 16-byte reads per head");
        float mw[kWaves], lw[kWaves], ow[kWaves];
        *reinterpret_cast<float4 *>(mw) = *reinterpret_cast<const float4 *>(wm + hh * kWaves);
        *reinterpret_cast<float4 *>(mw + 4) = *reinterpret_cast<const float4 *>(wm + hh * kWaves + 4);
        *reinterpret_cast<float4 *>(lw) = *reinterpret_cast<const float4 *>(wl + hh * kWaves);
        *reinterpret_cast<float4 *>(lw + 4) = *reinterpret_cast<const float4 *>(wl + hh * kWaves + 4);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ow[w] = wo[(w * 16 + hh) * D + (c ^ (16 * (hh & 3)))];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
        // a wave that saw no key holds (-inf, 0, 0), whose weight 2^-inf is 0;
        // a chunk with no key at all (M = -inf) gives the identity (0, -inf)
        float lt = 0.f, at = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = exp2_fast(mw[w] - M);
            lt = fmaf(lw[w], e, lt);
            at = fmaf(ow[w], e, at);
        }
        const bool empty = M == -INFINITY;
        const size_t ob = ((size_t)b * Hq + g * G + hh) * n_splits + s;
        // hardware reciprocal and log2 (about 1 ulp): the partials' bf16-input
        // tolerances are orders of magnitude wider
        part_o[ob * D + c] = empty ? 0.f : at * __builtin_amdgcn_rcpf(lt);
        if (c == 0) part_lse[ob] = empty ? -INFINITY : (M + __builtin_amdgcn_logf(lt)) * kLn2;
    }
}

}  // namespace

// The kernel addresses one (batch, kv head)'s cache through a buffer resource
// with 32-bit byte offsets: L d 2 bytes (plus a tile of slack) must stay below
// 2^31.
bool decode_mfma_supported(int dt, int d, int G, int L)
{
    return dt == kBF16 && (d == 64 || d == 128) && G <= 16 && (long)L * d * 2 + 65536 < (1L << 31);
}

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
