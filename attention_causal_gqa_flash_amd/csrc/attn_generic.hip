// attn_generic.hip -- vector-ALU kernels for every supported (dtype, head dim):
// the f32 path, small head dims, the backward preprocess, split-KV decode and
// the log-sum-exp merge.
//
// The forward keeps, per query row, the three running values of the streaming
// softmax -- running max m, running sum l, running weighted sum acc -- while the
// keys stream past once ("tang -- differentiable computing in Rust", "How tang
// works" part 3, equation (6)).  Arithmetic is f32 with accurate expf/logf.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

#include <algorithm>

namespace attn {

// ---------------------------------------------------------------------------
// Forward, one thread per query row; O of type OT (f32, or bf16 rounded to
// nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void put(float *p, float x) { *p = x; }
__device__ __forceinline__ void put(bf16_t *p, float x)
{
    p->bits = __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename T, int D, typename OT>
__global__ __launch_bounds__(64) void fwd_rowwise_kernel(const T *__restrict__ q,
                                                         const T *__restrict__ k,
                                                         const T *__restrict__ v,
                                                         OT *__restrict__ o,
                                                         float *__restrict__ lse, int Hq, int Hkv,
                                                         int Nq, int Nk, float scale, int causal,
                                                         Layouts L)
{
    // Nq queries against Nk >= Nq keys; query i sits at key position i + off
    const int i = blockIdx.x * 64 + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int off = Nk - Nq;
    const T *qh = q + b * L.q.b + h * L.q.h;
    const T *kg = k + b * L.k.b + g * L.k.h;
    const T *vg = v + b * L.v.b + g * L.v.h;
    const int row = i < Nq ? i : Nq - 1;

    float qr[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = to_f32(qh[(size_t)row * L.q.n + c]);
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int jend = causal ? row + off + 1 : Nk;
    // keys are read in lock-step across the wave (broadcast loads)
    const int wave_end = causal ? min(Nk, (int)(blockIdx.x * 64 + 64) + off) : Nk;
    for (int j = 0; j < wave_end; ++j) {
        if (j >= jend) continue;
        const T *kj = kg + (size_t)j * L.k.n;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s = fmaf(qr[c], to_f32(kj[c]), s);
        s *= scale;
        if (s > m) {                    // new running max: rescale the state
            const float a = expf(m - s);
            l *= a;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] *= a;
            m = s;
        }
        const float p = expf(s - m);
        l += p;
        const T *vj = vg + (size_t)j * L.v.n;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(p, to_f32(vj[c]), acc[c]);
    }
    if (i < Nq) {
        OT *oh = o + b * L.o.b + h * L.o.h + (size_t)i * L.o.n;
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < D; ++c) put(oh + c, acc[c] * inv);
        lse[((size_t)b * Hq + h) * Nq + i] = m + logf(l);
    }
}

// ---------------------------------------------------------------------------
// Backward preprocess: D_i = dout_i . o_i.  D/8 lanes per row, 8 elements each.
// ---------------------------------------------------------------------------
// Zero-fill n floats at a and at b (n a multiple of 4, 16-byte aligned).
__device__ __forceinline__ void zero2_grid_stride(float *a, float *b, long n)
{
    const long stride = (long)gridDim.x * blockDim.x;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n / 4; i += stride) {
        ((float4 *)a)[i] = z;
        ((float4 *)b)[i] = z;
    }
}

__global__ __launch_bounds__(256) void zero_fill2_kernel(float *__restrict__ a, float *__restrict__ b,
                                                         long n)
{
    zero2_grid_stride(a, b, n);
}

// Three f32 arrays rounded to bf16 (nearest even), eight elements a thread
// per step over their concatenation: array i holds 8 n8_i elements.
__global__ __launch_bounds__(256) void to_bf16_3_kernel(const float *__restrict__ s0, uint16_t *__restrict__ d0,
                                                        long n0, const float *__restrict__ s1,
                                                        uint16_t *__restrict__ d1, long n1,
                                                        const float *__restrict__ s2,
                                                        uint16_t *__restrict__ d2, long n2)
{
    const long total = n0 + n1 + n2;
    for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const bool a = i < n0, b = !a && i < n0 + n1;
        const float *src = a ? s0 : b ? s1 : s2;
        uint16_t *dst = a ? d0 : b ? d1 : d2;
        const long j = a ? i : b ? i - n0 : i - n0 - n1;
        const float4 x = ((const float4 *)src)[2 * j], y = ((const float4 *)src)[2 * j + 1];
        ((uint4 *)dst)[j] = make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y),
                                       pack_bf16x2(y.z, y.w));
    }
}

// Row r of the B*Hq*N rows is query row r % N of head (r / N) % Hq of batch
// r / (Hq N); dout and o have the strides of L.dout and L.o.
template <typename T, int D, typename OT>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T *__restrict__ dout,
                                                      const OT *__restrict__ o,
                                                      float *__restrict__ Dws, long rows,
                                                      float *__restrict__ zero,
                                                      float *__restrict__ zero2, long zero_len,
                                                      const float *__restrict__ dlse, int Hq, int N,
                                                      Layouts L)
{
    if (zero != nullptr) zero2_grid_stride(zero, zero2, zero_len);
    constexpr int LPR = D / 8;              // lanes per row
    constexpr int RPB = 256 / LPR;          // rows per block
    const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float s = 0.f;
    if (row < rows) {
        const long bh = row / N, bb = bh / Hq, hh = bh % Hq, ii = row % N;
        const size_t base = bb * L.o.b + hh * L.o.h + ii * L.o.n + part * 8;
        const size_t dbase = bb * L.dout.b + hh * L.dout.h + ii * L.dout.n + part * 8;
        float4 o0, o1;
        if constexpr (sizeof(OT) == 2) {
            const uint4 u = *(const uint4 *)((const uint16_t *)o + base);
            o0 = make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
            o1 = make_float4(bf16lo(u.z), bf16hi(u.z), bf16lo(u.w), bf16hi(u.w));
        } else {
            o0 = *(const float4 *)((const float *)o + base);
            o1 = *(const float4 *)((const float *)o + base + 4);
        }
        float dv[8];
        if constexpr (sizeof(T) == 2) {
            const uint4 u = *(const uint4 *)((const uint16_t *)dout + dbase);
            dv[0] = bf16lo(u.x); dv[1] = bf16hi(u.x); dv[2] = bf16lo(u.y); dv[3] = bf16hi(u.y);
            dv[4] = bf16lo(u.z); dv[5] = bf16hi(u.z); dv[6] = bf16lo(u.w); dv[7] = bf16hi(u.w);
        } else {
            const float4 a = *(const float4 *)((const float *)dout + dbase);
            const float4 c = *(const float4 *)((const float *)dout + dbase + 4);
            dv[0] = a.x; dv[1] = a.y; dv[2] = a.z; dv[3] = a.w;
            dv[4] = c.x; dv[5] = c.y; dv[6] = c.z; dv[7] = c.w;
        }
        s = dv[0] * o0.x + dv[1] * o0.y + dv[2] * o0.z + dv[3] * o0.w +
            dv[4] * o1.x + dv[5] * o1.y + dv[6] * o1.z + dv[7] * o1.w;
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    // an upstream gradient of lse enters as D - dlse (dS = P (dP - (D - dlse)))
    if (row < rows && part == 0) Dws[row] = dlse ? s - dlse[row] : s;
}

// ---------------------------------------------------------------------------
// Backward, dq: one thread per query row.  P is recomputed from lse.  Nq
// query rows against Nk >= Nq keys, query row i at key position i + Nk - Nq.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dq_rowwise_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ Dws,
    float *__restrict__ dq, int Hq, int Hkv, int Nq, int Nk, float scale, int causal, Layouts L)
{
    const int i = blockIdx.x * 64 + threadIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / (Hq / Hkv);
    const int off = Nk - Nq;
    const size_t qrow0 = ((size_t)b * Hq + h) * Nq;     // rows of lse and D
    const T *kg = k + b * L.k.b + g * L.k.h;
    const T *vg = v + b * L.v.b + g * L.v.h;
    const int row = i < Nq ? i : Nq - 1;
    const T *qrw = q + b * L.q.b + h * L.q.h + (size_t)row * L.q.n;
    const T *drw = dout + b * L.dout.b + h * L.dout.h + (size_t)row * L.dout.n;

    float qr[D], dor[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = to_f32(qrw[c]);
        dor[c] = to_f32(drw[c]);
        acc[c] = 0.f;
    }
    const float Li = lse[qrow0 + row], Di = Dws[qrow0 + row];
    const int jend = causal ? min(row + 1 + off, Nk) : Nk;
    const int wave_end = causal ? min(Nk, (int)(blockIdx.x * 64 + 64) + off) : Nk;
    for (int j = 0; j < wave_end; ++j) {
        if (j >= jend) continue;
        const T *kj = kg + (size_t)j * L.k.n;
        const T *vj = vg + (size_t)j * L.v.n;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            s = fmaf(qr[c], to_f32(kj[c]), s);
            dp = fmaf(dor[c], to_f32(vj[c]), dp);
        }
        const float p = expf(s * scale - Li);
        const float ds = p * (dp - Di);
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, to_f32(kj[c]), acc[c]);
    }
    if (i < Nq) {
#pragma unroll
        for (int c = 0; c < D; ++c) dq[b * L.dq.b + h * L.dq.h + (size_t)i * L.dq.n + c] = acc[c] * scale;
    }
}

// ---------------------------------------------------------------------------
// Backward, dk and dv: one thread per key row of a key/value head; the loop
// runs over the query heads of the group and over the queries that see the key
// (under the causal mask, query rows i >= j - (Nk - Nq)).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dkdv_colwise_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ Dws,
    float *__restrict__ dk, float *__restrict__ dv, int Hq, int Hkv, int Nq, int Nk, float scale,
    int causal, Layouts L)
{
    const int j = blockIdx.x * 64 + threadIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int off = Nk - Nq;
    const int row = j < Nk ? j : Nk - 1;
    const T *krw = k + b * L.k.b + g * L.k.h + (size_t)row * L.k.n;
    const T *vrw = v + b * L.v.b + g * L.v.h + (size_t)row * L.v.n;

    float kr[D], vr[D], dka[D], dva[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        kr[c] = to_f32(krw[c]);
        vr[c] = to_f32(vrw[c]);
        dka[c] = 0.f;
        dva[c] = 0.f;
    }
    const int istart = causal ? max(row - off, 0) : 0;
    const int wave_start = causal ? max((int)(blockIdx.x * 64) - off, 0) : 0;
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        const size_t qrow0 = ((size_t)b * Hq + h) * Nq;   // rows of lse and D
        for (int i = wave_start; i < Nq; ++i) {
            if (i < istart) continue;
            const T *qi = q + b * L.q.b + h * L.q.h + (size_t)i * L.q.n;
            const T *di = dout + b * L.dout.b + h * L.dout.h + (size_t)i * L.dout.n;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                s = fmaf(to_f32(qi[c]), kr[c], s);
                dp = fmaf(to_f32(di[c]), vr[c], dp);
            }
            const float p = expf(s * scale - lse[qrow0 + i]);
            const float ds = p * (dp - Dws[qrow0 + i]);
#pragma unroll
            for (int c = 0; c < D; ++c) {
                dva[c] = fmaf(p, to_f32(di[c]), dva[c]);
                dka[c] = fmaf(ds, to_f32(qi[c]), dka[c]);
            }
        }
    }
    if (j < Nk) {
#pragma unroll
        for (int c = 0; c < D; ++c) {
            dk[b * L.dk.b + g * L.dk.h + (size_t)j * L.dk.n + c] = dka[c] * scale;
            dv[b * L.dv.b + g * L.dv.h + (size_t)j * L.dv.n + c] = dva[c];
        }
    }
}

// ---------------------------------------------------------------------------
// Split-KV decode.  One workgroup per (split, key/value head, batch) handles
// all G query heads of the group, so each cached key and value is read from
// memory once.  Four waves share the chunk; within a wave, scores are computed
// one key per lane and the value sum one column pair per lane; the waves'
// running states are then combined with the associative softmax merge.
// ---------------------------------------------------------------------------
template <typename T, int D, int GM>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    float *__restrict__ part_o, float *__restrict__ part_lse, int Hq, int Hkv, int L,
    float scale, int n_splits)
{
    constexpr int CPL = D >= 64 ? D / 64 : 1;   // value columns per lane
    constexpr int ACT = D / CPL;                 // lanes that own columns
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = Hq / Hkv;
    const int w = threadIdx.x / 64, lane = threadIdx.x % 64;

    __shared__ float qs[GM][D];
    __shared__ float ps[4][64][GM];
    __shared__ float wm[4][GM], wl[4][GM];
    __shared__ float wacc[4][GM][D];

    for (int t = threadIdx.x; t < G * D; t += 256) {
        const int hh = t / D, c = t % D;
        qs[hh][c] = to_f32(q[((size_t)b * Hq + g * G + hh) * D + c]) * scale;
    }
    __syncthreads();

    const long C = ((long)L + n_splits - 1) / n_splits;
    const long j0 = (long)s * C;
    const long j1 = min((long)L, j0 + C);
    const T *kg = kc + ((size_t)b * Hkv + g) * (size_t)L * D;
    const T *vg = vc + ((size_t)b * Hkv + g) * (size_t)L * D;

    // G <= GM; loops run to the compile-time GM so the state stays in registers
    float m[GM], l[GM], acc[GM][CPL];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
        for (int c = 0; c < CPL; ++c) acc[hh][c] = 0.f;
    }

    // wave w takes rounds of 64 keys: [j0 + 64*(4r + w), +64)
    for (long base = j0 + 64 * w; base < j1; base += 256) {
        const long j = base + lane;
        const bool valid = j < j1;
        float sc[GM];
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) sc[hh] = 0.f;
        if (valid) {
            const T *kj = kg + (size_t)j * D;
            for (int c = 0; c < D; ++c) {
                const float kv = to_f32(kj[c]);
#pragma unroll
                for (int hh = 0; hh < GM; ++hh)
                    if (hh < G) sc[hh] = fmaf(qs[hh][c], kv, sc[hh]);
            }
        }
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) {
            if (hh >= G) continue;
            const float x = valid ? sc[hh] : -INFINITY;
            const float mx = wave_max(x);            // lane 0 is always valid: finite
            const float mnew = fmaxf(m[hh], mx);
            const float a = m[hh] == -INFINITY ? 0.f : expf(m[hh] - mnew);
            const float p = valid ? expf(x - mnew) : 0.f;
            l[hh] = l[hh] * a + wave_sum(p);
            for (int c = 0; c < CPL; ++c) acc[hh][c] *= a;
            m[hh] = mnew;
            ps[w][lane][hh] = p;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        const long nk = min((long)64, j1 - base);
        if (lane < ACT) {
            for (long t = 0; t < nk; ++t) {
                const T *vj = vg + (size_t)(base + t) * D + lane * CPL;
                float vv[CPL];
                for (int c = 0; c < CPL; ++c) vv[c] = to_f32(vj[c]);
#pragma unroll
                for (int hh = 0; hh < GM; ++hh) {
                    if (hh >= G) continue;
                    const float p = ps[w][t][hh];
                    for (int c = 0; c < CPL; ++c) acc[hh][c] = fmaf(p, vv[c], acc[hh][c]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // combine the four waves
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) { wm[w][hh] = m[hh]; wl[w][hh] = l[hh]; }
    }
    if (lane < ACT) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh)
            for (int c = 0; c < CPL; ++c) wacc[w][hh][lane * CPL + c] = acc[hh][c];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * D; t += 256) {
        const int hh = t / D, c = t % D;
        float M = -INFINITY;
        for (int x = 0; x < 4; ++x) M = fmaxf(M, wm[x][hh]);
        const size_t ob = ((size_t)b * Hq + g * G + hh) * n_splits + s;
        if (M == -INFINITY) {                    // empty chunk: the identity
            part_o[ob * D + c] = 0.f;
            if (c == 0) part_lse[ob] = -INFINITY;
            continue;
        }
        float lt = 0.f, at = 0.f;
        for (int x = 0; x < 4; ++x) {
            if (wm[x][hh] == -INFINITY) continue;
            const float e = expf(wm[x][hh] - M);
            lt = fmaf(wl[x][hh], e, lt);
            at = fmaf(wacc[x][hh][c], e, at);
        }
        part_o[ob * D + c] = at / lt;
        if (c == 0) part_lse[ob] = M + logf(lt);
    }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials: one workgroup per (query head,
// batch).  The split weights are computed once, in parallel, and staged in LDS;
// each thread then sums one output column with its loads unrolled.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block128_reduce(float v, float *red, bool is_max)
{
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
}

__global__ __launch_bounds__(128) void lse_merge_kernel(const float *__restrict__ part_o,
                                                        const float *__restrict__ part_lse,
                                                        float *__restrict__ o,
                                                        float *__restrict__ lse, int Hq,
                                                        int n_splits, int d)
{
    __shared__ float sw[128];
    __shared__ float red[2];
    const int tid = threadIdx.x;
    const size_t row = (size_t)blockIdx.y * Hq + blockIdx.x;
    const float *pl = part_lse + row * n_splits;
    const float *po = part_o + row * (size_t)n_splits * d;

    float M = -INFINITY;
    for (int s = tid; s < n_splits; s += 128) M = fmaxf(M, pl[s]);
    M = block128_reduce(M, red, true);

    float W = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += 128) {
        const int s = s0 + tid;
        float w = 0.f;
        if (s < n_splits && M != -INFINITY) {
            const float ls = pl[s];
            if (ls != -INFINITY) w = expf(ls - M);
        }
        W += w;
        __syncthreads();
        sw[tid] = w;
        __syncthreads();
        if (tid < d) {
            const int n = min(128, n_splits - s0);
            const float *pc = po + (size_t)s0 * d + tid;
#pragma unroll 8
            for (int i = 0; i < n; ++i) acc = fmaf(sw[i], pc[(size_t)i * d], acc);
        }
    }
    W = block128_reduce(W, red, false);
    if (tid < d) o[row * d + tid] = M == -INFINITY ? 0.f : acc / W;
    if (tid == 0) lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
}

// The same merge for at most NS <= 64 splits (the usual case): every lane
// loads its dim of all the partials at once, next to the splits' lse values
// (the same addresses in every lane), so the kernel waits for memory once;
// lane s of each wave computes split s's weight and the others read it from
// that lane, with no block reductions.  Indices past the last split or dim
// are clamped (the loads stay branch-free) and those splits get weight 0.
template <int NS>
__global__ __launch_bounds__(128) void lse_merge_small_kernel(const float *__restrict__ part_o,
                                                              const float *__restrict__ part_lse,
                                                              float *__restrict__ o,
                                                              float *__restrict__ lse, int Hq,
                                                              int n_splits, int d)
{
    static_assert(NS <= 64, "one split per lane");
    const int tid = threadIdx.x, lane = tid & 63, dc = min(tid, d - 1);
    const size_t row = (size_t)blockIdx.y * Hq + blockIdx.x;
    const float *pl = part_lse + row * n_splits;
    const float *po = part_o + row * (size_t)n_splits * d;
    float ls[NS], pv[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int sc = min(s, n_splits - 1);
        ls[s] = pl[sc];
        pv[s] = po[(size_t)sc * d + dc];
    }
    const float own = pl[min(lane, n_splits - 1)];    // split `lane`'s lse
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) M = fmaxf(M, ls[s]);
    // weight of split `lane`; all zero when every chunk is empty (M = -inf)
    const float w = (lane >= n_splits || M == -INFINITY || own == -INFINITY) ? 0.f : expf(own - M);
    float W = 0.f, acc = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
        W += ws;
        acc = fmaf(ws, pv[s], acc);
    }
    if (tid < d) o[row * d + tid] = M == -INFINITY ? 0.f : acc / W;
    if (tid == 0) lse[row] = M == -INFINITY ? -INFINITY : M + logf(W);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
#define ATTN_DISPATCH_D(d, ...)                              \
    switch (d) {                                             \
    case 16: { constexpr int D = 16; __VA_ARGS__; break; }   \
    case 32: { constexpr int D = 32; __VA_ARGS__; break; }   \
    case 64: { constexpr int D = 64; __VA_ARGS__; break; }   \
    case 128: { constexpr int D = 128; __VA_ARGS__; break; } \
    default: return hipErrorInvalidValue;                    \
    }

#define ATTN_DISPATCH_T(dt, ...)                                   \
    if (dt == kBF16) { typedef bf16_t T; __VA_ARGS__; }            \
    else { typedef float T; __VA_ARGS__; }

hipError_t fwd_rowwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                       float scale, const void *q, const void *k, const void *v, void *o,
                       float *lse, hipStream_t st, bool o_bf16, const Layouts *L)
{
    const Layouts lay = L ? *L : contiguous_layouts(Hq, Hkv, Nq, Nk, d);
    dim3 grid((Nq + 63) / 64, Hq, B);
    if (o_bf16) {
        ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL((fwd_rowwise_kernel<T, D, bf16_t>), grid,
                                                                  dim3(64), 0, st, (const T *)q,
                                                                  (const T *)k, (const T *)v,
                                                                  (bf16_t *)o, lse, Hq, Hkv, Nq, Nk,
                                                                  scale, causal, lay)));
    } else {
        ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL((fwd_rowwise_kernel<T, D, float>), grid,
                                                                  dim3(64), 0, st, (const T *)q,
                                                                  (const T *)k, (const T *)v,
                                                                  (float *)o, lse, Hq, Hkv, Nq, Nk,
                                                                  scale, causal, lay)));
    }
    return hipGetLastError();
}

hipError_t bwd_preprocess(int dt, int B, int Hq, int N, int d, const void *dout, const void *o,
                          float *Dws, float *zero, float *zero2, long zero_len, const float *dlse,
                          hipStream_t st, bool o_bf16, const Layouts *L)
{
    const Layouts lay = L ? *L : contiguous_layouts(Hq, Hq, N, N, d);
    const long rows = (long)B * Hq * N;
    const int rpb = 256 / (d / 8);
    dim3 grid((unsigned)((rows + rpb - 1) / rpb));
    if (o_bf16) {
        ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL((bwd_pre_kernel<T, D, bf16_t>), grid,
                                                                  dim3(256), 0, st, (const T *)dout,
                                                                  (const bf16_t *)o, Dws, rows, zero,
                                                                  zero2, zero_len, dlse, Hq, N, lay)));
    } else {
        ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL((bwd_pre_kernel<T, D, float>), grid,
                                                                  dim3(256), 0, st, (const T *)dout,
                                                                  (const float *)o, Dws, rows, zero,
                                                                  zero2, zero_len, dlse, Hq, N, lay)));
    }
    return hipGetLastError();
}

hipError_t to_bf16_3(const float *s0, uint16_t *d0, long n0, const float *s1, uint16_t *d1, long n1,
                     const float *s2, uint16_t *d2, long n2, hipStream_t st)
{
    if (n0 % 8 || n1 % 8 || n2 % 8) return hipErrorInvalidValue;
    const long total = (n0 + n1 + n2) / 8;
    const long blocks = std::min<long>((total + 255) / 256, 8192L);
    hipLaunchKernelGGL(to_bf16_3_kernel, dim3((unsigned)std::max<long>(blocks, 1)), dim3(256), 0, st, s0, d0,
                       n0 / 8, s1, d1, n1 / 8, s2, d2, n2 / 8);
    return hipGetLastError();
}

hipError_t zero_fill2(float *a, float *b, long n, hipStream_t st)
{
    const long blocks = std::min<long>((n / 4 + 255) / 256, 4096L);
    hipLaunchKernelGGL(zero_fill2_kernel, dim3((unsigned)std::max<long>(blocks, 1)), dim3(256), 0,
                       st, a, b, n);
    return hipGetLastError();
}

hipError_t bwd_dq_rowwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, const void *q, const void *k, const void *v,
                          const float *lse, const void *dout, const float *Dws, float *dq,
                          hipStream_t st, const Layouts *L)
{
    const Layouts lay = L ? *L : contiguous_layouts(Hq, Hkv, Nq, Nk, d);
    dim3 grid((Nq + 63) / 64, Hq, B);
    ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL(
                                               (bwd_dq_rowwise_kernel<T, D>), grid, dim3(64), 0,
                                               st, (const T *)q, (const T *)k, (const T *)v, lse,
                                               (const T *)dout, Dws, dq, Hq, Hkv, Nq, Nk,
                                               scale, causal, lay)));
    return hipGetLastError();
}

hipError_t bwd_dkdv_colwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            float scale, const void *q, const void *k, const void *v,
                            const float *lse, const void *dout, const float *Dws, float *dk,
                            float *dv, hipStream_t st, const Layouts *L)
{
    const Layouts lay = L ? *L : contiguous_layouts(Hq, Hkv, Nq, Nk, d);
    dim3 grid((Nk + 63) / 64, Hkv, B);
    ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL(
                                               (bwd_dkdv_colwise_kernel<T, D>), grid, dim3(64), 0,
                                               st, (const T *)q, (const T *)k, (const T *)v, lse,
                                               (const T *)dout, Dws, dk, dv, Hq, Hkv, Nq, Nk,
                                               scale, causal, lay)));
    return hipGetLastError();
}

hipError_t decode_split(int dt, int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                        const void *q, const void *kc, const void *vc, float *part_o,
                        float *part_lse, hipStream_t st)
{
    dim3 grid(n_splits, Hkv, B);
    const int G = Hq / Hkv;
#define ATTN_DEC_LAUNCH(GMV)                                                                     \
    ATTN_DISPATCH_T(dt, ATTN_DISPATCH_D(d, hipLaunchKernelGGL(                                  \
                                               (decode_split_kernel<T, D, GMV>), grid,           \
                                               dim3(256), 0, st, (const T *)q, (const T *)kc,   \
                                               (const T *)vc, part_o, part_lse, Hq, Hkv, L,     \
                                               scale, n_splits)))
    if (G <= 4) {
        ATTN_DEC_LAUNCH(4);
    } else if (G <= 8) {
        ATTN_DEC_LAUNCH(8);
    } else {
        ATTN_DEC_LAUNCH(16);
    }
#undef ATTN_DEC_LAUNCH
    return hipGetLastError();
}

hipError_t lse_merge(int B, int Hq, int n_splits, int d, const float *part_o,
                     const float *part_lse, float *o, float *lse, hipStream_t st)
{
    if (n_splits <= 16)
        hipLaunchKernelGGL(lse_merge_small_kernel<16>, dim3(Hq, B), dim3(128), 0, st, part_o, part_lse,
                           o, lse, Hq, n_splits, d);
    else if (n_splits <= 32)
        hipLaunchKernelGGL(lse_merge_small_kernel<32>, dim3(Hq, B), dim3(128), 0, st, part_o, part_lse,
                           o, lse, Hq, n_splits, d);
    else
        hipLaunchKernelGGL(lse_merge_kernel, dim3(Hq, B), dim3(128), 0, st, part_o, part_lse, o, lse,
                           Hq, n_splits, d);
    return hipGetLastError();
}

}  // namespace attn
