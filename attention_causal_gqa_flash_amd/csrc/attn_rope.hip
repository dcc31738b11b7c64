// attn_rope.hip -- rotary positions on the rows of q, k (and, transposed, on
// the gradients with respect to them).
//
// The pages list rotary position embeddings beside grouped-query attention
// among the derived ops ("tang -- differentiable computing in Rust", the "A
// transformer" panel; RustingBrain docs, "What is in the box") without a
// formula.  The rotation used (the usual one, on paired halves of the head
// dimension): for a row at position p and pair i in [0, d/2), theta_i =
// base^(-2i/d), a = p theta_i,
//     y_i = x_i cos a - x_{i+d/2} sin a,   y_{i+d/2} = x_i sin a + x_{i+d/2} cos a,
// and the transposed rotation (angle -a) for `inverse`.
//
// One elementwise pass, not a prologue inside the attention kernels: the
// dK/dV kernel streams Q tiles into LDS by direct global->LDS copies, which
// bypass the registers, so the backward needs the rotated Q in memory anyway;
// once written for it, the forward reads the same bytes as it would read the
// unrotated Q.  K is rotated once per key/value head here instead of once per
// query tile that loads it.
#include "attn_device.h"
#include "attn_launch.h"

#include <math.h>

#include <algorithm>

namespace attn {
namespace {

// Consecutive pairs per thread: 16 bytes of each half row (8 bf16, 4 f32),
// or the whole half row when it is shorter.
template <typename T>
__host__ __device__ constexpr int pairs_per_thread() { return sizeof(T) == 2 ? 8 : 4; }

__device__ __forceinline__ void load_pairs(const bf16_t *p, float (&v)[8])
{
    const uint4 u = *(const uint4 *)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo(w[j]); v[2 * j + 1] = bf16hi(w[j]); }
}
__device__ __forceinline__ void load_pairs(const float *p, float (&v)[4])
{
    const float4 u = *(const float4 *)p;
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}
__device__ __forceinline__ void store_pairs(bf16_t *p, const float (&v)[8])
{
    *(uint4 *)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                             pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ void store_pairs(float *p, const float (&v)[4])
{
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
}

// Rows of one tensor: row r of `rows` rows of d elements sits at position
// pos0 + r % N.
template <typename T>
struct RopeSeg {
    const T *x;
    T *y;
    long rows;
    int N;
    long pos0;
};

// One launch over one or two tensors (the second may have no rows).  A thread
// owns pairs i0 .. i0+KP-1 of its rows (16-byte accesses): the grid stride and
// the first tensor's thread count are multiples of the threads per row, so i0
// is fixed and its frequencies are computed once, in double.  The angle is
// reduced to whole turns in double before the f32 sine and cosine, so
// positions in the millions keep f32 accuracy: for bf16 rows on the hardware
// sine and cosine (about 1e-6, far below bf16's resolution), for f32 rows on
// the library's.  x and y may be the same buffer.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeSeg<T> s0, RopeSeg<T> s1, int d, double log2_base,
                                                   int inverse)
{
    constexpr int KP = pairs_per_thread<T>();
    const int half = d / 2, tpr = half / KP;
    const long t0 = (long)blockIdx.x * 256 + threadIdx.x;
    const long stride = (long)gridDim.x * 256;
    const long n0 = s0.rows * tpr, n = n0 + s1.rows * tpr;
    const int i0 = (int)(t0 % tpr) * KP;
    double th[KP];
#pragma unroll
    for (int e = 0; e < KP; ++e) th[e] = rope_theta(i0 + e, d, log2_base) * 0.15915494309189535;   // turns
    for (long t = t0; t < n; t += stride) {
        const bool first = t < n0;
        const RopeSeg<T> &sg = first ? s0 : s1;
        const long r = (first ? t : t - n0) / tpr;
        const double p = (double)(sg.pos0 + r % sg.N);
        float x0[KP], x1[KP], y0[KP], y1[KP];
        load_pairs(sg.x + r * d + i0, x0);
        load_pairs(sg.x + r * d + half + i0, x1);
#pragma unroll
        for (int e = 0; e < KP; ++e) {
            float s, c;
            if constexpr (sizeof(T) == 2) rope_sincos_turns(p * th[e], s, c);
            else rope_sincos(p * th[e] * 6.283185307179586, s, c);
            if (inverse) s = -s;
            y0[e] = x0[e] * c - x1[e] * s;
            y1[e] = x0[e] * s + x1[e] * c;
        }
        store_pairs(sg.y + r * d + i0, y0);
        store_pairs(sg.y + r * d + half + i0, y1);
    }
}

template <typename T>
hipError_t rope_launch(const RopeSeg<T> &s0, const RopeSeg<T> &s1, int d, double base, int inverse,
                       hipStream_t st)
{
    const long threads = (s0.rows + s1.rows) * (d / 2 / pairs_per_thread<T>());
    const unsigned blocks = (unsigned)std::min<long>((threads + 255) / 256, 2048L);
    hipLaunchKernelGGL(rope_kernel<T>, dim3(blocks), dim3(256), 0, st, s0, s1, d, log2(base), inverse);
    return hipGetLastError();
}

}  // namespace

hipError_t rope(int dt, long rows, int N, int d, long pos0, double base, int inverse, const void *x,
                void *y, hipStream_t st)
{
    return rope2(dt, rows, N, pos0, x, y, 0, 1, 0, nullptr, nullptr, d, base, inverse, st);
}

hipError_t rope2(int dt, long rows0, int N0, long pos00, const void *x0, void *y0, long rows1, int N1,
                 long pos01, const void *x1, void *y1, int d, double base, int inverse, hipStream_t st)
{
    if (dt == kBF16)
        return rope_launch<bf16_t>({(const bf16_t *)x0, (bf16_t *)y0, rows0, N0, pos00},
                                   {(const bf16_t *)x1, (bf16_t *)y1, rows1, N1, pos01}, d, base,
                                   inverse, st);
    return rope_launch<float>({(const float *)x0, (float *)y0, rows0, N0, pos00},
                              {(const float *)x1, (float *)y1, rows1, N1, pos01}, d, base, inverse, st);
}

}  // namespace attn
