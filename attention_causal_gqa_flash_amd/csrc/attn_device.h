// attn_device.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 is stored as a 16-bit word; widening to f32 is exact.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x.bits) << 16); }

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two f32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// D(32x32, f32) += A(32x16) * B(16x32), bf16 operands.
// Lane l supplies A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32], e = 0..7;
// accumulator register r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, result lane i, element k is
// element (i % 4) of the 4-element chunk addressed by lane 4k + i/4 of the group.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p)
{
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// Operand of v_mfma_f32_32x32x16_bf16 whose contraction runs down the rows of a
// row-major bf16 LDS tile: lane l gets column cbase + l%32 at rows
// kbase + 4*(l/32) + {0,1,2,3} (elements 0..3) and kbase + 8 + 4*(l/32) + {0..3}
// (elements 4..7).  That is exactly the row order in which the 32x32
// accumulator of the previous MFMA holds its rows (rows 8(r/4) + 4*(l/32) + r%4),
// so an accumulator repacked to bf16 pairs with this operand.  Two transposed
// LDS reads: lane i of each 16-lane group addresses row kbase + 4*(l/32) + i/4,
// columns cbase + 16*((l%32)/16) + 4*(i%4) .. +3.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int stride, int kbase, int cbase,
                                             int lane)
{
    const int hf = lane >> 5, i = lane & 15, g16 = (lane >> 4) & 1;
    const uint16_t *p = tile + (kbase + 4 * hf + (i >> 2)) * stride + cbase + 16 * g16 + 4 * (i & 3);
    const uint2 lo = lds_read_tr16(p);
    const uint2 hi = lds_read_tr16(p + 8 * stride);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Accumulator registers R0..R0+7 of a 32x32 MFMA packed to a bf16 operand.
template <int R0>
__device__ __forceinline__ bf16x8 pack_operand(f32x16 acc)
{
    return as_bf16x8(make_uint4(pack_bf16x2(acc[R0 + 0], acc[R0 + 1]), pack_bf16x2(acc[R0 + 2], acc[R0 + 3]),
                                pack_bf16x2(acc[R0 + 4], acc[R0 + 5]), pack_bf16x2(acc[R0 + 6], acc[R0 + 7])));
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace attn
