// attn_device.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

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

// Rotary positions: the frequency base^(-2i/d) of pair i (log2_base = log2 base),
// and the sine and cosine of an angle of any size, reduced to [-pi, pi] in
// double and then evaluated in f32.
__device__ __forceinline__ double rope_theta(int i, int d, double log2_base)
{
    return exp2(-2.0 * i / d * log2_base);
}
__device__ __forceinline__ void rope_sincos(double a, float &s, float &c)
{
    const double turns = rint(a * 0.15915494309189535);   // a / (2 pi)
    sincosf((float)fma(-6.283185307179586, turns, a), &s, &c);
}
// The same on the hardware sine and cosine (v_sin_f32 / v_cos_f32 take the
// angle in turns), for the matrix-core path's epilogues: a few instructions
// instead of the library's full-range code, accurate to about 1e-6.
__device__ __forceinline__ void rope_sincos_turns(double t, float &s, float &c)
{
    const float f = (float)(t - rint(t));                  // in [-1/2, 1/2]
    s = __builtin_amdgcn_sinf(f);
    c = __builtin_amdgcn_cosf(f);
}
__device__ __forceinline__ void rope_sincos_hw(double a, float &s, float &c)
{
    rope_sincos_turns(a * 0.15915494309189535, s, c);      // radians -> turns
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, result lane i, element k is
// element (i % 4) of the 4-element chunk addressed by lane 4k + i/4 of the group.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p)
{
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// Row-major bf16 tiles [rows][D] in LDS with their 16-byte chunks XOR-swizzled
// by row: logical chunk c of row r lives at chunk c ^ swz(r).  swz spreads the
// two read patterns of the kernels over the banks:
//   * 16 consecutive rows reading the same logical chunk (ds_read_b128 of an
//     MFMA operand row): swz takes 16 (D = 128) or 8 (D = 64) distinct values
//     over consecutive rows;
//   * 4 aligned rows x 2 adjacent chunks (the transposed reads of tr_operand):
//     swz(r) >> 1 differs between the 4 rows while its low bit is shared.
// That is conflict-free for 128 bytes a clock.  The gfx950 LDS serves 256
// bytes a clock (64 banks), and at that width this layout leaves 2-way
// conflicts (counted on MI355X: 24-33% of the LDS-active cycles of the
// forward, dQ and dK/dV kernels at d = 128).  ATTN_LDS_SWIZZLE_256 selects a
// layout that is conflict-free at 256 bytes (a bijection of 16 consecutive
// rows, and 4 distinct swz >> 2 over 4 aligned rows at D = 128; the same per
// row parity at D = 64): it removed every conflict, left the forward and
// dK/dV kernels' times unchanged (their LDS is 30-40% busy) and made the dQ
// kernel, which uses all 256 of its registers, spill 8 of them (+6%).  It is
// therefore not the default.
template <int D>
__device__ __forceinline__ int swz(int row)
{
    static_assert(D == 64 || D == 128, "swizzle defined for 8 or 16 chunks per row");
#ifdef ATTN_LDS_SWIZZLE_256
    if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        const int a = (row >> 1) & 7;
        return ((a & 1) << 2) | (a >> 1);
    }
#else
    const int f = ((row & 3) << 1) | ((row >> 2) & 1);
    return D == 128 ? (f | (row & 8)) : f;
#endif
}

template <int D>
__device__ __forceinline__ uint16_t *tile_chunk(uint16_t *tile, int row, int c)
{
    return tile + row * D + 8 * (c ^ swz<D>(row));
}

template <int D>
__device__ __forceinline__ const uint16_t *tile_chunk(const uint16_t *tile, int row, int c)
{
    return tile + row * D + 8 * (c ^ swz<D>(row));
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, stride 0): loads
// at byte offsets past `bytes` return zero.  Dword 3 = 0x00020000 is the
// gfx9 untyped 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Direct global -> LDS copy of a tile (buffer_load_dwordx4 ... lds, no
// registers).  One wave instruction moves 64 x 16 bytes into 1 KiB of LDS,
// lane L landing at byte 16 L of it; the LDS address is wave-uniform (M0).
// The tile of ROWS rows starting at row r0 of the [*][D] bf16 tensor behind
// the resource is filled in 1 KiB blocks, NW waves sharing them: wave w takes
// blocks w, w + NW, w + 2 NW, ...  Lane L of block j owns physical chunk
// 64 j + L and fetches the logical chunk the swizzle maps there.  Consecutive
// blocks of a wave lie 64 NW / (D/8) rows apart -- a multiple of the swizzle
// period -- so every block of a wave uses the same per-lane byte offset
// (computed once) plus a wave-uniform one.  Rows past the end of the resource
// read as zero.  The copy completes asynchronously: wait for vmcnt before the
// barrier that publishes it.  (The buffer form, unlike global_load_lds, lets
// the compiler keep partial LDS-read waits while a copy is in flight.)
// The rows of the tensor in memory lie ld elements apart (ld = D: contiguous
// rows; a larger ld: a strided layout such as [B][N][H][D]); the LDS tile is
// always [ROWS][D].
template <int D, int ROWS, int NW>
struct TileCopy {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int BLOCKS = ROWS * CPR / 64;
    static constexpr int PER_WAVE = BLOCKS / NW;      // copy instructions per wave
    static constexpr int RPB = 64 * NW / CPR;         // rows between a wave's blocks
    static_assert(ROWS * CPR % 64 == 0 && BLOCKS % NW == 0, "whole 1 KiB blocks per wave");
    static_assert(RPB % 16 == 0, "block stride keeps the swizzle");
    int voff;                                         // byte offset of this lane in block `wave`
    int ld;                                           // elements between rows in memory

    __device__ __forceinline__ TileCopy(int wave, int lane, int ld_ = D) : ld(ld_)
    {
        const int p = 64 * wave + lane;
        const int row = p / CPR;
        voff = (row * ld + 8 * ((p % CPR) ^ swz<D>(row))) * 2;
    }

    __device__ __forceinline__ void operator()(uint16_t *tile, __amdgpu_buffer_rsrc_t rs, int r0,
                                               int wave) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(tile + 512 * (wave + NW * i)), 16, voff,
                                                     (r0 + RPB * i) * ld * 2, 0, 0);
    }
};

__device__ __host__ __forceinline__ TL contiguous_tl(int H, int N, int D)
{
    return TL{(long)H * N * D, (long)N * D, D};
}
// Bytes a buffer resource over one head must cover: N rows of D elements, ld apart.
__device__ __forceinline__ uint32_t head_bytes(int N, int ld, int D, int esz)
{
    return (uint32_t)(((long)(N - 1) * ld + D) * esz);
}



// One f32 per lane, element r0 + lane of the f32 array behind the resource
// (zero past its end), into a register.
__device__ __forceinline__ float row_load(__amdgpu_buffer_rsrc_t rs, int r0, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (r0 + lane) * 4, 0, 0));
}

// 8 bf16 (logical chunk c) of one row: an MFMA operand whose contraction runs
// along the row.
template <int D>
__device__ __forceinline__ bf16x8 tile_row_operand(const uint16_t *tile, int row, int c)
{
    return as_bf16x8(*(const uint4 *)tile_chunk<D>(tile, row, c));
}

// Operand of v_mfma_f32_32x32x16_bf16 whose contraction runs down the rows of a
// swizzled tile: lane l gets column cbase + l%32 at rows kbase + 4*(l/32) +
// {0,1,2,3} (elements 0..3) and kbase + 8 + 4*(l/32) + {0..3} (elements 4..7).
// That is exactly the row order in which the 32x32 accumulator of the previous
// MFMA holds its rows (rows 8(r/4) + 4*(l/32) + r%4), so an accumulator
// repacked to bf16 pairs with this operand.  Two transposed LDS reads: lane i
// of each 16-lane group addresses row kbase + 4*(l/32) + i/4, columns
// cbase + 16*((l%32)/16) + 4*(i%4) .. +3.  cbase is a multiple of 16.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int kbase, int cbase, int lane)
{
    const int hf = lane >> 5, i = lane & 15, g16 = (lane >> 4) & 1;
    const int row = kbase + 4 * hf + (i >> 2);
    const int c = (cbase >> 3) + 2 * g16 + ((i & 3) >> 1);     // logical 16-byte chunk
    const int off = 4 * (i & 1);                                // element within the chunk
    const uint2 lo = lds_read_tr16(tile_chunk<D>(tile, row, c) + off);
    const uint2 hi = lds_read_tr16(tile_chunk<D>(tile, row + 8, c) + off);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Wait until at most N of this wave's vector-memory operations (direct
// global->LDS copies included) are outstanding; LDS and export counters are
// not waited on.  gfx9 s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// No instruction is scheduled across this point (keeps MFMAs issued before a
// wait instead of after it).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier for LDS data written before it -- by this wave's LDS
// stores, or by direct copies whose vmcnt each wave has already waited for --
// without the wait for every outstanding vector-memory operation that
// __syncthreads implies (its workgroup fence also covers the direct copies), so
// that copies of later tiles stay in flight across it.  The empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS tile buffers are separate __shared__ arrays chosen at compile time: the
// compiler then knows that a read of the current buffer does not alias the
// direct global->LDS copy in flight into the other one, and does not wait for
// that copy before the read.
template <int I>
struct Buf {
    static constexpr int value = I;
};

// Scheduling hint for the current basic block: NR LDS reads, NM MFMAs and NV
// vector-memory instructions (the next tile's direct copies) are interleaved as
// AHEAD reads first, then per MFMA: the MFMA, RPM reads while reads remain, and
// VPM copies while copies remain.  The reads for later MFMAs and the copies are
// issued while earlier MFMAs execute -- a wave that issues many copies back to
// back stalls until the memory pipeline accepts them, so they are spread out.
// (Masks: 0x008 = MFMA, 0x010 = vector memory, 0x100 = LDS read.)
template <int I, int NM, int REST, int RPM, int NV, int VPM>
struct SchedPipeStep {
    static __device__ __forceinline__ void emit()
    {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (I * RPM < REST) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
        if constexpr (I * VPM < NV) __builtin_amdgcn_sched_group_barrier(0x010, VPM, 0);
        if constexpr (I + 1 < NM) SchedPipeStep<I + 1, NM, REST, RPM, NV, VPM>::emit();
    }
};

template <int NR, int NM, int AHEAD, int RPM, int NV = 0>
__device__ __forceinline__ void sched_pipeline()
{
    static_assert(AHEAD <= NR && (NR - AHEAD) % RPM == 0, "reads must split evenly");
    constexpr int VPM = NV == 0 ? 1 : (NV + NM - 1) / NM;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
    SchedPipeStep<0, NM, NR - AHEAD, RPM, NV, VPM>::emit();
}

// Scheduling hint for a basic block of NM MFMAs and NR LDS reads: AHEAD reads
// first, then behind MFMA i as many as bring the reads issued to
// AHEAD + (i + 1) * NUM / DEN (the rate at which the MFMAs consume them), so
// that the reads stay a constant distance ahead until they run out.
// (Masks: 0x008 = MFMA, 0x100 = LDS read.)
template <int SID, int I, int NM, int NR, int AHEAD, int NUM, int DEN>
__device__ __forceinline__ void sched_lead_step()
{
    constexpr int c0 = AHEAD + I * NUM / DEN, c1 = AHEAD + (I + 1) * NUM / DEN;
    constexpr int n = (c1 < NR ? c1 : NR) - (c0 < NR ? c0 : NR);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SID);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, SID);
    if constexpr (I + 1 < NM) sched_lead_step<SID, I + 1, NM, NR, AHEAD, NUM, DEN>();
}
// SID: a sync id of its own per copy of the code, so that identical hints in
// different copies are never merged.
template <int SID, int NR, int NM, int AHEAD, int NUM, int DEN>
__device__ __forceinline__ void sched_lead()
{
    static_assert(AHEAD <= NR, "reads ahead");
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, SID);
    sched_lead_step<SID, 0, NM, NR, AHEAD, NUM, DEN>();
}

// Accumulator registers R0..R0+7 of a 32x32 MFMA packed to a bf16 operand.
template <int R0>
__device__ __forceinline__ bf16x8 pack_operand(f32x16 acc)
{
    return as_bf16x8(make_uint4(pack_bf16x2(acc[R0 + 0], acc[R0 + 1]), pack_bf16x2(acc[R0 + 2], acc[R0 + 3]),
                                pack_bf16x2(acc[R0 + 4], acc[R0 + 5]), pack_bf16x2(acc[R0 + 6], acc[R0 + 7])));
}

// Max / sum of x over the lane pair (l, l ^ 32), or (l, l ^ 16), in every lane
// of the pair, without the LDS round trip of a shuffle: v_permlane32_swap
// (v_permlane16_swap) exchanges the two 32-lane (16-lane) halves of two
// registers, so with both holding x each lane ends with its own value and its
// partner's, one in each result (which one is which does not matter to a
// symmetric combine).
__device__ __forceinline__ float pair32_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Workgroups are dispatched round-robin over the 8 XCDs of the chip (block i
// runs on XCD i % 8), and every XCD has its own L2.  For work items indexed by
// (key/value group, heaviest-first tile index, head in group) this returns the
// item of block i such that, when the group count is a multiple of 8, each XCD
// owns whole groups (their K and V stay in one L2) and runs its items
// heaviest tile first, the groups interleaved (so that the heavy items of all
// its groups start first).  Otherwise blocks take items in plain
// heaviest-first order.  Returns false for padding blocks (the grid is a
// multiple of 8).
// SNAKE, for grids whose workgroups are all resident at once: an XCD places
// its items on its CUs in dispatch order, one per CU a round, and odd rounds
// take their items in reverse, so that a CU holding a heavy item of one round
// holds a light one of the next (the CU's total then decides its end).  With
// more work than slots, blocks of later rounds start as slots free up and the
// plain order packs better, so it is the default.
struct WorkItem {
    int group, tile, head;
};

constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;   // MI355X: 256 CUs in 8 XCDs

template <bool SNAKE = false>
__device__ __forceinline__ bool xcd_work_item(int block, int groups, int tiles, int heads, WorkItem &w)
{
    const int total = groups * tiles * heads;
    if (groups % kXcds == 0) {
        const int per_xcd = total / kXcds, gpx = groups / kXcds;
        const int x = block % kXcds, kd = block / kXcds;
        if (kd >= per_xcd) return false;
        const int r = kd / kCusPerXcd, p = kd % kCusPerXcd;
        const int k = (SNAKE && (r & 1) && (r + 1) * kCusPerXcd <= per_xcd)
                          ? r * kCusPerXcd + kCusPerXcd - 1 - p : kd;
        const int level = k / (gpx * heads), rem = k % (gpx * heads);
        w.tile = tiles - 1 - level;
        w.group = x * gpx + rem / heads;
        w.head = rem % heads;
    } else {
        if (block >= total) return false;
        const int level = block / (groups * heads), rem = block % (groups * heads);
        w.tile = tiles - 1 - level;
        w.group = rem / heads;
        w.head = rem % heads;
    }
    return true;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace attn
