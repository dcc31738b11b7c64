// attn_launch.h -- host-side launchers of the gfx950 kernels (internal to libattn.so).
//
// Every launcher enqueues its kernels on `st` and returns hipGetLastError().
// Arguments have already been validated by the C ABI layer (attn_api.hip):
// shapes are positive, Hq % Hkv == 0, d is supported, pointers are non-null.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

enum Dtype { kF32 = 0, kBF16 = 1 };

// Element strides of a [B][H][N][D] tensor whose head dim is contiguous:
// element (b, h, n, c) sits at b*b + h*h + n*n + c (contiguous: n = D,
// h = N*D, b = H*N*D).
struct TL {
    long b, h;
    int n;
};

// The strides of every 4-D tensor of a call (a kernel argument; launchers
// take a pointer to one, null for contiguous tensors).
struct Layouts {
    TL q, k, v, o, dout, dq, dk, dv;
};

// Contiguous [B][H][N][d] tensors: q, o, dout, dq of Hq heads and Nq rows;
// k, v, dk, dv of Hkv heads and Nk rows.
inline Layouts contiguous_layouts(int Hq, int Hkv, int Nq, int Nk, int d)
{
    const TL a{(long)Hq * Nq * d, (long)Nq * d, d}, b{(long)Hkv * Nk * d, (long)Nk * d, d};
    return Layouts{a, b, b, a, a, a, b, b};
}

// Generic kernels: any supported (dtype, d); one thread per query row or key row.
// Forward of Nq queries against Nk >= Nq keys (query i at key position i + Nk - Nq);
// o is f32, or bf16 with o_bf16.
hipError_t fwd_rowwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                       float scale, const void *q, const void *k, const void *v, void *o,
                       float *lse, hipStream_t st, bool o_bf16 = false, const Layouts *L = nullptr);
// The backward launchers take Nq query rows against Nk >= Nq keys in the same
// alignment (Nq == Nk: the square case).
hipError_t bwd_dq_rowwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, const void *q, const void *k, const void *v,
                          const float *lse, const void *dout, const float *Dws, float *dq,
                          hipStream_t st, const Layouts *L = nullptr);
hipError_t bwd_dkdv_colwise(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            float scale, const void *q, const void *k, const void *v,
                            const float *lse, const void *dout, const float *Dws, float *dk,
                            float *dv, hipStream_t st, const Layouts *L = nullptr);

// D_i = dout_i . o_i for every query row (B*Hq*N rows; dout and o contiguous,
// or of the strides of L->dout and L->o).  With zero != nullptr the same
// launch also zero-fills `zero_len` floats at `zero` and at `zero2`.
hipError_t bwd_preprocess(int dt, int B, int Hq, int N, int d, const void *dout, const void *o,
                          float *Dws, float *zero, float *zero2, long zero_len, const float *dlse,
                          hipStream_t st, bool o_bf16 = false, const Layouts *L = nullptr);
// Rotary positions on `rows` rows of d elements of dtype dt, row r at position
// pos0 + r % N (inverse: the transposed rotation); x and y may alias.
hipError_t rope(int dt, long rows, int N, int d, long pos0, double base, int inverse, const void *x,
                void *y, hipStream_t st);
// The same over two tensors of one dtype and head dim in one launch.
hipError_t rope2(int dt, long rows0, int N0, long pos00, const void *x0, void *y0, long rows1, int N1,
                 long pos01, const void *x1, void *y1, int d, double base, int inverse, hipStream_t st);
// The current device's compute-unit count (256 when no device answers).
int device_cus();
// Reads `bytes` (a multiple of 16) at src once; writes *out only when the
// XOR of everything read equals a sentinel (a read-bandwidth reference).
hipError_t read_probe(const void *src, long bytes, unsigned *out, hipStream_t st);
// Zero-fill two float buffers of n elements each (a small fill kernel; no memset).
hipError_t zero_fill2(float *a, float *b, long n, hipStream_t st);
// s_i (f32, n_i elements, n_i a multiple of 8, 16-byte aligned) rounded to
// bf16 (nearest even) into d_i, in one launch.
hipError_t to_bf16_3(const float *s0, uint16_t *d0, long n0, const float *s1, uint16_t *d1, long n1,
                     const float *s2, uint16_t *d2, long n2, hipStream_t st);

// Matrix-core kernels: bf16 inputs, d in {64, 128}.  The gradient launchers'
// rope_lb (log2 of the rotary base; 0: none, so a base of 1 is left to the
// caller) carries dQ and dK, taken at rotated q and k, back through the
// transposed rotations in their epilogues.
bool mfma_supported(int dt, int d);
hipError_t fwd_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    const void *q, const void *k, const void *v, void *o, float *lse,
                    hipStream_t st, bool o_bf16 = false);
// The forward over tensors of any strides (L: every 4-D tensor's strides).
hipError_t fwd_mfma_strided(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                            const void *q, const void *k, const void *v, void *o, float *lse,
                            const Layouts &L, hipStream_t st, bool o_bf16);
// The forward over rotated queries: q unrotated, each lane rotating its row
// in the prologue (hardware sine and cosine of the angle reduced in double)
// and writing it to q_rot (bf16); k must already be rotated.
hipError_t fwd_mfma_rope_q(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           const void *q, const void *k, const void *v, void *q_rot, float *o,
                           float *lse, double rope_lb, hipStream_t st);
// Number of workgroups each group's query heads are split over by the dK/dV
// kernel; with more than one, dk and dv must be zero-filled before the launch
// (the kernel adds into them).
int dkdv_head_split(int B, int Hq, int Hkv, int Nk, int d);
// Whether the d = 128 dK/dV work takes the 128-key kernel (larger grids).
bool dkdv_use128(int B, int Hkv, int Nk, int d);
// The d = 128 dK/dV kernel (128 keys per workgroup) and its key-tile count.
int dkdv128_tiles(int Nk);
hipError_t bwd_dkdv128_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int causal, float scale,
                            const void *q, const void *k, const void *v, const float *lse,
                            const void *dout, const float *Dws, float *dk, float *dv, int hs,
                            hipStream_t st, double rope_lb, const Layouts *L);
hipError_t bwd_dkdv_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         const void *q, const void *k, const void *v, const float *lse,
                         const void *dout, const float *Dws, float *dk, float *dv, int hs,
                         hipStream_t st, double rope_lb = 0.0, const Layouts *L = nullptr);
hipError_t bwd_dq_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       const void *q, const void *k, const void *v, const float *lse,
                       const void *dout, const float *Dws, float *dq, hipStream_t st,
                       double rope_lb = 0.0, const Layouts *L = nullptr);
// dQ that also computes D_i = dO_i . O_i - dlse_i (O f32, dlse optional) into
// Dws for a dK/dV kernel launched after it (bf16, d = 128), and zeroes zf_n
// floats (a multiple of 4; 16-byte aligned) at zf_a and at zf_b for that
// kernel's atomic head subsets
hipError_t bwd_dq_pre_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           const void *q, const void *k, const void *v, const float *lse,
                           const void *dout, const float *o, const float *dlse, float *Dws,
                           float *dq, hipStream_t st, double rope_lb, const Layouts *L = nullptr,
                           float *zf_a = nullptr, float *zf_b = nullptr, long zf_n = 0);
// Whether the one-launch plan of a shape fits its kernel argument (at most
// 48 block groups); writes the group and block counts.  No device work.
bool bwd_fused_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int hs, int *groups,
                    int *blocks);
// dQ and dK/dV in one launch (dK/dV zero-filled beforehand when hs > 1);
// hipErrorInvalidValue, with nothing launched, when bwd_fused_plan is false.
hipError_t bwd_fused_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                          const void *q, const void *k, const void *v, const float *lse,
                          const void *dout, const float *Dws, float *dq, float *dk, float *dv,
                          int hs, hipStream_t st, double rope_lb = 0.0, const Layouts *L = nullptr);

// Split-KV decode and the log-sum-exp merge.
hipError_t decode_split(int dt, int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                        const void *q, const void *kc, const void *vc, float *part_o,
                        float *part_lse, hipStream_t st);
bool decode_mfma_supported(int dt, int d, int G, int L);
hipError_t decode_split_mfma(int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                             const void *q, const void *kc, const void *vc, float *part_o,
                             float *part_lse, hipStream_t st);
// One decode step of B sequences of their own lengths with cache append.
hipError_t decode_append_mfma(int B, int Hq, int Hkv, int L, int d, float scale, int n_splits,
                              const void *q, const void *k_new, const void *v_new, void *kc,
                              void *vc, const int *seq_lens, float *part_o, float *part_lse,
                              hipStream_t st);
hipError_t lse_merge(int B, int Hq, int n_splits, int d, const float *part_o,
                     const float *part_lse, float *o, float *lse, hipStream_t st);

}  // namespace attn
