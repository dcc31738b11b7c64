// attn_api.hip -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every entry point validates all of its arguments on the host before the
// first launch, so an invalid call enqueues nothing and leaves its outputs
// untouched (the fail-closed convention of the RustingBrain docs, "Training on
// a GPU": a device failure returns an error instead of silently continuing on
// the CPU).  No exception crosses the boundary; there is no host fallback.
#include "attn.h"
#include "attn_launch.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

namespace {

using attn::kBF16;
using attn::kF32;

constexpr long kMaxGridX = 2147483647L;
constexpr long kMaxGridYZ = 65535L;

bool aligned16(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

attn_status check_common(int dt, int B, int Hq, int Hkv, int N, int d, float scale)
{
    if (dt != ATTN_F32 && dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
    if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (!head_dim_ok(d)) return ATTN_ERR_UNSUPPORTED;
    // launch-shape limits of the kernels (grid x is linear, y/z are heads and batch)
    if ((long)Hq > kMaxGridYZ || (long)B > kMaxGridYZ) return ATTN_ERR_UNSUPPORTED;
    if ((long)((N + 63) / 64) * (long)B * (long)Hq > kMaxGridX) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

// The matrix-core kernels run softmax in base 2 on |scale|*log2(e) and need a
// nonzero scale; a zero scale (uniform attention) takes the generic kernels.
// They address one head's [N][d] bf16 rows through a buffer resource with
// 32-bit byte offsets, so heads of 2^31 bytes or more take the generic
// kernels too.
bool use_mfma(int dt, int N, int d, float scale)
{
    return attn::mfma_supported(dt, d) && scale != 0.f && (long)N * d * 2 < (1L << 31);
}

// With strided tensors (L), every bf16 tensor's head must span less than
// 2^31 bytes: (rows - 1) * row stride + d elements.
bool use_mfma(int dt, int Nk, int d, float scale, const attn::Layouts *L, int Nq)
{
    if (!use_mfma(dt, Nk, d, scale)) return false;
    if (L == nullptr) return true;
    auto fits = [&](const attn::TL &t, int rows) {
        return ((long)(rows - 1) * t.n + d) * 2 < (1L << 31);
    };
    return fits(L->q, Nq) && fits(L->dout, Nq) && fits(L->k, Nk) && fits(L->v, Nk);
}

attn_status hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

size_t workspace_bytes(int B, int Hq, int N)
{
    const size_t rows = (size_t)B * (size_t)Hq * (size_t)N;
    return (rows * sizeof(float) + 255) & ~(size_t)255;
}

// Kernel launches of the three backward stages (arguments already validated;
// Nq query rows against Nk >= Nq keys, Nq == Nk in the square entry points).
// dk/dv zero-fill piggybacked on the preprocess launch when the dK/dV kernel
// will accumulate into them (zero_dkdv), else plain preprocess.
hipError_t launch_bwd_preprocess(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                 const void *o, const void *dout, float *delta, float *dk,
                                 float *dv, bool zero_dkdv, hipStream_t st,
                                 const float *dlse = nullptr, bool o_bf16 = false,
                                 const attn::Layouts *L = nullptr)
{
    const long n = (long)B * Hkv * Nk * d;
    return attn::bwd_preprocess(dt, B, Hq, Nq, d, dout, o, delta, zero_dkdv ? dk : nullptr,
                                zero_dkdv ? dv : nullptr, n, dlse, st, o_bf16, L);
}

// Forward of Nq queries against Nk >= Nq keys (arguments already validated).
hipError_t launch_fwd(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                      float scale, const void *q, const void *k, const void *v, void *o,
                      float *lse, hipStream_t st, bool o_bf16 = false,
                      const attn::Layouts *L = nullptr)
{
    if (use_mfma(dt, Nk, d, scale, L, Nq)) {
        if (L)
            return attn::fwd_mfma_strided(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, o, lse, *L,
                                          st, o_bf16);
        return attn::fwd_mfma(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, o, lse, st, o_bf16);
    }
    return attn::fwd_rowwise(dt, B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, o, lse, st,
                             o_bf16, L);
}

// Head split of the dK/dV kernel (1 = plain stores; > 1 = atomics into zeroed dk/dv).
// (use_mfma on Nk covers the Nq <= Nk query rows as well.)
int dkdv_split(int dt, int B, int Hq, int Hkv, int Nk, int d, float scale,
               const attn::Layouts *L = nullptr)
{
    // strided dk / dv take no atomics (a zero-fill would have to follow their strides)
    return use_mfma(dt, Nk, d, scale) && L == nullptr ? attn::dkdv_head_split(B, Hq, Hkv, Nk, d) : 1;
}

// dk and dv must already be zero when hs > 1.
hipError_t launch_bwd_dkdv(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                           float scale, const void *q, const void *k, const void *v,
                           const float *lse, const void *dout, const float *delta, float *dk,
                           float *dv, int hs, hipStream_t st, double rope_lb = 0.0,
                           const attn::Layouts *L = nullptr)
{
    if (use_mfma(dt, Nk, d, scale, L, Nq))
        return attn::bwd_dkdv_mfma(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, lse, dout,
                                   delta, dk, dv, hs, st, rope_lb, L);
    return attn::bwd_dkdv_colwise(dt, B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, lse,
                                  dout, delta, dk, dv, st, L);
}

hipError_t launch_bwd_dq(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                         float scale, const void *q, const void *k, const void *v,
                         const float *lse, const void *dout, const float *delta, float *dq,
                         hipStream_t st, double rope_lb = 0.0, const attn::Layouts *L = nullptr)
{
    if (use_mfma(dt, Nk, d, scale, L, Nq))
        return attn::bwd_dq_mfma(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, lse, dout,
                                 delta, dq, st, rope_lb, L);
    return attn::bwd_dq_rowwise(dt, B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, lse, dout,
                                delta, dq, st, L);
}

// The gradient stage after the preprocess.  At d = 64 on the matrix-core path
// it is one launch whose grid holds both the dK/dV and the dQ work items,
// ordered heaviest first over both kinds (measured on MI355X, 4 x 1024 x 12/4
// heads, HIP-graph replay of the training step: 83.1 us with the two kernels
// side by side on two streams, 79.8-80.0 us with the one launch).  At d = 128
// the same holds for grids whose dK/dV work would take the 64-key kernel
// anyway: there the two kinds' short chains overlap (attn_bwd, 32/8 heads,
// causal: N = 128 20.5 -> 14.0 us, N = 512 37.6 -> 28.0 us).  Otherwise -- d =
// 128 on larger grids, where the one launch would give up the 128-key dK/dV
// kernel (N = 4096: 452 -> 538 us; N = 1024 about even), the row-wise
// fallback, and shapes whose one-launch plan does not fit its kernel argument
// -- the dQ kernel (which computes the row terms itself) and then the dK/dV
// kernel run on the caller's stream (side by side on two streams they gained
// nothing at d = 128: both are bound by the same CU resources).
bool fuse_bwd(int B, int Hkv, int Nk, int d)
{
    return d == 64 || (d == 128 && !attn::dkdv_use128(B, Hkv, Nk, d));
}

bool one_launch(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                int hs, int *groups = nullptr, int *blocks = nullptr, const attn::Layouts *L = nullptr)
{
    return use_mfma(dt, Nk, d, scale, L, Nq) && fuse_bwd(B, Hkv, Nk, d) &&
           attn::bwd_fused_plan(B, Hq, Hkv, Nq, Nk, d, causal, hs, groups, blocks);
}

// dQ, dK, dV from delta (dk/dv already zero when hs > 1).
attn_status launch_bwd_grads(int dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                             float scale, const void *q, const void *k, const void *v,
                             const float *lse, const void *dout, const float *delta, float *dq,
                             float *dk, float *dv, int hs, hipStream_t st, double rope_lb = 0.0,
                             const attn::Layouts *L = nullptr)
{
    if (one_launch(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, hs, nullptr, nullptr, L))
        return hip_status(attn::bwd_fused_mfma(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v,
                                               lse, dout, delta, dq, dk, dv, hs, st, rope_lb, L));
    if (launch_bwd_dq(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, lse, dout, delta, dq, st,
                      rope_lb, L) != hipSuccess)
        return ATTN_ERR_HIP;
    return hip_status(launch_bwd_dkdv(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, lse, dout,
                                      delta, dk, dv, hs, st, rope_lb, L));
}

// The whole backward of Nq query rows against Nk >= Nq keys: the preprocess
// (with the upstream lse gradient folded into delta when dlse is given), then
// the gradient stage.  At d = 128 on the matrix-core path with f32 o, the dQ
// kernel computes delta for its own rows instead and the dK/dV kernel follows
// it on the same stream: no preprocess launch (the two kernels gain nothing
// from running side by side, both being bound by the same CU resources).
attn_status bwd_whole(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                      float scale, const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dout, const float *dlse, float *dq, float *dk,
                      float *dv, void *workspace, size_t ws_bytes, void *stream, double rope_lb = 0.0,
                      bool o_bf16 = false, const attn::Layouts *L = nullptr)
{
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nk, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_INVALID_ARG;
    if (!aligned16(workspace) || ws_bytes < workspace_bytes(B, Hq, Nq)) return ATTN_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    float *delta = (float *)workspace;
    const int hs = dkdv_split(dt, B, Hq, Hkv, Nk, d, scale, L);
    if (use_mfma(dt, Nk, d, scale, L, Nq) && !fuse_bwd(B, Hkv, Nk, d) && !o_bf16) {
        // the dQ kernel also zeroes dk and dv for the dK/dV kernel's atomic head subsets
        if (attn::bwd_dq_pre_mfma(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k, v, lse, dout,
                                  (const float *)o, dlse, delta, dq, st, rope_lb, L, dk, dv,
                                  hs > 1 ? (long)B * Hkv * Nk * d : 0L) != hipSuccess)
            return ATTN_ERR_HIP;
        return hip_status(launch_bwd_dkdv(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, lse,
                                          dout, delta, dk, dv, hs, st, rope_lb, L));
    }
    if (launch_bwd_preprocess(dt, B, Hq, Hkv, Nq, Nk, d, o, dout, delta, dk, dv, hs > 1, st,
                              dlse, o_bf16, L) != hipSuccess)
        return ATTN_ERR_HIP;
    return launch_bwd_grads(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, lse, dout, delta,
                            dq, dk, dv, hs, st, rope_lb, L);
}

// The device array behind attn_bwd_noalloc: scratch for the backward's row
// terms D_i (one f32 per query row), for callers that cannot allocate.  Each
// device holds its own copy for the life of the process.  In host code the
// name is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, resolved once per device (with that device current)
// and kept in scratch_addr.
constexpr size_t kScratchBytes = (size_t)4 << 20;   // D for up to 2^20 query rows
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];

// The current device's address of `scratch`, or null when it cannot be had.
// Concurrent first calls may both resolve it; they store the same address.
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_addr[dev].store(p, std::memory_order_release);
    return p;
}

// Strides of one tensor from the caller's layout (null: contiguous [B][H][N][d]).
// Every stride must be positive, a row at least d elements long, and each
// stride a multiple of 16 bytes so that every row starts 16-byte aligned.
bool layout_of(const attn_layout *l, int H, int N, int d, int esz, attn::TL &t)
{
    if (l == nullptr) {
        t = attn::TL{(long)H * N * d, (long)N * d, d};
        return true;
    }
    const long long m = 16 / esz;
    if (l->batch <= 0 || l->head <= 0 || l->row < d || l->row > 0x7fffffffLL) return false;
    if (l->batch % m || l->head % m || l->row % m) return false;
    t = attn::TL{(long)l->batch, (long)l->head, (int)l->row};
    return true;
}

}  // namespace

extern "C" {

attn_status attn_fwd(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     const void *q, const void *k, const void *v, float *o, float *lse,
                     void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, N, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_fwd(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, o, lse,
                                 (hipStream_t)stream));
}

attn_status attn_fwd_kv(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, const void *q, const void *k, const void *v, float *o,
                        float *lse, void *stream)
{
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nq, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_fwd(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse,
                                 (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(attn_dtype dt, int B, int Hq, int Hkv, int N, int d)
{
    if (check_common(dt, B, Hq, Hkv, N, d, 1.0f) != ATTN_OK) return 0;
    return workspace_bytes(B, Hq, N);
}

attn_status attn_bwd_dlse(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, const void *q, const void *k, const void *v, const float *o,
                          const float *lse, const void *dout, const float *dlse, float *dq,
                          float *dk, float *dv, void *workspace, size_t ws_bytes, void *stream)
{
    if (!aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    return bwd_whole(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, o, lse, dout, dlse, dq, dk,
                     dv, workspace, ws_bytes, stream);
}

attn_status attn_fwd_ex(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                        int d, int causal, float scale, const void *q, const void *k,
                        const void *v, void *o, float *lse, void *stream)
{
    if (o_dt != ATTN_F32 && o_dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nk, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_fwd(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse,
                                 (hipStream_t)stream, o_dt == ATTN_BF16));
}

attn_status attn_bwd_ex(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                        int d, int causal, float scale, const void *q, const void *k,
                        const void *v, const void *o, const float *lse, const void *dout,
                        const float *dlse, float *dq, float *dk, float *dv, void *workspace,
                        size_t ws_bytes, void *stream)
{
    if (o_dt != ATTN_F32 && o_dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (dlse != nullptr && !aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    return bwd_whole(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, dout, dlse, dq, dk,
                     dv, workspace, ws_bytes, stream, 0.0, o_dt == ATTN_BF16);
}

// Workspace of attn_bwd_bf16grad: the row terms, then f32 dq, dk and dv, each
// section 256-byte aligned.
static size_t bf16grad_sections(int B, int Hq, int Hkv, int Nq, int Nk, int d, size_t *off_dq,
                                size_t *off_dk, size_t *off_dv)
{
    auto r256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nq = (size_t)B * Hq * Nq * d, nk = (size_t)B * Hkv * Nk * d;
    *off_dq = workspace_bytes(B, Hq, Nq);
    *off_dk = *off_dq + r256(nq * sizeof(float));
    *off_dv = *off_dk + r256(nk * sizeof(float));
    return *off_dv + r256(nk * sizeof(float));
}

size_t attn_bwd_bf16grad_workspace_bytes(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d)
{
    if (Nq <= 0 || Nk < Nq || check_common(dt, B, Hq, Hkv, Nk, d, 1.0f) != ATTN_OK) return 0;
    size_t a, b, c;
    return bf16grad_sections(B, Hq, Hkv, Nq, Nk, d, &a, &b, &c);
}

attn_status attn_bwd_bf16grad(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                              int d, int causal, float scale, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, const void *dout,
                              const float *dlse, void *dq, void *dk, void *dv, void *workspace,
                              size_t ws_bytes, void *stream)
{
    if (o_dt != ATTN_F32 && o_dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (dlse != nullptr && !aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nk, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_INVALID_ARG;
    size_t off_dq, off_dk, off_dv;
    const size_t need = bf16grad_sections(B, Hq, Hkv, Nq, Nk, d, &off_dq, &off_dk, &off_dv);
    if (!aligned16(workspace) || ws_bytes < need) return ATTN_ERR_WORKSPACE;
    char *w = (char *)workspace;
    float *dq32 = (float *)(w + off_dq), *dk32 = (float *)(w + off_dk), *dv32 = (float *)(w + off_dv);
    s = bwd_whole(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, dout, dlse, dq32, dk32,
                  dv32, workspace, off_dq, stream, 0.0, o_dt == ATTN_BF16);
    if (s != ATTN_OK) return s;
    const long nq = (long)B * Hq * Nq * d, nk = (long)B * Hkv * Nk * d;
    return hip_status(attn::to_bf16_3(dq32, (uint16_t *)dq, nq, dk32, (uint16_t *)dk, nk, dv32,
                                      (uint16_t *)dv, nk, (hipStream_t)stream));
}

attn_status attn_fwd_strided(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, float scale, const void *q, const attn_layout *lq,
                             const void *k, const attn_layout *lk, const void *v,
                             const attn_layout *lv, void *o, const attn_layout *lo, float *lse,
                             void *stream)
{
    if (o_dt != ATTN_F32 && o_dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nk, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    const int esz = dt == ATTN_BF16 ? 2 : 4, oesz = o_dt == ATTN_BF16 ? 2 : 4;
    attn::Layouts L = attn::contiguous_layouts(Hq, Hkv, Nq, Nk, d);
    if (!layout_of(lq, Hq, Nq, d, esz, L.q) || !layout_of(lk, Hkv, Nk, d, esz, L.k) ||
        !layout_of(lv, Hkv, Nk, d, esz, L.v) || !layout_of(lo, Hq, Nq, d, oesz, L.o))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_fwd(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse,
                                 (hipStream_t)stream, o_dt == ATTN_BF16, &L));
}

attn_status attn_bwd_strided(attn_dtype dt, attn_dtype o_dt, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, float scale, const void *q, const attn_layout *lq,
                             const void *k, const attn_layout *lk, const void *v,
                             const attn_layout *lv, const void *o, const attn_layout *lo,
                             const float *lse, const void *dout, const attn_layout *ldout,
                             const float *dlse, float *dq, const attn_layout *ldq, float *dk,
                             const attn_layout *ldk, float *dv, const attn_layout *ldv,
                             void *workspace, size_t ws_bytes, void *stream)
{
    if (o_dt != ATTN_F32 && o_dt != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
    if (dlse != nullptr && !aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    const int esz = dt == ATTN_BF16 ? 2 : 4, oesz = o_dt == ATTN_BF16 ? 2 : 4;
    attn::Layouts L = attn::contiguous_layouts(Hq, Hkv, Nq, Nk, d);
    if (!layout_of(lq, Hq, Nq, d, esz, L.q) || !layout_of(lk, Hkv, Nk, d, esz, L.k) ||
        !layout_of(lv, Hkv, Nk, d, esz, L.v) || !layout_of(lo, Hq, Nq, d, oesz, L.o) ||
        !layout_of(ldout, Hq, Nq, d, esz, L.dout) || !layout_of(ldq, Hq, Nq, d, 4, L.dq) ||
        !layout_of(ldk, Hkv, Nk, d, 4, L.dk) || !layout_of(ldv, Hkv, Nk, d, 4, L.dv))
        return ATTN_ERR_INVALID_ARG;
    return bwd_whole(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, dout, dlse, dq, dk,
                     dv, workspace, ws_bytes, stream, 0.0, o_dt == ATTN_BF16, &L);
}

attn_status attn_rope(attn_dtype dt, int B, int H, int N, int d, long long pos0, double base,
                      int inverse, const void *x, void *y, void *stream)
{
    attn_status s = check_common(dt, B, H, H, N, d, 1.0f);
    if (s != ATTN_OK) return s;
    if (!(base > 0.0) || !isfinite(base) || llabs(pos0) > (1LL << 40)) return ATTN_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y)) return ATTN_ERR_INVALID_ARG;
    return hip_status(attn::rope(dt, (long)B * H * N, N, d, (long)pos0, base, inverse != 0, x, y,
                                 (hipStream_t)stream));
}

attn_status attn_fwd_rope(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, double base, const void *q, const void *k, const void *v,
                          void *q_rot, void *k_rot, float *o, float *lse, void *stream)
{
    // one launch rotates q and k, then the forward
    if (Nq <= 0 || Nk < Nq) return ATTN_ERR_INVALID_ARG;
    attn_status s = check_common(dt, B, Hq, Hkv, Nk, d, scale);
    if (s != ATTN_OK) return s;
    if (!(base > 0.0) || !isfinite(base)) return ATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_rot) || !aligned16(k_rot) ||
        !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    // matrix-core path: one pass rotates k, the forward rotates each query row
    // in its prologue and writes q_rot; otherwise one pass rotates both
    // (log2 base = 0 means "no rotation" to the kernels: a base of 1 takes the pass)
    if (use_mfma(dt, Nk, d, scale) && log2(base) != 0.0 && q_rot != q) {
        if (attn::rope(dt, (long)B * Hkv * Nk, Nk, d, 0, base, 0, k, k_rot, st) != hipSuccess)
            return ATTN_ERR_HIP;
        return hip_status(attn::fwd_mfma_rope_q(B, Hq, Hkv, Nq, Nk, d, causal != 0, scale, q, k_rot, v,
                                                q_rot, o, lse, log2(base), st));
    }
    if (attn::rope2(dt, (long)B * Hq * Nq, Nq, Nk - Nq, q, q_rot, (long)B * Hkv * Nk, Nk, 0, k, k_rot, d,
                    base, 0, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return hip_status(launch_fwd(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q_rot, k_rot, v, o, lse, st));
}

attn_status attn_bwd_rope(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, double base, const void *q_rot, const void *k_rot,
                          const void *v, const float *o, const float *lse, const void *dout,
                          const float *dlse, float *dq, float *dk, float *dv, void *workspace,
                          size_t ws_bytes, void *stream)
{
    if (!(base > 0.0) || !isfinite(base)) return ATTN_ERR_INVALID_ARG;
    if (dlse != nullptr && !aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    // gradients with respect to the unrotated q and k: the transposed rotations,
    // in the gradient kernels' epilogues on the matrix-core path, else a pass
    // over dq and dk afterwards
    // (log2 base = 0 means "no rotation" to the kernels: a base of 1 takes the pass)
    const bool in_epilogue = use_mfma(dt, Nk, d, scale) && log2(base) != 0.0;
    attn_status s = bwd_whole(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q_rot, k_rot, v, o, lse,
                              dout, dlse, dq, dk, dv, workspace, ws_bytes, stream,
                              in_epilogue ? log2(base) : 0.0);
    if (s != ATTN_OK || in_epilogue) return s;
    hipStream_t st = (hipStream_t)stream;
    if (attn::rope2(kF32, (long)B * Hq * Nq, Nq, Nk - Nq, dq, dq, (long)B * Hkv * Nk, Nk, 0, dk, dk, d,
                    base, 1, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

attn_status attn_bwd_kv(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, const void *q, const void *k, const void *v, const float *o,
                        const float *lse, const void *dout, const float *dlse, float *dq,
                        float *dk, float *dv, void *workspace, size_t ws_bytes, void *stream)
{
    if (dlse != nullptr && !aligned16(dlse)) return ATTN_ERR_INVALID_ARG;
    return bwd_whole(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, dout, dlse, dq, dk,
                     dv, workspace, ws_bytes, stream);
}

attn_status attn_bwd(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     const void *q, const void *k, const void *v, const float *o,
                     const float *lse, const void *dout, float *dq, float *dk, float *dv,
                     void *workspace, size_t ws_bytes, void *stream)
{
    return bwd_whole(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, o, lse, dout, nullptr, dq,
                     dk, dv, workspace, ws_bytes, stream);
}

attn_status attn_bwd_noalloc(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                             float scale, const void *q, const void *k, const void *v,
                             const float *o, const float *lse, const void *dout, float *dq,
                             float *dk, float *dv, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, N, d, scale);
    if (s != ATTN_OK) return s;
    if (workspace_bytes(B, Hq, N) > kScratchBytes) return ATTN_ERR_WORKSPACE;
    void *ws = scratch_ptr();
    if (ws == nullptr) return ATTN_ERR_HIP;
    return bwd_whole(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, o, lse, dout, nullptr, dq,
                     dk, dv, ws, kScratchBytes, stream);
}

attn_status attn_bwd_preprocess(attn_dtype dt, int B, int Hq, int N, int d, const float *o,
                                const void *dout, float *delta, void *stream)
{
    attn_status s = check_common(dt, B, Hq, 1, N, d, 1.0f);
    if (s != ATTN_OK) return s;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_bwd_preprocess(dt, B, Hq, 1, N, N, d, o, dout, delta, nullptr,
                                            nullptr, false, (hipStream_t)stream));
}


attn_status attn_bwd_dkdv(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, const void *q, const void *k, const void *v,
                          const float *lse, const void *dout, const float *delta, float *dk,
                          float *dv, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, N, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(dout) ||
        !aligned16(delta) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    const int hs = dkdv_split(dt, B, Hq, Hkv, N, d, scale);
    if (hs > 1 && attn::zero_fill2(dk, dv, (long)B * Hkv * N * d, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return hip_status(launch_bwd_dkdv(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, lse, dout,
                                      delta, dk, dv, hs, st));
}

attn_status attn_bwd_dq(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                        float scale, const void *q, const void *k, const void *v, const float *lse,
                        const void *dout, const float *delta, float *dq, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, N, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(dout) ||
        !aligned16(delta) || !aligned16(dq))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(launch_bwd_dq(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, lse, dout,
                                    delta, dq, (hipStream_t)stream));
}

attn_status attn_bwd_grads(attn_dtype dt, int B, int Hq, int Hkv, int N, int d, int causal,
                           float scale, const void *q, const void *k, const void *v,
                           const float *lse, const void *dout, const float *delta, float *dq,
                           float *dk, float *dv, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, N, d, scale);
    if (s != ATTN_OK) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(lse) || !aligned16(dout) ||
        !aligned16(delta) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    const int hs = dkdv_split(dt, B, Hq, Hkv, N, d, scale);
    if (hs > 1 && attn::zero_fill2(dk, dv, (long)B * Hkv * N * d, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return launch_bwd_grads(dt, B, Hq, Hkv, N, N, d, causal, scale, q, k, v, lse, dout, delta, dq,
                            dk, dv, hs, st);
}

int attn_bwd_grads_plan(attn_dtype dt, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                        float scale, int *groups, int *blocks)
{
    if (groups) *groups = 0;
    if (blocks) *blocks = 0;
    if (Nq <= 0 || Nk < Nq || check_common(dt, B, Hq, Hkv, Nk, d, scale) != ATTN_OK) return 0;
    const int hs = dkdv_split(dt, B, Hq, Hkv, Nk, d, scale);
    return one_launch(dt, B, Hq, Hkv, Nq, Nk, d, causal, scale, hs, groups, blocks) ? 1 : 0;
}

attn_status attn_decode(attn_dtype dt, int B, int Hq, int Hkv, int L, int d, float scale,
                        int n_splits, const void *q, const void *k_cache, const void *v_cache,
                        float *part_o, float *part_lse, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, L, d, scale);
    if (s != ATTN_OK) return s;
    if (n_splits < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
    if ((long)n_splits > kMaxGridX || (long)Hkv > kMaxGridYZ) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(part_o) ||
        !aligned16(part_lse))
        return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (attn::decode_mfma_supported(dt, d, Hq / Hkv, L) && scale != 0.f)
        return hip_status(attn::decode_split_mfma(B, Hq, Hkv, L, d, scale, n_splits, q, k_cache,
                                                  v_cache, part_o, part_lse, st));
    return hip_status(attn::decode_split(dt, B, Hq, Hkv, L, d, scale, n_splits, q, k_cache,
                                         v_cache, part_o, part_lse, st));
}

attn_status attn_decode_merged(attn_dtype dt, int B, int Hq, int Hkv, int L, int d, float scale,
                               int n_splits, const void *q, const void *k_cache,
                               const void *v_cache, float *part_o, float *part_lse, float *o,
                               float *lse, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, L, d, scale);
    if (s != ATTN_OK) return s;
    if (n_splits < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
    if ((long)n_splits > kMaxGridX || (long)Hkv > kMaxGridYZ) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(part_o) ||
        !aligned16(part_lse) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (attn::decode_mfma_supported(dt, d, Hq / Hkv, L) && scale != 0.f)
        e = attn::decode_split_mfma(B, Hq, Hkv, L, d, scale, n_splits, q, k_cache, v_cache, part_o,
                                    part_lse, st);
    else
        e = attn::decode_split(dt, B, Hq, Hkv, L, d, scale, n_splits, q, k_cache, v_cache, part_o,
                               part_lse, st);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    return hip_status(attn::lse_merge(B, Hq, n_splits, d, part_o, part_lse, o, lse, st));
}

attn_status attn_decode_append(attn_dtype dt, int B, int Hq, int Hkv, int L_cap, int d,
                               float scale, int n_splits, const void *q, const void *k_new,
                               const void *v_new, void *k_cache, void *v_cache,
                               const int *seq_lens, float *part_o, float *part_lse, float *o,
                               float *lse, void *stream)
{
    attn_status s = check_common(dt, B, Hq, Hkv, L_cap, d, scale);
    if (s != ATTN_OK) return s;
    if (n_splits < 1) return ATTN_ERR_INVALID_ARG;
    if ((long)n_splits > kMaxGridX || (long)Hkv > kMaxGridYZ) return ATTN_ERR_UNSUPPORTED;
    if (!attn::decode_mfma_supported(dt, d, Hq / Hkv, L_cap) || scale == 0.f) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(part_o) || !aligned16(part_lse) || !aligned16(o) ||
        !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    if (seq_lens == nullptr || ((uintptr_t)seq_lens & 3) != 0) return ATTN_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (attn::decode_append_mfma(B, Hq, Hkv, L_cap, d, scale, n_splits, q, k_new, v_new, k_cache,
                                 v_cache, seq_lens, part_o, part_lse, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return hip_status(attn::lse_merge(B, Hq, n_splits, d, part_o, part_lse, o, lse, st));
}

attn_status attn_lse_merge(int B, int Hq, int n_splits, int d, const float *part_o,
                           const float *part_lse, float *o, float *lse, void *stream)
{
    if (B <= 0 || Hq <= 0 || n_splits < 1 || d <= 0) return ATTN_ERR_INVALID_ARG;
    if (!head_dim_ok(d)) return ATTN_ERR_UNSUPPORTED;
    if ((long)Hq > kMaxGridX || (long)B > kMaxGridYZ) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(part_o) || !aligned16(part_lse) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_INVALID_ARG;
    return hip_status(
        attn::lse_merge(B, Hq, n_splits, d, part_o, part_lse, o, lse, (hipStream_t)stream));
}

attn_status attn_read_probe(const void *src, size_t bytes, unsigned *out, void *stream)
{
    if (!aligned16(src) || out == nullptr || ((uintptr_t)out & 3u) != 0) return ATTN_ERR_INVALID_ARG;
    if (bytes == 0 || bytes % 16 != 0) return ATTN_ERR_INVALID_ARG;
    if (bytes > ((size_t)1 << 40)) return ATTN_ERR_UNSUPPORTED;
    return hip_status(attn::read_probe(src, (long)bytes, out, (hipStream_t)stream));
}

const char *attn_status_str(attn_status s)
{
    switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int attn_abi_version(void) { return 3; }

}  // extern "C"
