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
//   * K and V tiles stay row-major in LDS (16-byte chunks XOR-swizzled by row,
//     which keeps both the row reads and the transposed reads conflict-free),
//     double-buffered, filled by direct global->LDS loads (no staging
//     registers), one barrier per tile, the next tile's loads in flight during
//     the current MFMAs;
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
constexpr int kBN = 64;       // keys per tile (the key-split d = 64 kernel: 32)
constexpr float kLazy = 8.f;  // max growth tolerated before rescaling (log2 units)

// Per-wave state of the streaming softmax: this lane's query row, its Q^T
// operand, the O^T accumulator and the running max / partial sum.
template <int D>
struct FwdState {
    static constexpr int KS = D / 16;       // MFMA k-steps over the head dim
    static constexpr int DB = D / 32;       // 32-row blocks of O^T
    bf16x8 qf[KS];
    f32x16 oacc[DB];
    float m_run;    // running max of c2 * q.k for this lane's row (log2 units)
    float m_thr;    // m_run + kLazy: a tile max above it raises m_run
    float nm;       // exponent offset -m_run (0 while m_run = -inf)
    float lq[4];    // this lane's share of the running sum, in four chains
    __device__ __forceinline__ float l_sum() const { return (lq[0] + lq[1]) + (lq[2] + lq[3]); }
};

// One 64-key tile for one wave: S^T = K Q^T, the online-softmax update and
// O^T += V^T P^T.  With `mask` (wave-uniform: diagonal and tail tiles) keys
// after the query row's position qa and past the key count Nk are hidden.  `prefetch`
// issues the wave's NV direct copies of the next tile; they are interleaved
// with the S^T MFMAs.  PRIO raises the wave's issue priority while it issues
// its MFMAs, so that with two waves per SIMD one wave's matrix work goes
// first while the other's softmax fills the vector ALU.
template <int D, int NV, int NKB, bool PRIO, class Prefetch>
__device__ __forceinline__ void fwd_tile(FwdState<D> &st, const uint16_t *skb, const uint16_t *svb,
                                         float c2, int kv0, int qa, int Nk, int causal, bool mask,
                                         int lane, const Prefetch &prefetch)
{
    constexpr int KS = FwdState<D>::KS, DB = FwdState<D>::DB;
    const int l32 = lane & 31, hf = lane >> 5;
    prefetch();

    // S^T for the tile's NKB 32-key blocks; the K operands are read first and
    // interleaved with the MFMAs (4 reads ahead, then one per MFMA).
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    f32x16 sacc[NKB];
    bf16x8 ka[NKB][KS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[kb][ks] = tile_row_operand<D>(skb, kb * 32 + l32, 2 * ks + hf);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sacc[kb] = mfma32x32x16(ka[kb][ks], st.qf[ks], sacc[kb]);
    sched_pipeline<NKB * KS, NKB * KS, 4, 1, NV>();
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);

    // Row max on the raw scores (c2 > 0 commutes with max); masked scores are -inf.
    // Register r of block kb holds key kv0 + 4hf + c, c = 32kb + 8(r/4) + r%4
    // (a constant), kept iff c < lim: one compare and one select per score.
    if (mask) {
        const int lim = (causal ? min(qa + 1, Nk) : Nk) - (kv0 + 4 * hf);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
                sacc[kb][r] = c < lim ? sacc[kb][r] : -INFINITY;
            }
    }
    // Row max and row sum as four independent chains each (short dependency
    // chains matter: a wave's tile is a latency chain at small head dims);
    // the max chains start from the tile's first scores, the sum chains run
    // on across tiles (the vector ALU is what bounds small grids).
    float mq[4] = {sacc[0][0], sacc[0][1], sacc[0][2], sacc[0][3]};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = kb == 0 ? 4 : 0; r < 16; ++r) mq[r & 3] = fmaxf(mq[r & 3], sacc[kb][r]);
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = pair32_max(mx) * c2;
    // Lazy rescale: raise the running max only when some row of the wave grew
    // past it by more than kLazy.  A row that has seen no key yet keeps -inf
    // (its probabilities are then exact zeros, see nm).
    if (__any(mx > st.m_thr)) {
        const float m_new = fmaxf(st.m_run, mx);
        const float alpha = st.m_run == -INFINITY ? 0.f : exp2_fast(st.m_run - m_new);
#pragma unroll
        for (int c = 0; c < 4; ++c) st.lq[c] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
        st.m_run = m_new;
        st.m_thr = m_new + kLazy;
        st.nm = m_new == -INFINITY ? 0.f : -m_new;
    }
    // p = 2^(c2 s - m): one FMA and one exp per score (exp2(-inf) = 0; a row
    // with no key seen yet has only hidden scores, and m = -inf is taken as 0)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(sacc[kb][r], c2, st.nm));
            sacc[kb][r] = p;
            st.lq[r & 3] += p;
        }

    // O^T += V^T P^T, 2 NKB 16-key steps.  Step tt consumes accumulator
    // registers (tt&1)*8 .. +7 of block tt>>1, i.e. keys 16tt + 4hf + {0..3}
    // and 16tt + 8 + 4hf + {0..3}; tr_operand reads V^T in that order.
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    bf16x8 va[2 * NKB][DB];
#pragma unroll
    for (int tt = 0; tt < 2 * NKB; ++tt)
#pragma unroll
        for (int db = 0; db < DB; ++db) va[tt][db] = tr_operand<D>(svb, 16 * tt, db * 32, lane);
#pragma unroll
    for (int tt = 0; tt < 2 * NKB; ++tt) {
        const bf16x8 pb = (tt & 1) ? pack_operand<8>(sacc[tt >> 1]) : pack_operand<0>(sacc[tt >> 1]);
#pragma unroll
        for (int db = 0; db < DB; ++db) st.oacc[db] = mfma32x32x16(va[tt][db], pb, st.oacc[db]);
    }
    sched_pipeline<4 * NKB * DB, 2 * NKB * DB, 4, 2>();
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

// KSPLIT = 1: one workgroup = 4 waves = 128 query rows (32 per wave), every
// wave streaming all the key tiles of its query tile.
// KSPLIT = 2 (small grids): one workgroup = 64 query rows; waves (row half,
// key half) -- the two key halves stream disjoint halves of the key tiles
// side by side and their softmax states combine through LDS at the end with
// the associative merge, which halves the longest chain of tiles.  KSPLIT = 4
// (smaller grids; 32-key tiles): 32 query rows, the four waves each streaming
// a quarter of the key tiles.
// OBF: O is written in bf16 (rounded to nearest even) instead of f32.
// ROPE: q arrives unrotated; each lane turns its Q row (position i + Nk - Nq)
// by the rotary angles right after loading it -- the lane already holds both
// halves (i, i + D/2) of every pair, as chunks ks and ks + KS/2 of its
// operand -- and writes the rotated row, rounded to bf16, to Qrot (the
// backward takes it).  rope_lb = log2 of the rotary base.
// STR: q, k, v and o have the strides of L (else contiguous [B][H][N][D]).
template <int D, int KSPLIT, int TN, bool OBF, bool ROPE = false, bool STR = false>
__global__ __launch_bounds__(256, D == 128 && KSPLIT > 1 ? 1 : 2) void fwd_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, void *__restrict__ O, float *__restrict__ LSE, int B, int Hq,
    int Hkv, int Nq, int Nk, float scale, int causal, int nqt, uint16_t *__restrict__ Qrot,
    double rope_lb, Layouts L)
{
    static_assert(!(ROPE && STR), "the rotated forward takes contiguous tensors");
    constexpr int KS = FwdState<D>::KS, DB = FwdState<D>::DB;
    constexpr int RW = 4 / KSPLIT;           // row waves
    constexpr int BMW = 32 * RW;             // query rows per workgroup
    constexpr int TE = TN * D;               // elements of one tile (TN keys)
    // K and V tiles (one per key half), row-major with swizzled 16-byte
    // chunks, double-buffered in four separate arrays (see Buf)
    __shared__ __attribute__((aligned(16))) uint16_t sk0[KSPLIT * TE], sk1[KSPLIT * TE];
    __shared__ __attribute__((aligned(16))) uint16_t sv0[KSPLIT * TE], sv1[KSPLIT * TE];

    // Work item (query tile, batch, query head), XCD-aware (see xcd_work_item)
    const int G = Hq / Hkv;
    WorkItem w;
    // small grids (two or four key parts) are resident at once: snake order
    if (!xcd_work_item<(KSPLIT > 1)>(blockIdx.x, B * Hkv, nqt, G, w)) return;
    const int qt = w.tile;
    const int b = w.group / Hkv, g = w.group % Hkv;
    const int h = g * G + w.head;
    const int q0 = qt * BMW;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int rw = wave % RW, kh = wave / RW;                     // row wave, key half
    const int l32 = lane & 31, hf = lane >> 5;
    const int qw0 = q0 + rw * 32;           // first query row of this wave
    const int qi = qw0 + l32;               // this lane's query row

    // Nq queries against Nk >= Nq keys: query row i sits at key position
    // i + off (the queries are the last Nq positions; off = 0 for self-attention)
    const int off = Nk - Nq;
    const TL lq = STR ? L.q : contiguous_tl(Hq, Nq, D), lo = STR ? L.o : contiguous_tl(Hq, Nq, D);
    const TL lk = STR ? L.k : contiguous_tl(Hkv, Nk, D), lv = STR ? L.v : contiguous_tl(Hkv, Nk, D);
    const uint16_t *Qh = Q + b * lq.b + h * lq.h;
    const uint16_t *Kg = K + b * lk.b + g * lk.h;
    const uint16_t *Vg = V + b * lv.b + g * lv.h;

    // Softmax on c2 q.k with c2 = |scale| log2(e) > 0; a negative scale is
    // carried by negating q, which is exact in bf16.
    const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
    const float c2 = fabsf(scale) * kLog2e;

    FwdState<D> st;
    // Q^T operand, resident: lane holds q[qi][16ks + 8hf .. +7].  The tile's
    // Q rows go global -> LDS directly (whole rows; rows past Nq read as zero
    // and are never stored) into the second K and V buffers, 64 rows each
    // (the first 64 rows in sk1, the rest in sv1), which step 1's copy fills
    // only after step 0 has read them.
    static_assert(64 * D * sizeof(uint16_t) <= sizeof(sk1), "64 Q rows fit a buffer");
    {
        const uint32_t q_bytes = head_bytes(Nq, lq.n, D, 2);
        const TileCopy<D, 64, 4> qcopy(wave, lane, lq.n);
        qcopy(sk1, make_rsrc(Qh, q_bytes), q0, wave);
        if constexpr (BMW > 64) qcopy(sv1, make_rsrc(Qh, q_bytes), q0 + 64, wave);
    }
    // The Q rows of a wave lie in one of the two arrays (rows 0..63 in sk1,
    // 64..127 in sv1: a wave-uniform choice).  Each access names its array
    // directly rather than through a select, so that the compiler can tell it
    // from the step-0 copies into sk0 / sv0 still in flight and does not wait
    // for them.
    const int qr = rw * 32 + l32;            // this lane's row within the tile
    auto on_q_rows = [&](auto f) {
        if (BMW <= 64 || qr < 64) f(sk1); else f(sv1);
    };
    auto read_q = [&] {
        on_q_rows([&](const uint16_t *qt) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 u = *(const uint4 *)tile_chunk<D>(qt, qr & 63, 2 * ks + hf);
                u.x ^= qsign; u.y ^= qsign; u.z ^= qsign; u.w ^= qsign;
                st.qf[ks] = as_bf16x8(u);
            }
        });
    };
    // ROPE: the tile's Q rows, once in LDS, are turned in place, one pair of
    // chunks (ks, ks + KS/2) at a time; with two key halves both halves' waves
    // share the chunk pairs of their rows (all four SIMDs busy).  Pair
    // i = 16ks + 8hf + e turns by pos * r^i / (2 pi) turns, r = base^(-2/D):
    // one exp2 per lane for r, then products -- r^8 and r^16 by squaring, the
    // chunk's first frequency, and steps of r -- and then the rows are written
    // out whole by all threads as Qrot.
    auto rotate_q = [&] {
        on_q_rows([&](uint16_t *qt) {
            const double pos = (double)(qi + off);
            const double r1 = rope_theta(1, D, rope_lb);
            const double r2 = r1 * r1, r4 = r2 * r2, r8 = r4 * r4, r16 = r8 * r8;
            // frequency of pair 16 kh + 8 hf, in turns per position
            double f0 = (hf ? r8 : 1.0) * 0.15915494309189535;
            for (int j = 0; j < kh; ++j) f0 *= r16;
            double r16k = 1.0;
            for (int j = 0; j < KSPLIT; ++j) r16k *= r16;
#pragma unroll 1
            for (int ks = kh; ks < KS / 2; ks += KSPLIT, f0 *= r16k) {
                uint4 *p0 = (uint4 *)tile_chunk<D>(qt, qr & 63, 2 * ks + hf);
                uint4 *p1 = (uint4 *)tile_chunk<D>(qt, qr & 63, 2 * (ks + KS / 2) + hf);
                const uint4 a0 = *p0, a1 = *p1;
                const uint32_t w0[4] = {a0.x, a0.y, a0.z, a0.w}, w1[4] = {a1.x, a1.y, a1.z, a1.w};
                uint32_t o0[4], o1[4];
                double f = f0;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float y0[2], y1[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh, f *= r1) {
                        const float x0 = hh ? bf16hi(w0[e2]) : bf16lo(w0[e2]);
                        const float x1 = hh ? bf16hi(w1[e2]) : bf16lo(w1[e2]);
                        float sn, cs;
                        rope_sincos_turns(pos * f, sn, cs);
                        y0[hh] = x0 * cs - x1 * sn;
                        y1[hh] = x0 * sn + x1 * cs;
                    }
                    o0[e2] = pack_bf16x2(y0[0], y0[1]);
                    o1[e2] = pack_bf16x2(y1[0], y1[1]);
                }
                *p0 = make_uint4(o0[0], o0[1], o0[2], o0[3]);
                *p1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
            }
        });
        lds_barrier();
        constexpr int CPR = D / 8;           // 16-byte chunks per row
        uint16_t *qrot_h = Qrot + ((size_t)b * Hq + h) * (size_t)Nq * D;
        auto write_rows = [&](const uint16_t *qt, int r0) {
#pragma unroll 1
            for (int c = tid; c < (BMW < 64 ? BMW : 64) * CPR; c += 256) {
                const int r = c / CPR, ch = c % CPR;
                if (q0 + r0 + r < Nq)
                    *(uint4 *)(qrot_h + (size_t)(q0 + r0 + r) * D + 8 * ch) =
                        *(const uint4 *)tile_chunk<D>(qt, r, ch);
            }
        };
        write_rows(sk1, 0);
        if constexpr (BMW > 64) write_rows(sv1, 64);
    };
    const int kv_end = causal ? min(Nk, q0 + off + BMW) : Nk;
    const int ntiles = (kv_end + TN - 1) / TN;
    // Key part p (of KSPLIT) takes consecutive tiles from tile_of(p, 0); the
    // parts' counts differ by at most one, the later parts holding the extra
    // tiles.  A row may see no key of a part (its max stays -inf, its weights
    // are zeros); the part holding tile 0 holds key 0, which every row sees.
    const int kbase = ntiles / KSPLIT, krem = ntiles % KSPLIT;
    const int nsteps = kbase + (krem > 0 ? 1 : 0);
    auto tile_of = [&](int part, int s_) { return part * kbase + max(0, part - (KSPLIT - krem)) + s_; };
    auto valid = [&](int part, int s_) { return s_ < kbase + (part >= KSPLIT - krem ? 1 : 0); };

    // Tiles move global -> LDS directly (no staging registers); rows past N
    // read as zero, their scores are masked; copies of tiles that do not
    // exist read nothing (zero-byte resources).
    const uint32_t k_bytes = head_bytes(Nk, lk.n, D, 2), v_bytes = head_bytes(Nk, lv.n, D, 2);
    using Copy = TileCopy<D, TN, 4>;
    const Copy copy(wave, lane, lk.n), copyv(wave, lane, lv.n);
    auto copy_step = [&](uint16_t *skd, uint16_t *svd, int s_) {
#pragma unroll
        for (int half = 0; half < KSPLIT; ++half) {
            const bool ok = valid(half, s_);
            const int t_ = tile_of(half, s_);
            copy(skd + half * TE, make_rsrc(Kg, ok ? k_bytes : 0u), t_ * TN, wave);
            copyv(svd + half * TE, make_rsrc(Vg, ok ? v_bytes : 0u), t_ * TN, wave);
        }
    };
    copy_step(sk0, sv0, 0);

    // The resident Q rows, while the step-0 copies are in flight: wait for the
    // Q copies alone (issued first; loads complete in order), rotate them
    // (ROPE), read the operands, and free buffer 1 for step 1's copies.  The
    // softmax state is set up only afterwards, so the prologue's registers do
    // not add to the loop's.
    wait_vmcnt<2 * KSPLIT * Copy::PER_WAVE>();
    lds_barrier();
    if constexpr (ROPE) rotate_q();
    read_q();
    __syncthreads();

    st.m_run = -INFINITY;
    st.m_thr = -INFINITY;
    st.nm = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) st.lq[c] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;

    // Step s reads buffer s % 2 while step s+1 is copied into the other one.
    auto run_step = [&](auto bufc, int s_) {
        constexpr int BI = decltype(bufc)::value;
        uint16_t *skc = BI ? sk1 : sk0, *svc = BI ? sv1 : sv0;
        uint16_t *skn = BI ? sk0 : sk1, *svn = BI ? sv0 : sv1;
        wait_vmcnt<0>();                    // this wave's copies of step s have landed
        __syncthreads();                    // ... and every wave's; buffer s+1 is free
        // copies of step s+1 (branch-free, so they can interleave with MFMAs)
        auto prefetch = [&] { copy_step(skn, svn, s_ + 1); };
        const int kv0 = tile_of(kh, s_) * TN;
        if (valid(kh, s_) && qw0 < Nq && (!causal || kv0 <= qw0 + off + 31)) {
            const bool mask = (causal && kv0 + TN - 1 > qw0 + off) || kv0 + TN > Nk;
            fwd_tile<D, 2 * KSPLIT * Copy::PER_WAVE, TN / 32, D == 128 && KSPLIT == 1>(st, skc + kh * TE, svc + kh * TE, c2, kv0, qi + off,
                                                     Nk, causal, mask, lane, prefetch);
        } else {
            prefetch();
        }
        sched_fence();
    };
    for (int s_ = 0; s_ < nsteps; s_ += 2) {
        run_step(Buf<0>{}, s_);
        if (s_ + 1 < nsteps) run_step(Buf<1>{}, s_ + 1);
    }

    if constexpr (KSPLIT > 1) {
        // Key parts 1 .. KSPLIT-1 park (O^T, m, l) per lane in LDS and part 0
        // merges them: m = max of the parts' m, O = sum of O_p 2^(m_p - m), l
        // likewise.  The part that saw key 0 has a finite m; a part that saw no
        // key has m = -inf and weight 0.
        constexpr int SLOT = DB * 16 * 64;                               // floats of one parked O^T
        constexpr int CAP = (int)(sizeof(sk0) / (SLOT * sizeof(float))); // slots per array
        constexpr int NSLOT = RW * (KSPLIT - 1);
        static_assert(CAP >= 1 && NSLOT <= 2 * CAP, "parked O^T fits sk0 and sk1");
        static_assert(NSLOT * 2 * 64 * sizeof(float) <= sizeof(sv0), "parked m, l fit sv0");
        auto slot_o = [&](int slot) {
            float *a = reinterpret_cast<float *>(slot < CAP ? sk0 : sk1);
            return a + (slot % CAP) * SLOT;
        };
        float *pm = reinterpret_cast<float *>(sv0);                      // [slot][m, l][64]
        wait_vmcnt<0>();
        __syncthreads();
        if (kh > 0) {
            const int slot = rw * (KSPLIT - 1) + kh - 1;
            float *po = slot_o(slot);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) po[(db * 16 + r) * 64 + lane] = st.oacc[db][r];
            pm[(slot * 2 + 0) * 64 + lane] = st.m_run;
            pm[(slot * 2 + 1) * 64 + lane] = st.l_sum();
        }
        __syncthreads();
        if (kh > 0) return;
        float m = st.m_run;
#pragma unroll
        for (int p = 1; p < KSPLIT; ++p) m = fmaxf(m, pm[((rw * (KSPLIT - 1) + p - 1) * 2) * 64 + lane]);
        const float ea = exp2_fast(st.m_run - m);
        float l = st.l_sum() * ea;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.oacc[db][r] *= ea;
#pragma unroll
        for (int p = 1; p < KSPLIT; ++p) {
            const int slot = rw * (KSPLIT - 1) + p - 1;
            const float *po = slot_o(slot);
            const float e = exp2_fast(pm[(slot * 2 + 0) * 64 + lane] - m);
            l += pm[(slot * 2 + 1) * 64 + lane] * e;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[db][r] += po[(db * 16 + r) * 64 + lane] * e;
        }
        st.lq[0] = l;
        st.lq[1] = st.lq[2] = st.lq[3] = 0.f;
        st.m_run = m;
    }

    const float l_tot = pair32_sum(st.l_sum());
    if (qi < Nq) {
        const float inv = 1.f / l_tot;
        const size_t orow = b * lo.b + h * lo.h + (long)qi * lo.n;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = db * 32 + 8 * a + 4 * hf;
                const float o0 = st.oacc[db][4 * a + 0] * inv, o1 = st.oacc[db][4 * a + 1] * inv;
                const float o2 = st.oacc[db][4 * a + 2] * inv, o3 = st.oacc[db][4 * a + 3] * inv;
                if constexpr (OBF)
                    *(uint2 *)((uint16_t *)O + orow + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
                else
                    *(float4 *)((float *)O + orow + d0) = make_float4(o0, o1, o2, o3);
            }
        // lse = ln(sum exp(scale q.k)) = (m + log2 l) * ln 2
        if (hf == 0) LSE[((size_t)b * Hq + h) * Nq + qi] = (st.m_run + __log2f(l_tot)) * kLn2;
    }
}

}  // namespace

bool mfma_supported(int dt, int d) { return dt == kBF16 && (d == 64 || d == 128); }

namespace {

template <bool OBF, bool ROPE, bool STR>
hipError_t fwd_mfma_launch(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           const void *q, const void *k, const void *v, void *o, float *lse,
                           hipStream_t st, void *q_rot, double rope_lb, const Layouts &L)
{
    const int cus = device_cus();
    const int nqt = (Nq + kBM - 1) / kBM;
    // Key split of small grids.  d = 64 (32-key tiles, 32 KB of LDS, up to
    // three workgroups per CU): when the 128-row workgroups would not give
    // every CU two.  d = 128 (one split workgroup per CU: 128 KB of LDS): when
    // the 128-row workgroups would leave CUs empty.
    const long items = (long)nqt * B * Hq;
    const bool split = d == 64 ? items < 2L * cus : items < cus;
    // d = 64, four key parts (32-row workgroups, 64 KB of LDS, two per CU):
    // when all of them fit on the CUs at once, i.e. at most half a 128-row item
    // per CU.  Measured on MI355X (forward, causal): 96 items (1 x 12 heads x
    // 1024) 10.9 -> 8.3 us, 128 items 7.45 -> 6.4 us; at 192 and 256 items,
    // where the grid takes a second round, 7.9 -> 10.7 and 8.3 -> 11.1 us.
    const bool split4 = d == 64 && 2 * items <= cus;
    // d = 128, four key parts of 32-key tiles (128 KB of LDS, one per CU) when
    // they all fit at once (at most a quarter of a 128-row item per CU):
    // 32/8 heads x 128 tokens 6.3 -> 5.9 us, 8/2 heads x 512 10.0 -> 8.3 us.
    const bool split4_128 = d == 128 && 4 * items <= cus;
    auto grid_of = [&](int n_tiles) {
        return dim3((unsigned)(((long)n_tiles * B * Hq + kXcds - 1) / kXcds * kXcds));
    };
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *qr = (uint16_t *)q_rot;
    const int nqt64 = (Nq + 63) / 64;
    if (d == 128 && split4_128) {
        const int nqt32 = (Nq + 31) / 32;
        hipLaunchKernelGGL((fwd_mfma_kernel<128, 4, 32, OBF, ROPE, STR>), grid_of(nqt32), dim3(256), 0, st, qq, kk,
                           vv, o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt32, qr, rope_lb, L);
    } else if (d == 128 && !split) {
        hipLaunchKernelGGL((fwd_mfma_kernel<128, 1, kBN, OBF, ROPE, STR>), grid_of(nqt), dim3(256), 0, st, qq, kk, vv,
                           o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt, qr, rope_lb, L);
    } else if (d == 128) {
        hipLaunchKernelGGL((fwd_mfma_kernel<128, 2, kBN, OBF, ROPE, STR>), grid_of(nqt64), dim3(256), 0, st, qq, kk,
                           vv, o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt64, qr, rope_lb, L);
    } else if (d == 64 && !split) {
        hipLaunchKernelGGL((fwd_mfma_kernel<64, 1, kBN, OBF, ROPE, STR>), grid_of(nqt), dim3(256), 0, st, qq, kk, vv,
                           o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt, qr, rope_lb, L);
    } else if (d == 64 && split4) {
        const int nqt32 = (Nq + 31) / 32;
        hipLaunchKernelGGL((fwd_mfma_kernel<64, 4, 32, OBF, ROPE, STR>), grid_of(nqt32), dim3(256), 0, st, qq, kk, vv,
                           o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt32, qr, rope_lb, L);
    } else if (d == 64) {
        hipLaunchKernelGGL((fwd_mfma_kernel<64, 2, 32, OBF, ROPE, STR>), grid_of(nqt64), dim3(256), 0, st, qq, kk, vv,
                           o, lse, B, Hq, Hkv, Nq, Nk, scale, causal, nqt64, qr, rope_lb, L);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t fwd_mfma(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    const void *q, const void *k, const void *v, void *o, float *lse,
                    hipStream_t st, bool o_bf16)
{
    const Layouts none{};
    if (o_bf16)
        return fwd_mfma_launch<true, false, false>(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse,
                                                   st, nullptr, 0.0, none);
    return fwd_mfma_launch<false, false, false>(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, st,
                                                nullptr, 0.0, none);
}

hipError_t fwd_mfma_rope_q(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           const void *q, const void *k, const void *v, void *q_rot, float *o,
                           float *lse, double rope_lb, hipStream_t st)
{
    return fwd_mfma_launch<false, true, false>(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, st,
                                               q_rot, rope_lb, Layouts{});
}

hipError_t fwd_mfma_strided(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                            const void *q, const void *k, const void *v, void *o, float *lse,
                            const Layouts &L, hipStream_t st, bool o_bf16)
{
    if (o_bf16)
        return fwd_mfma_launch<true, false, true>(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, st,
                                                  nullptr, 0.0, L);
    return fwd_mfma_launch<false, false, true>(B, Hq, Hkv, Nq, Nk, d, causal, scale, q, k, v, o, lse, st,
                                               nullptr, 0.0, L);
}

}  // namespace attn
