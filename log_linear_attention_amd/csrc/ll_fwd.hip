// Chunkwise forward of log-linear attention (Mamba-2 form) for gfx950.
//
// The pages describe the parallel form as a chunk scan: dense work inside a
// chunk and hierarchical state passing between chunks, O(T log T) overall and
// rich in matrix products ("Log-Linear Attention", Portuguese page §2 "Forma
// Recorrente e Paralela", training bullet; French page §2 "Algorithmes
// Efficaces", training bullet), with custom kernels for the intra- and
// inter-chunk parts (Portuguese page §5, limitations).  Their kernel fuses
// levels to cut memory traffic and launches on another GPU (French page §3);
// this design keeps that goal and maps it to CDNA4 as follows.
//
// Chunk algebra.  With chunks of C tokens, a key in an earlier chunk c' is at
// level log2(C) + bit_length(c XOR c') from any query of chunk c, so the
// levels above log2(C) are a Fenwick tree over chunk indices: chunk c reads,
// for each set bit m-1 of c, the decayed state sum k v^T of the left block of
// 2^(m-1) chunks just below that bit.
//
// Three kernels, all on the caller's stream:
//  A  ll_group_state: for every group of G = 2^g consecutive chunks that can
//     precede another group, the group's state decayed to its end
//     (sum exp(decay) k v^T, fp32, dk x dv) and its total log-decay.  MFMA.
//  B  ll_left_blocks: from those, every left-child block state of the tree
//     over groups, stored in the exact register order the consuming MFMA
//     reads (bf16 or fp32).  Memory-bound, VALU.
//  C  ll_chunk_walk: one workgroup per (head, group) walks its G chunks in
//     order.  Per chunk it computes the intra-chunk part
//     (Q K^T ⊙ decay ⊙ lambda-level mask) V on MFMA, adds the levels inside
//     the group from a Fenwick stack of chunk states held in registers (the
//     recurrent decode rule applied at chunk granularity), adds the levels
//     above the group from B's block states, writes the output rows, and
//     folds the chunk's own state K^T diag(w) V into the stack.
// Nothing but the inputs, the output and the small group/block states touches
// HBM; the per-chunk states of the levels inside a group never leave
// registers.
#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

template <class DT, int DK_, int DV_, int C_>
struct Fwd {
    using T = typename DT::T;
    using Frag = typename DT::Frag;
    using DTag = DT;
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr int KB = DT::KB, EPL = DT::EPL;
    static constexpr int NW = DV / 16;           // waves: one 16-column slice of dv each
    static constexpr int NT = 64 * NW;
    static constexpr int NMT = C / 16;           // 16-row tiles per chunk
    static constexpr int CP = (C < KB) ? KB : C; // chunk contraction length (zero padded)
    static constexpr int NUC = CP / KB;          // units over chunk tokens
    static constexpr int NUK = DK / KB;          // units over dk
    static constexpr int NDT = DK / 16;          // accumulator tiles over dk rows
    static constexpr int PADE = DT::is_bf16 ? 8 : 4;
    static constexpr int LDK = DK + PADE;        // LDS row stride of Q, K tiles
    static constexpr int LDC = CP + PADE;        // LDS row stride of K^T, V^T, P tiles
    static constexpr int VEC = 16 / (int)sizeof(T);
    static_assert(DK % KB == 0, "dk must be a multiple of the MFMA unit");
    static_assert(DV % 16 == 0 && DV <= 128, "dv must be 16..128 in steps of 16");
    static_assert(C <= 64, "chunk scan handles at most one wave of tokens");
};

template <class F>
struct alignas(16) WalkSmem {
    using T = typename F::T;
    T Qs[F::C * F::LDK];
    T Ks[F::C * F::LDK];
    T Kts[F::DK * F::LDC];
    T Vts[F::DV * F::LDC];
    T Ps[F::C * F::LDC];
    float lam[F::C * kMaxLevels];
    float Aloc[F::C];
    float off[32];
    float gch;
};

template <class F>
struct alignas(16) StateSmem {
    using T = typename F::T;
    T Kts[F::DK * F::LDC];
    T Vts[F::DV * F::LDC];
    float Aloc[F::C];
    float gch;
};

// ---------------------------------------------------------------------------
// Staging helpers (all threads of the workgroup call them).
// ---------------------------------------------------------------------------

// Rows [t0, t0 + C) of a [*, D] tensor into a row-major LDS tile; rows past
// `valid` are zero.
template <class F, int D>
__device__ __forceinline__ void stage_rows(typename F::T *dst, const typename F::T *src, int valid, int tid)
{
    using T = typename F::T;
    constexpr int VPR = D / F::VEC;
    for (int idx = tid; idx < F::C * VPR; idx += F::NT) {
        const int j = idx / VPR, c = idx % VPR;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (j < valid)
            x = *reinterpret_cast<const uint4 *>(src + (size_t)j * D + c * F::VEC);
        *reinterpret_cast<uint4 *>(dst + j * F::LDK + c * F::VEC) = x;
    }
    (void)sizeof(T);
}

// Transposed staging: dst[d][j] = scale_j * src[j][d] for d < D, j < C, from
// rows with stride src_ld (global or LDS); rows past `valid` are zero.  Two
// rows at a time so each LDS store writes a pair of elements.
template <class F, int D, bool SCALE>
__device__ __forceinline__ void stage_transposed(typename F::T *dst, const typename F::T *src, int src_ld,
                                                 int valid, const float *Aloc, float gch, int tid)
{
    using T = typename F::T;
    constexpr int VPR = D / F::VEC;
    for (int idx = tid; idx < (F::C / 2) * VPR; idx += F::NT) {
        const int j = 2 * (idx / VPR), c = idx % VPR;
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        if (j < valid)
            x0 = *reinterpret_cast<const uint4 *>(src + (size_t)j * src_ld + c * F::VEC);
        if (j + 1 < valid)
            x1 = *reinterpret_cast<const uint4 *>(src + (size_t)(j + 1) * src_ld + c * F::VEC);
        const T *e0 = reinterpret_cast<const T *>(&x0);
        const T *e1 = reinterpret_cast<const T *>(&x1);
        float w0 = 1.f, w1 = 1.f;
        if (SCALE) {
            w0 = __expf(gch - Aloc[j]);
            w1 = __expf(gch - Aloc[j + 1]);
        }
#pragma unroll
        for (int x = 0; x < F::VEC; ++x) {
            T p0, p1;
            if (SCALE) {
                p0 = from_f32<T>(to_f32(e0[x]) * w0);
                p1 = from_f32<T>(to_f32(e1[x]) * w1);
            } else {
                p0 = e0[x];
                p1 = e1[x];
            }
            T *d = dst + (c * F::VEC + x) * F::LDC + j;
            d[0] = p0;
            d[1] = p1;
        }
    }
}

// Zero the padding columns [C, CP) of a transposed tile (bf16 with C < 32).
template <class F, int ROWS>
__device__ __forceinline__ void zero_pad_cols(typename F::T *dst, int tid)
{
    if constexpr (F::CP > F::C) {
        constexpr int W = F::CP - F::C;
        for (int idx = tid; idx < ROWS * W; idx += F::NT)
            dst[(idx / W) * F::LDC + F::C + idx % W] = from_f32<typename F::T>(0.f);
    }
}

// Inclusive within-chunk cumulative log-decay Aloc[i] = sum_{r=t0..t0+i} a_r
// (wave 0; tokens past `valid` contribute 0) and the chunk total.
template <class F>
__device__ __forceinline__ void stage_decay(float *Aloc, float *gch, const float *a, int valid, int tid)
{
    if (tid < 64) {
        float x = (tid < valid) ? a[tid] : 0.f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float y = __shfl_up(x, d, 64);
            if (tid >= d)
                x += y;
        }
        if (tid < F::C)
            Aloc[tid] = x;
        if (tid == F::C - 1)
            *gch = x;
    }
}

// ---------------------------------------------------------------------------
// Kernel A: group states.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(F::NT) void ll_group_state(const typename F::T *__restrict__ k,
                                                        const typename F::T *__restrict__ v,
                                                        const float *__restrict__ a, int Tlen, int g, int nG,
                                                        int nL, float *__restrict__ Sg, float *__restrict__ Gam)
{
    using T = typename F::T;
    __shared__ StateSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int bh = blockIdx.x / nL, sg = blockIdx.x % nL;
    const int G = 1 << g;

    zero_pad_cols<F, F::DK>(sm.Kts, tid);
    zero_pad_cols<F, F::DV>(sm.Vts, tid);

    floatx4 S[F::NDT];
#pragma unroll
    for (int rt = 0; rt < F::NDT; ++rt)
        S[rt] = zero4();
    float gsum = 0.f;

    for (int ci = 0; ci < G; ++ci) {
        const int t0 = (sg * G + ci) * F::C;
        const size_t row0 = (size_t)bh * Tlen + t0;
        __syncthreads();
        stage_decay<F>(sm.Aloc, &sm.gch, a + row0, F::C, tid);
        stage_transposed<F, F::DV, false>(sm.Vts, v + row0 * F::DV, F::DV, F::C, nullptr, 0.f, tid);
        __syncthreads();
        const float gch = sm.gch;
        stage_transposed<F, F::DK, true>(sm.Kts, k + row0 * F::DK, F::DK, F::C, sm.Aloc, gch, tid);
        __syncthreads();
        const float dec = __expf(gch);
#pragma unroll
        for (int rt = 0; rt < F::NDT; ++rt) {
            S[rt] *= dec;
#pragma unroll
            for (int u = 0; u < F::NUC; ++u)
                mma_unit(S[rt], lds_frag(sm.Kts, F::LDC, 16 * rt + li, u * F::KB, qd),
                         lds_frag(sm.Vts, F::LDC, 16 * w + li, u * F::KB, qd));
        }
        gsum += gch;
    }
    float *dst = Sg + ((size_t)bh * nL + sg) * F::DK * F::DV;
#pragma unroll
    for (int rt = 0; rt < F::NDT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dst[(16 * rt + 4 * qd + r) * F::DV + 16 * w + li] = S[rt][r];
    if (tid == 0)
        Gam[(size_t)bh * nG + sg] = gsum;
}

// ---------------------------------------------------------------------------
// Kernel B: left-child block states over groups, in MFMA B-operand order.
// One thread per (head, left block, 16-byte fragment).
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(256) void ll_left_blocks(const float *__restrict__ Sg, const float *__restrict__ Gam,
                                                      int BH, int nG, int nL, int nLeft,
                                                      typename F::T *__restrict__ Dg)
{
    using T = typename F::T;
    constexpr int NFV = F::DK * F::DV / F::EPL;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (size_t)BH * nLeft * NFV)
        return;
    const int fv = (int)(gid % NFV);
    const int lbg = (int)((gid / NFV) % nLeft);
    const int bh = (int)(gid / ((size_t)NFV * nLeft));
    int p = 0, lb = lbg;
    for (;;) {
        const int cnt = ((nL >> p) + 1) >> 1;
        if (lb < cnt)
            break;
        lb -= cnt;
        ++p;
    }
    const int first = (2 * lb) << p;             // first group of the block
    const int last = first + (1 << p) - 1;       // last group of the block
    const int w = fv / (F::NUK * 64), u = (fv / 64) % F::NUK, lane = fv % 64;
    const int qd = lane >> 4, col = 16 * w + (lane & 15);
    float acc[F::EPL];
#pragma unroll
    for (int e = 0; e < F::EPL; ++e)
        acc[e] = 0.f;
    float grun = 0.f;  // log-decay from the end of group gam to the end of the block
    for (int gam = last; gam >= first; --gam) {
        const float *src = Sg + ((size_t)bh * nL + gam) * F::DK * F::DV;
        const float dec = __expf(grun);
#pragma unroll
        for (int e = 0; e < F::EPL; ++e)
            acc[e] += dec * src[(u * F::KB + unit_row(e, qd)) * F::DV + col];
        grun += Gam[(size_t)bh * nG + gam];
    }
    T vals[F::EPL];
#pragma unroll
    for (int e = 0; e < F::EPL; ++e)
        vals[e] = from_f32<T>(acc[e]);
    *reinterpret_cast<uint4 *>(Dg + ((size_t)bh * nLeft + lbg) * F::DK * F::DV + (size_t)fv * F::EPL) =
        *reinterpret_cast<const uint4 *>(vals);
}

// ---------------------------------------------------------------------------
// Kernel C: the chunk walk.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(F::NT) void ll_chunk_walk(
    const typename F::T *__restrict__ q, const typename F::T *__restrict__ k, const typename F::T *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, typename F::T *__restrict__ out, int Tlen, int L,
    int log2C, int g, int N, int nG, int Plev, int nL, int nLeft, const float *__restrict__ Gam,
    const typename F::T *__restrict__ Dg)
{
    using T = typename F::T;
    using Frag = typename F::Frag;
    __shared__ WalkSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int bh = blockIdx.x / nG, sg = blockIdx.x % nG;
    const int G = 1 << g;
    const int nchunk = min(G, N - sg * G);

    zero_pad_cols<F, F::DK>(sm.Kts, tid);
    zero_pad_cols<F, F::DV>(sm.Vts, tid);
    zero_pad_cols<F, F::C>(sm.Ps, tid);

    // Log-decay from the end of each inter-group block to the start of this
    // group: the sum of the group totals strictly between them.
    if (w == 0) {
        for (int p = 0; p < Plev; ++p) {
            if (!((sg >> p) & 1))
                continue;
            const int lo = ((sg >> (p + 1)) << (p + 1)) + (1 << p);
            float s = 0.f;
            for (int gam = lo + lane; gam < sg; gam += 64)
                s += Gam[(size_t)bh * nG + gam];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1)
                s += __shfl_xor(s, d, 64);
            if (lane == 0)
                sm.off[p] = s;
        }
    }

    floatx4 stack[kMaxGroupLog2][F::NDT];
#pragma unroll
    for (int m = 0; m < kMaxGroupLog2; ++m)
#pragma unroll
        for (int rt = 0; rt < F::NDT; ++rt)
            stack[m][rt] = zero4();
    float agrun = 0.f;  // log-decay from the group start to the current chunk start

    for (int ci = 0; ci < nchunk; ++ci) {
        const int t0 = (sg * G + ci) * F::C;
        const int valid = min(F::C, Tlen - t0);
        const size_t row0 = (size_t)bh * Tlen + t0;
        __syncthreads();
        stage_rows<F, F::DK>(sm.Qs, q + row0 * F::DK, valid, tid);
        stage_rows<F, F::DK>(sm.Ks, k + row0 * F::DK, valid, tid);
        stage_transposed<F, F::DV, false>(sm.Vts, v + row0 * F::DV, F::DV, valid, nullptr, 0.f, tid);
        stage_decay<F>(sm.Aloc, &sm.gch, a + row0, valid, tid);
        for (int idx = tid; idx < F::C * kMaxLevels; idx += F::NT) {
            const int j = idx / kMaxLevels, l = idx % kMaxLevels;
            sm.lam[idx] = (j < valid && l < L) ? lam[(row0 + j) * L + l] : 0.f;
        }
        __syncthreads();
        const float gch = sm.gch;
        stage_transposed<F, F::DK, true>(sm.Kts, sm.Ks, F::LDK, valid, sm.Aloc, gch, tid);

        // Intra-chunk scores, masked by decay and the level weight.
        for (int tile = w; tile < F::NMT * F::NMT; tile += F::NW) {
            const int mt = tile / F::NMT, nt = tile % F::NMT;
            floatx4 s = zero4();
            if (nt <= mt) {
#pragma unroll
                for (int u = 0; u < F::NUK; ++u)
                    mma_unit(s, lds_frag(sm.Qs, F::LDK, 16 * mt + li, u * F::KB, qd),
                             lds_frag(sm.Ks, F::LDK, 16 * nt + li, u * F::KB, qd));
                const int j = 16 * nt + li;
                const float aj = sm.Aloc[j];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * qd + r;
                    float m = 0.f;
                    if (j <= i) {
                        const int lev = (i == j) ? 0 : bitlen_u32((uint32_t)(i ^ j));
                        m = __expf(sm.Aloc[i] - aj) * sm.lam[i * kMaxLevels + lev];
                    }
                    s[r] *= m;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.Ps[(16 * mt + 4 * qd + r) * F::LDC + 16 * nt + li] = from_f32<T>(s[r]);
        }
        __syncthreads();

        // O = P V for this wave's 16 output columns.
        floatx4 O[F::NMT];
#pragma unroll
        for (int mt = 0; mt < F::NMT; ++mt) {
            O[mt] = zero4();
#pragma unroll
            for (int u = 0; u < F::NUC; ++u)
                if (u * F::KB <= 16 * mt + 15)
                    mma_unit(O[mt], lds_frag(sm.Ps, F::LDC, 16 * mt + li, u * F::KB, qd),
                             lds_frag(sm.Vts, F::LDC, 16 * w + li, u * F::KB, qd));
        }

        // Levels inside the group: stack slot m holds the bucket of bit m of
        // ci, decayed to the end of the previous chunk.
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m) {
            if (m < g && ((ci >> m) & 1)) {
                const int lev = log2C + m + 1;
#pragma unroll
                for (int mt = 0; mt < F::NMT; ++mt) {
                    floatx4 tmp = zero4();
#pragma unroll
                    for (int u = 0; u < F::NUK; ++u)
                        mma_unit(tmp, lds_frag(sm.Qs, F::LDK, 16 * mt + li, u * F::KB, qd),
                                 acc_frag(stack[m], u, typename F::DTag{}));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * mt + 4 * qd + r;
                        O[mt][r] += sm.lam[i * kMaxLevels + lev] * __expf(sm.Aloc[i]) * tmp[r];
                    }
                }
            }
        }

        // Levels above the group: left-child block states from kernel B.
        for (int p = 0; p < Plev; ++p) {
            if (!((sg >> p) & 1))
                continue;
            int offp = 0;
            for (int pp = 0; pp < p; ++pp)
                offp += ((nL >> pp) + 1) >> 1;
            const T *blk = Dg + ((size_t)bh * nLeft + offp + (sg >> (p + 1))) * F::DK * F::DV;
            Frag bfr[F::NUK];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                bfr[u] = *reinterpret_cast<const Frag *>(blk + ((size_t)(w * F::NUK + u) * 64 + lane) * F::EPL);
            const int lev = log2C + g + 1 + p;
            const float base = agrun + sm.off[p];
#pragma unroll
            for (int mt = 0; mt < F::NMT; ++mt) {
                floatx4 tmp = zero4();
#pragma unroll
                for (int u = 0; u < F::NUK; ++u)
                    mma_unit(tmp, lds_frag(sm.Qs, F::LDK, 16 * mt + li, u * F::KB, qd), bfr[u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * mt + 4 * qd + r;
                    O[mt][r] += sm.lam[i * kMaxLevels + lev] * __expf(sm.Aloc[i] + base) * tmp[r];
                }
            }
        }

        // Output rows.
#pragma unroll
        for (int mt = 0; mt < F::NMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * qd + r;
                if (i < valid)
                    out[(row0 + i) * F::DV + 16 * w + li] = from_f32<T>(O[mt][r]);
            }

        // Fold this chunk's state into the stack (Fenwick carry on ci + 1).
        if (ci + 1 < nchunk) {
            floatx4 Hn[F::NDT];
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt) {
                Hn[rt] = zero4();
#pragma unroll
                for (int u = 0; u < F::NUC; ++u)
                    mma_unit(Hn[rt], lds_frag(sm.Kts, F::LDC, 16 * rt + li, u * F::KB, qd),
                             lds_frag(sm.Vts, F::LDC, 16 * w + li, u * F::KB, qd));
            }
            const float dec = __expf(gch);
            const int kc = __builtin_ctz((unsigned)(ci + 1));
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
#pragma unroll
                for (int rt = 0; rt < F::NDT; ++rt) {
                    stack[m][rt] *= dec;
                    if (m < kc)
                        Hn[rt] += stack[m][rt];
                }
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
                if (m == kc)
#pragma unroll
                    for (int rt = 0; rt < F::NDT; ++rt)
                        stack[m][rt] = Hn[rt];
        }
        agrun += gch;
    }
}

// ---------------------------------------------------------------------------
// Host side: plan and launch.
// ---------------------------------------------------------------------------

static int bit_length(int64_t x)
{
    int n = 0;
    while (x > 0) {
        ++n;
        x >>= 1;
    }
    return n;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FwdPlan fwd_plan(int B, int H, int T, int dk, int dv, int chunk, int group_log2, int elem_bytes)
{
    FwdPlan p;
    const int64_t BH = (int64_t)B * H;
    p.N = (T + chunk - 1) / chunk;
    int g = group_log2;
    if (g < 0) {
        // Largest group that still gives about four workgroups per CU.
        g = 0;
        while (g < kMaxGroupLog2 && (2 << g) <= p.N && BH * ((p.N + (2 << g) - 1) / (2 << g)) >= 1024)
            ++g;
    }
    if (g > kMaxGroupLog2)
        g = kMaxGroupLog2;
    p.g = g;
    p.G = 1 << g;
    p.nG = (p.N + p.G - 1) / p.G;
    p.nL = p.nG > 0 ? p.nG - 1 : 0;
    p.Plev = bit_length(p.nL);
    p.nLeft = 0;
    for (int lv = 0; lv < p.Plev; ++lv)
        p.nLeft += ((p.nL >> lv) + 1) >> 1;
    const size_t state = (size_t)dk * dv;
    p.off_Sg = 0;
    p.off_Gam = align256(p.off_Sg + (size_t)BH * p.nL * state * 4);
    p.off_Dg = align256(p.off_Gam + (size_t)BH * p.nG * 4);
    p.bytes = (p.nL > 0) ? align256(p.off_Dg + (size_t)BH * p.nLeft * state * elem_bytes) : 0;
    return p;
}

template <class F>
static hipError_t launch_fwd_t(const FwdArgs &A, const FwdPlan &P, hipStream_t s)
{
    using T = typename F::T;
    const int BH = A.B * A.H;
    char *ws = static_cast<char *>(A.workspace);
    float *Sg = reinterpret_cast<float *>(ws + P.off_Sg);
    float *Gam = reinterpret_cast<float *>(ws + P.off_Gam);
    T *Dg = reinterpret_cast<T *>(ws + P.off_Dg);
    const int log2C = bit_length(F::C) - 1;
    if (P.nL > 0) {
        prof_before("ll_group_state", s);
        hipLaunchKernelGGL(ll_group_state<F>, dim3(BH * P.nL), dim3(F::NT), 0, s, (const T *)A.k, (const T *)A.v,
                           A.a, A.T, P.g, P.nG, P.nL, Sg, Gam);
        prof_after(s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        constexpr int NFV = F::DK * F::DV / F::EPL;
        const size_t threads = (size_t)BH * P.nLeft * NFV;
        prof_before("ll_left_blocks", s);
        hipLaunchKernelGGL(ll_left_blocks<F>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                           (const float *)Sg, (const float *)Gam, BH, P.nG, P.nL, P.nLeft, Dg);
        prof_after(s);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    prof_before("ll_chunk_walk", s);
    hipLaunchKernelGGL(ll_chunk_walk<F>, dim3(BH * P.nG), dim3(F::NT), 0, s, (const T *)A.q, (const T *)A.k,
                       (const T *)A.v, A.a, A.lam, (T *)A.out, A.T, A.L, log2C, P.g, P.N, P.nG, P.Plev, P.nL,
                       P.nLeft, (const float *)Gam, (const T *)Dg);
    prof_after(s);
    return hipGetLastError();
}

typedef hipError_t (*FwdLauncher)(const FwdArgs &, const FwdPlan &, hipStream_t);

template <class DT, int DK, int DV, int C>
static FwdLauncher pick_c()
{
    if constexpr (DK % DT::KB != 0) {
        return nullptr;
    } else if constexpr (sizeof(WalkSmem<Fwd<DT, DK, DV, C>>) > 160 * 1024) {
        return nullptr;
    } else {
        return &launch_fwd_t<Fwd<DT, DK, DV, C>>;
    }
}

template <class DT, int DK, int DV>
static FwdLauncher pick_dv(int chunk)
{
    switch (chunk) {
    case 16: return pick_c<DT, DK, DV, 16>();
    case 32: return pick_c<DT, DK, DV, 32>();
    case 64: return pick_c<DT, DK, DV, 64>();
    default: return nullptr;
    }
}

template <class DT, int DK>
static FwdLauncher pick_dk(int dv, int chunk)
{
    switch (dv) {
    case 16: return pick_dv<DT, DK, 16>(chunk);
    case 32: return pick_dv<DT, DK, 32>(chunk);
    case 64: return pick_dv<DT, DK, 64>(chunk);
    case 128: return pick_dv<DT, DK, 128>(chunk);
    default: return nullptr;
    }
}

template <class DT>
static FwdLauncher pick(int dk, int dv, int chunk)
{
    switch (dk) {
    case 16: return pick_dk<DT, 16>(dv, chunk);
    case 32: return pick_dk<DT, 32>(dv, chunk);
    case 64: return pick_dk<DT, 64>(dv, chunk);
    case 128: return pick_dk<DT, 128>(dv, chunk);
    default: return nullptr;
    }
}

static FwdLauncher find_fwd(bool bf16, int dk, int dv, int chunk)
{
    return bf16 ? pick<TBF16>(dk, dv, chunk) : pick<TF32>(dk, dv, chunk);
}

bool fwd_supported(bool bf16, int dk, int dv, int chunk) { return find_fwd(bf16, dk, dv, chunk) != nullptr; }

hipError_t fwd_launch(const FwdArgs &args, const FwdPlan &plan, hipStream_t stream)
{
    FwdLauncher f = find_fwd(args.bf16, args.dk, args.dv, args.chunk);
    if (!f)
        return hipErrorInvalidValue;
    return f(args, plan, stream);
}

}  // namespace ll
