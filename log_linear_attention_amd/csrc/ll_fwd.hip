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
// Kernels, all on the caller's stream:
//  A  ll_group_state: for every group of G = 2^g consecutive chunks that can
//     precede another group, the group's state decayed to its end
//     (sum exp(decay) k v^T, fp32, dk x dv) and its total log-decay.  MFMA,
//     with the next chunk's k/v prefetched into registers.
//  B  ll_left_tree: the left-child block states of the binary tree over
//     groups, 64 leaves per thread in registers (one launch per 64x of tree
//     height), written in the exact register order the consuming MFMA reads.
//  C  ll_chunk_walk: one workgroup per (head, group) walks its G chunks in
//     order.  Per chunk it computes the intra-chunk part
//     (Q K^T ⊙ decay ⊙ lambda-level mask) V on MFMA, adds the levels inside
//     the group from a Fenwick stack of chunk states held in registers (the
//     recurrent decode rule applied at chunk granularity), adds the levels
//     above the group from B's block states, writes the output rows, and
//     folds the chunk's own state K^T diag(w) V into the stack.  The next
//     chunk's q/k/v/lambda/a are loaded into registers while the current one
//     computes.
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
    static constexpr int WPE = 1;                 // resident waves per SIMD the walk is built for
    static constexpr int NRES = DT::is_bf16 ? 4 : 2;  // inter-group levels kept in registers per group
    static constexpr int NMT = C / 16;           // 16-row tiles per chunk
    static constexpr int NCT = NMT * (NMT + 1) / 2;  // causal 16x16 score tiles
    static constexpr int CP = (C < KB) ? KB : C; // chunk contraction length (zero padded)
    static constexpr int NUC = CP / KB;          // units over chunk tokens
    static constexpr int NUK = DK / KB;          // units over dk
    static constexpr int NDT = DK / 16;          // accumulator tiles over dk rows
    static constexpr int PADE = DT::is_bf16 ? 8 : 4;
    static constexpr int LDK = DK + PADE;        // LDS row stride of Q, K tiles
    static constexpr int LDC = CP + PADE;        // LDS row stride of K^T, V^T, P tiles
    static constexpr int VEC = 16 / (int)sizeof(T);
    // register prefetch of one chunk
    static constexpr int QVEC = C * (DK / VEC);              // 16-byte vectors of a q (or k) chunk
    static constexpr int NQ = (QVEC + NT - 1) / NT;
    static constexpr int KPAIR = (C / 2) * (DK / VEC);       // k row-pair vectors
    static constexpr int NKP = (KPAIR + NT - 1) / NT;
    static constexpr int VPAIR = (C / 2) * (DV / VEC);       // v row-pair vectors
    static constexpr int NVP = (VPAIR + NT - 1) / NT;
    static constexpr int NLAM = (C * kMaxLevels + NT - 1) / NT;
    static_assert(DK % KB == 0, "dk must be a multiple of the MFMA unit");
    static_assert(DV % 16 == 0 && DV <= 128, "dv must be 16..128 in steps of 16");
    static_assert(C <= 64, "the decay scan handles at most one wave of tokens");
};

template <class F>
struct alignas(16) WalkSmem {
    using T = typename F::T;
    T Qs[F::C * F::LDK];
    T Ks[F::C * F::LDK];
    T Kts[F::DK * F::LDC];
    T Vts[F::DV * F::LDC];
    float lam[F::C * kMaxLevels];
    float Aloc[F::C];
    float off[32];          // log-decay from each inter-group block's end to the group start
    size_t blk[32];         // element offset of each inter-group block state
    int plist[32];          // set bits of the group index, low to high
    int npop;
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
// Shared device pieces.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint4 zero16() { return make_uint4(0, 0, 0, 0); }

// Zero a whole LDS array (used once per workgroup).
template <class F, class E>
__device__ __forceinline__ void lds_zero(E *dst, int n, int tid)
{
    for (int i = tid; i < n; i += F::NT)
        dst[i] = E(0.f);
}

// Inclusive within-chunk cumulative log-decay of wave 0's `x` (lane i holds
// a at token i of the chunk, 0 past the end): Aloc[i] = sum_{r<=i} a_r, and
// the chunk total.
template <class F>
__device__ __forceinline__ void scan_decay(float x, float *Aloc, float *gch, int tid)
{
    if (tid < 64) {
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

// Store a pair of rows j, j+1 (given as two 16-byte vectors of VEC elements
// starting at column c*VEC) transposed into dst[col][j], optionally scaled.
template <class F>
__device__ __forceinline__ void store_pair_t(typename F::T *dst, const uint4 &x0, const uint4 &x1, int j, int c,
                                             float w0, float w1, bool scale)
{
    using T = typename F::T;
    const T *e0 = reinterpret_cast<const T *>(&x0);
    const T *e1 = reinterpret_cast<const T *>(&x1);
#pragma unroll
    for (int x = 0; x < F::VEC; ++x) {
        T p0 = e0[x], p1 = e1[x];
        if (scale) {
            p0 = from_f32<T>(to_f32(e0[x]) * w0);
            p1 = from_f32<T>(to_f32(e1[x]) * w1);
        }
        T *d = dst + (c * F::VEC + x) * F::LDC + j;
        d[0] = p0;
        d[1] = p1;
    }
}

// K^T (row-major LDS K tile, scaled per token by w_j = exp(g - Aloc[j]))
// into the transposed tile Kts.
template <class F>
__device__ __forceinline__ void stage_kt_from_lds(typename F::T *Kts, const typename F::T *Ks, const float *Aloc,
                                                  float gch, int tid)
{
    constexpr int VPR = F::DK / F::VEC;
    for (int idx = tid; idx < F::KPAIR; idx += F::NT) {
        const int j = 2 * (idx / VPR), c = idx % VPR;
        const uint4 x0 = *reinterpret_cast<const uint4 *>(Ks + j * F::LDK + c * F::VEC);
        const uint4 x1 = *reinterpret_cast<const uint4 *>(Ks + (j + 1) * F::LDK + c * F::VEC);
        store_pair_t<F>(Kts, x0, x1, j, c, __expf(gch - Aloc[j]), __expf(gch - Aloc[j + 1]), true);
    }
}

// Unpack a B-operand fragment of unit u back into fp32 accumulator tiles,
// adding s * value (inverse of acc_frag).
__device__ __forceinline__ void frag_axpy(floatx4 *tiles, const floatx4 &f, int u, float s, TF32)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
        tiles[u][e] += s * f[e];
}

__device__ __forceinline__ void frag_axpy(floatx4 *tiles, const bf16x8 &f, int u, float s, TBF16)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        tiles[2 * u][e] += s * (float)f[e];
        tiles[2 * u + 1][e] += s * (float)f[e + 4];
    }
}

// ---------------------------------------------------------------------------
// Kernel A: group states.
// ---------------------------------------------------------------------------
template <class F>
struct StateRegs {
    uint4 k0[F::NKP], k1[F::NKP], v0[F::NVP], v1[F::NVP];
    float a;
};

template <class F>
__device__ __forceinline__ void state_load(StateRegs<F> &r, const typename F::T *k, const typename F::T *v,
                                           const float *a, size_t row0, int tid)
{
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NKP; ++i) {
        const int idx = tid + i * F::NT;
        const int j = 2 * (idx / KPR), c = idx % KPR;
        r.k0[i] = r.k1[i] = zero16();
        if (idx < F::KPAIR) {
            r.k0[i] = *reinterpret_cast<const uint4 *>(k + (row0 + j) * F::DK + c * F::VEC);
            r.k1[i] = *reinterpret_cast<const uint4 *>(k + (row0 + j + 1) * F::DK + c * F::VEC);
        }
    }
#pragma unroll
    for (int i = 0; i < F::NVP; ++i) {
        const int idx = tid + i * F::NT;
        const int j = 2 * (idx / VPR), c = idx % VPR;
        r.v0[i] = r.v1[i] = zero16();
        if (idx < F::VPAIR) {
            r.v0[i] = *reinterpret_cast<const uint4 *>(v + (row0 + j) * F::DV + c * F::VEC);
            r.v1[i] = *reinterpret_cast<const uint4 *>(v + (row0 + j + 1) * F::DV + c * F::VEC);
        }
    }
    r.a = (tid < F::C) ? a[row0 + tid] : 0.f;
}

template <class F>
__global__ __launch_bounds__(F::NT) void ll_group_state(const typename F::T *__restrict__ k,
                                                        const typename F::T *__restrict__ v,
                                                        const float *__restrict__ a, int Tlen, int g, int nG,
                                                        int nL, float *__restrict__ Sg, float *__restrict__ Gam)
{
    __shared__ StateSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int bh = blockIdx.x / nL, sg = blockIdx.x % nL;
    const int G = 1 << g;
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;

    lds_zero<F>(sm.Kts, F::DK * F::LDC, tid);
    lds_zero<F>(sm.Vts, F::DV * F::LDC, tid);

    floatx4 S[F::NDT];
#pragma unroll
    for (int rt = 0; rt < F::NDT; ++rt)
        S[rt] = zero4();
    float gsum = 0.f;

    StateRegs<F> pf;
    state_load<F>(pf, k, v, a, (size_t)bh * Tlen + (size_t)sg * G * F::C, tid);
    for (int ci = 0; ci < G; ++ci) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < F::NVP; ++i) {
            const int idx = tid + i * F::NT;
            if (idx < F::VPAIR)
                store_pair_t<F>(sm.Vts, pf.v0[i], pf.v1[i], 2 * (idx / VPR), idx % VPR, 1.f, 1.f, false);
        }
        scan_decay<F>(pf.a, sm.Aloc, &sm.gch, tid);
        __syncthreads();
        const float gch = sm.gch;
#pragma unroll
        for (int i = 0; i < F::NKP; ++i) {
            const int idx = tid + i * F::NT;
            if (idx < F::KPAIR) {
                const int j = 2 * (idx / KPR);
                store_pair_t<F>(sm.Kts, pf.k0[i], pf.k1[i], j, idx % KPR, __expf(gch - sm.Aloc[j]),
                                __expf(gch - sm.Aloc[j + 1]), true);
            }
        }
        if (ci + 1 < G)
            state_load<F>(pf, k, v, a, (size_t)bh * Tlen + ((size_t)sg * G + ci + 1) * F::C, tid);
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
// Kernel B: left-child block states of the tree over groups.
//
// Leaves are states of consecutive blocks at level p0 (groups for p0 = 0,
// blocks of 64 groups for p0 = 6, ...), each with its total log-decay.  One
// thread owns one state element of one tile of 64 leaves; it loads the 64
// leaves into registers, builds the six tree levels above them in registers
// (merge: exp(decay of the right half) * left + right), writes every
// complete left child in MFMA B-operand order, and the tile total for the
// next launch.  A block J at level p is complete when it ends at or before
// the last complete group: (J + 1) * 2^p <= nL.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(256) void ll_left_tree(const float *__restrict__ leaves,
                                                    const float *__restrict__ gleaves, int nleaves, int lstride,
                                                    int gstride, int p0, int nL, int nLeft,
                                                    typename F::T *__restrict__ Dg, float *__restrict__ tot,
                                                    float *__restrict__ gtot, int tstride)
{
    using T = typename F::T;
    constexpr int DKV = F::DK * F::DV;
    __shared__ float gsh[64];
    const int tid = threadIdx.x;
    const int elem = blockIdx.x * 256 + tid;
    const int tile = blockIdx.y, bh = blockIdx.z;
    const int base = tile * 64;
    if (tid < 64)
        gsh[tid] = (base + tid < nleaves) ? gleaves[(size_t)bh * gstride + base + tid] : 0.f;
    float x[64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
        x[i] = (base + i < nleaves && elem < DKV) ? leaves[((size_t)bh * lstride + base + i) * DKV + elem] : 0.f;
    __syncthreads();
    if (elem >= DKV)
        return;
    float G[64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
        G[i] = gsh[i];

    // Where this element sits inside a block state stored in B-operand order.
    const int d = elem / F::DV, c = elem % F::DV;
    const int u = d / F::KB, r = d % F::KB;
    const int e = 4 * (r >> 4) + (r & 3), qd = (r & 15) >> 2;
    const int fv = ((c >> 4) * F::NUK + u) * 64 + qd * 16 + (c & 15);
    const size_t frag_off = (size_t)fv * F::EPL + e;

    size_t offp = 0;  // first left block of level p0 + lv for this head
    for (int pp = 0; pp < p0; ++pp)
        offp += ((nL >> pp) + 1) >> 1;
#pragma unroll
    for (int lv = 0; lv < 6; ++lv) {
        const int p = p0 + lv;
        const int width = 64 >> lv;
        const int J0 = base >> lv;
#pragma unroll
        for (int j = 0; j < width; ++j) {
            const int J = J0 + j;
            if (((J & 1) == 0) && ((int64_t)(J + 1) << p) <= nL)
                Dg[((size_t)bh * nLeft + offp + (J >> 1)) * DKV + frag_off] = from_f32<T>(x[j]);
        }
        offp += ((nL >> p) + 1) >> 1;
#pragma unroll
        for (int j = 0; j < width / 2; ++j) {
            x[j] = __expf(G[2 * j + 1]) * x[2 * j] + x[2 * j + 1];
            G[j] = G[2 * j] + G[2 * j + 1];
        }
    }
    if (base + 64 <= nleaves && tot != nullptr) {
        tot[((size_t)bh * tstride + tile) * DKV + elem] = x[0];
        if (elem == 0)
            gtot[(size_t)bh * tstride + tile] = G[0];
    }
}

// ---------------------------------------------------------------------------
// Kernel C: the chunk walk.
// ---------------------------------------------------------------------------
template <class F>
struct WalkRegs {
    uint4 q[F::NQ], k[F::NQ], v0[F::NVP], v1[F::NVP];
    float lam[F::NLAM];
    float a;
};

template <class F>
__device__ __forceinline__ void walk_load(WalkRegs<F> &r, const typename F::T *q, const typename F::T *k,
                                          const typename F::T *v, const float *a, const float *lam, size_t row0,
                                          int valid, int L, int tid)
{
    constexpr int QPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NQ; ++i) {
        const int idx = tid + i * F::NT;
        const int j = idx / QPR, c = idx % QPR;
        r.q[i] = r.k[i] = zero16();
        if (idx < F::QVEC && j < valid) {
            r.q[i] = *reinterpret_cast<const uint4 *>(q + (row0 + j) * F::DK + c * F::VEC);
            r.k[i] = *reinterpret_cast<const uint4 *>(k + (row0 + j) * F::DK + c * F::VEC);
        }
    }
#pragma unroll
    for (int i = 0; i < F::NVP; ++i) {
        const int idx = tid + i * F::NT;
        const int j = 2 * (idx / VPR), c = idx % VPR;
        r.v0[i] = r.v1[i] = zero16();
        if (idx < F::VPAIR && j < valid)
            r.v0[i] = *reinterpret_cast<const uint4 *>(v + (row0 + j) * F::DV + c * F::VEC);
        if (idx < F::VPAIR && j + 1 < valid)
            r.v1[i] = *reinterpret_cast<const uint4 *>(v + (row0 + j + 1) * F::DV + c * F::VEC);
    }
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        const int j = idx / kMaxLevels, l = idx % kMaxLevels;
        r.lam[i] = (idx < F::C * kMaxLevels && j < valid && l < L) ? lam[(row0 + j) * L + l] : 0.f;
    }
    r.a = (tid < valid) ? a[row0 + tid] : 0.f;
}

template <class F>
__device__ __forceinline__ void walk_store(const WalkRegs<F> &r, WalkSmem<F> &sm, int tid)
{
    constexpr int QPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NQ; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::QVEC) {
            const int j = idx / QPR, c = idx % QPR;
            *reinterpret_cast<uint4 *>(sm.Qs + j * F::LDK + c * F::VEC) = r.q[i];
            *reinterpret_cast<uint4 *>(sm.Ks + j * F::LDK + c * F::VEC) = r.k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < F::NVP; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::VPAIR)
            store_pair_t<F>(sm.Vts, r.v0[i], r.v1[i], 2 * (idx / VPR), idx % VPR, 1.f, 1.f, false);
    }
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::C * kMaxLevels)
            sm.lam[idx] = r.lam[i];
    }
    scan_decay<F>(r.a, sm.Aloc, &sm.gch, tid);
}

// The walk works in transposed form: it forms S^T = K Q^T, so the masked
// tiles P^T are already in the register layout the B operand of
// O^T = V^T P^T needs (no LDS round trip for P), and every level adds
// D^T Q^T with the same Q^T fragments, which each wave loads from LDS once
// per chunk.  A wave owns 16 rows of O^T (16 output columns) and all query
// rows of the chunk; the per-query factors then vary along the accumulator's
// column, one value per lane and tile.

// O^T += (D^T Q^T) * f, f_i = lambda[i, lev] * exp(Aloc[i] + base), for one
// level whose state D is given as fragments (B operand of Q D, which is the
// A operand of D^T Q^T).
template <class F>
__device__ __forceinline__ void level_update(floatx4 *O, const typename F::Frag (*qf)[F::NUK],
                                             const typename F::Frag *d, const float *lam_s, const float *ai,
                                             int lev, float base, int li)
{
#pragma unroll
    for (int it = 0; it < F::NMT; ++it) {
        floatx4 tmp = zero4();
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            mma_unit(tmp, d[u], qf[it][u]);
        const int i = 16 * it + li;
        const float f = lam_s[i * kMaxLevels + lev] * __expf(ai[it] + base);
        O[it] += f * tmp;
    }
}

template <class F>
__global__ __launch_bounds__(F::NT, F::WPE) void ll_chunk_walk(
    const typename F::T *__restrict__ q, const typename F::T *__restrict__ k, const typename F::T *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, typename F::T *__restrict__ out, int Tlen, int L,
    int log2C, int g, int N, int nG, int Plev, int nL, int nLeft, const float *__restrict__ Gam,
    const typename F::T *__restrict__ Dg)
{
    using T = typename F::T;
    using Frag = typename F::Frag;
    using DTag = typename F::DTag;
    constexpr int NJT = F::CP / 16;  // key tiles covered by the PV units (zero padded past C)
    __shared__ WalkSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int bh = blockIdx.x / nG, sg = blockIdx.x % nG;
    const int G = 1 << g;
    const int nchunk = min(G, N - sg * G);

    WalkRegs<F> pf;
    walk_load<F>(pf, q, k, v, a, lam, (size_t)bh * Tlen + (size_t)sg * G * F::C,
                 min(F::C, Tlen - sg * G * F::C), L, tid);

    lds_zero<F>(sm.Kts, F::DK * F::LDC, tid);
    lds_zero<F>(sm.Vts, F::DV * F::LDC, tid);
    if (tid == 0) {
        int n = 0;
        size_t off = 0;
        for (int p = 0; p < Plev; ++p) {
            if ((sg >> p) & 1) {
                sm.plist[n] = p;
                sm.blk[n] = ((size_t)bh * nLeft + off + (sg >> (p + 1))) * F::DK * F::DV;
                ++n;
            }
            off += ((nL >> p) + 1) >> 1;
        }
        sm.npop = n;
    }
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

    __syncthreads();
    const int npop = sm.npop;
    // The first NRES inter-group levels stay in registers for the whole
    // group; further levels stream from L2.
    Frag bres[F::NRES][F::NUK];
#pragma unroll
    for (int ii = 0; ii < F::NRES; ++ii)
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            bres[ii][u] = (ii < npop)
                ? *reinterpret_cast<const Frag *>(Dg + sm.blk[ii] + ((size_t)(w * F::NUK + u) * 64 + lane) * F::EPL)
                : Frag{};

    // Fenwick stack of the levels inside the group, in fragment form.  Slot
    // m holds the bucket of bit m of the local chunk index, decayed to its own
    // end; gap[m] is the log-decay from that end to the current chunk start.
    Frag stk[kMaxGroupLog2][F::NUK];
    float gap[kMaxGroupLog2];
#pragma unroll
    for (int m = 0; m < kMaxGroupLog2; ++m) {
        gap[m] = 0.f;
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            stk[m][u] = Frag{};
    }
    float agrun = 0.f;  // log-decay from the group start to the current chunk start

    for (int ci = 0; ci < nchunk; ++ci) {
        const int t0 = (sg * G + ci) * F::C;
        const int valid = min(F::C, Tlen - t0);
        const size_t row0 = (size_t)bh * Tlen + t0;
        __syncthreads();
        walk_store<F>(pf, sm, tid);
        if (ci + 1 < nchunk)
            walk_load<F>(pf, q, k, v, a, lam, row0 + F::C, min(F::C, Tlen - t0 - F::C), L, tid);
        __syncthreads();
        const float gch = sm.gch;
        stage_kt_from_lds<F>(sm.Kts, sm.Ks, sm.Aloc, gch, tid);

        // Fragments reused for the whole chunk: Q^T (B operand, every query
        // tile), V^T (A operand of the PV product, this wave's columns), and
        // the decay of this lane's query rows.
        Frag qf[F::NMT][F::NUK];
        float ai[F::NMT];
#pragma unroll
        for (int it = 0; it < F::NMT; ++it) {
            ai[it] = sm.Aloc[16 * it + li];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                qf[it][u] = lds_frag(sm.Qs, F::LDK, 16 * it + li, u * F::KB, qd);
        }
        Frag vf[F::NUC];
#pragma unroll
        for (int u = 0; u < F::NUC; ++u)
            vf[u] = lds_frag(sm.Vts, F::LDC, 16 * w + li, u * F::KB, qd);

        // Intra-chunk: P^T tiles (key tile jt, query tile it), jt <= it.
        floatx4 pt[F::NMT][NJT];
#pragma unroll
        for (int it = 0; it < F::NMT; ++it)
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt)
                pt[it][jt] = zero4();
#pragma unroll
        for (int jt = 0; jt < F::NMT; ++jt) {
            Frag kf[F::NUK];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                kf[u] = lds_frag(sm.Ks, F::LDK, 16 * jt + li, u * F::KB, qd);
            float aj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                aj[r] = sm.Aloc[16 * jt + 4 * qd + r];
#pragma unroll
            for (int it = jt; it < F::NMT; ++it) {
                floatx4 s = zero4();
#pragma unroll
                for (int u = 0; u < F::NUK; ++u)
                    mma_unit(s, kf[u], qf[it][u]);
                const int i = 16 * it + li;
                if (jt < it) {
                    // every key of the tile sits in one bucket of query i
                    const float lm = sm.lam[i * kMaxLevels + 4 + bitlen_u32((uint32_t)(it ^ jt))];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pt[it][jt][r] = s[r] * __expf(ai[it] - aj[r]) * lm;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * jt + 4 * qd + r;
                        float m = 0.f;
                        if (j <= i) {
                            const int lev = (i == j) ? 0 : bitlen_u32((uint32_t)(i ^ j));
                            m = __expf(ai[it] - aj[r]) * sm.lam[i * kMaxLevels + lev];
                        }
                        pt[it][jt][r] = s[r] * m;
                    }
                }
            }
        }

        // O^T = V^T P^T for this wave's 16 output columns.
        floatx4 O[F::NMT];
#pragma unroll
        for (int it = 0; it < F::NMT; ++it) {
            O[it] = zero4();
#pragma unroll
            for (int u = 0; u < F::NUC; ++u)
                if (u * F::KB <= 16 * it + 15)
                    mma_unit(O[it], vf[u], acc_frag(pt[it], u, DTag{}));
        }

        // Levels inside the group.
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m)
            if (m < g && ((ci >> m) & 1))
                level_update<F>(O, qf, stk[m], sm.lam, ai, log2C + m + 1, gap[m], li);

        // Levels above the group.
#pragma unroll
        for (int ii = 0; ii < F::NRES; ++ii)
            if (ii < npop) {
                const int p = sm.plist[ii];
                level_update<F>(O, qf, bres[ii], sm.lam, ai, log2C + g + 1 + p, agrun + sm.off[p], li);
            }
        for (int ii = F::NRES; ii < npop; ++ii) {
            Frag bcur[F::NUK];
            const T *blk = Dg + sm.blk[ii];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                bcur[u] = *reinterpret_cast<const Frag *>(blk + ((size_t)(w * F::NUK + u) * 64 + lane) * F::EPL);
            const int p = sm.plist[ii];
            level_update<F>(O, qf, bcur, sm.lam, ai, log2C + g + 1 + p, agrun + sm.off[p], li);
        }

        // Output: lane holds O[i][16w + 4qd .. 16w + 4qd + 3] for i = 16it + li.
#pragma unroll
        for (int it = 0; it < F::NMT; ++it) {
            const int i = 16 * it + li;
            if (i < valid) {
                T vals[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vals[r] = from_f32<T>(O[it][r]);
                T *dst = out + (row0 + i) * F::DV + 16 * w + 4 * qd;
                if constexpr (sizeof(T) == 2)
                    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(vals);
                else
                    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(vals);
            }
        }

        // Fold this chunk's state into the stack (Fenwick carry on ci + 1):
        // slots below the lowest zero bit of ci merge with it into slot kc.
        if (ci + 1 < nchunk) {
            __syncthreads();  // K^T staged by every wave
            floatx4 Hn[F::NDT];
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt) {
                Hn[rt] = zero4();
#pragma unroll
                for (int u = 0; u < F::NUC; ++u)
                    mma_unit(Hn[rt], lds_frag(sm.Kts, F::LDC, 16 * rt + li, u * F::KB, qd), vf[u]);
            }
            const int kc = __builtin_ctz((unsigned)(ci + 1));
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m) {
                gap[m] += gch;
                if (m < kc) {
                    const float s = __expf(gap[m]);
#pragma unroll
                    for (int u = 0; u < F::NUK; ++u)
                        frag_axpy(Hn, stk[m][u], u, s, DTag{});
                }
            }
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
                if (m == kc) {
#pragma unroll
                    for (int u = 0; u < F::NUK; ++u)
                        stk[m][u] = acc_frag(Hn, u, DTag{});
                    gap[m] = 0.f;
                }
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
        // Largest group that still gives two resident workgroups per CU.
        g = 0;
        while (g < kMaxGroupLog2 && (2 << g) <= p.N && BH * ((p.N + (2 << g) - 1) / (2 << g)) >= 512)
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
    const size_t ntile = (size_t)(p.nL + 63) / 64;
    p.off_Sg = 0;
    p.off_Gam = align256(p.off_Sg + (size_t)BH * p.nL * state * 4);
    p.off_Dg = align256(p.off_Gam + (size_t)BH * p.nG * 4);
    p.off_tot = align256(p.off_Dg + (size_t)BH * p.nLeft * state * elem_bytes);
    p.off_gtot = align256(p.off_tot + 2 * (size_t)BH * ntile * state * 4);
    p.bytes = (p.nL > 0) ? align256(p.off_gtot + 2 * (size_t)BH * ntile * 4) : 0;
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
        // Tree over groups, 64 leaves per tile and six levels per launch.
        const size_t ntile_max = (size_t)(P.nL + 63) / 64;
        float *tot[2] = {reinterpret_cast<float *>(ws + P.off_tot),
                         reinterpret_cast<float *>(ws + P.off_tot) + (size_t)BH * ntile_max * F::DK * F::DV};
        float *gtot[2] = {reinterpret_cast<float *>(ws + P.off_gtot),
                          reinterpret_cast<float *>(ws + P.off_gtot) + (size_t)BH * ntile_max};
        const float *leaves = Sg, *gleaves = Gam;
        int nleaves = P.nL, lstride = P.nL, gstride = P.nG, p0 = 0, ping = 0;
        while (nleaves > 0) {
            const int ntiles = (nleaves + 63) / 64;
            const int complete = nleaves / 64;
            prof_before("ll_left_tree", s);
            hipLaunchKernelGGL(ll_left_tree<F>, dim3((F::DK * F::DV + 255) / 256, ntiles, BH), dim3(256), 0, s,
                               leaves, gleaves, nleaves, lstride, gstride, p0, P.nL, P.nLeft, Dg,
                               complete > 0 ? tot[ping] : nullptr, gtot[ping], ntiles);
            prof_after(s);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            if (complete == 0)
                break;
            leaves = tot[ping];
            gleaves = gtot[ping];
            lstride = gstride = ntiles;
            nleaves = complete;
            p0 += 6;
            ping ^= 1;
        }
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
