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
//     groups, 64 leaves in registers per thread (one launch per 64x of tree
//     height), written in the exact register order the consuming MFMA reads.
//  C  ll_chunk_walk: walks the chunks of a group in order.  Per chunk it
//     computes the intra-chunk part (Q K^T ⊙ decay ⊙ lambda-level mask) V on
//     MFMA, adds the levels inside the group from a Fenwick stack of chunk
//     states (the recurrent decode rule applied at chunk granularity), adds
//     the levels above the group from B's block states, writes the output
//     rows, and folds the chunk's own state K^T diag(w) V into the stack.
//     The next chunk's q/k/v/lambda/a are loaded while the current one
//     computes.  Three versions: fp32 with the stack in registers
//     (ll_chunk_walk_rs); bf16 with specialised compute and helper waves
//     (ll_chunk_walk_ws, each workgroup walking a group and its mirror);
//     and a bf16 fallback for shapes or lengths the latter does not take.
// Nothing but the inputs, the output and the small group/block states touches
// HBM; the per-chunk states of the levels inside a group stay on chip.
//
// Operands whose contraction runs over tokens (K^T and V^T) are read on the
// bf16 path straight from the row-major tiles with the CDNA4 LDS transpose
// read (ds_read_b64_tr_b16); the fp32 path has no such instruction for 32-bit
// elements and stores transposed copies instead.
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

// Row stride (in 16-bit elements) of a bf16 LDS tile with `cols` columns:
// a multiple of 8 elements (16-byte rows) chosen so that (a) the 16 lanes of
// a fragment read (rows li, 8 bytes each) and (b) the four 8-dword row
// segments of a transpose read fall in distinct banks of the 64-bank LDS.
constexpr bool stride_ok(int s, bool normal)
{
    bool used[64] = {};
    if (normal) {
        for (int li = 0; li < 16; ++li)
            for (int d = 0; d < 2; ++d) {
                const int b = (li * s + d) % 64;
                if (used[b])
                    return false;
                used[b] = true;
            }
    }
    bool used2[64] = {};
    for (int r = 0; r < 4; ++r)
        for (int d = 0; d < 8; ++d) {
            const int b = (r * s + d) % 64;
            if (used2[b])
                return false;
            used2[b] = true;
        }
    return true;
}

constexpr int bf16_stride(int cols, bool normal)
{
    int s = cols / 2;  // dwords
    while (s % 4 != 0 || !stride_ok(s, normal))
        ++s;
    return 2 * s;
}

// Row stride (in 16-bit elements) of a bf16 LDS tile read only by transpose
// reads and written by whole rows: the eight rows a half-wave's transpose
// read touches (8 dwords each) must fall in disjoint bank ranges, which
// holds when the stride in dwords is an odd multiple of 8.
constexpr int tr_stride(int cols)
{
    int s = cols / 2;
    while (s % 16 != 8)
        ++s;
    return 2 * s;
}

// Tile geometry.  SPLIT (the chunk walk) gives each 16-column slice of dv
// two waves that share the slice's state work and split the query tiles, so
// one workgroup keeps two waves per SIMD within the 256-register budget.
template <class DT, int DK_, int DV_, int C_, bool SPLIT = false>
struct Fwd {
    using T = typename DT::T;
    using Frag = typename DT::Frag;
    using DTag = DT;
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr bool TR = DT::is_bf16;          // transpose reads available
    static constexpr int KB = DT::KB, EPL = DT::EPL;
    static constexpr int NMT = C / 16;           // 16-row tiles per chunk
    static constexpr int NWC = DV / 16;          // 16-column slices of dv
    static constexpr int NH = (SPLIT && NMT >= 2 && DV <= 64) ? 2 : 1;  // waves per slice
    static constexpr int NW = NWC * NH;
    static constexpr int NT = 64 * NW;
    static constexpr int NQT = NMT / NH;         // query tiles per wave
    static constexpr int CP = (C < KB) ? KB : C; // chunk contraction length (zero padded)
    static constexpr int NUC = CP / KB;          // units over chunk tokens
    static constexpr int NUK = DK / KB;          // units over dk
    static constexpr int NDT = DK / 16;          // accumulator tiles over dk rows
    static constexpr int LDK = TR ? bf16_stride(DK, true) : DK + 4;   // Q, K row stride
    static constexpr int LDV = TR ? bf16_stride(DV, false) : DV + 4;  // V row stride
    static constexpr int LDC = CP + 4;           // fp32 transposed tiles K^T, V^T
    static constexpr int LDL = C + 1;            // lambda^T row stride
    static constexpr int VEC = 16 / (int)sizeof(T);
    // register prefetch of one chunk
    static constexpr int QVEC = C * (DK / VEC);  // 16-byte vectors of a q (or k) chunk
    static constexpr int NQ = (QVEC + NT - 1) / NT;
    static constexpr int VVEC = C * (DV / VEC);
    static constexpr int NV = (VVEC + NT - 1) / NT;
    static constexpr int NLAM = (C * kMaxLevels + NT - 1) / NT;
    // LDS bytes of everything but the resident inter-group states, and how
    // many of those states (one per level above the group) fit beside it.
    static constexpr int BASE_LDS = (int)sizeof(T) * (C * LDK + CP * LDK + (TR ? CP * LDV : 8) +
                                                       (TR ? 8 : DK * LDC) + (TR ? 8 : DV * LDC)) +
                                    4 * (kMaxLevels * LDL + C) + 1024;
    static constexpr int STATE_BYTES = DK * DV * (int)sizeof(T);
    static constexpr int NRES_FIT = (160 * 1024 - BASE_LDS) / STATE_BYTES;
    static constexpr int NRES = NRES_FIT < 0 ? 0 : (NRES_FIT > 8 ? 8 : NRES_FIT);
    // query tile x (0 .. NQT-1) of half h: pairs {0, NMT-1}, {1, NMT-2}
    // balance the causal work of the two halves.
    __device__ static constexpr int qtile(int h, int x) { return NH == 1 ? x : (x == 0 ? h : NMT - 1 - h); }
    static_assert(DK % KB == 0, "dk must be a multiple of the MFMA unit");
    static_assert(DV % 16 == 0 && DV <= 128, "dv must be 16..128 in steps of 16");
    static_assert(C <= 64, "the decay scan handles at most one wave of tokens");
    static_assert(NMT % NH == 0 && (NH == 1 || NQT <= 2), "query tiles split in pairs");
};

// Row-major q/k/v tiles (k and v padded with zero rows up to CP), lambda^T,
// and on the fp32 path the transposed copies of k and v.
template <class F>
struct alignas(16) WalkSmem {
    using T = typename F::T;
    T Qs[F::C * F::LDK];
    T Ks[F::CP * F::LDK];
    T Vs[F::TR ? F::CP * F::LDV : 8];
    T Kts[F::TR ? 8 : F::DK * F::LDC];
    T Vts[F::TR ? 8 : F::DV * F::LDC];
    float lamT[kMaxLevels * F::LDL];
    float Aloc[F::C];
    T Dres[F::NRES > 0 ? F::NRES * F::DK * F::DV : 8];  // inter-group states, fragment order
    float off[32];          // log-decay from each inter-group block's end to the group start
    size_t blk[32];         // element offset of each inter-group block state
    int plist[32];          // set bits of the group index, low to high
    int npop;
    float gch;
};

template <class F>
struct alignas(16) StateSmem {
    using T = typename F::T;
    T Ks[F::TR ? F::CP * F::LDK : 8];
    T Vs[F::TR ? F::CP * F::LDV : 8];
    T Kts[F::TR ? 8 : F::DK * F::LDC];
    T Vts[F::TR ? 8 : F::DV * F::LDC];
    float Aloc[F::C];
    float gch;
};

// ---------------------------------------------------------------------------
// Shared device pieces.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint4 zero16() { return make_uint4(0, 0, 0, 0); }

typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));

// Streaming 16-byte global access for data touched once (q, k, v, lambda in
// the chunk walk; the output rows).
__device__ __forceinline__ uint4 ld_stream(const void *p)
{
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}


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

// Paired-quad column layout of a bf16 LDS tile (used by the specialised
// walk for Q, K and P).  Inside every 32-column unit, logical column
// 16h + 4q + r is stored at 8q + 4h + r, so the two 4-element halves of a
// lane's operand fragment (columns 4q.. and 16 + 4q..) are adjacent and the
// fragment is one 16-byte read.  The contraction order is unchanged.
__device__ __forceinline__ bf16x8 pq_frag(const __bf16 *base, int ld, int row, int col0, int qd)
{
    return *reinterpret_cast<const bf16x8 *>(base + row * ld + col0 + 8 * qd);
}

// Position of the 4-column group starting at logical column 16h + 4q of a
// unit (relative to the unit start).
__device__ __forceinline__ constexpr int pq_pos(int h, int q) { return 8 * q + 4 * h; }

// Transpose-read fragment (as tr_frag) of the 16 logical columns
// 32u + 16t .. 32u + 16t + 15 of a paired-quad tile: rows jb .. jb+31.
__device__ __forceinline__ bf16x8 pq_tr_frag(const __bf16 *base, int ld, int jb, int u, int t, int li, int qd)
{
    const __bf16 *p = base + (jb + 4 * qd + (li >> 2)) * ld + 32 * u + pq_pos(t, li & 3);
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 16 * ld));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Scale the token-indexed fragment f of unit u by w_j = exp(g - Aloc[j])
// (the decay from token j to the chunk end); padding tokens j >= C get 0.
template <class F>
__device__ __forceinline__ floatx4 scale_tokens(const floatx4 &f, int u, const float *Aloc, float gch, int qd)
{
    floatx4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = u * F::KB + unit_row(e, qd);
        r[e] = (j < F::C) ? f[e] * __expf(gch - Aloc[j]) : 0.f;
    }
    return r;
}

template <class F>
__device__ __forceinline__ bf16x8 scale_tokens(const bf16x8 &f, int u, const float *Aloc, float gch, int qd)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = u * F::KB + unit_row(e, qd);
        r[e] = (__bf16)((j < F::C) ? (float)f[e] * __expf(gch - Aloc[j]) : 0.f);
    }
    return r;
}

// Fragments over tokens for the current chunk: K^T with rows d = 16*rt + li
// (A operand of the chunk state) and V with column e = 16*w + li (A operand
// of O^T = V^T P^T and B operand of the chunk state).
template <class F, class S>
__device__ __forceinline__ typename F::Frag kt_frag(const S &sm, int rt, int u, int li, int qd)
{
    if constexpr (F::TR)
        return tr_frag(sm.Ks, F::LDK, u * F::KB, 16 * rt, li, qd);
    else
        return lds_frag(sm.Kts, F::LDC, 16 * rt + li, u * F::KB, qd);
}

template <class F, class S>
__device__ __forceinline__ typename F::Frag v_frag(const S &sm, int w, int u, int li, int qd)
{
    if constexpr (F::TR)
        return tr_frag(sm.Vs, F::LDV, u * F::KB, 16 * w, li, qd);
    else
        return lds_frag(sm.Vts, F::LDC, 16 * w + li, u * F::KB, qd);
}

// Store a 16-byte vector holding row j, columns c*VEC .. of a tile: row-major
// (transpose-read path) or into the transposed copy (fp32 path).
template <class F>
__device__ __forceinline__ void store_row_vec(typename F::T *rowmajor, int ld, typename F::T *transposed, int j,
                                              int c, const uint4 &x)
{
    if constexpr (F::TR) {
        *reinterpret_cast<uint4 *>(rowmajor + j * ld + c * F::VEC) = x;
    } else {
        const typename F::T *e = reinterpret_cast<const typename F::T *>(&x);
#pragma unroll
        for (int i = 0; i < F::VEC; ++i)
            transposed[(c * F::VEC + i) * F::LDC + j] = e[i];
    }
}

// Unpack a fragment of unit u back into fp32 accumulator tiles, adding
// s * value (inverse of acc_frag).
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
    uint4 k[F::NQ], v[F::NV];
    float a;
};

// nrows: valid rows of the chunk (rows past it read as zero).
template <class F>
__device__ __forceinline__ void state_load(StateRegs<F> &r, const typename F::T *k, const typename F::T *v,
                                           const float *a, size_t row0, size_t krow0, int tid, int nrows = F::C)
{
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NQ; ++i) {
        const int idx = tid + i * F::NT;
        r.k[i] = zero16();
        if (idx < F::QVEC && idx / KPR < nrows)
            r.k[i] = *reinterpret_cast<const uint4 *>(k + (krow0 + idx / KPR) * F::DK + (idx % KPR) * F::VEC);
    }
#pragma unroll
    for (int i = 0; i < F::NV; ++i) {
        const int idx = tid + i * F::NT;
        r.v[i] = zero16();
        if (idx < F::VVEC && idx / VPR < nrows)
            r.v[i] = *reinterpret_cast<const uint4 *>(v + (row0 + idx / VPR) * F::DV + (idx % VPR) * F::VEC);
    }
    r.a = (tid < F::C && tid < nrows) ? a[row0 + tid] : 0.f;
}

template <class F>
__global__ __launch_bounds__(F::NT, (F::TR && F::NW >= 4) ? 2 : 1) void ll_group_state(const typename F::T *__restrict__ k,
                                                        const typename F::T *__restrict__ v,
                                                        const float *__restrict__ a, int Tlen, int g, int nG,
                                                        int nL, int rqk, float *__restrict__ Sg,
                                                        float *__restrict__ Gam, typename F::T *__restrict__ Nd,
                                                        float *__restrict__ GamC, int N)
{
    using Frag = typename F::Frag;
    __shared__ StateSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    // Node mode (Nd set): every group is walked (nG workgroups per head), the
    // Fenwick nodes inside the group and the chunk totals are written, and
    // the group state only for the nL groups that are tree leaves.
    const int ngw = Nd ? nG : nL;
    const int bh = blockIdx.x / ngw, sg = blockIdx.x % ngw;
    const int G = 1 << g;
    const size_t hrow = (size_t)bh * Tlen, krow = (size_t)(bh / rqk) * Tlen;   // k is shared by rqk heads
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;

    if constexpr (F::TR) {
        lds_zero<F>(sm.Ks, F::CP * F::LDK, tid);
        lds_zero<F>(sm.Vs, F::CP * F::LDV, tid);
    } else {
        lds_zero<F>(sm.Kts, F::DK * F::LDC, tid);
        lds_zero<F>(sm.Vts, F::DV * F::LDC, tid);
    }

    floatx4 S[F::NDT];
#pragma unroll
    for (int rt = 0; rt < F::NDT; ++rt)
        S[rt] = zero4();
    float gsum = 0.f;

    // node mode: the previous chunk's own state (for nodes of two chunks)
    floatx4 Xp[F::NDT];
#pragma unroll
    for (int rt = 0; rt < F::NDT; ++rt)
        Xp[rt] = zero4();
    const int nci = Nd ? min(G, N - sg * G) : G;   // chunks of this group
    auto rows_of = [&](int ci) { return min(F::C, Tlen - (sg * G + ci) * F::C); };

    StateRegs<F> pf;
    state_load<F>(pf, k, v, a, hrow + (size_t)sg * G * F::C, krow + (size_t)sg * G * F::C, tid, rows_of(0));
    for (int ci = 0; ci < nci; ++ci) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < F::NQ; ++i) {
            const int idx = tid + i * F::NT;
            if (idx < F::QVEC)
                store_row_vec<F>(sm.Ks, F::LDK, sm.Kts, idx / KPR, idx % KPR, pf.k[i]);
        }
#pragma unroll
        for (int i = 0; i < F::NV; ++i) {
            const int idx = tid + i * F::NT;
            if (idx < F::VVEC)
                store_row_vec<F>(sm.Vs, F::LDV, sm.Vts, idx / VPR, idx % VPR, pf.v[i]);
        }
        scan_decay<F>(pf.a, sm.Aloc, &sm.gch, tid);
        if (ci + 1 < nci)
            state_load<F>(pf, k, v, a, hrow + ((size_t)sg * G + ci + 1) * F::C, krow + ((size_t)sg * G + ci + 1) * F::C,
                          tid, rows_of(ci + 1));
        __syncthreads();
        const float gch = sm.gch;
        const float dec = __expf(gch);
        Frag vs[F::NUC];
#pragma unroll
        for (int u = 0; u < F::NUC; ++u)
            vs[u] = scale_tokens<F>(v_frag<F>(sm, w, u, li, qd), u, sm.Aloc, gch, qd);
        if (!Nd) {
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt) {
                S[rt] *= dec;
#pragma unroll
                for (int u = 0; u < F::NUC; ++u)
                    mma_unit(S[rt], kt_frag<F>(sm, rt, u, li, qd), vs[u]);
            }
        } else if constexpr (F::TR && F::DV % 32 == 0) {
            // this chunk's own state X, then S = exp(gch) S + X; the Fenwick
            // node of chunk ci inside the group: X (ci even), X + exp(gch) X of
            // the previous chunk (ci = 1 mod 4), S (ci = 3, chunks 0 .. 3).
            // Here the tiles are transposed (A = V^T, B = K): X[rt][r] is
            // element (dk 16 rt + li, dv 16 w + 4 qd + r).
            floatx4 X[F::NDT];
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt) {
                X[rt] = zero4();
#pragma unroll
                for (int u = 0; u < F::NUC; ++u)
                    mma_unit(X[rt], vs[u], kt_frag<F>(sm, rt, u, li, qd));
                S[rt] = dec * S[rt] + X[rt];
            }
            const int cc = sg * G + ci;   // chunk index
            if (tid == 0)
                GamC[(size_t)bh * N + cc] = gch;
            if (ci < G - 1 && cc < N - 1) {
                typename F::T *nd = Nd + ((size_t)bh * N + cc) * F::DK * F::DV;
#pragma unroll
                for (int rt = 0; rt < F::NDT; ++rt) {
                    floatx4 x = (ci & 1) == 0 ? X[rt] : (ci & 3) == 1 ? X[rt] + dec * Xp[rt] : S[rt];
                    // the backward's A-operand order: fragment (dk tile rt, dv
                    // unit w / 2), this lane, elements 4 (w & 1) ..
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        o[r] = (__bf16)x[r];
                    *reinterpret_cast<bf16x4 *>(nd + ((size_t)(rt * (F::DV / 32) + (w >> 1)) * 64 + lane) * 8 +
                                                4 * (w & 1)) = o;
                }
            }
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt)
                Xp[rt] = X[rt];
        }
        gsum += gch;
    }
    if (sg >= nL)
        return;   // the last group (node mode): not a tree leaf
    float *dst = Sg + ((size_t)bh * nL + sg) * F::DK * F::DV;
    if (F::TR && Nd) {
        // node mode: transposed tiles
#pragma unroll
        for (int rt = 0; rt < F::NDT; ++rt)
            *reinterpret_cast<floatx4 *>(dst + (16 * rt + li) * F::DV + 16 * w + 4 * qd) = S[rt];
    } else {
#pragma unroll
        for (int rt = 0; rt < F::NDT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * rt + 4 * qd + r) * F::DV + 16 * w + li] = S[rt][r];
    }
    if (tid == 0)
        Gam[(size_t)bh * nG + sg] = gsum;
}

// ---------------------------------------------------------------------------
// Kernel B: left-child block states of the tree over groups.
//
// Leaves are states of consecutive blocks at level p0 (groups for p0 = 0,
// blocks of 64 groups for p0 = 6, ...), each with its total log-decay.  A
// workgroup owns the state elements that make up one row of 16-byte
// fragments (unit u, lane quad qd: EPL rows x all dv columns) of one tile of
// 64 leaves; each thread loads its elements of the 64 leaves into registers
// and builds the six tree levels above them (merge: exp(decay of the right
// half) * left + right).  Every complete left child is staged in LDS in
// fragment order and then written with 16-byte stores, and the tile total
// goes out for the next launch.  A block J at level p is complete when it
// ends at or before the last complete group: (J + 1) * 2^p <= nL.  MODE
// selects the stored order: 1 the natural dk order of a fragment lane (lane
// quad qd holds dk 32u + 8qd ..; the specialised bf16 walk), 0 unit_row's
// (the other walks), 2 the backward's order (fragments over dv for each dk
// column; see FwdArgs::tree_yfrag), gathered from the staged lanes.
// ---------------------------------------------------------------------------
template <class F>
struct TreeGeom {
    static constexpr int NE = F::EPL / 4;          // elements per thread (rows e and e + 4)
    static constexpr int NTH = 4 * F::DV;          // threads: 4 row slots x dv columns
    static constexpr int NSLOT = 63;               // left children of six levels over 64 leaves
    static constexpr int CHUNK = F::EPL * (int)sizeof(typename F::T);   // bytes of one fragment lane
    static_assert(CHUNK == 16, "one fragment lane is 16 bytes");
};

template <class F, int MODE>
__global__ __launch_bounds__(TreeGeom<F>::NTH) void ll_left_tree(
    const float *__restrict__ leaves, const float *__restrict__ gleaves, int nleaves, int lstride, int gstride,
    int p0, int nL, int nLeft, typename F::T *__restrict__ Dg, float *__restrict__ tot, float *__restrict__ gtot,
    int tstride)
{
    using T = typename F::T;
    using TG = TreeGeom<F>;
    constexpr int DKV = F::DK * F::DV;
    __shared__ float gsh[64];
    __shared__ uint4 stage[TG::NSLOT * F::DV];   // [slot][column] fragment lanes
    const int tid = threadIdx.x;
    const int u = blockIdx.x >> 2, qd = blockIdx.x & 3;
    const int tile = blockIdx.y, bh = blockIdx.z;
    const int base = tile * 64;
    const int r = tid / F::DV, c = tid % F::DV;
    int dd[TG::NE];
#pragma unroll
    for (int h = 0; h < TG::NE; ++h)
        dd[h] = F::KB * u + (MODE != 0 ? 8 * qd + r + 4 * h : unit_row(r + 4 * h, qd));
    if (tid < 64)
        gsh[tid] = (base + tid < nleaves) ? gleaves[(size_t)bh * gstride + base + tid] : 0.f;
    float x[TG::NE][64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
#pragma unroll
        for (int h = 0; h < TG::NE; ++h)
            x[h][i] = (base + i < nleaves)
                          ? leaves[((size_t)bh * lstride + base + i) * DKV + (size_t)dd[h] * F::DV + c]
                          : 0.f;
    __syncthreads();
    float G[64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
        G[i] = gsh[i];

    // Fragment lane of this thread's elements: lane (qd, c % 16) of
    // fragment (c / 16, u); element e = r + 4h.
    T *st = reinterpret_cast<T *>(stage);
    int slot = 0;
#pragma unroll
    for (int lv = 0; lv < 6; ++lv) {
        const int width = 64 >> lv;
#pragma unroll
        for (int j = 0; j < width; j += 2, ++slot)
#pragma unroll
            for (int h = 0; h < TG::NE; ++h)
                st[((size_t)slot * F::DV + c) * F::EPL + r + 4 * h] = from_f32<T>(x[h][j]);
#pragma unroll
        for (int j = 0; j < width / 2; ++j) {
#pragma unroll
            for (int h = 0; h < TG::NE; ++h)
                x[h][j] = __expf(G[2 * j + 1]) * x[h][2 * j] + x[h][2 * j + 1];
            G[j] = G[2 * j] + G[2 * j + 1];
        }
    }
    if (base + 64 <= nleaves && tot != nullptr) {
#pragma unroll
        for (int h = 0; h < TG::NE; ++h)
            tot[((size_t)bh * tstride + tile) * DKV + (size_t)dd[h] * F::DV + c] = x[h][0];
        if (tid == 0)
            gtot[(size_t)bh * tstride + tile] = G[0];
    }
    __syncthreads();
    // Complete left children, one 16-byte fragment lane per thread and
    // column: slot s is child J = J0 + 2 * jj of level lv.
    size_t offp0 = 0;   // first left block of level p0 for this head
    for (int pp = 0; pp < p0; ++pp)
        offp0 += ((nL >> pp) + 1) >> 1;
    for (int idx = tid; idx < TG::NSLOT * F::DV; idx += TG::NTH) {
        const int s = idx / F::DV, cc = idx % F::DV;
        int lv = 0, first = 0;
        while (s >= first + (32 >> lv)) {
            first += 32 >> lv;
            ++lv;
        }
        const int p = p0 + lv;
        const int J = (base >> lv) + 2 * (s - first);
        if (((int64_t)(J + 1) << p) > nL)
            continue;
        size_t offp = offp0;
        for (int pp = p0; pp < p; ++pp)
            offp += ((nL >> pp) + 1) >> 1;
        T *blk = Dg + ((size_t)bh * nLeft + offp + (J >> 1)) * DKV;
        if constexpr (MODE == 2) {
            // piece (dk row d of this workgroup's eight, dv group pg): the
            // eight dv rows 32u' + 16(k/4) + 4qd' + k%4 of dk column d
            static_assert(F::EPL == 8 && F::DV % 32 == 0, "bf16 pieces over dv");
            const int dl = cc / (F::DV / 8), pg = cc % (F::DV / 8), uv = pg >> 2, qv = pg & 3;
            const int d = F::KB * u + 8 * qd + dl;
            bf16x8 y;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                y[k] = st[((size_t)s * F::DV + 32 * uv + 16 * (k >> 2) + 4 * qv + (k & 3)) * F::EPL + dl];
            const int fo = ((d >> 4) * (F::DV / 32) + uv) * 64 + (d & 15) + 16 * qv;
            *reinterpret_cast<bf16x8 *>(blk + (size_t)fo * 8) = y;
        } else {
            const int fv = ((cc >> 4) * F::NUK + u) * 64 + qd * 16 + (cc & 15);
            *reinterpret_cast<uint4 *>(blk + (size_t)fv * F::EPL) = stage[idx];
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel C: the chunk walk.
//
// The walk works in transposed form: it forms S^T = K Q^T, so the masked
// tiles P^T are already in the register layout the B operand of
// O^T = V^T P^T needs (no LDS round trip for P), and every level adds
// D^T Q^T with the same Q^T fragments, which each wave loads from LDS once
// per chunk.  A wave owns 16 rows of O^T (16 output columns) and all query
// rows of the chunk; the per-query factors vary along the accumulator's
// column, one value per lane and tile.
// ---------------------------------------------------------------------------
template <class F>
struct WalkRegs {
    uint4 q[F::NQ], k[F::NQ], v[F::NV];
    float lam[F::NLAM];
    float a;
};

template <class F>
__device__ __forceinline__ void walk_load(WalkRegs<F> &r, const typename F::T *q, const typename F::T *k,
                                          const typename F::T *v, const float *a, const float *lam, size_t row0,
                                          size_t qrow0, int valid, int L, float invL, int tid)
{
    constexpr int QPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NQ; ++i) {
        const int idx = tid + i * F::NT;
        const int j = idx / QPR, c = idx % QPR;
        r.q[i] = r.k[i] = zero16();
        if (idx < F::QVEC && j < valid) {
            r.q[i] = ld_stream(q + (qrow0 + j) * F::DK + c * F::VEC);
            r.k[i] = ld_stream(k + (qrow0 + j) * F::DK + c * F::VEC);
        }
    }
#pragma unroll
    for (int i = 0; i < F::NV; ++i) {
        const int idx = tid + i * F::NT;
        r.v[i] = zero16();
        if (idx < F::VVEC && idx / VPR < valid)
            r.v[i] = ld_stream(v + (row0 + idx / VPR) * F::DV + (idx % VPR) * F::VEC);
    }
    // lambda rows of the chunk are one contiguous block of valid * L floats
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        r.lam[i] = (idx < valid * L) ? __builtin_nontemporal_load(lam + row0 * L + idx) : 0.f;
    }
    r.a = (tid < valid) ? a[row0 + tid] : 0.f;
    (void)invL;
}

template <class F>
__device__ __forceinline__ void walk_store(const WalkRegs<F> &r, WalkSmem<F> &sm, int valid, int L, float invL,
                                           int tid)
{
    constexpr int QPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NQ; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::QVEC) {
            const int j = idx / QPR, c = idx % QPR;
            *reinterpret_cast<uint4 *>(sm.Qs + j * F::LDK + c * F::VEC) = r.q[i];
            *reinterpret_cast<uint4 *>(sm.Ks + j * F::LDK + c * F::VEC) = r.k[i];
            if constexpr (!F::TR)
                store_row_vec<F>(sm.Ks, F::LDK, sm.Kts, j, c, r.k[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < F::NV; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::VVEC)
            store_row_vec<F>(sm.Vs, F::LDV, sm.Vts, idx / VPR, idx % VPR, r.v[i]);
    }
    // lambda^T: only the valid entries are written; levels >= L stay zero
    // from the start of the kernel, and rows past a ragged chunk's end only
    // feed query rows that are never stored.
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < valid * L) {
            const int j = (int)(((float)idx + 0.5f) * invL);
            sm.lamT[(idx - j * L) * F::LDL + j] = r.lam[i];
        }
    }
    scan_decay<F>(r.a, sm.Aloc, &sm.gch, tid);
}

// O^T += (D^T Q^T) * f, f_i = lambda[i, lev] * exp(Aloc[i] + base), for one
// level whose state D is given as fragments (A operand of D^T Q^T), over this
// wave's query tiles.
template <class F>
__device__ __forceinline__ void level_update(floatx4 *O, const typename F::Frag (*qf)[F::NUK],
                                             const typename F::Frag *d, const float *lamT, const float *ai,
                                             int lev, float base, int h, int li)
{
#pragma unroll
    for (int x = 0; x < F::NQT; ++x) {
        floatx4 tmp = zero4();
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            mma_unit(tmp, d[u], qf[x][u]);
        const float f = lamT[lev * F::LDL + 16 * F::qtile(h, x) + li] * __expf(ai[x] + base);
        O[x] += f * tmp;
    }
}

// Intra-chunk part for the query tiles of half H (compile-time, so every
// tile index below is static): P^T = mask ⊙ (K Q^T) on the causal tiles and
// O^T = V^T P^T.
template <class F, int H>
__device__ __forceinline__ void intra_chunk(floatx4 *O, const typename F::Frag (*qf)[F::NUK], const float *ai,
                                            const typename F::Frag *vf, const WalkSmem<F> &sm, int li, int qd)
{
    using DTag = typename F::DTag;
    constexpr int NJT = F::CP / 16;
#pragma unroll
    for (int x = 0; x < F::NQT; ++x) {
        const int it = F::qtile(H, x);
        floatx4 pt[NJT];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
            pt[jt] = zero4();
#pragma unroll
        for (int jt = 0; jt < F::NMT; ++jt) {
            if (jt > it)
                break;
            __builtin_amdgcn_sched_barrier(0);  // keep one key tile's fragments live at a time
            floatx4 s = zero4();
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                mma_unit(s, lds_frag(sm.Ks, F::LDK, 16 * jt + li, u * F::KB, qd), qf[x][u]);
            const int i = 16 * it + li;
            if (jt < it) {
                // every key of the tile sits in one bucket of query i
                const float lm = sm.lamT[(4 + bitlen_u32((uint32_t)(it ^ jt))) * F::LDL + i];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    pt[jt][r] = s[r] * __expf(ai[x] - sm.Aloc[16 * jt + 4 * qd + r]) * lm;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * qd + r;
                    float m = 0.f;
                    if (j <= i) {
                        const int lev = (i == j) ? 0 : bitlen_u32((uint32_t)(i ^ j));
                        m = __expf(ai[x] - sm.Aloc[j]) * sm.lamT[lev * F::LDL + i];
                    }
                    pt[jt][r] = s[r] * m;
                }
            }
        }
        O[x] = zero4();
#pragma unroll
        for (int u = 0; u < F::NUC; ++u)
            if (u * F::KB <= 16 * it + 15)
                mma_unit(O[x], vf[u], acc_frag(pt, u, DTag{}));
    }
}

template <class F>
__global__ __launch_bounds__(F::NT) void ll_chunk_walk_rs(
    const typename F::T *__restrict__ q, const typename F::T *__restrict__ k, const typename F::T *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, typename F::T *__restrict__ out, int Tlen, int L,
    int log2C, int g, int N, int nG, int Plev, int nL, int nLeft, int rqk, const float *__restrict__ Gam,
    const typename F::T *__restrict__ Dg)
{
    using T = typename F::T;
    using Frag = typename F::Frag;
    using DTag = typename F::DTag;
    constexpr int DKV = F::DK * F::DV;
    __shared__ WalkSmem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int w = wave % F::NWC;   // this wave's 16 output columns
    const int h = wave / F::NWC;   // which half of the query tiles
    const int bh = blockIdx.x / nG, sg = blockIdx.x % nG;
    const int G = 1 << g;
    const int nchunk = min(G, N - sg * G);
    const float invL = 1.f / (float)L;

    WalkRegs<F> pf;
    const size_t qkrow = (size_t)(bh / rqk) * Tlen;   // q and k are shared by rqk heads
    walk_load<F>(pf, q, k, v, a, lam, (size_t)bh * Tlen + (size_t)sg * G * F::C, qkrow + (size_t)sg * G * F::C,
                 min(F::C, Tlen - sg * G * F::C), L, invL, tid);

    // Padding rows (CP > C) and the transposed copies start at zero.
    lds_zero<F>(sm.Ks, F::CP * F::LDK, tid);
    lds_zero<F>(sm.lamT, kMaxLevels * F::LDL, tid);
    if constexpr (F::TR) {
        lds_zero<F>(sm.Vs, F::CP * F::LDV, tid);
    } else {
        lds_zero<F>(sm.Kts, F::DK * F::LDC, tid);
        lds_zero<F>(sm.Vts, F::DV * F::LDC, tid);
    }
    if (tid == 0) {
        int n = 0;
        size_t off = 0;
        for (int p = 0; p < Plev; ++p) {
            if ((sg >> p) & 1) {
                sm.plist[n] = p;
                sm.blk[n] = ((size_t)bh * nLeft + off + (sg >> (p + 1))) * DKV;
                ++n;
            }
            off += ((nL >> p) + 1) >> 1;
        }
        sm.npop = n;
    }
    // Log-decay from the end of each inter-group block to the start of this
    // group: the sum of the group totals strictly between them.
    if (wave == 0) {
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
    // The inter-group level states are the same for every chunk of the group:
    // the first NRES are copied into LDS once, further ones stream from L2.
    const int nres = min(npop, F::NRES);
    for (int idx = tid; idx < nres * (DKV / F::VEC); idx += F::NT) {
        const int ii = idx / (DKV / F::VEC), e = idx % (DKV / F::VEC);
        *reinterpret_cast<uint4 *>(sm.Dres + (size_t)ii * DKV + e * F::VEC) =
            *reinterpret_cast<const uint4 *>(Dg + sm.blk[ii] + (size_t)e * F::VEC);
    }

    // Fenwick stack of the levels inside the group, in fragment form.  Slot
    // m holds the bucket of bit m of the local chunk index, decayed to its own
    // end; gap[m] is the log-decay from that end to the current chunk start.
    // Both waves of a column slice keep identical copies.
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
        walk_store<F>(pf, sm, valid, L, invL, tid);
        if (ci + 1 < nchunk)
            walk_load<F>(pf, q, k, v, a, lam, row0 + F::C, qkrow + t0 + F::C, min(F::C, Tlen - t0 - F::C), L, invL,
                         tid);
        __syncthreads();
        const float gch = sm.gch;

        // Q^T fragments of this wave's query tiles and the decay of this
        // lane's query rows, reused by every product of the chunk.
        Frag qf[F::NQT][F::NUK];
        float ai[F::NQT];
#pragma unroll
        for (int x = 0; x < F::NQT; ++x) {
            const int it = F::qtile(h, x);
            ai[x] = sm.Aloc[16 * it + li];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                qf[x][u] = lds_frag(sm.Qs, F::LDK, 16 * it + li, u * F::KB, qd);
        }
        Frag vf[F::NUC];
#pragma unroll
        for (int u = 0; u < F::NUC; ++u)
            vf[u] = v_frag<F>(sm, w, u, li, qd);

        // Intra-chunk: P^T tiles (key tile jt, query tile it), jt <= it, and
        // O^T = V^T P^T for this wave's columns.
        floatx4 O[F::NQT];
        if (h == 0)
            intra_chunk<F, 0>(O, qf, ai, vf, sm, li, qd);
        else
            intra_chunk<F, 1>(O, qf, ai, vf, sm, li, qd);

        // Levels inside the group.
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m)
            if (m < g && ((ci >> m) & 1))
                level_update<F>(O, qf, stk[m], sm.lamT, ai, log2C + m + 1, gap[m], h, li);

        // Levels above the group.
        for (int ii = 0; ii < npop; ++ii) {
            Frag d[F::NUK];
            const T *src = (ii < F::NRES) ? sm.Dres + (size_t)ii * DKV : Dg + sm.blk[ii];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                d[u] = *reinterpret_cast<const Frag *>(src + ((size_t)(w * F::NUK + u) * 64 + lane) * F::EPL);
            const int p = sm.plist[ii];
            level_update<F>(O, qf, d, sm.lamT, ai, log2C + g + 1 + p, agrun + sm.off[p], h, li);
        }

        // Output: lane holds O[i][16w + 4qd .. 16w + 4qd + 3] for i = 16it + li.
#pragma unroll
        for (int x = 0; x < F::NQT; ++x) {
            const int i = 16 * F::qtile(h, x) + li;
            if (i < valid) {
                T vals[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vals[r] = from_f32<T>(O[x][r]);
                T *dst = out + (row0 + i) * F::DV + 16 * w + 4 * qd;
                if constexpr (sizeof(T) == 2) {
                    typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x2 *>(vals), reinterpret_cast<u32x2 *>(dst));
                } else {
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(vals), reinterpret_cast<u32x4 *>(dst));
                }
            }
        }

        // Fold this chunk's state K^T diag(w) V into the stack (Fenwick carry
        // on ci + 1): slots below the lowest zero bit of ci merge with it into
        // slot kc.
        if (ci + 1 < nchunk) {
            Frag vs[F::NUC];
#pragma unroll
            for (int u = 0; u < F::NUC; ++u)
                vs[u] = scale_tokens<F>(vf[u], u, sm.Aloc, gch, qd);
            floatx4 Hn[F::NDT];
#pragma unroll
            for (int rt = 0; rt < F::NDT; ++rt) {
                Hn[rt] = zero4();
#pragma unroll
                for (int u = 0; u < F::NUC; ++u)
                    mma_unit(Hn[rt], kt_frag<F>(sm, rt, u, li, qd), vs[u]);
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
// Kernel C' (bf16): the chunk walk with shared score tiles and an LDS stack.
//
// Same algorithm as ll_chunk_walk_rs, mapped so that no work is repeated
// across waves: every causal score tile of a chunk is formed once (by one of
// the waves that own its query tile) and shared through LDS as P[i][j];
// wave (it, cg) owns query tile it and CPW of the 16-column output tiles;
// the Fenwick stack of the levels inside the group lives in LDS in fragment
// order, and each wave builds its own fragments of a new stack slot.  Q^T
// fragments are loaded straight from global memory into registers (one
// chunk ahead), so LDS holds only K, V, P, lambda^T, the stack and the
// inter-group states.
// ---------------------------------------------------------------------------
template <class DT, int DK_, int DV_, int C_>
struct Walk4 {
    using T = typename DT::T;
    using Frag = typename DT::Frag;
    using DTag = DT;
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr bool TR = true;
    static constexpr int KB = DT::KB, EPL = DT::EPL;
    static constexpr int NMT = C / 16;                 // query (and key) tiles per chunk
    static constexpr int NWC = DV / 16;                // 16-column output tiles
    static constexpr int QPW = NMT >= 2 ? 2 : 1;       // query tiles per wave (pairs {g, NMT-1-g})
    static constexpr int NQG = NMT / QPW;              // query groups
    static constexpr int CPW = NQG * NWC > 16 ? 2 : 1; // output column tiles per wave
    static constexpr int NCG = NWC / CPW;              // column groups
    static constexpr int NW = NQG * NCG;
    static constexpr int NT = 64 * NW;
    static constexpr int CP = (C < KB) ? KB : C;
    static constexpr int NUC = CP / KB;
    static constexpr int NUK = DK / KB;
    static constexpr int LDK = bf16_stride(DK, true);
    static constexpr int LDV = bf16_stride(DV, false);
    static constexpr int LDP = bf16_stride(CP, true);
    static constexpr int LDL = C + 1;
    static constexpr int VEC = 8;
    static constexpr int SLOT = DK * DV;               // elements of one state
    static constexpr int NFRAG = NUK * NWC;            // 16-byte fragments per lane per state
    static constexpr int KVEC = C * (DK / VEC);
    static constexpr int NK = (KVEC + NT - 1) / NT;
    static constexpr int VVEC = C * (DV / VEC);
    static constexpr int NV = (VVEC + NT - 1) / NT;
    static constexpr int NLAM = (C * kMaxLevels + NT - 1) / NT;
    static constexpr int BASE_LDS = 2 * (C * LDK + CP * LDK + CP * LDV + C * LDP + kMaxGroupLog2 * SLOT) +
                                    4 * (kMaxLevels * LDL + C + CP) + 1024;
    static constexpr int NRES_FIT = (160 * 1024 - BASE_LDS) / (2 * SLOT);
    static constexpr int NRES = NRES_FIT < 0 ? 0 : (NRES_FIT > 8 ? 8 : NRES_FIT);
    static constexpr bool FITS = BASE_LDS <= 160 * 1024 && NW <= 16 && NWC % CPW == 0;
    __device__ static constexpr int qtile(int qg, int x) { return x == 0 ? qg : NMT - 1 - qg; }
};

template <class F>
struct alignas(16) Walk4Smem {
    using T = typename F::T;
    T Qs[F::C * F::LDK];
    T Ks[F::CP * F::LDK];
    T Vs[F::CP * F::LDV];
    T Ps[F::C * F::LDP];
    T stk[kMaxGroupLog2 * F::SLOT];
    T Dres[F::NRES > 0 ? F::NRES * F::SLOT : 8];
    float lamT[kMaxLevels * F::LDL];
    float Aloc[F::C];
    float wdec[F::CP];      // exp(chunk total - Aloc[j]): decay from token j to the chunk end
    float off[32];
    size_t blk[32];
    int plist[32];
    int npop;
    float gch;
};

template <class F>
struct Walk4Regs {
    uint4 q[F::NK], k[F::NK], v[F::NV];
    float lam[F::NLAM];
    float a;
};

template <class F>
__device__ __forceinline__ void walk4_load(Walk4Regs<F> &r, const typename F::T *q, const typename F::T *k,
                                           const typename F::T *v, const float *a, const float *lam, size_t row0,
                                           size_t qrow0, int valid, int L, int tid)
{
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NK; ++i) {
        const int idx = tid + i * F::NT;
        r.q[i] = r.k[i] = zero16();
        if (idx < F::KVEC && idx / KPR < valid) {
            r.q[i] = ld_stream(q + (qrow0 + idx / KPR) * F::DK + (idx % KPR) * F::VEC);
            r.k[i] = ld_stream(k + (qrow0 + idx / KPR) * F::DK + (idx % KPR) * F::VEC);
        }
    }
#pragma unroll
    for (int i = 0; i < F::NV; ++i) {
        const int idx = tid + i * F::NT;
        r.v[i] = zero16();
        if (idx < F::VVEC && idx / VPR < valid)
            r.v[i] = ld_stream(v + (row0 + idx / VPR) * F::DV + (idx % VPR) * F::VEC);
    }
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        r.lam[i] = (idx < valid * L) ? __builtin_nontemporal_load(lam + row0 * L + idx) : 0.f;
    }
    r.a = (tid < valid) ? a[row0 + tid] : 0.f;
}

template <class F>
__device__ __forceinline__ void walk4_store(const Walk4Regs<F> &r, Walk4Smem<F> &sm, int valid, int L, float invL,
                                            int tid)
{
    constexpr int KPR = F::DK / F::VEC, VPR = F::DV / F::VEC;
#pragma unroll
    for (int i = 0; i < F::NK; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::KVEC) {
            // 8 logical columns 8m .. 8m+7 = two 4-column groups (q = 2(m%2), 2(m%2)+1; h = (m/2)%2)
            const int m = idx % KPR;
            const int pos = (idx / KPR) * F::LDK + 32 * (m >> 2) + pq_pos((m >> 1) & 1, 2 * (m & 1));
            typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
            *reinterpret_cast<u32x2 *>(sm.Qs + pos) = u32x2{r.q[i].x, r.q[i].y};
            *reinterpret_cast<u32x2 *>(sm.Qs + pos + 8) = u32x2{r.q[i].z, r.q[i].w};
            *reinterpret_cast<u32x2 *>(sm.Ks + pos) = u32x2{r.k[i].x, r.k[i].y};
            *reinterpret_cast<u32x2 *>(sm.Ks + pos + 8) = u32x2{r.k[i].z, r.k[i].w};
        }
    }
#pragma unroll
    for (int i = 0; i < F::NV; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < F::VVEC)
            *reinterpret_cast<uint4 *>(sm.Vs + (idx / VPR) * F::LDV + (idx % VPR) * F::VEC) = r.v[i];
    }
#pragma unroll
    for (int i = 0; i < F::NLAM; ++i) {
        const int idx = tid + i * F::NT;
        if (idx < valid * L) {
            const int j = (int)(((float)idx + 0.5f) * invL);
            sm.lamT[(idx - j * L) * F::LDL + j] = r.lam[i];
        }
    }
    if (tid < 64) {
        float x = r.a;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float y = __shfl_up(x, d, 64);
            if (tid >= d)
                x += y;
        }
        const float g = __shfl(x, F::C - 1, 64);
        if (tid < F::C)
            sm.Aloc[tid] = x;
        if (tid < F::CP)
            sm.wdec[tid] = (tid < F::C) ? __expf(g - x) : 0.f;
        if (tid == 0)
            sm.gch = g;
    }
}

// Fragment (c, u) of a state stored in fragment order.
template <class F>
__device__ __forceinline__ typename F::Frag state_frag(const typename F::T *st, int c, int u, int lane)
{
    return *reinterpret_cast<const typename F::Frag *>(st + ((size_t)(c * F::NUK + u) * 64 + lane) * F::EPL);
}

// O^T[x][cc] += f[x] * (D^T Q^T) for the wave's query tiles x and column
// tiles cc; f[x] is this lane's query-row factor lambda[i, lev] *
// exp(Aloc[i] + base).  Each state fragment is loaded once and used for
// every query tile of the wave.
template <class F>
__device__ __forceinline__ void walk4_level(floatx4 (*O)[F::CPW], const typename F::Frag (*qf)[F::NUK],
                                            const typename F::T *st, int cg, const float *f, int lane)
{
#pragma unroll
    for (int cc = 0; cc < F::CPW; ++cc) {
        const int c = cg * F::CPW + cc;
        typename F::Frag d[F::NUK];
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            d[u] = state_frag<F>(st, c, u, lane);
#pragma unroll
        for (int x = 0; x < F::QPW; ++x) {
            floatx4 tmp = zero4();
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                mma_unit(tmp, d[u], qf[x][u]);
            O[x][cc] += f[x] * tmp;
        }
    }
}

// As walk4_level, with the wave's state fragments already in registers
// (d[cc][u]: column tile cg * CPW + cc, dk unit u).
template <class F>
__device__ __forceinline__ void walk4_level_regs(floatx4 (*O)[F::CPW], const typename F::Frag (*qf)[F::NUK],
                                                 const typename F::Frag (*d)[F::NUK], const float *f)
{
#pragma unroll
    for (int cc = 0; cc < F::CPW; ++cc) {
#pragma unroll
        for (int x = 0; x < F::QPW; ++x) {
            floatx4 tmp = zero4();
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                mma_unit(tmp, d[cc][u], qf[x][u]);
            O[x][cc] += f[x] * tmp;
        }
    }
}

template <class F>
__global__ __launch_bounds__(F::NT) void ll_chunk_walk(
    const typename F::T *__restrict__ q, const typename F::T *__restrict__ k, const typename F::T *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, typename F::T *__restrict__ out, int Tlen, int L,
    int log2C, int g, int N, int nG, int Plev, int nL, int nLeft, int rqk, const float *__restrict__ Gam,
    const typename F::T *__restrict__ Dg)
{
    using T = typename F::T;
    using Frag = typename F::Frag;
    using DTag = typename F::DTag;
    __shared__ Walk4Smem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int qg = wave % F::NQG;   // query group of this wave (query tiles qtile(qg, x))
    const int cg = wave / F::NQG;   // column group of this wave
    const int bh = blockIdx.x / nG, sg = blockIdx.x % nG;
    const int G = 1 << g;
    const int nchunk = min(G, N - sg * G);
    const float invL = 1.f / (float)L;

    Walk4Regs<F> pf;
    const size_t qkrow = (size_t)(bh / rqk) * Tlen;   // q and k are shared by rqk heads
    walk4_load<F>(pf, q, k, v, a, lam, (size_t)bh * Tlen + (size_t)sg * G * F::C, qkrow + (size_t)sg * G * F::C,
                  min(F::C, Tlen - sg * G * F::C), L, tid);

    // Padding rows of K and V, P (its upper tiles and padding columns are
    // never written) and lambda^T (levels >= L) start at zero.
    lds_zero<F>(sm.Ks, F::CP * F::LDK, tid);
    lds_zero<F>(sm.Vs, F::CP * F::LDV, tid);
    lds_zero<F>(sm.Ps, F::C * F::LDP, tid);
    lds_zero<F>(sm.lamT, kMaxLevels * F::LDL, tid);
    if (tid == 0) {
        int n = 0;
        size_t off = 0;
        for (int p = 0; p < Plev; ++p) {
            if ((sg >> p) & 1) {
                sm.plist[n] = p;
                sm.blk[n] = ((size_t)bh * nLeft + off + (sg >> (p + 1))) * F::SLOT;
                ++n;
            }
            off += ((nL >> p) + 1) >> 1;
        }
        sm.npop = n;
    }
    if (wave == 0) {
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
    const int nres = min(npop, F::NRES);
    for (int idx = tid; idx < nres * (F::SLOT / F::VEC); idx += F::NT) {
        const int ii = idx / (F::SLOT / F::VEC), e = idx % (F::SLOT / F::VEC);
        *reinterpret_cast<uint4 *>(sm.Dres + (size_t)ii * F::SLOT + e * F::VEC) =
            *reinterpret_cast<const uint4 *>(Dg + sm.blk[ii] + (size_t)e * F::VEC);
    }

    float gap[kMaxGroupLog2];
#pragma unroll
    for (int m = 0; m < kMaxGroupLog2; ++m)
        gap[m] = 0.f;
    float agrun = 0.f;

    for (int ci = 0; ci < nchunk; ++ci) {
        const int t0 = (sg * G + ci) * F::C;
        const int valid = min(F::C, Tlen - t0);
        const size_t row0 = (size_t)bh * Tlen + t0;
        __syncthreads();
        walk4_store<F>(pf, sm, valid, L, invL, tid);
        if (ci + 1 < nchunk)
            walk4_load<F>(pf, q, k, v, a, lam, row0 + F::C, qkrow + t0 + F::C, min(F::C, Tlen - t0 - F::C), L, tid);
        __syncthreads();
        const float gch = sm.gch;
        // This lane's query rows (one per query tile of the wave), their
        // decay and their Q^T fragments.
        int iq[F::QPW];
        float ai[F::QPW];
        Frag qf[F::QPW][F::NUK];
#pragma unroll
        for (int x = 0; x < F::QPW; ++x) {
            iq[x] = 16 * F::qtile(qg, x) + li;
            ai[x] = sm.Aloc[iq[x]];
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                qf[x][u] = lds_frag(sm.Qs, F::LDK, iq[x], u * F::KB, qd);
        }

        // Causal score tiles (jt, it) of the group's query tiles, dealt
        // round-robin to its column-group waves; masked by decay and level
        // weight and stored as P[i][j].
        {
            int n = 0;
#pragma unroll
            for (int x = 0; x < F::QPW; ++x) {
                const int it = F::qtile(qg, x);
                const int i = iq[x];
                for (int jt = 0; jt <= it; ++jt, ++n) {
                    if (n % F::NCG != cg)
                        continue;
                    floatx4 s = zero4();
#pragma unroll
                    for (int u = 0; u < F::NUK; ++u)
                        mma_unit(s, lds_frag(sm.Ks, F::LDK, 16 * jt + li, u * F::KB, qd), qf[x][u]);
                    float p[4];
                    if (jt < it) {
                        const float lm = sm.lamT[(4 + bitlen_u32((uint32_t)(it ^ jt))) * F::LDL + i];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            p[r] = s[r] * __expf(ai[x] - sm.Aloc[16 * jt + 4 * qd + r]) * lm;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = 16 * jt + 4 * qd + r;
                            float m = 0.f;
                            if (j <= i) {
                                const int lev = (i == j) ? 0 : bitlen_u32((uint32_t)(i ^ j));
                                m = __expf(ai[x] - sm.Aloc[j]) * sm.lamT[lev * F::LDL + i];
                            }
                            p[r] = s[r] * m;
                        }
                    }
                    bf16x4 pb;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pb[r] = (__bf16)p[r];
                    *reinterpret_cast<bf16x4 *>(sm.Ps + i * F::LDP + 16 * jt + 4 * qd) = pb;
                }
            }
        }
        __syncthreads();

        // O^T = V^T P^T for this wave's query and column tiles.
        floatx4 O[F::QPW][F::CPW];
#pragma unroll
        for (int cc = 0; cc < F::CPW; ++cc) {
            const int c = cg * F::CPW + cc;
#pragma unroll
            for (int x = 0; x < F::QPW; ++x)
                O[x][cc] = zero4();
#pragma unroll
            for (int u = 0; u < F::NUC; ++u) {
                const Frag vt = tr_frag(sm.Vs, F::LDV, u * F::KB, 16 * c, li, qd);
#pragma unroll
                for (int x = 0; x < F::QPW; ++x)
                    if (u * F::KB <= 16 * F::qtile(qg, x) + 15)
                        mma_unit(O[x][cc], vt, lds_frag(sm.Ps, F::LDP, iq[x], u * F::KB, qd));
            }
        }

        // Levels inside the group (stack slots in LDS).
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m)
            if (m < g && ((ci >> m) & 1)) {
                float f[F::QPW];
#pragma unroll
                for (int x = 0; x < F::QPW; ++x)
                    f[x] = sm.lamT[(log2C + m + 1) * F::LDL + iq[x]] * __expf(ai[x] + gap[m]);
                walk4_level<F>(O, qf, sm.stk + m * F::SLOT, cg, f, lane);
            }
        // Levels above the group.
        for (int ii = 0; ii < npop; ++ii) {
            const int p = sm.plist[ii];
            float f[F::QPW];
#pragma unroll
            for (int x = 0; x < F::QPW; ++x)
                f[x] = sm.lamT[(log2C + g + 1 + p) * F::LDL + iq[x]] * __expf(ai[x] + agrun + sm.off[p]);
            const T *st = (ii < F::NRES) ? sm.Dres + (size_t)ii * F::SLOT : Dg + sm.blk[ii];
            walk4_level<F>(O, qf, st, cg, f, lane);
        }

        // Output: lane holds O[i][16c + 4qd .. 16c + 4qd + 3] for i = iq[x].
#pragma unroll
        for (int x = 0; x < F::QPW; ++x) {
            if (iq[x] < valid) {
#pragma unroll
                for (int cc = 0; cc < F::CPW; ++cc) {
                    const int c = cg * F::CPW + cc;
                    typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
                    bf16x4 ob;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ob[r] = (__bf16)O[x][cc][r];
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x2 *>(&ob),
                                                reinterpret_cast<u32x2 *>(out + (row0 + iq[x]) * F::DV + 16 * c + 4 * qd));
                }
            }
        }

        // Fold this chunk's state into the stack: slot kc (not read during
        // this chunk) becomes the chunk state plus the decayed slots below it
        // (read, never written, during this chunk).  Each wave builds whole
        // fragments (c, u) of the new slot.
        if (ci + 1 < nchunk) {
            const int kc = __builtin_ctz((unsigned)(ci + 1));
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
                gap[m] += gch;
            for (int fr = wave; fr < F::NFRAG; fr += F::NW) {
                const int u = fr / F::NWC, c = fr % F::NWC;
                floatx4 Hn[2] = {zero4(), zero4()};
#pragma unroll
                for (int uj = 0; uj < F::NUC; ++uj) {
                    Frag vsf = tr_frag(sm.Vs, F::LDV, uj * F::KB, 16 * c, li, qd);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vsf[e] = (__bf16)((float)vsf[e] * sm.wdec[uj * F::KB + unit_row(e, qd)]);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        mma_unit(Hn[t], tr_frag(sm.Ks, F::LDK, uj * F::KB, 16 * (2 * u + t), li, qd), vsf);
                }
#pragma unroll
                for (int m = 0; m < kMaxGroupLog2; ++m)
                    if (m < kc)
                        frag_axpy(Hn, state_frag<F>(sm.stk + m * F::SLOT, c, u, lane), 0, __expf(gap[m]), DTag{});
                *reinterpret_cast<Frag *>(sm.stk + kc * F::SLOT + ((size_t)(c * F::NUK + u) * 64 + lane) * F::EPL) =
                    acc_frag(Hn, 0, DTag{});
            }
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
                if (m == kc)
                    gap[m] = 0.f;
        }
        agrun += gch;
    }
}

// ---------------------------------------------------------------------------
// Kernel C'' (bf16): the chunk walk with specialised waves.
//
// The same per-chunk algebra as ll_chunk_walk, split over two kinds of wave
// so that the parts of a chunk's work overlap on every SIMD instead of
// following each other:
//  * NX compute waves own the output tiles (query-tile pairs x 16-column
//    slices): masked score tiles -> P (shared through LDS), O^T = V^T P^T,
//    the levels inside and above the group, the output rows, and (when dk
//    has at least two units per query group) part of the state fold;
//  * NY helper waves fold each chunk's state into the Fenwick stack and
//    stream the chunks from HBM straight into LDS with LDS-direct buffer
//    loads (no register staging), and form each chunk's decay prefix.
// Every per-chunk LDS tile is double-buffered by chunk parity.  Two
// workgroup barriers per chunk: A (chunk staged, stack slots ready) and B (P
// complete).  Q and K of chunk kk+2 are requested right after barrier B of
// chunk kk (nobody reads chunk kk's Q/K after B); V, lambda and a of chunk
// kk+1 right after barrier A of chunk kk (chunk kk-1's copies are read until
// then).
//
// LDS layouts.  Q and K rows are unpadded with the 16-byte chunks of a row
// XOR-swizzled (qk_swz), so the sixteen rows of an operand-fragment read hit
// distinct banks; their dk order is the natural one (lane quad qd supplies
// dk 32u + 8qd .. 32u + 8qd + 7, one 16-byte read).  The Fenwick stack and
// the block states use the same dk order.  V keeps padded rows (read only by
// transpose reads); P uses the paired-quad order; lambda is row-major
// [token][level].
// ---------------------------------------------------------------------------
template <class DT, int DK_, int DV_, int C_>
struct WalkWS {
    using T = typename DT::T;
    using Frag = typename DT::Frag;
    using DTag = DT;
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr int KB = DT::KB, EPL = DT::EPL;
    static constexpr int NMT = C / 16;                 // query (and key) tiles per chunk
    static constexpr int NWC = DV / 16;                // 16-column output tiles
    static constexpr int QPW = NMT >= 2 ? 2 : 1;       // query tiles per compute wave
    static constexpr int NQG = NMT / QPW;              // query groups
    static constexpr int CPW = NQG * NWC > 8 ? 2 : 1;  // output column tiles per compute wave
    static constexpr int NCG = NWC / CPW;              // column groups
    static constexpr int NX = NQG * NCG;               // compute waves
    static constexpr int NY = 4;                       // helper waves
    static constexpr int NW = NX + NY;
    static constexpr int NT = 64 * NW;
    static constexpr int CP = (C < KB) ? KB : C;
    static constexpr int NUC = CP / KB;
    static constexpr int NUK = DK / KB;
    static constexpr int CPR = DK / 8;                 // 16-byte chunks per Q/K row
    static constexpr int G4 = CPR / 4;                 // groups of four chunks per row
    static constexpr int RW = CPR >= 16 ? 1 : 16 / CPR;  // rows sharing one pass over the 64 banks
    static constexpr int LDV = tr_stride(DV);          // V row stride (padded)
    static constexpr int VCR = LDV / 8;                // 16-byte chunks per V row, padding included
    static constexpr int LDP = bf16_stride(CP, true);
    static constexpr int NLV = 22;                     // lambda levels staged (T <= 2^21)
    static constexpr int SLOT = DK * DV;               // elements of one state
    static constexpr int VEC = 8;                      // bf16 elements per 16 bytes
    static constexpr int QKB = C * CPR / 64;           // 1-KB LDS-direct blocks of a Q (or K) tile
    static constexpr int VBLK = (C * VCR + 63) / 64;   // blocks of a V tile
    // The fold of a chunk's state is split by dk unit: when dk has at least
    // two units per query group, compute wave (qg, cg) folds unit XU0 + qg of
    // its own output columns (it has slack before barrier B) and the helpers
    // fold units 0 .. YU-1.  A helper wave folds unit u = yw % YU for the
    // columns c = yw / YU + (NY / YU) * kk, so its K^T fragments are loaded
    // once.
    static constexpr bool XF = (NUK >= 2 * NQG) && (NY % (NUK - NQG) == 0);
    static constexpr int XU0 = XF ? NUK - NQG : NUK;
    static constexpr int YU = XU0;
    static constexpr int CSTEP = NY / YU;
    static constexpr int NFY = (NWC + CSTEP - 1) / CSTEP;
    // Q/K blocks each helper wave requests after barrier B (equal for every
    // wave when they divide evenly; then the wave can wait for everything
    // older than them).
    static constexpr int NQKW = (2 * QKB) % NY == 0 ? 2 * QKB / NY : -1;
    static constexpr int BASE_LDS = 2 * (2 * C * DK + 2 * CP * DK + 2 * CP * LDV + C * LDP + kMaxGroupLog2 * SLOT) +
                                    4 * (2 * C * NLV + 2 * 64 + 2 * CP + 2 * C) + 1024;
    static constexpr int NRES_FIT = (160 * 1024 - BASE_LDS) / (2 * SLOT);
    static constexpr int NRES = NRES_FIT < 0 ? 0 : (NRES_FIT > 8 ? 8 : NRES_FIT);
    static constexpr bool FITS = BASE_LDS <= 160 * 1024 && NWC % CPW == 0 && NY % YU == 0 && C * CPR % 64 == 0;
    static constexpr int NPF = 2;                      // block states above the group prefetched into registers
    __device__ static constexpr int qtile(int qg, int x) { return x == 0 ? qg : NMT - 1 - qg; }
};

template <class F>
struct alignas(16) WalkWSSmem {
    using T = typename F::T;
    T Qs[2][F::C * F::DK];
    T Ks[2][F::CP * F::DK];
    T Vs[2][F::CP * F::LDV];
    T Ps[F::C * F::LDP];
    T stk[kMaxGroupLog2 * F::SLOT];
    T Dres[F::NRES > 0 ? F::NRES * F::SLOT : 8];
    alignas(16) float lam[2][F::C * F::NLV];  // [token][level], row length L
    alignas(16) float abuf[2][64];
    alignas(16) float wdec[2][F::CP];         // exp(chunk total - Aloc[j]): decay from token j to the chunk end
    alignas(16) float Aloc[2][F::C];
    float off[32];
    size_t blk[32];
    int plist[32];
    float gch[2];
};

// XOR swizzle of the 16-byte chunks of Q/K row r: a bit rotation of the
// row's index within CPR consecutive bank passes, so that (a) the sixteen
// rows of a fragment read land on distinct chunks of the 64 banks and (b)
// the rows of a transpose read fall in different 4-chunk groups.
template <class F>
__device__ __forceinline__ int qk_swz(int r)
{
    const int x = (r / F::RW) % F::CPR;
    return ((x % F::G4) << 2) | (x / F::G4);
}

// Element offset of logical 16-byte chunk lc of Q/K row r.
template <class F>
__device__ __forceinline__ int qk_off(int r, int lc)
{
    return r * F::DK + ((lc ^ qk_swz<F>(r)) << 3);
}

// Operand fragment (unit u, lane quad qd) of Q/K row r: dk 32u + 8qd ..
template <class F>
__device__ __forceinline__ bf16x8 qk_frag(const __bf16 *tile, int r, int u, int qd)
{
    return *reinterpret_cast<const bf16x8 *>(tile + qk_off<F>(r, 4 * u + qd));
}

// Transpose-read fragment of K^T for the chunk state: token rows jb ..
// jb+31 (k index, in the unit_row order of tr_frag), and for tile t of dk
// unit u the 16 rows of the result are dk 32u + 8(m/4) + 4t + m%4 (m = 0..15),
// so that the tile pair of an accumulator packs into a fragment in natural
// dk order.
template <class F>
__device__ __forceinline__ bf16x8 kt_frag_nat(const __bf16 *tile, int jb, int u, int t, int li, int qd)
{
    const int r = jb + 4 * qd + (li >> 2);
    const __bf16 *p0 = tile + qk_off<F>(r, 4 * u + (li & 3)) + 4 * t;
    const __bf16 *p1 = tile + qk_off<F>(r + 16, 4 * u + (li & 3)) + 4 * t;
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
    bf16x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return v;
}

// Inclusive prefix sum over the 64 lanes of a fully active wave, with DPP
// row shifts inside each 16-lane row and row broadcasts across rows (no LDS
// round trips).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_shift(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_prefix_sum(float x)
{
    x += dpp_shift<0x111, 0xf>(x);  // row_shr:1
    x += dpp_shift<0x112, 0xf>(x);  // row_shr:2
    x += dpp_shift<0x114, 0xf>(x);  // row_shr:4
    x += dpp_shift<0x118, 0xf>(x);  // row_shr:8
    x += dpp_shift<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_shift<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Per-head buffer descriptors of the walk's streamed inputs.  Loads through
// them take 32-bit offsets, and every byte past the head's last token reads
// as zero, which supplies the zero padding of a ragged last chunk.
struct WSBuf {
    __amdgpu_buffer_rsrc_t q, k, v, lam, a;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS-direct streaming load: lane l of the wave writes `size` bytes read at
// byte offset `off` of the descriptor's range to LDS address dst + l * size
// (dst is wave-uniform).  Completion is counted by vmcnt.
template <int SIZE>
__device__ __forceinline__ void ld_lds(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t off)
{
    static_assert(SIZE == 4 || SIZE == 16, "LDS-direct sizes used here");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, (int)off, 0, 0, 2);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 4, (int)off, 0, 0, 2);
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Helper wave yw's share of the Q and K rows of the chunk at token t0 into
// buffer `slot` (swizzled; rows past the head's end arrive as zeros).
template <class F>
__device__ __forceinline__ void ws_ld_qk(WalkWSSmem<F> &sm, const WSBuf &bf, int slot, int t0, int yw, int lane)
{
#pragma unroll
    for (int i = 0; i < (2 * F::QKB + F::NY - 1) / F::NY; ++i) {
        const int blk = yw + i * F::NY;
        if (blk < 2 * F::QKB) {
            const bool isk = blk >= F::QKB;
            const int bb = isk ? blk - F::QKB : blk;
            const int pc = bb * 64 + lane;   // physical 16-byte chunk of the tile
            const int r = pc / F::CPR;
            const int lc = (pc % F::CPR) ^ qk_swz<F>(r);
            const uint32_t off = ((uint32_t)(t0 + r) * F::DK + (uint32_t)lc * 8) * 2;
            __bf16 *dst = (isk ? sm.Ks[slot] : sm.Qs[slot]) + bb * 512;
            ld_lds<16>(isk ? bf.k : bf.q, dst, off);
        }
    }
}

// Helper wave yw's share of the V rows (padded; the padding lanes load a
// copy of the row's first chunk), the lambda rows and the decays a of the
// chunk at token t0 into buffer `slot`.
template <class F>
__device__ __forceinline__ void ws_ld_vla(WalkWSSmem<F> &sm, const WSBuf &bf, int slot, int t0, int L, int yw,
                                          int lane)
{
#pragma unroll
    for (int i = 0; i < (F::VBLK + F::NY - 1) / F::NY; ++i) {
        const int blk = yw + i * F::NY;
        if (blk < F::VBLK) {
            const int pc = blk * 64 + lane;
            const int r = pc / F::VCR, cc = pc % F::VCR;
            const uint32_t off = ((uint32_t)(t0 + r) * F::DV + (uint32_t)(cc < F::DV / 8 ? cc : 0) * 8) * 2;
            if (pc < F::C * F::VCR)
                ld_lds<16>(bf.v, sm.Vs[slot] + blk * 512, off);
        }
    }
    // lambda rows are contiguous (C * L floats): 16 bytes per lane.
    const int nlv = (F::C * L + 3) / 4;   // 16-byte pieces
    for (int blk = yw; blk * 64 < nlv; blk += F::NY) {
        const int idx = blk * 64 + lane;
        if (idx < nlv)
            ld_lds<16>(bf.lam, sm.lam[slot] + blk * 256, ((uint32_t)t0 * L + 4 * idx) * 4);
    }
    if (yw == F::NY - 1 && lane < F::C)
        ld_lds<4>(bf.a, sm.abuf[slot], (uint32_t)(t0 + lane) * 4);
}

// Decay prefix of the chunk in buffer `slot` (one helper wave, after its a
// has arrived): Aloc, the token weights w_j = exp(total - Aloc[j]) and the
// chunk total.
template <class F>
__device__ __forceinline__ void ws_scan(WalkWSSmem<F> &sm, int slot, int lane)
{
    const float x = wave_prefix_sum(lane < F::C ? sm.abuf[slot][lane] : 0.f);
    const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), F::C - 1));
    if (lane < F::C)
        sm.Aloc[slot][lane] = x;
    if (lane < F::CP)
        sm.wdec[slot][lane] = (lane < F::C) ? __expf(g - x) : 0.f;
    if (lane == 0)
        sm.gch[slot] = g;
}

// Weighted K^T fragments of dk unit u for the chunk state K^T diag(w) V.
template <class F>
__device__ __forceinline__ void ws_kfrags(const WalkWSSmem<F> &sm, int b, int u, int li, int qd,
                                          typename F::Frag (*kf)[2])
{
    using Frag = typename F::Frag;
#pragma unroll
    for (int uj = 0; uj < F::NUC; ++uj) {
        const floatx4 w0 = *reinterpret_cast<const floatx4 *>(&sm.wdec[b][uj * F::KB + 4 * qd]);
        const floatx4 w1 = *reinterpret_cast<const floatx4 *>(&sm.wdec[b][uj * F::KB + 16 + 4 * qd]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            Frag f = kt_frag_nat<F>(sm.Ks[b], uj * F::KB, u, t, li, qd);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = (__bf16)((float)f[e] * w0[e]);
                f[e + 4] = (__bf16)((float)f[e + 4] * w1[e]);
            }
            kf[uj][t] = f;
        }
    }
}

// Fragments kk in [K0, K1) of chunk ci's new stack slot kc for dk unit u
// (columns c0 + CS * kk): the chunk state plus the slots below it, decayed to
// the chunk end (gapc[m] = their decay factors).  The V^T reads are issued
// before the products.
template <class F, int K0, int K1, int CS>
__device__ __forceinline__ void ws_fold(WalkWSSmem<F> &sm, const typename F::Frag (*kf)[2], int b, int kc,
                                        const float *gapc, int u, int c0, int lane, int li, int qd)
{
    using Frag = typename F::Frag;
    if constexpr (K1 > K0) {
        Frag vf[K1 - K0][F::NUC];
#pragma unroll
        for (int kk = K0; kk < K1; ++kk) {
            const int c = min(c0 + CS * kk, F::NWC - 1);
#pragma unroll
            for (int uj = 0; uj < F::NUC; ++uj)
                vf[kk - K0][uj] = tr_frag(sm.Vs[b], F::LDV, uj * F::KB, 16 * c, li, qd);
        }
        floatx4 Hn[K1 - K0][2];
#pragma unroll
        for (int kk = K0; kk < K1; ++kk) {
            Hn[kk - K0][0] = Hn[kk - K0][1] = zero4();
#pragma unroll
            for (int uj = 0; uj < F::NUC; ++uj)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    mma_unit(Hn[kk - K0][t], kf[uj][t], vf[kk - K0][uj]);
        }
#pragma unroll
        for (int kk = K0; kk < K1; ++kk) {
            const int c = c0 + CS * kk;
            if (c < F::NWC) {
#pragma unroll
                for (int m = 0; m < kMaxGroupLog2; ++m)
                    if (m < kc)
                        frag_axpy(Hn[kk - K0], state_frag<F>(sm.stk + m * F::SLOT, c, u, lane), 0, gapc[m], TBF16{});
                *reinterpret_cast<Frag *>(sm.stk + kc * F::SLOT + ((size_t)(c * F::NUK + u) * 64 + lane) * F::EPL) =
                    acc_frag(Hn[kk - K0], 0, TBF16{});
            }
        }
    }
}

template <class F, class E>
__device__ __forceinline__ void ws_zero(E *dst, int n, int t, int nt)
{
    for (int i = t; i < n; i += nt)
        dst[i] = E(0.f);
}

// The groups one workgroup walks: a group sg and its mirror nG-1-sg of the
// same head (their numbers of set bits, and so of levels above the group,
// add up to about the same for every pair).
struct WSGroups {
    int n;          // 1 or 2
    int sg0, sg1;   // group indices
    int n0, n1;     // chunks in each (n1 = 0 when n = 1)
    __device__ int sg(int i) const { return i ? sg1 : sg0; }
    __device__ int nch(int i) const { return i ? n1 : n0; }
};

template <class F>
__device__ __forceinline__ int ws_token(const WSGroups &gr, int G, int kk)
{
    return kk < gr.n0 ? (gr.sg0 * G + kk) * F::C : (gr.sg1 * G + kk - gr.n0) * F::C;
}

template <class F>
__device__ __forceinline__ void ws_helper(WalkWSSmem<F> &sm, const typename F::T *q, const typename F::T *k,
                                          const typename F::T *v, const float *a, const float *lam, int Tlen, int L,
                                          int bh, int qbh, const WSGroups &gr, int G, int ty)
{
    using Frag = typename F::Frag;
    const int lane = ty & 63, yw = ty >> 6, qd = lane >> 4, li = lane & 15;
    const int u = yw % F::YU, c0 = yw / F::YU;
    const size_t hrow = (size_t)bh * Tlen, qrow = (size_t)qbh * Tlen;
    const WSBuf bf = {head_rsrc(q + qrow * F::DK, (uint32_t)Tlen * F::DK * 2),
                      head_rsrc(k + qrow * F::DK, (uint32_t)Tlen * F::DK * 2),
                      head_rsrc(v + hrow * F::DV, (uint32_t)Tlen * F::DV * 2),
                      head_rsrc(lam + hrow * L, (uint32_t)Tlen * L * 4), head_rsrc(a + hrow, (uint32_t)Tlen * 4)};
    // The chunks of both groups form one stream kk = 0 .. K-1, chunk kk in
    // LDS buffer kk & 1.
    const int K = gr.n0 + gr.n1;
    // Rows past the chunk (K and V when C < 32) and P (its upper tiles and
    // padding columns) are never loaded and stay zero.
    if constexpr (F::CP > F::C) {
        ws_zero<F>(&sm.Ks[0][F::C * F::DK], (F::CP - F::C) * F::DK, ty, 64 * F::NY);
        ws_zero<F>(&sm.Ks[1][F::C * F::DK], (F::CP - F::C) * F::DK, ty, 64 * F::NY);
        ws_zero<F>(&sm.Vs[0][F::C * F::LDV], (F::CP - F::C) * F::LDV, ty, 64 * F::NY);
        ws_zero<F>(&sm.Vs[1][F::C * F::LDV], (F::CP - F::C) * F::LDV, ty, 64 * F::NY);
    }
    ws_zero<F>(sm.Ps, F::C * F::LDP, ty, 64 * F::NY);
    ws_ld_qk<F>(sm, bf, 0, ws_token<F>(gr, G, 0), yw, lane);
    ws_ld_vla<F>(sm, bf, 0, ws_token<F>(gr, G, 0), L, yw, lane);
    wait_vm<0>();
    if (yw == F::NY - 1)
        ws_scan<F>(sm, 0, lane);
    if (K > 1)
        ws_ld_qk<F>(sm, bf, 1, ws_token<F>(gr, G, 1), yw, lane);
    __syncthreads();  // prologue
    int kk = 0;
    for (int gi = 0; gi < gr.n; ++gi) {
        if (gi > 0)
            __syncthreads();  // group boundary
        const int nchunk = gr.nch(gi);
        float gap[kMaxGroupLog2];
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m)
            gap[m] = 0.f;
        for (int ci = 0; ci < nchunk; ++ci, ++kk) {
            const int b = kk & 1;
            const bool more = ci + 1 < nchunk;
            const int kc = more ? __builtin_ctz((unsigned)(ci + 1)) : 0;
            __syncthreads();  // A
            const float gch = sm.gch[b];
            if (kk + 1 < K)
                ws_ld_vla<F>(sm, bf, b ^ 1, ws_token<F>(gr, G, kk + 1), L, yw, lane);
            if (more) {
                float gapc[kMaxGroupLog2];
#pragma unroll
                for (int m = 0; m < kMaxGroupLog2; ++m)
                    gapc[m] = __expf(gap[m] + gch);
                Frag kf[F::NUC][2];
                ws_kfrags<F>(sm, b, u, li, qd, kf);
                if constexpr (F::NFY <= 2) {
                    ws_fold<F, 0, F::NFY, F::CSTEP>(sm, kf, b, kc, gapc, u, c0, lane, li, qd);
                } else {
                    ws_fold<F, 0, (F::NFY + 1) / 2, F::CSTEP>(sm, kf, b, kc, gapc, u, c0, lane, li, qd);
                    __builtin_amdgcn_sched_barrier(0);
                    ws_fold<F, (F::NFY + 1) / 2, F::NFY, F::CSTEP>(sm, kf, b, kc, gapc, u, c0, lane, li, qd);
                }
            }
            __syncthreads();  // B
            if (kk + 2 < K)
                ws_ld_qk<F>(sm, bf, b, ws_token<F>(gr, G, kk + 2), yw, lane);
            // Everything but the Q/K requests just made (in flight over the
            // next chunk) must have landed before barrier A.
            if constexpr (F::NQKW >= 0) {
                if (kk + 2 < K)
                    wait_vm<F::NQKW>();
                else
                    wait_vm<0>();
            } else {
                wait_vm<0>();
            }
            if (kk + 1 < K && yw == F::NY - 1)
                ws_scan<F>(sm, b ^ 1, lane);
            if (more) {
#pragma unroll
                for (int m = 0; m < kMaxGroupLog2; ++m)
                    gap[m] = (m == kc) ? 0.f : gap[m] + gch;
            }
        }
    }
}

template <class F>
__device__ __forceinline__ void ws_compute(WalkWSSmem<F> &sm, typename F::T *out, int Tlen, int L, int log2C,
                                           int g, int bh, const WSGroups &gr, int nG, int Plev, int nL, int nLeft,
                                           const float *Gam, const typename F::T *Dg, int tid)
{
    using T = typename F::T;
    using Frag = typename F::Frag;
    const int lane = tid & 63, wave = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int qg = wave % F::NQG;   // query group of this wave (query tiles qtile(qg, x))
    const int cg = wave / F::NQG;   // column group of this wave
    int kk = 0;   // chunk index in the workgroup's stream (LDS buffer parity)
    for (int gi = 0; gi < gr.n; ++gi) {
        const int sg = gr.sg(gi), nchunk = gr.nch(gi);
        const int t0g = sg * (1 << g) * F::C;
        const size_t rowg = (size_t)bh * Tlen + t0g;
        if (gi > 0)
            __syncthreads();  // group boundary: the previous group's Dres, off and plist are no longer read
        // The group's blocks above it: one per set bit p of the group index,
        // with the block state's offset and the log-decay from its end to the
        // group start.  Every thread walks the bits itself, so the loads of the
        // LDS-resident block states are issued at once.
        constexpr int DPT = (F::SLOT / F::VEC + 64 * F::NX - 1) / (64 * F::NX);
        const int npop = __builtin_popcount((unsigned)sg);   // every set bit of sg is below Plev
        if (tid == 0) {
            int n = 0;
            size_t off = 0;
            for (int p = 0; p < Plev; ++p) {
                if ((sg >> p) & 1) {
                    sm.plist[n] = p;
                    sm.blk[n] = ((size_t)bh * nLeft + off + (sg >> (p + 1))) * F::SLOT;
                    ++n;
                }
                off += ((nL >> p) + 1) >> 1;
            }
        }
        // Resident block states, copied straight to LDS (no wave reads Dres
        // between the group boundary and the group's first barrier A).
#pragma unroll
        for (int ii = 0; ii < F::NRES; ++ii) {
            if (ii < npop) {
                unsigned x = (unsigned)sg;
#pragma unroll
                for (int k = 0; k < ii; ++k)
                    x &= x - 1;
                const int p = __builtin_ctz(x);   // the ii-th set bit
                size_t off = 0;
                for (int r = 0; r < p; ++r)
                    off += ((nL >> r) + 1) >> 1;
                const size_t blk = ((size_t)bh * nLeft + off + (sg >> (p + 1))) * F::SLOT;
#pragma unroll
                for (int e = 0; e < DPT; ++e) {
                    const int idx = tid + e * 64 * F::NX;
                    if (idx < F::SLOT / F::VEC)
                        *reinterpret_cast<uint4 *>(sm.Dres + (size_t)ii * F::SLOT + (size_t)idx * F::VEC) =
                            *reinterpret_cast<const uint4 *>(Dg + blk + (size_t)idx * F::VEC);
                }
            }
        }
        // off[p] = sum of the group log-decays over [lo_p, sg), lo_p the end of
        // the block of bit p; the ranges nest, so one pass over the longest one
        // (from 2^(top bit)) serves every bit.
        if (wave == 0 && sg > 0) {
            const int top = 31 - __builtin_clz((unsigned)sg);
            for (int p = 0; p < Plev; ++p)
                if (lane == p)
                    sm.off[p] = 0.f;
            for (int base = 1 << top; base < sg; base += 64) {
                const int j = base + lane;
                const float gj = (j < sg) ? Gam[(size_t)bh * nG + j] : 0.f;
                for (int p = 0; p <= top; ++p) {
                    if (!((sg >> p) & 1))
                        continue;
                    const int lo = ((sg >> (p + 1)) << (p + 1)) + (1 << p);
                    const float t = wave_prefix_sum(j >= lo ? gj : 0.f);
                    if (lane == 63)
                        sm.off[p] += t;
                }
            }
        }
        if (gi == 0)
            __syncthreads();  // prologue
        float gap[kMaxGroupLog2];
#pragma unroll
        for (int m = 0; m < kMaxGroupLog2; ++m)
            gap[m] = 0.f;
        float agrun = 0.f;
        for (int ci = 0; ci < nchunk; ++ci, ++kk) {
            const int b = kk & 1;
            const int valid = min(F::C, Tlen - t0g - ci * F::C);
            const size_t row0 = rowg + (size_t)ci * F::C;
            __syncthreads();  // A
            const float gch = sm.gch[b];
            const float *lamr = sm.lam[b];   // lambda of token i, level l at i * L + l
            const float *Aloc = sm.Aloc[b];
            int iq[F::QPW];
            float ai[F::QPW];
            Frag qf[F::QPW][F::NUK];
#pragma unroll
            for (int x = 0; x < F::QPW; ++x) {
                iq[x] = 16 * F::qtile(qg, x) + li;
                ai[x] = Aloc[iq[x]];
#pragma unroll
                for (int uk = 0; uk < F::NUK; ++uk)
                    qf[x][uk] = qk_frag<F>(sm.Qs[b], iq[x], uk, qd);
            }
            // Causal score tiles (jt, it) of the group's query tiles, dealt
            // round-robin to its column-group waves; masked by decay and level
            // weight and stored as P[i][j].  The diagonal tiles (dearer to
            // mask) take positions 1 .. QPW of the deal and the others fill
            // the rest, so no wave gets two diagonal tiles.
            {
                int noff = 0;
#pragma unroll
                for (int x = 0; x < F::QPW; ++x) {
                    const int it = F::qtile(qg, x);
                    const int i = iq[x];
                    for (int jt = 0; jt <= it; ++jt) {
                        const int n = (jt == it) ? 1 + x : (noff == 0 ? 0 : noff + F::QPW);
                        noff += (jt != it);
                        if (n % F::NCG != cg)
                            continue;
                        floatx4 s = zero4();
#pragma unroll
                        for (int uk = 0; uk < F::NUK; ++uk)
                            mma_unit(s, qk_frag<F>(sm.Ks[b], 16 * jt + li, uk, qd), qf[x][uk]);
                        float p[4];
                        const floatx4 aj = *reinterpret_cast<const floatx4 *>(Aloc + 16 * jt + 4 * qd);
                        if (jt < it) {
                            const float lm = lamr[i * L + 4 + bitlen_u32((uint32_t)(it ^ jt))];
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                p[r] = s[r] * __expf(ai[x] - aj[r]) * lm;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int j = 16 * jt + 4 * qd + r;
                                float m = 0.f;
                                if (j <= i) {
                                    const int lev = (i == j) ? 0 : bitlen_u32((uint32_t)(i ^ j));
                                    m = __expf(ai[x] - aj[r]) * lamr[i * L + lev];
                                }
                                p[r] = s[r] * m;
                            }
                        }
                        bf16x4 pb;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            pb[r] = (__bf16)p[r];
                        *reinterpret_cast<bf16x4 *>(sm.Ps + i * F::LDP + 32 * (jt >> 1) + pq_pos(jt & 1, qd)) = pb;
                    }
                }
            }
            // This wave's share of the fold (dk unit XU0 + qg of its own
            // output columns) while the helpers finish theirs.
            if constexpr (F::XF) {
                if (ci + 1 < nchunk) {
                    const int kc = __builtin_ctz((unsigned)(ci + 1));
                    float gapc[kMaxGroupLog2];
#pragma unroll
                    for (int m = 0; m < kMaxGroupLog2; ++m)
                        gapc[m] = __expf(gap[m] + gch);
                    Frag kf[F::NUC][2];
                    ws_kfrags<F>(sm, b, F::XU0 + qg, li, qd, kf);
                    ws_fold<F, 0, F::CPW, 1>(sm, kf, b, kc, gapc, F::XU0 + qg, cg * F::CPW, lane, li, qd);
                }
            }
            // The first NPF block states above the group that are not
            // LDS-resident are requested now, so their L2 latency is spent
            // across barrier B and the products before their level.
            Frag dpf[F::NPF][F::CPW][F::NUK];
#pragma unroll
            for (int j = 0; j < F::NPF; ++j)
                if (F::NRES + j < npop) {
                    const T *st = Dg + sm.blk[F::NRES + j];
#pragma unroll
                    for (int cc = 0; cc < F::CPW; ++cc)
#pragma unroll
                        for (int uk = 0; uk < F::NUK; ++uk)
                            dpf[j][cc][uk] = state_frag<F>(st, cg * F::CPW + cc, uk, lane);
                }
            __syncthreads();  // B

            // O^T = V^T P^T for this wave's query and column tiles.
            floatx4 O[F::QPW][F::CPW];
#pragma unroll
            for (int cc = 0; cc < F::CPW; ++cc) {
                const int c = cg * F::CPW + cc;
#pragma unroll
                for (int x = 0; x < F::QPW; ++x)
                    O[x][cc] = zero4();
#pragma unroll
                for (int uc = 0; uc < F::NUC; ++uc) {
                    const Frag vt = tr_frag(sm.Vs[b], F::LDV, uc * F::KB, 16 * c, li, qd);
#pragma unroll
                    for (int x = 0; x < F::QPW; ++x)
                        if (uc * F::KB <= 16 * F::qtile(qg, x) + 15)
                            mma_unit(O[x][cc], vt, pq_frag(sm.Ps, F::LDP, iq[x], uc * F::KB, qd));
                }
            }
            // Levels inside the group (stack slots in LDS).
#pragma unroll
            for (int m = 0; m < kMaxGroupLog2; ++m)
                if (m < g && ((ci >> m) & 1)) {
                    float f[F::QPW];
#pragma unroll
                    for (int x = 0; x < F::QPW; ++x)
                        f[x] = lamr[iq[x] * L + log2C + m + 1] * __expf(ai[x] + gap[m]);
                    walk4_level<F>(O, qf, sm.stk + m * F::SLOT, cg, f, lane);
                }
            // Levels above the group: LDS-resident states, then the
            // prefetched ones, then any others straight from L2.
            for (int ii = 0; ii < npop; ++ii) {
                if (ii >= F::NRES && ii < F::NRES + F::NPF)
                    continue;
                const int p = sm.plist[ii];
                float f[F::QPW];
#pragma unroll
                for (int x = 0; x < F::QPW; ++x)
                    f[x] = lamr[iq[x] * L + log2C + g + 1 + p] * __expf(ai[x] + agrun + sm.off[p]);
                const T *st = (ii < F::NRES) ? sm.Dres + (size_t)ii * F::SLOT : Dg + sm.blk[ii];
                walk4_level<F>(O, qf, st, cg, f, lane);
            }
#pragma unroll
            for (int j = 0; j < F::NPF; ++j)
                if (F::NRES + j < npop) {
                    const int p = sm.plist[F::NRES + j];
                    float f[F::QPW];
#pragma unroll
                    for (int x = 0; x < F::QPW; ++x)
                        f[x] = lamr[iq[x] * L + log2C + g + 1 + p] * __expf(ai[x] + agrun + sm.off[p]);
                    walk4_level_regs<F>(O, qf, dpf[j], f);
                }
            // Output: lane holds O[i][16c + 4qd .. 16c + 4qd + 3] for i = iq[x].
#pragma unroll
            for (int x = 0; x < F::QPW; ++x) {
                if (iq[x] < valid) {
#pragma unroll
                    for (int cc = 0; cc < F::CPW; ++cc) {
                        const int c = cg * F::CPW + cc;
                        typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
                        bf16x4 ob;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            ob[r] = (__bf16)O[x][cc][r];
                        __builtin_nontemporal_store(*reinterpret_cast<const u32x2 *>(&ob),
                                                    reinterpret_cast<u32x2 *>(out + (row0 + iq[x]) * F::DV + 16 * c + 4 * qd));
                    }
                }
            }
            if (ci + 1 < nchunk) {
                const int kc = __builtin_ctz((unsigned)(ci + 1));
#pragma unroll
                for (int m = 0; m < kMaxGroupLog2; ++m)
                    gap[m] = (m == kc) ? 0.f : gap[m] + gch;
            }
            agrun += gch;
        }
    }
}

template <class F>
__global__ __launch_bounds__(F::NT) void ll_chunk_walk_ws(
    const typename F::T *__restrict__ q, const typename F::T *__restrict__ k, const typename F::T *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, typename F::T *__restrict__ out, int Tlen, int L,
    int log2C, int g, int N, int nG, int Plev, int nL, int nLeft, int rqk, const float *__restrict__ Gam,
    const typename F::T *__restrict__ Dg)
{
    __shared__ WalkWSSmem<F> sm;
    const int tid = threadIdx.x, wave = tid >> 6;
    // Work item of this workgroup.  Workgroups b, b+8, b+16, ... run on the
    // same XCD (and share its L2); each XCD gets a contiguous range of items,
    // so the block states a head's groups read stay in one L2.  Items run
    // over (q/k head, group pair, head of that q/k head), so the rqk heads
    // that read the same q and k chunks run side by side on one XCD.
    const int nb = (int)gridDim.x, bid = (int)blockIdx.x;
    const int per = nb >> 3, rem = nb & 7, xcd = bid & 7;
    const int wid = xcd * per + min(xcd, rem) + (bid >> 3);
    const int npair = (nG + 1) >> 1;
    const int qbh = wid / (npair * rqk), pr = (wid / rqk) % npair;
    const int bh = qbh * rqk + wid % rqk;
    const int G = 1 << g;
    WSGroups gr;
    gr.sg0 = pr;
    gr.sg1 = nG - 1 - pr;
    gr.n = (gr.sg1 != pr) ? 2 : 1;
    gr.n0 = min(G, N - pr * G);
    gr.n1 = (gr.n == 2) ? min(G, N - gr.sg1 * G) : 0;
    if (wave >= F::NX)
        ws_helper<F>(sm, q, k, v, a, lam, Tlen, L, bh, qbh, gr, G, tid - 64 * F::NX);
    else
        ws_compute<F>(sm, out, Tlen, L, log2C, g, bh, gr, nG, Plev, nL, nLeft, Gam, Dg, tid);
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
static hipError_t launch_fwd_t(const FwdArgs &A, const FwdPlan &P, hipStream_t s, bool *nat_blocks)
{
    using T = typename F::T;
    const int BH = A.B * A.H;
    char *ws = static_cast<char *>(A.workspace);
    float *Sg = reinterpret_cast<float *>(ws + P.off_Sg);
    float *Gam = reinterpret_cast<float *>(ws + P.off_Gam);
    T *Dg = reinterpret_cast<T *>(ws + P.off_Dg);
    const int log2C = bit_length(F::C) - 1;
    using W4 = Walk4<typename F::DTag, F::DK, F::DV, F::C>;
    using WS = WalkWS<typename F::DTag, F::DK, F::DV, F::C>;
    bool use_ws = false;
    if constexpr (F::TR && WS::FITS) {
        // 32-bit buffer offsets within one head.
        const bool fits32 = (int64_t)A.T * (F::DK > F::DV ? F::DK : F::DV) * 2 < ((int64_t)1 << 31) &&
                            (int64_t)A.T * A.L * 4 < ((int64_t)1 << 31);
        use_ws = A.L <= WS::NLV && fits32;
    }
    if (A.tree_only)
        use_ws = A.tree_nat;
    if (nat_blocks)
        *nat_blocks = use_ws;
    if (A.tree_yfrag && (!F::TR || F::DV % 32 != 0 || !A.tree_only || !A.tree_nat))
        return hipErrorInvalidValue;   // the backward's fragment order: bf16, dv units of 32
    if (A.tree_nodes && !A.tree_yfrag)
        return hipErrorInvalidValue;   // nodes come only in the backward's fragment order
    if (P.nL > 0 || (A.tree_only && A.tree_nodes)) {
        ProfEvents pe = prof_events("ll_group_state");
        const bool nodes = A.tree_only && A.tree_nodes;
        hipExtLaunchKernelGGL(ll_group_state<F>, dim3(BH * (nodes ? P.nG : P.nL)), dim3(F::NT), 0, s, pe.start,
                              pe.stop, 0, (const T *)A.k, (const T *)A.v, A.a, A.T, P.g, P.nG, P.nL, A.rqk, Sg, Gam,
                              nodes ? (T *)A.tree_nodes : nullptr, nodes ? A.tree_gamc : nullptr, P.N);
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
        // (node mode with a single group: no tree)
        while (nleaves > 0) {
            const int ntiles = (nleaves + 63) / 64;
            const int complete = nleaves / 64;
            pe = prof_events("ll_left_tree");
            const dim3 tg(4 * F::NUK, ntiles, BH), tb(TreeGeom<F>::NTH);
            float *tt = complete > 0 ? tot[ping] : nullptr;
            bool nat = false;
            if constexpr (F::TR) {
                nat = use_ws;
                if (nat && A.tree_yfrag)
                    hipExtLaunchKernelGGL(ll_left_tree<F, (F::DV % 32 == 0) ? 2 : 1>, tg, tb, 0, s, pe.start, pe.stop, 0, leaves, gleaves,
                                          nleaves, lstride, gstride, p0, P.nL, P.nLeft, Dg, tt, gtot[ping], ntiles);
                else if (nat)
                    hipExtLaunchKernelGGL(ll_left_tree<F, 1>, tg, tb, 0, s, pe.start, pe.stop, 0, leaves, gleaves,
                                          nleaves, lstride, gstride, p0, P.nL, P.nLeft, Dg, tt, gtot[ping], ntiles);
            }
            if (!nat)
                hipExtLaunchKernelGGL(ll_left_tree<F, 0>, tg, tb, 0, s, pe.start, pe.stop, 0, leaves, gleaves,
                                      nleaves, lstride, gstride, p0, P.nL, P.nLeft, Dg, tt, gtot[ping], ntiles);
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
    if (A.tree_only)
        return hipSuccess;
    const ProfEvents pw = prof_events("ll_chunk_walk");
    if constexpr (F::TR && WS::FITS) {
        if (use_ws) {
            hipExtLaunchKernelGGL(ll_chunk_walk_ws<WS>, dim3(BH * ((P.nG + 1) / 2)), dim3(WS::NT), 0, s, pw.start,
                                  pw.stop, 0, (const T *)A.q, (const T *)A.k, (const T *)A.v, A.a, A.lam, (T *)A.out,
                                  A.T, A.L, log2C, P.g, P.N, P.nG, P.Plev, P.nL, P.nLeft, A.rqk, (const float *)Gam,
                                  (const T *)Dg);
            return hipGetLastError();
        }
    }
    if constexpr (F::TR && W4::FITS) {
        hipExtLaunchKernelGGL(ll_chunk_walk<W4>, dim3(BH * P.nG), dim3(W4::NT), 0, s, pw.start, pw.stop, 0,
                              (const T *)A.q, (const T *)A.k, (const T *)A.v, A.a, A.lam, (T *)A.out, A.T, A.L,
                              log2C, P.g, P.N, P.nG, P.Plev, P.nL, P.nLeft, A.rqk, (const float *)Gam,
                              (const T *)Dg);
    } else {
        using FW = Fwd<typename F::DTag, F::DK, F::DV, F::C, true>;
        hipExtLaunchKernelGGL(ll_chunk_walk_rs<FW>, dim3(BH * P.nG), dim3(FW::NT), 0, s, pw.start, pw.stop, 0,
                              (const T *)A.q, (const T *)A.k, (const T *)A.v, A.a, A.lam, (T *)A.out, A.T, A.L,
                              log2C, P.g, P.N, P.nG, P.Plev, P.nL, P.nLeft, A.rqk, (const float *)Gam,
                              (const T *)Dg);
    }
    return hipGetLastError();
}

typedef hipError_t (*FwdLauncher)(const FwdArgs &, const FwdPlan &, hipStream_t, bool *);

template <class DT, int DK, int DV, int C>
static FwdLauncher pick_c()
{
    if constexpr (DK % DT::KB != 0) {
        return nullptr;
    } else if constexpr (sizeof(WalkSmem<Fwd<DT, DK, DV, C, true>>) > 160 * 1024) {
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

hipError_t fwd_launch(const FwdArgs &args, const FwdPlan &plan, hipStream_t stream, bool *nat_blocks)
{
    FwdLauncher f = find_fwd(args.bf16, args.dk, args.dv, args.chunk);
    if (!f)
        return hipErrorInvalidValue;
    return f(args, plan, stream, nat_blocks);
}

}  // namespace ll
