// Backward pass of log-linear attention (Mamba-2 form) for gfx950.
//
// Gradients of sum_t do_t . o_t, with P(t,s) = w(t,s) (q_t.k_s)(do_t.v_s)
// and w(t,s) = exp(sum_{r=s+1..t} a_r) lambda_t[level(t,s)]:
//   dq_t        = sum_{s<=t} w(t,s) (do_t.v_s) k_s
//   dk_s        = sum_{t>=s} w(t,s) (do_t.v_s) q_t
//   dv_s        = sum_{t>=s} w(t,s) (q_t.k_s) do_t
//   dlambda_t[l]= sum_{s in bucket l of t} exp(sum a) (q_t.k_s)(do_t.v_s)
//   da_r        = sum_{t>=r} (sum_s P(t,s) - sum_t' P(t',t)),  r >= 1;  da_0 = 0
// The pages name backpropagation through the per-level weights as needing
// custom kernels ("Log-Linear Attention", French page §5 "Signification et
// Limites"); the chunkwise split mirrors the forward's intra- and inter-chunk
// parts (Portuguese page §2 "Forma Recorrente e Paralela").
//
// How each part is computed:
//  - dq: with bf16 inputs the chunk kernel forms it.  Inside the chunk,
//    dQ = (M.dP) K from the same masked matrix as dk; at a chunk level where
//    the chunk reads a left block, Y = D do_t from that block's state D gives
//    both dlambda_t = exp(decay) q_t . Y_t and dq_t += lambda_t exp(decay) Y_t.
//    Otherwise dq is the forward itself with the roles q <- do, k <- v,
//    v <- k (it weights by lambda of the output position, as dq does), run on
//    the forward kernels.
//  - Inside a chunk, the masked C x C matrices S = Q K^T and dP = dO V^T give
//    dk and dv ((M.dP)^T Q, (M.S)^T dO) and the in-chunk levels of dlambda
//    (row sums of exp(decay) S dP over each level's key range).
//  - A chunk-level bucket m of query chunk c is a left-child block of the tree
//    over chunks (one chunk per group), whose state sum exp(decay) k v^T the
//    forward's tree kernels store; dlambda_t[log2 C + m] = exp(decay) q_t^T D do_t.
//  - For key chunk c and a level m whose bit m-1 of c is clear, the queries
//    that see c at level m form the right sibling block R.  Its state
//    W = sum_{t in R} exp(A_t - A_e) lambda_t[log2 C + m] q_t do_t^T (e the
//    last key before R) gives dk_s += exp(A_e - A_s) W v_s and
//    dv_s += exp(A_e - A_s) W^T k_s.  W is built in two passes: pieces of up
//    to WP chunks (ll_bwd_wpiece), then their sum written as the two MFMA
//    operand layouts the chunk kernel reads (ll_bwd_wsum).
//  - da_r, the sum of P over the pairs s < r <= t, is assembled without
//    differences of large sums: for r in chunk c, the in-chunk pairs come from
//    the chunk's fp32 products, the pairs with one end in c from the chunk's
//    query-side and key-side sums, and the pairs that jump over c from the
//    per-level pair masses of the chunks of c's sibling block at each level
//    (ll_bwd_da).  (The textbook form, a reverse prefix sum of
//    sum_s P(t,s) - sum_t' P(t',t), cancels nearly every pair and amplifies
//    bf16 rounding with the sequence length.)
//
// Every product runs on MFMA with both operands in the natural k order: an
// operand fragment is EPL consecutive elements of one row (16 bytes).
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

template <class DT, int DK_, int DV_, int C_>
struct Bw {
    using T = typename DT::T;
    using Frag = typename DT::Frag;
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr int NT = 256;
    static constexpr int KB = DT::KB, EPL = DT::EPL;
    static constexpr int PAD = 16 / (int)sizeof(T);     // one 16-byte piece of padding per LDS row
    static constexpr int LQ = DK + PAD, LV = DV + PAD, LC = C + PAD;
    static constexpr int CT = C / 16, DKT = DK / 16, DVT = DV / 16;
    static constexpr int NUK = DK / KB, NUV = DV / KB, NUC = C / KB;
    // Chunk kernel: 8 waves when the dk and dv tiles split evenly over the
    // column groups, else 4.
    static constexpr int NW = (DKT % (8 / CT) == 0 && DVT % (8 / CT) == 0) ? 8 : 4;
    static constexpr int NTC = 64 * NW;
    static constexpr int NCG = NW / CT;                   // column groups per token tile
    static constexpr int KPW = DKT / NCG, VPW = DVT / NCG;  // dk / dv tiles per wave
    static constexpr int LOGC = C == 16 ? 4 : C == 32 ? 5 : 6;
    static constexpr int WP = 8;                          // chunks per W piece
    static constexpr int VEC = 16 / (int)sizeof(T);
    // bf16: token-indexed operands are read with transpose reads from the
    // row-major tiles; fp32 keeps transposed copies
    static constexpr bool TRD = DT::is_bf16;
    // LDS copy of one level's state (W and W^T with padded rows, or a block
    // state in fragment order), shared by all waves
    static constexpr int LW1 = DV + PAD, LW2 = DK + PAD;
    static constexpr int SSZ = DK * LW1 + DV * LW2;
    static constexpr int NSP = 2 * DK * DV / VEC;         // 16-byte pieces of a level's state
    static_assert(C % KB == 0 && DK % KB == 0 && DV % KB == 0, "units");
    static_assert(CT >= 1 && CT <= 4 && 4 % CT == 0 && DKT % NCG == 0 && DVT % NCG == 0, "wave layout");
    static_assert((C * kMaxLevels) % NTC == 0, "lambda staging");
};

template <class B>
struct BwSmemBase {
    using T = typename B::T;
    __attribute__((aligned(16))) T Qs[B::C][B::LQ];    // q rows
    __attribute__((aligned(16))) T QsT[B::TRD ? 1 : B::DK][B::TRD ? 8 : B::LC];  // q, [dk][token] (fp32)
    __attribute__((aligned(16))) T Ks[B::C][B::LQ];
    __attribute__((aligned(16))) T Vs[B::C][B::LV];
    __attribute__((aligned(16))) T dOs[B::C][B::LV];
    __attribute__((aligned(16))) T dOsT[B::TRD ? 1 : B::DV][B::TRD ? 8 : B::LC];
    __attribute__((aligned(16))) T PdT[B::C][B::LC];   // (M . dP)^T, [key][query]
    __attribute__((aligned(16))) T PsT[B::C][B::LC];   // (M . S)^T
    float G[B::C][B::C + 1];                            // exp(decay) S dP, [query][key]
    float lam[B::C][kMaxLevels + 1];                    // odd row stride: per-thread rows hit distinct banks
    float dlam[B::C][kMaxLevels + 1];
    float Aloc[B::C];                                   // inclusive prefix of a inside the chunk
    float part[8][B::C];                                // cross-wave row partial sums
    float off[kMaxLevels];                              // per-level log-decay offsets (chunk totals)
    float km[kMaxLevels];                               // key-side pair mass of this chunk per level
    // per-level partial sums of the level loop (a slot per level, so the loop
    // needs no barrier): query side [level][column group][token], key side
    // [level][wave]
    float lpart[kMaxLevels - B::LOGC][B::NCG][B::C];
    float lkw[kMaxLevels - B::LOGC][B::NW];
    float u[B::C], w[B::C];                             // per-token terms of the in-chunk part of da
    float kin[B::CT][B::C];                             // in-chunk pair masses of each key, per query tile
};

// The shared level-state buffer when it fits next to the rest.
template <class B>
struct BwSt {
    static constexpr bool SST = sizeof(BwSmemBase<B>) + (size_t)B::SSZ * sizeof(typename B::T) + 64 <= 160 * 1024;
};

template <class B>
struct BwSmem : BwSmemBase<B> {
    __attribute__((aligned(16))) typename B::T st[BwSt<B>::SST ? B::SSZ : 8];
};

// bf16 with the level states staged in LDS: the chunk kernel also forms dq
// (the in-chunk part from (M . dP) K, the chunk levels from the left block
// states it reads for dlambda), so no separate dq pass runs.
template <class B>
struct BwDq {
    static constexpr bool on = B::TRD && BwSt<B>::SST;
};

// Operand fragment: EPL consecutive elements of row `row` starting at unit u.
template <class B>
__device__ __forceinline__ typename B::Frag frag(const typename B::T *base, int ld, int row, int u, int qd)
{
    return *reinterpret_cast<const typename B::Frag *>(base + (size_t)row * ld + B::KB * u + B::EPL * qd);
}

// B-operand fragment (n-tile nt, k-unit u) of a state stored in fragment
// order with NU units along k.
template <class B, int NU>
__device__ __forceinline__ typename B::Frag gfrag(const typename B::T *st, int nt, int u, int lane)
{
    return *reinterpret_cast<const typename B::Frag *>(st + ((size_t)(nt * NU + u) * 64 + lane) * B::EPL);
}

template <class T>
__device__ __forceinline__ void put(T *p, float x)
{
    *p = from_f32<T>(x);
}

// Store element e (a compile-time index after unrolling) of a 16-byte piece
// as raw bits.
__device__ __forceinline__ void store_elem(float *dst, const uint4 &u, int e)
{
    const uint32_t w = e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
    *reinterpret_cast<uint32_t *>(dst) = w;
}

__device__ __forceinline__ void store_elem(__bf16 *dst, const uint4 &u, int e)
{
    const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
    *reinterpret_cast<unsigned short *>(dst) = (unsigned short)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

// Four consecutive elements of LDS as floats (one 8- or 16-byte read).
__device__ __forceinline__ floatx4 ld4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

__device__ __forceinline__ floatx4 ld4(const __bf16 *p)
{
    const bf16x4 y = *reinterpret_cast<const bf16x4 *>(p);
    return floatx4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}

// Four consecutive elements from an accumulator (8- or 16-byte store).
__device__ __forceinline__ void put4(float *p, const floatx4 &x)
{
    *reinterpret_cast<floatx4 *>(p) = x;
}

__device__ __forceinline__ void put4(__bf16 *p, const floatx4 &x)
{
    bf16x4 y;
    y[0] = (__bf16)x[0]; y[1] = (__bf16)x[1]; y[2] = (__bf16)x[2]; y[3] = (__bf16)x[3];
    *reinterpret_cast<bf16x4 *>(p) = y;
}

// Buffer resource over `bytes` bytes at p: loads past the range return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bw_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bw_load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// Chunk kernel: one workgroup per (head, chunk).
// ---------------------------------------------------------------------------
template <class B>
__global__ __launch_bounds__(B::NTC) void ll_bwd_chunk(
    const typename B::T *__restrict__ q, const typename B::T *__restrict__ k, const typename B::T *__restrict__ v,
    const typename B::T *__restrict__ dout, const float *__restrict__ a, const float *__restrict__ lamg,
    const typename B::T *__restrict__ Dg, const typename B::T *__restrict__ Nd, int gq,
    const double *__restrict__ Gp, const typename B::T *__restrict__ W1,
    const typename B::T *__restrict__ W2, typename B::T *__restrict__ dqg, typename B::T *__restrict__ dkg,
    typename B::T *__restrict__ dvg,
    float *__restrict__ dlamg, float *__restrict__ daloc, float *__restrict__ Mq, float *__restrict__ Mk, int Tlen,
    int L, int N, int nL, int nLeft, int NB)
{
    using T = typename B::T;
    using Frag = typename B::Frag;
    constexpr int C = B::C, DK = B::DK, DV = B::DV;
    __shared__ BwSmem<B> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, qd = lane >> 4;
    // Workgroups b, b+8, ... run on the same XCD and share its L2: give each
    // XCD a contiguous range of (head, chunk) items, so the chunks that read
    // the same level states read them through one L2.
    const int nb = gridDim.x, bid = blockIdx.x;
    const int per = nb >> 3, rem = nb & 7, xcd = bid & 7;
    const int wid = xcd * per + min(xcd, rem) + (bid >> 3);
    const int bh = wid / N, c = wid % N;
    const int t0 = c * C;
    const int nv = min(C, Tlen - t0);   // valid rows of this chunk
    const size_t row0 = (size_t)bh * Tlen + t0;

    const int mtop = bitlen_u32((uint32_t)(N - 1));

    // Level sources: kind 1 = query side (the left block is a stored block
    // state), 2 = key side (the right block R exists), 0 = nothing.
    auto kind_of = [&](int m) __attribute__((always_inline)) {
        if (m > mtop)
            return 0;
        if ((c >> (m - 1)) & 1)
            return 1;
        return ((c >> m) << m) + (1 << (m - 1)) < N ? 2 : 0;
    };
    // level m's state in global memory: p1 (the block state, or W) and p2
    // (W^T when stored, else p1)
    struct StatePtr {
        const T *p1, *p2;
    };
    auto state_ptr = [&](int m, int kind) __attribute__((always_inline)) {
        // the bases read up front and chosen by value (a choice between the
        // addresses of the captured pointers would keep them in scratch)
        const T *const nd = Nd, *const dg = Dg, *const w1 = W1, *const w2 = W2;
        size_t o;
        int src;
        if (kind == 1) {
            if (m <= gq) {
                // inside a group of 2^gq chunks: the Fenwick node of the left
                // block's last chunk
                const int e = ((c >> m) << m) + (1 << (m - 1)) - 1;
                o = (size_t)bh * N + e;
                src = 0;
            } else {
                // a left block of the tree over groups, at level m - 1 - gq
                size_t offp = 0;
                for (int r = 0; r < m - 1 - gq; ++r)
                    offp += ((nL >> r) + 1) >> 1;
                o = (size_t)bh * nLeft + offp + (c >> m);
                src = 1;
            }
        } else {
            size_t ob = 0;
            for (int r = 1; r < m; ++r) {
                const int hr = 1 << (r - 1);
                ob += N > hr ? (N - hr + (1 << r) - 1) >> r : 0;
            }
            o = (size_t)bh * NB + ob + (c >> m);
            src = 2;
        }
        o *= (size_t)DK * DV;
        const T *p1 = (src == 0 ? nd : src == 1 ? dg : w1) + o;   // block state, or W [dk][dv]
        const T *p2 = src == 2 && w2 ? w2 + o : p1;                 // W^T [dv][dk] when stored
        return StatePtr{p1, p2};
    };

    // bf16 with staged level states: the key-side levels (kind 2) are not
    // multiplied one by one.  With delta_s = exp(A_end - A_s) and rho_m the
    // decay from the chunk's end to R_m's start, the key-side terms of all
    // levels are delta_s (sum_m rho_m W_m) v_s for dk and the transposed
    // product for dv; the level's pair mass is rho_m <W_m, X>, where
    // X = sum_s delta_s k_s v_s^T.  So the W_m are read straight into
    // registers (in X's accumulator layout: row d, four consecutive e),
    // summed in fp32, and one product with the sum replaces a product per
    // level.
    constexpr bool KS = BwDq<B>::on;
    constexpr int NXT = (B::DKT * B::DVT + B::NW - 1) / B::NW;   // X tiles per wave
    constexpr int PRE = KS ? (16 / NXT < 1 ? 1 : 16 / NXT > 4 ? 4 : 16 / NXT) : 1;   // levels per batch
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    uint32_t k2 = 0;   // the key-side levels, bit m
    if constexpr (KS) {
        for (int m = 1; m <= mtop; ++m)
            if (kind_of(m) == 2)
                k2 |= 1u << m;
    }
    u32x2 wr[PRE][NXT];
    // loads the first PRE levels of `mask` into wr
    auto load_k2 = [&](uint32_t mask) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
            // a slot past the last level reads nothing (an empty range)
            const int m = mask ? __builtin_ctz(mask) : 1;
            const __amdgpu_buffer_rsrc_t r = bw_rsrc(state_ptr(m, 2).p1, mask ? DK * DV * (int)sizeof(T) : 0);
            mask &= mask - 1;
#pragma unroll
            for (int t = 0; t < NXT; ++t) {
                const int ti = wv * NXT + t;
                const int d = 16 * (ti / B::DVT) + li, e0 = 16 * (ti % B::DVT) + 4 * qd;
                const int off = ti < B::DKT * B::DVT ? (d * DV + e0) * (int)sizeof(T) : DK * DV * (int)sizeof(T);
                wr[j][t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
            }
        }
    };

    // ---- stage the chunk: 16-byte pieces, every load issued first ------------
    // All of the item's loads go out together, so that it waits for one round
    // trip: q, k, v, dO, lambda rows (contiguous, C*L floats), a, the fp64
    // chunk prefix for the level offsets, the key-side level states and the
    // first query-side level state.  They are buffer loads over the valid
    // range (zero beyond it) issued on every path: a load skipped on some
    // path would make the compiler wait for all loads before the first use.
    constexpr int VEC = B::VEC, QP = C * DK / VEC, VP = C * DV / VEC;
    constexpr int NQP = (QP + B::NTC - 1) / B::NTC, NVP = (VP + B::NTC - 1) / B::NTC;
    uint4 rq[NQP], rk[NQP], rv[NVP], ro[NVP];
    {
        const uint32_t nq = (uint32_t)(nv * DK * sizeof(T)), nvb = (uint32_t)(nv * DV * sizeof(T));
        const __amdgpu_buffer_rsrc_t r_q = bw_rsrc(q + row0 * DK, nq), r_k = bw_rsrc(k + row0 * DK, nq);
        const __amdgpu_buffer_rsrc_t r_v = bw_rsrc(v + row0 * DV, nvb), r_o = bw_rsrc(dout + row0 * DV, nvb);
#pragma unroll
        for (int j = 0; j < NQP; ++j) {
            const int off = (tid + B::NTC * j) * 16;
            rq[j] = bw_load16(r_q, off);
            rk[j] = bw_load16(r_k, off);
        }
#pragma unroll
        for (int j = 0; j < NVP; ++j) {
            const int off = (tid + B::NTC * j) * 16;
            rv[j] = bw_load16(r_v, off);
            ro[j] = bw_load16(r_o, off);
        }
    }
    static_assert(C <= 64, "one wave scans a");
    constexpr int NLL = C * kMaxLevels / B::NTC;
    float lv[NLL];
    {
        const __amdgpu_buffer_rsrc_t r_l = bw_rsrc(lamg + row0 * L, (uint32_t)(nv * L * 4));
#pragma unroll
        for (int j = 0; j < NLL; ++j)
            lv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_l, (tid + B::NTC * j) * 4, 0, 0));
    }
    const float av = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(bw_rsrc(a + row0, (uint32_t)(nv * 4)), lane * 4, 0, 0));
    // Per level: the log-decay between this chunk and the other block, from
    // the fp64 prefix of chunk totals (query side: from the left block's end
    // to this chunk's start; key side: from this chunk's end to R's start).
    // Thread m reads the two prefix entries of level m (none: past the end).
    double gpa, gpb;
    {
        int ia = N, ib = N;
        if (tid >= 1 && tid <= mtop) {
            const int m = tid, half = 1 << (m - 1), b0 = (c >> m) << m;
            if ((c >> (m - 1)) & 1) {
                ia = c;
                ib = b0 + half;
            } else if (b0 + half < N) {
                ia = b0 + half;
                ib = c + 1;
            }
        }
        const __amdgpu_buffer_rsrc_t r_g = bw_rsrc(Gp + (size_t)bh * N, (uint32_t)N * 8);
        gpa = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r_g, ia * 8, 0, 0));
        gpb = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r_g, ib * 8, 0, 0));
    }
    if constexpr (KS)
        load_k2(k2);
    constexpr bool SST = BwSt<B>::SST;
    constexpr int HP = DK * DV / VEC;   // pieces of one state
    // pieces of one level's LDS copy: the state (W and W^T when both are kept)
    // (not used when dq is formed here)
    constexpr int NSPT = BwDq<B>::on ? 1 : (2 * HP + B::NTC - 1) / B::NTC;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    // the next level's state pieces of the level loop (loaded one level ahead)
    u32x4 sp[NSPT];
    // the levels the level loop takes (bit m)
    auto loop_kind = [&](int m) __attribute__((always_inline)) {
        const int kd = kind_of(m);
        return KS && kd == 2 ? 0 : kd;
    };
    uint32_t lmask = 0;
    for (int m = 1; m <= mtop; ++m)
        if (loop_kind(m) != 0)
            lmask |= 1u << m;
    // loads level mn's state into sp (mn = 0: none, zeros)
    auto load_sp = [&](int mn) __attribute__((always_inline)) {
        const int nk = mn ? loop_kind(mn) : 0;
        const StatePtr sq = state_ptr(mn ? mn : 1, nk ? nk : 1);
        const bool two = nk == 2;   // W and W^T
        const __amdgpu_buffer_rsrc_t r1 = bw_rsrc(sq.p1, nk ? HP * 16 : 0), r2 = bw_rsrc(sq.p2, two ? HP * 16 : 0);
#pragma unroll
        for (int j = 0; j < NSPT; ++j) {
            const int i = tid + B::NTC * j;
            if (B::NTC * (j + 1) <= HP) {
                sp[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, i * 16, 0, 0));
            } else if (B::NTC * j >= HP) {
                sp[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, (i - HP) * 16, 0, 0));
            } else {
                // pieces on both sides of HP: one of the two loads is out of range
                sp[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, i * 16, 0, 0)) |
                        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, (i - HP) * 16, 0, 0));
            }
        }
    };
    if constexpr (SST && !BwDq<B>::on)
        load_sp(lmask ? __builtin_ctz(lmask) : 0);   // (with dq formed here: in the level loop)
#pragma unroll
    for (int j = 0; j < NQP; ++j) {
        const int i = tid + B::NTC * j;
        if (i < QP) {
            const int t = i / (DK / VEC), d0 = (i % (DK / VEC)) * VEC;
            *reinterpret_cast<uint4 *>(&sm.Qs[t][d0]) = rq[j];
            *reinterpret_cast<uint4 *>(&sm.Ks[t][d0]) = rk[j];
            if constexpr (!B::TRD) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    store_elem(&sm.QsT[d0 + e][t], rq[j], e);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NVP; ++j) {
        const int i = tid + B::NTC * j;
        if (i < VP) {
            const int t = i / (DV / VEC), e0 = (i % (DV / VEC)) * VEC;
            *reinterpret_cast<uint4 *>(&sm.Vs[t][e0]) = rv[j];
            *reinterpret_cast<uint4 *>(&sm.dOs[t][e0]) = ro[j];
            if constexpr (!B::TRD) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    store_elem(&sm.dOsT[e0 + e][t], ro[j], e);
            }
        }
    }
    for (int i = tid; i < C * B::LC * (int)sizeof(T) / 16; i += B::NTC) {
        reinterpret_cast<uint4 *>(&sm.PdT[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4 *>(&sm.PsT[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    {
        for (int i = tid; i < C * (kMaxLevels + 1); i += B::NTC) {
            (&sm.lam[0][0])[i] = 0.f;
            (&sm.dlam[0][0])[i] = 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NLL; ++j) {
            const int i = tid + B::NTC * j;
            if (i < nv * L)
                sm.lam[i / L][i % L] = lv[j];
        }
    }
    if (tid < kMaxLevels)
        sm.km[tid] = 0.f;
    if (tid >= 1 && tid <= mtop)
        sm.off[tid] = (float)(gpa - gpb);
    if (wv == 0) {
        // inclusive prefix of a over the chunk (zero past the end)
        float x = av;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (lane >= d)
                x += y;
        }
        if (lane < C)
            sm.Aloc[lane] = x;
    }
    __syncthreads();
    if constexpr (KS) {
        static_assert(C * B::LV <= B::SSZ, "delta V fits the state buffer");
        // delta_s v_s (bf16) into the state buffer, for X
#pragma unroll
        for (int j = 0; j < NVP; ++j) {
            const int i = tid + B::NTC * j;
            if (i < VP) {
                const int t = i / (DV / VEC), e0 = (i % (DV / VEC)) * VEC;
                const float dl = __expf(sm.Aloc[C - 1] - sm.Aloc[t]);
                const uint4 x = rv[j];
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                uint32_t o[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float lo = __uint_as_float(w[h] << 16) * dl, hi = __uint_as_float(w[h] & 0xffff0000u) * dl;
                    const __bf16 blo = (__bf16)lo, bhi = (__bf16)hi;
                    o[h] = (uint32_t)__builtin_bit_cast(unsigned short, blo) |
                           ((uint32_t)__builtin_bit_cast(unsigned short, bhi) << 16);
                }
                *reinterpret_cast<uint4 *>(sm.st + t * B::LV + e0) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }

    // ---- in-chunk scores: S = Q K^T, dP = dO V^T, causal tile pairs ---------
    for (int pr = wv; pr < B::CT * (B::CT + 1) / 2; pr += B::NW) {
        int tt = 0, rem = pr;
        while (rem > tt) {
            rem -= tt + 1;
            ++tt;
        }
        const int st = rem;   // st <= tt
        floatx4 S = zero4(), dP = zero4();
#pragma unroll
        for (int u = 0; u < B::NUK; ++u)
            mma_unit(S, frag<B>(&sm.Ks[0][0], B::LQ, 16 * st + li, u, qd),
                     frag<B>(&sm.Qs[0][0], B::LQ, 16 * tt + li, u, qd));
#pragma unroll
        for (int u = 0; u < B::NUV; ++u)
            mma_unit(dP, frag<B>(&sm.Vs[0][0], B::LV, 16 * st + li, u, qd),
                     frag<B>(&sm.dOs[0][0], B::LV, 16 * tt + li, u, qd));
        // accumulator lane layout (A = keys, B = queries): rows 4*qd+i are
        // keys s, column li is query t
        const int t = 16 * tt + li;
        float kin[4];   // the in-chunk pair masses P(t, s) of key s, summed over this tile's queries below
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * st + 4 * qd + i;
            float m = 0.f, g = 0.f, sv = S[i], dpv = dP[i];
            if (s <= t) {
                const float dec = __expf(sm.Aloc[t] - sm.Aloc[s]);
                const int lev = s == t ? 0 : bitlen_u32((uint32_t)(t ^ s));
                m = dec * sm.lam[t][lev];
                g = dec * sv * dpv;
            }
            put(&sm.PdT[s][t], m * dpv);
            put(&sm.PsT[s][t], m * sv);
            sm.G[t][s] = g;
            kin[i] = m * sv * dpv;
        }
        // sum over the 16 queries of the tile (lanes li of one lane quad)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kin[i] += __shfl_xor(kin[i], o, 64);
        if (li == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.kin[tt][16 * st + 4 * qd + i] = kin[i];
    }
    __syncthreads();

    // ---- in-chunk levels of dlambda: row sums of G over each level's keys ----
    for (int task = tid; task < C * (B::LOGC + 1); task += B::NTC) {
        const int t = task / (B::LOGC + 1), lev = task % (B::LOGC + 1);
        float x = 0.f;
        if (lev == 0) {
            x = sm.G[t][t];
        } else if ((t >> (lev - 1)) & 1) {
            const int s0 = (t >> lev) << lev;
            for (int s = s0; s < s0 + (1 << (lev - 1)); ++s)
                x += sm.G[t][s];
        }
        sm.dlam[t][lev] = x;
    }

    // ---- dk, dv accumulators: this wave's key tile and column tiles ----------
    const int kt = wv % B::CT, cg = wv / B::CT;
    floatx4 dK[B::KPW], dV[B::VPW];
#pragma unroll
    for (int j = 0; j < B::KPW; ++j)
        dK[j] = zero4();
#pragma unroll
    for (int j = 0; j < B::VPW; ++j)
        dV[j] = zero4();
    // in-chunk: dK = (M.dP)^T Q, dV = (M.S)^T dO (contraction over queries)
#pragma unroll
    for (int u = 0; u < B::NUC; ++u) {
        if constexpr (B::TRD) {
            // both operands in the permuted token order of the transpose read
            const Frag pd = lds_frag(&sm.PdT[0][0], B::LC, 16 * kt + li, B::KB * u, qd);
            const Frag ps = lds_frag(&sm.PsT[0][0], B::LC, 16 * kt + li, B::KB * u, qd);
#pragma unroll
            for (int j = 0; j < B::KPW; ++j)
                mma_unit(dK[j], tr_frag(&sm.Qs[0][0], B::LQ, B::KB * u, 16 * (cg + B::NCG * j), li, qd), pd);
#pragma unroll
            for (int j = 0; j < B::VPW; ++j)
                mma_unit(dV[j], tr_frag(&sm.dOs[0][0], B::LV, B::KB * u, 16 * (cg + B::NCG * j), li, qd), ps);
        } else {
            const Frag pd = frag<B>(&sm.PdT[0][0], B::LC, 16 * kt + li, u, qd);
            const Frag ps = frag<B>(&sm.PsT[0][0], B::LC, 16 * kt + li, u, qd);
#pragma unroll
            for (int j = 0; j < B::KPW; ++j)
                mma_unit(dK[j], frag<B>(&sm.QsT[0][0], B::LC, 16 * (cg + B::NCG * j) + li, u, qd), pd);
#pragma unroll
            for (int j = 0; j < B::VPW; ++j)
                mma_unit(dV[j], frag<B>(&sm.dOsT[0][0], B::LC, 16 * (cg + B::NCG * j) + li, u, qd), ps);
        }
    }
    // The accumulators hold dK^T and dV^T tiles: A = columns (dk / dv index,
    // rows 4*qd+i), B = keys (column li).
    constexpr bool FDQ = BwDq<B>::on;
    // dq of this wave's token tile (as a query) and dk tiles: in-chunk
    // dQ^T = K^T (M . dP)^T, contraction over the keys s (rows of K and of
    // (M . dP)^T, both read with transpose reads)
    floatx4 dQ[B::KPW];
#pragma unroll
    for (int j = 0; j < B::KPW; ++j)
        dQ[j] = zero4();
    if constexpr (FDQ) {
#pragma unroll
        for (int u = 0; u < B::NUC; ++u) {
            const Frag pdt = tr_frag(&sm.PdT[0][0], B::LC, B::KB * u, 16 * kt, li, qd);
#pragma unroll
            for (int j = 0; j < B::KPW; ++j)
                mma_unit(dQ[j], tr_frag(&sm.Ks[0][0], B::LQ, B::KB * u, 16 * (cg + B::NCG * j), li, qd), pdt);
        }
    }
    // X = sum_s delta_s k_s v_s^T, tiles wv*NXT + t: Xc[t][i] = X[d][e] with
    // d = 16 (tile / DVT) + li, e = 16 (tile % DVT) + 4 qd + i (A = delta V^T,
    // B = K^T, both by transpose reads over the tokens)
    floatx4 Xc[NXT], Wt[NXT];
#pragma unroll
    for (int t = 0; t < NXT; ++t) {
        Xc[t] = zero4();
        Wt[t] = zero4();
    }
    if constexpr (KS) {
#pragma unroll
        for (int t = 0; t < NXT; ++t) {
            const int ti = wv * NXT + t;
            if (ti < B::DKT * B::DVT) {
#pragma unroll
                for (int u = 0; u < B::NUC; ++u)
                    mma_unit(Xc[t], tr_frag(sm.st, B::LV, B::KB * u, 16 * (ti % B::DVT), li, qd),
                             tr_frag(&sm.Ks[0][0], B::LQ, B::KB * u, 16 * (ti / B::DVT), li, qd));
            }
        }
    }
    // adds the levels loaded into wr (the first PRE of `rest`, which drops
    // them): Wt += rho_m W_m, and the level's pair mass per wave
    auto add_k2 = [&](uint32_t &rest) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
            if (rest) {
                const int m = __builtin_ctz(rest);
                rest &= rest - 1;
                const float rho = __expf(sm.off[m]);
                float x = 0.f;
#pragma unroll
                for (int t = 0; t < NXT; ++t) {
                    const u32x2 w = wr[j][t];
                    const floatx4 w4 = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
                    Wt[t] += rho * w4;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        x += w4[i] * Xc[t][i];
                }
                x *= rho;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1)
                    x += __shfl_xor(x, o, 64);
                if (lane == 0)
                    sm.lkw[m][wv] = x;
            }
        }
    };

    // ---- chunk levels -------------------------------------------------------
    // pki: this lane's part of k_s . (dk_s from later chunks), fp32
    float pki = 0.f;
    uint32_t k2rest = k2;   // key-side levels not yet added
    if constexpr (KS) {
        add_k2(k2rest);
        if (k2rest)
            load_k2(k2rest);   // in flight during the query-side levels
    }
    // the level loop: the query-side levels (and the key-side ones when
    // they are not summed).  With dq formed here, the block states are
    // stored in the A-operand fragment order of the product below, and each
    // wave reads its fragments straight into registers, one level ahead (no
    // LDS copy, no barriers); otherwise, with the state copy in LDS, each
    // level's state was loaded one level ahead (the first one with the
    // chunk).
    Frag dnx[FDQ ? B::KPW : 1][FDQ ? B::NUV : 1];
    // loads level mn's fragments of this wave's dk tiles into dnx (mn = 0:
    // none, zeros); fragment (dk tile dt, dv unit u) is 64 lanes x 16 bytes
    auto load_df = [&](int mn) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = bw_rsrc(state_ptr(mn ? mn : 1, 1).p1, mn ? HP * 16 : 0);
#pragma unroll
        for (int j = 0; j < B::KPW; ++j)
#pragma unroll
            for (int u = 0; u < B::NUV; ++u)
                dnx[j][u] = __builtin_bit_cast(
                    Frag, __builtin_amdgcn_raw_buffer_load_b128(r, (((cg + B::NCG * j) * B::NUV + u) * 64 + lane) * 16,
                                                                0, 0));
    };
    // the same for every query-side level: this wave's dO fragments (B
    // operand, query tile kt) and q rows of its dk tiles
    Frag dof[FDQ ? B::NUV : 1];
    floatx4 qrow[FDQ ? B::KPW : 1];
    if constexpr (FDQ) {
        load_df(lmask ? __builtin_ctz(lmask) : 0);
#pragma unroll
        for (int u = 0; u < B::NUV; ++u)
            dof[u] = lds_frag(&sm.dOs[0][0], B::LV, 16 * kt + li, B::KB * u, qd);
#pragma unroll
        for (int j = 0; j < B::KPW; ++j)
            qrow[j] = ld4(&sm.Qs[16 * kt + li][16 * (cg + B::NCG * j) + 4 * qd]);
    }
    for (int m = 1; m <= mtop; ++m) {
        if (!((lmask >> m) & 1))
            continue;
        const int kind = loop_kind(m);
        const T *g1 = nullptr, *g2 = nullptr;   // the state in global memory (no LDS copy)
        Frag dcur[FDQ ? B::KPW : 1][FDQ ? B::NUV : 1];
        if constexpr (FDQ) {
#pragma unroll
            for (int j = 0; j < B::KPW; ++j)
#pragma unroll
                for (int u = 0; u < B::NUV; ++u)
                    dcur[j][u] = dnx[j][u];
            const uint32_t above = lmask & ~((2u << m) - 1u);
            load_df(above ? __builtin_ctz(above) : 0);
        } else if constexpr (SST) {
            __syncthreads();   // the previous level's reads of the copy are done
            if (kind != 0) {
                const int np = kind == 1 ? HP : 2 * HP;
#pragma unroll
                for (int j = 0; j < NSPT; ++j) {
                    const int i = tid + B::NTC * j;
                    if (i < np) {
                        T *dst;
                        if (kind == 1) {
                            dst = sm.st + (size_t)i * VEC;                       // fragment order
                        } else if (i < HP) {
                            const int e0 = i * VEC;
                            dst = sm.st + (e0 / DV) * B::LW1 + e0 % DV;          // W rows
                        } else {
                            const int e0 = (i - HP) * VEC;
                            dst = sm.st + DK * B::LW1 + (e0 / DK) * B::LW2 + e0 % DK;   // W^T rows
                        }
                        *reinterpret_cast<u32x4 *>(dst) = sp[j];
                    }
                }
            }
            {
                // the next level of the loop
                const uint32_t above = lmask & ~((2u << m) - 1u);
                load_sp(above ? __builtin_ctz(above) : 0);
            }
            __syncthreads();
        } else if (kind != 0) {
            const StatePtr sq = state_ptr(m, kind);
            g1 = sq.p1;
            g2 = sq.p2;
        }
        if (kind == 1 && FDQ) {
            if constexpr (FDQ) {
                // query side -> dlambda level LOGC + m and dq.  Y^T = D dO^T: A = D
                // (rows d, the fragments read above), B = dO (columns t); this
                // wave takes query tile kt and dk tiles cg, cg + NCG, ...
                // dlambda_t = exp(A_t + off) q_t . Y_t; dq_t += lambda_t exp(A_t + off) Y_t.
                const int t = 16 * kt + li;
                const float fac = sm.lam[t][B::LOGC + m] * __expf(sm.Aloc[t] + sm.off[m]);
                float xs = 0.f;
#pragma unroll
                for (int j = 0; j < B::KPW; ++j) {
                    floatx4 Y = zero4();
#pragma unroll
                    for (int u = 0; u < B::NUV; ++u)
                        mma_unit(Y, dcur[j][u], dof[u]);
                    // Y[i] = (D dO^T)[d = 16 (cg + NCG j) + 4 qd + i][t]
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xs += Y[i] * qrow[j][i];
                    dQ[j] += fac * Y;
                }
                xs += __shfl_xor(xs, 16, 64);
                xs += __shfl_xor(xs, 32, 64);
                if (qd == 0)
                    sm.lpart[m][cg][t] = xs;
            }
        } else if (kind == 1) {
            // query side -> dlambda level LOGC + m.  X^T = D^T Q^T: A = D^T
            // (rows e), B = Q (columns t); this wave takes query tile kt and
            // value tiles cg, cg + NCG, ...
            float xs = 0.f;
#pragma unroll
            for (int j = 0; j < B::VPW; ++j) {
                const int et = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUK; ++u) {
                    const Frag fd = SST ? gfrag<B, B::NUK>(sm.st, et, u, lane) : gfrag<B, B::NUK>(g1, et, u, lane);
                    mma_unit(X, fd, frag<B>(&sm.Qs[0][0], B::LQ, 16 * kt + li, u, qd));
                }
                // X[i] = (Q D)[t = 16 kt + li][e = 16 et + 4 qd + i]
                const floatx4 o4 = ld4(&sm.dOs[16 * kt + li][16 * et + 4 * qd]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xs += X[i] * o4[i];
            }
            // reduce over the four lane quads (the e rows)
            xs += __shfl_xor(xs, 16, 64);
            xs += __shfl_xor(xs, 32, 64);
            if (qd == 0)
                sm.lpart[m][cg][16 * kt + li] = xs;
        } else if (kind == 2) {
            // key side: the right block R sees this chunk at level m
            const float offR = sm.off[m];   // log-decay from the chunk's end to R's start
            // this wave's key rows: decay exp(A_e - A_s)
            const float dec = __expf(sm.Aloc[C - 1] - sm.Aloc[16 * kt + li] + offR);
            float km = 0.f;   // this lane's part of the level's key-side pair mass
#pragma unroll
            for (int j = 0; j < B::KPW; ++j) {
                const int dt = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUV; ++u) {
                    const Frag fw = SST ? frag<B>(sm.st, B::LW1, 16 * dt + li, u, qd)
                                        : frag<B>(g1, DV, 16 * dt + li, u, qd);
                    mma_unit(X, fw, frag<B>(&sm.Vs[0][0], B::LV, 16 * kt + li, u, qd));
                }
                dK[j] += dec * X;
                const floatx4 k4 = ld4(&sm.Ks[16 * kt + li][16 * dt + 4 * qd]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    km += dec * X[i] * k4[i];
            }
#pragma unroll
            for (int j = 0; j < B::VPW; ++j) {
                const int et = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUK; ++u) {
                    if constexpr (FDQ) {
                        // W^T (rows e) by transpose reads of the W copy, k in the
                        // permuted order on both operands
                        mma_unit(X, tr_frag(sm.st, B::LW1, B::KB * u, 16 * et, li, qd),
                                 lds_frag(&sm.Ks[0][0], B::LQ, 16 * kt + li, B::KB * u, qd));
                    } else {
                        const Frag fw = SST ? frag<B>(sm.st + DK * B::LW1, B::LW2, 16 * et + li, u, qd)
                                            : frag<B>(g2, DK, 16 * et + li, u, qd);
                        mma_unit(X, fw, frag<B>(&sm.Ks[0][0], B::LQ, 16 * kt + li, u, qd));
                    }
                }
                dV[j] += dec * X;
            }
            pki += km;
            // the level's key-side pair mass of the chunk: sum over keys of k_s . dk_s(level m)
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                km += __shfl_xor(km, o, 64);
            if (lane == 0)
                sm.lkw[m][wv] = km;
        }
    }
    if constexpr (KS) {
        // the remaining key-side levels, then one product with their sum
        while (k2rest) {
            add_k2(k2rest);
            if (k2rest)
                load_k2(k2rest);
        }
        if (k2) {
            __syncthreads();   // the loop's reads of the state copy are done
#pragma unroll
            for (int t = 0; t < NXT; ++t) {
                const int ti = wv * NXT + t;
                if (ti < B::DKT * B::DVT)
                    put4(sm.st + (16 * (ti / B::DVT) + li) * B::LW1 + 16 * (ti % B::DVT) + 4 * qd, Wt[t]);
            }
            __syncthreads();
            const float dec = __expf(sm.Aloc[C - 1] - sm.Aloc[16 * kt + li]);
            float km = 0.f;
#pragma unroll
            for (int j = 0; j < B::KPW; ++j) {
                const int dt = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUV; ++u)
                    mma_unit(X, frag<B>(sm.st, B::LW1, 16 * dt + li, u, qd),
                             frag<B>(&sm.Vs[0][0], B::LV, 16 * kt + li, u, qd));
                dK[j] += dec * X;
                const floatx4 k4 = ld4(&sm.Ks[16 * kt + li][16 * dt + 4 * qd]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    km += dec * X[i] * k4[i];
            }
#pragma unroll
            for (int j = 0; j < B::VPW; ++j) {
                const int et = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUK; ++u)
                    mma_unit(X, tr_frag(sm.st, B::LW1, B::KB * u, 16 * et, li, qd),
                             lds_frag(&sm.Ks[0][0], B::LQ, 16 * kt + li, B::KB * u, qd));
                dV[j] += dec * X;
            }
            pki += km;
        }
    }
    __syncthreads();
    // the level loop's reductions: dlambda of the query-side levels, the
    // key-side pair masses
    for (int i = tid; i < mtop * C; i += B::NTC) {
        const int m = 1 + i / C, t = i % C;
        if ((c >> (m - 1)) & 1) {
            float x = 0.f;
            for (int g2 = 0; g2 < B::NCG; ++g2)
                x += sm.lpart[m][g2][t];
            sm.dlam[t][B::LOGC + m] = __expf(sm.Aloc[t] + sm.off[m]) * x;
        } else if (t == 0) {
            float x = 0.f;
            if (((c >> m) << m) + (1 << (m - 1)) < N)
                for (int w2 = 0; w2 < B::NW; ++w2)
                    x += sm.lkw[m][w2];
            sm.km[m] = x;
        }
    }
    __syncthreads();

    // ---- outputs ------------------------------------------------------------
    // dk, dv: this wave's key tile kt, column tiles; rows are keys s = 16 kt + li
    const int s = 16 * kt + li;
    float pk = pki;
    if (s < nv) {
        if constexpr (FDQ) {
#pragma unroll
            for (int j = 0; j < B::KPW; ++j)
                put4(&dqg[(row0 + s) * DK + 16 * (cg + B::NCG * j) + 4 * qd], dQ[j]);
        }
#pragma unroll
        for (int j = 0; j < B::KPW; ++j)
            put4(&dkg[(row0 + s) * DK + 16 * (cg + B::NCG * j) + 4 * qd], dK[j]);
#pragma unroll
        for (int j = 0; j < B::VPW; ++j)
            put4(&dvg[(row0 + s) * DV + 16 * (cg + B::NCG * j) + 4 * qd], dV[j]);
    }
    pk += __shfl_xor(pk, 16, 64);
    pk += __shfl_xor(pk, 32, 64);
    if (qd == 0)
        sm.part[cg][s] = pk;
    __syncthreads();
    {
        // da inside the chunk, for r = t0 + i:
        //   sum_{t >= r} (sum of P(t, s) over s <= t) - sum_{s >= r} (in-chunk P(., s))
        //   + sum_{s < r} (P(., s) over later chunks)
        // The in-chunk sums of both sides come from the same fp32 scores S, dP.
        // Four threads per token (quarters of the key / level ranges).
        const int tk = tid >> 2, qq = tid & 3;
        float pki_in = 0.f, pq = 0.f;
        if (tk < C) {
            // key tk's in-chunk pair masses: the query tiles from its own on
            for (int tt = tk / 16 + qq; tt < B::CT; tt += 4)
                pki_in += sm.kin[tt][tk];
            for (int l = qq; l < L; l += 4)
                pq += sm.lam[tk][l] * sm.dlam[tk][l];
        }
        pki_in += __shfl_xor(pki_in, 1, 64);
        pki_in += __shfl_xor(pki_in, 2, 64);
        pq += __shfl_xor(pq, 1, 64);
        pq += __shfl_xor(pq, 2, 64);
        if (tk < C && qq == 0) {
            float pkx = 0.f;
            for (int g2 = 0; g2 < B::NCG; ++g2)
                pkx += sm.part[g2][tk];
            sm.u[tk] = pq - pki_in;
            sm.w[tk] = pkx;
        }
    }
    __syncthreads();
    if (wv == 0) {
        // suffix sum of u and exclusive prefix sum of w over the chunk (C <= 64)
        float su = lane < C ? sm.u[lane] : 0.f, pw = lane < C ? sm.w[lane] : 0.f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_down(su, d, 64);
            if (lane + d < 64)
                su += y;
            const float z = __shfl_up(pw, d, 64);
            if (lane >= d)
                pw += z;
        }
        pw -= lane < C ? sm.w[lane] : 0.f;
        if (lane < nv)
            daloc[row0 + lane] = su + pw;
    }
    // pair masses of this chunk per level (query side: into its left block;
    // key side: from its right block), for the pairs that jump over other
    // chunks; wave w takes levels w+1, w+1+NW, ...
    for (int m = 1 + wv; m <= mtop; m += B::NW) {
        float x = 0.f;
        if ((c >> (m - 1)) & 1)
            for (int t = lane; t < C; t += 64)
                x += sm.lam[t][B::LOGC + m] * sm.dlam[t][B::LOGC + m];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            x += __shfl_xor(x, o, 64);
        if (lane == 0) {
            Mq[((size_t)bh * kMaxLevels + m) * (N + 1) + c] = x;
            Mk[((size_t)bh * kMaxLevels + m) * (N + 1) + c] = sm.km[m];
        }
    }
    for (int i = tid; i < nv * L; i += B::NTC) {
        const int t = i / L, l = i % L;
        dlamg[(row0 + t) * L + l] = sm.dlam[t][l];
    }
}

// ---------------------------------------------------------------------------
// W pieces: for level m, right block R = [j 2^m + 2^(m-1), (j+1) 2^m) and its
// piece pi (chunks R0 + pi*WP ..), the sum over the piece's queries of
// exp(A_t - A_e) lambda_t[LOGC + m] q_t do_t^T, e = R0*C - 1.  A block of a
// single piece writes W ([dk][dv]) and W^T ([dv][dk]) in the input dtype
// directly; otherwise the piece goes out as an fp32 partial for ll_bwd_wsum.
// Grid: (pieces of all levels, BH).
// ---------------------------------------------------------------------------
template <class B>
struct WpSmem {
    using T = typename B::T;
    // weighted q and do: bf16 row-major [token][.] (transpose reads), fp32
    // transposed [.][token]
    __attribute__((aligned(16))) T QwT[B::TRD ? B::C : B::DK][B::TRD ? B::LQ : B::LC];
    __attribute__((aligned(16))) T dOT[B::TRD ? B::C : B::DV][B::TRD ? B::LV : B::LC];
    __attribute__((aligned(16))) float Wt[B::DK][B::DV + 4];   // the result, for coalesced stores
    float Aloc[B::C];
    float wt[B::C];                                     // per-token weights
    float off;
};

__device__ __forceinline__ int wnblk(int N, int m)
{
    const int h = 1 << (m - 1);
    return N > h ? (N - h + (1 << m) - 1) >> m : 0;
}

// Write an fp32 [DK][DV] tile from LDS as W (row-major, T) and W^T.
template <class B>
__device__ __forceinline__ void write_w(const float (*Wt)[B::DV + 4], typename B::T *w1, typename B::T *w2, int tid)
{
    for (int i = tid; i < B::DK * B::DV; i += B::NT) {
        const int d = i / B::DV, e = i % B::DV;
        put(&w1[i], Wt[d][e]);
    }
    if (!w2)
        return;   // W^T not needed (the chunk kernel transposes W as it reads it)
    for (int i = tid; i < B::DK * B::DV; i += B::NT) {
        const int e = i / B::DK, d = i % B::DK;
        put(&w2[i], Wt[d][e]);
    }
}

template <class B>
__global__ __launch_bounds__(256) void ll_bwd_wpiece(const typename B::T *__restrict__ q,
                                                     const typename B::T *__restrict__ dout,
                                                     const float *__restrict__ a, const float *__restrict__ lamg,
                                                     const double *__restrict__ Gp, float *__restrict__ Wp,
                                                     typename B::T *__restrict__ W1, typename B::T *__restrict__ W2,
                                                     int Tlen, int L, int N, int NP, int NB)
{
    constexpr int C = B::C, DK = B::DK, DV = B::DV, VEC = B::VEC;
    __shared__ WpSmem<B> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, qd = lane >> 4;
    const int bh = blockIdx.y;
    // decode (m, block j, piece pi) from the piece index
    int x = blockIdx.x, m = 1, bbase = 0;
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    int nb = 0, np = 0;
    for (; m <= mtop; ++m) {
        nb = wnblk(N, m);
        np = ((1 << (m - 1)) + B::WP - 1) / B::WP;
        if (x < nb * np)
            break;
        x -= nb * np;
        bbase += nb;
    }
    const int j = x / np, pi = x % np;
    const int half = 1 << (m - 1);
    const int R0 = j * (1 << m) + half;
    const int cA = R0 + pi * B::WP, cB = min(min(cA + B::WP, R0 + half), N);
    // every wave owns dk tiles wv, wv+4, .. x all dv tiles
    constexpr int KT = (B::DKT + 3) / 4;
    floatx4 acc[KT][B::DVT];
#pragma unroll
    for (int r = 0; r < KT; ++r)
#pragma unroll
        for (int e = 0; e < B::DVT; ++e)
            acc[r][e] = zero4();
    // log-decay from e to the current chunk's start
    float off = cA < N ? (float)(Gp[(size_t)bh * N + cA] - Gp[(size_t)bh * N + R0]) : 0.f;
    constexpr int QP = C * DK / VEC, VP = C * DV / VEC;
    constexpr int NQP = (QP + B::NT - 1) / B::NT, NVP = (VP + B::NT - 1) / B::NT;
    // Loads of a chunk (q, do, and a, lambda for wave 0) go into registers one
    // chunk ahead: issued right after the previous chunk is staged, so their
    // latency overlaps that chunk's products.
    uint4 rq[NQP], ro[NVP];
    float av, lv;
    auto issue = [&](int cc) {
        const int t0 = cc * C, nv = min(C, Tlen - t0);
        const size_t row0 = (size_t)bh * Tlen + t0;
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int jj = 0; jj < NQP; ++jj) {
            const int i = tid + B::NT * jj;
            rq[jj] = z4;
            if (i < QP && i / (DK / VEC) < nv)
                rq[jj] = *reinterpret_cast<const uint4 *>(q + row0 * DK + (size_t)i * VEC);
        }
#pragma unroll
        for (int jj = 0; jj < NVP; ++jj) {
            const int i = tid + B::NT * jj;
            ro[jj] = z4;
            if (i < VP && i / (DV / VEC) < nv)
                ro[jj] = *reinterpret_cast<const uint4 *>(dout + row0 * DV + (size_t)i * VEC);
        }
        av = 0.f;
        lv = 0.f;
        if (wv == 0 && lane < nv) {
            av = a[row0 + lane];
            lv = lamg[(row0 + lane) * L + B::LOGC + m];
        }
    };
    static_assert(C <= 64, "one wave scans a chunk");
    if (cA < cB)
        issue(cA);
    for (int cc = cA; cc < cB; ++cc) {
        __syncthreads();   // the previous chunk's products are done with the tiles
        if (wv == 0) {
            float y = av;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float z = __shfl_up(y, d, 64);
                if (lane >= d)
                    y += z;
            }
            if (lane < C) {
                sm.Aloc[lane] = y;
                sm.wt[lane] = __expf(off + y) * lv;   // lv is 0 past the end
            }
        }
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < NQP; ++jj) {
            const int i = tid + B::NT * jj;
            if constexpr (B::TRD) {
                if (i < QP) {
                    const int t = i / (DK / VEC), d0 = (i % (DK / VEC)) * VEC;
                    const float w = sm.wt[t];
                    const uint32_t wd[4] = {rq[jj].x, rq[jj].y, rq[jj].z, rq[jj].w};
                    bf16x8 y;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        y[e] = (__bf16)(w * __uint_as_float((e & 1) ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16)));
                    *reinterpret_cast<bf16x8 *>(&sm.QwT[t][d0]) = y;
                }
                continue;
            }
            if (i < QP) {
                const int t = i / (DK / VEC), d0 = (i % (DK / VEC)) * VEC;
                const float w = sm.wt[t];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const uint32_t wd = (VEC == 8) ? ((e >> 1) == 0 ? rq[jj].x : (e >> 1) == 1 ? rq[jj].y
                                                      : (e >> 1) == 2 ? rq[jj].z : rq[jj].w)
                                                   : (e == 0 ? rq[jj].x : e == 1 ? rq[jj].y : e == 2 ? rq[jj].z : rq[jj].w);
                    const float xv = (VEC == 8) ? __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16))
                                                : __uint_as_float(wd);
                    put(&sm.QwT[d0 + e][t], w * xv);
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < NVP; ++jj) {
            const int i = tid + B::NT * jj;
            if (i < VP) {
                const int t = i / (DV / VEC), e0 = (i % (DV / VEC)) * VEC;
                if constexpr (B::TRD) {
                    *reinterpret_cast<uint4 *>(&sm.dOT[t][e0]) = ro[jj];
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        store_elem(&sm.dOT[e0 + e][t], ro[jj], e);
                }
            }
        }
        if (cc + 1 < cB)
            issue(cc + 1);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < B::NUC; ++u) {
#pragma unroll
            for (int r = 0; r < KT; ++r) {
                const int dt = wv + 4 * r;
                if (dt < B::DKT) {
                    if constexpr (B::TRD) {
                        const auto fa = tr_frag(&sm.QwT[0][0], B::LQ, B::KB * u, 16 * dt, li, qd);
#pragma unroll
                        for (int e = 0; e < B::DVT; ++e)
                            mma_unit(acc[r][e], fa, tr_frag(&sm.dOT[0][0], B::LV, B::KB * u, 16 * e, li, qd));
                    } else {
                        const auto fa = frag<B>(&sm.QwT[0][0], B::LC, 16 * dt + li, u, qd);
#pragma unroll
                        for (int e = 0; e < B::DVT; ++e)
                            mma_unit(acc[r][e], fa, frag<B>(&sm.dOT[0][0], B::LC, 16 * e + li, u, qd));
                    }
                }
            }
        }
        off += sm.Aloc[C - 1];   // read before the next chunk's first barrier
    }
    // acc[r][e][i] = W[d = 16 dt + 4 qd + i][dv = 16 e + li]
#pragma unroll
    for (int r = 0; r < KT; ++r) {
        const int dt = wv + 4 * r;
        if (dt < B::DKT)
#pragma unroll
            for (int e = 0; e < B::DVT; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.Wt[16 * dt + 4 * qd + i][16 * e + li] = acc[r][e][i];
    }
    __syncthreads();
    if (np == 1) {
        const size_t wi = (size_t)bh * NB + bbase + j;
        write_w<B>(sm.Wt, W1 + wi * DK * DV, W2 ? W2 + wi * DK * DV : nullptr, tid);
    } else {
        float *dst = Wp + ((size_t)bh * NP + blockIdx.x) * DK * DV;
        for (int i = tid; i < DK * DV; i += B::NT)
            dst[i] = sm.Wt[i / DV][i % DV];
    }
}

// W states from spans (bf16): one workgroup of 8 waves per (head, aligned
// span of WP chunks) reads each chunk's q, do, lambda and a once, and forms
// for every level m at which the chunk lies in a right block R its share of
//     W(R) = sum over R's queries of exp(A_t - A_e) lambda_t[LOGC + m] q_t do_t^T
// (e the last key before R).  Blocks of at most WP chunks lie inside one span:
// their W is written whole (bf16).  A larger block takes a float32 partial
// from each of its spans, the pieces ll_bwd_wsum adds, at the index the piece
// enumeration gives.  The levels are taken NL at a time (a further pass
// re-reads the span).  Products W^T = dO^T (w q) on MFMA: wave w owns dk tile
// w and every dv tile; q and do are read with transpose reads, and each
// level's per-token weights scale the q fragment in registers.
// Grid: (spans, BH).
template <class B>
struct WsSmem {
    using T = typename B::T;
    static constexpr int NL = 8;   // levels per pass (one per wave in the weight table)
    __attribute__((aligned(16))) T Qs[B::C][B::LQ];
    __attribute__((aligned(16))) T dOs[B::C][B::LV];
    __attribute__((aligned(16))) float wt[NL][B::C];   // per level and token: exp(decay) lambda (0: no share)
    float Aloc[B::C];
};

template <class B>
__global__ __launch_bounds__(512) void ll_bwd_wspan(const typename B::T *__restrict__ q,
                                                    const typename B::T *__restrict__ dout,
                                                    const float *__restrict__ a, const float *__restrict__ lamg,
                                                    const double *__restrict__ Gp, float *__restrict__ Wp,
                                                    typename B::T *__restrict__ W1, int Tlen, int L, int N, int NP,
                                                    int NB)
{
    using T = typename B::T;
    using S = WsSmem<B>;
    constexpr int C = B::C, DK = B::DK, DV = B::DV, VEC = B::VEC, NL = S::NL;
    constexpr int NTW = 512;
    static_assert(B::TRD && C <= 64 && DK == 16 * 8, "bf16, one dk tile per wave of eight");
    static_assert(NL * 64 == NTW, "one weight per thread");
    __shared__ S sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, qd = lane >> 4;
    const int bh = blockIdx.y, sp = blockIdx.x;
    const int cA = sp * B::WP, cB = min(cA + B::WP, N);
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    const double *gp = Gp + (size_t)bh * N;
    // first W index and first piece index of each level
    auto bbase_of = [&](int m) {
        int x = 0;
        for (int r = 1; r < m; ++r)
            x += wnblk(N, r);
        return x;
    };
    auto pbase_of = [&](int m) {
        int x = 0;
        for (int r = 1; r < m; ++r)
            x += wnblk(N, r) * (((1 << (r - 1)) + B::WP - 1) / B::WP);
        return x;
    };
    constexpr int QP = C * DK / VEC, VP = C * DV / VEC;
    constexpr int NQP = (QP + NTW - 1) / NTW, NVP = (VP + NTW - 1) / NTW;
    uint4 rq[NQP], ro[NVP];
    float av = 0.f, lv = 0.f;
    for (int m0 = 1; m0 <= mtop; m0 += NL) {
        floatx4 acc[NL][B::DVT];
#pragma unroll
        for (int l = 0; l < NL; ++l)
#pragma unroll
            for (int ct = 0; ct < B::DVT; ++ct)
                acc[l][ct] = zero4();
        // chunk cc's inputs into registers (its lambda at level m0 + wave)
        auto issue = [&](int cc) {
            const int t0 = cc * C, nv = min(C, Tlen - t0);
            const size_t row0 = (size_t)bh * Tlen + t0;
            const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int j = 0; j < NQP; ++j) {
                const int i = tid + NTW * j;
                rq[j] = z4;
                if (i < QP && i / (DK / VEC) < nv)
                    rq[j] = *reinterpret_cast<const uint4 *>(q + row0 * DK + (size_t)i * VEC);
            }
#pragma unroll
            for (int j = 0; j < NVP; ++j) {
                const int i = tid + NTW * j;
                ro[j] = z4;
                if (i < VP && i / (DV / VEC) < nv)
                    ro[j] = *reinterpret_cast<const uint4 *>(dout + row0 * DV + (size_t)i * VEC);
            }
            const int m = m0 + w;
            lv = (lane < nv && m <= mtop) ? lamg[(row0 + lane) * L + B::LOGC + m] : 0.f;
            av = (w == 0 && lane < nv) ? a[row0 + lane] : 0.f;
        };
        issue(cA);
        for (int cc = cA; cc < cB; ++cc) {
            __syncthreads();   // the previous chunk's products are done with the tiles
#pragma unroll
            for (int j = 0; j < NQP; ++j) {
                const int i = tid + NTW * j;
                if (i < QP)
                    *reinterpret_cast<uint4 *>(&sm.Qs[i / (DK / VEC)][(i % (DK / VEC)) * VEC]) = rq[j];
            }
#pragma unroll
            for (int j = 0; j < NVP; ++j) {
                const int i = tid + NTW * j;
                if (i < VP)
                    *reinterpret_cast<uint4 *>(&sm.dOs[i / (DV / VEC)][(i % (DV / VEC)) * VEC]) = ro[j];
            }
            if (w == 0) {
                float y = av;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const float z = __shfl_up(y, d, 64);
                    if (lane >= d)
                        y += z;
                }
                if (lane < C)
                    sm.Aloc[lane] = y;
            }
            const float lvc = lv;
            __syncthreads();
            // weight of token `lane` at level m = m0 + w: zero unless the chunk
            // lies in the right block R of that level (R0 its first chunk)
            {
                const int m = m0 + w;
                float x = 0.f;
                if (m <= mtop && ((cc >> (m - 1)) & 1) && lane < C) {
                    const int R0 = ((cc >> m) << m) + (1 << (m - 1));
                    x = __expf((float)(gp[cc] - gp[R0]) + sm.Aloc[lane]) * lvc;
                }
                if (lane < C)
                    sm.wt[w][lane] = x;
            }
            if (cc + 1 < cB)
                issue(cc + 1);
            __syncthreads();
            // products: the do fragments (A, rows e) are shared by the levels
#pragma unroll
            for (int u = 0; u < B::NUC; ++u) {
                bf16x8 fa[B::DVT];
#pragma unroll
                for (int ct = 0; ct < B::DVT; ++ct)
                    fa[ct] = tr_frag(&sm.dOs[0][0], B::LV, B::KB * u, 16 * ct, li, qd);
                const bf16x8 fq = tr_frag(&sm.Qs[0][0], B::LQ, B::KB * u, 16 * w, li, qd);
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const int m = m0 + l;
                    if (m > mtop || !((cc >> (m - 1)) & 1))
                        continue;
                    // token of element e: KB u + 16 (e / 4) + 4 qd + e % 4
                    const floatx4 w0 = *reinterpret_cast<const floatx4 *>(&sm.wt[l][B::KB * u + 4 * qd]);
                    const floatx4 w1 = *reinterpret_cast<const floatx4 *>(&sm.wt[l][B::KB * u + 16 + 4 * qd]);
                    bf16x8 fb;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        fb[e] = (__bf16)((float)fq[e] * w0[e]);
                        fb[e + 4] = (__bf16)((float)fq[e + 4] * w1[e]);
                    }
#pragma unroll
                    for (int ct = 0; ct < B::DVT; ++ct)
                        acc[l][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ct], fb, acc[l][ct], 0, 0, 0);
                }
            }
            // blocks that end with this chunk (levels whose blocks fit the span)
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const int m = m0 + l;
                if (m > mtop || (1 << (m - 1)) > B::WP || !((cc >> (m - 1)) & 1))
                    continue;
                const int last = ((cc >> m) << m) + (1 << m) - 1;
                if (cc != last && cc != N - 1)
                    continue;
                // acc[l][ct][r] = W[d = 16 w + li][e = 16 ct + 4 qd + r]
                const size_t wi = (size_t)bh * NB + bbase_of(m) + (cc >> m);
                T *dst = W1 + wi * DK * DV + (size_t)(16 * w + li) * DV + 4 * qd;
#pragma unroll
                for (int ct = 0; ct < B::DVT; ++ct) {
                    put4(dst + 16 * ct, acc[l][ct]);
                    acc[l][ct] = zero4();
                }
            }
        }
        // partials of the larger blocks (the whole span lies in one block)
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int m = m0 + l;
            if (m > mtop || (1 << (m - 1)) <= B::WP || !((cA >> (m - 1)) & 1))
                continue;
            const int j = cA >> m, R0 = (j << m) + (1 << (m - 1));
            const int np = ((1 << (m - 1)) + B::WP - 1) / B::WP;
            const size_t pi = (size_t)bh * NP + pbase_of(m) + (size_t)j * np + (cA - R0) / B::WP;
            float *dst = Wp + pi * DK * DV + (size_t)(16 * w + li) * DV + 4 * qd;
#pragma unroll
            for (int ct = 0; ct < B::DVT; ++ct)
                *reinterpret_cast<floatx4 *>(dst + 16 * ct) = acc[l][ct];
        }
    }
}

// Sum of a multi-piece block's partials, written as W and W^T.
template <class B>
__global__ __launch_bounds__(256) void ll_bwd_wsum(const float *__restrict__ Wp, typename B::T *__restrict__ W1,
                                                   typename B::T *__restrict__ W2, int N, int NP, int NB)
{
    constexpr int DK = B::DK, DV = B::DV;
    __shared__ __attribute__((aligned(16))) float Wt[DK][DV + 4];
    const int bh = blockIdx.y;
    int x = blockIdx.x, m = 1, pbase = 0;
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    int nb = 0, np = 0;
    for (; m <= mtop; ++m) {
        nb = wnblk(N, m);
        np = ((1 << (m - 1)) + B::WP - 1) / B::WP;
        if (x < nb)
            break;
        x -= nb;
        pbase += nb * np;
    }
    if (np == 1)
        return;   // written by its only piece
    const int j = x, half = 1 << (m - 1);
    const int R0 = j * (1 << m) + half;
    int npv = 0;   // pieces that start inside the sequence
    for (int pi = 0; pi < np; ++pi)
        if (R0 + pi * B::WP < N)
            npv = pi + 1;
    const float *src = Wp + ((size_t)bh * NP + pbase + (size_t)j * np) * DK * DV;
    constexpr int PER = DK * DV / 256;   // elements per thread, 16-byte pieces
    static_assert(PER % 4 == 0, "thread layout");
    float4 acc[PER / 4];
#pragma unroll
    for (int r = 0; r < PER / 4; ++r)
        acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int pi = 0; pi < npv; ++pi) {
        const float4 *sp = reinterpret_cast<const float4 *>(src + (size_t)pi * DK * DV);
#pragma unroll
        for (int r = 0; r < PER / 4; ++r) {
            const float4 x = sp[threadIdx.x + 256 * r];
            acc[r].x += x.x; acc[r].y += x.y; acc[r].z += x.z; acc[r].w += x.w;
        }
    }
#pragma unroll
    for (int r = 0; r < PER / 4; ++r) {
        const int i = 4 * (threadIdx.x + 256 * r);
        Wt[i / DV][i % DV] = acc[r].x;
        Wt[i / DV][i % DV + 1] = acc[r].y;
        Wt[i / DV][i % DV + 2] = acc[r].z;
        Wt[i / DV][i % DV + 3] = acc[r].w;
    }
    __syncthreads();
    const size_t wi = (size_t)bh * NB + blockIdx.x;
    write_w<B>(Wt, W1 + wi * DK * DV, W2 ? W2 + wi * DK * DV : nullptr, threadIdx.x);
}

// The same sums when only W is kept (the spans kernel's pieces): each block
// is split over WQ workgroups by rows, and a thread adds its 16-byte slices
// of four pieces at a time, so that four loads per slice are in flight.
// Grid: (NB * WQ, BH).
template <class B>
__global__ __launch_bounds__(256) void ll_bwd_wsum_rows(const float *__restrict__ Wp, typename B::T *__restrict__ W1,
                                                        int N, int NP, int NB)
{
    constexpr int DK = B::DK, DV = B::DV, WQ = 4;
    constexpr int PER = DK * DV / WQ / 4 / 256;   // float4 slices per thread and piece
    static_assert(PER >= 1 && DK * DV == PER * 4 * 256 * WQ, "thread layout");
    const int bh = blockIdx.y, qt = blockIdx.x % WQ;
    int x = blockIdx.x / WQ, m = 1, pbase = 0;
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    int nb = 0, np = 0;
    for (; m <= mtop; ++m) {
        nb = wnblk(N, m);
        np = ((1 << (m - 1)) + B::WP - 1) / B::WP;
        if (x < nb)
            break;
        x -= nb;
        pbase += nb * np;
    }
    if (np == 1)
        return;   // written by its only piece
    const int j = x, R0 = j * (1 << m) + (1 << (m - 1));
    int npv = 0;   // pieces that start inside the sequence
    for (int pi = 0; pi < np; ++pi)
        if (R0 + pi * B::WP < N)
            npv = pi + 1;
    const float *src = Wp + ((size_t)bh * NP + pbase + (size_t)j * np) * DK * DV + (size_t)qt * (DK * DV / WQ);
    float4 acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r)
        acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < npv; p0 += 4) {
        float4 x4[4][PER];
        float f[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int pi = p0 + h;
            const bool ok = pi < npv;
            const float4 *sp = reinterpret_cast<const float4 *>(src + (size_t)(ok ? pi : 0) * DK * DV);
#pragma unroll
            for (int r = 0; r < PER; ++r)
                x4[h][r] = sp[threadIdx.x + 256 * r];
            f[h] = ok ? 1.f : 0.f;   // a past-the-end slot re-reads piece 0 and adds nothing
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                acc[r].x += f[h] * x4[h][r].x;
                acc[r].y += f[h] * x4[h][r].y;
                acc[r].z += f[h] * x4[h][r].z;
                acc[r].w += f[h] * x4[h][r].w;
            }
    }
    typename B::T *dst = W1 + ((size_t)bh * NB + blockIdx.x / WQ) * DK * DV + (size_t)qt * (DK * DV / WQ);
#pragma unroll
    for (int r = 0; r < PER; ++r)
        put4(dst + 4 * (threadIdx.x + 256 * r), floatx4{acc[r].x, acc[r].y, acc[r].z, acc[r].w});
}

// fp64 exclusive prefix of the chunk log-decay totals: Gp[c] = sum of
// gam[c'] over c' < c, c in [0, N) (gam is defined for the first N-1 chunks).
// One workgroup per head.
__global__ __launch_bounds__(256) void ll_bwd_gprefix(const float *__restrict__ Gam, double *__restrict__ Gp, int N)
{
    __shared__ double sums[256];
    const int tid = threadIdx.x, bh = blockIdx.x;
    const float *g = Gam + (size_t)bh * N;
    double *o = Gp + (size_t)bh * N;
    const int per = (N + 255) / 256;
    const int lo = min(N, tid * per), hi = min(N, lo + per);
    double x = 0.0;
    for (int c = lo; c < hi; ++c)
        x += c < N - 1 ? (double)g[c] : 0.0;
    sums[tid] = x;
    __syncthreads();
    double b = 0.0;
    for (int j = 0; j < tid; ++j)
        b += sums[j];
    for (int c = lo; c < hi; ++c) {
        o[c] = b;
        b += c < N - 1 ? (double)g[c] : 0.0;
    }
}

// Exclusive prefix sums over chunks of the per-level pair masses, in place:
// one workgroup per (level, head).
__global__ __launch_bounds__(256) void ll_bwd_mscan(float *__restrict__ Mq, float *__restrict__ Mk, int N)
{
    __shared__ float sums[2][256];
    const int tid = threadIdx.x, m = blockIdx.x + 1, bh = blockIdx.y;
    float *q = Mq + ((size_t)bh * kMaxLevels + m) * (N + 1);
    float *k = Mk + ((size_t)bh * kMaxLevels + m) * (N + 1);
    const int per = (N + 1 + 255) / 256;
    const int lo = min(N + 1, tid * per), hi = min(N + 1, lo + per);
    float xq = 0.f, xk = 0.f;
    for (int x = lo; x < hi; ++x) {
        xq += x < N ? q[x] : 0.f;
        xk += x < N ? k[x] : 0.f;
    }
    sums[0][tid] = xq;
    sums[1][tid] = xk;
    __syncthreads();
    float bq = 0.f, bk = 0.f;
    for (int jj = 0; jj < tid; ++jj) {
        bq += sums[0][jj];
        bk += sums[1][jj];
    }
    for (int x = lo; x < hi; ++x) {
        const float vq = x < N ? q[x] : 0.f, vk = x < N ? k[x] : 0.f;
        q[x] = bq;
        k[x] = bk;
        bq += vq;
        bk += vk;
    }
}

// da_r = da inside r's chunk (daloc) + the pairs that jump over that chunk:
// at every chunk level m the chunk c lies in one of the two sibling blocks
// B (left) and R (right) of the pair set of that level, and the jumping pairs
// are R's queries after c into B (query-side masses Mq) or B's keys before c
// seen from R (key-side masses Mk), read from the prefix sums.  One thread per
// position.
__global__ __launch_bounds__(256) void ll_bwd_da(const float *__restrict__ daloc, const float *__restrict__ Mq,
                                                 const float *__restrict__ Mk, float *__restrict__ da, int Tlen, int N,
                                                 int C, int mtop)
{
    const int bh = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= Tlen)
        return;
    const int c = r / C;
    float X = 0.f;
    for (int m = 1; m <= mtop; ++m) {
        const float *q = Mq + ((size_t)bh * kMaxLevels + m) * (N + 1);
        const float *k = Mk + ((size_t)bh * kMaxLevels + m) * (N + 1);
        const int b0 = (c >> m) << m, half = 1 << (m - 1);
        if ((c >> (m - 1)) & 1)
            X += q[min(b0 + 2 * half, N)] - q[c + 1];
        else
            X += k[c] - k[b0];
    }
    const size_t h = (size_t)bh * Tlen;
    da[h + r] = r == 0 ? 0.f : daloc[h + r] + X;
}

// ---------------------------------------------------------------------------
// q/k shared by several heads.  The gradient of a shared q or k row is the
// sum of the per-head gradients of the heads that read it; the backward runs
// per head on a copy of q and k laid out per head and then sums.
// ---------------------------------------------------------------------------

// dst row block of head bh <- src row block of q/k head bh / rqk (16-byte
// vectors; hv vectors per head).
__global__ __launch_bounds__(256) void ll_bcast_heads(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                      size_t hv, int rqk, size_t total)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const size_t bh = i / hv, e = i - bh * hv;
        dst[i] = src[(bh / rqk) * hv + e];
    }
}

// dst[qbh] = sum over the rqk heads j of src[qbh * rqk + j], four elements
// per thread, fp32 accumulation (he elements per head).
template <class T>
__global__ __launch_bounds__(256) void ll_sum_heads(const T *__restrict__ src, T *__restrict__ dst, size_t he,
                                                    int rqk, size_t total4)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total4; i += (size_t)gridDim.x * 256) {
        const size_t qbh = (4 * i) / he, e = 4 * i - qbh * he;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < rqk; ++j) {
            const T *x = src + ((size_t)qbh * rqk + j) * he + e;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] += to_f32(x[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dst[4 * i + c] = from_f32<T>(acc[c]);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int bwd_levels(int N)
{
    int n = 0;
    for (int x = N - 1; x > 0; x >>= 1)
        ++n;
    return n;
}

static void bwd_counts(int N, int &NP, int &NB, int wp)
{
    NP = NB = 0;
    for (int m = 1; m <= bwd_levels(N); ++m) {
        const int h = 1 << (m - 1);
        const int nb = N > h ? (N - h + (1 << m) - 1) >> m : 0;
        NB += nb;
        NP += nb * ((h + wp - 1) / wp);
    }
}

typedef hipError_t (*BwdLauncher)(const BwdArgs &, const BwdPlan &, hipStream_t);

template <class DT, int DK, int DV, int C>
static hipError_t launch_bwd_t(const BwdArgs &A, const BwdPlan &P, hipStream_t s)
{
    using B = Bw<DT, DK, DV, C>;
    using T = typename B::T;
    const int BH = A.B * A.H;
    char *ws = static_cast<char *>(A.workspace);
    const int N = (A.T + C - 1) / C;
    // 1. left block states: with the chunk kernel forming dq (bf16), a tree
    //    over groups of up to 8 chunks plus the Fenwick nodes inside each
    //    group; otherwise a tree over chunks (one chunk per group)
    const bool g8 = BwDq<B>::on;
    const FwdPlan &TP = g8 ? P.tree8 : P.tree;
    FwdArgs tree{nullptr, A.k, A.v, A.a, A.lam, nullptr, A.B, A.H, A.T, DK, DV, C, A.L, A.bf16, ws + P.off_tree};
    tree.tree_only = true;
    tree.tree_nat = A.bf16;
    if (g8) {
        // block states and nodes in the A-operand fragment order of the
        // chunk kernel's query-side product
        tree.tree_yfrag = true;
        tree.tree_nodes = ws + P.off_tree + P.off_nd;
        tree.tree_gamc = reinterpret_cast<float *>(ws + P.off_tree + P.off_gamc);
    }
    hipError_t e = fwd_launch(tree, TP, s, nullptr);
    if (e != hipSuccess)
        return e;
    // 2. dq: the forward with q <- do, k <- v, v <- k (unless the chunk
    //    kernel forms it)
    if (!BwDq<B>::on) {
        FwdArgs fq{A.dout, A.v, A.k, A.a, A.lam, A.gq, A.B, A.H, A.T, DV, DK, C, A.L, A.bf16, ws + P.off_fq};
        e = fwd_launch(fq, P.fq, s, nullptr);
        if (e != hipSuccess)
            return e;
    }
    // chunk totals (the tree's leaves are chunks, or the node pass wrote them)
    const float *Gam = g8 ? reinterpret_cast<const float *>(ws + P.off_tree + P.off_gamc)
                          : reinterpret_cast<const float *>(ws + P.off_tree + P.tree.off_Gam);
    const T *Dg = reinterpret_cast<const T *>(ws + P.off_tree + TP.off_Dg);
    const T *Nd = g8 ? reinterpret_cast<const T *>(ws + P.off_tree + P.off_nd) : nullptr;
    float *Wp = reinterpret_cast<float *>(ws + P.off_wp);
    T *W1 = reinterpret_cast<T *>(ws + P.off_w1);
    T *W2 = g8 ? nullptr : reinterpret_cast<T *>(ws + P.off_w2);   // W^T, when the chunk kernel needs it
    float *daloc = reinterpret_cast<float *>(ws + P.off_pq);
    double *Gp = reinterpret_cast<double *>(ws + P.off_gp);
    if (N > 1) {
        ProfEvents pg = prof_events("ll_bwd_gprefix");
        hipExtLaunchKernelGGL(ll_bwd_gprefix, dim3(BH), dim3(256), 0, s, pg.start, pg.stop, 0, Gam, Gp, N);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    float *Mq = reinterpret_cast<float *>(ws + P.off_mq);
    float *Mk = reinterpret_cast<float *>(ws + P.off_mk);
    // 3. W pieces and their sums
    if (P.NP > 0 && g8) {
        if constexpr (BwDq<B>::on && B::DK == 128 && B::C <= 64) {
            ProfEvents pe = prof_events("ll_bwd_wspan");
            hipExtLaunchKernelGGL(ll_bwd_wspan<B>, dim3((N + B::WP - 1) / B::WP, BH), dim3(512), 0, s, pe.start,
                                  pe.stop, 0, (const T *)A.q, (const T *)A.dout, A.a, A.lam, (const double *)Gp, Wp,
                                  W1, A.T, A.L, N, P.NP, P.NB);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
            pe = prof_events("ll_bwd_wsum");
            hipExtLaunchKernelGGL(ll_bwd_wsum_rows<B>, dim3(P.NB * 4, BH), dim3(256), 0, s, pe.start, pe.stop,
                                  0, (const float *)Wp, W1, N, P.NP, P.NB);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
    }
    if (P.NP > 0 && !(g8 && BwDq<B>::on && B::DK == 128 && B::C <= 64)) {
        ProfEvents pe = prof_events("ll_bwd_wpiece");
        hipExtLaunchKernelGGL(ll_bwd_wpiece<B>, dim3(P.NP, BH), dim3(256), 0, s, pe.start, pe.stop, 0,
                              (const T *)A.q, (const T *)A.dout, A.a, A.lam, (const double *)Gp, Wp, W1, W2, A.T,
                              A.L, N, P.NP,
                              P.NB);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        pe = prof_events("ll_bwd_wsum");
        hipExtLaunchKernelGGL(ll_bwd_wsum<B>, dim3(P.NB, BH), dim3(256), 0, s, pe.start, pe.stop, 0,
                              (const float *)Wp, W1, W2, N, P.NP, P.NB);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    // 4. chunk kernel
    ProfEvents pe = prof_events("ll_bwd_chunk");
    hipExtLaunchKernelGGL(ll_bwd_chunk<B>, dim3(BH * N), dim3(B::NTC), 0, s, pe.start, pe.stop, 0, (const T *)A.q,
                          (const T *)A.k, (const T *)A.v, (const T *)A.dout, A.a, A.lam, Dg, Nd, g8 ? TP.g : 0,
                          (const double *)Gp, (const T *)W1, (const T *)W2, (T *)A.gq, (T *)A.gk, (T *)A.gv, A.glam,
                          daloc, Mq, Mk, A.T, A.L, N, TP.nL, TP.nLeft, P.NB);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // 5. da
    const int mt = bwd_levels(N);
    if (mt > 0) {
        pe = prof_events("ll_bwd_mscan");
        hipExtLaunchKernelGGL(ll_bwd_mscan, dim3(mt, BH), dim3(256), 0, s, pe.start, pe.stop, 0, Mq, Mk, N);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    pe = prof_events("ll_bwd_da");
    hipExtLaunchKernelGGL(ll_bwd_da, dim3((A.T + 255) / 256, BH), dim3(256), 0, s, pe.start, pe.stop, 0,
                          (const float *)daloc, (const float *)Mq, (const float *)Mk, A.ga, A.T, N, C, mt);
    return hipGetLastError();
}

template <class DT, int DK, int DV, int C>
static BwdLauncher bwd_pick_c()
{
    using B = Bw<DT, DK, DV, C>;
    if constexpr (C % DT::KB != 0 || 4 % (C / 16) != 0 || (DK / 16) % (4 / (C / 16)) != 0 ||
                  (DV / 16) % (4 / (C / 16)) != 0) {
        return nullptr;
    } else if constexpr (sizeof(BwSmem<B>) > 160 * 1024 || sizeof(WpSmem<B>) > 160 * 1024) {
        return nullptr;
    } else {
        return &launch_bwd_t<DT, DK, DV, C>;
    }
}

template <class DT, int DK, int DV>
static BwdLauncher bwd_pick_chunk(int chunk)
{
    switch (chunk) {
    case 32: return bwd_pick_c<DT, DK, DV, 32>();
    case 64: return bwd_pick_c<DT, DK, DV, 64>();
    default: return nullptr;
    }
}

template <class DT, int DK>
static BwdLauncher bwd_pick_dv(int dv, int chunk)
{
    switch (dv) {
    case 32: return bwd_pick_chunk<DT, DK, 32>(chunk);
    case 64: return bwd_pick_chunk<DT, DK, 64>(chunk);
    case 128: return bwd_pick_chunk<DT, DK, 128>(chunk);
    default: return nullptr;
    }
}

template <class DT>
static BwdLauncher bwd_pick(int dk, int dv, int chunk)
{
    switch (dk) {
    case 32: return bwd_pick_dv<DT, 32>(dv, chunk);
    case 64: return bwd_pick_dv<DT, 64>(dv, chunk);
    case 128: return bwd_pick_dv<DT, 128>(dv, chunk);
    default: return nullptr;
    }
}

static BwdLauncher find_bwd(bool bf16, int dk, int dv, int chunk)
{
    return bf16 ? bwd_pick<TBF16>(dk, dv, chunk) : bwd_pick<TF32>(dk, dv, chunk);
}

bool bwd_supported(bool bf16, int dk, int dv, int chunk)
{
    return find_bwd(bf16, dk, dv, chunk) != nullptr && fwd_supported(bf16, dk, dv, chunk) &&
           fwd_supported(bf16, dv, dk, chunk);
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdPlan bwd_plan(int B, int H, int T, int dk, int dv, int chunk, int rqk)
{
    BwdPlan p;
    const size_t BH = (size_t)B * H;
    const int N = (T + chunk - 1) / chunk;
    p.tree = fwd_plan(B, H, T, dk, dv, chunk, 0, 4);
    p.g8 = N >= 8 ? 3 : N >= 4 ? 2 : N >= 2 ? 1 : 0;
    p.tree8 = fwd_plan(B, H, T, dk, dv, chunk, p.g8, 4);
    p.off_nd = al256(p.tree8.bytes);
    p.off_gamc = al256(p.off_nd + BH * (size_t)N * dk * dv * 2);
    const size_t tree_bytes = std::max(p.tree.bytes, al256(p.off_gamc + BH * (size_t)N * 4));
    p.fq = fwd_plan(B, H, T, dv, dk, chunk, -1, 4);
    bwd_counts(N, p.NP, p.NB, 8);
    const size_t st = (size_t)dk * dv;
    p.off_tree = 0;
    p.off_fq = al256(p.off_tree + tree_bytes);
    p.off_wp = al256(p.off_fq + p.fq.bytes);
    p.off_w1 = al256(p.off_wp + BH * p.NP * st * 4);
    p.off_w2 = al256(p.off_w1 + BH * p.NB * st * 4);
    p.off_pq = al256(p.off_w2 + BH * p.NB * st * 4);
    p.off_mq = al256(p.off_pq + BH * T * 4);
    p.off_mk = al256(p.off_mq + BH * kMaxLevels * (size_t)(N + 1) * 4);
    p.off_gp = al256(p.off_mk + BH * kMaxLevels * (size_t)(N + 1) * 4);
    p.bytes = al256(p.off_gp + BH * (size_t)N * 8);
    if (rqk > 1) {
        // per-head copies of q and k and per-head dq, dk (sized for float32)
        const size_t hq = BH * (size_t)T * dk * 4;
        p.off_qx = p.bytes;
        p.off_kx = al256(p.off_qx + hq);
        p.off_gqx = al256(p.off_kx + hq);
        p.off_gkx = al256(p.off_gqx + hq);
        p.bytes = al256(p.off_gkx + hq);
    }
    return p;
}

static unsigned grid_for(size_t n)
{
    const size_t g = (n + 255) / 256;
    return (unsigned)(g < 16384 ? (g > 0 ? g : 1) : 16384);
}

hipError_t bwd_launch(const BwdArgs &args, const BwdPlan &plan, hipStream_t stream)
{
    BwdLauncher f = find_bwd(args.bf16, args.dk, args.dv, args.chunk);
    if (!f)
        return hipErrorInvalidValue;
    if (args.rqk <= 1)
        return f(args, plan, stream);
    // Shared q/k: per-head copies in, per-head dq/dk out, then the sums.
    char *ws = static_cast<char *>(args.workspace);
    const size_t es = args.bf16 ? 2 : 4;
    const size_t BH = (size_t)args.B * args.H;
    const size_t he = (size_t)args.T * args.dk;   // elements per head
    const size_t hv = he * es / 16, total = BH * hv;
    BwdArgs a = args;
    a.q = ws + plan.off_qx;
    a.k = ws + plan.off_kx;
    a.gq = ws + plan.off_gqx;
    a.gk = ws + plan.off_gkx;
    ProfEvents pe = prof_events("ll_bcast_heads");
    hipExtLaunchKernelGGL(ll_bcast_heads, dim3(grid_for(total)), dim3(256), 0, stream, pe.start, pe.stop, 0,
                          (const uint4 *)args.q, (uint4 *)(ws + plan.off_qx), hv, args.rqk, total);
    pe = prof_events("ll_bcast_heads");
    hipExtLaunchKernelGGL(ll_bcast_heads, dim3(grid_for(total)), dim3(256), 0, stream, pe.start, pe.stop, 0,
                          (const uint4 *)args.k, (uint4 *)(ws + plan.off_kx), hv, args.rqk, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if ((e = f(a, plan, stream)) != hipSuccess)
        return e;
    const size_t total4 = BH / args.rqk * he / 4;
    for (int which = 0; which < 2; ++which) {
        const void *src = which ? a.gk : a.gq;
        void *dst = which ? args.gk : args.gq;
        pe = prof_events("ll_sum_heads");
        if (args.bf16)
            hipExtLaunchKernelGGL(ll_sum_heads<__bf16>, dim3(grid_for(total4)), dim3(256), 0, stream, pe.start,
                                  pe.stop, 0, (const __bf16 *)src, (__bf16 *)dst, he, args.rqk, total4);
        else
            hipExtLaunchKernelGGL(ll_sum_heads<float>, dim3(grid_for(total4)), dim3(256), 0, stream, pe.start,
                                  pe.stop, 0, (const float *)src, (float *)dst, he, args.rqk, total4);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace ll
