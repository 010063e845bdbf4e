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
//  - dq is the forward itself with the roles q <- do, k <- v, v <- k (it
//    weights by lambda of the output position, as dq does); the host runs the
//    forward kernels for it.
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
    static constexpr int NCG = 4 / CT;                    // column groups per token tile (4 waves)
    static constexpr int KPW = DKT / NCG, VPW = DVT / NCG;  // dk / dv tiles per wave
    static constexpr int LOGC = C == 16 ? 4 : C == 32 ? 5 : 6;
    static constexpr int WP = 8;                          // chunks per W piece
    static constexpr int VEC = 16 / (int)sizeof(T);
    static_assert(C % KB == 0 && DK % KB == 0 && DV % KB == 0, "units");
    static_assert(CT >= 1 && CT <= 4 && 4 % CT == 0 && DKT % NCG == 0 && DVT % NCG == 0, "wave layout");
};

template <class B>
struct BwSmem {
    using T = typename B::T;
    __attribute__((aligned(16))) T Qs[B::C][B::LQ];    // q rows
    __attribute__((aligned(16))) T QsT[B::DK][B::LC];  // q, [dk][token]
    __attribute__((aligned(16))) T Ks[B::C][B::LQ];
    __attribute__((aligned(16))) T Vs[B::C][B::LV];
    __attribute__((aligned(16))) T dOs[B::C][B::LV];
    __attribute__((aligned(16))) T dOsT[B::DV][B::LC];
    __attribute__((aligned(16))) T PdT[B::C][B::LC];   // (M . dP)^T, [key][query]
    __attribute__((aligned(16))) T PsT[B::C][B::LC];   // (M . S)^T
    float G[B::C][B::C + 1];                            // exp(decay) S dP, [query][key]
    float lam[B::C][kMaxLevels];
    float dlam[B::C][kMaxLevels];
    float Aloc[B::C];                                   // inclusive prefix of a inside the chunk
    float part[4][B::C];                                // cross-wave row partial sums
    float off[kMaxLevels];                              // per-level log-decay offsets (chunk totals)
    float km[kMaxLevels];                               // key-side pair mass of this chunk per level
    float kw[4];
    float u[B::C], w[B::C];                             // per-token terms of the in-chunk part of da
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

// Sum of the chunk log-decay totals gam[c0 .. c1) over one wave.
__device__ __forceinline__ float wave_range_sum(const float *gam, int c0, int c1, int lane)
{
    float x = 0.f;
    for (int c = c0 + lane; c < c1; c += 64)
        x += gam[c];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

// ---------------------------------------------------------------------------
// Chunk kernel: one workgroup per (head, chunk).
// ---------------------------------------------------------------------------
template <class B>
__global__ __launch_bounds__(256) void ll_bwd_chunk(
    const typename B::T *__restrict__ q, const typename B::T *__restrict__ k, const typename B::T *__restrict__ v,
    const typename B::T *__restrict__ dout, const float *__restrict__ a, const float *__restrict__ lamg,
    const typename B::T *__restrict__ Dg, const float *__restrict__ Gam, const typename B::T *__restrict__ W1,
    const typename B::T *__restrict__ W2, typename B::T *__restrict__ dkg, typename B::T *__restrict__ dvg,
    float *__restrict__ dlamg, float *__restrict__ daloc, float *__restrict__ Mq, float *__restrict__ Mk, int Tlen,
    int L, int N, int nL, int nLeft, int NB)
{
    using T = typename B::T;
    using Frag = typename B::Frag;
    constexpr int C = B::C, DK = B::DK, DV = B::DV;
    __shared__ BwSmem<B> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, qd = lane >> 4;
    const int bh = blockIdx.x / N, c = blockIdx.x % N;
    const int t0 = c * C;
    const int nv = min(C, Tlen - t0);   // valid rows of this chunk
    const size_t row0 = (size_t)bh * Tlen + t0;

    // ---- stage the chunk --------------------------------------------------
    for (int i = tid; i < C * DK; i += B::NT) {
        const int t = i / DK, d = i % DK;
        const T zq = t < nv ? q[(row0 + t) * DK + d] : from_f32<T>(0.f);
        const T zk = t < nv ? k[(row0 + t) * DK + d] : from_f32<T>(0.f);
        sm.Qs[t][d] = zq;
        sm.QsT[d][t] = zq;
        sm.Ks[t][d] = zk;
    }
    for (int i = tid; i < C * DV; i += B::NT) {
        const int t = i / DV, e = i % DV;
        const T zv = t < nv ? v[(row0 + t) * DV + e] : from_f32<T>(0.f);
        const T zo = t < nv ? dout[(row0 + t) * DV + e] : from_f32<T>(0.f);
        sm.Vs[t][e] = zv;
        sm.dOs[t][e] = zo;
        sm.dOsT[e][t] = zo;
    }
    for (int i = tid; i < C * B::LC; i += B::NT) {
        (&sm.PdT[0][0])[i] = from_f32<T>(0.f);
        (&sm.PsT[0][0])[i] = from_f32<T>(0.f);
    }
    for (int i = tid; i < C * kMaxLevels; i += B::NT) {
        const int t = i / kMaxLevels, l = i % kMaxLevels;
        sm.lam[t][l] = (t < nv && l < L) ? lamg[(row0 + t) * L + l] : 0.f;
        sm.dlam[t][l] = 0.f;
    }
    if (tid < kMaxLevels)
        sm.km[tid] = 0.f;
    if (wv == 0) {
        // inclusive prefix of a over the chunk (zero past the end)
        for (int base = 0; base < C; base += 64) {
            float x = (base + lane < nv) ? a[row0 + base + lane] : 0.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x, d, 64);
                if (lane >= d)
                    x += y;
            }
            const float carry = base > 0 ? sm.Aloc[base - 1] : 0.f;
            if (base + lane < C)
                sm.Aloc[base + lane] = x + carry;
        }
    }
    __syncthreads();

    // ---- in-chunk scores: S = Q K^T, dP = dO V^T, causal tile pairs ---------
    for (int pr = wv; pr < B::CT * (B::CT + 1) / 2; pr += 4) {
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
        }
    }
    __syncthreads();

    // ---- in-chunk levels of dlambda: row sums of G over each level's keys ----
    for (int task = tid; task < C * (B::LOGC + 1); task += B::NT) {
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
        const Frag pd = frag<B>(&sm.PdT[0][0], B::LC, 16 * kt + li, u, qd);
        const Frag ps = frag<B>(&sm.PsT[0][0], B::LC, 16 * kt + li, u, qd);
#pragma unroll
        for (int j = 0; j < B::KPW; ++j)
            mma_unit(dK[j], frag<B>(&sm.QsT[0][0], B::LC, 16 * (cg + B::NCG * j) + li, u, qd), pd);
#pragma unroll
        for (int j = 0; j < B::VPW; ++j)
            mma_unit(dV[j], frag<B>(&sm.dOsT[0][0], B::LC, 16 * (cg + B::NCG * j) + li, u, qd), ps);
    }
    // The accumulators hold dK^T and dV^T tiles: A = columns (dk / dv index,
    // rows 4*qd+i), B = keys (column li).

    // ---- chunk levels -------------------------------------------------------
    // pki: this lane's part of k_s . (dk_s from later chunks), fp32
    float pki = 0.f;
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    const float *gam = Gam + (size_t)bh * N;   // chunk log-decay totals (chunks < N-1)
    for (int m = 1; m <= mtop; ++m) {
        const int half = 1 << (m - 1);
        const int b0 = (c >> m) << m;
        if ((c >> (m - 1)) & 1) {
            // query side: the left block [b0, b0 + half) -> dlambda level LOGC + m
            __syncthreads();
            if (wv == 0) {
                const float o = wave_range_sum(gam, b0 + half, c, lane);
                if (lane == 0)
                    sm.off[0] = o;
            }
            __syncthreads();
            const float offB = sm.off[0];   // log-decay from the block's end to the chunk start
            size_t offp = 0;
            for (int r = 0; r < m - 1; ++r)
                offp += ((nL >> r) + 1) >> 1;
            const T *blk = Dg + ((size_t)bh * nLeft + offp + (c >> m)) * DK * DV;
            // X^T = D^T Q^T: A = D^T (rows e), B = Q (columns t); this wave
            // takes query tile kt and value tiles cg, cg + NCG, ...
            float xs = 0.f;
#pragma unroll
            for (int j = 0; j < B::VPW; ++j) {
                const int et = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUK; ++u)
                    mma_unit(X, gfrag<B, B::NUK>(blk, et, u, lane), frag<B>(&sm.Qs[0][0], B::LQ, 16 * kt + li, u, qd));
                // X[i] = (Q D)[t = 16 kt + li][e = 16 et + 4 qd + i]
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xs += X[i] * to_f32(sm.dOs[16 * kt + li][16 * et + 4 * qd + i]);
            }
            // reduce over the four lane quads (the e rows), then over column groups
            xs += __shfl_xor(xs, 16, 64);
            xs += __shfl_xor(xs, 32, 64);
            if (qd == 0)
                sm.part[cg][16 * kt + li] = xs;
            __syncthreads();
            if (tid < C) {
                float x = 0.f;
                for (int g2 = 0; g2 < B::NCG; ++g2)
                    x += sm.part[g2][tid];
                sm.dlam[tid][B::LOGC + m] = __expf(sm.Aloc[tid] + offB) * x;
            }
        } else if (b0 + half < N) {
            // key side: the right block R = [b0 + half, b0 + 2 half) sees this chunk at level m
            __syncthreads();
            if (wv == 0) {
                const float o = wave_range_sum(gam, c + 1, b0 + half, lane);
                if (lane == 0)
                    sm.off[0] = o;
            }
            __syncthreads();
            const float offR = sm.off[0];   // log-decay from the chunk's end to R's start
            size_t ob = 0;
            for (int r = 1; r < m; ++r) {
                const int hr = 1 << (r - 1);
                ob += N > hr ? (N - hr + (1 << r) - 1) >> r : 0;
            }
            const size_t wi = (size_t)bh * NB + ob + (c >> m);
            const T *w1 = W1 + wi * DK * DV;   // W^T operand: k = dv, n = dk
            const T *w2 = W2 + wi * DK * DV;   // W operand:   k = dk, n = dv
            // this wave's key rows: decay exp(A_e - A_s)
            const float dec = __expf(sm.Aloc[C - 1] - sm.Aloc[16 * kt + li] + offR);
            float km = 0.f;   // this lane's part of the level's key-side pair mass
#pragma unroll
            for (int j = 0; j < B::KPW; ++j) {
                const int dt = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUV; ++u)
                    mma_unit(X, gfrag<B, B::NUV>(w1, dt, u, lane), frag<B>(&sm.Vs[0][0], B::LV, 16 * kt + li, u, qd));
                dK[j] += dec * X;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    km += dec * X[i] * to_f32(sm.Ks[16 * kt + li][16 * dt + 4 * qd + i]);
            }
#pragma unroll
            for (int j = 0; j < B::VPW; ++j) {
                const int et = cg + B::NCG * j;
                floatx4 X = zero4();
#pragma unroll
                for (int u = 0; u < B::NUK; ++u)
                    mma_unit(X, gfrag<B, B::NUK>(w2, et, u, lane), frag<B>(&sm.Ks[0][0], B::LQ, 16 * kt + li, u, qd));
                dV[j] += dec * X;
            }
            pki += km;
            // the level's key-side pair mass of the chunk: sum over keys of k_s . dk_s(level m)
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                km += __shfl_xor(km, o, 64);
            if (lane == 0)
                sm.kw[wv] = km;
            __syncthreads();
            if (tid == 0)
                sm.km[m] = sm.kw[0] + sm.kw[1] + sm.kw[2] + sm.kw[3];
        }
    }
    __syncthreads();

    // ---- outputs ------------------------------------------------------------
    // dk, dv: this wave's key tile kt, column tiles; rows are keys s = 16 kt + li
    const int s = 16 * kt + li;
    float pk = pki;
#pragma unroll
    for (int j = 0; j < B::KPW; ++j) {
        const int dt = cg + B::NCG * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 16 * dt + 4 * qd + i;
            if (s < nv)
                put(&dkg[(row0 + s) * DK + d], dK[j][i]);
        }
    }
#pragma unroll
    for (int j = 0; j < B::VPW; ++j) {
        const int et = cg + B::NCG * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 16 * et + 4 * qd + i;
            if (s < nv)
                put(&dvg[(row0 + s) * DV + e], dV[j][i]);
        }
    }
    pk += __shfl_xor(pk, 16, 64);
    pk += __shfl_xor(pk, 32, 64);
    if (qd == 0)
        sm.part[cg][s] = pk;
    __syncthreads();
    if (tid < C) {
        // da inside the chunk, for r = t0 + i:
        //   sum_{t >= r} (sum of P(t, s) over s <= t) - sum_{s >= r} (in-chunk P(., s))
        //   + sum_{s < r} (P(., s) over later chunks)
        // The in-chunk sums of both sides come from the same fp32 products.
        float pki_in = 0.f;
        for (int t = tid; t < C; ++t) {
            const int lev = t == tid ? 0 : bitlen_u32((uint32_t)(t ^ tid));
            pki_in += sm.lam[t][lev] * sm.G[t][tid];
        }
        float pkx = 0.f;
        for (int g2 = 0; g2 < B::NCG; ++g2)
            pkx += sm.part[g2][tid];
        float pq = 0.f;
        for (int l = 0; l < kMaxLevels; ++l)
            pq += sm.lam[tid][l] * sm.dlam[tid][l];
        sm.u[tid] = pq - pki_in;
        sm.w[tid] = pkx;
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
        // pair masses of this chunk per level (query side: into its left
        // block; key side: from its right block), for the pairs that jump
        // over other chunks
        for (int m = 1; m <= mtop; ++m) {
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
    }
    for (int i = tid; i < nv * L; i += B::NT) {
        const int t = i / L, l = i % L;
        dlamg[(row0 + t) * L + l] = sm.dlam[t][l];
    }
}

// ---------------------------------------------------------------------------
// W pieces: for level m, right block R = [j 2^m + 2^(m-1), (j+1) 2^m) and its
// piece pi (chunks R0 + pi*WP ..), the partial sum over the piece's queries of
// exp(A_t - A_e) lambda_t[LOGC + m] q_t do_t^T, e = R0*C - 1, fp32 row-major
// [dk][dv].  Grid: (pieces of all levels, BH).
// ---------------------------------------------------------------------------
template <class B>
struct WpSmem {
    using T = typename B::T;
    __attribute__((aligned(16))) T QwT[B::DK][B::LC];   // weighted q, [dk][token]
    __attribute__((aligned(16))) T dOT[B::DV][B::LC];   // do, [dv][token]
    float Aloc[B::C];
    float off;
};

__device__ __forceinline__ int wnblk(int N, int m)
{
    const int h = 1 << (m - 1);
    return N > h ? (N - h + (1 << m) - 1) >> m : 0;
}

template <class B>
__global__ __launch_bounds__(256) void ll_bwd_wpiece(const typename B::T *__restrict__ q,
                                                     const typename B::T *__restrict__ dout,
                                                     const float *__restrict__ a, const float *__restrict__ lamg,
                                                     const float *__restrict__ Gam, float *__restrict__ Wp, int Tlen,
                                                     int L, int N, int NP)
{
    using T = typename B::T;
    constexpr int C = B::C, DK = B::DK, DV = B::DV;
    __shared__ WpSmem<B> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, qd = lane >> 4;
    const int bh = blockIdx.y;
    // decode (m, block j, piece pi) from the piece index
    int x = blockIdx.x, m = 1;
    const int mtop = bitlen_u32((uint32_t)(N - 1));
    int nb = 0, np = 0;
    for (; m <= mtop; ++m) {
        nb = wnblk(N, m);
        np = ((1 << (m - 1)) + B::WP - 1) / B::WP;
        if (x < nb * np)
            break;
        x -= nb * np;
    }
    float *dst = Wp + ((size_t)bh * NP + blockIdx.x) * DK * DV;
    const int j = x / np, pi = x % np;
    const int half = 1 << (m - 1);
    const int R0 = j * (1 << m) + half;
    const int cA = R0 + pi * B::WP, cB = min(min(cA + B::WP, R0 + half), N);
    const float *gam = Gam + (size_t)bh * N;
    // every wave owns dk tiles wv, wv+4, .. x all dv tiles
    constexpr int KT = (B::DKT + 3) / 4;
    floatx4 acc[KT][B::DVT];
#pragma unroll
    for (int r = 0; r < KT; ++r)
#pragma unroll
        for (int e = 0; e < B::DVT; ++e)
            acc[r][e] = zero4();
    if (wv == 0) {
        const float o = wave_range_sum(gam, R0, cA, lane);
        if (lane == 0)
            sm.off = o;
    }
    __syncthreads();
    float off = sm.off;   // log-decay from e to the current chunk's start
    for (int cc = cA; cc < cB; ++cc) {
        const int t0 = cc * C, nv = min(C, Tlen - t0);
        const size_t row0 = (size_t)bh * Tlen + t0;
        __syncthreads();
        if (wv == 0) {
            for (int base = 0; base < C; base += 64) {
                float y = (base + lane < nv) ? a[row0 + base + lane] : 0.f;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const float z = __shfl_up(y, d, 64);
                    if (lane >= d)
                        y += z;
                }
                const float carry = base > 0 ? sm.Aloc[base - 1] : 0.f;
                if (base + lane < C)
                    sm.Aloc[base + lane] = y + carry;
            }
        }
        __syncthreads();
        for (int i = tid; i < C * DK; i += B::NT) {
            const int t = i / DK, d = i % DK;
            float w = 0.f;
            if (t < nv)
                w = __expf(off + sm.Aloc[t]) * lamg[(row0 + t) * L + B::LOGC + m] * to_f32(q[(row0 + t) * DK + d]);
            put(&sm.QwT[d][t], w);
        }
        for (int i = tid; i < C * DV; i += B::NT) {
            const int t = i / DV, e = i % DV;
            sm.dOT[e][t] = t < nv ? dout[(row0 + t) * DV + e] : from_f32<T>(0.f);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < B::NUC; ++u) {
#pragma unroll
            for (int r = 0; r < KT; ++r) {
                const int dt = wv + 4 * r;
                if (dt < B::DKT) {
                    const auto fa = frag<B>(&sm.QwT[0][0], B::LC, 16 * dt + li, u, qd);
#pragma unroll
                    for (int e = 0; e < B::DVT; ++e)
                        mma_unit(acc[r][e], fa, frag<B>(&sm.dOT[0][0], B::LC, 16 * e + li, u, qd));
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
                    dst[(size_t)(16 * dt + 4 * qd + i) * DV + 16 * e + li] = acc[r][e][i];
    }
}

// Sum of a block's pieces, written as the two operand layouts of the chunk
// kernel: W1 (k = dv, n = dk) and W2 (k = dk, n = dv), fragment order.
template <class B>
__global__ __launch_bounds__(256) void ll_bwd_wsum(const float *__restrict__ Wp, typename B::T *__restrict__ W1,
                                                   typename B::T *__restrict__ W2, int N, int NP, int NB)
{
    constexpr int DK = B::DK, DV = B::DV, KB = B::KB, EPL = B::EPL;
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
    const int j = x, half = 1 << (m - 1);
    const int R0 = j * (1 << m) + half;
    int npv = 0;   // pieces that start inside the sequence
    for (int pi = 0; pi < np; ++pi)
        if (R0 + pi * B::WP < N)
            npv = pi + 1;
    const float *src = Wp + ((size_t)bh * NP + pbase + (size_t)j * np) * DK * DV;
    typename B::T *w1 = W1 + ((size_t)bh * NB + blockIdx.x) * DK * DV;
    typename B::T *w2 = W2 + ((size_t)bh * NB + blockIdx.x) * DK * DV;
    for (int i = threadIdx.x; i < DK * DV; i += 256) {
        const int d = i / DV, e = i % DV;
        float s = 0.f;
        for (int pi = 0; pi < npv; ++pi)
            s += src[(size_t)pi * DK * DV + i];
        {   // W2: k = d, n = e
            const int u = d / KB, xk = d % KB, qd = xk / EPL, ee = xk % EPL;
            const int fv = ((e >> 4) * (DK / KB) + u) * 64 + qd * 16 + (e & 15);
            put(&w2[(size_t)fv * EPL + ee], s);
        }
        {   // W1: k = e, n = d
            const int u = e / KB, xk = e % KB, qd = xk / EPL, ee = xk % EPL;
            const int fv = ((d >> 4) * (DV / KB) + u) * 64 + qd * 16 + (d & 15);
            put(&w1[(size_t)fv * EPL + ee], s);
        }
    }
}

// da_r = da inside r's chunk (daloc) + the pairs that jump over that chunk:
// at every chunk level m the chunk c lies in one of the two sibling blocks
// B (left) and R (right) of the pair set of that level, and the jumping pairs
// are R's queries after c into B (query-side masses Mq) or B's keys before c
// seen from R (key-side masses Mk).  One workgroup per head; the masses are
// turned into exclusive prefix sums over chunks in place, level by level.
__global__ __launch_bounds__(256) void ll_bwd_da(const float *__restrict__ daloc, float *__restrict__ Mq,
                                                 float *__restrict__ Mk, float *__restrict__ da, int Tlen, int N,
                                                 int C, int mtop)
{
    __shared__ float sums[2][256];
    const int tid = threadIdx.x, bh = blockIdx.x;
    const int per = (N + 1 + 255) / 256;
    for (int m = 1; m <= mtop; ++m) {
        float *q = Mq + ((size_t)bh * kMaxLevels + m) * (N + 1);
        float *k = Mk + ((size_t)bh * kMaxLevels + m) * (N + 1);
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
        for (int j = 0; j < tid; ++j) {
            bq += sums[0][j];
            bk += sums[1][j];
        }
        for (int x = lo; x < hi; ++x) {
            const float vq = x < N ? q[x] : 0.f, vk = x < N ? k[x] : 0.f;
            q[x] = bq;
            k[x] = bk;
            bq += vq;
            bk += vk;
        }
        __syncthreads();
    }
    const size_t h = (size_t)bh * Tlen;
    int cprev = -1;
    float X = 0.f;
    for (int r = tid; r < Tlen; r += 256) {
        const int c = r / C;
        if (c != cprev) {
            X = 0.f;
            for (int m = 1; m <= mtop; ++m) {
                const float *q = Mq + ((size_t)bh * kMaxLevels + m) * (N + 1);
                const float *k = Mk + ((size_t)bh * kMaxLevels + m) * (N + 1);
                const int b0 = (c >> m) << m, half = 1 << (m - 1);
                if ((c >> (m - 1)) & 1)
                    X += q[min(b0 + 2 * half, N)] - q[c + 1];
                else
                    X += k[c] - k[b0];
            }
            cprev = c;
        }
        da[h + r] = r == 0 ? 0.f : daloc[h + r] + X;
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
    // 1. group states (one chunk per group) and the tree over chunks
    FwdArgs tree{nullptr, A.k, A.v, A.a, A.lam, nullptr, A.B, A.H, A.T, DK, DV, C, A.L, A.bf16, ws + P.off_tree};
    tree.tree_only = true;
    tree.tree_nat = A.bf16;
    hipError_t e = fwd_launch(tree, P.tree, s, nullptr);
    if (e != hipSuccess)
        return e;
    // 2. dq: the forward with q <- do, k <- v, v <- k
    FwdArgs fq{A.dout, A.v, A.k, A.a, A.lam, A.gq, A.B, A.H, A.T, DV, DK, C, A.L, A.bf16, ws + P.off_fq};
    e = fwd_launch(fq, P.fq, s, nullptr);
    if (e != hipSuccess)
        return e;
    const float *Gam = reinterpret_cast<const float *>(ws + P.off_tree + P.tree.off_Gam);
    const T *Dg = reinterpret_cast<const T *>(ws + P.off_tree + P.tree.off_Dg);
    float *Wp = reinterpret_cast<float *>(ws + P.off_wp);
    T *W1 = reinterpret_cast<T *>(ws + P.off_w1);
    T *W2 = reinterpret_cast<T *>(ws + P.off_w2);
    float *daloc = reinterpret_cast<float *>(ws + P.off_pq);
    float *Mq = reinterpret_cast<float *>(ws + P.off_mq);
    float *Mk = reinterpret_cast<float *>(ws + P.off_mk);
    // 3. W pieces and their sums
    if (P.NP > 0) {
        ProfEvents pe = prof_events("ll_bwd_wpiece");
        hipExtLaunchKernelGGL(ll_bwd_wpiece<B>, dim3(P.NP, BH), dim3(256), 0, s, pe.start, pe.stop, 0,
                              (const T *)A.q, (const T *)A.dout, A.a, A.lam, Gam, Wp, A.T, A.L, N, P.NP);
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
    hipExtLaunchKernelGGL(ll_bwd_chunk<B>, dim3(BH * N), dim3(256), 0, s, pe.start, pe.stop, 0, (const T *)A.q,
                          (const T *)A.k, (const T *)A.v, (const T *)A.dout, A.a, A.lam, Dg, Gam, (const T *)W1,
                          (const T *)W2, (T *)A.gk, (T *)A.gv, A.glam, daloc, Mq, Mk, A.T, A.L, N, P.tree.nL,
                          P.tree.nLeft, P.NB);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // 5. da
    pe = prof_events("ll_bwd_da");
    hipExtLaunchKernelGGL(ll_bwd_da, dim3(BH), dim3(256), 0, s, pe.start, pe.stop, 0, (const float *)daloc, Mq, Mk,
                          A.ga, A.T, N, C, bwd_levels(N));
    return hipGetLastError();
}

template <class DT, int DK, int DV, int C>
static BwdLauncher bwd_pick_c()
{
    using B = Bw<DT, DK, DV, C>;
    if constexpr (C % DT::KB != 0 || 4 % (C / 16) != 0 || (DK / 16) % (4 / (C / 16)) != 0 ||
                  (DV / 16) % (4 / (C / 16)) != 0) {
        return nullptr;
    } else if constexpr (sizeof(BwSmem<B>) > 160 * 1024 || sizeof(WpSmem<B>) > 64 * 1024) {
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

BwdPlan bwd_plan(int B, int H, int T, int dk, int dv, int chunk)
{
    BwdPlan p;
    const size_t BH = (size_t)B * H;
    const int N = (T + chunk - 1) / chunk;
    p.tree = fwd_plan(B, H, T, dk, dv, chunk, 0, 4);
    p.fq = fwd_plan(B, H, T, dv, dk, chunk, -1, 4);
    bwd_counts(N, p.NP, p.NB, 8);
    const size_t st = (size_t)dk * dv;
    p.off_tree = 0;
    p.off_fq = al256(p.off_tree + p.tree.bytes);
    p.off_wp = al256(p.off_fq + p.fq.bytes);
    p.off_w1 = al256(p.off_wp + BH * p.NP * st * 4);
    p.off_w2 = al256(p.off_w1 + BH * p.NB * st * 4);
    p.off_pq = al256(p.off_w2 + BH * p.NB * st * 4);
    p.off_mq = al256(p.off_pq + BH * T * 4);
    p.off_mk = al256(p.off_mq + BH * kMaxLevels * (size_t)(N + 1) * 4);
    p.bytes = al256(p.off_mk + BH * kMaxLevels * (size_t)(N + 1) * 4);
    return p;
}

hipError_t bwd_launch(const BwdArgs &args, const BwdPlan &plan, hipStream_t stream)
{
    BwdLauncher f = find_bwd(args.bf16, args.dk, args.dv, args.chunk);
    if (!f)
        return hipErrorInvalidValue;
    return f(args, plan, stream);
}

}  // namespace ll
