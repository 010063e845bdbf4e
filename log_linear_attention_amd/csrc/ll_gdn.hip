// Log-Linear Gated DeltaNet forward (float32), gfx950.
//
// The log-linear construction multiplies a linear-attention model's own
// attention matrix elementwise with the hierarchical (Fenwick) mask,
// P = A ⊙ M_H, O = P V ("Log-Linear Attention", Portuguese page §2
// "Metodologia", hierarchical-mask point; French page §3 "Contributions
// Clés"), and the pages name Gated DeltaNet as the second model so treated.
// Gated DeltaNet's recurrence (its own publication) is
//   S_t = S_{t-1} M_t + beta_t v_t k_t^T,  M_t = exp(a_t) (I - beta_t k_t k_t^T),
// o_t = S_t q_t, so its attention matrix is A[t,s] = beta_s k_s^T M_{s+1}..M_t q_t
// and the log-linear output is o_t = sum_s lambda_t[level(t,s)] A[t,s] v_s.
//
// Chunkwise evaluation (chunk of C tokens starting at c0; Aloc = in-chunk
// inclusive prefix of a, gamma_i = exp(Aloc[i])):
//  - In-chunk pairs.  With pseudo-values u (S_t = sum_s (gamma_t/gamma_s) u_s k_s^T
//    for a zero incoming state), u solves X u = diag(beta) v where
//    X = I + strictly-lower(beta_i (gamma_i/gamma_j) k_i.k_j); hence
//    A = ((Q K^T) ⊙ Gamma ⊙ causal) X^{-1} diag(beta) for the chunk's pairs.
//    Z = Y X^{-1} is multiplied by the in-chunk levels' lambda.
//  - Product of the chunk's transitions.  Without the scalar decays the
//    product of (I - beta_r k_r k_r^T) over r = 0..i is I - sum_{r<=i} w_r k_r^T
//    with w_i = beta_i (k_i - sum_{j<i} (k_i.k_j) w_j) (a compact WY form),
//    i.e. X0 W = diag(beta) K with X0 = I + strictly-lower(beta_i k_i.k_j), so
//    Phi_c = M_0 .. M_{C-1} = gamma_{C-1} (I - W^T K) and the query carried to
//    the chunk start is qt_i = M_0 .. M_i q_i = gamma_i (q_i - sum_{r<=i} (q_i.k_r) w_r).
//  - X = Gamma X0 Gamma^{-1}, so one inverse serves the three systems:
//    T = X0^{-1} is formed by 16 x 16 blocks (diagonal blocks by
//    substitution, the others from block rows of X0 T = I on MFMA), then
//    W = T diag(beta) K, U = X^{-1} diag(beta) V and Z are MFMA products,
//    with X^{-1}[i][j] = (gamma_i/gamma_j) T[i][j].
//  - Chunk state (keys of the chunk, at its end): H = sum_s (gamma_end/gamma_s) u_s k_s^T.
//  - Tree over chunks (left child L, right child R): D = D_L Phi_R + D_R,
//    Phi = Phi_L Phi_R.  Stored transposed (Phi^T [dk][dk], D^T [dk][dv]) so
//    the walk's reads run along rows.
//  - Walk: for chunk c and each set bit m-1 of c, the level-(log2 C + m)
//    bucket is the left-child block at tree level m-1; its contribution to
//    row i is lambda_i[log2 C + m] D qt_i^(m), where qt^(m) is qt carried
//    through the finer buckets' blocks: qt^(m') = Phi(block m) qt^(m) for
//    the next set bit m' > m.
//
// All arithmetic is float32 (FMA and fp32 MFMA); decays enter only as exp
// of non-positive differences for a <= 0.
#include <hip/hip_ext.h>

#include <type_traits>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

// Buffer resource over `bytes` bytes at p (loads past the range return zero)
// and a 16-byte load through it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gdn_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ float4 gdn_load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <class DT, int DK_, int DV_, int C_>
struct Gdn {
    using T = typename DT::T;   // q, k, v and out; everything else is float32
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static constexpr int NT = 256;
    // chunk kernel threads: its LDS allows one workgroup per CU at chunk 64
    // (16 waves) and two at chunk 32 (8 waves each)
    static constexpr int CNT = C == 64 ? 1024 : 512;
    // walk threads: up to 512, at most C rows per 4-column group of either product
    static constexpr int WNT = C * (DK < DV ? DK : DV) / 4 < 512 ? C * (DK < DV ? DK : DV) / 4 : 512;
    static constexpr int LOGC = C == 32 ? 5 : 6;
    static_assert(C * DV % NT == 0 && C * DK % NT == 0 && NT % DV == 0 && NT % DK == 0, "thread layout");
    // The pseudo-values U get a buffer of their own (and are formed beside W
    // and Z) when the chunk kernel's LDS allows one.
    static constexpr int LDS_WITH_U = 4 * (C * (DK + 4) * 2 + C * (DV + 4) * 2 + 3 * C * (C + 4) + C * (LOGC + 4));
    static constexpr bool SEPU = LDS_WITH_U <= 160 * 1024;
    static_assert(C / 16 <= CNT / 64, "one wave per off-diagonal block of the inverse");
};

template <class G>
struct GdnChunkSmem {
    // rows padded to a multiple of four floats (16-byte rows for float4 reads)
    __attribute__((aligned(16))) float QW[G::C][G::DK + 4];   // Q, then W
    __attribute__((aligned(16))) float Ks[G::C][G::DK + 4];
    __attribute__((aligned(16))) float Vs[G::C][G::DV + 4];   // V, then the pseudo-values U
    __attribute__((aligned(16))) float M1[G::C][G::C + 4];    // S = Q K^T
    __attribute__((aligned(16))) float M2[G::C][G::C + 4];    // X0 (lower) and blocks of the inverse (upper); then Z, the weighted A
    __attribute__((aligned(16))) float M3[G::C][G::C + 4];    // T = X0^{-1} (lower)
    __attribute__((aligned(16))) float Us[G::SEPU ? G::C : 1][G::DV + 4];   // pseudo-values (when separate)
    float Aloc[G::C];
    float beta[G::C];
    float wend[G::C];         // exp(Aloc[C-1] - Aloc[s])
    float lam[G::C][G::LOGC + 1];
};

// Workgroups b, b + 8, b + 16, ... run on one XCD (workgroups are dealt
// round-robin over the eight XCDs).  This numbering gives each XCD a
// contiguous range of the nb items, so items that read the same data share
// that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nb)
{
    const int per = nb >> 3, rem = nb & 7, xcd = bid & 7;
    return xcd * per + min(xcd, rem) + (bid >> 3);
}

__device__ __forceinline__ int bitlen(unsigned x) { return x ? 32 - __builtin_clz(x) : 0; }

// Tree offsets: level p holds N >> p blocks; levels are stored one after
// another per head.
__device__ __forceinline__ size_t gdn_level_off(int N, int p)
{
    size_t off = 0;
    for (int r = 0; r < p; ++r)
        off += (size_t)(N >> r);
    return off;
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Four consecutive input elements as float32.
__device__ __forceinline__ float4 ld4t(const float *p) { return ld4(p); }
__device__ __forceinline__ float4 ld4t(const __bf16 *p)
{
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

// The same through a buffer resource (zero past its range): elements
// 4 e4 .. 4 e4 + 3 of the resource's base.
__device__ __forceinline__ float4 ld4b(__amdgpu_buffer_rsrc_t r, int e4, const float *)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * e4, 0, 0));
}
__device__ __forceinline__ float4 ld4b(__amdgpu_buffer_rsrc_t r, int e4, const __bf16 *)
{
    const bf16x4 x = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, 8 * e4, 0, 0));
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

__device__ __forceinline__ void st4t(float *p, const float4 &x) { *reinterpret_cast<float4 *>(p) = x; }
__device__ __forceinline__ void st4t(__bf16 *p, const float4 &x)
{
    const bf16x4 y = {(__bf16)x.x, (__bf16)x.y, (__bf16)x.z, (__bf16)x.w};
    *reinterpret_cast<bf16x4 *>(p) = y;
}

// U tile (si, sc) of U = X^{-1} diag(beta) V, with X^{-1}[i][j] =
// (gamma_i / gamma_j) T[i][j] (T = X0^{-1} in M3, lower triangle), the decay
// applied to each T element as it is loaded (the factor is exp of a
// non-positive difference on and below the diagonal; zero above it).
template <class G, class SM>
__device__ __forceinline__ floatx4 gdn_u_tile(const SM &sm, int si, int sc, int li, int qd)
{
    constexpr int C = G::C;
    floatx4 acc = zero4();
    const int i = 16 * si + li;   // this lane's row of the A operand
    const float ai = sm.Aloc[i];
    for (int j0 = 0; j0 <= 16 * si; j0 += 16) {
        floatx4 af = lds_frag(&sm.M3[0][0], C + 4, i, j0, qd), bf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 4 * qd + e;
            af[e] = j <= i ? af[e] * __expf(ai - sm.Aloc[j]) : 0.f;
            bf[e] = sm.beta[j] * sm.Vs[j][16 * sc + li];
        }
        mma_unit(acc, af, bf);
    }
    return acc;
}

template <class G>
__global__ __launch_bounds__(G::CNT) void ll_gdn_chunk(const typename G::T *__restrict__ q,
                                                      const typename G::T *__restrict__ k,
                                                      const typename G::T *__restrict__ v, const float *__restrict__ a,
                                                      const float *__restrict__ beta, const float *__restrict__ lam,
                                                      float *__restrict__ out, float *__restrict__ qt,
                                                      float *__restrict__ Phit, float *__restrict__ Dt, int Tlen,
                                                      int L, int N, int NBT)
{
    constexpr int C = G::C, DK = G::DK, DV = G::DV, NT = G::CNT;
    __shared__ GdnChunkSmem<G> sm;
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / N, c = blockIdx.x % N;
    const int t0 = c * C, valid = min(C, Tlen - t0);
    const size_t row0 = (size_t)bh * Tlen + t0;

    // ---- stage the chunk (rows past the sequence end: zero keys, values,
    // queries, beta and a, i.e. identity transitions and no writes) ----
    // every load is issued before the first LDS store, as buffer loads over
    // the valid rows (zero past them) on every path, so that the chunk waits
    // for one round trip
    using T = typename G::T;
    constexpr int NQ4 = (C * DK / 4 + NT - 1) / NT, NV4 = (C * DV / 4 + NT - 1) / NT;
    constexpr int NL = (C * (G::LOGC + 1) + NT - 1) / NT;
    float4 rq[NQ4], rk[NQ4], rv[NV4];
    float rl[NL], rbeta, ra;
    {
        const int es = (int)sizeof(T);
        const __amdgpu_buffer_rsrc_t r_q = gdn_rsrc(q + row0 * DK, valid * DK * es);
        const __amdgpu_buffer_rsrc_t r_k = gdn_rsrc(k + row0 * DK, valid * DK * es);
        const __amdgpu_buffer_rsrc_t r_v = gdn_rsrc(v + row0 * DV, valid * DV * es);
        const __amdgpu_buffer_rsrc_t r_l = gdn_rsrc(lam + row0 * L, valid * L * 4);
#pragma unroll
        for (int u = 0; u < NQ4; ++u) {
            const int e = tid + u * NT;
            const int e4 = e < C * DK / 4 ? e : C * DK / 4;   // past the tile: past the range
            rq[u] = ld4b(r_q, e4, q);
            rk[u] = ld4b(r_k, e4, k);
        }
#pragma unroll
        for (int u = 0; u < NV4; ++u) {
            const int e = tid + u * NT;
            rv[u] = ld4b(r_v, e < C * DV / 4 ? e : C * DV / 4, v);
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = tid + u * NT, i = e / (G::LOGC + 1), l = e % (G::LOGC + 1);
            const int off = (e < C * (G::LOGC + 1) && l < L) ? (i * L + l) * 4 : valid * L * 4;
            rl[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_l, off, 0, 0));
        }
        rbeta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gdn_rsrc(beta + row0, valid * 4), tid * 4, 0, 0));
        ra = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(gdn_rsrc(a + row0, valid * 4), tid * 4, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < NQ4; ++u) {
        const int e = tid + u * NT, i = e / (DK / 4), d = 4 * (e % (DK / 4));
        if (e < C * DK / 4) {
            *reinterpret_cast<float4 *>(&sm.QW[i][d]) = rq[u];
            *reinterpret_cast<float4 *>(&sm.Ks[i][d]) = rk[u];
        }
    }
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
        const int e = tid + u * NT, i = e / (DV / 4), d = 4 * (e % (DV / 4));
        if (e < C * DV / 4)
            *reinterpret_cast<float4 *>(&sm.Vs[i][d]) = rv[u];
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int e = tid + u * NT;
        if (e < C * (G::LOGC + 1))
            sm.lam[e / (G::LOGC + 1)][e % (G::LOGC + 1)] = rl[u];
    }
    if (tid < C) {
        sm.beta[tid] = rbeta;
        sm.Aloc[tid] = ra;
    }
    __syncthreads();
    if (tid < 64) {
        // inclusive prefix of a over the chunk (C <= 64), one wave
        float x = tid < C ? sm.Aloc[tid] : 0.f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (tid >= d)
                x += y;
        }
        if (tid < C)
            sm.Aloc[tid] = x;
    }
    __syncthreads();
    if (tid < C)
        sm.wend[tid] = __expf(sm.Aloc[C - 1] - sm.Aloc[tid]);

    const int lane = tid & 63, wv = tid >> 6, qd = lane >> 4, li = lane & 15;
    constexpr int NWV = NT / 64, TB = C / 16;

    // ---- S = Q K^T and X0[i][j] = beta_i k_i.k_j (j < i): 16 x 16 tiles on fp32 MFMA,
    // one tile per wave at a time (the strictly upper tiles of K K^T skipped) ----
    {
        for (int b = wv; b < 2 * TB * TB; b += NWV) {
            const bool isg = b >= TB * TB;
            const int bb = isg ? b - TB * TB : b;
            const int si = bb / TB, sj = bb % TB;
            if (isg && sj > si)
                continue;
            // two independent accumulators over alternate 16-wide units
            floatx4 acc = zero4(), acc1 = zero4();
            const float *A = isg ? &sm.Ks[0][0] : &sm.QW[0][0];
#pragma unroll 2
            for (int k0 = 0; k0 < DK; k0 += 32) {
                mma_unit(acc, lds_frag(A, DK + 4, 16 * si + li, k0, qd), lds_frag(&sm.Ks[0][0], DK + 4, 16 * sj + li, k0, qd));
                mma_unit(acc1, lds_frag(A, DK + 4, 16 * si + li, k0 + 16, qd),
                         lds_frag(&sm.Ks[0][0], DK + 4, 16 * sj + li, k0 + 16, qd));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] += acc1[r];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * si + 4 * qd + r, j = 16 * sj + li;
                if (!isg)
                    sm.M1[i][j] = acc[r];
                else if (j < i)
                    sm.M2[i][j] = sm.beta[i] * acc[r];
            }
        }
    }
    __syncthreads();

    // ---- T = X0^{-1} (unit lower triangular) into M3, by 16 x 16 blocks.
    // Diagonal blocks by substitution, one column per thread:
    //   T_bb[r][c] = delta_rc - sum_{m<r} X0_bb[r][m] T_bb[m][c] ----
    if (tid < C) {
        const int b0 = 16 * (tid >> 4), cc = tid & 15;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = r == cc ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m)
                x -= sm.M2[b0 + r][b0 + m] * t[m];
            t[r] = x;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sm.M3[b0 + r][b0 + cc] = t[r];
    }
    __syncthreads();
    // Blocks below the diagonal, one block distance dd = i - j at a time, one
    // wave per block: T_ij = -T_ii R with R = sum_{m=j}^{i-1} X0_im T_mj (from
    // block row i of X0 T = I).  R waits in M2's strictly upper block (j, i),
    // which holds nothing else.
    for (int dd = 1; dd < TB; ++dd) {
        if (wv < TB - dd) {
            const int j = wv, i = wv + dd;
            floatx4 acc = zero4();
            for (int m = j; m < i; ++m) {
                floatx4 bf;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bf[e] = sm.M3[16 * m + 4 * qd + e][16 * j + li];
                mma_unit(acc, lds_frag(&sm.M2[0][0], C + 4, 16 * i + li, 16 * m, qd), bf);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.M2[16 * j + 4 * qd + r][16 * i + li] = acc[r];
        }
        __syncthreads();
        if (wv < TB - dd) {
            const int j = wv, i = wv + dd;
            floatx4 acc = zero4(), bf;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bf[e] = sm.M2[16 * j + 4 * qd + e][16 * i + li];
            mma_unit(acc, lds_frag(&sm.M3[0][0], C + 4, 16 * i + li, 16 * i, qd), bf);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.M3[16 * i + 4 * qd + r][16 * j + li] = -acc[r];
        }
        __syncthreads();
    }

    // ---- products of T, side by side on fp32 MFMA (T's blocks above the
    // diagonal are never read):
    //  W = T diag(beta) K over Q's storage;
    //  U = X^{-1} diag(beta) V into its own buffer (when there is one);
    //  Z = Y X^{-1} into M2, Z[i][j] = (gamma_i / gamma_j) sum_{j<=r<=i} S[i][r] T[r][j]
    //  (the decays of Y = S ⊙ Gamma and of X^{-1} meet in one factor per element) ----
    {
        constexpr int TD = DK / 16, TV = DV / 16;
        constexpr int NWT = TB * TD, NUT = G::SEPU ? TB * TV : 0, NZT = TB * (TB + 1) / 2;
        for (int b = wv; b < NWT + NUT + NZT; b += NWV) {
            if (b < NWT) {
                const int si = b / TD, sd = b % TD;
                floatx4 acc = zero4();
                for (int j0 = 0; j0 <= 16 * si; j0 += 16) {
                    floatx4 bf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = j0 + 4 * qd + e;
                        bf[e] = sm.beta[r] * sm.Ks[r][16 * sd + li];
                    }
                    mma_unit(acc, bf, lds_frag(&sm.M3[0][0], C + 4, 16 * si + li, j0, qd));   // transposed tile
                }
                *reinterpret_cast<float4 *>(&sm.QW[16 * si + li][16 * sd + 4 * qd]) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else if (b < NWT + NUT) {
                if constexpr (G::SEPU) {
                    const int si = (b - NWT) / TV, sc = (b - NWT) % TV;
                    const floatx4 acc = gdn_u_tile<G>(sm, si, sc, li, qd);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sm.Us[16 * si + 4 * qd + r][16 * sc + li] = acc[r];
                }
            } else {
                int sj = b - NWT - NUT, si = 0;   // lower tile (si, sj), sj <= si
                while (sj > si) {
                    sj -= si + 1;
                    ++si;
                }
                const int i = 16 * si + li;
                floatx4 acc = zero4();
                for (int rb = sj; rb <= si; ++rb) {
                    floatx4 af = lds_frag(&sm.M1[0][0], C + 4, i, 16 * rb, qd), bf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * rb + 4 * qd + e;
                        if (r > i)
                            af[e] = 0.f;   // S is used on and below the diagonal
                        bf[e] = sm.M3[r][16 * sj + li];
                    }
                    mma_unit(acc, bf, af);   // transposed tile: row i, columns 4qd .. 4qd + 3
                }
                float4 z;
                float *zp = &z.x;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = 16 * sj + 4 * qd + r;
                    zp[r] = jj <= i ? __expf(sm.Aloc[i] - sm.Aloc[jj]) * acc[r] : 0.f;
                }
                *reinterpret_cast<float4 *>(&sm.M2[i][16 * sj + 4 * qd]) = z;
            }
        }
    }
    __syncthreads();

    // ---- carried queries qt_i = gamma_i (q_i - sum_{r<=i} S[i][r] w_r), 16 x 16 tiles
    // formed transposed so that a lane writes four consecutive columns of its row;
    // weighted in-chunk attention A'[i][j] = lambda_i[level(i,j)] Z[i][j] beta_j (j <= i) ----
    float *qtc = qt + ((size_t)bh * N + c) * C * DK;
    {
        constexpr int TD = DK / 16;
        for (int b = wv; b < TB * TD; b += NWV) {
            const int si = b / TD, sd = b % TD;
            floatx4 acc = zero4();
            const int i = 16 * si + li;   // this lane's row of the A operand
            for (int r0 = 0; r0 <= 16 * si; r0 += 16) {
                floatx4 af = lds_frag(&sm.M1[0][0], C + 4, i, r0, qd), bf;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r0 + 4 * qd + e;
                    if (r > i)
                        af[e] = 0.f;   // S is used on and below the diagonal
                    bf[e] = sm.QW[r][16 * sd + li];
                }
                mma_unit(acc, bf, af);   // transposed tile: row i, columns 4qd .. 4qd + 3
            }
            const int d = 16 * sd + 4 * qd;
            const float4 qv = i < valid ? ld4t(q + (row0 + i) * DK + d) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float gq = __expf(sm.Aloc[i]);
            *reinterpret_cast<float4 *>(qtc + (size_t)i * DK + d) =
                make_float4(gq * (qv.x - acc[0]), gq * (qv.y - acc[1]), gq * (qv.z - acc[2]), gq * (qv.w - acc[3]));
        }
    }
    for (int e = tid; e < C * C; e += NT) {
        const int i = e / C, j = e % C;
        if (j <= i)
            sm.M2[i][j] *= sm.lam[i][bitlen((unsigned)(i ^ j))] * sm.beta[j];
    }
    __syncthreads();

    // ---- in-chunk output O = A' V: 16 x 16 tiles on fp32 MFMA ----
    {
        constexpr int TV = DV / 16;
        for (int b = wv; b < TB * TV; b += NWV) {
            const int si = b / TV, sc = b % TV;
            floatx4 acc = zero4();
            for (int j0 = 0; j0 <= 16 * si; j0 += 16) {   // A' is zero above the diagonal
                floatx4 bf;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bf[e] = sm.Vs[j0 + 4 * qd + e][16 * sc + li];
                mma_unit(acc, bf, lds_frag(&sm.M2[0][0], C + 4, 16 * si + li, j0, qd));   // transposed tile
            }
            const int i = 16 * si + li;
            if (i < valid)
                *reinterpret_cast<float4 *>(out + (row0 + i) * DV + 16 * sc + 4 * qd) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }

    // ---- pseudo-values in place of V when they have no buffer of their own:
    // every U tile held in registers until all reads of V are done ----
    if constexpr (!G::SEPU) {
        constexpr int TV = DV / 16, NUT = TB * TV, PER = (NUT + NWV - 1) / NWV;
        floatx4 ut[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int b = wv + p * NWV;
            if (b < NUT)
                ut[p] = gdn_u_tile<G>(sm, b / TV, b % TV, li, qd);
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int b = wv + p * NWV;
            if (b < NUT) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm.Vs[16 * (b / TV) + 4 * qd + r][16 * (b % TV) + li] = ut[p][r];
            }
        }
    }
    __syncthreads();

    // ---- level-0 tree entries of this chunk: Phi^T = gamma_end (I - K^T W), D^T = K^T diag(wend) U ----
    const size_t blk = (size_t)bh * NBT + c;
    float *P = Phit + blk * DK * DK;
    float *D = Dt + blk * DK * DV;
    const float gend = __expf(sm.Aloc[C - 1]);
    {
        // Phi^T[k][n] = gend (delta - sum_r K[r][k] W[r][n]);  D^T[d][c] = sum_s wend[s] K[s][d] U[s][c].
        // One 32 x 32 block (2 x 2 tiles) per wave at a time: each operand
        // fragment serves two tiles, and the four accumulators are independent.
        constexpr int TK = DK / 16, TV = DV / 16, NPB = (TK / 2) * (TK / 2), NDB = (TK / 2) * (TV / 2);
        static_assert(TK % 2 == 0 && TV % 2 == 0, "2 x 2 tiles");
        const float (*U)[DV + 4] = G::SEPU ? sm.Us : sm.Vs;
        for (int b = wv; b < NPB + NDB; b += NWV) {
            const bool isd = b >= NPB;
            const int bb = isd ? b - NPB : b, tn = isd ? TV / 2 : TK / 2;
            const int sk = 2 * (bb / tn), sn = 2 * (bb % tn);
            // tiles formed transposed (rows k, columns n) so that each lane
            // holds four consecutive columns of a stored row: one 16-byte store
            floatx4 acc[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
#pragma unroll 2
            for (int r0 = 0; r0 < C; r0 += 16) {
                floatx4 af[2], bf[2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r0 + 4 * qd + e;
                    const float wk = isd ? sm.wend[r] : 1.f;
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        af[x][e] = isd ? U[r][16 * (sn + x) + li] : sm.QW[r][16 * (sn + x) + li];
                        bf[x][e] = wk * sm.Ks[r][16 * (sk + x) + li];
                    }
                }
#pragma unroll
                for (int y = 0; y < 2; ++y)
#pragma unroll
                    for (int x = 0; x < 2; ++x)
                        mma_unit(acc[y][x], af[x], bf[y]);
            }
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int row = 16 * (sk + y) + li, col = 16 * (sn + x) + 4 * qd;   // acc[rr]: (row, col + rr)
                    const floatx4 &v = acc[y][x];
                    if (isd) {
                        *reinterpret_cast<float4 *>(D + (size_t)row * DV + col) = make_float4(v[0], v[1], v[2], v[3]);
                    } else {
                        float4 o;
                        o.x = gend * ((row == col ? 1.f : 0.f) - v[0]);
                        o.y = gend * ((row == col + 1 ? 1.f : 0.f) - v[1]);
                        o.z = gend * ((row == col + 2 ? 1.f : 0.f) - v[2]);
                        o.w = gend * ((row == col + 3 ? 1.f : 0.f) - v[3]);
                        *reinterpret_cast<float4 *>(P + (size_t)row * DK + col) = o;
                    }
                }
        }
    }
}

// One tree level p >= 1: block j from its children 2j (L) and 2j+1 (R) at
// level p-1:  Phi^T = Phi_R^T Phi_L^T,  D^T = Phi_R^T D_L^T + D_R^T.
// Output [DK rows] x [DK + DV columns] in 64 x 64 tiles (rows x columns;
// DK < 64: DK rows) on fp32 MFMA, 16 x 16 subtiles spread over the four
// waves, each formed transposed (B^T A^T) so that a lane holds four
// consecutive columns of a row and writes them with one 16-byte store.
// Both operands are staged through LDS 32 contraction rows at a time with
// 16-byte loads; the next slice is loaded into registers before
// the current one is multiplied, so its latency overlaps the MFMAs.
template <class G>
__global__ __launch_bounds__(256) void ll_gdn_tree(float *__restrict__ Phit, float *__restrict__ Dt, int N, int NBT,
                                                   int p)
{
    constexpr int DK = G::DK, DV = G::DV, NC = DK + DV;
    constexpr int TS = DK < 64 ? DK : 64;            // tile edge (rows and columns)
    constexpr int TR = DK / TS, TN = (NC + TS - 1) / TS;
    constexpr int KS = 32;                            // contraction rows per stage (two MFMA units)
    static_assert(DK % KS == 0, "stage width divides dk");
    constexpr int SR = TS / 16, ST = SR * SR, NSW = (ST + 3) / 4;   // 16 x 16 subtiles, per wave
    constexpr int NA = (TS * KS / 4 + 255) / 256, NB = (KS * TS / 4 + 255) / 256;   // float4 loads per thread
    __shared__ __attribute__((aligned(16))) float As[TS][KS + 4];   // As[r][k] = Phi_R^T[row0 + r][k0 + k]
    __shared__ __attribute__((aligned(16))) float Bs[KS][TS + 4];   // Bs[k][n] = [Phi_L^T | D_L^T][k0 + k][col0 + n]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    const int bh = blockIdx.y;
    // the tiles of one merge, and neighbouring merges, on one XCD
    const int bx = xcd_contiguous(blockIdx.x, gridDim.x);
    const int tile = bx % (TR * TN), j = bx / (TR * TN);
    const int tr = tile / TN, tn = tile % TN;
    const size_t child0 = (size_t)bh * NBT + gdn_level_off(N, p - 1);
    const size_t L = child0 + 2 * (size_t)j, R = L + 1;
    const size_t self = (size_t)bh * NBT + gdn_level_off(N, p) + j;
    const float *PR = Phit + R * DK * DK;
    const float *PL = Phit + L * DK * DK;
    const float *DL = Dt + L * DK * DV;
    const int row0 = TS * tr, col0 = TS * tn;

    float4 ra[NA], rb[NB];
    // Slice k0 of both operands into registers.  Columns come in groups of
    // four that never straddle the Phi / D boundary (dk and dv are multiples
    // of 16); columns past DK + DV read as zero.
    // The loads are issued on every path (the pieces past the operands, and
    // the columns past DK + DV, read as zero from buffer loads past their
    // range): a load skipped on some path would make the compiler wait for
    // every outstanding load, the prefetched slice included, at the next use.
    const __amdgpu_buffer_rsrc_t rPR = gdn_rsrc(PR, DK * DK * 4), rPL = gdn_rsrc(PL, DK * DK * 4),
                                 rDL = gdn_rsrc(DL, DK * DV * 4);
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int e = tid + 256 * i;
            const int r = e / (KS / 4), k4 = 4 * (e % (KS / 4));
            const int off = e < TS * KS / 4 ? ((row0 + r) * DK + k0 + k4) * 4 : DK * DK * 4;
            ra[i] = gdn_load16(rPR, off);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i;
            const int kk = e / (TS / 4), col = col0 + 4 * (e % (TS / 4));
            const bool in = e < KS * TS / 4;
            // one of the two loads is past its range (or both, past the columns)
            const int offL = in && col < DK ? ((k0 + kk) * DK + col) * 4 : DK * DK * 4;
            const int offD = in && col >= DK && col < NC ? ((k0 + kk) * DV + col - DK) * 4 : DK * DV * 4;
            const float4 a = gdn_load16(rPL, offL), b = gdn_load16(rDL, offD);
            rb[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        }
    };

    floatx4 acc[NSW];
#pragma unroll
    for (int x = 0; x < NSW; ++x)
        acc[x] = zero4();
    gload(0);
    for (int k0 = 0; k0 < DK; k0 += KS) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int e = tid + 256 * i;
            if (e < TS * KS / 4)
                *reinterpret_cast<float4 *>(&As[e / (KS / 4)][4 * (e % (KS / 4))]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int e = tid + 256 * i;
            if (e < KS * TS / 4)
                *reinterpret_cast<float4 *>(&Bs[e / (TS / 4)][4 * (e % (TS / 4))]) = rb[i];
        }
        __syncthreads();
        if (k0 + KS < DK)
            gload(k0 + KS);
#pragma unroll
        for (int ku = 0; ku < KS; ku += 16) {
            if constexpr (SR == 4) {
                // wave w: column subtile w, row subtiles 0..3 (one B fragment per unit)
                floatx4 bf;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bf[e] = Bs[ku + 4 * qd + e][16 * w + li];
#pragma unroll
                for (int x = 0; x < NSW; ++x)
                    mma_unit(acc[x], bf, lds_frag(&As[0][0], KS + 4, 16 * x + li, ku, qd));
            } else {
#pragma unroll
                for (int x = 0; x < NSW; ++x) {
                    const int st = w + 4 * x;
                    if (st < ST) {
                        const int sr = st / SR, sc = st % SR;
                        floatx4 bf;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bf[e] = Bs[ku + 4 * qd + e][16 * sc + li];
                        mma_unit(acc[x], bf, lds_frag(&As[0][0], KS + 4, 16 * sr + li, ku, qd));
                    }
                }
            }
        }
    }
#pragma unroll
    for (int x = 0; x < NSW; ++x) {
        const int st = SR == 4 ? 4 * x + w : w + 4 * x;   // row subtile x, column subtile w when SR == 4
        if (st < ST) {
            const int sr = st / SR, sc = st % SR;
            // transposed tile: lane (li, qd) holds row li, columns 4qd .. 4qd + 3
            const int row = row0 + 16 * sr + li, col = col0 + 16 * sc + 4 * qd;
            float4 o = make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
            if (col < DK) {
                *reinterpret_cast<float4 *>(Phit + self * DK * DK + (size_t)row * DK + col) = o;
            } else if (col < NC) {
                const float4 d = ld4(Dt + R * DK * DV + (size_t)row * DV + col - DK);
                o.x += d.x; o.y += d.y; o.z += d.z; o.w += d.w;
                *reinterpret_cast<float4 *>(Dt + self * DK * DV + (size_t)row * DV + col - DK) = o;
            }
        }
    }
}

constexpr int kGdnKS = 16;   // rows of the walk's right operand staged at a time (one fp32 MFMA unit)

// Tiles of Y B (Y: C x DK rows in LDS, B: DK x NB row-major in global memory)
// on fp32 MFMA, 16 x 16 output tiles t = w, w + NW, ... of wave w; B is
// staged through LDS (Bs) one 16-row unit at a time, read once per
// workgroup, with the next three units in flight in registers while the
// current one is multiplied.  Every thread of the workgroup (NW waves) must call
// this.  Tiles are formed transposed (B^T Y^T), so acc tile j of the wave
// holds row 16 * (t / (NB/16)) + li, columns 16 * (t % (NB/16)) + 4*qd + r.
template <int NTW, int NW, int C, int DK, int LDY, int NB, bool DIRECT>
__device__ __forceinline__ void gdn_tiles_mma(const float (*Y)[LDY], const float *B, float *Bs, int w, int li, int qd,
                                              floatx4 (&acc)[NTW])
{
    constexpr int TN = NB / 16, TT = (C / 16) * TN;
    constexpr int NTH = 64 * NW, NE = kGdnKS * NB / 4, NR = (NE + NTH - 1) / NTH;   // float4 per thread and unit
    constexpr int NU = DK / kGdnKS, PD = NU < 3 ? NU : 3;   // units, and units in flight
    const int tid = threadIdx.x;
    if constexpr (DIRECT && NW % TN == 0) {
        // The wave's column tile nt is fixed: it reads its own B fragments
        // (rows k0 + 4 qd + e, column 16 nt + li) straight from global memory,
        // three units ahead, with no LDS stage and no barrier.  Y must be
        // visible to every wave on entry.
        constexpr int PB = NU < 3 ? NU : 3;
        const __amdgpu_buffer_rsrc_t rB = gdn_rsrc(B, DK * NB * 4);
        const int col = 16 * (w % TN) + li;
        floatx4 bq[PB];
        auto ldb = [&](int k, floatx4 &r) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rB, ((k * kGdnKS + 4 * qd + e) * NB + col) * 4, 0, 0));
        };
#pragma unroll
        for (int k = 0; k < PB; ++k)
            ldb(k, bq[k]);
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            acc[j] = zero4();
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const floatx4 bf = bq[k % PB];
            if (k + PB < NU)
                ldb(k + PB, bq[k % PB]);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int t = w + NW * j;
                if (t < TT)
                    mma_unit(acc[j], bf, lds_frag(&Y[0][0], LDY, 16 * (t / TN) + li, k * kGdnKS, qd));
            }
        }
        return;
    }
    // unit k of B into registers: buffer loads issued on every path (past the
    // unit's elements: past the range, zero), so the compiler waits for
    // exactly the unit it stores and the later ones stay in flight
    const __amdgpu_buffer_rsrc_t rB = gdn_rsrc(B, DK * NB * 4);
    float4 rb[PD][NR];
    auto ld_unit = [&](int k, float4 (&r)[NR]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e = tid + NTH * i;
            r[i] = gdn_load16(rB, e < NE ? (k * kGdnKS * NB + 4 * e) * 4 : DK * NB * 4);
        }
    };
#pragma unroll
    for (int k = 0; k < PD; ++k)
        ld_unit(k, rb[k]);
#pragma unroll
    for (int j = 0; j < NTW; ++j)
        acc[j] = zero4();
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        const int k0 = k * kGdnKS;
        __syncthreads();   // the previous unit has been read
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (tid + NTH * i < NE)
                *reinterpret_cast<float4 *>(Bs + 4 * (tid + NTH * i)) = rb[k % PD][i];
        __syncthreads();
        if (k + PD < NU)
            ld_unit(k + PD, rb[k % PD]);
        if constexpr (NW % TN == 0) {
            // the wave's column tile is the same for all its tiles: one B fragment
            const int nt = w % TN;
            floatx4 bf;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bf[e] = Bs[(4 * qd + e) * NB + 16 * nt + li];
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int t = w + NW * j;
                if (t < TT)
                    mma_unit(acc[j], bf, lds_frag(&Y[0][0], LDY, 16 * (t / TN) + li, k0, qd));
            }
        } else {
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int t = w + NW * j;
                if (t < TT) {
                    const int it = t / TN, nt = t % TN;
                    const floatx4 af = lds_frag(&Y[0][0], LDY, 16 * it + li, k0, qd);
                    floatx4 bf;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        bf[e] = Bs[(4 * qd + e) * NB + 16 * nt + li];
                    mma_unit(acc[j], bf, af);
                }
            }
        }
    }
}

// Chunk-level buckets: out[i] = obuf[i] + sum over set bits m-1 of c of
// lambda_i[log2 C + m] D_m qt_i^(m), with the carried query moved through
// each used block's transition before the next, coarser one.  The products
// run on fp32 MFMA.
template <class G>
__global__ __launch_bounds__(G::WNT) void ll_gdn_walk(const float *__restrict__ lam, const float *__restrict__ qt,
                                                     const float *__restrict__ Phit, const float *__restrict__ Dt,
                                                     const float *obuf, typename G::T *out, int Tlen, int L, int N,
                                                     int NBT)
{
    constexpr int C = G::C, DK = G::DK, DV = G::DV, NT = G::WNT, NW = NT / 64;
    constexpr int T1 = (C / 16) * (DV / 16), T2 = (C / 16) * (DK / 16);
    constexpr int N1 = (T1 + NW - 1) / NW, N2 = (T2 + NW - 1) / NW;
    // right operands read straight from global memory (no LDS stage) for
    // states of at most 128 x 64 (larger ones would take more registers than
    // two workgroups per CU allow)
    constexpr bool DIRECT = DK * DV <= 128 * 64;
    __shared__ __attribute__((aligned(16))) float Y[2][C][DK + 4];
    __shared__ __attribute__((aligned(16))) float Bs[kGdnKS * (DK > DV ? DK : DV)];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;
    // neighbouring chunks of a head (which read the same finer blocks) on one XCD
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const int bh = item / N, c = item % N;
    const int t0 = c * C, valid = min(C, Tlen - t0);
    const size_t row0 = (size_t)bh * Tlen + t0;
    if (c == 0) {
        // no chunk-level bucket: the in-chunk output is the output
        if constexpr (!std::is_same<typename G::T, float>::value)
            for (int e = tid; e < valid * DV / 4; e += NT)
                st4t(out + row0 * DV + 4 * e, ld4(obuf + row0 * DV + 4 * e));
        return;
    }
    const float *qtc = qt + ((size_t)bh * N + c) * C * DK;
    for (int e = tid; e < C * DK / 4; e += NT) {
        const int i = e / (DK / 4), d4 = e % (DK / 4);
        *reinterpret_cast<float4 *>(&Y[0][i][4 * d4]) = *reinterpret_cast<const float4 *>(qtc + (size_t)i * DK + 4 * d4);
    }
    __syncthreads();   // Y[0] visible to every wave
    floatx4 acc[N1];
#pragma unroll
    for (int j = 0; j < N1; ++j)
        acc[j] = zero4();
    int cur = 0;
    const int top = bitlen((unsigned)c);
    for (int m = 1; m <= top; ++m) {
        if (!((c >> (m - 1)) & 1))
            continue;
        const int p = m - 1, jb = (c >> m) << 1;
        const size_t blk = (size_t)bh * NBT + gdn_level_off(N, p) + jb;
        floatx4 tmp[N1];
        gdn_tiles_mma<N1, NW, C, DK, DK + 4, DV, DIRECT>(Y[cur], Dt + blk * DK * DV, Bs, w, li, qd, tmp);
#pragma unroll
        for (int j = 0; j < N1; ++j) {
            const int t = w + NW * j;
            if (t < T1) {
                const int i = 16 * (t / (DV / 16)) + li;
                const float lw = i < valid ? lam[(row0 + i) * L + G::LOGC + m] : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[j][r] += lw * tmp[j][r];
            }
        }
        if ((c >> m) == 0)
            break;   // no coarser bucket
        // carry the queries through this block: Y' = Y Phi^T
        floatx4 ny[N2];
        gdn_tiles_mma<N2, NW, C, DK, DK + 4, DK, DIRECT>(Y[cur], Phit + blk * DK * DK, Bs, w, li, qd, ny);
#pragma unroll
        for (int j = 0; j < N2; ++j) {
            const int t = w + NW * j;
            if (t < T2) {
                const int i = 16 * (t / (DK / 16)) + li, n = 16 * (t % (DK / 16)) + 4 * qd;
                *reinterpret_cast<float4 *>(&Y[cur ^ 1][i][n]) = make_float4(ny[j][0], ny[j][1], ny[j][2], ny[j][3]);
            }
        }
        __syncthreads();
        cur ^= 1;
    }
#pragma unroll
    for (int j = 0; j < N1; ++j) {
        const int t = w + NW * j;
        if (t < T1) {
            const int i = 16 * (t / (DV / 16)) + li, n = 16 * (t % (DV / 16)) + 4 * qd;
            if (i < valid) {
                const size_t o = (row0 + i) * DV + n;
                const float4 b = ld4(obuf + o);
                st4t(out + o, make_float4(b.x + acc[j][0], b.y + acc[j][1], b.z + acc[j][2], b.w + acc[j][3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int host_bitlen(int x)
{
    int n = 0;
    while (x > 0) {
        ++n;
        x >>= 1;
    }
    return n;
}

GdnPlan gdn_plan(int B, int H, int T, int dk, int dv, int chunk)
{
    GdnPlan p;
    const size_t BH = (size_t)B * H;
    p.N = (T + chunk - 1) / chunk;
    p.P = p.N > 1 ? host_bitlen(p.N - 1) - 1 : 0;   // deepest tree level the walk reads
    p.NBT = 0;
    for (int r = 0; r <= p.P; ++r)
        p.NBT += p.N >> r;
    const size_t qt = BH * p.N * chunk * dk * 4;
    const size_t ph = BH * p.NBT * (size_t)dk * dk * 4;
    const size_t dd = BH * p.NBT * (size_t)dk * dv * 4;
    p.off_qt = 0;
    p.off_phi = (qt + 255) & ~(size_t)255;
    p.off_d = (p.off_phi + ph + 255) & ~(size_t)255;
    p.off_oi = (p.off_d + dd + 255) & ~(size_t)255;   // float32 in-chunk output (bf16 inputs)
    p.bytes = (p.off_oi + BH * (size_t)T * dv * 4 + 255) & ~(size_t)255;
    return p;
}

typedef hipError_t (*GdnLauncher)(const GdnArgs &, const GdnPlan &, hipStream_t);

template <class DT, int DK, int DV, int C>
static hipError_t launch_gdn_t(const GdnArgs &A, const GdnPlan &P, hipStream_t s)
{
    using G = Gdn<DT, DK, DV, C>;
    using T = typename G::T;
    constexpr bool F32 = std::is_same<T, float>::value;
    const int BH = A.B * A.H;
    char *ws = static_cast<char *>(A.workspace);
    float *qt = reinterpret_cast<float *>(ws + P.off_qt);
    float *Phit = reinterpret_cast<float *>(ws + P.off_phi);
    float *Dt = reinterpret_cast<float *>(ws + P.off_d);
    // float32 outputs are accumulated in place; bf16 ones through a float32 buffer
    float *obuf = F32 ? static_cast<float *>(A.out) : reinterpret_cast<float *>(ws + P.off_oi);
    ProfEvents pe = prof_events("ll_gdn_chunk");
    hipExtLaunchKernelGGL(ll_gdn_chunk<G>, dim3(BH * P.N), dim3(G::CNT), 0, s, pe.start, pe.stop, 0,
                          (const T *)A.q, (const T *)A.k, (const T *)A.v, A.a, A.beta, A.lam, obuf, qt, Phit, Dt,
                          A.T, A.L, P.N, P.NBT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    constexpr int TS = DK < 64 ? DK : 64;
    constexpr int tiles = (DK / TS) * ((DK + DV + TS - 1) / TS);
    for (int p = 1; p <= P.P; ++p) {
        pe = prof_events("ll_gdn_tree");
        hipExtLaunchKernelGGL(ll_gdn_tree<G>, dim3(tiles * (P.N >> p), BH), dim3(256), 0, s, pe.start, pe.stop, 0,
                              Phit, Dt, P.N, P.NBT, p);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    if (P.N > 1 || !F32) {
        pe = prof_events("ll_gdn_walk");
        hipExtLaunchKernelGGL(ll_gdn_walk<G>, dim3(BH * P.N), dim3(G::WNT), 0, s, pe.start, pe.stop, 0, A.lam,
                              (const float *)qt, (const float *)Phit, (const float *)Dt, (const float *)obuf,
                              (T *)A.out, A.T, A.L, P.N, P.NBT);
        e = hipGetLastError();
    }
    return e;
}

template <class DT, int DK, int DV>
static GdnLauncher gdn_pick_c(int chunk)
{
    switch (chunk) {
    case 32: return &launch_gdn_t<DT, DK, DV, 32>;
    case 64: return &launch_gdn_t<DT, DK, DV, 64>;
    default: return nullptr;
    }
}

template <class DT, int DK>
static GdnLauncher gdn_pick_dv(int dv, int chunk)
{
    switch (dv) {
    case 32: return gdn_pick_c<DT, DK, 32>(chunk);
    case 64: return gdn_pick_c<DT, DK, 64>(chunk);
    case 128: return gdn_pick_c<DT, DK, 128>(chunk);
    default: return nullptr;
    }
}

template <class DT>
static GdnLauncher gdn_pick(int dk, int dv, int chunk)
{
    switch (dk) {
    case 32: return gdn_pick_dv<DT, 32>(dv, chunk);
    case 64: return gdn_pick_dv<DT, 64>(dv, chunk);
    case 128: return gdn_pick_dv<DT, 128>(dv, chunk);
    default: return nullptr;
    }
}

static GdnLauncher find_gdn(bool bf16, int dk, int dv, int chunk)
{
    return bf16 ? gdn_pick<TBF16>(dk, dv, chunk) : gdn_pick<TF32>(dk, dv, chunk);
}

bool gdn_supported(int dk, int dv, int chunk) { return find_gdn(false, dk, dv, chunk) != nullptr; }

hipError_t gdn_launch(const GdnArgs &args, const GdnPlan &plan, hipStream_t stream)
{
    GdnLauncher f = find_gdn(args.bf16, args.dk, args.dv, args.chunk);
    if (!f)
        return hipErrorInvalidValue;
    return f(args, plan, stream);
}

}  // namespace ll
