// Decode stack left by a prefill (a forward over a prompt of T tokens), gfx950.
//
// The recurrent form keeps, for the most recent position, one state per
// Fenwick level ("Log-Linear Attention", Portuguese page §2 "Forma Recorrente
// e Paralela", decoding bullet; French page §2 "Algorithmes Efficaces").
// After a prompt whose last token sits at p = T - 1, slot 0 holds that token's
// k v^T and slot l >= 1 holds the level-l bucket of p, the 2^(l-1) keys
// [lo, lo + 2^(l-1)) with lo = (p >> l) << l, present iff bit l-1 of p is set
// (Portuguese page §2 "Particionamento Hierárquico").  Each slot is stored as
// (hat S, g), true state exp(g) hat S, with
//   hat S = sum_{s in bucket} exp(sum of a over (s, hi-1]) k_s v_s^T
//   g     = sum of a over [hi, p],          hi = one past the bucket's last key,
// i.e. decayed to the bucket's own end, as the decode step keeps its slots.
//
// The forward has already formed the state of every group of G*C tokens but
// the last (fp32, decayed to the group's end) and each group's decay total.
// A bucket of at least G*C keys is a union of whole groups, so its hat S is a
// decay-weighted sum of group states; a smaller bucket lies inside the
// prompt's last group and is summed from k, v and a.
//
// One workgroup per (head, slot, slice of 16 dk rows); each thread owns a few
// elements of the slice, so every output element is written once, in
// row-major [dk][dv] order.  Free slots are not written.
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

template <class DT, int DK_, int DV_>
struct Stk {
    using T = typename DT::T;
    static constexpr int DK = DK_, DV = DV_;
    static constexpr int NT = 256;
    static constexpr int RS = 16;          // dk rows per workgroup
    static constexpr int NTR = NT / DV;    // rows covered by one pass of the threads
    static constexpr int NE = RS / NTR;    // elements per thread
    static constexpr int TB = 64;          // keys staged per pass
    static constexpr int MAXB = NT;        // longest bucket summed from keys
    static_assert(NT % DV == 0 && RS % NTR == 0, "thread layout");
    static_assert(DK % RS == 0, "dk slices");
};

__device__ __forceinline__ float block_sum(float x, float *red)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0)
        red[tid >> 6] = x;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        s += red[w];
    return s;
}

template <class D>
__global__ __launch_bounds__(256) void ll_prefill_stack(const typename D::T *__restrict__ k,
                                                        const typename D::T *__restrict__ v,
                                                        const float *__restrict__ a, const float *__restrict__ Sg,
                                                        const float *__restrict__ Gam, int Tlen, int lgc, int nG,
                                                        int nL, float *__restrict__ state,
                                                        float *__restrict__ logscale, int Lcap)
{
    constexpr int DK = D::DK, DV = D::DV, NE = D::NE, NTR = D::NTR;
    __shared__ float wl[D::MAXB];
    __shared__ float ks[D::TB][D::RS];
    __shared__ float vs[D::TB][DV];
    __shared__ float red[4];

    const int tid = threadIdx.x;
    const int nsl = DK / D::RS;
    const int bh = blockIdx.x / nsl, row0 = (blockIdx.x % nsl) * D::RS;
    const int l = blockIdx.y;
    const int p = Tlen - 1;
    if (l > 0 && !((p >> (l - 1)) & 1))
        return;  // free slot
    const int lo = l == 0 ? p : (p >> l) << l;
    const int n = l == 0 ? 1 : 1 << (l - 1);
    const int hi = lo + n;
    const int t0 = (p >> lgc) << lgc;  // first key of the prompt's last group
    const bool whole = l >= 1 && l - 1 >= lgc;
    const int c = tid % DV, rr = tid / DV;
    const size_t head = (size_t)bh * Tlen;

    // g: decay from the bucket's end to p, over whole groups then keys
    float gt = 0.f;
    if (whole) {
        const int gl = p >> lgc;
        for (int j = (hi >> lgc) + tid; j < gl; j += D::NT)
            gt += Gam[(size_t)bh * nG + j];
    }
    for (int r = max(hi, t0) + tid; r <= p; r += D::NT)
        gt += a[head + r];
    gt = block_sum(gt, red);

    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
        acc[e] = 0.f;

    if (whole) {
        // Groups j1-1 down to j0, each weighted by the decay of the groups
        // after it inside the bucket; four group states in flight.
        const int j0 = lo >> lgc, j1 = hi >> lgc;
        const float *gam = Gam + (size_t)bh * nG;
        const float *base = Sg + ((size_t)bh * nL * DK + row0 + rr) * DV + c;
        float run = 0.f;
        for (int j = j1 - 1; j >= j0; j -= 4) {
            float x[4][NE], gj[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = j - u >= j0;
                gj[u] = ok ? gam[j - u] : 0.f;
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    x[u][e] = ok ? base[((size_t)(j - u) * DK + NTR * e) * DV] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w = __expf(run);
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    acc[e] += w * x[u][e];
                run += gj[u];
            }
        }
    } else {
        // Keys lo .. hi-1 (n <= MAXB): log-weight of key lo+i is the sum of
        // a over (lo+i, hi-1], a suffix scan over the bucket.
        wl[tid] = (tid + 1 < n) ? a[head + lo + tid + 1] : 0.f;
        __syncthreads();
        for (int off = 1; off < n; off <<= 1) {
            const float y = wl[tid] + ((tid + off < n) ? wl[tid + off] : 0.f);
            __syncthreads();
            wl[tid] = y;
            __syncthreads();
        }
        wl[tid] = __expf(wl[tid]);
        for (int b0 = 0; b0 < n; b0 += D::TB) {
            const int cnt = min(D::TB, n - b0);
            __syncthreads();
            for (int i = tid; i < cnt * D::RS; i += D::NT) {
                const int t = i / D::RS, r = i % D::RS;
                ks[t][r] = to_f32(k[(head + lo + b0 + t) * DK + row0 + r]);
            }
            for (int i = tid; i < cnt * DV; i += D::NT) {
                const int t = i / DV, cc = i % DV;
                vs[t][cc] = to_f32(v[(head + lo + b0 + t) * DV + cc]);
            }
            __syncthreads();
            for (int t = 0; t < cnt; ++t) {
                const float wv = wl[b0 + t] * vs[t][c];
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    acc[e] += ks[t][rr + NTR * e] * wv;
            }
        }
    }

    float *dst = state + (((size_t)bh * Lcap + l) * DK + row0 + rr) * DV + c;
#pragma unroll
    for (int e = 0; e < NE; ++e)
        dst[(size_t)NTR * e * DV] = acc[e];
    if (row0 == 0 && tid == 0)
        logscale[(size_t)bh * Lcap + l] = gt;
}

typedef hipError_t (*StackLauncher)(const StackArgs &, hipStream_t);

template <class DT, int DK, int DV>
static hipError_t launch_stack_t(const StackArgs &A, hipStream_t s)
{
    using D = Stk<DT, DK, DV>;
    using T = typename D::T;
    const ProfEvents pe = prof_events("ll_prefill_stack");
    const dim3 grid(A.BH * (DK / D::RS), A.Lcap);
    hipExtLaunchKernelGGL(ll_prefill_stack<D>, grid, dim3(D::NT), 0, s, pe.start, pe.stop, 0, (const T *)A.k,
                          (const T *)A.v, A.a, A.Sg, A.Gam, A.T, A.lgc, A.nG, A.nL, A.state, A.logscale, A.Lcap);
    return hipGetLastError();
}

template <class DT, int DK>
static StackLauncher stk_pick_dv(int dv)
{
    switch (dv) {
    case 16: return &launch_stack_t<DT, DK, 16>;
    case 32: return &launch_stack_t<DT, DK, 32>;
    case 64: return &launch_stack_t<DT, DK, 64>;
    case 128: return &launch_stack_t<DT, DK, 128>;
    default: return nullptr;
    }
}

template <class DT>
static StackLauncher stk_pick(int dk, int dv)
{
    switch (dk) {
    case 16: return stk_pick_dv<DT, 16>(dv);
    case 32: return stk_pick_dv<DT, 32>(dv);
    case 64: return stk_pick_dv<DT, 64>(dv);
    case 128: return stk_pick_dv<DT, 128>(dv);
    default: return nullptr;
    }
}

bool stack_supported(bool bf16, int dk, int dv)
{
    return (bf16 ? stk_pick<TBF16>(dk, dv) : stk_pick<TF32>(dk, dv)) != nullptr;
}

hipError_t stack_launch(const StackArgs &args, hipStream_t stream)
{
    StackLauncher f = args.bf16 ? stk_pick<TBF16>(args.dk, args.dv) : stk_pick<TF32>(args.dk, args.dv);
    if (!f || args.lgc < 0 || args.lgc > 9)
        return hipErrorInvalidValue;
    return f(args, stream);
}

}  // namespace ll
