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
// A bucket of at least one group (G*C keys) is exactly one of the left-child
// block states the forward's tree has stored for its chunk walk (decayed to
// the block's end, in fragment order and the input dtype), or, after the
// one-launch forward, the Fenwick node of its last group, so it is copied
// out in row-major order.  A smaller bucket lies inside the prompt's last
// group and is summed from k, v and a: the decay-weighted keys and the values
// are staged in LDS and contracted over keys with fp32 MFMA.
//
// One workgroup per (head, slot, slice of 16 dk rows).  Free slots are not
// written.  In a batch of prompts padded to one length, each sequence's
// stack is that of its own last position: every bucket of a position p lies
// in [0, p], so the padding never enters, and the whole-group buckets are
// tree blocks that end before p's group.
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

template <class DT, int DK_, int DV_>
struct Stk {
    using T = typename DT::T;
    using DTag = DT;
    static constexpr int DK = DK_, DV = DV_;
    static constexpr int NT = 256;
    static constexpr int RS = 16;                 // dk rows per workgroup
    static constexpr int NE = RS * DV / NT;       // block-state copy: one row, NE consecutive columns per thread
    static constexpr int TB = 64;                 // keys staged per pass
    static constexpr int MAXB = NT;               // longest bucket summed from keys
    static constexpr int VEC = 16 / (int)sizeof(T);  // elements of one 16-byte load
    static constexpr int KV = RS / VEC;           // 16-byte pieces of a key's row slice
    static constexpr int VV = DV / VEC;           // 16-byte pieces of a value row
    static constexpr int NKL = (TB * KV + NT - 1) / NT;
    static constexpr int NVL = (TB * VV + NT - 1) / NT;
    static constexpr int LDK = RS + 4;            // LDS rows: the four lane quads of an operand read
    static constexpr int LDV = DV + 4;            // land on disjoint bank groups
    static constexpr int NTL = DV / 16;           // 16x16 output tiles of the slice
    static constexpr int TPW = (NTL + 3) / 4;     // tiles per wave
    static constexpr int NPASS = MAXB / TB;       // passes of the longest bucket
    static constexpr int PF = sizeof(T) == 2 ? NPASS : 2;  // passes in flight (register budget)
    static constexpr int KB = DT::KB, EPL = DT::EPL, NUK = DK / KB;
    static_assert(NE >= 1 && RS * DV == NE * NT && NE <= 16, "thread layout");
    static_assert(DK % RS == 0 && RS % VEC == 0 && DV % VEC == 0, "vector layout");
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

// Unpack one 16-byte piece of T into floats.
__device__ __forceinline__ void unpack16(float *dst, const uint4 &u, float)
{
    dst[0] = __uint_as_float(u.x); dst[1] = __uint_as_float(u.y);
    dst[2] = __uint_as_float(u.z); dst[3] = __uint_as_float(u.w);
}

__device__ __forceinline__ void unpack16(float *dst, const uint4 &u, __bf16)
{
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dst[2 * i] = __uint_as_float(w[i] << 16);
        dst[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Position of state row x (0 <= x < KB) of a unit inside its fragment: lane
// quad and element within the lane's 16 bytes.
template <class DT>
__device__ __forceinline__ void frag_pos(int x, bool nat, int &qd, int &e)
{
    if constexpr (DT::EPL == 8) {
        if (nat) {
            qd = x >> 3;
            e = x & 7;
        } else {   // unit_row: x = 16 (e >> 2) + 4 qd + (e & 3)
            qd = (x >> 2) & 3;
            e = ((x >> 4) << 2) | (x & 3);
        }
    } else {       // fp32 units: x = 4 qd + e
        qd = x >> 2;
        e = x & 3;
    }
}

template <class D>
__global__ __launch_bounds__(256) void ll_prefill_stack(const typename D::T *__restrict__ k,
                                                        const typename D::T *__restrict__ v,
                                                        const float *__restrict__ a,
                                                        const typename D::T *__restrict__ Dg,
                                                        const float *__restrict__ Gam, int Tlen, int lgc, int nG,
                                                        int nL, int nLeft, int nat, float *__restrict__ state,
                                                        float *__restrict__ logscale, int Lcap, int rqk,
                                                        const int *__restrict__ lens, int H, int fused)
{
    using T = typename D::T;
    constexpr int DK = D::DK, DV = D::DV, VEC = D::VEC;
    __shared__ float wl[D::MAXB];
    __shared__ __attribute__((aligned(16))) float ks[D::TB][D::LDK];  // decay-weighted key rows
    __shared__ __attribute__((aligned(16))) float vs[D::TB][D::LDV];
    __shared__ float red[4];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nsl = DK / D::RS;
    const int bh = blockIdx.x / nsl, row0 = (blockIdx.x % nsl) * D::RS;
    // Dispatch order: the longest bucket summed from keys first (its sum is
    // the longest chain of work), then the block-state buckets from the top
    // down, then the shorter key buckets.
    const int lb = min(lgc, Lcap - 1), y = blockIdx.y;
    const int l = y == 0 ? lb : (y <= Lcap - 1 - lb ? Lcap - y : Lcap - 1 - y);
    // Prompt length of this sequence: Tlen, or its own length in a batch of
    // prompts padded to Tlen.  A length outside [0, Tlen] cannot be served:
    // every logscale entry of the sequence becomes NaN and no state is
    // written; an empty prompt leaves an empty stack (nothing written).
    const int Tb = lens ? lens[bh / H] : Tlen;
    if (Tb < 0 || Tb > Tlen) {
        if (row0 == 0 && tid == 0)
            logscale[(size_t)bh * Lcap + l] = __builtin_nanf("");
        return;
    }
    if (Tb == 0)
        return;
    const int p = Tb - 1;
    if (l > 0 && !((p >> (l - 1)) & 1))
        return;  // free slot
    const int lo = l == 0 ? p : (p >> l) << l;
    const int n = l == 0 ? 1 : 1 << (l - 1);
    const int hi = lo + n;
    const int t0 = (p >> lgc) << lgc;  // first key of the prompt's last group
    const bool whole = l >= 1 && l - 1 >= lgc;
    const size_t head = (size_t)bh * Tlen, khead = (size_t)(bh / rqk) * Tlen;   // k is shared by rqk heads
    float *slot = state + (((size_t)bh * Lcap + l) * DK + row0) * DV;

    // Independent loads first: the tail decay's terms, the bucket's decays,
    // and the key passes that fit in registers.
    float gt = 0.f;
    if (whole) {
        const int gl = p >> lgc;
        if (fused) {
            // the groups between the bucket and p's group are the Fenwick
            // nodes of the set bits of gl below the bucket's bit
            for (int kk = tid; kk < l - lgc - 1; kk += D::NT)
                if ((gl >> kk) & 1)
                    gt += Gam[(size_t)bh * nG + ((gl >> (kk + 1)) << (kk + 1)) + (1 << kk) - 1];
        } else {
            for (int j = (hi >> lgc) + tid; j < gl; j += D::NT)
                gt += Gam[(size_t)bh * nG + j];
        }
    }
    for (int t = max(hi, t0) + tid; t <= p; t += D::NT)
        gt += a[head + t];
    float av = 0.f;
    uint4 kr[D::PF][D::NKL], vr[D::PF][D::NVL];
    auto issue = [&](int b0, uint4 (&kq)[D::NKL], uint4 (&vq)[D::NVL]) {
        const int cnt = min(D::TB, n - b0);
#pragma unroll
        for (int u = 0; u < D::NKL; ++u) {
            const int i = tid + D::NT * u;
            if (i < cnt * D::KV)
                kq[u] = *reinterpret_cast<const uint4 *>(k + (khead + lo + b0 + i / D::KV) * DK + row0 +
                                                          (i % D::KV) * VEC);
        }
#pragma unroll
        for (int u = 0; u < D::NVL; ++u) {
            const int i = tid + D::NT * u;
            if (i < cnt * D::VV)
                vq[u] = *reinterpret_cast<const uint4 *>(v + (head + lo + b0) * DV + (size_t)i * VEC);
        }
    };
    if (!whole) {
        av = (tid + 1 < n) ? a[head + lo + tid + 1] : 0.f;
#pragma unroll
        for (int pp = 0; pp < D::PF; ++pp)
            if (pp * D::TB < n)
                issue(pp * D::TB, kr[pp], vr[pp]);
    }

    if (whole) {
        // Left child at tree level pl = l - lgc - 1 (blocks of 2^pl groups),
        // index 2 * (gl >> (pl + 1)); the tree stores level pl's left children
        // after those of the levels below it.
        const int pl = l - lgc - 1, gl = p >> lgc;
        const T *blk;
        if (fused) {
            // the node of the bucket's last group (2^pl groups ending there)
            blk = Dg + ((size_t)bh * nG + ((gl >> (pl + 1)) << (pl + 1)) + (1 << pl) - 1) * DK * DV;
        } else {
            size_t off = 0;
            for (int r = 0; r < pl; ++r)
                off += ((nL >> r) + 1) >> 1;
            blk = Dg + ((size_t)bh * nLeft + off + (gl >> (pl + 1))) * DK * DV;
        }
        const int r = tid / (DV / D::NE), c0 = (tid % (DV / D::NE)) * D::NE;
        const int row = row0 + r, u = row / D::KB;
        int qd, e;
        frag_pos<typename D::DTag>(row % D::KB, nat != 0, qd, e);
        float x[D::NE];
#pragma unroll
        for (int j = 0; j < D::NE; ++j) {
            const int col = c0 + j;
            const int fv = ((col >> 4) * D::NUK + u) * 64 + qd * 16 + (col & 15);
            x[j] = to_f32(blk[(size_t)fv * D::EPL + e]);
        }
        float *dst = slot + (size_t)r * DV + c0;
        if constexpr (D::NE % 4 == 0) {
#pragma unroll
            for (int j = 0; j < D::NE / 4; ++j)
                reinterpret_cast<float4 *>(dst)[j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < D::NE; ++j)
                dst[j] = x[j];
        }
    } else {
        // Keys lo .. hi-1 (n <= MAXB): the log-weight of key lo+i is the sum
        // of a over (lo+i, hi-1], a suffix scan over the bucket: within each
        // wave by shuffles, then across the four waves.
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float t = __shfl_down(av, d, 64);
            if (lane + d < 64)
                av += t;
        }
        if (lane == 0)
            red[wv] = av;
        __syncthreads();
        for (int w2 = wv + 1; w2 < 4; ++w2)
            av += red[w2];
        wl[tid] = __expf(av);

        // Each wave owns output tiles wv, wv+4, ... (16 rows x 16 columns)
        // and sums them with fp32 MFMA over 16 keys at a time.
        floatx4 dacc[D::TPW];
#pragma unroll
        for (int j = 0; j < D::TPW; ++j)
            dacc[j] = zero4();
        const int li = lane & 15, qd = lane >> 4;
        auto pass = [&](int b0, uint4 (&kq)[D::NKL], uint4 (&vq)[D::NVL]) {
            const int cnt = min(D::TB, n - b0);
            const int cnt16 = (cnt + 15) & ~15;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < D::NKL; ++u) {
                const int i = tid + D::NT * u;
                if (i < cnt * D::KV) {
                    const int t = i / D::KV, rr = (i % D::KV) * VEC;
                    float x[VEC];
                    unpack16(x, kq[u], T{});
                    const float w = wl[b0 + t];
#pragma unroll
                    for (int j = 0; j < VEC; j += 4)
                        *reinterpret_cast<float4 *>(&ks[t][rr + j]) =
                            make_float4(w * x[j], w * x[j + 1], w * x[j + 2], w * x[j + 3]);
                }
            }
#pragma unroll
            for (int u = 0; u < D::NVL; ++u) {
                const int i = tid + D::NT * u;
                if (i < cnt * D::VV) {
                    const int t = i / D::VV, cc = (i % D::VV) * VEC;
                    float x[VEC];
                    unpack16(x, vq[u], T{});
#pragma unroll
                    for (int j = 0; j < VEC; j += 4)
                        *reinterpret_cast<float4 *>(&vs[t][cc + j]) = make_float4(x[j], x[j + 1], x[j + 2], x[j + 3]);
                }
            }
            // keys past the bucket's end in the last 16-key unit are zero
            for (int i = tid; i < (cnt16 - cnt) * (D::RS + DV); i += D::NT) {
                const int t = cnt + i / (D::RS + DV), rc = i % (D::RS + DV);
                if (rc < D::RS)
                    ks[t][rc] = 0.f;
                else
                    vs[t][rc - D::RS] = 0.f;
            }
            if (b0 + D::PF * D::TB < n)
                issue(b0 + D::PF * D::TB, kq, vq);
            __syncthreads();
            for (int t = 0; t < cnt16; t += 16) {
                const int tk = t + 4 * qd;
                const floatx4 ka = {ks[tk][li], ks[tk + 1][li], ks[tk + 2][li], ks[tk + 3][li]};
#pragma unroll
                for (int j = 0; j < D::TPW; ++j) {
                    const int c = 16 * (wv + 4 * j) + li;
                    if (wv + 4 * j < D::NTL) {
                        const floatx4 vb = {vs[tk][c], vs[tk + 1][c], vs[tk + 2][c], vs[tk + 3][c]};
                        mma_unit(dacc[j], ka, vb);
                    }
                }
            }
        };
#pragma unroll
        for (int pp = 0; pp < D::NPASS; ++pp)
            if (pp * D::TB < n)
                pass(pp * D::TB, kr[pp % D::PF], vr[pp % D::PF]);
        // accumulator lane layout: rows 4*qd .. 4*qd+3 of column li
        float *dst = slot + (size_t)(4 * qd) * DV + li;
#pragma unroll
        for (int j = 0; j < D::TPW; ++j) {
            const int tt = wv + 4 * j;
            if (tt < D::NTL)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(size_t)i * DV + 16 * tt] = dacc[j][i];
        }
    }
    __syncthreads();  // red is reused
    gt = block_sum(gt, red);
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
                          (const T *)A.v, A.a, (const T *)A.Dg, A.Gam, A.T, A.lgc, A.nG, A.nL, A.nLeft, (int)A.nat,
                          A.state, A.logscale, A.Lcap, A.rqk, A.lens, A.H, (int)A.fused);
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
