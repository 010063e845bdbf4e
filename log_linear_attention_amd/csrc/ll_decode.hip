// Batched decode step of log-linear attention (Mamba-2 form) for gfx950.
//
// The recurrent form keeps O(log T) states per sequence; each new token goes
// into the finest level and the levels are merged and promoted the way a
// Fenwick tree carries ("Log-Linear Attention", Portuguese page §2 "Forma
// Recorrente e Paralela", decoding bullet; French page §2 "Algorithmes
// Efficaces", inference bullet).  With the new token at position t and
// kc = number of trailing zero bits of t, the buckets of levels 0..kc of the
// previous position merge into level kc+1, every older bucket only decays, and
// the new token alone forms level 0.
//
// Each slot stores (hat S, g) with true state exp(g) hat S, so buckets that
// only decay cost one scalar update instead of a 32 KiB rewrite; the step
// reads each occupied slot once and writes two (the merged bucket and the new
// token).  The work is memory-bound: one workgroup per (sequence, head) streams
// its occupied slots with 16-byte loads, accumulates q^T S per column group in
// registers and reduces over dk in LDS.
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

template <class DT, int DK_, int DV_>
struct Dec {
    using T = typename DT::T;
    static constexpr int DK = DK_, DV = DV_;
    static constexpr int NT = 256;
    static constexpr int NV4 = DK * DV / 4;                  // float4 vectors per slot
    static constexpr int NPT = (NV4 + NT - 1) / NT;          // vectors per thread
    static constexpr int CG = DV / 4;                        // column groups
    static_assert((NT * 4) % DV == 0, "a thread must keep one column group");
};

// Stack slots are touched once per step: stream them past the caches.
__device__ __forceinline__ float4 nt_load(const float4 *p)
{
    const floatx4 x = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void nt_store(float4 *p, const float4 &v)
{
    const floatx4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<floatx4 *>(p));
}

// Accumulate one slot's share x (this thread's float4 vectors) either into
// the merged bucket M (levels <= kc) or into the read-out partial sums.
template <class D>
__device__ __forceinline__ void decode_slot(const float4 *x, float4 *M, float *part, bool merge, float scale,
                                            const float *qs, int tid)
{
#pragma unroll
    for (int r = 0; r < D::NPT; ++r) {
        const int idx = tid + D::NT * r;
        if (idx < D::NV4) {
            if (merge) {
                M[r].x += scale * x[r].x; M[r].y += scale * x[r].y;
                M[r].z += scale * x[r].z; M[r].w += scale * x[r].w;
            } else {
                const float qc = scale * qs[idx * 4 / D::DV];
                part[0] += qc * x[r].x; part[1] += qc * x[r].y;
                part[2] += qc * x[r].z; part[3] += qc * x[r].w;
            }
        }
    }
}

// Slots a step at position t reads: slot 0 and one per set bit of t - 1
// (none for t = 0 or a position the stack cannot hold).
__device__ __forceinline__ int decode_occ(int64_t t, int Lcap)
{
    if (t <= 0 || t >= ((int64_t)1 << (Lcap - 1)))
        return 0;
    return 1 + __popcll((unsigned long long)(t - 1));
}

// The (sequence, head) this workgroup serves.  The work of a step grows with
// the slots a sequence reads (1 to Lcap), and the workgroups of one launch
// are spread over the CUs in rounds of 256, workgroup b landing beside
// b + 256, b + 512, ...  The sequences are ranked by slot count (heaviest
// first, ties by index) and dealt out in a snake over the rounds (round r
// runs backwards when r is odd), so that each CU gets heavy and light
// sequences alike.  All threads of the workgroup must call this; it returns
// the same value to each.
__device__ int decode_item(const int64_t *__restrict__ pos, int S, int H, int Lcap, int *hist, int *sel)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nwv = blockDim.x >> 6;
    const int b = blockIdx.x, SH = S * H;
    const int r = b >> 8, c = b & 255;
    const int rho = ((r & 1) && r * 256 + 255 < SH) ? r * 256 + 255 - c : b;
    const int target = rho / H;   // rank of the sequence wanted
    if (tid == 0)
        *sel = target;   // replaced below; the ranks are a permutation of the sequences
    // histogram of slot counts: lane l of each wave counts count l
    int cnt = 0;
    for (int g = wv; g * 64 < S; g += nwv) {
        const int sq = g * 64 + lane;
        const int o = sq < S ? decode_occ(pos[sq], Lcap) : -1;
        for (int k = 0; k <= Lcap; ++k) {
            const unsigned long long m = __ballot(o == k);
            if (lane == k)
                cnt += __popcll(m);
        }
    }
    if (lane <= Lcap)
        hist[wv * 33 + lane] = cnt;
    __syncthreads();
    if (tid < 64) {
        // bucket of the target rank (heaviest bucket first), then the index
        // of the sequence within it
        int start = 0, cstar = 0, jrem = 0;
        for (int k = Lcap; k >= 0; --k) {
            int n = 0;
            for (int w = 0; w < nwv; ++w)
                n += hist[w * 33 + k];
            if (target < start + n) {
                cstar = k;
                jrem = target - start;
                break;
            }
            start += n;
        }
        for (int g = 0; g * 64 < S; ++g) {
            const int sq = g * 64 + lane;
            const int o = sq < S ? decode_occ(pos[sq], Lcap) : -1;
            unsigned long long m = __ballot(o == cstar);
            const int n = __popcll(m);
            if (jrem < n) {
                for (int q = 0; q < jrem; ++q)
                    m &= m - 1;
                if (lane == 0)
                    *sel = g * 64 + __ffsll((long long)m) - 1;
                break;
            }
            jrem -= n;
        }
    }
    __syncthreads();
    return *sel * H + rho % H;
}

template <class D>
__global__ __launch_bounds__(256) void ll_decode(const typename D::T *__restrict__ q,
                                                 const typename D::T *__restrict__ k,
                                                 const typename D::T *__restrict__ v,
                                                 const float *__restrict__ a, const float *__restrict__ lam,
                                                 float *__restrict__ state, float *__restrict__ logscale,
                                                 const int64_t *__restrict__ pos, typename D::T *__restrict__ out,
                                                 int H, int Lcap, int rqk)
{
    using T = typename D::T;
    constexpr int DK = D::DK, DV = D::DV;
    __shared__ float qs[DK], ks[DK], vs[DV];
    __shared__ float lam_s[kMaxLevels], g_s[kMaxLevels];
    __shared__ float red[D::NT][4];
    __shared__ int slots[kMaxLevels];
    __shared__ int nslots;
    __shared__ float qk_s;
    __shared__ int hist[4 * 33];
    __shared__ int sel;

    const int tid = threadIdx.x;
    const int sh = decode_item(pos, gridDim.x / H, H, Lcap, hist, &sel);   // sequence * H + head
    const int s = sh / H;
    const int64_t t = pos[s];
    T *o = out + (size_t)sh * DV;

    if (t < 0 || t >= ((int64_t)1 << (Lcap - 1))) {
        // Not representable with Lcap slots: NaN output, stack untouched.
        for (int e = tid; e < DV; e += D::NT)
            o[e] = from_f32<T>(__builtin_nanf(""));
        return;
    }

    const size_t qkrow = (size_t)(sh / rqk) * DK;   // q and k are shared by rqk heads
    for (int d = tid; d < DK; d += D::NT) {
        qs[d] = to_f32(q[qkrow + d]);
        ks[d] = to_f32(k[qkrow + d]);
    }
    for (int e = tid; e < DV; e += D::NT)
        vs[e] = to_f32(v[(size_t)sh * DV + e]);
    for (int l = tid; l < Lcap; l += D::NT) {
        lam_s[l] = lam[(size_t)sh * Lcap + l];
        g_s[l] = logscale[(size_t)sh * Lcap + l];
    }
    if (tid == 0) {
        // occupied slots of the previous position: 0, and l >= 1 for each set
        // bit l-1 of t-1 (none when the stack is empty, t == 0)
        int n = 0;
        if (t > 0) {
            const int64_t prev = t - 1;
            slots[n++] = 0;
            for (int l = 1; l < Lcap; ++l)
                if ((prev >> (l - 1)) & 1)
                    slots[n++] = l;
        }
        nslots = n;
    }
    __syncthreads();
    if (tid < 64) {
        float x = 0.f;
        for (int d = tid; d < DK; d += 64)
            x += qs[d] * ks[d];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
            x += __shfl_xor(x, m, 64);
        if (tid == 0)
            qk_s = x;
    }

    const float at = a[sh];
    float *st = state + (size_t)sh * Lcap * DK * DV;
    const int c0 = (tid * 4) % DV;  // this thread's four output columns
    const int kc = t > 0 ? __builtin_ctzll((unsigned long long)t) : -1;  // levels 0..kc merge into kc+1
    const int n = nslots;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    float4 M[D::NPT];
#pragma unroll
    for (int r = 0; r < D::NPT; ++r)
        M[r] = make_float4(0.f, 0.f, 0.f, 0.f);

    // Stream the occupied slots two at a time.
    for (int i = 0; i < n; i += 2) {
        const int l0 = slots[i];
        const int l1 = (i + 1 < n) ? slots[i + 1] : -1;
        float4 x0[D::NPT], x1[D::NPT];
        const float4 *s0 = reinterpret_cast<const float4 *>(st + (size_t)l0 * DK * DV);
#pragma unroll
        for (int r = 0; r < D::NPT; ++r) {
            const int idx = tid + D::NT * r;
            if (idx < D::NV4)
                x0[r] = nt_load(s0 + idx);
        }
        if (l1 >= 0) {
            const float4 *s1 = reinterpret_cast<const float4 *>(st + (size_t)l1 * DK * DV);
#pragma unroll
            for (int r = 0; r < D::NPT; ++r) {
                const int idx = tid + D::NT * r;
                if (idx < D::NV4)
                    x1[r] = nt_load(s1 + idx);
            }
        }
        decode_slot<D>(x0, M, part, l0 <= kc, l0 <= kc ? __expf(g_s[l0]) : lam_s[l0] * __expf(g_s[l0] + at), qs,
                       tid);
        if (l1 >= 0)
            decode_slot<D>(x1, M, part, l1 <= kc,
                           l1 <= kc ? __expf(g_s[l1]) : lam_s[l1] * __expf(g_s[l1] + at), qs, tid);
    }

    // Merged bucket (true state, stored with logscale 0) and the new token's
    // own state in slot 0.
    const float dec = __expf(at);
    float4 *dst0 = reinterpret_cast<float4 *>(st);
    float4 *dstM = reinterpret_cast<float4 *>(st + (size_t)(kc + 1) * DK * DV);
    const float lm = t > 0 ? lam_s[kc + 1] : 0.f;
#pragma unroll
    for (int r = 0; r < D::NPT; ++r) {
        const int idx = tid + D::NT * r;
        if (idx < D::NV4) {
            const int row = idx * 4 / DV;
            const float kr = ks[row];
            nt_store(dst0 + idx, make_float4(kr * vs[c0], kr * vs[c0 + 1], kr * vs[c0 + 2], kr * vs[c0 + 3]));
            if (t > 0) {
                const float4 m = make_float4(dec * M[r].x, dec * M[r].y, dec * M[r].z, dec * M[r].w);
                nt_store(dstM + idx, m);
                const float qc = lm * qs[row];
                part[0] += qc * m.x; part[1] += qc * m.y; part[2] += qc * m.z; part[3] += qc * m.w;
            }
        }
    }

    red[tid][0] = part[0];
    red[tid][1] = part[1];
    red[tid][2] = part[2];
    red[tid][3] = part[3];
    __syncthreads();
    if (tid < D::CG) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int x = tid; x < D::NT; x += D::CG) {
            acc[0] += red[x][0]; acc[1] += red[x][1]; acc[2] += red[x][2]; acc[3] += red[x][3];
        }
        const float d0 = lam_s[0] * qk_s;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            o[4 * tid + c] = from_f32<T>(acc[c] + d0 * vs[4 * tid + c]);
    }
    if (tid == 0) {
        float *gl = logscale + (size_t)sh * Lcap;
        gl[0] = 0.f;
        if (t > 0) {
            const int64_t prev = t - 1;
            for (int l = kc + 2; l < Lcap; ++l)
                if ((prev >> (l - 1)) & 1)
                    gl[l] = g_s[l] + at;
            gl[kc + 1] = 0.f;
        }
    }
}

typedef hipError_t (*DecLauncher)(const DecodeArgs &, hipStream_t);

template <class DT, int DK, int DV>
static hipError_t launch_dec_t(const DecodeArgs &A, hipStream_t s)
{
    using D = Dec<DT, DK, DV>;
    using T = typename D::T;
    const ProfEvents pe = prof_events("ll_decode");
    hipExtLaunchKernelGGL(ll_decode<D>, dim3(A.S * A.H), dim3(D::NT), 0, s, pe.start, pe.stop, 0, (const T *)A.q,
                          (const T *)A.k, (const T *)A.v, A.a, A.lam, A.state, A.logscale, A.pos, (T *)A.out, A.H,
                          A.Lcap, A.rqk);
    return hipGetLastError();
}

template <class DT, int DK>
static DecLauncher dec_pick_dv(int dv)
{
    switch (dv) {
    case 16: return &launch_dec_t<DT, DK, 16>;
    case 32: return &launch_dec_t<DT, DK, 32>;
    case 64: return &launch_dec_t<DT, DK, 64>;
    case 128: return &launch_dec_t<DT, DK, 128>;
    default: return nullptr;
    }
}

template <class DT>
static DecLauncher dec_pick(int dk, int dv)
{
    switch (dk) {
    case 16: return dec_pick_dv<DT, 16>(dv);
    case 32: return dec_pick_dv<DT, 32>(dv);
    case 64: return dec_pick_dv<DT, 64>(dv);
    case 128: return dec_pick_dv<DT, 128>(dv);
    default: return nullptr;
    }
}

static DecLauncher find_dec(bool bf16, int dk, int dv) { return bf16 ? dec_pick<TBF16>(dk, dv) : dec_pick<TF32>(dk, dv); }

bool decode_supported(bool bf16, int dk, int dv) { return find_dec(bf16, dk, dv) != nullptr; }

hipError_t decode_launch(const DecodeArgs &args, hipStream_t stream)
{
    DecLauncher f = find_dec(args.bf16, args.dk, args.dv);
    if (!f)
        return hipErrorInvalidValue;
    return f(args, stream);
}

}  // namespace ll
