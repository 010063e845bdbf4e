// One-launch forward of log-linear attention (Mamba-2 form), bf16 inputs,
// for gfx950.
//
// The pages' parallel form splits the sequence into blocks: dense work inside
// a block and hierarchical state passing between blocks ("Log-Linear
// Attention", Portuguese page §2 "Forma Recorrente e Paralela", training
// bullet; French page §2 "Algorithmes Efficaces"), and their kernel fuses the
// levels to save memory traffic and launches (French page §3 "Contributions
// Clés").  Here the whole forward is one launch (plus a tiny flag reset).
//
// Groups of TG = 128 consecutive tokens.  Inside a group every level
// (bit_length(t XOR s) <= 7) is evaluated densely:
//     O_in = (Q K^T ⊙ M) V,  M[t,s] = exp(A_t - A_s) lambda_t[level(t,s)], s <= t,
// on bf16 MFMA with float32 accumulation.  A key in an earlier group j' sits
// at level 8 + bit_length(j XOR j') - 1 from every query of group j, so the
// coarser levels form a Fenwick tree over group indices: group j reads, for
// every set bit k of j, the decayed state sum k v^T of the 2^k groups just
// below that bit.  That block is the Fenwick node of its last group
// e = ((j >> (k+1)) << (k+1)) + 2^k - 1, which covers the lowbit(e+1) groups
// ending at e:
//     N_j = S_j + sum over the trailing one bits k of j of
//           exp(decay from node e_k's end to group j's end) N_{e_k},
// with S_j = K_j^T diag(exp(decay to the group end)) V_j — the merge rule of
// the recurrent form (a new block absorbs the finer ones below it) applied
// at group granularity.
//
// The grid holds two kinds of work items, one workgroup each, in rounds of
// a few groups: state items (group j's state, merged with the nodes of j's
// trailing bits, published as node j) and output items (the in-group part
// and the levels above the group, read from the published nodes), the state
// items dispatched a round ahead of the output items.  The chains of nodes
// (N_j waits for N_{j-1}, N_{j-2}, N_{j-4}, ...) thus run among light items
// that do nothing else, ahead of the output items that read them.
//
// Nodes live in the workspace (bf16, in the MFMA fragment order their
// readers load, with their total log-decay in float32) and carry a ready
// flag.  Every wait is for an item with a smaller workgroup index, which the
// in-order dispatch of workgroups started earlier, so every wait ends (and
// each is bounded all the same).  Node data moves between workgroups with
// agent-coherent (sc1) stores and loads: a writer raises the flag only after
// its node stores are complete, and readers load only after seeing the flag,
// so no cache-wide write-back or invalidation is needed and the XCD a
// workgroup lands on does not matter for correctness.  The mapping of items
// to workgroups keeps a head's items on one XCD when the dispatch deals
// workgroups round-robin over the XCDs.  A small preparation kernel clears
// the flags first.
#include <hip/hip_ext.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {
namespace fz {

template <int DK_, int DV_>
struct Cfg {
    static constexpr int DK = DK_, DV = DV_;
    static constexpr int TG = 128;            // tokens per group (work item)
    static constexpr int LTG = 7;             // log2 TG
    static constexpr int NQT = TG / 16;       // 16-row query (and key) tiles
    static constexpr int NW = 4;              // waves; wave w owns query tiles w and 7 - w
    static constexpr int NT = 64 * NW;
    static constexpr int NUK = DK / 32;       // 32-wide dk units (one bf16 MFMA each)
    static constexpr int NCT = DV / 16;       // 16-wide dv tiles
    static constexpr int CPR = DK / 8;        // 16-byte chunks per K row
    static constexpr int VPR = DV / 8;        // 16-byte chunks per V row
    static constexpr int NIN = LTG + 1;       // lambda levels inside a group (0 .. 7)
    static constexpr int NODE = DK * DV;      // elements of a node
    static constexpr int LDD = TG + 16;       // row stride of the level-major lambda table
    static_assert(DK == 128 && DV == 64, "shape of this kernel");
    static_assert(CPR == 16 && VPR == 8, "the K and V swizzles assume these row lengths");
    static_assert(NUK == NW, "wave w forms dk unit w of the group state");
    static_assert(TG * DK >= 2 * NODE && TG * DV >= NODE, "node buffers fit the K and V regions");
    // Query tiles of wave w: {w, 7 - w} carry w/2 + 1 + (7-w)/2 + 1 = 5 causal key pairs.
    __device__ static constexpr int qtile(int w, int x) { return x == 0 ? w : NQT - 1 - w; }
};

template <class F>
struct alignas(16) Smem {
    __bf16 K[F::TG * F::DK];      // keys (swizzled rows); node staging in the level phase
    __bf16 V[F::TG * F::DV];      // values (swizzled rows); node staging in the level phase
    float Aloc[F::TG];            // inclusive prefix of a inside the group
    float gam;                    // group total log-decay
    int ready;
    float off[32];                // decay from node e_k's end to the group start, per bit k
    float lamd[5][F::LDD];        // lambda levels 0 .. 4 of every token, level-major
};

// Physical 16-byte chunk of logical chunk c in K row r: a bijection on the 16
// chunks per row that (a) sends rows 0..15 of one logical chunk to 16
// distinct chunks (fragment reads: 16 lanes, 16 rows) and (b) sends the two
// chunks of a transpose read of 8 consecutive rows to 16 distinct chunks.
__device__ __forceinline__ int kswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <class F>
__device__ __forceinline__ int koff(int r, int c)
{
    return r * F::DK + ((c ^ kswz(r)) << 3);
}

// V rows are 128 bytes, half of the 64 banks; rows of the same parity share
// a bank half.  A transpose read touches 8 consecutive rows, 32 bytes (a
// pair of chunks) each: XOR-ing the chunk pair index with (r/2) mod 4 puts
// the four rows of each parity on four different pairs, so the read is
// conflict-free.
__device__ __forceinline__ int vswz(int r) { return ((r >> 1) & 3) << 1; }

template <class F>
__device__ __forceinline__ int voff(int r, int col)
{
    return r * F::DV + ((((col >> 3) ^ vswz(r))) << 3) + (col & 7);
}

// Fragment whose k-index runs over tokens of the swizzled V tile (as tr_frag
// of a plain row-major tile): rows jb + unit_row(e, qd), column c0 + li.
template <class F>
__device__ __forceinline__ bf16x8 v_frag(const __bf16 *V, int jb, int c0, int li, int qd)
{
    const int r = jb + 4 * qd + (li >> 2);
    const int col = c0 + 4 * (li & 3);
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(V + voff<F>(r, col)));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(V + voff<F>(r + 16, col)));
    bf16x8 x;
    x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
    x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
    return x;
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of a coherent access: sc1, i.e. performed at agent scope (the
// level every XCD sees), not in one XCD's L2.
constexpr int kCoherent = 16;

// LDS-direct load: lane l writes 16 bytes read at byte `off` of the
// descriptor's range to LDS dst + 16 l (dst wave-uniform); bytes past the
// range read as zero.
template <int CPOL = 0>
__device__ __forceinline__ void ld_lds16(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, (int)off, 0, 0, CPOL);
}

typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));

// ---- node exchange between workgroups --------------------------------------
// Node data, node totals and flags move between workgroups with
// agent-coherent (sc1) stores and loads only, so the XCD a workgroup lands on
// never matters and no cache-wide write-back or invalidation is needed: a
// writer raises a node's flag after its node stores are complete, and
// readers load the node only after they saw the flag.
__device__ __forceinline__ bf16x8 ld_frag_c(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent));
}

__device__ __forceinline__ float ld_f32_c(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherent));
}

__device__ __forceinline__ void st_frag_c(__amdgpu_buffer_rsrc_t r, int byte_off, const bf16x8 &f)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f), r, byte_off, 0, kCoherent);
}

__device__ __forceinline__ void st_f32_c(__amdgpu_buffer_rsrc_t r, int byte_off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, byte_off, 0, kCoherent);
}

__device__ __forceinline__ bool flag_up(const int *f)
{
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Spin until a node's flag is up.  Bounded: after 2^20 polls the wait gives
// up and the failure is counted, so a broken dependency cannot hang the GPU.
__device__ __forceinline__ bool wait_flag(const int *f)
{
    for (int n = 0; n < (1 << 20); ++n) {
        if (flag_up(f))
            return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Items of one kind per round of the workgroup order (the groups of a round
// are this many over the heads, at least one), and the rounds by which the
// state items run ahead of the output items.
constexpr int kRoundItems = 64;
constexpr int kLag = 2;

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes of a fully active wave.
__device__ __forceinline__ float wave_scan(float x)
{
    x += dpp<0x111, 0xf>(x);
    x += dpp<0x112, 0xf>(x);
    x += dpp<0x114, 0xf>(x);
    x += dpp<0x118, 0xf>(x);
    x += dpp<0x142, 0xa>(x);
    x += dpp<0x143, 0xc>(x);
    return x;
}

// K^T fragment for the group state (A operand, rows = dk, k = tokens): token
// rows jb + unit_row(e, qd) of dk column 32u + 8*(li/4) + 4t + li%4, so that
// the accumulator tile pair (t = 0, 1) of unit u holds rows 32u + 8qd + e in
// natural order (the node fragment order).
template <class F>
__device__ __forceinline__ bf16x8 kt_frag(const __bf16 *K, int jb, int u, int t, int li, int qd)
{
    const int r = jb + 4 * qd + (li >> 2);
    const int c = 4 * u + (li & 3);
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(K + koff<F>(r, c) + 4 * t));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(K + koff<F>(r + 16, c) + 4 * t));
    bf16x8 x;
    x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
    x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
    return x;
}

// K fragment for S^T = K Q^T (A operand, rows = keys, k = dk natural order):
// row r, dk 32u + 8qd .. +7: one 16-byte read.
template <class F>
__device__ __forceinline__ bf16x8 k_frag(const __bf16 *K, int r, int u, int qd)
{
    return *reinterpret_cast<const bf16x8 *>(K + koff<F>(r, 4 * u + qd));
}

__device__ __forceinline__ bf16x8 pack_frag(const floatx4 &lo, const floatx4 &hi)
{
    bf16x8 f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f[r] = (__bf16)lo[r];
        f[r + 4] = (__bf16)hi[r];
    }
    return f;
}

// Level weights of one query row for the key tiles left of the diagonal
// (levels 5 .. 7), held in registers; the level of such a tile is known at
// compile time, so no indexing is involved.  The diagonal tile's levels
// 0 .. 4 vary per element and are read from LDS.
struct Lam3 {
    float l5, l6, l7;
    __device__ __forceinline__ float at(int l) const { return l == 5 ? l5 : l == 6 ? l6 : l7; }
};

struct Ws {
    __bf16 *node;     // [BH][nG][NODE] fragment order
    float *gamN;      // [BH][nG] total log-decay of each node
    int *flag;        // [BH][nG]
    int *fail;        // [1] waits that gave up (0 in a correct run)
};

// Node fragment (ct, u) of lane `lane`: 8 consecutive bf16 (element offset).
template <class F>
__device__ __forceinline__ int frag_off(int ct, int u, int lane)
{
    return ((ct * F::NUK + u) * 64 + lane) * 8;
}

// In-group part for query tile qt, whose keys are the NP key pairs (32 keys
// each) up to the diagonal: P^T = M ⊙ (K Q^T) per 16-key tile, then
// O^T += V^T P^T.  A key tile left of the diagonal sits in one bucket of
// every query of the tile (level 4 + bit_length(kt XOR qt)); the diagonal
// tile takes the level per element.  NP is a template parameter, so the loop
// is fully unrolled and the products of different pairs overlap.
template <class F, int NP>
__device__ __forceinline__ void in_group(floatx4 (&O)[F::NCT], const bf16x8 (&qf)[F::NUK], const Lam3 &lam,
                                         const Smem<F> &sm, int qt, int li, int qd)
{
    const int tl = 16 * qt + li;   // query token in the group
    const float At = sm.Aloc[tl];
    const bool odd = (qt & 1) != 0;
#pragma unroll
    for (int kp = 0; kp < NP; ++kp) {
        // keep one key pair's fragments live at a time
        __builtin_amdgcn_sched_barrier(0);
        const bool two = kp < NP - 1 || odd;
        floatx4 s[2] = {zero4(), zero4()};
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag<F>(sm.K, 32 * kp + li, u, qd), qf[u], s[0], 0, 0, 0);
        if (two) {
#pragma unroll
            for (int u = 0; u < F::NUK; ++u)
                s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_frag<F>(sm.K, 32 * kp + 16 + li, u, qd), qf[u],
                                                               s[1], 0, 0, 0);
        }
        bf16x8 p;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kt = 2 * kp + h;
            const floatx4 As = *reinterpret_cast<const floatx4 *>(&sm.Aloc[16 * kt + 4 * qd]);
            if (kt < qt) {
                // qt is 2 NP - 2 or 2 NP - 1, so for kt < qt the level is fixed at compile time
                const int lev = kt < 2 * NP - 2 ? 4 + bitlen_u32((uint32_t)(kt ^ (2 * NP - 2))) : 5;
                const float lm = lam.at(lev);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[4 * h + r] = (__bf16)(s[h][r] * __expf(At - As[r]) * lm);
            } else if (kt == qt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int sk = 16 * kt + 4 * qd + r;
                    float m = 0.f;
                    if (sk <= tl)
                        m = __expf(At - As[r]) * sm.lamd[sk == tl ? 0 : bitlen_u32((uint32_t)(sk ^ tl))][tl];
                    p[4 * h + r] = (__bf16)(s[h][r] * m);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[4 * h + r] = (__bf16)0.f;
            }
        }
#pragma unroll
        for (int c = 0; c < F::NCT; ++c)
            O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_frag<F>(sm.V, 32 * kp, 16 * c, li, qd), p, O[c], 0,
                                                           0, 0);
    }
}

template <class F>
__device__ __forceinline__ void in_group_tile(floatx4 (&O)[F::NCT], const bf16x8 (&qf)[F::NUK], const Lam3 &lam,
                                              const Smem<F> &sm, int qt, int li, int qd)
{
    switch (qt >> 1) {
    case 0: in_group<F, 1>(O, qf, lam, sm, qt, li, qd); break;
    case 1: in_group<F, 2>(O, qf, lam, sm, qt, li, qd); break;
    case 2: in_group<F, 3>(O, qf, lam, sm, qt, li, qd); break;
    default: in_group<F, 4>(O, qf, lam, sm, qt, li, qd); break;
    }
}

template <class F>
__global__ __launch_bounds__(F::NT) __attribute__((amdgpu_waves_per_eu(3, 3))) void ll_fused_fwd(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ a, const float *__restrict__ lam, __bf16 *__restrict__ out, int BH, int Tlen, int L,
    int nG, int rqk, int kRound, Ws ws)
{
    __shared__ Smem<F> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, qd = lane >> 4, li = lane & 15;

    // ---- work item of this workgroup ----
    // Workgroups are dispatched in the order of their index, and every item
    // waits only for items with smaller workgroup indices (below): those were
    // dispatched first, so every wait ends.
    // Workgroups come in rounds of kRound groups (all heads; about
    // kRoundItems items of each kind), the state
    // items running kLag rounds ahead of the output items:
    //     S_0 .. S_{kLag-1}, then S_{m+kLag}, O_m for m = 0, 1, ..., then the
    //     last output rounds.
    // A state item publishes its group's Fenwick node (the chains of nodes
    // run among these light items); an output item does the in-group part
    // and reads the nodes of earlier groups of its head, published rounds
    // before.  Every wait is thus for a smaller workgroup index.
    // Within a round, with a multiple of 8 heads, item i = 8r + x (it runs
    // on XCD x when workgroups are dealt round-robin over the 8 XCDs) is head
    // x + 8 (r mod nh), group r / nh of the round: all items of a head share
    // one XCD and its L2.  Otherwise the order is group-major.
    bool state_item;
    int bh, j;
    {
        int b = blockIdx.x, m, i;
        const int rs = BH * kRound;                          // items of one kind in a full round
        const int M = (nG + kRound - 1) / kRound;            // rounds
        const int cl = BH * (nG - (M - 1) * kRound);         // items of one kind in the last round
        // the leading state rounds (the last of them may be the short one)
        const int nA = min(kLag, M);
        const int lenA = (nA - 1) * rs + (kLag >= M ? cl : rs);
        const int P = max(M - kLag, 0);                      // pairs (S_{m+kLag}, O_m)
        const int lenB = P > 0 ? (P - 1) * 2 * rs + cl + rs : 0;
        if (b < lenA) {
            state_item = true;
            m = b / rs;
            i = b - m * rs;
        } else if ((b -= lenA) < lenB) {
            const int p = b / (2 * rs);
            const int ssz = p == P - 1 ? cl : rs;            // only the last pair holds the short state round
            i = b - p * 2 * rs;
            state_item = i < ssz;
            m = state_item ? p + kLag : p;
            if (!state_item)
                i -= ssz;
        } else {
            b -= lenB;
            state_item = false;
            m = P + b / rs;
            i = b - (m - P) * rs;
        }
        const int g0 = m * kRound;
        if ((BH & 7) == 0) {
            const int nh = BH >> 3, x = i & 7, r = i >> 3;
            bh = x + 8 * (r % nh);
            j = g0 + r / nh;
        } else {
            bh = i % BH;
            j = g0 + i / BH;
        }
    }
    const int t0 = j * F::TG;
    const int qbh = bh / rqk;
    const size_t hrow = (size_t)bh * Tlen, qrow = (size_t)qbh * Tlen;

    // ---- stage K and V of the group (swizzled); Q, lambda and a to
    //      registers.  Every load is issued before the one wait below, so
    //      the phase costs a single memory round trip. ----
    // decay of tokens lane and 64 + lane (wave 0 scans them)
    float a0 = 0.f, a1 = 0.f;
    if (w == 0) {
        if (t0 + lane < Tlen)
            a0 = a[hrow + t0 + lane];
        if (t0 + 64 + lane < Tlen)
            a1 = a[hrow + t0 + 64 + lane];
    }
    {
        const __amdgpu_buffer_rsrc_t rk = rsrc(k + (qrow + t0) * F::DK, (uint32_t)(Tlen - t0) * F::DK * 2);
        const __amdgpu_buffer_rsrc_t rv = rsrc(v + (hrow + t0) * F::DV, (uint32_t)(Tlen - t0) * F::DV * 2);
        constexpr int KBLK = F::TG * F::CPR / 64;   // 1 KB blocks of 64 lanes
        static_assert(KBLK % F::NW == 0, "even K staging");
#pragma unroll
        for (int x = 0; x < KBLK / F::NW; ++x) {
            const int b = w + x * F::NW;
            const int pc = b * 64 + lane;
            const int r = pc / F::CPR, c = (pc % F::CPR) ^ kswz(r);
            ld_lds16(rk, sm.K + b * 512, ((uint32_t)r * F::DK + (uint32_t)c * 8) * 2);
        }
        constexpr int VBLK = F::TG * F::VPR / 64;
        static_assert(VBLK % F::NW == 0, "even V staging");
#pragma unroll
        for (int x = 0; x < VBLK / F::NW; ++x) {
            const int b = w + x * F::NW;
            const int pc = b * 64 + lane;
            const int r = pc / F::VPR, c = (pc % F::VPR) ^ vswz(r);
            ld_lds16(rv, sm.V + b * 512, ((uint32_t)r * F::DV + (uint32_t)c * 8) * 2);
        }
    }
    bf16x8 qf[2][F::NUK];
    Lam3 lamr[2];
    if (!state_item) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int tq = t0 + 16 * F::qtile(w, x) + li;
        const int tc = tq < Tlen ? tq : Tlen - 1;
        const __bf16 *qp = q + (qrow + tc) * F::DK + 8 * qd;
#pragma unroll
        for (int u = 0; u < F::NUK; ++u)
            qf[x][u] = *reinterpret_cast<const bf16x8 *>(qp + 32 * u);
        const float *lp = lam + (hrow + tc) * L;
        lamr[x] = Lam3{lp[5], lp[6], lp[7]};
    }
    }
    // lambda levels 0 .. 4 of the group's tokens (0 past the end): entry
    // i = tid + NT x is token i / 5, level i mod 5
    // (entries past the table repeat its last one: loads and stores stay
    // unconditional, so no load is sunk below the wait)
    constexpr int NLD = (5 * F::TG + F::NT - 1) / F::NT;
    float lv[NLD];
    if (!state_item) {
#pragma unroll
        for (int x = 0; x < NLD; ++x) {
            const int i = min(tid + x * F::NT, 5 * F::TG - 1), r = i / 5;
            lv[x] = lam[(hrow + min(t0 + r, Tlen - 1)) * L + (i - 5 * r)];
        }
    }
    wait_vm0();
    if (!state_item) {
#pragma unroll
        for (int x = 0; x < NLD; ++x) {
            const int i = min(tid + x * F::NT, 5 * F::TG - 1), r = i / 5;
            sm.lamd[i - 5 * r][r] = t0 + r < Tlen ? lv[x] : 0.f;
        }
    }
    // decay prefix of the group (wave 0)
    if (w == 0) {
        const float x0 = wave_scan(a0);
        const float tot0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x0), 63));
        const float x1 = wave_scan(a1) + tot0;
        sm.Aloc[lane] = x0;
        sm.Aloc[64 + lane] = x1;
        if (lane == 63)
            sm.gam = x1;
    }
    __syncthreads();
    const float gam = sm.gam;

    // ---- group state S_j = K^T diag(exp(gam - Aloc)) V: wave w forms dk
    //      unit w for every dv tile (tile pair t = 0, 1 per dv tile) ----
    const int su = w;
    floatx4 S[F::NCT][2];
    auto group_state = [&]() {
#pragma unroll
        for (int c = 0; c < F::NCT; ++c)
            S[c][0] = S[c][1] = zero4();
#pragma unroll
        for (int ju = 0; ju < F::TG / 32; ++ju) {
            const floatx4 A0 = *reinterpret_cast<const floatx4 *>(&sm.Aloc[32 * ju + 4 * qd]);
            const floatx4 A1 = *reinterpret_cast<const floatx4 *>(&sm.Aloc[32 * ju + 16 + 4 * qd]);
            float w0[4], w1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w0[e] = __expf(gam - A0[e]);
                w1[e] = __expf(gam - A1[e]);
            }
            bf16x8 kf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 f = kt_frag<F>(sm.K, 32 * ju, su, t, li, qd);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = (__bf16)((float)f[e] * w0[e]);
                    f[e + 4] = (__bf16)((float)f[e + 4] * w1[e]);
                }
                kf[t] = f;
            }
#pragma unroll
            for (int c = 0; c < F::NCT; ++c) {
                const bf16x8 vf = v_frag<F>(sm.V, 32 * ju, 16 * c, li, qd);
                S[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0], vf, S[c][0], 0, 0, 0);
                S[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1], vf, S[c][1], 0, 0, 0);
            }
        }
    };

    // ---- Fenwick bookkeeping ----
    const int tz = __builtin_ctz(~(unsigned)j);          // trailing one bits: nodes merged into N_j
    const int npop = __builtin_popcount((unsigned)j);    // set bits: nodes the levels read
    const size_t nbase = (size_t)bh * nG;
    const __amdgpu_buffer_rsrc_t rmine = rsrc(ws.node + (nbase + j) * F::NODE, (uint32_t)F::NODE * 2);

    // ---- state item: publish node j, N_j = S_j + sum_k exp(decay) N_{e_k}
    //      over the trailing one bits k of j (e_k = j - 2^k) ----
    if (state_item) {
        group_state();
        if (w == 0) {
            const bool okw = lane >= tz || wait_flag(&ws.flag[nbase + j - (1 << lane)]);
            if (__ballot(!okw) != 0 && lane == 0)
                atomicAdd(ws.fail, 1);
        }
        __syncthreads();
        float dec = gam, node_gam = gam;   // decay from node e_k's end to group j's end
        for (int kb = 0; kb < tz; ++kb) {
            const int e = j - (1 << kb);
            const __amdgpu_buffer_rsrc_t rn = rsrc(ws.node + (nbase + e) * F::NODE, (uint32_t)F::NODE * 2);
            bf16x8 f[F::NCT];
#pragma unroll
            for (int c = 0; c < F::NCT; ++c)
                f[c] = ld_frag_c(rn, frag_off<F>(c, su, lane) * 2);
            const float ge = __hip_atomic_load(&ws.gamN[nbase + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float sc = __expf(dec);
#pragma unroll
            for (int c = 0; c < F::NCT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    S[c][0][r] += sc * (float)f[c][r];
                    S[c][1][r] += sc * (float)f[c][r + 4];
                }
            dec += ge;
            node_gam += ge;
        }
#pragma unroll
        for (int c = 0; c < F::NCT; ++c)
            st_frag_c(rmine, frag_off<F>(c, su, lane) * 2, pack_frag(S[c][0], S[c][1]));
        if (tid == 0)
            __hip_atomic_store(&ws.gamN[nbase + j], node_gam, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every node store is complete (agent-coherent) before the flag
        wait_vm0();
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(&ws.flag[nbase + j], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---- output item: in-group part, O^T = V^T (M ⊙ K Q^T)^T for both query tiles ----
    floatx4 O[2][F::NCT];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int c = 0; c < F::NCT; ++c)
            O[x][c] = zero4();
        in_group_tile<F>(O[x], qf[x], lamr[x], sm, F::qtile(w, x), li, qd);
    }

    // ---- levels above the group: one node per set bit of j ----
    if (npop > 0) {
        // Level weights of the first four set bits for both rows, loaded
        // before the waits so that their memory latency overlaps them.
        float lwp[2][4];
        {
            unsigned bits = (unsigned)j;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int kb = bits ? __builtin_ctz(bits) : 0;
                bits &= bits - 1;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int tq = t0 + 16 * F::qtile(w, x) + li;
                    lwp[x][n] = lam[(hrow + (tq < Tlen ? tq : Tlen - 1)) * L + min(F::LTG + 1 + kb, L - 1)];
                }
            }
        }
        // Wave 0 waits for every node at once (lane kb for bit kb) and forms
        // the decay from each node's end to the group start: the totals of
        // the finer nodes between, an exclusive prefix over the set bits.
        if (w == 0) {
            const bool mine = lane < 31 && ((j >> lane) & 1);
            const int e = mine ? ((j >> (lane + 1)) << (lane + 1)) + (1 << lane) - 1 : 0;
            const bool okw = !mine || wait_flag(&ws.flag[nbase + e]);
            if (__ballot(!okw) != 0 && lane == 0)
                atomicAdd(ws.fail, 1);
            const float ge =
                mine ? __hip_atomic_load(&ws.gamN[nbase + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
            const float incl = wave_scan(ge);
            if (lane < 32)
                sm.off[lane] = incl - ge;
        }
        __syncthreads();   // also: every wave is done with K and V
        float At[2];
        const float *lrow[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int tl = 16 * F::qtile(w, x) + li;
            At[x] = sm.Aloc[tl];
            const int tq = t0 + tl;
            lrow[x] = lam + (hrow + (tq < Tlen ? tq : Tlen - 1)) * L;
        }
        // node buffers: the two halves of the key region and the value region
        auto slot_ptr = [&](int slot) -> __bf16 * { return slot == 0 ? sm.K : slot == 1 ? sm.K + F::NODE : sm.V; };
        constexpr int NBLK = F::NODE * 2 / 1024;
        static_assert(NBLK % F::NW == 0, "each wave stages the same number of blocks");
        constexpr int PER = NBLK / F::NW;   // staging loads per wave and node
        auto stage = [&](int kb, __bf16 *dst) {
            const int e = ((j >> (kb + 1)) << (kb + 1)) + (1 << kb) - 1;
            const __amdgpu_buffer_rsrc_t rn = rsrc(ws.node + (nbase + e) * F::NODE, (uint32_t)F::NODE * 2);
#pragma unroll
            for (int x = 0; x < PER; ++x) {
                const int bb = w + x * F::NW;
                ld_lds16<kCoherent>(rn, dst + bb * 512, (uint32_t)(bb * 64 + lane) * 16);
            }
        };
        // set bits of j, low to high; up to three nodes in flight
        unsigned rest = (unsigned)j;
        int kbs[3];
        int issued = 0;
        for (; issued < 3 && rest; ++issued) {
            kbs[issued] = __builtin_ctz(rest);
            rest &= rest - 1;
            stage(kbs[issued], slot_ptr(issued));
        }
        for (int n = 0; n < npop; ++n) {
            const int slot = n % 3;
            const int kb = slot == 0 ? kbs[0] : slot == 1 ? kbs[1] : kbs[2];
            // the level weights of this node (preloaded for the first four)
            float lw0, lw1;
            if (n < 4) {
                lw0 = n == 0 ? lwp[0][0] : n == 1 ? lwp[0][1] : n == 2 ? lwp[0][2] : lwp[0][3];
                lw1 = n == 0 ? lwp[1][0] : n == 1 ? lwp[1][1] : n == 2 ? lwp[1][2] : lwp[1][3];
            } else {
                lw0 = lrow[0][F::LTG + 1 + kb];
                lw1 = lrow[1][F::LTG + 1 + kb];
            }
            const int ahead = issued - n - 1;   // stages issued after node n's
            if (ahead >= 2)
                wait_vm<2 * PER>();
            else if (ahead == 1)
                wait_vm<PER>();
            else
                wait_vm<0>();
            __syncthreads();   // node n is in LDS
            const __bf16 *nd = slot_ptr(slot);
            const float f0 = lw0 * __expf(At[0] + sm.off[kb]);
            const float f1 = lw1 * __expf(At[1] + sm.off[kb]);
            // one dv tile at a time: its four fragments serve both query tiles
#pragma unroll
            for (int c = 0; c < F::NCT; ++c) {
                floatx4 y0 = zero4(), y1 = zero4();
#pragma unroll
                for (int u = 0; u < F::NUK; ++u) {
                    const bf16x8 nf = *reinterpret_cast<const bf16x8 *>(nd + frag_off<F>(c, u, lane));
                    y0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nf, qf[0][u], y0, 0, 0, 0);
                    y1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nf, qf[1][u], y1, 0, 0, 0);
                }
                O[0][c] += f0 * y0;
                O[1][c] += f1 * y1;
            }
            if (rest) {
                __syncthreads();   // every wave is done with this slot
                const int kn = __builtin_ctz(rest);
                rest &= rest - 1;
                if (slot == 0)
                    kbs[0] = kn;
                else if (slot == 1)
                    kbs[1] = kn;
                else
                    kbs[2] = kn;
                stage(kn, slot_ptr(slot));
                ++issued;
            }
        }
    }

    // ---- output rows ----
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int tq = t0 + 16 * F::qtile(w, x) + li;
        if (tq < Tlen) {
            __bf16 *op = out + (hrow + tq) * F::DV + 4 * qd;
#pragma unroll
            for (int c = 0; c < F::NCT; ++c) {
                bf16x4 o4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o4[r] = (__bf16)O[x][c][r];
                *reinterpret_cast<bf16x4 *>(op + 16 * c) = o4;
            }
        }
    }
}

// Clears the ready flags and the wait-failure counter.
__global__ void ll_fused_prep(int *flag, int n, int *fail)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        flag[i] = 0;
    if (i == 0)
        *fail = 0;
}

}  // namespace fz

size_t fused_workspace_bytes(int B, int H, int T, int dk, int dv)
{
    const size_t BH = (size_t)B * H;
    const size_t nG = ((size_t)T + 127) / 128;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al(BH * nG * dk * dv * 2) + al(BH * nG * 4) + al(BH * nG * 4) + 256;
}

bool fused_supported(bool bf16, int dk, int dv, int T, int L)
{
    // One group (T <= 128) has no level above it: the chunk walk serves it
    // without a workspace.
    return bf16 && dk == 128 && dv == 64 && T > fz::Cfg<128, 64>::TG && L <= kMaxLevels &&
           (int64_t)T * 128 * 2 < ((int64_t)1 << 31) && (int64_t)T * L * 4 < ((int64_t)1 << 31);
}

FusedNodes fused_nodes(const FwdArgs &A)
{
    using F = fz::Cfg<128, 64>;
    const size_t BH = (size_t)A.B * A.H;
    const int nG = (A.T + F::TG - 1) / F::TG;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const char *p = static_cast<const char *>(A.workspace);
    return FusedNodes{p, reinterpret_cast<const float *>(p + al(BH * nG * F::NODE * 2)), nG, F::LTG};
}

hipError_t fused_launch(const FwdArgs &A, hipStream_t s)
{
    using F = fz::Cfg<128, 64>;
    const int BH = A.B * A.H;
    const int nG = (A.T + F::TG - 1) / F::TG;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *p = static_cast<char *>(A.workspace);
    fz::Ws ws;
    ws.node = reinterpret_cast<__bf16 *>(p);
    p += al((size_t)BH * nG * F::NODE * 2);
    ws.gamN = reinterpret_cast<float *>(p);
    p += al((size_t)BH * nG * 4);
    ws.flag = reinterpret_cast<int *>(p);
    p += al((size_t)BH * nG * 4);
    ws.fail = reinterpret_cast<int *>(p);
    const int nflag = BH * nG;
    ProfEvents pe = prof_events("ll_fused_prep");
    hipExtLaunchKernelGGL(fz::ll_fused_prep, dim3((nflag + 255) / 256), dim3(256), 0, s, pe.start, pe.stop, 0,
                          ws.flag, nflag, ws.fail);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    pe = prof_events("ll_fused_fwd");
    hipExtLaunchKernelGGL(fz::ll_fused_fwd<F>, dim3(2 * BH * nG), dim3(F::NT), 0, s, pe.start, pe.stop, 0,
                          (const __bf16 *)A.q, (const __bf16 *)A.k, (const __bf16 *)A.v, A.a, A.lam,
                          (__bf16 *)A.out, BH, A.T, A.L, nG, A.rqk, std::max(1, fz::kRoundItems / BH), ws);
    return hipGetLastError();
}

}  // namespace ll
