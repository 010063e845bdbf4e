// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ll {

constexpr int kMaxLevels = 32;     // lambda entries per token the kernels stage (T < 2^31)
constexpr int kMaxGroupLog2 = 3;   // local Fenwick stack depth of the chunk walk (<= 8 chunks)

// How the chunked forward splits a sequence.
//  N chunks of C tokens; groups of G = 2^g consecutive chunks, nG groups.
//  Levels whose buckets stay inside a group are carried in registers by the
//  chunk walk; coarser ones come from left-child block states built over the
//  nL = nG - 1 complete groups that can precede another group.
struct FwdPlan {
    int N = 0, g = 0, G = 1, nG = 0, nL = 0, Plev = 0, nLeft = 0;
    size_t off_Sg = 0, off_Gam = 0, off_Dg = 0, off_tot = 0, off_gtot = 0, bytes = 0;
};

// group_log2 < 0 picks automatically.  elem_bytes is the size used for the
// stored block states (4 covers both dtypes).
FwdPlan fwd_plan(int B, int H, int T, int dk, int dv, int chunk, int group_log2, int elem_bytes);

struct FwdArgs {
    const void *q, *k, *v;
    const float *a, *lam;
    void *out;
    int B, H, T, dk, dv, chunk, L;
    bool bf16;
    void *workspace;
    // Only the group states and the tree over groups (no chunk walk, q,
    // lambda and out unused), with the block states in the natural dk order
    // when tree_nat is set (bf16 only).
    bool tree_only = false;
    bool tree_nat = false;
    // With tree_nat (bf16): the block states in the backward's fragment
    // order instead: fragment (dk tile dt, dv unit u) of 64 lanes x 8
    // elements, lane li + 16 qd holding dv rows 32u + 16(k/4) + 4qd + k%4
    // (k = 0..7) of dk column 16 dt + li.  Required with tree_nodes.
    bool tree_yfrag = false;
    // With tree_only, bf16 and groups of at most 8 chunks: also the Fenwick
    // nodes inside each group (the node of chunk e covers the 2^z chunks
    // ending at e, z its trailing one bits; bf16 [B*H][N][dk*dv] in the
    // backward's fragment order) and every chunk's total log-decay
    // ([B*H][N] float32); every group, the last one included, is walked.
    void *tree_nodes = nullptr;
    float *tree_gamc = nullptr;
    // Heads that share one q/k head: q and k are [B, H / rqk, T, dk] and
    // head h reads q/k head h / rqk.
    int rqk = 1;
};

// Profiling hook (implemented by the ABI layer): while profiling is on, a
// pair of events that the next launch records as part of its own dispatch
// (hipExtLaunchKernelGGL), so they time the kernel and nothing else; null
// events otherwise.
struct ProfEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events(const char *name);

bool fwd_supported(bool bf16, int dk, int dv, int chunk);
// nat_blocks (optional) receives the dk order of the stored block states:
// true for the natural order inside each 16-byte fragment lane (lane quad qd
// of unit u holds dk KB*u + 8*qd + e), false for unit_row's.
hipError_t fwd_launch(const FwdArgs &args, const FwdPlan &plan, hipStream_t stream, bool *nat_blocks = nullptr);

// One-launch forward (bf16, dk = 128, dv = 64): groups of 128 tokens, the
// levels above a group from Fenwick nodes that the work items publish to each
// other through the workspace.  Used for the plain forward with automatic
// group size; fused_workspace_bytes is its workspace (any dtype).
size_t fused_workspace_bytes(int B, int H, int T, int dk, int dv);
bool fused_supported(bool bf16, int dk, int dv, int T, int L);
hipError_t fused_launch(const FwdArgs &args, hipStream_t stream);
// After fused_launch: the Fenwick nodes (bf16, fragment order, dk natural
// inside a fragment lane, each decayed to its last group's end) and their
// log-decay totals, [BH][nG] each, in the launch's workspace.
struct FusedNodes {
    const void *node;
    const float *gamN;
    int nG, lg;   // groups, log2 of the group length in tokens
};
FusedNodes fused_nodes(const FwdArgs &args);

struct DecodeArgs {
    const void *q, *k, *v;
    const float *a, *lam;
    float *state, *logscale;
    const int64_t *pos;
    void *out;
    int S, H, dk, dv, Lcap;
    bool bf16;
    int rqk = 1;   // heads per q/k head: q, k are [S, H / rqk, dk]
};

bool decode_supported(bool bf16, int dk, int dv);
hipError_t decode_launch(const DecodeArgs &args, hipStream_t stream);

// Decode stack of the prompt's last position, written after the forward
// from its left-child block states (Dg, Gam: NULL when the prompt is one
// group) and the keys of the last group.  lgc = log2 of the group length in
// tokens; nat = the block states' dk order (see fwd_launch).
struct StackArgs {
    const void *k, *v;
    const float *a;
    const void *Dg;        // left-child block states (fragment order, input dtype)
    const float *Gam;      // per-group log-decay totals
    float *state, *logscale;
    int BH, T, dk, dv, lgc, nG, nL, nLeft, Lcap;
    bool bf16, nat;
    int rqk = 1;   // heads per k head: k is [BH / rqk, T, dk]
    // Per-sequence prompt lengths [BH / H] on the device (NULL: all T).
    const int *lens = nullptr;
    int H = 1;
    // Dg and Gam are the one-launch forward's Fenwick nodes and node totals
    // (a bucket of whole groups is the node of its last group; lgc = log2 of
    // the group length, nG groups; nL, nLeft unused; nat must be true).
    bool fused = false;
};

bool stack_supported(bool bf16, int dk, int dv);

// Backward.  Gradients gq, gk, gv in the input dtype; ga [BH, T] and
// glam [BH, T, L] fp32.
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *a, *lam;
    void *gq, *gk, *gv;
    float *ga, *glam;
    int B, H, T, dk, dv, chunk, L;
    bool bf16;
    void *workspace;
    int rqk = 1;   // heads per q/k head: q, k, gq, gk are [B, H / rqk, T, dk]
};

// Workspace of the backward: the tree over chunks (one chunk per group) of
// k, v; the forward that forms dq; the W pieces and sums; the in-chunk part
// of da and the per-level pair masses of every chunk.
struct BwdPlan {
    // tree: one chunk per group (float32 inputs); tree8: groups of up to 8
    // chunks with the Fenwick nodes inside each group (bf16 inputs), its
    // nodes and chunk totals at off_nd and off_gamc inside the tree region
    FwdPlan tree, tree8, fq;
    int NP = 0, NB = 0, g8 = 0;
    size_t off_nd = 0, off_gamc = 0;
    size_t off_tree = 0, off_fq = 0, off_wp = 0, off_w1 = 0, off_w2 = 0, off_pq = 0, off_mq = 0, off_mk = 0, off_gp = 0, bytes = 0;
    // shared q/k (rqk > 1): per-head copies of q, k and per-head dq, dk
    size_t off_qx = 0, off_kx = 0, off_gqx = 0, off_gkx = 0;
};

BwdPlan bwd_plan(int B, int H, int T, int dk, int dv, int chunk, int rqk = 1);
bool bwd_supported(bool bf16, int dk, int dv, int chunk);
hipError_t bwd_launch(const BwdArgs &args, const BwdPlan &plan, hipStream_t stream);
hipError_t stack_launch(const StackArgs &args, hipStream_t stream);

// Log-Linear Gated DeltaNet forward (float32 arithmetic; q, k, v, out in
// float32 or bf16): q, k [BH, T, dk], v and out [BH, T, dv], a and beta
// [BH, T], lam [BH, T, L].
struct GdnArgs {
    const void *q, *k, *v;       // input dtype
    const float *a, *beta, *lam;
    void *out;                   // input dtype
    int B, H, T, dk, dv, chunk, L;
    void *workspace;
    bool bf16 = false;
};

// Workspace: carried queries [BH][N*C][dk], then the tree over chunks
// (levels 0..P, level p holding N >> p blocks) of transposed transitions
// [dk][dk] and transposed states [dk][dv].
struct GdnPlan {
    int N = 0, P = 0, NBT = 0;
    size_t off_qt = 0, off_phi = 0, off_d = 0, off_oi = 0, bytes = 0;
};

GdnPlan gdn_plan(int B, int H, int T, int dk, int dv, int chunk);
bool gdn_supported(int dk, int dv, int chunk);
hipError_t gdn_launch(const GdnArgs &args, const GdnPlan &plan, hipStream_t stream);

}  // namespace ll
