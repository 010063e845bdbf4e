/*
 * loglinear.h — C ABI of the MI355X (gfx950) log-linear attention library.
 *
 * The operation.  Log-linear attention in its Mamba-2 form.  For every batch
 * b, head h and position t (0-indexed):
 *
 *   o[t,:] = sum_{s <= t} exp(sum_{r=s+1..t} a[r]) * lambda[t, level(t,s)]
 *                         * (q[t,:] . k[s,:]) * v[s,:]
 *   level(t,s) = 0 if s == t, else bit_length(t XOR s)
 *
 * This is O = (Q K^T ⊙ M_H) V with a hierarchical mask M_H ("Log-Linear
 * Attention" summary page, French, §2 "Matrice de Masque Hiérarchique";
 * Portuguese page §2 "Máscara Hierárquica"), whose levels are the Fenwick-tree
 * buckets of sizes 1, 2, 4, 8, ... of the prefix (Portuguese page §2
 * "Particionamento Hierárquico"), each level weighted by a per-token,
 * data-dependent lambda_t^(l) (French page §2), composed with Mamba-2's
 * decay exp(sum a) (both pages: Mamba-2 is one of the two instances built).
 * The forward is the chunkwise parallel form, O(T log T) (Portuguese page
 * §2 "Forma Recorrente e Paralela", training bullet); the decode step is the
 * recurrent form over O(log T) states (same section, decoding bullet; French
 * page §2 "Algorithmes Efficaces").
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), contiguous and row-major.  q, k, v, out and state must be
 *    16-byte aligned, the workspace 256-byte aligned, pos 8-byte aligned and
 *    the float32 vectors (a, lambda, logscale) 4-byte aligned.  Host pointers
 *    are an error the library cannot detect; the kernels would fault.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream); nothing is synchronised.  Results are visible after the caller
 *    synchronises that stream.  A kernel fault surfaces at that sync.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates or frees device memory in these calls and keeps no pointer
 *    after returning.  Inputs are never written.
 *  - Errors: validation happens on the host before any launch; a non-zero
 *    status is returned and a message is available from loglinear_last_error()
 *    (thread-local).  No call aborts, throws across the ABI or prints.
 *  - Zero-sized problems (B, H, T or S equal to 0) are valid and launch nothing.
 */
#ifndef LOGLINEAR_H
#define LOGLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LL_OK = 0,
    LL_EINVAL = -1,       /* null/misaligned pointer, negative size, bad dtype  */
    LL_EUNSUPPORTED = -2, /* valid request outside the compiled shape set       */
    LL_EDEVICE = -3,      /* a HIP launch or runtime call failed                */
    LL_EWORKSPACE = -4    /* workspace missing or smaller than required         */
} ll_status;

typedef enum {
    LL_F32 = 0, /* q, k, v, out are float32                                  */
    LL_BF16 = 1, /* q, k, v, out are bfloat16; accumulation is float32       */
    /* Not dtypes.  They widen the enum's range to every 32-bit int, so a
     * caller's out-of-range value is a valid ll_dtype in C++ too and reaches
     * the library's own check (LL_EINVAL) instead of being undefined. */
    LL_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    LL_DTYPE_RANGE_MAX_ = 0x7fffffff
} ll_dtype;

/* Number of lambda entries per token for a sequence of T tokens:
 * 1 + ceil(log2 T) (1 for T <= 1): level 0 plus one per possible bucket.
 * Returns -1 for T < 0. */
int loglinear_num_levels(int64_t T);

/* Bytes of device workspace loglinear_fwd needs for this shape (0 when no
 * workspace is needed).  Depends only on the arguments.  Returns 0 for
 * invalid or unsupported shapes (loglinear_fwd reports those). */
size_t loglinear_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/* Forward pass (chunkwise parallel form).
 *  q      [B,H,T,dk]  dtype
 *  k      [B,H,T,dk]  dtype
 *  v      [B,H,T,dv]  dtype
 *  a      [B,H,T]     float32, per-token log-decay (a[...,0] never enters;
 *                     values are expected <= 0 as in Mamba-2)
 *  lambda [B,H,T,L]   float32, L = loglinear_num_levels(T); entries for
 *                     levels that are empty for a row are ignored
 *  out    [B,H,T,dv]  dtype, written; must not alias any input
 *  chunk  tokens per chunk: 16, 32 or 64.  The result does not depend on it
 *         beyond rounding.  T need not be a multiple of chunk.
 *  workspace / workspace_bytes: caller-owned device scratch of at least
 *         loglinear_fwd_workspace_bytes(...) bytes (may be NULL when that is
 *         0).  Its contents on entry do not matter and are clobbered.
 * Supported: dtype F32 with dk, dv in {16, 32, 64, 128}; dtype BF16 with
 * dk in {32, 64, 128} and dv in {16, 32, 64, 128}; T < 2^31; B*H <= 65535.
 * Anything else (every other head size, e.g. 48, 96 or 256) returns
 * LL_EUNSUPPORTED: the kernels are compiled for these power-of-two tiles.
 * Errors: LL_EINVAL, LL_EUNSUPPORTED, LL_EWORKSPACE, LL_EDEVICE. */
ll_status loglinear_fwd(const void *q, const void *k, const void *v,
                        const float *a, const float *lambda, void *out,
                        int B, int H, int T, int dk, int dv, int chunk,
                        ll_dtype dtype, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Same as loglinear_fwd / loglinear_fwd_workspace_bytes with an explicit
 * group size: the chunk walk carries the levels inside groups of
 * 2^group_log2 consecutive chunks in registers and reads coarser levels from
 * the workspace.  group_log2 < 0 selects automatically (what the plain calls
 * do); values above 3 return LL_EUNSUPPORTED.  The result does not depend on
 * it beyond rounding; it exists for tuning and for tests.  The workspace
 * size must be queried with the same group_log2. */
size_t loglinear_fwd_workspace_bytes_ex(int B, int H, int T, int dk, int dv, int chunk, int group_log2);
ll_status loglinear_fwd_ex(const void *q, const void *k, const void *v,
                           const float *a, const float *lambda, void *out,
                           int B, int H, int T, int dk, int dv, int chunk,
                           ll_dtype dtype, void *workspace, size_t workspace_bytes,
                           void *stream, int group_log2);

/* Device scratch that loglinear_fwd_noalloc holds on every GPU it runs on. */
#define LL_FWD_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)

/* loglinear_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation and kernels as loglinear_fwd (automatic group size); its
 * workspace comes from a scratch array of LL_FWD_NOALLOC_SCRATCH_BYTES in the
 * library's device code object (each GPU holds its own copy from the load of
 * the library's kernels until the process ends) instead of an argument.  The
 * call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  The caller passes the inputs and out as for loglinear_fwd.
 *  stream  must belong to the current device (NULL: its null stream).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (each call clears what it needs cleared with a kernel of
 * its own): calls that overlap on one GPU (several streams, or threads
 * without ordering) race and give wrong results; calls ordered on one stream
 * are safe.
 * Errors: those of loglinear_fwd; LL_EWORKSPACE when the shape needs more
 * than LL_FWD_NOALLOC_SCRATCH_BYTES of workspace (it needs at most
 * loglinear_fwd_workspace_bytes(...)); LL_EINVAL for a stream of another
 * device. */
ll_status loglinear_fwd_noalloc(const void *q, const void *k, const void *v,
                                const float *a, const float *lambda, void *out,
                                int B, int H, int T, int dk, int dv, int chunk,
                                ll_dtype dtype, void *stream);

/* One decode step for S sequences x H heads (the recurrent form).
 * Stack convention: for a sequence whose previous token sat at position p,
 * slot 0 holds that token's own state k v^T and slot l >= 1 holds the
 * level-l bucket state iff bit l-1 of p is set (Fenwick occupancy); other
 * slots are free and never read.  A slot stores (hat S, g) meaning the state
 * exp(g) * hat S, so buckets that only decay are never rewritten.
 *  q, k   [S,H,dk]          dtype, the new token
 *  v      [S,H,dv]          dtype
 *  a      [S,H]             float32 log-decay of the new token
 *  lambda [S,H,Lcap]        float32 per-level weights of the new token
 *  state  [S,H,Lcap,dk,dv]  float32 hat S, updated in place
 *  logscale [S,H,Lcap]      float32 g, updated in place
 *  pos    [S]               int64, 0-indexed position of the new token
 *                           (read only; the caller advances it).  pos == 0
 *                           means the stack is empty.
 *  out    [S,H,dv]          dtype, written
 * The step merges the levels below the lowest set bit of pos into one
 * bucket, puts the new token in slot 0, and reads out
 * o = sum over occupied levels l of lambda[l] * q^T S_l.
 * A position outside [0, 2^(Lcap-1)) cannot be represented: that sequence
 * gets NaN outputs and its stack is left unchanged (checked on the device,
 * since pos lives there).
 * Supported: dk, dv in {16, 32, 64, 128}, 2 <= Lcap <= 32, both dtypes.
 * Errors: LL_EINVAL, LL_EUNSUPPORTED, LL_EDEVICE. */
ll_status loglinear_decode_step(const void *q, const void *k, const void *v,
                                const float *a, const float *lambda,
                                float *state, float *logscale, const int64_t *pos,
                                void *out, int S, int H, int dk, int dv, int Lcap,
                                ll_dtype dtype, void *stream);

/* Backward: gradients of the scalar sum over (b, h, t) of dout[t,:] . out[t,:]
 * with respect to q, k, v, a and lambda, for the forward above (the pages
 * name backpropagation through the per-level weights lambda as needing
 * custom kernels: French page §5 "Signification et Limites").  With
 * w(t,s) = exp(sum_{r=s+1..t} a[r]) * lambda[t, level(t,s)] for s <= t:
 *   dq[t]        = sum_s w(t,s) (dout[t].v[s]) k[s]
 *   dk[s]        = sum_t w(t,s) (dout[t].v[s]) q[t]
 *   dv[s]        = sum_t w(t,s) (q[t].k[s]) dout[t]
 *   dlambda[t,l] = sum over keys s of level l: exp(decay) (q[t].k[s]) (dout[t].v[s])
 *   da[r]        = sum over pairs s < r <= t of w(t,s) (q[t].k[s]) (dout[t].v[s]),
 *                  da[...,0] = 0 (a[...,0] never enters)
 *  q, k, v, a, lambda: the forward's inputs (same shapes and dtype)
 *  dout   [B,H,T,dv]  dtype, the gradient of the loss with respect to out
 *  dq, dk [B,H,T,dk]  dtype, written
 *  dv     [B,H,T,dv]  dtype, written
 *  da     [B,H,T]     float32, written
 *  dlambda [B,H,T,L]  float32, written (0 for levels that are empty for a row)
 *  workspace: caller-owned device scratch of loglinear_bwd_workspace_bytes
 *         bytes, 256-byte aligned; contents on entry do not matter.
 * Outputs must not alias each other, the inputs or the workspace.
 * Supported: dk, dv in {32, 64, 128} with chunk 32 or 64 in bf16, and with
 * chunk 32 in float32 (float32 chunk 64 only for dk = dv = 32: the larger
 * chunk kernels do not fit in LDS).  Anything else, including every other
 * multiple of 16 up to 256, returns LL_EUNSUPPORTED.  Accumulation is float32 throughout; in bf16
 * the operands of the matrix products are bf16, as in the forward.
 * Errors: LL_EINVAL, LL_EUNSUPPORTED, LL_EWORKSPACE, LL_EDEVICE. */
size_t loglinear_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
ll_status loglinear_bwd(const void *q, const void *k, const void *v,
                        const float *a, const float *lambda, const void *dout,
                        void *dq, void *dk_out, void *dv_out, float *da, float *dlambda,
                        int B, int H, int T, int dk, int dv, int chunk, ll_dtype dtype,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Prefill: the forward of loglinear_fwd_ex over a prompt of T tokens, which
 * also writes the decode stack the prompt leaves for its next token, so that
 * decoding can continue at position T (the recurrent form takes over from
 * the parallel one: Portuguese page §2 "Forma Recorrente e Paralela";
 * buckets: same page §2 "Particionamento Hierárquico").
 *  q, k, v, a, lambda, out, B, H, T, dk, dv, chunk, dtype, workspace,
 *  workspace_bytes, stream, group_log2: as for loglinear_fwd_ex (the same
 *         workspace size, loglinear_fwd_workspace_bytes_ex).
 *  state    [B,H,Lcap,dk,dv] float32, written: the stack of position T-1 in
 *           loglinear_decode_step's convention (slot 0 = token T-1's k v^T;
 *           slot l >= 1 = its level-l bucket iff bit l-1 of T-1 is set).
 *           Free slots are not written.
 *  logscale [B,H,Lcap] float32, written for the occupied slots (each slot is
 *           stored decayed to its own last key; g is the decay from there to
 *           position T-1).
 *  Lcap     slots per (sequence, head): 2 <= Lcap <= 32 (else
 *           LL_EUNSUPPORTED) and Lcap >= loglinear_num_levels(T + 1) =
 *           1 + bit_length(T) (else LL_EINVAL): the stack of position T-1
 *           needs loglinear_num_levels(T) slots, and the decode step at
 *           position T needs T < 2^(Lcap-1).
 * Sequence b of the forward is decode sequence b: call
 * loglinear_decode_step next with pos[b] = T.  T == 0 leaves an empty stack
 * (pos = 0) and writes nothing.  state and logscale must not alias the
 * inputs, out or the workspace.  Supported: the shapes loglinear_fwd supports
 * with dk, dv in {16, 32, 64, 128}.
 * In bf16, the stack's coarse slots (buckets of at least one chunk group)
 * carry the rounding of the forward's bf16 products; finer slots are summed
 * in float32.
 * Errors: LL_EINVAL, LL_EUNSUPPORTED, LL_EWORKSPACE, LL_EDEVICE. */
ll_status loglinear_prefill(const void *q, const void *k, const void *v,
                            const float *a, const float *lambda, void *out,
                            float *state, float *logscale,
                            int B, int H, int T, int dk, int dv, int chunk, int Lcap,
                            ll_dtype dtype, void *workspace, size_t workspace_bytes,
                            void *stream, int group_log2);

/* ---- q and k shared across heads ----------------------------------------
 * Mamba-2 lets several heads read one q/k head (its "groups"); the pages
 * build log-linear attention on top of Mamba-2 (Portuguese page §2
 * "Metodologia", its point on generalisation; French page §3 "Contributions
 * Clés") without saying whether q and k are per head.  These calls take Hqk q/k heads for H heads (H a positive multiple
 * of Hqk; Hqk = H is the per-head case of the calls above): head h reads q/k
 * head h / (H / Hqk), i.e. consecutive heads share one q/k head.  Everything
 * else (arguments, layouts, workspace sizes, errors) is as in the call each
 * one extends, except:
 *  q, k   [B,Hqk,T,dk] (forward, prefill, backward) or [S,Hqk,dk] (decode)
 *  dq, dk [B,Hqk,T,dk]: the backward sums the gradients of the heads that
 *         share a q/k head (in float32, rounded once to the dtype).
 * The backward's workspace is loglinear_bwd_grouped_workspace_bytes (the
 * forward's and prefill's sizes do not depend on Hqk).  An H that is not a
 * positive multiple of Hqk returns LL_EINVAL (workspace query: 0). */
ll_status loglinear_fwd_grouped(const void *q, const void *k, const void *v,
                                const float *a, const float *lambda, void *out,
                                int B, int H, int Hqk, int T, int dk, int dv, int chunk,
                                ll_dtype dtype, void *workspace, size_t workspace_bytes,
                                void *stream, int group_log2);
ll_status loglinear_prefill_grouped(const void *q, const void *k, const void *v,
                                    const float *a, const float *lambda, void *out,
                                    float *state, float *logscale,
                                    int B, int H, int Hqk, int T, int dk, int dv, int chunk, int Lcap,
                                    ll_dtype dtype, void *workspace, size_t workspace_bytes,
                                    void *stream, int group_log2);
ll_status loglinear_decode_step_grouped(const void *q, const void *k, const void *v,
                                        const float *a, const float *lambda,
                                        float *state, float *logscale, const int64_t *pos,
                                        void *out, int S, int H, int Hqk, int dk, int dv, int Lcap,
                                        ll_dtype dtype, void *stream);
size_t loglinear_bwd_grouped_workspace_bytes(int B, int H, int Hqk, int T, int dk, int dv, int chunk);
ll_status loglinear_bwd_grouped(const void *q, const void *k, const void *v,
                                const float *a, const float *lambda, const void *dout,
                                void *dq, void *dk_out, void *dv_out, float *da, float *dlambda,
                                int B, int H, int Hqk, int T, int dk, int dv, int chunk, ll_dtype dtype,
                                void *workspace, size_t workspace_bytes, void *stream);

/* ---- batches of prompts of different lengths -----------------------------
 * A batch of B prompts padded to one length T: sequence b holds lens[b]
 * tokens at positions 0 .. lens[b]-1, and whatever follows is padding.  The
 * form is causal (row t of the forward reads keys s <= t only: the
 * hierarchical mask is lower triangular, French page §2 "Matrice de Masque
 * Hiérarchique"), so the forward and the backward of the plain calls already
 * serve such a batch:
 *  - rows t < lens[b] of the forward do not depend on the padding, which
 *    must hold finite values (a <= 0 as everywhere); padded rows of out hold
 *    unspecified values;
 *  - with dout zero on the padded rows, the backward's gradients of the real
 *    rows are those of each prompt alone, and those of the padded rows are 0.
 * What differs per sequence is the decode stack a prefill leaves, which
 * belongs to each prompt's own last position:
 *  lens  [B] int32 on the device, 0 <= lens[b] <= T, 4-byte aligned.
 *        lens[b] == 0 leaves an empty stack (nothing written; decode with
 *        pos[b] = 0).  A length outside [0, T] cannot be checked on the host
 *        (lens lives on the device): every logscale entry of that sequence
 *        becomes NaN (so its next decode step returns NaN) and no state is
 *        written.
 * Then loglinear_decode_step continues sequence b at pos[b] = lens[b].
 * Everything else is as in loglinear_prefill_grouped (Hqk = H for per-head
 * q and k); out is the padded forward.  lens == NULL returns LL_EINVAL
 * unless the batch is empty. */
ll_status loglinear_prefill_varlen(const void *q, const void *k, const void *v,
                                   const float *a, const float *lambda, void *out,
                                   float *state, float *logscale, const int *lens,
                                   int B, int H, int Hqk, int T, int dk, int dv, int chunk, int Lcap,
                                   ll_dtype dtype, void *workspace, size_t workspace_bytes,
                                   void *stream, int group_log2);

/* ---- Log-Linear Gated DeltaNet (forward, float32 arithmetic) --------------
 * The pages turn a linear-attention model into its log-linear form by
 * multiplying the model's own attention matrix elementwise with the
 * hierarchical mask, P = A ⊙ M_H (Portuguese page §2 "Metodologia",
 * hierarchical-mask point; French page §3 "Contributions Clés"), and name
 * Gated DeltaNet as the second model so treated.  With Gated DeltaNet's own
 * recurrence  S_t = S_{t-1} M_t + beta_t v_t k_t^T,
 * M_t = exp(a_t) (I - beta_t k_t k_t^T),  o_t = S_t q_t,  this computes
 *   o_t = sum_{s<=t} lambda[t, level(t,s)] * beta_s (k_s^T M_{s+1} ... M_t q_t) * v_s
 * with level() as for loglinear_fwd (lambda = 1 gives Gated DeltaNet).
 *  q, k   [B,H,T,dk]  dtype (k is expected unit-norm, as Gated DeltaNet
 *                     normalises it; not checked)
 *  v      [B,H,T,dv]  dtype
 *  a      [B,H,T]     float32 log of the gate alpha_t (expected <= 0)
 *  beta   [B,H,T]     float32 write strength (expected in [0, 1])
 *  lambda [B,H,T,L]   float32, L = loglinear_num_levels(T)
 *  out    [B,H,T,dv]  dtype, written; must not alias inputs or workspace
 *  q, k, v, out must be 16-byte aligned; a, beta, lambda 4-byte aligned.
 *  chunk  32 or 64; dk, dv in {32, 64, 128}; dtype LL_F32 or LL_BF16 (bf16
 *         inputs are widened on load, all arithmetic is float32, and out is
 *         rounded once); B*H <= 65535.
 *  workspace: loglinear_gdn_fwd_workspace_bytes(...) bytes, 256-byte
 *         aligned (about 4*B*H*T*(dk+dv) + 8*B*H*(T/chunk)*dk*(dk+dv) bytes;
 *         the same for both dtypes).
 * Errors: LL_EINVAL, LL_EUNSUPPORTED, LL_EWORKSPACE, LL_EDEVICE. */
size_t loglinear_gdn_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
ll_status loglinear_gdn_fwd(const void *q, const void *k, const void *v,
                            const float *a, const float *beta, const float *lambda, void *out,
                            int B, int H, int T, int dk, int dv, int chunk, ll_dtype dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Message for the last failing call on this thread ("" if none).  Valid
 * until the next call into the library on the same thread. */
const char *loglinear_last_error(void);

/* ---- measurement support -------------------------------------------------
 * While profiling is on, every kernel the library launches carries a pair of
 * HIP events that its own dispatch records on the launch stream
 * (hipExtLaunchKernelGGL; timing-only events without a system-scope fence,
 * no synchronisation).
 * loglinear_profile_end synchronises those events and returns, per kernel
 * name, the number of launches and the summed device time.  The profiler is
 * process-wide: while it is on, launches from every thread are recorded (a
 * mutex guards its records; with profiling off a launch only reads one
 * atomic flag).  Meant for benchmarks.  Creating the event pool in
 * loglinear_profile_begin may allocate host/driver resources. */
typedef struct {
    char name[48];
    int launches;
    double total_ms;
} ll_kernel_stat;

ll_status loglinear_profile_begin(int max_launches);
ll_status loglinear_profile_end(ll_kernel_stat *stats, int max_stats, int *n_stats);

#ifdef __cplusplus
}
#endif

#endif /* LOGLINEAR_H */
