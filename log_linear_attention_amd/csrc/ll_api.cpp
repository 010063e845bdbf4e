// C ABI of the log-linear attention library: argument validation, error
// reporting, dispatch to the gfx950 kernels and optional launch profiling.
// Validation runs entirely on the host and makes no HIP call, so every error
// path can be exercised on a machine without a GPU (the forward without
// allocation looks up its scratch only after every argument check).
#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <climits>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/loglinear.h"
#include "ll_internal.h"

namespace {

thread_local std::string g_err;

ll_status fail(ll_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

ll_status ok()
{
    g_err.clear();
    return LL_OK;
}

bool aligned(const void *p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

int levels_for(int64_t T)
{
    if (T <= 1)
        return 1;
    int n = 0;
    for (int64_t x = T - 1; x > 0; x >>= 1)
        ++n;
    return 1 + n;
}

// ---- profiling -------------------------------------------------------------
struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};

struct Profiler {
    int used = 0;
    bool overflow = false;
    std::vector<hipEvent_t> pool;
    std::vector<ProfRecord> recs;
};

// The profiler is shared by every thread of the process.  Launches test the
// atomic flag without locking (one relaxed load when profiling is off); the
// event pool and the records are only touched under the mutex.
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
Profiler g_prof;

}  // namespace

namespace ll {

ProfEvents prof_events(const char *name)
{
    if (!g_prof_on.load(std::memory_order_relaxed))
        return {};
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on.load(std::memory_order_relaxed))
        return {};
    if (g_prof.used + 2 > (int)g_prof.pool.size()) {
        g_prof.overflow = true;
        return {};
    }
    ProfRecord r{name, g_prof.pool[g_prof.used], g_prof.pool[g_prof.used + 1]};
    g_prof.used += 2;
    g_prof.recs.push_back(r);
    return {r.start, r.stop};
}

}  // namespace ll

extern "C" {

int loglinear_num_levels(int64_t T)
{
    if (T < 0)
        return -1;
    return levels_for(T);
}

static ll_status check_fwd_shape(const char *who, int B, int H, int T, int dk, int dv, int chunk)
{
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0)
        return fail(LL_EINVAL, "%s: negative or zero size (B=%d H=%d T=%d dk=%d dv=%d)", who, B, H, T, dk, dv);
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(LL_EUNSUPPORTED, "%s: chunk must be 16, 32 or 64 (got %d)", who, chunk);
    const int64_t BH = (int64_t)B * H;
    if (BH * ((int64_t)T / chunk + 1) > INT_MAX)
        return fail(LL_EUNSUPPORTED, "%s: B*H*T/chunk too large for one launch", who);
    return LL_OK;
}

// Hqk q/k heads shared by H heads: Hqk >= 1 and H a multiple of it (with
// H = 0 there is nothing to share and any Hqk >= 0 passes).
static ll_status check_qk_heads(const char *who, int H, int Hqk)
{
    if (H == 0 && Hqk >= 0)
        return LL_OK;
    if (Hqk <= 0 || H % Hqk != 0)
        return fail(LL_EINVAL, "%s: H=%d must be a positive multiple of Hqk=%d", who, H, Hqk);
    return LL_OK;
}

size_t loglinear_fwd_workspace_bytes_ex(int B, int H, int T, int dk, int dv, int chunk, int group_log2)
{
    if (check_fwd_shape("loglinear_fwd_workspace_bytes", B, H, T, dk, dv, chunk) != LL_OK)
        return 0;
    if ((int64_t)B * H * T == 0)
        return 0;
    size_t bytes = ll::fwd_plan(B, H, T, dk, dv, chunk, group_log2, 4).bytes;
    // the one-launch forward may serve this shape (the query has no dtype)
    if (group_log2 < 0 && ll::fused_supported(true, dk, dv, T, levels_for(T)))
        bytes = std::max(bytes, ll::fused_workspace_bytes(B, H, T, dk, dv));
    return bytes;
}

size_t loglinear_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk)
{
    return loglinear_fwd_workspace_bytes_ex(B, H, T, dk, dv, chunk, -1);
}

}  // extern "C"

// ---- scratch of the forward for callers that cannot allocate ---------------
// Each GPU that loads the library's kernels holds its own copy.  On the host,
// `scratch` names a host-side stand-in, not device memory: kernels get the
// address that hipGetSymbolAddress returns for the device in question.
static __device__ __align__(256) unsigned char scratch[LL_FWD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];

// Device address of the current device's scratch, looked up once per device
// with that device current.  The launch stream must belong to it.
ll_status scratch_address(const char *who, void *stream, void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(LL_EDEVICE, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess)
            return fail(LL_EDEVICE, "%s: hipStreamGetDevice failed: %s", who, hipGetErrorString(e));
        if (sdev != dev)
            return fail(LL_EINVAL, "%s: the stream belongs to device %d but device %d is current", who, (int)sdev,
                        dev);
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(LL_EUNSUPPORTED, "%s: device %d beyond the %d this entry point serves", who, dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(LL_EDEVICE, "%s: hipGetSymbolAddress of the scratch failed: %s", who,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return LL_OK;
}

}  // namespace

extern "C" {

// Decode stack a prefill writes (NULL: a plain forward).
struct StackOut {
    float *state, *logscale;
    int Lcap;
    const int *lens = nullptr;   // per-sequence prompt lengths (device), NULL: all T
};

static ll_status run_fwd(const char *who, const void *q, const void *k, const void *v, const float *a,
                         const float *lambda, void *out, int B, int H, int Hqk, int T, int dk, int dv, int chunk,
                         ll_dtype dtype, void *workspace, size_t workspace_bytes, void *stream, int group_log2,
                         const StackOut *so, bool use_scratch = false)
{
    if (dtype != LL_F32 && dtype != LL_BF16)
        return fail(LL_EINVAL, "%s: unknown dtype %d", who, (int)dtype);
    ll_status st = check_fwd_shape(who, B, H, T, dk, dv, chunk);
    if (st != LL_OK)
        return st;
    if ((st = check_qk_heads(who, H, Hqk)) != LL_OK)
        return st;
    if (group_log2 > ll::kMaxGroupLog2)
        return fail(LL_EUNSUPPORTED, "%s: group_log2 %d above %d", who, group_log2, ll::kMaxGroupLog2);
    if ((int64_t)B * H > 65535)
        return fail(LL_EUNSUPPORTED, "%s: B*H above 65535", who);
    const bool bf16 = dtype == LL_BF16;
    if (!ll::fwd_supported(bf16, dk, dv, chunk))
        return fail(LL_EUNSUPPORTED, "%s: no kernel for dtype=%s dk=%d dv=%d chunk=%d", who,
                    bf16 ? "bf16" : "f32", dk, dv, chunk);
    if (so) {
        if (so->Lcap < 1)
            return fail(LL_EINVAL, "%s: Lcap must be >= 1 (got %d)", who, so->Lcap);
        if (so->Lcap < 2 || so->Lcap > ll::kMaxLevels)
            return fail(LL_EUNSUPPORTED, "%s: Lcap must be in [2, %d] (got %d)", who, ll::kMaxLevels, so->Lcap);
        // The stack of position T-1 needs levels_for(T) slots, and the decode
        // step that continues at position T needs T < 2^(Lcap-1), i.e.
        // Lcap >= 1 + bit_length(T) = levels_for(T + 1).
        if (levels_for((int64_t)T + 1) > so->Lcap)
            return fail(LL_EINVAL, "%s: decoding position %d after the prompt needs Lcap >= %d, got %d", who, T,
                        levels_for((int64_t)T + 1), so->Lcap);
        if (!ll::stack_supported(bf16, dk, dv))
            return fail(LL_EUNSUPPORTED, "%s: no stack kernel for dk=%d dv=%d", who, dk, dv);
        if ((int64_t)B * H * (dk / 16) > INT_MAX)
            return fail(LL_EUNSUPPORTED, "%s: B*H too large for the stack launch", who);
    }
    const int64_t rows = (int64_t)B * H * T;
    if (rows == 0)
        return ok();
    const size_t es = bf16 ? 2 : 4;
    const size_t nq = (size_t)B * Hqk * T * dk * es, nv = (size_t)rows * dv * es;
    const void *ptrs[] = {q, k, v, out};
    const char *names[] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i) {
        if (!ptrs[i])
            return fail(LL_EINVAL, "%s: %s is NULL", who, names[i]);
        if (!aligned(ptrs[i], 16))
            return fail(LL_EINVAL, "%s: %s is not 16-byte aligned", who, names[i]);
    }
    if (!a || !lambda)
        return fail(LL_EINVAL, "%s: %s is NULL", who, !a ? "a" : "lambda");
    if (!aligned(a, 4) || !aligned(lambda, 4))
        return fail(LL_EINVAL, "%s: a and lambda must be 4-byte aligned", who);
    const int L = levels_for(T);
    if (L > ll::kMaxLevels)
        return fail(LL_EUNSUPPORTED, "%s: T=%d needs %d levels (max %d)", who, T, L, ll::kMaxLevels);
    const size_t na = (size_t)rows * 4, nl = (size_t)rows * L * 4;
    if (overlaps(out, nv, q, nq) || overlaps(out, nv, k, nq) || overlaps(out, nv, v, nv) ||
        overlaps(out, nv, a, na) || overlaps(out, nv, lambda, nl))
        return fail(LL_EINVAL, "%s: out aliases an input", who);
    const ll::FwdPlan plan = ll::fwd_plan(B, H, T, dk, dv, chunk, group_log2, 4);
    // The forward with automatic groups runs as one launch where it can (the
    // prefill's stack then reads the one-launch forward's Fenwick nodes).
    const bool fused = group_log2 < 0 && ll::fused_supported(bf16, dk, dv, T, L);
    const size_t need = fused ? ll::fused_workspace_bytes(B, H, T, dk, dv) : plan.bytes;
    if (use_scratch && need > 0) {
        // the library's own scratch stands in for the workspace argument
        if (need > LL_FWD_NOALLOC_SCRATCH_BYTES)
            return fail(LL_EWORKSPACE, "%s: this shape needs %zu bytes of scratch, above the %zu the library holds",
                        who, need, (size_t)LL_FWD_NOALLOC_SCRATCH_BYTES);
        if ((st = scratch_address(who, stream, &workspace)) != LL_OK)
            return st;
        workspace_bytes = LL_FWD_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0) {
        if (!workspace)
            return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got NULL", who, need);
        if (workspace_bytes < need)
            return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need,
                        workspace_bytes);
        if (!aligned(workspace, 256))
            return fail(LL_EINVAL, "%s: workspace must be 256-byte aligned", who);
        if (overlaps(workspace, need, out, nv) || overlaps(workspace, need, q, nq) ||
            overlaps(workspace, need, k, nq) || overlaps(workspace, need, v, nv) ||
            overlaps(workspace, need, a, na) || overlaps(workspace, need, lambda, nl))
            return fail(LL_EINVAL, "%s: workspace aliases an input or the output", who);
    }
    const size_t bh = (size_t)B * H;
    if (so) {
        if (!so->state || !so->logscale)
            return fail(LL_EINVAL, "%s: %s is NULL", who, !so->state ? "state" : "logscale");
        if (!aligned(so->state, 16) || !aligned(so->logscale, 4))
            return fail(LL_EINVAL, "%s: state must be 16-byte and logscale 4-byte aligned", who);
        const size_t nst = bh * so->Lcap * dk * dv * 4, nls = bh * so->Lcap * 4;
        const void *others[] = {q, k, v, a, lambda, out, workspace};
        const size_t sizes[] = {nq, nq, nv, na, nl, nv, need};
        for (int i = 0; i < 7; ++i)
            if (overlaps(so->state, nst, others[i], sizes[i]) || overlaps(so->logscale, nls, others[i], sizes[i]))
                return fail(LL_EINVAL, "%s: state and logscale must not alias the inputs, out or the workspace", who);
        if (overlaps(so->state, nst, so->logscale, nls))
            return fail(LL_EINVAL, "%s: state and logscale overlap", who);
        if (so->lens && !aligned(so->lens, 4))
            return fail(LL_EINVAL, "%s: lens must be 4-byte aligned", who);
        if (so->lens && (overlaps(so->state, nst, so->lens, (size_t)B * 4) ||
                         overlaps(so->logscale, nls, so->lens, (size_t)B * 4)))
            return fail(LL_EINVAL, "%s: state and logscale must not alias lens", who);
    }
    ll::FwdArgs args{q, k, v, a, lambda, out, B, H, T, dk, dv, chunk, L, bf16, workspace};
    args.rqk = H / Hqk;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (fused) {
        hipError_t e = ll::fused_launch(args, s);
        if (e != hipSuccess)
            return fail(LL_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
        if (so) {
            const ll::FusedNodes fn = ll::fused_nodes(args);
            ll::StackArgs sa{k, v, a, fn.node, fn.gamN, so->state, so->logscale, (int)bh, T, dk, dv, fn.lg, fn.nG,
                             0, 0, so->Lcap, bf16, true};
            sa.rqk = H / Hqk;
            sa.lens = so->lens;
            sa.H = H;
            sa.fused = true;
            e = ll::stack_launch(sa, s);
            if (e != hipSuccess)
                return fail(LL_EDEVICE, "%s: stack launch failed: %s", who, hipGetErrorString(e));
        }
        return ok();
    }
    bool nat = false;
    hipError_t e = ll::fwd_launch(args, plan, s, &nat);
    if (e != hipSuccess)
        return fail(LL_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
    if (so) {
        const char *ws = static_cast<const char *>(workspace);
        const int lgc = plan.g + (chunk == 16 ? 4 : chunk == 32 ? 5 : 6);
        ll::StackArgs sa{k, v, a,
                         plan.nL > 0 ? static_cast<const void *>(ws + plan.off_Dg) : nullptr,
                         plan.nL > 0 ? reinterpret_cast<const float *>(ws + plan.off_Gam) : nullptr,
                         so->state, so->logscale, (int)bh, T, dk, dv, lgc, plan.nG, plan.nL, plan.nLeft, so->Lcap,
                         bf16, nat};
        sa.rqk = H / Hqk;
        sa.lens = so->lens;
        sa.H = H;
        e = ll::stack_launch(sa, s);
        if (e != hipSuccess)
            return fail(LL_EDEVICE, "%s: stack launch failed: %s", who, hipGetErrorString(e));
    }
    return ok();
}

ll_status loglinear_fwd_ex(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                           void *out, int B, int H, int T, int dk, int dv, int chunk, ll_dtype dtype,
                           void *workspace, size_t workspace_bytes, void *stream, int group_log2)
{
    return run_fwd("loglinear_fwd", q, k, v, a, lambda, out, B, H, H, T, dk, dv, chunk, dtype, workspace,
                   workspace_bytes, stream, group_log2, nullptr);
}

ll_status loglinear_fwd_grouped(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                                void *out, int B, int H, int Hqk, int T, int dk, int dv, int chunk, ll_dtype dtype,
                                void *workspace, size_t workspace_bytes, void *stream, int group_log2)
{
    return run_fwd("loglinear_fwd_grouped", q, k, v, a, lambda, out, B, H, Hqk, T, dk, dv, chunk, dtype, workspace,
                   workspace_bytes, stream, group_log2, nullptr);
}

ll_status loglinear_prefill(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                            void *out, float *state, float *logscale, int B, int H, int T, int dk, int dv,
                            int chunk, int Lcap, ll_dtype dtype, void *workspace, size_t workspace_bytes,
                            void *stream, int group_log2)
{
    const StackOut so{state, logscale, Lcap};
    return run_fwd("loglinear_prefill", q, k, v, a, lambda, out, B, H, H, T, dk, dv, chunk, dtype, workspace,
                   workspace_bytes, stream, group_log2, &so);
}

ll_status loglinear_prefill_varlen(const void *q, const void *k, const void *v, const float *a,
                                   const float *lambda, void *out, float *state, float *logscale,
                                   const int *lens, int B, int H, int Hqk, int T, int dk, int dv, int chunk,
                                   int Lcap, ll_dtype dtype, void *workspace, size_t workspace_bytes, void *stream,
                                   int group_log2)
{
    if (!lens && (int64_t)B * H * T > 0)
        return fail(LL_EINVAL, "loglinear_prefill_varlen: lens is NULL");
    StackOut so{state, logscale, Lcap};
    so.lens = lens;
    return run_fwd("loglinear_prefill_varlen", q, k, v, a, lambda, out, B, H, Hqk, T, dk, dv, chunk, dtype,
                   workspace, workspace_bytes, stream, group_log2, &so);
}

ll_status loglinear_prefill_grouped(const void *q, const void *k, const void *v, const float *a,
                                    const float *lambda, void *out, float *state, float *logscale, int B, int H,
                                    int Hqk, int T, int dk, int dv, int chunk, int Lcap, ll_dtype dtype,
                                    void *workspace, size_t workspace_bytes, void *stream, int group_log2)
{
    const StackOut so{state, logscale, Lcap};
    return run_fwd("loglinear_prefill_grouped", q, k, v, a, lambda, out, B, H, Hqk, T, dk, dv, chunk, dtype,
                   workspace, workspace_bytes, stream, group_log2, &so);
}

ll_status loglinear_fwd(const void *q, const void *k, const void *v, const float *a, const float *lambda, void *out,
                        int B, int H, int T, int dk, int dv, int chunk, ll_dtype dtype, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    return loglinear_fwd_ex(q, k, v, a, lambda, out, B, H, T, dk, dv, chunk, dtype, workspace, workspace_bytes,
                            stream, -1);
}

ll_status loglinear_fwd_noalloc(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                                void *out, int B, int H, int T, int dk, int dv, int chunk, ll_dtype dtype,
                                void *stream)
{
    return run_fwd("loglinear_fwd_noalloc", q, k, v, a, lambda, out, B, H, H, T, dk, dv, chunk, dtype, nullptr, 0,
                   stream, -1, nullptr, true);
}

size_t loglinear_bwd_grouped_workspace_bytes(int B, int H, int Hqk, int T, int dk, int dv, int chunk)
{
    if (check_fwd_shape("loglinear_bwd_workspace_bytes", B, H, T, dk, dv, chunk) != LL_OK)
        return 0;
    if (Hqk <= 0 || (H > 0 && H % Hqk != 0))
        return 0;
    if ((int64_t)B * H * T == 0)
        return 0;
    return ll::bwd_plan(B, H, T, dk, dv, chunk, H / Hqk).bytes;
}

size_t loglinear_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk)
{
    return loglinear_bwd_grouped_workspace_bytes(B, H, H > 0 ? H : 1, T, dk, dv, chunk);
}

static ll_status run_bwd(const char *who, const void *q, const void *k, const void *v, const float *a,
                         const float *lambda, const void *dout, void *dq, void *dk_out, void *dv_out, float *da,
                         float *dlambda, int B, int H, int Hqk, int T, int dk, int dv, int chunk, ll_dtype dtype,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != LL_F32 && dtype != LL_BF16)
        return fail(LL_EINVAL, "%s: unknown dtype %d", who, (int)dtype);
    ll_status st = check_fwd_shape(who, B, H, T, dk, dv, chunk);
    if (st != LL_OK)
        return st;
    if ((st = check_qk_heads(who, H, Hqk)) != LL_OK)
        return st;
    const bool bf16 = dtype == LL_BF16;
    if (!ll::bwd_supported(bf16, dk, dv, chunk))
        return fail(LL_EUNSUPPORTED, "%s: no kernel for dtype=%s dk=%d dv=%d chunk=%d", who, bf16 ? "bf16" : "f32",
                    dk, dv, chunk);
    if ((int64_t)B * H > 65535)
        return fail(LL_EUNSUPPORTED, "%s: B*H above 65535", who);
    const int64_t rows = (int64_t)B * H * T;
    if (rows == 0)
        return ok();
    const int L = levels_for(T);
    if (L > ll::kMaxLevels)
        return fail(LL_EUNSUPPORTED, "%s: T=%d needs %d levels (max %d)", who, T, L, ll::kMaxLevels);
    const size_t es = bf16 ? 2 : 4;
    const size_t nq = (size_t)B * Hqk * T * dk * es, nv = (size_t)rows * dv * es, na = (size_t)rows * 4,
                 nl = (size_t)rows * L * 4;
    const void *ins[] = {q, k, v, dout};
    const char *inames[] = {"q", "k", "v", "dout"};
    void *outs[] = {dq, dk_out, dv_out};
    const char *onames[] = {"dq", "dk", "dv"};
    for (int i = 0; i < 4; ++i) {
        if (!ins[i])
            return fail(LL_EINVAL, "%s: %s is NULL", who, inames[i]);
        if (!aligned(ins[i], 16))
            return fail(LL_EINVAL, "%s: %s is not 16-byte aligned", who, inames[i]);
    }
    for (int i = 0; i < 3; ++i) {
        if (!outs[i])
            return fail(LL_EINVAL, "%s: %s is NULL", who, onames[i]);
        if (!aligned(outs[i], 16))
            return fail(LL_EINVAL, "%s: %s is not 16-byte aligned", who, onames[i]);
    }
    if (!a || !lambda || !da || !dlambda)
        return fail(LL_EINVAL, "%s: a, lambda, da and dlambda must be non-NULL", who);
    if (!aligned(a, 4) || !aligned(lambda, 4) || !aligned(da, 4) || !aligned(dlambda, 4))
        return fail(LL_EINVAL, "%s: a, lambda, da and dlambda must be 4-byte aligned", who);
    const ll::BwdPlan plan = ll::bwd_plan(B, H, T, dk, dv, chunk, H / Hqk);
    if (!workspace)
        return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got NULL", who, plan.bytes);
    if (workspace_bytes < plan.bytes)
        return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, plan.bytes, workspace_bytes);
    if (!aligned(workspace, 256))
        return fail(LL_EINVAL, "%s: workspace must be 256-byte aligned", who);
    // every output must be disjoint from every input, every other output and the workspace
    const void *all[] = {q, k, v, dout, a, lambda, workspace, dq, dk_out, dv_out, da, dlambda};
    const size_t sz[] = {nq, nq, nv, nv, na, nl, plan.bytes, nq, nq, nv, na, nl};
    for (int i = 7; i < 12; ++i)
        for (int j = 0; j < 12; ++j)
            if (j != i && overlaps(all[i], sz[i], all[j], sz[j]))
                return fail(LL_EINVAL, "%s: outputs must not alias each other, an input or the workspace", who);
    if (overlaps(workspace, plan.bytes, q, nq) || overlaps(workspace, plan.bytes, k, nq) ||
        overlaps(workspace, plan.bytes, v, nv) || overlaps(workspace, plan.bytes, dout, nv))
        return fail(LL_EINVAL, "%s: workspace aliases an input", who);
    ll::BwdArgs args{q, k, v, dout, a, lambda, dq, dk_out, dv_out, da, dlambda, B, H, T, dk, dv, chunk, L, bf16,
                     workspace};
    args.rqk = H / Hqk;
    hipError_t e = ll::bwd_launch(args, plan, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(LL_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ok();
}

ll_status loglinear_bwd(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                        const void *dout, void *dq, void *dk_out, void *dv_out, float *da, float *dlambda, int B,
                        int H, int T, int dk, int dv, int chunk, ll_dtype dtype, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    return run_bwd("loglinear_bwd", q, k, v, a, lambda, dout, dq, dk_out, dv_out, da, dlambda, B, H, H, T, dk, dv,
                   chunk, dtype, workspace, workspace_bytes, stream);
}

ll_status loglinear_bwd_grouped(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                                const void *dout, void *dq, void *dk_out, void *dv_out, float *da, float *dlambda,
                                int B, int H, int Hqk, int T, int dk, int dv, int chunk, ll_dtype dtype,
                                void *workspace, size_t workspace_bytes, void *stream)
{
    return run_bwd("loglinear_bwd_grouped", q, k, v, a, lambda, dout, dq, dk_out, dv_out, da, dlambda, B, H, Hqk,
                   T, dk, dv, chunk, dtype, workspace, workspace_bytes, stream);
}

static ll_status run_decode(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                            float *state, float *logscale, const int64_t *pos, void *out, int S, int H, int Hqk,
                            int dk, int dv, int Lcap, ll_dtype dtype, void *stream)
{
    if (dtype != LL_F32 && dtype != LL_BF16)
        return fail(LL_EINVAL, "loglinear_decode_step: unknown dtype %d", (int)dtype);
    if (S < 0 || H < 0 || dk <= 0 || dv <= 0)
        return fail(LL_EINVAL, "loglinear_decode_step: bad size (S=%d H=%d dk=%d dv=%d)", S, H, dk, dv);
    if (check_qk_heads("loglinear_decode_step", H, Hqk) != LL_OK)
        return LL_EINVAL;
    if (Lcap < 1)
        return fail(LL_EINVAL, "loglinear_decode_step: Lcap must be >= 1 (got %d)", Lcap);
    if (Lcap < 2 || Lcap > ll::kMaxLevels)
        return fail(LL_EUNSUPPORTED, "loglinear_decode_step: Lcap must be in [2, %d] (got %d)", ll::kMaxLevels, Lcap);
    const bool bf16 = dtype == LL_BF16;
    if (!ll::decode_supported(bf16, dk, dv))
        return fail(LL_EUNSUPPORTED, "loglinear_decode_step: no kernel for dk=%d dv=%d", dk, dv);
    if ((int64_t)S * H > INT_MAX)
        return fail(LL_EUNSUPPORTED, "loglinear_decode_step: S*H too large");
    if ((int64_t)S * H == 0)
        return ok();
    const void *ptrs[] = {q, k, v, out, state};
    const char *names[] = {"q", "k", "v", "out", "state"};
    for (int i = 0; i < 5; ++i) {
        if (!ptrs[i])
            return fail(LL_EINVAL, "loglinear_decode_step: %s is NULL", names[i]);
        if (!aligned(ptrs[i], 16))
            return fail(LL_EINVAL, "loglinear_decode_step: %s is not 16-byte aligned", names[i]);
    }
    if (!a || !lambda || !logscale || !pos)
        return fail(LL_EINVAL, "loglinear_decode_step: a, lambda, logscale and pos must be non-NULL");
    if (!aligned(a, 4) || !aligned(lambda, 4) || !aligned(logscale, 4) || !aligned(pos, 8))
        return fail(LL_EINVAL, "loglinear_decode_step: misaligned a/lambda/logscale/pos");
    const size_t sh = (size_t)S * H;
    const size_t es = bf16 ? 2 : 4;
    const size_t nst = sh * Lcap * dk * dv * 4, nout = sh * dv * es, nq = (size_t)S * Hqk * dk * es;
    // Every written buffer (state, logscale, out) must be disjoint from every
    // other buffer of the call.
    const void *all[] = {state, logscale, out, q, k, v, a, lambda, pos};
    const size_t sz[] = {nst, sh * Lcap * 4, nout, nq, nq, nout, sh * 4, sh * Lcap * 4, (size_t)S * 8};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 9; ++j)
            if (j != i && overlaps(all[i], sz[i], all[j], sz[j]))
                return fail(LL_EINVAL,
                            "loglinear_decode_step: state, logscale and out must not alias each other or inputs");
    ll::DecodeArgs args{q, k, v, a, lambda, state, logscale, pos, out, S, H, dk, dv, Lcap, bf16};
    args.rqk = H / Hqk;
    hipError_t e = ll::decode_launch(args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(LL_EDEVICE, "loglinear_decode_step: launch failed: %s", hipGetErrorString(e));
    return ok();
}

ll_status loglinear_decode_step(const void *q, const void *k, const void *v, const float *a, const float *lambda,
                                float *state, float *logscale, const int64_t *pos, void *out, int S, int H, int dk,
                                int dv, int Lcap, ll_dtype dtype, void *stream)
{
    return run_decode(q, k, v, a, lambda, state, logscale, pos, out, S, H, H, dk, dv, Lcap, dtype, stream);
}

ll_status loglinear_decode_step_grouped(const void *q, const void *k, const void *v, const float *a,
                                        const float *lambda, float *state, float *logscale, const int64_t *pos,
                                        void *out, int S, int H, int Hqk, int dk, int dv, int Lcap, ll_dtype dtype,
                                        void *stream)
{
    return run_decode(q, k, v, a, lambda, state, logscale, pos, out, S, H, Hqk, dk, dv, Lcap, dtype, stream);
}

size_t loglinear_gdn_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk)
{
    if (check_fwd_shape("loglinear_gdn_fwd_workspace_bytes", B, H, T, dk, dv, chunk) != LL_OK)
        return 0;
    if ((int64_t)B * H * T == 0 || !ll::gdn_supported(dk, dv, chunk))
        return 0;
    return ll::gdn_plan(B, H, T, dk, dv, chunk).bytes;
}

ll_status loglinear_gdn_fwd(const void *q, const void *k, const void *v, const float *a, const float *beta,
                            const float *lambda, void *out, int B, int H, int T, int dk, int dv, int chunk,
                            ll_dtype dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    const char *who = "loglinear_gdn_fwd";
    if (dtype != LL_F32 && dtype != LL_BF16)
        return fail(LL_EINVAL, "%s: unknown dtype %d", who, (int)dtype);
    ll_status st = check_fwd_shape(who, B, H, T, dk, dv, chunk);
    if (st != LL_OK)
        return st;
    if (!ll::gdn_supported(dk, dv, chunk))
        return fail(LL_EUNSUPPORTED, "%s: no kernel for dk=%d dv=%d chunk=%d", who, dk, dv, chunk);
    if ((int64_t)B * H > 65535)
        return fail(LL_EUNSUPPORTED, "%s: B*H above 65535", who);
    const int64_t rows = (int64_t)B * H * T;
    if (rows == 0)
        return ok();
    const int L = levels_for(T);
    if (L > ll::kMaxLevels)
        return fail(LL_EUNSUPPORTED, "%s: T=%d needs %d levels (max %d)", who, T, L, ll::kMaxLevels);
    const void *ptrs[] = {q, k, v, a, beta, lambda, out};
    const char *names[] = {"q", "k", "v", "a", "beta", "lambda", "out"};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i])
            return fail(LL_EINVAL, "%s: %s is NULL", who, names[i]);
        // q, k, v, out are read and written four elements at a time
        if (!aligned(ptrs[i], (i < 3 || i == 6) ? 16 : 4))
            return fail(LL_EINVAL, "%s: %s is misaligned", who, names[i]);
    }
    const ll::GdnPlan plan = ll::gdn_plan(B, H, T, dk, dv, chunk);
    if (!workspace)
        return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got NULL", who, plan.bytes);
    if (workspace_bytes < plan.bytes)
        return fail(LL_EWORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, plan.bytes, workspace_bytes);
    if (!aligned(workspace, 256))
        return fail(LL_EINVAL, "%s: workspace must be 256-byte aligned", who);
    const size_t es = dtype == LL_BF16 ? 2 : 4;
    const size_t nq = (size_t)rows * dk * es, nv = (size_t)rows * dv * es, na = (size_t)rows * 4,
                 nl = (size_t)rows * L * 4;
    const void *all[] = {q, k, v, a, beta, lambda, workspace};
    const size_t sz[] = {nq, nq, nv, na, na, nl, plan.bytes};
    for (int i = 0; i < 7; ++i)
        if (overlaps(out, nv, all[i], sz[i]))
            return fail(LL_EINVAL, "%s: out aliases an input or the workspace", who);
    for (int i = 0; i < 6; ++i)
        if (overlaps(workspace, plan.bytes, all[i], sz[i]))
            return fail(LL_EINVAL, "%s: workspace aliases an input", who);
    ll::GdnArgs args{q, k, v, a, beta, lambda, out, B, H, T, dk, dv, chunk, L, workspace};
    args.bf16 = dtype == LL_BF16;
    hipError_t e = ll::gdn_launch(args, plan, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(LL_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ok();
}

const char *loglinear_last_error(void) { return g_err.c_str(); }

ll_status loglinear_profile_begin(int max_launches)
{
    if (max_launches <= 0)
        return fail(LL_EINVAL, "loglinear_profile_begin: max_launches must be positive");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_relaxed);
    for (hipEvent_t e : g_prof.pool)
        (void)hipEventDestroy(e);
    g_prof = Profiler();
    g_prof.pool.resize(2 * (size_t)max_launches);
    for (size_t i = 0; i < g_prof.pool.size(); ++i) {
        // Timing-only events: no system-scope fence, so recording them adds no
        // cache writeback or invalidation to the launches they time.
        hipError_t e = hipEventCreateWithFlags(&g_prof.pool[i], hipEventDisableSystemFence);
        if (e != hipSuccess) {
            g_prof.pool.resize(i);
            return fail(LL_EDEVICE, "loglinear_profile_begin: hipEventCreate failed: %s", hipGetErrorString(e));
        }
    }
    g_prof.recs.reserve(max_launches);
    g_prof_on.store(true, std::memory_order_relaxed);
    return ok();
}

ll_status loglinear_profile_end(ll_kernel_stat *stats, int max_stats, int *n_stats)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on.load(std::memory_order_relaxed))
        return fail(LL_EINVAL, "loglinear_profile_end: profiling is not on");
    g_prof_on.store(false, std::memory_order_relaxed);
    std::vector<ll_kernel_stat> out;
    for (const ProfRecord &r : g_prof.recs) {
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess)
            return fail(LL_EDEVICE, "loglinear_profile_end: %s", hipGetErrorString(e));
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, r.start, r.stop);
        size_t i = 0;
        for (; i < out.size(); ++i)
            if (std::strcmp(out[i].name, r.name) == 0)
                break;
        if (i == out.size()) {
            ll_kernel_stat s{};
            std::snprintf(s.name, sizeof s.name, "%s", r.name);
            out.push_back(s);
        }
        out[i].launches += 1;
        out[i].total_ms += ms;
    }
    const int n = (int)out.size() < max_stats ? (int)out.size() : max_stats;
    for (int i = 0; i < n; ++i)
        stats[i] = out[i];
    if (n_stats)
        *n_stats = n;
    const bool overflow = g_prof.overflow;
    for (hipEvent_t e : g_prof.pool)
        (void)hipEventDestroy(e);
    g_prof = Profiler();
    if (overflow)
        return fail(LL_EINVAL, "loglinear_profile_end: event pool overflowed; some launches were not timed");
    return ok();
}

}  // extern "C"
