"""Python binding of libloglinear.so (gfx950 log-linear attention).

Argument marshalling only: every step of the forward and the decode runs in
the library's HIP kernels.  torch is used for device memory and streams; the
functions take torch CUDA tensors, check dtype/device/contiguity, and pass raw
pointers.  If the library has not been built this module raises on first use;
there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LOGLINEAR_LIB names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("LOGLINEAR_LIB") or os.path.join(_HERE, "libloglinear.so")

LL_OK, LL_EINVAL, LL_EUNSUPPORTED, LL_EDEVICE, LL_EWORKSPACE = 0, -1, -2, -3, -4
LL_F32, LL_BF16 = 0, 1
FWD_NOALLOC_SCRATCH_BYTES = 80 << 20   # LL_FWD_NOALLOC_SCRATCH_BYTES

_STATUS_NAMES = {
    LL_EINVAL: "LL_EINVAL",
    LL_EUNSUPPORTED: "LL_EUNSUPPORTED",
    LL_EDEVICE: "LL_EDEVICE",
    LL_EWORKSPACE: "LL_EWORKSPACE",
}


class LLError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library (loads it on first call)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m log_linear_attention_amd.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
        L.loglinear_num_levels.argtypes = [I64]
        L.loglinear_num_levels.restype = I
        L.loglinear_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.loglinear_fwd_workspace_bytes.restype = Z
        L.loglinear_fwd_workspace_bytes_ex.argtypes = [I, I, I, I, I, I, I]
        L.loglinear_fwd_workspace_bytes_ex.restype = Z
        L.loglinear_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        L.loglinear_fwd.restype = I
        L.loglinear_fwd_ex.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P, I]
        L.loglinear_fwd_ex.restype = I
        L.loglinear_fwd_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P]
        L.loglinear_fwd_noalloc.restype = I
        L.loglinear_prefill.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, Z, P, I]
        L.loglinear_prefill.restype = I
        L.loglinear_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.loglinear_bwd_workspace_bytes.restype = Z
        L.loglinear_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        L.loglinear_bwd.restype = I
        L.loglinear_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P]
        L.loglinear_decode_step.restype = I
        L.loglinear_fwd_grouped.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, Z, P, I]
        L.loglinear_fwd_grouped.restype = I
        L.loglinear_prefill_grouped.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, Z, P, I]
        L.loglinear_prefill_grouped.restype = I
        L.loglinear_prefill_varlen.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, Z, P, I]
        L.loglinear_prefill_varlen.restype = I
        L.loglinear_gdn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.loglinear_gdn_fwd_workspace_bytes.restype = Z
        L.loglinear_gdn_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
        L.loglinear_gdn_fwd.restype = I
        L.loglinear_decode_step_grouped.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
        L.loglinear_decode_step_grouped.restype = I
        L.loglinear_bwd_grouped_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.loglinear_bwd_grouped_workspace_bytes.restype = Z
        L.loglinear_bwd_grouped.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, Z, P]
        L.loglinear_bwd_grouped.restype = I
        L.loglinear_last_error.argtypes = []
        L.loglinear_last_error.restype = ctypes.c_char_p
        L.loglinear_profile_begin.argtypes = [I]
        L.loglinear_profile_begin.restype = I
        L.loglinear_profile_end.argtypes = [ctypes.POINTER(KernelStat), I, ctypes.POINTER(I)]
        L.loglinear_profile_end.restype = I
        _lib = L
    return _lib


def last_error() -> str:
    return lib().loglinear_last_error().decode()


def _check(status: int) -> None:
    if status != LL_OK:
        raise LLError(status, last_error())


def num_levels(T: int) -> int:
    return int(lib().loglinear_num_levels(int(T)))


def fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int, group_log2: int = -1) -> int:
    return int(lib().loglinear_fwd_workspace_bytes_ex(B, H, T, dk, dv, chunk, group_log2))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LL_F32
    if t.dtype == torch.bfloat16:
        return LL_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _keep_for_stream(t, stream) -> None:
    """Tie a tensor that this module allocated to the launch stream.

    The caching allocator reuses a freed block as soon as the stream it was
    allocated on is done with it.  The tensors allocated here (workspaces and
    default outputs) are allocated on torch's current stream, while the
    kernels run asynchronously on ``stream``; recording that stream keeps the
    block from being handed out again before the kernels that use it finish."""
    if t is None or stream is None:
        return
    if isinstance(stream, torch.cuda.Stream):
        ts = stream
    else:
        handle = int(stream)
        if handle == torch.cuda.current_stream().cuda_stream:
            return
        ts = torch.cuda.ExternalStream(handle)
    if ts.cuda_stream != torch.cuda.current_stream().cuda_stream:
        t.record_stream(ts)


def _qkv_shapes(q, k, v):
    """(B, H, Hqk, T, dk, dv) from q, k [B,Hqk,T,dk] and v [B,H,T,dv]; H must
    be a multiple of Hqk (Hqk = H: one q/k head per head)."""
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[0] != q.shape[0] or v.shape[2] != q.shape[2]:
        raise ValueError("q, k must be [B,Hqk,T,dk] and v [B,H,T,dv]")
    B, Hqk, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    if Hqk == 0 or H % Hqk != 0:
        raise ValueError(f"the number of heads H={H} must be a multiple of the q/k heads Hqk={Hqk}")
    return B, H, Hqk, T, dk, dv


def alloc_workspace(B, H, T, dk, dv, chunk, group_log2=-1, device="cuda") -> torch.Tensor | None:
    n = fwd_workspace_bytes(B, H, T, dk, dv, chunk, group_log2)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def fwd(q, k, v, a, lam, chunk: int = 64, out=None, workspace=None, group_log2: int = -1, stream=None):
    """Forward pass.  q,k [B,Hqk,T,dk], v [B,H,T,dv] (float32 or bfloat16,
    same dtype; Hqk = H, or H a multiple of Hqk when consecutive heads share
    a q/k head), a [B,H,T] float32, lam [B,H,T,L] float32 with
    L = num_levels(T).  Returns out [B,H,T,dv] in the input dtype.
    Asynchronous on ``stream``."""
    B, H, Hqk, T, dk, dv = _qkv_shapes(q, k, v)
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    L = num_levels(T)
    if tuple(a.shape) != (B, H, T) or tuple(lam.shape) != (B, H, T, L):
        raise ValueError(f"a must be [B,H,T] and lam [B,H,T,{L}]")
    own = []
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
        own.append(out)
    elif tuple(out.shape) != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    need = fwd_workspace_bytes(B, H, T, dk, dv, chunk, group_log2)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if Hqk == H:
        st = lib().loglinear_fwd_ex(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
            _dev(out, "out"), B, H, T, dk, dv, chunk, code, ws_ptr, ws_bytes, _stream(stream), group_log2)
    else:
        st = lib().loglinear_fwd_grouped(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
            _dev(out, "out"), B, H, Hqk, T, dk, dv, chunk, code, ws_ptr, ws_bytes, _stream(stream), group_log2)
    for t in own:
        _keep_for_stream(t, stream)
    _check(st)
    return out


def fwd_noalloc(q, k, v, a, lam, out, chunk: int = 64, stream=None):
    """loglinear_fwd_noalloc: the forward with the library's per-GPU scratch
    as its workspace, for callers that cannot allocate.  Same arguments as
    fwd with one q/k head per head; out [B,H,T,dv] is required (nothing is
    allocated).  Calls that overlap on one GPU race on the scratch.
    Asynchronous on ``stream``."""
    B, H, Hqk, T, dk, dv = _qkv_shapes(q, k, v)
    if Hqk != H:
        raise ValueError("fwd_noalloc takes one q/k head per head")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    L = num_levels(T)
    if tuple(a.shape) != (B, H, T) or tuple(lam.shape) != (B, H, T, L):
        raise ValueError(f"a must be [B,H,T] and lam [B,H,T,{L}]")
    if tuple(out.shape) != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    _check(lib().loglinear_fwd_noalloc(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
        _dev(out, "out"), B, H, T, dk, dv, chunk, code, _stream(stream)))
    return out


def prefill(q, k, v, a, lam, state, logscale, chunk: int = 64, out=None, workspace=None, group_log2: int = -1,
            stream=None, lengths=None):
    """Forward over a prompt that also writes the decode stack of its last
    position.  Inputs as for ``fwd``; state [B,H,Lcap,dk,dv] and logscale
    [B,H,Lcap] float32 are written (free slots untouched).  Decoding continues
    with ``decode_step`` at pos = T.  Returns out [B,H,T,dv].

    ``lengths`` (optional int32 GPU tensor [B]): the batch holds prompts of
    these lengths padded to T; each sequence's stack is that of its own last
    position, and decoding continues at pos = lengths."""
    B, H, Hqk, T, dk, dv = _qkv_shapes(q, k, v)
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    L = num_levels(T)
    if tuple(a.shape) != (B, H, T) or tuple(lam.shape) != (B, H, T, L):
        raise ValueError(f"a must be [B,H,T] and lam [B,H,T,{L}]")
    if state.dim() != 5:
        raise ValueError("state must be [B,H,Lcap,dk,dv]")
    Lcap = state.shape[2]
    if tuple(state.shape) != (B, H, Lcap, dk, dv) or tuple(logscale.shape) != (B, H, Lcap):
        raise ValueError("state must be [B,H,Lcap,dk,dv] and logscale [B,H,Lcap]")
    own = []
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
        own.append(out)
    elif tuple(out.shape) != (B, H, T, dv) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    need = fwd_workspace_bytes(B, H, T, dk, dv, chunk, group_log2)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptrs = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
            _dev(out, "out"), _dev(state, "state", torch.float32), _dev(logscale, "logscale", torch.float32))
    if lengths is not None:
        if tuple(lengths.shape) != (B,):
            raise ValueError("lengths must be [B]")
        st = lib().loglinear_prefill_varlen(*ptrs, _dev(lengths, "lengths", torch.int32), B, H, Hqk, T, dk, dv,
                                            chunk, Lcap, code, ws_ptr, ws_bytes, _stream(stream), group_log2)
    elif Hqk == H:
        st = lib().loglinear_prefill(*ptrs, B, H, T, dk, dv, chunk, Lcap, code, ws_ptr, ws_bytes, _stream(stream),
                                     group_log2)
    else:
        st = lib().loglinear_prefill_grouped(*ptrs, B, H, Hqk, T, dk, dv, chunk, Lcap, code, ws_ptr, ws_bytes,
                                             _stream(stream), group_log2)
    for t in own:
        _keep_for_stream(t, stream)
    _check(st)
    return out


def bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int, Hqk: int | None = None) -> int:
    if Hqk is None or Hqk == H:
        return int(lib().loglinear_bwd_workspace_bytes(B, H, T, dk, dv, chunk))
    return int(lib().loglinear_bwd_grouped_workspace_bytes(B, H, Hqk, T, dk, dv, chunk))


def bwd(q, k, v, a, lam, dout, chunk: int = 64, workspace=None, stream=None):
    """Backward of ``fwd``: gradients of sum(dout * fwd(q, k, v, a, lam)).
    Returns (dq, dk, dv, da, dlam): dq, dk, dv in the input dtype (dq, dk
    shaped like q, k: with shared q/k heads they sum over the heads sharing
    each), da and dlam float32.  Asynchronous on ``stream``."""
    B, H, Hqk, T, dk, dv = _qkv_shapes(q, k, v)
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("q, k, v, dout must share one dtype")
    L = num_levels(T)
    if tuple(a.shape) != (B, H, T) or tuple(lam.shape) != (B, H, T, L) or tuple(dout.shape) != (B, H, T, dv):
        raise ValueError(f"a must be [B,H,T], lam [B,H,T,{L}] and dout [B,H,T,dv]")
    dq = torch.empty_like(q)
    dk_ = torch.empty_like(k)
    dv_ = torch.empty_like(v)
    da = torch.empty_like(a)
    dlam = torch.empty_like(lam)
    own = [dq, dk_, dv_, da, dlam]
    need = bwd_workspace_bytes(B, H, T, dk, dv, chunk, Hqk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptrs = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
            _dev(dout, "dout"), _dev(dq, "dq"), _dev(dk_, "dk"), _dev(dv_, "dv"), _dev(da, "da", torch.float32),
            _dev(dlam, "dlam", torch.float32))
    if Hqk == H:
        st = lib().loglinear_bwd(*ptrs, B, H, T, dk, dv, chunk, code, ws_ptr, ws_bytes, _stream(stream))
    else:
        st = lib().loglinear_bwd_grouped(*ptrs, B, H, Hqk, T, dk, dv, chunk, code, ws_ptr, ws_bytes,
                                         _stream(stream))
    for t in own:
        _keep_for_stream(t, stream)
    _check(st)
    return dq, dk_, dv_, da, dlam


def decode_step(q, k, v, a, lam, state, logscale, pos, out=None, stream=None):
    """One decode step.  q,k [S,Hqk,dk], v [S,H,dv] (float32 or bfloat16;
    Hqk = H, or H a multiple of Hqk), a [S,H], lam [S,H,Lcap],
    state [S,H,Lcap,dk,dv] and logscale [S,H,Lcap] float32 (updated in place),
    pos [S] int64.  Returns out [S,H,dv]."""
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [S,Hqk,dk] and v [S,H,dv]")
    S, Hqk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    if Hqk == 0 or H % Hqk != 0:
        raise ValueError(f"the number of heads H={H} must be a multiple of the q/k heads Hqk={Hqk}")
    Lcap = state.shape[2]
    code = _dtype_code(q)
    if tuple(state.shape) != (S, H, Lcap, dk, dv) or tuple(logscale.shape) != (S, H, Lcap):
        raise ValueError("state must be [S,H,Lcap,dk,dv] and logscale [S,H,Lcap]")
    if tuple(lam.shape) != (S, H, Lcap) or tuple(a.shape) != (S, H) or tuple(pos.shape) != (S,):
        raise ValueError("lam must be [S,H,Lcap], a [S,H], pos [S]")
    own = []
    if out is None:
        out = torch.empty((S, H, dv), dtype=q.dtype, device=q.device)
        own.append(out)
    ptrs = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", torch.float32), _dev(lam, "lam", torch.float32),
            _dev(state, "state", torch.float32), _dev(logscale, "logscale", torch.float32),
            _dev(pos, "pos", torch.int64), _dev(out, "out"))
    if Hqk == H:
        st = lib().loglinear_decode_step(*ptrs, S, H, dk, dv, Lcap, code, _stream(stream))
    else:
        st = lib().loglinear_decode_step_grouped(*ptrs, S, H, Hqk, dk, dv, Lcap, code, _stream(stream))
    for t in own:
        _keep_for_stream(t, stream)
    _check(st)
    return out


def gdn_fwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, chunk: int) -> int:
    return int(lib().loglinear_gdn_fwd_workspace_bytes(B, H, T, dk, dv, chunk))


def gdn_fwd(q, k, v, a, beta, lam, chunk: int = 64, out=None, workspace=None, stream=None):
    """Log-Linear Gated DeltaNet forward.  q, k [B,H,T,dk], v [B,H,T,dv]
    (float32 or bfloat16, same dtype; arithmetic in float32), a and beta
    [B,H,T] and lam [B,H,T,L] float32 with L = num_levels(T).  Returns out
    [B,H,T,dv] in the input dtype.  Asynchronous on ``stream``."""
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,T,dk] and v [B,H,T,dv]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T)
    if tuple(a.shape) != (B, H, T) or tuple(beta.shape) != (B, H, T) or tuple(lam.shape) != (B, H, T, L):
        raise ValueError(f"a and beta must be [B,H,T] and lam [B,H,T,{L}]")
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    own = []
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
        own.append(out)
    need = gdn_fwd_workspace_bytes(B, H, T, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    f32 = torch.float32
    st = lib().loglinear_gdn_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(a, "a", f32), _dev(beta, "beta", f32),
        _dev(lam, "lam", f32), _dev(out, "out", q.dtype), B, H, T, dk, dv, chunk, code, ws_ptr, ws_bytes,
        _stream(stream))
    for t in own:
        _keep_for_stream(t, stream)
    _check(st)
    return out


def profile_begin(max_launches: int = 4096) -> None:
    _check(lib().loglinear_profile_begin(max_launches))


def profile_end() -> dict:
    """Per-kernel {name: (launches, total_ms)} for launches since profile_begin."""
    arr = (KernelStat * 64)()
    n = ctypes.c_int(0)
    _check(lib().loglinear_profile_end(arr, 64, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}
