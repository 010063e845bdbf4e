"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments on the host with the
documented status codes before any device call."""

import ctypes
import os
import re

import pytest

import log_linear_attention_amd as ll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loglinear.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ll.LIB_PATH):
        from log_linear_attention_amd import build

        build.build(verbose=False)
    return ll.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(loglinear_\w+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("loglinear_fwd", "loglinear_decode_step", "loglinear_last_error",
                 "loglinear_num_levels", "loglinear_fwd_workspace_bytes"):
        assert must in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), f"{name} declared in loglinear.h but not exported"


def test_num_levels(L):
    assert [ll.num_levels(T) for T in (0, 1, 2, 3, 4, 5, 256, 257, 2048, 16384, 65536)] == \
        [1, 1, 2, 3, 3, 4, 9, 10, 12, 15, 17]
    assert L.loglinear_num_levels(-1) == -1


def test_workspace_bytes_is_deterministic_and_zero_when_unneeded(L):
    a = ll.fwd_workspace_bytes(1, 16, 16384, 128, 64, 64)
    b = ll.fwd_workspace_bytes(1, 16, 16384, 128, 64, 64)
    assert a == b and a > 0 and a % 256 == 0
    # a single chunk needs no inter-chunk state
    assert ll.fwd_workspace_bytes(1, 1, 64, 128, 64, 64) == 0
    assert ll.fwd_workspace_bytes(0, 16, 16384, 128, 64, 64) == 0
    # invalid shapes report 0
    assert ll.fwd_workspace_bytes(1, 1, 100, 128, 64, 48) == 0


FAKE = 1 << 20  # 16-byte aligned fake device address; never dereferenced on error paths


def _fwd(L, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, lam=FAKE + 0x400000,
                out=FAKE + 0x8000000, B=1, H=1, T=128, dk=128, dv=64, chunk=64, dtype=ll.LL_BF16,
                ws=None, wsb=0, stream=None, g=-1)
    args.update(kw)
    return L.loglinear_fwd_ex(args["q"], args["k"], args["v"], args["a"], args["lam"], args["out"],
                              args["B"], args["H"], args["T"], args["dk"], args["dv"], args["chunk"],
                              args["dtype"], args["ws"], args["wsb"], args["stream"], args["g"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), ll.LL_EINVAL),
    (dict(B=-1), ll.LL_EINVAL),
    (dict(T=-5), ll.LL_EINVAL),
    (dict(dk=0), ll.LL_EINVAL),
    (dict(chunk=48), ll.LL_EUNSUPPORTED),
    (dict(chunk=128), ll.LL_EUNSUPPORTED),
    (dict(dk=96), ll.LL_EUNSUPPORTED),
    (dict(dv=48), ll.LL_EUNSUPPORTED),
    (dict(dk=16), ll.LL_EUNSUPPORTED),           # bf16 needs dk >= 32
    (dict(dk=256, dtype=ll.LL_F32), ll.LL_EUNSUPPORTED),
    (dict(g=4), ll.LL_EUNSUPPORTED),
    (dict(q=None), ll.LL_EINVAL),
    (dict(out=None), ll.LL_EINVAL),
    (dict(q=FAKE + 8), ll.LL_EINVAL),            # misaligned
    (dict(a=FAKE + 0x300002), ll.LL_EINVAL),     # misaligned float vector
    (dict(lam=None), ll.LL_EINVAL),
    (dict(out=FAKE + 0x100), ll.LL_EINVAL),      # out overlaps q
    (dict(T=1000), ll.LL_EWORKSPACE),            # needs a workspace, none given
    (dict(T=1000, ws=FAKE + 0x10000000, wsb=16), ll.LL_EWORKSPACE),
])
def test_fwd_rejects_bad_arguments(L, kw, status):
    assert _fwd(L, **kw) == status
    assert ll.last_error() != ""


def test_fwd_misaligned_workspace(L):
    need = ll.fwd_workspace_bytes(1, 1, 1000, 128, 64, 64)
    assert _fwd(L, T=1000, ws=FAKE + 0x10000010, wsb=need) == ll.LL_EINVAL


def test_fwd_empty_problem_is_a_no_op(L):
    # zero sizes: valid, nothing launched, pointers not touched
    assert _fwd(L, B=0, q=None, k=None, v=None, out=None, a=None, lam=None) == ll.LL_OK
    assert _fwd(L, T=0, q=None, k=None, v=None, out=None, a=None, lam=None) == ll.LL_OK


def _dec(L, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, lam=FAKE + 0x400000,
                state=FAKE + 0x1000000, logscale=FAKE + 0x9000000, pos=FAKE + 0xa000000,
                out=FAKE + 0xb000000, S=2, H=2, dk=128, dv=64, Lcap=17, dtype=ll.LL_BF16, stream=None)
    args.update(kw)
    return L.loglinear_decode_step(args["q"], args["k"], args["v"], args["a"], args["lam"], args["state"],
                                   args["logscale"], args["pos"], args["out"], args["S"], args["H"], args["dk"],
                                   args["dv"], args["Lcap"], args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), ll.LL_EINVAL),
    (dict(S=-1), ll.LL_EINVAL),
    (dict(Lcap=0), ll.LL_EINVAL),
    (dict(Lcap=1), ll.LL_EUNSUPPORTED),
    (dict(Lcap=33), ll.LL_EUNSUPPORTED),
    (dict(dk=96), ll.LL_EUNSUPPORTED),
    (dict(dv=256), ll.LL_EUNSUPPORTED),
    (dict(state=None), ll.LL_EINVAL),
    (dict(pos=None), ll.LL_EINVAL),
    (dict(pos=FAKE + 0xa000004), ll.LL_EINVAL),
    (dict(state=FAKE + 4), ll.LL_EINVAL),
    (dict(out=FAKE + 0x1000000), ll.LL_EINVAL),  # out inside state
])
def test_decode_rejects_bad_arguments(L, kw, status):
    assert _dec(L, **kw) == status
    assert ll.last_error() != ""


def test_decode_empty_is_a_no_op(L):
    assert _dec(L, S=0, q=None, state=None) == ll.LL_OK


def test_profile_end_without_begin(L):
    n = ctypes.c_int(0)
    arr = (ll.KernelStat * 4)()
    assert L.loglinear_profile_end(arr, 4, ctypes.byref(n)) == ll.LL_EINVAL
    assert L.loglinear_profile_begin(0) == ll.LL_EINVAL


def _pre(L, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, lam=FAKE + 0x400000,
                out=FAKE + 0x8000000, state=FAKE + 0x10000000, logscale=FAKE + 0x20000000,
                B=1, H=1, T=64, dk=128, dv=64, chunk=64, Lcap=17, dtype=ll.LL_BF16,
                ws=None, wsb=0, stream=None, g=-1)
    args.update(kw)
    return L.loglinear_prefill(args["q"], args["k"], args["v"], args["a"], args["lam"], args["out"],
                               args["state"], args["logscale"], args["B"], args["H"], args["T"], args["dk"],
                               args["dv"], args["chunk"], args["Lcap"], args["dtype"], args["ws"], args["wsb"],
                               args["stream"], args["g"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), ll.LL_EINVAL),
    (dict(T=-1), ll.LL_EINVAL),
    (dict(chunk=8), ll.LL_EUNSUPPORTED),
    (dict(Lcap=0), ll.LL_EINVAL),
    (dict(Lcap=1), ll.LL_EUNSUPPORTED),
    (dict(Lcap=33), ll.LL_EUNSUPPORTED),
    (dict(T=129, Lcap=8), ll.LL_EINVAL),         # position 128 needs slot 8
    (dict(dk=256, dtype=ll.LL_F32), ll.LL_EUNSUPPORTED),
    (dict(state=None), ll.LL_EINVAL),
    (dict(logscale=None), ll.LL_EINVAL),
    (dict(state=FAKE + 0x10000004), ll.LL_EINVAL),  # misaligned
    (dict(logscale=FAKE + 0x20000002), ll.LL_EINVAL),
    (dict(state=FAKE + 0x100), ll.LL_EINVAL),        # state overlaps q
    (dict(logscale=FAKE + 0x8000000), ll.LL_EINVAL),  # logscale overlaps out
    (dict(logscale=FAKE + 0x10000100), ll.LL_EINVAL),  # logscale inside state
    (dict(T=1000), ll.LL_EWORKSPACE),
])
def test_prefill_rejects_bad_arguments(L, kw, status):
    assert _pre(L, **kw) == status
    assert ll.last_error().startswith("loglinear_prefill")


def test_prefill_lcap_fits_exactly(L):
    # After a prompt of T tokens decoding continues at position T, which the
    # decode step represents only when T < 2^(Lcap-1): Lcap >= 1 + bit_length(T).
    # B = 0, so nothing is launched and only validation runs.
    assert _pre(L, T=127, Lcap=8, B=0) == ll.LL_OK    # position 127 < 2^7
    assert _pre(L, T=128, Lcap=9, B=0) == ll.LL_OK    # position 128 < 2^8
    # num_levels(T) slots hold the stack of position T-1, but for a power of
    # two T the next position needs one more: the old minimum is rejected
    for T in (16, 128, 1024, 16384):
        assert _pre(L, T=T, Lcap=ll.num_levels(T), B=0) == ll.LL_EINVAL
        assert _pre(L, T=T, Lcap=ll.num_levels(T + 1), B=0) == ll.LL_OK
    assert _pre(L, T=128, Lcap=7, B=0) == ll.LL_EINVAL


def test_fwd_rejects_too_many_heads_before_any_launch(L):
    # B*H above 65535 is refused on the host (no launch is attempted, so the
    # fake pointers are never touched)
    need = ll.fwd_workspace_bytes(1, 70000, 1000, 128, 64, 64)
    assert _fwd(L, B=1, H=70000, T=1000, ws=FAKE + 0x10000000, wsb=max(need, 1 << 30)) == ll.LL_EUNSUPPORTED
    assert "65535" in ll.last_error()


def test_fwd_noalloc_checks_arguments_before_any_device_call(L):
    # 64 heads of 64K tokens need far more workspace than the library's
    # scratch: LL_EWORKSPACE, found on the host (fake pointers 4 GiB apart so
    # that no alias check fires first; nothing is launched)
    B, H, T, dk, dv = 1, 64, 65536, 128, 64
    assert ll.fwd_workspace_bytes(B, H, T, dk, dv, 64) > ll.FWD_NOALLOC_SCRATCH_BYTES
    p = [FAKE + i * (1 << 32) for i in range(6)]
    assert L.loglinear_fwd_noalloc(*p, B, H, T, dk, dv, 64, ll.LL_BF16, None) == ll.LL_EWORKSPACE
    assert "scratch" in ll.last_error()
    # argument errors come before the scratch lookup (which would need a GPU)
    assert L.loglinear_fwd_noalloc(None, *p[1:], B, H, 1000, dk, dv, 64, ll.LL_BF16, None) == ll.LL_EINVAL
    assert L.loglinear_fwd_noalloc(*p, B, H, 1000, dk, dv, 48, ll.LL_BF16, None) == ll.LL_EUNSUPPORTED
    assert L.loglinear_fwd_noalloc(*p, B, H, 1000, dk, dv, 64, 7, None) == ll.LL_EINVAL


@pytest.mark.parametrize("kw", [
    dict(state=FAKE),                    # state over q
    dict(state=FAKE + 0x100000),         # state over k
    dict(logscale=FAKE + 0x300000),      # logscale over a
    dict(logscale=FAKE + 0x400000),      # logscale over lambda
    dict(logscale=FAKE + 0xa000000),     # logscale over pos
    dict(out=FAKE + 0x300000),           # out over a
    dict(out=FAKE + 0x400000),           # out over lambda
    dict(out=FAKE + 0xa000000),          # out over pos
    dict(state=FAKE + 0x400000),         # state over lambda
    dict(state=FAKE + 0xa000000 - 0x100),  # state running into pos
])
def test_decode_rejects_every_output_alias(L, kw):
    assert _dec(L, **kw) == ll.LL_EINVAL
    assert "alias" in ll.last_error()


def test_prefill_empty_prompt_is_a_no_op(L):
    assert _pre(L, T=0, q=None, k=None, v=None, out=None, a=None, lam=None, state=None, logscale=None) == ll.LL_OK


def _bwd(L, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, lam=FAKE + 0x400000,
                do=FAKE + 0x500000, dq=FAKE + 0x1000000, dk=FAKE + 0x2000000, dv=FAKE + 0x3000000,
                da=FAKE + 0x4000000, dlam=FAKE + 0x5000000, B=1, H=1, T=64, dk_=128, dv_=64, chunk=64,
                dtype=ll.LL_BF16, ws=FAKE + 0x10000000, wsb=1 << 30, stream=None)
    args.update(kw)
    return L.loglinear_bwd(args["q"], args["k"], args["v"], args["a"], args["lam"], args["do"], args["dq"],
                           args["dk"], args["dv"], args["da"], args["dlam"], args["B"], args["H"], args["T"],
                           args["dk_"], args["dv_"], args["chunk"], args["dtype"], args["ws"], args["wsb"],
                           args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=9), ll.LL_EINVAL),
    (dict(T=-2), ll.LL_EINVAL),
    (dict(chunk=16), ll.LL_EUNSUPPORTED),
    (dict(dk_=16), ll.LL_EUNSUPPORTED),
    (dict(dv_=96), ll.LL_EUNSUPPORTED),
    (dict(dtype=ll.LL_F32, chunk=64, dk_=128, dv_=128), ll.LL_EUNSUPPORTED),   # fp32 chunk 64 does not fit LDS
    (dict(B=70000), ll.LL_EUNSUPPORTED),
    (dict(q=None), ll.LL_EINVAL),
    (dict(do=None), ll.LL_EINVAL),
    (dict(dq=None), ll.LL_EINVAL),
    (dict(da=None), ll.LL_EINVAL),
    (dict(dk=FAKE + 0x2000008), ll.LL_EINVAL),       # misaligned
    (dict(dlam=FAKE + 0x5000002), ll.LL_EINVAL),
    (dict(dq=FAKE + 0x100), ll.LL_EINVAL),           # dq overlaps q
    (dict(dv=FAKE + 0x2000000), ll.LL_EINVAL),       # dv overlaps dk
    (dict(ws=None), ll.LL_EWORKSPACE),
    (dict(wsb=16), ll.LL_EWORKSPACE),
    (dict(ws=FAKE + 0x10000010), ll.LL_EINVAL),      # misaligned workspace
])
def test_bwd_rejects_bad_arguments(L, kw, status):
    assert _bwd(L, **kw) == status
    assert ll.last_error().startswith("loglinear_bwd")


def test_bwd_workspace_and_empty(L):
    n = ll.bwd_workspace_bytes(1, 16, 16384, 128, 64, 64)
    assert n > 0 and n % 256 == 0 and n == ll.bwd_workspace_bytes(1, 16, 16384, 128, 64, 64)
    assert ll.bwd_workspace_bytes(0, 16, 16384, 128, 64, 64) == 0
    assert _bwd(L, T=0, q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None, da=None, dlam=None,
                ws=None, wsb=0) == ll.LL_OK


# --- q/k shared across heads ---------------------------------------------------

def _fwd_g(L, **kw):
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, lam=FAKE + 0x400000,
                out=FAKE + 0x8000000, B=1, H=4, Hqk=2, T=64, dk=128, dv=64, chunk=64, dtype=ll.LL_BF16,
                ws=None, wsb=0, stream=None, g=-1)
    args.update(kw)
    return L.loglinear_fwd_grouped(args["q"], args["k"], args["v"], args["a"], args["lam"], args["out"],
                                   args["B"], args["H"], args["Hqk"], args["T"], args["dk"], args["dv"],
                                   args["chunk"], args["dtype"], args["ws"], args["wsb"], args["stream"], args["g"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hqk=3), ll.LL_EINVAL),                 # 4 heads cannot share 3 q/k heads
    (dict(Hqk=0), ll.LL_EINVAL),
    (dict(Hqk=-2), ll.LL_EINVAL),
    (dict(Hqk=8), ll.LL_EINVAL),                 # more q/k heads than heads
    (dict(q=None), ll.LL_EINVAL),
    (dict(out=FAKE + 0x7ff0), ll.LL_EINVAL),     # out overlaps the end of q (2 q/k heads: 32 KiB)
    (dict(chunk=48), ll.LL_EUNSUPPORTED),
])
def test_fwd_grouped_rejects_bad_arguments(L, kw, status):
    assert _fwd_g(L, **kw) == status
    assert ll.last_error().startswith("loglinear_fwd_grouped")


def test_fwd_grouped_q_size_follows_qk_heads(L):
    # q of 2 heads x 64 tokens x 128 bf16 = 32 KiB: an out placed right after it is legal on the host side
    # (the call fails only later, at the launch, which is not reached without a GPU: the workspace check
    # comes first and T=1000 needs one)
    assert _fwd_g(L, T=1000, out=FAKE + 2 * 1000 * 128 * 2) == ll.LL_EWORKSPACE
    assert _fwd_g(L, T=1000, out=FAKE + 2 * 1000 * 128 * 2 - 16) == ll.LL_EINVAL


def test_decode_grouped_rejects_bad_heads(L):
    st = L.loglinear_decode_step_grouped(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                         FAKE + 0x1000000, FAKE + 0x9000000, FAKE + 0xa000000, FAKE + 0xb000000,
                                         2, 6, 4, 128, 64, 17, ll.LL_BF16, None)
    assert st == ll.LL_EINVAL
    assert "Hqk" in ll.last_error()
    # no heads: nothing to do
    assert L.loglinear_decode_step_grouped(None, None, None, None, None, None, None, None, None,
                                           2, 0, 1, 128, 64, 17, ll.LL_BF16, None) == ll.LL_OK


def test_prefill_grouped_rejects_bad_heads(L):
    st = L.loglinear_prefill_grouped(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                     FAKE + 0x8000000, FAKE + 0x9000000, FAKE + 0xa000000, 1, 4, 3, 64, 128, 64,
                                     64, 17, ll.LL_BF16, None, 0, None, -1)
    assert st == ll.LL_EINVAL
    assert ll.last_error().startswith("loglinear_prefill_grouped")


def test_bwd_grouped_workspace_and_heads(L):
    per_head = ll.bwd_workspace_bytes(1, 16, 4096, 128, 64, 64)
    shared = ll.bwd_workspace_bytes(1, 16, 4096, 128, 64, 64, Hqk=2)
    # the shared form adds per-head copies of q, k and of their gradients
    assert shared > per_head and shared % 256 == 0
    assert ll.bwd_workspace_bytes(1, 16, 4096, 128, 64, 64, Hqk=16) == per_head
    assert L.loglinear_bwd_grouped_workspace_bytes(1, 16, 3, 4096, 128, 64, 64) == 0
    st = L.loglinear_bwd_grouped(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                 FAKE + 0x500000, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                                 FAKE + 0x4000000, FAKE + 0x5000000, 1, 4, 3, 64, 128, 64, 64, ll.LL_BF16,
                                 FAKE + 0x10000000, 1 << 30, None)
    assert st == ll.LL_EINVAL
    assert ll.last_error().startswith("loglinear_bwd_grouped")


def test_prefill_varlen_needs_lens(L):
    args = (FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x8000000,
            FAKE + 0x9000000, FAKE + 0xa000000)
    st = L.loglinear_prefill_varlen(*args, None, 2, 2, 2, 64, 128, 64, 64, 17, ll.LL_BF16, None, 0, None, -1)
    assert st == ll.LL_EINVAL and "lens" in ll.last_error()
    st = L.loglinear_prefill_varlen(*args, FAKE + 0xb000002, 2, 2, 2, 64, 128, 64, 64, 17, ll.LL_BF16, None, 0,
                                    None, -1)
    assert st == ll.LL_EINVAL and "lens" in ll.last_error()
    # an empty batch needs nothing
    assert L.loglinear_prefill_varlen(*args, None, 0, 2, 2, 64, 128, 64, 64, 17, ll.LL_BF16, None, 0, None,
                                      -1) == ll.LL_OK


def test_gdn_rejects_bad_arguments(L):
    def call(**kw):
        args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, a=FAKE + 0x300000, beta=FAKE + 0x380000,
                    lam=FAKE + 0x400000, out=FAKE + 0x8000000, B=1, H=2, T=64, dk=128, dv=64, chunk=64,
                    dtype=ll.LL_F32, ws=FAKE + 0x10000000, wsb=1 << 30, stream=None)
        args.update(kw)
        return L.loglinear_gdn_fwd(args["q"], args["k"], args["v"], args["a"], args["beta"], args["lam"],
                                   args["out"], args["B"], args["H"], args["T"], args["dk"], args["dv"],
                                   args["chunk"], args["dtype"], args["ws"], args["wsb"], args["stream"])

    assert call(dtype=7) == ll.LL_EINVAL
    assert call(q=FAKE + 4) == ll.LL_EINVAL                         # q is read four elements at a time
    assert call(chunk=16) == ll.LL_EUNSUPPORTED
    assert call(dk=16) == ll.LL_EUNSUPPORTED
    assert call(beta=None) == ll.LL_EINVAL
    assert call(ws=None) == ll.LL_EWORKSPACE
    assert call(wsb=64) == ll.LL_EWORKSPACE
    assert call(out=FAKE + 0x100) == ll.LL_EINVAL                  # out overlaps q
    assert call(T=0, q=None, k=None, v=None, a=None, beta=None, lam=None, out=None, ws=None, wsb=0) == ll.LL_OK
    assert ll.last_error().startswith("loglinear_gdn_fwd") or ll.last_error() == ""
    n = ll.gdn_fwd_workspace_bytes(1, 16, 16384, 128, 64, 64)
    assert n > 0 and n % 256 == 0
    assert ll.gdn_fwd_workspace_bytes(1, 16, 16384, 128, 64, 16) == 0


# ---- the shape support matrix, checked exhaustively on the host --------------
# Every dk, dv that is a multiple of 16 up to 256, both dtypes, every chunk:
# with an empty batch (B = 0, or S = 0 for decode) nothing is launched, and the
# call returns LL_OK exactly for the shapes the header lists as supported and
# LL_EUNSUPPORTED for every other one.
DIMS = list(range(16, 257, 16))
P4 = {16, 32, 64, 128}


def _fwd_ok(dtype, dk, dv, chunk):
    if dtype == ll.LL_F32:
        return dk in P4 and dv in P4
    return dk in {32, 64, 128} and dv in P4


@pytest.mark.parametrize("dtype", [ll.LL_F32, ll.LL_BF16])
def test_forward_support_matrix(L, dtype):
    for chunk in (16, 32, 64):
        for dk in DIMS:
            for dv in DIMS:
                st = _fwd(L, B=0, q=None, k=None, v=None, out=None, a=None, lam=None, dk=dk, dv=dv, chunk=chunk,
                          dtype=dtype)
                want = ll.LL_OK if _fwd_ok(dtype, dk, dv, chunk) else ll.LL_EUNSUPPORTED
                assert st == want, (dtype, dk, dv, chunk, st, ll.last_error())


@pytest.mark.parametrize("dtype", [ll.LL_F32, ll.LL_BF16])
def test_decode_support_matrix(L, dtype):
    for dk in DIMS:
        for dv in DIMS:
            st = _dec(L, S=0, q=None, k=None, v=None, a=None, lam=None, state=None, logscale=None, pos=None,
                      out=None, dk=dk, dv=dv, dtype=dtype)
            want = ll.LL_OK if dk in P4 and dv in P4 else ll.LL_EUNSUPPORTED
            assert st == want, (dtype, dk, dv, st, ll.last_error())


def _bwd_ok(dtype, dk, dv, chunk):
    if dk not in {32, 64, 128} or dv not in {32, 64, 128}:
        return False
    if dtype == ll.LL_BF16:
        return chunk in (32, 64)
    return chunk == 32 or (chunk == 64 and dk == dv == 32)


@pytest.mark.parametrize("dtype", [ll.LL_F32, ll.LL_BF16])
def test_backward_support_matrix(L, dtype):
    for chunk in (16, 32, 64):
        for dk in DIMS:
            for dv in DIMS:
                st = _bwd(L, B=0, q=None, k=None, v=None, a=None, lam=None, do=None, dq=None, dk=None, dv=None,
                          da=None, dlam=None, ws=None, wsb=0, dk_=dk, dv_=dv, chunk=chunk, dtype=dtype)
                want = ll.LL_OK if _bwd_ok(dtype, dk, dv, chunk) else ll.LL_EUNSUPPORTED
                assert st == want, (dtype, dk, dv, chunk, st, ll.last_error())


@pytest.mark.parametrize("dtype", [ll.LL_F32, ll.LL_BF16])
def test_gdn_support_matrix(L, dtype):
    for chunk in (16, 32, 64):
        for dk in DIMS:
            for dv in DIMS:
                st = L.loglinear_gdn_fwd(None, None, None, None, None, None, None, 0, 1, 64, dk, dv, chunk, dtype,
                                         None, 0, None)
                ok = dk in {32, 64, 128} and dv in {32, 64, 128} and chunk in (32, 64)
                assert st == (ll.LL_OK if ok else ll.LL_EUNSUPPORTED), (dtype, dk, dv, chunk, st, ll.last_error())


@pytest.mark.parametrize("dtype", [ll.LL_F32, ll.LL_BF16])
def test_prefill_support_matrix(L, dtype):
    for dk in DIMS:
        for dv in DIMS:
            st = _pre(L, B=0, q=None, k=None, v=None, out=None, a=None, lam=None, state=None, logscale=None,
                      dk=dk, dv=dv, dtype=dtype)
            want = ll.LL_OK if _fwd_ok(dtype, dk, dv, 64) else ll.LL_EUNSUPPORTED
            assert st == want, (dtype, dk, dv, st, ll.last_error())
