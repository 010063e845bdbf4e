"""fp64 oracle for log-linear attention (Mamba-2 form): forward and decode.

TEST INFRASTRUCTURE ONLY.  The library never imports, links or calls this
package; only ``tests/``, the smoke check and the benchmark's CPU baseline do.
It shares no code with the HIP path.

Sources, cited by page title, language and section:
  [LLA-pt] "Log-Linear Attention" summary page, Portuguese
           (gist.science/pt/paper/2506.04761).
  [LLA-fr] "Log-Linear Attention" summary page, French
           (gist.science/fr/paper/2506.04761).

Forward (``fwd``, ``fwd_rows``): the plain O(T^2) evaluation, in C
(``ll_oracle.c``), of
    o[t] = sum_{s<=t} exp(sum_{r=s+1..t} a_r) * lambda_t[level(t,s)] * (q_t.k_s) v_s,
i.e. O = (Q K^T ⊙ M_H) V with the hierarchical mask [LLA-fr §2 "Matrice de
Masque Hiérarchique"] composed with Mamba-2's decay, with Fenwick buckets of
sizes 1, 2, 4, 8, ... [LLA-pt §2 "Particionamento Hierárquico"] and per-level
weights lambda_t^(l) [LLA-fr §2].

Decode (``decode_step``, ``decode_sequence``): the recurrent form — O(log T)
states; the new token fills the finest level and the levels below the lowest
zero bit of the previous position merge into the next one, as a Fenwick tree
carries [LLA-pt §2 "Forma Recorrente e Paralela", decoding bullet; LLA-fr §2
"Algorithmes Efficaces", inference bullet].  Written from that description
in numpy fp64, one (sequence, head) at a time.

Backward (``bwd``, ``bwd_rows``): the gradients of sum(do * o) with respect
to q, k, v, a and lambda, each differentiated term by term from the forward
definition and evaluated plainly in C (``ll_oracle.c``, backward section).

Prefill (``prefill_stack``): the stack that a whole prompt leaves for the
decode of the next token, summed bucket by bucket from the same definition
the forward uses.

Log-Linear Gated DeltaNet: ``oracle/gdn.py`` (its own module; numpy fp64).

Shared q/k heads (``expand_heads``, ``fwd_grouped``, ``bwd_grouped``): each
head reads its q/k head; the gradient of a shared entry sums over the heads
that read it.

Stack convention for decode: slot l holds the state of level-l bucket of the
most recent query position.  Occupancy follows the position's bits: for
position p, slot 0 is always occupied and slot l >= 1 is occupied iff bit
l-1 of p is set.  A stored pair (hat S_l, g_l) means the true state
exp(g_l) * hat S_l.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ll_oracle.c")
# ORACLE_LIB names another build of the same C source (the host-sanitizer
# build of the CPU tests); by default the in-tree build is loaded.
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "libll_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  No fast-math."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.ll_oracle_level.argtypes = [I, I]
        lib.ll_oracle_level.restype = ctypes.c_int
        lib.ll_oracle_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
        lib.ll_oracle_fwd.restype = ctypes.c_int
        lib.ll_oracle_fwd_rows.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P]
        lib.ll_oracle_fwd_rows.restype = ctypes.c_int
        lib.ll_oracle_bwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P, P]
        lib.ll_oracle_bwd.restype = ctypes.c_int
        lib.ll_oracle_bwd_qrows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P, P]
        lib.ll_oracle_bwd_qrows.restype = ctypes.c_int
        lib.ll_oracle_bwd_krows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P, P]
        lib.ll_oracle_bwd_krows.restype = ctypes.c_int
        lib.ll_oracle_da_window.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, I, P]
        lib.ll_oracle_da_window.restype = ctypes.c_int
        lib.ll_oracle_num_threads.argtypes = []
        lib.ll_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def level(t: int, s: int) -> int:
    """Fenwick level of key s seen from query t (the C oracle's function)."""
    return int(_load().ll_oracle_level(int(t), int(s)))


def num_threads() -> int:
    return int(_load().ll_oracle_num_threads())


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().to(dtype=__import__("torch").float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, a, lam) -> np.ndarray:
    """All rows.  q,k [B,H,T,dk], v [B,H,T,dv], a [B,H,T], lam [B,H,T,L]
    (any float dtype; upcast exactly to fp64).  Returns fp64 [B,H,T,dv]."""
    q, k, v, a, lam = (_f64(x) for x in (q, k, v, a, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    rc = _load().ll_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam),
                               B * H, T, dk, dv, L, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle fwd failed (code {rc}): lambda narrower than the levels used?")
    return out


def fwd_rows(q, k, v, a, lam, rows) -> np.ndarray:
    """Selected rows: ``rows`` is int [n, 2] of (b*H + h, t).  Returns [n, dv]."""
    q, k, v, a, lam = (_f64(x) for x in (q, k, v, a, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    out = np.zeros((rows.shape[0], dv), dtype=np.float64)
    rc = _load().ll_oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam),
                                    B * H, T, dk, dv, L, rows.shape[0], _ptr(rows), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle fwd_rows failed (code {rc})")
    return out


# ---------------------------------------------------------------------------
# Backward: gradients of the forward definition.
# ---------------------------------------------------------------------------

def bwd(q, k, v, a, lam, do):
    """Gradients of sum(do * fwd(q, k, v, a, lam)) with respect to every
    input, by the term-by-term derivative of the definition (C, fp64,
    O(T^2)).  Returns dict(dq, dk, dv, da, dlam) shaped like the inputs;
    da[..., 0] is 0 because a_0 never enters."""
    q, k, v, a, lam, do = (_f64(x) for x in (q, k, v, a, lam, do))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "da": np.zeros_like(a), "dlam": np.zeros_like(lam)}
    rc = _load().ll_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam), _ptr(do), B * H, T, dk, dv, L,
                               _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["da"]),
                               _ptr(out["dlam"]))
    if rc != 0:
        raise ValueError(f"oracle bwd failed (code {rc})")
    return out


def bwd_rows(q, k, v, a, lam, do, qrows, krows):
    """Selected rows of the gradients: ``qrows`` [n, 2] of (b*H + h, t) for
    dq [n, dk] and dlam [n, L]; ``krows`` [m, 2] of (b*H + h, s) for
    dk [m, dk] and dv [m, dv]."""
    q, k, v, a, lam, do = (_f64(x) for x in (q, k, v, a, lam, do))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    qrows = np.ascontiguousarray(np.asarray(qrows, dtype=np.int64).reshape(-1, 2))
    krows = np.ascontiguousarray(np.asarray(krows, dtype=np.int64).reshape(-1, 2))
    dq = np.zeros((qrows.shape[0], dk)); dlam = np.zeros((qrows.shape[0], L))
    dkk = np.zeros((krows.shape[0], dk)); dvv = np.zeros((krows.shape[0], dv))
    lib = _load()
    rc = lib.ll_oracle_bwd_qrows(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam), _ptr(do), B * H, T, dk, dv, L,
                                 qrows.shape[0], _ptr(qrows), _ptr(dq), _ptr(dlam))
    rc = rc or lib.ll_oracle_bwd_krows(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam), _ptr(do), B * H, T, dk, dv,
                                       L, krows.shape[0], _ptr(krows), _ptr(dkk), _ptr(dvv))
    if rc != 0:
        raise ValueError(f"oracle bwd_rows failed (code {rc})")
    return {"dq": dq, "dlam": dlam, "dk": dkk, "dv": dvv}


def da_window(q, k, v, a, lam, do, rows, W: int) -> np.ndarray:
    """da at selected (b*H + h, r) rows (r >= 1) from the pairs s < r <= t
    with both ends within W tokens of r (exact when W >= T)."""
    q, k, v, a, lam, do = (_f64(x) for x in (q, k, v, a, lam, do))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    out = np.zeros(rows.shape[0])
    rc = _load().ll_oracle_da_window(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(lam), _ptr(do), B * H, T, dk, dv, L,
                                     rows.shape[0], _ptr(rows), int(W), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle da_window failed (code {rc})")
    return out


# ---------------------------------------------------------------------------
# q and k shared across heads (Mamba-2's groups; the pages build on Mamba-2,
# [LLA-pt §2 "Metodologia", generalisation point], and leave open whether q
# and k are per head).  Head h of H reads q/k head h // (H // Hqk).
# ---------------------------------------------------------------------------

def expand_heads(x, H: int) -> np.ndarray:
    """x [B, Hqk, ...] -> [B, H, ...] with head h taken from x head
    h // (H // Hqk) (each q/k head repeated for its consecutive heads)."""
    x = _f64(x)
    Hqk = x.shape[1]
    if Hqk <= 0 or H % Hqk != 0:
        raise ValueError(f"H={H} is not a multiple of Hqk={Hqk}")
    return np.repeat(x, H // Hqk, axis=1)


def fwd_grouped(q, k, v, a, lam) -> np.ndarray:
    """Forward with q, k [B,Hqk,T,dk] shared by the heads of v [B,H,T,dv]:
    the per-head definition applied to each head's q/k head."""
    H = v.shape[1]
    return fwd(expand_heads(q, H), expand_heads(k, H), v, a, lam)


def bwd_grouped(q, k, v, a, lam, do):
    """Gradients of sum(do * fwd_grouped(q, k, v, a, lam)).  A shared q or k
    entry enters the output of every head that reads it, so its gradient is
    the sum of those heads' per-head gradients (chain rule through the
    repetition); dv, da and dlam are per head."""
    H = v.shape[1]
    B, Hqk, T, dk = q.shape
    g = bwd(expand_heads(q, H), expand_heads(k, H), v, a, lam, do)
    for n in ("dq", "dk"):
        g[n] = g[n].reshape(B, Hqk, H // Hqk, T, dk).sum(axis=2)
    return g


# ---------------------------------------------------------------------------
# Decode: the recurrent form, one token per (sequence, head) per step.
# ---------------------------------------------------------------------------

def occupied(p: int, Lcap: int) -> list[int]:
    """Slots holding a bucket for query position p (p >= 0)."""
    return [0] + [l for l in range(1, Lcap) if (p >> (l - 1)) & 1]


def _trailing_zeros(x: int) -> int:
    n = 0
    while x % 2 == 0:
        x //= 2
        n += 1
    return n


def decode_step(state, logscale, pos, q, k, v, a, lam):
    """One decode step for every (sequence, head), fp64.

    state [S,H,Lcap,dk,dv] (stored hat S), logscale [S,H,Lcap] (g), pos [S]
    (0-indexed position t of the new token), q,k [S,H,dk], v [S,H,dv], a [S,H],
    lam [S,H,Lcap].

    Returns (o [S,H,dv], new_true_state [S,H,Lcap,dk,dv], occ [S,Lcap] bool):
    the stack after the step, materialised as true states (exp(g) * hat S),
    with unoccupied slots set to zero.  A position outside [0, 2^(Lcap-1))
    yields NaN output and the incoming stack unchanged (materialised).
    """
    state, logscale, q, k, v, a, lam = (_f64(x) for x in (state, logscale, q, k, v, a, lam))
    pos = np.asarray(pos.detach().cpu().numpy() if hasattr(pos, "detach") else pos, dtype=np.int64)
    S, H, Lcap, dk, dv = state.shape
    o = np.zeros((S, H, dv))
    new = np.zeros_like(state)
    occ = np.zeros((S, Lcap), dtype=bool)
    for s in range(S):
        t = int(pos[s])
        if t < 0 or t >= (1 << (Lcap - 1)):
            o[s] = np.nan
            if t >= 1:  # report the untouched incoming stack
                for l in occupied(t - 1, Lcap):
                    new[s, :, l] = np.exp(logscale[s, :, l])[:, None, None] * state[s, :, l]
            continue
        for h in range(H):
            fresh = np.outer(k[s, h], v[s, h])  # level 0: the token itself
            stack = {}
            if t == 0:
                stack[0] = fresh
            else:
                prev = {l: np.exp(logscale[s, h, l]) * state[s, h, l] for l in occupied(t - 1, Lcap)}
                carry = _trailing_zeros(t)  # levels 0..carry of t-1 merge into carry+1
                decay = np.exp(a[s, h])
                merged = np.zeros((dk, dv))
                for l, st in prev.items():
                    if l <= carry:
                        merged += st
                    else:
                        stack[l] = decay * st
                stack[carry + 1] = decay * merged
                stack[0] = fresh
            assert sorted(stack) == occupied(t, Lcap)
            for l, st in stack.items():
                o[s, h] += lam[s, h, l] * (q[s, h] @ st)
                new[s, h, l] = st
        for l in occupied(t, Lcap):
            occ[s, l] = True
    return o, new, occ


def decode_sequence(q, k, v, a, lam, Lcap: int | None = None) -> np.ndarray:
    """Run the recurrence from an empty stack over a whole sequence.

    q,k [B,H,T,dk], v [B,H,T,dv], a [B,H,T], lam [B,H,T,L].  Returns the
    outputs [B,H,T,dv] (fp64).  Treats each (b, h) as one decode 'sequence'.
    """
    q, k, v, a, lam = (_f64(x) for x in (q, k, v, a, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    Lcap = max(L, 2) if Lcap is None else Lcap
    BH = B * H
    qs, ks, vs = q.reshape(BH, 1, T, dk), k.reshape(BH, 1, T, dk), v.reshape(BH, 1, T, dv)
    As, lams = a.reshape(BH, 1, T), lam.reshape(BH, 1, T, L)
    state = np.zeros((BH, 1, Lcap, dk, dv))
    logscale = np.zeros((BH, 1, Lcap))
    out = np.zeros((BH, 1, T, dv))
    lam_pad = np.zeros((BH, 1, T, Lcap))
    lam_pad[..., :L] = lams
    for t in range(T):
        pos = np.full(BH, t, dtype=np.int64)
        o, new, _ = decode_step(state, logscale, pos, qs[:, :, t], ks[:, :, t], vs[:, :, t],
                                As[:, :, t], lam_pad[:, :, t])
        out[:, :, t] = o
        state = new
    return out.reshape(B, H, T, dv)


def prefill_stack(k, v, a, Lcap: int):
    """The decode stack a prompt of T tokens leaves for the next token, fp64.

    The prompt's last token sits at position p = T - 1.  Slot l holds the true
    state of that position's level-l bucket, straight from the definition of
    the buckets: every key s <= p lands in slot level(p, s) with the weight
    exp(sum_{r=s+1..p} a_r) it carries in the forward [LLA-fr §2 "Matrice de
    Masque Hiérarchique"; LLA-pt §2 "Particionamento Hierárquico"], so
    sum_l lambda_p[l] q_p^T S_l is row p of the forward.

    k [B,H,T,dk], v [B,H,T,dv], a [B,H,T].  Returns (true_state
    [B,H,Lcap,dk,dv] with unoccupied slots zero, occ [Lcap] bool).
    """
    k, v, a = (_f64(x) for x in (k, v, a))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    state = np.zeros((B, H, Lcap, dk, dv))
    occ = np.zeros(Lcap, dtype=bool)
    if T == 0:
        return state, occ
    p = T - 1
    # log-weight of key s: sum of a over (s, p]
    logw = np.zeros((B, H, T))
    for s in range(p - 1, -1, -1):
        logw[:, :, s] = logw[:, :, s + 1] + a[:, :, s + 1]
    lev = np.array([level(p, s) for s in range(T)])
    if lev.max() >= Lcap:
        raise ValueError(f"position {p} needs {lev.max() + 1} slots, Lcap is {Lcap}")
    for l in range(Lcap):
        sel = np.nonzero(lev == l)[0]
        if sel.size == 0:
            continue
        occ[l] = True
        kw = k[:, :, sel, :] * np.exp(logw[:, :, sel])[..., None]
        state[:, :, l] = np.swapaxes(kw, -1, -2) @ v[:, :, sel, :]
    return state, occ


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 in fp64."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((x - ref) ** 2))
    return float(num / den) if den > 0 else float(num)
