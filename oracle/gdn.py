"""fp64 oracle for Log-Linear Gated DeltaNet (forward).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the library never
imports or calls it.

What is computed.  The pages turn a linear-attention model into its
log-linear variant by multiplying the model's own attention matrix A
elementwise with the hierarchical mask: P = A ⊙ M_H, O = P V
("Log-Linear Attention", Portuguese page §2 "Metodologia", hierarchical-mask
point; French page §3 "Contributions Clés", the unified framework that
replaces a model's temporal mask), and name Gated DeltaNet as the second
model so treated (same sections).  They do not restate Gated DeltaNet, so
its recurrence is taken from its own publication (Yang, Kautz, Hatamizadeh,
"Gated Delta Networks", 2024):

    S_t = S_{t-1} M_t + beta_t v_t k_t^T,   M_t = alpha_t (I - beta_t k_t k_t^T),
    o_t = S_t q_t,                          S in R^{dv x dk}, alpha_t = exp(a_t).

Unrolled, o_t = sum_{s<=t} A[t,s] v_s with
    A[t,s] = beta_s k_s^T M_{s+1} M_{s+2} ... M_t q_t,
so the log-linear form reads
    o_t = sum_{s<=t} lambda_t[level(t,s)] A[t,s] v_s,
with the same Fenwick level(t,s) = bit length of t xor s as the Mamba-2
form.  With lambda = 1 it is Gated DeltaNet itself.

Two independent evaluations:
  ``gdn_fwd`` / ``gdn_fwd_rows``: the pairwise sum above, walking s from t
      down to 0 and applying one M per step to the query side;
  ``gdn_recurrent``: the recurrent form, one state per Fenwick level, every
      state right-multiplied by M_t at each step, the new token's
      beta_t v_t k_t^T in level 0, and the levels below the lowest set bit
      of t merged into the next one (the same carry rule as the decode of
      the Mamba-2 form).
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().to(dtype=__import__("torch").float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _levels(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """bit length of t xor s, elementwise (0 for s == t)."""
    x = np.bitwise_xor(t, s).astype(np.int64)
    out = np.zeros_like(x)
    while np.any(x > 0):
        nz = x > 0
        out[nz] += 1
        x = x >> 1
    return out


def _rows(q, k, v, a, beta, lam, bh_rows, t_rows):
    """Outputs of the selected (head, query) pairs, all at once: the query
    side y = M_{s+1} ... M_t q_t is built one key at a time, distance
    d = t - s = 0, 1, 2, ... (one M applied per step)."""
    n = len(t_rows)
    dv = v.shape[-1]
    out = np.zeros((n, dv))
    y = q[bh_rows, t_rows].copy()            # [n, dk], M-product empty at d = 0
    tmax = int(t_rows.max()) if n else -1
    for d in range(tmax + 1):
        act = t_rows >= d
        if not np.any(act):
            break
        ia = np.nonzero(act)[0]
        bh = bh_rows[ia]
        s = t_rows[ia] - d
        ks = k[bh, s]                         # [m, dk]
        dot = np.einsum("ij,ij->i", ks, y[ia])
        coef = beta[bh, s] * dot              # A[t, s]
        lv = _levels(t_rows[ia], s)
        w = lam[bh, t_rows[ia], lv] * coef
        out[ia] += w[:, None] * v[bh, s]
        # move the query side one key further back: y <- M_s y
        alpha = np.exp(a[bh, s])
        y[ia] = alpha[:, None] * (y[ia] - (beta[bh, s] * dot)[:, None] * ks)
    return out


def gdn_fwd(q, k, v, a, beta, lam) -> np.ndarray:
    """All rows.  q, k [B,H,T,dk], v [B,H,T,dv], a, beta [B,H,T],
    lam [B,H,T,L].  Returns fp64 [B,H,T,dv]."""
    q, k, v, a, beta, lam = (_f64(x) for x in (q, k, v, a, beta, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    BH = B * H
    rs = lambda x: x.reshape((BH,) + x.shape[2:])
    q, k, v, a, beta, lam = (rs(x) for x in (q, k, v, a, beta, lam))
    bh_rows = np.repeat(np.arange(BH), T)
    t_rows = np.tile(np.arange(T), BH)
    out = _rows(q, k, v, a, beta, lam, bh_rows, t_rows)
    return out.reshape(B, H, T, dv)


def gdn_fwd_rows(q, k, v, a, beta, lam, rows) -> np.ndarray:
    """Selected rows: ``rows`` int [n, 2] of (b*H + h, t).  Returns [n, dv]."""
    q, k, v, a, beta, lam = (_f64(x) for x in (q, k, v, a, beta, lam))
    B, H = q.shape[:2]
    BH = B * H
    rs = lambda x: x.reshape((BH,) + x.shape[2:])
    q, k, v, a, beta, lam = (rs(x) for x in (q, k, v, a, beta, lam))
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    return _rows(q, k, v, a, beta, lam, rows[:, 0], rows[:, 1])


def gdn_recurrent(q, k, v, a, beta, lam) -> np.ndarray:
    """The recurrent form over Fenwick level states (one (b, h) at a time,
    fp64).  Same arguments and result as ``gdn_fwd``."""
    q, k, v, a, beta, lam = (_f64(x) for x in (q, k, v, a, beta, lam))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            states = {}
            for t in range(T):
                kt, vt = k[b, h, t], v[b, h, t]
                Mt = np.exp(a[b, h, t]) * (np.eye(dk) - beta[b, h, t] * np.outer(kt, kt))
                if t > 0:
                    # levels 0 .. c of position t-1 merge into level c+1
                    c = (t & -t).bit_length() - 1
                    merged = np.zeros((dv, dk))
                    for l in [l for l in states if l <= c]:
                        merged += states.pop(l)
                    states[c + 1] = merged
                for l in states:
                    states[l] = states[l] @ Mt
                states[0] = beta[b, h, t] * np.outer(vt, kt)
                for l, S in states.items():
                    out[b, h, t] += lam[b, h, t, l] * (S @ q[b, h, t])
    return out


def gdn_serial(q, k, v, a, beta) -> np.ndarray:
    """Gated DeltaNet itself (one state, no levels), for the lambda = 1 pin."""
    q, k, v, a, beta = (_f64(x) for x in (q, k, v, a, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk))
            for t in range(T):
                kt = k[b, h, t]
                S = np.exp(a[b, h, t]) * (S - beta[b, h, t] * np.outer(S @ kt, kt)) \
                    + beta[b, h, t] * np.outer(v[b, h, t], kt)
                out[b, h, t] = S @ q[b, h, t]
    return out
