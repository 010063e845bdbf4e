"""Pins for the fp64 oracle, each against something other than the oracle's
own formula: the bucket structure the pages describe, a hand-worked example,
textbook recurrences and matrix products, and the recurrent (decode) form.

Pages: "Log-Linear Attention" summaries (pt and fr, gist.science 2506.04761).
"""

import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_inputs(rng, B, H, T, dk, dv, L, a_scale=0.3):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    a = -np.abs(rng.standard_normal((B, H, T))) * a_scale
    lam = rng.random((B, H, T, L))
    return q, k, v, a, lam


def _L(T):
    return 1 if T <= 1 else 1 + (T - 1).bit_length()


# --- level function: the Fenwick buckets (pt §2 "Particionamento Hierárquico",
# fr §2 "Partitionnement par Arbre de Fenwick"): sizes 1, 2, 4, 8, ...; recent
# tokens in small buckets; O(log T) buckets per position. ----------------------

def test_level_buckets_partition_prefix(oracle_mod):
    for t in range(0, 300):
        buckets = {}
        for s in range(t + 1):
            buckets.setdefault(oracle_mod.level(t, s), []).append(s)
        assert buckets[0] == [t]
        covered = []
        # walk from the finest (rightmost) bucket to the coarsest
        right_edge = t  # exclusive upper end for the next-coarser bucket
        for lev in sorted(buckets):
            members = buckets[lev]
            assert members == list(range(members[0], members[-1] + 1)), "bucket not contiguous"
            if lev == 0:
                continue
            assert (t >> (lev - 1)) & 1 == 1, "non-empty bucket on a clear bit"
            assert len(members) == 2 ** (lev - 1), "bucket size is not 2^(l-1)"
            assert members[-1] == right_edge - 1, "buckets not ordered finer-to-the-right"
            right_edge = members[0]
            covered += members
        assert right_edge == 0 or t == 0
        assert sorted(covered + [t]) == list(range(t + 1))
        # number of non-empty buckets = 1 + popcount(t) <= 1 + ceil(log2(t+1))
        assert len(buckets) == 1 + bin(t).count("1")


def test_level_hand_examples(oracle_mod):
    lv = oracle_mod.level
    # t = 3: {3} level 0, {2} level 1, {0,1} level 2
    assert [lv(3, s) for s in range(4)] == [2, 2, 1, 0]
    # t = 6: {6} level 0, level 1 empty, {4,5} level 2, {0..3} level 3
    assert [lv(6, s) for s in range(7)] == [3, 3, 3, 3, 2, 2, 0]
    # large positions: top level is the bit length of t XOR s
    assert lv(1 << 20, 0) == 21
    assert lv((1 << 20) + 5, (1 << 20) + 4) == 1


# --- hand-worked example ------------------------------------------------------

def test_hand_example_forward(oracle_mod):
    g = json.load(open(os.path.join(HERE, "golden", "hand_T4.json")))
    T = 4
    q = np.array(g["q"]).reshape(1, 1, T, 1)
    k = np.array(g["k"]).reshape(1, 1, T, 1)
    v = np.array(g["v"]).reshape(1, 1, T, 2)
    a = np.array(g["a"]).reshape(1, 1, T)
    lam = np.array(g["lam"]).reshape(1, 1, T, 3)
    o = oracle_mod.fwd(q, k, v, a, lam)[0, 0]
    np.testing.assert_allclose(o, np.array(g["expected_o"]), rtol=1e-13, atol=1e-13)
    # the recurrent form gives the same rows
    o2 = oracle_mod.decode_sequence(q, k, v, a, lam)[0, 0]
    np.testing.assert_allclose(o2, np.array(g["expected_o"]), rtol=1e-13, atol=1e-13)


def test_hand_example_decode_stack(oracle_mod):
    g = json.load(open(os.path.join(HERE, "golden", "hand_T4.json")))
    T, Lcap = 4, 3
    q = np.array(g["q"]).reshape(T, 1)
    k = np.array(g["k"]).reshape(T, 1)
    v = np.array(g["v"]).reshape(T, 2)
    a = np.array(g["a"])
    lam = np.array(g["lam"])
    state = np.zeros((1, 1, Lcap, 1, 2))
    logscale = np.zeros((1, 1, Lcap))
    for t in range(T):
        o, state, occ = oracle_mod.decode_step(
            state, logscale, np.array([t]), q[t].reshape(1, 1, 1), k[t].reshape(1, 1, 1),
            v[t].reshape(1, 1, 2), a[t].reshape(1, 1), lam[t].reshape(1, 1, Lcap))
        np.testing.assert_allclose(o[0, 0], g["expected_o"][t], rtol=1e-13, atol=1e-13)
    assert occ[0].tolist() == [True, True, True]
    for slot, want in g["expected_stack_after_t3"].items():
        np.testing.assert_allclose(state[0, 0, int(slot)], np.array(want), rtol=1e-13, atol=1e-15)


# --- reductions to textbook operators -----------------------------------------

def test_lambda_one_is_mamba2_recurrence(oracle_mod):
    """lambda == 1 removes the hierarchy: decayed linear attention, whose
    scalar recurrence is S_t = exp(a_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t."""
    rng = np.random.default_rng(1)
    B, H, T, dk, dv = 1, 2, 45, 5, 3
    q, k, v, a, _ = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    lam = np.ones((B, H, T, _L(T)))
    o = oracle_mod.fwd(q, k, v, a, lam)
    ref = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                S = np.exp(a[b, h, t]) * S + np.outer(k[b, h, t], v[b, h, t])
                ref[b, h, t] = q[b, h, t] @ S
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-11)


def test_lambda_onehot_level0_is_diagonal(oracle_mod):
    rng = np.random.default_rng(2)
    B, H, T, dk, dv = 1, 1, 33, 4, 6
    q, k, v, a, _ = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    lam = np.zeros((B, H, T, _L(T)))
    lam[..., 0] = 1.0
    o = oracle_mod.fwd(q, k, v, a, lam)
    ref = np.sum(q * k, axis=-1)[..., None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_no_decay_unit_lambda_is_causal_linear_attention(oracle_mod):
    """a == 0 and lambda == 1: O = tril(Q K^T) V, a plain matrix product."""
    rng = np.random.default_rng(3)
    B, H, T, dk, dv = 2, 1, 40, 7, 3
    q, k, v, _, _ = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    a = np.zeros((B, H, T))
    lam = np.ones((B, H, T, _L(T)))
    o = oracle_mod.fwd(q, k, v, a, lam)
    for b in range(B):
        ref = np.tril(q[b, 0] @ k[b, 0].T) @ v[b, 0]
        np.testing.assert_allclose(o[b, 0], ref, rtol=1e-11, atol=1e-11)


def test_onehot_level_reads_only_its_bucket(oracle_mod):
    """With lambda = one-hot(l), row t sums exactly the keys of bucket l,
    built here from t's binary digits: [(t>>l)<<l, (t>>l)<<l + 2^(l-1)) when
    bit l-1 of t is set.  Summing over l recovers the full lambda (linearity)."""
    rng = np.random.default_rng(4)
    B, H, T, dk, dv = 1, 1, 70, 3, 2
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, L)
    total = np.zeros((B, H, T, dv))
    for lev in range(L):
        lam1 = np.zeros_like(lam)
        lam1[..., lev] = lam[..., lev]
        o = oracle_mod.fwd(q, k, v, a, lam1)
        total += o
        ref = np.zeros((T, dv))
        for t in range(T):
            if lev == 0:
                members = [t]
            elif (t >> (lev - 1)) & 1:
                lo = (t >> lev) << lev
                members = range(lo, lo + 2 ** (lev - 1))
            else:
                members = []
            for s in members:
                decay = np.exp(np.sum(a[0, 0, s + 1:t + 1]))
                ref[t] += decay * lam[0, 0, t, lev] * (q[0, 0, t] @ k[0, 0, s]) * v[0, 0, s]
        np.testing.assert_allclose(o[0, 0], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(total, oracle_mod.fwd(q, k, v, a, lam), rtol=1e-11, atol=1e-12)


def test_prefix_consistency(oracle_mod):
    rng = np.random.default_rng(5)
    B, H, T, dk, dv = 1, 2, 50, 4, 4
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    full = oracle_mod.fwd(q, k, v, a, lam)
    for Tp in (1, 7, 32, 33):
        Lp = _L(Tp)
        part = oracle_mod.fwd(q[:, :, :Tp], k[:, :, :Tp], v[:, :, :Tp], a[:, :, :Tp], lam[:, :, :Tp, :Lp])
        np.testing.assert_allclose(part, full[:, :, :Tp], rtol=1e-13, atol=1e-13)


def test_rows_match_full(oracle_mod):
    rng = np.random.default_rng(6)
    B, H, T, dk, dv = 2, 2, 64, 8, 4
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    full = oracle_mod.fwd(q, k, v, a, lam)
    rows = np.array([[0, 0], [1, 63], [3, 17], [2, 32]])
    got = oracle_mod.fwd_rows(q, k, v, a, lam, rows)
    for i, (bh, t) in enumerate(rows):
        np.testing.assert_array_equal(got[i], full.reshape(B * H, T, dv)[bh, t])


def test_too_narrow_lambda_is_an_error(oracle_mod):
    rng = np.random.default_rng(7)
    q, k, v, a, lam = _rand_inputs(rng, 1, 1, 9, 2, 2, 4)
    with pytest.raises(ValueError):
        oracle_mod.fwd(q, k, v, a, lam[..., :3])


# --- forward (O(T^2) sum) versus the recurrent decode form ----------------------

@pytest.mark.parametrize("T", [1, 2, 5, 16, 37, 64])
def test_forward_equals_serial_fenwick_recurrence(oracle_mod, T):
    rng = np.random.default_rng(10 + T)
    B, H, dk, dv = 1, 2, 5, 3
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, _L(T))
    o1 = oracle_mod.fwd(q, k, v, a, lam)
    o2 = oracle_mod.decode_sequence(q, k, v, a, lam)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)


def test_decode_stack_holds_decayed_bucket_sums(oracle_mod):
    """After step t, slot l holds sum over bucket l of t of
    exp(sum_{r=s+1..t} a_r) k_s v_s^T (bucket built from t's digits)."""
    rng = np.random.default_rng(20)
    T, dk, dv, Lcap = 37, 3, 2, 7
    q, k, v, a, lam = _rand_inputs(rng, 1, 1, T, dk, dv, Lcap)
    q, k, v, a, lam = q[0, 0], k[0, 0], v[0, 0], a[0, 0], lam[0, 0]
    state = np.zeros((1, 1, Lcap, dk, dv))
    logscale = np.zeros((1, 1, Lcap))
    for t in range(T):
        _, state, occ = oracle_mod.decode_step(
            state, logscale, np.array([t]), q[t][None, None], k[t][None, None], v[t][None, None],
            a[t].reshape(1, 1), lam[t][None, None])
        for lev in range(Lcap):
            if lev == 0:
                members = [t]
            elif (t >> (lev - 1)) & 1:
                lo = (t >> lev) << lev
                members = list(range(lo, lo + 2 ** (lev - 1)))
            else:
                members = []
            assert occ[0, lev] == bool(members)
            want = np.zeros((dk, dv))
            for s in members:
                want += np.exp(np.sum(a[s + 1:t + 1])) * np.outer(k[s], v[s])
            np.testing.assert_allclose(state[0, 0, lev], want, rtol=1e-12, atol=1e-13)


def test_decode_uses_logscale(oracle_mod):
    """A stored pair (hat S, g) is the state exp(g) hat S: scaling hat S by
    e^c and g by -c changes nothing."""
    rng = np.random.default_rng(21)
    S, H, Lcap, dk, dv = 3, 2, 6, 4, 3
    state = rng.standard_normal((S, H, Lcap, dk, dv))
    logscale = rng.standard_normal((S, H, Lcap)) * 0.5
    pos = np.array([5, 12, 31])
    q = rng.standard_normal((S, H, dk)); k = rng.standard_normal((S, H, dk))
    v = rng.standard_normal((S, H, dv)); a = -np.abs(rng.standard_normal((S, H)))
    lam = rng.random((S, H, Lcap))
    o1, n1, _ = oracle_mod.decode_step(state, logscale, pos, q, k, v, a, lam)
    c = rng.standard_normal((S, H, Lcap))
    o2, n2, _ = oracle_mod.decode_step(state * np.exp(c)[..., None, None], logscale - c, pos, q, k, v, a, lam)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(n1, n2, rtol=1e-12, atol=1e-12)


def test_decode_out_of_range_position(oracle_mod):
    rng = np.random.default_rng(22)
    S, H, Lcap, dk, dv = 2, 1, 4, 2, 2
    state = rng.standard_normal((S, H, Lcap, dk, dv))
    logscale = np.zeros((S, H, Lcap))
    pos = np.array([8, 3])  # 8 >= 2^(Lcap-1) is out of range
    q = rng.standard_normal((S, H, dk)); k = rng.standard_normal((S, H, dk))
    v = rng.standard_normal((S, H, dv)); a = -np.abs(rng.standard_normal((S, H)))
    lam = rng.random((S, H, Lcap))
    o, new, _ = oracle_mod.decode_step(state, logscale, pos, q, k, v, a, lam)
    assert np.all(np.isnan(o[0])) and np.all(np.isfinite(o[1]))
    for l in oracle_mod.occupied(7, Lcap):
        np.testing.assert_array_equal(new[0, 0, l], state[0, 0, l])


# --- prefill: the stack a prompt leaves for the next token -----------------------

def test_prefill_stack_hand_example(oracle_mod):
    """The hand-worked stack after the fourth token of the T=4 example."""
    g = json.load(open(os.path.join(HERE, "golden", "hand_T4.json")))
    T, Lcap = 4, 3
    k = np.array(g["k"]).reshape(1, 1, T, 1)
    v = np.array(g["v"]).reshape(1, 1, T, 2)
    a = np.array(g["a"]).reshape(1, 1, T)
    st, occ = oracle_mod.prefill_stack(k, v, a, Lcap)
    assert occ.tolist() == [True, True, True]
    for slot, want in g["expected_stack_after_t3"].items():
        np.testing.assert_allclose(st[0, 0, int(slot)], np.array(want), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("T", [1, 2, 3, 8, 9, 37, 64, 65])
def test_prefill_stack_equals_decode_recurrence(oracle_mod, T):
    """The stack summed bucket by bucket equals the one the recurrent form
    builds by merging and promoting token by token."""
    rng = np.random.default_rng(30 + T)
    H, dk, dv, Lcap = 2, 3, 2, 8
    q, k, v, a, lam = _rand_inputs(rng, 1, H, T, dk, dv, Lcap)
    state = np.zeros((1, H, Lcap, dk, dv))
    logscale = np.zeros((1, H, Lcap))
    for t in range(T):
        _, state, occ = oracle_mod.decode_step(state, logscale, np.array([t]), q[:, :, t], k[:, :, t], v[:, :, t],
                                               a[:, :, t], lam[:, :, t])
    st, occ2 = oracle_mod.prefill_stack(k, v, a, Lcap)
    assert occ2.tolist() == occ[0].tolist()
    np.testing.assert_allclose(st, state, rtol=1e-12, atol=1e-13)


def test_prefill_occupancy_follows_position_bits(oracle_mod):
    rng = np.random.default_rng(31)
    for T in list(range(1, 70)) + [127, 128, 129, 255, 256, 300]:
        k = rng.standard_normal((1, 1, T, 1))
        v = rng.standard_normal((1, 1, T, 1))
        a = np.zeros((1, 1, T))
        _, occ = oracle_mod.prefill_stack(k, v, a, 10)
        assert np.nonzero(occ)[0].tolist() == oracle_mod.occupied(T - 1, 10), T


def test_prefill_readout_is_last_forward_row(oracle_mod):
    """Reading the stack with the last token's query and weights gives the
    forward's last row: sum_l lambda_p[l] q_p^T S_l = o_p."""
    rng = np.random.default_rng(32)
    T, dk, dv = 45, 4, 3
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, 2, 2, T, dk, dv, L)
    st, occ = oracle_mod.prefill_stack(k, v, a, L)
    o = oracle_mod.fwd(q, k, v, a, lam)[:, :, T - 1]
    read = np.einsum("bhl,bhd,bhlde->bhe", lam[:, :, T - 1] * occ, q[:, :, T - 1], st)
    np.testing.assert_allclose(read, o, rtol=1e-12, atol=1e-12)


def test_prefill_without_decay_sums_to_kv(oracle_mod):
    """With a == 0 the buckets partition the prefix: the slots add up to K^T V."""
    rng = np.random.default_rng(33)
    T, dk, dv = 29, 5, 3
    k = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    st, _ = oracle_mod.prefill_stack(k, v, np.zeros((1, 1, T)), 6)
    np.testing.assert_allclose(st.sum(axis=2)[0, 0], k[0, 0].T @ v[0, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [1, 6, 16, 31, 40])
def test_prefill_then_decode_continues_the_forward(oracle_mod, T):
    """Decoding token T from the stack of tokens 0..T-1 gives row T of the
    forward over tokens 0..T."""
    rng = np.random.default_rng(34 + T)
    H, dk, dv, Lcap = 2, 4, 3, 8
    q, k, v, a, lam = _rand_inputs(rng, 1, H, T + 1, dk, dv, _L(T + 1))
    st, _ = oracle_mod.prefill_stack(k[:, :, :T], v[:, :, :T], a[:, :, :T], Lcap)
    lam_pad = np.zeros((1, H, Lcap))
    lam_pad[..., :lam.shape[-1]] = lam[:, :, T]
    o, _, _ = oracle_mod.decode_step(st, np.zeros((1, H, Lcap)), np.array([T]), q[:, :, T], k[:, :, T],
                                     v[:, :, T], a[:, :, T], lam_pad)
    want = oracle_mod.fwd(q, k, v, a, lam)[:, :, T]
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)


def test_prefill_stack_too_few_slots_is_an_error(oracle_mod):
    k = np.zeros((1, 1, 9, 1)); v = np.zeros((1, 1, 9, 1)); a = np.zeros((1, 1, 9))
    with pytest.raises(ValueError):
        oracle_mod.prefill_stack(k, v, a, 4)  # position 8 needs slot 4


# --- backward: gradients of sum(do * o) -------------------------------------------

def _loss(oracle_mod, q, k, v, a, lam, do):
    return float(np.sum(do * oracle_mod.fwd(q, k, v, a, lam)))


@pytest.mark.parametrize("T", [1, 2, 7, 16, 23])
def test_bwd_matches_finite_differences(oracle_mod, T):
    """Central differences of the forward oracle along random directions,
    input by input (the step keeps the fp64 truncation error near 1e-9)."""
    rng = np.random.default_rng(40 + T)
    B, H, dk, dv = 1, 2, 3, 2
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, L)
    do = rng.standard_normal((B, H, T, dv))
    g = oracle_mod.bwd(q, k, v, a, lam, do)
    args = {"q": q, "k": k, "v": v, "a": a, "lam": lam}
    eps = 1e-5
    for name, x in args.items():
        for _ in range(3):
            d = rng.standard_normal(x.shape)
            if name == "a":
                d[..., 0] = 0.0  # a_0 never enters: its gradient is 0 by construction
            plus = dict(args); plus[name] = x + eps * d
            minus = dict(args); minus[name] = x - eps * d
            fd = (_loss(oracle_mod, **plus, do=do) - _loss(oracle_mod, **minus, do=do)) / (2 * eps)
            an = float(np.sum(g["d" + name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
    assert np.all(g["da"][..., 0] == 0.0)


def _torch_masked_forward(torch, q, k, v, a, lam):
    """O = ((Q K^T) ⊙ M) V with M[t,s] = exp(A_t - A_s) * lam[t, level(t,s)]
    for s <= t (A = prefix sums of a from index 1), built with plain torch
    ops so that autograd differentiates it independently of the oracle."""
    T = q.shape[-2]
    A = torch.cumsum(torch.cat([torch.zeros_like(a[..., :1]), a[..., 1:]], dim=-1), dim=-1)
    t_idx = torch.arange(T).view(T, 1)
    s_idx = torch.arange(T).view(1, T)
    x = (t_idx ^ s_idx).clamp(min=0)
    lev = torch.zeros((T, T), dtype=torch.int64)
    for b in range(max(T, 1).bit_length() + 1):
        lev = torch.where(x >= (1 << b), torch.full_like(lev, b + 1), lev)
    causal = s_idx <= t_idx
    lev = torch.where(causal, lev, torch.zeros_like(lev))
    lam_ts = torch.gather(lam, -1, lev.expand(*lam.shape[:-2], T, T))
    decay = torch.exp(torch.where(causal, A.unsqueeze(-1) - A.unsqueeze(-2), torch.full_like(lam_ts, -1e300)))
    M = decay * lam_ts * causal
    return ((q @ k.transpose(-1, -2)) * M) @ v


@pytest.mark.parametrize("T", [1, 5, 16, 33])
def test_bwd_matches_torch_autograd_of_masked_form(oracle_mod, T):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(50 + T)
    B, H, dk, dv = 2, 1, 4, 3
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, L)
    do = rng.standard_normal((B, H, T, dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, lam)]
    o = _torch_masked_forward(torch, *ts)
    np.testing.assert_allclose(o.detach().numpy(), oracle_mod.fwd(q, k, v, a, lam), rtol=1e-12, atol=1e-12)
    (o * torch.tensor(do)).sum().backward()
    g = oracle_mod.bwd(q, k, v, a, lam, do)
    for name, t in zip(("dq", "dk", "dv", "da", "dlam"), ts):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_bwd_decay_shift_invariance(oracle_mod):
    """Adding a constant c to every a_r (r >= 1) multiplies each pair's
    weight by exp(c (t - s)); the derivative in c at 0 is sum_r da_r, which
    must equal sum_t sum_s (t - s) P(t,s) — checked against a direct sum."""
    rng = np.random.default_rng(60)
    T, dk, dv = 19, 3, 2
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, 1, 1, T, dk, dv, L)
    do = rng.standard_normal((1, 1, T, dv))
    g = oracle_mod.bwd(q, k, v, a, lam, do)
    total = 0.0
    for t in range(T):
        for s in range(t + 1):
            w = np.exp(np.sum(a[0, 0, s + 1:t + 1])) * lam[0, 0, t, oracle_mod.level(t, s)]
            total += (t - s) * w * (q[0, 0, t] @ k[0, 0, s]) * (do[0, 0, t] @ v[0, 0, s])
    np.testing.assert_allclose(np.sum(g["da"]), total, rtol=1e-12, atol=1e-12)


def test_bwd_rows_match_full(oracle_mod):
    rng = np.random.default_rng(61)
    T, dk, dv = 40, 5, 3
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, 2, 2, T, dk, dv, L)
    do = rng.standard_normal((2, 2, T, dv))
    g = oracle_mod.bwd(q, k, v, a, lam, do)
    rows = np.array([[0, 0], [1, 17], [3, 39], [2, 5]])
    r = oracle_mod.bwd_rows(q, k, v, a, lam, do, rows, rows)
    for i, (bh, t) in enumerate(rows):
        b, h = divmod(bh, 2)
        np.testing.assert_allclose(r["dq"][i], g["dq"][b, h, t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["dlam"][i], g["dlam"][b, h, t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["dk"][i], g["dk"][b, h, t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["dv"][i], g["dv"][b, h, t], rtol=1e-13, atol=1e-13)


def test_da_window_is_exact_with_full_window(oracle_mod):
    rng = np.random.default_rng(62)
    T, dk, dv = 37, 3, 2
    L = _L(T)
    q, k, v, a, lam = _rand_inputs(rng, 1, 2, T, dk, dv, L)
    do = rng.standard_normal((1, 2, T, dv))
    g = oracle_mod.bwd(q, k, v, a, lam, do)
    rows = np.array([[0, 1], [0, 17], [1, 36], [1, 8]])
    got = oracle_mod.da_window(q, k, v, a, lam, do, rows, W=T)
    want = np.array([g["da"][0, bh, r] for bh, r in rows])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # a short window drops the far pairs: with a strong decay they are tiny
    a_strong = a * 40.0
    g2 = oracle_mod.bwd(q, k, v, a_strong, lam, do)
    got2 = oracle_mod.da_window(q, k, v, a_strong, lam, do, rows, W=8)
    want2 = np.array([g2["da"][0, bh, r] for bh, r in rows])
    np.testing.assert_allclose(got2, want2, rtol=1e-6, atol=1e-9)


# --- q/k shared across heads (Mamba-2 groups) --------------------------------

def _brute_grouped(q, k, v, a, lam):
    """Pure-Python loops over the definition, with head h reading q/k head
    h // (H // Hqk): decay as an explicit sum of a, the level from the bit
    length of t xor s."""
    B, Hqk, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    r = H // Hqk
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            g = h // r
            for t in range(T):
                for s in range(t + 1):
                    lev = 0 if s == t else (t ^ s).bit_length()
                    w = np.exp(sum(a[b, h, x] for x in range(s + 1, t + 1))) * lam[b, h, t, lev]
                    out[b, h, t] += w * float(np.dot(q[b, g, t], k[b, g, s])) * v[b, h, s]
    return out


def test_grouped_forward_brute_force(oracle_mod):
    rng = np.random.default_rng(70)
    B, H, Hqk, T, dk, dv = 2, 6, 2, 11, 3, 2
    L = _L(T)
    _, _, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, L)
    q = rng.standard_normal((B, Hqk, T, dk))
    k = rng.standard_normal((B, Hqk, T, dk))
    got = oracle_mod.fwd_grouped(q, k, v, a, lam)
    np.testing.assert_allclose(got, _brute_grouped(q, k, v, a, lam), rtol=1e-12, atol=1e-12)
    # heads 0..2 share q/k head 0: with equal v, a and lambda they agree
    v2, a2, lam2 = v.copy(), a.copy(), lam.copy()
    v2[:, 1] = v2[:, 0]; a2[:, 1] = a2[:, 0]; lam2[:, 1] = lam2[:, 0]
    o2 = oracle_mod.fwd_grouped(q, k, v2, a2, lam2)
    np.testing.assert_array_equal(o2[:, 0], o2[:, 1])
    # one q/k head per head is the per-head forward
    qf = rng.standard_normal((B, H, T, dk))
    kf = rng.standard_normal((B, H, T, dk))
    np.testing.assert_array_equal(oracle_mod.fwd_grouped(qf, kf, v, a, lam), oracle_mod.fwd(qf, kf, v, a, lam))


def test_grouped_bwd_matches_finite_differences(oracle_mod):
    """The shared q/k gradients sum over the heads that read them: central
    differences of the grouped forward along random directions."""
    rng = np.random.default_rng(71)
    B, H, Hqk, T, dk, dv = 1, 4, 2, 9, 3, 2
    L = _L(T)
    _, _, v, a, lam = _rand_inputs(rng, B, H, T, dk, dv, L)
    q = rng.standard_normal((B, Hqk, T, dk))
    k = rng.standard_normal((B, Hqk, T, dk))
    do = rng.standard_normal((B, H, T, dv))
    g = oracle_mod.bwd_grouped(q, k, v, a, lam, do)
    assert g["dq"].shape == q.shape and g["dk"].shape == k.shape
    args = {"q": q, "k": k, "v": v, "a": a, "lam": lam}

    def loss(**kw):
        return float(np.sum(do * oracle_mod.fwd_grouped(**kw)))

    eps = 1e-5
    for name, x in args.items():
        for _ in range(2):
            d = rng.standard_normal(x.shape)
            if name == "a":
                d[..., 0] = 0.0
            plus = dict(args); plus[name] = x + eps * d
            minus = dict(args); minus[name] = x - eps * d
            fd = (loss(**plus) - loss(**minus)) / (2 * eps)
            an = float(np.sum(g["d" + name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_expand_heads_needs_a_multiple(oracle_mod):
    x = np.zeros((1, 3, 2, 2))
    assert oracle_mod.expand_heads(x, 6).shape == (1, 6, 2, 2)
    with pytest.raises(ValueError):
        oracle_mod.expand_heads(x, 4)
