"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a library routine, a closed
form worked by hand, an algebraic invariant, an independent brute force with a
different written form of the update, or an identity between two routes that
must agree. Chosen so that a dropped term, a wrong sign, a swapped operand or
a wrong index in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import workloads as W
from oracle import oracle as O


# ------------------------------------------------------------------ helpers

def _rand_pregated(T, K, V, seed, g_scale=0.3, unit_k=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, K))
    k = r.standard_normal((T, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = r.standard_normal((T, V))
    g = -np.abs(r.standard_normal((T, K))) * g_scale
    b = r.uniform(0.05, 0.95, T)
    S0 = 0.1 * r.standard_normal((K, V))
    return q, k, v, g, b, S0


def _widen(t: torch.Tensor) -> np.ndarray:
    """bf16 -> fp64 through torch's own conversion (independent of the oracle)."""
    return t.float().double().numpy()


def brute_force(case: W.Case, groups, lower_bound, scale):
    """Dense-matrix form of the update, written independently of the oracle:
        S <- (I - beta k k^T) diag(alpha) S + beta k v^T ,   o = scale S^T q
    with the gate from numpy/scipy library routines (logaddexp, expit).
    ``groups``: list of (row0, n, slot, read_initial). Returns (out, states)."""
    H, K, V = case.H, case.K, case.V
    qkv = _widen(case.inputs["mixed_qkv"])
    rg = _widen(case.inputs["raw_g"])
    rb = _widen(case.inputs["raw_beta"])
    A_log = case.inputs["A_log"].double().numpy()
    dtb = case.inputs["dt_bias"].double().numpy()
    pool = case.pool.double().numpy()
    out = np.zeros((case.rows, H, V))
    states = []
    for row0, n, slot, read_init in groups:
        st = np.zeros((H, K, V))
        for h in range(H):
            if slot < 0:
                continue
            S = pool[slot, h].copy() if read_init else np.zeros((K, V))
            a = math.exp(A_log[h])
            for t in range(row0, row0 + n):
                q = qkv[t, h * K:(h + 1) * K]
                k = qkv[t, H * K + h * K:H * K + (h + 1) * K]
                v = qkv[t, 2 * H * K + h * V:2 * H * K + (h + 1) * V]
                x = rg[t, h * K:(h + 1) * K] + dtb[h * K:(h + 1) * K]
                if lower_bound is None:
                    g = -a * np.logaddexp(0.0, x)
                else:
                    g = lower_bound * sps.expit(a * x)
                beta = sps.expit(rb[t, h])
                S = (np.eye(K) - beta * np.outer(k, k)) @ np.diag(np.exp(g)) @ S + beta * np.outer(k, v)
                out[t, h] = scale * (S.T @ q)
            st[h] = S
        states.append(st)
    return out, np.stack(states) if states else np.zeros((0, H, K, V))


def _rel(a, b):
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


# ------------------------------------------------------------ scalar pieces

def test_bf16_widening_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, 4000).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80],
                                          dtype=np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([O.bf16_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_gate_closed_forms():
    # raw_g + dt_bias = 0: softplus(0) = ln 2, sigmoid(0) = 1/2.
    for A_log in (0.0, math.log(3.0), math.log(16.0)):
        assert O.gate(0.0, A_log, 0.0, None) == pytest.approx(-math.exp(A_log) * math.log(2.0), rel=1e-15)
        assert O.gate(0.0, A_log, 0.0, -5.0) == pytest.approx(-2.5, rel=1e-15)
    # dt_bias is added before the activation: (x, b) and (x + b, 0) agree.
    assert O.gate(0.7, 0.3, -0.2, None) == pytest.approx(O.gate(0.5, 0.3, 0.0, None), rel=1e-15)
    # Library routines: -a*logaddexp(0, x) and lb*expit(a*x).
    for x in np.linspace(-40, 40, 81):
        for A_log in (0.0, 1.3, 2.77):
            a = math.exp(A_log)
            assert O.gate(x, A_log, 0.0, None) == pytest.approx(-a * np.logaddexp(0.0, x), rel=1e-14, abs=1e-300)
            assert O.gate(x, A_log, 0.0, -5.0) == pytest.approx(-5.0 * sps.expit(a * x), rel=1e-14, abs=1e-300)
            lbv = O.gate(x, A_log, 0.0, -5.0)
            assert -5.0 <= lbv <= 0.0
            assert O.gate(x, A_log, 0.0, None) <= 0.0
    # Large-argument limits of softplus: x -> +inf gives -a x, x -> -inf gives -a e^x.
    assert O.gate(50.0, 0.0, 0.0, None) == pytest.approx(-50.0, rel=1e-15)
    assert O.gate(-50.0, 0.0, 0.0, None) == pytest.approx(-math.exp(-50.0), rel=1e-12)


def test_beta_is_logistic():
    assert O.beta(0.0) == 0.5
    for x in np.linspace(-30, 30, 61):
        assert O.beta(x) == pytest.approx(sps.expit(x), rel=1e-14)


# ------------------------------------------------------- brute force (P-a)

@pytest.mark.parametrize("lower_bound", [None, -5.0])
@pytest.mark.parametrize("K,V,H", [(4, 4, 2), (4, 6, 3), (8, 5, 1)])
def test_decode_matches_brute_force(K, V, H, lower_bound):
    case = W.decode_case("bf", H, K, V, num_seqs=5, tokens_per_seq=3, num_slots=11,
                         index_stride=3, lower_bound=lower_bound, seed=17, std=0.3,
                         null_rows=(2,), scale=0.7)
    out, fs, pool_after = O.decode_packed(case.inputs, case.pool, case.state_indices, H, K, V,
                                          tokens_per_seq=3, lower_bound=lower_bound, scale=0.7)
    idx = case.state_indices.tolist()
    groups = [(3 * n, 3, idx[n], True) for n in range(5)]
    ref_out, ref_st = brute_force(case, groups, lower_bound, 0.7)
    assert _rel(out, ref_out) < 1e-12
    for n in range(5):
        if idx[n] >= 0:
            assert _rel(fs[n], ref_st[n]) < 1e-12
            np.testing.assert_array_equal(pool_after[idx[n]].reshape(H, K, V),
                                          ref_st[n].astype(np.float32))
    assert np.all(out[6:9] == 0.0)  # null slot rows


def _spec_brute(case: W.Case, lower_bound, scale):
    """Per-token states of the spec-decode reading through the dense brute
    force: request n starts from the slot in column num_accepted[n]-1 and its
    state after token t is the brute-force state after t+1 tokens."""
    T = case.tokens_per_seq
    tab = case.block_table.tolist()
    acc = case.num_accepted.tolist()
    N = len(tab)
    out = np.zeros((case.rows, case.H, case.V))
    states = np.zeros((N, T, case.H, case.K, case.V))
    for n in range(N):
        s0 = tab[n][acc[n] - 1]
        for t in range(T):
            o, st = brute_force(case, [(n * T, t + 1, s0, True)], lower_bound, scale)
            out[n * T + t] = o[n * T + t]
            states[n, t] = st[0] if s0 >= 0 else 0.0
    return out, states


@pytest.mark.parametrize("lower_bound", [None, -5.0])
@pytest.mark.parametrize("T", [1, 3, 4])
def test_spec_decode_states_match_brute_force(T, lower_bound):
    """Initial state from column num_accepted-1, the state after token t in
    column t, a padded request (null slots) touching nothing."""
    H, K, V, N = 2, 4, 5, 4
    case = W.spec_decode_case("sd", H, K, V, N, T, num_slots=N * 4 + 3, lower_bound=lower_bound,
                              seed=71 + T, width=4, std=0.3, null_rows=(2,))
    out, states, pool_after = O.spec_decode(case.inputs, case.pool, case.block_table, case.num_accepted,
                                            H, K, V, T, lower_bound=lower_bound, scale=0.6)
    ref_out, ref_states = _spec_brute(case, lower_bound, 0.6)
    assert _rel(out, ref_out) < 1e-12
    assert _rel(states, ref_states) < 1e-12
    tab = case.block_table.tolist()
    written = set()
    for n in range(N):
        for t in range(T):
            sl = tab[n][t]
            if sl >= 0 and n != 2:
                written.add(sl)
                np.testing.assert_array_equal(pool_after[sl].reshape(H, K, V),
                                              ref_states[n, t].astype(np.float32))
    before = case.pool.reshape(case.pool.shape[0], -1).numpy()
    for sl in range(case.pool.shape[0]):
        if sl not in written:
            np.testing.assert_array_equal(pool_after[sl], before[sl])
    assert np.all(out[2 * T:3 * T] == 0.0)


def test_spec_decode_skips_null_columns_and_selects_by_accepted_count():
    H, K, V, N, T = 1, 4, 4, 3, 4
    case = W.spec_decode_case("sdn", H, K, V, N, T, num_slots=N * 4, lower_bound=-5.0, seed=91,
                              width=4, std=0.3, null_cols=((0, 1), (1, 3)), accepted=[3, 2, 1])
    out, states, pool_after = O.spec_decode(case.inputs, case.pool, case.block_table, case.num_accepted,
                                            H, K, V, T, lower_bound=-5.0)
    tab = case.block_table.tolist()
    before = case.pool.reshape(N * 4, -1).numpy()
    # The null entries are skipped; every other column holds its token's state.
    for n in range(N):
        for t in range(T):
            sl = tab[n][t]
            if sl >= 0:
                np.testing.assert_array_equal(pool_after[sl], states[n, t].reshape(-1).astype(np.float32))
    # Request 0 started from column 2: its first output equals a one-token
    # decode from that slot's original state.
    single = W.decode_case("one", H, K, V, 1, 1, N * 4, 1, -5.0, seed=91)
    single.inputs = {k: (v[0:1] if v.dim() and v.shape[0] == N * T else v) for k, v in case.inputs.items()}
    single.pool = case.pool
    single.block_table = torch.tensor([[tab[0][2]]], dtype=torch.int32)
    o1, _ = brute_force(single, [(0, 1, tab[0][2], True)], -5.0, 1.0)
    np.testing.assert_allclose(out[0], o1[0], rtol=0, atol=1e-12)
    assert np.isfinite(before).all()


@pytest.mark.parametrize("lower_bound", [None, -5.0])
def test_prefill_matches_brute_force(lower_bound):
    lens = [1, 9, 0, 23, 40]
    case = W.prefill_case("bf", 2, 6, 5, lens, 9, lower_bound, seed=23, std=0.2,
                          has_initial=[1, 0, 1, 1, 0])
    out, fs, _ = O.prefill(case.inputs, case.pool, case.state_indices, case.cu_seqlens.tolist(),
                           2, 6, 5, has_initial_state=[1, 0, 1, 1, 0], lower_bound=lower_bound)
    cu = case.cu_seqlens.tolist()
    idx = case.state_indices.tolist()
    groups = [(cu[i], cu[i + 1] - cu[i], idx[i], [1, 0, 1, 1, 0][i]) for i in range(5)]
    ref_out, ref_st = brute_force(case, groups, lower_bound, 1.0)
    assert _rel(out, ref_out) < 1e-12
    for i in (0, 1, 3, 4):
        assert _rel(fs[i], ref_st[i]) < 1e-12


# ------------------------------------------------ chunked = recurrent (P-b)

@pytest.mark.parametrize("C", [1, 2, 3, 16, 64])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 130])
def test_chunked_equals_recurrent(C, T):
    q, k, v, g, b, S0 = _rand_pregated(T, 8, 6, seed=C * 1000 + T)
    o1, S1 = O.recurrent_pregated(q, k, v, g, b, S0, scale=0.9)
    o2, S2 = O.chunked_pregated(q, k, v, g, b, S0, C, scale=0.9)
    assert _rel(o2, o1) < 1e-11
    assert _rel(S2, S1) < 1e-11


def test_chunked_survives_huge_decay():
    """Per-token decays down to -90 (cumulated -5000 over a chunk): the pairwise
    exponentials of the chunked form must not overflow, and it must still equal
    the recurrence."""
    q, k, v, g, b, S0 = _rand_pregated(130, 8, 4, seed=5)
    g = -np.random.default_rng(6).uniform(0.0, 90.0, g.shape)
    o1, S1 = O.recurrent_pregated(q, k, v, g, b, S0)
    o2, S2 = O.chunked_pregated(q, k, v, g, b, S0, 64)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(S2))
    assert _rel(o2, o1) < 1e-11


# ---------------------------------------------- delta-rule invariant (P-c)

def test_delta_rule_invariant():
    """alpha = 1, beta = 1, |k| = 1: after the write, S^T k = v exactly."""
    T, K, V = 12, 16, 7
    q, k, v, _, _, S0 = _rand_pregated(T, K, V, seed=3)
    g = np.zeros((T, K))
    b = np.ones(T)
    S = S0.copy()
    for t in range(T):
        _, S = O.recurrent_pregated(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], b[t:t + 1], S)
        np.testing.assert_allclose(S.T @ k[t], v[t], rtol=0, atol=1e-13)


# ---------------------------------------------------- closed forms (P-d)

def test_no_write_no_decay_is_plain_readout():
    """beta = 0 and g = 0: the state is unchanged and o = scale S0^T q."""
    q, k, v, _, _, S0 = _rand_pregated(4, 6, 5, seed=9)
    o, S = O.recurrent_pregated(q, k, v, np.zeros((4, 6)), np.zeros(4), S0, scale=0.5)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, 0.5 * q @ S0, rtol=1e-14, atol=1e-15)


def test_full_forget_full_write():
    """alpha = 0 and beta = 1: S = k v^T and o = scale v (k.q)."""
    q, k, v, _, _, S0 = _rand_pregated(1, 6, 5, seed=11, unit_k=False)
    o, S = O.recurrent_pregated(q, k, v, np.full((1, 6), -1e4), np.ones(1), S0, scale=2.0)
    np.testing.assert_allclose(S, np.outer(k[0], v[0]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0], 2.0 * v[0] * (k[0] @ q[0]), rtol=1e-14)


def test_scalar_recurrence_worked_by_hand():
    """K = V = 1 worked by hand.  s0 = 4.
    t0: alpha=1/2 -> 2; u = 1/4 (2 - 2*1) = 0 -> s = 2; o = 3 * 2 = 6.
    t1: alpha=1 -> 2; u = 1 (5 - 2) = 3 -> s = 5; o = 3 * 5 = 15.
    t2: alpha=1/4 -> 1.25; k = 2: u = 1/2 (1 - 2*1.25) = -0.75;
        s = 1.25 + 2*(-0.75) = -0.25; q = -2: o = 0.5.  (scale 1)"""
    q = np.array([[3.0], [3.0], [-2.0]])
    k = np.array([[1.0], [1.0], [2.0]])
    v = np.array([[2.0], [5.0], [1.0]])
    g = np.log(np.array([[0.5], [1.0], [0.25]]))
    b = np.array([0.25, 1.0, 0.5])
    o, S = O.recurrent_pregated(q, k, v, g, b, np.array([[4.0]]))
    np.testing.assert_allclose(o[:, 0], [6.0, 15.0, 0.5], rtol=1e-14)
    np.testing.assert_allclose(S, [[-0.25]], rtol=1e-14)
    o2, S2 = O.chunked_pregated(q, k, v, g, b, np.array([[4.0]]), 2)
    np.testing.assert_allclose(o2[:, 0], [6.0, 15.0, 0.5], rtol=1e-13)


def test_two_by_two_worked_by_hand():
    """K = V = 2, S0 = I, alpha = (1, 1/2), beta = 1/2, k = e1, v = (1, 1), q = (1, 1).
    decay: S = diag(1, 1/2);  S^T k = (1, 0);  u = 1/2 ((1,1) - (1,0)) = (0, 1/2);
    S = [[1, 1/2], [0, 1/2]];  o = S^T q = (1, 1)."""
    o, S = O.recurrent_pregated(np.array([[1.0, 1.0]]), np.array([[1.0, 0.0]]),
                                np.array([[1.0, 1.0]]), np.log(np.array([[1.0, 0.5]])),
                                np.array([0.5]), np.eye(2))
    np.testing.assert_allclose(S, [[1.0, 0.5], [0.0, 0.5]], rtol=1e-15)
    np.testing.assert_allclose(o[0], [1.0, 1.0], rtol=1e-15)


# --------------------------------------------------------- linearity (P-e)

def test_linear_in_initial_state_and_values():
    q, k, v, g, b, S0 = _rand_pregated(20, 8, 6, seed=13)
    o_full, S_full = O.recurrent_pregated(q, k, v, g, b, S0)
    o_s, S_s = O.recurrent_pregated(q, k, np.zeros_like(v), g, b, S0)
    o_v, S_v = O.recurrent_pregated(q, k, v, g, b, np.zeros_like(S0))
    np.testing.assert_allclose(o_full, o_s + o_v, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_full, S_s + S_v, rtol=0, atol=1e-13)


def test_segment_maps_compose_to_the_whole_sequence():
    """A run of tokens maps the state affinely: S_out = M S_in + B, with M the
    end state reached from the identity with zero values and B the end state
    reached from zero. Walking S_{j+1} = M_j S_j + B_j over consecutive
    segments reproduces the uncut end state, and rerunning each segment from
    its S_j reproduces the uncut outputs (the segment-parallel inter-chunk
    pass relies on both)."""
    T, K, V = 150, 8, 6
    q, k, v, g, b, S0 = _rand_pregated(T, K, V, seed=17)
    o_all, S_all = O.recurrent_pregated(q, k, v, g, b, S0)
    S = S0.copy()
    outs = []
    for a, e in [(0, 64), (64, 128), (128, 150)]:
        M = O.recurrent_pregated(q[a:e], k[a:e], np.zeros((e - a, K)), g[a:e], b[a:e], np.eye(K))[1]
        B = O.recurrent_pregated(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], np.zeros((K, V)))[1]
        o_seg, S_seg = O.recurrent_pregated(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], S)
        np.testing.assert_allclose(S_seg, M @ S + B, rtol=0, atol=1e-13)
        assert np.abs(M - np.eye(K)).max() > 1e-3   # the segment does change the state
        outs.append(o_seg)
        S = M @ S + B
    np.testing.assert_allclose(S, S_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.concatenate(outs), o_all, rtol=0, atol=1e-13)


# ------------------------------------------------------ equivariance (P-f)

def test_value_columns_permute_and_heads_are_independent():
    q, k, v, g, b, S0 = _rand_pregated(10, 8, 6, seed=21)
    perm = np.random.default_rng(1).permutation(6)
    o, S = O.recurrent_pregated(q, k, v, g, b, S0)
    op, Sp = O.recurrent_pregated(q, k, v[:, perm], g, b, S0[:, perm])
    np.testing.assert_allclose(op, o[:, perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Sp, S[:, perm], rtol=1e-14, atol=1e-15)
    # Heads: changing head 1's inputs leaves head 0's outputs bit-identical.
    case = W.decode_case("eq", 2, 4, 4, 3, 2, 6, 1, -5.0, seed=5, std=0.3)
    out_a, _, _ = O.decode_packed(case.inputs, case.pool, case.state_indices, 2, 4, 4, 2, -5.0)
    qkv = case.inputs["mixed_qkv"].clone()
    qkv[:, 4:8] = -qkv[:, 4:8]           # q of head 1
    qkv[:, 2 * 2 * 4 + 4:] *= 3          # v of head 1
    mod = dict(case.inputs, mixed_qkv=qkv)
    out_b, _, _ = O.decode_packed(mod, case.pool, case.state_indices, 2, 4, 4, 2, -5.0)
    np.testing.assert_array_equal(out_a[:, 0], out_b[:, 0])
    assert not np.array_equal(out_a[:, 1], out_b[:, 1])


# ---------------------------------------------------- cross-path (P-g/P-h)

def _single_seq_case(T, seed, lb=-5.0):
    return W.prefill_case("x", 2, 8, 8, [T], 3, lb, seed=seed, std=0.2)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_decodes_equal_prefill_equal_spec_verify(T):
    case = _single_seq_case(T, seed=31 + T)
    idx = case.state_indices
    pre_out, pre_fs, pre_pool = O.prefill(case.inputs, case.pool, idx, [0, T], 2, 8, 8, lower_bound=-5.0)
    spec_out, spec_fs, spec_pool = O.decode_packed(case.inputs, case.pool, idx, 2, 8, 8,
                                                   tokens_per_seq=T, lower_bound=-5.0)
    np.testing.assert_allclose(spec_out, pre_out, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(spec_pool, pre_pool)
    # T single-token decodes, threading the fp32 pool through.
    pool = case.pool.clone()
    outs = []
    for t in range(T):
        rows = {kk: (vv[t:t + 1] if vv.dim() and vv.shape[0] == T else vv)
                for kk, vv in case.inputs.items()}
        o, _, p = O.decode_packed(rows, pool, idx, 2, 8, 8, 1, -5.0)
        pool = torch.from_numpy(p).view_as(case.pool)
        outs.append(o)
    dec = np.concatenate(outs)
    # Each decode step re-reads an fp32-rounded state, so agreement is to fp32 rounding.
    assert _rel(dec, pre_out) < 1e-6


def test_prefill_split_equals_whole():
    T1, T2 = 70, 59
    case = _single_seq_case(T1 + T2, seed=41, lb=None)
    idx = case.state_indices
    whole, whole_fs, _ = O.prefill(case.inputs, case.pool, idx, [0, T1 + T2], 2, 8, 8)
    first = {kk: (vv[:T1] if vv.shape[0] == T1 + T2 else vv) for kk, vv in case.inputs.items()}
    second = {kk: (vv[T1:] if vv.shape[0] == T1 + T2 else vv) for kk, vv in case.inputs.items()}
    o1, _, p1 = O.prefill(first, case.pool, idx, [0, T1], 2, 8, 8)
    o2, fs2, _ = O.prefill(second, torch.from_numpy(p1).view_as(case.pool), idx, [0, T2], 2, 8, 8)
    assert _rel(np.concatenate([o1, o2]), whole) < 1e-6
    assert _rel(fs2, whole_fs) < 1e-6


def test_mixed_equals_separate_calls():
    case = W.mixed_case("m", 2, 8, 8, 5, [1, 17, 66], 16, -5.0, seed=51, index_stride=4)
    idx = case.state_indices
    D = 5
    out, fs, pool = O.mixed_batch(case.inputs, case.pool, idx, D, case.cu_seqlens.tolist(), 2, 8, 8,
                                  lower_bound=-5.0)
    dec_in = {kk: (vv[:D] if vv.shape[0] == case.rows else vv) for kk, vv in case.inputs.items()}
    pre_in = {kk: (vv[D:] if vv.shape[0] == case.rows else vv) for kk, vv in case.inputs.items()}
    o_d, _, p_d = O.decode_packed(dec_in, case.pool, idx[:D], 2, 8, 8, 1, -5.0)
    o_p, _, p_p = O.prefill(pre_in, torch.from_numpy(p_d).view_as(case.pool), idx[D:],
                            case.cu_seqlens.tolist(), 2, 8, 8, lower_bound=-5.0)
    np.testing.assert_array_equal(out, np.concatenate([o_d, o_p]))
    np.testing.assert_array_equal(pool, p_p)


@pytest.mark.parametrize("lb", [None, -5.0])
def test_length_one_sequences_through_chunked_form(lb):
    """Length-1 sequences in the chunked form are finite and equal the decode
    (the NaN-for-length-1 failure of the chunk kernel described in PR #50649)."""
    lens = [1, 1, 5, 1]
    case = W.prefill_case("l1", 2, 8, 8, lens, 8, lb, seed=61, std=0.2)
    idx = case.state_indices
    chunk_out, chunk_fs, _ = O.prefill(case.inputs, case.pool, idx, case.cu_seqlens.tolist(), 2, 8, 8,
                                       lower_bound=lb, form=64)
    rec_out, rec_fs, _ = O.prefill(case.inputs, case.pool, idx, case.cu_seqlens.tolist(), 2, 8, 8,
                                   lower_bound=lb, form=0)
    assert np.all(np.isfinite(chunk_out)) and np.all(np.isfinite(chunk_fs))
    assert _rel(chunk_out, rec_out) < 1e-12
    assert _rel(chunk_fs, rec_fs) < 1e-12


# ----------------------------------------------------------- slot handling

def test_null_and_untouched_slots_are_bit_identical():
    case = W.decode_case("ns", 2, 4, 4, 4, 2, 10, 8, -5.0, seed=71, null_rows=(1, 3))
    out, _, pool_after = O.decode_packed(case.inputs, case.pool, case.state_indices, 2, 4, 4, 2, -5.0)
    before = case.pool.reshape(10, -1).numpy()
    touched = {s for s in case.state_indices.tolist() if s >= 0}
    for s in range(10):
        if s not in touched:
            np.testing.assert_array_equal(pool_after[s], before[s])
        else:
            assert not np.array_equal(pool_after[s], before[s])
    assert np.all(out[2:4] == 0.0) and np.all(out[6:8] == 0.0)


def test_no_initial_state_means_zero_state():
    case = W.prefill_case("z", 2, 8, 8, [7, 3], 4, -5.0, seed=81, std=0.3)
    idx = case.state_indices
    o0, fs0, _ = O.prefill(case.inputs, case.pool, idx, case.cu_seqlens.tolist(), 2, 8, 8,
                           has_initial_state=[0, 0], lower_bound=-5.0)
    zero_pool = torch.zeros_like(case.pool)
    o1, fs1, _ = O.prefill(case.inputs, zero_pool, idx, case.cu_seqlens.tolist(), 2, 8, 8,
                           lower_bound=-5.0)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(fs0, fs1)


def test_padded_slot_stride_is_honoured():
    case = W.decode_case("pad", 2, 4, 4, 3, 1, 5, 2, -5.0, seed=91, slot_pad=13)
    assert case.pool.stride(0) == 2 * 4 * 4 + 13
    out_a, fs_a, _ = O.decode_packed(case.inputs, case.pool, case.state_indices, 2, 4, 4, 1, -5.0)
    dense = case.pool.contiguous()
    out_b, fs_b, _ = O.decode_packed(case.inputs, dense, case.state_indices, 2, 4, 4, 1, -5.0)
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(fs_a, fs_b)


# ------------------------------------------------ gated RMSNorm epilogue (R20)

def _bf16_rows(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def _norm_inputs(rows=3, H=2, V=8, seed=71):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, H, V))
    z = _bf16_rows(rng.standard_normal((rows, H * V)).tolist())
    w = torch.tensor(rng.uniform(0.5, 1.5, V), dtype=torch.float32)
    return o, z, w


def _rms(y):
    return np.sqrt((y ** 2).mean(axis=-1))


def test_gated_rmsnorm_unit_rms_and_direction():
    """eps = 0, unit weights and an activation of 1 (sigmoid of a large gate):
    every head's output has RMS 1 and points along o."""
    o, _, _ = _norm_inputs()
    z = _bf16_rows([[88.0] * 16] * 3)   # sigmoid(88) = 1 in fp64
    y = O.gated_rmsnorm(o, z, torch.ones(8), 0.0, "sigmoid")
    np.testing.assert_allclose(_rms(y), 1.0, rtol=1e-14)
    ratio = y / o
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-13)
    assert np.all(ratio > 0)


def test_gated_rmsnorm_activation_special_values():
    """sigmoid(0) = 1/2 halves the RMS; z sigmoid(z) is 0 at z = 0 and about
    z for a large gate."""
    o, _, _ = _norm_inputs()
    zeros = _bf16_rows([[0.0] * 16] * 3)
    big = _bf16_rows([[88.0] * 16] * 3)
    w = torch.ones(8)
    np.testing.assert_allclose(_rms(O.gated_rmsnorm(o, zeros, w, 0.0, "sigmoid")), 0.5, rtol=1e-14)
    assert np.all(O.gated_rmsnorm(o, zeros, w, 0.0, "silu") == 0.0)
    np.testing.assert_allclose(_rms(O.gated_rmsnorm(o, big, w, 0.0, "silu")), 88.0, rtol=1e-14)


def test_gated_rmsnorm_scaling_identity_fixes_eps():
    """Scaling o by lambda equals dividing eps by lambda^2:
    y(lambda o; eps) = y(o; eps / lambda^2) (eps sits under the root, beside
    the mean square); with eps = 0 the output is scale-invariant and odd."""
    o, z, w = _norm_inputs(seed=73)
    for lam in (0.01, 3.0, 250.0):
        np.testing.assert_allclose(O.gated_rmsnorm(lam * o, z, w, 0.3),
                                   O.gated_rmsnorm(o, z, w, 0.3 / lam ** 2), rtol=1e-12)
        np.testing.assert_allclose(O.gated_rmsnorm(lam * o, z, w, 0.0), O.gated_rmsnorm(o, z, w, 0.0),
                                   rtol=1e-12)
    np.testing.assert_allclose(O.gated_rmsnorm(-o, z, w, 0.3), -O.gated_rmsnorm(o, z, w, 0.3), rtol=1e-15)
    # eps > 0 shrinks the output of a small row well below unit RMS.
    tiny = 1e-3 * o
    assert np.all(_rms(O.gated_rmsnorm(tiny, _bf16_rows([[88.0] * 16] * 3), torch.ones(8), 1.0)) < 2e-3)


def test_gated_rmsnorm_weight_is_per_channel_and_gate_per_head():
    o, _, _ = _norm_inputs(seed=75)
    H, V = 2, 8
    onehot = torch.zeros(V)
    onehot[5] = 2.0
    big = _bf16_rows([[88.0] * 16] * 3)
    y = O.gated_rmsnorm(o, big, onehot, 0.0)
    assert np.count_nonzero(y[..., [0, 1, 2, 3, 4, 6, 7]]) == 0
    assert np.all(y[..., 5] != 0)
    # Head 0's gate 0 (sigmoid 1/2), head 1's gate large (sigmoid 1).
    z = _bf16_rows([[0.0] * V + [88.0] * V] * 3)
    y = O.gated_rmsnorm(o, z, torch.ones(V), 0.0)
    np.testing.assert_allclose(_rms(y)[:, 0], 0.5, rtol=1e-14)
    np.testing.assert_allclose(_rms(y)[:, 1], 1.0, rtol=1e-14)
    # Heads are independent: changing head 1's outputs leaves head 0's alone.
    o2 = o.copy()
    o2[:, 1] *= -7.0
    y2 = O.gated_rmsnorm(o2, z, torch.ones(V), 0.1)
    np.testing.assert_array_equal(y2[:, 0], O.gated_rmsnorm(o, z, torch.ones(V), 0.1)[:, 0])


# ------------------------------------------------ short conv prologue (R22)

def _conv_setup(lens, H=2, K=4, V=3, Wd=4, slots=6, seed=81, bias=True):
    g = torch.Generator().manual_seed(seed)
    D = 2 * H * K + H * V
    rows = sum(lens)
    x = torch.randn(rows, D, generator=g).to(torch.bfloat16)
    w = torch.randn(D, Wd, generator=g) * 0.5
    b = torch.randn(D, generator=g) * 0.1 if bias else None
    state = torch.randn(slots, Wd - 1, D, generator=g).to(torch.bfloat16).double()
    idx = torch.randperm(slots, generator=g)[:len(lens)].to(torch.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return D, x, w, b, state, idx, cu


def _silu(a):
    return torch.nn.functional.silu(torch.as_tensor(a, dtype=torch.float64)).numpy()


def test_short_conv_matches_numpy_convolution_per_channel():
    """Pre-activation = numpy's convolution of [history; inputs] with the
    flipped taps, then torch's silu; q and k of each head are then unit
    vectors along the same direction."""
    H, K, V, Wd = 2, 4, 3, 4
    lens = [5, 1, 9]
    D, x, w, b, state, idx, cu = _conv_setup(lens, H, K, V, Wd)
    y, _ = O.short_conv(x, w, b, state, idx, cu, H, K, V, l2_eps=1e-300)
    xf = x.double().numpy()
    raw = np.zeros_like(y)
    for s in range(len(lens)):
        hist = state[int(idx[s])].numpy()          # [W-1, D], oldest first
        seq = np.concatenate([hist, xf[cu[s]:cu[s + 1]]])
        for c in range(D):
            a = np.convolve(seq[:, c], w[c].double().numpy()[::-1], mode="valid") + float(b[c])
            raw[cu[s]:cu[s + 1], c] = _silu(a)
    np.testing.assert_allclose(y[:, 2 * H * K:], raw[:, 2 * H * K:], rtol=1e-13, atol=1e-15)
    for part in range(2):
        for h in range(H):
            sl = slice(part * H * K + h * K, part * H * K + (h + 1) * K)
            ref = raw[:, sl] / np.linalg.norm(raw[:, sl], axis=1, keepdims=True)
            np.testing.assert_allclose(y[:, sl], ref, rtol=1e-12, atol=1e-14)


def test_short_conv_single_taps_are_shifts():
    """One-hot taps: the last tap passes the current input, the first passes
    the input W-1 rows back (from the conv state for the first rows)."""
    H, K, V, Wd = 1, 4, 4, 4
    D, x, _, _, state, idx, cu = _conv_setup([6], H, K, V, Wd, seed=83)
    for tap, back in ((Wd - 1, 0), (0, Wd - 1)):
        w = torch.zeros(D, Wd)
        w[:, tap] = 1.0
        y, _ = O.short_conv(x, w, None, state, idx, cu, H, K, V)
        v = y[:, 2 * H * K:]
        hist = state[int(idx[0])].numpy()
        seq = np.concatenate([hist, x.double().numpy()])[:, 2 * H * K:]
        np.testing.assert_allclose(v, _silu(seq[Wd - 1 - back: Wd - 1 - back + 6]), rtol=1e-14)


def test_short_conv_state_carries_across_calls():
    """One call over a sequence equals two calls with the conv state carried
    between them, and T one-row calls equal one T-row call; a sequence
    shorter than W-1 shifts the old state."""
    H, K, V, Wd = 2, 4, 3, 4
    D, x, w, b, state, idx, cu = _conv_setup([7], H, K, V, Wd, seed=85)
    y_all, st_all = O.short_conv(x, w, b, state, idx, cu, H, K, V)
    cuts = [0, 2, 3, 7]
    st = state.clone()
    ys = []
    for a, e in zip(cuts[:-1], cuts[1:]):
        y, st_np = O.short_conv(x[a:e], w, b, st, idx, [0, e - a], H, K, V)
        st = torch.from_numpy(st_np)
        ys.append(y)
    np.testing.assert_allclose(np.concatenate(ys), y_all, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(st.numpy(), st_all)
    # The new state is the last W-1 inputs of the sequence.
    np.testing.assert_array_equal(st_all[int(idx[0])], x[-(Wd - 1):].double().numpy())
    # A 1-row call shifts the old state by one row and appends the input.
    _, st1 = O.short_conv(x[:1], w, b, state, idx, [0, 1], H, K, V)
    old = state[int(idx[0])].numpy()
    np.testing.assert_array_equal(st1[int(idx[0])], np.concatenate([old[1:], x[:1].double().numpy()]))


def test_short_conv_null_slot_and_no_initial_state():
    H, K, V, Wd = 2, 4, 3, 3
    D, x, w, b, state, idx, cu = _conv_setup([4, 3], H, K, V, Wd, seed=87)
    null = idx.clone()
    null[0] = -1
    y_null, st_null = O.short_conv(x, w, b, state, null, cu, H, K, V)
    y_zero, st_zero = O.short_conv(x, w, b, state, idx, cu, H, K, V, has_initial_state=[0, 1])
    # Both read zeros before the first row; the null slot writes no state
    # (only the second sequence's slot changes).
    np.testing.assert_array_equal(y_null, y_zero)
    others = [s for s in range(state.shape[0]) if s != int(idx[1])]
    np.testing.assert_array_equal(st_null[others], state.numpy()[others])
    assert not np.array_equal(st_zero[int(idx[0])], state[int(idx[0])].numpy())
    y_init, _ = O.short_conv(x, w, b, state, idx, cu, H, K, V)
    assert not np.allclose(y_init[:Wd - 1], y_zero[:Wd - 1])
    np.testing.assert_array_equal(y_init[Wd - 1:4], y_zero[Wd - 1:4])   # history no longer reached
