"""The block (WY) form of a short request's tokens, in fp64 on the CPU.

The spec-verify block kernel does not run the token recurrence step by step.
With G_t the running sum of the log decays through token t it forms, from the
initial state S0 alone,
    X_t = S0^T (e^{G_t} k_t),   Y_t = S0^T (e^{G_t} q_t),
    A_ts = sum_i k_s k_t e^{G_t - G_s}  (s < t),   P_ts likewise with q_t (s <= t),
then u_t = beta_t (v_t - X_t - sum_{s<t} A_ts u_s), o_t = scale (Y_t + sum_{s<=t}
P_ts u_s), and the state S_t = diag(e^{g_t}) S_{t-1} + k_t u_t^T. Under a lower
bound it takes A and P from the factored product (e^{G} k)^T (e^{-G} k). The
kernel evaluates the recurrence for u in matrix form: with
M = I + diag(beta) A_strict and Tb = M^{-1} diag(beta), u = Tb (v - X) and
o = scale (Y + P Tb (v - X)); the block's state is
diag(e^{G_last}) S0 + sum_t (e^{G_last - G_t} k_t) u_t^T. These tests restate
that algebra in numpy and check it against the oracle's token-by-token
recurrence, so the reformulation itself is pinned apart from the GPU: a
dropped term, a wrong sign, or an exclusive running sum fails them.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _block_form(q, k, v, g, b, S0, scale, factored=False):
    T = q.shape[0]
    G = np.cumsum(g, axis=0)                       # inclusive running sums
    X = (np.exp(G) * k) @ S0                      # [T, V]
    Y = (np.exp(G) * q) @ S0
    if factored:
        A = (np.exp(G) * k) @ (np.exp(-G) * k).T  # A[t, s] = sum_i k_t k_s e^{G_t - G_s}
        P = (np.exp(G) * q) @ (np.exp(-G) * k).T
    else:
        A = np.zeros((T, T))
        P = np.zeros((T, T))
        for t in range(T):
            for s in range(t + 1):
                d = np.exp(G[t] - G[s])
                A[t, s] = np.sum(k[s] * k[t] * d)
                P[t, s] = np.sum(k[s] * q[t] * d)
    u = np.zeros_like(v)
    o = np.zeros_like(v)
    for t in range(T):
        u[t] = b[t] * (v[t] - X[t] - sum(A[t, s] * u[s] for s in range(t)))
        o[t] = scale * (Y[t] + sum(P[t, s] * u[s] for s in range(t + 1)))
    S = S0.copy()
    for t in range(T):
        S = np.exp(g[t])[:, None] * S + np.outer(k[t], u[t])
    return o, S


def _block_form_matrix(q, k, v, g, b, S0, scale):
    """The matrix form: Tb and P Tb from the token-pair tables, u and o as
    products with d = v - X, the state as one rank-T update of the decayed
    initial state."""
    T = q.shape[0]
    G = np.cumsum(g, axis=0)
    X = (np.exp(G) * k) @ S0
    Y = (np.exp(G) * q) @ S0
    A = (np.exp(G) * k) @ (np.exp(-G) * k).T
    P = (np.exp(G) * q) @ (np.exp(-G) * k).T
    M = np.eye(T) + np.diag(b) @ np.tril(A, -1)
    Tb = np.linalg.solve(M, np.diag(b))
    PT = np.tril(P) @ Tb
    d = v - X
    u = Tb @ d
    o = scale * (Y + PT @ d)
    C = np.exp(G[-1][None, :] - G) * k             # [T, K]
    S = np.exp(G[-1])[:, None] * S0 + C.T @ u
    return o, S


def _case(T, K, V, lb, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, K))
    k = r.standard_normal((T, K))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, V))
    g = lb * r.uniform(0.0, 1.0, (T, K)) if lb is not None else -np.exp(r.standard_normal((T, K)))
    b = r.uniform(0.1, 0.9, T)
    S0 = 0.3 * r.standard_normal((K, V))
    return q, k, v, g, b, S0


@pytest.mark.parametrize("T", [2, 3, 5, 8])
@pytest.mark.parametrize("lb", [-5.0, None])
def test_block_form_equals_recurrence(T, lb):
    q, k, v, g, b, S0 = _case(T, 16, 8, lb, 300 + T)
    o_ref, S_ref = O.recurrent_pregated(q, k, v, g, b, S0, scale=0.7)
    o, S = _block_form(q, k, v, g, b, S0, 0.7)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T", [2, 4, 7, 8])
@pytest.mark.parametrize("lb", [-5.0, None])
def test_matrix_form_equals_recurrence(T, lb):
    q, k, v, g, b, S0 = _case(T, 16, 8, lb, 320 + T)
    o_ref, S_ref = O.recurrent_pregated(q, k, v, g, b, S0, scale=0.7)
    o, S = _block_form_matrix(q, k, v, g, b, S0, 0.7)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-10, atol=1e-12)


def test_matrix_form_padded_places_are_inert():
    # Padded places (q = k = v = 0, g = 0, beta = 0) give zero rows and
    # columns of Tb, zero u there, and leave the state that of the real tokens.
    q, k, v, g, b, S0 = _case(3, 16, 8, -5.0, 431)
    pad = lambda a: np.concatenate([a, np.zeros((5,) + a.shape[1:])])
    o8, S8 = _block_form_matrix(pad(q), pad(k), pad(v), pad(g), pad(b), S0, 1.0)
    o_ref, S_ref = O.recurrent_pregated(q, k, v, g, b, S0, scale=1.0)
    np.testing.assert_allclose(o8[:3], o_ref, rtol=1e-10, atol=1e-12)
    assert np.all(o8[3:] == 0.0)
    np.testing.assert_allclose(S8, S_ref, rtol=1e-10, atol=1e-12)


def test_factored_tables_under_a_bound_equal_the_recurrence():
    # Eight tokens at lb = -7.5: running sums down to -60, the factors e^{+-G}
    # within [e^-60, e^60].
    q, k, v, g, b, S0 = _case(8, 16, 8, -7.5, 399)
    g[:, 0] = -7.5                                 # one channel at the bound on every token
    o_ref, S_ref = O.recurrent_pregated(q, k, v, g, b, S0, scale=1.0)
    o, S = _block_form(q, k, v, g, b, S0, 1.0, factored=True)
    np.testing.assert_allclose(o, o_ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-9, atol=1e-12)


def test_padded_token_places_change_nothing():
    # A request of 5 tokens in 8 places: places 5..7 carry q = k = v = 0,
    # g = 0 and beta = 0, so outputs and state are those of the 5 tokens.
    q, k, v, g, b, S0 = _case(5, 16, 8, -5.0, 411)
    pad = lambda a: np.concatenate([a, np.zeros((3,) + a.shape[1:])])
    o8, S8 = _block_form(pad(q), pad(k), pad(v), pad(g), pad(b), S0, 1.0)
    o_ref, S_ref = O.recurrent_pregated(q, k, v, g, b, S0, scale=1.0)
    np.testing.assert_allclose(o8[:5], o_ref, rtol=1e-11, atol=1e-12)
    assert np.all(o8[5:] == 0.0)
    np.testing.assert_allclose(S8, S_ref, rtol=1e-11, atol=1e-12)
