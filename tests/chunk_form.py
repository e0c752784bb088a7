"""Chunked (WY / UT) evaluation of the gated delta rule in fp64 numpy.

Test helper, not part of the product: it evaluates the same recurrence as the
oracle by a different algorithm, chunk by chunk, so that agreement across
chunk sizes pins both the oracle and the chunk algebra the kernels rely on.

Within a chunk of rows r = 1..C with entering state S0 and G_r = sum_{j<=r} g_j
(per key channel), the token recurrence of the "Delta Rule formulation"
(page "feat(kda): integrate KDA attention with tokamax backend and CP
support", Implementation Details) unrolls exactly to
    A[r,i]   = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)        i < r
    Aqk[r,i] = sum_c q_rc k_ic exp(G_rc - G_ic)               i <= r
    T = (I + A)^-1,  W = T diag(beta) (K * exp(G)),  U = T diag(beta) V
    Delta = U - W S0                     (row r: beta_r times the residual)
    O = scale [ (Q * exp(G)) S0 + Aqk Delta ]
    S_C = diag(exp(G_C)) S0 + (K * exp(G_C - G))^T Delta
"""
import numpy as np
from scipy.linalg import solve_triangular


def chunk_forward(q, k, v, g, beta, scale, chunk, initial_state=None):
    """One segment per row, no in-kernel normalisation.  Returns (o, final)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, T, H, V))
    fin = np.zeros((B, H, K, V))
    for b in range(B):
        for h in range(H):
            S = np.zeros((K, V)) if initial_state is None else \
                np.asarray(initial_state[b, h], dtype=np.float64).copy()
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(t0 + chunk, T))
                Q, Kc, Vc, gc, bc = q[b, sl, h], k[b, sl, h], v[b, sl, h], g[b, sl, h], beta[b, sl, h]
                n = Q.shape[0]
                G = np.cumsum(gc, axis=0)
                diff = G[:, None, :] - G[None, :, :]            # [r, i, c] = G_rc - G_ic
                lower = np.tril(np.ones((n, n), dtype=bool))
                diff = np.where(lower[:, :, None], diff, -np.inf)
                E = np.exp(diff)
                A = bc[:, None] * np.einsum("rc,ic,ric->ri", Kc, Kc, E)
                A = np.tril(A, -1)
                Aqk = np.einsum("rc,ic,ric->ri", Q, Kc, E)
                Gam = np.exp(G)
                IA = np.eye(n) + A
                W = solve_triangular(IA, bc[:, None] * Kc * Gam, lower=True, unit_diagonal=True)
                U = solve_triangular(IA, bc[:, None] * Vc, lower=True, unit_diagonal=True)
                D = U - W @ S
                o[b, sl, h] = scale * ((Q * Gam) @ S + Aqk @ D)
                S = np.exp(G[-1])[:, None] * S + (Kc * np.exp(G[-1][None, :] - G)).T @ D
            fin[b, h] = S
    return o, fin
