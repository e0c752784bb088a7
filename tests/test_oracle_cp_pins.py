"""Pins of the context-parallel oracle (transition and slice plan) against
closed forms, the token-loop oracle and a hand-worked example.  Source: the
page "feat(kda): integrate KDA attention with tokamax backend and CP support"
(Context Parallelism Support; its CP tests: splitting T over 2 or 4 ranks
reproduces the unsplit forward, with packed segments that cross a split or
begin exactly at one) and the Delta Rule formulation on the same page.
None of these re-types the oracle: each compares it with a closed form, the
separate token-loop oracle in C, or an invariant."""
import numpy as np
import pytest

import oracle
from oracle import cp


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(B, T, H, K, V, seed):
    q, k, v = _unit(_rand((B, T, H, K), seed)), _unit(_rand((B, T, H, K), seed + 1)), _rand((B, T, H, V), seed + 2)
    g = np.log(1 / (1 + np.exp(-_rand((B, T, H, K), seed + 3))))
    beta = 1 / (1 + np.exp(-_rand((B, T, H), seed + 4)))
    f = lambda a: a.astype(np.float32)
    return f(q), f(k), f(v), f(g), f(beta)


# ---------------------------------------------------------------- transition

def test_transition_with_zero_beta_is_the_total_decay():
    """beta = 0 leaves only the decay: M = diag(exp(sum_t g_t))."""
    B, T, H, K = 1, 9, 2, 6
    _, k, _, g, _ = _case(B, T, H, K, 3, 10)
    M = cp.transition(k, g, np.zeros((B, T, H), np.float32))
    for h in range(H):
        np.testing.assert_allclose(M[0, h], np.diag(np.exp(g[0, :, h].astype(np.float64).sum(0))), rtol=1e-13,
                                   atol=1e-300)


def test_transition_with_orthonormal_keys_is_a_projector():
    """g = 0, beta = 1 and orthonormal keys: each step removes one key
    direction, M = I - sum_t k_t k_t^T."""
    K, T = 16, 5
    had = np.array([[1.0]])
    while had.shape[0] < K:                       # Sylvester's Hadamard matrix: rows / 4 are
        had = np.block([[had, had], [had, -had]])  # orthonormal and exact in fp32
    k = (had[[3, 12, 0, 7, 9]] / 4.0).astype(np.float32)[None, :, None, :]
    M = cp.transition(k, np.zeros_like(k), np.ones((1, T, 1), np.float32))
    kd = k[0, :, 0].astype(np.float64)
    np.testing.assert_allclose(M[0, 0], np.eye(K) - kd.T @ kd, atol=1e-12)


@pytest.mark.parametrize("l2norm", [False, True])
def test_transition_is_the_derivative_of_the_final_state(l2norm):
    """The token-loop oracle's end state is affine in the start state with
    slope M: fin(S0) - fin(0) = M S0 (fp64 build)."""
    B, T, H, K, V = 2, 40, 2, 8, 5
    q, k, v, g, beta = _case(B, T, H, K, V, 20)
    if l2norm:
        k = (3.0 * _rand(k.shape, 25)).astype(np.float32)
    S0 = _rand((B, H, K, V), 26).astype(np.float32)
    _, f1 = oracle.kda_forward(q, k, v, g, beta, initial_state=S0, output_final_state=True, use_qk_l2norm=l2norm)
    _, f0 = oracle.kda_forward(q, k, v, g, beta, output_final_state=True, use_qk_l2norm=l2norm)
    M = cp.transition(k, g, beta, use_qk_l2norm=l2norm)
    np.testing.assert_allclose(f1 - f0, M @ S0.astype(np.float64), rtol=1e-9, atol=1e-11)


def test_transition_composes_over_a_split():
    """The product runs latest-first: M(whole row) = M(second part) M(first part)."""
    B, T, H, K = 1, 30, 1, 6
    _, k, _, g, beta = _case(B, T, H, K, 2, 30)
    M = cp.transition(k, g, beta)
    for t1 in (1, 13, 29):
        M1 = cp.transition(k[:, :t1], g[:, :t1], beta[:, :t1])
        M2 = cp.transition(k[:, t1:], g[:, t1:], beta[:, t1:])
        np.testing.assert_allclose(M, M2 @ M1, rtol=1e-11, atol=1e-14)


def test_transition_is_zero_without_one_spanning_segment():
    """A boundary or padding anywhere between the first and the last token
    cuts the end state off from the start state; one segment over the whole
    row (any id) gives the same M as no segment ids."""
    B, T, H, K = 5, 12, 1, 4
    _, k, _, g, beta = _case(B, T, H, K, 2, 40)
    seg = np.ones((B, T), np.int32)
    seg[0, 6:] = 2          # a boundary
    seg[1, -1] = 0          # padding at the end
    seg[2, 0] = 0           # padding at the start
    seg[3, 5] = 0           # padding inside
    seg[4] = 7              # one segment, another id
    M = cp.transition(k, g, beta, segment_ids=seg)
    assert np.all(M[:4] == 0.0)
    np.testing.assert_array_equal(M[4], cp.transition(k[4:], g[4:], beta[4:])[0])


# ---------------------------------------------------------------- slice plan

def test_plan_on_a_hand_worked_example():
    """Row ids, cut into 4 slices of 4 tokens:
        [1 1 1 2 | 2 2 0 3 | 3 3 3 3 | 4 5 5 0]
    Segments in order: 0 = '1' (0-3), 1 = '2' (3-6), 2 = '3' (7-12), 3 = '4'
    (12-13), 4 = '5' (13-15).  Slice 1 continues segment 1, slice 2 continues
    segment 2, slice 3 begins with a new segment exactly at the cut.  A
    second row is padding except for one segment that starts at a cut and
    one that runs over two cuts:
        [0 0 0 0 | 1 1 1 1 | 0 2 2 2 | 2 2 2 2]"""
    seg = np.array([[1, 1, 1, 2, 2, 2, 0, 3, 3, 3, 3, 3, 4, 5, 5, 0],
                    [0, 0, 0, 0, 1, 1, 1, 1, 0, 2, 2, 2, 2, 2, 2, 2]], np.int32)
    expect = np.array([[[0, 0, 2, 0], [1, 1, 2, 0], [1, 2, 1, 0], [0, 3, 2, 0]],
                       [[0, 0, 0, 0], [0, 0, 1, 0], [0, 1, 1, 0], [1, 1, 1, 0]]], np.int32)
    np.testing.assert_array_equal(cp.cp_plan(seg, 2, 16, 4, 5), expect)
    over = cp.cp_plan(seg, 2, 16, 4, 4)
    np.testing.assert_array_equal(over[0, :, 3], [0, 0, 0, 1])     # segment 4 has no slot
    fixed = cp.cp_plan(None, 2, 16, 4, 1)
    np.testing.assert_array_equal(fixed[:, :, 0], [[0, 1, 1, 1]] * 2)
    assert np.all(fixed[:, :, 1] == 0) and np.all(fixed[:, :, 2] == 1) and np.all(fixed[:, :, 3] == 0)


def test_plan_counts_add_up():
    """Over a row, the segments a slice begins (count minus continued) sum to
    the row's segment count, and consecutive slices' first indices follow."""
    rng = np.random.default_rng(50)
    B, T, P = 6, 48, 6
    seg = np.repeat(rng.integers(0, 4, (B, T // 3)), 3, axis=1).astype(np.int32)
    plan = cp.cp_plan(seg, B, T, P, 64)
    for b in range(B):
        n = len(cp.segment_runs(seg[b]))
        assert int(np.sum(plan[b, :, 2] - plan[b, :, 0])) == n
        for r in range(1, P):
            assert plan[b, r, 1] == plan[b, r - 1, 1] + plan[b, r - 1, 2] - plan[b, r, 0]


# ------------------------------------------------- chaining in the oracle

def _cp_run(q, k, v, g, beta, seg, S0, n_states, P):
    """The state chaining written out with the oracle alone: every slice runs
    with a zero start state for the segment it continues, the chain
    C_{r+1} = E_r + [slice r continues] M_r C_r gives the true carried
    states, and a second run of each slice starts from them.  Per-segment
    states move between the row layout and the slice layout by the plan."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    L = T // P
    plan = cp.cp_plan(seg, B, T, P, n_states)
    o = np.zeros((B, T, H, V))
    fin = np.zeros((B, n_states, H, K, V))

    def run_slice(b, r, carried_state):
        cont, first, count, _ = plan[b, r]
        sl = slice(r * L, (r + 1) * L)
        local = np.zeros((1, max(count, 1), H, K, V))
        for l in range(count):
            if l == 0 and cont:
                local[0, 0] = carried_state
            elif S0 is not None:
                local[0, l] = S0[b, first + l]
        args = [a[b:b + 1, sl] for a in (q, k, v, g, beta)]
        ol, fl = oracle.kda_forward(*args, initial_state=local.astype(np.float32), output_final_state=True,
                                    segment_ids=seg[b:b + 1, sl], max_segments=max(count, 1))
        M = cp.transition(args[1], args[3], args[4], segment_ids=seg[b:b + 1, sl])[0]
        return ol[0], fl[0], M, sl, first, count

    for b in range(B):
        carries = [np.zeros((H, K, V)) for _ in range(P)]
        for r in range(P - 1):                                  # pass 1 and the chain
            _, fl, M, _, _, count = run_slice(b, r, np.zeros((H, K, V)))
            if plan[b, r + 1, 0]:
                end = fl[count - 1]
                carries[r + 1] = end + (M @ carries[r] if plan[b, r, 0] else 0.0)
        for r in range(P):                                      # pass 2
            ol, fl, _, sl, first, count = run_slice(b, r, carries[r])
            o[b, sl] = ol
            for l in range(count):
                fin[b, first + l] = fl[l]                       # a later slice overwrites
    return o, fin


@pytest.mark.parametrize("P", [2, 4])
def test_chaining_reproduces_the_unsplit_run(P):
    """CP equivalence, the pages' check, on the oracle: cutting rows into P
    slices and chaining the state gives the unsplit result (segments crossing
    a cut, one beginning exactly at a cut, padding at a cut, start states)."""
    B, T, H, K, V = 2, 32, 2, 6, 5
    q, k, v, g, beta = _case(B, T, H, K, V, 60)
    seg = np.zeros((B, T), np.int32)
    seg[0, 0:5], seg[0, 5:19], seg[0, 19:24], seg[0, 24:31] = 1, 2, 3, 4     # 24 = a cut for P = 4
    seg[1, 0:8], seg[1, 9:32] = 1, 2                                     # padding at token 8 (a cut's start)
    n_states = 5
    S0 = _rand((B, n_states, H, K, V), 61, 0.5).astype(np.float32)
    o, fin = oracle.kda_forward(q, k, v, g, beta, initial_state=S0, output_final_state=True, segment_ids=seg,
                                max_segments=n_states)
    oc, fc = _cp_run(q, k, v, g, beta, seg, S0, n_states, P)
    # the oracle takes start states in fp32, so each carried state is rounded once
    assert oracle.rel_err(oc, o) < 1e-6
    assert oracle.rel_err(fc, fin) < 1e-6


def _cp_bwd_run(q, k, v, g, beta, seg, S0, d_o, d_fin, n_states, P):
    """The gradient chaining written out with the oracle alone: the slices'
    start states come from the forward chain; each slice's backward first
    runs with a zero gradient for the state it hands on, the reverse chain
    X_r = [r+1 continues] (dInit_{r+1} + M_{r+1}^T X_{r+1}) gives the true
    hand-off gradients, and a second backward of each slice uses them."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    L = T // P
    plan = cp.cp_plan(seg, B, T, P, n_states)
    out = {n: np.zeros(a.shape) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    d_init = np.zeros((B, n_states, H, K, V))
    for b in range(B):
        # forward chain: the state each continued slice starts from
        carries = [np.zeros((H, K, V)) for _ in range(P)]
        for r in range(P - 1):
            cont, first, count, _ = plan[b, r]
            sl = slice(r * L, (r + 1) * L)
            local = np.zeros((1, max(count, 1), H, K, V))
            for l in range(count):
                local[0, l] = carries[r] if (l == 0 and cont) else (S0[b, first + l] if S0 is not None else 0.0)
            args = [a[b:b + 1, sl] for a in (q, k, v, g, beta)]
            _, fl = oracle.kda_forward(*args, initial_state=local.astype(np.float32), output_final_state=True,
                                       segment_ids=seg[b:b + 1, sl], max_segments=max(count, 1))
            if plan[b, r + 1, 0]:
                carries[r + 1] = fl[0, count - 1]

        def slice_bwd(r, x_out):
            cont, first, count, _ = plan[b, r]
            sl = slice(r * L, (r + 1) * L)
            local = np.zeros((1, max(count, 1), H, K, V))
            dfl = np.zeros((1, max(count, 1), H, K, V))
            for l in range(count):
                local[0, l] = carries[r] if (l == 0 and cont) else (S0[b, first + l] if S0 is not None else 0.0)
                handed_on = l == count - 1 and r + 1 < P and plan[b, r + 1, 0]
                dfl[0, l] = x_out if handed_on else d_fin[b, first + l]
            args = [a[b:b + 1, sl] for a in (q, k, v, g, beta)]
            gr = oracle.kda_backward(*args, d_o[b:b + 1, sl], initial_state=local.astype(np.float32),
                                     d_final_state=dfl, segment_ids=seg[b:b + 1, sl], max_segments=max(count, 1))
            M = cp.transition(args[1], args[3], args[4], segment_ids=seg[b:b + 1, sl])[0]
            return gr, M, sl, first, count, cont

        # pass 1 and the reverse chain
        X = [np.zeros((H, K, V)) for _ in range(P)]
        for r in range(P - 1, 0, -1):
            gr, M, _, _, _, cont = slice_bwd(r, np.zeros((H, K, V)))   # pass 1: nothing handed on
            if cont:
                X[r - 1] = gr["d_initial_state"][0, 0] + np.swapaxes(M, -1, -2) @ X[r]
        # pass 2
        for r in range(P):
            gr, _, sl, first, count, cont = slice_bwd(r, X[r])
            for n in out:
                out[n][b, sl] = gr[n][0]
            for l in range(count):
                if not (l == 0 and cont):
                    d_init[b, first + l] = gr["d_initial_state"][0, l]
    out["d_initial_state"] = d_init
    return out


@pytest.mark.parametrize("P", [2, 4])
def test_gradient_chaining_reproduces_the_unsplit_backward(P):
    """CP gradient equivalence, the pages' check, on the oracle."""
    B, T, H, K, V = 2, 32, 2, 6, 5
    q, k, v, g, beta = _case(B, T, H, K, V, 70)
    seg = np.zeros((B, T), np.int32)
    seg[0, 0:5], seg[0, 5:19], seg[0, 19:24], seg[0, 24:31] = 1, 2, 3, 4
    seg[1, 0:8], seg[1, 9:32] = 1, 2
    n_states = 5
    S0 = _rand((B, n_states, H, K, V), 71, 0.5).astype(np.float32)
    d_o = _rand((B, T, H, V), 72)
    d_fin = _rand((B, n_states, H, K, V), 73)
    ref = oracle.kda_backward(q, k, v, g, beta, d_o, initial_state=S0, d_final_state=d_fin, segment_ids=seg,
                              max_segments=n_states)
    got = _cp_bwd_run(q, k, v, g, beta, seg, S0, d_o, d_fin, n_states, P)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"):
        # the oracle takes start states in fp32, so each carried state is rounded once
        assert oracle.rel_err(got[n], ref[n]) < 1e-5, n
