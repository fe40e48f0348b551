"""Pins of the pair-decay oracle (oracle/vector_decay.py), CPU only.

  * reduction: when every pair of a head has the same decay, each form equals the
    scalar-decay oracle (itself pinned by brute force, closed forms and library cases);
  * decomposition: the score is a sum over coordinate pairs, so retention with pair
    decays equals the sum over pairs j of scalar retention with decay gamma[h, j] applied
    to q, k (and the initial state's rows) restricted to pair j — a decay read from the
    wrong pair, a per-coordinate instead of per-pair index or a transposed [H, d_k/2]
    table fails it;
  * the brute-force sum, the parallel, recurrent and chunkwise forms agree (ragged last
    chunk, positions, initial and final state), and two chained chunkwise calls equal one.
A dropped decay factor, an off-by-one exponent (xi = gamma^j instead of gamma^(j+1), zeta
= gamma^(L-j)) or a decay applied once per pair instead of per coordinate row fails one
of them.
"""
import numpy as np
import pytest

import oracle as O


def inputs(seed, B=1, H=2, N=11, dk=6, dv=4, spread=(0.35, 0.999)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    gamma = rng.uniform(*spread, (H, dk // 2))
    theta = rng.uniform(0.05, 1.2, dk // 2)
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    return q, k, v, gamma, theta, S0


def pair_only(x, j):
    y = np.zeros_like(x)
    y[..., 2 * j:2 * j + 2] = x[..., 2 * j:2 * j + 2]
    return y


def test_equal_pair_decays_reduce_to_the_scalar_oracle():
    q, k, v, _, theta, S0 = inputs(1, B=2, H=3, N=13, dk=8, dv=5)
    gs = np.array([0.9, 0.55, 1.0])
    gv = np.repeat(gs[:, None], 4, axis=1)
    np.testing.assert_allclose(O.brute_force_vec(q, k, v, gv, theta, 3, 0.8, S0),
                               O.brute_force(q, k, v, gs, theta, 3, 0.8, S0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.parallel_vec(q, k, v, gv, theta, 5, 0.7, norm_r=True),
                               O.parallel(q, k, v, gs, theta, 5, 0.7, norm_r=True), rtol=1e-12, atol=1e-12)
    o1, s1 = O.recurrent_vec(q, k, v, gv, theta, 2, 1.1, S0)
    o2, s2 = O.recurrent(q, k, v, gs, theta, 2, 1.1, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)
    o1, s1 = O.chunkwise_vec(q, k, v, gv, theta, 5, 7, 0.9, S0)
    o2, s2 = O.chunkwise(q, k, v, gs, theta, 5, 7, 0.9, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)
    d1, t1 = O.recurrent_step_vec(q[:, :, 0], k[:, :, 0], v[:, :, 0], gv, theta, 40, 0.6, S0)
    d2, t2 = O.recurrent_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], gs, theta, 40, 0.6, S0)
    np.testing.assert_allclose(d1, d2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(t1, t2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("form", ["brute", "parallel", "recurrent", "chunkwise", "step"])
def test_pair_decays_decompose_into_scalar_retentions(form):
    q, k, v, gv, theta, S0 = inputs(2, B=1, H=2, N=9, dk=6, dv=3)
    H, P = gv.shape
    if form == "step":
        got, got_s = O.recurrent_step_vec(q[:, :, 3], k[:, :, 3], v[:, :, 3], gv, theta, 17, 0.9, S0)
    elif form == "brute":
        got = O.brute_force_vec(q, k, v, gv, theta, 4, 0.9, S0)
    elif form == "parallel":
        got = O.parallel_vec(q, k, v, gv, theta, 4, 0.9)
    elif form == "recurrent":
        got, got_s = O.recurrent_vec(q, k, v, gv, theta, 4, 0.9, S0)
    else:
        got, got_s = O.chunkwise_vec(q, k, v, gv, theta, 4, 4, 0.9, S0)
    want = np.zeros_like(got)
    want_s = np.zeros_like(S0)
    for h in range(H):
        for j in range(P):
            gj = np.full(H, gv[h, j])
            qj, kj, sj = pair_only(q, j), pair_only(k, j), np.zeros_like(S0)
            sj[:, :, 2 * j:2 * j + 2] = S0[:, :, 2 * j:2 * j + 2]
            if form == "step":
                o, s = O.recurrent_step(qj[:, :, 3], kj[:, :, 3], v[:, :, 3], gj, theta, 17, 0.9, sj)
            elif form == "brute":
                o, s = O.brute_force(qj, kj, v, gj, theta, 4, 0.9, sj), None
            elif form == "parallel":
                o, s = O.parallel(qj, kj, v, gj, theta, 4, 0.9), None
            elif form == "recurrent":
                o, s = O.recurrent(qj, kj, v, gj, theta, 4, 0.9, sj)
            else:
                o, s = O.chunkwise(qj, kj, v, gj, theta, 4, 4, 0.9, sj)
            want[:, h] += o[:, h]
            if s is not None:
                # only pair j's rows of the state belong to this retention
                want_s[:, h, 2 * j:2 * j + 2] = s[:, h, 2 * j:2 * j + 2]
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    if form in ("recurrent", "chunkwise", "step"):
        np.testing.assert_allclose(got_s, want_s, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("chunk,pos0,alpha", [(1, 0, 1.0), (4, 9, 0.6), (5, 0, 1.0), (11, 1000, 1.2),
                                              (30, 3, 0.5)])
def test_forms_agree_with_the_brute_force_sum(chunk, pos0, alpha):
    q, k, v, gv, theta, S0 = inputs(3, B=2, H=2, N=11, dk=8, dv=5, spread=(0.05, 1.0))
    ref = O.brute_force_vec(q, k, v, gv, theta, pos0, alpha, S0)
    rec, s_rec = O.recurrent_vec(q, k, v, gv, theta, pos0, alpha, S0)
    chk, s_chk = O.chunkwise_vec(q, k, v, gv, theta, chunk, pos0, alpha, S0)
    np.testing.assert_allclose(rec, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(chk, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s_chk, s_rec, rtol=1e-11, atol=1e-11)
    par = O.parallel_vec(q, k, v, gv, theta, pos0, alpha)
    ref0 = O.brute_force_vec(q, k, v, gv, theta, pos0, alpha)
    np.testing.assert_allclose(par, ref0, rtol=1e-11, atol=1e-11)


def test_final_state_is_the_decayed_sum_of_outer_products():
    """S_N = diag(γ^N) S0 + Σ_s diag(γ^(N-1-s)) Kh_s^T V_s, written out per state row."""
    q, k, v, gv, theta, S0 = inputs(4, B=1, H=1, N=7, dk=4, dv=3)
    _, S = O.chunkwise_vec(q, k, v, gv, theta, 3, 2, 1.0, S0)
    kh = O.rotate(k, np.arange(7) + 2, theta)
    for d in range(4):
        g = gv[0, d // 2]
        want = g ** 7 * S0[0, 0, d] + sum(g ** (6 - s) * kh[0, 0, s, d] * v[0, 0, s] for s in range(7))
        np.testing.assert_allclose(S[0, 0, d], want, rtol=1e-12, atol=1e-12)


def test_chained_chunkwise_calls_equal_one_call():
    q, k, v, gv, theta, S0 = inputs(5, B=1, H=2, N=14, dk=6, dv=4)
    full, s_full = O.chunkwise_vec(q, k, v, gv, theta, 4, 10, 1.0, S0)
    M = 6
    a, s_mid = O.chunkwise_vec(q[:, :, :M], k[:, :, :M], v[:, :, :M], gv, theta, 4, 10, 1.0, S0)
    b, s_end = O.chunkwise_vec(q[:, :, M:], k[:, :, M:], v[:, :, M:], gv, theta, 4, 10 + M, 1.0, s_mid)
    np.testing.assert_allclose(np.concatenate([a, b], axis=2), full, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s_end, s_full, rtol=1e-11, atol=1e-11)
