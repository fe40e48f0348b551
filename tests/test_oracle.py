"""Pins for the fp64 oracle: brute force, closed forms, invariants and library
special cases. None of these compares the oracle with itself through a retyped
formula; each would fail under a plausible slip (dropped term, wrong sign,
wrong pairing, transposed operand, off-by-one decay, wrong variance).
CPU only."""
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = Path(__file__).parent / "golden"


def rand(rng, *shape):
    return rng.standard_normal(shape)


def tiny_inputs(seed=0, B=1, H=2, N=12, dk=6, dv=5):
    rng = np.random.default_rng(seed)
    q, k, v = rand(rng, B, H, N, dk), rand(rng, B, H, N, dk), rand(rng, B, H, N, dv)
    gamma = np.array([0.9, 0.6, 0.97, 0.8][:H])
    theta = rng.uniform(0.1, 1.3, dk // 2)
    return q, k, v, gamma, theta


# ---- T1: brute-force sum of the defining closed form --------------------------------

@pytest.mark.parametrize("pos0,alpha", [(0, 1.0), (3, 0.7), (1000, 1.3)])
def test_t1_forms_match_brute_force(pos0, alpha):
    q, k, v, gamma, theta = tiny_inputs(1)
    ref = O.brute_force(q, k, v, gamma, theta, pos0, alpha)
    par = O.parallel(q, k, v, gamma, theta, pos0, alpha)
    rec, _ = O.recurrent(q, k, v, gamma, theta, pos0, alpha)
    chk, _ = O.chunkwise(q, k, v, gamma, theta, 5, pos0, alpha)
    for x in (par, rec, chk):
        np.testing.assert_allclose(x, ref, rtol=1e-11, atol=1e-11)


def test_t1_brute_force_with_initial_state():
    q, k, v, gamma, theta = tiny_inputs(2)
    rng = np.random.default_rng(7)
    S0 = rand(rng, 1, 2, 6, 5)
    ref = O.brute_force(q, k, v, gamma, theta, 4, 0.9, S0)
    rec, _ = O.recurrent(q, k, v, gamma, theta, 4, 0.9, S0)
    chk, _ = O.chunkwise(q, k, v, gamma, theta, 4, 4, 0.9, S0)
    np.testing.assert_allclose(rec, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(chk, ref, rtol=1e-11, atol=1e-11)


# ---- T2/T3: the three forms agree; structural special cases -------------------------

@pytest.mark.parametrize("chunk", [1, 3, 16, 23, 5, 40])
def test_t2_chunkwise_equals_recurrent(chunk):
    q, k, v, gamma, theta = tiny_inputs(3, B=2, H=3, N=23, dk=8, dv=7)
    rng = np.random.default_rng(11)
    S0 = rand(rng, 2, 3, 8, 7)
    rec, Sr = O.recurrent(q, k, v, gamma, theta, 2, 1.1, S0)
    chk, Sc = O.chunkwise(q, k, v, gamma, theta, chunk, 2, 1.1, S0)
    np.testing.assert_allclose(chk, rec, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Sc, Sr, rtol=1e-11, atol=1e-11)


def test_t3_chunk_n_zero_state_is_parallel():
    q, k, v, gamma, theta = tiny_inputs(4, N=17)
    chk, _ = O.chunkwise(q, k, v, gamma, theta, 17, 0, 0.5)
    par = O.parallel(q, k, v, gamma, theta, 0, 0.5)
    np.testing.assert_allclose(chk, par, rtol=1e-11, atol=1e-11)


def test_state_closed_form():
    """S_N = Σ_s γ^(N-1-s) Kh_s^T v_s (the [hwhale] unrolled state sum with A = γ)."""
    q, k, v, gamma, theta = tiny_inputs(5, N=9)
    _, S = O.recurrent(q, k, v, gamma, theta, 3, 1.0)
    pos = np.arange(9) + 3
    for h in range(2):
        kh = np.array([[complex(k[0, h, s, 2 * j], k[0, h, s, 2 * j + 1]) * np.exp(1j * pos[s] * theta[j])
                        for j in range(3)] for s in range(9)])
        kr = np.empty((9, 6))
        kr[:, 0::2], kr[:, 1::2] = kh.real, kh.imag
        ref = sum(gamma[h] ** (8 - s) * np.outer(kr[s], v[0, h, s]) for s in range(9))
        np.testing.assert_allclose(S[0, h], ref, rtol=1e-12, atol=1e-12)


def test_recurrent_step_chain_equals_recurrent():
    q, k, v, gamma, theta = tiny_inputs(6, N=7)
    rng = np.random.default_rng(3)
    S = rand(rng, 1, 2, 6, 5)
    rec, Sr = O.recurrent(q, k, v, gamma, theta, 10, 0.8, S)
    for t in range(7):
        o, S = O.recurrent_step(q[:, :, t], k[:, :, t], v[:, :, t], gamma, theta, 10 + t, 0.8, S)
        np.testing.assert_allclose(o, rec[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sr, rtol=1e-12, atol=1e-12)


# ---- T4: closed forms ---------------------------------------------------------------

def test_t4a_geometric_series_golden():
    """θ=0, q=k=e0, v≡1 ⇒ O_t = Σ_{m<=t} γ^m = (1-γ^{t+1})/(1-γ): exact rationals
    stored in tests/golden/geometric_series.txt."""
    lines = (GOLDEN / "geometric_series.txt").read_text().split("\n")
    rows = [l.split() for l in lines if l and not l.startswith("#")]
    gam = float(Fraction(rows[0][1]))
    N = len(rows) - 1
    q = np.zeros((1, 1, N, 2)); q[..., 0] = 1
    v = np.ones((1, 1, N, 1))
    for form in ("parallel", "recurrent", "chunkwise"):
        if form == "parallel":
            out = O.parallel(q, q, v, [gam], [0.0])
        elif form == "recurrent":
            out, _ = O.recurrent(q, q, v, [gam], [0.0])
        else:
            out, _ = O.chunkwise(q, q, v, [gam], [0.0], 7)
        for t, row in enumerate(rows[1:]):
            assert int(row[0]) == t
            assert abs(out[0, 0, t, 0] - float(Fraction(row[1]))) < 1e-13


@pytest.mark.parametrize("gam,th", [(0.9, 0.3), (0.75, 2.0), (1.0, 0.1)])
def test_t4b_rotation_sign_closed_form(gam, th):
    """d_k=2, q=(1,0), k=(0,1), v≡1 ⇒ Qh_t·Kh_s = sin((t-s)θ) and
    O_t = Im[(1-(γe^{iθ})^{t+1})/(1-γe^{iθ})]. The sign pins e^{+ipθ} on both q and k
    with k conjugated."""
    N = 20
    q = np.zeros((1, 1, N, 2)); q[..., 0] = 1
    k = np.zeros((1, 1, N, 2)); k[..., 1] = 1
    v = np.ones((1, 1, N, 1))
    z = gam * np.exp(1j * th)
    ref = np.array([((1 - z ** (t + 1)) / (1 - z)).imag for t in range(N)])
    for out in (O.parallel(q, k, v, [gam], [th], 5),
                O.recurrent(q, k, v, [gam], [th], 5)[0],
                O.chunkwise(q, k, v, [gam], [th], 6, 5)[0],
                O.brute_force(q, k, v, [gam], [th], 5)):
        np.testing.assert_allclose(out[0, 0, :, 0], ref, atol=1e-12)


def test_t4b_adjacent_pairing():
    """d_k=4 with distinct angles: e0 and e1 form one pair (adjacent reading), so the
    score of q=e0 with k=e1 is sin((t-s)θ_0); under a half-split pairing it would be 0."""
    N, th = 10, [0.4, 1.7]
    q = np.zeros((1, 1, N, 4)); q[..., 0] = 1
    k = np.zeros((1, 1, N, 4)); k[..., 1] = 1
    v = np.ones((1, 1, N, 1))
    z = 0.8 * np.exp(1j * th[0])
    ref = np.array([((1 - z ** (t + 1)) / (1 - z)).imag for t in range(N)])
    np.testing.assert_allclose(O.parallel(q, k, v, [0.8], th)[0, 0, :, 0], ref, atol=1e-12)
    np.testing.assert_allclose(O.recurrent(q, k, v, [0.8], th)[0][0, 0, :, 0], ref, atol=1e-12)


def test_t4c_impulse_causality():
    q, k, v, gamma, theta = tiny_inputs(8, N=15)
    s0 = 6
    v = np.zeros_like(v); v[:, :, s0, :] = [1.0, -2.0, 0.5, 3.0, 1.5]
    out, _ = O.chunkwise(q, k, v, gamma, theta, 4, 2, 1.0)
    pos = np.arange(15) + 2
    qh, kh = O.rotate(q, pos, theta), O.rotate(k, pos, theta)
    for h in range(2):
        for t in range(15):
            if t < s0:
                assert np.all(out[0, h, t] == 0.0)
            else:
                c = gamma[h] ** (t - s0) * (qh[0, h, t] @ kh[0, h, s0])
                np.testing.assert_allclose(out[0, h, t], c * v[0, h, s0], rtol=1e-12, atol=1e-12)


def _unit_case(N, ksign=None):
    q = np.zeros((1, 1, N, 2)); q[..., 0] = 1
    k = q.copy()
    if ksign is not None:
        k[0, 0, :, 0] = ksign
    v = np.ones((1, 1, N, 1))
    return q, k, v


def test_t4d_both_rescalings_give_one():
    """θ=0, q=k=e0, v≡1, α=1 with D̃ and R̃ ⇒ O_t = 1 for every t."""
    gam = 0.93
    q, k, v = _unit_case(30)
    out = O.parallel(q, k, v, [gam], [0.0], norm_d=True, norm_r=True)
    np.testing.assert_allclose(out[0, 0, :, 0], 1.0, atol=1e-12)


def test_t4d_row_rescalings_separately():
    gam, N = 0.9, 40
    q, k, v = _unit_case(N)
    G = np.array([(1 - gam ** (t + 1)) / (1 - gam) for t in range(N)])
    # D̃ only: O_t = G_t / sqrt(G_t)
    np.testing.assert_allclose(O.parallel(q, k, v, [gam], [0.0], norm_d=True)[0, 0, :, 0],
                               np.sqrt(G), rtol=1e-12)
    # R̃ only with α = 0.1: O_t = 0.1 G_t / max(0.1 G_t, 1)
    np.testing.assert_allclose(O.parallel(q, k, v, [gam], [0.0], alpha=0.1, norm_r=True)[0, 0, :, 0],
                               0.1 * G / np.maximum(0.1 * G, 1.0), rtol=1e-12)


def test_t4d_signed_row_sum():
    """k_s = (-1)^s e0 gives R_ts = γ^{t-s}(-1)^s; the SIGNED row sum is small, so
    max(|Σ|,1) = 1 and O_t = Σ_s R_ts; a sum of |R| would divide by G_t instead."""
    gam, N = 0.8, 12
    q, k, v = _unit_case(N, ksign=(-1.0) ** np.arange(N))
    out = O.parallel(q, k, v, [gam], [0.0], norm_r=True)[0, 0, :, 0]
    ref = np.array([sum(gam ** (t - s) * (-1) ** s for s in range(t + 1)) for t in range(N)])
    assert np.all(np.abs(ref) <= 1.0)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


# ---- T5: GroupNorm ------------------------------------------------------------------

def test_t5_groupnorm_matches_torch_group_norm():
    """Per-(token, head) statistics over d_v equal torch's group_norm with one group per
    head over channels laid out as [head, d_v]."""
    rng = np.random.default_rng(9)
    B, H, N, dv = 2, 3, 5, 8
    x = rand(rng, B, H, N, dv)
    w, b = rand(rng, H, dv), rand(rng, H, dv)
    ours = O.group_norm(x, 1e-5, w, b)
    xt = torch.from_numpy(x).permute(0, 2, 1, 3).reshape(B * N, H * dv)
    ref = torch.nn.functional.group_norm(xt, H, torch.from_numpy(w).reshape(-1),
                                         torch.from_numpy(b).reshape(-1), 1e-5)
    ref = ref.reshape(B, N, H, dv).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-10)


def test_t5_scale_invariance_closed_form():
    """GN_ε(c·x) = (x-μ)/sqrt(σ² + ε/c²); at ε=0 GN(cx) = GN(x) (the [hwhale] remark that
    the rescalings only multiply the GN input by a per-row constant)."""
    rng = np.random.default_rng(10)
    x = rand(rng, 1, 2, 4, 16)
    mu = x.mean(-1, keepdims=True)
    var = x.var(-1, keepdims=True)
    for c in (1e-3, 0.5, 7.0):
        np.testing.assert_allclose(O.group_norm(c * x, 1e-5), (x - mu) / np.sqrt(var + 1e-5 / c ** 2),
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(O.group_norm(c * x, 0.0), O.group_norm(x, 0.0), rtol=1e-10, atol=1e-12)
    y = O.group_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(-1), 1.0, rtol=1e-12)


def test_t5_rescalings_leave_gn_unchanged_at_eps0():
    q, k, v, gamma, theta = tiny_inputs(12, N=14)
    a = O.group_norm(O.parallel(q, k, v, gamma, theta, 0, 1.0), 0.0)
    b = O.group_norm(O.parallel(q, k, v, gamma, theta, 0, 0.25, norm_d=True, norm_r=True), 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


# ---- T6-T10 -------------------------------------------------------------------------

def test_t6_relative_position_shift():
    q, k, v, gamma, theta = tiny_inputs(13, N=11)
    a = O.parallel(q, k, v, gamma, theta, 0)
    b = O.parallel(q, k, v, gamma, theta, 12345)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_t7_resume():
    q, k, v, gamma, theta = tiny_inputs(14, N=20)
    full, Sf = O.chunkwise(q, k, v, gamma, theta, 4, 0)
    M = 9
    a, Sa = O.chunkwise(q[:, :, :M], k[:, :, :M], v[:, :, :M], gamma, theta, 4, 0)
    b, Sb = O.chunkwise(q[:, :, M:], k[:, :, M:], v[:, :, M:], gamma, theta, 4, M, 1.0, Sa)
    np.testing.assert_allclose(np.concatenate([a, b], 2), full, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Sb, Sf, rtol=1e-11, atol=1e-11)
    S = Sa
    for t in range(M, 20):
        o, S = O.recurrent_step(q[:, :, t], k[:, :, t], v[:, :, t], gamma, theta, t, 1.0, S)
        np.testing.assert_allclose(o, full[:, :, t], rtol=1e-11, atol=1e-11)


def test_t8_linear_attention_limit():
    """γ=1, θ=0: o_t = q_t · Σ_{s<=t} k_s^T v_s (causal linear attention by cumulative sum)."""
    q, k, v, _, _ = tiny_inputs(15, N=13)
    kv = np.cumsum(k[..., :, None] * v[..., None, :], axis=2)
    ref = np.einsum("bhtd,bhtde->bhte", q, kv)
    th = np.zeros(3)
    np.testing.assert_allclose(O.parallel(q, k, v, [1.0, 1.0], th), ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(O.chunkwise(q, k, v, [1.0, 1.0], th, 5)[0], ref, rtol=1e-11, atol=1e-11)


def test_t9_swish():
    assert O.swish(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.swish(np.array([40.0])), [40.0], rtol=1e-15)
    np.testing.assert_allclose(O.swish(np.array([-40.0])), [0.0], atol=1e-15)
    g = np.linspace(-5, 5, 11)
    np.testing.assert_allclose(O.swish(g), g * torch.sigmoid(torch.from_numpy(g)).numpy(), rtol=1e-14)


def test_t10_nan_propagates_only_forward():
    """A NaN in v_{s0}[c] reaches exactly the outputs that depend on it in the
    recurrent form: channel c from t = s0 on, in that head only. The matrix forms
    multiply masked (s > t) entries by 0, so inside the chunk holding s0 a NaN may
    also reach earlier rows (0·NaN); other heads and channels stay finite."""
    q, k, v, gamma, theta = tiny_inputs(16, N=10)
    v[0, 1, 4, 2] = np.nan
    out, S = O.recurrent(q, k, v, gamma, theta)
    assert np.all(np.isfinite(out[0, 0]))           # other head untouched
    assert np.all(np.isfinite(out[0, 1, :4]))       # earlier tokens untouched
    assert np.all(np.isnan(out[0, 1, 4:, 2]))       # channel 2 poisoned from t=4
    assert np.all(np.isfinite(out[0, 1, :, [0, 1, 3, 4]]))
    assert np.all(np.isnan(S[0, 1, :, 2])) and np.all(np.isfinite(S[0, 0]))
    out, S = O.chunkwise(q, k, v, gamma, theta, 3)   # chunk [3,6) holds s0 = 4
    assert np.all(np.isfinite(out[0, 1, :3])) and np.all(np.isnan(out[0, 1, 4:, 2]))
    assert np.all(np.isfinite(out[0, 0])) and np.all(np.isfinite(out[0, 1, :, [0, 1, 3, 4]]))


def test_rotation_is_orthogonal_pairwise():
    rng = np.random.default_rng(17)
    x = rand(rng, 3, 8)
    pos = np.array([0, 5, 70000])
    th = rng.uniform(0, 2, 4)
    y = O.rotate(x, pos, th)
    np.testing.assert_allclose(y[0], x[0], atol=0)
    for t in range(3):
        for j in range(4):
            assert math.isclose(np.hypot(*y[t, 2 * j:2 * j + 2]), np.hypot(*x[t, 2 * j:2 * j + 2]),
                                rel_tol=1e-13)
