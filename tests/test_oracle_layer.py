"""Pins of the layer oracle (oracle/layer.py), CPU only.

  * brute force: the layer evaluated with explicit loops on a tiny input — projections as
    sums over the model dimension, head h reading feature h*d + i, retention by the
    brute-force sum (itself pinned), GroupNorm from explicit means, the gate, the output
    projection as a sum over the concatenated features;
  * identity projections: with d_model = H d_k = H d_v and every W the identity, the
    layer is the retention oracle run on the input's head slices, concatenated;
  * head permutation: permuting the heads (their weight columns, decays, GroupNorm
    parameters and W_O rows together) leaves the output unchanged, while permuting the
    decays alone changes it.
A transposed weight, a head read from the wrong columns, heads concatenated in the wrong
order or a gate applied to another head's output fails one of them.
"""
import math

import numpy as np
import pytest

import oracle as O


def layer_inputs(seed, B=1, N=7, d_model=8, H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, d_model))
    w = {"w_q": rng.standard_normal((d_model, H * dk)) / 3,
         "w_k": rng.standard_normal((d_model, H * dk)) / 3,
         "w_v": rng.standard_normal((d_model, H * dv)) / 3,
         "w_g": rng.standard_normal((d_model, H * dv)) / 3,
         "w_o": rng.standard_normal((H * dv, d_model)) / 3}
    theta = rng.uniform(0.1, 1.0, dk // 2)
    gnw = 1 + 0.3 * rng.standard_normal((H, dv))
    gnb = 0.1 * rng.standard_normal((H, dv))
    return x, w, theta, gnw, gnb


def loop_layer(x, w, gamma, theta, H, dk, dv, pos0, eps, gnw, gnb):
    B, N, D = x.shape
    out = np.zeros((B, N, D))
    for b in range(B):
        # per-head q, k, v, g by explicit sums
        q = np.zeros((1, H, N, dk)); k = np.zeros((1, H, N, dk))
        v = np.zeros((1, H, N, dv)); g = np.zeros((1, H, N, dv))
        for t in range(N):
            for h in range(H):
                for i in range(dk):
                    q[0, h, t, i] = sum(x[b, t, m] * w["w_q"][m, h * dk + i] for m in range(D))
                    k[0, h, t, i] = sum(x[b, t, m] * w["w_k"][m, h * dk + i] for m in range(D))
                for i in range(dv):
                    v[0, h, t, i] = sum(x[b, t, m] * w["w_v"][m, h * dv + i] for m in range(D))
                    g[0, h, t, i] = sum(x[b, t, m] * w["w_g"][m, h * dv + i] for m in range(D))
        ret = O.brute_force(q, k, v, gamma, theta, pos0)
        for t in range(N):
            feat = []
            for h in range(H):
                row = ret[0, h, t]
                mu = sum(row) / dv
                var = sum((r - mu) ** 2 for r in row) / dv
                for i in range(dv):
                    y = (row[i] - mu) / math.sqrt(var + eps) * gnw[h, i] + gnb[h, i]
                    gg = g[0, h, t, i]
                    feat.append(y * gg / (1.0 + math.exp(-gg)))
            for m in range(D):
                out[b, t, m] = sum(feat[f] * w["w_o"][f, m] for f in range(H * dv))
    return out


def test_layer_matches_explicit_loops():
    x, w, theta, gnw, gnb = layer_inputs(1, B=2)
    gamma = np.array([0.9, 0.6])
    got, _ = O.msr_layer(x, **w, gamma=gamma, theta=theta, H=2, chunk=3, pos0=5, eps=1e-5,
                         gn_weight=gnw, gn_bias=gnb)
    want = loop_layer(x, w, gamma, theta, 2, 4, 3, 5, 1e-5, gnw, gnb)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("pair", [False, True])
def test_identity_projections_reduce_to_head_slices(pair):
    rng = np.random.default_rng(2)
    B, N, H, d = 2, 9, 3, 4
    x = rng.standard_normal((B, N, H * d))
    eye = np.eye(H * d)
    theta = rng.uniform(0.1, 1.0, d // 2)
    gamma = rng.uniform(0.5, 1.0, (H, d // 2)) if pair else np.array([0.95, 0.8, 0.6])
    got, S = O.msr_layer(x, eye, eye, eye, eye, eye, gamma, theta, H, chunk=4)
    heads = np.stack([x[:, :, h * d:(h + 1) * d] for h in range(H)], axis=1)   # [B,H,N,d]
    if pair:
        ret, S_ref = O.chunkwise_vec(heads, heads, heads, gamma, theta, 4)
    else:
        ret, S_ref = O.chunkwise(heads, heads, heads, gamma, theta, 4)
    y = O.groupnorm_gate(ret, heads)
    want = np.concatenate([y[:, h] for h in range(H)], axis=-1)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-11)


def test_permuting_heads_consistently_leaves_the_output_unchanged():
    H, dk, dv, D = 3, 4, 2, 6
    x, w, theta, gnw, gnb = layer_inputs(3, N=8, d_model=D, H=H, dk=dk, dv=dv)
    gamma = np.array([0.95, 0.7, 0.4])
    base, _ = O.msr_layer(x, **w, gamma=gamma, theta=theta, H=H, gn_weight=gnw, gn_bias=gnb)
    perm = [2, 0, 1]

    def cols(m, d):
        return np.concatenate([m[:, p * d:(p + 1) * d] for p in perm], axis=1)

    wp = {"w_q": cols(w["w_q"], dk), "w_k": cols(w["w_k"], dk), "w_v": cols(w["w_v"], dv),
          "w_g": cols(w["w_g"], dv),
          "w_o": np.concatenate([w["w_o"][p * dv:(p + 1) * dv] for p in perm], axis=0)}
    same, _ = O.msr_layer(x, **wp, gamma=gamma[perm], theta=theta, H=H, gn_weight=gnw[perm],
                          gn_bias=gnb[perm])
    np.testing.assert_allclose(same, base, rtol=1e-11, atol=1e-11)
    other, _ = O.msr_layer(x, **w, gamma=gamma[perm], theta=theta, H=H, gn_weight=gnw, gn_bias=gnb)
    assert np.abs(other - base).max() > 1e-3
