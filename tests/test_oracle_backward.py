"""Pins of the gradient oracle (oracle/backward.py) against the forward oracle.

The loss is a fixed random linear functional of the call's results,
    L = sum(out * R1) + sum(S_N * R2),
computed with the forward oracle (chunkwise form, then GroupNorm and the gate), and
every gradient the backward oracle returns is compared with central differences of L,
element by element, in float64 on tiny inputs. A dropped term, a wrong sign, a missing
transpose or a misplaced decay factor in the backward formulas fails one of them.
"""
import numpy as np
import pytest

import oracle as O
from oracle.backward import backward


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def forward_loss(x, R1, R2, gamma, theta, pos0, alpha, gn, eps, chunk):
    out, S = O.chunkwise(x["q"], x["k"], x["v"], gamma, theta, chunk, pos0, alpha, x["state0"])
    if gn:
        out = O.groupnorm_gate(out, x.get("gate"), eps, x.get("weight"), x.get("bias"))
    return float((out * R1).sum() + (S * R2).sum())


def finite_diff(x, name, loss, h=1e-6):
    g = np.zeros_like(x[name])
    flat = x[name].reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + h
        lp = loss(x)
        flat[i] = keep - h
        lm = loss(x)
        flat[i] = keep
        gf[i] = (lp - lm) / (2 * h)
    return g


CASES = [
    # gn, gate, pos0, alpha, gammas, chunk
    (False, False, 0, 1.0, [0.9, 0.5], 3),
    (False, False, 17, 0.25, [1.0, 0.8], 4),
    (True, True, 5, 1.0, [0.95, 0.7], 2),
    (True, False, 1000, 0.5, [0.99, 0.6], 6),
]


@pytest.mark.parametrize("gn,use_gate,pos0,alpha,gammas,chunk", CASES)
def test_gradients_match_finite_differences(gn, use_gate, pos0, alpha, gammas, chunk):
    rng = np.random.default_rng(7 + pos0)
    B, H, N, dk, dv = 1, 2, 6, 4, 3
    gamma = np.array(gammas, dtype=np.float32)
    theta = np.array([0.7, 0.013], dtype=np.float32)
    x = {"q": rand(rng, B, H, N, dk), "k": rand(rng, B, H, N, dk), "v": rand(rng, B, H, N, dv),
         "state0": rand(rng, B, H, dk, dv, scale=0.5)}
    if use_gate:
        x["gate"] = rand(rng, B, H, N, dv)
    if gn:
        x["weight"] = 1.0 + rand(rng, H, dv, scale=0.3)
        x["bias"] = rand(rng, H, dv, scale=0.1)
    R1 = rand(rng, B, H, N, dv)
    R2 = rand(rng, B, H, dk, dv)
    eps = 1e-5
    loss = lambda xx: forward_loss(xx, R1, R2, gamma, theta, pos0, alpha, gn, eps, chunk)
    got = backward(x["q"], x["k"], x["v"], gamma, theta, R1, pos0=pos0, alpha=alpha,
                   state0=x["state0"], dstate_out=R2, gate=x.get("gate"), gn=gn, eps=eps,
                   weight=x.get("weight"), bias=x.get("bias"))
    pairs = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("state0", "dstate0")]
    if use_gate:
        pairs.append(("gate", "dgate"))
    if gn:
        pairs += [("weight", "dweight"), ("bias", "dbias")]
    for name, gname in pairs:
        fd = finite_diff(x, name, loss)
        err = np.abs(got[gname] - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-6, (gname, err)


def test_gradient_of_chained_calls_is_the_gradient_of_one_call():
    """Splitting the sequence into two calls joined by the state (prefix's state_out ->
    suffix's state_in) gives the same gradients: the suffix's dstate0 is the gradient
    flowing into the prefix's final state."""
    rng = np.random.default_rng(3)
    B, H, N, dk, dv, M = 1, 2, 9, 4, 3, 4
    gamma = np.array([0.9, 0.75], dtype=np.float32)
    theta = np.array([0.3, 0.05], dtype=np.float32)
    q, k, v = rand(rng, B, H, N, dk), rand(rng, B, H, N, dk), rand(rng, B, H, N, dv)
    dout = rand(rng, B, H, N, dv)
    full = backward(q, k, v, gamma, theta, dout, pos0=2)
    sl1, sl2 = slice(0, M), slice(M, N)
    _, S_mid = O.chunkwise(q[:, :, sl1], k[:, :, sl1], v[:, :, sl1], gamma, theta, 3, 2)
    tail = backward(q[:, :, sl2], k[:, :, sl2], v[:, :, sl2], gamma, theta, dout[:, :, sl2],
                    pos0=2 + M, state0=S_mid)
    head = backward(q[:, :, sl1], k[:, :, sl1], v[:, :, sl1], gamma, theta, dout[:, :, sl1],
                    pos0=2, dstate_out=tail["dstate0"])
    for n in ("dq", "dk", "dv"):
        both = np.concatenate([head[n], tail[n]], axis=2)
        assert np.allclose(both, full[n], rtol=1e-10, atol=1e-12), n
