"""fp64 CPU oracle for the gradients of the retention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests alone; shares no code with the HIP
path. Pinned by central finite differences of the forward oracle (tests/test_oracle.py).

The forward pass of one (batch, head) with an initial state S0 is, in closed form
([hwhale] parallel-form equation for the first term; the recurrent equation unrolled
from S0 for the second and for the final state; [hwhale] chunkwise equation, which
computes the same thing):
    Qh = rot(q, p),  Kh = rot(k, p)                       p_t = pos0 + t
    A  = alpha (Qh Kh^T) ⊙ D,   D_ts = gamma^(t-s) for t >= s, else 0
    O  = A V + alpha diag(xi) Qh S0,                      xi_t = gamma^(t+1)
    S_N = gamma^N S0 + Kh^T diag(zeta) V,                 zeta_s = gamma^(N-1-s)
followed by the optional GroupNorm over d_v per row and the swish gate. Given the
gradient of a loss with respect to the call's output (dout) and to its final state
(dstate_out), the gradients below are that closed form differentiated:
    dA  = dO V^T
    dQh = alpha (dA ⊙ D) Kh + alpha diag(xi) dO S0^T
    dKh = alpha (dA ⊙ D)^T Qh + diag(zeta) V dS_N^T
    dV  = A^T dO + diag(zeta) Kh dS_N
    dS0 = alpha Qh^T diag(xi) dO + gamma^N dS_N
and, the rotation being orthogonal per coordinate pair, dq = rot(dQh, -p),
dk = rot(dKh, -p). GroupNorm (one group per head and row, biased variance, eps
inside the square root, affine w, b) and the gate out = y * swish(g) are
differentiated per row:
    dy  = dout * swish(g),   dg = dout * y * swish'(g),
    swish'(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))
    xh  = (x - mean) r,  r = 1 / sqrt(var + eps),  dxh = dy * w
    dx  = r (dxh - mean(dxh) - xh mean(dxh * xh))
    dw  = sum over (batch, rows) of dy * xh,   db = sum of dy.
"""
from __future__ import annotations

import numpy as np

from .retention import decay_matrix, rotate, to64

__all__ = ["backward"]


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def backward(q, k, v, gamma, theta, dout, *, pos0=0, alpha=1.0, state0=None,
             dstate_out=None, gate=None, gn=False, eps=1e-5, weight=None, bias=None):
    """Gradients of (out, S_N) -> loss with respect to q, k, v, the initial state, the
    gate and the GroupNorm affine parameters.

    q, k: [B,H,N,d_k]; v, dout, gate: [B,H,N,d_v]; state0, dstate_out: [B,H,d_k,d_v] or
    None (zeros); weight, bias: [H, d_v] (or [H*d_v]) or None (identity).
    Returns a dict with dq, dk, dv, dstate0 and, when present, dgate, dweight, dbias.
    """
    q, k, v, dout = to64(q), to64(k), to64(v), to64(dout)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    pos = pos0 + np.arange(N, dtype=np.int64)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    S0 = np.zeros((B, H, dk, dv)) if state0 is None else to64(state0)
    dSN = np.zeros((B, H, dk, dv)) if dstate_out is None else to64(dstate_out)
    g = None if gate is None else to64(gate)
    w = np.ones((H, dv)) if weight is None else to64(weight).reshape(H, dv)
    bvec = np.zeros((H, dv)) if bias is None else to64(bias).reshape(H, dv)

    res = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v))}
    res["dstate0"] = np.zeros((B, H, dk, dv))
    if g is not None:
        res["dgate"] = np.zeros_like(g)
    if gn:
        res["dweight"] = np.zeros((H, dv))
        res["dbias"] = np.zeros((H, dv))
    t_idx = np.arange(N, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            gm = float(gamma[h])
            D = decay_matrix(gm, N)
            xi = gm ** (t_idx + 1.0)
            zeta = gm ** (N - 1.0 - t_idx)
            Qh, Kh, V = qh[b, h], kh[b, h], v[b, h]
            A = alpha * (Qh @ Kh.T) * D
            O = A @ V + alpha * xi[:, None] * (Qh @ S0[b, h])
            dO = dout[b, h]
            if gn:
                mu = O.mean(axis=-1, keepdims=True)
                var = ((O - mu) ** 2).mean(axis=-1, keepdims=True)
                r = 1.0 / np.sqrt(var + eps)
                xh = (O - mu) * r
                y = xh * w[h] + bvec[h]
                dy = dO
                if g is not None:
                    sg = _sigmoid(g[b, h])
                    res["dgate"][b, h] = dO * y * sg * (1.0 + g[b, h] * (1.0 - sg))
                    dy = dO * g[b, h] * sg
                res["dweight"][h] += (dy * xh).sum(axis=0)
                res["dbias"][h] += dy.sum(axis=0)
                dxh = dy * w[h]
                dO = r * (dxh - dxh.mean(axis=-1, keepdims=True)
                          - xh * (dxh * xh).mean(axis=-1, keepdims=True))
            dA = dO @ V.T
            dAD = alpha * dA * D
            dQh = dAD @ Kh + alpha * xi[:, None] * (dO @ S0[b, h].T)
            dKh = dAD.T @ Qh + zeta[:, None] * (V @ dSN[b, h].T)
            res["dv"][b, h] = A.T @ dO + zeta[:, None] * (Kh @ dSN[b, h])
            res["dstate0"][b, h] = alpha * Qh.T @ (xi[:, None] * dO) + gm ** N * dSN[b, h]
            res["dq"][b, h] = rotate(dQh[None, None], -pos, theta)[0, 0]
            res["dk"][b, h] = rotate(dKh[None, None], -pos, theta)[0, 0]
    return res
