"""fp64 CPU oracle for retention with one decay per coordinate pair — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module;
it shares no code with the HIP path. Pinned by tests/test_oracle_vector.py (reduction to
the scalar-decay oracle when a head's decays are equal, decomposition into one scalar
retention per coordinate pair, agreement of the independently written forms, chained
calls).

The form before the pages simplify the decay to one number per head: the transition of
the recurrence is diagonalised as A = Λ diag(γ e^{iθ}) Λ^{-1} with γ and θ both vectors
over the complex dimensions ([hwhale] the diagonalisation of A; [m0nads] "Retention",
where γ and θ are introduced as two d-vectors before γ is replaced by a scalar). With Λ
absorbed into the projections, complex dimension j (the coordinate pair (2j, 2j+1) of
the real layout, as for θ) evolves as γ_j^n e^{i n θ_j}, so the score of query t and key
s becomes
    s_ts = α Re Σ_j γ_j^(t-s) ẑq_{t,j} conj(ẑk_{s,j})       (t >= s)
with ẑ the rotated pairs. Per head, gamma is a [d_k/2] vector: gamma[h, j] decays pair j.
In the real layout that is a decay per row of the d_k x d_v state, both rows of a pair
sharing it. The decay no longer factors out of Q K^T, so every form applies it inside
the sum over d_k.
"""
from __future__ import annotations

import numpy as np

from .retention import rotate, to64

__all__ = [
    "row_decays", "brute_force_vec", "parallel_vec", "recurrent_vec",
    "recurrent_step_vec", "chunkwise_vec",
]


def row_decays(gamma) -> np.ndarray:
    """[H, d_k/2] pair decays -> [H, d_k] decay of each real coordinate (2j and 2j+1 share
    gamma[h, j])."""
    g = np.asarray(gamma, dtype=np.float64)
    return np.repeat(g, 2, axis=-1)


def _positions(N: int, pos0: int) -> np.ndarray:
    return np.arange(N, dtype=np.int64) + int(pos0)


def brute_force_vec(q, k, v, gamma, theta, pos0=0, alpha=1.0, state0=None):
    """O_t = α Σ_{s<=t} Re[Σ_j γ_j^(t-s) ẑq_{t,j} conj(ẑk_{s,j})] V_s  (+ initial state).

    The un-simplified sum, term by term in complex arithmetic with plain loops. A
    nonzero initial state S0 adds α Σ_d Qh_{t,d} γ_{d}^(t+1) S0[d, :] (the recurrence
    run from S0). Tiny sizes only.
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    th = np.asarray(theta, dtype=np.float64)
    gm = np.asarray(gamma, dtype=np.float64)
    S0 = None if state0 is None else to64(state0)
    out = np.zeros((B, H, N, dv))
    for b in range(B):
        for h in range(H):
            for t in range(N):
                zq = [complex(q[b, h, t, 2 * j], q[b, h, t, 2 * j + 1]) *
                      np.exp(1j * (pos0 + t) * th[j]) for j in range(dk // 2)]
                acc = np.zeros(dv)
                for s in range(t + 1):
                    sc = 0j
                    for j in range(dk // 2):
                        zk = complex(k[b, h, s, 2 * j], k[b, h, s, 2 * j + 1]) * \
                            np.exp(1j * (pos0 + s) * th[j])
                        sc += gm[h, j] ** (t - s) * zq[j] * np.conj(zk)
                    acc += alpha * sc.real * v[b, h, s]
                if S0 is not None:
                    for j in range(dk // 2):
                        w = alpha * gm[h, j] ** (t + 1)
                        acc += w * (zq[j].real * S0[b, h, 2 * j] + zq[j].imag * S0[b, h, 2 * j + 1])
                out[b, h, t] = acc
    return out


def _decayed_scores(qh, kh, g_rows, alpha):
    """R_ts = α Σ_d Qh_{t,d} γ_d^(t-s) Kh_{s,d} for t >= s, else 0 (one head).

    qh, kh: [..., T, d_k]; g_rows: [d_k]."""
    T = qh.shape[-2]
    dist = np.arange(T)[:, None] - np.arange(T)[None, :]
    causal = dist >= 0
    G = np.where(causal[..., None], g_rows[None, None, :] ** np.maximum(dist, 0)[..., None], 0.0)
    return alpha * np.einsum("...td,tsd,...sd->...ts", qh, G, kh)


def parallel_vec(q, k, v, gamma, theta, pos0=0, alpha=1.0, norm_r=False):
    """Parallel form with pair decays: O = R V, R_ts = α Σ_d Qh_{t,d} γ_d^(t-s) Kh_{s,d}
    (causal), optionally R̃_ts = R_ts / max(|Σ_{s'<=t} R_ts'|, 1) ([hwhale] third of the
    listed rescalings). The D-row rescaling is defined by the scalar decay matrix and has
    no counterpart here."""
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, _ = q.shape
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    gr = row_decays(gamma)
    out = np.empty(v.shape)
    for h in range(H):
        R = _decayed_scores(qh[:, h], kh[:, h], gr[h], alpha)
        if norm_r:
            R = R / np.maximum(np.abs(R.sum(axis=-1, keepdims=True)), 1.0)
        out[:, h] = R @ v[:, h]
    return out


def recurrent_vec(q, k, v, gamma, theta, pos0=0, alpha=1.0, state0=None):
    """S_n = diag(γ) S_{n-1} + Kh_n^T V_n ; o_n = α Qh_n S_n, where diag(γ) scales state
    row d by the decay of its pair ([hwhale] recurrent equations with the diagonal
    transition left as a vector). Returns (O, S_final)."""
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else to64(state0).copy()
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    g = row_decays(gamma)[None, :, :, None]
    out = np.empty((B, H, N, dv))
    for t in range(N):
        S = g * S + kh[:, :, t, :, None] * v[:, :, t, None, :]
        out[:, :, t] = alpha * np.einsum("bhd,bhde->bhe", qh[:, :, t], S)
    return out, S


def recurrent_step_vec(q, k, v, gamma, theta, pos, alpha=1.0, state=None):
    """One decode step at absolute position ``pos`` with pair decays: S <- diag(γ) S +
    Kh^T v ; o = α Qh S. q, k: [B,H,d_k] (or [B,H,1,d_k]); v: [B,H,d_v]."""
    q, k, v = to64(q), to64(k), to64(v)
    if q.ndim == 4:
        q, k, v = q[:, :, 0], k[:, :, 0], v[:, :, 0]
    B, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state is None else to64(state)
    p = np.array([pos], dtype=np.int64)
    qh = rotate(q[:, :, None], p, theta)[:, :, 0]
    kh = rotate(k[:, :, None], p, theta)[:, :, 0]
    g = row_decays(gamma)[None, :, :, None]
    S = g * S + kh[..., :, None] * v[..., None, :]
    return alpha * np.einsum("bhd,bhde->bhe", qh, S), S


def chunkwise_vec(q, k, v, gamma, theta, chunk, pos0=0, alpha=1.0, state0=None):
    """Chunkwise form with pair decays ([hwhale] chunkwise equation, decay kept per row
    of the state). For chunk i covering rows [iC, iC+L), j the 0-based row in the chunk:
      inner_t = Σ_{s in chunk, s<=t} (Σ_d Qh_{t,d} γ_d^(t-s) Kh_{s,d}) V_s
      cross_t = Σ_d Qh_{t,d} γ_d^(j+1) S_i[d, :]
      O_t     = α (inner_t + cross_t)
      S_{i+1} = diag(γ^L) S_i + Σ_j (Kh_j ⊙ γ^(L-1-j))^T V_j
    The last chunk may be shorter. Returns (O, S_final)."""
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else to64(state0).copy()
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    gr = row_decays(gamma)
    out = np.empty((B, H, N, dv))
    for c0 in range(0, N, chunk):
        L = min(chunk, N - c0)
        sl = slice(c0, c0 + L)
        j = np.arange(L, dtype=np.float64)
        for h in range(H):
            g = gr[h]
            Qc, Kc, Vc = qh[:, h, sl], kh[:, h, sl], v[:, h, sl]
            inner = _decayed_scores(Qc, Kc, g, 1.0) @ Vc
            xi = g[None, :] ** (j[:, None] + 1.0)            # [L, d_k]
            cross = (Qc * xi[None]) @ S[:, h]
            out[:, h, sl] = alpha * (inner + cross)
            zeta = g[None, :] ** (L - 1.0 - j[:, None])      # [L, d_k]
            S[:, h] = (g ** L)[None, :, None] * S[:, h] + np.swapaxes(Kc * zeta[None], -1, -2) @ Vc
    return out, S
