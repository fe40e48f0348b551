"""fp64 CPU oracle for the multi-scale retention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP path.

Every function is the plain definition (or the plain algorithm) written out in
float64 numpy, with no blocking, fusion or reordering beyond what the cited
passage states. Inputs are taken exactly as the GPU sees them (bf16 or fp32
values upcast exactly; gamma and theta are the float32 values the caller
passes, upcast).

Sources (the four pages gathered on RetNet, "Retentive Network"):
  [hwhale]  hwhale.com article 285883, Chinese notes on RetNet
  [sdkjxy]  m.sdkjxy.cn walkthrough "RetNet 架構解讀"
  [m0nads]  m0nads.wordpress.com "Retentive Network notes"
  [eepw]    eepw.com.cn translation of the paper's related-work/experiments

Notation: positions p_t = pos0 + t with 0-based t (the pages count from 1);
alpha = qk_scale; gamma = the head's decay; Qh/Kh = rotated q/k.

Readings taken where the pages are silent or garbled (all listed in the design
notes):
  * rotation pairs are adjacent coordinates (2j, 2j+1) read as the real and
    imaginary part of one complex number ([sdkjxy] "Retention 機制", the
    paragraph that groups a vector's elements two by two); both q and k are
    multiplied by e^{+i p theta_j} and the score conjugates k ([hwhale] closed
    form of O_n with the conjugate transpose); the real part is kept.
  * alpha multiplies q (so the recurrent state never contains alpha).
  * the chunk state update weights each key row by gamma^(L-1-j), obtained by
    unrolling the recurrent update L times ([hwhale] recurrent equation);
    xi_j = gamma^(j+1) with j the 0-based row inside the chunk ([hwhale]
    chunkwise equation).
  * the D and R row normalisations apply to the parallel form only, in the
    listed order, over causal entries, with the signed row sum for R.
  * GroupNorm: one group per head, statistics per token over d_v, biased
    variance, eps inside the square root, optional affine (identity default).
  * swish gate: out = GN(x) * g * sigmoid(g).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rotate", "scores", "decay_matrix", "brute_force", "parallel", "recurrent",
    "recurrent_step", "chunkwise", "group_norm", "swish", "groupnorm_gate",
    "apply_epilogue", "to64",
]


def to64(x) -> np.ndarray:
    """Exact upcast of a torch tensor / numpy array to float64 numpy."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def rotate(x: np.ndarray, pos: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """xPos-style rotation of the last axis.

    [hwhale] definition Q = (X W_Q) ⊙ Θ with Θ_n = e^{i n θ}; [sdkjxy]
    "Retention 機制": a d-vector's elements are taken two by two as the real and
    imaginary part of a complex number. Pair j = (x_{2j}, x_{2j+1}) is
    multiplied by e^{i p θ_j}; the angle p·θ_j is formed in float64.

    x: [..., T, d] ; pos: [T] integer positions ; theta: [d/2].
    """
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * np.asarray(theta, dtype=np.float64)[None, :]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    zr = z * np.exp(1j * ang)
    out = np.empty_like(x)
    out[..., 0::2] = zr.real
    out[..., 1::2] = zr.imag
    return out


def scores(qh: np.ndarray, kh: np.ndarray, alpha: float) -> np.ndarray:
    """s_ts = alpha · (Qh_t · Kh_s): the real part of (Q_t e^{itθ})(K_s e^{isθ})†."""
    return alpha * (qh @ np.swapaxes(kh, -1, -2))


def decay_matrix(gamma: float, N: int) -> np.ndarray:
    """D_nm = γ^(n-m) for n >= m else 0 ([hwhale] definition of D, diagonal = 1)."""
    n = np.arange(N)[:, None]
    m = np.arange(N)[None, :]
    D = np.where(n >= m, float(gamma) ** np.maximum(n - m, 0).astype(np.float64), 0.0)
    return D


def _positions(N: int, pos0: int) -> np.ndarray:
    return np.arange(N, dtype=np.int64) + int(pos0)


def brute_force(q, k, v, gamma, theta, pos0=0, alpha=1.0, state0=None):
    """O_t = α Σ_{s<=t} γ^(t-s) Re[(Q_t e^{i p_t θ})(K_s e^{i p_s θ})†] V_s  (+ initial state).

    The sum defining retention in the [hwhale] closed form of O_n (after the
    diagonalisation), evaluated term by term in complex arithmetic with plain
    loops. A nonzero initial state S0 enters through the recurrence
    S_t = γ^(t+1) S0 + Σ γ^(t-s) Kh_s^T v_s, i.e. the extra term α γ^(t+1) Qh_t S0.
    Tiny sizes only.
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    th = np.asarray(theta, dtype=np.float64)
    S0 = None if state0 is None else to64(state0)
    out = np.zeros((B, H, N, dv))
    for b in range(B):
        for h in range(H):
            g = float(gamma[h])
            for t in range(N):
                pt = pos0 + t
                zq = [complex(q[b, h, t, 2 * j], q[b, h, t, 2 * j + 1]) *
                      np.exp(1j * pt * th[j]) for j in range(dk // 2)]
                acc = np.zeros(dv)
                for s in range(t + 1):
                    ps = pos0 + s
                    sc = 0j
                    for j in range(dk // 2):
                        zk = complex(k[b, h, s, 2 * j], k[b, h, s, 2 * j + 1]) * np.exp(1j * ps * th[j])
                        sc += zq[j] * np.conj(zk)
                    acc += (g ** (t - s)) * alpha * sc.real * v[b, h, s]
                if S0 is not None:
                    qr = np.empty(dk)
                    qr[0::2] = [z.real for z in zq]
                    qr[1::2] = [z.imag for z in zq]
                    acc += alpha * g ** (t + 1) * (qr @ S0[b, h])
                out[b, h, t] = acc
    return out


def parallel(q, k, v, gamma, theta, pos0=0, alpha=1.0, norm_d=False, norm_r=False):
    """Parallel retention: (QK^T ⊙ D) V  ([hwhale] parallel-form equation and the
    ParallelRetention listing), with the optional rescalings of [hwhale]'s list
    of three normalisations, applied in the listed order:
      1. α = 1/√d on QK^T (passed as ``alpha``),
      2. D̃_nm = D_nm / √(Σ_{i<=n} D_ni)          (``norm_d``),
      3. R = QK^T ⊙ D̃ ; R̃_nm = R_nm / max(|Σ_{i<=n} R_ni|, 1)   (``norm_r``).
    Returns O [B, H, N, d_v] (float64, before GroupNorm).
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, _ = q.shape
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    out = np.empty(v.shape[:-1] + (v.shape[-1],))
    for h in range(H):
        D = decay_matrix(gamma[h], N)
        if norm_d:
            D = D / np.sqrt(D.sum(axis=-1, keepdims=True))
        R = scores(qh[:, h], kh[:, h], alpha) * D[None]
        if norm_r:
            R = R / np.maximum(np.abs(R.sum(axis=-1, keepdims=True)), 1.0)
        out[:, h] = R @ v[:, h]
    return out


def recurrent(q, k, v, gamma, theta, pos0=0, alpha=1.0, state0=None):
    """Recurrent retention ([hwhale] recurrent equations and RecurrentRetention
    listing): S_n = γ S_{n-1} + K_n^T V_n ; o_n = Q_n S_n (current token included).
    The initial state is zero unless given ([sdkjxy] "Retention 機制": the
    derivation starts from an all-zero state).
    Returns (O [B,H,N,d_v], S_final [B,H,d_k,d_v]).
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else to64(state0).copy()
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    g = np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    out = np.empty((B, H, N, dv))
    for t in range(N):
        S = g * S + kh[:, :, t, :, None] * v[:, :, t, None, :]
        out[:, :, t] = alpha * np.einsum("bhd,bhde->bhe", qh[:, :, t], S)
    return out, S


def recurrent_step(q, k, v, gamma, theta, pos, alpha=1.0, state=None):
    """One decode step at absolute position ``pos``: S <- γS + Kh^T v ; o = α Qh S.

    q, k: [B,H,d_k] or [B,H,1,d_k]; v: [B,H,d_v] or [B,H,1,d_v]. Returns
    (o [B,H,d_v], S_new)."""
    q, k, v = to64(q), to64(k), to64(v)
    if q.ndim == 4:
        q, k, v = q[:, :, 0], k[:, :, 0], v[:, :, 0]
    B, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state is None else to64(state)
    p = np.array([pos], dtype=np.int64)
    qh = rotate(q[:, :, None], p, theta)[:, :, 0]
    kh = rotate(k[:, :, None], p, theta)[:, :, 0]
    g = np.asarray(gamma, dtype=np.float64)[None, :, None, None]
    S = g * S + kh[..., :, None] * v[..., None, :]
    o = alpha * np.einsum("bhd,bhde->bhe", qh, S)
    return o, S


def chunkwise(q, k, v, gamma, theta, chunk, pos0=0, alpha=1.0, state0=None):
    """Chunkwise recurrent retention ([hwhale] chunkwise equation and the
    ChunkwiseRetention listing; [m0nads] "Chunkwise representation").

    For chunk i covering rows [iC, iC+L):
      inner  = (Qh_[i] Kh_[i]^T ⊙ D) V_[i]          (D the L×L decay mask)
      cross  = (Qh_[i] S_i) ⊙ ξ,   ξ_j = γ^(j+1)    (j = 0-based row in chunk)
      O_[i]  = α (inner + cross)
      S_{i+1} = γ^L S_i + Σ_j γ^(L-1-j) Kh_j^T V_j
    The last chunk may be shorter (L < C). Returns (O, S_final).
    """
    q, k, v = to64(q), to64(k), to64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if state0 is None else to64(state0).copy()
    pos = _positions(N, pos0)
    qh = rotate(q, pos, theta)
    kh = rotate(k, pos, theta)
    out = np.empty((B, H, N, dv))
    for c0 in range(0, N, chunk):
        L = min(chunk, N - c0)
        sl = slice(c0, c0 + L)
        for h in range(H):
            g = float(gamma[h])
            D = decay_matrix(g, L)
            xi = g ** (np.arange(L, dtype=np.float64) + 1.0)
            zeta = g ** (L - 1.0 - np.arange(L, dtype=np.float64))
            Qc, Kc, Vc = qh[:, h, sl], kh[:, h, sl], v[:, h, sl]
            inner = ((Qc @ np.swapaxes(Kc, -1, -2)) * D[None]) @ Vc
            cross = (Qc @ S[:, h]) * xi[None, :, None]
            out[:, h, sl] = alpha * (inner + cross)
            S[:, h] = (g ** L) * S[:, h] + np.swapaxes(Kc, -1, -2) @ (Vc * zeta[None, :, None])
    return out, S


def group_norm(x, eps=1e-5, weight=None, bias=None):
    """Per-head GroupNorm ([hwhale] closing paragraph on heads; [sdkjxy] "Gated
    Multi-Scale Retention"; [eepw] Sub-LayerNorm paragraph): one group per head,
    statistics per token over that head's d_v outputs, biased variance, eps
    inside the square root; optional per-(head, channel) affine [H, d_v]."""
    x = to64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    H, dv = x.shape[1], x.shape[-1]
    if weight is not None:
        y = y * to64(weight).reshape(1, H, *([1] * (x.ndim - 3)), dv)
    if bias is not None:
        y = y + to64(bias).reshape(1, H, *([1] * (x.ndim - 3)), dv)
    return y


def swish(g):
    """swish(g) = g · sigmoid(g) ([m0nads] "Gated Multi-Scale Retention": swish gate)."""
    g = to64(g)
    return g / (1.0 + np.exp(-g))


def groupnorm_gate(x, gate=None, eps=1e-5, weight=None, bias=None):
    """out = GN(x) ⊙ swish(gate) (gate optional)."""
    y = group_norm(x, eps, weight, bias)
    return y if gate is None else y * swish(gate)


def apply_epilogue(o, *, gn=False, gate=None, eps=1e-5, weight=None, bias=None):
    """Optional GroupNorm (+ swish gate) applied to a retention output."""
    if not gn:
        return to64(o)
    return groupnorm_gate(o, gate, eps, weight, bias)
