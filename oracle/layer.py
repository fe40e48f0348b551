"""fp64 CPU oracle for the gated multi-scale retention layer — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this module;
it shares no code with the HIP path. Pinned by tests/test_oracle_layer.py.

The layer ([m0nads] "Gated Multi-Scale Retention"; [hwhale] "Gated Multi-Scale
Retention"; [sdkjxy] the multi-scale retention block): the input X is projected to
Q = X W_Q, K = X W_K, V = X W_V; head h takes the h-th block of d_k (Q, K) or d_v (V)
columns and runs retention with its own decay; each head's output is normalised on its
own (GroupNorm, one group per head), the heads are concatenated, multiplied by
swish(X W_G) and projected by W_O:
    MSR(X) = (swish(X W_G) ⊙ GN_h(Concat_h Retention_h(X))) W_O.
The pages state W_G and W_O as d x d; with a value width H d_v different from d they are
d x (H d_v) and (H d_v) x d (the reading taken for the 6.7B shape, d_v = 2 d_k).
"""
from __future__ import annotations

import numpy as np

from .retention import chunkwise, group_norm, swish, to64
from .vector_decay import chunkwise_vec

__all__ = ["split_heads", "merge_heads", "msr_layer"]


def split_heads(y: np.ndarray, H: int) -> np.ndarray:
    """[B, N, H*d] -> [B, H, N, d]: head h owns columns [h d, (h+1) d)."""
    B, N, W = y.shape
    return y.reshape(B, N, H, W // H).transpose(0, 2, 1, 3)


def merge_heads(y: np.ndarray) -> np.ndarray:
    """[B, H, N, d] -> [B, N, H*d] (concatenation of the heads along the features)."""
    B, H, N, d = y.shape
    return y.transpose(0, 2, 1, 3).reshape(B, N, H * d)


def msr_layer(x, w_q, w_k, w_v, w_g, w_o, gamma, theta, H, *, chunk=64, pos0=0, alpha=1.0,
              eps=1e-5, gn_weight=None, gn_bias=None, state0=None, gate=True):
    """Returns (MSR(X) [B, N, d_model], final states [B, H, d_k, d_v]).

    x: [B, N, d_model]; w_q, w_k: [d_model, H d_k]; w_v, w_g: [d_model, H d_v];
    w_o: [H d_v, d_model]; gamma: [H] (one decay per head) or [H, d_k/2] (one per
    coordinate pair); gn_weight, gn_bias: [H, d_v] or None. With ``gate=False`` the
    swish gate is left out (w_g unused)."""
    x = to64(x)
    q = split_heads(x @ to64(w_q), H)
    k = split_heads(x @ to64(w_k), H)
    v = split_heads(x @ to64(w_v), H)
    g = np.asarray(gamma)
    if g.ndim == 2:
        ret, S = chunkwise_vec(q, k, v, g, theta, chunk, pos0, alpha, state0)
    else:
        ret, S = chunkwise(q, k, v, g, theta, chunk, pos0, alpha, state0)
    y = group_norm(ret, eps, gn_weight, gn_bias)
    if gate:
        y = y * swish(split_heads(x @ to64(w_g), H))
    return merge_heads(y) @ to64(w_o), S
