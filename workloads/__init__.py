"""Seeded synthetic inputs for the retention forward pass.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds only input recipes (shapes, seeds, value distributions, the per-head
decay and per-pair angle hyper-parameters) and draws random numbers; it
contains none of the retention arithmetic, and it imports neither the oracle
nor the GPU package.

Shapes follow the listings on the hwhale.com RetNet notes (ParallelRetention /
RecurrentRetention / ChunkwiseRetention argument comments):
q, k: [B, H, N, d_k]; v, gate: [B, H, N, d_v]; state: [B, H, d_k, d_v].

Draw order for one workload: q, k, v, gate, state, each as float32 from
``numpy.random.default_rng(seed)``; tensors that the workload declares bf16
are rounded float32 -> bfloat16 with round-to-nearest-even (torch's CPU
conversion), and both the GPU path and the oracle consume the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "theta_default", "gamma_small", "gamma_wide",
    "gamma_pairs_wide", "gamma_pairs_spread", "make_inputs", "make_decode_step_inputs",
    "LAYER_D_MODEL", "make_layer_inputs",
]


def theta_default(d_k: int) -> np.ndarray:
    """One angle per coordinate pair: theta_j = 10000^(-2j/d_k), j < d_k/2 (float32)."""
    j = np.arange(d_k // 2, dtype=np.float64)
    return (10000.0 ** (-2.0 * j / d_k)).astype(np.float32)


def gamma_small(H: int) -> np.ndarray:
    """Per-head decay 1 - 2^(-5-h) (tiny and 1.3B-shaped workloads), float32."""
    h = np.arange(H, dtype=np.float64)
    return (1.0 - 2.0 ** (-5.0 - h)).astype(np.float32)


def gamma_wide(H: int) -> np.ndarray:
    """Per-head decay 1 - 2^(-5 - 4h/H) (6.7B-shaped workloads, H=16), float32."""
    h = np.arange(H, dtype=np.float64)
    return (1.0 - 2.0 ** (-5.0 - 4.0 * h / H)).astype(np.float32)


def gamma_pairs_wide(H: int, d_k: int) -> np.ndarray:
    """One decay per (head, coordinate pair): 1 - 2^-(5 + 4h/H + 4j/(P-1)), P = d_k/2.
    Each head spans four octaves of 1 - gamma across its pairs, the heads together the
    range 1 - 2^-5 .. 1 - 2^-13 (float32 [H, P])."""
    P = d_k // 2
    h = np.arange(H, dtype=np.float64)[:, None]
    j = np.arange(P, dtype=np.float64)[None, :]
    return (1.0 - 2.0 ** (-(5.0 + 4.0 * h / H + 4.0 * j / max(P - 1, 1)))).astype(np.float32)


def gamma_pairs_spread(H: int, d_k: int, seed: int) -> np.ndarray:
    """Pair decays over a wide range, for checking robustness: gamma = exp(-u) with u
    log-uniform in [1e-5, 10] (gamma from 0.99999 down to 4.5e-5), pair 0 of head 0 set to
    1e-6 and pair 1 of head 0 to exactly 1 (float32 [H, d_k/2])."""
    rng = np.random.default_rng([seed, 77])
    u = np.exp(rng.uniform(np.log(1e-5), np.log(10.0), (H, d_k // 2)))
    g = np.exp(-u)
    g[0, 0] = 1e-6
    if d_k >= 4:
        g[0, 1] = 1.0
    return g.astype(np.float32)


def _gamma(kind: str, H: int, d_k: int, seed: int) -> np.ndarray:
    if kind == "small":
        return gamma_small(H)
    if kind == "wide":
        return gamma_wide(H)
    if kind == "pair_wide":
        return gamma_pairs_wide(H, d_k)
    if kind == "pair_spread":
        return gamma_pairs_spread(H, d_k, seed)
    raise ValueError(kind)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    form: str            # "parallel" | "chunkwise" | "recurrent" | "all"
    B: int
    H: int
    N: int
    d_k: int
    d_v: int
    dtype: str           # "f32" | "bf16" (q, k, v, gate)
    chunk: int = 0
    qk_scale: float = 1.0
    norm_d: bool = False
    norm_r: bool = False
    gn: bool = False
    gate: bool = False
    gn_eps: float = 1e-5
    gamma_kind: str = "small"   # "small" | "wide" (per head) | "pair_wide" | "pair_spread" (per pair)
    qkv_std: float = 1.0        # q,k,v ~ N(0, qkv_std^2)
    state_std: float = 0.0      # initial state ~ N(0, state_std^2); 0 = no state
    steps: int = 0              # decode steps (recurrent workload)
    seed: int = 0

    def gamma(self) -> np.ndarray:
        return _gamma(self.gamma_kind, self.H, self.d_k, self.seed)

    def theta(self) -> np.ndarray:
        return theta_default(self.d_k)


_S = 1.0 / math.sqrt(256.0)

WORKLOADS = {
    # tiny oracle check: fp32, all three forms + GroupNorm(eps=1e-5)
    "tiny": Workload("tiny", "all", B=1, H=2, N=64, d_k=16, d_v=16, dtype="f32",
                     chunk=16, gn_eps=1e-5, gamma_kind="small", qkv_std=1.0, seed=1),
    # parallel form, 1.3B-shaped, all three rescalings + GroupNorm
    "parallel_1p3b": Workload("parallel_1p3b", "parallel", B=8, H=8, N=2048, d_k=256,
                              d_v=512, dtype="bf16", qk_scale=_S, norm_d=True,
                              norm_r=True, gn=True, gamma_kind="small", qkv_std=_S,
                              seed=2),
    # chunkwise form, 6.7B-shaped training: GroupNorm + swish gate, fp32 state out
    "chunkwise_6p7b": Workload("chunkwise_6p7b", "chunkwise", B=2, H=16, N=8192, d_k=256,
                               d_v=512, dtype="bf16", chunk=256, gn=True, gate=True,
                               gamma_kind="wide", qkv_std=_S, seed=3),
    # recurrent decode step, 6.7B-shaped: batch 128, state ~ N(0, 0.1^2), 1024 steps
    "decode_6p7b": Workload("decode_6p7b", "recurrent", B=128, H=16, N=1, d_k=256,
                            d_v=512, dtype="bf16", gamma_kind="wide", qkv_std=_S,
                            state_std=0.1, steps=1024, seed=4),
    # the 6.7B training shape with one decay per (head, coordinate pair)
    "chunkwise_6p7b_pair": Workload("chunkwise_6p7b_pair", "chunkwise", B=2, H=16, N=8192,
                                    d_k=256, d_v=512, dtype="bf16", chunk=256, gn=True,
                                    gate=True, gamma_kind="pair_wide", qkv_std=_S, seed=6),
    # long-sequence chunkwise: 128 chunks of 512, GroupNorm
    "chunkwise_long": Workload("chunkwise_long", "chunkwise", B=1, H=16, N=65536,
                               d_k=256, d_v=512, dtype="bf16", chunk=512, gn=True,
                               gamma_kind="wide", qkv_std=_S, seed=5),
}


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(w: Workload, *, N: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Draw q, k, v, gate, state for workload ``w`` (optionally resized).

    Returns CPU torch tensors in the workload dtype (q, k, v, gate) and float32
    (state, or None), plus float32 numpy ``gamma`` ([H], or [H, d_k/2] for the pair
    kinds) and ``theta`` [d_k/2].
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal((B, H, N, w.d_k), dtype=np.float32) * np.float32(w.qkv_std)
    k = rng.standard_normal((B, H, N, w.d_k), dtype=np.float32) * np.float32(w.qkv_std)
    v = rng.standard_normal((B, H, N, w.d_v), dtype=np.float32) * np.float32(w.qkv_std)
    gate = rng.standard_normal((B, H, N, w.d_v), dtype=np.float32) if w.gate else None
    state = None
    if w.state_std > 0:
        state = rng.standard_normal((B, H, w.d_k, w.d_v), dtype=np.float32) * np.float32(w.state_std)
    gamma = _gamma(w.gamma_kind, H, w.d_k, w.seed)
    return {
        "q": _round(q, w.dtype), "k": _round(k, w.dtype), "v": _round(v, w.dtype),
        "gate": None if gate is None else _round(gate, w.dtype),
        "state": None if state is None else torch.from_numpy(state),
        "gamma": gamma, "theta": w.theta(),
    }


def make_decode_step_inputs(w: Workload, step: int, *, B: Optional[int] = None) -> dict:
    """q, k, v for one decode step (seed (w.seed, step)), shape [B, H, 1, d]."""
    B = w.B if B is None else B
    rng = np.random.default_rng([w.seed, step])
    q = rng.standard_normal((B, w.H, 1, w.d_k), dtype=np.float32) * np.float32(w.qkv_std)
    k = rng.standard_normal((B, w.H, 1, w.d_k), dtype=np.float32) * np.float32(w.qkv_std)
    v = rng.standard_normal((B, w.H, 1, w.d_v), dtype=np.float32) * np.float32(w.qkv_std)
    return {"q": _round(q, w.dtype), "k": _round(k, w.dtype), "v": _round(v, w.dtype)}


def initial_state(w: Workload, *, B: Optional[int] = None) -> torch.Tensor:
    """The decode workload's initial state, ~ N(0, state_std^2), float32 [B, H, d_k, d_v]."""
    B = w.B if B is None else B
    rng = np.random.default_rng([w.seed, 1 << 20])
    s = rng.standard_normal((B, w.H, w.d_k, w.d_v), dtype=np.float32) * np.float32(w.state_std)
    return torch.from_numpy(s)


# Model width of the 6.7B-shaped layer (16 heads of d_k = 256 -> H d_k = 4096).
LAYER_D_MODEL = 4096


def make_layer_inputs(w: Workload, d_model: int, *, N: Optional[int] = None,
                      B: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Input and synthetic weights of the gated multi-scale layer on workload ``w``'s heads.

    x ~ N(0, 1) [B, N, d_model]; W_Q, W_K, W_V ~ N(0, 1/(d_k d_model)) so that q, k, v have
    the retention workloads' scale N(0, 1/d_k); W_G ~ N(0, 1/d_model) (gate ~ N(0, 1));
    W_O ~ N(0, 1/(H d_v)). All drawn as float32 in the order x, W_Q, W_K, W_V, W_G, W_O from
    ``default_rng([seed, 9])`` and rounded to bf16. Returns CPU tensors plus ``gamma`` and
    ``theta`` as make_inputs does."""
    B = w.B if B is None else B
    N = w.N if N is None else N
    rng = np.random.default_rng([w.seed if seed is None else seed, 9])
    H, dk, dv = w.H, w.d_k, w.d_v

    def draw(shape, std):
        return _round(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), "bf16")

    x = draw((B, N, d_model), 1.0)
    s_qkv = 1.0 / math.sqrt(dk * d_model)
    return {
        "x": x,
        "w_q": draw((d_model, H * dk), s_qkv), "w_k": draw((d_model, H * dk), s_qkv),
        "w_v": draw((d_model, H * dv), s_qkv), "w_g": draw((d_model, H * dv), 1.0 / math.sqrt(d_model)),
        "w_o": draw((H * dv, d_model), 1.0 / math.sqrt(H * dv)),
        "gamma": _gamma(w.gamma_kind, H, dk, w.seed), "theta": w.theta(),
    }
