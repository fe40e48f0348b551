"""GPU parity of the chunkwise backward (rn_retention_chunkwise_backward) against the
gradient oracle (oracle/backward.py, pinned by finite differences of the forward oracle).

Tolerances (about five times the largest error measured):
  * float32 inputs: the products run in float32; per (b, h),
    ||gpu - ref||_inf <= 5e-6 ||ref||_inf (measured at most 8.9e-7).
  * bf16 inputs: the tile products run on matrix cores with their operands rounded to IEEE
    half (relative 2^-11) and float32 accumulation, as the forward's matrix-core paths do;
    a gradient element is a signed sum of many such terms, plus half a bf16 ulp of the
    reference for the bf16 store: |gpu - ref| <= 1e-2 ||ref||_inf + 2^-8 |ref| (measured
    at most 0.26 of that bound). (The state scans stay in float32.)
"""
import numpy as np
import pytest
import torch

import oracle as O
from errlog import record
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rn():
    import linear_recurrent_sequence_rn_amd as m
    return m


def dev(x):
    return None if x is None else x.to(DEV)


def close(gpu, ref, bf16=False, rel=5e-6):
    g, r = O.to64(gpu), O.to64(ref)
    lead = r.shape[:2] if r.ndim >= 3 else (1,)
    nrm = np.abs(r).reshape(*lead, -1).max(-1).reshape(*lead, *([1] * (r.ndim - len(lead))))
    bound = rel * np.maximum(nrm, 1e-30)
    if bf16:
        bound = bound + np.abs(r) * 2.0 ** -8
    e = float((np.abs(g - r) / bound).max())
    record(f"bw_ratio_at_{rel:g}", e)
    return e


def make(dtype, B, H, N, dk, dv, seed, gate=False, state=False):
    w = W.Workload(name="bw", form="chunkwise", B=B, H=H, N=N, d_k=dk, d_v=dv, dtype=dtype,
                   chunk=64, gamma_kind="wide", qkv_std=1 / 8, seed=seed, gate=gate,
                   state_std=0.1 if state else 0.0)
    x = W.make_inputs(w)
    rng = np.random.default_rng(seed + 1)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x["dout"] = torch.from_numpy(rng.standard_normal((B, H, N, dv)).astype(np.float32)).to(tdt)
    x["dstate_out"] = (torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.1)
                       if state else None)
    return x


@pytest.mark.parametrize("N,pos0,alpha", [(70, 0, 1.0), (600, 33, 0.5), (513, 70000, 1.0)])
def test_raw_gradients_fp32(N, pos0, alpha):
    """No epilogue; with an initial state and a gradient for the final state; the 256-token
    state blocks are crossed by N = 513 and 600."""
    x = make("f32", 2, 2, N, 16, 24, seed=N, state=True)
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 64, dev(x["dout"]),
        state_in=dev(x["state"]), dstate_out=dev(x["dstate_out"]), want_dstate_in=True,
        pos0=pos0, qk_scale=alpha)
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], pos0=pos0,
                     alpha=alpha, state0=x["state"], dstate_out=x["dstate_out"])
    for n, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dstate_in", "dstate0")):
        assert close(got[n].cpu(), ref[rname]) <= 1.0, n


def test_gn_gate_affine_gradients_fp32():
    x = make("f32", 1, 3, 300, 32, 40, seed=5, gate=True)
    H, dv = 3, 40
    gw = torch.randn(H * dv, generator=torch.Generator().manual_seed(8)) * 0.3 + 1
    gb = torch.randn(H * dv, generator=torch.Generator().manual_seed(9)) * 0.1
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 128, dev(x["dout"]),
        gate=dev(x["gate"]), gn=True, gn_weight=dev(gw), gn_bias=dev(gb))
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], gate=x["gate"],
                     gn=True, weight=gw.reshape(H, dv), bias=gb.reshape(H, dv))
    for n in ("dq", "dk", "dv", "dgate"):
        assert close(got[n].cpu(), ref[n]) <= 1.0, n
    assert close(got["dgn_weight"].cpu().reshape(1, H, dv), ref["dweight"][None]) <= 1.0
    assert close(got["dgn_bias"].cpu().reshape(1, H, dv), ref["dbias"][None]) <= 1.0


def test_bf16_6p7b_head_shape():
    """The 6.7B head shape (d_k 256, d_v 512), bf16 inputs and gradients, GroupNorm + gate,
    N = 300 (two state blocks)."""
    x = make("bf16", 1, 2, 300, 256, 512, seed=11, gate=True)
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 256, dev(x["dout"]),
        gate=dev(x["gate"]), gn=True)
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], gate=x["gate"], gn=True)
    for n in ("dq", "dk", "dv", "dgate"):
        assert close(got[n].cpu(), ref[n], bf16=True, rel=1e-2) <= 1.0, n


@pytest.mark.parametrize("N,pos0,dk,dv", [(513, 70000, 64, 96), (77, 3, 48, 40), (600, 0, 256, 512),
                                         (130, 5, 20, 12)])
def test_bf16_state_positions_other_shapes(N, pos0, dk, dv):
    """Matrix-core paths with an initial state, a gradient for the final state, positions
    and ragged tiles; head shapes below the 6.7B one are zero-padded in the products (d_k
    and d_v multiples of 8 take the half-operand path with transposed copies, 20 / 12 the
    one that stages float32 operands)."""
    x = make("bf16", 2, 2, N, dk, dv, seed=N + dk, state=True)
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 64, dev(x["dout"]),
        state_in=dev(x["state"]), dstate_out=dev(x["dstate_out"]), want_dstate_in=True,
        pos0=pos0, qk_scale=0.5)
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], pos0=pos0,
                     alpha=0.5, state0=x["state"], dstate_out=x["dstate_out"])
    for n, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv")):
        assert close(got[n].cpu(), ref[rname], bf16=True, rel=1e-2) <= 1.0, n
    assert close(got["dstate_in"].cpu(), ref["dstate0"], rel=1e-2) <= 1.0


def test_bf16_inputs_register_staged_kernels():
    """bf16 inputs through the kernels that stage their operands through registers with
    64-bit addressing (RN_FORCE_GENERIC; the path taken where a head's arrays pass the
    copy-fed kernels' 2 GB buffer range): operands staged in float32 and rounded to IEEE
    half for the MFMA products, float32 accumulation and scans. Bar: 2e-3 of the head's
    norm plus the bf16 store (measured at most 3.5e-4 of the norm beyond the store's
    rounding)."""
    x = make("bf16", 1, 2, 130, 64, 96, seed=31, gate=True, state=True)
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 64, dev(x["dout"]),
        gate=dev(x["gate"]), gn=True, state_in=dev(x["state"]), dstate_out=dev(x["dstate_out"]),
        want_dstate_in=True, pos0=9, force_generic=True)
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], gate=x["gate"],
                     gn=True, pos0=9, state0=x["state"], dstate_out=x["dstate_out"])
    for n in ("dq", "dk", "dv", "dgate"):
        assert close(got[n].cpu(), ref[n], bf16=True, rel=2e-3) <= 1.0, n
    assert close(got["dstate_in"].cpu(), ref["dstate0"], rel=2e-3) <= 1.0


def test_bf16_gn_affine_gradients():
    x = make("bf16", 1, 2, 300, 256, 512, seed=21, gate=True)
    H, dv = 2, 512
    gw = torch.randn(H * dv, generator=torch.Generator().manual_seed(18)) * 0.3 + 1
    gb = torch.randn(H * dv, generator=torch.Generator().manual_seed(19)) * 0.1
    got = rn().rn_retention_chunkwise_backward(
        dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 256, dev(x["dout"]),
        gate=dev(x["gate"]), gn=True, gn_weight=dev(gw), gn_bias=dev(gb))
    ref = O.backward(x["q"], x["k"], x["v"], x["gamma"], x["theta"], x["dout"], gate=x["gate"],
                     gn=True, weight=gw.reshape(H, dv), bias=gb.reshape(H, dv))
    for n in ("dq", "dk", "dv", "dgate"):
        assert close(got[n].cpu(), ref[n], bf16=True, rel=1e-2) <= 1.0, n
    assert close(got["dgn_weight"].cpu().reshape(1, H, dv), ref["dweight"][None], rel=1e-2) <= 1.0
    assert close(got["dgn_bias"].cpu().reshape(1, H, dv), ref["dbias"][None], rel=1e-2) <= 1.0
