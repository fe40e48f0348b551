"""GPU parity: the HIP kernels against the fp64 oracle on the same seeded inputs.

Tolerances (about five times the largest error measured over the GPU suite):
  * float32 arithmetic paths (generic kernels, decode, GroupNorm): per (b, h) slice,
    ||gpu - ref||_inf <= F32_BAR ||ref||_inf (raw outputs, GroupNorm outputs and final
    states alike). Measured at most 1.0e-6 (the generic parallel kernel; the full decode
    workload over 1024 steps: 6.8e-7 for outputs, 5.7e-7 for the final states).
  * a bf16 output after GroupNorm: 2e-2 max-abs plus half a bf16 ulp of the reference.
"""
import numpy as np
import pytest
import torch

import oracle as O
from errlog import record
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32_BAR = 5e-6


def rn():
    import linear_recurrent_sequence_rn_amd as m
    return m


def rel_inf(gpu, ref):
    """max over (b,h) of ||gpu - ref||_inf / ||ref||_inf."""
    g = O.to64(gpu)
    r = O.to64(ref)
    err = np.abs(g - r).reshape(r.shape[0], r.shape[1], -1).max(-1)
    nrm = np.abs(r).reshape(r.shape[0], r.shape[1], -1).max(-1)
    e = float((err / np.maximum(nrm, 1e-30)).max())
    record("rel", e)
    return e


def dev(x):
    return None if x is None else x.to(DEV)


def inputs(name, **kw):
    w = W.WORKLOADS[name]
    x = W.make_inputs(w, **kw)
    return w, x


# ---- tiny workload: float32, all three forms, raw and GroupNorm ----------------------

@pytest.mark.parametrize("gn", [False, True])
def test_tiny_parallel_fp32(gn):
    w, x = inputs("tiny")
    out = rn().rn_retention_parallel(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"],
                                     gn=gn, gn_eps=w.gn_eps)
    ref = O.brute_force(x["q"], x["k"], x["v"], x["gamma"], x["theta"])
    ref = O.apply_epilogue(ref, gn=gn, eps=w.gn_eps)
    assert rel_inf(out.cpu(), ref) <= F32_BAR


@pytest.mark.parametrize("gn", [False, True])
@pytest.mark.parametrize("chunk", [16, 5, 64, 1])
def test_tiny_chunkwise_fp32(gn, chunk):
    w, x = inputs("tiny")
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], chunk, state_out=True, gn=gn, gn_eps=w.gn_eps)
    ref = O.brute_force(x["q"], x["k"], x["v"], x["gamma"], x["theta"])
    _, Sref = O.recurrent(x["q"], x["k"], x["v"], x["gamma"], x["theta"])
    assert rel_inf(out.cpu(), O.apply_epilogue(ref, gn=gn, eps=w.gn_eps)) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR


@pytest.mark.parametrize("gn", [False, True])
def test_tiny_recurrent_fp32(gn):
    w, x = inputs("tiny")
    B, H, N, dk = x["q"].shape
    dv = x["v"].shape[-1]
    S = torch.zeros(B, H, dk, dv, device=DEV)
    outs = []
    for t in range(N):
        sl = slice(t, t + 1)
        outs.append(rn().rn_retention_recurrent_step(dev(x["q"][:, :, sl].contiguous()),
                                                     dev(x["k"][:, :, sl].contiguous()),
                                                     dev(x["v"][:, :, sl].contiguous()),
                                                     x["gamma"], x["theta"], S, t, gn=gn,
                                                     gn_eps=w.gn_eps))
    out = torch.cat(outs, 2).cpu()
    ref = O.brute_force(x["q"], x["k"], x["v"], x["gamma"], x["theta"])
    _, Sref = O.recurrent(x["q"], x["k"], x["v"], x["gamma"], x["theta"])
    assert rel_inf(out, O.apply_epilogue(ref, gn=gn, eps=w.gn_eps)) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR


def test_tiny_parallel_rescaled_fp32():
    """The parallel form with the 1.3B workload's flags: alpha = 1/sqrt(d_k), D and R row
    normalisation, GroupNorm."""
    w, x = inputs("tiny")
    a = 1.0 / 4.0
    for nd, nr in ((True, False), (False, True), (True, True)):
        out = rn().rn_retention_parallel(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], qk_scale=a, norm_d=nd, norm_r=nr)
        ref = O.parallel(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 0, a, nd, nr)
        assert rel_inf(out.cpu(), ref) <= F32_BAR, (nd, nr)
    out = rn().rn_retention_parallel(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"],
                                     qk_scale=a, norm_d=True, norm_r=True, gn=True)
    ref = O.group_norm(O.parallel(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 0, a, True, True))
    assert rel_inf(out.cpu(), ref) <= F32_BAR


def test_tiny_state_in_pos0_gate_affine_fp32():
    """Initial state, a nonzero start position, ragged chunks, the swish gate and a GN affine."""
    w = W.WORKLOADS["tiny"]
    x = W.make_inputs(W.Workload(**{**w.__dict__, "gate": True, "state_std": 0.3}))
    B, H, N, dk = x["q"].shape
    dv = x["v"].shape[-1]
    gw = torch.randn(H * dv, generator=torch.Generator().manual_seed(5))
    gb = torch.randn(H * dv, generator=torch.Generator().manual_seed(6))
    pos0 = 70000
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 7, gate=dev(x["gate"]),
                                         state_in=dev(x["state"]), state_out=True, pos0=pos0,
                                         gn=True, gn_weight=dev(gw), gn_bias=dev(gb))
    raw, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 7, pos0, 1.0, x["state"])
    ref = O.groupnorm_gate(raw, x["gate"], 1e-5, gw.reshape(H, dv), gb.reshape(H, dv))
    assert rel_inf(out.cpu(), ref) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR


# ---- decode step ---------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_match_oracle(dtype):
    """Reduced-batch decode workload (6.7B head shape): 6 steps in place from a random
    state at positions near 65536; every output and the final state."""
    w = W.Workload(**{**W.WORKLOADS["decode_6p7b"].__dict__, "B": 3, "dtype": dtype})
    S0 = W.initial_state(w)
    S = dev(S0.clone())
    Sref = S0
    for i in range(6):
        pos = 65536 - 6 + i
        x = W.make_decode_step_inputs(w, i)
        out = rn().rn_retention_recurrent_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.gamma(),
                                               w.theta(), S, pos, out_dtype=torch.float32)
        o_ref, Sref = O.recurrent_step(x["q"], x["k"], x["v"], w.gamma(), w.theta(), pos, 1.0, Sref)
        assert rel_inf(out.cpu()[:, :, 0], o_ref) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR


def test_decode_1024_steps_full_shape():
    """The full decode workload in the benchmark's launch configuration: batch 128, 16
    heads, 256 x 512 float32 states updated in place over 1024 steps at positions 0..1023.
    After the first step every (b, h) output and state is checked; at every step, the
    outputs of 16 sampled (b, h), whose states the oracle carries along in float64; after
    the last step, those 16 states."""
    w = W.WORKLOADS["decode_6p7b"]
    g, th = w.gamma(), w.theta()
    S0 = W.initial_state(w)
    S = dev(S0)
    rng = np.random.default_rng(0)
    bs = rng.choice(w.B, 16, replace=False)
    hs = rng.integers(0, w.H, 16)
    bi, hi = torch.as_tensor(bs, device=DEV), torch.as_tensor(hs, device=DEV)
    Sref = [S0[b:b + 1, h:h + 1] for b, h in zip(bs, hs)]
    worst_o = 0.0
    for i in range(w.steps):
        x = W.make_decode_step_inputs(w, i)
        out = rn().rn_retention_recurrent_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), g, th, S, i,
                                               out_dtype=torch.float32)
        osel = out[bi, hi].cpu()                      # [16, 1, d_v]
        if i == 0:
            oall, Sall = out.cpu(), S.cpu()
            for b0 in range(0, w.B, 16):
                sl = (slice(b0, b0 + 16),)
                o_ref, s_ref = O.recurrent_step(x["q"][sl], x["k"][sl], x["v"][sl], g, th, 0, 1.0,
                                                S0[sl])
                assert rel_inf(oall[sl][:, :, 0], o_ref) <= F32_BAR, b0
                assert rel_inf(Sall[sl], s_ref) <= F32_BAR, b0
            del oall, Sall
        for j, (b, h) in enumerate(zip(bs, hs)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            o_ref, Sref[j] = O.recurrent_step(x["q"][sl], x["k"][sl], x["v"][sl], g[h:h + 1], th, i,
                                              1.0, Sref[j])
            worst_o = max(worst_o, rel_inf(osel[j:j + 1], o_ref))
        assert worst_o <= F32_BAR, (i, worst_o)
    Sfin = S[bi, hi].cpu()                            # [16, d_k, d_v]
    worst_s = max(rel_inf(Sfin[j][None, None], Sref[j]) for j in range(16))
    print(f"decode 1024 steps: worst output {worst_o:.2e}, worst final state {worst_s:.2e}")
    assert worst_s <= F32_BAR


@pytest.mark.parametrize("dk,dv", [(256, 256), (128, 128), (64, 256), (48, 512), (256, 384)])
def test_decode_other_shapes(dk, dv):
    """Decode at other head shapes: the pipelined kernel's d_v = 256 and 128 layouts
    (G = 8 and 16 row groups), and shapes it does not take (d_k not a multiple of 8G,
    d_v outside {128, 256, 512}), which run the one-batch kernel; 3 chained steps."""
    w = W.Workload(**{**W.WORKLOADS["decode_6p7b"].__dict__, "B": 2, "H": 3, "d_k": dk, "d_v": dv})
    S0 = W.initial_state(w)
    S = dev(S0.clone())
    Sref = S0
    for i in range(3):
        x = W.make_decode_step_inputs(w, i)
        out = rn().rn_retention_recurrent_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.gamma(),
                                               w.theta(), S, 100 + i, out_dtype=torch.float32)
        o_ref, Sref = O.recurrent_step(x["q"], x["k"], x["v"], w.gamma(), w.theta(), 100 + i, 1.0, Sref)
        assert rel_inf(out.cpu()[:, :, 0], o_ref) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR


def test_decode_gn_gate_bf16_out():
    w = W.Workload(**{**W.WORKLOADS["decode_6p7b"].__dict__, "B": 2})
    S0 = W.initial_state(w)
    x = W.make_decode_step_inputs(w, 3)
    g = torch.randn(2, 16, 1, 512, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    S = dev(S0.clone())
    out = rn().rn_retention_recurrent_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.gamma(),
                                           w.theta(), S, 17, gate=dev(g), gn=True)
    o_ref, _ = O.recurrent_step(x["q"], x["k"], x["v"], w.gamma(), w.theta(), 17, 1.0, S0)
    ref = O.groupnorm_gate(o_ref[:, :, None], g)
    d = np.abs(O.to64(out.cpu()) - ref)
    # bf16 output: GN values are O(1); allow the bar plus half a bf16 ulp of the reference
    assert (d <= 2e-2 + np.abs(ref) * 2.0 ** -8).all()


# ---- standalone GroupNorm + gate ----------------------------------------------------

@pytest.mark.parametrize("dt,dv", [(torch.float32, 512), (torch.bfloat16, 512), (torch.float32, 37),
                                   (torch.bfloat16, 100)])
def test_groupnorm_gate(dt, dv):
    gen = torch.Generator().manual_seed(dv)
    x = (torch.randn(2, 3, 5, dv, generator=gen) * 3 + 1).to(dt)
    g = torch.randn(2, 3, 5, dv, generator=gen).to(dt)
    w = torch.randn(3 * dv, generator=gen)
    b = torch.randn(3 * dv, generator=gen)
    out = rn().rn_groupnorm_gate(dev(x), dev(g), dev(w), dev(b), 1e-5, out_dtype=torch.float32)
    ref = O.groupnorm_gate(x, g, 1e-5, w.reshape(3, dv), b.reshape(3, dv))
    assert rel_inf(out.cpu(), ref) <= F32_BAR
    out2 = rn().rn_groupnorm_gate(dev(x), None, None, None, 1e-5, out_dtype=torch.float32)
    assert rel_inf(out2.cpu(), O.group_norm(x, 1e-5)) <= F32_BAR


# ---- generic path with bf16 inputs ---------------------------------------------------

def test_generic_bf16_inputs_fp32_accuracy():
    """The plain kernels compute in float32 from bf16 inputs: 1e-4 relative holds."""
    w = W.Workload("g", "all", B=2, H=3, N=45, d_k=32, d_v=24, dtype="bf16", chunk=8, seed=21)
    x = W.make_inputs(w)
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 8, state_out=True, out_dtype=torch.float32,
                                         pos0=3, force_generic=True)
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 8, 3)
    assert rel_inf(out.cpu(), ref) <= F32_BAR
    assert rel_inf(S.cpu(), Sref) <= F32_BAR
    out = rn().rn_retention_parallel(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"],
                                     out_dtype=torch.float32, pos0=3, force_generic=True)
    assert rel_inf(out.cpu(), O.parallel(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 3)) <= F32_BAR
