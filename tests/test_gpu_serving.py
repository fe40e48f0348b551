"""GPU parity of the serving path: prompts of different lengths and starting positions,
padded into one batch, go through rn_retention_chunkwise_varlen (prefill). Its final
states are handed to batched decode steps, rn_retention_recurrent_step_at, with one
position per sequence. The oracle runs every sequence on its own: its true length, its
own positions, no padding.

Tolerances are those of the other GPU parity files:
  * decode and the generic chunkwise kernel (float32 arithmetic): per (b, h),
    ||gpu - ref||_inf <= F32_BAR ||ref||_inf;
  * fused MFMA chunkwise kernel (half operands): raw outputs and states at MFMA_BAR of the
    slice maximum (measured at most 3.9e-4 here); after GroupNorm, 2e-2 * max(1,
    |swish(gate)|) max-abs (measured 2.0e-3). A decode step that continues from an
    MFMA-made state inherits that state's MFMA_BAR bound.
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
MFMA_BAR = 3e-3
SENTINEL = 1234.5   # value of padded output rows before the call; must survive it


def rn():
    import linear_recurrent_sequence_rn_amd as m
    return m


def rel_inf(gpu, ref):
    g, r = O.to64(gpu), O.to64(ref)
    err = np.abs(g - r).reshape(r.shape[0], r.shape[1], -1).max(-1)
    nrm = np.abs(r).reshape(r.shape[0], r.shape[1], -1).max(-1)
    e = float((err / np.maximum(nrm, 1e-30)).max())
    record("rel", e)
    return e


def dev(x):
    return None if x is None else x.to(DEV)


def wl(**kw):
    base = dict(name="serving", form="chunkwise", B=4, H=2, N=200, d_k=256, d_v=512,
                dtype="bf16", chunk=64, gamma_kind="wide", qkv_std=1 / 16, seed=57)
    base.update(kw)
    return W.Workload(**base)


def seq_arrays(pos, lengths):
    return (torch.tensor(pos, dtype=torch.int64, device=DEV),
            None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device=DEV))


def check_gated(out, ref, gate):
    sw = np.abs(O.swish(gate)) if gate is not None else 1.0
    bound = 2e-2 * np.maximum(1.0, sw)
    d = np.abs(O.to64(out) - ref)
    record("gated", (d / np.maximum(1.0, sw)).max())
    assert (d <= bound).all(), float((d / bound).max())


# ---- decode with a position per sequence ---------------------------------------------

@pytest.mark.parametrize("dk,dv", [(256, 512), (64, 96)])
def test_decode_step_at_per_sequence_positions(dk, dv):
    """Four sequences at unrelated positions (0, 9, 65535, 1000003), three chained steps,
    each sequence against the oracle's step at its own position. (256, 512) runs the
    pipelined kernel, (64, 96) the one-batch kernel."""
    w = W.Workload(**{**W.WORKLOADS["decode_6p7b"].__dict__, "B": 4, "H": 3, "d_k": dk, "d_v": dv})
    S0 = W.initial_state(w)
    S = dev(S0.clone())
    Sref = [S0[b:b + 1] for b in range(4)]
    p0 = [0, 9, 65535, 1000003]
    pos = torch.tensor(p0, dtype=torch.int64, device=DEV)
    for i in range(3):
        x = W.make_decode_step_inputs(w, i)
        out = rn().rn_retention_recurrent_step_at(dev(x["q"]), dev(x["k"]), dev(x["v"]), w.gamma(),
                                                  w.theta(), S, pos, out_dtype=torch.float32)
        out = out.cpu()
        for b in range(4):
            o_ref, Sref[b] = O.recurrent_step(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1],
                                              w.gamma(), w.theta(), p0[b] + i, 1.0, Sref[b])
            assert rel_inf(out[b:b + 1, :, 0], o_ref) <= F32_BAR, (b, i)
        pos += 1   # the positions advance on the device
    Sg = S.cpu()
    for b in range(4):
        assert rel_inf(Sg[b:b + 1], Sref[b]) <= F32_BAR


def test_decode_step_at_equal_positions_is_the_plain_step():
    """With every pos[b] equal to p, the per-sequence entry computes what the plain step
    at position p does, bit for bit (same kernel, same angles)."""
    w = W.Workload(**{**W.WORKLOADS["decode_6p7b"].__dict__, "B": 3, "H": 4})
    S0 = W.initial_state(w)
    x = W.make_decode_step_inputs(w, 5)
    g = torch.randn(3, 4, 1, 512, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    S1, S2 = dev(S0.clone()), dev(S0.clone())
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), w.gamma(), w.theta())
    o1 = rn().rn_retention_recurrent_step(*args, S1, 4097, gate=dev(g), gn=True)
    pos = torch.full((3,), 4097, dtype=torch.int64, device=DEV)
    o2 = rn().rn_retention_recurrent_step_at(*args, S2, pos, gate=dev(g), gn=True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ---- prefill over a padded batch -----------------------------------------------------

CASES = [
    # lengths (N = 200 padded rows), first positions
    ([200, 0, 1, 131], [0, 5, 70000, 3]),
    ([64, 65, 127, 199], [1000, 0, 7, 123456]),
]


@pytest.mark.parametrize("lengths,pos", CASES)
@pytest.mark.parametrize("path", ["segmented", "sequential", "pair", "generic"])
def test_chunkwise_varlen_outputs_and_states(lengths, pos, path):
    """Each sequence's rows and final state against the oracle's chunkwise form on that
    sequence alone (its length, its positions, its initial state); padded rows keep the
    value they had; a length of 0 hands the initial state through."""
    w = wl(state_std=0.05)
    x = W.make_inputs(w)
    posd, lens = seq_arrays(pos, lengths)
    out = torch.full((4, 2, 200, 512), SENTINEL, dtype=torch.float32, device=DEV)
    _, S = rn().rn_retention_chunkwise_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                              x["theta"], 64, pos=posd, lengths=lens,
                                              state_in=dev(x["state"]), state_out=True, out=out,
                                              out_dtype=torch.float32, force_generic=path == "generic",
                                              chunk_parallel=path == "pair",
                                              segmented=path == "segmented")
    out, S = out.cpu(), S.cpu()
    tol = F32_BAR if path == "generic" else MFMA_BAR
    for b, (L, p) in enumerate(zip(lengths, pos)):
        sb = slice(b, b + 1)
        assert (out[sb, :, L:] == SENTINEL).all(), f"padded rows of sequence {b} written"
        if L == 0:
            assert rel_inf(S[sb], x["state"][sb]) <= 1e-6
            continue
        ref, Sref = O.chunkwise(x["q"][sb, :, :L], x["k"][sb, :, :L], x["v"][sb, :, :L],
                                x["gamma"], x["theta"], 64, p, 1.0, x["state"][sb])
        assert rel_inf(out[sb, :, :L], ref) <= tol, b
        assert rel_inf(S[sb], Sref) <= tol, b


@pytest.mark.parametrize("generic", [False, True])
def test_chunkwise_varlen_gn_gate(generic):
    """GroupNorm + gate epilogue per valid row (float32 output), from zero states."""
    w = wl(gate=True, N=150)
    x = W.make_inputs(w)
    lengths, pos = [150, 37, 64, 100], [0, 11, 2048, 99]
    posd, lens = seq_arrays(pos, lengths)
    out, _ = rn().rn_retention_chunkwise_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                                x["theta"], 64, pos=posd, lengths=lens,
                                                gate=dev(x["gate"]), gn=True,
                                                out_dtype=torch.float32, force_generic=generic)
    out = out.cpu()
    for b, (L, p) in enumerate(zip(lengths, pos)):
        sb = (slice(b, b + 1), slice(None), slice(0, L))
        raw, _ = O.chunkwise(x["q"][sb], x["k"][sb], x["v"][sb], x["gamma"], x["theta"], 64, p)
        check_gated(out[sb], O.groupnorm_gate(raw, x["gate"][sb]), x["gate"][sb])
        assert (out[b, :, L:] == 0).all()   # the binding zero-fills a new output's padding


def test_chunkwise_varlen_full_lengths_is_the_plain_call():
    """lengths = N and pos = pos0 everywhere: the fused kernel computes exactly what the
    plain chunkwise call does (bit for bit)."""
    w = wl(gate=True, N=300, state_std=0.05)
    x = W.make_inputs(w)
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 64)
    kw = dict(gate=dev(x["gate"]), gn=True, state_in=dev(x["state"]), state_out=True)
    o1, s1 = rn().rn_retention_chunkwise(*args, pos0=77, **kw)
    posd, lens = seq_arrays([77] * 4, [300] * 4)
    o2, s2 = rn().rn_retention_chunkwise_varlen(*args, pos=posd, lengths=lens, **kw)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---- the handoff: prefill, then decode -----------------------------------------------

def test_prefill_then_decode_matches_recurrent_oracle():
    """Serving end to end at the 6.7B head shape: three prompts (lengths 192, 77, 130;
    the third continues an earlier context at position 1000) prefilled in one padded
    call, then four batched decode steps continuing from the prefill's states at each
    sequence's next position. Every decode output is checked against the oracle's
    recurrent form run over the whole sequence (prompt + decoded tokens), an
    independent path from the chunkwise one."""
    w = wl(B=3, H=4, N=192, seed=91)
    x = W.make_inputs(w)
    lengths, pos = [192, 77, 130], [0, 0, 1000]
    posd, lens = seq_arrays(pos, lengths)
    _, S = rn().rn_retention_chunkwise_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                              x["theta"], 64, pos=posd, lengths=lens,
                                              state_out=True, out_dtype=torch.float32)
    step_pos = posd + lens.to(torch.int64)
    steps = []
    for i in range(4):
        d = W.make_decode_step_inputs(w, 100 + i)
        o = rn().rn_retention_recurrent_step_at(dev(d["q"]), dev(d["k"]), dev(d["v"]), x["gamma"],
                                                x["theta"], S, step_pos, out_dtype=torch.float32)
        steps.append((d, o.cpu()))
        step_pos += 1
    for b, (L, p) in enumerate(zip(lengths, pos)):
        cat = {n: torch.cat([x[n][b:b + 1, :, :L]] + [d[n][b:b + 1] for d, _ in steps], dim=2)
               for n in ("q", "k", "v")}
        ref, _ = O.recurrent(cat["q"], cat["k"], cat["v"], x["gamma"], x["theta"], p)
        for i, (_, o) in enumerate(steps):
            assert rel_inf(o[b:b + 1, :, 0], ref[:, :, L + i]) <= MFMA_BAR, (b, i)
