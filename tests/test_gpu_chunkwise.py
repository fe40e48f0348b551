"""GPU parity of the MFMA chunkwise schedules (bf16 q/k/v, d_k = 256): the sequential
single kernel (the default), the segmented schedule (RN_CHUNK_SEGMENTED: segment-local
states, a scan over segments, then the outputs; d_v = 512) and the chunk-parallel pair
(RN_CHUNK_PARALLEL: state snapshots, then outputs; d_v = 512).

Tolerances (half-precision MFMA operands, fp32 accumulation), about five times the
largest error measured over these tests:
  * raw outputs and final states: per (b, h), ||gpu - ref||_inf <= MFMA_BAR ||ref||_inf.
    Qh, Kh, V, the copy of the state used by the cross term and the decayed scores are
    each rounded to IEEE half (relative 2^-11); an output is a sum of many such terms
    of mixed sign, so the error of one element is a few 2^-11 of the typical magnitude
    (measured at most 5.2e-4 of the slice maximum; 3.0e-4 for the states of the 6.7B
    and long-sequence workloads).
  * after GroupNorm (fp32 output): max-abs 2e-2; with the gate, 2e-2 * max(1, |swish(g)|)
    (measured at most 3.9e-3; 2.9e-3 on the 6.7B and long-sequence workloads).
  * bf16 output: the same bound plus half a bf16 ulp of the reference.
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
    base = dict(name="t", form="chunkwise", B=1, H=2, N=200, d_k=256, d_v=512, dtype="bf16",
                chunk=64, gamma_kind="wide", qkv_std=1 / 16, seed=31)
    base.update(kw)
    return W.Workload(**base)


def check_gated(out, ref, gate):
    sw = np.abs(O.swish(gate)) if gate is not None else 1.0
    bound = 2e-2 * np.maximum(1.0, sw)
    d = np.abs(O.to64(out) - ref)
    record("gated", ((d - (np.abs(ref) * 2.0 ** -8 if out.dtype == torch.bfloat16 else 0.0))
                     / np.maximum(1.0, sw)).max())
    if out.dtype == torch.bfloat16:
        bound = bound + np.abs(ref) * 2.0 ** -8
    assert (d <= bound).all(), float((d / bound).max())


def ws_for(q, v, gamma, theta, chunk, **kw):
    n = rn().rn_chunkwise_workspace_bytes(q, v, gamma, theta, chunk, **kw)
    return torch.zeros(n, dtype=torch.uint8, device=DEV)


STATUS_BYTES = 256   # every matrix-core schedule's call status word leads its workspace


def counters(ws, heads):
    """Per-head counter blocks of the sequential kernel (64 words each, after the status)."""
    c = ws[STATUS_BYTES: STATUS_BYTES + heads * 256].view(torch.int32).reshape(heads, 64)
    return c.cpu().numpy()


def slices_per_xcd(c):
    """Words 2-3 of each counter block: the 64-bit arrival word, nibble x = slices on XCD x."""
    out = []
    for lo, hi in c[:, 2:4]:
        a = (int(lo) & 0xFFFFFFFF) | ((int(hi) & 0xFFFFFFFF) << 32)
        out.append([(a >> (4 * x)) & 15 for x in range(16)])
    return out


SCHEDULES = ["segmented", "sequential", "pair"]
MFMA_BAR = 3e-3      # raw outputs and states: ||gpu - ref||_inf / ||ref||_inf per (b, h)
STATE_BAR = MFMA_BAR


def sk(schedule):
    """Binding keywords that select a schedule."""
    return dict(chunk_parallel=schedule == "pair", segmented=schedule == "segmented")


@pytest.mark.parametrize("cp", SCHEDULES)
@pytest.mark.parametrize("N,pos0", [(200, 0), (64, 5), (1, 70000), (129, 3), (700, 11)])
def test_raw_output_and_state(N, pos0, cp):
    w = wl(N=N, state_std=0.05)
    x = W.make_inputs(w)
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 64, state_in=dev(x["state"]), state_out=True,
                                         out_dtype=torch.float32, pos0=pos0, **sk(cp))
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 64, pos0, 1.0, x["state"])
    assert rel_inf(out.cpu(), ref) <= MFMA_BAR
    assert rel_inf(S.cpu(), Sref) <= MFMA_BAR


@pytest.mark.parametrize("cp", SCHEDULES)
def test_gn_gate_affine_fp32_and_bf16_out(cp):
    w = wl(N=333, gate=True)
    x = W.make_inputs(w)
    H, dv = 2, 512
    gw = torch.randn(H * dv, generator=torch.Generator().manual_seed(3)) * 0.5 + 1
    gb = torch.randn(H * dv, generator=torch.Generator().manual_seed(4)) * 0.1
    raw, _ = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 256)
    ref = O.groupnorm_gate(raw, x["gate"], 1e-5, gw.reshape(H, dv), gb.reshape(H, dv))
    for od in (torch.float32, torch.bfloat16):
        out, _ = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                             x["theta"], 256, gate=dev(x["gate"]), gn=True,
                                             gn_weight=dev(gw), gn_bias=dev(gb), out_dtype=od,
                                             **sk(cp))
        check_gated(out.cpu(), ref, x["gate"])


@pytest.mark.parametrize("dv", [64, 128, 256])
def test_value_dims(dv):
    w = wl(d_v=dv, N=150, H=3)
    x = W.make_inputs(w)
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 32, state_out=True, out_dtype=torch.float32)
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 32)
    assert rel_inf(out.cpu(), ref) <= MFMA_BAR
    assert rel_inf(S.cpu(), Sref) <= MFMA_BAR
    out, _ = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 32, gn=True, out_dtype=torch.float32)
    check_gated(out.cpu(), O.group_norm(ref), None)


def test_exchange_diagnostics_and_determinism():
    """Sequential kernel: every slice of a head reports the same XCD (the L2 exchange path is the one in
    use), no wait hit its time limit, and two runs agree bit for bit."""
    w = wl(N=300, H=4, gate=True)
    x = W.make_inputs(w)
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 64)
    ws = ws_for(args[0], args[2], x["gamma"], x["theta"], 64, gn=True, gate=x["gate"])
    outs = []
    for _ in range(2):
        o, s = rn().rn_retention_chunkwise(*args, gate=dev(x["gate"]), gn=True, state_out=True,
                                           workspace=ws)
        outs.append((o.cpu(), s.cpu()))
    torch.cuda.synchronize()
    c = counters(ws, 4)
    nibbles = slices_per_xcd(c)
    print("xcc per slice:", c[:, 8:16].tolist(), "slices per XCD:", nibbles)
    assert (c[:, 4] == 0).all(), "an exchange wait hit its time limit"
    # all 8 slices arrived, all on one XCD, and the XCD each slice recorded agrees
    assert all(sorted(n)[-1] == 8 and sum(n) == 8 for n in nibbles), "slices of a head span XCDs"
    assert all(n[int(c[h, 8])] == 8 and len(set(c[h, 8:16].tolist())) == 1
               for h, n in enumerate(nibbles))
    # 5 blocks x 8 slices x 4 waves (counters are cleared per launch): the 8 ring slots
    # and the 8 statistics slots count blocks 0..4 once each
    assert c[:, 16:24].tolist() == [[32, 32, 32, 32, 32, 0, 0, 0]] * 4
    assert c[:, 24:32].tolist() == [[32, 32, 32, 32, 32, 0, 0, 0]] * 4
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("cp", SCHEDULES)
def test_more_heads_than_one_launch(cp):
    """80 heads: more than one co-resident launch of the sequential kernel (48 heads x 8
    slices fill 256 CUs) and more than one 64-head group of the chunk-parallel pair."""
    w = wl(B=5, H=16, N=70)
    x = W.make_inputs(w)
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                         x["theta"], 64, state_out=True, out_dtype=torch.float32,
                                         **sk(cp))
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 64)
    assert rel_inf(out.cpu(), ref) <= MFMA_BAR
    assert rel_inf(S.cpu(), Sref) <= MFMA_BAR


def gated_err(out, ref, gate):
    """max |out - ref| / max(1, |swish(gate)|): the error in units of the post-GroupNorm bar."""
    sw = np.abs(O.swish(gate)) if gate is not None else 1.0
    return float((np.abs(O.to64(out) - ref) / np.maximum(1.0, sw)).max())


def test_6p7b_training_shape_all_heads():
    """The 6.7B-shaped training workload (B=2, H=16, N=8192, chunk 256, GroupNorm + gate)
    in the launch configuration the benchmark times, for all three schedules; every one of
    the 32 (b, h) checked in full against the oracle (outputs and final states)."""
    w = W.WORKLOADS["chunkwise_6p7b"]
    x = W.make_inputs(w)
    res = {}
    for cp in SCHEDULES:
        out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                             x["theta"], w.chunk, gate=dev(x["gate"]), gn=True,
                                             state_out=True, out_dtype=torch.float32, **sk(cp))
        res[cp] = (out.cpu(), S.cpu())
        del out, S
        assert torch.isfinite(res[cp][0]).all(), cp
    worst = {cp: [0.0, 0.0] for cp in SCHEDULES}
    for b in range(w.B):
        for h in range(w.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            raw, Sref = O.chunkwise(x["q"][sl], x["k"][sl], x["v"][sl], x["gamma"][h:h + 1],
                                    x["theta"], w.chunk)
            ref = O.groupnorm_gate(raw, x["gate"][sl])
            for cp in SCHEDULES:
                out, S = res[cp]
                check_gated(out[sl], ref, x["gate"][sl])
                worst[cp][0] = max(worst[cp][0], gated_err(out[sl], ref, x["gate"][sl]))
                worst[cp][1] = max(worst[cp][1], rel_inf(S[sl], Sref))
    print("6.7B training shape, worst (gated output, relative state):", worst)
    for cp in SCHEDULES:
        assert worst[cp][1] <= STATE_BAR, (cp, worst[cp])


def test_long_sequence_four_heads():
    """Long-sequence workload (B=1, H=16, N=65536, chunk 512, GroupNorm) for all three
    schedules, each run twice (bit-identical: no exchange race); heads 0, 5, 11 and 15 (the
    fastest to the slowest decay) checked in full. The workspace does not grow with N (the
    chunk-parallel pair and the segmented schedule run windows of 32 chunks and carry the
    state between them)."""
    w = W.WORKLOADS["chunkwise_long"]
    x = W.make_inputs(w)
    heads = [0, 5, 11, 15]
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], w.chunk)
    res = {}
    for cp in SCHEDULES:
        sizes = [rn().rn_chunkwise_workspace_bytes(x["q"][:, :, :n], x["v"][:, :, :n], x["gamma"],
                                                   x["theta"], 512, gn=True, **sk(cp))
                 for n in (8192 + 256, 65536)]
        assert sizes[0] == sizes[1], cp
        kw = dict(gn=True, state_out=True, out_dtype=torch.float32, **sk(cp))
        out, S = rn().rn_retention_chunkwise(*args, **kw)
        out2, S2 = rn().rn_retention_chunkwise(*args, **kw)
        assert torch.equal(out, out2) and torch.equal(S, S2), (cp, "runs differ: exchange race")
        res[cp] = (out[:, heads].cpu(), S[:, heads].cpu())
        del out, S, out2, S2
    worst = {cp: [0.0, 0.0] for cp in SCHEDULES}
    for i, h in enumerate(heads):
        sl = (slice(0, 1), slice(h, h + 1))
        raw, Sref = O.chunkwise(x["q"][sl], x["k"][sl], x["v"][sl], x["gamma"][h:h + 1],
                                x["theta"], 2048)
        ref = O.group_norm(raw)
        for cp in SCHEDULES:
            out, S = res[cp]
            got = out[:, i:i + 1]
            check_gated(got, ref, None)
            worst[cp][0] = max(worst[cp][0], gated_err(got, ref, None))
            worst[cp][1] = max(worst[cp][1], rel_inf(S[:, i:i + 1], Sref))
    print("long sequence, worst (output, relative state):", worst)
    for cp in SCHEDULES:
        assert worst[cp][1] <= STATE_BAR, (cp, worst[cp])


def test_chunk_parallel_snapshots_are_the_chunk_states():
    """The chunk-parallel pair's first kernel leaves, in the caller's workspace, the state
    at the start of every 256-token chunk (rounded to half, stored transposed in pieces of
    32 d_k rows: [head][chunk][piece][d_v][32]); each is checked against the oracle's state
    after the chunk's prefix."""
    w = wl(B=1, H=2, N=600, state_std=0.05)
    x = W.make_inputs(w)
    ws = ws_for(x["q"], x["v"], x["gamma"], x["theta"], 256, chunk_parallel=True)
    rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 256,
                                state_in=dev(x["state"]), workspace=ws, out_dtype=torch.float32,
                                chunk_parallel=True)
    torch.cuda.synchronize()
    snap = ws[STATUS_BYTES: STATUS_BYTES + 2 * 32 * 256 * 512 * 2].view(torch.float16).reshape(2, 32, 8, 512, 32)
    for c in range(3):
        # [head, piece, d_v, 32] -> [head, piece, 32, d_v] -> S [head, d_k, d_v]
        got = snap[:, c].permute(0, 1, 3, 2).reshape(2, 256, 512).cpu().to(torch.float64).numpy()[None]
        if c == 0:
            ref = O.to64(x["state"])
        else:
            sl = slice(0, 256 * c)
            _, ref = O.chunkwise(x["q"][:, :, sl], x["k"][:, :, sl], x["v"][:, :, sl], x["gamma"],
                                 x["theta"], 256, 0, 1.0, x["state"])
        assert rel_inf(got, ref) <= MFMA_BAR, c


def test_small_decay_takes_a_schedule_without_a_decay_limit():
    """A head with gamma^32 < 2^-6 (gamma = 0.8) is outside the sequential kernel's operand
    range; the default call then takes the segmented schedule, which applies the decay in
    float32 (as does the chunk-parallel pair). Both checked against the oracle, outputs and
    state."""
    w = wl(N=300, state_std=0.05)
    x = W.make_inputs(w)
    gamma = np.array([0.8, 0.97], dtype=np.float32)
    n_default = rn().rn_chunkwise_workspace_bytes(x["q"], x["v"], gamma, x["theta"], 64)
    n_seg = rn().rn_chunkwise_workspace_bytes(x["q"], x["v"], gamma, x["theta"], 64, segmented=True)
    assert n_default == n_seg
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], gamma, x["theta"], 64, 0, 1.0, x["state"])
    for kw in (dict(), dict(chunk_parallel=True)):
        out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), gamma, x["theta"],
                                             64, state_in=dev(x["state"]), state_out=True,
                                             out_dtype=torch.float32, **kw)
        assert rel_inf(out.cpu(), ref) <= MFMA_BAR, kw
        assert rel_inf(S.cpu(), Sref) <= MFMA_BAR, kw


def test_segmented_states_in_the_workspace():
    """The segmented schedule's intermediate states, read back from the caller's workspace
    ([heads][32 chunks][d_v][d_k] half L, then [heads][4][d_v][d_k] float32 E, then
    [heads][4][d_v][d_k] half T): T_g is the state at segment g's start (2048 tokens
    apart), and L at a chunk start plus gamma^(c0 - s_g) T_g is the state there."""
    w = wl(B=1, H=2, N=2048 + 600, state_std=0.05)
    x = W.make_inputs(w)
    ws = ws_for(x["q"], x["v"], x["gamma"], x["theta"], 256, segmented=True)
    rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"], x["theta"], 256,
                                state_in=dev(x["state"]), workspace=ws, out_dtype=torch.float32,
                                segmented=True)
    torch.cuda.synchronize()
    heads, snap = 2, 256 * 512
    L = ws[STATUS_BYTES: STATUS_BYTES + heads * 32 * snap * 2].view(torch.float16).reshape(heads, 32, 512, 256)
    off = STATUS_BYTES + heads * 32 * snap * 2 + heads * 4 * snap * 4
    T = ws[off: off + heads * 4 * snap * 2].view(torch.float16).reshape(heads, 4, 512, 256)

    def state_at(t):
        if t == 0:
            return O.to64(x["state"])
        sl = slice(0, t)
        return O.chunkwise(x["q"][:, :, sl], x["k"][:, :, sl], x["v"][:, :, sl], x["gamma"],
                           x["theta"], 256, 0, 1.0, x["state"])[1]

    def host(t):   # [heads, d_v, d_k] half -> [1, heads, d_k, d_v] float64
        return t.permute(0, 2, 1).cpu().to(torch.float64).numpy()[None]

    g = np.asarray(x["gamma"], dtype=np.float64)[None, :, None, None]
    for seg in (0, 1):
        assert rel_inf(host(T[:, seg]), state_at(2048 * seg)) <= MFMA_BAR, seg
    for c in (1, 5, 9, 10):
        c0, s0 = 256 * c, 2048 * (c // 8)
        got = host(L[:, c]) + g ** (c0 - s0) * host(T[:, c // 8])
        assert rel_inf(got, state_at(c0)) <= MFMA_BAR, c


@pytest.mark.parametrize("gammas", [(1.0, 0.999), (0.5, 1e-6)])
def test_segmented_decays_without_a_limit(gammas):
    """The segmented schedule applies the decay only as factors at most 1 (operands) or in
    float32 (scores, row scales), so decays from 1 down to 1e-6 hold, across segment
    boundaries (2048 tokens) and a window boundary (8192): N = 8192 + 300 with an initial
    state, raw outputs and final state against the oracle."""
    w = wl(N=8192 + 300, state_std=0.05)
    x = W.make_inputs(w)
    gamma = np.array(gammas, dtype=np.float32)
    out, S = rn().rn_retention_chunkwise(dev(x["q"]), dev(x["k"]), dev(x["v"]), gamma, x["theta"], 256,
                                         state_in=dev(x["state"]), state_out=True,
                                         out_dtype=torch.float32, segmented=True)
    ref, Sref = O.chunkwise(x["q"], x["k"], x["v"], gamma, x["theta"], 256, 0, 1.0, x["state"])
    assert torch.isfinite(out).all() and torch.isfinite(S).all()
    assert rel_inf(out.cpu(), ref) <= MFMA_BAR
    assert rel_inf(S.cpu(), Sref) <= MFMA_BAR


def status(q, v, gamma, theta, chunk, ws, **kw):
    return rn().rn_chunkwise_check(q, v, gamma, theta, chunk, ws, **kw)


@pytest.mark.parametrize("od", [torch.float32, torch.bfloat16])
def test_forced_time_out_is_reported_and_outputs_are_nan(od):
    """RN_TEST_FORCE_TIMEOUT makes every exchange wait of the sequential kernel give up at
    once, as a wait past its time limit does: the call's status reads RN_ERR_EXCHANGE and
    every output and final state is NaN. The next call on the same workspace starts from a
    clear status and matches the oracle."""
    w = wl(N=300, H=2, gate=True, state_std=0.05)
    x = W.make_inputs(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    kw = dict(gate=dev(x["gate"]), gn=True, out_dtype=od)
    ws = ws_for(q, v, x["gamma"], x["theta"], 64, **kw)
    call = dict(state_in=dev(x["state"]), state_out=True, workspace=ws, **kw)
    out, S = rn().rn_retention_chunkwise(q, k, v, x["gamma"], x["theta"], 64,
                                         test_force_timeout=True, **call)
    assert status(q, v, x["gamma"], x["theta"], 64, ws, **kw) == rn().RN_ERR_EXCHANGE
    assert torch.isnan(out).all() and torch.isnan(S).all()
    assert counters(ws, 2)[:, 4].tolist() == [1, 1]
    out, S = rn().rn_retention_chunkwise(q, k, v, x["gamma"], x["theta"], 64, **call)
    assert status(q, v, x["gamma"], x["theta"], 64, ws, **kw) == rn().RN_OK
    raw, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 64, 0, 1.0, x["state"])
    check_gated(out.cpu(), O.groupnorm_gate(raw, x["gate"]), x["gate"])
    assert rel_inf(S.cpu(), Sref) <= STATE_BAR


def finite_or_reported(out, S, st):
    """Outputs are either all finite with status RN_OK, or the status says RN_ERR_NONFINITE."""
    finite = bool(torch.isfinite(out).all()) and bool(torch.isfinite(S).all())
    assert st in (rn().RN_OK, rn().RN_ERR_NONFINITE), st
    assert finite == (st == rn().RN_OK), (finite, st)
    return finite


def test_no_decay_constant_inputs_over_64k_tokens():
    """gamma = 1 and q = k = v = 1 over N = 65536 (the state grows with every token and is
    never decayed): the default schedule either matches the oracle or reports
    RN_ERR_NONFINITE; never an unreported infinity or NaN."""
    N = 65536
    q = torch.ones(1, 1, N, 256, dtype=torch.bfloat16)
    v = torch.ones(1, 1, N, 512, dtype=torch.bfloat16)
    g, th = np.ones(1, dtype=np.float32), W.theta_default(256)
    ws = ws_for(dev(q), dev(v), g, th, 512)
    out, S = rn().rn_retention_chunkwise(dev(q), dev(q), dev(v), g, th, 512, state_out=True,
                                         workspace=ws, out_dtype=torch.float32)
    st = status(dev(q), dev(v), g, th, 512, ws)
    if finite_or_reported(out, S, st):
        raw, Sref = O.chunkwise(q, q, v, g, th, 2048)
        e = rel_inf(out.cpu(), raw)
        print(f"gamma = 1, constant inputs, N = 65536: relative error {e:.2e}, "
              f"max |S| {float(np.abs(Sref).max()):.3g}")
        assert e <= MFMA_BAR
        assert rel_inf(S.cpu(), Sref) <= STATE_BAR
    else:
        print("gamma = 1, constant inputs, N = 65536: reported RN_ERR_NONFINITE")


@pytest.mark.parametrize("cp", SCHEDULES)
@pytest.mark.parametrize("mag", [1 / 16, 2e3, 1e5])
def test_large_inputs_match_or_are_reported(mag, cp):
    """q, k, v ~ N(0, mag^2): beyond the half-precision operand range each matrix-core
    schedule reports RN_ERR_NONFINITE rather than returning unreported infinities or NaNs;
    within it, the outputs match the oracle and the status is RN_OK."""
    w = wl(N=1000, H=2, qkv_std=mag, seed=41)
    x = W.make_inputs(w)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    ws = ws_for(q, v, x["gamma"], x["theta"], 64, **sk(cp))
    out, S = rn().rn_retention_chunkwise(q, k, v, x["gamma"], x["theta"], 64, state_out=True,
                                         workspace=ws, out_dtype=torch.float32, **sk(cp))
    st = status(q, v, x["gamma"], x["theta"], 64, ws, **sk(cp))
    if finite_or_reported(out, S, st):
        raw, Sref = O.chunkwise(x["q"], x["k"], x["v"], x["gamma"], x["theta"], 64)
        assert rel_inf(out.cpu(), raw) <= MFMA_BAR
        assert rel_inf(S.cpu(), Sref) <= STATE_BAR
    if mag < 1:
        assert st == rn().RN_OK
    print(f"{cp}: inputs ~ N(0, {mag:g}^2): status {st}")


def test_near_the_decay_and_operand_limits():
    """gamma^32 just above 2^-6 (the smallest decay the sequential kernel takes: its half
    operands carry factors up to gamma^-31 ~ 2^6) with |k| up to ~500: finite, status
    RN_OK, and within the raw-output bar of the oracle."""
    w = wl(N=700, H=2, seed=43)
    x = W.make_inputs(w)
    gen = torch.Generator().manual_seed(44)
    kbig = (torch.randn(x["k"].shape, generator=gen) * 100).to(torch.bfloat16)
    g = np.full(2, 2.0 ** (-6 / 32) + 1e-6, dtype=np.float32)
    q, k, v = dev(x["q"]), dev(kbig), dev(x["v"])
    ws = ws_for(q, v, g, x["theta"], 64)
    assert ws.numel() == ws_for(q, v, np.full(2, 0.99, np.float32), x["theta"], 64).numel()
    out, S = rn().rn_retention_chunkwise(q, k, v, g, x["theta"], 64, state_out=True, workspace=ws,
                                         out_dtype=torch.float32)
    assert status(q, v, g, x["theta"], 64, ws) == rn().RN_OK
    # the sequential kernel ran (8 slices arrived per head)
    assert [sum(n) for n in slices_per_xcd(counters(ws, 2))] == [8, 8]
    raw, Sref = O.chunkwise(x["q"], kbig, x["v"], g, x["theta"], 64)
    e = rel_inf(out.cpu(), raw)
    print(f"gamma^32 = 2^-6, max |k| {float(kbig.abs().max()):.0f}: relative error {e:.2e}")
    assert e <= MFMA_BAR
    assert rel_inf(S.cpu(), Sref) <= STATE_BAR
