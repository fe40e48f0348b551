"""GPU parity of the gated multi-scale retention layer (rn_msr_layer_forward) against the
layer oracle (oracle/layer.py, float64 throughout).

Tolerance. The GPU path rounds Q, K, V, G and the heads' outputs to bf16 (relative
2^-9 each) and runs the retention with half operands (about 4e-3 after GroupNorm, the
retention bar being 2e-2); the output projection sums H d_v such terms with independent
rounding, so its error is of the size of one term's relative error times the output's
scale. Bar: per batch row, max-abs error <= 2e-2 of the row block's max |ref| and RMS
error <= 1e-2 of its RMS (measured well below both); a bf16 output adds half a bf16 ulp
of the reference. A head read from the wrong columns or concatenated in the wrong place
gives errors of the output's own size.
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


def check(out, ref):
    g = O.to64(out)
    for b in range(ref.shape[0]):
        err = np.abs(g[b] - ref[b])
        bound = 2e-2 * np.abs(ref[b]).max()
        if out.dtype == torch.bfloat16:
            err = err - np.abs(ref[b]) * 2.0 ** -9
        record("layer_max", err.max() / np.abs(ref[b]).max())
        assert err.max() <= bound, (b, float(err.max() / bound))
        rms = np.sqrt(((g[b] - ref[b]) ** 2).mean())
        record("layer_rms", rms / np.sqrt((ref[b] ** 2).mean()))
        assert rms <= 1e-2 * np.sqrt((ref[b] ** 2).mean()), (b, rms)


def wl(**kw):
    base = dict(name="layer", form="chunkwise", B=2, H=2, N=300, d_k=256, d_v=512, dtype="bf16",
                chunk=256, gn=True, gate=True, gamma_kind="wide", seed=61)
    base.update(kw)
    return W.Workload(**base)


def run(w, D, *, gate=True, gn=True, out_dtype=None, state=False, pos0=0, gamma=None, gnp=False):
    x = W.make_layer_inputs(w, D)
    gm = x["gamma"] if gamma is None else gamma
    g_dev = torch.from_numpy(gm).to(DEV) if np.ndim(gm) == 2 else gm
    H, dv = w.H, w.d_v
    gw = gb = None
    if gnp:
        gw = torch.randn(H * dv, generator=torch.Generator().manual_seed(8)) * 0.3 + 1
        gb = torch.randn(H * dv, generator=torch.Generator().manual_seed(9)) * 0.1
    s0 = None
    if state:
        s0 = torch.randn(w.B, H, w.d_k, dv, generator=torch.Generator().manual_seed(10)) * 0.05
    out, S = rn().rn_msr_layer_forward(
        dev(x["x"]), dev(x["w_q"]), dev(x["w_k"]), dev(x["w_v"]), dev(x["w_g"]) if gate else None,
        dev(x["w_o"]), g_dev, x["theta"], H, w.d_k, dv, w.chunk, state_in=dev(s0), state_out=True,
        out_dtype=out_dtype, pos0=pos0, gn=gn, gn_weight=dev(gw), gn_bias=dev(gb))
    torch.cuda.synchronize()
    if gn:
        ref, Sref = O.msr_layer(x["x"], x["w_q"], x["w_k"], x["w_v"], x["w_g"], x["w_o"], gm,
                                x["theta"], H, chunk=w.chunk, pos0=pos0, state0=s0,
                                gn_weight=None if gw is None else gw.reshape(H, dv),
                                gn_bias=None if gb is None else gb.reshape(H, dv), gate=gate)
    else:
        # without GroupNorm: the heads' raw retention, gated, projected (composition of
        # the oracle's pieces)
        xx = O.to64(x["x"])
        q = O.split_heads(xx @ O.to64(x["w_q"]), H)
        k = O.split_heads(xx @ O.to64(x["w_k"]), H)
        v = O.split_heads(xx @ O.to64(x["w_v"]), H)
        ret, Sref = O.chunkwise(q, k, v, gm, x["theta"], w.chunk, pos0, 1.0, s0)
        if gate:
            ret = ret * O.swish(O.split_heads(xx @ O.to64(x["w_g"]), H))
        ref = O.merge_heads(ret) @ O.to64(x["w_o"])
    return out.cpu(), S.cpu(), ref, Sref


def test_layer_fused_retention_path():
    out, S, ref, Sref = run(wl(), 512)
    check(out, ref)
    assert np.abs(O.to64(S) - Sref).max() <= 1e-2 * np.abs(Sref).max()


def test_layer_state_in_positions_affine_fp32_out():
    out, S, ref, Sref = run(wl(N=257), 512, out_dtype=torch.float32, state=True, pos0=1000, gnp=True)
    check(out, ref)
    assert np.abs(O.to64(S) - Sref).max() <= 1e-2 * np.abs(Sref).max()


def test_layer_pair_decays():
    w = wl(N=333, gamma_kind="pair_wide")
    out, S, ref, Sref = run(w, 512)
    check(out, ref)


def test_layer_generic_retention_shape_without_gate():
    """d_k = 64 runs the retention on the float32 generic kernel; no gate."""
    w = wl(H=4, d_k=64, d_v=64, N=100, gamma_kind="small")
    out, S, ref, Sref = run(w, 256, gate=False)
    check(out, ref)


def test_layer_without_groupnorm_or_gate():
    """The gate goes with GroupNorm (as in the retention entry points); without both, the
    layer is the heads' raw retention concatenated and projected."""
    out, S, ref, Sref = run(wl(N=130), 512, gn=False, gate=False)
    check(out, ref)


def test_layer_6p7b_shape_one_batch_row():
    """The 6.7B layer shape (d_model 4096, 16 heads of 256/512, N = 8192, batch 2) in the
    launch configuration the benchmark times; batch row 1 is checked in full against the
    oracle (its float64 projections take seconds on the host)."""
    w = W.WORKLOADS["chunkwise_6p7b"]
    x = W.make_layer_inputs(w, W.LAYER_D_MODEL)
    out, S = rn().rn_msr_layer_forward(
        dev(x["x"]), dev(x["w_q"]), dev(x["w_k"]), dev(x["w_v"]), dev(x["w_g"]), dev(x["w_o"]),
        x["gamma"], x["theta"], w.H, w.d_k, w.d_v, w.chunk, state_out=True)
    torch.cuda.synchronize()
    out, S = out.cpu(), S.cpu()
    ref, Sref = O.msr_layer(x["x"][1:2], x["w_q"], x["w_k"], x["w_v"], x["w_g"], x["w_o"],
                            x["gamma"], x["theta"], w.H, chunk=w.chunk)
    check(out[1:2], ref)
    assert np.abs(O.to64(S[1:2]) - Sref).max() <= 1e-2 * np.abs(Sref).max()
