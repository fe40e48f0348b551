"""rn_retention_chunkwise_noalloc (the chunkwise form on the library's own device buffer,
for callers that cannot allocate) against rn_retention_chunkwise with a caller workspace:
the same kernels run, so outputs and final states agree bit for bit. Two calls in a row,
the second smaller than the first (the buffer keeps the first call's contents), then a
schedule with a larger workspace, and a call whose workspace would not fit."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rn():
    import linear_recurrent_sequence_rn_amd as m
    return m


def dev(x):
    return None if x is None else x.to(DEV)


def wl(**kw):
    base = dict(name="t", form="chunkwise", B=1, H=2, N=200, d_k=256, d_v=512, dtype="bf16",
                chunk=256, gamma_kind="wide", qkv_std=1 / 16, seed=71, gate=True, state_std=0.05)
    base.update(kw)
    return W.Workload(**base)


def both(x, chunk, **kw):
    """The same call through both entry points, outputs preallocated for the new one."""
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    args = (q, k, v, x["gamma"], x["theta"], chunk)
    common = dict(gate=dev(x["gate"]), state_in=dev(x["state"]), gn=True, **kw)
    ref_out, ref_S = rn().rn_retention_chunkwise(*args, state_out=True, **common)
    out = torch.full_like(ref_out, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    got_out, got_S = rn().rn_retention_chunkwise_noalloc(*args, out=out, state_out=S, **common)
    torch.cuda.synchronize()
    assert got_out.data_ptr() == out.data_ptr() and got_S.data_ptr() == S.data_ptr()
    return (got_out.cpu(), got_S.cpu()), (ref_out.cpu(), ref_S.cpu())


def test_two_calls_in_a_row_the_second_smaller():
    big = W.make_inputs(wl(B=2, H=16, N=2048))
    (o1, s1), (r1, t1) = both(big, 256)
    assert torch.equal(o1, r1) and torch.equal(s1, t1)
    small = W.make_inputs(wl(B=1, H=2, N=300, seed=72))
    (o2, s2), (r2, t2) = both(small, 64)
    assert torch.equal(o2, r2) and torch.equal(s2, t2)
    # and the smaller call against the oracle, at the chunkwise tests' bars
    raw, Sref = O.chunkwise(small["q"], small["k"], small["v"], small["gamma"], small["theta"],
                            64, 0, 1.0, small["state"])
    ref = O.groupnorm_gate(raw, small["gate"])
    d = np.abs(O.to64(o2) - ref)
    assert (d <= 2e-2 * np.maximum(1.0, np.abs(O.swish(small["gate"])))).all()
    err = np.abs(O.to64(s2) - Sref).max() / np.abs(Sref).max()
    assert err <= 3e-3


def test_segmented_schedule_fits_for_two_heads():
    x = W.make_inputs(wl(B=1, H=2, N=700, seed=73))
    (o, s), (r, t) = both(x, 256, segmented=True)
    assert torch.equal(o, r) and torch.equal(s, t)


def test_workspace_beyond_the_buffer_is_rejected():
    """d_v = 256 with 64 heads needs 34 MiB: rejected before any launch, outputs untouched."""
    x = W.make_inputs(wl(B=4, H=16, N=64, d_v=256, gate=False, state_std=0.0))
    out = torch.zeros(4, 16, 64, 256, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rn().RnError, match="RN_ERR_UNSUPPORTED"):
        rn().rn_retention_chunkwise_noalloc(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["gamma"],
                                            x["theta"], 64, out=out)
    assert int(torch.count_nonzero(out)) == 0
