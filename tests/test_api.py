"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, and rejects invalid arguments before any HIP call.
Pointers passed here are never dereferenced: validation fails first."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import linear_recurrent_sequence_rn_amd as rn

ROOT = Path(__file__).resolve().parents[1]
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def header_symbols():
    txt = "\n".join(p.read_text() for p in (ROOT / "include").glob("*.h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(rn_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    syms = header_symbols()
    for s in ("rn_retention_parallel", "rn_retention_chunkwise", "rn_retention_recurrent_step",
              "rn_groupnorm_gate"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(str(rn.LIB_PATH))
    for s in header_symbols():
        assert hasattr(so, s), s
    assert set(header_symbols()) == set(rn.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    assert re.match(r"\d+\.\d+\.\d+", rn.rn_version())
    assert rn.lib.rn_status_str(rn.RN_ERR_WORKSPACE) == b"RN_ERR_WORKSPACE"
    assert rn.lib.rn_status_str(-99) == b"RN_ERR_UNKNOWN"


def desc(**kw):
    p = dict(B=1, H=2, N=8, d_k=16, d_v=16, in_dtype=rn.RN_BF16, out_dtype=rn.RN_F32,
             gamma=[0.9, 0.8], theta=np.ones(8), flags=0, pos0=0, qk_scale=1.0, gn_eps=1e-5)
    p.update(kw)
    g, th = p.pop("gamma"), p.pop("theta")
    B, H, N, dk, dv, i, o = (p.pop(x) for x in ("B", "H", "N", "d_k", "d_v", "in_dtype", "out_dtype"))
    return rn.make_desc(B, H, N, dk, dv, i, o, g, th, **p)


def par(d, gate=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return rn.lib.rn_retention_parallel(ctypes.byref(d), FAKE, FAKE, FAKE, gate, FAKE, ws, ws_bytes, None)


def chk(d, chunk=4, ws_bytes=1 << 30, ws=FAKE):
    return rn.lib.rn_retention_chunkwise(ctypes.byref(d), chunk, FAKE, FAKE, FAKE, FAKE, None,
                                         None, FAKE, ws, ws_bytes, None)


def step(d, state=FAKE):
    return rn.lib.rn_retention_recurrent_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, state,
                                              FAKE, None)


def chk_varlen(d, pos=FAKE, lengths=FAKE, chunk=4, ws_bytes=1 << 30):
    return rn.lib.rn_retention_chunkwise_varlen(ctypes.byref(d), chunk, pos, lengths, FAKE, FAKE,
                                                FAKE, FAKE, None, None, FAKE, FAKE, ws_bytes, None)


def step_at(d, pos=FAKE, state=FAKE):
    return rn.lib.rn_retention_recurrent_step_at(ctypes.byref(d), pos, FAKE, FAKE, FAKE, FAKE,
                                                 state, FAKE, None)


BAD_DESCS = [
    (dict(B=0), rn.RN_ERR_INVALID_ARG),
    (dict(N=0), rn.RN_ERR_INVALID_ARG),
    (dict(d_k=15, theta=np.ones(7)), rn.RN_ERR_INVALID_ARG),
    (dict(d_k=258, theta=np.ones(129)), rn.RN_ERR_UNSUPPORTED),
    (dict(d_v=513), rn.RN_ERR_UNSUPPORTED),
    (dict(H=129, gamma=np.full(129, 0.9)), rn.RN_ERR_UNSUPPORTED),
    (dict(in_dtype=7), rn.RN_ERR_INVALID_ARG),
    (dict(out_dtype=-1), rn.RN_ERR_INVALID_ARG),
    (dict(flags=1 << 20), rn.RN_ERR_INVALID_ARG),
    (dict(flags=rn.RN_EPI_GATE), rn.RN_ERR_INVALID_ARG),          # gate without GN
    (dict(gamma=[0.9, 0.0]), rn.RN_ERR_INVALID_ARG),
    (dict(gamma=[0.9, 1.5]), rn.RN_ERR_INVALID_ARG),
    (dict(gamma=[float("nan"), 0.5]), rn.RN_ERR_INVALID_ARG),
    (dict(theta=np.r_[np.ones(7), np.inf]), rn.RN_ERR_INVALID_ARG),
    (dict(qk_scale=float("inf")), rn.RN_ERR_INVALID_ARG),
    (dict(flags=rn.RN_EPI_GN, gn_eps=-1.0), rn.RN_ERR_INVALID_ARG),
    (dict(pos0=-1), rn.RN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,code", BAD_DESCS)
def test_invalid_descriptors_rejected_everywhere(kw, code):
    d, keep = desc(**kw)
    assert par(d) == code, rn.lib.rn_last_error()
    assert rn.lib.rn_last_error() != b""
    assert chk(d) == code
    assert chk_varlen(d) == code
    assert chk_varlen(d, pos=None, lengths=None) == code
    d1, keep1 = desc(**{**kw, "N": 1} if "N" not in kw else kw)
    assert step(d1) == code
    assert step_at(d1) == code
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 4) == 0
    assert rn.lib.rn_parallel_workspace_bytes(ctypes.byref(d)) == 0


def test_null_desc_and_pointers():
    P = rn.lib.rn_retention_parallel
    assert P(None, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == rn.RN_ERR_INVALID_ARG
    d, keep = desc()
    assert P(ctypes.byref(d), None, FAKE, FAKE, None, FAKE, None, 0, None) == rn.RN_ERR_INVALID_ARG
    assert P(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None, 0, None) == rn.RN_ERR_INVALID_ARG
    d, keep = desc(flags=rn.RN_EPI_GN | rn.RN_EPI_GATE)
    assert par(d, gate=None) == rn.RN_ERR_INVALID_ARG     # gate flag without a gate tensor


def test_chunkwise_specific_errors():
    d, keep = desc()
    assert chk(d, chunk=0) == rn.RN_ERR_INVALID_ARG
    need = rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 4)
    assert need > 0
    assert chk(d, ws_bytes=need - 1) == rn.RN_ERR_WORKSPACE
    assert chk(d, ws=None) == rn.RN_ERR_WORKSPACE
    d, keep = desc(flags=rn.RN_NORM_D_ROW)
    assert chk(d) == rn.RN_ERR_INVALID_ARG                 # rescalings: parallel form only
    d, keep = desc(flags=rn.RN_NORM_R_ROW, N=1)
    assert step(d) == rn.RN_ERR_INVALID_ARG


def test_workspace_independent_of_sequence_length():
    sizes = set()
    for N in (64, 8192, 65536):
        d, keep = desc(N=N, d_k=256, d_v=512, theta=np.ones(128), H=16, gamma=np.full(16, 0.9))
        sizes.add(rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 256))
    assert len(sizes) == 1 and sizes.pop() > 0


def test_chunkwise_schedule_flags():
    """The two explicit schedules are exclusive; each has its own workspace size, which does
    not grow with N (windows of 32 chunks carry the state between them)."""
    big = dict(d_k=256, d_v=512, theta=np.ones(128), H=16, gamma=np.full(16, 0.9))
    d, keep = desc(**big, flags=rn.RN_CHUNK_PARALLEL | rn.RN_CHUNK_SEGMENTED)
    assert chk(d) == rn.RN_ERR_INVALID_ARG
    assert b"exclusive" in rn.lib.rn_last_error()
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 256) == 0
    sizes = {}
    for name, flags in (("sequential", 0), ("pair", rn.RN_CHUNK_PARALLEL), ("segmented", rn.RN_CHUNK_SEGMENTED)):
        got = set()
        for N in (64, 8192, 65536):
            d, keep = desc(**dict(big, N=N), flags=flags)
            got.add(rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 256))
        assert len(got) == 1 and min(got) > 0, name
        sizes[name] = got.pop()
    assert len(set(sizes.values())) == 3, sizes


def test_matrix_core_paths_stop_at_32_bit_head_extents():
    """Each matrix-core path reads a head's arrays through buffer resources with 32-bit
    offsets; past 2 GB per head (float32 outputs and dout included) the calls take the
    generic kernels, whose workspace sizes differ."""
    big = dict(d_k=256, d_v=512, theta=np.ones(128), H=1, gamma=[0.9])
    # backward: (N + 64) * 512 * 4 < 2^31 <=> N < 2^20 - 64
    def bw_ws(N, flags=0):
        d, keep = desc(**big, N=N, flags=flags)
        return rn.lib.rn_chunkwise_backward_workspace_bytes(ctypes.byref(d), 256)
    lo, hi = (1 << 20) - 65, (1 << 20) - 64
    assert bw_ws(lo) != bw_ws(lo, rn.RN_FORCE_GENERIC)         # matrix cores below the bound
    assert bw_ws(hi) == bw_ws(hi, rn.RN_FORCE_GENERIC) > 0     # generic kernels from it on
    # forward: the sequential kernel while N * 512 * 4 < 2^31, then another schedule
    lo, keep_lo = desc(**big, N=(1 << 20) - 1)
    hi, keep_hi = desc(**big, N=1 << 20)
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(lo), 256) != \
        rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(hi), 256)
    # parallel: the matrix-core kernel needs its workspace, the generic one none
    lo, keep_lo = desc(**big, N=(1 << 20) - 1)
    hi, keep_hi = desc(**big, N=1 << 20)
    assert rn.lib.rn_parallel_workspace_bytes(ctypes.byref(lo)) > 0
    assert rn.lib.rn_parallel_workspace_bytes(ctypes.byref(hi)) == 0


def test_parallel_workspace():
    big = dict(d_k=256, d_v=512, theta=np.ones(128), H=8, gamma=np.full(8, 0.9), N=2048)
    d, keep = desc(**big)
    need = rn.lib.rn_parallel_workspace_bytes(ctypes.byref(d))
    assert need == 8 * 2048 * (256 + 512) * 2              # k rotated + v transposed, half
    assert par(d, ws_bytes=need - 1) == rn.RN_ERR_WORKSPACE
    assert par(d, ws=None) == rn.RN_ERR_WORKSPACE
    assert par(d, ws=ctypes.c_void_p(0x1010), ws_bytes=need) == rn.RN_ERR_INVALID_ARG   # misaligned
    d, keep = desc(**big, flags=rn.RN_FORCE_GENERIC)
    assert rn.lib.rn_parallel_workspace_bytes(ctypes.byref(d)) == 0


def test_step_specific_errors():
    d, keep = desc(N=2)
    assert step(d) == rn.RN_ERR_INVALID_ARG                # decode takes one token
    d, keep = desc(N=1)
    assert step(d, state=None) == rn.RN_ERR_INVALID_ARG
    assert step(d, state=ctypes.c_void_p(0x1004)) == rn.RN_ERR_INVALID_ARG  # misaligned


def test_groupnorm_errors():
    f = rn.lib.rn_groupnorm_gate
    assert f(0, 1, 1, 8, rn.RN_F32, rn.RN_F32, FAKE, None, None, None, 1e-5, FAKE, None) == rn.RN_ERR_INVALID_ARG
    assert f(1, 1, 1, 600, rn.RN_F32, rn.RN_F32, FAKE, None, None, None, 1e-5, FAKE, None) == rn.RN_ERR_UNSUPPORTED
    assert f(1, 1, 1, 8, 5, rn.RN_F32, FAKE, None, None, None, 1e-5, FAKE, None) == rn.RN_ERR_INVALID_ARG
    assert f(1, 1, 1, 8, rn.RN_F32, rn.RN_F32, None, None, None, None, 1e-5, FAKE, None) == rn.RN_ERR_INVALID_ARG
    assert f(1, 1, 1, 8, rn.RN_F32, rn.RN_F32, FAKE, None, None, None, -1.0, FAKE, None) == rn.RN_ERR_INVALID_ARG
    assert f(1, 1, 1, 8, rn.RN_F32, rn.RN_BF16, FAKE, None, None, None, 1e-5, FAKE, None) == rn.RN_ERR_INVALID_ARG  # in place, dtype change


def test_serving_entry_point_errors():
    """Per-sequence arrays are device pointers: their alignment is checked on the host,
    the decode variant requires its positions, and the common checks still apply."""
    d, keep = desc()
    assert chk_varlen(d, pos=ctypes.c_void_p(0x1004)) == rn.RN_ERR_INVALID_ARG    # int64 misaligned
    assert b"pos" in rn.lib.rn_last_error()
    assert chk_varlen(d, lengths=ctypes.c_void_p(0x1002)) == rn.RN_ERR_INVALID_ARG
    assert b"lengths" in rn.lib.rn_last_error()
    assert chk_varlen(d, chunk=0) == rn.RN_ERR_INVALID_ARG
    need = rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 4)
    assert chk_varlen(d, ws_bytes=need - 1) == rn.RN_ERR_WORKSPACE
    d1, keep1 = desc(N=1)
    assert step_at(d1, pos=None) == rn.RN_ERR_INVALID_ARG
    assert step_at(d1, pos=ctypes.c_void_p(0x1004)) == rn.RN_ERR_INVALID_ARG
    assert step_at(d1, state=None) == rn.RN_ERR_INVALID_ARG
    d2, keep2 = desc(N=2)
    assert step_at(d2) == rn.RN_ERR_INVALID_ARG                          # one token per call


def test_binding_checks_sequence_arrays():
    """The Python layer rejects per-sequence arrays of the wrong dtype or shape before
    any call (CPU tensors never reach the library)."""
    import torch
    q = torch.zeros(2, 1, 4, 16, dtype=torch.bfloat16)
    v = torch.zeros(2, 1, 4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rn._seq_array(torch.zeros(3, dtype=torch.int64), 2, torch.int64, "pos")
    with pytest.raises(ValueError):
        rn._seq_array(torch.zeros(2, dtype=torch.int32), 2, torch.int64, "pos")
    with pytest.raises(ValueError):   # tensors must be on the GPU
        rn._seq_array(torch.zeros(2, dtype=torch.int32), 2, torch.int32, "lengths")
    with pytest.raises(ValueError):
        rn.rn_retention_recurrent_step_at(q[:, :, :1], q[:, :, :1], v[:, :, :1], [0.9], np.ones(8),
                                          torch.zeros(2, 1, 16, 16), None)


def bwd(d, dgate=FAKE, ws=FAKE, ws_bytes=1 << 40, dq=FAKE):
    return rn.lib.rn_retention_chunkwise_backward(
        ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, dq, FAKE, FAKE, dgate,
        None, None, None, ws, ws_bytes, None)


def test_backward_errors():
    d, keep = desc()
    assert bwd(d, dq=None) == rn.RN_ERR_INVALID_ARG
    need = rn.lib.rn_chunkwise_backward_workspace_bytes(ctypes.byref(d), 4)
    assert need > 0
    assert bwd(d, ws_bytes=need - 1) == rn.RN_ERR_WORKSPACE
    assert bwd(d, ws=ctypes.c_void_p(0x1010), ws_bytes=need) == rn.RN_ERR_INVALID_ARG
    d, keep = desc(flags=rn.RN_EPI_GN | rn.RN_EPI_GATE)
    assert bwd(d, dgate=None) == rn.RN_ERR_INVALID_ARG       # gate flag needs dgate
    d, keep = desc(B=600, H=128, gamma=np.full(128, 0.9))
    assert bwd(d) == rn.RN_ERR_UNSUPPORTED                   # B*H above one grid dimension
    d, keep = desc(flags=rn.RN_NORM_D_ROW)
    assert bwd(d) == rn.RN_ERR_INVALID_ARG                   # rescalings: parallel form only


def test_pair_decay_descriptor():
    """One decay per (head, coordinate pair) travels as a device array (gamma_pair); the
    host checks its alignment and the combinations the forms accept, never its values.
    Here the array is a host copy, which only calls that fail or size a workspace see."""
    big = dict(d_k=256, d_v=512, theta=np.ones(128), H=4, N=1000)
    gp = np.full((4, 128), 0.9, dtype=np.float32)
    d, keep = desc(**big, gamma=gp)
    assert not d.gamma and d.gamma_pair
    # chunkwise runs the chunk-parallel pair at this shape: its workspace, not the
    # sequential kernel's
    dcp, keep_cp = desc(**big, gamma=np.full(4, 0.9), flags=rn.RN_CHUNK_PARALLEL)
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 256) == \
        rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(dcp), 256) > 0
    assert rn.lib.rn_parallel_workspace_bytes(ctypes.byref(d)) == 0       # generic parallel
    assert chk(d, ws_bytes=1000) == rn.RN_ERR_WORKSPACE
    dn, keep_n = desc(**big, gamma=gp, flags=rn.RN_NORM_D_ROW)
    assert par(dn) == rn.RN_ERR_INVALID_ARG                               # scalar-decay rescaling
    assert b"RN_NORM_D_ROW" in rn.lib.rn_last_error()
    assert bwd(d) == rn.RN_ERR_UNSUPPORTED                                # backward: per-head decay
    assert rn.lib.rn_chunkwise_backward_workspace_bytes(ctypes.byref(d), 256) == 0
    d.gamma_pair = 0x1002
    assert chk(d) == rn.RN_ERR_INVALID_ARG                                # misaligned
    d.gamma_pair = None
    assert chk(d) == rn.RN_ERR_INVALID_ARG                                # no decay at all
    with pytest.raises(ValueError):
        desc(**big, gamma=np.full((4, 127), 0.9, dtype=np.float32))


def layer(d, d_model=64, chunk=16, ws=FAKE, ws_bytes=1 << 40, w_g=FAKE, x=FAKE):
    return rn.lib.rn_msr_layer_forward(ctypes.byref(d), d_model, chunk, x, FAKE, FAKE, FAKE, w_g,
                                       FAKE, None, None, FAKE, ws, ws_bytes, None)


def test_layer_errors_and_workspace():
    d, keep = desc(flags=rn.RN_EPI_GN | rn.RN_EPI_GATE)
    need = rn.lib.rn_msr_layer_workspace_bytes(ctypes.byref(d), 64, 16)
    # q, k (d_k) + v, g, head outputs (d_v), each 256-aligned, + the retention workspace
    tok = 1 * 2 * 8
    a = lambda n: (n + 255) // 256 * 256
    d_ret, keep_ret = desc(flags=rn.RN_EPI_GN | rn.RN_EPI_GATE, out_dtype=rn.RN_BF16)
    ret = rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d_ret), 16)
    assert need == 2 * a(tok * 16 * 2) + 3 * a(tok * 16 * 2) + a(ret)
    assert layer(d, ws_bytes=need - 1) == rn.RN_ERR_WORKSPACE
    assert layer(d, ws=ctypes.c_void_p(0x1010), ws_bytes=need) == rn.RN_ERR_INVALID_ARG
    assert layer(d, w_g=None) == rn.RN_ERR_INVALID_ARG          # gate flag needs w_g
    assert layer(d, x=None) == rn.RN_ERR_INVALID_ARG
    assert layer(d, d_model=0) == rn.RN_ERR_INVALID_ARG
    assert layer(d, chunk=0) == rn.RN_ERR_INVALID_ARG
    d32, keep32 = desc(in_dtype=rn.RN_F32)
    assert layer(d32) == rn.RN_ERR_UNSUPPORTED                  # bf16 GEMM operands only
    dodd, keep_odd = desc(d_v=12)
    assert layer(dodd) == rn.RN_ERR_UNSUPPORTED                 # d_v % 8
    dbad, keep_bad = desc(B=0)
    assert layer(dbad) == rn.RN_ERR_INVALID_ARG
    assert rn.lib.rn_msr_layer_workspace_bytes(ctypes.byref(dbad), 64, 16) == 0


SEQ = dict(d_k=256, d_v=512, theta=np.ones(128), H=2, gamma=np.full(2, 0.99), N=300)


def status_image(word, nbytes):
    """A host copy of a sequential-kernel workspace whose status word is ``word``."""
    img = np.zeros(nbytes // 4, dtype=np.uint32)
    img[0] = word
    return img


def chk_status(d, img, chunk=64, nbytes=None):
    nb = img.nbytes if nbytes is None else nbytes
    return rn.lib.rn_chunkwise_check(ctypes.byref(d), chunk, img.ctypes.data_as(ctypes.c_void_p),
                                     nb, None)


def test_chunkwise_check_reads_the_status_word():
    """The status word leads the sequential kernel's workspace: bit 0 is an exchange wait
    that hit its time limit, bit 1 a non-finite output or state. A host copy of the
    workspace is read directly, so every code is reachable without a GPU."""
    d, keep = desc(**SEQ)
    n = rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 64)
    assert n >= 256
    assert chk_status(d, status_image(0, n)) == rn.RN_OK
    assert chk_status(d, status_image(1, n)) == rn.RN_ERR_EXCHANGE
    assert b"time limit" in rn.lib.rn_last_error()
    assert chk_status(d, status_image(2, n)) == rn.RN_ERR_NONFINITE
    assert chk_status(d, status_image(3, n)) == rn.RN_ERR_EXCHANGE     # the time-out wins
    assert rn.lib.rn_status_str(rn.RN_ERR_EXCHANGE) == b"RN_ERR_EXCHANGE"
    assert rn.lib.rn_status_str(rn.RN_ERR_NONFINITE) == b"RN_ERR_NONFINITE"
    # argument errors
    assert rn.lib.rn_chunkwise_check(ctypes.byref(d), 64, None, n, None) == rn.RN_ERR_INVALID_ARG
    assert chk_status(d, status_image(0, n), nbytes=2) == rn.RN_ERR_WORKSPACE
    assert chk_status(d, status_image(0, n), chunk=0) == rn.RN_ERR_INVALID_ARG
    assert rn.lib.rn_chunkwise_check(None, 64, FAKE, n, None) == rn.RN_ERR_INVALID_ARG


def test_chunkwise_check_other_schedules():
    """The segmented and chunk-parallel schedules keep the status word too (their waits are
    kernel boundaries, so only the non-finite bit is ever set); the float32 kernels keep
    none, and the check is RN_OK whatever the workspace holds."""
    for flags in (rn.RN_CHUNK_PARALLEL, rn.RN_CHUNK_SEGMENTED):
        d, keep = desc(**SEQ, flags=flags)
        assert chk_status(d, status_image(0, 1024)) == rn.RN_OK, flags
        assert chk_status(d, status_image(2, 1024)) == rn.RN_ERR_NONFINITE, flags
        assert b"segmented" in rn.lib.rn_last_error() or b"chunk-parallel" in rn.lib.rn_last_error()
    d, keep = desc(**dict(SEQ, gamma=np.full(2, 0.8)))       # gamma^32 < 2^-6: segmented
    assert chk_status(d, status_image(2, 1024)) == rn.RN_ERR_NONFINITE
    d, keep = desc(**SEQ, flags=rn.RN_FORCE_GENERIC)
    assert chk_status(d, status_image(3, 1024)) == rn.RN_OK
    d, keep = desc(**dict(SEQ, in_dtype=rn.RN_F32))             # float32 inputs: generic
    assert chk_status(d, status_image(3, 1024)) == rn.RN_OK


def test_chunkwise_check_binding_with_a_host_copy():
    import torch
    q = torch.zeros(1, 2, 300, 256, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 300, 512, dtype=torch.bfloat16)
    g, th = [0.99, 0.99], np.ones(128)
    n = rn.rn_chunkwise_workspace_bytes(q, v, g, th, 64)
    for word, code in ((0, rn.RN_OK), (1, rn.RN_ERR_EXCHANGE), (2, rn.RN_ERR_NONFINITE)):
        img = torch.from_numpy(status_image(word, n).view(np.uint8))
        assert rn.rn_chunkwise_check(q, v, g, th, 64, img) == code
    with pytest.raises(RuntimeError):
        rn.rn_chunkwise_check(q, v, g, th, 0, img)


def test_test_force_timeout_flag_is_known():
    d, keep = desc(flags=rn.RN_TEST_FORCE_TIMEOUT)
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 4) > 0
    d, keep = desc(flags=1 << 30)
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 4) == 0


def test_sequence_length_limit():
    d, keep = desc(N=(1 << 30) + 1)
    assert chk(d) == rn.RN_ERR_UNSUPPORTED
    assert b"2^30" in rn.lib.rn_last_error()


def test_binding_checks_gate_and_affine():
    """The gate must match v (shape, dtype, device) and the GroupNorm weight and bias
    must be float32 with H*d_v elements on the call's device; all rejected before any call."""
    import torch
    q = torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16)
    g, th = [0.9, 0.8], np.ones(8)
    base = (q, q, v, g, th, None, 0, 0, 1.0, 1e-5)
    for gate in (torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16),          # shape
                 torch.zeros(1, 2, 8, 32, dtype=torch.float32),           # dtype
                 torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16, device="meta")):   # device
        with pytest.raises(ValueError, match="gate"):
            rn._qkv_desc(*base, None, None, gate)
    for w in (torch.ones(64, dtype=torch.bfloat16), torch.ones(63), torch.ones(64, device="meta")):
        with pytest.raises(ValueError, match="gn_weight"):
            rn._qkv_desc(*base, w, None)
        with pytest.raises(ValueError, match="gn_weight"):
            rn._qkv_desc(*base, None, w)
    with pytest.raises(ValueError, match="gate"):
        rn.rn_groupnorm_gate(v, gate=torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16, device="meta"))
    with pytest.raises(ValueError, match="gn_weight"):
        rn.rn_groupnorm_gate(v, weight=torch.ones(63))


def test_noalloc_entry_point_validates_first():
    """The call without allocation validates like rn_retention_chunkwise and rejects a
    workspace beyond its 32 MiB buffer before any HIP call."""
    f = rn.lib.rn_retention_chunkwise_noalloc
    d, keep = desc(N=0)
    assert f(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == rn.RN_ERR_INVALID_ARG
    d, keep = desc()
    assert f(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == rn.RN_ERR_INVALID_ARG
    big = dict(d_k=256, d_v=256, theta=np.ones(128), H=16, gamma=np.full(16, 0.99), B=4, N=64)
    d, keep = desc(**big)
    assert rn.lib.rn_chunkwise_workspace_bytes(ctypes.byref(d), 64) > 32 << 20
    assert f(ctypes.byref(d), 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == rn.RN_ERR_UNSUPPORTED
    assert b"workspace" in rn.lib.rn_last_error()
