"""The C-ABI boundary without a GPU: the library loads, exports every symbol
include/ssd.h declares, sizes its workspace, and rejects every invalid call on
the host (status code + detail) before any HIP call is made."""

import ctypes
import os
import subprocess

import pytest

from selective_state_space_amd import ssd

pytestmark = pytest.mark.skipif(not os.path.exists(ssd.LIB_PATH),
                                reason="libssd.so not built (python -m selective_state_space_amd.build)")

# Fake, 16-byte aligned, never dereferenced: every call below fails validation first.
P16 = ctypes.c_void_p(0x1000)
P_MIS = ctypes.c_void_p(0x1004)


def lib():
    return ssd.load_library()


def dims(Bt=2, T=300, H=8, P=64, N=128, G=2, io=ssd.SSD_BF16):
    return ssd.Dims(Bt, T, H, P, N, G, io)


def test_exports_every_declared_symbol():
    names = ssd.header_functions()
    assert {"ssd_chunked_fwd", "ssd_decode_step", "ssd_chunked_fwd_workspace_size"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib(), n)


def test_version_and_status_strings():
    assert lib().ssd_version() >= 100
    for code in ssd.STATUS:
        assert lib().ssd_status_string(code).decode().startswith(ssd.STATUS[code])


def test_workspace_size_and_layout():
    d = dims(8, 4096, 80, 64, 128, 1)
    nc = 16
    units = 8 * 80 * nc
    size = ssd.ssd_chunked_fwd_workspace_size(d, 256)
    off = ssd.ssd_chunked_fwd_workspace_layout(d, 256)
    assert off[0] == 0
    assert off[1] >= units * 256 * 4 and off[1] % 256 == 0
    assert off[2] >= off[1] + units * 256 * 4 and off[2] % 256 == 0
    assert off[3] >= off[2] + units * 64 * 128 * 4 and off[3] % 256 == 0
    assert size >= off[3] + units * 64 * 128 * 2
    # fp32 io keeps h_prev in fp32
    d32 = dims(8, 4096, 80, 64, 128, 1, ssd.SSD_F32)
    assert ssd.ssd_chunked_fwd_workspace_size(d32, 256) >= off[3] + units * 64 * 128 * 4
    # ragged T rounds up to whole chunks
    assert (ssd.ssd_chunked_fwd_workspace_size(dims(1, 257, 4), 256)
            == ssd.ssd_chunked_fwd_workspace_size(dims(1, 512, 4), 256))
    # empty and invalid shapes need none
    assert ssd.ssd_chunked_fwd_workspace_size(dims(Bt=0), 256) == 0
    assert ssd.ssd_chunked_fwd_workspace_size(dims(T=0), 256) == 0
    assert ssd.ssd_chunked_fwd_workspace_size(dims(N=100), 256) == 0
    assert ssd.ssd_chunked_fwd_workspace_size(dims(), 96) == 0


def _fwd(d, L=256, x=P16, dt=P16, A=P16, B=P16, C=P16, D=P16, init=None, y=P16, fin=None,
         ws=P16, wsb=1 << 40):
    return lib().ssd_chunked_fwd(x, dt, A, B, C, D, L, init, y, fin,
                                 None if d is None else ctypes.byref(d), ws, wsb, None)


def _detail():
    return lib().ssd_last_error_detail().decode()


@pytest.mark.parametrize("field", ["x", "dt", "A", "B", "C", "D", "y", "ws"])
def test_null_pointers(field):
    st = _fwd(dims(), **{field: None})
    assert st == -1
    assert (field if field != "ws" else "workspace") in _detail()


def test_null_dims():
    assert _fwd(None) == -1


@pytest.mark.parametrize("kw,code,word", [
    (dict(H=6, G=4), -2, "multiple"),
    (dict(H=0), -2, "nheads"),
    (dict(G=0), -2, "ngroups"),
    (dict(Bt=-1), -2, "batch"),
    (dict(T=-5), -2, "seqlen"),
    (dict(P=32), -3, "headdim"),
    (dict(N=256), -3, "dstate"),
    (dict(io=7), -3, "io_dtype"),
])
def test_bad_shapes(kw, code, word):
    assert _fwd(dims(**kw)) == code
    assert word in _detail()


@pytest.mark.parametrize("L", [0, 32, 100, 512])
def test_unsupported_chunk_size(L):
    assert _fwd(dims(), L=L) == -3
    assert "chunk_size" in _detail()


@pytest.mark.parametrize("field", ["x", "dt", "A", "B", "C", "D", "y", "init", "fin", "ws"])
def test_misaligned(field):
    assert _fwd(dims(), **{field: P_MIS}) == -4
    assert "aligned" in _detail()


def test_short_workspace():
    d = dims()
    need = ssd.ssd_chunked_fwd_workspace_size(d, 256)
    assert _fwd(d, wsb=need - 1) == -5
    assert str(need) in _detail()


def test_too_large_for_one_launch():
    assert _fwd(dims(Bt=1 << 20, T=1 << 20, H=1 << 10, G=1)) == -2


def test_stage_calls_validate_too():
    d = dims()
    L = lib()
    assert L.ssd_chunk_cumsum(None, P16, 256, ctypes.byref(d), P16, 1 << 40, None) == -1
    assert L.ssd_chunk_state(P16, P_MIS, 256, ctypes.byref(d), P16, 1 << 40, None) == -4
    assert L.ssd_state_passing(None, None, 256, ctypes.byref(d), P16, 10, None) == -5
    assert L.ssd_chunk_scan(P16, P16, P16, None, P16, 256, ctypes.byref(d), P16, 1 << 40,
                            None) == -1
    assert L.ssd_state_fwd(None, P16, None, P16, 256, ctypes.byref(d), P16, 1 << 40, None) == -1
    assert L.ssd_state_fwd(P16, P16, P_MIS, P16, 256, ctypes.byref(d), P16, 1 << 40, None) == -4
    assert L.ssd_state_fwd(P16, P16, None, None, 256, ctypes.byref(d), P16, 10, None) == -5


def test_path_query_and_override():
    out = ctypes.c_int(-1)
    q = lambda d: lib().ssd_chunked_fwd_path(ctypes.byref(d), 256, ctypes.byref(out))
    default = ssd.PATH_STATE_FWD
    try:
        assert lib().ssd_set_path_override(-1, 0, 0) == 0
        assert q(dims(Bt=8, T=4096, H=80, G=1)) == 0 and out.value == default
        assert q(dims(Bt=4, T=2048, H=32, G=1)) == 0 and out.value == default
        assert q(dims(Bt=8, T=4096, H=80, G=1, io=ssd.SSD_F32)) == 0 and out.value == 0
        ssd.set_path_override(ssd.PATH_FOUR_STAGE)
        assert q(dims(Bt=8, T=4096, H=80, G=1)) == 0 and out.value == 0
        ssd.set_path_override(ssd.PATH_FUSED)
        assert q(dims(Bt=8, T=4096, H=80, G=1)) == 0 and out.value == ssd.PATH_FUSED
        ssd.set_path_override(ssd.PATH_STATE_FWD, 2)
        assert q(dims(Bt=1, T=4096, H=8, G=1)) == 0 and out.value == ssd.PATH_STATE_FWD
        # an override the shape does not support is ignored (fp32 io: four stages only)
        assert q(dims(io=ssd.SSD_F32)) == 0 and out.value == 0
        # bad values are rejected and leave the override as it was
        assert lib().ssd_set_path_override(3, 0, 0) == -3
        assert lib().ssd_set_path_override(-1, 3, 0) == -3
        assert lib().ssd_set_path_override(-1, 0, 8) == -3
        assert q(dims(Bt=1, T=4096, H=8, G=1)) == 0 and out.value == ssd.PATH_STATE_FWD
    finally:
        ssd.set_path_override(-1, 0, 0)
    assert lib().ssd_chunked_fwd_path(ctypes.byref(dims()), 256, None) == -1
    assert q(dims(P=32)) == -3


def test_state_fwd_needs_bf16_and_32bit_row_spans():
    L = lib()
    d = dims(io=ssd.SSD_F32)
    assert L.ssd_state_fwd(P16, P16, None, P16, 256, ctypes.byref(d), P16, 1 << 40, None) == -3
    assert "bf16" in L.ssd_last_error_detail().decode()
    # 256 tokens * 65536 heads * 64 * 2 bytes = 2^31: per-chunk x offsets leave 32 bits
    d = dims(Bt=1, T=256, H=1 << 16, G=1)
    assert L.ssd_state_fwd(P16, P16, None, P16, 256, ctypes.byref(d), P16, 1 << 60, None) == -3
    d = dims(Bt=1, T=256, H=(1 << 16) - 8, G=1)
    assert L.ssd_state_fwd(P16, P16, None, P16, 256, ctypes.byref(d), P16, 10, None) == -5


def _dec(d, state=P16, x=P16, dt=P16, B=P16, C=P16, A=P16, D=P16, y=P16):
    return lib().ssd_decode_step(state, x, dt, B, C, A, D, y,
                                 None if d is None else ctypes.byref(d), None)


@pytest.mark.parametrize("field", ["state", "x", "dt", "B", "C", "A", "D", "y"])
def test_decode_null_and_misaligned(field):
    assert _dec(dims(), **{field: None}) == -1
    assert _dec(dims(), **{field: P_MIS}) == -4


def test_decode_shapes():
    assert _dec(dims(H=8, G=3)) == -2
    assert _dec(dims(N=32)) == -3
    assert _dec(None) == -1


def test_empty_batch_is_a_no_op():
    # batch 0: valid, nothing to launch, no workspace needed
    assert _fwd(dims(Bt=0), ws=None, wsb=0) == 0
    assert _dec(dims(Bt=0)) == 0


def test_detail_cleared_on_success():
    _fwd(dims(), x=None)
    assert _detail()
    assert _fwd(dims(Bt=0), ws=None, wsb=0) == 0
    assert _detail() == ""


def test_empty_sequence_allows_null_token_tensors():
    # seqlen 0: nothing to read but the state; validation passes up to the
    # state pointers (a misaligned final_state is still caught)
    d = dims(T=0)
    assert _fwd(d, x=None, dt=None, A=None, B=None, C=None, D=None, y=None, ws=None, wsb=0,
                fin=P_MIS) == -4
    # with tokens present the same NULLs are errors
    assert _fwd(dims(), x=None) == -1


def test_layer_opts_are_validated():
    L = lib()
    d = dims()
    bad = ssd.LayerOpts(None, 1, 7, None)          # y_io_dtype is 0 or 1
    assert L.ssd_chunked_fwd_opts(P16, P16, P16, P16, P16, P16, 256, None, P16, None,
                                  ctypes.byref(bad), ctypes.byref(d), P16, 1 << 40, None) == -3
    assert "y_io_dtype" in L.ssd_last_error_detail().decode()
    assert L.ssd_decode_step_opts(P16, P16, P16, P16, P16, P16, P16, P16, ctypes.byref(bad),
                                  ctypes.byref(d), None) == -3
    # y in the io dtype passes validation (short workspace is the error here)
    yio = ssd.LayerOpts(None, 0, 1, None)
    assert L.ssd_chunked_fwd_opts(P16, P16, P16, P16, P16, P16, 256, None, P16, None,
                                  ctypes.byref(yio), ctypes.byref(d), P16, 10, None) == -5
    mis = ssd.LayerOpts(None, 0, 0, P_MIS)
    assert L.ssd_chunked_fwd_opts(P16, P16, P16, P16, P16, P16, 256, None, P16, None,
                                  ctypes.byref(mis), ctypes.byref(d), P16, 1 << 40, None) == -4
    misb = ssd.LayerOpts(P_MIS, 0, 0, None)
    assert L.ssd_decode_step_opts(P16, P16, P16, P16, P16, P16, P16, P16, ctypes.byref(misb),
                                  ctypes.byref(d), None) == -4
    # NULL options fall through to the usual validation (short workspace)
    assert L.ssd_chunked_fwd_opts(P16, P16, P16, P16, P16, P16, 256, None, P16, None, None,
                                  ctypes.byref(d), P16, 10, None) == -5


def multi(d, snaps=P16, parent=None, flags=0, opts=None, y=P16, state=P16):
    return lib().ssd_decode_multi(state, P16, P16, P16, P16, P16, P16, y, snaps, parent, flags,
                                  opts, ctypes.byref(d), None)


def test_decode_multi_is_validated():
    L = lib()
    d = dims(T=4)
    assert multi(d, flags=2) == -3
    assert "flags" in L.ssd_last_error_detail().decode()
    assert multi(d, snaps=None, parent=P16) == -1
    assert "parent" in L.ssd_last_error_detail().decode()
    assert multi(d, snaps=P_MIS) == -4
    assert multi(d, parent=P_MIS) == -4
    assert multi(d, y=None) == -1
    assert multi(d, state=P_MIS) == -4
    assert multi(dims(T=-1)) == -2
    assert multi(dims(T=(1 << 16) + 1)) == -2
    assert multi(dims(Bt=1 << 30, T=1 << 16, H=1 << 10, G=1)) == -2
    assert multi(dims(N=96, T=4)) == -3
    bad = ssd.LayerOpts(None, 0, 2, None)        # y_io_dtype is 0 or 1
    assert multi(d, opts=ctypes.byref(bad)) == -3
    # nothing to do: no HIP call is made, so these succeed without a GPU
    assert multi(dims(T=0)) == 0
    assert multi(dims(Bt=0, T=4)) == 0
    assert multi(dims(T=0), snaps=None, flags=1) == 0
    assert lib().ssd_decode_multi(P16, None, None, None, None, None, None, None, None, None, 0,
                                  None, ctypes.byref(dims(T=0)), None) == 0
    assert lib().ssd_decode_multi(None, None, None, None, None, None, None, None, None, None, 0,
                                  None, ctypes.byref(dims(T=0)), None) == -1   # state


def lp(fmt, d=None, state=P16, y=P16):
    d = d or dims(T=1)
    f = None if fmt is None else ctypes.byref(fmt)
    return lib().ssd_decode_step_lp(state, f, P16, P16, P16, P16, P16, P16, y, None,
                                    ctypes.byref(d), None)


def test_decode_step_lp_is_validated():
    L = lib()
    SF = ssd.StateFormat
    assert lp(None) == -1
    assert lp(SF(7, 0, 0, None)) == -3
    assert lp(SF(2, 10, 0, None)) == -3                     # stochastic bf16
    assert lp(SF(1, 11, 0, None)) == -3                     # 0..10 rounds
    assert lp(SF(1, -1, 0, None)) == -3
    assert lp(SF(3, 0, 0, None)) == -1                      # int16 without scales
    assert "scale" in L.ssd_last_error_detail().decode()
    assert lp(SF(1, 0, 0, 0x1000)) == -3                    # scales on an fp16 state
    assert lp(SF(3, 0, 0, 0x1004)) == -4
    assert lp(SF(3, 0, 0, 0x1000), state=P_MIS) == -4
    assert lp(SF(1, 1, 5, None), y=None) == -1
    assert lp(SF(1, 1, 5, None), d=dims(N=96)) == -3
    assert lp(SF(0, 0, 0, None), state=None) == -1          # fp32: the plain step's checks
    assert lp(SF(3, 0, 0, 0x1000), d=dims(Bt=0)) == 0       # empty batch: no HIP call


def test_chunked_bwd_workspace_and_validation():
    L = lib()
    d = dims(8, 4096, 80, 64, 128, 1)
    fwd = ssd.ssd_chunked_fwd_workspace_size(d, 256)
    bwd = ssd.ssd_chunked_bwd_workspace_size(d, 256)
    nc, bh = 16, 8 * 80
    assert bwd >= fwd + bh * 64 * 128 * 4 + 8 * nc * 256 * 256 * 4 + 3 * bh * nc * 256 * 4
    assert bwd % 256 == 0
    assert ssd.ssd_chunked_bwd_workspace_size(dims(N=96), 256) == 0
    args = [P16] * 6 + [256] + [None, P16, None] + [P16] * 6 + [None]
    call = lambda a, dd=dims(), ws=P16, wsb=1 << 40: L.ssd_chunked_bwd(
        *a, ctypes.byref(dd), ws, wsb, None)
    bad = list(args); bad[8] = None                      # dy
    assert call(bad) == -1
    bad = list(args); bad[12] = None                     # dA
    assert call(bad) == -1
    bad = list(args); bad[16] = P_MIS                    # dinit
    assert call(bad) == -4
    assert call(args, wsb=10) == -5
    assert call(args, ws=None) == -1
    assert call(args, dd=dims(N=96)) == -3
    assert L.ssd_chunked_bwd(*args[:6], 100, *args[7:], ctypes.byref(dims()), P16, 1 << 40,
                             None) == -3
    # empty batch: no HIP call is made
    assert call(args, dd=dims(Bt=0)) == 0


def test_noalloc_refuses_large_shapes_before_any_hip_call():
    # host arithmetic only: runs without a GPU
    L = lib()
    d = dims(Bt=8, T=4096, H=80, G=1)   # the 2.7B layer: about 0.5 GB of workspace
    st = L.ssd_chunked_fwd_noalloc(P16, P16, P16, P16, P16, P16, 256, None, P16, None, None,
                                   ctypes.byref(d), None)
    assert st == -5
    assert "scratch" in L.ssd_last_error_detail().decode()
    assert L.ssd_chunked_fwd_noalloc(P16, P16, P16, P16, P16, P16, 100, None, P16, None, None,
                                     ctypes.byref(d), None) == -3
    assert L.ssd_chunked_fwd_noalloc(P16, P16, P16, P16, P16, P16, 256, None, P16, None, None,
                                     None, None) == -1
    # nothing to compute: no HIP call either
    assert L.ssd_chunked_fwd_noalloc(None, None, None, None, None, None, 256, None, None, None,
                                     None, ctypes.byref(dims(Bt=0)), None) == 0
