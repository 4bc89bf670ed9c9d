"""Host-side checks of the C ABI: no GPU needed, no device work queued.

The library must load, export every entry point include/nbw.h declares, and
reject bad arguments with the documented status codes before any HIP call.
"""
import ctypes
import os
import re

import pytest

import nested_bit_weight_amd as nbw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nbw.h")

OK, EINVAL, EALIGN, ERANGE, EUNSUPPORTED = 0, 1, 2, 3, 4
FAKE = 0x7F0000001000  # a 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    return nbw.library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^(\n]*?\b(nbw_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in nbw.h but not exported"
    assert set(names) == set(nbw.EXPORTS)


def test_plane_bytes(lib):
    assert lib.nbw_plane_bytes(1, 128) == 16 * 16
    assert lib.nbw_plane_bytes(16, 4096) == 16 * 512
    assert lib.nbw_plane_bytes(17, 4096) == 32 * 512
    assert lib.nbw_plane_bytes(0, 128) == -1
    assert lib.nbw_plane_bytes(16, 100) == -1
    assert lib.nbw_packed_bytes(6144, 4096, 3) == 3 * 6144 * 512
    assert lib.nbw_packed_bytes(16, 128, 9) == -1


def _view(lib, n=64, k=256, nplanes=8, ptr=FAKE):
    v = nbw.WView()
    st = lib.nbw_make_view(ctypes.c_void_p(ptr), n, k, nplanes, ctypes.byref(v))
    return st, v


def test_make_and_slice_view(lib):
    st, v = _view(lib)
    assert st == OK and v.nplanes == 8 and v.layout == 1 and v.plane_bytes == 64 * 32
    c = nbw.WView()
    assert lib.nbw_slice_view(ctypes.byref(v), 3, ctypes.byref(c)) == OK
    assert c.planes == v.planes and c.nplanes == 3 and c.plane_bytes == v.plane_bytes
    c2 = nbw.WView()
    assert lib.nbw_slice_view(ctypes.byref(c), 4, ctypes.byref(c2)) == ERANGE
    assert lib.nbw_slice_view(ctypes.byref(v), 0, ctypes.byref(c2)) == ERANGE
    assert lib.nbw_slice_view(ctypes.byref(v), 9, ctypes.byref(c2)) == ERANGE
    assert lib.nbw_slice_view(None, 2, ctypes.byref(c2)) == EINVAL
    assert _view(lib, ptr=FAKE + 8)[0] == EALIGN
    assert _view(lib, k=200)[0] == EINVAL
    assert _view(lib, n=0)[0] == EINVAL
    assert _view(lib, nplanes=0)[0] == ERANGE
    assert _view(lib, ptr=0)[0] == EINVAL


def test_qgemm_validation_before_any_hip_call(lib):
    _, v = _view(lib)
    p = ctypes.c_void_p
    q = lib.nbw_qgemm_kernel
    args = dict(x=p(FAKE), b=4, s=p(FAKE), r=4, y=p(FAKE), kern=0)

    def call(**kw):
        a = dict(args, **kw)
        return q(a["x"], a["b"], ctypes.byref(kw.get("view", v)), a["s"], a["r"], a["y"], a["kern"],
                 None)

    assert call(x=p(0)) == EINVAL
    assert call(y=p(0)) == EINVAL
    assert call(s=p(0)) == EINVAL
    assert call(b=-1) == EINVAL
    assert call(r=0) == ERANGE
    assert call(r=9) == ERANGE
    assert call(kern=7) == EUNSUPPORTED
    assert call(x=p(FAKE + 2)) == EALIGN
    assert call(y=p(FAKE + 4)) == EALIGN
    assert call(s=p(FAKE + 1)) == EALIGN
    assert call(s=p(FAKE + 2)) == EALIGN
    child = nbw.WView()
    lib.nbw_slice_view(ctypes.byref(v), 2, ctypes.byref(child))
    assert call(view=child, r=3) == ERANGE
    bad = nbw.WView.from_buffer_copy(v)
    bad.layout = 9
    assert call(view=bad) == EUNSUPPORTED
    bad = nbw.WView.from_buffer_copy(v)
    bad.plane_bytes += 16
    assert call(view=bad) == EINVAL
    # the empty product is valid and touches nothing
    assert call(b=0, x=p(0), y=p(0), s=p(0)) == OK


def test_pack_and_unpack_validation(lib):
    p = ctypes.c_void_p
    pb = lib.nbw_plane_bytes(64, 256)
    assert lib.nbw_pack_bitplanes(p(0), 64, 256, p(FAKE), 8 * pb, None) == EINVAL
    assert lib.nbw_pack_bitplanes(p(FAKE), 64, 256, p(FAKE), 8 * pb - 1, None) == EINVAL
    assert lib.nbw_pack_bitplanes(p(FAKE), 64, 250, p(FAKE), 8 * pb, None) == EINVAL
    assert lib.nbw_pack_bitplanes(p(FAKE + 4), 64, 256, p(FAKE), 8 * pb, None) == EALIGN
    _, v = _view(lib)
    assert lib.nbw_unpack_codes(ctypes.byref(v), 9, p(FAKE), None) == ERANGE
    assert lib.nbw_unpack_codes(ctypes.byref(v), 3, p(0), None) == EINVAL
    assert lib.nbw_unpack_codes(ctypes.byref(v), 3, p(FAKE + 1), None) == EALIGN


def test_status_strings(lib):
    for s in range(7):
        assert lib.nbw_status_str(s)
    assert b"gfx950" in lib.nbw_version()
    assert lib.nbw_last_hip_error() == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nbw.pack_bitplanes(torch.zeros((16, 128), dtype=torch.uint8))


def test_qgemm_ex_validation(lib):
    _, v = _view(lib, n=64, k=256)
    p = ctypes.c_void_p

    def call(opts=None, b=4, y=FAKE, x=FAKE):
        o = None if opts is None else ctypes.byref(opts)
        return lib.nbw_qgemm_ex(p(x), b, ctypes.byref(v), p(FAKE), 4, p(y), o, None)

    def opts(**kw):
        o = nbw.QgemmOpts()
        for key, val in kw.items():
            setattr(o, key, val)
        return o

    assert call(opts(ldx=255)) == EINVAL            # below k
    assert call(opts(ldy=63)) == EINVAL             # below n
    assert call(opts(ldx=260)) == EALIGN            # rows would lose 16-byte alignment
    assert call(opts(y_dtype=2)) == EUNSUPPORTED
    assert call(opts(kernel=9)) == EUNSUPPORTED
    assert call(opts(zeros_bf16=FAKE + 2)) == EALIGN
    assert call(opts(workspace=FAKE, workspace_bytes=-1)) == EINVAL
    assert call(opts(workspace=FAKE + 16, workspace_bytes=4096)) == EALIGN   # not 256-aligned
    assert call(opts(), b=0, x=0, y=0) == OK        # empty product


def test_workspace_bytes_without_device_work(lib):
    # Bad arguments and the kernels that never split answer without a device query.
    assert lib.nbw_qgemm_workspace_bytes(-1, 4096, 4096, 4, 0) == -1
    assert lib.nbw_qgemm_workspace_bytes(0, 4096, 4096, 4, 0) == 0     # empty batch: no launch
    assert lib.nbw_qgemm_workspace_bytes(256, 4096, 100, 4, 0) == -1
    assert lib.nbw_qgemm_workspace_bytes(256, 4096, 4096, 9, 0) == -1
    assert lib.nbw_qgemm_workspace_bytes(256, 4096, 4096, 4, 7) == -1
    assert lib.nbw_qgemm_workspace_bytes(1, 4096, 4096, 4, 0) == 0     # GEMV
    assert lib.nbw_qgemm_workspace_bytes(16, 4096, 4096, 4, 0) == 0    # small-batch kernel
    assert lib.nbw_qgemm_workspace_bytes(256, 4096, 4096, 4, 2) == 0   # forced small-batch kernel


def test_choose_codes_validation(lib):
    p = ctypes.c_void_p
    i32 = ctypes.c_int32
    dbl = ctypes.c_double

    def call(widths, lambdas, n=16, k=128, w=FAKE):
        wa = (i32 * max(1, len(widths)))(*widths)
        la = (dbl * max(1, len(lambdas)))(*lambdas)
        return lib.nbw_choose_codes(p(w), n, k, p(FAKE), wa, la, len(widths), p(FAKE), None)

    assert call([], []) == EINVAL
    assert call([3, 4, 8, 1, 2, 5, 6, 7, 8], [1.0] * 9) == EINVAL
    assert call([9], [1.0]) == ERANGE
    assert call([0], [1.0]) == ERANGE
    assert call([8], [-1.0]) == EINVAL
    assert call([8], [float("nan")]) == EINVAL
    assert call([8], [float("inf")]) == EINVAL
    assert call([8], [1.0], k=100) == EINVAL
    assert call([8], [1.0], w=0) == EINVAL
    assert call([8], [1.0], w=FAKE + 2) == EALIGN


def test_stream_read_validation(lib):
    vp = ctypes.c_void_p
    assert lib.nbw_stream_sink_words() >= 1024
    assert lib.nbw_stream_read(None, 1024, vp(FAKE), None) == EINVAL
    assert lib.nbw_stream_read(vp(FAKE), 1024, None, None) == EINVAL
    assert lib.nbw_stream_read(vp(FAKE), -16, vp(FAKE), None) == EINVAL
    assert lib.nbw_stream_read(vp(FAKE), 1000, vp(FAKE), None) == EINVAL   # not a multiple of 16
    assert lib.nbw_stream_read(vp(FAKE + 8), 1024, vp(FAKE), None) == EALIGN
    assert lib.nbw_stream_read(vp(FAKE), 1024, vp(FAKE + 2), None) == EALIGN


def test_mfma_rate_validation(lib):
    # argument checks come before the device is queried (no GPU here)
    vp = ctypes.c_void_p
    assert lib.nbw_mfma_rate(None, 1, vp(FAKE), None) == EINVAL
    assert lib.nbw_mfma_rate(vp(FAKE), 1, None, None) == EINVAL
    assert lib.nbw_mfma_rate(vp(FAKE), 0, vp(FAKE), None) == EINVAL
    assert lib.nbw_mfma_rate(vp(FAKE + 8), 1, vp(FAKE), None) == EALIGN
    assert lib.nbw_mfma_rate(vp(FAKE), 1, vp(FAKE + 2), None) == EALIGN


def test_noalloc_rejects_before_any_device_work(lib):
    p = ctypes.c_void_p
    _, v = _view(lib)
    o = nbw.QgemmOpts(0, 0, 0, 0, None, FAKE, 4096)   # a caller workspace is refused
    assert lib.nbw_qgemm_noalloc(p(FAKE), 4, ctypes.byref(v), p(FAKE), 4, p(FAKE), ctypes.byref(o),
                                 None) == EINVAL
    o = nbw.QgemmOpts()
    assert lib.nbw_qgemm_noalloc(p(FAKE), 4, ctypes.byref(v), p(FAKE), 9, p(FAKE), ctypes.byref(o),
                                 None) == ERANGE
    o.kernel = 7
    assert lib.nbw_qgemm_noalloc(p(FAKE), 4, ctypes.byref(v), p(FAKE), 4, p(FAKE), ctypes.byref(o),
                                 None) == EUNSUPPORTED
    assert b"scratch" in lib.nbw_status_str(6)
