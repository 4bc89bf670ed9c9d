"""nested_bit_weight_amd -- sliced r-bit qgemm over nested bit-plane weights, MI355X.

A thin ctypes binding over ``libnbw.so`` (C ABI in ``include/nbw.h``).  It only
marshals arguments: PyTorch provides device memory and the current stream; every
step of the computation runs in the library's HIP kernels.  If the library is not
built, every call raises -- there is no fallback path.

    planes = pack_bitplanes(codes)            # uint8 [n][k] on the GPU -> PackedWeight
    child = slice_view(planes, r)             # the r-bit child: same storage, r planes
    y = qgemm(x, child, scales, r)            # x bf16 [B][k], scales bf16 [n][k/128] -> fp32 [B][n]

(MatGPTQ: Efficient and Accurate Inference over Nested Quantized Models, Abstract:
one sliceable parent; an r-bit model reads exactly r bits; kernels for batch sizes
beyond one.)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnbw.so")

NBW_LAYOUT_T16 = 1
KERNELS = {"auto": 0, "gemv": 1, "smallb": 2, "gemm": 3}
_STATUS = {0: "NBW_OK", 1: "NBW_EINVAL", 2: "NBW_EALIGN", 3: "NBW_ERANGE",
           4: "NBW_EUNSUPPORTED", 5: "NBW_EHIP", 6: "NBW_ESCRATCH"}


class NBWError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        lib = _lib()
        text = lib.nbw_status_str(status).decode()
        extra = f" (hipError {lib.nbw_last_hip_error()})" if status == 5 else ""
        super().__init__(f"{what}: {_STATUS.get(status, status)} {text}{extra}")


class WView(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("nplanes", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("plane_bytes", ctypes.c_int64)]


class QgemmOpts(ctypes.Structure):
    _fields_ = [("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64), ("y_dtype", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("zeros_bf16", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


Y_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class Problem(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("batch", ctypes.c_int64), ("w", WView),
                ("scales_bf16", ctypes.c_void_p), ("r", ctypes.c_int32), ("y", ctypes.c_void_p)]


class FileInfo(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("nplanes", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("plane_bytes", ctypes.c_int64),
                ("scales_offset", ctypes.c_int64), ("scales_bytes", ctypes.c_int64),
                ("planes_offset", ctypes.c_int64), ("planes_present", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


FILE_HEADER_BYTES = 4096

_LIB = None

EXPORTS = ("nbw_plane_bytes", "nbw_packed_bytes", "nbw_pack_bitplanes", "nbw_make_view",
           "nbw_slice_view", "nbw_qgemm", "nbw_qgemm_kernel", "nbw_qgemm_ex", "nbw_qgemm_noalloc",
           "nbw_qgemm_workspace_bytes", "nbw_qgemm_grouped",
           "nbw_choose_codes", "nbw_unpack_codes", "nbw_stream_sink_words", "nbw_stream_read",
           "nbw_mfma_rate_sink_floats", "nbw_mfma_rate",
           "nbw_file_prefix_bytes", "nbw_file_header", "nbw_file_parse",
           "nbw_kernel_name", "nbw_status_str", "nbw_last_hip_error", "nbw_version")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        pv = ctypes.POINTER(WView)
        lib.nbw_plane_bytes.argtypes = [i64, i64]
        lib.nbw_plane_bytes.restype = i64
        lib.nbw_packed_bytes.argtypes = [i64, i64, i32]
        lib.nbw_packed_bytes.restype = i64
        lib.nbw_pack_bitplanes.argtypes = [vp, i64, i64, vp, i64, vp]
        lib.nbw_pack_bitplanes.restype = ctypes.c_int
        lib.nbw_make_view.argtypes = [vp, i64, i64, i32, pv]
        lib.nbw_make_view.restype = ctypes.c_int
        lib.nbw_slice_view.argtypes = [pv, i32, pv]
        lib.nbw_slice_view.restype = ctypes.c_int
        lib.nbw_qgemm.argtypes = [vp, i64, pv, vp, i32, vp, vp]
        lib.nbw_qgemm.restype = ctypes.c_int
        lib.nbw_qgemm_kernel.argtypes = [vp, i64, pv, vp, i32, vp, ctypes.c_int, vp]
        lib.nbw_qgemm_kernel.restype = ctypes.c_int
        lib.nbw_qgemm_ex.argtypes = [vp, i64, pv, vp, i32, vp, ctypes.POINTER(QgemmOpts), vp]
        lib.nbw_qgemm_ex.restype = ctypes.c_int
        lib.nbw_qgemm_noalloc.argtypes = [vp, i64, pv, vp, i32, vp, ctypes.POINTER(QgemmOpts), vp]
        lib.nbw_qgemm_noalloc.restype = ctypes.c_int
        lib.nbw_choose_codes.argtypes = [vp, i64, i64, vp, ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(ctypes.c_double), i32, vp, vp]
        lib.nbw_choose_codes.restype = ctypes.c_int
        lib.nbw_qgemm_grouped.argtypes = [ctypes.POINTER(Problem), i32, vp]
        lib.nbw_qgemm_grouped.restype = ctypes.c_int
        lib.nbw_unpack_codes.argtypes = [pv, i32, vp, vp]
        lib.nbw_unpack_codes.restype = ctypes.c_int
        lib.nbw_qgemm_workspace_bytes.argtypes = [i64, i64, i64, i32, ctypes.c_int]
        lib.nbw_qgemm_workspace_bytes.restype = i64
        lib.nbw_stream_sink_words.argtypes = []
        lib.nbw_stream_sink_words.restype = i32
        lib.nbw_stream_read.argtypes = [vp, i64, vp, vp]
        lib.nbw_stream_read.restype = ctypes.c_int
        lib.nbw_mfma_rate_sink_floats.argtypes = []
        lib.nbw_mfma_rate_sink_floats.restype = i64
        lib.nbw_mfma_rate.argtypes = [vp, i32, vp, vp]
        lib.nbw_mfma_rate.restype = ctypes.c_int
        lib.nbw_status_str.argtypes = [ctypes.c_int]
        lib.nbw_status_str.restype = ctypes.c_char_p
        lib.nbw_last_hip_error.argtypes = []
        lib.nbw_last_hip_error.restype = i32
        lib.nbw_kernel_name.argtypes = [i64, i64, i64, i32, ctypes.c_int]
        lib.nbw_kernel_name.restype = ctypes.c_char_p
        lib.nbw_version.argtypes = []
        lib.nbw_version.restype = ctypes.c_char_p
        lib.nbw_file_prefix_bytes.argtypes = [i64, i64, i32]
        lib.nbw_file_prefix_bytes.restype = i64
        lib.nbw_file_header.argtypes = [i64, i64, vp]
        lib.nbw_file_header.restype = ctypes.c_int
        lib.nbw_file_parse.argtypes = [vp, i64, ctypes.POINTER(FileInfo)]
        lib.nbw_file_parse.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes handle of libnbw.so (raises if it is not built)."""
    return _lib()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise NBWError(status, what)


def _raw_stream(device_index: int) -> int:
    """Raw handle of the current HIP stream of a device."""
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


def _stream(t: torch.Tensor):
    """The current HIP stream of t's device (the handle only; cheap)."""
    idx = t.device.index if t.device.index is not None else torch.cuda.current_device()
    return ctypes.c_void_p(_raw_stream(idx))


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def plane_bytes(n: int, k: int) -> int:
    v = _lib().nbw_plane_bytes(n, k)
    if v < 0:
        raise ValueError(f"bad shape n={n}, k={k} (need n >= 1, k a positive multiple of 128)")
    return int(v)


def packed_bytes(n: int, k: int, r: int) -> int:
    v = _lib().nbw_packed_bytes(n, k, r)
    if v < 0:
        raise ValueError(f"bad shape or bit-width n={n}, k={k}, r={r}")
    return int(v)


class PackedWeight:
    """Bit-planes of an n x k weight: ``nplanes`` planes (8 = parent, r = child).

    ``storage`` is the uint8 device tensor holding at least ``nplanes`` planes; a child
    made by ``slice_view`` shares it."""

    def __init__(self, storage: torch.Tensor, n: int, k: int, nplanes: int):
        self.storage = storage
        self.n, self.k, self.nplanes = n, k, nplanes
        self.view = WView()
        _check(_lib().nbw_make_view(ctypes.c_void_p(storage.data_ptr()), n, k, nplanes,
                                    ctypes.byref(self.view)), "nbw_make_view")

    @property
    def plane_bytes(self) -> int:
        return int(self.view.plane_bytes)

    @property
    def nbytes(self) -> int:
        """Bytes of plane data this view reads (nplanes * plane_bytes)."""
        return self.nplanes * self.plane_bytes

    def slice_view(self, r: int) -> "PackedWeight":
        return slice_view(self, r)

    def __repr__(self):
        return f"PackedWeight(n={self.n}, k={self.k}, nplanes={self.nplanes})"


def pack_bitplanes(codes: torch.Tensor, out: torch.Tensor | None = None) -> PackedWeight:
    """uint8 parent codes [n][k] (GPU) -> 8-plane PackedWeight."""
    _need(codes, "codes", torch.uint8, 2)
    n, k = codes.shape
    need = 8 * plane_bytes(n, k)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=codes.device)
    else:
        _need(out, "out", torch.uint8, 1)
        if out.numel() < need or out.device != codes.device:
            raise ValueError("out is too small or on another device")
    _check(_lib().nbw_pack_bitplanes(ctypes.c_void_p(codes.data_ptr()), n, k,
                                     ctypes.c_void_p(out.data_ptr()), out.numel(),
                                     _stream(codes)), "nbw_pack_bitplanes")
    return PackedWeight(out, n, k, 8)


def slice_view(w: PackedWeight, r: int) -> PackedWeight:
    """The r-bit child of ``w``: the first r planes of the same storage (host only)."""
    child = WView()
    _check(_lib().nbw_slice_view(ctypes.byref(w.view), r, ctypes.byref(child)), "nbw_slice_view")
    out = PackedWeight.__new__(PackedWeight)
    out.storage, out.n, out.k, out.nplanes, out.view = w.storage, w.n, w.k, r, child
    return out


def _need_rows(t: torch.Tensor, name: str, dtype, cols: int) -> None:
    """A 2-d tensor whose rows are contiguous (row stride may exceed `cols`)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.shape[1] != cols or (t.shape[0] > 1 and t.stride(0) < cols) or \
            (cols > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be [rows][{cols}] with unit column stride")


def qgemm(x: torch.Tensor, w: PackedWeight, scales: torch.Tensor, r: int,
          out: torch.Tensor | None = None, kernel: str = "auto", zeros: torch.Tensor | None = None,
          out_dtype=torch.float32, workspace="auto") -> torch.Tensor:
    """Y [B][n] = X . dequant_r(W)^T for the r-bit child of ``w``.

    ``x`` may have a row stride larger than k (e.g. a column slice of a wider
    tensor), as may ``out``; ``zeros`` (bf16 [n][k/128]) selects asymmetric
    children; ``out_dtype`` is torch.float32 or torch.bfloat16.  ``workspace``:
    "auto" (the binding's buffer for this device and stream), a uint8 device
    tensor, or None (a large-batch launch then runs unsplit)."""
    _need(scales, "scales", torch.bfloat16, 2)
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-d tensor")
    b, k = x.shape
    if k != w.k:
        raise ValueError(f"x has k={k}, weights have k={w.k}")
    _need_rows(x, "x", torch.bfloat16, k)
    if tuple(scales.shape) != (w.n, w.k // 128):
        raise ValueError(f"scales must be [{w.n}][{w.k // 128}], got {tuple(scales.shape)}")
    if scales.device != x.device or w.storage.device != x.device:
        raise ValueError("x, scales and weights must be on the same GPU")
    if out_dtype not in Y_DTYPES:
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    if zeros is not None:
        _need(zeros, "zeros", torch.bfloat16, 2)
        if tuple(zeros.shape) != (w.n, w.k // 128) or zeros.device != x.device:
            raise ValueError(f"zeros must be [{w.n}][{w.k // 128}] on the same GPU")
    if out is None:
        out = torch.empty((b, w.n), dtype=out_dtype, device=x.device)
    else:
        _need_rows(out, "out", out_dtype, w.n)
        if out.shape[0] != b or out.device != x.device:
            raise ValueError(f"out must be [{b}][{w.n}] on the same GPU")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', a tensor or None")
        dev = x.device.index if x.device.index is not None else torch.cuda.current_device()
        workspace = _workspace(dev, _raw_stream(dev), workspace_bytes(b, w.n, w.k, r, kernel))
    if workspace is not None and (workspace.device != x.device or workspace.dtype != torch.uint8):
        raise ValueError("workspace must be a uint8 tensor on the inputs' GPU")
    opts = QgemmOpts(x.stride(0) if b > 1 else k, out.stride(0) if b > 1 else w.n,
                     Y_DTYPES[out_dtype], KERNELS[kernel],
                     zeros.data_ptr() if zeros is not None else None,
                     workspace.data_ptr() if workspace is not None else None,
                     workspace.numel() if workspace is not None else 0)
    _check(_lib().nbw_qgemm_ex(ctypes.c_void_p(x.data_ptr()), b, ctypes.byref(w.view),
                               ctypes.c_void_p(scales.data_ptr()), r,
                               ctypes.c_void_p(out.data_ptr()), ctypes.byref(opts), _stream(x)),
           "nbw_qgemm")
    return out


def choose_codes(w: torch.Tensor, scales: torch.Tensor, widths=(3, 4, 8),
                 lambdas=(1.0, 1.0, 1.0)) -> torch.Tensor:
    """Parent codes uint8 [n][k] for fp32 weights [n][k] (GPU): per weight, the
    code minimising sum_t lambdas[t] * (w - dequant_{widths[t]}(code))^2."""
    _need(w, "w", torch.float32, 2)
    _need(scales, "scales", torch.bfloat16, 2)
    n, k = w.shape
    if tuple(scales.shape) != (n, k // 128) or k % 128:
        raise ValueError(f"scales must be [{n}][{k // 128}] and k a multiple of 128")
    widths = list(widths)
    lambdas = list(lambdas)
    if len(widths) != len(lambdas):
        raise ValueError("widths and lambdas must have the same length")
    wa = (ctypes.c_int32 * max(1, len(widths)))(*widths)
    la = (ctypes.c_double * max(1, len(lambdas)))(*lambdas)
    out = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    _check(_lib().nbw_choose_codes(ctypes.c_void_p(w.data_ptr()), n, k,
                                   ctypes.c_void_p(scales.data_ptr()), wa, la, len(widths),
                                   ctypes.c_void_p(out.data_ptr()), _stream(w)), "nbw_choose_codes")
    return out


_WORKSPACES = {}


def workspace_bytes(batch: int, n: int, k: int, r: int, kernel: str = "auto") -> int:
    """Bytes of split-k workspace nbw_qgemm_ex uses for this problem (0: none)."""
    nb = _lib().nbw_qgemm_workspace_bytes(batch, n, k, r, KERNELS[kernel])
    if nb < 0:
        raise ValueError("workspace_bytes: bad arguments")
    return nb


def _workspace(device_index: int, stream: int, nbytes: int):
    """The binding's split-k workspace for (device, stream): calls on one
    stream never overlap, so one buffer per stream suffices."""
    if nbytes <= 0:
        return None
    key = (device_index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device("cuda", device_index))
        _WORKSPACES[key] = ws
    return ws


class QgemmCall:
    """One qgemm with its arguments checked and marshalled once.

    Calling it issues the product on the current stream of the inputs' device (or on
    ``stream``, a raw HIP stream handle) with a single library call; the tensors are
    kept alive by the object.  Use it where per-call Python cost matters, e.g. when a
    decode step is captured into a HIP graph or launched in a tight loop."""

    __slots__ = ("x", "w", "scales", "r", "out", "kernel", "_args", "_fn", "_dev", "_nb", "_ws",
                 "_opts", "_view")

    def __init__(self, x, w, scales, r, out=None, kernel="auto"):
        _need(x, "x", torch.bfloat16, 2)
        _need(scales, "scales", torch.bfloat16, 2)
        b, k = x.shape
        if k != w.k:
            raise ValueError(f"x has k={k}, weights have k={w.k}")
        if tuple(scales.shape) != (w.n, w.k // 128):
            raise ValueError(f"scales must be [{w.n}][{w.k // 128}], got {tuple(scales.shape)}")
        if scales.device != x.device or w.storage.device != x.device:
            raise ValueError("x, scales and weights must be on the same GPU")
        if out is None:
            out = torch.empty((b, w.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, "out", torch.float32, 2)
            if tuple(out.shape) != (b, w.n) or out.device != x.device:
                raise ValueError(f"out must be [{b}][{w.n}] on the same GPU")
        if kernel not in KERNELS:
            raise ValueError(f"unknown kernel {kernel!r}")
        self.x, self.w, self.scales, self.r, self.out, self.kernel = x, w, scales, r, out, kernel
        self._dev = x.device.index if x.device.index is not None else torch.cuda.current_device()
        # split-k workspace: the binding's buffer of the stream each call runs on
        # (calls on one stream never overlap; calls on two streams never share one)
        self._nb = workspace_bytes(b, w.n, w.k, r, kernel)
        self._ws = {}
        self._opts = {}
        self._view = WView.from_buffer_copy(w.view)
        self._args = (ctypes.c_void_p(x.data_ptr()), b, ctypes.byref(self._view),
                      ctypes.c_void_p(scales.data_ptr()), r, ctypes.c_void_p(out.data_ptr()))
        self._fn = _lib().nbw_qgemm_ex

    def _opts_for(self, stream: int):
        opts = self._opts.get(stream)
        if opts is None:
            ws = _workspace(self._dev, stream, self._nb)
            opts = QgemmOpts(0, 0, 0, KERNELS[self.kernel], None,
                             ws.data_ptr() if ws is not None else None,
                             ws.numel() if ws is not None else 0)
            self._ws[stream] = ws  # keeps the buffer alive with the prepared call
            self._opts[stream] = opts
        return opts

    def __call__(self, stream=None):
        if stream is None:
            stream = _raw_stream(self._dev)
        st = self._fn(*self._args, ctypes.byref(self._opts_for(stream)), ctypes.c_void_p(stream))
        if st != 0:
            raise NBWError(st, "nbw_qgemm")
        return self.out


def qgemm_grouped(items, outs=None):
    """Several products in as few dispatches as possible.

    ``items``: sequence of ``(x, w, scales, r)`` as for :func:`qgemm`.  Returns the
    fp32 outputs (or fills ``outs``).  Batch 1..4 products run as grouped launches of
    the streaming kernel (one for batch 1, one for batch 2..4), batch-5..16 products
    as one of the small-batch kernel (k/128 a multiple of 4 for both); the rest one
    by one."""
    items = list(items)
    if outs is None:
        outs = [None] * len(items)
    arr = (Problem * max(1, len(items)))()
    results = []
    for j, ((x, w, scales, r), out) in enumerate(zip(items, outs)):
        _need(x, "x", torch.bfloat16, 2)
        _need(scales, "scales", torch.bfloat16, 2)
        b, k = x.shape
        if k != w.k or tuple(scales.shape) != (w.n, w.k // 128):
            raise ValueError(f"problem {j}: shapes of x / scales do not match the weights")
        if out is None:
            out = torch.empty((b, w.n), dtype=torch.float32, device=x.device)
        else:
            _need(out, "out", torch.float32, 2)
            if tuple(out.shape) != (b, w.n):
                raise ValueError(f"problem {j}: out must be [{b}][{w.n}]")
        arr[j].x_bf16 = x.data_ptr()
        arr[j].batch = b
        arr[j].w = w.view
        arr[j].scales_bf16 = scales.data_ptr()
        arr[j].r = r
        arr[j].y = out.data_ptr()
        results.append(out)
    if items:
        _check(_lib().nbw_qgemm_grouped(arr, len(items), _stream(items[0][0])), "nbw_qgemm_grouped")
    return results


def unpack_codes(w: PackedWeight, r: int) -> torch.Tensor:
    """Child codes q_r [n][k] (uint8) decoded on the GPU from planes 0..r-1 (test hook)."""
    out = torch.empty((w.n, w.k), dtype=torch.uint8, device=w.storage.device)
    _check(_lib().nbw_unpack_codes(ctypes.byref(w.view), r, ctypes.c_void_p(out.data_ptr()),
                                   _stream(out)), "nbw_unpack_codes")
    return out


def stream_sink(device=None) -> torch.Tensor:
    """A sink buffer for stream_read (nbw_stream_sink_words() uint32 words)."""
    return torch.empty(_lib().nbw_stream_sink_words(), dtype=torch.int32,
                       device=device if device is not None else "cuda")


def stream_read(src: torch.Tensor, nbytes: int, sink: torch.Tensor) -> None:
    """Launch the plain streaming read of the first nbytes of src (bandwidth reference)."""
    if sink.numel() < _lib().nbw_stream_sink_words() or sink.dtype != torch.int32:
        raise ValueError(f"stream_read: sink needs {_lib().nbw_stream_sink_words()} int32 words")
    if nbytes > src.numel() * src.element_size():
        raise ValueError("stream_read: nbytes exceeds the source tensor")
    _check(_lib().nbw_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                  ctypes.c_void_p(sink.data_ptr()), _stream(src)), "nbw_stream_read")


MFMA_RATE_OPS_BYTES = 16 * 64 * 16  # 16 fragments x 64 lanes x 16 bytes


def mfma_rate_sink(device=None) -> torch.Tensor:
    """A sink buffer for mfma_rate (nbw_mfma_rate_sink_floats() floats)."""
    nf = _lib().nbw_mfma_rate_sink_floats()
    if nf < 0:
        raise NBWError("nbw_mfma_rate_sink_floats: no device")
    return torch.empty(nf, dtype=torch.float32, device=device if device is not None else "cuda")


def mfma_rate_flops(sink: torch.Tensor, iters: int) -> int:
    """Flops of one mfma_rate launch of `iters` rounds (64 MFMAs of 32768 flops per wave and round)."""
    return sink.numel() // 64 * iters * 64 * 32768


def mfma_rate(ops: torch.Tensor, iters: int, sink: torch.Tensor) -> None:
    """Launch the matrix-unit rate loop on the 16 KB of operand fragments in ops (compute reference)."""
    if ops.numel() * ops.element_size() < MFMA_RATE_OPS_BYTES:
        raise ValueError(f"mfma_rate: ops needs {MFMA_RATE_OPS_BYTES} bytes")
    if sink.dtype != torch.float32 or sink.numel() < _lib().nbw_mfma_rate_sink_floats():
        raise ValueError(f"mfma_rate: sink needs {_lib().nbw_mfma_rate_sink_floats()} float32 values")
    _check(_lib().nbw_mfma_rate(ctypes.c_void_p(ops.data_ptr()), int(iters), ctypes.c_void_p(sink.data_ptr()),
                                _stream(ops)), "nbw_mfma_rate")


def file_prefix_bytes(n: int, k: int, r: int) -> int:
    """Bytes at the head of a parent file that hold everything an r-bit child needs."""
    v = _lib().nbw_file_prefix_bytes(n, k, r)
    if v < 0:
        raise ValueError(f"bad shape or bit-width n={n}, k={k}, r={r}")
    return int(v)


def save_parent(path, w: PackedWeight, scales: torch.Tensor) -> None:
    """Write the 8-plane parent ``w`` and its bf16 scales [n][k/128] to ``path``
    (header, scales, planes 0..7: the library's file layout, whose r-bit child is
    the file's first ``file_prefix_bytes(n, k, r)`` bytes).  The planes and scales
    may live on the GPU or on the host; they are copied to the host to be written."""
    if w.nplanes != 8:
        raise ValueError("save_parent needs the 8-plane parent")
    if not isinstance(scales, torch.Tensor) or scales.dtype != torch.bfloat16:
        raise ValueError("scales must be a bf16 tensor (host or device)")
    if tuple(scales.shape) != (w.n, w.k // 128):
        raise ValueError(f"scales must be [{w.n}][{w.k // 128}]")
    hdr = ctypes.create_string_buffer(FILE_HEADER_BYTES)
    _check(_lib().nbw_file_header(w.n, w.k, hdr), "nbw_file_header")
    info = FileInfo()
    _check(_lib().nbw_file_parse(hdr, file_prefix_bytes(w.n, w.k, 8), ctypes.byref(info)),
           "nbw_file_parse")
    sbytes = scales.contiguous().view(torch.uint8).reshape(-1).cpu().numpy().tobytes()
    planes = w.storage[: 8 * w.plane_bytes].cpu().numpy().tobytes()
    with open(path, "wb") as f:
        f.write(hdr.raw)
        f.write(sbytes)
        f.write(b"\0" * (info.planes_offset - info.scales_offset - len(sbytes)))
        f.write(planes)


def file_info(path) -> FileInfo:
    """Header of a parent (or child) file, checked, with the planes its size holds."""
    with open(path, "rb") as f:
        hdr = f.read(FILE_HEADER_BYTES)
    if len(hdr) < FILE_HEADER_BYTES:
        raise ValueError(f"{path}: shorter than a header")
    info = FileInfo()
    _check(_lib().nbw_file_parse(hdr, os.path.getsize(path), ctypes.byref(info)), "nbw_file_parse")
    return info


def load_child(path, r: int, device="cuda"):
    """The r-bit child of the parent stored in ``path``: reads only the file's first
    ``file_prefix_bytes(n, k, r)`` bytes (header, scales, planes 0..r-1).  Returns
    (PackedWeight with r planes, bf16 scales [n][k/128]) on ``device``."""
    info = file_info(path)
    if not 1 <= r <= info.planes_present:
        raise ValueError(f"{path}: r={r} needs {r} planes, the file holds {info.planes_present}")
    n, k = int(info.n), int(info.k)
    with open(path, "rb") as f:
        f.seek(info.scales_offset)
        sb = f.read(info.scales_bytes)
        f.seek(info.planes_offset)
        pb = f.read(r * info.plane_bytes)
    if len(sb) != info.scales_bytes or len(pb) != r * info.plane_bytes:
        raise ValueError(f"{path}: short read")
    # fresh tensors on the device (aligned as the views require), filled from the bytes read
    scales = torch.empty((n, k // 128), dtype=torch.bfloat16, device=device)
    scales.view(torch.uint8).reshape(-1).copy_(torch.frombuffer(bytearray(sb), dtype=torch.uint8))
    planes = torch.empty(r * info.plane_bytes, dtype=torch.uint8, device=device)
    planes.copy_(torch.frombuffer(bytearray(pb), dtype=torch.uint8))
    return PackedWeight(planes, n, k, r), scales


def kernel_name(batch: int, n: int, k: int, r: int, kernel: str = "auto") -> str:
    """Name of the kernel instance nbw_qgemm would launch (as profilers print it)."""
    return _lib().nbw_kernel_name(batch, n, k, r, KERNELS[kernel]).decode()


def version() -> str:
    return _lib().nbw_version().decode()


__all__ = ["pack_bitplanes", "slice_view", "save_parent", "load_child", "file_info",
           "file_prefix_bytes", "qgemm", "QgemmCall", "qgemm_grouped", "workspace_bytes", "choose_codes", "unpack_codes", "stream_read", "stream_sink", "mfma_rate", "mfma_rate_sink", "mfma_rate_flops", "plane_bytes",
           "packed_bytes", "PackedWeight", "NBWError", "KERNELS", "library", "kernel_name",
           "version"]
