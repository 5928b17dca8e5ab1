"""ctypes binding of libw4a16.so: argument marshalling only.

Every entry point has the name of its C function (include/w4a16.h). Device buffers are
torch tensors on a HIP device (torch provides memory and streams, nothing else); host
buffers are NumPy arrays. All arithmetic happens in the library.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libw4a16.so")

W4A16_OK = 0
W4A16_ERR_INVALID_ARG = -1
W4A16_ERR_UNSUPPORTED = -2
W4A16_ERR_ALIGNMENT = -3
W4A16_ERR_NONFINITE = -4
W4A16_ERR_HIP = -5

W4A16_KERNEL_AUTO = 0
W4A16_KERNEL_SKINNY = 1
W4A16_KERNEL_PREFILL = 2
W4A16_TILE_LDS = 1
W4A16_TILE_REGISTER_B = 2
W4A16_TILE_ASYNC = 3
W4A16_LAYOUT_LINEAR = 0
W4A16_LAYOUT_INTERLEAVED = 1

GROUP_SIZE = 128


class W4A16Error(RuntimeError):
    def __init__(self, code, func, detail):
        self.code = code
        super().__init__(f"{func} failed: {code} ({strerror(code)}): {detail}")


class w4a16_plan_t(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("kc", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("row_tiles", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("cols", ctypes.c_int32), ("seg", ctypes.c_int32)]

    def as_dict(self):
        return {"kernel": self.kernel, "kc": self.kc, "splits": self.splits,
                "row_tiles": self.row_tiles, "tile": self.tile, "waves": self.waves,
                "cols": self.cols, "seg": self.seg}


class w4a16_matrix_t(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("x", ctypes.c_void_p), ("M", ctypes.c_int64)]


MAX_GROUP_MATS = 16


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "w4a16_pack": ([_P, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "w4a16_pack_ex": ([_P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P], ctypes.c_int),
    "w4a16_unpack": ([_P, _I64, _I64, _P], ctypes.c_int),
    "w4a16_unpack_ex": ([_P, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "w4a16_matmul": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "w4a16_matmul_ex": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P,
                         ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_matmul_fmt": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, _P,
                          ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_matmul_grouped": ([_P, ctypes.POINTER(w4a16_matrix_t), ctypes.c_int, _I64, _I64, _I64, ctypes.c_int, _P,
                              ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_matmul_noalloc": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, _P,
                              ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_plan": ([_I64, _I64, _I64, _I64, ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_dequant": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "w4a16_dequant_fmt": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "w4a8_quantize_activations": ([_P, _P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "w4a8_matmul": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "w4a8_matmul_ex": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int, _P],
                       ctypes.c_int),
    "w4a16_read_probe": ([_P, _I64, _P, _P], ctypes.c_int),
    "w4a16_autotune": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, _P,
                        ctypes.POINTER(w4a16_plan_t), ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "w4a16_set_plan": ([_I64, _I64, _I64, _I64, ctypes.POINTER(w4a16_plan_t)], ctypes.c_int),
    "w4a16_clear_plans": ([], ctypes.c_int),
    "w4a16_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "w4a16_last_error_detail": ([], ctypes.c_char_p),
    "w4a16_version": ([], ctypes.c_int),
}


def _bind_hip_runtime():
    """Make the library use the HIP runtime that torch already uses.

    torch ships its own libamdhip64 with the same soname (libamdhip64.so.7) as the ROCm
    one libw4a16.so is linked against. Loaded after torch, the library binds to torch's
    copy, so device pointers and stream handles from torch belong to the runtime the
    library calls. Loaded first, it would pull in a second HIP and HSA runtime, whose
    streams are not torch's and which may not see the device at all.
    """
    try:
        import torch  # noqa: F401
    except ImportError:          # no torch in the process: the ROCm runtime is the only one
        pass


def hip_runtimes_loaded():
    """Paths of the libamdhip64 files mapped into this process (Linux)."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(line.split()[-1])
    except OSError:
        pass
    return sorted(paths)


def load(build_if_missing=True):
    """Load libw4a16.so (building it in-tree first if it is absent). Raises if it cannot."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise ImportError(f"{LIB_PATH} is not built")
        from . import build as _build
        _build.build()
    _bind_hip_runtime()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def strerror(code):
    return load().w4a16_strerror(code).decode()


def _check(rc, func):
    if rc != W4A16_OK:
        raise W4A16Error(rc, func, load().w4a16_last_error_detail().decode())


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, dtype):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# ---- host entry points ------------------------------------------------------------------

_LAYOUTS = {"linear": 0, "interleaved": 1}


def _layout_id(layout):
    """"linear" / "interleaved" (or the W4A16_LAYOUT_* integer) -> the ABI's integer."""
    if isinstance(layout, str):
        if layout not in _LAYOUTS:
            raise ValueError(f"unknown layout {layout!r}")
        return _LAYOUTS[layout]
    return int(layout)


def w4a16_pack(W, group_size=GROUP_SIZE, symmetric=False, layout="linear"):
    """W fp32 [K, N] (NumPy) -> (qweight int32 [K/8, N], scales fp16, zeros fp16).
    symmetric=True selects the +8 zero-point quantiser; layout "interleaved" the
    pre-permuted packing (w4a16_pack_ex)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    K, N = W.shape
    G = K // group_size if group_size > 0 else 0
    qweight = np.empty((K // 8, N), dtype=np.int32)
    scales = np.empty((max(G, 0), N), dtype=np.float16)
    zeros = np.empty((max(G, 0), N), dtype=np.float16)
    rc = load().w4a16_pack_ex(W.ctypes.data, K, N, group_size, 1 if symmetric else 0,
                              _layout_id(layout), qweight.ctypes.data, scales.ctypes.data,
                              zeros.ctypes.data)
    _check(rc, "w4a16_pack_ex")
    return qweight, scales, zeros


def w4a16_unpack(qweight, layout="linear"):
    """qweight int32 [K/8, N] (NumPy) -> codes uint8 [K, N] in natural K order."""
    qweight = np.ascontiguousarray(qweight, dtype=np.int32)
    P, N = qweight.shape
    codes = np.empty((P * 8, N), dtype=np.uint8)
    _check(load().w4a16_unpack_ex(qweight.ctypes.data, P * 8, N, _layout_id(layout), codes.ctypes.data),
           "w4a16_unpack_ex")
    return codes


def _make_plan(d):
    return w4a16_plan_t(kernel=d.get("kernel", 0), kc=d.get("kc", 0), splits=d.get("splits", 0),
                        row_tiles=d.get("row_tiles", 0), tile=d.get("tile", 0),
                        waves=d.get("waves", 0), cols=d.get("cols", 0), seg=d.get("seg", 0))


def w4a16_plan(M, N, K, group_size=GROUP_SIZE, **plan):
    """The completed plan for (M, N, K): the dispatcher's, or a forced one filled in."""
    pl = _make_plan(plan)
    _check(load().w4a16_plan(M, N, K, group_size, ctypes.byref(pl)), "w4a16_plan")
    return pl.as_dict()


# ---- device entry points ------------------------------------------------------------------

def w4a16_matmul(x, qweight, scales, zeros, y=None, group_size=GROUP_SIZE, stream=None, plan=None,
                 layout="linear"):
    """y[M, N] = x[M, K] . dequant(qweight, scales, zeros); torch tensors on one device.

    x fp16 [M, K]; qweight int32 [K/8, N]; scales, zeros fp16 [K/g, N]; y fp16 [M, N]
    (allocated when None). Enqueued on `stream` (default: torch's current stream).
    `plan` (dict with kernel/kc/row_tiles/waves/tile) forces the execution plan; `layout`
    names the packing of qweight ("linear" or "interleaved").
    """
    import torch
    if x.dim() != 2 or qweight.dim() != 2:
        raise ValueError("x and qweight must be 2-D")
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError(f"qweight rows {qweight.shape[0]} do not match K={K}")
    if scales.shape != (K // group_size, N) or zeros.shape != (K // group_size, N):
        raise ValueError("scales/zeros must be [K/group_size, N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    args = [_dev_ptr(x, "x", torch.float16), _dev_ptr(qweight, "qweight", torch.int32),
            _dev_ptr(scales, "scales", torch.float16), _dev_ptr(zeros, "zeros", torch.float16),
            _dev_ptr(y, "y", torch.float16), M, N, K, group_size, _stream_ptr(stream, x.device)]
    lay = _layout_id(layout)
    if plan is None and lay == 0:
        rc = load().w4a16_matmul(*args)
        _check(rc, "w4a16_matmul")
    elif lay == 0:
        pl = _make_plan(plan)
        rc = load().w4a16_matmul_ex(*args, ctypes.byref(pl))
        _check(rc, "w4a16_matmul_ex")
    else:
        pl = ctypes.byref(_make_plan(plan)) if plan is not None else None
        rc = load().w4a16_matmul_fmt(*args[:-1], lay, args[-1], pl)
        _check(rc, "w4a16_matmul_fmt")
    return y


def w4a16_autotune(x, qweight, scales, zeros, y=None, group_size=GROUP_SIZE, stream=None, layout="linear"):
    """Time the plans of this shape on the device (w4a16_autotune) and keep the fastest for
    later calls of (M, N, K, group_size) in this process. Synchronous. Returns (plan dict,
    seconds per call); y (allocated when None) holds the product afterwards."""
    import torch
    if x.dim() != 2 or qweight.dim() != 2:
        raise ValueError("x and qweight must be 2-D")
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError(f"qweight rows {qweight.shape[0]} do not match K={K}")
    if scales_shape_bad(scales, zeros, K, N, group_size):
        raise ValueError("scales/zeros must be [K/group_size, N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    pl = w4a16_plan_t()
    sec = ctypes.c_double(0.0)
    rc = load().w4a16_autotune(_dev_ptr(x, "x", torch.float16), _dev_ptr(qweight, "qweight", torch.int32),
                               _dev_ptr(scales, "scales", torch.float16), _dev_ptr(zeros, "zeros", torch.float16),
                               _dev_ptr(y, "y", torch.float16), M, N, K, group_size, _layout_id(layout),
                               _stream_ptr(stream, x.device), ctypes.byref(pl), ctypes.byref(sec))
    _check(rc, "w4a16_autotune")
    return pl.as_dict(), sec.value


def w4a16_set_plan(M, N, K, plan, group_size=GROUP_SIZE):
    """Make `plan` (a dict as w4a16_plan returns, or None to remove) the plan that later calls
    of (M, N, K, group_size) take when they leave the plan to the dispatcher."""
    pl = ctypes.byref(_make_plan(plan)) if plan is not None else None
    _check(load().w4a16_set_plan(M, N, K, group_size, pl), "w4a16_set_plan")


def w4a16_clear_plans():
    """Forget every plan set by w4a16_autotune or w4a16_set_plan."""
    _check(load().w4a16_clear_plans(), "w4a16_clear_plans")


def w4a16_matmul_grouped(x, weights, ys=None, group_size=GROUP_SIZE, stream=None, plan=None, layout="linear"):
    """y_i = x_i . dequant(W_i) for the matrices in `weights` (a list of (qweight, scales, zeros)
    or (qweight, scales, zeros, x_i), 1..16 of them; x_i defaults to x; an x_i of M_i <= M rows
    gives y_i of M_i rows) in one call of w4a16_matmul_grouped; returns the list of y_i
    (allocated when `ys` is None)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    if not 1 <= len(weights) <= MAX_GROUP_MATS:
        raise ValueError(f"1..{MAX_GROUP_MATS} weight matrices")
    weights = [tuple(w) if len(w) == 4 else tuple(w) + (None,) for w in weights]
    rows = [M if w[3] is None else w[3].shape[0] for w in weights]
    if ys is None:
        ys = [torch.empty((m, w[0].shape[1]), dtype=torch.float16, device=x.device) for m, w in zip(rows, weights)]
    arr = (w4a16_matrix_t * len(weights))()
    for i, ((qw, s, z, xi), y, Mi) in enumerate(zip(weights, ys, rows)):
        if xi is not None and (xi.dim() != 2 or xi.shape[1] != K or not 1 <= Mi <= M):
            raise ValueError(f"matrix {i}: its x must be [M_i, K] with 1 <= M_i <= M = {M}, K = {K}")
        N = qw.shape[1]
        if qw.dim() != 2 or qw.shape[0] * 8 != K:
            raise ValueError(f"matrix {i}: qweight must be [K/8, N] with K={K}")
        if scales_shape_bad(s, z, K, N, group_size):
            raise ValueError(f"matrix {i}: scales/zeros must be [K/group_size, N]")
        if y.shape != (Mi, N):
            raise ValueError(f"matrix {i}: y must be [M_i, N]")
        arr[i] = w4a16_matrix_t(_dev_ptr(qw, "qweight", torch.int32), _dev_ptr(s, "scales", torch.float16),
                                _dev_ptr(z, "zeros", torch.float16), _dev_ptr(y, "y", torch.float16), N,
                                None if xi is None else _dev_ptr(xi, "x", torch.float16), Mi)
    pl = ctypes.byref(_make_plan(plan)) if plan is not None else None
    rc = load().w4a16_matmul_grouped(_dev_ptr(x, "x", torch.float16), arr, len(weights), M, K, group_size,
                                     _layout_id(layout), _stream_ptr(stream, x.device), pl)
    _check(rc, "w4a16_matmul_grouped")
    return ys


def scales_shape_bad(scales, zeros, K, N, group_size):
    return group_size <= 0 or scales.shape != (K // group_size, N) or zeros.shape != (K // group_size, N)


def w4a16_matmul_noalloc(x, qweight, scales, zeros, y, group_size=GROUP_SIZE, stream=None, plan=None,
                         layout="linear"):
    """w4a16_matmul through the entry point that allocates nothing (split-K partials in the
    library's static scratch). y fp16 [M, N] must be given: nothing is allocated here either."""
    import torch
    if x.dim() != 2 or qweight.dim() != 2:
        raise ValueError("x and qweight must be 2-D")
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError(f"qweight rows {qweight.shape[0]} do not match K={K}")
    if scales.shape != (K // group_size, N) or zeros.shape != (K // group_size, N):
        raise ValueError("scales/zeros must be [K/group_size, N]")
    if y is None or y.shape != (M, N):
        raise ValueError("y must be an fp16 [M, N] tensor")
    pl = ctypes.byref(_make_plan(plan)) if plan is not None else None
    rc = load().w4a16_matmul_noalloc(_dev_ptr(x, "x", torch.float16), _dev_ptr(qweight, "qweight", torch.int32),
                                     _dev_ptr(scales, "scales", torch.float16), _dev_ptr(zeros, "zeros", torch.float16),
                                     _dev_ptr(y, "y", torch.float16), M, N, K, group_size, _layout_id(layout),
                                     _stream_ptr(stream, x.device), pl)
    _check(rc, "w4a16_matmul_noalloc")
    return y


def w4a16_matmul_ex(x, qweight, scales, zeros, y=None, plan=None, group_size=GROUP_SIZE,
                    stream=None):
    """w4a16_matmul with a forced plan (dict: kernel, kc, row_tiles, waves, tile)."""
    return w4a16_matmul(x, qweight, scales, zeros, y=y, group_size=group_size, stream=stream,
                        plan=plan if plan is not None else {})


def w4a16_dequant(qweight, scales, zeros, codes=True, weights=True, group_size=GROUP_SIZE,
                  stream=None, layout="linear"):
    """The GPU's unpack/dequant: returns (codes uint8 [K, N] or None, w fp16 [K, N] or None),
    both in natural K order."""
    import torch
    if qweight.dim() != 2:
        raise ValueError("qweight must be 2-D")
    K = qweight.shape[0] * 8
    N = qweight.shape[1]
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    if scales.shape != (K // group_size, N) or zeros.shape != (K // group_size, N):
        raise ValueError("scales/zeros must be [K/group_size, N]")
    c = torch.empty((K, N), dtype=torch.uint8, device=qweight.device) if codes else None
    w = torch.empty((K, N), dtype=torch.float16, device=qweight.device) if weights else None
    rc = load().w4a16_dequant_fmt(_dev_ptr(qweight, "qweight", torch.int32),
                                  _dev_ptr(scales, "scales", torch.float16),
                                  _dev_ptr(zeros, "zeros", torch.float16),
                                  ctypes.c_void_p(c.data_ptr()) if c is not None else None,
                                  ctypes.c_void_p(w.data_ptr()) if w is not None else None,
                                  N, K, group_size, _layout_id(layout), _stream_ptr(stream, qweight.device))
    _check(rc, "w4a16_dequant_fmt")
    return c, w


def w4a8_quantize(x, stream=None):
    """Per-row E4M3 quantisation of fp16 activations on the device: returns (xq uint8 [M, K],
    sx float32 [M], xsum float32 [K/128, Ms]) with x ~= dec(xq) * sx[:, None] and xsum the
    per-128-column block sums of dec(xq) (Ms = M rounded up to 4, padding rows 0)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    xsum = torch.empty((K // 128, w4a8_sum_stride(M)), dtype=torch.float32, device=x.device)
    rc = load().w4a8_quantize_activations(_dev_ptr(x, "x", torch.float16), _dev_ptr(xq, "xq", torch.uint8),
                                          _dev_ptr(sx, "sx", torch.float32), _dev_ptr(xsum, "xsum", torch.float32),
                                          M, K, _stream_ptr(stream, x.device))
    _check(rc, "w4a8_quantize_activations")
    return xq, sx, xsum


def w4a8_sum_stride(M):
    """Row stride of the block sums: M rounded up to a multiple of 4."""
    return (M + 3) // 4 * 4


def w4a8_matmul(xq, sx, xsum, qweight, scales, zeros, y=None, group_size=GROUP_SIZE, layout="linear", stream=None,
                splits=0):
    """y[M, N] = sx * sum_g s_g * (dec(xq) . (q - z)) per group (W4A8, q - z exact); xsum are
    the block sums w4a8_quantize returns; `splits` forces the split-K count (0: the
    library's choice)."""
    import torch
    if xq.dim() != 2 or qweight.dim() != 2 or sx.dim() != 1:
        raise ValueError("xq and qweight must be 2-D, sx 1-D")
    M, K = xq.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K or sx.shape[0] != M:
        raise ValueError("xq, sx and qweight disagree on M or K")
    if tuple(xsum.shape) != (K // 128, w4a8_sum_stride(M)):
        raise ValueError("xsum must be [K/128, M rounded up to 4]")
    if scales.shape != (K // group_size, N) or zeros.shape != (K // group_size, N):
        raise ValueError("scales/zeros must be [K/group_size, N]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=xq.device)
    elif y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    rc = load().w4a8_matmul_ex(_dev_ptr(xq, "xq", torch.uint8), _dev_ptr(sx, "sx", torch.float32),
                               _dev_ptr(xsum, "xsum", torch.float32),
                               _dev_ptr(qweight, "qweight", torch.int32), _dev_ptr(scales, "scales", torch.float16),
                               _dev_ptr(zeros, "zeros", torch.float16), _dev_ptr(y, "y", torch.float16), M, N, K,
                               group_size, _layout_id(layout), splits, _stream_ptr(stream, xq.device))
    _check(rc, "w4a8_matmul_ex")
    return y


def w4a16_version():
    return load().w4a16_version()
