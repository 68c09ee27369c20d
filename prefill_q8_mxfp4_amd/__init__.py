"""Python binding of libqgemm (the C ABI in include/qgemm.h).

Argument marshalling only: every step of the product runs in the HIP
kernels of ``csrc/``.  PyTorch supplies device memory and the stream.  If
``libqgemm.so`` has not been built, :func:`lib` raises: there is no fallback.

    import prefill_q8_mxfp4_amd as q
    buf = q.pack("q8_0", N, K, codes, scales)             # host bytes
    w = torch.from_numpy(buf).cuda()
    plan = q.Plan("q8_0", N, K, act="f32", out="f32", math="fp32")
    plan.run(x, w, y)                                     # y = x @ dequant(W)^T
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMM_LIB_PATH selects another build of the same library (the debug build
# with its extra environment overrides, for tests)
LIB_PATH = os.environ.get("QGEMM_LIB_PATH") or os.path.join(_HERE, "libqgemm.so")

OK, EINVAL, ENOTSUP, EHIP, ENOMEM = 0, 1, 2, 3, 4
FORMATS = {"q8_0": 0, "mxfp4": 1, "nvfp4": 2, "fp8": 3}
DTYPES = {"f32": 0, "bf16": 1}
EPILOGUES = {"none": 0, "swiglu": 1}
MATHS = {"fp32": 0, "bf16": 1}
TIERS = {1: "skinny", 2: "tiled", 3: "gemv"}
FLAG_FORCE_SKINNY = 0x1
FLAG_FORCE_TILED = 0x2
FLAG_FORCE_GEMV = 0x4
ALIGN = 256
MAX_TENSORS = 60

EXPORTS = ("qgemm_weight_bytes", "qgemm_pack", "qgemm_create", "qgemm_run", "qgemm_run_ws",
           "qgemm_run_noalloc", "qgemm_run_grouped", "qgemm_grouped_tier",
           "qgemm_workspace_bytes", "qgemm_plan_tier", "qgemm_init_device", "qgemm_xcd_local",
           "qgemm_device_status",
           "qgemm_destroy", "qgemm_dequantize", "qgemm_read_bytes", "qgemm_mfma_rate", "qgemm_strerror",
           "qgemm_last_error",
           "qgemm_version")
DEV_XCD_MISMATCH = 0x1
DEV_BAD_OFFSETS = 0x2
SCRATCH_BYTES = 64 << 20          # QGEMM_SCRATCH_BYTES
SCRATCH_COUNTER_BYTES = 1 << 20   # QGEMM_SCRATCH_COUNTER_BYTES

_lib = None


class QgemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qgemm status {status}: {msg}")
        self.status = status


def lib():
    """Load libqgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m prefill_q8_mxfp4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, u32, i32, sz = (ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int,
                             ctypes.c_size_t)
    L.qgemm_weight_bytes.restype = sz
    L.qgemm_weight_bytes.argtypes = [i32, i64, i64]
    L.qgemm_pack.restype = i32
    L.qgemm_pack.argtypes = [i32, i64, i64, vp, vp, vp, i64, vp, sz]
    L.qgemm_create.restype = i32
    L.qgemm_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i32, i64, i64, u32]
    L.qgemm_run.restype = i32
    L.qgemm_run.argtypes = [vp, i64, vp, vp, vp, vp]
    L.qgemm_run_ws.restype = i32
    L.qgemm_run_ws.argtypes = [vp, i64, vp, vp, vp, vp, sz, vp]
    L.qgemm_run_noalloc.restype = i32
    L.qgemm_run_noalloc.argtypes = [vp, i64, vp, vp, vp, vp]
    L.qgemm_run_grouped.restype = i32
    L.qgemm_run_grouped.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    L.qgemm_grouped_tier.restype = i32
    L.qgemm_grouped_tier.argtypes = [vp, i64, i64]
    L.qgemm_workspace_bytes.restype = sz
    L.qgemm_workspace_bytes.argtypes = [vp, i64]
    L.qgemm_plan_tier.restype = i32
    L.qgemm_plan_tier.argtypes = [vp, i64]
    L.qgemm_destroy.restype = i32
    L.qgemm_destroy.argtypes = [vp]
    L.qgemm_dequantize.restype = i32
    L.qgemm_dequantize.argtypes = [i32, vp, vp, i64, i64, vp]
    L.qgemm_mfma_rate.restype = i32
    L.qgemm_mfma_rate.argtypes = [i32, i32, vp, vp]
    L.qgemm_read_bytes.restype = i32
    L.qgemm_read_bytes.argtypes = [vp, sz, vp, i32, vp]
    L.qgemm_strerror.restype = ctypes.c_char_p
    L.qgemm_strerror.argtypes = [i32]
    L.qgemm_last_error.restype = ctypes.c_char_p
    L.qgemm_last_error.argtypes = []
    L.qgemm_version.restype = i32
    L.qgemm_version.argtypes = []
    L.qgemm_xcd_local.restype = i32
    L.qgemm_xcd_local.argtypes = []
    L.qgemm_init_device.restype = i32
    L.qgemm_init_device.argtypes = []
    L.qgemm_device_status.restype = i32
    L.qgemm_device_status.argtypes = [ctypes.POINTER(u32), i32, vp]
    _lib = L
    return L


_inited = set()


def init_device(device=None):
    """qgemm_init_device on a CUDA (HIP) device (default: the current one),
    once per device and process: the dispatch probe that enables the
    XCD-local K-split exchange.  Plans run without it (device-coherent
    exchange); the binding calls it before a device's first launch."""
    import torch

    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx in _inited:
        return
    with torch.cuda.device(idx):
        _check(lib().qgemm_init_device())
    _inited.add(idx)


def device_status(clear: bool = False, stream=None) -> int:
    """The current device's status word (DEV_* bits set by kernels since the
    last clear), after synchronising `stream` (default: the current one)."""
    bits = ctypes.c_uint32(0)
    _check(lib().qgemm_device_status(ctypes.byref(bits), int(bool(clear)), _stream_ptr(stream)))
    return int(bits.value)


def _check(status: int):
    if status != OK:
        raise QgemmError(status, lib().qgemm_last_error().decode())


def weight_bytes(fmt: str, N: int, K: int) -> int:
    return int(lib().qgemm_weight_bytes(FORMATS[fmt], N, K))


def pack(fmt: str, N: int, K: int, codes: np.ndarray, scales: np.ndarray, g=None) -> np.ndarray:
    """Pack logical arrays (host numpy) into the device layout (host uint8).

    codes: Q8_0 int8 [N][K]; FP4 uint8 [N][K] (one code per byte); FP8 uint8
    [N][K] E4M3 codes.
    scales: Q8_0 uint16 fp16 bits [N][K/32]; MXFP4 uint8 [N][K/32]; NVFP4 uint8 [N][K/16];
    FP8 float32 [N][ceil(K/128)].
    g: NVFP4 tensor scales (1..60 fp32 values; rows split evenly among them).
    """
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    if codes.shape != (N, K) or codes.itemsize != 1:
        raise QgemmError(EINVAL, f"codes must be one byte per weight, shape ({N}, {K})")
    want = {"q8_0": (np.uint16, K // 32), "mxfp4": (np.uint8, K // 32),
            "nvfp4": (np.uint8, K // 16), "fp8": (np.float32, -(-K // 128))}[fmt]
    if scales.dtype != want[0] or scales.shape != (N, want[1]):
        raise QgemmError(EINVAL, f"{fmt} scales must be {np.dtype(want[0]).name} [{N}][{want[1]}]")
    nbytes = weight_bytes(fmt, N, K)
    if nbytes == 0:
        raise QgemmError(EINVAL, f"bad shape for {fmt}: N={N} K={K}")
    out = np.empty(nbytes, dtype=np.uint8)
    gp, nt = None, 0
    if g is not None:
        g = np.ascontiguousarray(g, dtype=np.float32).ravel()
        gp, nt = g.ctypes.data_as(ctypes.c_void_p), g.size
    _check(lib().qgemm_pack(FORMATS[fmt], N, K, codes.ctypes.data_as(ctypes.c_void_p),
                            scales.ctypes.data_as(ctypes.c_void_p), gp, nt,
                            out.ctypes.data_as(ctypes.c_void_p), nbytes))
    return out


def pack_logical(w: dict) -> np.ndarray:
    """Pack a dict with keys fmt, codes, scales, g (the synthetic-input form)."""
    n, k = w["codes"].shape
    return pack(w["fmt"], n, k, w["codes"], w["scales"], w.get("g"))


def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """A validated problem shape (qgemm_create); run() launches on a stream."""

    def __init__(self, fmt: str, N: int, K: int, act: str = "bf16", out: str = "f32",
                 epilogue: str = "none", math: str | None = None, tier: str | None = None):
        if math is None:
            math = "fp32" if act == "f32" else "bf16"
        flags = 0
        if tier == "skinny":
            flags = FLAG_FORCE_SKINNY
        elif tier == "tiled":
            flags = FLAG_FORCE_TILED
        elif tier == "gemv":
            flags = FLAG_FORCE_GEMV
        elif tier is not None:
            raise ValueError(tier)
        self.fmt, self.N, self.K, self.act, self.out, self.epilogue, self.math = (
            fmt, N, K, act, out, epilogue, math)
        h = ctypes.c_void_p()
        _check(lib().qgemm_create(ctypes.byref(h), FORMATS[fmt], DTYPES[act], DTYPES[out],
                                  EPILOGUES[epilogue], MATHS[math], N, K, flags))
        self._h = h

    @property
    def out_cols(self) -> int:
        return self.N // 2 if self.epilogue == "swiglu" else self.N

    def tier(self, B: int) -> str:
        return TIERS.get(lib().qgemm_plan_tier(self._h, B), "invalid")

    def grouped_tier(self, E: int, T: int) -> str:
        """The route run_grouped takes for E experts and T rows: "skinny" (the
        small-batch order, bf16 math with few rows per expert), "tiled", or
        "invalid" (no route for this plan)."""
        return TIERS.get(lib().qgemm_grouped_tier(self._h, E, T), "invalid")

    def workspace_bytes(self, B: int) -> int:
        return int(lib().qgemm_workspace_bytes(self._h, B))

    def _workspace(self, B, device, stream):
        """Plan-owned zeroed workspace, grown on demand.  It is zeroed on the
        stream the call is launched on (so the kernels see it zeroed), and a
        replaced buffer is kept alive until that stream's work on it is done
        (record_stream).  Calls on one plan object must not overlap."""
        import torch

        need = self.workspace_bytes(B)
        if need == 0:
            return None
        ws = getattr(self, "_ws", None)
        if ws is None or ws.numel() < need or ws.device != device:
            with torch.cuda.stream(stream):
                ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
            old = getattr(self, "_ws", None)
            if old is not None and old.device == device and not torch.cuda.is_current_stream_capturing():
                old.record_stream(stream)
            self._ws = ws
        if not torch.cuda.is_current_stream_capturing():
            ws.record_stream(stream)
        return ws

    def run(self, x, w, y, stream=None, B: int | None = None, workspace="auto"):
        """y[B][out_cols] = x[B][K] (x) W; tensors on the GPU, contiguous.

        workspace: "auto" (a plan-owned buffer: calls on one plan object must
        not overlap), None (no K split), or a zero-initialised uint8 tensor."""
        import torch

        if B is None:
            B = x.shape[0]
        want_x = torch.float32 if self.act == "f32" else torch.bfloat16
        want_y = torch.float32 if self.out == "f32" else torch.bfloat16
        if x.dtype != want_x or y.dtype != want_y or w.dtype != torch.uint8:
            raise TypeError("dtype mismatch: x %s, w %s, y %s" % (x.dtype, w.dtype, y.dtype))
        if x.numel() < B * self.K or y.numel() < B * self.out_cols:
            raise ValueError("x or y too small for B")
        if w.numel() < weight_bytes(self.fmt, self.N, self.K):
            raise ValueError("packed weight buffer too small")
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        init_device(x.device)
        if isinstance(workspace, str):
            workspace = self._workspace(B, x.device, stream) if B > 0 else None
        wsp, wsn = None, 0
        if workspace is not None:
            wsp, wsn = _dev_ptr(workspace, "workspace"), workspace.numel()
        _check(lib().qgemm_run_ws(self._h, B, _dev_ptr(w, "w"), _dev_ptr(x, "x"),
                                  _dev_ptr(y, "y"), wsp, wsn, _stream_ptr(stream)))
        return y

    def run_noalloc(self, x, w, y, stream=None, B: int | None = None):
        """qgemm_run_noalloc: as run() with the library's static per-device
        scratch instead of a workspace (no allocation anywhere in the call;
        calls that overlap in time on one device race)."""
        import torch

        if B is None:
            B = x.shape[0]
        want_x = torch.float32 if self.act == "f32" else torch.bfloat16
        want_y = torch.float32 if self.out == "f32" else torch.bfloat16
        if x.dtype != want_x or y.dtype != want_y or w.dtype != torch.uint8:
            raise TypeError("dtype mismatch: x %s, w %s, y %s" % (x.dtype, w.dtype, y.dtype))
        if x.numel() < B * self.K or y.numel() < B * self.out_cols:
            raise ValueError("x or y too small for B")
        if w.numel() < weight_bytes(self.fmt, self.N, self.K):
            raise ValueError("packed weight buffer too small")
        init_device(x.device)
        _check(lib().qgemm_run_noalloc(self._h, B, _dev_ptr(w, "w"), _dev_ptr(x, "x"),
                                       _dev_ptr(y, "y"), _stream_ptr(stream)))
        return y

    def run_grouped(self, x, w_table, offsets, y, stream=None):
        """Routed experts: rows offsets[e] .. offsets[e+1]-1 of x and y use the
        packed weights at device address w_table[e].  w_table: int64 tensor of
        E device addresses (e.g. [t.data_ptr() for t in expert_buffers]) on the
        GPU; offsets: int32 [E + 1] on the GPU; x [T][K], y [T][out_cols]."""
        import torch

        T = x.shape[0]
        E = w_table.numel()
        want_x = torch.float32 if self.act == "f32" else torch.bfloat16
        want_y = torch.float32 if self.out == "f32" else torch.bfloat16
        if x.dtype != want_x or y.dtype != want_y:
            raise TypeError("dtype mismatch: x %s, y %s" % (x.dtype, y.dtype))
        if w_table.dtype != torch.int64 or offsets.dtype != torch.int32 or offsets.numel() != E + 1:
            raise TypeError("w_table must be int64 [E], offsets int32 [E + 1]")
        if x.numel() < T * self.K or y.numel() < T * self.out_cols:
            raise ValueError("x or y too small")
        init_device(x.device)
        _check(lib().qgemm_run_grouped(self._h, E, T, _dev_ptr(w_table, "w_table"),
                                       _dev_ptr(offsets, "offsets"), _dev_ptr(x, "x"),
                                       _dev_ptr(y, "y"), _stream_ptr(stream)))
        return y

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().qgemm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dequantize(fmt: str, w, N: int, K: int, stream=None):
    """Device decode of a packed buffer -> torch float32 [N][K] on the same device."""
    import torch

    out = torch.empty((N, K), dtype=torch.float32, device=w.device)
    _check(lib().qgemm_dequantize(FORMATS[fmt], _dev_ptr(w, "w"), _dev_ptr(out, "out"), N, K,
                                  _stream_ptr(stream)))
    return out


def read_bytes(buf, sink, wgs: int = 0, nbytes: int | None = None, stream=None):
    """qgemm_read_bytes: a plain 16-byte-load read of a device buffer (the
    achieved-bandwidth ceiling of the weight stream); sink: int32 tensor of
    at least wgs (default 2048) elements on the same device."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if sink.numel() < (wgs or 2048):
        raise ValueError("sink too small")
    _check(lib().qgemm_read_bytes(_dev_ptr(buf, "buf"), n, _dev_ptr(sink, "sink"), wgs,
                                  _stream_ptr(stream)))


MFMA_RATE_MODES = {0: ("bf16 16x16x32", 32), 1: ("i8 16x16x32", 32), 2: ("i8 16x16x64", 64),
                   3: ("i8 16x16x32 + per-32 scale (int8 tier loop)", 32),
                   4: ("bf16 16x16x32 + per-32 scale FMA", 32),
                   5: ("scaled 16x16x128 e4m3 x e2m1", 128), 6: ("scaled 16x16x128 e2m1 x e2m1", 128),
                   7: ("scaled 16x16x128 e4m3 x e4m3", 128)}


def mfma_rate(mode: int, iters: int, sink, stream=None):
    """qgemm_mfma_rate: one launch of the matrix-core loop `mode` (see
    MFMA_RATE_MODES: name, K per MFMA); sink: int32 tensor of 4096 elements."""
    if sink.numel() < 4096:
        raise ValueError("sink too small")
    _check(lib().qgemm_mfma_rate(mode, iters, _dev_ptr(sink, "sink"), _stream_ptr(stream)))


def xcd_local() -> int:
    """Dispatch probe outcome on the current device (see qgemm_xcd_local):
    1 XCD-local K-split exchange, 0 device-coherent, -1 not initialised."""
    return int(lib().qgemm_xcd_local())


def version() -> tuple:
    v = lib().qgemm_version()
    return (v >> 16, v & 0xFFFF)
