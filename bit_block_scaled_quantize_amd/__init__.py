"""Thin Python binding of libnvfp4 (include/nvfp4.h): NVFP4 quantization and block-scaled
GEMMs on MI355X.

Every function marshals torch tensors (device memory, current stream) into the C ABI and
returns; all arithmetic runs in the HIP kernels. If the library is not built the import
still succeeds but every call raises, so nothing can silently fall back to another path.

Names follow the C entry points: quantize, quantize_noalloc, rht_quantize, rht_rows_quantize,
gemm, gemm_ex, grouped_gemm, grouped_gemm_k, amax, amax_pair, mx_quantize, mx_quantize_columns, mx_gemm, dequantize.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

NVFP4_OK = 0
_STATUS = {-1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "HIP error"}
_DTYPE = {torch.bfloat16: 0, torch.float32: 1}
_BLOCK = {"1x16": 0, "16x16": 1}
_ROUND = {"rn": 0, "sr": 1}
OP_QUANTIZE, OP_RHT_QUANTIZE, OP_GEMM, OP_GROUPED_GEMM, OP_AMAX_PAIR, OP_GEMM_EX = 0, 1, 2, 3, 4, 5
OUT_FP32, OUT_FP32_ACCUMULATE, OUT_BF16 = 0, 1, 2

EXPORTED = ("nvfp4_quantize", "nvfp4_quantize_noalloc", "nvfp4_rht_quantize", "nvfp4_gemm", "nvfp4_gemm_ex", "nvfp4_grouped_gemm",
            "mxfp4_quantize", "mxfp4_quantize_columns", "mxfp4_gemm", "nvfp4_rht_rows_quantize",
            "nvfp4_grouped_gemm_k",
            "nvfp4_amax", "nvfp4_amax_pair", "nvfp4_workspace_size", "nvfp4_last_error",
            "nvfp4_dequantize")


class NVFP4Error(RuntimeError):
    pass


class _CTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class _CMXTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NVFP4Error(f"{LIB_PATH} is not built; run bit_block_scaled_quantize_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, u64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    pt = ctypes.POINTER(_CTensor)
    lib.nvfp4_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                   u64, u64, vp, i64, vp, pt, pt, vp, sz, vp]
    lib.nvfp4_quantize_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                           u64, u64, vp, i64, vp, pt, pt, vp]
    lib.nvfp4_rht_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_uint16,
                                       ctypes.c_int, u64, u64, vp, i64, vp, pt, vp, sz, vp]
    lib.nvfp4_gemm.argtypes = [pt, pt, vp, i64, vp]
    mpt = ctypes.POINTER(_CMXTensor)
    lib.mxfp4_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, u64, u64, mpt, vp]
    lib.mxfp4_quantize_columns.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, u64, u64, mpt, vp]
    lib.mxfp4_gemm.argtypes = [mpt, mpt, vp, i64, vp]
    lib.nvfp4_rht_rows_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_uint16, ctypes.c_int,
                                            u64, u64, vp, pt, vp, sz, vp]
    lib.nvfp4_gemm_ex.argtypes = [pt, pt, vp, i64, ctypes.c_int, vp, vp, sz, vp]
    lib.nvfp4_grouped_gemm.argtypes = [i64, vp, pt, pt, i64, vp, i64, vp, sz, vp]
    lib.nvfp4_grouped_gemm_k.argtypes = [i64, vp, pt, pt, vp, i64, vp]
    lib.nvfp4_amax.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, ctypes.c_int,
                               ctypes.c_uint16, vp, vp, sz, vp]
    lib.nvfp4_amax_pair.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_uint16, vp, vp, sz, vp]
    lib.nvfp4_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.nvfp4_workspace_size.restype = sz
    lib.nvfp4_last_error.restype = ctypes.c_char_p
    lib.nvfp4_dequantize.argtypes = [pt, vp, i64, vp, vp]
    for name in EXPORTED:
        if name not in ("nvfp4_workspace_size", "nvfp4_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises NVFP4Error if it is not built)."""
    return _load()


def _check(status: int):
    if status != NVFP4_OK:
        msg = _load().nvfp4_last_error().decode()
        raise NVFP4Error(f"{_STATUS.get(status, status)}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Runs a binding function with its `stream` argument (when given) as torch's current
    stream, so every workspace and default output it allocates belongs to the stream its
    kernels are enqueued on. torch's caching allocator hands a freed block out again only to
    work on the stream it belongs to, so a workspace freed when the function returns cannot be
    given to other work while these kernels may still be using it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


@dataclass
class NVFP4Tensor:
    """Device buffers of one NVFP4 tensor [rows, cols] quantized along cols."""
    codes: torch.Tensor         # uint8 [rows, cols/2]
    scales: torch.Tensor        # uint8 [rows, cols/16] (E4M3 codes)
    global_scale: torch.Tensor  # float32 [nseg]
    rows: int
    cols: int

    @classmethod
    def empty(cls, rows: int, cols: int, nseg: int = 1, device="cuda"):
        return cls(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                   torch.empty((rows, cols // 16), dtype=torch.uint8, device=device),
                   torch.empty((nseg,), dtype=torch.float32, device=device), rows, cols)

    def c(self) -> _CTensor:
        return _CTensor(self.codes.data_ptr(), self.scales.data_ptr(),
                        self.global_scale.data_ptr(), self.rows, self.cols)


@dataclass
class MXFP4Tensor:
    """Device buffers of one MXFP4 tensor [rows, cols] quantized along cols. The E8M0 scales
    are stored K step by K step: [ceil(cols/128), rows, 4], scale j of row r at [j // 4, r,
    j % 4] (one 128-element step's scales of all rows contiguous, as the GEMM reads them)."""
    codes: torch.Tensor         # uint8 [rows, cols/2]
    scales: torch.Tensor        # uint8 [ceil(cols/128), rows, 4] (E8M0 codes)
    rows: int
    cols: int

    @classmethod
    def empty(cls, rows: int, cols: int, device="cuda"):
        return cls(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                   torch.empty(((cols + 127) // 128, rows, 4), dtype=torch.uint8, device=device), rows, cols)

    def scales_by_row(self) -> torch.Tensor:
        """The scales as [rows, cols/32] (row r's j-th scale at [r, j]), a copy."""
        steps = (self.cols + 127) // 128
        s = self.scales.reshape(steps, self.rows, 4).permute(1, 0, 2).reshape(self.rows, steps * 4)
        return s[:, : self.cols // 32].contiguous()

    def c(self) -> _CMXTensor:
        return _CMXTensor(self.codes.data_ptr(), self.scales.data_ptr(), self.rows, self.cols)


def _input(x: torch.Tensor):
    if x.dtype not in _DTYPE:
        raise NVFP4Error(f"unsupported input dtype {x.dtype}")
    if x.dim() != 2 or x.stride(1) != 1 or x.device.type != "cuda":
        raise NVFP4Error("input must be a 2-D GPU tensor with unit column stride")
    return _DTYPE[x.dtype], x.shape[0], x.shape[1], x.stride(0)


def _check_q(q, nseg: int = 1, what: str = "tensor"):
    """The C ABI sees only pointers: make sure the torch buffers behind an NVFP4/MXFP4 tensor
    are as large as its rows and cols say (and contiguous), so no kernel writes past them."""
    mx = isinstance(q, MXFP4Tensor)
    need = ((q.codes, q.rows * (q.cols // 2)),
            (q.scales, q.rows * 4 * ((q.cols + 127) // 128) if mx else q.rows * (q.cols // 16)))
    if not mx:
        need += ((q.global_scale, nseg),)
    for t, n in need:
        if t.numel() < n or not t.is_contiguous() or t.device.type != "cuda":
            raise NVFP4Error(f"{what}: buffer of {t.numel()} elements (contiguous, on the GPU) needed {n}")


def _check_out(out: torch.Tensor, rows: int, cols: int, dtype, what: str = "out"):
    """A 2-D output with at least rows x cols elements, unit column stride, the given dtype."""
    if out.dtype != dtype or out.dim() != 2 or out.stride(1) != 1 or out.device.type != "cuda":
        raise NVFP4Error(f"{what} must be a 2-D {dtype} GPU tensor with unit column stride")
    if out.shape[0] < rows or out.shape[1] < cols:
        raise NVFP4Error(f"{what} shape {tuple(out.shape)} smaller than ({rows}, {cols})")


def _check_table(t, what: str):
    """Segment / offset tables are int64 GPU tensors with at least two entries."""
    if t is not None and (t.dtype != torch.int64 or t.device.type != "cuda" or t.numel() < 2
                          or not t.is_contiguous()):
        raise NVFP4Error(f"{what} must be a contiguous int64 GPU tensor of at least 2 entries")


def _check_vec(t, n: int, what: str):
    if t is not None and (t.dtype != torch.float32 or t.numel() < n or t.device.type != "cuda"
                          or not t.is_contiguous()):
        raise NVFP4Error(f"{what} must be a contiguous float32 GPU tensor of at least {n} elements")


def workspace_size(op: int, rows: int, cols: int, nseg: int = 1) -> int:
    return int(_load().nvfp4_workspace_size(op, rows, cols, nseg))


def _workspace(op, rows, cols, nseg, device):
    n = workspace_size(op, rows, cols, nseg)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=device), n


@_on_stream
def quantize(x: torch.Tensor, block: str = "1x16", rounding: str = "rn", seed: int = 0,
             offset: int = 0, segments: torch.Tensor | None = None, amax: torch.Tensor | None = None,
             emit_transposed: bool = False, out: NVFP4Tensor | None = None,
             out_t: NVFP4Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """nvfp4_quantize. Returns (q, q_t) where q_t is None unless emit_transposed."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    nseg = 1 if segments is None else segments.numel() - 1
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, nseg, x.device)
    if emit_transposed and out_t is None:
        # a segmented stack of nseg equal blocks: each block's transpose, stacked
        out_t = (NVFP4Tensor.empty(cols, rows, 1, x.device) if segments is None
                 else NVFP4Tensor.empty(nseg * cols, rows // nseg, nseg, x.device))
    ws_n = 0
    if amax is None:
        if workspace is None:
            workspace, ws_n = _workspace(OP_QUANTIZE, rows, cols, nseg, x.device)
        else:
            ws_n = workspace.numel()
    _check_table(segments, "segments")
    _check_vec(amax, nseg, "amax")
    _check_q(out, nseg, "out")
    if emit_transposed:
        _check_q(out_t, nseg if segments is not None else 1, "out_t")
    oc = out.c()
    otc = out_t.c() if emit_transposed else None
    st = lib.nvfp4_quantize(_ptr(x), dt, rows, cols, ld, _BLOCK[block], _ROUND[rounding],
                            seed & (2 ** 64 - 1), offset & (2 ** 64 - 1), _ptr(segments), nseg,
                            _ptr(amax), ctypes.byref(oc),
                            ctypes.byref(otc) if otc is not None else None,
                            _ptr(workspace) if amax is None else None, ws_n, _stream(stream))
    _check(st)
    return out, (out_t if emit_transposed else None)


@_on_stream
def quantize_noalloc(x: torch.Tensor, block: str = "1x16", rounding: str = "rn", seed: int = 0,
                     offset: int = 0, segments: torch.Tensor | None = None, amax: torch.Tensor | None = None,
                     emit_transposed: bool = False, out: NVFP4Tensor | None = None,
                     out_t: NVFP4Tensor | None = None, stream=None):
    """nvfp4_quantize_noalloc: nvfp4_quantize without a workspace (the library's static device
    array holds the amax partials). With `out` (and `out_t` when emit_transposed) given, this
    allocates nothing; calls overlapping on one device race. Returns (q, q_t)."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    nseg = 1 if segments is None else segments.numel() - 1
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, nseg, x.device)
    if emit_transposed and out_t is None:
        out_t = (NVFP4Tensor.empty(cols, rows, 1, x.device) if segments is None
                 else NVFP4Tensor.empty(nseg * cols, rows // nseg, nseg, x.device))
    _check_table(segments, "segments")
    _check_vec(amax, nseg, "amax")
    _check_q(out, nseg, "out")
    if emit_transposed:
        _check_q(out_t, nseg if segments is not None else 1, "out_t")
    oc = out.c()
    otc = out_t.c() if emit_transposed else None
    st = lib.nvfp4_quantize_noalloc(_ptr(x), dt, rows, cols, ld, _BLOCK[block], _ROUND[rounding],
                                    seed & (2 ** 64 - 1), offset & (2 ** 64 - 1), _ptr(segments), nseg,
                                    _ptr(amax), ctypes.byref(oc),
                                    ctypes.byref(otc) if otc is not None else None, _stream(stream))
    _check(st)
    return out, (out_t if emit_transposed else None)


@_on_stream
def rht_rows_quantize(x: torch.Tensor, sign_mask: int, rounding: str = "rn", seed: int = 0,
                      offset: int = 0, amax: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_rht_rows_quantize: each row's 16-blocks through the random-sign Hadamard
    transform, then 1x16 quantization along the rows (same shape as x)."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    if out is None:
        out = NVFP4Tensor.empty(rows, cols, 1, x.device)
    ws_n = 0
    if amax is None:
        if workspace is None:
            workspace, ws_n = _workspace(OP_QUANTIZE, rows, cols, 1, x.device)
        else:
            ws_n = workspace.numel()
    _check_vec(amax, 1, "amax")
    _check_q(out, 1, "out")
    oc = out.c()
    _check(lib.nvfp4_rht_rows_quantize(_ptr(x), dt, rows, cols, ld, sign_mask & 0xFFFF, _ROUND[rounding],
                                       seed & (2 ** 64 - 1), offset & (2 ** 64 - 1), _ptr(amax),
                                       ctypes.byref(oc), _ptr(workspace) if amax is None else None, ws_n,
                                       _stream(stream)))
    return out


@_on_stream
def mx_quantize(x: torch.Tensor, rounding: str = "rn", seed: int = 0, offset: int = 0,
                out: MXFP4Tensor | None = None, stream=None) -> MXFP4Tensor:
    """mxfp4_quantize: x[rows, cols] -> MXFP4 (E8M0 scale per 32 elements)."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    if out is None:
        out = MXFP4Tensor.empty(rows, cols, x.device)
    _check_q(out, what="out")
    oc = out.c()
    _check(lib.mxfp4_quantize(_ptr(x), dt, rows, cols, ld, _ROUND[rounding], seed & (2 ** 64 - 1),
                              offset & (2 ** 64 - 1), ctypes.byref(oc), _stream(stream)))
    return out


@_on_stream
def mx_quantize_columns(x: torch.Tensor, rounding: str = "rn", seed: int = 0, offset: int = 0,
                        out: MXFP4Tensor | None = None, stream=None) -> MXFP4Tensor:
    """mxfp4_quantize_columns: x[rows, cols] -> MXFP4 of x^T, [cols, rows] (E8M0 per 32 rows)."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    if out is None:
        out = MXFP4Tensor.empty(cols, rows, x.device)
    _check_q(out, what="out")
    oc = out.c()
    _check(lib.mxfp4_quantize_columns(_ptr(x), dt, rows, cols, ld, _ROUND[rounding], seed & (2 ** 64 - 1),
                                      offset & (2 ** 64 - 1), ctypes.byref(oc), _stream(stream)))
    return out


@_on_stream
def mx_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxfp4_gemm: D[M, N] = A[M, K] * B[N, K]^T (FP32) on the block-scaled FP4 matrix cores."""
    lib = _load()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.codes.device)
    _check_q(a, what="A")
    _check_q(b, what="B")
    _check_out(out, a.rows, b.rows, torch.float32)
    ac, bc = a.c(), b.c()
    _check(lib.mxfp4_gemm(ctypes.byref(ac), ctypes.byref(bc), _ptr(out), out.stride(0), _stream(stream)))
    return out


@_on_stream
def rht_quantize(x: torch.Tensor, sign_mask: int, rounding: str = "rn", seed: int = 0,
                 offset: int = 0, amax: torch.Tensor | None = None,
                 out: NVFP4Tensor | None = None, workspace: torch.Tensor | None = None,
                 segments: torch.Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_rht_quantize: x[tokens, cols] -> NVFP4 tensor [cols, tokens] (segments: token
    ranges with one global scale each)."""
    lib = _load()
    dt, tokens, cols, ld = _input(x)
    nseg = 1 if segments is None else segments.numel() - 1
    if out is None:
        out = NVFP4Tensor.empty(cols, tokens, nseg, x.device)
    ws_n = 0
    if amax is None:
        if workspace is None:
            workspace, ws_n = _workspace(OP_RHT_QUANTIZE, tokens, cols, nseg, x.device)
        else:
            ws_n = workspace.numel()
    _check_table(segments, "segments")
    _check_vec(amax, nseg, "amax")
    _check_q(out, nseg, "out")
    oc = out.c()
    st = lib.nvfp4_rht_quantize(_ptr(x), dt, tokens, cols, ld, sign_mask & 0xFFFF,
                                _ROUND[rounding], seed & (2 ** 64 - 1), offset & (2 ** 64 - 1),
                                _ptr(segments), nseg, _ptr(amax), ctypes.byref(oc),
                                _ptr(workspace) if amax is None else None, ws_n, _stream(stream))
    _check(st)
    return out


@_on_stream
def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_gemm: D[M, N] = A[M, K] * B[N, K]^T (FP32)."""
    lib = _load()
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.codes.device)
    _check_q(a, what="A")
    _check_q(b, what="B")
    _check_out(out, a.rows, b.rows, torch.float32)
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm(ctypes.byref(ac), ctypes.byref(bc), _ptr(out), out.stride(0),
                          _stream(stream)))
    return out


@_on_stream
def gemm_ex(a: NVFP4Tensor, b: NVFP4Tensor, out: torch.Tensor | None = None,
            out_dtype: torch.dtype = torch.float32, accumulate: bool = False,
            amax_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """nvfp4_gemm_ex: D = A * B^T stored as float32 or bfloat16, or (accumulate, float32) added
    to `out`; amax_out (float32 [1]) receives max |D| as stored."""
    lib = _load()
    if accumulate:
        if out is None or out.dtype != torch.float32:
            raise NVFP4Error("accumulate needs a float32 `out`")
        kind = OUT_FP32_ACCUMULATE
    else:
        kind = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_FP32
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise NVFP4Error(f"unsupported output dtype {out_dtype}")
        if out is None:
            out = torch.empty((a.rows, b.rows), dtype=out_dtype, device=a.codes.device)
        elif out.dtype != out_dtype:
            raise NVFP4Error("out dtype does not match out_dtype")
    _check_q(a, what="A")
    _check_q(b, what="B")
    _check_out(out, a.rows, b.rows, out.dtype)
    if amax_out is not None and (amax_out.numel() < 1 or amax_out.dtype != torch.float32):
        raise NVFP4Error("amax_out must be a float32 tensor of at least one element")
    if workspace is None:
        workspace, ws_n = _workspace(OP_GEMM_EX, a.rows, b.rows, 1, a.codes.device)
    else:
        ws_n = workspace.numel()
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm_ex(ctypes.byref(ac), ctypes.byref(bc), _ptr(out), out.stride(0), kind,
                             _ptr(amax_out), _ptr(workspace), ws_n, _stream(stream)))
    return out


@_on_stream
def grouped_gemm(m_offsets: torch.Tensor, a: NVFP4Tensor, b: NVFP4Tensor, n: int,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_grouped_gemm: per group g, rows m_offsets[g]:m_offsets[g+1] of A against rows
    g*n:(g+1)*n of B."""
    lib = _load()
    G = m_offsets.numel() - 1
    if out is None:
        out = torch.empty((a.rows, n), dtype=torch.float32, device=a.codes.device)
    _check_q(a, G, "A")
    _check_q(b, G, "B")
    _check_out(out, a.rows, n, torch.float32)
    if m_offsets.dtype != torch.int64 or m_offsets.device.type != "cuda":
        raise NVFP4Error("m_offsets must be an int64 GPU tensor")
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_grouped_gemm(G, _ptr(m_offsets), ctypes.byref(ac), ctypes.byref(bc), n,
                                  _ptr(out), out.stride(0), None, 0, _stream(stream)))
    return out


@_on_stream
def grouped_gemm_k(k_offsets: torch.Tensor, a: NVFP4Tensor, b: NVFP4Tensor,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_grouped_gemm_k: for each group g, columns k_offsets[g]:k_offsets[g+1] of A [M, K]
    and B [N, K] into rows g*M:(g+1)*M of D [G*M, N] (FP32)."""
    lib = _load()
    G = k_offsets.numel() - 1
    if out is None:
        out = torch.empty((G * a.rows, b.rows), dtype=torch.float32, device=a.codes.device)
    _check_q(a, G, "A")
    _check_q(b, G, "B")
    _check_out(out, G * a.rows, b.rows, torch.float32)
    if k_offsets.dtype != torch.int64 or k_offsets.device.type != "cuda":
        raise NVFP4Error("k_offsets must be an int64 GPU tensor")
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_grouped_gemm_k(G, _ptr(k_offsets), ctypes.byref(ac), ctypes.byref(bc),
                                    _ptr(out), out.stride(0), _stream(stream)))
    return out


@_on_stream
def amax(x: torch.Tensor, segments: torch.Tensor | None = None, rht: bool | int = False,
         sign_mask: int = 0, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """nvfp4_amax: max|x| per segment, or of the Hadamard-transformed tensor: rht = True (or 1)
    along tokens as rht_quantize, rht = 2 along each row as rht_rows_quantize."""
    lib = _load()
    dt, rows, cols, ld = _input(x)
    nseg = 1 if segments is None else segments.numel() - 1
    if out is None:
        out = torch.empty((nseg,), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace, ws_n = _workspace(OP_RHT_QUANTIZE if int(rht) == 1 else OP_QUANTIZE, rows, cols, nseg, x.device)
    else:
        ws_n = workspace.numel()
    _check_table(segments, "segments")
    _check_vec(out, nseg, "out")
    _check(lib.nvfp4_amax(_ptr(x), dt, rows, cols, ld, _ptr(segments), nseg, int(rht),
                          sign_mask & 0xFFFF, _ptr(out), _ptr(workspace), ws_n, _stream(stream)))
    return out


@_on_stream
def amax_pair(x: torch.Tensor, sign_mask: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_amax_pair: float32 [2] = (max|x|, max of the Hadamard-transformed tensor)."""
    lib = _load()
    dt, tokens, cols, ld = _input(x)
    if out is None:
        out = torch.empty((2,), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace, ws_n = _workspace(OP_AMAX_PAIR, tokens, cols, 1, x.device)
    else:
        ws_n = workspace.numel()
    _check_vec(out, 2, "out")
    _check(lib.nvfp4_amax_pair(_ptr(x), dt, tokens, cols, ld, sign_mask & 0xFFFF, _ptr(out),
                               _ptr(workspace), ws_n, _stream(stream)))
    return out


@_on_stream
def dequantize(q: NVFP4Tensor, segments: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """nvfp4_dequantize (test helper): FP32 [rows, cols]."""
    lib = _load()
    nseg = 1 if segments is None else segments.numel() - 1
    _check_table(segments, "segments")
    _check_q(q, nseg, "q")
    y = torch.empty((q.rows, q.cols), dtype=torch.float32, device=q.codes.device)
    qc = q.c()
    _check(lib.nvfp4_dequantize(ctypes.byref(qc), _ptr(segments), nseg, _ptr(y), _stream(stream)))
    return y
