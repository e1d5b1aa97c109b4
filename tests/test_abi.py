"""C-ABI checks that need no GPU: the built library loads, exports every entry point that
include/nvfp4.h declares, and rejects invalid arguments on the host with the documented
status codes before anything is enqueued (all cases below fail validation, so no HIP call
is made)."""
import ctypes
import os
import re

import pytest
import torch

import bit_block_scaled_quantize_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:nvfp4|mxfp4)_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv.LIB_PATH):
        pytest.skip("libnvfp4.so not built")
    return nv.library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(nv.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def _tensor(rows, cols, codes=FAKE, scales=FAKE, gs=FAKE):
    return nv._CTensor(codes, scales, gs, rows, cols)


def _q(lib, **kw):
    a = dict(x=FAKE, dt=0, rows=32, cols=64, ld=64, blk=0, rnd=0, seed=0, offset=0, seg=None,
             nseg=1, amax=None, out=_tensor(32, 64), out_t=None, ws=FAKE, ws_n=8192, stream=None)
    a.update(kw)
    out_t = ctypes.byref(a["out_t"]) if a["out_t"] is not None else None
    out = ctypes.byref(a["out"]) if a["out"] is not None else None
    return lib.nvfp4_quantize(a["x"], a["dt"], a["rows"], a["cols"], a["ld"], a["blk"], a["rnd"],
                              a["seed"], a["offset"], a["seg"], a["nseg"], a["amax"], out, out_t,
                              a["ws"], a["ws_n"], a["stream"])


def test_quantize_validation(lib):
    assert _q(lib, x=None) == INVALID
    assert b"x is NULL" in lib.nvfp4_last_error()
    assert _q(lib, cols=60, ld=64) == INVALID
    assert _q(lib, ld=32) == INVALID
    assert _q(lib, dt=7) == INVALID
    assert _q(lib, blk=5) == INVALID
    assert _q(lib, rnd=9) == INVALID
    assert _q(lib, blk=1, rows=24, out=_tensor(24, 64)) == INVALID         # 16x16 rows % 16
    assert _q(lib, nseg=3) == INVALID                                       # nseg without table
    assert _q(lib, nseg=0) == INVALID
    assert _q(lib, out_t=_tensor(64, 32)) == INVALID                        # out_t needs 16x16
    assert _q(lib, blk=1, rnd=1) == UNSUPPORTED                             # SR on weights
    assert _q(lib, blk=1, seg=FAKE, nseg=3, out_t=_tensor(192, 32)) == UNSUPPORTED  # 32 % 3
    assert _q(lib, blk=1, seg=FAKE, nseg=4, out_t=_tensor(256, 8)) == UNSUPPORTED   # 8 rows each
    assert _q(lib, blk=1, seg=FAKE, nseg=2, out_t=_tensor(64, 32)) == INVALID       # [2*64, 16]
    assert _q(lib, out=None) == INVALID
    assert _q(lib, out=_tensor(32, 48)) == INVALID                          # shape mismatch
    assert _q(lib, out=_tensor(32, 64, codes=None)) == INVALID
    assert _q(lib, blk=1, out_t=_tensor(32, 64)) == INVALID                 # out_t must be [cols, rows]
    assert _q(lib, ws=None) == WORKSPACE
    assert _q(lib, ws_n=4) == WORKSPACE
    assert _q(lib, ws=FAKE + 4) == WORKSPACE                                # misaligned
    assert _q(lib, x=FAKE + 2) == UNSUPPORTED                               # misaligned input
    assert _q(lib, ld=68, cols=64) == UNSUPPORTED                           # row stride not 16-byte


def _qn(lib, **kw):
    a = dict(x=FAKE, dt=0, rows=32, cols=64, ld=64, blk=0, rnd=0, seed=0, offset=0, seg=None,
             nseg=1, amax=None, out=_tensor(32, 64), out_t=None, stream=None)
    a.update(kw)
    out_t = ctypes.byref(a["out_t"]) if a["out_t"] is not None else None
    out = ctypes.byref(a["out"]) if a["out"] is not None else None
    return lib.nvfp4_quantize_noalloc(a["x"], a["dt"], a["rows"], a["cols"], a["ld"], a["blk"], a["rnd"],
                                      a["seed"], a["offset"], a["seg"], a["nseg"], a["amax"], out, out_t,
                                      a["stream"])


def test_quantize_noalloc_validation(lib):
    # the allocation-free form validates like nvfp4_quantize, before touching its device array
    assert _qn(lib, x=None) == INVALID
    assert _qn(lib, cols=60, ld=64) == INVALID
    assert _qn(lib, blk=1, rnd=1) == UNSUPPORTED
    assert _qn(lib, out=None) == INVALID
    assert _qn(lib, x=FAKE + 2) == UNSUPPORTED
    # more segments than its 64 KiB device array holds: a clear error, nothing enqueued
    assert _qn(lib, seg=FAKE, nseg=16385) == UNSUPPORTED
    assert b"at most 16384 segments" in lib.nvfp4_last_error()


def test_rht_validation(lib):
    out = _tensor(64, 32)
    f = lib.nvfp4_rht_quantize
    assert f(FAKE, 0, 30, 64, 64, 0, 0, 0, 0, None, 1, None, ctypes.byref(out), FAKE, 8192, None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 0, 3, 0, 0, None, 1, None, ctypes.byref(out), FAKE, 8192, None) == INVALID
    bad = _tensor(32, 64)                                                    # must be [cols, tokens]
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, 0, None, 1, None, ctypes.byref(bad), FAKE, 8192, None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, 0, None, 1, None, ctypes.byref(out), None, 0, None) == WORKSPACE
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, 0, None, 3, None, ctypes.byref(out), FAKE, 8192, None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, 0, FAKE, 0, None, ctypes.byref(out), FAKE, 8192, None) == INVALID


def test_amax_pair_validation(lib):
    f = lib.nvfp4_amax_pair
    assert f(None, 0, 32, 64, 64, 0, FAKE, FAKE, 8192, None) == INVALID
    assert f(FAKE, 0, 30, 64, 64, 0, FAKE, FAKE, 8192, None) == INVALID     # tokens % 16
    assert f(FAKE, 0, 32, 64, 64, 0, None, FAKE, 8192, None) == INVALID     # amax_out
    assert f(FAKE, 2, 32, 64, 64, 0, FAKE, FAKE, 8192, None) == INVALID     # dtype
    assert f(FAKE, 0, 32, 64, 60, 0, FAKE, FAKE, 8192, None) == INVALID     # ld < cols
    assert f(FAKE, 0, 32, 64, 64, 0, FAKE, None, 0, None) == WORKSPACE
    assert f(FAKE, 0, 32, 64, 64, 0, FAKE, FAKE, 4096, None) == WORKSPACE   # needs two arrays
    assert f(FAKE + 2, 0, 32, 64, 64, 0, FAKE, FAKE, 8192, None) == UNSUPPORTED


def test_gemm_validation(lib):
    a, b = _tensor(64, 128), _tensor(32, 128)
    g = lib.nvfp4_gemm
    assert g(None, ctypes.byref(b), FAKE, 32, None) == INVALID
    assert g(ctypes.byref(a), ctypes.byref(_tensor(32, 96)), FAKE, 32, None) == INVALID   # K
    assert g(ctypes.byref(a), ctypes.byref(b), None, 32, None) == INVALID
    assert g(ctypes.byref(a), ctypes.byref(b), FAKE, 16, None) == INVALID                # ldd
    assert g(ctypes.byref(_tensor(64, 100)), ctypes.byref(b), FAKE, 32, None) == INVALID  # K % 16
    gg = lib.nvfp4_grouped_gemm
    assert gg(0, FAKE, ctypes.byref(a), ctypes.byref(b), 32, FAKE, 32, None, 0, None) == INVALID
    assert gg(2, None, ctypes.byref(a), ctypes.byref(b), 16, FAKE, 16, None, 0, None) == INVALID
    assert gg(2, FAKE, ctypes.byref(a), ctypes.byref(b), 8, FAKE, 8, None, 0, None) == INVALID  # B rows


def test_gemm_operand_size_limit(lib):
    # 2^20 rows x 4096 codes bytes = 4 GiB: beyond the kernels' 32-bit buffer offsets
    a, b = _tensor(1 << 20, 8192), _tensor(32, 8192)
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), FAKE, 32, None) == UNSUPPORTED
    assert lib.nvfp4_gemm(ctypes.byref(b), ctypes.byref(a), FAKE, 1 << 20, None) == UNSUPPORTED
    assert lib.nvfp4_grouped_gemm_k(1, FAKE, ctypes.byref(a), ctypes.byref(b), FAKE, 32, None) == UNSUPPORTED


def test_gemm_ex_validation(lib):
    a, b = _tensor(64, 128), _tensor(32, 128)
    g = lib.nvfp4_gemm_ex
    A, B = ctypes.byref(a), ctypes.byref(b)
    assert g(None, B, FAKE, 32, 0, None, None, 0, None) == INVALID
    assert g(A, ctypes.byref(_tensor(32, 96)), FAKE, 32, 0, None, None, 0, None) == INVALID   # K
    assert g(A, B, None, 32, 0, None, None, 0, None) == INVALID                              # D
    assert g(A, B, FAKE, 16, 0, None, None, 0, None) == INVALID                              # ldd
    assert g(A, B, FAKE, 32, 3, None, None, 0, None) == INVALID                              # kind
    assert g(A, B, FAKE + 2, 32, 0, None, None, 0, None) == INVALID                          # FP32 align
    assert g(A, B, FAKE + 1, 32, 2, None, None, 0, None) == INVALID                          # BF16 align
    # a partial last round needs the split workspace: 640 tiles of 256 x 256 on 256 CUs
    big_a, big_b = _tensor(8192, 128), _tensor(5120, 128)
    need = lib.nvfp4_workspace_size(nv.OP_GEMM_EX, 8192, 5120, 1)
    assert need > 0
    assert g(ctypes.byref(big_a), ctypes.byref(big_b), FAKE, 5120, 2, None, None, 0, None) == WORKSPACE
    assert g(ctypes.byref(big_a), ctypes.byref(big_b), FAKE, 5120, 2, None, FAKE, need - 256, None) == WORKSPACE
    assert g(ctypes.byref(big_a), ctypes.byref(big_b), FAKE, 5120, 2, None, FAKE + 16, need, None) == INVALID


def test_grouped_gemm_k_validation(lib):
    a, b = _tensor(64, 128), _tensor(32, 128)
    f = lib.nvfp4_grouped_gemm_k
    assert f(0, FAKE, ctypes.byref(a), ctypes.byref(b), FAKE, 32, None) == INVALID          # G
    assert f(2, None, ctypes.byref(a), ctypes.byref(b), FAKE, 32, None) == INVALID          # offsets
    assert f(2, FAKE, ctypes.byref(a), ctypes.byref(_tensor(32, 96)), FAKE, 32, None) == INVALID
    assert f(2, FAKE, ctypes.byref(a), ctypes.byref(b), None, 32, None) == INVALID          # D
    assert f(2, FAKE, ctypes.byref(a), ctypes.byref(b), FAKE, 16, None) == INVALID          # ldd
    assert f(2, FAKE, ctypes.byref(_tensor(64, 96)), ctypes.byref(_tensor(32, 96)), FAKE, 32,
             None) == UNSUPPORTED                                                         # K % 64


def test_workspace_sizes(lib):
    assert lib.nvfp4_workspace_size(nv.OP_QUANTIZE, 10, 16, 1) == 4096      # 1024 partial maxima
    assert lib.nvfp4_workspace_size(nv.OP_QUANTIZE, 10, 16, 2000) == 8192   # one slot per segment
    assert lib.nvfp4_workspace_size(nv.OP_RHT_QUANTIZE, 16, 16, 1) == 4096
    assert lib.nvfp4_workspace_size(nv.OP_RHT_QUANTIZE, 16, 16, 3000) == 12032   # one per segment
    assert lib.nvfp4_workspace_size(nv.OP_AMAX_PAIR, 16, 16, 1) == 8192
    assert lib.nvfp4_workspace_size(nv.OP_GEMM, 16, 16, 1) == 0
    assert lib.nvfp4_workspace_size(nv.OP_GROUPED_GEMM, 16, 16, 1) == 0
    # K-split partial round of the linear-layer GEMM: two 256 x 256 FP32 partial tiles per
    # split tile (sizes for 256 compute units, the count assumed without a device)
    assert lib.nvfp4_workspace_size(nv.OP_GEMM_EX, 8192, 20480, 1) == 0          # 10 whole rounds
    assert lib.nvfp4_workspace_size(nv.OP_GEMM_EX, 8192, 5120, 1) == 128 * 2 * 256 * 256 * 4
    # 64 tiles left over (a quarter of the units or fewer): each becomes four 256 x 64 column
    # tiles over all of K, with no partial tiles to park
    assert lib.nvfp4_workspace_size(nv.OP_GEMM_EX, 20480, 5120, 1) == 0
    assert lib.nvfp4_workspace_size(nv.OP_GEMM_EX, 256 * 200, 256, 1) == 0       # 200 > 128 left over


def test_python_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(nv, "_lib", None)
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(nv.NVFP4Error):
        nv.library()


def test_product_package_does_not_import_oracle():
    pkg = os.path.dirname(nv.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f


def test_mx_quantize_validation(lib):
    f = lib.mxfp4_quantize
    out = nv._CMXTensor(FAKE, FAKE, 32, 64)
    o = ctypes.byref(out)
    assert f(None, 0, 32, 64, 64, 0, 0, 0, o, None) == INVALID                  # x
    assert f(FAKE, 0, 32, 48, 48, 0, 0, 0, ctypes.byref(nv._CMXTensor(FAKE, FAKE, 32, 48)), None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 2, 0, 0, o, None) == INVALID                  # rounding
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, None, None) == INVALID               # out
    assert f(FAKE, 0, 16, 64, 64, 0, 0, 0, o, None) == INVALID                  # shape
    assert f(FAKE + 2, 0, 32, 64, 64, 0, 0, 0, o, None) == UNSUPPORTED          # alignment


def test_mx_quantize_columns_validation(lib):
    f = lib.mxfp4_quantize_columns
    out = nv._CMXTensor(FAKE, FAKE, 64, 32)                                      # [cols, rows]
    o = ctypes.byref(out)
    assert f(None, 0, 32, 64, 64, 0, 0, 0, o, None) == INVALID                  # x
    assert f(FAKE, 0, 48, 64, 64, 0, 0, 0, ctypes.byref(nv._CMXTensor(FAKE, FAKE, 64, 48)), None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 2, 0, 0, o, None) == INVALID                  # rounding
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, None, None) == INVALID               # out
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, ctypes.byref(nv._CMXTensor(FAKE, FAKE, 32, 64)), None) == INVALID
    assert f(FAKE, 0, 32, 64, 64, 0, 0, 0, ctypes.byref(nv._CMXTensor(FAKE + 8, FAKE, 64, 32)), None) == INVALID
    assert f(FAKE + 2, 0, 32, 64, 64, 0, 0, 0, o, None) == UNSUPPORTED          # pair alignment


def test_binding_checks_buffers_before_calling(lib):
    # the C ABI sees only pointers: the binding refuses host tensors, short buffers and
    # outputs smaller than the result before anything reaches the library
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(torch.zeros((16, 32), dtype=torch.bfloat16))            # host input
    q = nv.NVFP4Tensor(torch.zeros(8, dtype=torch.uint8), torch.zeros(2, dtype=torch.uint8),
                       torch.ones(1), 16, 32)
    with pytest.raises(nv.NVFP4Error):
        nv._check_q(q, 1, "q")                                              # 8 < 16*16 codes
    with pytest.raises(nv.NVFP4Error):
        nv._check_out(torch.zeros((4, 8)), 4, 8, torch.float32)             # host output
    with pytest.raises(nv.NVFP4Error):
        nv._check_table(torch.zeros(3, dtype=torch.int32), "segments")      # not int64 / GPU
    with pytest.raises(nv.NVFP4Error):
        nv._check_vec(torch.zeros(1), 2, "amax")


def test_rht_rows_quantize_validation(lib):
    f = lib.nvfp4_rht_rows_quantize
    out = _tensor(32, 64)
    o = ctypes.byref(out)
    assert f(None, 0, 32, 64, 64, 0x6E04, 0, 0, 0, None, o, FAKE, 4096, None) == INVALID       # x
    assert f(FAKE, 0, 32, 40, 40, 0x6E04, 0, 0, 0, None, ctypes.byref(_tensor(32, 40)), FAKE, 4096,
             None) in (INVALID, UNSUPPORTED)                                                    # cols % 16
    assert f(FAKE, 0, 32, 64, 64, 0x6E04, 7, 0, 0, None, o, FAKE, 4096, None) == INVALID         # rounding
    assert f(FAKE, 0, 16, 64, 64, 0x6E04, 0, 0, 0, None, o, FAKE, 4096, None) == INVALID         # out shape
    assert f(FAKE, 0, 32, 64, 64, 0x6E04, 0, 0, 0, None, o, None, 0, None) == WORKSPACE         # no amax, no ws
    # nvfp4_amax with the rowwise selector takes no segments
    a = lib.nvfp4_amax
    assert a(FAKE, 0, 32, 64, 64, FAKE, 2, 2, 0x6E04, FAKE, None, 0, None) == UNSUPPORTED
    assert a(FAKE, 0, 32, 64, 64, None, 1, 3, 0x6E04, FAKE, FAKE, 4096, None) == INVALID         # selector
