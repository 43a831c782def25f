"""FP8 table generator: a GPU filler for HBM and a CPU row rebuilder.

Both implement the same counter-based recipe (Philox4x64-10, see
csrc/tablegen_host.c), so the CPU side can rebuild any row the GPU wrote.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import inputs

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libplegen_host.so")
HIP_LIB = os.path.join(_HERE, "libplegen_hip.so")

_host = None
_hip = None
_thr = None


def thresholds() -> np.ndarray:
    global _thr
    if _thr is None:
        _thr = inputs.e4m3_magnitude_thresholds()
    return _thr


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.gen_table_rows.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.c_void_p]
        lib.gen_table_rows.restype = None
        lib.gen_philox4x64_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.gen_philox4x64_10.restype = None
        lib.gen_table_span.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.gen_table_span.restype = None
        lib.gen_table_slices.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.gen_table_slices.restype = None
        lib.gen_scales.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32,
                                   ctypes.c_uint32, ctypes.c_void_p]
        lib.gen_scales.restype = None
        lib.gen_nvfp4_rows.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        lib.gen_nvfp4_rows.restype = None
        _host = lib
    return _host


def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint64))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64))
    o = np.zeros(4, dtype=np.uint64)
    _host_lib().gen_philox4x64_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


def rows_cpu(ids, seed: int = inputs.TABLE_SEED):
    """Rebuild table rows `ids` on the CPU: (codes uint8[n][2560], scales float32[n])."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int64).reshape(-1))
    n = len(ids)
    rows = np.empty((n, inputs.D), dtype=np.uint8)
    scales = np.empty(n, dtype=np.float32)
    thr = np.ascontiguousarray(thresholds())
    if n:
        _host_lib().gen_table_rows(seed, ids.ctypes.data, n, thr.ctypes.data,
                                   inputs.SCALE_M_LO, inputs.SCALE_M_SPAN,
                                   rows.ctypes.data, scales.ctypes.data)
    return rows, scales


HEADS = 16
SLICE = inputs.D // HEADS   # 160 bytes per head-table row


def slices_cpu(heads, ids, R: int, seed: int = inputs.TABLE_SEED):
    """Rows `ids` of head tables `heads` in the 16 x [R][160] view of the same
    table bytes: (codes uint8[n][160], scales float32[n]); element g =
    (h R + r) 160 + j, scale number h R + r."""
    heads = np.asarray(heads, dtype=np.int64).reshape(-1)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    n = len(ids)
    codes = np.empty((n, SLICE), dtype=np.uint8)
    q = np.ascontiguousarray(heads * R + ids)
    thr = np.ascontiguousarray(thresholds())
    lib = _host_lib()
    if n:
        lib.gen_table_slices(seed, q.ctypes.data, n, thr.ctypes.data, codes.ctypes.data)
    scales = np.empty(n, dtype=np.float32)
    if n:
        lib.gen_scales(seed, q.ctypes.data, n, inputs.SCALE_M_LO, inputs.SCALE_M_SPAN, scales.ctypes.data)
    return codes, scales


def nvfp4_rows_cpu(ids, seed: int = inputs.TABLE_SEED):
    """Rows `ids` of the NVFP4 table: (codes uint8[n][1280] packed E2M1, low
    nibble first; blocks uint8[n][160] E4M3 scale per 16 elements; scales
    float32[n], the fp32 row scales)."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int64).reshape(-1))
    n = len(ids)
    codes = np.empty((n, inputs.D // 2), dtype=np.uint8)
    blocks = np.empty((n, inputs.D // 16), dtype=np.uint8)
    thr = np.ascontiguousarray(inputs.e2m1_magnitude_thresholds())
    lib = _host_lib()
    if n:
        lib.gen_nvfp4_rows(seed, ids.ctypes.data, n, thr.ctypes.data, inputs.NVFP4_BLOCK_CODE_LO,
                           inputs.NVFP4_BLOCK_CODES, codes.ctypes.data, blocks.ctypes.data)
    scales = np.empty(n, dtype=np.float32)
    if n:
        lib.gen_scales(seed, ids.ctypes.data, n, inputs.SCALE_M_LO, inputs.SCALE_M_SPAN, scales.ctypes.data)
    return codes, blocks, scales


def _hip_lib():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (torch's HIP runtime must be the one loaded)
        if not os.path.exists(HIP_LIB):
            raise RuntimeError(f"{HIP_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HIP_LIB)
        lib.gen_fill_table.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_void_p]
        lib.gen_fill_table.restype = ctypes.c_int
        lib.gen_fill_scales.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_void_p]
        lib.gen_fill_scales.restype = ctypes.c_int
        lib.gen_fill_nvfp4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        lib.gen_fill_nvfp4.restype = ctypes.c_int
        _hip = lib
    return _hip


def table_gpu(R: int, seed: int = inputs.TABLE_SEED, device="cuda"):
    """Allocate and fill (codes uint8[R][2560], scales float32[R]) on the GPU."""
    import torch
    table = torch.empty((R, inputs.D), dtype=torch.uint8, device=device)
    scales = torch.empty((R,), dtype=torch.float32, device=device)
    thr = torch.from_numpy(thresholds().astype(np.int64)).to(torch.int32).to(device)
    stream = torch.cuda.current_stream(table.device).cuda_stream
    rc = _hip_lib().gen_fill_table(table.data_ptr(), scales.data_ptr(), R, seed, thr.data_ptr(),
                                   inputs.SCALE_M_LO, inputs.SCALE_M_SPAN, stream)
    if rc != 0:
        raise RuntimeError(f"gen_fill_table failed: {rc}")
    torch.cuda.current_stream(table.device).synchronize()
    del thr
    return table, scales


def head_scales_gpu(R: int, seed: int = inputs.TABLE_SEED, device="cuda"):
    """The 16 R row scales of the 16 x [R][160] head view, float32 [16][R], on the GPU."""
    import torch
    scales = torch.empty((HEADS, R), dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream(scales.device).cuda_stream
    rc = _hip_lib().gen_fill_scales(scales.data_ptr(), HEADS * R, seed, inputs.SCALE_M_LO,
                                    inputs.SCALE_M_SPAN, stream)
    if rc != 0:
        raise RuntimeError(f"gen_fill_scales failed: {rc}")
    torch.cuda.current_stream(scales.device).synchronize()
    return scales


def nvfp4_gpu(R: int, seed: int = inputs.TABLE_SEED, device="cuda"):
    """The NVFP4 table on the GPU: codes uint8 [R][1280], blocks uint8
    [R][160], row scales float32 [R]."""
    import torch
    codes = torch.empty((R, inputs.D // 2), dtype=torch.uint8, device=device)
    blocks = torch.empty((R, inputs.D // 16), dtype=torch.uint8, device=device)
    scales = torch.empty((R,), dtype=torch.float32, device=device)
    thr = torch.from_numpy(inputs.e2m1_magnitude_thresholds().astype(np.int64)).to(torch.int32).to(device)
    stream = torch.cuda.current_stream(codes.device).cuda_stream
    rc = _hip_lib().gen_fill_nvfp4(codes.data_ptr(), blocks.data_ptr(), R, seed, thr.data_ptr(),
                                   inputs.NVFP4_BLOCK_CODE_LO, inputs.NVFP4_BLOCK_CODES, stream)
    if rc != 0:
        raise RuntimeError(f"gen_fill_nvfp4 failed: {rc}")
    rc = _hip_lib().gen_fill_scales(scales.data_ptr(), R, seed, inputs.SCALE_M_LO, inputs.SCALE_M_SPAN, stream)
    if rc != 0:
        raise RuntimeError(f"gen_fill_scales failed: {rc}")
    torch.cuda.current_stream(codes.device).synchronize()
    del thr
    return codes, blocks, scales
