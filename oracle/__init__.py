"""CPU oracle of the PLE n-gram embedding path — TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrapper around `ple_oracle.c` (plain C, fp64). Only the
tests, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may
import this package; the product path (`sparse_memory_gather_amd`) never
does and shares no source with it.

`forward()` strings the definition's steps together for one chunk of S
sequences: n-gram IDs -> gather/dequant -> projection (bf16 output) ->
gate -> causal short conv with carried state -> residual add. Table rows come from a
`row_source(ids) -> (codes uint8[n][2560], scales float32[n])` callable so
that a 51.2 GB table never has to be materialised on the host.

Parity status of each step (see the pins under tests/):
  ngram_ids, hist_update  pinned (SplitMix64 published vectors, key-field
                          decode, brute-force invariants)
  e4m3_value              pinned (all 256 codes vs torch.float8_e4m3fn)
  gather_dequant          pinned (raw bytes vs generator rows; rounding
                          properties against the exact rational sum)
  e2m1_value,             pinned (OCP MX v1.0 E2M1 table; the E2M1 grid
  gather_dequant_nvfp4    of the generator); x vs torch fp32 with nibble
                          order and block placement checked
  ngram_ids_heads,        pinned (SplitMix64 published stream for the head
  gather_dequant_heads    offsets; heads 0/8 equal the 2-lookup IDs; raw
                          bytes vs generator; torch fp32 product; placement)
  project                 pinned (numpy fp64 matmul; W = I)
  round_bf16              pinned (exact rational round-half-even; ties,
                          single rounding, subnormal step, overflow)
  gate                    pinned (closed forms e = +/-h, e = 0)
  conv_fuse               pinned (torch conv1d; impulse response; chunked
                          equals unchunked)
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

D = 2560
_HERE = os.path.dirname(os.path.abspath(__file__))
# PLE_ORACLE_LIB: another build of the same source (the sanitizer run loads
# the UBSan build through it)
LIB = os.environ.get("PLE_ORACLE_LIB") or os.path.join(_HERE, "libple_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        sig = {
            "oracle_num_threads": ([], ctypes.c_int),
            "oracle_set_num_threads": ([ctypes.c_int], None),
            "oracle_mix64": ([ctypes.c_uint64], ctypes.c_uint64),
            "oracle_key2": ([ctypes.c_uint32, ctypes.c_uint32], ctypes.c_uint64),
            "oracle_key3": ([ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32], ctypes.c_uint64),
            "oracle_ngram_ids": ([_P, _P, _I32, _P, _P, _I64, _P], None),
            "oracle_head_mix": ([ctypes.c_uint64, ctypes.c_int32], ctypes.c_uint64),
            "oracle_ngram_ids_heads": ([_P, _P, _I32, _P, _P, _I64, _P], None),
            "oracle_gather_dequant_heads": ([_P, _I64, _P, _P, _P, _P], None),
            "oracle_e2m1_value": ([ctypes.c_uint8], ctypes.c_double),
            "oracle_gather_dequant_nvfp4": ([_P, _I64, _P, _P, _P, _P, _P], None),
            "oracle_hist_update": ([_P, _P, _I32, _P, _P, _P, _P], None),
            "oracle_e4m3_value": ([ctypes.c_uint8], ctypes.c_double),
            "oracle_bf16_rne": ([ctypes.c_float], ctypes.c_uint16),
            "oracle_gather_dequant": ([_P, _I64, _P, _P, _P, _P], None),
            "oracle_project": ([_P, _I64, _P, _P], None),
            "oracle_round_bf16": ([_P, _I64, _P], None),
            "oracle_gate": ([_P, _P, _I64, ctypes.c_double, _P], None),
            "oracle_conv_fuse": ([_P, _P, _P, _I64, _P, _I32, _P, _P, _P, _P, _P], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _ptr(a):
    return a.ctypes.data if a is not None else None


# --- scalar helpers -------------------------------------------------------

def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls; results do not depend on it."""
    _load().oracle_set_num_threads(int(n))


def mix64(z: int) -> int:
    return int(_load().oracle_mix64(z & (2 ** 64 - 1)))


def key2(a: int, b: int) -> int:
    return int(_load().oracle_key2(a, b))


def key3(a: int, b: int, c: int) -> int:
    return int(_load().oracle_key3(a, b, c))


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(code))


def bf16_rne(f: float) -> int:
    return int(_load().oracle_bf16_rne(f))


# --- steps ------------------------------------------------------------------

def ngram_ids(tokens, cu_seqlens, hist_ids, hist_len, R: int) -> np.ndarray:
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    hist_ids = _c(hist_ids, np.int32).reshape(S, 2)
    hist_len = _c(hist_len, np.int32).reshape(S)
    out = np.full((len(tokens), 2), -7, dtype=np.int32)
    _load().oracle_ngram_ids(_ptr(tokens), _ptr(cu), S, _ptr(hist_ids), _ptr(hist_len), R, _ptr(out))
    return out


def head_mix(key: int, head: int) -> int:
    return int(_load().oracle_head_mix(key, head))


def ngram_ids_heads(tokens, cu_seqlens, hist_ids, hist_len, R: int) -> np.ndarray:
    """Row IDs [T][16] of the 16-lookup layout (R rows per head table)."""
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    hist_ids = _c(hist_ids, np.int32).reshape(S, 2)
    hist_len = _c(hist_len, np.int32).reshape(S)
    out = np.full((len(tokens), 16), -7, dtype=np.int32)
    _load().oracle_ngram_ids_heads(_ptr(tokens), _ptr(cu), S, _ptr(hist_ids), _ptr(hist_len), R, _ptr(out))
    return out


def hist_update(tokens, cu_seqlens, hist_ids, hist_len):
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    hist_ids = _c(hist_ids, np.int32).reshape(S, 2)
    hist_len = _c(hist_len, np.int32).reshape(S)
    hid = np.empty_like(hist_ids)
    hln = np.empty_like(hist_len)
    _load().oracle_hist_update(_ptr(tokens), _ptr(cu), S, _ptr(hist_ids), _ptr(hist_len),
                               _ptr(hid), _ptr(hln))
    return hid, hln


def gather_dequant(row_ids, table, scales, raw: bool = False):
    """x (bf16 bits [T][2560]) from rows of `table` (uint8[n][2560]) and
    `scales` (float32[n]); row_ids index into that table (-1 = missing)."""
    row_ids = _c(row_ids, np.int32).reshape(-1, 2)
    table = _c(table, np.uint8)
    scales = _c(scales, np.float32)
    T = row_ids.shape[0]
    x = np.empty((T, D), dtype=np.uint16)
    r = np.empty((T, 2, D), dtype=np.uint8) if raw else None
    _load().oracle_gather_dequant(_ptr(row_ids), T, _ptr(table), _ptr(scales), _ptr(x), _ptr(r))
    return (x, r) if raw else x


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(code))


def gather_dequant_nvfp4(row_ids, codes, blocks, scales, raw: bool = False):
    """x (bf16 bits [T][2560]) from NVFP4 rows: codes uint8[n][1280] (packed
    E2M1, low nibble first), blocks uint8[n][160] (E4M3 per 16 elements),
    scales float32[n]; row_ids [T][2] index them (-1 = missing)."""
    row_ids = _c(row_ids, np.int32).reshape(-1, 2)
    codes = _c(codes, np.uint8)
    blocks = _c(blocks, np.uint8)
    scales = _c(scales, np.float32)
    T = row_ids.shape[0]
    x = np.empty((T, D), dtype=np.uint16)
    r = np.empty((T, 2, D // 2), dtype=np.uint8) if raw else None
    _load().oracle_gather_dequant_nvfp4(_ptr(row_ids), T, _ptr(codes), _ptr(blocks), _ptr(scales), _ptr(x), _ptr(r))
    return (x, r) if raw else x


def gather_dequant_heads(idx, slices, scales, raw: bool = False):
    """x (bf16 bits [T][2560]) of the 16-lookup layout from 160-byte rows
    `slices` (uint8[n][160]) and `scales` (float32[n]); idx[t][h] indexes
    them (-1 = missing)."""
    idx = _c(idx, np.int32).reshape(-1, 16)
    slices = _c(slices, np.uint8)
    scales = _c(scales, np.float32)
    T = idx.shape[0]
    x = np.empty((T, D), dtype=np.uint16)
    r = np.empty((T, 16, 160), dtype=np.uint8) if raw else None
    _load().oracle_gather_dequant_heads(_ptr(idx), T, _ptr(slices), _ptr(scales), _ptr(x), _ptr(r))
    return (x, r) if raw else x


def project(x_bf16, W_bf16) -> np.ndarray:
    x = _c(x_bf16, np.uint16).reshape(-1, D)
    W = _c(W_bf16, np.uint16).reshape(D, D)
    e = np.empty((x.shape[0], D), dtype=np.float64)
    _load().oracle_project(_ptr(x), x.shape[0], _ptr(W), _ptr(e))
    return e


def round_bf16(a) -> np.ndarray:
    """Nearest bf16 value of each fp64 element (ties to even, one rounding),
    returned as fp64."""
    a = _c(a, np.float64)
    out = np.empty_like(a)
    _load().oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def gate(h_bf16, e, eps: float = 1e-6) -> np.ndarray:
    h = _c(h_bf16, np.uint16).reshape(-1, D)
    e = _c(e, np.float64).reshape(-1, D)
    g = np.empty(h.shape[0], dtype=np.float64)
    _load().oracle_gate(_ptr(h), _ptr(e), h.shape[0], eps, _ptr(g))
    return g


def conv_fuse(h_bf16, e, g, cu_seqlens, conv_w_bf16, state):
    h = _c(h_bf16, np.uint16).reshape(-1, D)
    e = _c(e, np.float64).reshape(-1, D)
    g = _c(g, np.float64)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    w = _c(conv_w_bf16, np.uint16).reshape(D, 4)
    st = _c(state, np.float64).reshape(S, 3, D)
    T = h.shape[0]
    y = np.empty((T, D), dtype=np.float64)
    out = np.empty((T, D), dtype=np.float64)
    st_out = np.empty_like(st)
    _load().oracle_conv_fuse(_ptr(h), _ptr(e), _ptr(g), T, _ptr(cu), S, _ptr(w), _ptr(st),
                             _ptr(y), _ptr(out), _ptr(st_out))
    return y, out, st_out


# --- whole chunk ------------------------------------------------------------

def forward(tokens, cu_seqlens, h_bf16, W_bf16, conv_w_bf16, R: int, row_source,
            hist_ids=None, hist_len=None, conv_state=None, eps: float = 1e-6):
    """One chunk through the whole path. Returns a dict with row_ids, x, e
    (the exact projection, fp64), e_b (its bf16 rounding: the projection's
    output tensor, which the gate and the conv consume; outside the routed
    experts the model's weights are BF16, bittide model card copy,
    "模型简介"), g, y, out (fp64,
    unrounded), and the new hist_ids / hist_len / conv_state (conv_state kept
    in fp64 so chained chunks equal one long chunk)."""
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    if hist_ids is None:
        hist_ids = np.zeros((S, 2), np.int32)
    if hist_len is None:
        hist_len = np.zeros(S, np.int32)
    if conv_state is None:
        conv_state = np.zeros((S, 3, D), np.float64)
    row_ids = ngram_ids(tokens, cu, hist_ids, hist_len, R)
    valid = row_ids[row_ids >= 0]
    uniq, inv = np.unique(valid, return_inverse=True)
    codes, scales = row_source(uniq)
    compact = np.full(row_ids.shape, -1, dtype=np.int32)
    compact[row_ids >= 0] = inv.astype(np.int32)
    x = gather_dequant(compact, codes, scales)
    e = project(x, W_bf16)
    e_b = round_bf16(e)
    g = gate(h_bf16, e_b, eps)
    y, out, st = conv_fuse(h_bf16, e_b, g, cu, conv_w_bf16, conv_state)
    hid, hln = hist_update(tokens, cu, hist_ids, hist_len)
    return dict(row_ids=row_ids, x=x, e=e, e_b=e_b, g=g, y=y, out=out,
                hist_ids=hid, hist_len=hln, conv_state=st)


def forward_nvfp4(tokens, cu_seqlens, h_bf16, W_bf16, conv_w_bf16, R: int, row_source,
                  hist_ids=None, hist_len=None, conv_state=None, eps: float = 1e-6):
    """forward() over the NVFP4 table: rows from row_source(ids) -> (codes
    uint8[n][1280], blocks uint8[n][160], scales float32[n]); IDs, projection,
    gate, conv and fuse as in forward()."""
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    if hist_ids is None:
        hist_ids = np.zeros((S, 2), np.int32)
    if hist_len is None:
        hist_len = np.zeros(S, np.int32)
    if conv_state is None:
        conv_state = np.zeros((S, 3, D), np.float64)
    row_ids = ngram_ids(tokens, cu, hist_ids, hist_len, R)
    valid = row_ids[row_ids >= 0]
    uniq, inv = np.unique(valid, return_inverse=True)
    codes, blocks, scales = row_source(uniq)
    compact = np.full(row_ids.shape, -1, dtype=np.int32)
    compact[row_ids >= 0] = inv.astype(np.int32)
    x = gather_dequant_nvfp4(compact, codes, blocks, scales)
    e = project(x, W_bf16)
    e_b = round_bf16(e)
    g = gate(h_bf16, e_b, eps)
    y, out, st = conv_fuse(h_bf16, e_b, g, cu, conv_w_bf16, conv_state)
    hid, hln = hist_update(tokens, cu, hist_ids, hist_len)
    return dict(row_ids=row_ids, x=x, e=e, e_b=e_b, g=g, y=y, out=out,
                hist_ids=hid, hist_len=hln, conv_state=st)


def forward_heads(tokens, cu_seqlens, h_bf16, W_bf16, conv_w_bf16, R: int, slice_source,
                  hist_ids=None, hist_len=None, conv_state=None, eps: float = 1e-6):
    """forward() for the 16-lookup layout: row IDs [T][16] into 16 head
    tables of R rows x 160 bytes, rows from slice_source(heads, rows) ->
    (codes uint8[n][160], scales float32[n]); the rest of the path is the
    same."""
    tokens = _c(tokens, np.int32)
    cu = _c(cu_seqlens, np.int32)
    S = len(cu) - 1
    if hist_ids is None:
        hist_ids = np.zeros((S, 2), np.int32)
    if hist_len is None:
        hist_len = np.zeros(S, np.int32)
    if conv_state is None:
        conv_state = np.zeros((S, 3, D), np.float64)
    row_ids = ngram_ids_heads(tokens, cu, hist_ids, hist_len, R)
    heads = np.broadcast_to(np.arange(16, dtype=np.int64), row_ids.shape)
    valid = row_ids >= 0
    q = heads[valid] * R + row_ids[valid]
    uniq, inv = np.unique(q, return_inverse=True)
    codes, scales = slice_source(uniq // R, uniq % R)
    compact = np.full(row_ids.shape, -1, dtype=np.int32)
    compact[valid] = inv.astype(np.int32)
    x = gather_dequant_heads(compact, codes, scales)
    e = project(x, W_bf16)
    e_b = round_bf16(e)
    g = gate(h_bf16, e_b, eps)
    y, out, st = conv_fuse(h_bf16, e_b, g, cu, conv_w_bf16, conv_state)
    hid, hln = hist_update(tokens, cu, hist_ids, hist_len)
    return dict(row_ids=row_ids, x=x, e=e, e_b=e_b, g=g, y=y, out=out,
                hist_ids=hid, hist_len=hln, conv_state=st)
