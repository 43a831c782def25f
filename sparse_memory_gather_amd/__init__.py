"""Python binding of libple, the MI355X PLE n-gram embedding lookup.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/ple.h. Torch provides device memory
and the current stream. There is no CPU fallback: if libple.so is missing,
or torch has no GPU, the calls raise.

The operation (Qwen3.8-Flash-Next pages; mengman.github.io "Qwen3.8-Flash-
Next 端侧部署 01", n-gram embedding section): per token, hash the recent
token IDs into bigram/trigram row IDs, gather and dequantize the FP8 rows,
project, gate, short-convolve with carried state and add to the hidden
state. Exact formulas are in include/ple.h.
"""

from __future__ import annotations

import ctypes
import os

import torch

D = 2560
CONV_TAPS = 4
MAX_VOCAB = 1 << 20
DEFAULT_VOCAB = 248_320
DEFAULT_EPS = 1e-6

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libple.so")

PLE_OK = 0
STATUS_NAMES = {0: "PLE_OK", -1: "PLE_ERR_NULL", -2: "PLE_ERR_SHAPE", -3: "PLE_ERR_RANGE",
                -4: "PLE_ERR_ALIGN", -5: "PLE_ERR_ALIAS", -6: "PLE_ERR_WORKSPACE", -7: "PLE_ERR_HIP"}
DEVERR_TOKEN_RANGE = 1
DEVERR_CU_SEQLENS = 2
DEVERR_HIST_LEN = 4
DEVERR_ROW_RANGE = 8
DEVERR_SYNC = 16


class PLEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p


class ForwardArgs(ctypes.Structure):
    """Mirror of ple_forward_args (include/ple.h), same field order."""
    _fields_ = [
        ("tokens", _P), ("T", ctypes.c_int64), ("cu_seqlens", _P), ("S", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32), ("table", _P), ("scales", _P), ("R", ctypes.c_int64),
        ("W", _P), ("conv_w", _P), ("h", _P), ("out", _P), ("hist_ids", _P), ("hist_len", _P),
        ("conv_state", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
        ("dev_err", _P), ("eps", ctypes.c_float), ("row_ids_out", _P), ("x_out", _P),
        ("e_out", _P), ("gate_out", _P), ("y_out", _P),
    ]


_lib = None

EXPORTS = ("ple_hash", "ple_lookup", "ple_proj", "ple_forward", "ple_forward_profiled",
           "ple_forward_workspace_size", "ple_hash_heads", "ple_lookup_heads", "ple_forward_heads",
           "ple_forward_heads_profiled", "ple_forward_heads_workspace_size", "ple_forward_x",
           "ple_lookup_nvfp4", "ple_forward_nvfp4", "ple_forward_nvfp4_profiled",
           "ple_status_string", "ple_last_error", "ple_proj_tiling", "ple_forward_noalloc",
           "ple_forward_noalloc_max_tokens", "ple_forward_noalloc_max_sequences", "ple_forward_one_launch",
           "ple_forward_staged")
HEADS = 16            # 16-lookup layout: head tables of 160-byte rows
SLICE = D // HEADS


def load_library(path: str = LIB_PATH):
    """Load libple.so (torch is imported first so that its HIP runtime is the
    one the library binds to)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libple is not built ({path} missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    for name in ("ple_hash", "ple_hash_heads"):
        getattr(lib, name).argtypes = [_P, I64, _P, I32, _P, _P, I32, I64, _P, _P, _P]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("ple_lookup", "ple_lookup_heads"):
        getattr(lib, name).argtypes = [_P, I64, _P, _P, I64, _P, _P, _P, _P]
        getattr(lib, name).restype = ctypes.c_int
    lib.ple_proj.argtypes = [_P, I64, _P, _P, _P]
    lib.ple_proj.restype = ctypes.c_int
    for name in ("ple_forward", "ple_forward_heads", "ple_forward_staged"):
        getattr(lib, name).argtypes = [ctypes.POINTER(ForwardArgs), _P]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("ple_forward_profiled", "ple_forward_heads_profiled"):
        getattr(lib, name).argtypes = [ctypes.POINTER(ForwardArgs), _P, ctypes.POINTER(_P)]
        getattr(lib, name).restype = ctypes.c_int
    lib.ple_forward_x.argtypes = [ctypes.POINTER(ForwardArgs), _P, _P]
    lib.ple_forward_x.restype = ctypes.c_int
    lib.ple_lookup_nvfp4.argtypes = [_P, I64, _P, _P, _P, I64, _P, _P, _P, _P]
    lib.ple_lookup_nvfp4.restype = ctypes.c_int
    lib.ple_forward_nvfp4.argtypes = [ctypes.POINTER(ForwardArgs), _P, _P]
    lib.ple_forward_nvfp4.restype = ctypes.c_int
    lib.ple_forward_nvfp4_profiled.argtypes = [ctypes.POINTER(ForwardArgs), _P, _P, ctypes.POINTER(_P)]
    lib.ple_forward_nvfp4_profiled.restype = ctypes.c_int
    for name in ("ple_forward_workspace_size", "ple_forward_heads_workspace_size"):
        getattr(lib, name).argtypes = [I64, I32]
        getattr(lib, name).restype = ctypes.c_size_t
    lib.ple_status_string.argtypes = [ctypes.c_int]
    lib.ple_status_string.restype = ctypes.c_char_p
    lib.ple_last_error.argtypes = []
    lib.ple_last_error.restype = ctypes.c_char_p
    lib.ple_proj_tiling.argtypes = [I64]
    lib.ple_proj_tiling.restype = ctypes.c_int
    lib.ple_forward_one_launch.argtypes = [I64, I32]
    lib.ple_forward_one_launch.restype = ctypes.c_int
    lib.ple_forward_noalloc.argtypes = [ctypes.POINTER(ForwardArgs), _P]
    lib.ple_forward_noalloc.restype = ctypes.c_int
    for name in ("ple_forward_noalloc_max_tokens", "ple_forward_noalloc_max_sequences"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_size_t
    _lib = lib
    return lib


PROJ_TILINGS = {0: None, 1: "proj_small_kernel", 2: "proj_mid_kernel", 3: "proj_kernel", 4: "proj_w320_kernel"}


def proj_tiling(T: int):
    """Name of the projection kernel a T-token forward runs (None for T <= 0)."""
    return PROJ_TILINGS[int(load_library().ple_proj_tiling(int(T)))]


def one_launch(T: int, S: int) -> bool:
    """Whether ple_forward runs a T-token call of S sequences (FP8 table) as
    one kernel launch."""
    return bool(load_library().ple_forward_one_launch(int(T), int(S)))


def _check(status: int):
    if status != PLE_OK:
        raise PLEError(status, load_library().ple_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _opt(t, name, dtype, shape):
    return None if t is None else _dev(t, name, dtype, shape)


def workspace_size(max_T: int, max_S: int, heads: bool = False) -> int:
    lib = load_library()
    f = lib.ple_forward_heads_workspace_size if heads else lib.ple_forward_workspace_size
    return int(f(max_T, max_S))


def _table(table, R: int):
    """The table's bytes, [R][2560] or (16-lookup layout) [16][R][160]."""
    if not isinstance(table, torch.Tensor) or table.numel() != R * D:
        raise ValueError(f"table must hold R x 2560 = {R * D} bytes")
    return _dev(table, "table", torch.uint8)


def _rows_of(table, scales, heads: bool) -> int:
    """R (rows, per head table in the 16-lookup layout) from the scales' shape."""
    if heads:
        if scales.dim() != 2 or scales.shape[0] != HEADS:
            raise ValueError("scales must be float32 [16][R] in the 16-lookup layout")
        return scales.shape[1]
    return table.shape[0]


def ple_hash(tokens, cu_seqlens, hist_ids, hist_len, R: int, vocab_size: int = DEFAULT_VOCAB,
             row_ids=None, dev_err=None, stream=None, heads: bool = False):
    """a1: row IDs int32 [T][2] (bigram, trigram; -1 when missing), or
    [T][16] in the 16-lookup layout (heads=True)."""
    T = tokens.numel()
    S = cu_seqlens.numel() - 1
    n = HEADS if heads else 2
    if row_ids is None:
        row_ids = torch.empty((T, n), dtype=torch.int32, device=tokens.device)
    lib = load_library()
    _check((lib.ple_hash_heads if heads else lib.ple_hash)(
        _dev(tokens, "tokens", torch.int32, (T,)), T, _dev(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        S, _dev(hist_ids, "hist_ids", torch.int32, (S, 2)), _dev(hist_len, "hist_len", torch.int32, (S,)),
        vocab_size, R, _dev(row_ids, "row_ids", torch.int32, (T, n)),
        _opt(dev_err, "dev_err", torch.int32, (1,)), _stream(stream)))
    return row_ids


def ple_lookup(row_ids, table, scales, x=None, raw=None, dev_err=None, stream=None, heads: bool = False):
    """a2: x bf16 [T][2560] = bf16(sum of the two dequantized rows); with
    heads=True the 16-lookup layout (scales [16][R], row_ids [T][16], raw
    [T][16][160])."""
    T = row_ids.shape[0]
    R = _rows_of(table, scales, heads)
    if x is None:
        x = torch.empty((T, D), dtype=torch.bfloat16, device=row_ids.device)
    lib = load_library()
    n = HEADS if heads else 2
    _check((lib.ple_lookup_heads if heads else lib.ple_lookup)(
        _dev(row_ids, "row_ids", torch.int32, (T, n)), T, _table(table, R),
        _dev(scales, "scales", torch.float32, (HEADS, R) if heads else (R,)), R,
        _dev(x, "x", torch.bfloat16, (T, D)),
        _opt(raw, "raw", torch.uint8, (T, HEADS, SLICE) if heads else (T, 2, D)),
        _opt(dev_err, "dev_err", torch.int32, (1,)), _stream(stream)))
    return x


def ple_lookup_nvfp4(row_ids, codes, blocks, scales, x=None, raw=None, dev_err=None, stream=None):
    """a2 over the NVFP4 table: codes uint8 [R][1280], blocks uint8 [R][160],
    scales float32 [R]; raw (optional) uint8 [T][2][1280]."""
    T = row_ids.shape[0]
    R = scales.shape[0]
    if x is None:
        x = torch.empty((T, D), dtype=torch.bfloat16, device=row_ids.device)
    _check(load_library().ple_lookup_nvfp4(
        _dev(row_ids, "row_ids", torch.int32, (T, 2)), T, _dev(codes, "codes", torch.uint8, (R, D // 2)),
        _dev(blocks, "blocks", torch.uint8, (R, D // 16)), _dev(scales, "scales", torch.float32, (R,)), R,
        _dev(x, "x", torch.bfloat16, (T, D)), _opt(raw, "raw", torch.uint8, (T, 2, D // 2)),
        _opt(dev_err, "dev_err", torch.int32, (1,)), _stream(stream)))
    return x


def ple_proj(x, W, e=None, stream=None):
    """a3: e fp32 [T][2560] = x W^T."""
    T = x.shape[0]
    if e is None:
        e = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _check(load_library().ple_proj(_dev(x, "x", torch.bfloat16, (T, D)), T,
                                   _dev(W, "W", torch.bfloat16, (D, D)),
                                   _dev(e, "e", torch.float32, (T, D)), _stream(stream)))
    return e


class State:
    """Per-sequence carried state: the last two token IDs and the last three
    gated vectors of each of S sequences (zeros = fresh sequences)."""

    def __init__(self, S: int, device="cuda"):
        self.hist_ids = torch.zeros((S, 2), dtype=torch.int32, device=device)
        self.hist_len = torch.zeros((S,), dtype=torch.int32, device=device)
        self.conv_state = torch.zeros((S, 3, D), dtype=torch.float32, device=device)

    @property
    def S(self) -> int:
        return self.hist_len.numel()

    def clone(self) -> "State":
        c = State.__new__(State)
        c.hist_ids = self.hist_ids.clone()
        c.hist_len = self.hist_len.clone()
        c.conv_state = self.conv_state.clone()
        return c


class Workspace:
    """Caller-owned scratch for ple_forward, grown on demand (allocation
    happens here, in torch, never inside libple). Allocated zeroed: its first
    256 bytes are the one-launch path's counters, which must be zero before
    the first call (libple leaves them zero)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, T: int, S: int, heads: bool = False) -> torch.Tensor:
        need = workspace_size(T, S, heads)
        if self.buf is None or self.buf.numel() < need:
            self.buf = torch.zeros((max(need, 256),), dtype=torch.uint8, device=self.device)
        return self.buf


class Forward:
    """One ple_forward call prepared once: every tensor is checked and the C
    argument struct built at construction; each call passes the struct
    straight to the library. For loops that run the same buffers again (a
    decode loop copying each step's tokens and hidden states into fixed
    device buffers). The tensors given must keep their storage while the
    object is in use; arguments as for ple_forward."""

    def __init__(self, tokens, cu_seqlens, table, scales, W, conv_w, h, state: State, out=None,
                 workspace=None, vocab_size: int = DEFAULT_VOCAB, eps: float = DEFAULT_EPS,
                 dev_err=None, debug: bool = False, heads: bool = False, nvfp4_blocks=None,
                 noalloc: bool = False, staged: bool = False):
        T = tokens.numel()
        S = cu_seqlens.numel() - 1
        nv = nvfp4_blocks is not None
        if nv and heads:
            raise ValueError("the NVFP4 table is read with two lookups per token")
        if staged and (noalloc or heads or nv):
            raise ValueError("staged runs the two-lookup FP8 table through ple_forward_staged")
        R = scales.shape[0] if nv else _rows_of(table, scales, heads)
        n = HEADS if heads else 2
        dev = tokens.device
        if out is None:
            out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        if noalloc:
            # ple_forward_noalloc: the library's own device array is the workspace
            if workspace is not None or heads or nv:
                raise ValueError("noalloc runs the two-lookup FP8 table with the library's own workspace")
            ws = None
        else:
            if workspace is None:
                workspace = Workspace(dev)
            ws = workspace.get(T, S, heads) if isinstance(workspace, Workspace) else workspace
        dbg = {}
        if debug:
            dbg = dict(row_ids=torch.empty((T, n), dtype=torch.int32, device=dev),
                       x=torch.empty((T, D), dtype=torch.bfloat16, device=dev),
                       e=torch.empty((T, D), dtype=torch.float32, device=dev),
                       gate=torch.empty((T,), dtype=torch.float32, device=dev),
                       y=torch.empty((T, D), dtype=torch.float32, device=dev))
        a = ForwardArgs()
        a.tokens = _dev(tokens, "tokens", torch.int32, (T,))
        a.T = T
        a.cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,))
        a.S = S
        a.vocab_size = vocab_size
        a.table = _dev(table, "table", torch.uint8, (R, D // 2)) if nv else _table(table, R)
        a.scales = _dev(scales, "scales", torch.float32, (HEADS, R) if heads else (R,))
        a.R = R
        a.W = _dev(W, "W", torch.bfloat16, (D, D))
        a.conv_w = _dev(conv_w, "conv_w", torch.bfloat16, (D, CONV_TAPS))
        a.h = _dev(h, "h", torch.bfloat16, (T, D))
        a.out = _dev(out, "out", torch.bfloat16, (T, D))
        a.hist_ids = _dev(state.hist_ids, "hist_ids", torch.int32, (S, 2))
        a.hist_len = _dev(state.hist_len, "hist_len", torch.int32, (S,))
        a.conv_state = _dev(state.conv_state, "conv_state", torch.float32, (S, 3, D))
        a.workspace = None if ws is None else _dev(ws, "workspace", torch.uint8)
        a.workspace_bytes = 0 if ws is None else ws.numel()
        a.dev_err = _opt(dev_err, "dev_err", torch.int32, (1,))
        a.eps = eps
        if debug:
            a.row_ids_out = dbg["row_ids"].data_ptr()
            a.x_out = dbg["x"].data_ptr()
            a.e_out = dbg["e"].data_ptr()
            a.gate_out = dbg["gate"].data_ptr()
            a.y_out = dbg["y"].data_ptr()
        lib = load_library()
        self.args, self.out, self.debug = a, out, dbg if debug else None
        byref = ctypes.byref(a)
        # the tensors whose addresses the struct holds stay referenced here
        self._keep = (tokens, cu_seqlens, table, scales, W, conv_w, h, state, ws, dev_err, nvfp4_blocks)
        if noalloc:
            self._run = lambda st: lib.ple_forward_noalloc(byref, st)
            self._run_ev = None
        elif staged:
            self._run = lambda st: lib.ple_forward_staged(byref, st)
            self._run_ev = None
        elif nv:
            blk = _dev(nvfp4_blocks, "nvfp4_blocks", torch.uint8, (R, D // 16))
            self._run = lambda st: lib.ple_forward_nvfp4(byref, blk, st)
            self._run_ev = lambda st, ev: lib.ple_forward_nvfp4_profiled(byref, blk, st, ev)
        elif heads:
            self._run = lambda st: lib.ple_forward_heads(byref, st)
            self._run_ev = lambda st, ev: lib.ple_forward_heads_profiled(byref, st, ev)
        else:
            self._run = lambda st: lib.ple_forward(byref, st)
            self._run_ev = lambda st, ev: lib.ple_forward_profiled(byref, st, ev)

    def __call__(self, stream=None, events=None):
        """Enqueue the call on `stream` (default: torch's current stream);
        returns out, or the debug dict. `events` as for ple_forward."""
        if events is None:
            _check(self._run(_stream(stream)))
        elif self._run_ev is None:
            raise ValueError("per-stage events are recorded by ple_forward_profiled only (not by noalloc or staged)")
        else:
            _check(self._run_ev(_stream(stream), (_P * 5)(*[ctypes.c_void_p(int(e)) for e in events])))
        if self.debug is not None:
            self.debug["out"] = self.out
            return self.debug
        return self.out


def ple_forward(tokens, cu_seqlens, table, scales, W, conv_w, h, state: State, out=None,
                workspace=None, vocab_size: int = DEFAULT_VOCAB, eps: float = DEFAULT_EPS,
                dev_err=None, debug: bool = False, stream=None, events=None, heads: bool = False,
                nvfp4_blocks=None, noalloc: bool = False, staged: bool = False):
    """a1..a4 for one chunk. Updates `state` in place; returns out (bf16
    [T][2560]) or, with debug=True, a dict with out, row_ids, x, e, gate, y.
    `events`: optional sequence of five hipEvent_t handles (ints) recorded
    around the four stages (ple_forward_profiled). heads=True: the 16-lookup
    layout (scales [16][R], row_ids [T][16]). nvfp4_blocks (uint8 [R][160]):
    the NVFP4 table, `table` then being the packed codes uint8 [R][1280].
    noalloc=True: ple_forward_noalloc (no workspace; up to
    noalloc_limits() tokens and sequences). staged=True: ple_forward_staged
    (every stage its own launch, also for the calls ple_forward runs as one)."""
    return Forward(tokens, cu_seqlens, table, scales, W, conv_w, h, state, out=out, workspace=workspace,
                   vocab_size=vocab_size, eps=eps, dev_err=dev_err, debug=debug, heads=heads,
                   nvfp4_blocks=nvfp4_blocks, noalloc=noalloc, staged=staged)(stream=stream, events=events)


def noalloc_limits():
    """(max tokens, max sequences) of one ple_forward_noalloc call."""
    lib = load_library()
    return int(lib.ple_forward_noalloc_max_tokens()), int(lib.ple_forward_noalloc_max_sequences())


def ple_forward_x(x, tokens, cu_seqlens, W, conv_w, h, state: State, out=None, workspace=None,
                  eps: float = DEFAULT_EPS, dev_err=None, debug: bool = False, stream=None):
    """a3..a4 from x (bf16 [T][2560]) gathered ahead by ple_hash + ple_lookup
    (e.g. on another stream, with the history the chunk starts from): the
    same projection, gate, conv, fuse and state update as ple_forward. With
    debug=True returns a dict with out, e, gate, y."""
    T = tokens.numel()
    S = cu_seqlens.numel() - 1
    dev = tokens.device
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = Workspace(dev)
    ws = workspace.get(T, S) if isinstance(workspace, Workspace) else workspace
    dbg = {}
    if debug:
        dbg = dict(e=torch.empty((T, D), dtype=torch.float32, device=dev),
                   gate=torch.empty((T,), dtype=torch.float32, device=dev),
                   y=torch.empty((T, D), dtype=torch.float32, device=dev))
    a = ForwardArgs()
    a.tokens = _dev(tokens, "tokens", torch.int32, (T,))
    a.T = T
    a.cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,))
    a.S = S
    a.W = _dev(W, "W", torch.bfloat16, (D, D))
    a.conv_w = _dev(conv_w, "conv_w", torch.bfloat16, (D, CONV_TAPS))
    a.h = _dev(h, "h", torch.bfloat16, (T, D))
    a.out = _dev(out, "out", torch.bfloat16, (T, D))
    a.hist_ids = _dev(state.hist_ids, "hist_ids", torch.int32, (S, 2))
    a.hist_len = _dev(state.hist_len, "hist_len", torch.int32, (S,))
    a.conv_state = _dev(state.conv_state, "conv_state", torch.float32, (S, 3, D))
    a.workspace = _dev(ws, "workspace", torch.uint8)
    a.workspace_bytes = ws.numel()
    a.dev_err = _opt(dev_err, "dev_err", torch.int32, (1,))
    a.eps = eps
    if debug:
        a.e_out = dbg["e"].data_ptr()
        a.gate_out = dbg["gate"].data_ptr()
        a.y_out = dbg["y"].data_ptr()
    _check(load_library().ple_forward_x(ctypes.byref(a), _dev(x, "x", torch.bfloat16, (T, D)), _stream(stream)))
    if debug:
        dbg["out"] = out
        return dbg
    return out
