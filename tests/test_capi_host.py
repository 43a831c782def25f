"""Host-side checks of the C ABI that need no GPU: the library loads, every
symbol include/ple.h declares is exported, and argument validation rejects
bad calls before anything is enqueued (so these calls never reach a kernel).
"""

import ctypes
import os
import re
import subprocess

import pytest
import torch

import sparse_memory_gather_amd as ple

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ple.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ple.LIB_PATH), reason="libple.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ple_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = _declared()
    assert set(names) == set(ple.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ple.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
    lib = ple.load_library()
    for n in names:
        assert hasattr(lib, n)


def test_projection_tiling_by_call_size():
    # small-T up to 256 tokens, mid-size up to 3200, then whichever of the
    # 256 x 256 and 256 x 320 tilings needs fewer (weighted) rounds of 256 blocks
    expect = {0: None, 1: "proj_small_kernel", 256: "proj_small_kernel", 257: "proj_mid_kernel",
              3200: "proj_mid_kernel", 3201: "proj_kernel", 6144: "proj_kernel", 8100: "proj_w320_kernel",
              8192: "proj_w320_kernel", 12000: "proj_kernel", 16384: "proj_w320_kernel",
              24576: "proj_w320_kernel", 32768: "proj_w320_kernel"}
    for T, name in expect.items():
        assert ple.proj_tiling(T) == name, T


def test_forward_args_struct_matches_header_field_order():
    src = open(HEADER).read()
    body = src[src.index("typedef struct ple_forward_args"):src.index("} ple_forward_args;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b([a-zA-Z_]+)\s*;", body)
    assert fields == [f[0] for f in ple.ForwardArgs._fields_]


def test_status_strings_and_workspace_size():
    lib = ple.load_library()
    assert lib.ple_status_string(0) == b"ok"
    assert lib.ple_status_string(-6) == b"workspace too small"
    # workspace: the one-launch path's counters (256 bytes), row ids + x + e
    # (bf16) per token, conv-state copy per sequence
    T, S = 1000, 3
    need = ple.workspace_size(T, S)
    assert need >= 256 + T * (8 + 2560 * 2 * 2) + S * 3 * 2560 * 4
    assert need % 256 == 0 and ple.workspace_size(0, 0) == 256


# Every call below fails validation, so no kernel is launched; fake device
# addresses are fine. Skipped where a GPU is present, so that a validation
# bug can never turn one of them into a real launch.
cpu_only = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only checks")
FAKE = 0x7F0000000000


def _fwd_args(**over):
    a = ple.ForwardArgs()
    T, S = 64, 2
    base = FAKE
    vals = dict(tokens=base, T=T, cu_seqlens=base + 0x1000, S=S, vocab_size=248320,
                table=base + 0x100000, scales=base + 0x200000, R=1000, W=base + 0x400000,
                conv_w=base + 0x1400000, h=base + 0x2000000, out=base + 0x3000000,
                hist_ids=base + 0x4000000, hist_len=base + 0x4001000, conv_state=base + 0x5000000,
                workspace=base + 0x6000000, workspace_bytes=ple.workspace_size(T, S), eps=1e-6)
    vals.update(over)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


def _call(a):
    return ple.load_library().ple_forward(ctypes.byref(a), None)


@cpu_only
@pytest.mark.parametrize("over,status", [
    (dict(R=0), -3), (dict(R=2 ** 31), -3), (dict(vocab_size=0), -3),
    (dict(vocab_size=(1 << 20) + 1), -3), (dict(S=0), -2), (dict(T=-1), -2),
    (dict(T=2 ** 31), -2),                            # beyond int32 cu_seqlens
    (dict(eps=-1.0), -3), (dict(eps=float("nan")), -3),
    (dict(tokens=None), -1), (dict(table=None), -1), (dict(conv_state=None), -1),
    (dict(workspace=None), -6), (dict(workspace_bytes=1000), -6),
    (dict(h=FAKE + 0x2000000 + 2), -4), (dict(workspace=FAKE + 0x6000000 + 16), -4),
    (dict(table=FAKE + 0x100000 + 8), -4),
    (dict(out=FAKE + 0x2000000 + 256), -5),          # partial overlap with h
    (dict(conv_state=FAKE + 0x3000000), -5),         # state inside out
    (dict(x_out=FAKE + 0x2000000), -5),              # debug output over h
])
def test_forward_rejects_bad_arguments(over, status):
    st = _call(_fwd_args(**over))
    assert st == status
    assert ple.load_library().ple_last_error() != b""


@cpu_only
def test_forward_in_place_and_empty_calls_pass_validation_without_launch():
    # T = 0 returns OK without touching anything (pointers may be anything)
    assert _call(_fwd_args(T=0, tokens=None, h=None)) == 0
    assert ple.load_library().ple_last_error() == b""


@cpu_only
def test_hash_lookup_proj_reject_bad_arguments():
    lib = ple.load_library()
    assert lib.ple_hash(FAKE, 10, FAKE + 0x100, 0, FAKE, FAKE, 100, 10, FAKE + 0x1000, None, None) == -2
    assert lib.ple_hash(FAKE, 10, FAKE + 0x100, 1, FAKE, FAKE, 100, 0, FAKE + 0x1000, None, None) == -3
    assert lib.ple_hash(FAKE, 10, FAKE + 0x100, 1, FAKE, FAKE, 100, 10, FAKE + 0x1004, None, None) == -4
    assert lib.ple_hash(FAKE, 10, FAKE + 0x100, 1, FAKE, FAKE, 100, 10, FAKE, None, None) == -5
    assert lib.ple_hash(FAKE, 0, None, 1, None, None, 100, 10, None, None, None) == 0
    assert lib.ple_hash(FAKE, 2 ** 31, FAKE + 0x100, 1, FAKE, FAKE, 100, 10, FAKE + 0x1000, None, None) == -2
    assert lib.ple_lookup(FAKE, 4, FAKE + 0x10000, None, 10, FAKE + 0x100000, None, None, None) == -1
    assert lib.ple_lookup(FAKE, 4, FAKE + 0x10008, FAKE + 0x90000, 10, FAKE + 0x100000, None, None,
                          None) == -4
    assert lib.ple_lookup(FAKE, 4, FAKE + 0x10000, FAKE + 0x90000, 10, FAKE + 0x10000, None, None,
                          None) == -5
    assert lib.ple_proj(FAKE, 4, FAKE + 0x100000, FAKE + 0x100000, None) == -5
    assert lib.ple_proj(FAKE, -1, FAKE + 0x100000, FAKE + 0x10000000, None) == -2


@cpu_only
def test_forward_x_and_heads_reject_bad_arguments():
    lib = ple.load_library()
    X = FAKE + 0x8000000
    # x NULL; debug outputs that ple_forward_x does not produce; x misaligned;
    # x overlapping a written buffer
    assert lib.ple_forward_x(ctypes.byref(_fwd_args()), None, None) == -1
    assert lib.ple_forward_x(ctypes.byref(_fwd_args(x_out=FAKE + 0x9000000)), X, None) == -2
    assert lib.ple_forward_x(ctypes.byref(_fwd_args()), X + 8, None) == -4
    assert lib.ple_forward_x(ctypes.byref(_fwd_args()), FAKE + 0x3000000, None) == -5    # x inside out
    # table, scales, R and vocab_size are not used by ple_forward_x
    assert lib.ple_forward_x(ctypes.byref(_fwd_args(T=0, table=None, R=0)), X, None) == 0
    # 16-lookup layout: row_ids must be 16-byte aligned; scales span 16 R
    assert lib.ple_hash_heads(FAKE, 10, FAKE + 0x100, 1, FAKE, FAKE, 100, 10, FAKE + 0x1008, None, None) == -4
    # x placed 320 bytes after the scales: outside 10 scales, inside 16 x 10
    assert lib.ple_lookup_heads(FAKE, 4, FAKE + 0x10000, FAKE + 0x90000, 10, FAKE + 0x90140, None, None,
                                None) == -5


def test_binding_refuses_cpu_tensors_and_bad_dtypes():
    # the binding only marshals: CPU tensors are refused (there is no CPU
    # fallback), as are wrong dtypes, shapes and non-contiguous tensors
    toks = torch.zeros(4, dtype=torch.int32)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    hist = torch.zeros((1, 2), dtype=torch.int32)
    hl = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        ple.ple_hash(toks, cu, hist, hl, 10)
    with pytest.raises(ValueError, match="GPU"):
        ple.ple_lookup(torch.zeros((4, 2), dtype=torch.int32), torch.zeros((10, 2560), dtype=torch.uint8),
                       torch.zeros(10))
    with pytest.raises(ValueError, match="GPU"):
        ple.ple_proj(torch.zeros((4, 2560), dtype=torch.bfloat16), torch.zeros((2560, 2560), dtype=torch.bfloat16))
    # the device is checked first, whatever else is wrong; non-tensors are refused
    with pytest.raises(ValueError, match="GPU"):
        ple._dev(torch.zeros(4, dtype=torch.int64), "tokens", torch.int32)
    with pytest.raises(TypeError):
        ple._dev([1, 2, 3], "tokens", torch.int32)


def test_binding_raises_when_the_library_is_missing(tmp_path, monkeypatch):
    # a missing libple.so is an error, never a silent fallback
    monkeypatch.setattr(ple, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        ple.load_library(str(tmp_path / "libple.so"))


@cpu_only
def test_noalloc_refuses_oversize_calls_and_a_workspace_before_any_launch():
    lib = ple.load_library()
    assert lib.ple_forward_noalloc_max_tokens() == 2048 and lib.ple_forward_noalloc_max_sequences() == 256
    # beyond the array's limits: PLE_ERR_SHAPE, with the limits in the message
    for over in (dict(T=2049), dict(S=257)):
        a = _fwd_args(workspace=None, workspace_bytes=0, **over)
        assert lib.ple_forward_noalloc(ctypes.byref(a), None) == -2
        assert b"beyond its limits" in lib.ple_last_error()
    # the call brings no workspace of its own
    a = _fwd_args()
    assert lib.ple_forward_noalloc(ctypes.byref(a), None) == -6
    assert lib.ple_forward_noalloc(None, None) == -1


def test_traffic_hashes_cover_every_file_a_kernel_is_built_from():
    """bench.py reports a recorded HBM-traffic figure only while the hash of
    the kernel's source files matches: the list must hold the .hip file and
    every header it includes, directly or not."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    csrc = os.path.join(root, "sparse_memory_gather_amd", "csrc")

    def closure(name, seen):
        if name in seen:
            return seen
        seen.add(name)
        for inc in re.findall(r'^#include "([^"]+)"', open(os.path.join(csrc, name)).read(), re.M):
            if os.path.exists(os.path.join(csrc, inc)):
                closure(inc, seen)
        return seen

    for kernel, files in bench.KERNEL_SOURCES.items():
        names = {os.path.basename(f) for f in files}
        hip = [n for n in names if n.endswith(".hip")]
        assert len(hip) == 1, kernel
        assert closure(hip[0], set()) == names, kernel
