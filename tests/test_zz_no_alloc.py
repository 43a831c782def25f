"""ple_forward_noalloc, whose workspace is the library's own device array,
called through the C ABI against ple_forward on the same inputs, bit for bit:
consecutive calls that continue the carried state, the second smaller than
the first (the array keeps the first call's contents), in place too; and the
host-side refusal of calls beyond the array's limits, before anything runs."""

import numpy as np
import pytest
import torch

import sparse_memory_gather_amd as ple
from gen import inputs, table

from parity_util import D, dev_bf16, dev_i32, host_bits

pytestmark = pytest.mark.gpu


def _case(rng, lengths):
    T = int(sum(lengths))
    toks = inputs.uniform_tokens(rng, T)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h = inputs.normal_bf16(rng, (T, D))
    return toks, cu, h


def test_noalloc_equals_forward_on_consecutive_calls(weights):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    ple.load_library()
    W, cw = weights
    Wd, cwd = dev_bf16(W, dev), dev_bf16(cw, dev)
    tab, sc = table.table_gpu(65_536, device=dev)
    max_t, max_s = ple.noalloc_limits()
    assert (max_t, max_s) == (2048, 256)
    rng = np.random.default_rng(77)
    S = 5
    st_ref, st = ple.State(S, dev), ple.State(S, dev)
    ws = ple.Workspace(dev)
    # 2048 tokens (the limit; the streaming fuse), then 300 (the one-token
    # fuse), then 9: each continues the state the previous call left
    for lengths in ([700, 1, 0, 900, 447], [3, 1, 0, 250, 46], [1, 2, 1, 0, 5]):
        toks, cu, h = _case(rng, lengths)
        print("noalloc call", lengths, flush=True)
        t_d, cu_d, h_d = dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev)
        ref = host_bits(ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, h_d, st_ref, workspace=ws))
        got = host_bits(ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, h_d, st, noalloc=True))
        assert np.array_equal(got, ref), lengths
        assert torch.equal(st.conv_state, st_ref.conv_state), lengths
        assert torch.equal(st.hist_ids, st_ref.hist_ids) and torch.equal(st.hist_len, st_ref.hist_len)
    # debug outputs and an in-place call (out == h: the h rows other blocks
    # overwrite are copied into the array first)
    toks, cu, h = _case(rng, [600, 0, 1100, 3, 40])
    t_d, cu_d = dev_i32(toks, dev), dev_i32(cu, dev)
    a = ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, dev_bf16(h, dev), st_ref, workspace=ws, debug=True)
    b = ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, dev_bf16(h, dev), st, noalloc=True, debug=True)
    for k in ("row_ids", "x", "e", "gate", "y", "out"):
        assert torch.equal(a[k], b[k]), k
    h_a, h_b = dev_bf16(h, dev), dev_bf16(h, dev)
    ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, h_a, st_ref, out=h_a, workspace=ws)
    ple.ple_forward(t_d, cu_d, tab, sc, Wd, cwd, h_b, st, out=h_b, noalloc=True)
    assert torch.equal(h_a, h_b)
    assert torch.equal(st.conv_state, st_ref.conv_state)
    torch.cuda.synchronize()
    # beyond the limits: refused on the host, state untouched
    before = st.conv_state.clone()
    for lengths in ([max_t + 1], [1] * (max_s + 1)):
        toks, cu, h = _case(rng, lengths)
        stx = ple.State(len(lengths), dev)
        with pytest.raises(ple.PLEError) as ei:
            ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, Wd, cwd, dev_bf16(h, dev), stx,
                            noalloc=True)
        assert ei.value.status == -2
    assert torch.equal(st.conv_state, before)
