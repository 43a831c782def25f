"""GPU parity at the full workload sizes (20,000,096-row, 51.2 GB FP8 table
in HBM), in the same launch configuration the bench times: every row ID is
compared with the oracle; sampled tokens (sequence starts, chunk and step
boundaries, random interior positions) are recomputed one by one by the
oracle and compared on x, e, gate, y and out."""

import numpy as np
import pytest
import torch

import oracle
import sparse_memory_gather_amd as ple
from gen import inputs, table

from parity_util import (D, check_samples, dev_bf16, dev_i32, gather_debug, host_bits,
                         oracle_samples)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def full_table(dev):
    t = table.table_gpu(inputs.R_FULL, device=dev)
    yield t
    del t
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def dev_weights(dev, weights):
    W, cw = weights
    return dev_bf16(W, dev), dev_bf16(cw, dev)


def _run(dev, tab, sc, dw, toks, cu, h, state, ws, debug):
    return ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dw[0], dw[1],
                           dev_bf16(h, dev), state, workspace=ws, debug=debug)


def _interior(rng, lo, hi, n):
    return sorted(set(int(v) for v in rng.integers(lo, hi, n)))


def test_full_table_generator_sample_matches_cpu(dev, full_table):
    tab, sc = full_table
    ids = np.concatenate([np.random.default_rng(11).integers(0, inputs.R_FULL, 10_000),
                          [0, inputs.R_FULL - 1]])
    codes, scales = table.rows_cpu(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(tab[it].cpu().numpy(), codes)
    assert np.array_equal(sc[it].cpu().numpy(), scales)


@pytest.mark.parametrize("name", ["prefill", "ragged"])
def test_single_chunk_workloads(dev, full_table, dev_weights, weights, name):
    W, cw = weights
    tab, sc = full_table
    wl = inputs.make_workload(name)
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    ws = ple.Workspace(dev)
    st_a = ple.State(wl.S, dev)
    out = host_bits(_run(dev, tab, sc, dev_weights, toks, cu, h, st_a, ws, debug=False))
    st_b = ple.State(wl.S, dev)
    res = _run(dev, tab, sc, dev_weights, toks, cu, h, st_b, ws, debug=True)
    assert np.array_equal(host_bits(res["out"]), out)       # debug outputs change nothing
    assert torch.equal(st_a.conv_state, st_b.conv_state)
    # every row id
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((wl.S, 2), np.int32), np.zeros(wl.S, np.int32), wl.R)
    assert np.array_equal(res["row_ids"].cpu().numpy(), ref_ids)
    # sampled tokens: starts of sequences, their 2nd/3rd/4th tokens, ends, interior
    rng = np.random.default_rng(12)
    seqs, samples = [], []
    pick = [0] if wl.S == 1 else [0, 1, 2, 3, 63]
    for s in pick:
        a, b = int(cu[s]), int(cu[s + 1])
        seqs.append((toks[a:b], h[a:b]))
        pos = [0, 1, 2, 3, b - a - 1] + _interior(rng, 4, b - a - 1, 6 if wl.S == 1 else 2)
        samples += [(len(seqs) - 1, p) for p in sorted(set(pos))]
    ref = oracle_samples(seqs, samples, W, cw, wl.R)
    idx = [int(cu[pick[si]]) + p for si, p in samples]
    stats = check_samples(gather_debug(res, idx), ref, W, name)
    print(name, stats)
    # carried state of the last sequence: hist = its last two tokens
    last = wl.S - 1
    assert list(st_a.hist_ids[last].cpu().numpy()) == list(toks[int(cu[last + 1]) - 2:int(cu[last + 1])])


def test_long_context_chunks(dev, full_table, dev_weights, weights):
    W, cw = weights
    tab, sc = full_table
    wl = inputs.make_workload("long")
    ws = ple.Workspace(dev)
    st = ple.State(1, dev)
    all_toks = np.concatenate([c[0] for c in wl.chunks])
    hs, outs, samples_idx = [], [], []
    rng = np.random.default_rng(13)
    check_chunks = {0, 1, 7, 15}
    got_rows = []
    pos0 = 0
    for i, (toks, cu) in enumerate(wl.chunks):
        h = wl.hidden(i)
        hs.append(h)
        debug = i in check_chunks
        res = _run(dev, tab, sc, dev_weights, toks, cu, h, st, ws, debug=debug)
        if debug:
            n = len(toks)
            pos = sorted(set([0, 1, 2, 3, n - 1] + _interior(rng, 4, n - 1, 5)))
            got_rows.append(gather_debug(res, pos))
            samples_idx += [pos0 + p for p in pos]
            ids = res["row_ids"].cpu().numpy()
            ref_ids = oracle.ngram_ids(all_toks[:pos0 + n], np.array([0, pos0 + n], np.int32),
                                       np.zeros((1, 2), np.int32), np.zeros(1, np.int32), wl.R)[pos0:]
            assert np.array_equal(ids, ref_ids), i
        pos0 += len(toks)
    h_all = np.concatenate(hs)
    ref = oracle_samples([(all_toks, h_all)], [(0, p) for p in samples_idx], W, cw, wl.R)
    got = {k: np.concatenate([g[k] for g in got_rows]) for k in got_rows[0]}
    print("long", check_samples(got, ref, W, "long"))
    assert list(st.hist_ids[0].cpu().numpy()) == list(all_toks[-2:])


def test_decode_steps_after_history(dev, full_table, dev_weights, weights):
    W, cw = weights
    tab, sc = full_table
    wl = inputs.make_workload("decode", decode_steps=16)
    S = wl.S
    hist = wl.history[0]                                   # [8][4096]
    hlen = hist.shape[1]
    h_hist = wl.history_hidden(S * hlen)
    ws = ple.Workspace(dev)
    st = ple.State(S, dev)
    cu_h = np.arange(0, S * hlen + 1, hlen, dtype=np.int32)
    _run(dev, tab, sc, dev_weights, hist.reshape(-1), cu_h, h_hist, st, ws, debug=False)
    assert np.array_equal(st.hist_ids.cpu().numpy(), hist[:, -2:])
    steps = []
    for k, (toks, cu) in enumerate(wl.chunks):
        h = wl.hidden(k)
        res = _run(dev, tab, sc, dev_weights, toks, cu, h, st, ws, debug=True)
        steps.append((toks, h, gather_debug(res, np.arange(S))))
    # sequences as the oracle sees them: history then one token per step
    seqs = []
    for s in range(S):
        t = np.concatenate([hist[s], [st_[0][s] for st_ in steps]]).astype(np.int32)
        hh = np.concatenate([h_hist[s * hlen:(s + 1) * hlen], np.stack([st_[1][s] for st_ in steps])])
        seqs.append((t, hh))
    check_k = [0, 1, 2, 15]
    samples = [(s, hlen + k) for k in check_k for s in range(S)]
    ref = oracle_samples(seqs, samples, W, cw, wl.R)
    got = {key: np.concatenate([steps[k][2][key] for k in check_k]) for key in steps[0][2]}
    print("decode", check_samples(got, ref, W, "decode"))


def test_prefill_heads_layout(dev, full_table, dev_weights, weights):
    # the 16-lookup layout on the same 51.2 GB of table bytes: 16 head tables
    # of 20,000,096 rows x 160 bytes, 16 x 20,000,096 scales
    W, cw = weights
    tab, _ = full_table
    R = inputs.R_FULL
    sc16 = table.head_scales_gpu(R, device=dev)
    rng = np.random.default_rng(15)
    hs, rs = rng.integers(0, 16, 500), rng.integers(0, R, 500)
    _, want = table.slices_cpu(hs, rs, R)
    assert np.array_equal(sc16[torch.as_tensor(hs, device=dev), torch.as_tensor(rs, device=dev)].cpu().numpy(),
                          want)
    wl = inputs.make_workload("prefill")
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    st = ple.State(1, dev)
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc16, dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), st, debug=True, heads=True)
    ref_ids = oracle.ngram_ids_heads(toks, cu, np.zeros((1, 2), np.int32), np.zeros(1, np.int32), R)
    assert np.array_equal(res["row_ids"].cpu().numpy(), ref_ids)
    pos = sorted(set([0, 1, 2, 3, len(toks) - 1] + _interior(rng, 4, len(toks) - 1, 8)))
    ref = oracle_samples([(toks, h)], [(0, p) for p in pos], W, cw, R, heads=True)
    print("prefill heads", check_samples(gather_debug(res, pos), ref, W, "prefill heads"))
    del sc16


def test_prefill_nvfp4_table(dev, dev_weights, weights):
    # the NVFP4 table at the full row count: 20,000,096 rows x (1280 code
    # bytes + 160 block scales + 4-byte row scale) = 28.9 GB in HBM
    W, cw = weights
    R = inputs.R_FULL
    codes, blocks, scales = table.nvfp4_gpu(R, device=dev)
    rng = np.random.default_rng(19)
    ids = np.concatenate([rng.integers(0, R, 2000), [0, R - 1]])
    c, b, s = table.nvfp4_rows_cpu(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(codes[it].cpu().numpy(), c)
    assert np.array_equal(blocks[it].cpu().numpy(), b)
    assert np.array_equal(scales[it].cpu().numpy(), s)
    wl = inputs.make_workload("prefill")
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    st = ple.State(1, dev)
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), codes, scales, dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), st, debug=True, nvfp4_blocks=blocks)
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((1, 2), np.int32), np.zeros(1, np.int32), R)
    assert np.array_equal(res["row_ids"].cpu().numpy(), ref_ids)
    pos = sorted(set([0, 1, 2, 3, len(toks) - 1] + _interior(rng, 4, len(toks) - 1, 8)))
    ref = oracle_samples([(toks, h)], [(0, p) for p in pos], W, cw, R, nvfp4=True)
    print("prefill nvfp4", check_samples(gather_debug(res, pos), ref, W, "prefill nvfp4"))
    del res, codes, blocks, scales
    torch.cuda.empty_cache()


def test_max_size_single_call(dev, dev_weights, weights):
    # one call of 2^20 tokens in four uneven sequences: byte offsets of the
    # bf16 rows pass 2^31, so any 32-bit index arithmetic would show here
    W, cw = weights
    R = 65_536
    tab, sc = table.table_gpu(R, device=dev)
    T = 1 << 20
    lengths = [1, (1 << 19) - 1, (1 << 19) - 3, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(17)
    toks = inputs.uniform_tokens(rng, T)
    g = torch.Generator(device=dev)
    g.manual_seed(1717)
    h = torch.randn((T, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    st = ple.State(len(lengths), dev)
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1], h,
                          st, debug=True)
    ids = res["row_ids"]
    probe = np.array([0, 1, 2, 3, 4, cu[2] - 1, cu[2], cu[2] + 3, cu[3] - 1, cu[3], T - 3, T - 1,
                      (1 << 19) + 12345, 900_001])
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((4, 2), np.int32), np.zeros(4, np.int32), R)
    assert np.array_equal(ids[torch.as_tensor(probe, device=dev)].cpu().numpy(), ref_ids[probe])
    assert int((ids.cpu().numpy() != ref_ids).sum()) == 0
    # sampled outputs, each recomputed from its own sequence
    seqs, samples, idx = [], [], []
    for s in range(4):
        a, b = int(cu[s]), int(cu[s + 1])
        pos = sorted(set(p for p in (0, 1, 2, 3, b - a - 1, (b - a) // 2) if 0 <= p < b - a))
        # only the hidden rows the samples read (each sample and the three before it)
        need = sorted(set(q for p in pos for q in range(max(0, p - 3), p + 1)))
        hh = np.zeros((b - a, D), np.uint16)
        hh[need] = host_bits(h[torch.as_tensor(np.array(need) + a, device=dev)])
        seqs.append((toks[a:b], hh))
        samples += [(s, p) for p in pos]
        idx += [a + p for p in pos]
    ref = oracle_samples(seqs, samples, W, cw, R)
    print("max size", check_samples(gather_debug(res, idx), ref, W, "max size"))
    del res, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["heads", "nvfp4"])
def test_ragged_other_layouts(dev, full_table, dev_weights, weights, layout):
    # the ragged workload (64 x 256 tokens, 20,000,096 rows) in the 16-lookup
    # layout (the 51.2 GB table read as 16 head tables) and over the NVFP4
    # table (28.9 GB): every row ID, and sampled tokens of five sequences
    W, cw = weights
    wl = inputs.make_workload("ragged")
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    R = wl.R
    if layout == "heads":
        tab, sc, kw = full_table[0], table.head_scales_gpu(R, device=dev), dict(heads=True)
        ref_ids = oracle.ngram_ids_heads(toks, cu, np.zeros((wl.S, 2), np.int32), np.zeros(wl.S, np.int32), R)
    else:
        codes, blocks, sc = table.nvfp4_gpu(R, device=dev)
        tab, kw = codes, dict(nvfp4_blocks=blocks)
        ref_ids = oracle.ngram_ids(toks, cu, np.zeros((wl.S, 2), np.int32), np.zeros(wl.S, np.int32), R)
    st = ple.State(wl.S, dev)
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), st, debug=True, **kw)
    assert np.array_equal(res["row_ids"].cpu().numpy(), ref_ids)
    rng = np.random.default_rng(21)
    seqs, samples, idx = [], [], []
    for s in (0, 1, 31, 62, 63):
        a, b = int(cu[s]), int(cu[s + 1])
        seqs.append((toks[a:b], h[a:b]))
        pos = sorted(set([0, 1, 2, 3, b - a - 1] + _interior(rng, 4, b - a - 1, 2)))
        samples += [(len(seqs) - 1, p) for p in pos]
        idx += [a + p for p in pos]
    ref = oracle_samples(seqs, samples, W, cw, R, heads=layout == "heads", nvfp4=layout == "nvfp4")
    print("ragged", layout, check_samples(gather_debug(res, idx), ref, W, f"ragged {layout}"))
    del res
    if layout == "nvfp4":
        del codes, blocks
    torch.cuda.empty_cache()
