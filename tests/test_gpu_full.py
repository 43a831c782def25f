"""GPU parity at the full workload sizes (20,000,096-row, 51.2 GB FP8 table
in HBM), in the launch configuration the bench times.

Against the oracle on EVERY token of every workload (all 16 chunks of the
long context, every one of 64 decode steps): the row IDs, the gathered FP8
bytes (ple_lookup's raw copy, on the forward's own IDs) and x, bit for bit.
e, g, y and out are compared within the derived bounds at:
  - sequence starts (first four tokens) and ends, random interior tokens;
  - every block-range start of the streaming fuse (ranges of ceil(T/256)
    tokens for these calls): the range's first four tokens, whose conv taps
    come from the three tokens before it, and those three tokens;
  - decode: every 8th step and the last;
and the carried conv state after the call against the oracle's last three v
of every sequence. Each call runs twice on copies of the state, once with
the debug outputs (which switch the streaming fuse to its general path) and
once without (the path the bench times): outputs and state must agree bit
for bit."""

import numpy as np
import pytest
import torch

import oracle
import sparse_memory_gather_amd as ple
from gen import inputs, table

from parity_util import (D, check_samples, dev_bf16, dev_i32, gather_debug, host_bits, oracle_windows,
                         OUT_ATOL, OUT_RTOL)

pytestmark = pytest.mark.gpu

STREAM_BLOCKS = 256   # the streaming fuse splits a long call into ranges of ceil(T / 256) tokens


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


def _interior(rng, lo, hi, n):
    return sorted(set(int(v) for v in rng.integers(lo, hi, n)))


def _state_copy(st):
    return st.clone()


def _run_pair(dev, tab, sc, dw, toks_d, cu_d, h_d, st_fast, st_dbg, ws, **kw):
    """One call without debug outputs (the timed path) on st_fast and one with
    them on st_dbg; outputs and the updated states must agree bit for bit."""
    out = host_bits(ple.ple_forward(toks_d, cu_d, tab, sc, dw[0], dw[1], h_d, st_fast, workspace=ws, **kw))
    res = ple.ple_forward(toks_d, cu_d, tab, sc, dw[0], dw[1], h_d, st_dbg, workspace=ws, debug=True, **kw)
    assert np.array_equal(host_bits(res["out"]), out), "debug outputs changed out"
    assert torch.equal(st_fast.conv_state, st_dbg.conv_state)
    assert torch.equal(st_fast.hist_ids, st_dbg.hist_ids) and torch.equal(st_fast.hist_len, st_dbg.hist_len)
    return res


def check_every_token_gather(dev, tab, sc, res, ref_ids, label):
    """Every token of a call: row IDs against the oracle's, then x (the
    forward's own) and the gathered FP8 bytes (ple_lookup with a raw copy on
    the forward's IDs) against oracle.gather_dequant over the rows the CPU
    generator rebuilds. Returns the number of valid lookups and distinct rows."""
    rid_d = res["row_ids"]
    rid = rid_d.cpu().numpy()
    assert np.array_equal(rid, ref_ids), f"{label}: row ids"
    T = rid.shape[0]
    valid = rid >= 0
    uniq, inv = np.unique(rid[valid], return_inverse=True)
    codes, scales = table.rows_cpu(uniq)
    compact = np.full(rid.shape, -1, np.int32)
    compact[valid] = inv.astype(np.int32)
    x_ref = oracle.gather_dequant(compact, codes, scales)
    assert np.array_equal(host_bits(res["x"]), x_ref), f"{label}: x"
    raw = torch.empty((T, 2, D), dtype=torch.uint8, device=dev)
    x2 = ple.ple_lookup(rid_d, tab, sc, raw=raw)
    assert torch.equal(x2, res["x"]), f"{label}: ple_lookup x differs from the forward's"
    want = np.zeros((T, 2, D), np.uint8)
    want[valid] = codes[inv]
    assert np.array_equal(raw.cpu().numpy(), want), f"{label}: gathered bytes"
    del raw, x2
    return int(valid.sum()), len(uniq)


def boundary_windows(starts, T, pb, seq_of_pos):
    """Windows around every streaming-fuse range start k pb (k >= 1): outputs
    k pb - 3 .. k pb + 3 (clipped to the sequence), as (seq, lo, hi) in
    sequence coordinates; seq_of_pos maps a call position to (seq, offset)."""
    out = []
    for b in range(pb, T, pb):
        s, off = seq_of_pos(b)
        lo = max(0, off - 3)
        hi = min(starts[s + 1] - starts[s], off + 4)
        out.append((s, lo, hi))
        if off < 3 and s > 0:   # the range starts within 3 tokens of a sequence start: the previous one's end
            n = starts[s] - starts[s - 1]
            out.append((s - 1, max(0, n - (3 - off)), n))
    return out


def check_state(st, seqs, W, cw, R, label):
    """Carried conv state (last three v of every sequence of >= 3 tokens)
    against the oracle's within dv (derived bound) and the history IDs."""
    wins = [(s, len(t) - 3, len(t)) for s, (t, _) in enumerate(seqs)]
    ref = oracle_windows(seqs, wins, W, cw, R)
    got = st.conv_state.cpu().numpy().astype(np.float64).reshape(-1, D)
    dv = np.abs(ref["v"] - got)
    assert np.all(dv <= ref["dv"] + 1e-7), f"{label}: conv state off by {np.max(dv - ref['dv']):.3g} over its bound"
    hid = st.hist_ids.cpu().numpy()
    for s, (t, _) in enumerate(seqs):
        assert list(hid[s]) == list(t[-2:]), f"{label}: history of sequence {s}"
    assert np.all(st.hist_len.cpu().numpy() == 2)
    return float(np.max(dv / (ref["dv"] + 1e-30)))


def test_full_table_generator_sample_matches_cpu(dev, full_table):
    tab, sc = full_table
    ids = np.concatenate([np.random.default_rng(11).integers(0, inputs.R_FULL, 10_000),
                          [0, inputs.R_FULL - 1]])
    codes, scales = table.rows_cpu(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(tab[it].cpu().numpy(), codes)
    assert np.array_equal(sc[it].cpu().numpy(), scales)


@pytest.mark.parametrize("name", ["tiny", "prefill", "ragged"])
def test_single_chunk_workloads(dev, full_table, dev_weights, weights, name):
    W, cw = weights
    wl = inputs.make_workload(name)
    if name == "tiny":
        tab, sc = table.table_gpu(wl.R, device=dev)
    else:
        tab, sc = full_table
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    T, S = len(toks), wl.S
    print(f"[{name}] T={T} S={S}", flush=True)
    ws = ple.Workspace(dev)
    st_fast, st_dbg = ple.State(S, dev), ple.State(S, dev)
    res = _run_pair(dev, tab, sc, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                    st_fast, st_dbg, ws)
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((S, 2), np.int32), np.zeros(S, np.int32), wl.R)
    n_look, n_uniq = check_every_token_gather(dev, tab, sc, res, ref_ids, name)
    print(f"[{name}] every token: ids, x, bytes bit-exact ({n_look} lookups, {n_uniq} distinct rows)", flush=True)

    seqs = [(toks[cu[s]:cu[s + 1]], h[cu[s]:cu[s + 1]]) for s in range(S)]
    rng = np.random.default_rng(12)
    wins = []
    for s in ([0] if S == 1 else [0, 1, 2, 31, 62, 63]):
        n = int(cu[s + 1] - cu[s])
        wins += [(s, 0, 4), (s, n - 1, n)] + [(s, p, p + 1) for p in _interior(rng, 4, n - 1, 6)]
    if T > 1024:
        pb = -(-T // STREAM_BLOCKS)
        seq_of_pos = lambda p: (int(np.searchsorted(cu, p, side="right") - 1),
                                int(p - cu[np.searchsorted(cu, p, side="right") - 1]))
        wins += boundary_windows(cu, T, pb, seq_of_pos)
    else:
        wins = [(0, 0, T)]   # tiny: every token
    ref = oracle_windows(seqs, wins, W, cw, wl.R)
    idx = [int(cu[s]) + p for s, lo, hi in wins for p in range(lo, hi)]
    stats = check_samples(gather_debug(res, idx), ref, W, name)
    print(f"[{name}] {len(idx)} outputs in {len(wins)} windows: {stats}", flush=True)
    if name == "tiny":
        # a fresh sequence's first token adds nothing: out == h bit for bit
        assert np.array_equal(host_bits(res["out"][:1])[0], h[0]) and float(res["gate"][0]) == 0.5
    print(f"[{name}] state", check_state(st_fast, seqs, W, cw, wl.R, name), flush=True)


def test_long_context_every_chunk(dev, full_table, dev_weights, weights):
    W, cw = weights
    tab, sc = full_table
    wl = inputs.make_workload("long")
    ws = ple.Workspace(dev)
    st_fast, st_dbg = ple.State(1, dev), ple.State(1, dev)
    all_toks = np.concatenate([c[0] for c in wl.chunks])
    N = len(all_toks)
    ref_ids = oracle.ngram_ids(all_toks, np.array([0, N], np.int32), np.zeros((1, 2), np.int32),
                               np.zeros(1, np.int32), wl.R)
    rng = np.random.default_rng(13)
    hs, got_rows, wins = [], [], []
    pos0 = 0
    for i, (toks, cu) in enumerate(wl.chunks):
        h = wl.hidden(i)
        hs.append(h)
        n = len(toks)
        print(f"[long] chunk {i} at {pos0}", flush=True)
        res = _run_pair(dev, tab, sc, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                        st_fast, st_dbg, ws)
        check_every_token_gather(dev, tab, sc, res, ref_ids[pos0:pos0 + n], f"long chunk {i}")
        pb = -(-n // STREAM_BLOCKS)
        starts = list(range(pb, n, pb))
        if i not in (1, 15):
            starts = sorted(int(v) for v in rng.choice(starts, 16, replace=False))
        cw_ = [(0, pos0, pos0 + 4), (0, pos0 + n - 1, pos0 + n)]     # chunk start (carried state) and end
        cw_ += [(0, pos0 + p, pos0 + p + 1) for p in _interior(rng, 4, n - 1, 4)]
        cw_ += [(0, pos0 + b - 3, pos0 + b + 4) for b in starts]
        wins += cw_
        local = [p - pos0 for _, lo, hi in cw_ for p in range(lo, hi)]
        got_rows.append(gather_debug(res, local))
        pos0 += n
        del res
    h_all = np.concatenate(hs)
    del hs
    ref = oracle_windows([(all_toks, h_all)], wins, W, cw, wl.R)
    got = {k: np.concatenate([g[k] for g in got_rows]) for k in got_rows[0]}
    print("[long]", len(got["x"]), "outputs:", check_samples(got, ref, W, "long"), flush=True)
    print("[long] state", check_state(st_fast, [(all_toks, h_all)], W, cw, wl.R, "long"), flush=True)


def test_decode_64_steps_after_history(dev, full_table, dev_weights, weights):
    W, cw = weights
    tab, sc = full_table
    wl = inputs.make_workload("decode", decode_steps=64)
    S = wl.S
    hist = wl.history[0]                                   # [8][4096]
    hlen = hist.shape[1]
    h_hist = wl.history_hidden(S * hlen)
    ws = ple.Workspace(dev)
    st = ple.State(S, dev)
    cu_h = np.arange(0, S * hlen + 1, hlen, dtype=np.int32)
    print("[decode] history 8 x 4096", flush=True)
    ple.ple_forward(dev_i32(hist.reshape(-1), dev), dev_i32(cu_h, dev), tab, sc, dev_weights[0], dev_weights[1],
                    dev_bf16(h_hist, dev), st, workspace=ws)
    assert np.array_equal(st.hist_ids.cpu().numpy(), hist[:, -2:])
    st_dbg = st.clone()
    st_ip = st.clone()      # the same steps in place (out == h), also one launch
    # the sequences as the oracle sees them: history, then one token per step
    steps_toks = np.stack([c[0] for c in wl.chunks], axis=1)      # [8][64]
    full = np.concatenate([hist, steps_toks], axis=1).astype(np.int32)
    ref_ids = oracle.ngram_ids(full.reshape(-1), np.arange(0, full.size + 1, full.shape[1], dtype=np.int32),
                               np.zeros((S, 2), np.int32), np.zeros(S, np.int32), wl.R).reshape(S, -1, 2)
    hs, check_k, got = [], list(range(0, 64, 8)) + [63], []
    for k, (toks, cu) in enumerate(wl.chunks):
        h = wl.hidden(k)
        hs.append(h)
        res = _run_pair(dev, tab, sc, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                        st, st_dbg, ws)
        h_ip = dev_bf16(h, dev)
        ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1], h_ip, st_ip,
                        out=h_ip, workspace=ws)
        assert np.array_equal(host_bits(h_ip), host_bits(res["out"])), f"decode step {k}: in place"
        check_every_token_gather(dev, tab, sc, res, ref_ids[:, hlen + k], f"decode step {k}")
        if k in check_k:
            got.append(gather_debug(res, np.arange(S)))
    seqs = []
    for s in range(S):
        hh = np.concatenate([h_hist[s * hlen:(s + 1) * hlen], np.stack([hk[s] for hk in hs])])
        seqs.append((full[s], hh))
    wins = [(s, hlen + k, hlen + k + 1) for k in check_k for s in range(S)]
    ref = oracle_windows(seqs, wins, W, cw, wl.R)
    got = {key: np.concatenate([g[key] for g in got]) for key in got[0]}
    print("[decode] steps", check_k, check_samples(got, ref, W, "decode"), flush=True)
    print("[decode] state after 64 steps", check_state(st, seqs, W, cw, wl.R, "decode"), flush=True)
    assert torch.equal(st_ip.conv_state, st.conv_state) and torch.equal(st_ip.hist_ids, st.hist_ids)


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
    T = len(toks)
    st_fast, st_dbg = ple.State(1, dev), ple.State(1, dev)
    res = _run_pair(dev, tab, sc16, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                    st_fast, st_dbg, ple.Workspace(dev), heads=True)
    ref_ids = oracle.ngram_ids_heads(toks, cu, np.zeros((1, 2), np.int32), np.zeros(1, np.int32), R)
    rid_d = res["row_ids"]
    rid = rid_d.cpu().numpy()
    assert np.array_equal(rid, ref_ids)
    # every token: x and the gathered 160-byte rows
    valid = rid >= 0
    head = np.broadcast_to(np.arange(16), rid.shape)
    q = head[valid].astype(np.int64) * R + rid[valid]
    uniq, inv = np.unique(q, return_inverse=True)
    codes, scales = table.slices_cpu(uniq // R, uniq % R, R)
    compact = np.full(rid.shape, -1, np.int32)
    compact[valid] = inv.astype(np.int32)
    assert np.array_equal(host_bits(res["x"]), oracle.gather_dequant_heads(compact, codes, scales))
    raw = torch.empty((T, 16, 160), dtype=torch.uint8, device=dev)
    assert torch.equal(ple.ple_lookup(rid_d, tab, sc16, raw=raw, heads=True), res["x"])
    want = np.zeros((T, 16, 160), np.uint8)
    want[valid] = codes[inv]
    assert np.array_equal(raw.cpu().numpy(), want)
    del raw, want
    pos = sorted(set([0, 1, 2, 3, T - 1] + _interior(rng, 4, T - 1, 8)))
    wins = [(0, p, p + 1) for p in pos] + [(0, b - 3, b + 4) for b in range(128, T, 128 * 16)]
    ref = oracle_windows([(toks, h)], wins, W, cw, R, heads=True)
    idx = [p for _, lo, hi in wins for p in range(lo, hi)]
    print("prefill heads", check_samples(gather_debug(res, idx), ref, W, "prefill heads"))
    del sc16


def test_prefill_nvfp4_table(dev, dev_weights, weights):
    # the NVFP4 table at the full row count: 20,000,096 rows x (1280 code
    # bytes + 160 block scales + 4-byte row scale) = 28.9 GB in HBM
    W, cw = weights
    R = inputs.R_FULL
    codes_d, blocks_d, scales_d = table.nvfp4_gpu(R, device=dev)
    rng = np.random.default_rng(19)
    ids = np.concatenate([rng.integers(0, R, 2000), [0, R - 1]])
    c, b, s = table.nvfp4_rows_cpu(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(codes_d[it].cpu().numpy(), c)
    assert np.array_equal(blocks_d[it].cpu().numpy(), b)
    assert np.array_equal(scales_d[it].cpu().numpy(), s)
    wl = inputs.make_workload("prefill")
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    T = len(toks)
    st_fast, st_dbg = ple.State(1, dev), ple.State(1, dev)
    res = _run_pair(dev, codes_d, scales_d, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                    st_fast, st_dbg, ple.Workspace(dev), nvfp4_blocks=blocks_d)
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((1, 2), np.int32), np.zeros(1, np.int32), R)
    rid_d = res["row_ids"]
    rid = rid_d.cpu().numpy()
    assert np.array_equal(rid, ref_ids)
    valid = rid >= 0
    uniq, inv = np.unique(rid[valid], return_inverse=True)
    c, b, s = table.nvfp4_rows_cpu(uniq)
    compact = np.full(rid.shape, -1, np.int32)
    compact[valid] = inv.astype(np.int32)
    assert np.array_equal(host_bits(res["x"]), oracle.gather_dequant_nvfp4(compact, c, b, s))
    raw = torch.empty((T, 2, D // 2), dtype=torch.uint8, device=dev)
    assert torch.equal(ple.ple_lookup_nvfp4(rid_d, codes_d, blocks_d, scales_d, raw=raw), res["x"])
    want = np.zeros((T, 2, D // 2), np.uint8)
    want[valid] = c[inv]
    assert np.array_equal(raw.cpu().numpy(), want)
    del raw, want
    pos = sorted(set([0, 1, 2, 3, T - 1] + _interior(rng, 4, T - 1, 8)))
    wins = [(0, p, p + 1) for p in pos] + [(0, b_ - 3, b_ + 4) for b_ in range(128, T, 128 * 16)]
    ref = oracle_windows([(toks, h)], wins, W, cw, R, nvfp4=True)
    idx = [p for _, lo, hi in wins for p in range(lo, hi)]
    print("prefill nvfp4", check_samples(gather_debug(res, idx), ref, W, "prefill nvfp4"))
    del res, codes_d, blocks_d, scales_d
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
    ref_ids = oracle.ngram_ids(toks, cu, np.zeros((4, 2), np.int32), np.zeros(4, np.int32), R)
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
        samples += [(s, p, p + 1) for p in pos]
        idx += [a + p for p in pos]
    ref = oracle_windows(seqs, samples, W, cw, R)
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
    st_fast, st_dbg = ple.State(wl.S, dev), ple.State(wl.S, dev)
    res = _run_pair(dev, tab, sc, dev_weights, dev_i32(toks, dev), dev_i32(cu, dev), dev_bf16(h, dev),
                    st_fast, st_dbg, ple.Workspace(dev), **kw)
    assert np.array_equal(res["row_ids"].cpu().numpy(), ref_ids)
    rng = np.random.default_rng(21)
    seqs = [(toks[cu[s]:cu[s + 1]], h[cu[s]:cu[s + 1]]) for s in range(wl.S)]
    wins = []
    for s in (0, 1, 31, 62, 63):
        n = int(cu[s + 1] - cu[s])
        wins += [(s, 0, 4), (s, n - 1, n)] + [(s, p, p + 1) for p in _interior(rng, 4, n - 1, 2)]
        wins += [(s, 61, 68), (s, 125, 132)]     # streaming-fuse range starts (64-token ranges)
    ref = oracle_windows(seqs, wins, W, cw, R, heads=layout == "heads", nvfp4=layout == "nvfp4")
    idx = [int(cu[s]) + p for s, lo, hi in wins for p in range(lo, hi)]
    print("ragged", layout, check_samples(gather_debug(res, idx), ref, W, f"ragged {layout}"))
    del res
    if layout == "nvfp4":
        del codes, blocks
    torch.cuda.empty_cache()
