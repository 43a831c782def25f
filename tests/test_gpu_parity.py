"""GPU parity of every entry point against the CPU oracle at small sizes that
still span several tiles, ragged tails and every sequence-boundary case.
All calls go through the C ABI (libple.so) via the Python binding."""

import numpy as np
import pytest
import torch

import oracle
import sparse_memory_gather_amd as ple
from gen import inputs, table

from parity_util import (D, check_samples, dev_bf16, dev_i32, e_bound, gate_bound, gather_debug, head_rows,
                         host_bits, oracle_samples, oracle_windows, rows, state_bound, y_bound, E_REL, OUT_ATOL,
                         OUT_RTOL)

pytestmark = pytest.mark.gpu

R_SMALL = 65_536


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ple.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def small_table(dev):
    return table.table_gpu(R_SMALL, device=dev)


@pytest.fixture(scope="module")
def dev_weights(dev, weights):
    W, cw = weights
    return dev_bf16(W, dev), dev_bf16(cw, dev)


def _case(seed, lengths, hist_lens, vocab=inputs.VOCAB):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    toks = inputs.uniform_tokens(rng, T, vocab)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S = len(lengths)
    hist = inputs.uniform_tokens(rng, 2 * S, vocab).reshape(S, 2)
    hl = np.array(hist_lens, np.int32)
    h = inputs.normal_bf16(rng, (T, D))
    return toks, cu, hist, hl, h


def test_table_generator_gpu_matches_cpu(dev, small_table):
    tab, sc = small_table
    ids = np.concatenate([np.arange(8), np.random.default_rng(0).integers(0, R_SMALL, 2000),
                          [R_SMALL - 1]])
    codes, scales = rows(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(tab[it].cpu().numpy(), codes)
    assert np.array_equal(sc[it].cpu().numpy(), scales)


def test_hash_parity_sequence_boundaries(dev):
    lengths = [0, 1, 2, 3, 5, 300, 0, 1, 700]
    hl = [0, 0, 1, 2, 0, 1, 2, 2, 2]
    toks, cu, hist, hlen, _ = _case(1, lengths, hl)
    toks[:4] = [0, inputs.VOCAB - 1, 0, inputs.VOCAB - 1]  # vocabulary edges
    # the kernels reduce mod R by multiplying with a precomputed reciprocal:
    # R at 1, 2, 3, powers of two and their neighbours, primes, the full row
    # count and the largest allowed
    for R in (1, 2, 3, 7, 1009, 1 << 16, (1 << 20) - 1, 1 << 30, 20_000_096, 2 ** 31 - 1):
        ref = oracle.ngram_ids(toks, cu, hist, hlen, R)
        got = ple.ple_hash(dev_i32(toks, dev), dev_i32(cu, dev), dev_i32(hist, dev), dev_i32(hlen, dev), R)
        assert np.array_equal(got.cpu().numpy(), ref), R
        ref16 = oracle.ngram_ids_heads(toks, cu, hist, hlen, R)
        got16 = ple.ple_hash(dev_i32(toks, dev), dev_i32(cu, dev), dev_i32(hist, dev), dev_i32(hlen, dev), R,
                             heads=True)
        assert np.array_equal(got16.cpu().numpy(), ref16), R


@pytest.mark.parametrize("R", [1, 3, 1009])
def test_ids_computed_inside_the_gather(dev, dev_weights, R):
    # calls of up to 1024 tokens compute the IDs in the gather kernel
    lengths = [1, 2, 3, 5, 300, 0, 700]
    hl = [0, 1, 2, 0, 1, 2, 2]
    toks, cu, hist, hlen, h = _case(2, lengths, hl)
    tab, sc = table.table_gpu(R, device=dev)
    st = ple.State(len(lengths), dev)
    st.hist_ids.copy_(dev_i32(hist, dev))
    st.hist_len.copy_(dev_i32(hlen, dev))
    res = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    assert np.array_equal(res["row_ids"].cpu().numpy(), oracle.ngram_ids(toks, cu, hist, hlen, R))


def test_lookup_parity_raw_bytes_and_x(dev, small_table):
    tab, sc = small_table
    rng = np.random.default_rng(2)
    T = 333
    ids = rng.integers(-1, R_SMALL, (T, 2)).astype(np.int32)
    ids[ids[:, 0] < 0, 1] = -1
    ids[3] = [-1, -1]
    ids[4] = [17, 17]
    ids[5] = [-1, 9]          # trigram without bigram: only that row
    ids[6] = [R_SMALL - 1, 0]
    raw = torch.empty((T, 2, D), dtype=torch.uint8, device=dev)
    x = ple.ple_lookup(dev_i32(ids, dev), tab, sc, raw=raw)
    uniq = np.unique(ids[ids >= 0])
    codes, scales = rows(uniq)
    remap = np.full(ids.shape, -1, np.int32)
    remap[ids >= 0] = np.searchsorted(uniq, ids[ids >= 0])
    xr, rr = oracle.gather_dequant(remap, codes, scales, raw=True)
    assert np.array_equal(raw.cpu().numpy(), rr)
    assert np.array_equal(host_bits(x), xr)


def test_lookup_decodes_every_e4m3_code(dev):
    # 256 rows; row r holds code r everywhere; scale 1 -> x = bf16(decode(r))
    codes = np.repeat(np.arange(256, dtype=np.uint8)[:, None], D, axis=1)
    tab = torch.from_numpy(codes).to(dev)
    sc = torch.ones(256, dtype=torch.float32, device=dev)
    ids = np.stack([np.arange(256), np.full(256, -1)], axis=1).astype(np.int32)
    x = host_bits(ple.ple_lookup(dev_i32(ids, dev), tab, sc))
    ref = oracle.gather_dequant(ids, codes, np.ones(256, np.float32))
    nan = np.array([c & 0x7F == 0x7F for c in range(256)])
    assert np.array_equal(x[~nan], ref[~nan])
    f = torch.from_numpy(x[nan].view(np.int16)).view(torch.bfloat16).float()
    assert torch.isnan(f).all()


def test_proj_parity_ragged_tail(dev, dev_weights, weights):
    W, _ = weights
    rng = np.random.default_rng(3)
    for T in (1, 37, 300, 513):
        x = inputs.normal_bf16(rng, (T, D), std=0.08)
        e = ple.ple_proj(dev_bf16(x, dev), dev_weights[0]).cpu().numpy().astype(np.float64)
        ref = oracle.project(x, W)
        bound = E_REL * e_bound(x, W) + 1e-7
        assert np.all(np.abs(e - ref) <= bound), T


def _forward(dev, tab, sc, dw, toks, cu, h, state, debug=True, **kw):
    return ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dw[0], dw[1], dev_bf16(h, dev),
                           state, debug=debug, **kw)


def _same_without_debug(dev, tab, sc, dw, toks, cu, h, state_in, res, state_out):
    """The call again without debug outputs (the streaming fuse's fast path
    for steps inside a sequence) on a copy of the incoming state: out and the
    new state must equal the debug run's bit for bit."""
    st = state_in.clone()
    out = _forward(dev, tab, sc, dw, toks, cu, h, st, debug=False)
    assert np.array_equal(host_bits(out), host_bits(res["out"]))
    assert torch.equal(st.conv_state, state_out.conv_state)
    assert torch.equal(st.hist_ids, state_out.hist_ids) and torch.equal(st.hist_len, state_out.hist_len)


def test_forward_tiny_workload_full_parity(dev, small_table, dev_weights, weights):
    W, cw = weights
    tab, sc = small_table
    wl = inputs.make_workload("tiny")
    toks, cu = wl.chunks[0]
    h = wl.hidden(0)
    st = ple.State(1, dev)
    res = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    ref = oracle.forward(toks, cu, h, W, cw, wl.R, rows)
    got = gather_debug(res, np.arange(len(toks)))
    assert np.array_equal(got["row_ids"], ref["row_ids"])
    assert np.array_equal(got["x"], ref["x"])
    # token 0 of a fresh sequence: nothing to add, out == h bit-exactly
    assert np.array_equal(got["out"][0], h[0]) and got["g"][0] == 0.5
    seqs = [(toks, h)]
    samples = [(0, p) for p in range(len(toks))]
    refs = oracle_samples(seqs, samples, W, cw, wl.R)
    check_samples(got, refs, W, "tiny")
    # carried state equals the oracle's (conv state within the derived v bound)
    assert np.array_equal(st.hist_ids.cpu().numpy(), ref["hist_ids"])
    assert np.array_equal(st.hist_len.cpu().numpy(), ref["hist_len"])
    dst = np.abs(st.conv_state.cpu().numpy() - ref["conv_state"])
    assert np.all(dst <= state_bound(ref, cu, cw, W, h))


def test_forward_sequence_edge_cases_with_carried_state(dev, small_table, dev_weights, weights):
    W, cw = weights
    tab, sc = small_table
    lengths = [0, 1, 2, 3, 17, 300, 5, 1]
    hl = [2, 0, 1, 2, 0, 1, 2, 1]
    toks, cu, hist, hlen, h = _case(4, lengths, hl)
    S = len(lengths)
    rng = np.random.default_rng(5)
    state0 = (0.05 * rng.standard_normal((S, 3, D))).astype(np.float32)
    st = ple.State(S, dev)
    st.hist_ids.copy_(dev_i32(hist, dev))
    st.hist_len.copy_(dev_i32(hlen, dev))
    st.conv_state.copy_(torch.from_numpy(state0).to(dev))
    res = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    ref = oracle.forward(toks, cu, h, W, cw, R_SMALL, rows, hist, hlen, state0.astype(np.float64))
    got = gather_debug(res, np.arange(len(toks)))
    assert np.array_equal(got["row_ids"], ref["row_ids"])
    assert np.array_equal(got["x"], ref["x"])
    out = inputs.bf16_bits_to_f32(got["out"]).astype(np.float64)
    assert np.all(np.abs(out - ref["out"]) <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"]))
    assert np.all(np.abs(got["g"] - ref["g"]) <= gate_bound(ref, h, W))
    assert np.all(np.abs(got["y"] - ref["y"]) <= y_bound(ref, cu, cw, state0.astype(np.float64), W, h))
    hid = st.hist_ids.cpu().numpy()
    hln = st.hist_len.cpu().numpy()
    assert np.array_equal(hln, ref["hist_len"])
    for s in range(S):
        k = ref["hist_len"][s]
        assert np.array_equal(hid[s][2 - k:], ref["hist_ids"][s][2 - k:]), s
    # conv state: v of this call within the derived bound, carried values
    # (sequences of fewer than three tokens shift them) bit for bit
    dst = np.abs(st.conv_state.cpu().numpy() - ref["conv_state"])
    assert np.all(dst <= state_bound(ref, cu, cw, W, h))
    # the empty sequence 0 keeps its state bit-exactly
    assert np.array_equal(st.conv_state[0].cpu().numpy(), state0[0])


def test_chunked_equals_unchunked_and_decode_equals_prefill(dev, small_table, dev_weights):
    tab, sc = small_table
    rng = np.random.default_rng(6)
    n = 270
    toks = inputs.uniform_tokens(rng, n)
    h = inputs.normal_bf16(rng, (n, D))

    def run(cuts):
        st = ple.State(1, dev)
        outs, pos = [], 0
        for L in cuts:
            r = _forward(dev, tab, sc, dev_weights, toks[pos:pos + L], np.array([0, L], np.int32),
                         h[pos:pos + L], st)
            outs.append(host_bits(r["out"]))
            pos += L
        return np.concatenate(outs), st.conv_state.cpu().numpy(), st.hist_ids.cpu().numpy()

    full = run([n])
    # pieces of up to 256 tokens run the small-T projection (16 feature rows
    # per block for 1-32 tokens, 32 rows and 1, 2 or 4 token tiles per block
    # above), 257 and more the mid-size one
    for cuts in ([1, 2, 3, 264], [256, 14], [100, 0, 170], [1] * 20 + [250], [40, 64, 33, 32, 101],
                 [150, 120], [200, 70]):
        got = run(cuts)
        for a, b in zip(got, full):
            assert np.array_equal(a, b), cuts


def test_kernel_variants_agree_bit_exactly(dev, small_table, dev_weights):
    # a 4000-token call runs the tiled projection, the ID kernel and the
    # streaming fuse; its pieces run, by size, the mid-size projection (257-
    # 3200 tokens, both ends included), the tiled one again (3201 and more),
    # the small-T one (<= 256), IDs computed in the gather and the one-token
    # fuse (<= 1024): every output and the carried state must match bit for
    # bit
    tab, sc = small_table
    rng = np.random.default_rng(16)
    n = 4000
    toks = inputs.uniform_tokens(rng, n)
    h = inputs.normal_bf16(rng, (n, D))

    def run(cuts):
        st = ple.State(1, dev)
        outs, pos = [], 0
        for L in cuts:
            r = _forward(dev, tab, sc, dev_weights, toks[pos:pos + L], np.array([0, L], np.int32),
                         h[pos:pos + L], st)
            outs.append(host_bits(r["out"]))
            pos += L
        return np.concatenate(outs), st.conv_state.cpu().numpy(), st.hist_ids.cpu().numpy()

    full = run([n])
    for cuts in ([1024, 2976], [1500, 2500], [200, 1100, 2700], [3, 3997], [257, 3200, 543], [3201, 799]):
        assert sum(cuts) == n
        got = run(cuts)
        for a, b in zip(got, full):
            assert np.array_equal(a, b), cuts


def test_projection_tilings_agree_bit_exactly(dev, small_table, dev_weights):
    # an 8100-token call runs the 256 x 320 tiling (its last token tile has
    # 164 tokens); its halves run the 256 x 256 one, a 3200-token piece the
    # mid-size one and a 1-token piece the small-T one: outputs and the carried
    # state must match bit for bit
    tab, sc = small_table
    rng = np.random.default_rng(17)
    n = 8100
    toks = inputs.uniform_tokens(rng, n)
    h = inputs.normal_bf16(rng, (n, D))
    assert ple.proj_tiling(n) == "proj_w320_kernel" and ple.proj_tiling(n // 2) == "proj_kernel"

    def run(cuts):
        st = ple.State(1, dev)
        outs, pos = [], 0
        for L in cuts:
            r = _forward(dev, tab, sc, dev_weights, toks[pos:pos + L], np.array([0, L], np.int32),
                         h[pos:pos + L], st)
            outs.append(host_bits(r["out"]))
            pos += L
        return np.concatenate(outs), st.conv_state.cpu().numpy(), st.hist_ids.cpu().numpy()

    full = run([n])
    for cuts in ([4050, 4050], [3200, 4900], [8099, 1]):
        assert sum(cuts) == n
        got = run(cuts)
        for a, b in zip(got, full):
            assert np.array_equal(a, b), cuts


@pytest.mark.parametrize("lengths", [[3000], [1500, 1, 2595]])
def test_mid_size_tilings_against_oracle(dev, small_table, dev_weights, weights, lengths):
    # a call of 257-3200 tokens runs the 128-token tiles of the projection
    # and one of 3201-6400 tokens (4096 here) the 256 x 256 tiles: e, g, y and
    # out against the oracle at every sequence's first and last tokens,
    # random interior tokens and every 16th block-range start of the
    # streaming fuse, and the carried conv state of every sequence
    W, cw = weights
    tab, sc = small_table
    toks, cu, hist, hlen, h = _case(301 + len(lengths), lengths, [0] * len(lengths))
    T, S = int(cu[-1]), len(lengths)
    assert ple.proj_tiling(T) == ("proj_mid_kernel" if T <= 3200 else "proj_kernel")
    st = ple.State(S, dev)
    res = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    _same_without_debug(dev, tab, sc, dev_weights, toks, cu, h, ple.State(S, dev), res, st)
    seqs = [(toks[cu[s]:cu[s + 1]], h[cu[s]:cu[s + 1]]) for s in range(S)]
    rng = np.random.default_rng(303)
    wins = []
    for s in range(S):
        n = int(cu[s + 1] - cu[s])
        wins += [(s, 0, min(4, n)), (s, max(0, n - 4), n)]
        wins += [(s, int(p), int(p) + 1) for p in sorted(set(rng.integers(0, n, 6).tolist()))]
    pb = -(-T // 256)
    for b in range(pb, T, 16 * pb):
        s = int(np.searchsorted(cu, b, side="right") - 1)
        off = b - int(cu[s])
        wins.append((s, max(0, off - 3), min(int(cu[s + 1] - cu[s]), off + 4)))
    ref = oracle_windows(seqs, wins, W, cw, R_SMALL)
    idx = [int(cu[s]) + p for s, lo, hi in wins for p in range(lo, hi)]
    check_samples(gather_debug(res, idx), ref, W, f"T={T}")
    # the carried state: the last three v of each sequence of 3 or more tokens
    full = [s for s in range(S) if cu[s + 1] - cu[s] >= 3]
    sref = oracle_windows(seqs, [(s, int(cu[s + 1] - cu[s]) - 3, int(cu[s + 1] - cu[s])) for s in full],
                          W, cw, R_SMALL)
    got = st.conv_state.cpu().numpy().astype(np.float64)[full].reshape(-1, D)
    assert np.all(np.abs(sref["v"] - got) <= sref["dv"] + 1e-7)


def test_streaming_fuse_equals_per_sequence_calls(dev, small_table, dev_weights):
    # one 1380-token call of fourteen sequences (three empty, which must keep
    # their state) with carried state runs the streaming fuse (block ranges of
    # 8 tokens cross sequence starts and ends); each sequence alone (<= 1024
    # tokens) runs the one-token fuse and the small-T projection: outputs,
    # gates and the new state must be equal
    tab, sc = small_table
    lengths = [1, 2, 0, 3, 5, 40, 33, 700, 0, 31, 500, 1, 64, 0]
    hl = [0, 1, 2, 2, 2, 0, 2, 1, 1, 2, 2, 2, 0, 2]
    toks, cu, hist, hlen, h = _case(91, lengths, hl)
    S = len(lengths)
    rng = np.random.default_rng(92)
    state0 = (rng.standard_normal((S, 3, D)) * 0.5).astype(np.float32)
    state0[np.array(hl) == 0] = 0.0

    def fresh(sl):
        st = ple.State(len(range(*sl.indices(S))), dev)
        st.hist_ids.copy_(dev_i32(hist[sl], dev))
        st.hist_len.copy_(dev_i32(hlen[sl], dev))
        st.conv_state.copy_(torch.from_numpy(state0[sl]).to(dev))
        return st

    st = fresh(slice(0, S))
    whole = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    _same_without_debug(dev, tab, sc, dev_weights, toks, cu, h, fresh(slice(0, S)), whole, st)
    for i in range(S):
        a, b = int(cu[i]), int(cu[i + 1])
        si = fresh(slice(i, i + 1))
        one = _forward(dev, tab, sc, dev_weights, toks[a:b], np.array([0, b - a], np.int32), h[a:b], si)
        assert np.array_equal(host_bits(one["out"]), host_bits(whole["out"][a:b])), i
        assert torch.equal(one["gate"], whole["gate"][a:b]), i
        assert torch.equal(one["y"], whole["y"][a:b]), i
        assert torch.equal(si.conv_state[0], st.conv_state[i]), i
        assert torch.equal(si.hist_ids[0], st.hist_ids[i]) and torch.equal(si.hist_len[0], st.hist_len[i]), i


@pytest.mark.parametrize("T,lengths", [(1000, [1000]), (4000, [1500, 1, 2499]), (9000, [9000])])
def test_in_place_equals_out_of_place_both_fuse_kernels(dev, small_table, dev_weights, T, lengths):
    # out == h: the h rows a block reads but does not own come from a copy
    # taken before the fuse (1000 tokens: one-token fuse, all of h; longer:
    # streaming fuse, three rows per block range)
    tab, sc = small_table
    rng = np.random.default_rng(T)
    toks = inputs.uniform_tokens(rng, T)
    h = inputs.normal_bf16(rng, (T, D))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S = len(lengths)
    ref = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), ple.State(S, dev))
    hd = dev_bf16(h, dev)
    st = ple.State(S, dev)
    out = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                          hd, st, out=hd)
    assert out.data_ptr() == hd.data_ptr()
    assert np.array_equal(host_bits(hd), host_bits(ref))


@pytest.mark.parametrize("T", [8, 300, 2000])
def test_forward_flags_bad_inputs_on_the_device(dev, small_table, dev_weights, T):
    # 8 tokens: the one-launch kernel; 300 tokens: IDs computed inside the
    # gather, one-token fuse; 2000: the ID kernel and the streaming fuse.
    # Bad values the host cannot see are
    # flagged in dev_err (1: token ID outside the vocabulary, 4: hist_len
    # outside 0..2, 2: malformed cu_seqlens) and every kernel stays in bounds.
    tab, sc = small_table
    rng = np.random.default_rng(T)
    h = dev_bf16(inputs.normal_bf16(rng, (T, D)), dev)

    def run(toks, cu, hist_len):
        st = ple.State(len(cu) - 1, dev)
        st.hist_len.copy_(dev_i32(hist_len, dev))
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1], h,
                              st, dev_err=err)
        torch.cuda.synchronize()
        return int(err.item()), out

    toks = inputs.uniform_tokens(rng, T)
    good_cu = np.array([0, T // 2, T], np.int32)
    assert run(toks, good_cu, [0, 0])[0] == 0
    bad = toks.copy()
    bad[T // 3] = inputs.VOCAB + 7
    assert run(bad, good_cu, [0, 0])[0] == 1
    assert run(toks, good_cu, [0, 5])[0] == 4
    err, out = run(toks, np.array([0, T // 2, T // 4, T - 1], np.int32), [0, 0, 0])
    assert err == 2
    assert out.shape == (T, D)


def test_prepared_forward_reuses_its_buffers(dev, small_table, dev_weights):
    # a prepared call run on fixed buffers whose contents change between
    # steps (a decode loop) equals ple_forward on each step's inputs
    tab, sc = small_table
    rng = np.random.default_rng(33)
    S = 8
    cu = dev_i32(np.arange(S + 1), dev)
    toks_buf = torch.empty(S, dtype=torch.int32, device=dev)
    h_buf = torch.empty((S, D), dtype=torch.bfloat16, device=dev)
    st_a, st_b = ple.State(S, dev), ple.State(S, dev)
    call = ple.Forward(toks_buf, cu, tab, sc, dev_weights[0], dev_weights[1], h_buf, st_a)
    for step in range(4):
        toks = inputs.uniform_tokens(rng, S)
        h = inputs.normal_bf16(rng, (S, D))
        toks_buf.copy_(dev_i32(toks, dev))
        h_buf.copy_(dev_bf16(h, dev))
        got = host_bits(call())
        want = host_bits(ple.ple_forward(dev_i32(toks, dev), cu, tab, sc, dev_weights[0], dev_weights[1],
                                         dev_bf16(h, dev), st_b))
        assert np.array_equal(got, want), step
    assert torch.equal(st_a.conv_state, st_b.conv_state) and torch.equal(st_a.hist_ids, st_b.hist_ids)


@pytest.mark.parametrize("T,S", [(8, 8), (1300, 2), (8192, 4)])
def test_graph_captured_forward_replays_like_eager(dev, small_table, dev_weights, T, S):
    # a prepared call captured into a HIP graph (nothing in the path records a
    # memset) and replayed three times, with eager work and synchronizations
    # in between, advances the state exactly as three eager calls do
    tab, sc = small_table
    rng = np.random.default_rng(T)
    toks = dev_i32(inputs.uniform_tokens(rng, T), dev)
    cu = dev_i32(np.linspace(0, T, S + 1).astype(np.int32), dev)
    h = dev_bf16(inputs.normal_bf16(rng, (T, D)), dev)
    st_g, st_e = ple.State(S, dev), ple.State(S, dev)
    out_g = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    call = ple.Forward(toks, cu, tab, sc, dev_weights[0], dev_weights[1], h, st_g, out=out_g)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call()                                   # warm-up outside the graph
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    st_g.hist_ids.zero_()
    st_g.hist_len.zero_()
    st_g.conv_state.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    # capture does not run the work: the state is still fresh
    assert int(st_g.hist_len.abs().sum().item()) == 0
    for rep in range(3):
        g.replay()
        want = ple.ple_forward(toks, cu, tab, sc, dev_weights[0], dev_weights[1], h, st_e)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out_g), host_bits(want)), rep
        assert torch.equal(st_g.conv_state, st_e.conv_state) and torch.equal(st_g.hist_ids, st_e.hist_ids), rep
        _ = torch.randn(1000, device=dev).sum().item()   # unrelated eager work between replays



def test_graph_captured_in_place_one_launch_replays_like_eager(dev, small_table, dev_weights):
    # a short call in place (out == h): one launch, whose finishers read the
    # earlier tokens' h rows from the copy the projection blocks take;
    # captured once and replayed three times against three eager calls
    tab, sc = small_table
    T, S = 16, 4
    assert ple.one_launch(T, S)
    rng = np.random.default_rng(31)
    toks = dev_i32(inputs.uniform_tokens(rng, T), dev)
    cu = dev_i32(np.array([0, 1, 6, 10, 16], np.int32), dev)
    h0 = dev_bf16(inputs.normal_bf16(rng, (T, D)), dev)
    h_g, h_e = h0.clone(), h0.clone()
    st_g, st_e = ple.State(S, dev), ple.State(S, dev)
    call = ple.Forward(toks, cu, tab, sc, dev_weights[0], dev_weights[1], h_g, st_g, out=h_g)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call()                                   # warm-up outside the graph
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    h_g.copy_(h0)
    st_g.hist_ids.zero_()
    st_g.hist_len.zero_()
    st_g.conv_state.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    assert torch.equal(h_g, h0)                  # capture does not run the work
    for rep in range(3):
        g.replay()
        ple.ple_forward(toks, cu, tab, sc, dev_weights[0], dev_weights[1], h_e, st_e, out=h_e)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(h_g), host_bits(h_e)), rep
        assert torch.equal(st_g.conv_state, st_e.conv_state) and torch.equal(st_g.hist_ids, st_e.hist_ids), rep
        _ = torch.randn(1000, device=dev).sum().item()   # unrelated eager work between replays

def test_in_place_out_equals_h(dev, small_table, dev_weights):
    tab, sc = small_table
    rng = np.random.default_rng(7)
    toks = inputs.uniform_tokens(rng, 300)
    h = inputs.normal_bf16(rng, (300, D))
    cu = np.array([0, 120, 300], np.int32)
    ref = _forward(dev, tab, sc, dev_weights, toks, cu, h, ple.State(2, dev))
    hd = dev_bf16(h, dev)
    out = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                          hd, ple.State(2, dev), out=hd)
    assert out.data_ptr() == hd.data_ptr()
    assert np.array_equal(host_bits(hd), host_bits(ref["out"]))


def test_save_restore_state_resumes_identically(dev, small_table, dev_weights):
    tab, sc = small_table
    rng = np.random.default_rng(8)
    toks = inputs.uniform_tokens(rng, 64)
    h = inputs.normal_bf16(rng, (64, D))
    cu = np.array([0, 32], np.int32)
    st = ple.State(1, dev)
    _forward(dev, tab, sc, dev_weights, toks[:32], cu, h[:32], st)
    saved = st.clone()
    a = _forward(dev, tab, sc, dev_weights, toks[32:], cu, h[32:], st)
    b = _forward(dev, tab, sc, dev_weights, toks[32:], cu, h[32:], saved)
    assert np.array_equal(host_bits(a["out"]), host_bits(b["out"]))
    assert torch.equal(st.conv_state, saved.conv_state)


# ---------------------------------------------------------------------------
# 16-lookup layout (16 head tables of 160-byte rows)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_head_scales(dev):
    return table.head_scales_gpu(R_SMALL, device=dev)


def test_heads_scales_generator_gpu_matches_cpu(dev, small_head_scales):
    rng = np.random.default_rng(50)
    hs, rs = rng.integers(0, 16, 3000), rng.integers(0, R_SMALL, 3000)
    _, want = table.slices_cpu(hs, rs, R_SMALL)
    got = small_head_scales[torch.as_tensor(hs, device=dev), torch.as_tensor(rs, device=dev)].cpu().numpy()
    assert np.array_equal(got, want)


def test_heads_hash_lookup_bit_exact(dev, small_table, small_head_scales):
    tab, _ = small_table
    lengths = [0, 1, 2, 3, 5, 129, 1, 300]
    hl = [2, 0, 1, 2, 0, 1, 2, 0]
    toks, cu, hist, hlen, _ = _case(51, lengths, hl)
    rid = ple.ple_hash(dev_i32(toks, dev), dev_i32(cu, dev), dev_i32(hist, dev), dev_i32(hlen, dev),
                       R_SMALL, heads=True)
    ref_ids = oracle.ngram_ids_heads(toks, cu, hist, hlen, R_SMALL)
    assert np.array_equal(rid.cpu().numpy(), ref_ids)
    T = len(toks)
    raw = torch.empty((T, 16, 160), dtype=torch.uint8, device=dev)
    x = ple.ple_lookup(rid, tab, small_head_scales, raw=raw, heads=True)
    heads = np.broadcast_to(np.arange(16), ref_ids.shape)
    valid = ref_ids >= 0
    q = heads[valid] * R_SMALL + ref_ids[valid]
    uniq, inv = np.unique(q, return_inverse=True)
    codes, scales = head_rows(R_SMALL)(uniq // R_SMALL, uniq % R_SMALL)
    compact = np.full(ref_ids.shape, -1, np.int32)
    compact[valid] = inv
    want_x, want_raw = oracle.gather_dequant_heads(compact, codes, scales, raw=True)
    assert np.array_equal(raw.cpu().numpy(), want_raw)
    assert np.array_equal(host_bits(x), want_x)


def test_heads_lookup_out_of_range_ids_flagged_and_zero(dev, small_table, small_head_scales):
    tab, _ = small_table
    ids = np.full((4, 16), 7, np.int32)
    ids[1, 3] = R_SMALL          # out of range -> treated as missing, flagged
    ids[2, 15] = -5              # below -1 -> same
    ids[3, :] = -1               # all missing -> x = +0
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    x = host_bits(ple.ple_lookup(dev_i32(ids, dev), tab, small_head_scales, dev_err=err, heads=True))
    assert err.item() & 8
    assert np.all(x[1, 480:640] == 0) and np.all(x[2, 2400:2560] == 0) and np.all(x[3] == 0)
    assert np.any(x[1, :480] != 0)


def test_heads_forward_parity_with_edge_cases(dev, small_table, small_head_scales, dev_weights, weights):
    W, cw = weights
    tab, _ = small_table
    lengths = [1, 2, 3, 40, 300, 4]
    hl = [0, 1, 2, 2, 0, 1]
    toks, cu, hist, hlen, h = _case(52, lengths, hl)
    S = len(lengths)
    st = ple.State(S, dev)
    st.hist_ids.copy_(dev_i32(hist, dev))
    st.hist_len.copy_(dev_i32(hlen, dev))
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, small_head_scales, dev_weights[0],
                          dev_weights[1], dev_bf16(h, dev), st, debug=True, heads=True)
    ref = oracle.forward_heads(toks, cu, h, W, cw, R_SMALL, head_rows(R_SMALL), hist, hlen)
    got = gather_debug(res, np.arange(len(toks)))
    assert np.array_equal(got["row_ids"], ref["row_ids"])
    assert np.array_equal(got["x"], ref["x"])
    out = inputs.bf16_bits_to_f32(got["out"]).astype(np.float64)
    assert np.all(np.abs(out - ref["out"]) <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"]))
    assert np.all(np.abs(got["g"] - ref["g"]) <= gate_bound(ref, h, W))
    assert np.all(np.abs(got["y"] - ref["y"]) <= y_bound(ref, cu, cw, np.zeros((S, 3, D)), W, h))
    assert np.array_equal(st.hist_len.cpu().numpy(), ref["hist_len"])
    np.testing.assert_allclose(st.conv_state.cpu().numpy(), ref["conv_state"], rtol=2e-2, atol=1e-4)
    # tokens whose four conv taps lie in this chunk, through the shared checker
    # (e, bf16 flips, g, y, out); each becomes its own short oracle segment
    seqs, samples, idx = [], [], []
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        full = np.concatenate([hist[s][2 - hl[s]:], toks[a:b]]).astype(np.int32)
        hh = np.concatenate([np.zeros((hl[s], D), np.uint16), h[a:b]])
        seqs.append((full, hh))
        samples += [(s, hl[s] + p) for p in range(3, b - a)]
        idx += [a + p for p in range(3, b - a)]
    refs = oracle_samples(seqs, samples, W, cw, R_SMALL, heads=True)
    check_samples(gather_debug(res, idx), refs, W, "heads")


# ---------------------------------------------------------------------------
# ID-ahead form: rows gathered on another stream, ple_forward_x consumes x
# ---------------------------------------------------------------------------

def test_forward_x_pipelined_equals_forward(dev, small_table, dev_weights):
    # chunk i+1's IDs and rows are computed on a side stream while chunk i
    # runs; the history each chunk starts from comes from the token stream
    tab, sc = small_table
    rng = np.random.default_rng(60)
    cuts = [1, 300, 2, 517, 64]
    n = sum(cuts)
    toks = inputs.uniform_tokens(rng, n)
    h = inputs.normal_bf16(rng, (n, D))

    st_ref = ple.State(1, dev)
    ref, pos = [], 0
    for L in cuts:
        ref.append(host_bits(ple.ple_forward(dev_i32(toks[pos:pos + L], dev), dev_i32([0, L], dev), tab, sc,
                                             dev_weights[0], dev_weights[1], dev_bf16(h[pos:pos + L], dev),
                                             st_ref)))
        pos += L

    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream(dev)
    st = ple.State(1, dev)
    chunks, pos = [], 0
    for L in cuts:
        k = min(2, pos)
        hist = np.zeros((1, 2), np.int32)
        hist[0, 2 - k:] = toks[pos - k:pos]
        chunks.append(dict(t=dev_i32(toks[pos:pos + L], dev), cu=dev_i32([0, L], dev),
                           hist=dev_i32(hist, dev), hl=dev_i32([k], dev), h=dev_bf16(h[pos:pos + L], dev)))
        pos += L
    torch.cuda.synchronize()
    xs, ready = [], []
    for c in chunks:   # all rows ahead, on the side stream
        with torch.cuda.stream(side):
            rid = ple.ple_hash(c["t"], c["cu"], c["hist"], c["hl"], R_SMALL)
            xs.append(ple.ple_lookup(rid, tab, sc))
            ev = torch.cuda.Event()
            ev.record(side)
            ready.append(ev)
    outs = []
    for c, x, ev in zip(chunks, xs, ready):
        main.wait_event(ev)
        outs.append(ple.ple_forward_x(x, c["t"], c["cu"], dev_weights[0], dev_weights[1], c["h"], st))
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert np.array_equal(host_bits(a), b)
    assert torch.equal(st.conv_state, st_ref.conv_state)
    assert torch.equal(st.hist_ids, st_ref.hist_ids) and torch.equal(st.hist_len, st_ref.hist_len)


def test_forward_x_with_several_sequences_and_debug_outputs(dev, small_table, dev_weights):
    tab, sc = small_table
    lengths = [0, 3, 40, 1, 290]
    toks, cu, hist, hlen, h = _case(61, lengths, [2, 1, 0, 2, 1])
    S = len(lengths)
    st_a, st_b = ple.State(S, dev), ple.State(S, dev)
    for st in (st_a, st_b):
        st.hist_ids.copy_(dev_i32(hist, dev))
        st.hist_len.copy_(dev_i32(hlen, dev))
    a = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                        dev_bf16(h, dev), st_a, debug=True)
    rid = ple.ple_hash(dev_i32(toks, dev), dev_i32(cu, dev), st_b.hist_ids, st_b.hist_len, R_SMALL)
    x = ple.ple_lookup(rid, tab, sc)
    b = ple.ple_forward_x(x, dev_i32(toks, dev), dev_i32(cu, dev), dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), st_b, debug=True)
    for k in ("out", "e", "gate", "y"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(st_a.conv_state, st_b.conv_state) and torch.equal(st_a.hist_ids, st_b.hist_ids)


def test_forward_x_against_oracle(dev, small_table, dev_weights, weights):
    # rows gathered ahead (ple_hash + ple_lookup with the carried history),
    # then ple_forward_x: e, g, y, out and the updated state against the
    # oracle's forward over the same chunk, with carried history and conv
    # state, empty and one- and two-token sequences; the same call is made
    # twice, with and without debug outputs (over 1024 tokens: the streaming
    # fuse, whose no-debug path differs), and must agree bit for bit
    W, cw = weights
    tab, sc = small_table
    for lengths, hls in (([0, 1, 2, 3, 40, 290], [2, 1, 2, 0, 1, 2]),
                         ([2, 0, 700, 1, 5, 333, 64], [1, 2, 2, 0, 2, 1, 2])):
        toks, cu, hist, hlen, h = _case(62 + len(lengths), lengths, hls)
        S = len(lengths)
        rng = np.random.default_rng(63)
        state0 = (0.3 * rng.standard_normal((S, 3, D))).astype(np.float32)
        state0[np.array(hls) == 0] = 0.0
        st = ple.State(S, dev)
        st.hist_ids.copy_(dev_i32(hist, dev))
        st.hist_len.copy_(dev_i32(hlen, dev))
        st.conv_state.copy_(torch.from_numpy(state0).to(dev))
        st_fast = st.clone()
        rid = ple.ple_hash(dev_i32(toks, dev), dev_i32(cu, dev), st.hist_ids, st.hist_len, R_SMALL)
        x = ple.ple_lookup(rid, tab, sc)
        res = ple.ple_forward_x(x, dev_i32(toks, dev), dev_i32(cu, dev), dev_weights[0], dev_weights[1],
                                dev_bf16(h, dev), st, debug=True)
        out_fast = ple.ple_forward_x(x, dev_i32(toks, dev), dev_i32(cu, dev), dev_weights[0], dev_weights[1],
                                     dev_bf16(h, dev), st_fast)
        assert np.array_equal(host_bits(out_fast), host_bits(res["out"]))
        assert torch.equal(st_fast.conv_state, st.conv_state)
        ref = oracle.forward(toks, cu, h, W, cw, R_SMALL, rows, hist, hlen, state0.astype(np.float64))
        assert np.array_equal(rid.cpu().numpy(), ref["row_ids"])
        assert np.array_equal(host_bits(x), ref["x"])
        e = res["e"].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(e - ref["e"]) <= E_REL * e_bound(ref["x"], W) + 1e-7)
        assert np.all(np.abs(res["gate"].cpu().numpy() - ref["g"]) <= gate_bound(ref, h, W))
        s64 = state0.astype(np.float64)
        assert np.all(np.abs(res["y"].cpu().numpy() - ref["y"]) <= y_bound(ref, cu, cw, s64, W, h))
        out = inputs.bf16_bits_to_f32(host_bits(res["out"])).astype(np.float64)
        assert np.all(np.abs(out - ref["out"]) <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"]))
        assert np.array_equal(st.hist_len.cpu().numpy(), ref["hist_len"])
        hid = st.hist_ids.cpu().numpy()
        for s_ in range(S):
            k = ref["hist_len"][s_]
            assert np.array_equal(hid[s_][2 - k:], ref["hist_ids"][s_][2 - k:]), s_
        dst = np.abs(st.conv_state.cpu().numpy() - ref["conv_state"])
        assert np.all(dst <= state_bound(ref, cu, cw, W, h))
        assert np.array_equal(st.conv_state[lengths.index(0)].cpu().numpy(), state0[lengths.index(0)])


# ---------------------------------------------------------------------------
# NVFP4 table (E2M1 codes, E4M3 per 16 elements, fp32 row scale)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_nvfp4(dev):
    return table.nvfp4_gpu(R_SMALL, device=dev)


def test_nvfp4_generator_gpu_matches_cpu(dev, small_nvfp4):
    codes, blocks, scales = small_nvfp4
    ids = np.concatenate([np.arange(4), np.random.default_rng(80).integers(0, R_SMALL, 1500), [R_SMALL - 1]])
    c, b, s = table.nvfp4_rows_cpu(ids)
    it = torch.as_tensor(ids, device=dev)
    assert np.array_equal(codes[it].cpu().numpy(), c)
    assert np.array_equal(blocks[it].cpu().numpy(), b)
    assert np.array_equal(scales[it].cpu().numpy(), s)


def test_nvfp4_lookup_bit_exact_with_missing_and_bad_ids(dev, small_nvfp4):
    codes, blocks, scales = small_nvfp4
    rng = np.random.default_rng(81)
    ids = rng.integers(0, R_SMALL, (333, 2)).astype(np.int32)
    ids[rng.random((333, 2)) < 0.1] = -1
    ids[5] = [-1, -1]
    ids[7, 1] = R_SMALL + 3         # out of range: treated as missing, flagged
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    raw = torch.empty((333, 2, 1280), dtype=torch.uint8, device=dev)
    x = ple.ple_lookup_nvfp4(dev_i32(ids, dev), codes, blocks, scales, raw=raw, dev_err=err)
    assert err.item() & 8
    ref_ids = ids.copy()
    ref_ids[7, 1] = -1
    valid = ref_ids[ref_ids >= 0]
    uniq, inv = np.unique(valid, return_inverse=True)
    c, b, s = table.nvfp4_rows_cpu(uniq)
    compact = np.full(ref_ids.shape, -1, np.int32)
    compact[ref_ids >= 0] = inv
    want_x, want_raw = oracle.gather_dequant_nvfp4(compact, c, b, s, raw=True)
    assert np.array_equal(host_bits(x), want_x)
    assert np.array_equal(raw.cpu().numpy(), want_raw)


def test_nvfp4_forward_parity_with_edge_cases(dev, small_nvfp4, dev_weights, weights):
    W, cw = weights
    codes, blocks, scales = small_nvfp4
    lengths = [1, 2, 3, 40, 300, 4]
    hl = [0, 1, 2, 2, 0, 1]
    toks, cu, hist, hlen, h = _case(82, lengths, hl)
    S = len(lengths)
    st = ple.State(S, dev)
    st.hist_ids.copy_(dev_i32(hist, dev))
    st.hist_len.copy_(dev_i32(hlen, dev))
    res = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), codes, scales, dev_weights[0], dev_weights[1],
                          dev_bf16(h, dev), st, debug=True, nvfp4_blocks=blocks)
    ref = oracle.forward_nvfp4(toks, cu, h, W, cw, R_SMALL, table.nvfp4_rows_cpu, hist, hlen)
    got = gather_debug(res, np.arange(len(toks)))
    assert np.array_equal(got["row_ids"], ref["row_ids"])
    assert np.array_equal(got["x"], ref["x"])
    out = inputs.bf16_bits_to_f32(got["out"]).astype(np.float64)
    assert np.all(np.abs(out - ref["out"]) <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"]))
    assert np.all(np.abs(got["g"] - ref["g"]) <= gate_bound(ref, h, W))
    assert np.all(np.abs(got["y"] - ref["y"]) <= y_bound(ref, cu, cw, np.zeros((S, 3, D)), W, h))
    eb = e_bound(ref["x"], W)
    assert np.all(np.abs(got["e"].astype(np.float64) - ref["e"]) <= E_REL * eb + 1e-7)
    assert np.array_equal(st.hist_len.cpu().numpy(), ref["hist_len"])
    np.testing.assert_allclose(st.conv_state.cpu().numpy(), ref["conv_state"], rtol=2e-2, atol=1e-4)


@pytest.mark.parametrize("layout", ["heads", "nvfp4"])
def test_other_layouts_chunked_equals_unchunked(dev, small_table, small_head_scales, small_nvfp4, dev_weights,
                                                layout):
    # calls of up to 1024 tokens compute the row IDs inside the gather, longer
    # ones run the ID kernel: the 16-lookup and NVFP4 paths must agree bit
    # for bit across the switch, state included
    rng = np.random.default_rng(40)
    n = 1300
    toks = inputs.uniform_tokens(rng, n)
    h = inputs.normal_bf16(rng, (n, D))
    if layout == "heads":
        tab, sc, kw = small_table[0], small_head_scales, dict(heads=True)
    else:
        tab, sc, kw = small_nvfp4[0], small_nvfp4[2], dict(nvfp4_blocks=small_nvfp4[1])

    def run(cuts):
        st = ple.State(1, dev)
        outs, ids, pos = [], [], 0
        for L in cuts:
            r = _forward(dev, tab, sc, dev_weights, toks[pos:pos + L], np.array([0, L], np.int32),
                         h[pos:pos + L], st, **kw)
            outs.append(host_bits(r["out"]))
            ids.append(r["row_ids"].cpu().numpy())
            pos += L
        return np.concatenate(outs), np.concatenate(ids), st.conv_state.cpu().numpy(), st.hist_ids.cpu().numpy()

    full = run([n])
    for cuts in ([1024, 276], [300, 1000], [1, 2, 1297], [8] * 10 + [1220]):
        got = run(cuts)
        for a, b in zip(got, full):
            assert np.array_equal(a, b), (layout, cuts)


@pytest.mark.parametrize("seed", range(6))
def test_streaming_fuse_random_sequence_structures(dev, small_table, dev_weights, seed):
    # random sequence structures (empty, short and long sequences, random
    # history lengths and carried state) in one call of more than 1024 tokens
    # (streaming fuse, block ranges crossing sequence starts and ends at
    # random places) against each sequence alone (one-token fuse or, above
    # 1024 tokens, the streaming fuse on its own ranges), bit for bit
    tab, sc = small_table
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.integers(2, 14))
    lengths = []
    for _ in range(S):
        kind = rng.integers(0, 4)
        lengths.append(0 if kind == 0 else int(rng.integers(1, 8)) if kind == 1 else int(rng.integers(30, 700)))
    lengths[int(rng.integers(0, S))] += 1100 - sum(lengths) if sum(lengths) < 1100 else 0
    hl = [int(v) for v in rng.integers(0, 3, S)]
    toks, cu, hist, hlen, h = _case(2000 + seed, lengths, hl)
    T = int(cu[-1])
    assert T > 1024 and T >= 32 * S
    state0 = (rng.standard_normal((S, 3, D)) * 0.5).astype(np.float32)

    def fresh(lo, hi):
        st = ple.State(hi - lo, dev)
        st.hist_ids.copy_(dev_i32(hist[lo:hi], dev))
        st.hist_len.copy_(dev_i32(hlen[lo:hi], dev))
        st.conv_state.copy_(torch.from_numpy(state0[lo:hi]).to(dev))
        return st

    st = fresh(0, S)
    whole = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    _same_without_debug(dev, tab, sc, dev_weights, toks, cu, h, fresh(0, S), whole, st)
    for i in range(S):
        a, b = int(cu[i]), int(cu[i + 1])
        si = fresh(i, i + 1)
        one = _forward(dev, tab, sc, dev_weights, toks[a:b], np.array([0, b - a], np.int32), h[a:b], si)
        assert np.array_equal(host_bits(one["out"]), host_bits(whole["out"][a:b])), (seed, i, lengths)
        assert torch.equal(si.conv_state[0], st.conv_state[i]), (seed, i, lengths)
        assert torch.equal(si.hist_ids[0], st.hist_ids[i]) and torch.equal(si.hist_len[0], st.hist_len[i])


def test_streaming_fuse_many_short_sequences(dev, small_table, dev_weights):
    # about 150 sequences of 0-8 tokens (and a few longer ones) in one call of
    # more than 1024 tokens: the streaming fuse, whose 8-token block ranges
    # hold several sequence starts and ends each, against each sequence alone
    # (the one-token fuse), bit for bit, carried state included
    tab, sc = small_table
    rng = np.random.default_rng(3000)
    lengths = []
    while sum(lengths) < 1100:
        kind = rng.integers(0, 10)
        lengths.append(0 if kind == 0 else 1 if kind < 4 else int(rng.integers(2, 9)) if kind < 9
                       else int(rng.integers(20, 61)))
    S = len(lengths)
    hl = [int(v) for v in rng.integers(0, 3, S)]
    toks, cu, hist, hlen, h = _case(3001, lengths, hl)
    T = int(cu[-1])
    assert T > 1024 and T >= 2 * S and T < 8 * S
    state0 = (rng.standard_normal((S, 3, D)) * 0.5).astype(np.float32)

    def fresh(lo, hi):
        st = ple.State(hi - lo, dev)
        st.hist_ids.copy_(dev_i32(hist[lo:hi], dev))
        st.hist_len.copy_(dev_i32(hlen[lo:hi], dev))
        st.conv_state.copy_(torch.from_numpy(state0[lo:hi]).to(dev))
        return st

    st = fresh(0, S)
    whole = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    _same_without_debug(dev, tab, sc, dev_weights, toks, cu, h, fresh(0, S), whole, st)
    whole_out = host_bits(whole["out"])
    for i in range(S):
        a, b = int(cu[i]), int(cu[i + 1])
        si = fresh(i, i + 1)
        one = _forward(dev, tab, sc, dev_weights, toks[a:b], np.array([0, b - a], np.int32), h[a:b], si)
        assert np.array_equal(host_bits(one["out"]), whole_out[a:b]), (i, lengths[i])
        assert torch.equal(si.conv_state[0], st.conv_state[i]), (i, lengths[i])
        assert torch.equal(si.hist_ids[0], st.hist_ids[i]) and torch.equal(si.hist_len[0], st.hist_len[i])


# ---------------------------------------------------------------------------
# One launch for short calls (up to 16 tokens and 256 sequences): projection
# blocks and one finisher per token, ordered by counters in the workspace.
# ple_forward_staged runs the same calls as three launches. In place
# (out == h), the finishers read the earlier tokens' h rows from a copy the
# projection blocks take.
# ---------------------------------------------------------------------------

ONE_LAUNCH_CASES = [
    ([1] * 8, [2] * 8),                                     # a decode step
    ([16], [0]),                                            # a fresh 16-token chunk
    ([0, 1, 5, 2, 0, 4, 3, 1], [2, 1, 0, 2, 1, 2, 0, 1]),   # empty, short and longer sequences
    ([1] * 14 + [0] * 186 + [2], [2] * 100 + [1] * 101),    # 201 sequences, most empty
    ([0] * 120 + [1] * 16 + [0] * 120, [2, 1, 0, 2] * 64),   # the limits: 256 sequences, 16 tokens
]


@pytest.mark.parametrize("case", range(len(ONE_LAUNCH_CASES)))
def test_one_launch_equals_three_launches(dev, small_table, dev_weights, case):
    lengths, hls = ONE_LAUNCH_CASES[case]
    tab, sc = small_table
    toks, cu, hist, hlen, h = _case(700 + case, lengths, hls)
    S, T = len(lengths), int(cu[-1])
    assert ple.one_launch(T, S) and not ple.one_launch(17, S)
    rng = np.random.default_rng(701 + case)
    state0 = (0.4 * rng.standard_normal((S, 3, D))).astype(np.float32)
    state0[np.array(hls) == 0] = 0.0

    def fresh():
        st = ple.State(S, dev)
        st.hist_ids.copy_(dev_i32(hist, dev))
        st.hist_len.copy_(dev_i32(hlen, dev))
        st.conv_state.copy_(torch.from_numpy(state0).to(dev))
        return st

    ws = ple.Workspace(dev)
    st1, st2, st3, st4, st5 = fresh(), fresh(), fresh(), fresh(), fresh()
    one = _forward(dev, tab, sc, dev_weights, toks, cu, h, st1, workspace=ws)        # one launch, debug
    three = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                            dev_bf16(h, dev), st2, debug=True, staged=True)         # three launches
    fast = _forward(dev, tab, sc, dev_weights, toks, cu, h, st3, debug=False, workspace=ws)
    h4 = dev_bf16(h, dev)
    ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1], h4, st4,
                    out=h4, workspace=ws)                                            # one launch, in place
    h5 = dev_bf16(h, dev)
    ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1], h5, st5,
                    out=h5, staged=True)                                             # three launches, in place
    for k in ("row_ids", "x", "e", "gate", "y"):
        assert torch.equal(one[k], three[k]), k
    want = host_bits(three["out"])
    for got in (one["out"], fast, h4, h5):
        assert np.array_equal(host_bits(got), want)
    for st in (st1, st3, st4, st5):
        assert torch.equal(st.conv_state, st2.conv_state)
        assert torch.equal(st.hist_ids, st2.hist_ids) and torch.equal(st.hist_len, st2.hist_len)
    # every call leaves the counters at zero
    torch.cuda.synchronize()
    assert int(ws.buf[:256].to(torch.int32).abs().sum().item()) == 0


def test_one_launch_against_oracle(dev, small_table, dev_weights, weights):
    W, cw = weights
    tab, sc = small_table
    lengths, hls = ONE_LAUNCH_CASES[2]
    toks, cu, hist, hlen, h = _case(710, lengths, hls)
    S = len(lengths)
    rng = np.random.default_rng(711)
    state0 = (0.4 * rng.standard_normal((S, 3, D))).astype(np.float32)
    st = ple.State(S, dev)
    st.hist_ids.copy_(dev_i32(hist, dev))
    st.hist_len.copy_(dev_i32(hlen, dev))
    st.conv_state.copy_(torch.from_numpy(state0).to(dev))
    res = _forward(dev, tab, sc, dev_weights, toks, cu, h, st)
    ref = oracle.forward(toks, cu, h, W, cw, R_SMALL, rows, hist, hlen, state0.astype(np.float64))
    got = gather_debug(res, np.arange(len(toks)))
    assert np.array_equal(got["row_ids"], ref["row_ids"])
    assert np.array_equal(got["x"], ref["x"])
    assert np.all(np.abs(got["e"].astype(np.float64) - ref["e"]) <= E_REL * e_bound(ref["x"], W) + 1e-7)
    assert np.all(np.abs(got["g"] - ref["g"]) <= gate_bound(ref, h, W))
    s64 = state0.astype(np.float64)
    assert np.all(np.abs(got["y"] - ref["y"]) <= y_bound(ref, cu, cw, s64, W, h))
    out = inputs.bf16_bits_to_f32(got["out"]).astype(np.float64)
    assert np.all(np.abs(out - ref["out"]) <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"]))
    assert np.array_equal(st.hist_len.cpu().numpy(), ref["hist_len"])
    hid = st.hist_ids.cpu().numpy()
    for s in range(S):
        k = ref["hist_len"][s]
        assert np.array_equal(hid[s][2 - k:], ref["hist_ids"][s][2 - k:]), s
    assert np.all(np.abs(st.conv_state.cpu().numpy() - ref["conv_state"]) <= state_bound(ref, cu, cw, W, h))
    assert np.array_equal(st.conv_state[0].cpu().numpy(), state0[0])        # empty sequence untouched


def test_one_launch_flags_a_workspace_whose_counters_are_not_zero(dev, small_table, dev_weights):
    # a ticket counter far past the grid: every block takes a ticket beyond
    # its roles and exits at once, flagging PLE_DEVERR_SYNC (nothing waits)
    tab, sc = small_table
    toks, cu, hist, hlen, h = _case(720, [1] * 8, [2] * 8)
    ws = ple.Workspace(dev)
    ws.get(8, 8)
    ws.buf[:4].view(torch.int32).fill_(1000)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                    dev_bf16(h, dev), ple.State(8, dev), workspace=ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ple.DEVERR_SYNC
    # cleared again, the same workspace serves a normal call
    ws.buf[:256].zero_()
    err.zero_()
    st_a, st_b = ple.State(8, dev), ple.State(8, dev)
    a = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                        dev_bf16(h, dev), st_a, workspace=ws, dev_err=err)
    b = ple.ple_forward(dev_i32(toks, dev), dev_i32(cu, dev), tab, sc, dev_weights[0], dev_weights[1],
                        dev_bf16(h, dev), st_b, staged=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(host_bits(a), host_bits(b))
