"""Checks of the seeded input generators (CPU side)."""

import os

import numpy as np
import torch

from gen import inputs, table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_matches_numpy_and_kat():
    # numpy's Philox is Philox4x64-10; it increments the counter before use
    rng = np.random.default_rng(0)
    for _ in range(20):
        ctr = [int(v) for v in rng.integers(0, 2 ** 63, 4)]
        key = [int(v) for v in rng.integers(0, 2 ** 63, 2)]
        bg = np.random.Philox(counter=ctr, key=key)
        ref = bg.random_raw(4)
        nxt = list(ctr)
        nxt[0] = (nxt[0] + 1) % 2 ** 64
        assert np.array_equal(table.philox4x64_10(nxt, key), ref)
    with open(os.path.join(GOLDEN, "philox4x64_10.txt")) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            v = [int(t, 16) for t in ln.split()]
            assert [int(o) for o in table.philox4x64_10(v[:4], v[4:6])] == v[6:]


def test_thresholds_follow_half_normal():
    thr = table.thresholds().astype(np.float64) / 2 ** 31
    grid = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    # P(|Z| <= 1.0625) (midpoint of 1.0 and 1.125) = erf(1.0625/sqrt2) = 0.7120...
    k = int(np.where(grid == 1.0)[0][0])
    assert abs(thr[k] - 0.71200) < 1e-4
    assert thr[-1] == 1.0


def test_table_rows_statistics_and_independence_of_R():
    rows, scales = table.rows_cpu(np.arange(2000))
    v = torch.from_numpy(rows.reshape(-1)).view(torch.float8_e4m3fn).double().numpy()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    assert not np.any((rows & 0x7F) == 0x7F)     # never a NaN code
    again, sc2 = table.rows_cpu(np.array([1999, 5, 0]))
    assert np.array_equal(again, rows[[1999, 5, 0]]) and np.array_equal(sc2, scales[[1999, 5, 0]])
    other, _ = table.rows_cpu(np.array([5]), seed=inputs.TABLE_SEED + 1)
    assert not np.array_equal(other[0], rows[5])


def test_workloads_shapes():
    w = inputs.make_workload("tiny")
    assert w.R == 65_536 and w.total_tokens == 128
    toks = w.chunks[0][0]
    assert toks.dtype == np.int32 and toks.min() >= 0 and toks.max() < inputs.VOCAB
    rg = inputs.make_workload("ragged")
    assert rg.S == 64 and list(rg.chunks[0][1][:3]) == [0, 256, 512] and rg.chunks[0][1][-1] == 16_384
    dc = inputs.make_workload("decode", decode_steps=3)
    assert dc.history[0].shape == (8, 4096) and len(dc.chunks) == 3
    assert list(dc.chunks[0][1]) == list(range(9))


def test_zipf_is_truncated_and_heavy_headed():
    rng = np.random.Generator(np.random.PCG64(1))
    t = inputs.zipf_tokens(rng, 200_000)
    assert t.min() >= 0 and t.max() < inputs.VOCAB
    p0 = np.mean(t == 0)
    ranks = np.arange(1, inputs.VOCAB + 1, dtype=np.float64)
    expect = 1.0 / np.sum(ranks ** -1.1)
    assert abs(p0 - expect) < 0.005


def test_long_context_reuse():
    rng = np.random.Generator(np.random.PCG64(2))
    t = inputs.long_context_tokens(rng, 16_384)
    bigrams = t[:-1].astype(np.int64) * inputs.VOCAB + t[1:]
    frac_unique = len(np.unique(bigrams)) / len(bigrams)
    assert 0.5 < frac_unique < 0.95


def test_bf16_normals():
    rng = np.random.Generator(np.random.PCG64(3))
    h = inputs.normal_bf16(rng, (64, 2560))
    f = inputs.bf16_bits_to_f32(h)
    assert abs(f.std() - 1.0) < 0.01 and h.dtype == np.uint16
