"""Pins of the CPU oracle against things other than itself.

Every step of the oracle is checked here against a published value, a
library routine, a closed form or a brute-force invariant, chosen so that a
plausible slip (dropped term, wrong sign, wrong index or tap order,
transposed operand) fails at least one test.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gen import inputs, table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 2560
M64 = 2 ** 64 - 1


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _rows(ids):
    return table.rows_cpu(ids)


# ---------------------------------------------------------------------------
# n-gram IDs
# ---------------------------------------------------------------------------

def test_mix64_matches_published_splitmix64_sequence():
    for seed, idx, out in _golden("splitmix64.txt"):
        state = (int(seed) + int(idx) * 0x9E3779B97F4A7C15) & M64
        assert oracle.mix64(state) == int(out)


def test_key_fields_decode():
    rng = np.random.default_rng(5)
    for a, b, c in rng.integers(0, 2 ** 20, size=(200, 3)):
        k2 = oracle.key2(int(a), int(b))
        assert k2 >> 60 == 2 and (k2 >> 20) & (2 ** 40 - 1) == a and k2 & (2 ** 20 - 1) == b
        k3 = oracle.key3(int(a), int(b), int(c))
        assert k3 >> 60 == 3
        assert (k3 >> 40) & (2 ** 20 - 1) == a
        assert (k3 >> 20) & (2 ** 20 - 1) == b
        assert k3 & (2 ** 20 - 1) == c


def test_ngram_ids_missing_history_and_range():
    R = 1009
    toks = np.array([5, 9, 9, 5, 7, 1, 2, 3], np.int32)
    cu = np.array([0, 0, 1, 3, 8], np.int32)          # lengths 0, 1, 2, 5
    hist = np.array([[0, 0], [0, 0], [0, 77], [0, 0]], np.int32)
    hl = np.array([0, 0, 1, 2], np.int32)
    hist[3] = [11, 12]
    ids = oracle.ngram_ids(toks, cu, hist, hl, R)
    # seq 1 (len 1, no history): token 0 has neither n-gram
    assert list(ids[0]) == [-1, -1]
    # seq 2 (len 2, one history token): bigram everywhere, trigram from the 2nd
    assert ids[1][0] >= 0 and ids[1][1] == -1
    assert ids[2][0] >= 0 and ids[2][1] >= 0
    # seq 3 (two history tokens): everything present
    assert np.all(ids[3:] >= 0)
    assert np.all(ids < R)
    # the ID of an n-gram does not depend on where it occurs: bigram (77, 9)
    # then (9, 9); trigram (77, 9, 9)
    fresh = oracle.ngram_ids(np.array([77, 9, 9], np.int32), np.array([0, 3], np.int32),
                             np.zeros((1, 2), np.int32), np.zeros(1, np.int32), R)
    assert list(fresh[1]) == [ids[1][0], -1]
    assert list(fresh[2]) == list(ids[2])


def test_ngram_ids_are_mix_of_key_mod_R():
    R = 20_000_096
    rng = np.random.default_rng(1)
    toks = rng.integers(0, inputs.VOCAB, 50).astype(np.int32)
    ids = oracle.ngram_ids(toks, np.array([0, 50], np.int32), np.zeros((1, 2), np.int32),
                           np.zeros(1, np.int32), R)
    for j in range(2, 50):
        a, b, c = (int(v) for v in toks[j - 2:j + 1])
        assert ids[j][0] == oracle.mix64(oracle.key2(b, c)) % R
        assert ids[j][1] == oracle.mix64(oracle.key3(a, b, c)) % R


def test_ngram_ids_repeated_phrase_repeats_ids_and_brute_force_distinct():
    R = 2 ** 31 - 1
    rng = np.random.default_rng(2)
    phrase = rng.integers(0, inputs.VOCAB, 20).astype(np.int32)
    filler = rng.integers(0, inputs.VOCAB, 13).astype(np.int32)
    seq = np.concatenate([phrase, filler, phrase])
    ids = oracle.ngram_ids(seq, np.array([0, len(seq)], np.int32), np.zeros((1, 2), np.int32),
                           np.zeros(1, np.int32), R)
    a = ids[2:20]
    b = ids[33 + 2:33 + 20]
    assert np.array_equal(a, b)
    # over a tiny vocabulary every bigram and trigram key is distinct, and the
    # 64-bit mix is a bijection, so with R = 2^31-1 collisions are rare
    v = 12
    keys2 = {oracle.key2(x, y) for x in range(v) for y in range(v)}
    keys3 = {oracle.key3(x, y, z) for x in range(v) for y in range(v) for z in range(v)}
    assert len(keys2) == v * v and len(keys3) == v ** 3 and not (keys2 & keys3)


def test_hist_update_cases():
    toks = np.array([5, 6, 7, 8, 9], np.int32)
    cu = np.array([0, 0, 1, 2, 5], np.int32)
    hist = np.array([[3, 4], [0, 4], [0, 0], [1, 2]], np.int32)
    hl = np.array([2, 1, 0, 2], np.int32)
    hid, hln = oracle.hist_update(toks, cu, hist, hl)
    assert list(hln) == [2, 2, 1, 2]
    assert list(hid[0]) == [3, 4]          # empty segment: unchanged
    assert list(hid[1]) == [4, 5]          # one history + one token
    assert hid[2][1] == 6                  # fresh + one token
    assert list(hid[3]) == [8, 9]          # last two tokens


def test_ngram_ids_chunked_equals_unchunked():
    R = 65_536
    rng = np.random.default_rng(3)
    seq = rng.integers(0, inputs.VOCAB, 40).astype(np.int32)
    full = oracle.ngram_ids(seq, np.array([0, 40], np.int32), np.zeros((1, 2), np.int32),
                            np.zeros(1, np.int32), R)
    for cuts in ([1, 1, 1, 37], [2, 3, 35], [0, 5, 0, 35]):
        hid, hln = np.zeros((1, 2), np.int32), np.zeros(1, np.int32)
        pos, parts = 0, []
        for L in cuts:
            chunk = seq[pos:pos + L]
            cu = np.array([0, L], np.int32)
            parts.append(oracle.ngram_ids(chunk, cu, hid, hln, R))
            hid, hln = oracle.hist_update(chunk, cu, hid, hln)
            pos += L
        assert np.array_equal(np.concatenate(parts), full)


# ---------------------------------------------------------------------------
# FP8 decode and bf16 rounding
# ---------------------------------------------------------------------------

def test_e4m3_ocp_table_values():
    for code, val in _golden("e4m3fn_ocp.txt"):
        got = oracle.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_rne_matches_torch_including_ties():
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    # force exact ties and near-ties in part of the sample
    bits[:5000] = (bits[:5000] & 0xFFFF0000) | 0x8000
    bits[5000:7000] = (bits[5000:7000] & 0xFFFF0000) | 0x7FFF
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(ref, got)


# ---------------------------------------------------------------------------
# Gather + dequant
# ---------------------------------------------------------------------------

def _gather_case(n_rows=64, T=96, seed=6):
    rng = np.random.default_rng(seed)
    row_numbers = rng.choice(20_000_096, n_rows, replace=False)
    codes, scales = _rows(row_numbers)
    ids = rng.integers(-1, n_rows, (T, 2)).astype(np.int32)
    ids[ids[:, 0] < 0, 1] = -1            # no trigram without a bigram
    ids[5] = [7, 7]                       # bigram and trigram on the same row
    return codes, scales, ids


def test_gather_raw_bytes_equal_rows():
    codes, scales, ids = _gather_case()
    _, raw = oracle.gather_dequant(ids, codes, scales, raw=True)
    for t in range(ids.shape[0]):
        for k in range(2):
            r = ids[t, k]
            expect = codes[r] if r >= 0 else np.zeros(D, np.uint8)
            assert raw[t, k].tobytes() == expect.tobytes()


def test_gather_dequant_matches_torch_fp32_reduction():
    codes, scales, ids = _gather_case()
    x = oracle.gather_dequant(ids, codes, scales)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(scales)
    for t in range(ids.shape[0]):
        acc = torch.zeros(D, dtype=torch.float32)
        r0, r1 = ids[t]
        if r0 >= 0:
            acc = dec[r0] * sc[r0]
        if r1 >= 0:
            acc = acc + dec[r1] * sc[r1]
        ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ref, x[t]), t


def test_gather_dequant_close_to_exact_rational_sum():
    codes, scales, ids = _gather_case(n_rows=8, T=6, seed=9)
    x = oracle.gather_dequant(ids, codes, scales)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for t in range(ids.shape[0]):
        for c in range(0, D, 7):
            exact = Fraction(0)
            for r in ids[t]:
                if r >= 0:
                    exact += Fraction(float(dec[r, c])) * Fraction(float(scales[r]))
            got = Fraction(float(inputs.bf16_bits_to_f32(np.array([x[t, c]], np.uint16))[0]))
            if exact == 0:
                assert got == 0
                continue
            ulp = Fraction(2) ** (math.floor(math.log2(abs(float(exact)))) - 7)
            # one fp32 rounding then one bf16 rounding: within half a bf16 ulp
            # plus half an fp32 ulp
            assert abs(got - exact) <= ulp / 2 + ulp / 2 ** 16


def test_scales_exact_and_in_range():
    _, scales = _rows(np.arange(5000))
    m = scales.astype(np.float64) * 2 ** 23
    assert np.all(m == np.round(m)) and np.all(m < 2 ** 20)
    assert scales.min() >= 0.01 and scales.max() < 0.1


# ---------------------------------------------------------------------------
# Projection, gate, conv
# ---------------------------------------------------------------------------

def test_project_matches_numpy_fp64(weights):
    W, _ = weights
    rng = np.random.default_rng(7)
    x = inputs.normal_bf16(rng, (9, D), std=0.1)
    e = oracle.project(x, W)
    ref = inputs.bf16_bits_to_f32(x).astype(np.float64) @ inputs.bf16_bits_to_f32(W).astype(np.float64).T
    np.testing.assert_allclose(e, ref, rtol=1e-12, atol=1e-13)


def test_project_identity_weight():
    I = torch.eye(D, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(8)
    x = inputs.normal_bf16(rng, (3, D))
    e = oracle.project(x, I)
    assert np.array_equal(e, inputs.bf16_bits_to_f32(x).astype(np.float64))


def test_project_uses_w_rows_as_outputs():
    # W with a single non-zero W[o][c] = 1 maps x[:, c] to e[:, o] (catches a transpose)
    W = np.zeros((D, D), np.uint16)
    W[11, 1234] = 0x3F80  # 1.0 in bf16
    x = np.zeros((1, D), np.uint16)
    x[0, 1234] = 0x4040   # 3.0
    e = oracle.project(x, W)
    assert e[0, 11] == 3.0 and np.count_nonzero(e) == 1


def _rne_bf16_exact(v: float) -> float:
    """Round-half-even of a double to 8 significant bits with bf16's range,
    in exact rational arithmetic (independent of the oracle's frexp/nearbyint)."""
    if v == 0.0 or math.isinf(v) or math.isnan(v):
        return v
    a = abs(Fraction(v))
    ex = a.numerator.bit_length() - a.denominator.bit_length()   # 2^ex <= a < 2^(ex+1), up to one
    if Fraction(2) ** ex > a:
        ex -= 1
    step = Fraction(2) ** max(ex - 7, -133)
    n, rem = divmod(a, step)
    if rem > step / 2 or (rem == step / 2 and n % 2 == 1):
        n += 1
    r = n * step
    if r > Fraction(255) * Fraction(2) ** 120:                    # beyond the largest finite bf16
        return math.copysign(math.inf, v)
    return math.copysign(float(r), v)


def test_round_bf16_matches_exact_rational_rne():
    rng = np.random.default_rng(31)
    # random 53-bit significands over normal and subnormal bf16 exponents
    m = 1.0 + rng.random(4000)
    ex = rng.integers(-140, 128, 4000)
    v = np.ldexp(m, ex) * np.where(rng.random(4000) < 0.5, -1.0, 1.0)
    # exact ties and near-ties at a few scales
    base = np.ldexp(1.0 + np.arange(1, 60) * 2.0 ** -7, rng.integers(-20, 20, 59))
    ulp = base * 2.0 ** -8 / (1.0 + np.arange(1, 60) * 2.0 ** -7)
    v = np.concatenate([v, base + ulp, base - ulp, base + ulp * (1 + 2 ** -30), base + ulp * (1 - 2 ** -30)])
    got = oracle.round_bf16(v)
    want = np.array([_rne_bf16_exact(float(a)) for a in v])
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_single_rounding_and_range():
    r = oracle.round_bf16(np.array([
        1 + 2.0 ** -8,               # tie -> 1 (even)
        1 + 3 * 2.0 ** -8,           # tie -> 1 + 2^-6 (even)
        1 + 2.0 ** -8 + 2.0 ** -40,  # just above the tie: up; a pass through fp32 would give 1
        -(1 + 2.0 ** -8 + 2.0 ** -40),
        1.5 * 2.0 ** -133,           # subnormal tie -> 2^-132 (even)
        2.0 ** -134,                 # tie between 0 and 2^-133 -> +0
        -(2.0 ** -134),
        3.4e38,                      # past the overflow midpoint -> inf
        3.3961e38,                   # below it -> largest finite
        -0.0]))
    want = [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -(1 + 2.0 ** -7), 2.0 ** -132, 0.0, -0.0,
            math.inf, 255 * 2.0 ** 120, -0.0]
    for a, b in zip(r, want):
        assert a == b and math.copysign(1, a) == math.copysign(1, b)


def test_round_bf16_matches_torch_on_fp32_inputs():
    # torch rounds float32 -> bfloat16 directly (RNE); on float32 inputs the
    # single rounding from fp64 must agree with it
    rng = np.random.default_rng(32)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(f.astype(np.float64)), want)


def test_gate_closed_forms():
    rng = np.random.default_rng(10)
    h = inputs.normal_bf16(rng, (4, D))
    hf = inputs.bf16_bits_to_f32(h).astype(np.float64)
    e = np.stack([0.37 * hf[0], -2.0 * hf[1], np.zeros(D), np.zeros(D)])
    # row 3: exactly orthogonal to h[3]
    e[3, 0] = hf[3, 1]
    e[3, 1] = -hf[3, 0]
    g = oracle.gate(h, e, eps=1e-6)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    assert abs(g[0] - sig(math.sqrt(D))) < 1e-12 and g[0] > 0.999999
    assert abs(g[1] - sig(-math.sqrt(D))) < 1e-12 and g[1] < 1e-6
    assert g[2] == 0.5
    assert abs(g[3] - 0.5) < 1e-15


def _unit(v):
    return v / np.linalg.norm(v)


def test_gate_mid_range_cosine_closed_form():
    # with RMS-normalised rows, <h^, e^> / sqrt(D) = sqrt(D) cos(h, e); pick
    # e at a known angle to h so that the sigmoid argument is 0.5 and -1.25
    rng = np.random.default_rng(16)
    h = inputs.normal_bf16(rng, (2, D))
    hf = inputs.bf16_bits_to_f32(h).astype(np.float64)
    e = np.empty((2, D))
    for i, z in enumerate((0.5, -1.25)):
        cos = z / math.sqrt(D)
        u = _unit(hf[i])
        p = rng.standard_normal(D)
        p = _unit(p - (p @ u) * u)
        e[i] = 3.0 * (cos * u + math.sqrt(1 - cos * cos) * p)
    g = oracle.gate(h, e, eps=0.0)
    assert abs(g[0] - 1 / (1 + math.exp(-0.5))) < 1e-12
    assert abs(g[1] - 1 / (1 + math.exp(1.25))) < 1e-12


def test_gate_eps_damps_tiny_rows():
    rng = np.random.default_rng(17)
    h = inputs.normal_bf16(rng, (1, D))
    hf = inputs.bf16_bits_to_f32(h).astype(np.float64)
    e = 0.01 * hf + rng.standard_normal((1, D))
    g_big = oracle.gate(h, e, eps=1e-6)[0]
    g_big0 = oracle.gate(h, e, eps=0.0)[0]
    assert abs(g_big - g_big0) < 1e-5            # eps is negligible at unit scale
    # shrinking e by 1e-4 (mean(e^2) ~ 1e-8 << eps) pulls the gate towards 1/2
    g_small = oracle.gate(h, e * 1e-4, eps=1e-6)[0]
    g_small0 = oracle.gate(h, e * 1e-4, eps=0.0)[0]
    assert abs(g_small0 - g_big0) < 1e-12        # scale invariant without eps
    assert g_big0 > 0.55 and 0.5 < g_small < g_big0 - 0.05


def _conv_torch(v, w, state):
    """Causal depthwise conv by torch.nn.functional.conv1d (cross-correlation)."""
    full = np.concatenate([state, v], axis=0)          # [3 + L, D]
    inp = torch.from_numpy(full.T.copy())[None]         # [1, D, 3+L]
    ker = torch.from_numpy(w.copy())[:, None, :]        # [D, 1, 4]
    y = torch.nn.functional.conv1d(inp, ker, groups=D)  # valid conv -> L outputs
    return y[0].numpy().T


def test_conv_matches_torch_conv1d_with_state():
    rng = np.random.default_rng(11)
    L = 9
    h = inputs.normal_bf16(rng, (L, D))
    e = rng.standard_normal((L, D))
    g = rng.random(L)
    _, cw = inputs.weights()
    w = inputs.bf16_bits_to_f32(cw).astype(np.float64)
    state = rng.standard_normal((1, 3, D))
    y, out, st = oracle.conv_fuse(h, e, g, np.array([0, L], np.int32), cw, state)
    ref = _conv_torch(g[:, None] * e, w, state[0])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out, inputs.bf16_bits_to_f32(h).astype(np.float64) + y)
    np.testing.assert_array_equal(st[0], g[-3:, None] * e[-3:])


def test_conv_impulse_response_tap_order():
    L = 7
    h = np.zeros((L, D), np.uint16)
    e = np.zeros((L, D))
    e[2, :] = 1.0
    g = np.ones(L)
    _, cw = inputs.weights()
    w = inputs.bf16_bits_to_f32(cw).astype(np.float64)
    y, _, _ = oracle.conv_fuse(h, e, g, np.array([0, L], np.int32), cw, np.zeros((1, 3, D)))
    for k in range(4):
        np.testing.assert_array_equal(y[2 + k], w[:, 3 - k])
    assert np.all(y[:2] == 0) and np.all(y[6:] == 0)


def test_conv_short_segments_carry_state():
    rng = np.random.default_rng(12)
    _, cw = inputs.weights()
    state = rng.standard_normal((3, 3, D))
    e = rng.standard_normal((3, D))
    g = rng.random(3)
    cu = np.array([0, 0, 1, 3], np.int32)               # lengths 0, 1, 2
    h = np.zeros((3, D), np.uint16)
    _, _, st = oracle.conv_fuse(h, e, g, cu, cw, state)
    np.testing.assert_array_equal(st[0], state[0])                       # unchanged
    np.testing.assert_array_equal(st[1][:2], state[1][1:])                # shifted
    np.testing.assert_array_equal(st[1][2], g[0] * e[0])
    np.testing.assert_array_equal(st[2][0], state[2][2])
    np.testing.assert_array_equal(st[2][1:], g[1:, None] * e[1:])


# ---------------------------------------------------------------------------
# NVFP4 table (E2M1 codes, E4M3 scale per 16 elements, fp32 row scale)
# ---------------------------------------------------------------------------

def _e2m1_golden():
    return {int(c, 16): float(v) for c, v in _golden("e2m1_ocp.txt")}


def test_e2m1_values_match_ocp_table_and_generator_grid():
    gold = _e2m1_golden()
    assert len(gold) == 16
    for c, v in gold.items():
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    assert tuple(gold[c] for c in range(8)) == inputs.E2M1_GRID


def _nvfp4_torch(ids, codes, blocks, scales):
    """x by torch fp32 ops: E2M1 by table lookup, E4M3 by torch's float8."""
    gold = _e2m1_golden()
    lut = torch.tensor([gold[c] for c in range(16)], dtype=torch.float32)
    c = torch.from_numpy(codes).to(torch.int64)
    nib = torch.stack([c & 15, c >> 4], dim=-1).reshape(codes.shape[0], -1)   # element 2k = low nibble
    q = lut[nib] * torch.from_numpy(blocks).view(torch.float8_e4m3fn).to(torch.float32).repeat_interleave(16, 1)
    p = q * torch.from_numpy(scales)[:, None]
    out = []
    for r0, r1 in ids:
        acc = None
        for r in (r0, r1):
            if r >= 0:
                acc = p[r] if acc is None else acc + p[r]
        acc = torch.zeros(D) if acc is None else acc
        out.append(acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    return np.stack(out)


def test_gather_dequant_nvfp4_matches_torch_fp32():
    rng = np.random.default_rng(70)
    n = 40
    codes = rng.integers(0, 256, (n, 1280), dtype=np.uint8)
    blocks = rng.integers(0, 0x7F, (n, 160), dtype=np.uint8)          # positive, no NaN
    blocks[:, ::7] |= 0x80                                              # and some negative
    scales = rng.uniform(0.01, 0.1, n).astype(np.float32)
    ids = rng.integers(-1, n, (30, 2)).astype(np.int32)
    x, raw = oracle.gather_dequant_nvfp4(ids, codes, blocks, scales, raw=True)
    assert np.array_equal(x, _nvfp4_torch(ids, codes, blocks, scales))
    for t, (r0, r1) in enumerate(ids):
        for k, r in enumerate((r0, r1)):
            assert np.array_equal(raw[t, k], codes[r] if r >= 0 else np.zeros(1280, np.uint8))


def test_gather_dequant_nvfp4_close_to_exact_rational_sum():
    # the E2M1 values are taken from the OCP table (not from the oracle's
    # decoder) and the sum is formed exactly: each row's product is rounded to
    # fp32 once (code x block is exact), their sum once more, then to bf16
    rng = np.random.default_rng(71)
    n = 6
    codes = rng.integers(0, 256, (n, 1280), dtype=np.uint8)
    blocks = rng.integers(0x20, 0x58, (n, 160), dtype=np.uint8)
    blocks[:, ::5] |= 0x80
    scales = rng.uniform(0.01, 0.1, n).astype(np.float32)
    ids = np.array([[0, 1], [2, -1], [-1, 3], [4, 4], [5, 0], [-1, -1]], np.int32)
    x = oracle.gather_dequant_nvfp4(ids, codes, blocks, scales)
    e2m1 = {c: Fraction(v) for c, v in _e2m1_golden().items()}   # tests/golden/e2m1_ocp.txt
    blk = torch.from_numpy(blocks).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for t in range(ids.shape[0]):
        for c in range(0, D, 7):
            terms = []
            for r in ids[t]:
                if r >= 0:
                    nib = (int(codes[r, c // 2]) >> (4 * (c & 1))) & 15
                    val = e2m1[nib]
                    terms.append(val * Fraction(float(blk[r, c // 16])) * Fraction(float(scales[r])))
            exact = sum(terms, Fraction(0))
            got = Fraction(float(inputs.bf16_bits_to_f32(np.array([x[t, c]], np.uint16))[0]))
            if not terms or all(v == 0 for v in terms):
                assert got == 0
                continue
            mag = max(abs(exact), abs(got), Fraction(2) ** -126)
            ulp = Fraction(2) ** (math.floor(math.log2(float(mag))) - 7)
            fp32_err = sum(abs(v) for v in terms) / 2 ** 23 + abs(exact) / 2 ** 24
            assert abs(got - exact) <= ulp / 2 + fp32_err, (t, c)


def test_gather_dequant_nvfp4_element_and_block_placement():
    codes = np.zeros((1, 1280), np.uint8)
    blocks = np.zeros((1, 160), np.uint8)
    codes[0, 8] = 0x20            # element 17 (high nibble of byte 8) = E2M1 1.0
    blocks[0, 1] = 0x38           # block 1 (elements 16..31) = E4M3 1.0
    x = oracle.gather_dequant_nvfp4(np.array([[0, -1]], np.int32), codes, blocks, np.array([0.5], np.float32))
    nz = np.flatnonzero(x[0] & 0x7FFF)
    assert list(nz) == [17] and x[0, 17] == 0x3F00          # bf16 0.5


def test_nvfp4_generator_codes_follow_the_e2m1_half_normal():
    codes, blocks, scales = table.nvfp4_rows_cpu(np.arange(64))
    nib = np.concatenate([(codes & 15).ravel(), (codes >> 4).ravel()])
    freq = np.bincount(nib & 7, minlength=8) / nib.size
    edges = [0.0] + [0.5 * (inputs.E2M1_GRID[k] + inputs.E2M1_GRID[k + 1]) / 2 for k in range(7)] + [math.inf]
    want = [math.erf(edges[k + 1] / math.sqrt(2)) - math.erf(edges[k] / math.sqrt(2)) for k in range(8)]
    assert np.allclose(freq, want, atol=0.01)
    assert 0.45 < np.mean(nib >= 8) < 0.55
    assert blocks.min() >= inputs.NVFP4_BLOCK_CODE_LO
    assert blocks.max() < inputs.NVFP4_BLOCK_CODE_LO + inputs.NVFP4_BLOCK_CODES
    _, sc = table.rows_cpu(np.arange(64))
    assert np.array_equal(scales, sc)                         # the FP8 table's row scales


def test_forward_nvfp4_fresh_sequence(weights):
    W, cw = weights
    toks, h = _small_stream(4, seed=71)
    r = oracle.forward_nvfp4(toks, np.array([0, 4], np.int32), h, W, cw, 65_536, table.nvfp4_rows_cpu)
    assert np.all(r["x"][0] == 0) and r["g"][0] == 0.5
    assert np.array_equal(r["out"][0], inputs.bf16_bits_to_f32(h[0]).astype(np.float64))
    assert np.any(r["x"][1] != 0)


# ---------------------------------------------------------------------------
# 16-lookup layout (16 head tables of 160-byte rows)
# ---------------------------------------------------------------------------

GAMMA = 0x9E3779B97F4A7C15


def test_head_mix_is_the_published_splitmix64_stream():
    # head h of a key is output h + 1 of SplitMix64 started one increment
    # before the key; heads 8..15 repeat heads 0..7 on the trigram key
    for seed, idx, out in _golden("splitmix64.txt"):
        k = int(idx) - 1
        if 0 <= k < 8:
            key = (int(seed) + GAMMA) & M64
            assert oracle.head_mix(key, k) == int(out)
            assert oracle.head_mix(key, 8 + k) == int(out)


def test_ngram_ids_heads_against_keys_and_two_lookup_ids():
    R = 20_000_096
    rng = np.random.default_rng(41)
    toks = inputs.uniform_tokens(rng, 40)
    cu = np.array([0, 1, 2, 5, 40], np.int32)
    hist = np.array([[0, 0], [0, 11], [3, 4], [0, 0]], np.int32)
    hl = np.array([0, 1, 2, 0], np.int32)
    heads = oracle.ngram_ids_heads(toks, cu, hist, hl, R)
    two = oracle.ngram_ids(toks, cu, hist, hl, R)
    assert np.array_equal(heads[:, 0], two[:, 0]) and np.array_equal(heads[:, 8], two[:, 1])
    for s in range(4):
        seq = list(hist[s][2 - hl[s]:]) + list(toks[cu[s]:cu[s + 1]])
        for i in range(cu[s], cu[s + 1]):
            j = hl[s] + i - cu[s]
            for h in range(16):
                if h < 8:
                    want = -1 if j < 1 else oracle.head_mix(oracle.key2(seq[j - 1], seq[j]), h) % R
                else:
                    want = -1 if j < 2 else oracle.head_mix(oracle.key3(seq[j - 2], seq[j - 1], seq[j]), h) % R
                assert heads[i, h] == want, (s, i, h)
    full = heads[heads[:, 15] >= 0]
    assert all(len(set(r[:8])) == 8 and len(set(r[8:])) == 8 for r in full)   # heads read distinct rows


def test_head_slices_are_the_table_bytes_at_their_linear_offset():
    R = 65_536
    rng = np.random.default_rng(42)
    hs, rs = rng.integers(0, 16, 40), rng.integers(0, R, 40)
    codes, scales = table.slices_cpu(hs, rs, R)
    for h, r, c in zip(hs, rs, codes):
        g = (int(h) * R + int(r)) * 160
        row, _ = table.rows_cpu([g // 2560])
        assert np.array_equal(c, row[0][g % 2560:g % 2560 + 160])
    _, sc_rows = table.rows_cpu(rs)
    _, sc_head0 = table.slices_cpu(np.zeros(40, np.int64), rs, R)
    assert np.array_equal(sc_head0, sc_rows)          # head 0 shares the 2560-wide rows' scales


def test_gather_dequant_heads_torch_product_placement_and_missing_rows():
    rng = np.random.default_rng(43)
    n = 50
    codes = rng.integers(0, 256, (n, 160), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x80             # no NaN codes; keep some -0
    scales = (rng.uniform(0.01, 0.1, n)).astype(np.float32)
    idx = rng.integers(0, n, (12, 16)).astype(np.int32)
    idx[rng.random((12, 16)) < 0.25] = -1
    x, raw = oracle.gather_dequant_heads(idx, codes, scales, raw=True)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(scales)
    for t in range(12):
        for h in range(16):
            r = idx[t, h]
            got = x[t, 160 * h:160 * h + 160]
            if r < 0:
                assert np.all(got == 0) and np.all(raw[t, h] == 0)      # +0, not -0
            else:
                want = (dec[r] * sc[r]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got, want), (t, h)
                assert np.array_equal(raw[t, h], codes[r])


def test_forward_heads_fresh_sequence_and_bigram_only_token(weights):
    W, cw = weights
    R = 65_536
    toks, h = _small_stream(5, seed=44)
    r = oracle.forward_heads(toks, np.array([0, 5], np.int32), h, W, cw, R,
                             lambda hs, rs: table.slices_cpu(hs, rs, R))
    assert np.all(r["x"][0] == 0) and r["g"][0] == 0.5
    assert np.array_equal(r["out"][0], inputs.bf16_bits_to_f32(h[0]).astype(np.float64))
    assert np.all(r["row_ids"][1, :8] >= 0) and np.all(r["row_ids"][1, 8:] == -1)
    assert np.any(r["x"][1, :1280] != 0) and np.all(r["x"][1, 1280:] == 0)
    assert np.all(r["row_ids"][2:] >= 0)


# ---------------------------------------------------------------------------
# Whole path
# ---------------------------------------------------------------------------

def _small_stream(n, seed=13):
    rng = np.random.default_rng(seed)
    return inputs.uniform_tokens(rng, n), inputs.normal_bf16(rng, (n, D))


def test_fresh_sequence_token0_is_identity_and_token1_uses_bigram_only(weights):
    W, cw = weights
    toks, h = _small_stream(6)
    r = oracle.forward(toks, np.array([0, 6], np.int32), h, W, cw, 65_536, _rows)
    assert np.all(r["x"][0] == 0) and r["g"][0] == 0.5
    assert np.array_equal(r["out"][0], inputs.bf16_bits_to_f32(h[0]).astype(np.float64))
    assert r["row_ids"][1][1] == -1 and r["row_ids"][1][0] >= 0
    codes, scales = _rows([r["row_ids"][1][0]])
    x1 = oracle.gather_dequant(np.array([[0, -1]], np.int32), codes, scales)
    assert np.array_equal(x1[0], r["x"][1])


def test_forward_gate_and_conv_consume_the_bf16_projection(weights):
    # the gate and the conv act on e_b = bf16(e); recompute both in torch
    # (fp64) from forward()'s own exact e and check the rounding matters
    W, cw = weights
    n = 7
    toks, h = _small_stream(n, seed=33)
    r = oracle.forward(toks, np.array([0, n], np.int32), h, W, cw, 65_536, _rows)
    flat = r["e"].ravel()
    e_b = np.array([_rne_bf16_exact(float(a)) for a in flat]).reshape(r["e"].shape)
    np.testing.assert_array_equal(r["e_b"], e_b)
    hf = torch.from_numpy(inputs.bf16_bits_to_f32(h).astype(np.float64))
    w = inputs.bf16_bits_to_f32(cw).astype(np.float64)

    def gate_and_y(e):
        et = torch.from_numpy(e)
        hn = hf / torch.sqrt((hf * hf).mean(dim=1, keepdim=True) + 1e-6)
        en = et / torch.sqrt((et * et).mean(dim=1, keepdim=True) + 1e-6)
        g = torch.sigmoid((hn * en).sum(dim=1) / math.sqrt(D)).numpy()
        return g, _conv_torch(g[:, None] * e, w, np.zeros((3, D)))

    g_ref, y_ref = gate_and_y(e_b)
    np.testing.assert_allclose(r["g"], g_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["y"], y_ref, rtol=1e-12, atol=1e-13)
    g_raw, y_raw = gate_and_y(r["e"])
    assert np.max(np.abs(y_raw - r["y"])) > 1e-5      # a dropped rounding would fail the check above


def _run_chunks(toks, h, cuts, W, cw, R):
    hid, hln = np.zeros((1, 2), np.int32), np.zeros(1, np.int32)
    st = np.zeros((1, 3, D))
    pos, outs, ys = 0, [], []
    for L in cuts:
        r = oracle.forward(toks[pos:pos + L], np.array([0, L], np.int32), h[pos:pos + L], W, cw, R,
                           _rows, hid, hln, st)
        hid, hln, st = r["hist_ids"], r["hist_len"], r["conv_state"]
        outs.append(r["out"])
        ys.append(r["y"])
        pos += L
    return np.concatenate(outs), np.concatenate(ys)


def test_chunked_equals_unchunked_and_decode_equals_prefill(weights):
    W, cw = weights
    n = 24
    toks, h = _small_stream(n, seed=14)
    full_out, full_y = _run_chunks(toks, h, [n], W, cw, 65_536)
    for cuts in ([1, 2, 3, 18], [5, 0, 19], [1] * n):
        out, y = _run_chunks(toks, h, cuts, W, cw, 65_536)
        assert np.array_equal(out, full_out) and np.array_equal(y, full_y)


def test_sequences_in_one_call_are_independent(weights):
    W, cw = weights
    toks, h = _small_stream(30, seed=15)
    cu = np.array([0, 4, 4, 5, 30], np.int32)
    r = oracle.forward(toks, cu, h, W, cw, 65_536, _rows)
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        alone = oracle.forward(toks[a:b], np.array([0, b - a], np.int32), h[a:b], W, cw, 65_536, _rows)
        assert np.array_equal(alone["out"], r["out"][a:b])
        assert np.array_equal(alone["row_ids"], r["row_ids"][a:b])


def test_results_do_not_depend_on_the_thread_count(weights):
    # the bench reports the oracle on all host cores and on one thread; each
    # output element is computed by one thread in one fixed order
    W, cw = weights
    toks, h = _small_stream(40, seed=16)
    cu = np.array([0, 7, 40], np.int32)
    before = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        one = oracle.forward(toks, cu, h, W, cw, 65_536, _rows)
        oracle.set_num_threads(4)
        four = oracle.forward(toks, cu, h, W, cw, 65_536, _rows)
    finally:
        oracle.set_num_threads(before)
    for k in ("row_ids", "x", "e", "g", "y", "out", "conv_state"):
        assert np.array_equal(one[k], four[k]), k
