"""Shared helpers of the GPU parity tests: host<->device bf16 plumbing and
the oracle reference for sampled tokens.

Tolerances:
  row IDs, gathered bytes, x           bit-exact
  e (fp32 MFMA accumulation, K=2560)   |de| <= delta = 2e-5 * sum_c |x_c W_oc| + 1e-7
  g                                    |dg| <= gb, derived per token (gate_bound)
  y                                    |dy| <= sum_k |w_k| dv_k + 2^-22 sum_k |w_k v_k| + 1e-7
  out (bf16)                           |dout| <= 2e-2 + 1e-2 |out_ref|
The e bound: bf16 x bf16 products are exact in fp32; each output takes 160
MFMA k-steps of 16 products into an fp32 accumulator, so even with every
internal add rounded the error is at most (15 + 160) u sum |x_c W_oc| =
1.04e-5 sum |...| (u = 2^-24), doubled for margin.
The projection's output is bf16 on both sides (the oracle rounds its exact e
once, the GPU its fp32 accumulator), so an element of the GPU's bf16 e can
differ from the oracle's e_b only where e -/+ delta straddles a rounding
boundary: de_b = max |round_bf16(e -/+ delta) - e_b| (0 almost everywhere).
A flip of a large element beside a large h moves the gate measurably, so
the gate bound carries it:
  z = <h, e_b> / (rh re sqrt(D)),  gb = 1/4 (dz) + 1e-7,
  dz = (sum |h| de_b + U sum |h e_b|) / (rh re sqrt(D))
       + |z| ((sum (2 |e_b| de_b + de_b^2) / D) / (2 (mean e_b^2 + eps)) + U),
U = 46 u, u = 2^-24: the fuse kernel's fp32 reduction is at most 46 roundings
deep per sum (two bf16 dot products, four DPP steps, 40 row partials). Then
  dv = gb (|e_b| + de_b) + g de_b + 2^-23 |g e_b| per tap.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from gen import inputs, table

D = inputs.D

E_REL = 2e-5
Y_FP32 = 2.0 ** -22
U_SUM = 46 * 2.0 ** -24
OUT_ATOL = 2e-2
OUT_RTOL = 1e-2


def dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def rows(ids):
    return table.rows_cpu(ids)


def e_bound(x_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """sum_c |x_c W_oc| for each token row of x (fp64)."""
    xa = np.abs(inputs.bf16_bits_to_f32(x_bits).astype(np.float64))
    Wa = np.abs(inputs.bf16_bits_to_f32(W_bits).astype(np.float64))
    return xa @ Wa.T


def _de_b(ref: dict, W) -> np.ndarray:
    """max |round_bf16(e -/+ delta) - e_b| per element."""
    delta = E_REL * e_bound(ref["x"], W) + 1e-7
    lo = oracle.round_bf16(ref["e"] - delta)
    hi = oracle.round_bf16(ref["e"] + delta)
    return np.maximum(np.abs(lo - ref["e_b"]), np.abs(hi - ref["e_b"]))


def gate_bound(ref: dict, h_bits, W, eps: float = 1e-6) -> np.ndarray:
    """Per-token bound on |g_gpu - g_ref| (see the module docstring)."""
    de = _de_b(ref, W)
    eb = ref["e_b"]
    hf = inputs.bf16_bits_to_f32(np.asarray(h_bits).reshape(eb.shape)).astype(np.float64)
    rh = np.sqrt((hf * hf).mean(axis=1) + eps)
    re = np.sqrt((eb * eb).mean(axis=1) + eps)
    norm = rh * re * np.sqrt(D)
    z = (hf * eb).sum(axis=1) / norm
    dz = (np.abs(hf) * de).sum(axis=1) / norm + U_SUM * np.abs(hf * eb).sum(axis=1) / norm
    dz += np.abs(z) * (((2 * np.abs(eb) * de + de * de).sum(axis=1) / D) / (2 * (re * re)) + U_SUM)
    return 0.25 * dz + 1e-7


def dv_bound(ref: dict, W, h_bits) -> np.ndarray:
    """Per-element bound on |v_gpu - v_ref| for the tokens of an oracle
    forward() result (see the module docstring)."""
    de_b = _de_b(ref, W)
    gb = gate_bound(ref, h_bits, W)[:, None]
    g = np.abs(ref["g"])[:, None]
    eb = np.abs(ref["e_b"])
    return gb * (eb + de_b) + g * de_b + 2.0 ** -23 * g * eb


def y_bound(ref: dict, cu, cw, state, W, h_bits) -> np.ndarray:
    """y tolerance per element for a whole oracle forward() result whose
    incoming conv state the GPU received exactly: sum_k |w_k| dv_k over the
    taps inside the chunk, plus fp32 rounding of the conv, via the oracle's
    own conv on absolute values."""
    wa = np.asarray(cw) & 0x7FFF
    zero_h = np.zeros(ref["e"].shape, np.uint16)
    ydv, _, _ = oracle.conv_fuse(zero_h, dv_bound(ref, W, h_bits), np.ones(len(ref["g"])), cu, wa,
                                 np.zeros_like(state))
    yabs, _, _ = oracle.conv_fuse(zero_h, np.abs(ref["e_b"]), np.abs(ref["g"]), cu, wa, np.abs(state))
    return ydv + Y_FP32 * yabs + 1e-7


def head_rows(R: int):
    """Row source of the 16-lookup layout for oracle.forward_heads."""
    return lambda hs, rs: table.slices_cpu(hs, rs, R)


def oracle_windows(seqs, windows, W, cw, R, eps=1e-6, heads: bool = False, nvfp4: bool = False):
    """Reference outputs of windows of consecutive tokens.

    seqs: list of (tokens int32[n], h bf16 bits [n][D]) — whole sequences
          from their first token (history included), fresh state at 0.
    windows: list of (seq index, lo, hi): the outputs at positions lo..hi-1.
    Each window becomes its own segment: positions max(0, lo - 3) .. hi-1,
    with the two tokens before it as n-gram history. An output depends on
    its own n-grams and on v of the three tokens before it, nothing earlier,
    so rows lo..hi-1 of each segment are exact references. Returns the
    concatenated rows (window order) of row_ids, x, e, e_b, g, y, out, v
    (= g e_b, what the conv state carries) and the tolerances ytol, gtol."""
    toks, hs, cu, hid, hln, keep = [], [], [0], [], [], []
    for si, lo, hi in windows:
        st, hh = seqs[si]
        assert 0 <= lo < hi <= len(st), (si, lo, hi)
        q = max(0, lo - 3)
        toks.append(st[q:hi])
        hs.append(hh[q:hi])
        keep.extend(range(cu[-1] + lo - q, cu[-1] + hi - q))
        cu.append(cu[-1] + hi - q)
        k = min(2, q)
        hist = np.zeros(2, np.int32)
        if k:
            hist[2 - k:] = st[q - k:q]
        hid.append(hist)
        hln.append(k)
    S = len(windows)
    if nvfp4:
        fwd, src = oracle.forward_nvfp4, table.nvfp4_rows_cpu
    elif heads:
        fwd, src = oracle.forward_heads, head_rows(R)
    else:
        fwd, src = oracle.forward, rows
    cu = np.array(cu, np.int32)
    r = fwd(np.concatenate(toks), cu, np.concatenate(hs), W, cw, R,
            src, np.array(hid, np.int32), np.array(hln, np.int32), np.zeros((S, 3, D)), eps)
    keep = np.array(keep, np.int64)
    # tolerances: per token of the segments, then the kept rows. The y bound
    # sums |w_k| (dv + fp32 rounding of v) over the taps inside the segment;
    # taps before a sequence start are zero on both sides
    h_all = np.concatenate(hs)
    dv = dv_bound(r, W, h_all)
    wa = np.asarray(cw) & 0x7FFF
    zero_h = np.zeros(r["e"].shape, np.uint16)
    v = np.abs(r["g"][:, None] * r["e_b"])
    ytol, _, _ = oracle.conv_fuse(zero_h, dv + Y_FP32 * v, np.ones(len(r["g"])), cu, wa, np.zeros((S, 3, D)))
    gtol = gate_bound(r, h_all, W)
    return dict(row_ids=r["row_ids"][keep], x=r["x"][keep], e=r["e"][keep], e_b=r["e_b"][keep],
                g=r["g"][keep], y=r["y"][keep], out=r["out"][keep], v=(r["g"][:, None] * r["e_b"])[keep],
                dv=dv[keep], ytol=ytol[keep] + 1e-7, gtol=gtol[keep])


def oracle_samples(seqs, samples, W, cw, R, eps=1e-6, heads: bool = False, nvfp4: bool = False):
    """Reference outputs of sampled tokens: samples = (seq index, position)
    pairs, each a one-token window of oracle_windows."""
    return oracle_windows(seqs, [(si, p, p + 1) for si, p in samples], W, cw, R, eps, heads, nvfp4)


def state_bound(ref: dict, cu, cw, W, h_bits) -> np.ndarray:
    """Per-element bound on |conv_state_gpu - conv_state_ref| after a chunk
    whose incoming state the GPU received exactly: the new state holds the
    last three v of each sequence (dv_bound each, fp32 storage included) or,
    for sequences shorter than three tokens, shifted carried values (copied,
    exact). The oracle's own state update applied to dv with g = 1 and a
    zero carried state places each bound where its v went."""
    wa = np.asarray(cw) & 0x7FFF
    S = len(cu) - 1
    zero_h = np.zeros(ref["e"].shape, np.uint16)
    _, _, st = oracle.conv_fuse(zero_h, dv_bound(ref, W, h_bits), np.ones(len(ref["g"])), cu, wa,
                                np.zeros((S, 3, D)))
    return st + 1e-7


def check_samples(got: dict, ref: dict, W, label=""):
    """Compare GPU debug outputs at sampled tokens against oracle_samples()."""
    assert np.array_equal(got["row_ids"], ref["row_ids"]), f"{label}: row ids"
    assert np.array_equal(got["x"], ref["x"]), f"{label}: x"
    eb = e_bound(ref["x"], W)
    de = np.abs(got["e"].astype(np.float64) - ref["e"])
    assert np.all(de <= E_REL * eb + 1e-7), f"{label}: e off by {np.max(de / (eb + 1e-30)):.3g} rel"
    # the GPU's bf16 e is the RNE of its fp32 accumulator: count where it
    # differs from the oracle's rounding of the exact e
    e16 = torch.from_numpy(np.ascontiguousarray(got["e"], np.float32)).to(torch.bfloat16).double().numpy()
    flips = int(np.count_nonzero(e16 != ref["e_b"]))
    dg = np.abs(got["g"].astype(np.float64) - ref["g"])
    assert np.all(dg <= ref["gtol"]), f"{label}: gate off by {np.max(dg / ref['gtol']):.3g} of its bound"
    dy = np.abs(got["y"].astype(np.float64) - ref["y"])
    assert np.all(dy <= ref["ytol"]), f"{label}: y off by {np.max(dy / ref['ytol']):.3g} of its bound"
    out = inputs.bf16_bits_to_f32(got["out"]).astype(np.float64)
    do = np.abs(out - ref["out"])
    assert np.all(do <= OUT_ATOL + OUT_RTOL * np.abs(ref["out"])), f"{label}: out off by {do.max():.3g}"
    return dict(max_de_rel=float(np.max(de / (eb + 1e-30))), e_bf16_flips=flips, max_dg=float(dg.max()),
                max_dg_of_bound=float(np.max(dg / ref["gtol"])),
                max_dy=float(dy.max()), max_dy_of_bound=float(np.max(dy / ref["ytol"])),
                max_dout=float(do.max()))


def gather_debug(res: dict, idx) -> dict:
    """Pick rows `idx` of a debug ple_forward result, as host arrays."""
    ii = torch.as_tensor(np.asarray(idx, dtype=np.int64), device=res["out"].device)
    return dict(row_ids=res["row_ids"][ii].cpu().numpy(), x=host_bits(res["x"][ii]),
                e=res["e"][ii].cpu().numpy(), g=res["gate"][ii].cpu().numpy(),
                y=res["y"][ii].cpu().numpy(), out=host_bits(res["out"][ii]))
