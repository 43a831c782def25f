// a4 device code shared by the fuse kernels and the one-launch decode step:
// the gate, the short conv, the residual add and the state updates, with one
// operation order wherever they run, so that a token's result does not depend
// on which kernel computes it.
//
// After the projection the looked-up vector is gated, short-convolved and
// fused into the hidden states (mengman.github.io "Qwen3.8-Flash-Next 端侧部署
// 01", n-gram embedding section); with e the projection's bf16 output:
//   g = sigmoid(<h/rms(h), e/rms(e)> / sqrt(2560)), rms(z) = sqrt(mean(z^2)+eps),
//   v = g e,  y[t][c] = sum_k w[c][k] v[t-3+k][c],  out = bf16(h + y),
// with v before a sequence's first token taken from the carried state.
//
// A block has 640 threads and thread i owns features 4i .. 4i+3 (packed
// bf16, 8 bytes of a row):
//   - gate sums e^2, h.e, h^2 straight from the packed pairs with the bf16
//     dot-product instruction (products of bf16 values are exact in fp32);
//     each row of 16 lanes reduces to one sum with DPP, and one thread per
//     token adds the block's 40 row sums in row order;
//   - v = g e; y = the four taps in one fixed FMA order, taps before a
//     sequence's first token taken from the carried state; out = bf16(h + y).
#pragma once

#include "ple_ngram.h"

namespace ple {
namespace fuse {

constexpr int FPT = 4;                 // features per thread
constexpr int kThreads = kD / FPT;     // 640
constexpr int kWaves = kThreads / 64;  // 10
constexpr int kRows = kWaves * 4;      // rows of 16 lanes in a block

__device__ __forceinline__ void unpack4(const u32x2& q, float v[4]) {
    v[0] = bf16_to_f32(q[0] & 0xFFFFu);
    v[1] = bf16_to_f32(q[0] >> 16);
    v[2] = bf16_to_f32(q[1] & 0xFFFFu);
    v[3] = bf16_to_f32(q[1] >> 16);
}

// y = sum_k w_k v_k in one fixed FMA order
__device__ __forceinline__ float conv4(const float w[kTaps], float v0, float v1, float v2, float v3) {
    return fmaf(w[3], v3, fmaf(w[2], v2, fmaf(w[1], v1, w[0] * v0)));
}

// v moved across lanes by a DPP pattern (rows of 16 lanes)
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                                 0xF, 0xF, false));
}

// sum over each row of 16 lanes, complete in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: quads
    v += dpp<0x141>(v);  // row_half_mirror: eights
    v += dpp<0x140>(v);  // row_mirror: sixteens
    return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi on packed bf16 pairs
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// the gate from a token's three sums (fixed operation order, no contraction)
__device__ __forceinline__ float gate_of(float ee, float he, float hh, float eps) {
#pragma clang fp contract(off)
    const float rh = sqrtf(hh * (1.0f / kD) + eps);
    const float re = sqrtf(ee * (1.0f / kD) + eps);
    const float z = he / (rh * re) * (1.0f / 50.596443f);  // 1/sqrt(2560)
    return 1.0f / (1.0f + expf(-z));
}

// gate sums of one token over this thread's four features, reduced over the
// row of 16 lanes; lane 15 of each row stores them in red[row]
__device__ __forceinline__ void gate_rows(const u32x2& qe, const u32x2& qh, int lane, int wave,
                                          float (*red)[3]) {
    float ee = dot2(qe[1], qe[1], dot2(qe[0], qe[0], 0.0f));
    float he = dot2(qh[1], qe[1], dot2(qh[0], qe[0], 0.0f));
    float hh = dot2(qh[1], qh[1], dot2(qh[0], qh[0], 0.0f));
    ee = row_sum(ee);
    he = row_sum(he);
    hh = row_sum(hh);
    if ((lane & 15) == 15) {
        float* r = red[wave * 4 + (lane >> 4)];
        r[0] = ee;
        r[1] = he;
        r[2] = hh;
    }
}

// a token's gate from its 40 row sums, added in row order
__device__ __forceinline__ float gate_reduce(const float (*red)[3], float eps) {
    float ee = 0.0f, he = 0.0f, hh = 0.0f;
#pragma unroll 8
    for (int r = 0; r < kRows; ++r) {
        ee += red[r][0];
        he += red[r][1];
        hh += red[r][2];
    }
    return gate_of(ee, he, hh, eps);
}

// conv_w of this thread's four features as fp32, w[feature][tap]
__device__ __forceinline__ void load_conv_w(const uint16_t* __restrict__ conv_w, int tid, float w[FPT][kTaps]) {
    const u32x4* wp = reinterpret_cast<const u32x4*>(conv_w + tid * FPT * kTaps);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x4 q = wp[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = i * 8 + 2 * j;  // element index within the 4 x 4 block
            w[idx / 4][idx % 4] = bf16_to_f32(q[j] & 0xFFFFu);
            w[(idx + 1) / 4][(idx + 1) % 4] = bf16_to_f32(q[j] >> 16);
        }
    }
}

// n-gram history of sequence s after its last token en-1 (sequence start st)
__device__ __forceinline__ void update_history(const int32_t* tokens, int32_t* hist_ids, int32_t* hist_len,
                                               int s, int64_t st, int64_t en) {
    int hl = hist_len[s];
    if (hl < 0 || hl > 2) hl = 0;
    const int64_t L = en - st;
    if (L >= 2) {
        hist_ids[2 * s] = tokens[en - 2];
        hist_ids[2 * s + 1] = tokens[en - 1];
        hist_len[s] = 2;
    } else if (hl >= 1) {
        hist_ids[2 * s] = hist_ids[2 * s + 1];
        hist_ids[2 * s + 1] = tokens[en - 1];
        hist_len[s] = 2;
    } else {
        hist_ids[2 * s + 1] = tokens[en - 1];
        hist_len[s] = 1;
    }
}

// One token, one block of kThreads. Window slot k is token t-3+k; slots
// below `first` lie before the sequence start and take the carried state.
struct TokenFuse {
    int s;
    int64_t st, en;
    int first;
    const float* sbase;   // where the carried state is read (the copy, or conv_state)
    f32x4 c[3];           // carried-state taps (k < first)
    u32x2 hp[4], ep[4];   // h and e of the window (k >= first)
    float w[FPT][kTaps];
};

// the token's sequence and window, its h rows and conv weights: everything
// that does not need e or the carried state. hw: where the h rows of the
// three earlier tokens are read (a copy when out is h), or NULL for h.
// window = false leaves those three rows out (token_window reads them later).
// cu, tokens may be copies in LDS.
__device__ __forceinline__ void token_begin(TokenFuse& f, int64_t t, int64_t T, const int32_t* cu, int32_t S,
                                            const uint16_t* __restrict__ h, const uint16_t* __restrict__ hw,
                                            const uint16_t* __restrict__ conv_w, const float* snap,
                                            const float* conv_state, int tid, bool window = true) {
    const uint32_t cb = (uint32_t)tid * FPT * 2;
    f.s = seq_of(cu, S, t);
    f.st = cu[f.s];
    f.en = cu[f.s + 1];
    if (f.st < 0 || f.st > t) f.st = t;  // malformed cu_seqlens (flagged elsewhere): stay in bounds
    if (f.en <= t || f.en > T) f.en = t + 1;
    f.first = f.st > t - 3 ? (int)(f.st - (t - 3)) : 0;
    // one token per block: a one-token sequence reads and rewrites its own
    // state in this block, so it was not copied
    f.sbase = state_needs_copy(f.st, f.en, 1) ? snap : conv_state;
    const uint16_t* hwin = hw ? hw : h;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k >= f.first && (window || k == 3)) {
            const int64_t p = t - 3 + k;
            f.hp[k] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>((k < 3 ? hwin : h) + p * kD) + cb);
        } else {
            f.hp[k] = u32x2{0u, 0u};
        }
    }
    load_conv_w(conv_w, tid, f.w);
}

// the h rows of the window's earlier tokens, from hw, after a token_begin
// with window = false
__device__ __forceinline__ void token_window(TokenFuse& f, int64_t t, const uint16_t* __restrict__ hw, int tid) {
    const uint32_t cb = (uint32_t)tid * FPT * 2;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (k >= f.first)
            f.hp[k] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(hw + (t - 3 + k) * kD) + cb);
}

// the carried-state taps of the window
__device__ __forceinline__ void token_state(TokenFuse& f, int tid) {
#pragma unroll
    for (int k = 0; k < 3; ++k)
        f.c[k] = k < f.first
                     ? *reinterpret_cast<const f32x4*>(f.sbase + ((int64_t)f.s * 3 + 3 - (f.first - k)) * kD + tid * FPT)
                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// e rows, gate, conv, out; the new state and history when t ends its
// sequence. red_s, g_s: LDS of the block; every thread of the block calls it.
__device__ __forceinline__ void token_end(TokenFuse& f, int64_t t, const uint16_t* __restrict__ e16,
                                          const int32_t* __restrict__ tokens, float* conv_state, int32_t* hist_ids,
                                          int32_t* hist_len, uint16_t* out, float eps, float* gate_out,
                                          float* y_out, float (*red_s)[kRows][3], float* g_s, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t cb = (uint32_t)tid * FPT * 2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k >= f.first) {
            const int64_t p = t - 3 + k;
            f.ep[k] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(e16 + p * kD) + cb);
        } else {
            f.ep[k] = u32x2{0u, 0u};
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (k >= f.first) gate_rows(f.ep[k], f.hp[k], lane, wave, red_s[k]);
    __syncthreads();
    if (tid < 4 && tid >= f.first) {
        const float g = gate_reduce(red_s[tid], eps);
        g_s[tid] = g;
        if (gate_out && tid == 3) gate_out[t] = g;
    }
    __syncthreads();

    // taps: v = g e inside the sequence, the carried state before it
    float a[4][FPT];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < f.first) {
#pragma unroll
            for (int q = 0; q < FPT; ++q) a[k][q] = f.c[k][q];
        } else {
            float e[FPT];
            unpack4(f.ep[k], e);
            const float g = g_s[k];
#pragma unroll
            for (int q = 0; q < FPT; ++q) a[k][q] = g * e[q];
        }
    }
    float y[FPT], hv[FPT];
#pragma unroll
    for (int q = 0; q < FPT; ++q) y[q] = conv4(f.w[q], a[0][q], a[1][q], a[2][q], a[3][q]);
    unpack4(f.hp[3], hv);
    const u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(reinterpret_cast<char*>(out + t * kD) + cb));
    if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + tid * FPT) = f32x4{y[0], y[1], y[2], y[3]};
    if (t == f.en - 1) {
        // last token of sequence s: new conv state = v at t-2, t-1, t
        float* dp = conv_state + (int64_t)f.s * 3 * kD + tid * FPT;
#pragma unroll
        for (int r = 0; r < 3; ++r)
            *reinterpret_cast<f32x4*>(dp + r * kD) = f32x4{a[r + 1][0], a[r + 1][1], a[r + 1][2], a[r + 1][3]};
        if (tid == 0) update_history(tokens, hist_ids, hist_len, f.s, f.st, f.en);
    }
}

}  // namespace fuse
}  // namespace ple
