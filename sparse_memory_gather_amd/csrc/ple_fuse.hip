// a4: gate, causal short conv with carried state, residual add.
//
// After the projection the looked-up vector is gated, short-convolved and
// fused into the hidden states (mengman.github.io "Qwen3.8-Flash-Next 端侧部署
// 01", n-gram embedding section); the short conv is its own op in the vLLM
// port (kipfel.ltd Thor article, section 5, qwen4_exp_ple_short_conv). Here,
// with e the projection's bf16 output:
//   g = sigmoid(<h/rms(h), e/rms(e)> / sqrt(2560)), rms(z) = sqrt(mean(z^2)+eps),
//   v = g e,  y[t][c] = sum_k w[c][k] v[t-3+k][c],  out = bf16(h + y),
// with v before a sequence's first token taken from the carried state.
//
// One block of 640 threads owns BT consecutive tokens; thread i owns
// features 4i .. 4i+3 and loads, up front, e and h of the block's tokens and
// of the three before them (packed bf16, 8 bytes a row). BT is 16 for long
// calls and 1 for short ones (decode steps), whose tokens then run side by
// side; a token's result does not depend on BT. The kernel is bound
// by vector ALU issue (no packed fp32 here), so the arithmetic is kept lean:
//   - gate sums e^2, h.e, h^2 straight from the packed pairs with the bf16
//     dot-product instruction (products of bf16 values are exact in fp32);
//     each wave reduces its lanes to four row sums with DPP, and after a
//     barrier one thread per token adds the 40 row sums of the block, always
//     in the same order, so a token's gate does not depend on which block or
//     chunk computes it;
//   - v = g e is formed once per window position; an output whose four taps
//     lie in its own sequence (all but a sequence's first three tokens)
//     convolves straight from those registers, the others take the taps
//     before the sequence start from the carried state (a scalar test:
//     sequence bounds are wave-uniform).
// The block holding a sequence's last token writes the new conv state and
// n-gram history; the old state is read from a copy taken before this
// kernel, so the in-place update cannot race with readers.
#include "ple_kernels.h"

namespace ple {
namespace {

constexpr int FPT = 4;                 // features per thread
constexpr int kThreads = kD / FPT;     // 640
constexpr int kWaves = kThreads / 64;  // 10
constexpr int kSmallT = 1024;          // calls up to this many tokens run one token per block

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

__device__ __forceinline__ int seq_of(const int32_t* cu, int32_t S, int64_t t) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// BT tokens per block (16 for long calls; 1 for short ones, so that decode
// steps, whose tokens each start a sequence, run side by side)
template <int BT>
__global__ void __launch_bounds__(kThreads)
fuse_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16, int64_t T,
            const int32_t* __restrict__ cu, int32_t S, const int32_t* __restrict__ tokens,
            const uint16_t* __restrict__ conv_w, const float* __restrict__ snap,
            float* __restrict__ conv_state, int32_t* __restrict__ hist_ids,
            int32_t* __restrict__ hist_len, uint16_t* out, float eps, float* __restrict__ gate_out,
            float* __restrict__ y_out) {
    constexpr int kWin = BT + 3;       // tokens whose v the block needs
    constexpr int kRows = kWaves * 4;  // rows of 16 lanes in the block
    __shared__ float red_s[kRows][kWin][3];
    __shared__ float g_s[kWin];
    __shared__ int seg_s[kWin], start_s[kWin], end_s[kWin];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * BT;
    const uint32_t cb = (uint32_t)tid * FPT * 2;  // byte offset of this thread's features in a row

    // this thread's e and h of the 19-token window
    const u32x2 zero = {0u, 0u};
    u32x2 ep[kWin], hp[kWin];
    if (t0 >= 3 && t0 + BT <= T) {
        // interior block: one uniform base, 32-bit per-lane offsets
        const char* eb = reinterpret_cast<const char*>(e16) + (t0 - 3) * (kD * 2);
        const char* hb = reinterpret_cast<const char*>(h) + (t0 - 3) * (kD * 2);
#pragma unroll
        for (int i = 0; i < kWin; ++i) {
            const uint32_t off = cb + (uint32_t)(i * kD * 2);
            ep[i] = *reinterpret_cast<const u32x2*>(eb + off);
            hp[i] = *reinterpret_cast<const u32x2*>(hb + off);
        }
    } else {
        // first and last blocks: unconditional loads from a clamped (in-bounds)
        // row, then a select, so no branches around the loads
#pragma unroll
        for (int i = 0; i < kWin; ++i) {
            const int64_t t = t0 - 3 + i;
            const bool in = t >= 0 && t < T;
            const int64_t tc = t < 0 ? 0 : (t >= T ? T - 1 : t);
            const u32x2 qe = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(e16) + tc * (kD * 2) + cb);
            const u32x2 qh = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(h) + tc * (kD * 2) + cb);
            ep[i] = in ? qe : zero;
            hp[i] = in ? qh : zero;
        }
    }

    // gate sums: four features per thread (bf16 dot products), then the rows
    // of 16 lanes; lane 15 of each row keeps the row's sums
#pragma unroll
    for (int i = 0; i < kWin; ++i) {
        const u32x2 qe = ep[i], qh = hp[i];
        float ee = dot2(qe[1], qe[1], dot2(qe[0], qe[0], 0.0f));
        float he = dot2(qh[1], qe[1], dot2(qh[0], qe[0], 0.0f));
        float hh = dot2(qh[1], qh[1], dot2(qh[0], qh[0], 0.0f));
        ee = row_sum(ee);
        he = row_sum(he);
        hh = row_sum(hh);
        if ((lane & 15) == 15) {
            const int r = wave * 4 + (lane >> 4);
            red_s[r][i][0] = ee;
            red_s[r][i][1] = he;
            red_s[r][i][2] = hh;
        }
    }
    __syncthreads();
    if (tid < kWin) {
        const int64_t t = t0 - 3 + tid;
        if (t >= 0 && t < T) {
            float ee = 0.0f, he = 0.0f, hh = 0.0f;
#pragma unroll 8
            for (int r = 0; r < kRows; ++r) {
                ee += red_s[r][tid][0];
                he += red_s[r][tid][1];
                hh += red_s[r][tid][2];
            }
            const float rh = sqrtf(hh * (1.0f / kD) + eps);
            const float re = sqrtf(ee * (1.0f / kD) + eps);
            const float z = he / (rh * re) * (1.0f / 50.596443f);  // 1/sqrt(2560)
            const float g = 1.0f / (1.0f + expf(-z));
            g_s[tid] = g;
            if (gate_out && tid >= 3) gate_out[t] = g;
            const int s = seq_of(cu, S, t);
            int64_t st = cu[s], en = cu[s + 1];
            if (st < 0 || st > t) st = t;            // malformed cu_seqlens: stay in bounds
            if (en <= t || en > T) en = t + 1;
            seg_s[tid] = s;
            start_s[tid] = (int)st;
            end_s[tid] = (int)en;
        } else {
            g_s[tid] = 0.0f;
            seg_s[tid] = 0;
            start_s[tid] = 0;
            end_s[tid] = 0;
        }
    }
    __syncthreads();

    float w[FPT][kTaps];
    {
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

    // v = g e at every window position
    float v[kWin][FPT];
#pragma unroll
    for (int j = 0; j < kWin; ++j) {
        float e[FPT];
        unpack4(ep[j], e);
        const float g = g_s[j];
#pragma unroll
        for (int q = 0; q < FPT; ++q) v[j][q] = g * e[q];
    }
    char* ob = reinterpret_cast<char*>(out) + t0 * (kD * 2);
#pragma unroll
    for (int i = 0; i < BT; ++i) {
        const int64_t t = t0 + i;
        if (t >= T) break;
        // sequence bounds of token t are the same in every lane: keep them scalar
        const int s = __builtin_amdgcn_readfirstlane(seg_s[i + 3]);
        const int st = __builtin_amdgcn_readfirstlane(start_s[i + 3]);
        const int en = __builtin_amdgcn_readfirstlane(end_s[i + 3]);
        // tap k is position t-3+k (window slot i+k); before the sequence start
        // it comes from the carried state
        auto tap = [&](int k, float a[FPT]) {
            const int p = (int)t - 3 + k;
            if (p >= st) {
#pragma unroll
                for (int q = 0; q < FPT; ++q) a[q] = v[i + k][q];
            } else {
                const f32x4 c = *reinterpret_cast<const f32x4*>(snap + ((int64_t)s * 3 + 3 - (st - p)) * kD +
                                                                tid * FPT);
#pragma unroll
                for (int q = 0; q < FPT; ++q) a[q] = c[q];
            }
        };
        float y[FPT];
        if ((int)t - 3 >= st) {
#pragma unroll
            for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], v[i][q], v[i + 1][q], v[i + 2][q], v[i + 3][q]);
        } else {
            float a0[FPT], a1[FPT], a2[FPT], a3[FPT];
            tap(0, a0);
            tap(1, a1);
            tap(2, a2);
            tap(3, a3);
#pragma unroll
            for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], a0[q], a1[q], a2[q], a3[q]);
        }
        float hv[FPT];
        unpack4(hp[i + 3], hv);
        const u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(ob + (cb + (uint32_t)(i * kD * 2))));
        if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + tid * FPT) = f32x4{y[0], y[1], y[2], y[3]};
        if ((int)t == en - 1) {
            // last token of sequence s: new conv state = v at t-2, t-1, t
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                float a[FPT];
                tap(r + 1, a);
                *reinterpret_cast<f32x4*>(conv_state + ((int64_t)s * 3 + r) * kD + tid * FPT) =
                    f32x4{a[0], a[1], a[2], a[3]};
            }
            if (tid == 0) {
                int hl = hist_len[s];
                if (hl < 0 || hl > 2) hl = 0;
                const int L = en - st;
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
        }
    }
}

}  // namespace

hipError_t launch_fuse(const uint16_t* h, const uint16_t* e16, int64_t T, const int32_t* cu,
                       int32_t S, const int32_t* tokens, const uint16_t* conv_w,
                       const float* state_snap, float* conv_state, int32_t* hist_ids,
                       int32_t* hist_len, uint16_t* out, float eps, float* gate_out, float* y_out,
                       hipStream_t stream) {
    if (T <= kSmallT) {
        hipLaunchKernelGGL(fuse_kernel<1>, dim3((unsigned)T), dim3(kThreads), 0, stream, h, e16, T, cu,
                           S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out, eps,
                           gate_out, y_out);
    } else {
        const int64_t blocks = (T + 15) / 16;
        hipLaunchKernelGGL(fuse_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, e16, T,
                           cu, S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out, eps,
                           gate_out, y_out);
    }
    return hipGetLastError();
}

}  // namespace ple
