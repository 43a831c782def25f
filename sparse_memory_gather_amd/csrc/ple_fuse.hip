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
// One block of 640 threads owns 16 consecutive tokens; thread i owns
// features 4i .. 4i+3 and loads, up front, e of the block's tokens and the
// three before them and h of its own tokens (packed bf16, 8 bytes a row).
// The gates of those 19 tokens are formed by whole waves: wave w takes
// tokens w and w + 10 of the window, reads the two 5 KB rows with 16-byte
// loads (L2 hits: the block's own loads of the same rows are in flight),
// sums e^2, h.e and h^2 over its 40 features per lane and reduces across the
// wave with DPP, always in the same order, so a token's gate does not depend
// on which block or chunk computes it. Each output then takes its four taps
// from registers, or from the carried state where a tap lies before its
// sequence's first token (a wave-uniform test). The block holding a
// sequence's last token writes the new conv state and n-gram history; the
// old state is read from a copy taken before this kernel, so the in-place
// update cannot race with readers.
#include "ple_kernels.h"

namespace ple {
namespace {

constexpr int BT = 16;                 // tokens per block
constexpr int FPT = 4;                 // features per thread
constexpr int kThreads = kD / FPT;     // 640
constexpr int kWaves = kThreads / 64;  // 10
constexpr int kWin = BT + 3;           // tokens whose v the block needs
constexpr int kXcds = 8;               // accelerator complex dies on MI355X

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

// v moved across lanes by a DPP pattern; lanes of rows outside kRowMask get 0
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                                 kRowMask, 0xF, false));
}

// sum over the 64 lanes of a wave, complete in lane 63
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]: pairs
    v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]: quads
    v += dpp<0x141>(v);       // row_half_mirror: eights
    v += dpp<0x140>(v);       // row_mirror: rows of 16
    v += dpp<0x142, 0xA>(v);  // row_bcast15: rows 1, 3 add rows 0, 2
    v += dpp<0x143, 0xC>(v);  // row_bcast31: rows 2, 3 add rows 0 + 1
    return v;
}

__device__ __forceinline__ int seq_of(const int32_t* cu, int32_t S, int64_t t) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ void __launch_bounds__(kThreads)
fuse_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16, int64_t T,
            const int32_t* __restrict__ cu, int32_t S, const int32_t* __restrict__ tokens,
            const uint16_t* __restrict__ conv_w, const float* __restrict__ snap,
            float* __restrict__ conv_state, int32_t* __restrict__ hist_ids,
            int32_t* __restrict__ hist_len, uint16_t* out, float eps, float* __restrict__ gate_out,
            float* __restrict__ y_out) {
    __shared__ float sum_s[kWin][3];
    __shared__ float g_s[kWin];
    __shared__ int seg_s[kWin], start_s[kWin], end_s[kWin];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // consecutive token blocks on one XCD, so that the three-token overlap of
    // neighbouring blocks is served by that XCD's L2
    const int nb = gridDim.x, b = blockIdx.x;
    const int per = nb / kXcds, rem = nb % kXcds, xcd = b % kXcds;
    const int64_t t0 = (int64_t)(xcd * per + (xcd < rem ? xcd : rem) + b / kXcds) * BT;
    const int c0 = tid * FPT;

    // this thread's e of the 19-token window and h of the block's tokens
    const u32x2 zero = {0u, 0u};
    u32x2 ep[kWin], hp[BT];
#pragma unroll
    for (int i = 0; i < kWin; ++i) {
        const int64_t t = t0 - 3 + i;
        ep[i] = (t >= 0 && t < T) ? *reinterpret_cast<const u32x2*>(e16 + t * kD + c0) : zero;
    }
#pragma unroll
    for (int i = 0; i < BT; ++i) {
        const int64_t t = t0 + i;
        hp[i] = t < T ? *reinterpret_cast<const u32x2*>(h + t * kD + c0) : zero;
    }

    // gate sums: one wave per window token, lane l holds features 8l + 512 s + 0..7
    for (int i = wave; i < kWin; i += kWaves) {
        const int64_t t = t0 - 3 + i;
        if (t < 0 || t >= T) continue;
        const u32x4* hr = reinterpret_cast<const u32x4*>(h + t * kD) + lane;
        const u32x4* er = reinterpret_cast<const u32x4*>(e16 + t * kD) + lane;
        u32x4 hv[5], ev[5];
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            hv[s] = hr[s * 64];
            ev[s] = er[s * 64];
        }
        float ee = 0.0f, he = 0.0f, hh = 0.0f;
#pragma unroll
        for (int s = 0; s < 5; ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float h0 = bf16_to_f32(hv[s][q] & 0xFFFFu), h1 = bf16_to_f32(hv[s][q] >> 16);
                const float e0 = bf16_to_f32(ev[s][q] & 0xFFFFu), e1 = bf16_to_f32(ev[s][q] >> 16);
                ee = fmaf(e1, e1, fmaf(e0, e0, ee));
                he = fmaf(h1, e1, fmaf(h0, e0, he));
                hh = fmaf(h1, h1, fmaf(h0, h0, hh));
            }
        ee = wave_sum(ee);
        he = wave_sum(he);
        hh = wave_sum(hh);
        if (lane == 63) {
            sum_s[i][0] = ee;
            sum_s[i][1] = he;
            sum_s[i][2] = hh;
        }
    }
    __syncthreads();
    if (tid < kWin) {
        const int64_t t = t0 - 3 + tid;
        if (t >= 0 && t < T) {
            const float rh = sqrtf(sum_s[tid][2] * (1.0f / kD) + eps);
            const float re = sqrtf(sum_s[tid][0] * (1.0f / kD) + eps);
            const float z = sum_s[tid][1] / (rh * re) * (1.0f / 50.596443f);  // 1/sqrt(2560)
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
        const u32x4* wp = reinterpret_cast<const u32x4*>(conv_w + c0 * kTaps);
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

#pragma unroll
    for (int i = 0; i < BT; ++i) {
        const int64_t t = t0 + i;
        if (t >= T) break;
        const int s = seg_s[i + 3];
        const int64_t st = start_s[i + 3], en = end_s[i + 3];
        // v at positions t-3 .. t (window slots i .. i+3)
        float v[kTaps][FPT];
#pragma unroll
        for (int k = 0; k < kTaps; ++k) {
            const int64_t p = t - 3 + k;
            if (p >= st) {
                float e[FPT];
                unpack4(ep[i + k], e);
                const float g = g_s[i + k];
#pragma unroll
                for (int q = 0; q < FPT; ++q) v[k][q] = g * e[q];
            } else {
                const f32x4 a = *reinterpret_cast<const f32x4*>(snap + ((int64_t)s * 3 + 3 - (st - p)) * kD + c0);
#pragma unroll
                for (int q = 0; q < FPT; ++q) v[k][q] = a[q];
            }
        }
        float hv[FPT], y[FPT];
        unpack4(hp[i], hv);
#pragma unroll
        for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], v[0][q], v[1][q], v[2][q], v[3][q]);
        const u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + t * kD + c0));
        if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + c0) = f32x4{y[0], y[1], y[2], y[3]};
        if (t == en - 1) {
            // last token of sequence s: new conv state = v at t-2, t-1, t
#pragma unroll
            for (int r = 0; r < 3; ++r)
                *reinterpret_cast<f32x4*>(conv_state + ((int64_t)s * 3 + r) * kD + c0) =
                    f32x4{v[r + 1][0], v[r + 1][1], v[r + 1][2], v[r + 1][3]};
            if (tid == 0) {
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
        }
    }
}

}  // namespace

hipError_t launch_fuse(const uint16_t* h, const uint16_t* e16, int64_t T, const int32_t* cu,
                       int32_t S, const int32_t* tokens, const uint16_t* conv_w,
                       const float* state_snap, float* conv_state, int32_t* hist_ids,
                       int32_t* hist_len, uint16_t* out, float eps, float* gate_out, float* y_out,
                       hipStream_t stream) {
    const int64_t blocks = (T + BT - 1) / BT;
    hipLaunchKernelGGL(fuse_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, e16, T, cu,
                       S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out, eps,
                       gate_out, y_out);
    return hipGetLastError();
}

}  // namespace ple
