// a4: gate, causal short conv with carried state, residual add.
//
// After the projection the looked-up vector is gated, short-convolved and
// fused into the hidden states (mengman.github.io "Qwen3.8-Flash-Next 端侧部署
// 01", n-gram embedding section); the short conv is its own op in the vLLM
// port (kipfel.ltd Thor article, section 5, qwen4_exp_ple_short_conv). Here:
//   g = sigmoid(<h/rms(h), e/rms(e)> / sqrt(2560)), rms(z) = sqrt(mean(z^2)+eps),
//   v = g e,  y[t][c] = sum_k w[c][k] v[t-3+k][c],  out = bf16(h + y),
// with v before a sequence's first token taken from the carried state.
//
// One block of 320 threads owns 16 consecutive tokens; thread i owns
// features 8i .. 8i+7 and slides a three-token window of v down its column
// in registers. The gate of each token (and of the three before the block)
// is finished once per block from the projection's per-slice partial sums.
// The block that holds a sequence's last token writes the new conv state
// and n-gram history; the old state is read from a copy taken before this
// kernel, so the in-place update cannot race with readers.
#include "ple_kernels.h"

namespace ple {
namespace {

constexpr int BT = 16;
constexpr int kThreads = kD / 8;  // 320

__device__ __forceinline__ void load8_bf16(const uint16_t* p, float v[8]) {
    u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(q[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
    }
}

__global__ void __launch_bounds__(kThreads)
fuse_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16,
            const float* __restrict__ parts, int64_t T, const int32_t* __restrict__ cu, int32_t S,
            const int32_t* __restrict__ tokens, const uint16_t* __restrict__ conv_w,
            const float* __restrict__ snap, float* __restrict__ conv_state,
            int32_t* __restrict__ hist_ids, int32_t* __restrict__ hist_len, uint16_t* out,
            float eps, float* __restrict__ gate_out, float* __restrict__ y_out) {
    __shared__ float g_s[BT + 3];
    __shared__ int seg_s[BT + 3], start_s[BT + 3], end_s[BT + 3];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * BT;

    if (tid < BT + 3) {
        const int64_t t = t0 - 3 + tid;
        if (t >= 0 && t < T) {
            int lo = 0, hi = S - 1;
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
            }
            int64_t st = cu[lo], en = cu[lo + 1];
            if (st < 0 || st > t) st = t;            // malformed cu_seqlens: stay in bounds
            if (en <= t || en > T) en = t + 1;
            float ee = 0.0f, he = 0.0f, hh = 0.0f;
            const f32x4* p = reinterpret_cast<const f32x4*>(parts + t * kParts * kPartStride);
#pragma unroll
            for (int k = 0; k < kParts; ++k) {
                f32x4 q = p[k];
                ee += q[0];
                he += q[1];
                hh += q[2];
            }
            const float rh = sqrtf(hh * (1.0f / kD) + eps);
            const float re = sqrtf(ee * (1.0f / kD) + eps);
            const float z = he / (rh * re) * (1.0f / 50.596443f);  // 1/sqrt(2560)
            const float g = 1.0f / (1.0f + expf(-z));
            g_s[tid] = g;
            seg_s[tid] = lo;
            start_s[tid] = (int)st;
            end_s[tid] = (int)en;
            if (gate_out && tid >= 3) gate_out[t] = g;
        } else {
            g_s[tid] = 0.0f;
            seg_s[tid] = -1;
            start_s[tid] = 0;
            end_s[tid] = 0;
        }
    }
    __syncthreads();

    const int c0 = tid * 8;
    float w[8][4];
    {
        const u32x4* wp = reinterpret_cast<const u32x4*>(conv_w + c0 * kTaps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 q = wp[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = i * 8 + 2 * j;  // element index within the 8 x 4 block
                w[idx / 4][idx % 4] = bf16_to_f32(q[j] & 0xFFFFu);
                w[(idx + 1) / 4][(idx + 1) % 4] = bf16_to_f32(q[j] >> 16);
            }
        }
    }

    // v of token p (p in [t0-3, t0+BT)) for a token of sequence s starting at st
    auto v_at = [&](int64_t p, int s, int64_t st, float v[8]) {
        if (p >= st) {
            float e[8];
            load8_bf16(e16 + p * kD + c0, e);
            const float g = g_s[p - t0 + 3];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = g * e[q];
        } else {
            const f32x4* sp = reinterpret_cast<const f32x4*>(
                snap + ((int64_t)s * 3 + 3 - (st - p)) * kD + c0);
            f32x4 a = sp[0], b = sp[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[q] = a[q];
                v[4 + q] = b[q];
            }
        }
    };

    float win[3][8];
    for (int i = 0; i < BT; ++i) {
        const int64_t t = t0 + i;
        if (t >= T) break;
        const int s = seg_s[i + 3];
        const int64_t st = start_s[i + 3], en = end_s[i + 3];
        if (i == 0 || t == st) {
            v_at(t - 3, s, st, win[0]);
            v_at(t - 2, s, st, win[1]);
            v_at(t - 1, s, st, win[2]);
        }
        float vt[8], hv[8];
        v_at(t, s, st, vt);
        load8_bf16(h + t * kD + c0, hv);
        float y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            y[q] = w[q][0] * win[0][q] + w[q][1] * win[1][q] + w[q][2] * win[2][q] + w[q][3] * vt[q];
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(hv[2 * q] + y[2 * q], hv[2 * q + 1] + y[2 * q + 1]);
        *reinterpret_cast<u32x4*>(out + t * kD + c0) = o;
        if (y_out) {
            f32x4* yp = reinterpret_cast<f32x4*>(y_out + t * kD + c0);
            yp[0] = f32x4{y[0], y[1], y[2], y[3]};
            yp[1] = f32x4{y[4], y[5], y[6], y[7]};
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            win[0][q] = win[1][q];
            win[1][q] = win[2][q];
            win[2][q] = vt[q];
        }
        if (t == en - 1) {
            // last token of sequence s: new conv state = last three v, oldest first
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                f32x4* dp = reinterpret_cast<f32x4*>(conv_state + ((int64_t)s * 3 + r) * kD + c0);
                dp[0] = f32x4{win[r][0], win[r][1], win[r][2], win[r][3]};
                dp[1] = f32x4{win[r][4], win[r][5], win[r][6], win[r][7]};
            }
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

hipError_t launch_fuse(const uint16_t* h, const uint16_t* e16, const float* parts, int64_t T,
                       const int32_t* cu, int32_t S, const int32_t* tokens,
                       const uint16_t* conv_w, const float* state_snap, float* conv_state,
                       int32_t* hist_ids, int32_t* hist_len, uint16_t* out, float eps,
                       float* gate_out, float* y_out, hipStream_t stream) {
    const int64_t blocks = (T + BT - 1) / BT;
    hipLaunchKernelGGL(fuse_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, e16, parts,
                       T, cu, S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out,
                       eps, gate_out, y_out);
    return hipGetLastError();
}

}  // namespace ple
