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
// One block of 640 threads owns 16 consecutive tokens; thread i owns
// features 4i .. 4i+3. The gates of the block's tokens and of the three
// before them are finished once per block from the projection's per-slice
// partial sums: 380 partial vectors are loaded in parallel into LDS, then
// summed in a fixed order. A block whose 19-token window lies inside one
// sequence that goes on past the block (every block of a long prefill but
// the first and the last) issues all its e and h loads up front and
// convolves from registers. Other blocks walk their tokens with a
// three-token window that restarts from the carried state at a sequence
// start; the block holding a sequence's last token writes the new conv state
// and n-gram history. The old state is read from a copy taken before this
// kernel, so the in-place update cannot race with readers.
#include "ple_kernels.h"

namespace ple {
namespace {

constexpr int BT = 16;                 // tokens per block
constexpr int FPT = 4;                 // features per thread
constexpr int kThreads = kD / FPT;     // 640
constexpr int kWin = BT + 3;           // tokens whose gate the block needs

__device__ __forceinline__ void load4_bf16(const uint16_t* p, float v[4]) {
    u32x2 q = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16_to_f32(q[0] & 0xFFFFu);
    v[1] = bf16_to_f32(q[0] >> 16);
    v[2] = bf16_to_f32(q[1] & 0xFFFFu);
    v[3] = bf16_to_f32(q[1] >> 16);
}

// y = sum_k w_k v_k in one fixed FMA order, shared by both paths so that a
// token's result does not depend on which path (or chunking) produced it
__device__ __forceinline__ float conv4(const float w[kTaps], float v0, float v1, float v2, float v3) {
    return fmaf(w[3], v3, fmaf(w[2], v2, fmaf(w[1], v1, w[0] * v0)));
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
fuse_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16,
            const float* __restrict__ parts, int64_t T, const int32_t* __restrict__ cu, int32_t S,
            const int32_t* __restrict__ tokens, const uint16_t* __restrict__ conv_w,
            const float* __restrict__ snap, float* __restrict__ conv_state,
            int32_t* __restrict__ hist_ids, int32_t* __restrict__ hist_len, uint16_t* out,
            float eps, float* __restrict__ gate_out, float* __restrict__ y_out) {
    __shared__ f32x4 part_s[kWin][kParts];
    __shared__ float g_s[kWin];
    __shared__ int seg_s[kWin], start_s[kWin], end_s[kWin];
    __shared__ int fast_s;
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * BT;

    // gate partial sums of tokens t0-3 .. t0+BT-1, one 16-byte vector per thread
    if (tid < kWin * kParts) {
        const int i = tid / kParts, k = tid % kParts;
        const int64_t t = t0 - 3 + i;
        if (t >= 0 && t < T)
            part_s[i][k] = *reinterpret_cast<const f32x4*>(parts + (t * kParts + k) * kPartStride);
    }
    __syncthreads();
    if (tid < kWin) {
        const int64_t t = t0 - 3 + tid;
        if (t >= 0 && t < T) {
            float ee = 0.0f, he = 0.0f, hh = 0.0f;
#pragma unroll
            for (int k = 0; k < kParts; ++k) {  // fixed order: deterministic
                const f32x4 q = part_s[tid][k];
                ee += q[0];
                he += q[1];
                hh += q[2];
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
            seg_s[tid] = -1;
            start_s[tid] = 0;
            end_s[tid] = 0;
        }
    }
    __syncthreads();
    if (tid == 0) {
        // fast: the 19-token window lies in one sequence that goes on past the block
        const int64_t tl = t0 + BT - 1;
        fast_s = (t0 >= 3 && tl < T && start_s[kWin - 1] <= t0 - 3 && end_s[kWin - 1] > tl + 1) ? 1 : 0;
    }
    __syncthreads();

    const int c0 = tid * FPT;
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

    if (fast_s) {
        float e[kWin][FPT], hv[BT][FPT];
#pragma unroll
        for (int i = 0; i < kWin; ++i) load4_bf16(e16 + (t0 - 3 + i) * kD + c0, e[i]);
#pragma unroll
        for (int i = 0; i < BT; ++i) load4_bf16(h + (t0 + i) * kD + c0, hv[i]);
#pragma unroll
        for (int i = 0; i < kWin; ++i) {
            const float g = g_s[i];
#pragma unroll
            for (int q = 0; q < FPT; ++q) e[i][q] *= g;  // e[i] now holds v
        }
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int64_t t = t0 + i;
            float y[FPT];
#pragma unroll
            for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], e[i][q], e[i + 1][q], e[i + 2][q], e[i + 3][q]);
            u32x2 o = {pack_bf16x2(hv[i][0] + y[0], hv[i][1] + y[1]),
                       pack_bf16x2(hv[i][2] + y[2], hv[i][3] + y[3])};
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + t * kD + c0));
            if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + c0) = f32x4{y[0], y[1], y[2], y[3]};
        }
        return;
    }

    // general path: sequence starts and ends inside the block, the first block, the tail
    auto v_at = [&](int64_t p, int s, int64_t st, float v[FPT]) {
        if (p >= st) {
            float e[FPT];
            load4_bf16(e16 + p * kD + c0, e);
            const float g = g_s[p - t0 + 3];
#pragma unroll
            for (int q = 0; q < FPT; ++q) v[q] = g * e[q];
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(
                snap + ((int64_t)s * 3 + 3 - (st - p)) * kD + c0);
#pragma unroll
            for (int q = 0; q < FPT; ++q) v[q] = a[q];
        }
    };
    float win[3][FPT];
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
        float vt[FPT], hv[FPT];
        v_at(t, s, st, vt);
        load4_bf16(h + t * kD + c0, hv);
        float y[FPT];
#pragma unroll
        for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], win[0][q], win[1][q], win[2][q], vt[q]);
        u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + t * kD + c0));
        if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + c0) = f32x4{y[0], y[1], y[2], y[3]};
#pragma unroll
        for (int q = 0; q < FPT; ++q) {
            win[0][q] = win[1][q];
            win[1][q] = win[2][q];
            win[2][q] = vt[q];
        }
        if (t == en - 1) {
            // last token of sequence s: new conv state = last three v, oldest first
#pragma unroll
            for (int r = 0; r < 3; ++r)
                *reinterpret_cast<f32x4*>(conv_state + ((int64_t)s * 3 + r) * kD + c0) =
                    f32x4{win[r][0], win[r][1], win[r][2], win[r][3]};
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
