// a4: gate, causal short conv with carried state, residual add.
//
// The arithmetic (gate sums, gate, conv taps, residual add, state and
// history updates) is in ple_fuse_common.h, shared by both kernels here and
// by the one-launch decode step, so that a token's result does not depend on
// which kernel runs it; the short conv is its own op in the vLLM port
// (kipfel.ltd Thor article, section 5, qwen4_exp_ple_short_conv).
// fuse_token_kernel (short calls: decode steps, and calls of many short
// sequences): one token per block, so the tokens of a call run side by side.
// fuse_stream_kernel (long calls): one block per CU walks a contiguous range
// of tokens, kStep at a time, with one barrier per step (the gates of step i
// are added up while step i-1 is convolved). The e and h rows of the next
// step are loaded while the current ones are computed, and the v of the last
// three tokens stay in registers (a ring reset from the carried state at
// each sequence start), so every row of e and h is read once; a block first
// runs the three tokens before its range (without output) to fill the ring.
// Whichever block holds a sequence's last token writes the new conv state
// and n-gram history; the old state is read from a copy taken before this
// kernel, so the in-place update cannot race with readers.
#include "ple_fuse_common.h"

namespace ple {
namespace {

using namespace fuse;

constexpr int kSmallT = 1024;          // calls up to this many tokens run one token per block
constexpr int kStep = 6;               // fuse_stream_kernel: tokens per step
constexpr int kStreamBlocks = 256;     // fuse_stream_kernel: one block per CU
constexpr int kMinRange = 8;           // fuse_stream_kernel: fewest tokens per block
constexpr int kMinAvgSeq = 2;          // fuse_stream_kernel: fewest tokens per sequence on average

// One token per block (short calls). The token's sequence is found first, so
// that the carried-state taps load beside e and h; window rows before the
// sequence start are neither loaded nor gated (a decode step, whose tokens
// each start a sequence, reads its own row only). hw: where the h rows of the
// three earlier tokens are read (a copy when out is h), or NULL for h.
__global__ void __launch_bounds__(kThreads)
fuse_token_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16, int64_t T,
                  const int32_t* __restrict__ cu, int32_t S, const int32_t* __restrict__ tokens,
                  const uint16_t* __restrict__ conv_w, const float* __restrict__ snap,
                  float* __restrict__ conv_state, int32_t* __restrict__ hist_ids,
                  int32_t* __restrict__ hist_len, uint16_t* out, float eps, float* __restrict__ gate_out,
                  float* __restrict__ y_out, const uint16_t* __restrict__ hw) {
    __shared__ float red_s[4][kRows][3];
    __shared__ float g_s[4];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    TokenFuse f;
    token_begin(f, t, T, cu, S, h, hw, conv_w, snap, conv_state, tid);
    token_state(f, tid);
    token_end(f, t, e16, tokens, conv_state, hist_ids, hist_len, out, eps, gate_out, y_out, red_s, g_s, tid);
}

// e and h of tokens t .. t+kStep-1 for this thread; tokens past `last` read
// row `last` (in bounds; their results are never used). The row clamp is
// scalar and no branch surrounds the loads, so the compiler can count them
// and wait only for the step a computation needs.
template <int kN>
__device__ __forceinline__ void load_step(const uint16_t* __restrict__ e16, const uint16_t* __restrict__ h,
                                          int64_t t, int64_t last, uint32_t cb, u32x2 (&pe)[kN],
                                          u32x2 (&ph)[kN]) {
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        const int64_t r = t + j < last ? t + j : last;
        pe[j] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(e16 + r * kD) + cb);
        ph[j] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(h + r * kD) + cb);
    }
}

// One block per CU walks tokens a .. b-1 (and up to three before a, without
// output, to fill the ring) kN at a time, with one barrier per step: step
// i's gate row sums go to LDS, then after the barrier one wave adds them up
// while every wave convolves and writes step i-1, whose gates were formed
// after the previous barrier. Three e/h register buffers rotate (step i+1
// loading, step i gated, step i-1 convolved), the loop unrolled by three so
// each is named statically. A step that neither starts nor ends a sequence
// convolves from one statically indexed window with no per-token
// bookkeeping; v of the last three tokens stays in registers, reset from the
// carried state at a sequence start.
template <int kN>
__global__ void __launch_bounds__(kThreads)
fuse_stream_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ e16, int64_t T,
                 const int32_t* __restrict__ cu, int32_t S, const int32_t* __restrict__ tokens,
                 const uint16_t* __restrict__ conv_w, const float* __restrict__ snap,
                 float* __restrict__ conv_state, int32_t* __restrict__ hist_ids,
                 int32_t* __restrict__ hist_len, uint16_t* out, float eps, float* __restrict__ gate_out,
                 float* __restrict__ y_out, int64_t per_block, const uint16_t* __restrict__ halo) {
    static_assert(kN >= 3, "the three tokens before a range must fit in the first step");
    __shared__ float red_s[2][kN][kRows][3];
    __shared__ float g_s[2][kN];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t cb = (uint32_t)tid * FPT * 2;
    const int64_t a = (int64_t)blockIdx.x * per_block;
    if (a >= T) return;
    const int64_t b = a + per_block < T ? a + per_block : T;
    int s = seq_of(cu, S, a);
    int64_t st = cu[s], en = cu[s + 1];
    if (st < 0 || st > a) st = a;
    if (en <= a || en > T) en = a + 1;
    const int64_t a0 = a - 3 > st ? a - 3 : st;

    float w[FPT][kTaps];
    load_conv_w(conv_w, tid, w);
    float r0[FPT] = {}, r1[FPT] = {}, r2[FPT] = {};

    // gates of step tb from red_s[sel] (threads < kN)
    auto reduce = [&](int64_t tb, int sel) {
        if (tid < kN) {
            const float g = gate_reduce(red_s[sel][tid], eps);
            g_s[sel][tid] = g;
            const int64_t t = tb + tid;
            if (gate_out && t >= a && t < b) gate_out[t] = g;
        }
    };
    // conv, out and state of step tb with the gates in g_s[sel]
    auto convolve = [&](int64_t tb, const u32x2 (&ce)[kN], const u32x2 (&ch)[kN], int sel) {
        char* ob = reinterpret_cast<char*>(out) + tb * (kD * 2);
        if (tb >= a && tb + kN <= b && st < tb && en > tb + kN && !y_out) {
            float vw[kN + 3][FPT];
#pragma unroll
            for (int q = 0; q < FPT; ++q) {
                vw[0][q] = r0[q];
                vw[1][q] = r1[q];
                vw[2][q] = r2[q];
            }
#pragma unroll
            for (int j = 0; j < kN; ++j) {
                float e[FPT];
                unpack4(ce[j], e);
                const float g = g_s[sel][j];
#pragma unroll
                for (int q = 0; q < FPT; ++q) vw[j + 3][q] = g * e[q];
            }
#pragma unroll
            for (int j = 0; j < kN; ++j) {
                float y[FPT], hv[FPT];
#pragma unroll
                for (int q = 0; q < FPT; ++q) y[q] = conv4(w[q], vw[j][q], vw[j + 1][q], vw[j + 2][q], vw[j + 3][q]);
                unpack4(ch[j], hv);
                const u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
                __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(ob + (cb + (uint32_t)(j * kD * 2))));
            }
#pragma unroll
            for (int q = 0; q < FPT; ++q) {
                r0[q] = vw[kN][q];
                r1[q] = vw[kN + 1][q];
                r2[q] = vw[kN + 2][q];
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < kN; ++j) {
            const int64_t t = tb + j;
            if (t >= b) break;
            while (t >= en && s + 1 < S) {
                ++s;
                st = en;
                en = cu[s + 1];
            }
            if (st < 0 || st > t) st = t;
            if (en <= t || en > T) en = t + 1;
            if (t == st) {
                // the copy, unless this sequence starts and ends in this block
                const float* sp = (state_needs_copy(st, en, per_block) ? snap : conv_state) +
                                  (int64_t)s * 3 * kD + tid * FPT;
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(sp);
                const f32x4 c1 = *reinterpret_cast<const f32x4*>(sp + kD);
                const f32x4 c2 = *reinterpret_cast<const f32x4*>(sp + 2 * kD);
#pragma unroll
                for (int q = 0; q < FPT; ++q) {
                    r0[q] = c0[q];
                    r1[q] = c1[q];
                    r2[q] = c2[q];
                }
            }
            float e[FPT], v[FPT], y[FPT];
            unpack4(ce[j], e);
            const float g = g_s[sel][j];
#pragma unroll
            for (int q = 0; q < FPT; ++q) {
                v[q] = g * e[q];
                y[q] = conv4(w[q], r0[q], r1[q], r2[q], v[q]);
                r0[q] = r1[q];
                r1[q] = r2[q];
                r2[q] = v[q];
            }
            if (t < a) continue;
            float hv[FPT];
            unpack4(ch[j], hv);
            const u32x2 o = {pack_bf16x2(hv[0] + y[0], hv[1] + y[1]), pack_bf16x2(hv[2] + y[2], hv[3] + y[3])};
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(ob + (cb + (uint32_t)(j * kD * 2))));
            if (y_out) *reinterpret_cast<f32x4*>(y_out + t * kD + tid * FPT) = f32x4{y[0], y[1], y[2], y[3]};
            if (t == en - 1) {
                float* dp = conv_state + (int64_t)s * 3 * kD + tid * FPT;
                *reinterpret_cast<f32x4*>(dp) = f32x4{r0[0], r0[1], r0[2], r0[3]};
                *reinterpret_cast<f32x4*>(dp + kD) = f32x4{r1[0], r1[1], r1[2], r1[3]};
                *reinterpret_cast<f32x4*>(dp + 2 * kD) = f32x4{r2[0], r2[1], r2[2], r2[3]};
                if (tid == 0) update_history(tokens, hist_ids, hist_len, s, st, en);
            }
        }
    };

    u32x2 be[3][kN], bh[3][kN];
    load_step<kN>(e16, h, a0, b - 1, cb, be[0], bh[0]);
    if (halo) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (a0 + j < a)
                bh[0][j] = *reinterpret_cast<const u32x2*>(
                    reinterpret_cast<const char*>(halo) +
                    ((int64_t)blockIdx.x * 3 + 3 - (a - (a0 + j))) * (kD * 2) + cb);
    }
    // iteration i: load step i+1, gate step i, barrier, reduce step i and
    // convolve step i-1; one extra iteration convolves the last step
    const int64_t nsteps = (b - a0 + kN - 1) / kN;
    auto iter = [&](int64_t i, u32x2 (&ce)[kN], u32x2 (&ch)[kN], u32x2 (&pe)[kN], u32x2 (&ph)[kN],
                    u32x2 (&ne)[kN], u32x2 (&nh)[kN]) {
        const int64_t tb = a0 + i * kN;
        const int sel = (int)(i & 1);
        load_step<kN>(e16, h, tb + kN, b - 1, cb, ne, nh);  // past b: row b-1 again, unused
        if (i < nsteps) {
#pragma unroll
            for (int j = 0; j < kN; ++j) gate_rows(ce[j], ch[j], lane, wave, red_s[sel][j]);
        }
        __syncthreads();
        if (i < nsteps) reduce(tb, sel);
        if (i >= 1) convolve(tb - kN, pe, ph, sel ^ 1);
    };
    for (int64_t i = 0; i <= nsteps; i += 3) {
        iter(i, be[0], bh[0], be[2], bh[2], be[1], bh[1]);
        if (i + 1 > nsteps) break;
        iter(i + 1, be[1], bh[1], be[0], bh[0], be[2], bh[2]);
        if (i + 2 > nsteps) break;
        iter(i + 2, be[2], bh[2], be[1], bh[1], be[0], bh[0]);
    }
}

// out is h: the three h rows before each streaming block's range, copied to
// halo [blocks][3][kD] before the fuse kernel overwrites them
__global__ void __launch_bounds__(kThreads)
halo_copy_kernel(const uint16_t* __restrict__ h, int64_t per_block, uint16_t* __restrict__ halo) {
    const int64_t a = (int64_t)blockIdx.x * per_block;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int64_t t = a - 3 + k;
        if (t < 0) continue;
        const u32x2 q = *reinterpret_cast<const u32x2*>(h + t * kD + threadIdx.x * FPT);
        *reinterpret_cast<u32x2*>(halo + ((int64_t)blockIdx.x * 3 + k) * kD + threadIdx.x * FPT) = q;
    }
}

}  // namespace

int64_t fuse_block_tokens(int64_t T, int32_t S) {
    // short calls, or calls of mostly one-token sequences (every token would
    // start a sequence and stall a streaming block on its carried state): one
    // token per block. From two tokens per sequence on average the streaming
    // kernel is faster (16384 tokens in 4096 sequences: 117 against 199 us)
    if (T <= kSmallT || T < (int64_t)kMinAvgSeq * S) return 1;
    int64_t blocks = (T + kMinRange - 1) / kMinRange;
    if (blocks > kStreamBlocks) blocks = kStreamBlocks;
    return (T + blocks - 1) / blocks;
}

hipError_t launch_fuse(const uint16_t* h, const uint16_t* e16, int64_t T, const int32_t* cu,
                       int32_t S, const int32_t* tokens, const uint16_t* conv_w,
                       const float* state_snap, float* conv_state, int32_t* hist_ids,
                       int32_t* hist_len, uint16_t* out, float eps, float* gate_out, float* y_out,
                       uint16_t* h_copy, hipStream_t stream) {
    const bool in_place = out == h;
    const int64_t per_block = fuse_block_tokens(T, S);
    if (T <= kSmallT || T < (int64_t)kMinAvgSeq * S) {
        // one token per block (per_block == 1)
        if (in_place) {
            hipError_t e = hipMemcpyAsync(h_copy, h, (size_t)T * kD * 2, hipMemcpyDeviceToDevice, stream);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(fuse_token_kernel, dim3((unsigned)T), dim3(kThreads), 0, stream, h, e16, T, cu,
                           S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out, eps,
                           gate_out, y_out, in_place ? h_copy : nullptr);
    } else {
        const int64_t blocks = (T + per_block - 1) / per_block;
        if (in_place) {
            hipLaunchKernelGGL(halo_copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, per_block,
                               h_copy);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((fuse_stream_kernel<kStep>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, e16, T,
                           cu, S, tokens, conv_w, state_snap, conv_state, hist_ids, hist_len, out, eps,
                           gate_out, y_out, per_block, in_place ? h_copy : nullptr);
    }
    return hipGetLastError();
}

}  // namespace ple
