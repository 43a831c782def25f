// a3: projection e = x W^T (bf16 in, fp32 accumulate) on gfx950 MFMA.
//
// The looked-up vector is projected before the gate and the short conv
// (mengman.github.io "Qwen3.8-Flash-Next 端侧部署 01", n-gram embedding
// section). It is the only dense contraction on the path: [T x 2560] times
// [2560 x 2560]^T, both operands K-contiguous.
//
// Block tile 256 tokens x 256 features x 64 k, four waves in a 2x2 grid,
// each wave a 128 x 128 sub-tile of 4x4 v_mfma_f32_32x32x16_bf16 tiles. W
// rows feed the MFMA A operand and tokens the B operand, so a lane's
// accumulators hold one token and runs of four consecutive features (8-byte
// bf16 stores). Operands are double-buffered in LDS (128 KB), with the 16-byte
// chunks of each 128-byte row XOR-swizzled by (row & 7) so that the MFMA
// fragment reads are bank-conflict free.
//
// Forward mode also reduces, per token and per 128-feature slice, the sums
// e^2, h.e and h^2 that the gate needs (fp32, before e is rounded to bf16).
#include <atomic>

#include "ple_kernels.h"

namespace ple {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;  // tokens per block
constexpr int BN = 256;  // features per block
constexpr int BK = 64;   // k per stage
constexpr int KT = kD / BK;
constexpr int kThreads = 256;
constexpr int kLdsBytes = 2 * (BM + BN) * BK * 2;  // 131072

template <bool kFwd>
__global__ void __launch_bounds__(kThreads, 1)
proj_kernel(const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ W,
            float* __restrict__ e32, uint16_t* __restrict__ e16, const uint16_t* __restrict__ h,
            float* __restrict__ parts) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t* sW = lds;                  // [2][BN][BK]
    uint16_t* sX = lds + 2 * BN * BK;    // [2][BM][BK]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fh = wave & 1, th = wave >> 1;
    const int n0 = blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;

    // global -> LDS copy assignment: chunk (row = lrow + 32 i, 16-byte column lc)
    const int lrow = tid >> 3, lc = tid & 7;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 gw[8], gx[8];

    auto gload = [&](int kt) {
        const int k0 = kt * BK + lc * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = lrow + 32 * i;
            gw[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)(n0 + row) * kD + k0);
            const int64_t tok = m0 + row;
            gx[i] = tok < M ? *reinterpret_cast<const u32x4*>(x + tok * kD + k0) : zero;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = lrow + 32 * i;
            const int off = row * BK + ((lc ^ (row & 7)) * 8);
            *reinterpret_cast<u32x4*>(sW + buf * BN * BK + off) = gw[i];
            *reinterpret_cast<u32x4*>(sX + buf * BM * BK + off) = gx[i];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload(0);
    lstore(0);
    __syncthreads();

    const int fr = lane & 31, kh = lane >> 5, sw = fr & 7;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint16_t* cW = sW + cur * BN * BK;
        const uint16_t* cX = sX + cur * BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ((ks * 2 + kh) ^ sw) * 8;
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(cW + (fh * 128 + i * 32 + fr) * BK + c);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(cX + (th * 128 + j * 32 + fr) * BK + c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds token (.. + fr) and features (.. + 8 g + 4 kh + 0..3)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t tok = m0 + th * 128 + j * 32 + fr;
        const bool live = tok < M;
        float ee = 0.0f, he = 0.0f, hh = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int f = n0 + fh * 128 + i * 32 + g * 8 + kh * 4;
                const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                if (!live) continue;
                const int64_t off = tok * kD + f;
                if (!kFwd || e32) {
                    f32x4 o = {v0, v1, v2, v3};
                    *reinterpret_cast<f32x4*>(e32 + off) = o;
                }
                if (kFwd) {
                    u32x2 hb = *reinterpret_cast<const u32x2*>(h + off);
                    const float h0 = bf16_to_f32(hb[0] & 0xFFFFu), h1 = bf16_to_f32(hb[0] >> 16);
                    const float h2 = bf16_to_f32(hb[1] & 0xFFFFu), h3 = bf16_to_f32(hb[1] >> 16);
                    ee += v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
                    he += h0 * v0 + h1 * v1 + h2 * v2 + h3 * v3;
                    hh += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
                    u32x2 ob = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                    *reinterpret_cast<u32x2*>(e16 + off) = ob;
                }
            }
        }
        if (kFwd) {
            ee += __shfl_xor(ee, 32);
            he += __shfl_xor(he, 32);
            hh += __shfl_xor(hh, 32);
            if (live && kh == 0) {
                const int part = (n0 + fh * 128) / kPartCols;
                f32x4 p = {ee, he, hh, 0.0f};
                *reinterpret_cast<f32x4*>(parts + (tok * kParts + part) * kPartStride) = p;
            }
        }
        // keep each token tile's loads and stores together (bounds register pressure)
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool kFwd>
hipError_t launch(const uint16_t* x, int64_t T, const uint16_t* W, float* e32, uint16_t* e16,
                  const uint16_t* h, float* parts, hipStream_t stream) {
    // the 128 KB of dynamic LDS must be allowed once per device
    static std::atomic<uint64_t> allowed{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(allowed.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&proj_kernel<kFwd>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (err != hipSuccess) return err;
        allowed.fetch_or(bit, std::memory_order_acq_rel);
    }
    dim3 grid(kD / BN, (unsigned)((T + BM - 1) / BM));
    hipLaunchKernelGGL(proj_kernel<kFwd>, grid, dim3(kThreads), kLdsBytes, stream, x, T, W, e32,
                       e16, h, parts);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj(const uint16_t* x, int64_t T, const uint16_t* W, float* e32,
                       uint16_t* e16, const uint16_t* h, float* parts, hipStream_t stream) {
    if (h) return launch<true>(x, T, W, e32, e16, h, parts, stream);
    return launch<false>(x, T, W, e32, nullptr, nullptr, nullptr, stream);
}

}  // namespace ple
