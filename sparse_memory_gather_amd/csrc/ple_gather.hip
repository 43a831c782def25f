// a2: gather the bigram and trigram rows of each token and dequantize.
//
// The table is FP8 (bittide copy of the SSD-Stream model card, "模型简介");
// rows are read by ID and dequantized before the projection (mengman.github.io
// "Qwen3.8-Flash-Next 端侧部署 01", n-gram embedding section). Here the whole
// table sits in HBM; each 64-lane wave owns one token:
//   - both row IDs and scales are wave-uniform (scalar registers);
//   - a 2560-byte row is 160 chunks of 16 bytes; lane l takes chunks l, l+64
//     and (l < 32) l+128 of both rows, all six loads issued before any use;
//   - E4M3FN -> fp32 with the hardware conversion, times the row scale, the
//     two products added in fp32 (no FMA contraction), rounded once to bf16;
//   - each 16-byte input chunk becomes 32 contiguous output bytes.
#include "ple_kernels.h"

namespace ple {
namespace {

constexpr int kTokPerBlock = 4;  // one wave per token
constexpr int kChunks = kD / 16;  // 160

__device__ __forceinline__ void decode16(const u32x4& q, float s, float out[16]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], false);
        f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], true);
        out[4 * w + 0] = lo[0] * s;
        out[4 * w + 1] = lo[1] * s;
        out[4 * w + 2] = hi[0] * s;
        out[4 * w + 3] = hi[1] * s;
    }
}

__device__ __forceinline__ void emit(uint16_t* __restrict__ xrow, int chunk, const u32x4& qa, float sa,
                                     bool va, const u32x4& qb, float sb, bool vb) {
#pragma clang fp contract(off)
    float pa[16], pb[16], acc[16];
    decode16(qa, sa, pa);
    decode16(qb, sb, pb);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = va ? (vb ? pa[i] + pb[i] : pa[i]) : (vb ? pb[i] : 0.0f);
    u32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o0[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        o1[i] = pack_bf16x2(acc[8 + 2 * i], acc[8 + 2 * i + 1]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(xrow) + 2 * chunk;
    dst[0] = o0;
    dst[1] = o1;
}

__global__ void __launch_bounds__(64 * kTokPerBlock)
gather_kernel(const int32_t* __restrict__ row_ids, int64_t T, const uint8_t* __restrict__ table,
              const float* __restrict__ scales, int64_t R, uint16_t* __restrict__ x,
              uint8_t* __restrict__ raw, int32_t* dev_err) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int2 ids = reinterpret_cast<const int2*>(row_ids)[t];
    int r0 = __builtin_amdgcn_readfirstlane(ids.x);
    int r1 = __builtin_amdgcn_readfirstlane(ids.y);
    if (r0 < -1 || (int64_t)r0 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r0 = -1;
    }
    if (r1 < -1 || (int64_t)r1 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r1 = -1;
    }
    const bool v0 = r0 >= 0, v1 = r1 >= 0;
    const u32x4* row0 = reinterpret_cast<const u32x4*>(table + (int64_t)(v0 ? r0 : 0) * kD);
    const u32x4* row1 = reinterpret_cast<const u32x4*>(table + (int64_t)(v1 ? r1 : 0) * kD);
    const bool third = lane < kChunks - 128;
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 a0 = z, a1 = z, a2 = z, b0 = z, b1 = z, b2 = z;
    if (v0) {
        a0 = row0[lane];
        a1 = row0[lane + 64];
        if (third) a2 = row0[lane + 128];
    }
    if (v1) {
        b0 = row1[lane];
        b1 = row1[lane + 64];
        if (third) b2 = row1[lane + 128];
    }
    const float s0 = v0 ? scales[r0] : 0.0f;
    const float s1 = v1 ? scales[r1] : 0.0f;
    uint16_t* xrow = x + t * kD;
    emit(xrow, lane, a0, s0, v0, b0, s1, v1);
    emit(xrow, lane + 64, a1, s0, v0, b1, s1, v1);
    if (third) emit(xrow, lane + 128, a2, s0, v0, b2, s1, v1);
    if (raw) {
        u32x4* d0 = reinterpret_cast<u32x4*>(raw + (t * 2 + 0) * kD);
        u32x4* d1 = reinterpret_cast<u32x4*>(raw + (t * 2 + 1) * kD);
        d0[lane] = a0;
        d0[lane + 64] = a1;
        d1[lane] = b0;
        d1[lane + 64] = b1;
        if (third) {
            d0[lane + 128] = a2;
            d1[lane + 128] = b2;
        }
    }
}

}  // namespace

hipError_t launch_gather(const int32_t* row_ids, int64_t T, const uint8_t* table,
                         const float* scales, int64_t R, uint16_t* x, uint8_t* raw,
                         int32_t* dev_err, hipStream_t stream) {
    int64_t blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(64 * kTokPerBlock), 0, stream,
                       row_ids, T, table, scales, R, x, raw, dev_err);
    return hipGetLastError();
}

}  // namespace ple
