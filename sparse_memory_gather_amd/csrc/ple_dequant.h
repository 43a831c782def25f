// FP8 E4M3FN dequantization of the two rows of a token (bigram, trigram),
// shared by the gather kernel and the one-launch decode step so that both
// produce the same x bits:
//   x = bf16_rne(fl32(fl32(dec(c2) s2) + fl32(dec(c3) s3)))
// dec = the hardware E4M3FN -> fp32 conversion (OCP on gfx950), one fp32
// scale per row multiplied in, no FMA contraction, one rounding to bf16; a
// missing row (-1) contributes nothing, not even a signed zero.
#pragma once

#include "ple_kernels.h"

namespace ple {

// 8 FP8 codes of one row times its scale
__device__ __forceinline__ void decode8(const u32x2& q, float s, float out[8]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], false);
        f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], true);
        out[4 * w + 0] = lo[0] * s;
        out[4 * w + 1] = lo[1] * s;
        out[4 * w + 2] = hi[0] * s;
        out[4 * w + 3] = hi[1] * s;
    }
}

// 8 consecutive elements of x from the same 8 bytes of both rows: codes a
// (scale sa, row present va) and b (sb, vb); returned as 8 packed bf16
__device__ __forceinline__ u32x4 dequant_pair8(const u32x2& a, float sa, bool va, const u32x2& b, float sb,
                                               bool vb) {
#pragma clang fp contract(off)
    float pa[8], pb[8], acc[8];
    decode8(a, sa, pa);
    decode8(b, sb, pb);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = va ? (vb ? pa[i] + pb[i] : pa[i]) : (vb ? pb[i] : 0.0f);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    return o;
}

}  // namespace ple
