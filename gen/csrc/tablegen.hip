// GPU side of the FP8 table generator (input data, not part of the PLE method).
//
// Fills a [R][2560] E4M3FN code table and its [R] fp32 scales in HBM with the
// same bytes the CPU generator (tablegen_host.c) rebuilds on demand:
// Philox4x64-10 (Salmon et al., SC 2011) with key = (seed, 0);
//   codes: counter (g / 8, 0, 0, 0), g = r * 2560 + c, eight 32-bit words per
//          call (low half of each 64-bit output first); bit 31 = sign,
//          magnitude code = number of thresholds <= (word & 0x7fffffff);
//   scale: counter (r, 1, 0, 0), m = lo + hi32(out[0]) % span, scale = m * 2^-23.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kRow = 2560;

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        if (i > 0) {
            k0 += 0x9E3779B97F4A7C15ULL;
            k1 += 0xBB67AE8584CAA73BULL;
        }
        const uint64_t m0 = 0xD2E7470EE14C6C93ULL, m1 = 0xCA5A826395121157ULL;
        uint64_t lo0 = m0 * c[0], hi0 = __umul64hi(m0, c[0]);
        uint64_t lo1 = m1 * c[2], hi1 = __umul64hi(m1, c[2]);
        uint64_t n0 = hi1 ^ c[1] ^ k0;
        uint64_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    }
}

__device__ __forceinline__ uint32_t code_of(uint32_t w, const uint32_t* thr) {
    uint32_t u = w & 0x7FFFFFFFu;
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (thr[mid] <= u) lo = mid + 1; else hi = mid;
    }
    return ((w >> 31) << 7) | (uint32_t)lo;
}

__global__ void __launch_bounds__(256) fill_codes(uint8_t* __restrict__ table, uint64_t n_calls,
                                                  uint64_t seed, const uint32_t* __restrict__ thr_g) {
    __shared__ uint32_t thr[128];
    if (threadIdx.x < 126) thr[threadIdx.x] = thr_g[threadIdx.x];
    __syncthreads();
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; n < n_calls; n += stride) {
        uint64_t c[4] = {n, 0, 0, 0};
        philox4x64_10(c, seed, 0);
        uint64_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint64_t word = c[j / 2];
            uint32_t w = (j & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
            packed |= (uint64_t)code_of(w, thr) << (8 * j);
        }
        reinterpret_cast<uint64_t*>(table)[n] = packed;
    }
}

__global__ void __launch_bounds__(256) fill_scales(float* __restrict__ scales, uint64_t R, uint64_t seed,
                                                   uint32_t lo, uint32_t span) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R; r += stride) {
        uint64_t c[4] = {r, 1, 0, 0};
        philox4x64_10(c, seed, 0);
        uint32_t m = lo + (uint32_t)(c[0] >> 32) % span;
        scales[r] = (float)m * (1.0f / 8388608.0f);
    }
}

}  // namespace

extern "C" int gen_fill_table(uint8_t* table, float* scales, int64_t R, uint64_t seed,
                              const uint32_t* thr_dev, uint32_t scale_lo, uint32_t scale_span,
                              void* stream) {
    if (!table || !scales || !thr_dev || R <= 0) return -1;
    if (reinterpret_cast<uintptr_t>(table) % 8) return -2;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint64_t n_calls = (uint64_t)R * kRow / 8;
    uint64_t want = (n_calls + 255) / 256;
    unsigned grid = (unsigned)(want < 65536 * 8 ? want : 65536 * 8);
    hipLaunchKernelGGL(fill_codes, dim3(grid), dim3(256), 0, s, table, n_calls, seed, thr_dev);
    uint64_t want_s = ((uint64_t)R + 255) / 256;
    unsigned grid_s = (unsigned)(want_s < 65536 ? want_s : 65536);
    hipLaunchKernelGGL(fill_scales, dim3(grid_s), dim3(256), 0, s, scales, (uint64_t)R, seed,
                       scale_lo, scale_span);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// scales number 0 .. n-1 (e.g. the 16 R scales of the 16 x 160-byte head view)
extern "C" int gen_fill_scales(float* scales, int64_t n, uint64_t seed, uint32_t scale_lo,
                               uint32_t scale_span, void* stream) {
    if (!scales || n <= 0) return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint64_t want_s = ((uint64_t)n + 255) / 256;
    unsigned grid_s = (unsigned)(want_s < 65536 ? want_s : 65536);
    hipLaunchKernelGGL(fill_scales, dim3(grid_s), dim3(256), 0, s, scales, (uint64_t)n, seed, scale_lo,
                       scale_span);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// NVFP4 table (see tablegen_host.c): codes [R][1280], block scales [R][160]
__global__ void __launch_bounds__(256) fill_nvfp4_codes(uint8_t* __restrict__ codes, uint64_t n_calls,
                                                        uint64_t seed, const uint32_t* __restrict__ thr7) {
    uint32_t thr[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) thr[k] = thr7[k];
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t n = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; n < n_calls; n += stride) {
        uint64_t c[4] = {n, 0, 0, 0};
        philox4x64_10(c, seed, 1);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint64_t word = c[j / 2];
            uint32_t w = (j & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
            uint32_t u = w & 0x7FFFFFFFu, m = 0;
#pragma unroll
            for (int k = 0; k < 7; ++k) m += thr[k] <= u ? 1u : 0u;
            packed |= (((w >> 31) << 3) | m) << (4 * j);
        }
        reinterpret_cast<uint32_t*>(codes)[n] = packed;
    }
}

__global__ void __launch_bounds__(256) fill_nvfp4_blocks(uint8_t* __restrict__ blocks, uint64_t n_blocks,
                                                         uint64_t seed, uint32_t lo, uint32_t span) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n_blocks; q += stride) {
        uint64_t c[4] = {q, 2, 0, 0};
        philox4x64_10(c, seed, 1);
        blocks[q] = (uint8_t)(lo + (uint32_t)(c[0] >> 32) % span);
    }
}

extern "C" int gen_fill_nvfp4(uint8_t* codes, uint8_t* blocks, int64_t R, uint64_t seed, const uint32_t* thr7_dev,
                              uint32_t block_lo, uint32_t block_span, void* stream) {
    if (!codes || !blocks || !thr7_dev || R <= 0) return -1;
    if (reinterpret_cast<uintptr_t>(codes) % 4) return -2;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint64_t n_calls = (uint64_t)R * kRow / 8;
    uint64_t want = (n_calls + 255) / 256;
    unsigned grid = (unsigned)(want < 65536 * 8 ? want : 65536 * 8);
    hipLaunchKernelGGL(fill_nvfp4_codes, dim3(grid), dim3(256), 0, s, codes, n_calls, seed, thr7_dev);
    uint64_t n_blocks = (uint64_t)R * (kRow / 16);
    uint64_t want_b = (n_blocks + 255) / 256;
    unsigned grid_b = (unsigned)(want_b < 65536 * 8 ? want_b : 65536 * 8);
    hipLaunchKernelGGL(fill_nvfp4_blocks, dim3(grid_b), dim3(256), 0, s, blocks, n_blocks, seed, block_lo,
                       block_span);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
