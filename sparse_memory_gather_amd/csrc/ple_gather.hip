// a2: gather the bigram and trigram rows of each token and dequantize.
//
// The table is FP8 (bittide copy of the SSD-Stream model card, "模型简介");
// rows are read by ID and dequantized before the projection (mengman.github.io
// "Qwen3.8-Flash-Next 端侧部署 01", n-gram embedding section). Here the whole
// table sits in HBM; each 64-lane wave owns one token:
//   - both row IDs and scales are wave-uniform (scalar registers);
//   - a 2560-byte row is five 512-byte spans; lane l reads bytes 8l .. 8l+7
//     of every span of both rows, all ten loads issued before any use;
//   - E4M3FN -> fp32 with the hardware conversion, times the row scale, the
//     two products added in fp32 (no FMA contraction), rounded once to bf16;
//   - each span becomes 1 KB of output written by one store instruction
//     (16 contiguous bytes per lane); 32 bytes per lane per 16-byte load
//     (each store instruction covering every other 16-byte slot) took 29%
//     longer. The stores are plain, not non-temporal: x then stays in the
//     memory-side cache, and its write-back to HBM overlaps the
//     compute-bound projection that reads it next (a 32K-token call: 54-55
//     us against 60-61 us with non-temporal stores, the projection no
//     slower). A gather run back to back with itself, as in an isolated
//     timing loop, is the opposite case: each run then pays for the
//     previous run's write-back, and non-temporal stores are faster.
#include "ple_dequant.h"
#include "ple_ngram.h"

namespace ple {
namespace {

constexpr int kTokPerBlock = 4;  // one wave per token
constexpr int kSpans = kD / 512;  // 5

// kIds (all three gathers): each wave computes its token's row IDs itself
// (short calls: one launch instead of the ID kernel and the gather). The
// launch then also checks cu_seqlens (block 0) and copies the carried conv
// state (grid row 1), as the ID kernel would. False for the copy blocks.
template <bool kIds>
__device__ __forceinline__ bool ids_prologue(const IdSource& src, int64_t T, int32_t* dev_err) {
    if (!kIds) return true;
    if (blockIdx.y == 1) {
        copy_state(src.conv_state, src.snap, src.cu, src.S, src.snap_pb, blockIdx.x, gridDim.x);
        return false;
    }
    if (blockIdx.x == 0) check_cu(src.cu, src.S, T, dev_err);
    return true;
}

// the token's two rows (wave-uniform): computed (kIds) or read from row_ids
template <bool kIds>
__device__ __forceinline__ void pair_rows(int64_t t, const int32_t* row_ids, const IdSource& src,
                                          int32_t* dev_err, int lane, int& r0, int& r1) {
    if (kIds) {
        const NgramKeys k = ngram_keys(t, src.tokens, src.cu, src.S, src.hist_ids, src.hist_len, src.vocab,
                                       dev_err);
        const ModR mr{src.mod_R, src.mod_m};
        r0 = __builtin_amdgcn_readfirstlane(bigram_row(k, mr));
        r1 = __builtin_amdgcn_readfirstlane(trigram_row(k, mr));
        if (src.row_ids_out && lane == 0) reinterpret_cast<int2*>(src.row_ids_out)[t] = make_int2(r0, r1);
    } else {
        const int2 ids = reinterpret_cast<const int2*>(row_ids)[t];
        r0 = __builtin_amdgcn_readfirstlane(ids.x);
        r1 = __builtin_amdgcn_readfirstlane(ids.y);
    }
}

template <bool kIds>
__global__ void __launch_bounds__(64 * kTokPerBlock)
gather_kernel(const int32_t* __restrict__ row_ids, int64_t T, const uint8_t* __restrict__ table,
              const float* __restrict__ scales, int64_t R, uint16_t* __restrict__ x,
              uint8_t* __restrict__ raw, int32_t* dev_err, IdSource src) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    if (!ids_prologue<kIds>(src, T, dev_err)) return;
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int r0, r1;
    pair_rows<kIds>(t, row_ids, src, dev_err, lane, r0, r1);
    if (r0 < -1 || (int64_t)r0 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r0 = -1;
    }
    if (r1 < -1 || (int64_t)r1 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r1 = -1;
    }
    const bool v0 = r0 >= 0, v1 = r1 >= 0;
    const u32x2* row0 = reinterpret_cast<const u32x2*>(table + (int64_t)(v0 ? r0 : 0) * kD) + lane;
    const u32x2* row1 = reinterpret_cast<const u32x2*>(table + (int64_t)(v1 ? r1 : 0) * kD) + lane;
    const u32x2 z = {0u, 0u};
    u32x2 a[kSpans], b[kSpans];
#pragma unroll
    for (int s = 0; s < kSpans; ++s) {
        a[s] = v0 ? row0[s * 64] : z;
        b[s] = v1 ? row1[s * 64] : z;
    }
    const float s0 = v0 ? scales[r0] : 0.0f;
    const float s1 = v1 ? scales[r1] : 0.0f;
    u32x4* xrow = reinterpret_cast<u32x4*>(x + t * kD) + lane;
#pragma unroll
    for (int s = 0; s < kSpans; ++s) *(xrow + s * 64) = dequant_pair8(a[s], s0, v0, b[s], s1, v1);
    if (raw) {
        u32x2* d0 = reinterpret_cast<u32x2*>(raw + (t * 2 + 0) * kD) + lane;
        u32x2* d1 = reinterpret_cast<u32x2*>(raw + (t * 2 + 1) * kD) + lane;
#pragma unroll
        for (int s = 0; s < kSpans; ++s) {
            d0[s * 64] = a[s];
            d1[s * 64] = b[s];
        }
    }
}

// 16-lookup layout: the table as 16 head tables of R rows x 160 bytes and
// one scale per (head, row). Head h's row fills x columns 160h .. 160h+159;
// a missing n-gram leaves its heads' columns +0. One wave per token (two
// tokens per wave, all loads issued first, measured slower), the same five
// 512-element spans as above: lane l of span s covers elements 512s + 8l .. +7, which
// lie in one head (160 is a multiple of 8); lanes 0..15 load a token's 16 row
// IDs and scales and the others take theirs with a lane shuffle.
constexpr int kHeadTokPerWave = 1;

template <bool kIds>
__global__ void __launch_bounds__(64 * kTokPerBlock)
gather_heads_kernel(const int32_t* __restrict__ row_ids, int64_t T, const uint8_t* __restrict__ table,
                    const float* __restrict__ scales, int64_t R, uint16_t* __restrict__ x,
                    uint8_t* __restrict__ raw, int32_t* dev_err, IdSource src) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    if (!ids_prologue<kIds>(src, T, dev_err)) return;
    const int64_t t0 = ((int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6)) * kHeadTokPerWave;
    if (t0 >= T) return;
    u32x2 a[kHeadTokPerWave][kSpans];
    float sc[kHeadTokPerWave][kSpans];
    bool ok[kHeadTokPerWave][kSpans];
    int head[kSpans], off[kSpans];
#pragma unroll
    for (int s = 0; s < kSpans; ++s) {
        const int e0 = 512 * s + 8 * lane;
        head[s] = e0 / 160;
        off[s] = e0 - 160 * head[s];
    }
#pragma unroll
    for (int k = 0; k < kHeadTokPerWave; ++k) {
        const int64_t t = t0 + k;
        int my_id = -1;
        float my_scale = 0.0f;
        if (kIds && t < T) {
            // lane h < 16 computes head h's row (the keys are wave-uniform)
            const NgramKeys kk = ngram_keys(t, src.tokens, src.cu, src.S, src.hist_ids, src.hist_len, src.vocab,
                                            dev_err);
            if (lane < 16) {
                my_id = head_row(kk, lane, ModR{src.mod_R, src.mod_m});
                if (src.row_ids_out) src.row_ids_out[t * 16 + lane] = my_id;
                if (my_id >= 0) my_scale = scales[(int64_t)lane * R + my_id];
            }
        } else if (lane < 16 && t < T) {
            int r = row_ids[t * 16 + lane];
            if (r < -1 || (int64_t)r >= R) {
                flag_error(dev_err, 8);
                r = -1;
            }
            my_id = r;
            if (r >= 0) my_scale = scales[(int64_t)lane * R + r];
        }
#pragma unroll
        for (int s = 0; s < kSpans; ++s) {
            const int r = __shfl(my_id, head[s]);
            sc[k][s] = __shfl(my_scale, head[s]);
            ok[k][s] = r >= 0;
            const u32x2 z = {0u, 0u};
            a[k][s] = ok[k][s] ? *reinterpret_cast<const u32x2*>(table + ((int64_t)head[s] * R + r) * 160 + off[s])
                               : z;
        }
    }
#pragma unroll
    for (int k = 0; k < kHeadTokPerWave; ++k) {
        const int64_t t = t0 + k;
        if (t >= T) break;
        u32x4* xrow = reinterpret_cast<u32x4*>(x + t * kD) + lane;
#pragma unroll
        for (int s = 0; s < kSpans; ++s) {
            float p[8];
            decode8(a[k][s], sc[k][s], p);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = ok[k][s] ? pack_bf16x2(p[2 * i], p[2 * i + 1]) : 0u;
            *(xrow + s * 64) = o;
        }
        if (raw) {
#pragma unroll
            for (int s = 0; s < kSpans; ++s)
                *reinterpret_cast<u32x2*>(raw + (t * 16 + head[s]) * 160 + off[s]) = a[k][s];
        }
    }
}

// NVFP4 table (the Spark deployment's packed PLE table: 4-bit codes with an
// FP8 scale per group of 16): row r = 1280 bytes of OCP E2M1 codes (element
// 2k in the low nibble of byte k), 160 E4M3 block scales (block b covers
// elements 16b .. 16b+15) and the fp32 row scale;
//   p = fl32(fl32(e2m1 * e4m3) * scale)   (the inner product exact),
// the two rows combined as in the FP8 table. Same wave-per-token plan: lane
// l of span s covers elements 512s + 8l .. +7, i.e. code word 64s + l and
// block 32s + l/2 of each row. E2M1 pairs are decoded by
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 (exact; low nibble first).
__device__ __forceinline__ void decode_nvfp4(uint32_t w, float block, float s, float out[8]) {
#pragma clang fp contract(off)
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const float e[8] = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = e[i] * block;
        out[i] = q * s;
    }
}

template <bool kIds>
__global__ void __launch_bounds__(64 * kTokPerBlock)
gather_nvfp4_kernel(const int32_t* __restrict__ row_ids, int64_t T, const uint8_t* __restrict__ codes,
                    const uint8_t* __restrict__ blocks, const float* __restrict__ scales, int64_t R,
                    uint16_t* __restrict__ x, uint8_t* __restrict__ raw, int32_t* dev_err, IdSource src) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    if (!ids_prologue<kIds>(src, T, dev_err)) return;
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int r0, r1;
    pair_rows<kIds>(t, row_ids, src, dev_err, lane, r0, r1);
    if (r0 < -1 || (int64_t)r0 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r0 = -1;
    }
    if (r1 < -1 || (int64_t)r1 >= R) {
        if (lane == 0) flag_error(dev_err, 8);
        r1 = -1;
    }
    const bool v0 = r0 >= 0, v1 = r1 >= 0;
    const uint32_t* c0 = reinterpret_cast<const uint32_t*>(codes + (int64_t)(v0 ? r0 : 0) * (kD / 2)) + lane;
    const uint32_t* c1 = reinterpret_cast<const uint32_t*>(codes + (int64_t)(v1 ? r1 : 0) * (kD / 2)) + lane;
    const uint8_t* b0 = blocks + (int64_t)(v0 ? r0 : 0) * (kD / 16) + lane / 2;
    const uint8_t* b1 = blocks + (int64_t)(v1 ? r1 : 0) * (kD / 16) + lane / 2;
    uint32_t a[kSpans], b[kSpans], ba[kSpans], bb[kSpans];
#pragma unroll
    for (int s = 0; s < kSpans; ++s) {
        a[s] = v0 ? c0[s * 64] : 0u;
        b[s] = v1 ? c1[s * 64] : 0u;
        ba[s] = v0 ? b0[s * 32] : 0u;
        bb[s] = v1 ? b1[s * 32] : 0u;
    }
    const float s0 = v0 ? scales[r0] : 0.0f;
    const float s1 = v1 ? scales[r1] : 0.0f;
    u32x4* xrow = reinterpret_cast<u32x4*>(x + t * kD) + lane;
#pragma unroll
    for (int s = 0; s < kSpans; ++s) {
        const float blk0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ba[s], false)[0];
        const float blk1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bb[s], false)[0];
        float pa[8], pb[8], acc[8];
        decode_nvfp4(a[s], blk0, s0, pa);
        decode_nvfp4(b[s], blk1, s1, pb);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = v0 ? (v1 ? pa[i] + pb[i] : pa[i]) : (v1 ? pb[i] : 0.0f);
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
        *(xrow + s * 64) = o;
    }
    if (raw) {
        uint32_t* d0 = reinterpret_cast<uint32_t*>(raw + (t * 2 + 0) * (kD / 2)) + lane;
        uint32_t* d1 = reinterpret_cast<uint32_t*>(raw + (t * 2 + 1) * (kD / 2)) + lane;
#pragma unroll
        for (int s = 0; s < kSpans; ++s) {
            d0[s * 64] = a[s];
            d1[s * 64] = b[s];
        }
    }
}

}  // namespace

hipError_t launch_gather_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes, const uint8_t* blocks,
                               const float* scales, int64_t R, uint16_t* x, uint8_t* raw, int32_t* dev_err,
                               hipStream_t stream) {
    int64_t blocks_n = (T + kTokPerBlock - 1) / kTokPerBlock;
    hipLaunchKernelGGL(gather_nvfp4_kernel<false>, dim3((unsigned)blocks_n), dim3(64 * kTokPerBlock), 0, stream,
                       row_ids, T, codes, blocks, scales, R, x, raw, dev_err, IdSource{});
    return hipGetLastError();
}

hipError_t launch_gather_heads(const int32_t* row_ids, int64_t T, const uint8_t* table,
                               const float* scales, int64_t R, uint16_t* x, uint8_t* raw,
                               int32_t* dev_err, hipStream_t stream) {
    const int64_t per_block = (int64_t)kTokPerBlock * kHeadTokPerWave;
    int64_t blocks = (T + per_block - 1) / per_block;
    hipLaunchKernelGGL(gather_heads_kernel<false>, dim3((unsigned)blocks), dim3(64 * kTokPerBlock), 0, stream,
                       row_ids, T, table, scales, R, x, raw, dev_err, IdSource{});
    return hipGetLastError();
}

hipError_t launch_gather(const int32_t* row_ids, int64_t T, const uint8_t* table,
                         const float* scales, int64_t R, uint16_t* x, uint8_t* raw,
                         int32_t* dev_err, hipStream_t stream) {
    int64_t blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
    hipLaunchKernelGGL(gather_kernel<false>, dim3((unsigned)blocks), dim3(64 * kTokPerBlock), 0, stream,
                       row_ids, T, table, scales, R, x, raw, dev_err, IdSource{});
    return hipGetLastError();
}

hipError_t launch_gather_ids(const IdSource& src, int layout, int64_t T, const uint8_t* table,
                             const uint8_t* nv_blocks, const float* scales, int64_t R, uint16_t* x,
                             int32_t* dev_err, hipStream_t stream) {
    int64_t blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
    // grid row 1 copies the state, one sequence per block and round
    const int64_t snap_blocks = src.snap ? src.S : 0;
    if (snap_blocks > blocks) blocks = snap_blocks < 65536 ? snap_blocks : 65536;
    if (blocks < 1) blocks = 1;
    IdSource s = src;
    const ModR mr = make_mod((uint64_t)R);
    s.mod_R = mr.R;
    s.mod_m = mr.m;
    const dim3 grid((unsigned)blocks, src.snap ? 2 : 1), block(64 * kTokPerBlock);
    if (layout == kLayoutHeads)
        hipLaunchKernelGGL(gather_heads_kernel<true>, grid, block, 0, stream, nullptr, T, table, scales, R, x,
                           nullptr, dev_err, s);
    else if (layout == kLayoutNvfp4)
        hipLaunchKernelGGL(gather_nvfp4_kernel<true>, grid, block, 0, stream, nullptr, T, table, nv_blocks, scales,
                           R, x, nullptr, dev_err, s);
    else
        hipLaunchKernelGGL(gather_kernel<true>, grid, block, 0, stream, nullptr, T, table, scales, R, x, nullptr,
                           dev_err, s);
    return hipGetLastError();
}

}  // namespace ple
