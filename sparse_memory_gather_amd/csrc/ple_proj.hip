// a3: projection e = x W^T (bf16 in, fp32 accumulate) on gfx950 MFMA.
//
// The looked-up vector is projected before the gate and the short conv
// (mengman.github.io "Qwen3.8-Flash-Next 端侧部署 01", n-gram embedding
// section). It is the only dense contraction on the path: [T x 2560] times
// [2560 x 2560]^T, both operands K-contiguous.
//
// Block tile 256 features x 256 tokens x 64 k, eight waves (two per SIMD, so
// one wave's LDS waits overlap the other's MFMAs), each wave a 128-feature x
// 64-token sub-tile of 4x2 v_mfma_f32_32x32x16_bf16 tiles. W rows feed the
// MFMA A operand and tokens the B operand, so a lane's accumulators hold one
// token and runs of four consecutive features (8-byte bf16 stores).
//
// Operands move global -> LDS with global_load_lds_dwordx4 (no register
// staging) into two 64 KB stages; each wave-level load fills 1 KB of LDS
// (eight 128-byte rows). The 16-byte chunks of a row are XOR-swizzled by
// (row >> 1) & 7: gfx950's LDS serves a ds_read_b128 sixteen lanes at a time
// across 256 bytes, and 16 consecutive 128-byte rows then hit 16 distinct
// 16-byte bank groups.
//
// The k loop is software-pipelined: the fragment reads of k-step ks+1 are
// interleaved with the MFMAs of ks (pinned with sched_group_barrier), and
// the wait for the next stage, the barrier and the DMA into the stage just
// read sit inside the last k-step of each stage, so the first fragments of
// the next stage load while its MFMAs drain.
//
// Forward mode writes e as bf16 (the projection's output tensor), staged
// through LDS into 256-byte token rows; the fp32 accumulators can also be
// written for checking.
//
// Four tilings by call size, all with the same MFMA sequence over k for
// every output element, so a token's e does not depend on the call it is
// in: a small-T kernel (up to 256 tokens), 128 x 256 tiles (up to 3200),
// and for larger calls the 256 x 256 tiles above or 256 x 320 tiles,
// whichever needs fewer rounds of blocks on the 256 CUs.
#include <atomic>

#include "ple_fragments.h"
#include "ple_kernels.h"

namespace ple {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int BM = 256;  // tokens per block
constexpr int BN = 256;  // features per block
constexpr int BK = 64;   // k per stage
constexpr int KT = kD / BK;
constexpr int CH = BK / 8;               // 16-byte chunks per row of a stage
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int RPL = 64 / CH;             // rows filled by one wave-level load
constexpr int LPW = BM / (kWaves * RPL); // loads per wave per operand per stage
constexpr int STAGE = (BM + BN) * BK;    // bf16 elements per stage
constexpr int kNTiles = kD / BN;         // feature tiles per token tile
constexpr int kXcds = 8;                 // accelerator complex dies on MI355X
constexpr int kLdsBytes = 2 * STAGE * 2; // 131072
constexpr int kSmallT = 256;            // token counts served by proj_small_kernel

__device__ __forceinline__ int swz(int row) { return (row >> 1) & (CH - 1); }

// Output of one lane for one 32-token tile of a 128-feature slice: vals[i] are
// the lane's 16 accumulators of feature tile i (features fbase + 32 i + 8 g +
// 4 kh + 0..3, g = r / 4) for token `tok`. Writes e as fp32 (if e32) and, in
// forward mode, as bf16: to global memory, or with kStage to the wave's LDS
// staging tile, row `srow` (the token within the wave's 64), 16-byte chunk
// (feature offset / 8) XOR (srow & 15), so that the 32 rows a store
// instruction touches spread over all 64 banks.
template <bool kFwd, bool kStage>
__device__ __forceinline__ void emit_slice(const float (&vals)[4][16], int64_t tok, int64_t M, int fbase,
                                           int kh, float* __restrict__ e32, uint16_t* __restrict__ e16,
                                           uint16_t* stage = nullptr, int srow = 0) {
    if (tok >= M) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int f = fbase + i * 32 + g * 8 + kh * 4;
            const float v0 = vals[i][4 * g + 0], v1 = vals[i][4 * g + 1];
            const float v2 = vals[i][4 * g + 2], v3 = vals[i][4 * g + 3];
            const int64_t off = tok * kD + f;
            if (!kFwd || e32) *reinterpret_cast<f32x4*>(e32 + off) = f32x4{v0, v1, v2, v3};
            if (kFwd) {
                const u32x2 ob = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                if (kStage)
                    *reinterpret_cast<u32x2*>(stage + srow * 128 + ((4 * i + g) ^ (srow & 15)) * 8 + kh * 4) = ob;
                else
                    *reinterpret_cast<u32x2*>(e16 + off) = ob;
            }
        }
    }
}

template <bool kFwd>
__global__ void __launch_bounds__(kThreads, 1)
proj_kernel(const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ W,
            float* __restrict__ e32, uint16_t* __restrict__ e16) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fh = wave & 1, tq = wave >> 1;  // 128-feature half, 64-token quarter
    // Workgroups are handed to the 8 XCDs round-robin (block b -> XCD b % 8).
    // Give each XCD a contiguous run of tiles, feature tiles fastest, so the
    // blocks resident on one XCD share their x panels in that XCD's L2.
    const int nb = gridDim.x, b = blockIdx.x;
    const int per = nb / kXcds, rem = nb % kXcds, xcd = b % kXcds;
    const int tile = xcd * per + (xcd < rem ? xcd : rem) + b / kXcds;
    const int n0 = (tile % kNTiles) * BN;
    const int64_t m0 = (int64_t)(tile / kNTiles) * BM;

    // DMA assignment: load i of this wave fills rows R = (wave*LPW + i)*RPL ..
    // +RPL of both operands; lane l writes row R + l/CH, physical chunk l%CH,
    // which holds logical chunk (l%CH) ^ swz(row).
    const uint16_t* gW[LPW];
    const uint16_t* gX[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = (wave * LPW + i) * RPL + lane / CH;
        const int c = (lane % CH) ^ swz(row);
        gW[i] = W + (int64_t)(n0 + row) * kD + c * 8;
        const int64_t tok = m0 + row;
        // rows past the last token read token 0 (in bounds); their results are never stored
        gX[i] = x + (tok < M ? tok : 0) * kD + c * 8;
    }
    auto issue = [&](int kt) {
        uint16_t* sbase = lds + (kt & 1) * STAGE;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            uint16_t* dW = sbase + (wave * LPW + i) * RPL * BK;
            __builtin_amdgcn_global_load_lds((gbl_void*)(gW[i] + k0), (lds_void*)dW, 16, 0, 0);
            uint16_t* dX = sbase + BN * BK + (wave * LPW + i) * RPL * BK;
            __builtin_amdgcn_global_load_lds((gbl_void*)(gX[i] + k0), (lds_void*)dX, 16, 0, 0);
        }
    };

    // fragments of one k-step: 4 W tiles (A operand) and 2 token tiles (B)
    const int fr = lane & 31, kh = lane >> 5, sw = swz(fr);
    const int offA = (fh * 128 + fr) * BK, offB = BN * BK + (tq * 64 + fr) * BK;
    bf16x8 fa[2][4], fb[2][2];
    auto read = [&](int kt, int ks, int buf) {
        const uint16_t* base = lds + (kt & 1) * STAGE;
        const int c = ((ks * 2 + kh) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8*>(base + offA + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8*>(base + offB + j * 32 * BK + c);
    };
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // MFMAs lo .. hi-1 of one k-step (q = 2 i + j), each tile's k order unchanged
    auto mfma = [&](int buf, int lo, int hi) {
#pragma unroll
        for (int q = lo; q < hi; ++q)
            acc[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][q >> 1], fb[buf][q & 1],
                                                                         acc[q >> 1][q & 1], 0, 0, 0);
    };

    issue(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt untouched
    __builtin_amdgcn_s_barrier();
    issue(1);
    read(0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ks = 0; ks < BK / 16 - 1; ++ks) {
            read(kt, ks + 1, (ks + 1) & 1);
            mfma(ks & 1, 0, 8);
            // one fragment read between consecutive MFMAs
#pragma unroll
            for (int q = 0; q < 6; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        // last k-step of stage kt (fragments in buffer 1): this wave's reads
        // of the stage are complete; once every wave has passed the barrier
        // the stage may be refilled, and stage kt+1 (DMA issued one stage
        // ago) has landed for every wave
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        mfma(1, 0, 4);
        if (kt + 1 < KT) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __builtin_amdgcn_s_barrier();
            if (kt + 2 < KT) issue(kt + 2);
            read(kt + 1, 0, 0);
        }
        mfma(1, 4, 8);
    }

    // epilogue: lane holds token (.. + fr) and features (.. + 8 g + 4 kh + 0..3).
    // In forward mode the bf16 e tile of each wave (64 tokens x 128 features,
    // 16 KB) is staged in LDS, which every wave must have finished reading.
    uint16_t* stage = lds + wave * (64 * 128);
    if (kFwd) __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float vals[4][16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) vals[i][r] = acc[i][j][r];
        emit_slice<kFwd, kFwd>(vals, m0 + tq * 64 + j * 32 + fr, M, n0 + fh * 128, kh, e32, e16, stage,
                               j * 32 + fr);
    }
    if (kFwd) {
        // the lanes read staging rows other lanes of the wave wrote: a
        // wave-scope fence orders those LDS writes before the reads. Each
        // store instruction writes four 256-byte token rows; plain stores
        // leave e in the memory-side cache for the fuse kernel, which reads
        // it next.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const int c = lane & 15;
#pragma unroll 4
        for (int q = 0; q < 16; ++q) {
            const int r = q * 4 + (lane >> 4);
            const int64_t tok = m0 + tq * 64 + r;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 128 + (c ^ (r & 15)) * 8);
            if (tok < M)
                *reinterpret_cast<u32x4*>(e16 + tok * kD + n0 + fh * 128 + c * 8) = v;
        }
    }
}

// Small-T projection (decode steps, short chunks): one block per kRows
// features and kTiles consecutive 32-token tiles, eight waves, wave w holding
// the fragments of k-steps 20w .. 20w+19, all loaded up front. A tile's
// accumulator passes from wave to wave through LDS, so it sees the same MFMA
// sequence over k as in proj_kernel and every output element is
// bit-identical to what proj_kernel produces. kRows < 32 leaves the MFMA's
// other A rows zero (an output element depends only on its own row and
// column), so that an 8-token step spreads its W loads over 160 CUs. With
// kTiles > 1 the tiles' chains are pipelined through the waves with the same
// W fragments: in step s wave w runs its segment of tile s - w, so the block
// takes kW + kTiles - 1 steps instead of kW x kTiles, each wave loading its x
// fragments of the next tile during its segment of the current one;
// calls of up to 256 tokens take one round of blocks (one block per CU fits
// at this register use). With 32 rows a block loads W and its first token
// tile in 64-byte runs (ple_fragments.h), a quarter of the address-unit time
// of loads in the MFMA layout, and wave w moves them into that layout during
// the step before its first segment (passing w barriers first, so only
// wave 0's exchange precedes the first segment).
template <bool kFwd, int kRows, int kTiles>
__global__ void __launch_bounds__(512)
proj_small_kernel(const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ W,
                  float* __restrict__ e32, uint16_t* __restrict__ e16) {
    static_assert(kRows == 16 || kRows == 32, "feature rows per block");
    constexpr int KS = kD / 16;        // 160 k-steps
    constexpr int kW = 8;              // waves
    constexpr int SPW = KS / kW;       // k-steps per wave
    __shared__ f32x16 acc_s[kTiles][64];  // each tile's accumulator between waves
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int fr = lane & 31, kh = lane >> 5;
    const int f0 = blockIdx.x * kRows;
    bf16x8 fa[SPW], fb[SPW];
    // a tile's segment on this wave: k-steps 20 wave .. 20 wave + 19 of tile
    // t, the accumulator from the wave before (or zero), to the wave after
    // (or e for the last wave)
    auto segment = [&](int t) {
        f32x16 acc;
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        } else {
            acc = acc_s[t][lane];
        }
        if (t + 1 < kTiles) {
            // the next tile's fragment q replaces this one's as soon as its
            // MFMA has issued, so those loads are in flight during the
            // segment. Tokens past the last read token 0 (in bounds): their
            // columns of the product are never stored, and loads under a
            // per-lane condition would make the compiler wait for the first
            // of them before issuing the rest
            const int64_t tok = ((int64_t)blockIdx.y * kTiles + t + 1) * 32 + fr;
            const uint16_t* xrow = x + (tok < M ? tok : 0) * kD + wave * SPW * 16 + kh * 8;
#pragma unroll
            for (int q = 0; q < SPW; ++q) {
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q], fb[q], acc, 0, 0, 0);
                fb[q] = *reinterpret_cast<const bf16x8*>(xrow + q * 16);
                // one MFMA, then one load (without this the compiler issues
                // 15 of the MFMAs before the first load)
                __builtin_amdgcn_sched_group_barrier(0x8, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x20, 1, 0);  // VMEM read
            }
        } else {
#pragma unroll
            for (int q = 0; q < SPW; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q], fb[q], acc, 0, 0, 0);
        }
        if (wave + 1 < kW) {
            acc_s[t][lane] = acc;
            return;
        }
        const int64_t tok = ((int64_t)blockIdx.y * kTiles + t) * 32 + fr;
        if (tok < M) {
            // lane holds token `tok` and features f0 + 8 g + 4 kh + 0..3
#pragma unroll
            for (int g = 0; g < kRows / 8; ++g) {
                const float v0 = acc[4 * g], v1 = acc[4 * g + 1], v2 = acc[4 * g + 2], v3 = acc[4 * g + 3];
                const int64_t off = tok * kD + f0 + g * 8 + kh * 4;
                if (!kFwd || e32) *reinterpret_cast<f32x4*>(e32 + off) = f32x4{v0, v1, v2, v3};
                if (kFwd) *reinterpret_cast<u32x2*>(e16 + off) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            }
        }
    };
    if constexpr (kRows == 32) {
        // W rows f0 .. f0+31 and token tile 0 in runs; tokens past the last
        // read token 0 (in bounds), whose columns are never stored
        const int kb = wave * SPW * 16;
        const int64_t t0 = (int64_t)blockIdx.y * kTiles * 32;
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int r = run_row(q, lane);
            fa[q] = *reinterpret_cast<const bf16x8*>(W + (int64_t)(f0 + r) * kD + kb + run_chunk(q, lane) * 8);
            const int64_t tok = t0 + r;
            fb[q] = *reinterpret_cast<const bf16x8*>(x + (tok < M ? tok : 0) * kD + kb + run_chunk(q, lane) * 8);
        }
        // wave w runs tile t in step w + t; every wave passes kW + kTiles - 1
        // barriers, one at the end of each step
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        for (int i = 0; i + 1 < wv; ++i) __syncthreads();
        runs_to_fragments(fa);
        runs_to_fragments(fb);
        if (wv > 0) __syncthreads();
        for (int t = 0; t < kTiles; ++t) {
            segment(t);
            __syncthreads();
        }
        for (int i = wv; i + 1 < kW; ++i) __syncthreads();
    } else {
        // 16 rows and one token tile (a decode step's few tokens): W and x in
        // the MFMA layout, the lanes of the MFMA's other 16 A rows and of the
        // tokens past the last loading nothing (zeros). Here that is fewer
        // pieces for the address unit than runs over all 32 rows and tokens
        static_assert(kTiles == 1, "16-row blocks take one token tile");
        const bf16x8 zero = {};
        const bool row = fr < kRows;
        const uint16_t* wrow = W + (int64_t)(f0 + (row ? fr : 0)) * kD + wave * SPW * 16 + kh * 8;
        const int64_t tok = (int64_t)blockIdx.y * 32 + fr;
        const bool live = tok < M;
        const uint16_t* xrow = x + (live ? tok : 0) * kD + wave * SPW * 16 + kh * 8;
#pragma unroll
        for (int q = 0; q < SPW; ++q) fa[q] = row ? *reinterpret_cast<const bf16x8*>(wrow + q * 16) : zero;
#pragma unroll
        for (int q = 0; q < SPW; ++q) fb[q] = live ? *reinterpret_cast<const bf16x8*>(xrow + q * 16) : zero;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        for (int w = 0; w < kW; ++w) {
            if (wave == w) {
                if (w > 0) acc = acc_s[0][lane];
#pragma unroll
                for (int q = 0; q < SPW; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q], fb[q], acc, 0, 0, 0);
                if (w + 1 < kW) acc_s[0][lane] = acc;
            }
            __syncthreads();
        }
        if (wave == kW - 1 && live) {
            // lane holds token `tok` and features f0 + 8 g + 4 kh + 0..3
#pragma unroll
            for (int g = 0; g < kRows / 8; ++g) {
                const float v0 = acc[4 * g], v1 = acc[4 * g + 1], v2 = acc[4 * g + 2], v3 = acc[4 * g + 3];
                const int64_t off = tok * kD + f0 + g * 8 + kh * 4;
                if (!kFwd || e32) *reinterpret_cast<f32x4*>(e32 + off) = f32x4{v0, v1, v2, v3};
                if (kFwd) *reinterpret_cast<u32x2*>(e16 + off) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            }
        }
    }
}

// Mid-size calls (257-3200 tokens): tiles of 128 tokens x 256 features so
// that more blocks share the chip (the 256 x 256 tiles give such calls only
// 20-130 blocks); up to 3200 tokens the grid (at most 250 blocks) is one
// round on the 256 CUs. Eight waves, each 64 features x 64 tokens (2 x 2
// MFMA tiles); both operands through LDS as in proj_kernel, 48 KB stages.
// The bf16 tile is staged through LDS as 512-byte token rows (16-byte chunk
// c of row r at chunk c ^ (r & 31)), so that each store instruction writes
// two whole row segments; stores straight from the accumulators (16 bytes
// per row per instruction) took up to 60% longer. The k order of every
// output is proj_kernel's, so the bits are the same.
constexpr int kMidT = 3200;           // largest call served by proj_mid_kernel
constexpr int BMM = 128;              // tokens per block
constexpr int STM = (BN + BMM) * BK;  // bf16 elements per stage
constexpr int kMidLds = 2 * STM * 2;  // 98304

template <bool kFwd>
__global__ void __launch_bounds__(kThreads, 1)
proj_mid_kernel(const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ W,
                float* __restrict__ e32, uint16_t* __restrict__ e16) {
    constexpr int LX = BMM / (kWaves * RPL);  // x loads per wave per stage
    constexpr int LW = BN / (kWaves * RPL);   // W loads per wave per stage
    static_assert(BMM * BN * 2 <= kMidLds && BMM == kWaves * 16, "bf16 tile staging");
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ff = wave & 3, tt = wave >> 2;  // 64-feature quarter, 64-token half
    const int nb = gridDim.x, b = blockIdx.x;
    const int per = nb / kXcds, rem = nb % kXcds, xcd = b % kXcds;
    const int tile = xcd * per + (xcd < rem ? xcd : rem) + b / kXcds;
    const int n0 = (tile % kNTiles) * BN;
    const int64_t m0 = (int64_t)(tile / kNTiles) * BMM;

    const uint16_t* gW[LW];
    const uint16_t* gX[LX];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int row = (wave * LW + i) * RPL + lane / CH;
        gW[i] = W + (int64_t)(n0 + row) * kD + ((lane % CH) ^ swz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < LX; ++i) {
        const int row = (wave * LX + i) * RPL + lane / CH;
        const int64_t tok = m0 + row;
        // rows past the last token read token 0 (in bounds); their results are never stored
        gX[i] = x + (tok < M ? tok : 0) * kD + ((lane % CH) ^ swz(row)) * 8;
    }
    auto issue = [&](int kt) {
        uint16_t* sbase = lds + (kt & 1) * STM;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < LW; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void*)(gW[i] + k0), (lds_void*)(sbase + (wave * LW + i) * RPL * BK),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < LX; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void*)(gX[i] + k0),
                                             (lds_void*)(sbase + BN * BK + (wave * LX + i) * RPL * BK), 16, 0, 0);
    };
    const int fr = lane & 31, kh = lane >> 5, sw = swz(fr);
    const int offA = (ff * 64 + fr) * BK, offB = BN * BK + (tt * 64 + fr) * BK;
    bf16x8 fa[2][2], fb[2][2];
    auto read = [&](int kt, int ks, int buf) {
        const uint16_t* base = lds + (kt & 1) * STM;
        const int c = ((ks * 2 + kh) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            fa[buf][i] = *reinterpret_cast<const bf16x8*>(base + offA + i * 32 * BK + c);
            fb[buf][i] = *reinterpret_cast<const bf16x8*>(base + offB + i * 32 * BK + c);
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    auto mfma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };
    issue(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue(1);
    read(0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ks = 0; ks < BK / 16 - 1; ++ks) {
            read(kt, ks + 1, (ks + 1) & 1);
            mfma(ks & 1);
        }
        // this wave's reads of stage kt are complete; after the barrier every
        // wave's are, and stage kt+1 has landed
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        mfma(1);
        if (kt + 1 < KT) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __builtin_amdgcn_s_barrier();
            if (kt + 2 < KT) issue(kt + 2);
            read(kt + 1, 0, 0);
        }
    }
    // lane holds token m0 + 64 tt + 32 j + fr and features n0 + 64 ff + 32 i + 8 g + 4 kh + 0..3
    if (!kFwd || e32) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t tok = m0 + tt * 64 + 32 * j + fr;
            if (tok >= M) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t off = tok * kD + n0 + ff * 64 + 32 * i + 8 * g + 4 * kh;
                    *reinterpret_cast<f32x4*>(e32 + off) =
                        f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                }
        }
    }
    if (kFwd) {
        // every wave has finished reading the stages before they are reused
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = tt * 64 + 32 * j + fr;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = ff * 8 + 4 * i + g;
                    *reinterpret_cast<u32x2*>(lds + r * 256 + (c ^ (r & 31)) * 8 + kh * 4) =
                        u32x2{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                              pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                }
        }
        __syncthreads();
        // wave w stores rows 16 w .. 16 w + 15, two 512-byte rows per instruction
        const int c = lane & 31;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = wave * 16 + q * 2 + (lane >> 5);
            const int64_t tok = m0 + r;
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * 256 + (c ^ (r & 31)) * 8);
            if (tok < M) *reinterpret_cast<u32x4*>(e16 + tok * kD + n0 + c * 8) = v;
        }
    }
}

// Tiles of 256 tokens x 320 features (8 per token tile instead of 10):
// fewer, larger tiles, so that token counts whose 256 x 256 grid ends in a
// partly filled round of 256 blocks fill whole rounds instead (8192 tokens:
// 256 tiles, one round, against 320; 16384 tokens: 512 against 640), and
// 10% fewer operand bytes per flop from L2. Eight waves of 160 features x 64
// tokens (5 x 2 MFMA tiles), both operands through LDS in two 72 KB stages,
// the main loop of proj_kernel with one more A fragment per k-step; the k
// order of every output is proj_kernel's, so the bits are the same. The bf16
// tile leaves in two passes of 128 tokens staged as 656-byte rows (320
// features and 16 bytes of padding, so that the 32 rows an MFMA-layout store
// touches spread over the LDS banks), stored as whole 640-byte segments.
constexpr int BNW = 320;                   // features per block
constexpr int kNTilesW = kD / BNW;         // feature tiles per token tile
constexpr int NFW = BNW / 2 / 32;          // A tiles per wave
constexpr int LWW = BNW / (kWaves * RPL);  // W loads per wave per stage
constexpr int STW = (BNW + BM) * BK;       // bf16 elements per stage
constexpr int kLdsW = 2 * STW * 2;         // 147456
constexpr int kPadRow = BNW + 8;           // staging row in bf16 elements

__global__ void __launch_bounds__(kThreads, 1)
proj_w320_kernel(const uint16_t* __restrict__ x, int64_t M, const uint16_t* __restrict__ W,
                 float* __restrict__ e32, uint16_t* __restrict__ e16) {
    static_assert(BNW % (kWaves * RPL) == 0 && 128 * kPadRow * 2 <= kLdsW, "tile shape");
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fh = wave & 1, tq = wave >> 1;  // 160-feature half, 64-token quarter
    const int nb = gridDim.x, b = blockIdx.x;
    const int per = nb / kXcds, rem = nb % kXcds, xcd = b % kXcds;
    const int tile = xcd * per + (xcd < rem ? xcd : rem) + b / kXcds;
    const int n0 = (tile % kNTilesW) * BNW;
    const int64_t m0 = (int64_t)(tile / kNTilesW) * BM;

    const uint16_t* gW[LWW];
    const uint16_t* gX[LPW];
#pragma unroll
    for (int i = 0; i < LWW; ++i) {
        const int row = (wave * LWW + i) * RPL + lane / CH;
        gW[i] = W + (int64_t)(n0 + row) * kD + ((lane % CH) ^ swz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = (wave * LPW + i) * RPL + lane / CH;
        const int64_t tok = m0 + row;
        // rows past the last token read token 0 (in bounds); their results are never stored
        gX[i] = x + (tok < M ? tok : 0) * kD + ((lane % CH) ^ swz(row)) * 8;
    }
    auto issue = [&](int kt) {
        uint16_t* sbase = lds + (kt & 1) * STW;
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < LWW; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void*)(gW[i] + k0), (lds_void*)(sbase + (wave * LWW + i) * RPL * BK),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void*)(gX[i] + k0),
                                             (lds_void*)(sbase + BNW * BK + (wave * LPW + i) * RPL * BK), 16, 0, 0);
    };
    const int fr = lane & 31, kh = lane >> 5, sw = swz(fr);
    const int offA = (fh * (BNW / 2) + fr) * BK, offB = BNW * BK + (tq * 64 + fr) * BK;
    bf16x8 fa[2][NFW], fb[2][2];
    auto read = [&](int kt, int ks, int buf) {
        const uint16_t* base = lds + (kt & 1) * STW;
        const int c = ((ks * 2 + kh) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < NFW; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8*>(base + offA + i * 32 * BK + c);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8*>(base + offB + j * 32 * BK + c);
    };
    f32x16 acc[NFW][2];
#pragma unroll
    for (int i = 0; i < NFW; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    constexpr int NQ = 2 * NFW;  // MFMAs per k-step
    auto mfma = [&](int buf, int lo, int hi) {
#pragma unroll
        for (int q = lo; q < hi; ++q)
            acc[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][q >> 1], fb[buf][q & 1],
                                                                         acc[q >> 1][q & 1], 0, 0, 0);
    };
    issue(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue(1);
    read(0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ks = 0; ks < BK / 16 - 1; ++ks) {
            read(kt, ks + 1, (ks + 1) & 1);
            mfma(ks & 1, 0, NQ);
            // one fragment read between consecutive MFMAs
#pragma unroll
            for (int q = 0; q < NFW + 2; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NQ - NFW - 2, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        mfma(1, 0, NQ / 2);
        if (kt + 1 < KT) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __builtin_amdgcn_s_barrier();
            if (kt + 2 < KT) issue(kt + 2);
            read(kt + 1, 0, 0);
        }
        mfma(1, NQ / 2, NQ);
    }
    // lane holds token m0 + 64 tq + 32 j + fr and features n0 + 160 fh + 32 i + 8 g + 4 kh + 0..3
    if (e32) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t tok = m0 + tq * 64 + 32 * j + fr;
            if (tok >= M) continue;
#pragma unroll
            for (int i = 0; i < NFW; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4*>(e32 + tok * kD + n0 + fh * (BNW / 2) + 32 * i + 8 * g + 4 * kh) =
                        f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        // the stages (pass 0) or the previous pass's staging are no longer read
        __syncthreads();
        const int pr = tq * 32 + fr;  // staged row: token m0 + 64 (pr / 32) + 32 j + pr % 32
#pragma unroll
        for (int i = 0; i < NFW; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<u32x2*>(lds + pr * kPadRow + fh * (BNW / 2) + 32 * i + 8 * g + 4 * kh) =
                    u32x2{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                          pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
        __syncthreads();
        // 128 rows x 40 chunks of 16 bytes, chunk q = tid + 512 k
#pragma unroll
        for (int k = 0; k < 128 * (BNW / 8) / kThreads; ++k) {
            const int q = tid + kThreads * k;
            const int row = q / (BNW / 8), col = q % (BNW / 8);
            const int64_t tok = m0 + (row >> 5) * 64 + j * 32 + (row & 31);
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kPadRow + col * 8);
            if (tok < M) *reinterpret_cast<u32x4*>(e16 + tok * kD + n0 + col * 8) = v;
        }
    }
}

// Whether the 256 x 320 tiling is expected to finish first: rounds of 256
// blocks, its tiles weighted 1.2x (measured per full round) against the
// 256 x 256 tiles'.
__host__ inline bool use_w320(int64_t T) {
    const int64_t tt = (T + BM - 1) / BM;
    const int64_t r256 = (kNTiles * tt + 255) / 256, r320 = (kNTilesW * tt + 255) / 256;
    return 6 * r320 <= 5 * r256;
}

template <bool kFwd>
hipError_t launch(const uint16_t* x, int64_t T, const uint16_t* W, float* e32, uint16_t* e16,
                  hipStream_t stream) {
    // the dynamic LDS (128 KB, 96 KB, 144 KB) must be allowed once per device
    static std::atomic<uint64_t> allowed{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(allowed.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&proj_kernel<kFwd>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (err != hipSuccess) return err;
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&proj_mid_kernel<kFwd>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMidLds);
        if (err != hipSuccess) return err;
        if (kFwd) {
            err = hipFuncSetAttribute(reinterpret_cast<const void*>(&proj_w320_kernel),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsW);
            if (err != hipSuccess) return err;
        }
        allowed.fetch_or(bit, std::memory_order_acq_rel);
    }
    if (T <= kSmallT) {
        // about 160 blocks: one token tile runs 16 features per block, up to
        // 3 tiles one block per (32-feature, tile), more tiles 2 or 4 per block
        const unsigned tiles = (unsigned)((T + 31) / 32);
        if (tiles == 1)
            hipLaunchKernelGGL((proj_small_kernel<kFwd, 16, 1>), dim3(kD / 16, 1), dim3(512), 0, stream, x, T, W,
                               e32, e16);
        else if (tiles <= 3)
            hipLaunchKernelGGL((proj_small_kernel<kFwd, 32, 1>), dim3(kD / 32, tiles), dim3(512), 0, stream, x, T,
                               W, e32, e16);
        else if (tiles <= 6)
            hipLaunchKernelGGL((proj_small_kernel<kFwd, 32, 2>), dim3(kD / 32, (tiles + 1) / 2), dim3(512), 0, stream,
                               x, T, W, e32, e16);
        else
            hipLaunchKernelGGL((proj_small_kernel<kFwd, 32, 4>), dim3(kD / 32, (tiles + 3) / 4), dim3(512), 0, stream,
                               x, T, W, e32, e16);
        return hipGetLastError();
    }
    if (T <= kMidT) {
        hipLaunchKernelGGL(proj_mid_kernel<kFwd>, dim3((unsigned)(kNTiles * ((T + BMM - 1) / BMM))), dim3(kThreads),
                           kMidLds, stream, x, T, W, e32, e16);
        return hipGetLastError();
    }
    if (kFwd && use_w320(T)) {
        hipLaunchKernelGGL(proj_w320_kernel, dim3((unsigned)(kNTilesW * ((T + BM - 1) / BM))), dim3(kThreads), kLdsW,
                           stream, x, T, W, e32, e16);
        return hipGetLastError();
    }
    dim3 grid((unsigned)(kNTiles * ((T + BM - 1) / BM)));
    hipLaunchKernelGGL(proj_kernel<kFwd>, grid, dim3(kThreads), kLdsBytes, stream, x, T, W, e32, e16);
    return hipGetLastError();
}

}  // namespace

int proj_tiling(int64_t T) {
    if (T <= 0) return 0;
    if (T <= kSmallT) return 1;
    if (T <= kMidT) return 2;
    return use_w320(T) ? 4 : 3;
}

hipError_t launch_proj(const uint16_t* x, int64_t T, const uint16_t* W, float* e32,
                       uint16_t* e16, hipStream_t stream) {
    if (e16) return launch<true>(x, T, W, e32, e16, stream);
    return launch<false>(x, T, W, e32, nullptr, stream);
}

}  // namespace ple
