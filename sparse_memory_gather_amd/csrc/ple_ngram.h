// n-gram keys of one token (segment-aware, with carried history), shared by
// the ID kernel and the gather variant that computes its own IDs.
//
// The rows an n-gram embedding reads depend only on the recent token IDs,
// positions and sequence boundaries (mengman.github.io "Qwen3.8-Flash-Next
// 端侧部署 01", section on the n-gram embedding path; reactapp.top RTX 3090
// article, section "n-gram表格": hashed bigram and trigram keys):
//   bigram  key (2<<60)|(a<<20)|b,  trigram key (3<<60)|(a<<40)|(b<<20)|c
// finalized with SplitMix64 and reduced mod R (unsigned 64-bit); the token
// before a sequence's first comes from its carried history.
#pragma once

#include "ple_kernels.h"

namespace ple {

__device__ __forceinline__ uint64_t splitmix_finalize(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

// z mod R without a division (the GPU has none for 64-bit integers): with
// m = floor((2^64 - 1) / R), the high half of z * m is floor(z / R) or one
// less (Barrett reduction), so one conditional subtraction of R gives the
// exact remainder; a second one is kept as a guard.
struct ModR {
    uint64_t R, m;
};

inline ModR make_mod(uint64_t R) { return ModR{R, ~0ULL / R}; }

__device__ __forceinline__ uint32_t mod_r(uint64_t z, const ModR& d) {
    const uint64_t q = __umul64hi(z, d.m);
    uint64_t r = z - q * d.R;
    if (r >= d.R) r -= d.R;
    if (r >= d.R) r -= d.R;
    return (uint32_t)r;
}

// sequence of token t: the last s with cu[s] <= t
__device__ __forceinline__ int seq_of(const int32_t* cu, int32_t S, int64_t t) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct NgramKeys {
    uint64_t k2, k3;  // bigram and trigram keys
    int64_t j;        // index of the token in history ++ chunk (j >= 1: bigram, j >= 2: trigram)
};

// keys of token t; flags 1 (token ID outside [0, vocab)) and 4 (hist_len
// outside 0..2) in dev_err. Stays in bounds for malformed cu_seqlens (which
// the caller checks once per launch).
__device__ __forceinline__ NgramKeys ngram_keys(int64_t t, const int32_t* __restrict__ tokens,
                                                const int32_t* __restrict__ cu, int32_t S,
                                                const int32_t* __restrict__ hist_ids,
                                                const int32_t* __restrict__ hist_len, int32_t vocab,
                                                int32_t* dev_err) {
    const int s = seq_of(cu, S, t);
    int64_t start = cu[s];
    if (start < 0 || start > t) start = t;
    int hl = hist_len[s];
    if (hl < 0 || hl > 2) {
        flag_error(dev_err, 4);
        hl = 0;
    }
    NgramKeys k;
    k.j = hl + (t - start);
    auto seq_at = [&](int64_t idx) -> uint32_t {
        const int32_t v = idx < hl ? hist_ids[2 * s + 2 - hl + idx] : tokens[start + idx - hl];
        if (v < 0 || v >= vocab) flag_error(dev_err, 1);
        return (uint32_t)v & 0xFFFFFu;
    };
    const uint32_t c = seq_at(k.j);
    k.k2 = 0;
    k.k3 = 0;
    if (k.j >= 1) {
        const uint32_t b = seq_at(k.j - 1);
        k.k2 = (2ULL << 60) | ((uint64_t)b << 20) | c;
        if (k.j >= 2) k.k3 = (3ULL << 60) | ((uint64_t)seq_at(k.j - 2) << 40) | ((uint64_t)b << 20) | c;
    }
    return k;
}

// two-lookup rows: bigram and trigram, -1 where the sequence is too short
__device__ __forceinline__ int32_t bigram_row(const NgramKeys& k, const ModR& mr) {
    return k.j >= 1 ? (int32_t)mod_r(splitmix_finalize(k.k2), mr) : -1;
}
__device__ __forceinline__ int32_t trigram_row(const NgramKeys& k, const ModR& mr) {
    return k.j >= 2 ? (int32_t)mod_r(splitmix_finalize(k.k3), mr) : -1;
}

// 16-lookup layout: heads 0..7 on the bigram key, 8..15 on the trigram key,
// head h finalizing key + (h mod 8) * 0x9E3779B97F4A7C15 (the h-th SplitMix64
// output from the key), so heads 0 and 8 equal the two-lookup rows
constexpr uint64_t kHeadGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ int32_t head_row(const NgramKeys& k, int h, const ModR& mr) {
    const bool tri = h >= 8;
    if (k.j < (tri ? 2 : 1)) return -1;
    return (int32_t)mod_r(splitmix_finalize((tri ? k.k3 : k.k2) + (uint64_t)(h & 7) * kHeadGamma), mr);
}

// cu_seqlens checks (one block of a launch): cu[0] == 0, non-decreasing, cu[S] == T
__device__ __forceinline__ void check_cu(const int32_t* cu, int32_t S, int64_t T, int32_t* dev_err) {
    for (int i = threadIdx.x; i <= S; i += blockDim.x) {
        const int32_t c = cu[i];
        const bool bad = (i == 0 && c != 0) || (i == S && c != T) || (i < S && c > cu[i + 1]);
        if (bad) flag_error(dev_err, 2);
    }
}

// Sequence [st, en) needs its carried conv state copied before the fuse
// runs when its first and last tokens fall in different fuse blocks of pb
// tokens: the block holding the last token rewrites the state in place while
// another may still read the old one. Within one block the state is read at
// the first token and written at the last by the same thread, in order.
__device__ __forceinline__ bool state_needs_copy(int64_t st, int64_t en, int64_t pb) {
    return en > st && st / pb != (en - 1) / pb;
}

// Copy of the conv state ([S][3][kD] floats) of the sequences that need it:
// block `blk` of `nblk` takes sequences blk, blk + nblk, ..., its threads
// the float4s of each.
__device__ __forceinline__ void copy_state(const float* __restrict__ from, float* __restrict__ to,
                                           const int32_t* __restrict__ cu, int32_t S, int64_t pb,
                                           int64_t blk, int64_t nblk) {
    constexpr int kPerSeq = 3 * kD / 4;  // float4s per sequence
    const f32x4* src = reinterpret_cast<const f32x4*>(from);
    f32x4* dst = reinterpret_cast<f32x4*>(to);
    for (int64_t s = blk; s < S; s += nblk) {
        if (!state_needs_copy(cu[s], cu[s + 1], pb)) continue;  // uniform in the block
        for (int i = threadIdx.x; i < kPerSeq; i += blockDim.x) dst[s * kPerSeq + i] = src[s * kPerSeq + i];
    }
}

}  // namespace ple
