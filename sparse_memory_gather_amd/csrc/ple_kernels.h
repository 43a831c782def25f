// Internal declarations shared by the libple HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ple {

constexpr int kD = 2560;          // row width = hidden size
constexpr int kTaps = 4;          // short-conv taps

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two floats -> two bf16 (round to nearest even), low element in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void flag_error(int32_t* dev_err, int bit) {
    if (dev_err) atomicOr(dev_err, bit);
}

// what a gather launch needs to compute its own row IDs (launch_gather_ids)
struct IdSource {
    const int32_t* tokens;
    const int32_t* cu;
    int32_t S;
    const int32_t* hist_ids;
    const int32_t* hist_len;
    int32_t vocab;
    int32_t* row_ids_out;     // int32 [T][2] (16-lookup layout: [T][16]), or NULL
    const float* conv_state;  // copied to snap when snap is not NULL (the sequences that need it)
    float* snap;
    int64_t snap_pb;          // the fuse's tokens per block (fuse_block_tokens)
    uint64_t mod_R, mod_m;  // set by launch_gather_ids (R and its reciprocal for mod_r)
};

// ---- launchers (each returns hipGetLastError()) ----------------------------

// n-gram IDs for T tokens (2 per token, or 16 with heads); optionally also
// copies conv_state [S][3][kD] into state_snap for the sequences whose state
// the fuse (snap_pb tokens per block) reads in one block and rewrites in
// another.
hipError_t launch_hash(const int32_t* tokens, int64_t T, const int32_t* cu, int32_t S,
                       const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab, int64_t R,
                       int32_t* row_ids, int32_t* dev_err, const float* conv_state,
                       float* state_snap, int64_t snap_pb, bool heads, hipStream_t stream);

// NVFP4 table: codes [R][1280] (E2M1, low nibble first), blocks [R][160]
// (E4M3 per 16 elements), scales [R]; raw (optional) [T][2][1280]
hipError_t launch_gather_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes, const uint8_t* blocks,
                               const float* scales, int64_t R, uint16_t* x, uint8_t* raw, int32_t* dev_err,
                               hipStream_t stream);

// copy of conv_state [S][3][kD] into state_snap (the sequences that need it)
hipError_t launch_state_copy(const float* conv_state, float* state_snap, const int32_t* cu, int32_t S,
                             int64_t pb, hipStream_t stream);

// Tokens per block of the fuse for a T-token call of S sequences (1 when it
// runs one token per block); the state copy and the fuse agree on it.
int64_t fuse_block_tokens(int64_t T, int32_t S);

// 16-lookup layout: table [16][R][160], scales [16][R], row_ids [T][16],
// raw (optional) [T][16][160].
hipError_t launch_gather_heads(const int32_t* row_ids, int64_t T, const uint8_t* table,
                               const float* scales, int64_t R, uint16_t* x, uint8_t* raw,
                               int32_t* dev_err, hipStream_t stream);

// a gather computing each token's row IDs itself (the ID kernel's work,
// cu_seqlens checks and state copy included): the FP8 table (two lookups),
// the 16-lookup layout, or the NVFP4 table (nv_blocks)
constexpr int kLayoutFp8 = 0, kLayoutHeads = 1, kLayoutNvfp4 = 2;
hipError_t launch_gather_ids(const IdSource& src, int layout, int64_t T, const uint8_t* table,
                             const uint8_t* nv_blocks, const float* scales, int64_t R, uint16_t* x,
                             int32_t* dev_err, hipStream_t stream);

hipError_t launch_gather(const int32_t* row_ids, int64_t T, const uint8_t* table,
                         const float* scales, int64_t R, uint16_t* x, uint8_t* raw,
                         int32_t* dev_err, hipStream_t stream);

// e = x W^T. Forward mode (e16 != nullptr): writes e as bf16 into e16, and
// as fp32 into e32 if e32 != nullptr. Projection-only mode: fp32 into e32.
hipError_t launch_proj(const uint16_t* x, int64_t T, const uint16_t* W, float* e32,
                       uint16_t* e16, hipStream_t stream);

// The tiling launch_proj uses in forward mode for T tokens (values as
// ple_proj_tiling in ple.h).
int proj_tiling(int64_t T);

// Gate (from h and the bf16 e), causal short conv with carried state,
// residual add; updates conv_state and the n-gram history in place.
hipError_t launch_fuse(const uint16_t* h, const uint16_t* e16, int64_t T, const int32_t* cu,
                       int32_t S, const int32_t* tokens, const uint16_t* conv_w,
                       const float* state_snap, float* conv_state, int32_t* hist_ids,
                       int32_t* hist_len, uint16_t* out, float eps, float* gate_out, float* y_out,
                       uint16_t* h_copy, hipStream_t stream);  // h_copy: T x 2560 bf16 scratch, used when out == h

// ---- the whole path of a short call in one launch (ple_decode.hip) ----------
constexpr int kDecodeMaxT = 16;    // tokens: their x tile is staged in LDS (82 KB at 16)
constexpr int kDecodeMaxS = 256;   // sequences: their metadata is staged in LDS

struct DecodeArgs {
    const int32_t* tokens;
    int64_t T;
    const int32_t* cu;
    int32_t S;
    int32_t vocab;
    int32_t* hist_ids;           // in/out
    int32_t* hist_len;           // in/out
    const uint8_t* table;
    const float* scales;
    int64_t R;
    uint64_t mod_R, mod_m;       // set by launch_decode_step
    const uint16_t* W;
    const uint16_t* conv_w;
    const uint16_t* h;           // read only (out may be h: see hw)
    uint16_t* out;
    uint16_t* hw;                // workspace: copy of h [T][kD] when out == h, else NULL
    float* conv_state;
    float* snap;                 // workspace: carried state of sequences spanning finishers
    uint16_t* e16;               // workspace: bf16 e [T][kD]
    uint32_t* sync;              // workspace: three counters, zero at the call, left zero
    float eps;
    int32_t* dev_err;
    int32_t* row_ids_out;
    uint16_t* x_out;
    float* e_out;
    float* gate_out;
    float* y_out;
};

// whether a T-token call of S sequences (FP8 table) runs as one launch
bool decode_one_launch(int64_t T, int32_t S);
hipError_t launch_decode_step(DecodeArgs a, hipStream_t stream);

}  // namespace ple
