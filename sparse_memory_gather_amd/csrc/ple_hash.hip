// a1: n-gram row IDs (segment-aware, carried history).
//
// The rows an n-gram embedding reads depend only on the recent token IDs,
// positions and sequence boundaries (mengman.github.io "Qwen3.8-Flash-Next
// 端侧部署 01", section on the n-gram embedding path; reactapp.top RTX 3090
// article, section "n-gram表格": hashed bigram and trigram keys). One thread
// per token: find the token's sequence in cu_seqlens, take the previous one
// or two IDs from the chunk or from the carried history, and hash
//   bigram  key (2<<60)|(a<<20)|b,  trigram key (3<<60)|(a<<40)|(b<<20)|c
// with the SplitMix64 finalizer, reduced mod R (unsigned 64-bit). Missing
// history gives -1.
//
// The 16-lookup layout (the model card's 16 lookups of 160-byte rows, SSD
// streaming page, "技术细节") writes 16 IDs per token: heads 0..7 on the
// bigram key, heads 8..15 on the trigram key, head h finalizing
// key + (h mod 8) * 0x9E3779B97F4A7C15 (the h-th SplitMix64 output from the
// key), so heads 0 and 8 equal the two-lookup IDs.
#include "ple_ngram.h"

namespace ple {
namespace {

constexpr int kHashBlock = 256;

// kHeads = 0: two IDs per token (bigram, trigram); 16: the 16-lookup layout
template <int kHeads>
__global__ void __launch_bounds__(kHashBlock)
hash_kernel(const int32_t* __restrict__ tokens, int64_t T, const int32_t* __restrict__ cu, int32_t S,
            const int32_t* __restrict__ hist_ids, const int32_t* __restrict__ hist_len,
            int32_t vocab, ModR mr, int32_t* __restrict__ row_ids, int32_t* dev_err,
            const float* __restrict__ conv_state, float* __restrict__ state_snap,
            int64_t snap_pb) {
    if (blockIdx.y == 1) {
        // copy of the carried conv state of the sequences that need one
        copy_state(conv_state, state_snap, cu, S, snap_pb, blockIdx.x, gridDim.x);
        return;
    }
    if (blockIdx.x == 0) check_cu(cu, S, T, dev_err);
    const int64_t t = (int64_t)blockIdx.x * kHashBlock + threadIdx.x;
    if (t >= T) return;
    const NgramKeys k = ngram_keys(t, tokens, cu, S, hist_ids, hist_len, vocab, dev_err);
    if (kHeads == 0) {
        reinterpret_cast<int2*>(row_ids)[t] = make_int2(bigram_row(k, mr), trigram_row(k, mr));
    } else {
        int32_t id[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) id[h] = head_row(k, h, mr);
        int4* dst = reinterpret_cast<int4*>(row_ids + t * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_int4(id[4 * q], id[4 * q + 1], id[4 * q + 2], id[4 * q + 3]);
    }
}

// the carried conv state alone (ple_forward_x: no ID kernel in the launch)
__global__ void __launch_bounds__(kHashBlock)
state_copy_kernel(const float* __restrict__ conv_state, float* __restrict__ state_snap,
                  const int32_t* __restrict__ cu, int32_t S, int64_t pb) {
    copy_state(conv_state, state_snap, cu, S, pb, blockIdx.x, gridDim.x);
}

}  // namespace

hipError_t launch_state_copy(const float* conv_state, float* state_snap, const int32_t* cu, int32_t S,
                             int64_t pb, hipStream_t stream) {
    int64_t blocks = S < 65536 ? S : 65536;  // one sequence per block and round
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(kHashBlock), 0, stream, conv_state,
                       state_snap, cu, S, pb);
    return hipGetLastError();
}

hipError_t launch_hash(const int32_t* tokens, int64_t T, const int32_t* cu, int32_t S,
                       const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab, int64_t R,
                       int32_t* row_ids, int32_t* dev_err, const float* conv_state,
                       float* state_snap, int64_t snap_pb, bool heads, hipStream_t stream) {
    int64_t blocks = (T + kHashBlock - 1) / kHashBlock;
    if (blocks < 1) blocks = 1;
    // grid row 1 copies the state, one sequence per block and round
    const int64_t snap_blocks = state_snap ? S : 0;
    if (snap_blocks > blocks) blocks = snap_blocks < 65536 ? snap_blocks : 65536;
    dim3 grid((unsigned)blocks, state_snap ? 2 : 1);
    if (heads)
        hipLaunchKernelGGL(hash_kernel<16>, grid, dim3(kHashBlock), 0, stream, tokens, T, cu, S, hist_ids,
                           hist_len, vocab, make_mod((uint64_t)R), row_ids, dev_err, conv_state, state_snap,
                           snap_pb);
    else
        hipLaunchKernelGGL(hash_kernel<0>, grid, dim3(kHashBlock), 0, stream, tokens, T, cu, S, hist_ids,
                           hist_len, vocab, make_mod((uint64_t)R), row_ids, dev_err, conv_state, state_snap,
                           snap_pb);
    return hipGetLastError();
}

}  // namespace ple
