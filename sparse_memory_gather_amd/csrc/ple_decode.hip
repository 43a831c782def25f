// The whole path of a short call in one launch: n-gram IDs, gather and
// dequant, projection, gate, short conv and residual add.
//
// A decode step carries a few tokens (one per sequence) through every stage,
// and each stage would be its own launch. The Thor vLLM deployment splits its
// CUDA graph at the PLE ops (kipfel.ltd, section "五、启动参数"), and the
// Spark deployment notes that decode cannot hide the lookup the way prefill
// can (mengman.github.io "Qwen3.8-Flash-Next 端侧部署 01", inference-flow
// section). Here a call of up to 16 tokens runs as one grid of
// kProj + T blocks of 640 threads, whose roles come from a ticket each block
// takes when it starts (an atomic counter in the caller's workspace):
//   - tickets 0 .. kProj-1: projection block p computes e for features
//     32p .. 32p+31 of every token (all 32 A rows of the MFMA). It computes
//     the tokens' row IDs once (the ID kernel's device code) while its other
//     waves issue their W loads (in 64-byte runs, moved into the MFMA's
//     fragment layout in registers later), loads the rows with coalesced
//     reads, dequantizes all of x into an LDS tile (the gather's device
//     code), and runs proj_small_kernel's k chain (ten waves of 16 k-steps
//     handing the accumulator on through LDS), so x and e are bit-identical
//     to the three-launch path. It writes e as bf16 into the workspace,
//     copies the carried state of sequences that need it, then releases and
//     increments the `done` counter. Each release writes back the L2 of the
//     block's XCD, and those of one XCD take turns, so fewer, wider blocks
//     publish sooner: 80 blocks of 32 features rather than 160 of 16.
//   - tickets kProj .. kProj+T-1: finisher i fuses token i exactly as the
//     one-token fuse kernel does (the same device code). It loads what does
//     not depend on e first (its sequence, h rows, conv weights, its own
//     carried state), waits for `done` to reach kProj, then reads e, gates,
//     convolves and writes out, the new state and the history.
// A finisher waits only for tickets below its own, held by blocks that have
// started and never wait, so the wait ends whether or not the whole grid is
// resident; no cooperative launch or grid barrier is needed. The wait is
// bounded all the same: past the spin limit the block flags
// PLE_DEVERR_SYNC and goes on. The last finisher resets the three counters,
// so the workspace holds zeros again after every call (no memset, so a
// captured call replays as it ran).
#include <atomic>

#include "ple_dequant.h"
#include "ple_fragments.h"
#include "ple_fuse_common.h"

namespace ple {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowsPerBlock = 32;            // features per projection block (the MFMA's A rows)
constexpr int kProj = kD / kRowsPerBlock;    // 80 projection blocks
constexpr int kChainWaves = fuse::kWaves;    // 10 waves of the 640-thread block
constexpr int kSteps = kD / 16 / kChainWaves;  // 16 k-steps per wave
constexpr uint32_t kSpinLimit = 1u << 21;    // polls of `done` before giving up (about a second)
constexpr int kDevErrSync = 16;              // PLE_DEVERR_SYNC

constexpr int kXRow = kD + 8;   // LDS row of the x tile in bf16: 16 bytes of padding spread the tokens over the banks

__global__ void __launch_bounds__(fuse::kThreads)
decode_step_kernel(const DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t x_s[];   // [T][kXRow] bf16 (projection blocks)
    __shared__ int s_ticket;
    __shared__ int32_t s_cu[kDecodeMaxS + 1];
    __shared__ int32_t s_tok[kDecodeMaxT];
    __shared__ int32_t s_hid[2 * kDecodeMaxS];
    __shared__ int32_t s_hlen[kDecodeMaxS];
    __shared__ int2 s_rows[kDecodeMaxT];
    __shared__ f32x16 acc_s[64];
    __shared__ float red_s[4][fuse::kRows][3];
    __shared__ float g_s[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = (int)a.T, S = a.S;
    const bf16x8 zero = {};
    // the ticket and the sequences' metadata, staged in LDS once per block
    // with every load in flight at once (a thread stages at most one element
    // of each array)
    static_assert(2 * kDecodeMaxS <= fuse::kThreads && kDecodeMaxT <= fuse::kThreads, "one element per thread");
    const int32_t v_cu = tid <= S ? a.cu[tid] : 0;
    const int32_t v_tok = tid < T ? a.tokens[tid] : 0;
    const int32_t v_hid = tid < 2 * S ? a.hist_ids[tid] : 0;
    const int32_t v_hlen = tid < S ? a.hist_len[tid] : 0;
    // after the loads: the compiler waits for the ticket right after taking it
    uint32_t tk = 0;
    if (tid == 0) tk = __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) s_ticket = (int)tk;
    if (tid <= S) s_cu[tid] = v_cu;
    if (tid < T) s_tok[tid] = v_tok;
    if (tid < 2 * S) s_hid[tid] = v_hid;
    if (tid < S) s_hlen[tid] = v_hlen;
    __syncthreads();
    const int ticket = s_ticket;
    if (ticket >= kProj + T) {
        // the counters were not zero when the call began (a workspace not
        // cleared before its first use)
        if (tid == 0) flag_error(a.dev_err, kDevErrSync);
        return;
    }

    if (ticket < kProj) {
        const int p = ticket;
        const int fr = lane & 31, kh = lane >> 5;
        const int k0 = wave * kSteps * 16 + kh * 8;  // this lane's first k
        const int f0 = p * kRowsPerBlock;
        if (p == 0) check_cu(s_cu, S, a.T, a.dev_err);
        // each token's two rows, once per block (the ID kernel's device code)
        if (tid < T) {
            const NgramKeys k = ngram_keys(tid, s_tok, s_cu, S, s_hid, s_hlen, a.vocab, a.dev_err);
            const ModR mr{a.mod_R, a.mod_m};
            s_rows[tid] = make_int2(bigram_row(k, mr), trigram_row(k, mr));
        }
        // W in 64-byte runs (ple_fragments.h), issued while wave 0 computes
        // the IDs: about a quarter of the address-unit time of loads in the
        // MFMA layout. The barrier below waits for LDS operations, not for
        // loads in flight
        static_assert(kRowsPerBlock == 32, "the runs cover the MFMA's 32 rows");
        const uint16_t* wp = a.W + (int64_t)f0 * kD + wave * kSteps * 16;
        bf16x8 fa[kSteps];
#pragma unroll
        for (int q = 0; q < kSteps; ++q)
            fa[q] = *reinterpret_cast<const bf16x8*>(wp + run_row(q, lane) * kD + run_chunk(q, lane) * 8);
        __syncthreads();
        // x of every token into LDS, 8 elements per piece (the gather's
        // device code): consecutive threads read consecutive 8-byte pieces of
        // a row, all loads in flight before the first conversion
        constexpr int kPieces = kDecodeMaxT * (kD / 8) / fuse::kThreads;  // per thread, at most
        const int n_pieces = T * (kD / 8);
        u32x2 ca[kPieces], cb[kPieces];
        float sa[kPieces], sb[kPieces];
        bool va[kPieces], vb[kPieces];
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            if (j * fuse::kThreads < n_pieces) {   // the same for every thread of the block
                const int c = tid + j * fuse::kThreads;
                const bool in = c < n_pieces;
                const int t = in ? c / (kD / 8) : 0, k8 = (c % (kD / 8)) * 8;
                const int2 r = s_rows[t];
                va[j] = in && r.x >= 0;
                vb[j] = in && r.y >= 0;
                // loads under a per-lane condition would need their values at
                // once (to merge with the zeros of the other lanes), and the
                // loads issued before them would be waited for too; row 0
                // stands in for a missing row instead, and the dequant drops
                // its bytes
                const int64_t rx = r.x >= 0 ? r.x : 0, ry = r.y >= 0 ? r.y : 0;
                ca[j] = *reinterpret_cast<const u32x2*>(a.table + rx * kD + k8);
                cb[j] = *reinterpret_cast<const u32x2*>(a.table + ry * kD + k8);
                sa[j] = a.scales[rx];
                sb[j] = a.scales[ry];
            }
        }
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int c = tid + j * fuse::kThreads;
            if (j * fuse::kThreads < n_pieces && c < n_pieces) {
                const int t = c / (kD / 8), k8 = (c % (kD / 8)) * 8;
                *reinterpret_cast<u32x4*>(x_s + t * kXRow + k8) = dequant_pair8(ca[j], sa[j], va[j], cb[j], sb[j], vb[j]);
            }
        }
        __syncthreads();
        if (p == 0) {
            // debug copies of the IDs and x
            if (a.row_ids_out && tid < T) reinterpret_cast<int2*>(a.row_ids_out)[tid] = s_rows[tid];
            if (a.x_out)
                for (int c = tid; c < T * (kD / 8); c += fuse::kThreads) {
                    const int t = c / (kD / 8), k8 = (c % (kD / 8)) * 8;
                    *reinterpret_cast<u32x4*>(a.x_out + (int64_t)t * kD + k8) =
                        *reinterpret_cast<const u32x4*>(x_s + t * kXRow + k8);
                }
        }
        // the k chain, wave by wave (proj_small_kernel's order over k); lanes
        // past the last token feed zeros. Wave v passes the v turns before its
        // own (a barrier each) and moves its W into the MFMA layout during the
        // turn before, so only wave 0's exchange delays the chain; every wave
        // passes kChainWaves barriers in all
        const bool live = fr < T;
        bf16x8 fb[kSteps];
#pragma unroll
        for (int q = 0; q < kSteps; ++q)
            fb[q] = live ? *reinterpret_cast<const bf16x8*>(x_s + fr * kXRow + k0 + q * 16) : zero;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        for (int i = 0; i + 1 < wv; ++i) __syncthreads();
        runs_to_fragments(fa);
        if (wv > 0) {
            __syncthreads();
            acc = acc_s[lane];
        }
#pragma unroll
        for (int q = 0; q < kSteps; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q], fb[q], acc, 0, 0, 0);
        if (wv + 1 < kChainWaves) acc_s[lane] = acc;
        if (wv == 0 && a.hw && lane < T * 4) {
            // in place (out == h): wave 0, done with its turn, copies this
            // block's 32 features of every token's h for the finishers that
            // read earlier tokens' rows; out overwrites h only after every
            // projection block has released
            const int64_t off = (int64_t)(lane >> 2) * kD + f0 + (lane & 3) * 8;
            *reinterpret_cast<u32x4*>(a.hw + off) = *reinterpret_cast<const u32x4*>(a.h + off);
        }
        for (int i = wv; i < kChainWaves; ++i) __syncthreads();
        if (wave == kChainWaves - 1 && live) {
            // lane holds token fr and features f0 + 8 g + 4 kh + 0..3
#pragma unroll
            for (int g = 0; g < kRowsPerBlock / 8; ++g) {
                const float e0 = acc[4 * g], e1 = acc[4 * g + 1], e2 = acc[4 * g + 2], e3 = acc[4 * g + 3];
                const int64_t off = (int64_t)fr * kD + f0 + g * 8 + kh * 4;
                if (a.e_out) *reinterpret_cast<f32x4*>(a.e_out + off) = f32x4{e0, e1, e2, e3};
                *reinterpret_cast<u32x2*>(a.e16 + off) = u32x2{pack_bf16x2(e0, e1), pack_bf16x2(e2, e3)};
            }
        }
        // carried state of the sequences whose first and last tokens are
        // different finishers (read there after the wait, rewritten by the
        // last one), block p taking sequences p, p + kProj, ...
        copy_state(a.conv_state, a.snap, s_cu, S, 1, p, kProj);
        // the barrier completes every wave's stores; one agent-scope release
        // (a write-back of this XCD's L2) then publishes them with the count
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(a.sync + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // finisher: token t
    const int64_t t = ticket - kProj;
    fuse::TokenFuse f;
    // in place, the earlier tokens' h rows are other finishers' out rows:
    // they are read from the projection blocks' copy after the wait
    fuse::token_begin(f, t, a.T, s_cu, S, a.h, nullptr, a.conv_w, a.snap, a.conv_state, tid, a.hw == nullptr);
    // a one-token sequence's state is read and rewritten by this block alone
    const bool own_state = f.sbase == a.conv_state;
    if (own_state) fuse::token_state(f, tid);
    if (tid == 0) {
        // relaxed polls (an acquire on every poll would invalidate this XCD's
        // L2 under the projection blocks still running on it), then one
        // acquire fence
        uint32_t polls = 0, done;
        while ((done = __hip_atomic_load(a.sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < (uint32_t)kProj) {
            if (++polls == kSpinLimit) {
                flag_error(a.dev_err, kDevErrSync);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (done > (uint32_t)kProj) flag_error(a.dev_err, kDevErrSync);  // counted before this call
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (a.hw) fuse::token_window(f, t, a.hw, tid);
    if (!own_state) fuse::token_state(f, tid);
    fuse::token_end(f, t, a.e16, a.tokens, a.conv_state, a.hist_ids, a.hist_len, a.out, a.eps, a.gate_out,
                    a.y_out, red_s, g_s, tid);
    // the last finisher out leaves the counters at zero for the next call
    __syncthreads();
    if (tid == 0) {
        // the counters publish no data: relaxed operations suffice
        const uint32_t n = __hip_atomic_fetch_add(a.sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n == (uint32_t)T - 1) {
            __hip_atomic_store(a.sync + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

bool decode_one_launch(int64_t T, int32_t S) { return T >= 1 && T <= kDecodeMaxT && S >= 1 && S <= kDecodeMaxS; }

hipError_t launch_decode_step(DecodeArgs a, hipStream_t stream) {
    // the x tile (up to 16 tokens: 82 KB) exceeds the default dynamic LDS
    // limit, which is raised once per device
    static std::atomic<uint64_t> allowed{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(allowed.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_step_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kDecodeMaxT * kXRow * 2);
        if (err != hipSuccess) return err;
        allowed.fetch_or(bit, std::memory_order_acq_rel);
    }
    const ModR mr = make_mod((uint64_t)a.R);
    a.mod_R = mr.R;
    a.mod_m = mr.m;
    hipLaunchKernelGGL(decode_step_kernel, dim3((unsigned)(kProj + a.T)), dim3(fuse::kThreads),
                       (size_t)a.T * kXRow * 2, stream, a);
    return hipGetLastError();
}

}  // namespace ple
