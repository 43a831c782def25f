// libple C ABI: argument validation, workspace layout and launch order.
//
// Every host-detectable error is reported before anything is enqueued; the
// kernels then run on the caller's stream in the order of the method
// (IDs -> gather/dequant -> projection -> gate/conv/fuse), nothing is
// synchronized and nothing is allocated.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "../../include/ple.h"
#include "ple_kernels.h"

using namespace ple;

namespace {

// calls up to this many tokens (one round of gather waves on 256 CUs) compute
// their row IDs inside the gather
constexpr int64_t kIdsInGatherMaxT = 1024;

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return PLE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
    bool writable;
};

Range rng(const char* name, const void* p, size_t bytes, bool writable) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo, writable};
}

// Writable ranges may not overlap any other range; the single exception is
// the pair (h, out) over the same extent (in-place fuse).
int check_alias(const Range* r, int n) {
    for (int i = 0; i < n; ++i) {
        if (r[i].lo == r[i].hi) continue;
        for (int j = i + 1; j < n; ++j) {
            if (r[j].lo == r[j].hi) continue;
            if (!r[i].writable && !r[j].writable) continue;
            const bool overlap = r[i].lo < r[j].hi && r[j].lo < r[i].hi;
            if (!overlap) continue;
            const bool same = r[i].lo == r[j].lo && r[i].hi == r[j].hi;
            const std::string a = r[i].name, b = r[j].name;
            const bool in_place = (a == "h" && b == "out") || (a == "out" && b == "h");
            if (same && in_place) continue;
            return fail(PLE_ERR_ALIAS, "%s overlaps %s", r[i].name, r[j].name);
        }
    }
    return PLE_OK;
}

struct WsLayout {
    size_t sync, row_ids, x, e16, snap, total;
};

constexpr size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

// row IDs per token: 2 (bigram, trigram) or 16 in the 16-lookup layout
constexpr int ids_per_token(bool heads) { return heads ? 16 : 2; }

constexpr WsLayout layout(int64_t T, int32_t S, bool heads) {
    WsLayout w{};
    size_t off = 0;
    // counters of the one-launch path: zero before the first call on a
    // workspace, left zero by every call; nothing else writes them
    w.sync = off;    off = 256;
    w.row_ids = off; off = up256(off + (size_t)T * ids_per_token(heads) * sizeof(int32_t));
    w.x = off;       off = up256(off + (size_t)T * kD * 2);
    w.e16 = off;     off = up256(off + (size_t)T * kD * 2);
    w.snap = off;    off = up256(off + (size_t)S * 3 * kD * sizeof(float));
    w.total = off;
    return w;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return PLE_OK;
    return fail(PLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_R(int64_t R) {
    if (R < 1 || R > 2147483647LL) return fail(PLE_ERR_RANGE, "R = %lld outside [1, 2^31-1]", (long long)R);
    return PLE_OK;
}

}  // namespace

extern "C" {

const char* ple_status_string(int status) {
    switch (status) {
        case PLE_OK: return "ok";
        case PLE_ERR_NULL: return "null pointer";
        case PLE_ERR_SHAPE: return "bad shape";
        case PLE_ERR_RANGE: return "value out of range";
        case PLE_ERR_ALIGN: return "misaligned pointer";
        case PLE_ERR_ALIAS: return "overlapping buffers";
        case PLE_ERR_WORKSPACE: return "workspace too small";
        case PLE_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* ple_last_error(void) { return g_last_error.c_str(); }

int ple_proj_tiling(int64_t T) { return ple::proj_tiling(T); }

int ple_forward_one_launch(int64_t T, int32_t S) { return ple::decode_one_launch(T, S) ? 1 : 0; }

size_t ple_forward_workspace_size(int64_t max_T, int32_t max_S) {
    if (max_T < 0 || max_S < 0) return 0;
    return layout(max_T, max_S, false).total;
}

size_t ple_forward_heads_workspace_size(int64_t max_T, int32_t max_S) {
    if (max_T < 0 || max_S < 0) return 0;
    return layout(max_T, max_S, true).total;
}

}  // extern "C"

static int hash_impl(const int32_t* tokens, int64_t T, const int32_t* cu_seqlens, int32_t S,
                     const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab_size, int64_t R,
                     int32_t* row_ids, int32_t* dev_err, void* stream, bool heads) {
    const char* fn = heads ? "ple_hash_heads" : "ple_hash";
    if (T < 0) return fail(PLE_ERR_SHAPE, "T = %lld < 0", (long long)T);
    if (T > 2147483647LL) return fail(PLE_ERR_SHAPE, "T = %lld > 2^31-1 (cu_seqlens are int32)", (long long)T);
    if (S < 1) return fail(PLE_ERR_SHAPE, "S = %d < 1", S);
    if (int st = check_R(R)) return st;
    if (vocab_size < 1 || vocab_size > PLE_MAX_VOCAB)
        return fail(PLE_ERR_RANGE, "vocab_size = %d outside [1, 2^20]", vocab_size);
    if (T == 0) return ok();
    if (!tokens || !cu_seqlens || !hist_ids || !hist_len || !row_ids)
        return fail(PLE_ERR_NULL, "%s: a required pointer is NULL", fn);
    if (!aligned(tokens, 4) || !aligned(cu_seqlens, 4) || !aligned(hist_ids, 4) ||
        !aligned(hist_len, 4) || !aligned(row_ids, heads ? 16 : 8) || !aligned(dev_err, 4))
        return fail(PLE_ERR_ALIGN, "%s: misaligned pointer", fn);
    const size_t ids = (size_t)T * ids_per_token(heads) * 4;
    Range r[] = {rng("tokens", tokens, T * 4, false), rng("cu_seqlens", cu_seqlens, (S + 1) * 4ull, false),
                 rng("hist_ids", hist_ids, S * 8ull, false), rng("hist_len", hist_len, S * 4ull, false),
                 rng("row_ids", row_ids, ids, true), rng("dev_err", dev_err, 4, true)};
    if (int st = check_alias(r, 6)) return st;
    hipError_t e = launch_hash(tokens, T, cu_seqlens, S, hist_ids, hist_len, vocab_size, R, row_ids,
                               dev_err, nullptr, nullptr, 1, heads, reinterpret_cast<hipStream_t>(stream));
    if (int st = hip_status(e, heads ? "ple_hash_heads launch" : "ple_hash launch")) return st;
    return ok();
}

static int lookup_impl(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
                       int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err, void* stream,
                       bool heads) {
    const char* fn = heads ? "ple_lookup_heads" : "ple_lookup";
    if (T < 0) return fail(PLE_ERR_SHAPE, "T = %lld < 0", (long long)T);
    if (int st = check_R(R)) return st;
    if (T == 0) return ok();
    if (!row_ids || !table || !scales || !x_bf16)
        return fail(PLE_ERR_NULL, "%s: a required pointer is NULL", fn);
    if (!aligned(row_ids, heads ? 16 : 8) || !aligned(table, 16) || !aligned(scales, 4) ||
        !aligned(x_bf16, 16) || !aligned(raw_opt, 16) || !aligned(dev_err, 4))
        return fail(PLE_ERR_ALIGN, "%s: misaligned pointer", fn);
    // both layouts: R x 2560 table bytes (16 x R x 160), raw T x 2560 x (2 or 1) bytes
    const size_t n_scales = (size_t)R * (heads ? 16 : 1);
    Range r[] = {rng("row_ids", row_ids, (size_t)T * ids_per_token(heads) * 4, false),
                 rng("table", table, (size_t)R * kD, false), rng("scales", scales, n_scales * 4, false),
                 rng("x", x_bf16, (size_t)T * kD * 2, true),
                 rng("raw", raw_opt, (size_t)T * kD * (heads ? 1 : 2), true), rng("dev_err", dev_err, 4, true)};
    if (int st = check_alias(r, 6)) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = heads ? launch_gather_heads(row_ids, T, table, scales, R, x_bf16, raw_opt, dev_err, s)
                         : launch_gather(row_ids, T, table, scales, R, x_bf16, raw_opt, dev_err, s);
    if (int st = hip_status(e, heads ? "ple_lookup_heads launch" : "ple_lookup launch")) return st;
    return ok();
}

extern "C" {

int ple_hash(const int32_t* tokens, int64_t T, const int32_t* cu_seqlens, int32_t S,
             const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab_size, int64_t R,
             int32_t* row_ids, int32_t* dev_err, void* stream) {
    return hash_impl(tokens, T, cu_seqlens, S, hist_ids, hist_len, vocab_size, R, row_ids, dev_err, stream,
                     false);
}

int ple_hash_heads(const int32_t* tokens, int64_t T, const int32_t* cu_seqlens, int32_t S,
                   const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab_size, int64_t R,
                   int32_t* row_ids, int32_t* dev_err, void* stream) {
    return hash_impl(tokens, T, cu_seqlens, S, hist_ids, hist_len, vocab_size, R, row_ids, dev_err, stream,
                     true);
}

int ple_lookup(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
               int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err, void* stream) {
    return lookup_impl(row_ids, T, table, scales, R, x_bf16, raw_opt, dev_err, stream, false);
}

int ple_lookup_heads(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
                     int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err, void* stream) {
    return lookup_impl(row_ids, T, table, scales, R, x_bf16, raw_opt, dev_err, stream, true);
}

int ple_lookup_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes, const uint8_t* blocks,
                     const float* scales, int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err,
                     void* stream) {
    if (T < 0) return fail(PLE_ERR_SHAPE, "T = %lld < 0", (long long)T);
    if (int st = check_R(R)) return st;
    if (T == 0) return ok();
    if (!row_ids || !codes || !blocks || !scales || !x_bf16)
        return fail(PLE_ERR_NULL, "ple_lookup_nvfp4: a required pointer is NULL");
    if (!aligned(row_ids, 8) || !aligned(codes, 16) || !aligned(blocks, 4) || !aligned(scales, 4) ||
        !aligned(x_bf16, 16) || !aligned(raw_opt, 16) || !aligned(dev_err, 4))
        return fail(PLE_ERR_ALIGN, "ple_lookup_nvfp4: misaligned pointer");
    Range r[] = {rng("row_ids", row_ids, (size_t)T * 8, false), rng("codes", codes, (size_t)R * (kD / 2), false),
                 rng("blocks", blocks, (size_t)R * (kD / 16), false), rng("scales", scales, (size_t)R * 4, false),
                 rng("x", x_bf16, (size_t)T * kD * 2, true), rng("raw", raw_opt, (size_t)T * kD, true),
                 rng("dev_err", dev_err, 4, true)};
    if (int st = check_alias(r, 7)) return st;
    hipError_t e = launch_gather_nvfp4(row_ids, T, codes, blocks, scales, R, x_bf16, raw_opt, dev_err,
                                       reinterpret_cast<hipStream_t>(stream));
    if (int st = hip_status(e, "ple_lookup_nvfp4 launch")) return st;
    return ok();
}

int ple_proj(const uint16_t* x_bf16, int64_t T, const uint16_t* W_bf16, float* e, void* stream) {
    if (T < 0) return fail(PLE_ERR_SHAPE, "T = %lld < 0", (long long)T);
    if (T == 0) return ok();
    if (!x_bf16 || !W_bf16 || !e) return fail(PLE_ERR_NULL, "ple_proj: a required pointer is NULL");
    if (!aligned(x_bf16, 16) || !aligned(W_bf16, 16) || !aligned(e, 16))
        return fail(PLE_ERR_ALIGN, "ple_proj: misaligned pointer");
    Range r[] = {rng("x", x_bf16, (size_t)T * kD * 2, false), rng("W", W_bf16, (size_t)kD * kD * 2, false),
                 rng("e", e, (size_t)T * kD * 4, true)};
    if (int st = check_alias(r, 3)) return st;
    hipError_t err = launch_proj(x_bf16, T, W_bf16, e, nullptr,
                                 reinterpret_cast<hipStream_t>(stream));
    if (int st = hip_status(err, "ple_proj launch")) return st;
    return ok();
}

}  // extern "C"

// x_in != NULL: ple_forward_x (x given; no ID or gather kernel, table,
// scales, R and vocab_size unused)
// nv_blocks != NULL: NVFP4 table (table = codes [R][1280], nv_blocks [R][160])
static int forward_impl(const ple_forward_args* a, void* stream, void* const* events, bool heads,
                        const uint16_t* x_in = nullptr, const uint8_t* nv_blocks = nullptr, bool staged = false) {
    if (!a) return fail(PLE_ERR_NULL, "ple_forward: args is NULL");
    const bool from_x = x_in != nullptr;
    const int64_t T = a->T;
    const int32_t S = a->S;
    if (T < 0) return fail(PLE_ERR_SHAPE, "T = %lld < 0", (long long)T);
    if (T > 2147483647LL) return fail(PLE_ERR_SHAPE, "T = %lld > 2^31-1 (cu_seqlens are int32)", (long long)T);
    if (S < 1) return fail(PLE_ERR_SHAPE, "S = %d < 1", S);
    if (!from_x) {
        if (int st = check_R(a->R)) return st;
        if (a->vocab_size < 1 || a->vocab_size > PLE_MAX_VOCAB)
            return fail(PLE_ERR_RANGE, "vocab_size = %d outside [1, 2^20]", a->vocab_size);
    }
    if (!(a->eps >= 0.0f) || !isfinite(a->eps)) return fail(PLE_ERR_RANGE, "eps must be finite and >= 0");
    if (from_x && (a->row_ids_out || a->x_out))
        return fail(PLE_ERR_SHAPE, "ple_forward_x: row_ids_out and x_out are not produced (x is an input)");
    if (T == 0) return ok();
    if (!a->tokens || !a->cu_seqlens || (!from_x && (!a->table || !a->scales)) || !a->W || !a->conv_w ||
        !a->h || !a->out || !a->hist_ids || !a->hist_len || !a->conv_state)
        return fail(PLE_ERR_NULL, "ple_forward: a required pointer is NULL");
    if (from_x && !aligned(x_in, 16)) return fail(PLE_ERR_ALIGN, "ple_forward_x: x is not 16-byte aligned");
    if (!a->workspace) return fail(PLE_ERR_WORKSPACE, "ple_forward: workspace is NULL");
    const WsLayout L = layout(T, S, heads);
    if (a->workspace_bytes < L.total)
        return fail(PLE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", a->workspace_bytes, L.total);
    if (!aligned(a->tokens, 4) || !aligned(a->cu_seqlens, 4) || !aligned(a->table, 16) ||
        !aligned(a->scales, 4) || !aligned(a->W, 16) || !aligned(a->conv_w, 16) || !aligned(a->h, 16) ||
        !aligned(a->out, 16) || !aligned(a->hist_ids, 4) || !aligned(a->hist_len, 4) ||
        !aligned(a->conv_state, 16) || !aligned(a->workspace, 256) || !aligned(a->dev_err, 4) ||
        !aligned(a->row_ids_out, heads ? 16 : 8) || !aligned(a->x_out, 16) || !aligned(a->e_out, 16) ||
        !aligned(a->gate_out, 4) || !aligned(a->y_out, 16))
        return fail(PLE_ERR_ALIGN, "ple_forward: misaligned pointer");
    const size_t act = (size_t)T * kD * 2;
    Range r[] = {
        rng("tokens", a->tokens, T * 4, false),
        rng("cu_seqlens", a->cu_seqlens, (S + 1) * 4ull, false),
        rng("table", from_x ? nullptr : a->table, (size_t)a->R * (nv_blocks ? kD / 2 : kD), false),
        rng("nvfp4_blocks", nv_blocks, (size_t)a->R * (kD / 16), false),
        rng("scales", from_x ? nullptr : a->scales, (size_t)a->R * (heads ? 16 : 1) * 4, false),
        rng("x", x_in, (size_t)T * kD * 2, false),
        rng("W", a->W, (size_t)kD * kD * 2, false),
        rng("conv_w", a->conv_w, (size_t)kD * kTaps * 2, false),
        rng("h", a->h, act, false),
        rng("out", a->out, act, true),
        rng("hist_ids", a->hist_ids, S * 8ull, true),
        rng("hist_len", a->hist_len, S * 4ull, true),
        rng("conv_state", a->conv_state, (size_t)S * 3 * kD * 4, true),
        rng("workspace", a->workspace, L.total, true),
        rng("dev_err", a->dev_err, 4, true),
        rng("row_ids_out", a->row_ids_out, (size_t)T * ids_per_token(heads) * 4, true),
        rng("x_out", a->x_out, act, true),
        rng("e_out", a->e_out, (size_t)T * kD * 4, true),
        rng("gate_out", a->gate_out, T * 4, true),
        rng("y_out", a->y_out, (size_t)T * kD * 4, true),
    };
    if (int st = check_alias(r, (int)(sizeof r / sizeof r[0]))) return st;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(a->workspace);
    int32_t* row_ids = a->row_ids_out ? a->row_ids_out : reinterpret_cast<int32_t*>(ws + L.row_ids);
    uint16_t* x = a->x_out ? a->x_out : reinterpret_cast<uint16_t*>(ws + L.x);
    uint16_t* e16 = reinterpret_cast<uint16_t*>(ws + L.e16);
    float* snap = reinterpret_cast<float*>(ws + L.snap);

    auto mark = [&](int i) -> hipError_t {
        return events ? hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s) : hipSuccess;
    };
    if (!from_x && !heads && !nv_blocks && !staged && decode_one_launch(T, S)) {
        // a short call: IDs, gather, projection and fuse in one launch (the
        // profiling events then put the whole kernel in the projection stage).
        // In place, the projection blocks copy h into the x region, which
        // this path does not otherwise use
        DecodeArgs d{};
        d.tokens = a->tokens;
        d.T = T;
        d.cu = a->cu_seqlens;
        d.S = S;
        d.vocab = a->vocab_size;
        d.hist_ids = a->hist_ids;
        d.hist_len = a->hist_len;
        d.table = a->table;
        d.scales = a->scales;
        d.R = a->R;
        d.W = a->W;
        d.conv_w = a->conv_w;
        d.h = a->h;
        d.out = a->out;
        d.hw = a->out == a->h ? reinterpret_cast<uint16_t*>(ws + L.x) : nullptr;
        d.conv_state = a->conv_state;
        d.snap = snap;
        d.e16 = e16;
        d.sync = reinterpret_cast<uint32_t*>(ws + L.sync);
        d.eps = a->eps;
        d.dev_err = a->dev_err;
        d.row_ids_out = a->row_ids_out;
        d.x_out = a->x_out;
        d.e_out = a->e_out;
        d.gate_out = a->gate_out;
        d.y_out = a->y_out;
        for (int i = 0; i < 3; ++i)
            if (int st = hip_status(mark(i), "ple_forward: event record")) return st;
        if (int st = hip_status(launch_decode_step(d, s), "ple_forward: one-launch kernel")) return st;
        for (int i = 3; i < 5; ++i)
            if (int st = hip_status(mark(i), "ple_forward: event record")) return st;
        return ok();
    }
    hipError_t e = mark(0);
    if (int st = hip_status(e, "ple_forward: event record")) return st;
    // short calls: the gather computes the IDs (one launch instead of two;
    // the ID stage's event pair then brackets nothing)
    const bool ids_in_gather = !from_x && T <= kIdsInGatherMaxT;
    // the fuse's block size decides which sequences' carried state is copied
    const int64_t pb = fuse_block_tokens(T, S);
    if (from_x) {
        x = const_cast<uint16_t*>(x_in);  // read only from here on
        e = launch_state_copy(a->conv_state, snap, a->cu_seqlens, S, pb, s);
        if (int st = hip_status(e, "ple_forward_x: state copy launch")) return st;
    } else if (!ids_in_gather) {
        e = launch_hash(a->tokens, T, a->cu_seqlens, S, a->hist_ids, a->hist_len, a->vocab_size,
                        a->R, row_ids, a->dev_err, a->conv_state, snap, pb, heads, s);
        if (int st = hip_status(e, "ple_forward: hash launch")) return st;
    }
    if (int st = hip_status(mark(1), "ple_forward: event record")) return st;
    if (ids_in_gather) {
        const IdSource src{a->tokens, a->cu_seqlens, S, a->hist_ids, a->hist_len, a->vocab_size,
                           a->row_ids_out, a->conv_state, snap, pb};
        e = launch_gather_ids(src, heads ? kLayoutHeads : nv_blocks ? kLayoutNvfp4 : kLayoutFp8, T, a->table,
                              nv_blocks, a->scales, a->R, x, a->dev_err, s);
        if (int st = hip_status(e, "ple_forward: gather launch")) return st;
    } else if (!from_x) {
        e = nv_blocks ? launch_gather_nvfp4(row_ids, T, a->table, nv_blocks, a->scales, a->R, x, nullptr,
                                            a->dev_err, s)
            : heads   ? launch_gather_heads(row_ids, T, a->table, a->scales, a->R, x, nullptr, a->dev_err, s)
                      : launch_gather(row_ids, T, a->table, a->scales, a->R, x, nullptr, a->dev_err, s);
        if (int st = hip_status(e, "ple_forward: gather launch")) return st;
    }
    if (int st = hip_status(mark(2), "ple_forward: event record")) return st;
    e = launch_proj(x, T, a->W, a->e_out, e16, s);
    if (int st = hip_status(e, "ple_forward: projection launch")) return st;
    if (int st = hip_status(mark(3), "ple_forward: event record")) return st;
    e = launch_fuse(a->h, e16, T, a->cu_seqlens, S, a->tokens, a->conv_w, snap, a->conv_state,
                    a->hist_ids, a->hist_len, a->out, a->eps, a->gate_out, a->y_out,
                    reinterpret_cast<uint16_t*>(ws + L.x), s);
    if (int st = hip_status(e, "ple_forward: fuse launch")) return st;
    if (int st = hip_status(mark(4), "ple_forward: event record")) return st;
    return ok();
}

static int check_events(void* const* events) {
    if (!events) return fail(PLE_ERR_NULL, "profiled forward: events is NULL");
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return fail(PLE_ERR_NULL, "profiled forward: events[%d] is NULL", i);
    return PLE_OK;
}

extern "C" {

int ple_forward(const ple_forward_args* a, void* stream) { return forward_impl(a, stream, nullptr, false); }

int ple_forward_staged(const ple_forward_args* a, void* stream) {
    return forward_impl(a, stream, nullptr, false, nullptr, nullptr, true);
}

int ple_forward_profiled(const ple_forward_args* a, void* stream, void* const* events) {
    if (int st = check_events(events)) return st;
    return forward_impl(a, stream, events, false);
}

int ple_forward_heads(const ple_forward_args* a, void* stream) {
    return forward_impl(a, stream, nullptr, true);
}

int ple_forward_heads_profiled(const ple_forward_args* a, void* stream, void* const* events) {
    if (int st = check_events(events)) return st;
    return forward_impl(a, stream, events, true);
}

int ple_forward_nvfp4(const ple_forward_args* a, const uint8_t* blocks, void* stream) {
    if (!blocks) return fail(PLE_ERR_NULL, "ple_forward_nvfp4: blocks is NULL");
    if (!aligned(blocks, 4)) return fail(PLE_ERR_ALIGN, "ple_forward_nvfp4: blocks is not 4-byte aligned");
    return forward_impl(a, stream, nullptr, false, nullptr, blocks);
}

int ple_forward_nvfp4_profiled(const ple_forward_args* a, const uint8_t* blocks, void* stream,
                               void* const* events) {
    if (int st = check_events(events)) return st;
    if (!blocks) return fail(PLE_ERR_NULL, "ple_forward_nvfp4: blocks is NULL");
    if (!aligned(blocks, 4)) return fail(PLE_ERR_ALIGN, "ple_forward_nvfp4: blocks is not 4-byte aligned");
    return forward_impl(a, stream, events, false, nullptr, blocks);
}

int ple_forward_x(const ple_forward_args* a, const uint16_t* x_bf16, void* stream) {
    if (!x_bf16) return fail(PLE_ERR_NULL, "ple_forward_x: x is NULL");
    return forward_impl(a, stream, nullptr, false, x_bf16);
}

}  // extern "C"

// ---- ple_forward_noalloc: the workspace in a static device array ----------
//
// For callers that cannot allocate device memory. The workspace of a call of
// up to kNoAllocMaxT tokens and kNoAllocMaxS sequences lives in `scratch`, a
// file-scope device array that each GPU the library runs on holds until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept in g_scratch. Every call on one GPU shares that GPU's array; the
// kernels write each region before reading it, so nothing has to start at
// zero, and calls that overlap on one GPU (on different streams, or from
// different threads without ordering) race on it.
namespace {
constexpr int64_t kNoAllocMaxT = 2048;
constexpr int32_t kNoAllocMaxS = 256;
constexpr size_t kScratchBytes = layout(kNoAllocMaxT, kNoAllocMaxS, false).total;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// device address of this device's scratch (looked up on the first call)
static int scratch_ptr(void** out) {
    int dev = 0;
    if (int st = hip_status(hipGetDevice(&dev), "ple_forward_noalloc: hipGetDevice")) return st;
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PLE_ERR_HIP, "ple_forward_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (int st = hip_status(e, "ple_forward_noalloc: hipGetSymbolAddress(scratch)")) return st;
        if (!p) return fail(PLE_ERR_HIP, "ple_forward_noalloc: no device address for the scratch array");
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PLE_OK;
}

extern "C" {

size_t ple_forward_noalloc_max_tokens(void) { return (size_t)kNoAllocMaxT; }

size_t ple_forward_noalloc_max_sequences(void) { return (size_t)kNoAllocMaxS; }

int ple_forward_noalloc(const ple_forward_args* a, void* stream) {
    if (!a) return fail(PLE_ERR_NULL, "ple_forward_noalloc: args is NULL");
    if (a->T > kNoAllocMaxT || a->S > kNoAllocMaxS)
        return fail(PLE_ERR_SHAPE, "ple_forward_noalloc: T = %lld, S = %d beyond its limits (T <= %lld, S <= %d)",
                    (long long)a->T, a->S, (long long)kNoAllocMaxT, kNoAllocMaxS);
    if (a->workspace || a->workspace_bytes)
        return fail(PLE_ERR_WORKSPACE, "ple_forward_noalloc: workspace must be NULL and workspace_bytes 0 "
                                       "(the call uses the library's own scratch)");
    void* ws = nullptr;
    if (int st = scratch_ptr(&ws)) return st;
    ple_forward_args b = *a;
    b.workspace = ws;
    b.workspace_bytes = kScratchBytes;
    return forward_impl(&b, stream, nullptr, false);
}

}  // extern "C"
