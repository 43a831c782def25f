/* libple — MI355X (gfx950) PLE n-gram embedding lookup, C ABI.
 *
 * The operation (Qwen3.8-Flash-Next pages):
 *  - mengman.github.io "【Qwen3.8-Flash-Next 端侧部署】01-模型架构与整体方案",
 *    section "n-gram embedding 是一条附加的条件记忆路径": the engine keeps token IDs,
 *    positions and sequence boundaries, computes n-gram IDs from them, reads
 *    the vectors from the large table, then dequantizes, projects, gates and
 *    short-convolves them and fuses the result into the hidden states; the
 *    IDs and the table reads need no hidden state.
 *  - reactapp.top "在配备 RTX 3090 的设备上，通过 llama.cpp 张量卸载技术运行
 *    Qwen3.8-Flash-Next", section "n-gram表格": the rows are keyed by hashed
 *    recent tokens (about 20 M bigram and trigram rows) and depend only on the
 *    input text.
 *  - bittide.aicompass.dev copy of the "Qwen3.8-Flash-Next-NVFP4-SSD-Stream"
 *    model card, sections "模型简介" and "技术细节": the table is FP8.
 *  - kipfel.ltd "Qwen3.8-Flash-Next-Uncensored in NVIDIA Jetson AGX Thor",
 *    section 2: hidden size 2560, vocabulary 248,320; section 5: the n-gram
 *    ID lookup and the PLE short conv are separate graph-splitting ops.
 *
 * Readings fixed by this library where the pages are silent:
 *  - row IDs: bigram  r2 = mix64((2<<60)|(a<<20)|b) mod R,
 *             trigram r3 = mix64((3<<60)|(a<<40)|(b<<20)|c) mod R,
 *    mix64 = SplitMix64 finalizer, unsigned 64-bit mod; -1 when the sequence
 *    (history + chunk) has too few tokens; a missing row contributes zero.
 *  - x = bf16_rne(fl32(fl32(dec(code_r2)*scale[r2]) + fl32(dec(code_r3)*scale[r3])))
 *    with dec = OCP FP8 E4M3FN decode and one fp32 scale per row.
 *  - e = bf16_rne(x W^T), W bf16 [2560 out][2560 in], fp32 accumulation: the
 *    projection is a bf16 layer (outside the routed experts the model's
 *    weights are BF16, the table FP8: bittide model card copy, "模型简介"),
 *    and the gate and the conv read its bf16 output.
 *  - g = sigmoid(<h/rms(h), e/rms(e)> / sqrt(2560)), rms(z) = sqrt(mean(z^2) + eps).
 *  - v = g e; y[t][c] = sum_{k=0..3} conv_w[c][k] v[t-3+k][c] (causal,
 *    depthwise, conv_w[c][3] on the current token, v before a sequence's
 *    first token taken from conv_state, oldest first); out = bf16_rne(h + y).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller. libple
 *    never allocates, frees, keeps a pointer past return, or synchronizes;
 *    it enqueues work only on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream). Stateful buffers are read and written in
 *    stream order.
 *  - bf16 arrays are passed as uint16_t bit patterns.
 *  - Return value: PLE_OK (0) or a negative ple_status. Every error that the
 *    host can detect (NULL pointer, bad size, misalignment, overlap, small
 *    workspace) is reported BEFORE anything is enqueued, so outputs and state
 *    are untouched. Data-dependent errors are detected on the device: the
 *    kernels OR a PLE_DEVERR_* bit into *dev_err (optional, may be NULL);
 *    outputs of the affected tokens are then unspecified but every access
 *    stays in bounds.
 *  - T = 0 is valid and enqueues nothing.
 *  - Thread-safe; the only global state is a thread-local error message, a
 *    per-device flag recording that the projection kernels' LDS size has
 *    been set (set once, under an atomic) and, for ple_forward_noalloc only,
 *    a per-device device array and its address (see that call).
 */
#ifndef PLE_H
#define PLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLE_D 2560          /* row width = hidden size */
#define PLE_CONV_TAPS 4     /* short-conv kernel size */
#define PLE_MAX_VOCAB (1 << 20)

typedef enum ple_status {
    PLE_OK = 0,
    PLE_ERR_NULL = -1,       /* a required pointer is NULL */
    PLE_ERR_SHAPE = -2,      /* T < 0 or (with cu_seqlens) T > 2^31-1, S < 1, sizes inconsistent */
    PLE_ERR_RANGE = -3,      /* R outside [1, 2^31-1], vocab outside [1, 2^20], eps < 0 */
    PLE_ERR_ALIGN = -4,      /* a pointer lacks the alignment stated below */
    PLE_ERR_ALIAS = -5,      /* an output overlaps another argument (out == h excepted) */
    PLE_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than ple_forward_workspace_size */
    PLE_ERR_HIP = -7         /* a HIP launch failed */
} ple_status;

/* Bits OR-ed into *dev_err by the kernels. */
#define PLE_DEVERR_TOKEN_RANGE 1  /* a token outside [0, vocab_size) */
#define PLE_DEVERR_CU_SEQLENS 2   /* cu_seqlens[0] != 0, decreasing, or cu_seqlens[S] != T */
#define PLE_DEVERR_HIST_LEN 4     /* hist_len[s] outside {0, 1, 2} (treated as 0) */
#define PLE_DEVERR_ROW_RANGE 8    /* ple_lookup: a row id outside [-1, R) (treated as -1) */
#define PLE_DEVERR_SYNC 16        /* one-launch path: its counters in the workspace were not zero at
                                     the call, or a wait passed its limit (outputs unspecified) */

/* a1 — n-gram row IDs (mengman page, "n-gram embedding" section: IDs from
 * token IDs, positions and sequence boundaries; reactapp page, "n-gram表格":
 * hashed bigrams and trigrams).
 *   tokens     int32 [T]          token IDs of this chunk, sequences concatenated
 *   cu_seqlens int32 [S+1]        sequence s = tokens[cu[s] .. cu[s+1]); cu[0]=0, cu[S]=T
 *   hist_ids   int32 [S][2]       carried history, most recent in slot 1
 *   hist_len   int32 [S]          number of valid history IDs (0, 1 or 2),
 *                                 right-aligned in hist_ids[s]
 *   vocab_size                    tokens must lie in [0, vocab_size), vocab_size <= 2^20
 *   R                             table rows, 1 <= R <= 2^31-1
 *   row_ids    int32 [T][2]  out  [t][0] bigram row, [t][1] trigram row, -1 if missing
 * Does not update hist_ids / hist_len. Alignment: 4 bytes (row_ids: 8 bytes). */
int ple_hash(const int32_t* tokens, int64_t T, const int32_t* cu_seqlens, int32_t S,
             const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab_size, int64_t R,
             int32_t* row_ids, int32_t* dev_err, void* stream);

/* a2 — gather + dequantize (mengman page, "n-gram embedding" section: read
 * the vectors, dequantize; bittide model card, "技术细节": FP8 rows).
 *   row_ids int32 [T][2]            rows to sum per token, -1 = none
 *   table   uint8 [R][2560]         E4M3FN codes, row-major; 16-byte aligned
 *   scales  float [R]               one scale per row
 *   x_bf16  uint16 [T][2560]   out  x (formula above); 16-byte aligned
 *   raw_opt uint8 [T][2][2560] out  optional (NULL to skip): the two rows'
 *                                   bytes, zero-filled for -1; 16-byte aligned
 * row_ids must be 8-byte aligned. Row ids outside [-1, R) are treated as -1
 * and flagged PLE_DEVERR_ROW_RANGE. */
int ple_lookup(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
               int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err, void* stream);

/* a3 — projection alone (mengman page, "n-gram embedding" section: 投影):
 *   x bf16 [T][2560], W bf16 [2560][2560] (W[out][in]) -> e float [T][2560],
 *   e = x W^T with fp32 accumulation. All pointers 16-byte aligned. */
int ple_proj(const uint16_t* x_bf16, int64_t T, const uint16_t* W_bf16, float* e, void* stream);

/* a1..a4 — the whole path for one chunk of S sequences (mengman page,
 * "n-gram embedding" section: IDs -> table read -> dequantize -> project ->
 * gate -> short conv -> fuse with the hidden states). */
typedef struct ple_forward_args {
    const int32_t* tokens;      /* int32 [T] */
    int64_t T;
    const int32_t* cu_seqlens;  /* int32 [S+1] */
    int32_t S;
    int32_t vocab_size;
    const uint8_t* table;       /* uint8 [R][2560] E4M3FN, 16-byte aligned */
    const float* scales;        /* float [R] */
    int64_t R;
    const uint16_t* W;          /* bf16 [2560][2560], W[out][in], 16-byte aligned */
    const uint16_t* conv_w;     /* bf16 [2560][4], 16-byte aligned */
    const uint16_t* h;          /* bf16 [T][2560] hidden states in, 16-byte aligned */
    uint16_t* out;              /* bf16 [T][2560] out; may equal h (in place: the h rows other
                                   blocks overwrite are first copied into the workspace),
                                   16-byte aligned; any partial overlap is rejected */
    int32_t* hist_ids;          /* int32 [S][2] in/out */
    int32_t* hist_len;          /* int32 [S] in/out */
    float* conv_state;          /* float [S][3][2560] in/out, last three v, oldest first; 16-byte aligned */
    void* workspace;            /* device scratch, >= ple_forward_workspace_size(T, S) bytes, 256-byte aligned;
                                   its first 256 bytes must be zero before the first call on it (see below) */
    size_t workspace_bytes;
    int32_t* dev_err;           /* optional */
    float eps;                  /* RMSNorm epsilon (>= 0), 1e-6 by convention */
    /* optional debug outputs, NULL to skip */
    int32_t* row_ids_out;       /* int32 [T][2], 8-byte aligned */
    uint16_t* x_out;            /* bf16 [T][2560] */
    float* e_out;               /* float [T][2560], projection accumulators before the bf16 rounding */
    float* gate_out;            /* float [T] */
    float* y_out;               /* float [T][2560], conv output before the residual add */
} ple_forward_args;

/* After the call: hist_ids/hist_len hold the last min(2, hist_len + L) IDs of
 * each sequence, conv_state the last three v (an empty sequence keeps its
 * state). Everything runs on `stream`; nothing is synchronized.
 *
 * Short calls (ple_forward_one_launch(T, S): up to 16 tokens and 256
 * sequences) run as ONE kernel launch: projection blocks and one finisher
 * block per token, ordered through three counters in the first 256 bytes of
 * the workspace (in place, the projection blocks also copy h into the
 * workspace, where the finishers read the earlier tokens' rows) (decode steps split into separate launches cannot
 * hide the table reads: mengman.github.io "Qwen3.8-Flash-Next 端侧部署 01",
 * inference-flow section; kipfel.ltd Thor article, section "五、启动参数").
 * Those bytes must be zero before the first call on a workspace; every call
 * leaves them zero and no other kernel writes them, so clearing the buffer
 * once when it is allocated suffices. Non-zero counters are flagged
 * PLE_DEVERR_SYNC. Calls that share a workspace must be ordered (one stream),
 * as for every other use of the workspace. Results equal the longer path's
 * bit for bit. */
int ple_forward(const ple_forward_args* args, void* stream);

/* 1 if ple_forward runs a T-token call of S sequences (FP8 table) as one
 * launch, else 0. Host-only, enqueues nothing. */
int ple_forward_one_launch(int64_t T, int32_t S);

/* ple_forward (the same operation, arguments, workspace, errors and results,
 * bit for bit) with every stage its own kernel launch at every call size:
 * the ID kernel (or IDs inside the gather for short calls), the gather, the
 * projection and the fuse, as ple_forward runs calls beyond
 * ple_forward_one_launch. For callers that want the stages as separate
 * launches, for instance to compare the two paths. */
int ple_forward_staged(const ple_forward_args* args, void* stream);

/* ple_forward with per-stage timing: the same launches on the same stream,
 * with events[0..4] (hipEvent_t, created by the caller) recorded before the
 * n-gram ID kernel and after the ID, gather/dequant, projection and
 * gate/conv/fuse kernels. Calls of up to 1024 tokens compute the IDs inside
 * the gather, so events[0] and events[1] then bracket no kernel; a
 * one-launch call records events[0..2] before its kernel and events[3..4]
 * after it. events may not be NULL. */
int ple_forward_profiled(const ple_forward_args* args, void* stream, void* const* events);

/* Workspace bytes ple_forward (and ple_forward_x) needs for up to max_T
 * tokens and max_S sequences. */
size_t ple_forward_workspace_size(int64_t max_T, int32_t max_S);

/* a3..a4 from rows gathered ahead: the IDs depend only on the tokens, so the
 * ID and table-read stages can run early, on another stream, before the
 * layer that needs them (SSD-streaming page, "技术细节" and the Spark
 * deployment page's scheduling section: rows are fetched ahead of the PLE
 * layer). x_bf16 (bf16 [T][2560], 16-byte aligned, read only) is the output
 * of ple_hash + ple_lookup (or their 16-lookup variants) for this chunk with
 * the history it had; this call runs the projection, gate, conv and fuse
 * exactly as ple_forward would and updates conv_state, hist_ids and
 * hist_len the same way. table, scales, R and vocab_size are not used;
 * row_ids_out and x_out must be NULL. Ordering x's producer before this call
 * (an event between the streams) is the caller's. */
int ple_forward_x(const ple_forward_args* args, const uint16_t* x_bf16, void* stream);

/* ---- The 16-lookup layout ------------------------------------------------
 * The SSD-streaming page's model card ("技术细节") speaks of 16 lookups of
 * 160-byte rows per token: the same 51,200,245,760-byte table read as 16
 * head tables of R = 20,000,096 rows x 160 bytes. Reading fixed by this
 * library where the pages are silent:
 *  - heads 0..7 take the bigram key, heads 8..15 the trigram key (same keys
 *    as above); head h's row = mix64(key + (h mod 8) * 0x9E3779B97F4A7C15)
 *    mod R, the h-th output of a SplitMix64 stream started at the key (heads
 *    0 and 8 equal ple_hash's two IDs); -1 when the n-gram is missing;
 *  - one fp32 scale per (head, row), scales[h][r];
 *  - x[t][160 h + j] = bf16_rne(fl32(dec(table[h][row_h][j]) * scales[h][row_h])),
 *    +0 for a missing head row. The projection, gate, conv and fuse are the
 *    same as above.
 * Error bits, ownership and stream rules are those of the two-lookup calls. */

/* a1, 16-lookup layout. As ple_hash, but
 *   row_ids int32 [T][16] out  [t][h] row of head h, -1 if missing; 16-byte aligned */
int ple_hash_heads(const int32_t* tokens, int64_t T, const int32_t* cu_seqlens, int32_t S,
                   const int32_t* hist_ids, const int32_t* hist_len, int32_t vocab_size, int64_t R,
                   int32_t* row_ids, int32_t* dev_err, void* stream);

/* a2, 16-lookup layout.
 *   row_ids int32 [T][16]             16-byte aligned
 *   table   uint8 [16][R][160]        E4M3FN codes (the same bytes as [R][2560]); 16-byte aligned
 *   scales  float [16][R]             one scale per head row
 *   x_bf16  uint16 [T][2560]     out  x (formula above); 16-byte aligned
 *   raw_opt uint8 [T][16][160]   out  optional: the 16 rows' bytes, zero for -1; 16-byte aligned
 * Row ids outside [-1, R) are treated as -1 and flagged PLE_DEVERR_ROW_RANGE. */
int ple_lookup_heads(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
                     int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err, void* stream);

/* a1..a4 in the 16-lookup layout: ple_forward with `table` read as
 * [16][R][160], `scales` as [16][R] (R = rows per head table), row_ids_out
 * (optional) as int32 [T][16] (16-byte aligned), and a workspace of
 * ple_forward_heads_workspace_size bytes. */
int ple_forward_heads(const ple_forward_args* args, void* stream);

/* ple_forward_heads with the five timing events of ple_forward_profiled. */
int ple_forward_heads_profiled(const ple_forward_args* args, void* stream, void* const* events);

/* Workspace bytes ple_forward_heads needs for up to max_T tokens and max_S sequences. */
size_t ple_forward_heads_workspace_size(int64_t max_T, int32_t max_S);

/* ---- NVFP4 table ------------------------------------------------------------
 * The Spark deployment's packed PLE table keeps 4-bit codes with an FP8
 * scale per group of 16 elements (26.82 GiB for the 51.2 G elements).
 * Reading fixed by this library: row r of R is
 *   codes  uint8 [R][1280]  OCP E2M1 codes, element 2k in the low nibble of byte k
 *   blocks uint8 [R][160]   E4M3FN scale of elements 16b .. 16b+15
 *   scales float [R]        one fp32 scale per row (as for the FP8 table)
 * and p = fl32(fl32(e2m1(code) * e4m3(block)) * scale) (the inner product is
 * exact); the bigram and trigram rows combine as in the FP8 table:
 * x = bf16_rne(fl32(p_bi + p_tri)), a missing row skipped. Row IDs, the
 * projection, gate, conv and fuse are those of ple_forward. */

/* a2 over the NVFP4 table.
 *   row_ids int32 [T][2]             8-byte aligned
 *   codes   uint8 [R][1280]          16-byte aligned
 *   blocks  uint8 [R][160]           4-byte aligned
 *   scales  float [R]
 *   x_bf16  uint16 [T][2560]    out  16-byte aligned
 *   raw_opt uint8 [T][2][1280]  out  optional: the two rows' code bytes, zero for -1
 * Row ids outside [-1, R) are treated as -1 and flagged PLE_DEVERR_ROW_RANGE. */
int ple_lookup_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes, const uint8_t* blocks,
                     const float* scales, int64_t R, uint16_t* x_bf16, uint8_t* raw_opt, int32_t* dev_err,
                     void* stream);

/* a1..a4 over the NVFP4 table: ple_forward with args->table = codes
 * [R][1280], args->scales = the row scales and `blocks` [R][160]; workspace
 * of ple_forward_workspace_size bytes. */
int ple_forward_nvfp4(const ple_forward_args* args, const uint8_t* blocks, void* stream);

/* ple_forward_nvfp4 with the five timing events of ple_forward_profiled. */
int ple_forward_nvfp4_profiled(const ple_forward_args* args, const uint8_t* blocks, void* stream,
                               void* const* events);

/* Which projection tiling ple_forward (and its variants) runs for a T-token
 * call: 0 none (T <= 0), 1 small-T (T <= 256: 16 or 32 features x 32-token
 * tiles, the k chain split over eight waves), 2 mid-size (T <= 3200: 128
 * tokens x 256 features), 3 256 x 256, 4 256 tokens x 320 features (chosen
 * over 3 when it needs fewer rounds of 256 blocks). All give the same bits.
 * Host-only, enqueues nothing; for labelling measurements. */
int ple_proj_tiling(int64_t T);

/* ---- One call that allocates nothing -----------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. ple_forward_noalloc is ple_forward (same arguments, kernels and
 * results, bit for bit) with args->workspace NULL and args->workspace_bytes 0:
 * its workspace is a device array inside the library, 28,852,480 bytes on
 * each GPU it runs on, held until the process ends, enough for a call of up
 * to ple_forward_noalloc_max_tokens() = 2048 tokens and
 * ple_forward_noalloc_max_sequences() = 256 sequences. Larger calls return
 * PLE_ERR_SHAPE before anything is enqueued; a non-NULL workspace returns
 * PLE_ERR_WORKSPACE. The call allocates and frees nothing (the array's device
 * address is looked up once per device, on the first call with that device
 * current). Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (two streams, or two threads without ordering) race and give
 * unspecified results; calls ordered on one stream are safe. The array starts
 * zeroed when the library is loaded, and the one-launch path's counters in
 * it are left zero by every call. */
int ple_forward_noalloc(const ple_forward_args* args, void* stream);
size_t ple_forward_noalloc_max_tokens(void);
size_t ple_forward_noalloc_max_sequences(void);

/* Static description of a status code. */
const char* ple_status_string(int status);

/* Message of the last error on the calling thread ("" if none). */
const char* ple_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PLE_H */
