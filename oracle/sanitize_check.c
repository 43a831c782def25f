/* Sanitizer run of the CPU oracle — TEST INFRASTRUCTURE ONLY.
 *
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer (oracle/build.py,
 * sanitize=True) and run by the CPU tests: every function of ple_oracle.c is
 * called on small inputs that reach its edge cases (empty sequences, one- and
 * two-token chunks, history lengths 0..2, missing rows, R = 1, special
 * floating-point values, several thread counts), so that any out-of-bounds
 * access, use of uninitialized or freed memory, or undefined arithmetic stops
 * the run. Alongside, invariants that hold by the definition are checked
 * (chunked equals unchunked for IDs, history and conv state; W = I gives
 * e = x; e = 0 gives g = 1/2; results independent of the thread count), so
 * the calls are meaningful, not just executed. The value pins themselves are
 * the Python tests, which also run against a UBSan build of the library. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define D 2560

int oracle_num_threads(void);
void oracle_set_num_threads(int n);
uint64_t oracle_mix64(uint64_t z);
uint64_t oracle_key2(uint32_t a, uint32_t b);
uint64_t oracle_key3(uint32_t a, uint32_t b, uint32_t c);
void oracle_ngram_ids(const int32_t* tokens, const int32_t* cu, int32_t S, const int32_t* hist_ids,
                      const int32_t* hist_len, int64_t R, int32_t* row_ids);
uint64_t oracle_head_mix(uint64_t key, int32_t head);
void oracle_ngram_ids_heads(const int32_t* tokens, const int32_t* cu, int32_t S, const int32_t* hist_ids,
                            const int32_t* hist_len, int64_t R, int32_t* row_ids);
void oracle_hist_update(const int32_t* tokens, const int32_t* cu, int32_t S, const int32_t* hist_ids,
                        const int32_t* hist_len, int32_t* hist_ids_out, int32_t* hist_len_out);
double oracle_e4m3_value(uint8_t b);
uint16_t oracle_bf16_rne(float f);
double oracle_bf16_value(uint16_t b);
void oracle_gather_dequant(const int32_t* row_ids, int64_t T, const uint8_t* table, const float* scales,
                           uint16_t* x, uint8_t* raw);
double oracle_e2m1_value(uint8_t code);
void oracle_gather_dequant_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes,
                                 const uint8_t* blocks, const float* scales, uint16_t* x, uint8_t* raw);
void oracle_gather_dequant_heads(const int32_t* idx, int64_t T, const uint8_t* slices, const float* scales,
                                 uint16_t* x, uint8_t* raw);
void oracle_project(const uint16_t* x, int64_t T, const uint16_t* W, double* e);
void oracle_round_bf16(const double* in, int64_t n, double* out);
void oracle_gate(const uint16_t* h, const double* e, int64_t T, double eps, double* g);
void oracle_conv_fuse(const uint16_t* h, const double* e, const double* g, int64_t T, const int32_t* cu,
                      int32_t S, const uint16_t* conv_w, const double* state, double* y, double* out,
                      double* state_out);

static int failures = 0;
#define CHECK(cond, what)                                     \
    do {                                                      \
        if (!(cond)) {                                        \
            fprintf(stderr, "check failed: %s\n", what);      \
            ++failures;                                       \
        }                                                     \
    } while (0)

static uint64_t rng_state = 0x5EED;
static uint32_t rnd(uint32_t n) {  /* xorshift64*, test data only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1DULL) >> 33) % n;
}
static uint16_t bf16_of(double v) { return oracle_bf16_rne((float)v); }
static double urand(void) { return (double)rnd(1u << 24) / (1u << 23) - 1.0; }
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

/* IDs and history: the whole sequence in one call equals it cut in pieces
 * of 0, 1, 2, 3 and more tokens, each piece carrying the history */
static void check_ids_and_history(void) {
    const int N = 23, R_list[3] = {1, 3, 1000003};
    int32_t toks[23];
    for (int i = 0; i < N; ++i) toks[i] = (int32_t)rnd(248320);
    for (int ri = 0; ri < 3; ++ri) {
        int64_t R = R_list[ri];
        int32_t cu_all[2] = {0, N}, hz[2] = {0, 0}, hl0 = 0;
        int32_t* all = xmalloc(sizeof(int32_t) * 2 * N);
        int32_t* allh = xmalloc(sizeof(int32_t) * 16 * N);
        oracle_ngram_ids(toks, cu_all, 1, hz, &hl0, R, all);
        oracle_ngram_ids_heads(toks, cu_all, 1, hz, &hl0, R, allh);
        CHECK(all[0] == -1 && all[1] == -1 && all[3] == -1 && all[2] >= 0, "missing history gives -1");
        for (int h = 0; h < 16; ++h) CHECK(allh[h] == -1, "token 0 has no head row");
        const int cuts[8] = {0, 1, 2, 0, 3, 1, 7, 9};  /* sums to 23 */
        int32_t hid[2] = {0, 0}, hln = 0, pos = 0;
        for (int k = 0; k < 8; ++k) {
            int L = cuts[k];
            int32_t cu[2] = {0, L};
            int32_t* part = xmalloc(sizeof(int32_t) * 2 * (L ? L : 1));
            int32_t* parth = xmalloc(sizeof(int32_t) * 16 * (L ? L : 1));
            oracle_ngram_ids(toks + pos, cu, 1, hid, &hln, R, part);
            oracle_ngram_ids_heads(toks + pos, cu, 1, hid, &hln, R, parth);
            CHECK(memcmp(part, all + 2 * pos, sizeof(int32_t) * 2 * L) == 0, "chunked IDs");
            CHECK(memcmp(parth, allh + 16 * pos, sizeof(int32_t) * 16 * L) == 0, "chunked head IDs");
            for (int t = 0; t < L; ++t)
                for (int j = 0; j < 2; ++j) CHECK(part[2 * t + j] >= -1 && part[2 * t + j] < R, "ID range");
            int32_t hid2[2], hln2;
            oracle_hist_update(toks + pos, cu, 1, hid, &hln, hid2, &hln2);
            hid[0] = hid2[0];
            hid[1] = hid2[1];
            hln = hln2;
            pos += L;
            free(part);
            free(parth);
        }
        CHECK(pos == N && hln == 2 && hid[0] == toks[N - 2] && hid[1] == toks[N - 1], "history after the pieces");
        free(all);
        free(allh);
    }
    /* several sequences in one call, including empty ones and every history length */
    int32_t toks2[6] = {5, 6, 7, 8, 9, 10}, cu[6] = {0, 0, 1, 3, 3, 6};
    int32_t hid[10] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 11}, hln[5] = {2, 1, 0, 2, 1}, ids[12], hid2[10], hln2[5];
    oracle_ngram_ids(toks2, cu, 5, hid, hln, 97, ids);
    oracle_hist_update(toks2, cu, 5, hid, hln, hid2, hln2);
    CHECK(hln2[0] == 2 && hid2[0] == 1 && hid2[1] == 2, "empty sequence keeps its history");
    CHECK(hln2[1] == 2 && hid2[2] == 4 && hid2[3] == 5, "one token after one of history");
    CHECK(hln2[2] == 2 && hid2[4] == 6 && hid2[5] == 7, "two fresh tokens");
    CHECK(oracle_key2(1, 2) != oracle_key3(0, 1, 2), "bigram and trigram keys differ");
    CHECK(oracle_head_mix(12345, 0) == oracle_mix64(12345) && oracle_head_mix(12345, 8) == oracle_mix64(12345),
          "heads 0 and 8 are the plain finalizer");
}

/* gathers of the three layouts with present and missing rows */
static void check_gathers(void) {
    const int n = 5, T = 4;
    uint8_t* table = xmalloc((size_t)n * D);
    float scales[5];
    for (int i = 0; i < n * D; ++i) table[i] = (uint8_t)rnd(256);
    for (int i = 0; i < n; ++i) scales[i] = 0.01f * (float)(i + 1);
    for (int c = 0; c < 256; ++c) {
        double v = oracle_e4m3_value((uint8_t)c);
        CHECK((isnan(v) != 0) == ((c & 0x7F) == 0x7F), "E4M3 NaN codes");
    }
    for (int c = 0; c < 16; ++c) CHECK(!isnan(oracle_e2m1_value((uint8_t)c)), "E2M1 values are finite");
    int32_t ids[8] = {-1, -1, 0, -1, -1, 4, 2, 2};
    uint16_t* x = xmalloc(sizeof(uint16_t) * T * D);
    uint8_t* raw = xmalloc((size_t)T * 2 * D);
    oracle_gather_dequant(ids, T, table, scales, x, raw);
    for (int c = 0; c < D; ++c) CHECK(x[c] == 0 && raw[c] == 0 && raw[D + c] == 0, "no rows: zeros");
    CHECK(memcmp(raw + 2 * D, table, D) == 0, "raw bytes of a present row");
    oracle_gather_dequant(ids, T, table, scales, x, NULL);
    /* NVFP4 rows: 1280 code bytes and 160 block scales per row */
    uint8_t* codes = xmalloc((size_t)n * D / 2);
    uint8_t* blocks = xmalloc((size_t)n * D / 16);
    for (int i = 0; i < n * D / 2; ++i) codes[i] = (uint8_t)rnd(256);
    for (int i = 0; i < n * D / 16; ++i) blocks[i] = (uint8_t)(0x28 + rnd(32));
    uint8_t* raw4 = xmalloc((size_t)T * D);
    oracle_gather_dequant_nvfp4(ids, T, codes, blocks, scales, x, raw4);
    for (int c = 0; c < D; ++c) CHECK(x[c] == 0, "NVFP4: no rows, zeros");
    /* 16-lookup layout: 160-byte slices */
    uint8_t* slices = xmalloc((size_t)n * 160);
    memcpy(slices, table, (size_t)n * 160);
    int32_t* hidx = xmalloc(sizeof(int32_t) * 16 * T);
    for (int i = 0; i < 16 * T; ++i) hidx[i] = (int32_t)rnd(n + 1) - 1;
    uint8_t* rawh = xmalloc((size_t)T * 16 * 160);
    oracle_gather_dequant_heads(hidx, T, slices, scales, x, rawh);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < 16; ++h)
            if (hidx[16 * t + h] < 0)
                for (int j = 0; j < 160; ++j) CHECK(x[(size_t)t * D + 160 * h + j] == 0, "missing head row: zeros");
    free(table); free(x); free(raw); free(codes); free(blocks); free(raw4); free(slices); free(hidx); free(rawh);
}

/* projection, rounding, gate and conv on a few tokens */
static void check_dense_steps(void) {
    const int T = 7;
    uint16_t* x = xmalloc(sizeof(uint16_t) * T * D);
    uint16_t* W = xmalloc(sizeof(uint16_t) * D * D);
    double* e = xmalloc(sizeof(double) * T * D);
    double* e1 = xmalloc(sizeof(double) * T * D);
    for (int i = 0; i < T * D; ++i) x[i] = bf16_of(urand());
    memset(W, 0, sizeof(uint16_t) * D * D);
    for (int i = 0; i < D; ++i) W[(size_t)i * D + i] = bf16_of(1.0);
    oracle_project(x, T, W, e);
    for (int i = 0; i < T * D; ++i) CHECK(e[i] == oracle_bf16_value(x[i]), "W = I gives e = x");
    for (int i = 0; i < D * D; ++i) W[i] = bf16_of(urand() / 50.0);
    int threads = oracle_num_threads();
    oracle_set_num_threads(1);
    oracle_project(x, T, W, e1);
    oracle_set_num_threads(threads > 1 ? threads : 4);
    oracle_project(x, T, W, e);
    oracle_set_num_threads(threads);
    CHECK(memcmp(e, e1, sizeof(double) * T * D) == 0, "projection independent of the thread count");
    oracle_project(x, 0, W, e);   /* an empty call touches nothing */

    double special[10] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e-45, -3e-39, 3.4e38, 1.0 + 1.0 / 256, 6.5e38};
    double rs[10];
    oracle_round_bf16(special, 10, rs);
    CHECK(rs[0] == 0.0 && signbit(rs[1]) && isinf(rs[2]) && isnan(rs[4]) && isinf(rs[9]), "rounding specials");

    uint16_t* h = xmalloc(sizeof(uint16_t) * T * D);
    for (int i = 0; i < T * D; ++i) h[i] = bf16_of(urand());
    double* g = xmalloc(sizeof(double) * T);
    double* ez = xmalloc(sizeof(double) * T * D);
    memset(ez, 0, sizeof(double) * T * D);
    oracle_gate(h, ez, T, 1e-6, g);
    for (int t = 0; t < T; ++t) CHECK(g[t] == 0.5, "e = 0 gives g = 1/2");
    oracle_round_bf16(e, (int64_t)T * D, e1);
    oracle_gate(h, e1, T, 1e-6, g);
    for (int t = 0; t < T; ++t) CHECK(g[t] > 0.0 && g[t] < 1.0, "gate in (0, 1)");

    /* conv: one call over 7 tokens equals pieces of 0, 1, 2 and 4 tokens
     * carrying the state */
    uint16_t cw[4 * D];
    for (int i = 0; i < 4 * D; ++i) cw[i] = bf16_of(urand());
    double* state = xmalloc(sizeof(double) * 3 * D);
    for (int i = 0; i < 3 * D; ++i) state[i] = urand();
    double* y = xmalloc(sizeof(double) * T * D);
    double* out = xmalloc(sizeof(double) * T * D);
    double* st_all = xmalloc(sizeof(double) * 3 * D);
    int32_t cu_all[2] = {0, T};
    oracle_conv_fuse(h, e1, g, T, cu_all, 1, cw, state, y, out, st_all);
    double* st = xmalloc(sizeof(double) * 3 * D);
    double* st2 = xmalloc(sizeof(double) * 3 * D);
    memcpy(st, state, sizeof(double) * 3 * D);
    const int cuts[4] = {0, 1, 2, 4};
    int pos = 0;
    for (int k = 0; k < 4; ++k) {
        int L = cuts[k];
        int32_t cu[2] = {0, L};
        double* yp = xmalloc(sizeof(double) * (L ? L : 1) * D);
        double* op = xmalloc(sizeof(double) * (L ? L : 1) * D);
        oracle_conv_fuse(h + (size_t)pos * D, e1 + (size_t)pos * D, g + pos, L, cu, 1, cw, st, yp, op, st2);
        CHECK(memcmp(yp, y + (size_t)pos * D, sizeof(double) * L * D) == 0, "chunked conv equals unchunked");
        memcpy(st, st2, sizeof(double) * 3 * D);
        pos += L;
        free(yp);
        free(op);
    }
    CHECK(memcmp(st, st_all, sizeof(double) * 3 * D) == 0, "conv state after the pieces");
    /* an empty sequence between two others keeps its state */
    int32_t cu3[4] = {0, 3, 3, 7};
    double* state3 = xmalloc(sizeof(double) * 9 * D);
    double* state3o = xmalloc(sizeof(double) * 9 * D);
    for (int i = 0; i < 9 * D; ++i) state3[i] = urand();
    oracle_conv_fuse(h, e1, g, T, cu3, 3, cw, state3, y, out, state3o);
    CHECK(memcmp(state3 + 3 * D, state3o + 3 * D, sizeof(double) * 3 * D) == 0, "empty sequence keeps its state");
    free(x); free(W); free(e); free(e1); free(h); free(g); free(ez); free(state); free(y); free(out);
    free(st_all); free(st); free(st2); free(state3); free(state3o);
}

int main(void) {
    check_ids_and_history();
    check_gathers();
    check_dense_steps();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
