/* CPU oracle of the PLE n-gram embedding path — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct definition of what the path computes,
 * used to check the HIP path. Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load it; the product path never does. It
 * shares no source with the HIP kernels.
 *
 * What the path computes, per token (Qwen3.8-Flash-Next pages):
 *  - n-gram IDs from the current token and the one or two before it, with
 *    sequence boundaries and carried history (mengman.github.io "Qwen3.8-
 *    Flash-Next 端侧部署 01", section "n-gram embedding 是一条附加的条件记忆路径";
 *    reactapp.top "...on RTX 3090s...", section "n-gram表格"): the table is
 *    keyed by hashed bigrams and trigrams of the recent tokens.
 *  - read the rows, dequantize, project, gate, short-convolve and fuse into
 *    the hidden state, in that order (mengman page, same section).
 *  - the table is FP8 (bittide model card copy, "模型简介").
 * The pages leave the hash, the row scale and the gate open; this file
 * follows the readings fixed for this library:
 *  - mix64 = SplitMix64 finalizer (Steele, Lea, Flood, OOPSLA 2014);
 *    bigram key (2<<60)|(a<<20)|b, trigram key (3<<60)|(a<<40)|(b<<20)|c;
 *    row = mix64(key) mod R (unsigned 64-bit); a missing n-gram (not enough
 *    history at a sequence start) has row -1 and contributes zero.
 *  - x = bf16_rne( fl32( fl32(dec(code_bi)*s_bi) + fl32(dec(code_tri)*s_tri) ) ),
 *    E4M3FN decode, one fp32 scale per row.
 *  - e = x W^T (W[out][in]), fp64 here. Outside the routed experts the
 *    model's weights are BF16 and only the table is FP8 (bittide model card
 *    copy, "模型简介"), so the projection is a bf16 layer whose output is the
 *    bf16 tensor e_b = bf16_rne(e) (one rounding from the exact value); the
 *    gate and the conv below act on e_b.
 *  - g = sigmoid( <h/rms(h), e_b/rms(e_b)> / sqrt(2560) ), rms(z) = sqrt(mean(z^2)+eps).
 *  - v = g e_b; y[t][c] = sum_{k=0..3} w[c][k] v[t-3+k][c] (causal depthwise,
 *    w[c][3] on the current token; v before a sequence start comes from the
 *    carried state, oldest first); out = h + y.
 * Floating point beyond the dequant step is fp64 throughout.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define D 2560
#define KTAPS 4

/* Threads the projection loop runs on (OpenMP), for reporting. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for later calls (each output element is still computed by one
 * thread in one fixed order, so results do not depend on the count). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* n-gram IDs                                                                */
/* ------------------------------------------------------------------------ */

/* SplitMix64 output mix (Steele, Lea & Flood 2014; Stafford's "Mix13"). */
uint64_t oracle_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t oracle_key2(uint32_t a, uint32_t b) {
    return (2ULL << 60) | ((uint64_t)a << 20) | (uint64_t)b;
}

uint64_t oracle_key3(uint32_t a, uint32_t b, uint32_t c) {
    return (3ULL << 60) | ((uint64_t)a << 40) | ((uint64_t)b << 20) | (uint64_t)c;
}

/* row_ids[t][0] = bigram row, row_ids[t][1] = trigram row, -1 when missing.
 * Sequence s covers tokens[cu[s] .. cu[s+1]); its history is the last
 * hist_len[s] entries of hist_ids[s][0..1] (most recent in slot 1). */
void oracle_ngram_ids(const int32_t* tokens, const int32_t* cu, int32_t S,
                      const int32_t* hist_ids, const int32_t* hist_len, int64_t R,
                      int32_t* row_ids) {
    for (int32_t s = 0; s < S; ++s) {
        int32_t start = cu[s], end = cu[s + 1];
        int32_t hl = hist_len[s];
        /* the sequence as seen by the hash: history then this chunk */
        int64_t n = hl + (end - start);
        for (int64_t j = hl; j < n; ++j) {
            int32_t t = start + (int32_t)(j - hl);
            /* Hs[j] */
#define HS(idx) ((idx) < hl ? hist_ids[2 * s + 2 - hl + (idx)] : tokens[start + (idx) - hl])
            uint32_t cur = (uint32_t)HS(j);
            int32_t bi = -1, tri = -1;
            if (j >= 1) {
                uint32_t p1 = (uint32_t)HS(j - 1);
                bi = (int32_t)(oracle_mix64(oracle_key2(p1, cur)) % (uint64_t)R);
                if (j >= 2) {
                    uint32_t p2 = (uint32_t)HS(j - 2);
                    tri = (int32_t)(oracle_mix64(oracle_key3(p2, p1, cur)) % (uint64_t)R);
                }
            }
#undef HS
            row_ids[2 * (int64_t)t + 0] = bi;
            row_ids[2 * (int64_t)t + 1] = tri;
        }
    }
}

/* The 16-lookup layout (the model card's 16 lookups of 160-byte rows per
 * token, SSD-streaming page, "技术细节"): the same table read as 16 head
 * tables of R rows x 160 bytes. Heads 0..7 hash the bigram, heads 8..15 the
 * trigram; head h's key is offset by (h mod 8) steps of SplitMix64's
 * increment before the same finalizer, i.e. the head-th output of a
 * SplitMix64 stream started at the key, so head 0 and head 8 give the
 * 2-lookup layout's bigram and trigram rows. */
#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

uint64_t oracle_head_mix(uint64_t key, int32_t head) {
    return oracle_mix64(key + (uint64_t)(head % 8) * GOLDEN_GAMMA);
}

/* row_ids[t][h], h = 0..15, -1 when the head's n-gram is missing. */
void oracle_ngram_ids_heads(const int32_t* tokens, const int32_t* cu, int32_t S,
                            const int32_t* hist_ids, const int32_t* hist_len, int64_t R,
                            int32_t* row_ids) {
    for (int32_t s = 0; s < S; ++s) {
        int32_t start = cu[s], end = cu[s + 1];
        int32_t hl = hist_len[s];
        int64_t n = hl + (end - start);
        for (int64_t j = hl; j < n; ++j) {
            int32_t t = start + (int32_t)(j - hl);
#define HS(idx) ((idx) < hl ? hist_ids[2 * s + 2 - hl + (idx)] : tokens[start + (idx) - hl])
            uint32_t cur = (uint32_t)HS(j);
            for (int h = 0; h < 16; ++h) {
                int32_t r = -1;
                if (h < 8 && j >= 1) {
                    uint32_t p1 = (uint32_t)HS(j - 1);
                    r = (int32_t)(oracle_head_mix(oracle_key2(p1, cur), h) % (uint64_t)R);
                } else if (h >= 8 && j >= 2) {
                    uint32_t p1 = (uint32_t)HS(j - 1), p2 = (uint32_t)HS(j - 2);
                    r = (int32_t)(oracle_head_mix(oracle_key3(p2, p1, cur), h) % (uint64_t)R);
                }
                row_ids[16 * (int64_t)t + h] = r;
            }
#undef HS
        }
    }
}

/* New history after a chunk: the last min(2, hist_len + L) IDs, right-aligned. */
void oracle_hist_update(const int32_t* tokens, const int32_t* cu, int32_t S,
                        const int32_t* hist_ids, const int32_t* hist_len,
                        int32_t* hist_ids_out, int32_t* hist_len_out) {
    for (int32_t s = 0; s < S; ++s) {
        int32_t hl = hist_len[s], L = cu[s + 1] - cu[s];
        int32_t seq[4];  /* up to 2 history + last 2 tokens */
        int n = 0;
        for (int i = 0; i < hl; ++i) seq[n++] = hist_ids[2 * s + 2 - hl + i];
        int32_t from = L > 2 ? L - 2 : 0;
        for (int32_t i = from; i < L; ++i) seq[n++] = tokens[cu[s] + i];
        int keep = n < 2 ? n : 2;
        hist_ids_out[2 * s + 0] = hist_ids[2 * s + 0];
        hist_ids_out[2 * s + 1] = hist_ids[2 * s + 1];
        for (int i = 0; i < keep; ++i) hist_ids_out[2 * s + 2 - keep + i] = seq[n - keep + i];
        hist_len_out[s] = keep;
    }
}

/* ------------------------------------------------------------------------ */
/* Gather + dequantize                                                       */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3FN: sign s, exponent e (bias 7), mantissa m; e = 0 is
 * subnormal m/8 * 2^-6; 0x7F/0xFF are NaN; no infinities. */
double oracle_e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* float -> bfloat16, round to nearest, ties to even (finite inputs). */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

double oracle_bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* x[t] = bf16( fl32(p_bi + p_tri) ), p = fl32(dec(code) * scale[row]);
 * rows with id -1 are skipped. raw (optional) gets the two rows' bytes,
 * zero for a missing row. */
void oracle_gather_dequant(const int32_t* row_ids, int64_t T, const uint8_t* table,
                           const float* scales, uint16_t* x, uint8_t* raw) {
    for (int64_t t = 0; t < T; ++t) {
        int32_t r0 = row_ids[2 * t], r1 = row_ids[2 * t + 1];
        for (int c = 0; c < D; ++c) {
            float acc = 0.0f;
            int have = 0;
            if (r0 >= 0) {
                float p = (float)oracle_e4m3_value(table[(int64_t)r0 * D + c]) * scales[r0];
                acc = p;
                have = 1;
            }
            if (r1 >= 0) {
                float p = (float)oracle_e4m3_value(table[(int64_t)r1 * D + c]) * scales[r1];
                acc = have ? acc + p : p;
            }
            x[t * D + c] = oracle_bf16_rne(acc);
        }
        if (raw) {
            for (int k = 0; k < 2; ++k) {
                int32_t r = row_ids[2 * t + k];
                uint8_t* dst = raw + (t * 2 + k) * D;
                if (r >= 0) memcpy(dst, table + (int64_t)r * D, D);
                else memset(dst, 0, D);
            }
        }
    }
}

/* OCP Microscaling formats (v1.0), FP4 E2M1: sign S, exponent E (2 bits,
 * bias 1), mantissa M (1 bit); E = 0 is subnormal 0.5 * M, otherwise
 * 2^(E-1) * (1 + M/2); no infinities or NaN. */
double oracle_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* NVFP4 table (the Spark deployment's packed PLE table: 4-bit codes with an
 * FP8 scale per group of 16): row r = 1280 bytes of E2M1 codes (element 2k
 * in the low nibble of byte k), 160 E4M3FN block scales (block b covers
 * elements 16b .. 16b+15) and the fp32 row scale. Per element
 *   p = fl32( fl32( e2m1(code) * e4m3(block) ) * scale ),
 * the inner product being exact (at most 2 x 4 significant bits); the two
 * rows combine as in the FP8 table: x = bf16(fl32(p_bi + p_tri)), a missing
 * row skipped. raw (optional) gets the rows' code bytes [T][2][1280]. */
void oracle_gather_dequant_nvfp4(const int32_t* row_ids, int64_t T, const uint8_t* codes,
                                 const uint8_t* blocks, const float* scales, uint16_t* x, uint8_t* raw) {
    for (int64_t t = 0; t < T; ++t) {
        int32_t rr[2] = {row_ids[2 * t], row_ids[2 * t + 1]};
        for (int c = 0; c < D; ++c) {
            float acc = 0.0f;
            int have = 0;
            for (int k = 0; k < 2; ++k) {
                int32_t r = rr[k];
                if (r < 0) continue;
                uint8_t byte = codes[(int64_t)r * (D / 2) + c / 2];
                uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
                float q = (float)(oracle_e2m1_value(nib) * oracle_e4m3_value(blocks[(int64_t)r * (D / 16) + c / 16]));
                float p = q * scales[r];
                acc = have ? acc + p : p;
                have = 1;
            }
            x[t * D + c] = oracle_bf16_rne(acc);
        }
        if (raw) {
            for (int k = 0; k < 2; ++k) {
                uint8_t* dst = raw + (t * 2 + k) * (D / 2);
                if (rr[k] >= 0) memcpy(dst, codes + (int64_t)rr[k] * (D / 2), D / 2);
                else memset(dst, 0, D / 2);
            }
        }
    }
}

/* 16-lookup layout: x[t][160 h + j] = bf16( fl32(dec(code_h[j]) * scale_h) )
 * for a present head row, +0 for a missing one; `slices` holds the rows
 * referenced by idx[t][h] (uint8 [n][160]) with their scales. raw (optional)
 * gets the 16 rows' bytes, zero for a missing row. */
void oracle_gather_dequant_heads(const int32_t* idx, int64_t T, const uint8_t* slices,
                                 const float* scales, uint16_t* x, uint8_t* raw) {
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < 16; ++h) {
            int32_t r = idx[16 * t + h];
            for (int j = 0; j < 160; ++j) {
                float v = 0.0f;
                if (r >= 0) v = (float)oracle_e4m3_value(slices[(int64_t)r * 160 + j]) * scales[r];
                x[t * D + 160 * h + j] = oracle_bf16_rne(v);
            }
            if (raw) {
                uint8_t* dst = raw + (t * 16 + h) * 160;
                if (r >= 0) memcpy(dst, slices + (int64_t)r * 160, 160);
                else memset(dst, 0, 160);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Projection, gate, conv, fuse                                              */
/* ------------------------------------------------------------------------ */

/* e[t][o] = sum_c x[t][c] * W[o][c], fp64 accumulation. */
void oracle_project(const uint16_t* x, int64_t T, const uint16_t* W, double* e) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double xr[D];
        for (int c = 0; c < D; ++c) xr[c] = oracle_bf16_value(x[t * D + c]);
        for (int o = 0; o < D; ++o) {
            const uint16_t* w = W + (int64_t)o * D;
            double acc = 0.0;
            for (int c = 0; c < D; ++c) acc += xr[c] * oracle_bf16_value(w[c]);
            e[t * D + o] = acc;
        }
    }
}

/* out[i] = the bf16 value nearest to in[i], ties to the even significand,
 * rounded once from the fp64 value: bf16 keeps 8 significant bits and
 * fp32's exponent range (subnormal step 2^-133); magnitudes at or beyond
 * the midpoint above the largest finite bf16 become infinite. */
void oracle_round_bf16(const double* in, int64_t n, double* out) {
    const double max_finite = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    const double overflow = ldexp(511.0, 119);     /* max_finite + half its step */
    for (int64_t i = 0; i < n; ++i) {
        double v = in[i];
        if (v == 0.0 || isnan(v) || isinf(v)) {
            out[i] = v;
            continue;
        }
        int ex;
        frexp(v, &ex);                              /* |v| = m 2^ex, 0.5 <= m < 1 */
        int q = ex - 8;                             /* step of an 8-bit significand */
        if (q < -133) q = -133;
        double r = nearbyint(ldexp(v, -q));        /* default mode: nearest, ties even */
        r = ldexp(r, q);
        if (fabs(v) >= overflow) r = copysign(INFINITY, v);
        else if (fabs(r) > max_finite) r = copysign(max_finite, v);
        out[i] = (r == 0.0) ? copysign(0.0, v) : r;
    }
}

/* g[t] = sigmoid( <h/rms(h), e/rms(e)> / sqrt(D) ). */
void oracle_gate(const uint16_t* h, const double* e, int64_t T, double eps, double* g) {
    for (int64_t t = 0; t < T; ++t) {
        double hh = 0.0, ee = 0.0, he = 0.0;
        for (int c = 0; c < D; ++c) {
            double hv = oracle_bf16_value(h[t * D + c]), ev = e[t * D + c];
            hh += hv * hv;
            ee += ev * ev;
            he += hv * ev;
        }
        double rh = sqrt(hh / D + eps), re = sqrt(ee / D + eps);
        double z = he / (rh * re) / sqrt((double)D);
        g[t] = 1.0 / (1.0 + exp(-z));
    }
}

/* v = g e; y[t][c] = sum_k w[c][k] v[t-3+k][c] with v before a sequence's
 * first token read from state[s][0..2] (oldest first); out = h + y.
 * state_out[s] = the last three v of (state[s] ++ this chunk's v). */
void oracle_conv_fuse(const uint16_t* h, const double* e, const double* g, int64_t T,
                      const int32_t* cu, int32_t S, const uint16_t* conv_w,
                      const double* state, double* y, double* out, double* state_out) {
    (void)T;
    for (int32_t s = 0; s < S; ++s) {
        int32_t start = cu[s], L = cu[s + 1] - cu[s];
        for (int c = 0; c < D; ++c) {
            double w[KTAPS];
            for (int k = 0; k < KTAPS; ++k) w[k] = oracle_bf16_value(conv_w[c * KTAPS + k]);
            /* V(j) for j = -3 .. L-1 */
#define V(j) ((j) < 0 ? state[((int64_t)s * 3 + 3 + (j)) * D + c] \
                      : g[start + (j)] * e[(int64_t)(start + (j)) * D + c])
            for (int32_t j = 0; j < L; ++j) {
                double acc = 0.0;
                for (int k = 0; k < KTAPS; ++k) acc += w[k] * V(j - 3 + k);
                int64_t t = start + j;
                y[t * D + c] = acc;
                out[t * D + c] = oracle_bf16_value(h[t * D + c]) + acc;
            }
            for (int i = 0; i < 3; ++i)
                state_out[((int64_t)s * 3 + i) * D + c] = V(L - 3 + i);
#undef V
        }
    }
}
