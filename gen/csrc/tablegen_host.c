/* CPU side of the FP8 table generator (input data, not part of the PLE method).
 *
 * Row r of the table is 2560 E4M3FN codes plus one fp32 scale. Every byte is
 * a pure function of (seed, r, c), so any row can be rebuilt here on demand
 * and compared with what the GPU generator wrote into HBM.
 *
 * Random bits: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), key = (seed, 0).
 *   codes: counter = (g / 8, 0, 0, 0) with g = r * 2560 + c; the four 64-bit
 *          outputs give eight 32-bit words, low half first; element g takes
 *          word g % 8. Bit 31 is the sign, bits 0..30 a uniform u; the
 *          magnitude code is the number of thresholds <= u.
 *   scale: counter = (r, 1, 0, 0); m = lo + (hi32(out[0]) % span);
 *          scale = m * 2^-23 (an exact fp32 with at most 20 significant bits).
 * NVFP4 table (a second table, key = (seed, 1)): element g = r * 2560 + c
 *   takes word g % 8 of Philox(counter (g / 8, 0, 0, 0)); bit 31 is the sign,
 *   the E2M1 magnitude is the number of the 7 thresholds <= bits 0..30;
 *   element 2k is the low nibble of byte k of the row. Block b (elements
 *   16b .. 16b+15) of row r: q = r * 160 + b, Philox(counter (q, 2, 0, 0)),
 *   E4M3 code = lo + hi32(out[0]) % span. The row scale is the FP8 table's.
 * The same bytes, read as 16 head tables of R rows x 160 bytes, give row r of
 * head h at element g = (h R + r) 160; its scale is scale number h R + r of
 * the same recipe (the first R being the 2560-wide rows' scales).
 */
#include <stdint.h>
#include <string.h>

#define ROW 2560

static void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    unsigned __int128 p = (unsigned __int128)a * b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void gen_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int i = 0; i < 10; ++i) {
        if (i > 0) {
            k0 += 0x9E3779B97F4A7C15ULL;
            k1 += 0xBB67AE8584CAA73BULL;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(0xD2E7470EE14C6C93ULL, c0, &hi0, &lo0);
        mulhilo64(0xCA5A826395121157ULL, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static uint8_t code_of(uint32_t w, const uint32_t* thr) {
    uint32_t u = w & 0x7FFFFFFFu;
    /* count thresholds <= u (thresholds are non-decreasing) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (thr[mid] <= u) lo = mid + 1; else hi = mid;
    }
    return (uint8_t)(((w >> 31) << 7) | (uint32_t)lo);
}

/* Rebuild rows ids[0..n) into rows_out[n][2560] and scales_out[n]. */
void gen_table_rows(uint64_t seed, const int64_t* ids, int64_t n, const uint32_t* thr,
                    uint32_t scale_lo, uint32_t scale_span,
                    uint8_t* rows_out, float* scales_out) {
    const uint64_t key[2] = {seed, 0};
    /* rows are independent: one thread per row */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = (uint64_t)ids[i];
        uint8_t* row = rows_out + i * ROW;
        for (int c8 = 0; c8 < ROW / 8; ++c8) {
            uint64_t g0 = r * ROW + (uint64_t)c8 * 8;
            uint64_t ctr[4] = {g0 / 8, 0, 0, 0}, o[4];
            gen_philox4x64_10(ctr, key, o);
            for (int j = 0; j < 8; ++j) {
                uint64_t word = o[j / 2];
                uint32_t w = (j & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
                row[c8 * 8 + j] = code_of(w, thr);
            }
        }
        uint64_t sc[4] = {r, 1, 0, 0}, so[4];
        gen_philox4x64_10(sc, key, so);
        uint32_t m = scale_lo + (uint32_t)(so[0] >> 32) % scale_span;
        float s = (float)m;            /* exact: m < 2^24 */
        s *= 1.0f / 8388608.0f;        /* * 2^-23, exact */
        scales_out[i] = s;
    }
}

/* Codes of elements g0 .. g0+n-1 (g0 and n multiples of 8) into out[n]. */
void gen_table_span(uint64_t seed, uint64_t g0, int64_t n, const uint32_t* thr, uint8_t* out) {
    const uint64_t key[2] = {seed, 0};
    for (int64_t c8 = 0; c8 < n / 8; ++c8) {
        uint64_t ctr[4] = {g0 / 8 + (uint64_t)c8, 0, 0, 0}, o[4];
        gen_philox4x64_10(ctr, key, o);
        for (int j = 0; j < 8; ++j) {
            uint64_t word = o[j / 2];
            uint32_t w = (j & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
            out[c8 * 8 + j] = code_of(w, thr);
        }
    }
}

/* 160-byte rows q[0..n) of the 16 x [R][160] view (row q = h R + r starts at
 * element 160 q) into out[n][160]. */
void gen_table_slices(uint64_t seed, const int64_t* q, int64_t n, const uint32_t* thr, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) gen_table_span(seed, (uint64_t)q[i] * 160, 160, thr, out + i * 160);
}

/* Scales number ids[0..n) into out[n]. */
void gen_scales(uint64_t seed, const int64_t* ids, int64_t n, uint32_t scale_lo, uint32_t scale_span,
                float* out) {
    const uint64_t key[2] = {seed, 0};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t sc[4] = {(uint64_t)ids[i], 1, 0, 0}, so[4];
        gen_philox4x64_10(sc, key, so);
        uint32_t m = scale_lo + (uint32_t)(so[0] >> 32) % scale_span;
        out[i] = (float)m * (1.0f / 8388608.0f);
    }
}

/* NVFP4 rows ids[0..n): codes_out[n][1280], blocks_out[n][160] (the fp32 row
 * scales are the FP8 table's, gen_table_rows). */
void gen_nvfp4_rows(uint64_t seed, const int64_t* ids, int64_t n, const uint32_t* thr7,
                    uint32_t block_lo, uint32_t block_span, uint8_t* codes_out, uint8_t* blocks_out) {
    const uint64_t key[2] = {seed, 1};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = (uint64_t)ids[i];
        uint8_t* codes = codes_out + i * (ROW / 2);
        for (int c8 = 0; c8 < ROW / 8; ++c8) {
            uint64_t ctr[4] = {(r * ROW) / 8 + (uint64_t)c8, 0, 0, 0}, o[4];
            gen_philox4x64_10(ctr, key, o);
            for (int j = 0; j < 8; j += 2) {
                uint8_t nib[2];
                for (int k = 0; k < 2; ++k) {
                    uint64_t word = o[(j + k) / 2];
                    uint32_t w = ((j + k) & 1) ? (uint32_t)(word >> 32) : (uint32_t)word;
                    uint32_t u = w & 0x7FFFFFFFu, m = 0;
                    while (m < 7 && thr7[m] <= u) ++m;
                    nib[k] = (uint8_t)(((w >> 31) << 3) | m);
                }
                codes[c8 * 4 + j / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
        for (int b = 0; b < ROW / 16; ++b) {
            uint64_t ctr[4] = {r * (ROW / 16) + (uint64_t)b, 2, 0, 0}, o[4];
            gen_philox4x64_10(ctr, key, o);
            blocks_out[i * (ROW / 16) + b] = (uint8_t)(block_lo + (uint32_t)(o[0] >> 32) % block_span);
        }
    }
}
