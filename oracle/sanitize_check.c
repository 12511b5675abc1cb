/*
 * Memory and undefined-behaviour check of the CPU oracle (test
 * infrastructure): tests/test_oracle_sanitize.py builds this driver together
 * with oracle.c under AddressSanitizer and UBSan on the host and runs it.
 * It calls every oracle entry point on small buffers sized exactly as each
 * function's contract states (so any read or write past them is reported),
 * including the degenerate cases: kv_len below 0 and above L_cap, k larger
 * than the visible context, index slots that are -1 or out of range, empty
 * sets, unallocated pages, and every FP8 code.  Exit status 0 means every
 * call finished without a report; a few results are also checked against
 * their closed forms so the calls are not optimised away.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
static int rand_int(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

/* bf16 bit pattern of a float (round toward zero is enough for test data) */
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;
#define EXPECT(cond, ...)                  \
    do {                                   \
        if (!(cond)) {                     \
            fprintf(stderr, __VA_ARGS__);  \
            fputc('\n', stderr);           \
            ++failures;                    \
        }                                  \
    } while (0)

static void check_scores_and_topk(void) {
    const int B = 3, Tq = 4, H_I = 5, D_I = 7, L_cap = 19;
    int8_t* qI = xmalloc((size_t)B * Tq * H_I * D_I);
    float* w = xmalloc(sizeof(float) * B * Tq * H_I);
    int8_t* kI = xmalloc((size_t)B * L_cap * D_I);
    int32_t kv_len[3] = {-2, 7, L_cap + 5};      /* below 0, inside, past L_cap */
    float* S = xmalloc(sizeof(float) * B * Tq * L_cap);
    for (int i = 0; i < B * Tq * H_I * D_I; ++i) qI[i] = (int8_t)rand_int(-128, 127);
    for (int i = 0; i < B * L_cap * D_I; ++i) kI[i] = (int8_t)rand_int(-128, 127);
    for (int i = 0; i < B * Tq * H_I; ++i) w[i] = 0.25f * (float)rand_int(-8, 8);
    oracle_indexer_scores(qI, w, kI, kv_len, B, Tq, H_I, D_I, L_cap, S);
    /* sequence 0 sees nothing: every score is -inf */
    for (int i = 0; i < Tq * L_cap; ++i) EXPECT(isinf(S[i]) && S[i] < 0, "seq 0 score %d visible", i);
    const int ks[3] = {1, 6, 40};                /* 40 > every visible count */
    for (int ki = 0; ki < 3; ++ki) {
        const int k = ks[ki];
        int32_t* idx = xmalloc(sizeof(int32_t) * B * Tq * k);
        oracle_topk_select(S, kv_len, B, Tq, L_cap, k, idx);
        for (int j = 0; j < Tq * k; ++j) EXPECT(idx[j] == -1, "seq 0 slot %d = %d", j, idx[j]);
        free(idx);
    }
    free(qI); free(w); free(kI); free(S);
}

static void check_attend(void) {
    const int B = 2, Tq = 3, H = 4, D = 12, D_v = 8, L_cap = 23, k = 9;
    uint16_t* Q = xmalloc(sizeof(uint16_t) * B * Tq * H * D);
    uint16_t* C = xmalloc(sizeof(uint16_t) * B * L_cap * D);
    int32_t* idx = xmalloc(sizeof(int32_t) * B * Tq * k);
    double* out = xmalloc(sizeof(double) * B * Tq * H * D_v);
    double* lse = xmalloc(sizeof(double) * B * Tq * H);
    for (int i = 0; i < B * Tq * H * D; ++i) Q[i] = bf16_of((float)rand_int(-40, 40) / 16.0f);
    for (int i = 0; i < B * L_cap * D; ++i) C[i] = bf16_of((float)rand_int(-40, 40) / 16.0f);
    for (int i = 0; i < B * Tq * k; ++i) idx[i] = rand_int(-3, L_cap + 3);
    for (int j = 0; j < k; ++j) idx[j] = -1;     /* (b=0, t=0): empty set */
    oracle_sparse_mla_attend(Q, C, idx, B, Tq, H, D, D_v, L_cap, k, 0.25f, out, lse);
    for (int h = 0; h < H; ++h) {
        EXPECT(isinf(lse[h]) && lse[h] < 0, "empty set lse %g", lse[h]);
        for (int v = 0; v < D_v; ++v) EXPECT(out[h * D_v + v] == 0.0, "empty set out");
    }

    /* FP8 cache: D_c = D_v latent codes, one exponent byte, D - D_v RoPE dims */
    const int D_c = D_v, D_r = D - D_v;
    uint8_t* C8 = xmalloc((size_t)B * L_cap * D_c);
    uint8_t* Ce = xmalloc((size_t)B * L_cap);
    uint16_t* Cr = xmalloc(sizeof(uint16_t) * B * L_cap * D_r);
    for (int i = 0; i < B * L_cap * D_c; ++i) C8[i] = (uint8_t)next_u32();
    for (int i = 0; i < B * L_cap; ++i) Ce[i] = (uint8_t)rand_int(120, 134);
    for (int i = 0; i < B * L_cap * D_r; ++i) Cr[i] = bf16_of((float)rand_int(-9, 9) / 4.0f);
    oracle_sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, B, Tq, H, D_c, D_r, L_cap, k, 0.25f, out, lse);
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3_to_double((uint8_t)c);
    EXPECT(oracle_e4m3_to_double(0x7E) == 448.0, "e4m3 max");

    /* access counts, invalid slots included */
    uint32_t* counts = xmalloc(sizeof(uint32_t) * B * L_cap);
    memset(counts, 0, sizeof(uint32_t) * B * L_cap);
    oracle_index_histogram(idx, B, Tq, k, L_cap, counts);
    long valid = 0, total = 0;
    for (int i = 0; i < B * Tq * k; ++i) valid += idx[i] >= 0 && idx[i] < L_cap;
    for (int i = 0; i < B * L_cap; ++i) total += counts[i];
    EXPECT(valid == total, "histogram total %ld != valid slots %ld", total, valid);

    free(Q); free(C); free(idx); free(out); free(lse); free(C8); free(Ce); free(Cr); free(counts);
}

static void check_paged(void) {
    const int B = 2, Tq = 2, H_I = 3, D_I = 5, bs = 4, max_blocks = 5, n_pages = 11;
    const int H = 2, D = 6, D_v = 4, k = 7;
    const int L_cap = max_blocks * bs;
    int32_t table[10];
    for (int i = 0; i < B * max_blocks; ++i) table[i] = i;
    table[3] = -1;                                /* unallocated block */
    table[6] = n_pages;                           /* past the pool: unallocated too */
    int8_t* qI = xmalloc((size_t)B * Tq * H_I * D_I);
    float* w = xmalloc(sizeof(float) * B * Tq * H_I);
    int8_t* kIp = xmalloc((size_t)n_pages * bs * D_I);
    int32_t kv_len[2] = {L_cap, 9};
    float* S = xmalloc(sizeof(float) * B * Tq * L_cap);
    for (int i = 0; i < B * Tq * H_I * D_I; ++i) qI[i] = (int8_t)rand_int(-8, 7);
    for (int i = 0; i < B * Tq * H_I; ++i) w[i] = 1.0f;
    for (int i = 0; i < n_pages * bs * D_I; ++i) kIp[i] = (int8_t)rand_int(-8, 7);
    oracle_indexer_scores_paged(qI, w, kIp, table, max_blocks, bs, n_pages, kv_len, B, Tq, H_I,
                                D_I, S);
    uint16_t* Q = xmalloc(sizeof(uint16_t) * B * Tq * H * D);
    uint16_t* Cp = xmalloc(sizeof(uint16_t) * n_pages * bs * D);
    int32_t* idx = xmalloc(sizeof(int32_t) * B * Tq * k);
    double* out = xmalloc(sizeof(double) * B * Tq * H * D_v);
    double* lse = xmalloc(sizeof(double) * B * Tq * H);
    for (int i = 0; i < B * Tq * H * D; ++i) Q[i] = bf16_of((float)rand_int(-9, 9) / 8.0f);
    for (int i = 0; i < n_pages * bs * D; ++i) Cp[i] = bf16_of((float)rand_int(-9, 9) / 8.0f);
    for (int i = 0; i < B * Tq * k; ++i) idx[i] = rand_int(-2, L_cap + 2);
    oracle_sparse_mla_attend_paged(Q, Cp, table, max_blocks, bs, n_pages, idx, B, Tq, H, D, D_v, k,
                                   0.5f, out, lse);
    free(qI); free(w); free(kIp); free(S); free(Q); free(Cp); free(idx); free(out); free(lse);
}

static void check_group(void) {
    const int B = 2, Tq = 3, L_cap = 30, H_I = 2, D_I = 4, k = 5, H = 2, D = 6, D_v = 4, n = 4;
    int8_t* qI[4];
    float* w[4];
    int8_t* kI[4];
    uint16_t* Q[4];
    uint16_t* C[4];
    double* out[4];
    double* lse[4];
    for (int l = 0; l < n; ++l) {
        qI[l] = xmalloc((size_t)B * Tq * H_I * D_I);
        w[l] = xmalloc(sizeof(float) * B * Tq * H_I);
        kI[l] = xmalloc((size_t)B * L_cap * D_I);
        Q[l] = xmalloc(sizeof(uint16_t) * B * Tq * H * D);
        C[l] = xmalloc(sizeof(uint16_t) * B * L_cap * D);
        out[l] = xmalloc(sizeof(double) * B * Tq * H * D_v);
        lse[l] = xmalloc(sizeof(double) * B * Tq * H);
        for (int i = 0; i < B * Tq * H_I * D_I; ++i) qI[l][i] = (int8_t)rand_int(-8, 7);
        for (int i = 0; i < B * Tq * H_I; ++i) w[l][i] = 0.5f;
        for (int i = 0; i < B * L_cap * D_I; ++i) kI[l][i] = (int8_t)rand_int(-8, 7);
        for (int i = 0; i < B * Tq * H * D; ++i) Q[l][i] = bf16_of((float)rand_int(-9, 9) / 8.0f);
        for (int i = 0; i < B * L_cap * D; ++i) C[l][i] = bf16_of((float)rand_int(-9, 9) / 8.0f);
    }
    int32_t kv_len[2] = {L_cap, 2};
    int32_t* idx = xmalloc(sizeof(int32_t) * B * Tq * k);
    float* S = xmalloc(sizeof(float) * B * Tq * L_cap);
    const int modes[3][2] = {{0, 0}, {1, 0}, {0, 1}};   /* shared, reuse, per-layer */
    for (int m = 0; m < 3; ++m)
        oracle_group_forward(B, Tq, L_cap, H_I, D_I, k, H, D, D_v, n, 0.4f,
                             (const int8_t* const*)qI, (const float* const*)w,
                             (const int8_t* const*)kI, kv_len, (const uint16_t* const*)Q,
                             (const uint16_t* const*)C, out, lse, idx, modes[m][0], modes[m][1], S);
    for (int l = 0; l < n; ++l) {
        free(qI[l]); free(w[l]); free(kI[l]); free(Q[l]); free(C[l]); free(out[l]); free(lse[l]);
    }
    free(idx); free(S);
}

int main(void) {
    for (int rep = 0; rep < 20; ++rep) {
        check_scores_and_topk();
        check_attend();
        check_paged();
        check_group();
    }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
