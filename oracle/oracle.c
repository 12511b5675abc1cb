/*
 * CPU oracle for one IndexShare layer group.  TEST INFRASTRUCTURE ONLY: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it; the GPU library neither links nor calls it, and the two share no
 * code, header, table or constant.
 *
 * Sources (the pages describing GLM-5.2's sparse attention):
 *  - "GLM-5.2 Explained: 1M Token Context AI Agent Model", section 2.1
 *    (IndexShare: Cross-Layer Index Sharing for DSA Sparse Attention): the
 *    lightning indexer scores every earlier token against the current query,
 *    I(t,s) = w * sigma(q_t . h_s), keeps the top-K positions, and attention
 *    loads keys and values only at those positions; the first layer of a
 *    group of index_topk_freq layers computes the set and the others reuse it.
 *    Section 2.2.1: only the first MTP draft step runs the indexer; later
 *    steps reuse its top-k and append nothing to the cache.
 *  - "GLM-5.2核心技术解析：IndexShare架构与MTP层优化详解", the config.json
 *    fragments: index_topk = 2048, index_topk_freq = 4,
 *    index_share_for_mtp_iteration = true, kv_lora_rank = 512.
 *  - "GLM-5.2 技术报告解读：IndexShare 稀疏注意力与反奖励作弊强化学习",
 *    section 1, training-strategy table (indexer only in the first of every
 *    four sparse layers; the other three reuse its top-k) and the MTP notes.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes):
 *  - sigma is ReLU and the score sums over indexer heads with one weight per
 *    (query, head): S = sum_h w_h * ReLU(q_h . k), one shared key per token;
 *  - a query at position pos sees keys 0..pos, itself included;
 *  - the set holds the min(k, pos+1) best keys under (score descending,
 *    position ascending), is listed in ascending position and padded with -1;
 *  - attention uses the absorbed latent form: the key is the whole latent
 *    row and the value is its first D_v entries.
 *
 * Arithmetic: indexer dot products in exact 64-bit integers; the head sum
 * and every attention quantity in double.  Built with -ffp-contract=off.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static long visible_len(const int32_t* kv_len, int b, int L_cap) {
    long len = kv_len[b];
    if (len < 0) len = 0;
    if (len > L_cap) len = L_cap;
    return len;
}

/* Position of query t of a sequence whose last query sits at len-1
 * (the Tq queries are the last Tq entries of the cache). */
static long query_pos(long len, int Tq, int t) { return len - Tq + t; }

void oracle_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                           const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                           int L_cap, float* S) {
    for (int b = 0; b < B; ++b) {
        long len = visible_len(kv_len, b, L_cap);
        for (int t = 0; t < Tq; ++t) {
            long pos = query_pos(len, Tq, t);
            const int8_t* q = qI + ((size_t)b * Tq + t) * H_I * D_I;
            const float* wt = w + ((size_t)b * Tq + t) * H_I;
            float* row = S + ((size_t)b * Tq + t) * L_cap;
            for (long s = 0; s < L_cap; ++s) {
                if (s > pos) {
                    row[s] = -INFINITY;
                    continue;
                }
                const int8_t* key = kI + ((size_t)b * L_cap + s) * D_I;
                double score = 0.0;
                for (int h = 0; h < H_I; ++h) {
                    long long dot = 0;
                    for (int d = 0; d < D_I; ++d)
                        dot += (long long)q[h * D_I + d] * (long long)key[d];
                    long long relu = dot > 0 ? dot : 0;
                    score += (double)wt[h] * (double)relu;
                }
                row[s] = (float)score;
            }
        }
    }
}

typedef struct {
    float v;
    int32_t s;
} scored_pos;

/* Total order of the selection: larger score first; equal scores (with -0.0
 * equal to +0.0, as float comparison gives) keep the lower position first. */
static int by_score_desc_pos_asc(const void* pa, const void* pb) {
    const scored_pos* a = (const scored_pos*)pa;
    const scored_pos* b = (const scored_pos*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->s > b->s) - (a->s < b->s);
}

static int by_int_asc(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

void oracle_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                        int k, int32_t* idx) {
    scored_pos* cand = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(L_cap > 0 ? L_cap : 1));
    for (int b = 0; b < B; ++b) {
        long len = visible_len(kv_len, b, L_cap);
        for (int t = 0; t < Tq; ++t) {
            long pos = query_pos(len, Tq, t);
            long n = pos + 1 > 0 ? pos + 1 : 0;
            const float* row = S + ((size_t)b * Tq + t) * L_cap;
            int32_t* out = idx + ((size_t)b * Tq + t) * k;
            for (long s = 0; s < n; ++s) {
                cand[s].v = row[s];
                cand[s].s = (int32_t)s;
            }
            qsort(cand, (size_t)n, sizeof(scored_pos), by_score_desc_pos_asc);
            long m = n < k ? n : k;
            for (long j = 0; j < m; ++j) out[j] = cand[j].s;
            qsort(out, (size_t)m, sizeof(int32_t), by_int_asc);
            for (long j = m; j < k; ++j) out[j] = -1;
        }
    }
    free(cand);
}

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                              int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                              float sm_scale, double* out, double* lse) {
    double* z = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    const double scale = (double)sm_scale;
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < Tq; ++t) {
            const int32_t* sel = idx + ((size_t)b * Tq + t) * k;
            for (int h = 0; h < H; ++h) {
                const uint16_t* q = Q + (((size_t)b * Tq + t) * H + h) * D;
                double* o = out + (((size_t)b * Tq + t) * H + h) * D_v;
                double m = -INFINITY;
                int n_valid = 0;
                for (int j = 0; j < k; ++j) {
                    int32_t s = sel[j];
                    if (s < 0 || s >= L_cap) continue;
                    const uint16_t* c = C + ((size_t)b * L_cap + s) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += bf16_to_double(q[d]) * bf16_to_double(c[d]);
                    z[j] = scale * dot;
                    if (z[j] > m) m = z[j];
                    ++n_valid;
                }
                for (int v = 0; v < D_v; ++v) o[v] = 0.0;
                if (n_valid == 0) {
                    if (lse) lse[((size_t)b * Tq + t) * H + h] = -INFINITY;
                    continue;
                }
                double denom = 0.0;
                for (int j = 0; j < k; ++j) {
                    int32_t s = sel[j];
                    if (s < 0 || s >= L_cap) continue;
                    double e = exp(z[j] - m);
                    denom += e;
                    const uint16_t* c = C + ((size_t)b * L_cap + s) * D;
                    for (int v = 0; v < D_v; ++v) o[v] += e * bf16_to_double(c[v]);
                }
                for (int v = 0; v < D_v; ++v) o[v] /= denom;
                if (lse) lse[((size_t)b * Tq + t) * H + h] = m + log(denom);
            }
        }
    }
    free(z);
}

/* OCP FP8 E4M3 (the "FN" variant): sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no
 * infinities; S.1111.111 is NaN; the largest finite magnitude is 448. */
double oracle_e4m3_to_double(uint8_t code) {
    const int sign = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Attention over an FP8 latent cache: every selected row is first written
 * out as the D = D_c + D_r values it stands for (E4M3 code times the row's
 * power-of-two scale 2^(Ce - 127) for d < D_c, the bf16 RoPE value after
 * that), then the attention is the same as oracle_sparse_mla_attend's. */
void oracle_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                  const uint16_t* Cr, const int32_t* idx, int B, int Tq, int H,
                                  int D_c, int D_r, int L_cap, int k, float sm_scale,
                                  double* out, double* lse) {
    const int D = D_c + D_r;
    const int D_v = D_c;
    double code_value[256];
    for (int c = 0; c < 256; ++c) code_value[c] = oracle_e4m3_to_double((uint8_t)c);
    double* rows = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)D);
    double* z = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    const double scale = (double)sm_scale;
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < Tq; ++t) {
            const int32_t* sel = idx + ((size_t)b * Tq + t) * k;
            for (int j = 0; j < k; ++j) {
                int32_t s = sel[j];
                if (s < 0 || s >= L_cap) continue;
                const size_t row = (size_t)b * L_cap + s;
                const double row_scale = ldexp(1.0, (int)Ce[row] - 127);
                double* r = rows + (size_t)j * D;
                for (int d = 0; d < D_c; ++d) r[d] = code_value[C8[row * D_c + d]] * row_scale;
                for (int d = 0; d < D_r; ++d) r[D_c + d] = bf16_to_double(Cr[row * D_r + d]);
            }
            for (int h = 0; h < H; ++h) {
                const uint16_t* q = Q + (((size_t)b * Tq + t) * H + h) * D;
                double* o = out + (((size_t)b * Tq + t) * H + h) * D_v;
                double m = -INFINITY;
                int n_valid = 0;
                for (int j = 0; j < k; ++j) {
                    int32_t s = sel[j];
                    if (s < 0 || s >= L_cap) continue;
                    const double* r = rows + (size_t)j * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += bf16_to_double(q[d]) * r[d];
                    z[j] = scale * dot;
                    if (z[j] > m) m = z[j];
                    ++n_valid;
                }
                for (int v = 0; v < D_v; ++v) o[v] = 0.0;
                if (n_valid == 0) {
                    if (lse) lse[((size_t)b * Tq + t) * H + h] = -INFINITY;
                    continue;
                }
                double denom = 0.0;
                for (int j = 0; j < k; ++j) {
                    int32_t s = sel[j];
                    if (s < 0 || s >= L_cap) continue;
                    const double* r = rows + (size_t)j * D;
                    double e = exp(z[j] - m);
                    denom += e;
                    for (int v = 0; v < D_v; ++v) o[v] += e * r[v];
                }
                for (int v = 0; v < D_v; ++v) o[v] /= denom;
                if (lse) lse[((size_t)b * Tq + t) * H + h] = m + log(denom);
            }
        }
    }
    free(z);
    free(rows);
}

/* Access counts of an index set (the per-position access frequency that
 * hot/cold cache placement reads): counts[b,s] += the number of slots of
 * idx[b,:,:] equal to s, for 0 <= s < L_cap; other slot values are ignored. */
void oracle_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                            uint32_t* counts) {
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < Tq; ++t)
            for (int j = 0; j < k; ++j) {
                const int32_t s = idx[((size_t)b * Tq + t) * k + j];
                if (s >= 0 && s < L_cap) counts[(size_t)b * L_cap + s] += 1u;
            }
}

/* Paged caches: the logical row s of sequence b is row
 * table[b][s / block_size] * block_size + s % block_size of the page pool
 * when that table entry is a page in [0, n_pages); otherwise the row is
 * unallocated.  Copies the logical cache out of the pool (unallocated rows
 * zero) and marks which logical rows exist. */
static void unpage_rows(const void* pool, size_t row_bytes, const int32_t* table, int B,
                        int max_blocks, int block_size, int n_pages, unsigned char* out,
                        unsigned char* valid) {
    const long L = (long)max_blocks * block_size;
    for (int b = 0; b < B; ++b)
        for (long s = 0; s < L; ++s) {
            const int32_t page = table[(size_t)b * max_blocks + s / block_size];
            unsigned char* dst = out + ((size_t)b * L + s) * row_bytes;
            const int ok = page >= 0 && page < n_pages;
            valid[(size_t)b * L + s] = (unsigned char)ok;
            if (ok)
                memcpy(dst, (const unsigned char*)pool +
                                ((size_t)page * block_size + s % block_size) * row_bytes,
                       row_bytes);
            else
                memset(dst, 0, row_bytes);
        }
}

void oracle_indexer_scores_paged(const int8_t* qI, const float* w, const int8_t* kI_pages,
                                 const int32_t* table, int max_blocks, int block_size,
                                 int n_pages, const int32_t* kv_len, int B, int Tq, int H_I,
                                 int D_I, float* S) {
    const long L = (long)max_blocks * block_size;
    int8_t* kI = (int8_t*)malloc((size_t)B * L * D_I);
    unsigned char* valid = (unsigned char*)malloc((size_t)B * L);
    unpage_rows(kI_pages, (size_t)D_I, table, B, max_blocks, block_size, n_pages,
                (unsigned char*)kI, valid);
    oracle_indexer_scores(qI, w, kI, kv_len, B, Tq, H_I, D_I, (int)L, S);
    /* positions on unallocated pages score -inf */
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < Tq; ++t)
            for (long s = 0; s < L; ++s)
                if (!valid[(size_t)b * L + s]) S[((size_t)b * Tq + t) * L + s] = -INFINITY;
    free(valid);
    free(kI);
}

void oracle_sparse_mla_attend_paged(const uint16_t* Q, const uint16_t* C_pages,
                                    const int32_t* table, int max_blocks, int block_size,
                                    int n_pages, const int32_t* idx, int B, int Tq, int H, int D,
                                    int D_v, int k, float sm_scale, double* out, double* lse) {
    const long L = (long)max_blocks * block_size;
    uint16_t* C = (uint16_t*)malloc((size_t)B * L * D * sizeof(uint16_t));
    unsigned char* valid = (unsigned char*)malloc((size_t)B * L);
    int32_t* idx2 = (int32_t*)malloc((size_t)B * Tq * k * sizeof(int32_t));
    unpage_rows(C_pages, (size_t)D * sizeof(uint16_t), table, B, max_blocks, block_size, n_pages,
                (unsigned char*)C, valid);
    /* slots on unallocated pages are skipped like -1 */
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < Tq; ++t)
            for (int j = 0; j < k; ++j) {
                const size_t o = ((size_t)b * Tq + t) * k + j;
                const int32_t s = idx[o];
                idx2[o] = (s >= 0 && s < L && valid[(size_t)b * L + s]) ? s : -1;
            }
    oracle_sparse_mla_attend(Q, C, idx2, B, Tq, H, D, D_v, (int)L, k, sm_scale, out, lse);
    free(idx2);
    free(valid);
    free(C);
}

void oracle_group_forward(int B, int Tq, int L_cap, int H_I, int D_I, int k, int H, int D,
                          int D_v, int n_layers, float sm_scale,
                          const int8_t* const* qI, const float* const* w,
                          const int8_t* const* kI, const int32_t* kv_len,
                          const uint16_t* const* Q, const uint16_t* const* C,
                          double* const* out, double* const* lse, int32_t* idx,
                          int reuse_idx, int per_layer_indexer, float* S_scratch) {
    if (!per_layer_indexer && !reuse_idx) {
        /* first layer of the group: indexer + top-k, written once */
        oracle_indexer_scores(qI[0], w[0], kI[0], kv_len, B, Tq, H_I, D_I, L_cap, S_scratch);
        oracle_topk_select(S_scratch, kv_len, B, Tq, L_cap, k, idx);
    }
    for (int l = 0; l < n_layers; ++l) {
        if (per_layer_indexer) {
            oracle_indexer_scores(qI[l], w[l], kI[l], kv_len, B, Tq, H_I, D_I, L_cap, S_scratch);
            oracle_topk_select(S_scratch, kv_len, B, Tq, L_cap, k, idx);
        }
        oracle_sparse_mla_attend(Q[l], C[l], idx, B, Tq, H, D, D_v, L_cap, k, sm_scale, out[l],
                                 lse ? lse[l] : 0);
    }
}
