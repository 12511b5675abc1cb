/*
 * CPU oracle for one IndexShare layer group: lightning-indexer scores, top-k
 * position select, sparse softmax attention over a latent cache, and the
 * group composition that computes the index set once and reuses it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library and the GPU library never calls it.
 *
 * Every pointer is a HOST pointer to a dense row-major array.  Plain,
 * single-threaded loops; no blocking, no fusion, no reordering beyond what the
 * definitions below state.
 */
#ifndef ISA_ORACLE_H
#define ISA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Indexer scores.  S[b,t,s] = sum_h w[b,t,h] * ReLU(sum_d qI[b,t,h,d] * kI[b,s,d])
 * for s <= pos(b,t) = len_b - Tq + t, and -inf otherwise, where len_b is
 * kv_len[b] clamped to [0, L_cap].  Dot products are exact integers, the head
 * sum is taken in double in ascending h and rounded once to float. */
void oracle_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                           const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                           int L_cap, float* S);

/* Top-k select.  For each (b,t) the candidates are s in [0, pos(b,t)].  The
 * min(k, pos+1) candidates that come first in the order (S descending, s
 * ascending) are written in ascending s, and the row is padded with -1 to k
 * entries.  -0.0 and +0.0 compare equal.  NaN scores are not supported. */
void oracle_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                        int k, int32_t* idx);

/* Sparse attention over the latent cache.  For each (b,t,h), the slots j of
 * idx[b,t,:] with 0 <= idx < L_cap are used (other values are skipped):
 * z_j = sm_scale * sum_{d<D} Q[b,t,h,d] * C[b,idx_j,d]; p = softmax(z);
 * out[b,t,h,v] = sum_j p_j * C[b,idx_j,v] for v < D_v; lse = log sum_j exp z_j.
 * All arithmetic in double.  An empty set gives out = 0 and lse = -inf.
 * Q and C hold bf16 bit patterns. */
void oracle_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                              int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                              float sm_scale, double* out, double* lse);

/* Value of an OCP FP8 E4M3 code (bias 7, subnormals m * 2^-9, no infinities,
 * S.1111.111 = NaN, largest finite 448). */
double oracle_e4m3_to_double(uint8_t code);

/* oracle_sparse_mla_attend over an FP8 latent cache: row s of sequence b
 * stands for C[b,s,d] = e4m3(C8[b,s,d]) * 2^(Ce[b,s] - 127) for d < D_c and
 * Cr[b,s,d-D_c] (bf16) for D_c <= d < D_c + D_r; D = D_c + D_r, D_v = D_c.
 * C8 [B,L_cap,D_c] codes, Ce [B,L_cap] exponent bytes, Cr [B,L_cap,D_r]. */
void oracle_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                  const uint16_t* Cr, const int32_t* idx, int B, int Tq, int H,
                                  int D_c, int D_r, int L_cap, int k, float sm_scale,
                                  double* out, double* lse);

/* counts [B,L_cap] += occurrences of each position s in [0, L_cap) among the
 * slots of idx [B,Tq,k]; other slot values are ignored. */
void oracle_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                            uint32_t* counts);

/* Paged caches: logical row s of sequence b is row
 * table[b][s / block_size] * block_size + s % block_size of the page pool
 * ([n_pages, block_size, row]) when that entry is in [0, n_pages), else
 * unallocated.  L_cap = max_blocks * block_size.  The scores equal
 * oracle_indexer_scores on the logical cache, with -inf at unallocated
 * positions; attention equals oracle_sparse_mla_attend on the logical cache
 * with slots at unallocated positions skipped. */
void oracle_indexer_scores_paged(const int8_t* qI, const float* w, const int8_t* kI_pages,
                                 const int32_t* table, int max_blocks, int block_size,
                                 int n_pages, const int32_t* kv_len, int B, int Tq, int H_I,
                                 int D_I, float* S);
void oracle_sparse_mla_attend_paged(const uint16_t* Q, const uint16_t* C_pages,
                                    const int32_t* table, int max_blocks, int block_size,
                                    int n_pages, const int32_t* idx, int B, int Tq, int H, int D,
                                    int D_v, int k, float sm_scale, double* out, double* lse);

/* One layer group.  When reuse_idx is 0 the index set is computed once from
 * (qI[0], w[0], kI[0]) and written to idx; when it is 1 idx is read as given
 * (later MTP draft steps).  When per_layer_indexer is 1 every layer l computes
 * its own set from (qI[l], w[l], kI[l]) and idx ends holding the last layer's.
 * Then out[l] = attend(Q[l], C[l], idx) for l < n_layers.  S_scratch must
 * hold B*Tq*L_cap floats. */
void oracle_group_forward(int B, int Tq, int L_cap, int H_I, int D_I, int k, int H, int D,
                          int D_v, int n_layers, float sm_scale,
                          const int8_t* const* qI, const float* const* w,
                          const int8_t* const* kI, const int32_t* kv_len,
                          const uint16_t* const* Q, const uint16_t* const* C,
                          double* const* out, double* const* lse, int32_t* idx,
                          int reuse_idx, int per_layer_indexer, float* S_scratch);

#ifdef __cplusplus
}
#endif
#endif
