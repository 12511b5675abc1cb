/*
 * isa.h - C ABI of the IndexShare sparse-attention library for MI355X (gfx950).
 *
 * One IndexShare layer group of DeepSeek-style sparse attention (DSA) as
 * GLM-5.2 uses it: a lightning indexer scores every cached token for each
 * query, a top-k keeps the best positions, and the layers of the group each
 * run sparse attention over their own latent cache at those same positions.
 * Sources (the pages describing the method):
 *   [P4]  "GLM-5.2 Explained: 1M Token Context AI Agent Model",
 *         section 2.1 (IndexShare: Cross-Layer Index Sharing for DSA Sparse
 *         Attention): the relevance score I(t,s) = w * sigma(q_t . h_s) over
 *         all earlier tokens, the top-K selection, attention that loads keys
 *         and values only at the selected positions, and the compute-or-reuse
 *         rule for the layers of a group; section 2.2.1: later MTP draft
 *         steps reuse the first step's top-k and append nothing to the cache.
 *   [P3]  "GLM-5.2核心技术解析：IndexShare架构与MTP层优化详解", the config.json
 *         fragments: index_topk = 2048, index_topk_freq = 4,
 *         index_share_for_mtp_iteration = true; kv_lora_rank = 512.
 *   [P1]  "GLM-5.2 技术报告解读：IndexShare 稀疏注意力与反奖励作弊强化学习",
 *         section 1, training-strategy table: the indexer sits in the first of
 *         every four sparse layers and the other three reuse its top-k;
 *         section 4: FP8 KV cache among the serving optimisations.
 *   [P5]  "GLM-5.2 深度技术解析：智谱百万上下文旗舰模型的架构创新与工程实践",
 *         HiSparse memory-management section: per-position access counts of
 *         the top-k sets drive hot/cold cache placement.
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays owned by
 *    the caller.  The library never allocates, frees or keeps caller memory;
 *    scratch memory comes only from the caller's workspace.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on that stream and returns without synchronising.
 *  - Sequence b holds kv_len[b] cache entries (a DEVICE array of B int32;
 *    kernels clamp each value to [0, L_cap]).  Its Tq queries are the last
 *    Tq entries, so query t sits at pos(b,t) = kv_len[b] - Tq + t and sees
 *    positions 0..pos(b,t), itself included.  A query with pos < 0 sees
 *    nothing.
 *  - Arguments are checked on the host before any GPU work.  A failed check
 *    returns a negative isa_status, launches nothing, and leaves a message
 *    for isa_last_error().  Faults that happen on the GPU surface at the
 *    caller's next synchronisation.
 *  - Workspaces: a call that needs scratch memory takes (ws, ws_bytes), sized
 *    by the matching *_workspace_bytes query, 256-byte aligned.  Its contents
 *    need no initialisation (each call clears what it needs with a fill
 *    kernel, never a memset, so calls can be captured in HIP graphs) and are
 *    meaningless after the call.  One workspace serves one call at a time.
 *  - The library keeps no mutable global state; calls on different streams
 *    with different workspaces may overlap.
 */
#ifndef ISA_H
#define ISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISA_ABI_VERSION 3
#define ISA_MAX_TOPK 2048            /* index_topk of [P3] */
#define ISA_MAX_LCAP (1 << 21)       /* positions must fit 21 bits */

typedef enum {
    ISA_OK = 0,
    ISA_ERR_INVALID_ARG = -1,  /* NULL pointer, non-positive size, k out of range, ... */
    ISA_ERR_UNSUPPORTED = -2,  /* shape outside the compiled set */
    ISA_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small */
    ISA_ERR_HIP = -4           /* a HIP launch or runtime call failed */
} isa_status;

/* ABI version of the loaded library (ISA_ABI_VERSION when it matches this header). */
int isa_abi_version(void);

/* Message of the last failed call on this thread ("" when none). */
const char* isa_last_error(void);

/*
 * Lightning-indexer scores ([P4] section 2.1, relevance score I(t,s)).
 *   S[b,t,s] = sum_h w[b,t,h] * ReLU( sum_d qI[b,t,h,d] * kI[b,s,d] )   for s <= pos(b,t)
 *   S[b,t,s] = -inf                                                    for s >  pos(b,t)
 * qI  [B,Tq,H_I,D_I] int8; w [B,Tq,H_I] fp32 (one weight per query and head);
 * kI  [B,L_cap,D_I] int8, one key per token shared by all indexer heads;
 * S   [B,Tq,L_cap] fp32 output.
 * Dot products are exact (int8 MFMA, int32 accumulate); the head sum is fp32.
 * When every partial head sum is exactly representable in fp32 (for example
 * int8 values in [-8,7], D_I <= 128 and weights in {1/4,1/2,1,2}) the result is
 * the exact score, identical to any other summation order.
 * Supported: H_I in {4,8,16,32,64}, D_I in {32,64,128}.
 */
isa_status isa_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                              const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                              int L_cap, float* S, void* stream);

/*
 * Top-k position select ([P4] section 2.1: keep the top-K positions;
 * K = index_topk of [P3]).  For every (b,t) the candidates are s in
 * [0, pos(b,t)]; the min(k, pos+1) of them that come first under the total
 * order (S descending, then s ascending) are written to idx[b,t,:] in
 * ascending s, followed by -1 up to k entries.  -0.0 equals +0.0; scores must
 * not be NaN (their placement is unspecified).
 * S [B,Tq,L_cap] fp32; idx [B,Tq,k] int32 output.  1 <= k <= ISA_MAX_TOPK,
 * L_cap <= ISA_MAX_LCAP.
 */
size_t isa_topk_workspace_bytes(int B, int Tq, int L_cap, int k);
isa_status isa_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                           int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse latent (absorbed-MLA) attention over the selected positions
 * ([P4] section 2.1: keys and values are loaded only at the selected
 * positions; the latent row is kv_lora_rank = 512 wide plus a RoPE slice).
 * For each (b,t,h), over the slots j with 0 <= idx[b,t,j] < L_cap (other
 * values, -1 padding included, are skipped):
 *   z_j = sm_scale * sum_{d<D} Q[b,t,h,d] * C[b,idx_j,d]
 *   out[b,t,h,:] = sum_j softmax(z)_j * C[b,idx_j,0:D_v]      (bf16, RNE)
 *   lse[b,t,h]   = log sum_j exp(z_j)                          (fp32, optional)
 * An empty set gives out = 0 and lse = -inf.
 * Q [B,Tq,H,D] bf16 (post-RoPE, absorbed); C [B,L_cap,D] bf16; idx [B,Tq,k];
 * out [B,Tq,H,D_v] bf16; lse [B,Tq,H] fp32 or NULL.
 * bf16 MFMA with fp32 accumulation and an fp32 online softmax.
 * Supported: (D, D_v) in {(576, 512), (160, 128)}, 1 <= H <= 64,
 * 1 <= k <= ISA_MAX_TOPK, sm_scale finite and > 0 (a softmax temperature).
 */
size_t isa_attend_workspace_bytes(int B, int Tq, int H, int D, int D_v, int k);
isa_status isa_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                                 int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                                 float sm_scale, uint16_t* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * The same attention over an FP8 latent cache (the FP8 KV cache the pages
 * name among the serving optimisations: [P1] section 4, [P4] section 3).
 * Row s of sequence b is stored as
 *   C8[b,s,0:D_c]  OCP FP8 E4M3 codes of the latent dims (bias 7, max 448),
 *   Ce[b,s]        one byte e: the row's scale is 2^(e - 127) (UE8M0),
 *   Cr[b,s,0:D_r]  the RoPE dims in bf16,
 * and stands for the bf16 row C[b,s,d] = e4m3(C8[b,s,d]) * 2^(Ce[b,s]-127)
 * for d < D_c and Cr[b,s,d-D_c] for D_c <= d < D_c + D_r.  The result is
 * isa_sparse_mla_attend on that row with D = D_c + D_r and D_v = D_c (the
 * values are the dequantized latent dims).  The kernel dequantizes to bf16,
 * which is exact while every dequantized value is a normal bf16 number (for
 * example e in [10, 246]); E4M3 NaN codes (0x7F, 0xFF) give unspecified
 * values.  Supported: (D_c, D_r) in {(512, 64), (128, 32)}; other conditions
 * and the workspace as for isa_sparse_mla_attend with D = D_c + D_r.
 */
size_t isa_attend_fp8_workspace_bytes(int B, int Tq, int H, int D_c, int D_r, int k);
isa_status isa_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                     const uint16_t* Cr, const int32_t* idx, int B, int Tq, int H,
                                     int D_c, int D_r, int L_cap, int k, float sm_scale,
                                     uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * Paged caches (the paged KV memory of serving engines, [P4] sections 3 and
 * 5).  A cache of rows (kI: D_I int8; C: D bf16) is split into pages of
 * block_size consecutive positions held in a pool [n_pages, block_size, row];
 * block_table [B, max_blocks] int32 maps logical block j of sequence b (its
 * positions j*block_size .. +block_size-1) to a pool page.  Entries outside
 * [0, n_pages) mark unallocated blocks: their positions score -inf in the
 * indexer and are skipped by attention.  The logical capacity is
 * L_cap = max_blocks * block_size; everything else (S, idx, out, positions)
 * is as for the contiguous calls, which these equal on the same logical
 * cache.  block_size is a power of two in [32, 65536];
 * n_pages * block_size < 2^31; L_cap <= ISA_MAX_LCAP.
 */
isa_status isa_indexer_scores_paged(const int8_t* qI, const float* w, const int8_t* kI_pages,
                                    const int32_t* block_table, int max_blocks, int block_size,
                                    int n_pages, const int32_t* kv_len, int B, int Tq, int H_I,
                                    int D_I, float* S, void* stream);
isa_status isa_sparse_mla_attend_paged(const uint16_t* Q, const uint16_t* C_pages,
                                       const int32_t* block_table, int max_blocks,
                                       int block_size, int n_pages, const int32_t* idx, int B,
                                       int Tq, int H, int D, int D_v, int k, float sm_scale,
                                       uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                       void* stream);

/*
 * Access counts of an index set, the input of hot/cold cache placement
 * ([P5] "GLM-5.2 深度技术解析：智谱百万上下文旗舰模型的架构创新与工程实践",
 * HiSparse memory-management section: every attention step adds one access to
 * each position the top-k selected):
 *   counts[b,s] += |{ (t,j) : idx[b,t,j] == s }|   for 0 <= s < L_cap.
 * Slot values outside [0, L_cap) (the -1 padding included) are ignored.
 * idx [B,Tq,k] int32; counts [B,L_cap] uint32, accumulated (the caller zeroes
 * it to start a count; a uint32 count wraps after 2^32 accesses).  The result
 * is exact and independent of the order of the additions.
 * 1 <= k <= ISA_MAX_TOPK, L_cap <= ISA_MAX_LCAP.
 */
isa_status isa_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                               uint32_t* counts, void* stream);

/*
 * One IndexShare layer group ([P1] section 1 table; [P4] sections 2.1 and
 * 2.2.1; index_topk_freq and index_share_for_mtp_iteration of [P3]).
 *  - reuse_idx = 0, per_layer_indexer = 0: indexer + top-k run once from
 *    (qI[0], w[0], kI[0]) and write idx; then every layer l < n_layers runs
 *    sparse attention out[l] = attend(Q[l], C[l], idx), in layer order.
 *  - reuse_idx = 1: idx is read as given and the indexer does not run (the
 *    later MTP draft steps, which reuse the first step's set).
 *  - per_layer_indexer = 1: the baseline without sharing; layer l runs its
 *    own indexer + top-k from (qI[l], w[l], kI[l]) before its attention, and
 *    idx ends holding the last layer's set.
 * The pointer arrays (qI, w, kI, Q, C, out, lse, C8, Ce, Cr) are HOST arrays
 * read during the call only; the tensors they point to are device memory.
 * lse may be NULL, or an array whose entries may be NULL.
 * kv_fp8 = 1: the layers' latent caches are FP8 as in isa_sparse_mla_attend_fp8
 * (D_c = D_v, D_r = D - D_v); C is ignored and C8, Ce, Cr hold n_layers entries.
 * paged = 1: kI and every layer's cache (C, or C8/Ce/Cr) are page pools of
 * n_pages pages sharing block_table (as in isa_sparse_mla_attend_paged), and
 * L_cap must equal max_blocks * block_size.
 */
typedef struct {
    int B, Tq, L_cap;
    int H_I, D_I, k;
    int H, D, D_v;
    int n_layers;                      /* index_topk_freq: 4 in GLM-5.2 */
    float sm_scale;
    const int8_t* const* qI;           /* 1 entry, or n_layers with per_layer_indexer */
    const float* const* w;
    const int8_t* const* kI;
    const int32_t* kv_len;             /* device [B] */
    const uint16_t* const* Q;          /* n_layers entries */
    const uint16_t* const* C;          /* n_layers entries */
    uint16_t* const* out;              /* n_layers entries */
    float* const* lse;                 /* NULL, or n_layers entries (each may be NULL) */
    int32_t* idx;                      /* device [B,Tq,k]: written, or read with reuse_idx */
    int reuse_idx;
    int per_layer_indexer;
    void* ws;
    size_t ws_bytes;
    int kv_fp8;
    const uint8_t* const* C8;          /* n_layers entries with kv_fp8 */
    const uint8_t* const* Ce;
    const uint16_t* const* Cr;
    int paged;
    const int32_t* block_table;        /* device [B, max_blocks] with paged */
    int max_blocks, block_size, n_pages;
} isa_group_args;

size_t isa_group_workspace_bytes(const isa_group_args* args);
isa_status isa_group_forward(const isa_group_args* args, void* stream);

/*
 * isa_group_forward for callers that cannot allocate memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call takes its scratch memory from a fixed array of
 * ISA_NOALLOC_SCRATCH_BYTES inside the library (one copy per GPU, held until
 * the process ends) instead of args->ws, which is ignored (ws and ws_bytes
 * may be 0); everything else, results included, is as for isa_group_forward.
 * It calls no hipMalloc, hipFree or other allocating routine.
 *  - A call whose isa_group_workspace_bytes(args) exceeds
 *    ISA_NOALLOC_SCRATCH_BYTES returns ISA_ERR_WORKSPACE and launches
 *    nothing (the decode shapes of up to 64 queries x 128K positions fit;
 *    a 4096-query prefill does not).
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents (each call clears what it needs first): calls that may
 *    overlap on one GPU (other streams, other threads) race with each other
 *    and must not be issued concurrently.
 *  - The first call on a device looks up the device address of the array
 *    (a failure there returns ISA_ERR_HIP).
 */
#define ISA_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t isa_group_noalloc_max_bytes(void);
isa_status isa_group_forward_noalloc(const isa_group_args* args, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ISA_H */
