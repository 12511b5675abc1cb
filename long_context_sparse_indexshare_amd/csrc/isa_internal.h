// Internal declarations shared by the HIP translation units of libisa.
// Not part of the public ABI (that is include/isa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace isa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

// Sum and maximum of x over lanes i and i ^ 32 of a wave, the same bits in
// both halves (the low half's value is always the left operand).
// v_permlane32_swap exchanges the two 32-lane halves in registers; a
// __shfl_xor(x, 32) goes through the LDS crossbar (ds_bpermute) and waits
// for it.
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Paged caches: logical position s of sequence b lives in row
// (page << shift) + (s & ((1 << shift) - 1)) of the page pool, where page =
// table[b * max_blocks + (s >> shift)]; pages outside [0, n_pages) are
// unallocated.  table == nullptr: the cache is contiguous, [B, L_cap, row].
struct PageMap {
    const int32_t* table;
    int max_blocks;
    int shift;                        // log2 of the page size (>= 5)
    int n_pages;
};

// Top-k geometry (shared by the host sizing code and the kernels).
constexpr int TOPK_THREADS = 1024;          // classify workgroup: 4 scores per thread
constexpr int TOPK_CHUNK = 4096;            // scores per workgroup
constexpr int TOPK_PER_THREAD = TOPK_CHUNK / TOPK_THREADS;
constexpr int TOPK_HIST_BITS = 12;          // first radix digit: key bits [31:20]
constexpr int TOPK_HIST_BINS = 1 << TOPK_HIST_BITS;
constexpr int TOPK_MAX_CHUNKS = (1 << 21) / TOPK_CHUNK;   // positions fit 21 bits

struct TopkLayout {
    size_t hist, hist2, alloc, zero_bytes;   // counters: [0, zero_bytes) is cleared per call
    size_t row_state, runs, ent, total;
    int rows, nchunks;
    uint32_t cap;                     // entries per row in the entry buffer
};
TopkLayout topk_layout(int rows, int L_cap);
// true when the one-workgroup-per-row select kernel serves (rows, L_cap)
bool topk_uses_select(int rows, int L_cap);

// Attention split geometry; the workspace of one call holds the partials.
struct AttendPlan {
    int splits;            // workgroups per (query, head block, column part) along the k slots
    int slots_per_split;
    int head_blocks;       // 32-head blocks per workgroup
    int col_parts;         // value-column parts (workgroups) per head block
    size_t part_o_off, part_ml_off, partial_bytes;   // 0 bytes when not split
};
AttendPlan attend_plan(int B, int Tq, int H, int D, int D_v, int k);

// Launchers (host side; argument checking happens in the API layer).
hipError_t launch_clear_u32(uint32_t* p, size_t n, hipStream_t stream);
// zero[0, zero_n): words the indexer grid also sets to 0 (the top-k counters of
// the group call that follows), or zero_n = 0
hipError_t launch_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                                 const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                                 int L_cap, float* S, uint32_t* zero, uint32_t zero_n,
                                 hipStream_t stream, PageMap pm = PageMap{nullptr, 0, 0, 0});
// counters_clear: the caller already zeroed the first topk_layout().zero_bytes
hipError_t launch_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                              int k, int32_t* idx, void* ws, bool counters_clear,
                              hipStream_t stream);
hipError_t launch_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                                    int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                                    float sm_scale, uint16_t* out, float* lse, void* partials,
                                    hipStream_t stream, PageMap pm = PageMap{nullptr, 0, 0, 0});

// FP8 latent cache: C8 [B,L_cap,D_v] E4M3 codes, Ce [B,L_cap] exponent bytes,
// Cr [B,L_cap,D-D_v] bf16 RoPE slices; otherwise as launch_sparse_mla_attend.
hipError_t launch_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                        const uint16_t* Cr, const int32_t* idx, int B, int Tq,
                                        int H, int D, int D_v, int L_cap, int k, float sm_scale,
                                        uint16_t* out, float* lse, void* partials,
                                        hipStream_t stream, PageMap pm = PageMap{nullptr, 0, 0, 0});

// counts [B,L_cap] += occurrences of each position in idx [B,Tq,k]
hipError_t launch_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                                  uint32_t* counts, hipStream_t stream);

bool indexer_shape_supported(int H_I, int D_I);
bool attend_shape_supported(int H, int D, int D_v);

}  // namespace isa
