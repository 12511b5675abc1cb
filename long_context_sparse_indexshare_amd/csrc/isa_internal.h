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

// Order-preserving 32-bit image of an fp32 score (larger score, larger
// key; -0.0 ranks as +0.0).  Key 0 is below every score's key (-inf maps
// to 0x007FFFFF) and marks "no value" in the top-k summaries.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of an unsigned value over the 64 lanes of a wave (every lane
// active), in registers: DPP row shifts take each 16-lane row's maximum to
// its lane 15, two row broadcasts carry it to lane 63.  0 is the identity.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    uint32_t v = x;
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

// Top-k summary of a wave's values: the M largest keys (with multiplicity)
// among the NV keys each lane holds, in descending order, each with the
// 8-bit code of its position (codes[i] belongs to k[i]); lane r < M writes
// the r-th to dst[r] and its code to cdst[r].  Key 0 (no value) pads the list
// when the wave holds fewer; which of several equal keys is kept is
// unspecified.  Every lane first sorts its own (key, code) pairs (a small
// sorting network), then each of the M rounds takes the wave maximum of the
// lanes' heads and advances the head of the lowest lane holding it.  All 64
// lanes must be active, and M <= 64 (the callers' M is at most 32).
template <int NV>
__device__ __forceinline__ void sort_keys_desc(uint32_t (&k)[NV], uint32_t (&c)[NV]) {
    auto cas = [&](int i, int j) {
        const bool sw = k[j] > k[i];
        const uint32_t a = k[i], b = k[j], ca = c[i], cb = c[j];
        k[i] = sw ? b : a;
        k[j] = sw ? a : b;
        c[i] = sw ? cb : ca;
        c[j] = sw ? ca : cb;
    };
    if constexpr (NV == 4) {
        cas(0, 1); cas(2, 3); cas(0, 2); cas(1, 3); cas(1, 2);
    } else if constexpr (NV == 8) {
        cas(0, 2); cas(1, 3); cas(4, 6); cas(5, 7);
        cas(0, 4); cas(1, 5); cas(2, 6); cas(3, 7);
        cas(0, 1); cas(2, 3); cas(4, 5); cas(6, 7);
        cas(2, 4); cas(3, 5);
        cas(1, 4); cas(3, 6);
        cas(1, 2); cas(3, 4); cas(5, 6);
    } else {
        static_assert(NV == 4 || NV == 8, "summary lanes hold 4 or 8 keys");
    }
}

template <int NV>
__device__ __forceinline__ void wave_top_m(uint32_t (&k)[NV], uint32_t (&c)[NV], int M,
                                           uint32_t* __restrict__ dst, uint8_t* __restrict__ cdst) {
    sort_keys_desc<NV>(k, c);
    const int lane = threadIdx.x & 63;
    uint32_t mine = 0u, mine_code = 0u;
    for (int r = 0; r < M; ++r) {
        const uint32_t m = wave_max_u32(k[0]);
        const uint64_t hit = __ballot(k[0] == m);
        const int winner = (int)__builtin_ctzll(hit);
        const uint32_t code = (uint32_t)__builtin_amdgcn_readlane((int)c[0], winner);
        // the r-th key and its code go straight into lane r (both are
        // uniform; the lane select is M0, since one VALU instruction reads
        // one SGPR here); the wait states cover the SGPRs just written by
        // v_readlane and the M0 write
        asm("s_nop 4\n\tv_writelane_b32 %0, %2, m0\n\tv_writelane_b32 %1, %3, m0"
            : "+v"(mine), "+v"(mine_code)
            : "s"(m), "s"(code), "{m0}"(r));
        // the winner's lane mask straight from the scalar unit (no compare)
        if (__builtin_amdgcn_inverse_ballot_w64(1ull << winner)) {
#pragma unroll
            for (int i = 0; i + 1 < NV; ++i) {
                k[i] = k[i + 1];
                c[i] = c[i + 1];
            }
            k[NV - 1] = 0u;
        }
    }
    if (lane < M) {
        dst[lane] = mine;
        cdst[lane] = (uint8_t)mine_code;
    }
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
constexpr int TOPK_THREADS = 1024;          // filter workgroup: 4 scores per thread
constexpr int TOPK_CHUNK = 4096;            // scores per filter workgroup
constexpr int TOPK_PER_THREAD = TOPK_CHUNK / TOPK_THREADS;
constexpr int TOPK_HIST_BITS = 12;          // first radix digit of the prefill path: key bits [31:20]
constexpr int TOPK_HIST_BINS = 1 << TOPK_HIST_BITS;
constexpr int TOPK_MAX_CHUNKS = (1 << 21) / TOPK_CHUNK;   // positions fit 21 bits
// The summary: for every set of 256 positions (a "wave chunk": the keys one
// wave of the indexer's decode workgroup scores), its M largest keys and the
// 8-bit code of each one's position.  Wave chunk 4c + w holds positions
// 1024c + 32w + 128q + j (q < 8, j < 32), position code 32q + j.  M is
// chosen per call (topk_layout).
constexpr int TOPK_WAVE_CHUNK = 256;
constexpr int TOPK_MAX_M = 16;              // filter path
constexpr int TOPK_DIRECT_MAX_M = 32;       // direct path
constexpr int TOPK_FEW_ROWS = 16;           // direct path: rows whose summary kernel is cheap
constexpr int TOPK_MAX_SUMMARY = 8192;      // summary keys per row at most (8 per filter thread)
// Entry slots per filter chunk: one per position, so a chunk's run always fits.
constexpr int TOPK_SLOT_CAP = TOPK_CHUNK;

struct TopkLayout {
    size_t zero_bytes;                // counters: [0, zero_bytes) is cleared per call
    size_t hist;                      // first-digit histograms (prefill select path)
    size_t summary, codes, counts, ent, total;
    int rows, nchunks;                // filter chunks of TOPK_CHUNK positions per row
    int nwchunks, M;                  // wave chunks per row, summary keys per wave chunk
    bool select;                      // one-workgroup-per-row select path (prefill)
    bool direct;                      // one workgroup per row from the summary (decode)
};
// Where the indexer writes the top-k summary (keys [rows][nwchunks][M] and
// their position codes, same shape); keys == nullptr: no summary.
struct SummaryOut {
    uint32_t* keys;
    uint8_t* codes;
    int M;
};
// fused: the indexer's epilogue writes the summary (decode group calls)
TopkLayout topk_layout(int rows, int L_cap, int k, bool fused = false);
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
// the group call that follows), or zero_n = 0.  summary.keys != nullptr: the
// indexer also writes the top-k summary (M keys and codes per wave chunk)
// when it can (indexer_writes_summary); the caller checks that first.
hipError_t launch_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                                 const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                                 int L_cap, float* S, uint32_t* zero, uint32_t zero_n,
                                 hipStream_t stream, PageMap pm = PageMap{nullptr, 0, 0, 0},
                                 SummaryOut summary = SummaryOut{nullptr, nullptr, 0});
bool indexer_writes_summary(int Tq, int H_I);
// counters_clear: the caller already zeroed the first topk_layout().zero_bytes;
// summary_ready: the summary in the workspace was written by the indexer
hipError_t launch_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                              int k, int32_t* idx, void* ws, bool counters_clear,
                              hipStream_t stream, bool summary_ready = false);
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
