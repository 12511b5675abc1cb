// Lightning-indexer scores on int8 MFMA (gfx950).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1, relevance score I(t,s) = w * sigma(q_t . h_s), read with sigma = ReLU,
// a sum over indexer heads and one weight per query and head):
//   S[b,t,s] = sum_h w[b,t,h] * ReLU(qI[b,t,h,:] . kI[b,s,:])  for s <= pos(b,t), else -inf.
//
// Work split: the GEMM rows are (query, head) pairs, 64 per workgroup
// (64 / H_I queries of one sequence); the columns are keys.  Each of the
// 4 waves owns a 32-key block per step, so the 64 query rows stay in
// registers (A operands) and every key byte is read from HBM exactly once
// per workgroup with 16-byte loads straight into B operands.  The MFMA is
// v_mfma_i32_32x32x32_i8 (exact int32 dot products).  The epilogue applies
// ReLU and the head weight in fp32 and reduces the heads of a query in
// registers plus one cross-lane swap; blocks past the last visible key of
// every query in the workgroup read a zero row instead of keys (no HBM
// traffic, no MFMA) and write -inf.  Each wave
// keeps the next two key blocks' loads in flight while it computes the
// current one; with one query per workgroup the scores are staged in LDS and
// written after the last block, four contiguous floats per thread.
#include <type_traits>

#include "isa_internal.h"

namespace isa {
namespace {

constexpr int IX_THREADS = 256;
constexpr int IX_ROWS = 64;              // (query, head) rows per workgroup
constexpr int IX_KEYS_PER_STEP = 128;    // 4 waves x 32 keys
constexpr int IX_STEPS = 8;
constexpr int IX_KEYS_PER_WG = IX_KEYS_PER_STEP * IX_STEPS;
constexpr int IX_DEPTH = 3;              // key blocks per wave: 1 computed + 2 in flight

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// Key bytes read by lanes that have no live key (the largest D_I is 128).
__device__ __attribute__((aligned(16))) int8_t g_zero_keys[128];
typedef const __attribute__((address_space(1))) v4i* global_v4i_ptr;

// Zeroes zero[0, zero_n) with the whole grid (the next launch's counters; it
// saves that launch a fill kernel of its own).
__device__ __forceinline__ void grid_clear(uint32_t* __restrict__ zero, uint32_t zero_n) {
    if (zero_n == 0) return;
    const uint32_t wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t nwg = gridDim.x * gridDim.y * gridDim.z;
    for (uint32_t i = wg * IX_THREADS + threadIdx.x; i < zero_n; i += nwg * IX_THREADS) zero[i] = 0u;
}

// First cache row of the 32-key block at logical position s0 (a multiple of
// 32) of sequence b, or -1 when its page is unallocated.  A page holds a
// power-of-two number (>= 32) of keys, so a block never straddles pages;
// s0 is wave-uniform, so the table read is a scalar load.
__device__ __forceinline__ long long key_block_row(const PageMap& pm, int b, int L_cap, int s0) {
    if (pm.table == nullptr) return (long long)b * L_cap + s0;
    const int blk = __builtin_amdgcn_readfirstlane(s0 >> pm.shift);
    const int page = pm.table[(size_t)b * pm.max_blocks + blk];
    if (page < 0 || page >= pm.n_pages) return -1;
    return ((long long)page << pm.shift) + (s0 & ((1 << pm.shift) - 1));
}

template <int H_I, int D_I>
__global__ __launch_bounds__(IX_THREADS) void indexer_scores_kernel(
    const int8_t* __restrict__ qI, const float* __restrict__ w, const int8_t* __restrict__ kI,
    const int32_t* __restrict__ kv_len, int Tq, int L_cap, float* __restrict__ S,
    uint32_t* __restrict__ zero, uint32_t zero_n, PageMap pm, SummaryOut summary) {
    grid_clear(zero, zero_n);
    constexpr int QPW = IX_ROWS / H_I;             // queries per workgroup
    constexpr int KS = D_I / 32;                   // MFMA k-steps over the indexer dim
    constexpr int NQL = H_I >= 8 ? 64 / H_I : 8;   // query slots held per lane
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int g = lane >> 5;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * QPW;
    const int len = clamp_len(kv_len[b], L_cap);
    const int t_last = min(t0 + QPW, Tq) - 1;
    const int pos_max = len - Tq + t_last;          // last key any query here can see

    // A operands: row m = 32*rb + j is (query m / H_I, head m % H_I); k bytes 32*ks + 16*g .. +16.
    v4i a[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int m = 32 * rb + j;
        const int t = t0 + m / H_I;
        const int h = m % H_I;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (t < Tq) {
                a[rb][ks] = *reinterpret_cast<const v4i*>(
                    qI + (((size_t)b * Tq + t) * H_I + h) * D_I + 32 * ks + 16 * g);
            } else {
                a[rb][ks] = v4i{0, 0, 0, 0};
            }
        }
    }
    // Head weight of every accumulator register: register r of block rb holds row
    // 32*rb + 8*(r/4) + 4*g + r%4 (the 32x32 MFMA output layout).
    float wr[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * rb + 8 * (r / 4) + 4 * g + (r % 4);
            const int t = t0 + m / H_I;
            wr[rb][r] = t < Tq ? w[((size_t)b * Tq + t) * H_I + (m % H_I)] : 0.0f;
        }
    }

    // B operands of one 32-key block: lane (key s0 + j, half g) holds k bytes
    // 32*ks + 16*g .. +16.  Lanes without a live key read the zero row instead:
    // the loads are unconditional, so the compiler can count them and wait
    // only for the block about to be used, not for the ones behind it.
    const uintptr_t zero_row = reinterpret_cast<uintptr_t>(g_zero_keys);
    auto load_keys = [&](int s0, v4i* bk) {
        const int s = s0 + j;
        const long long r0 = s0 <= pos_max && s0 < L_cap ? key_block_row(pm, b, L_cap, s0) : -1;
        const bool live = r0 >= 0 && s < L_cap;
        const uintptr_t src =
            (live ? reinterpret_cast<uintptr_t>(kI + (size_t)(r0 + j) * D_I) : zero_row) + 16 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bk[ks] = *(global_v4i_ptr)(src + 32 * ks);
    };

    // With one query per workgroup (H_I = 64) each step's scores wait in
    // registers and are written once after the loop: stores and loads share
    // one in-order counter, so a store between the key blocks would make the
    // wait for each later block also wait for the store.
    float res[IX_STEPS];
    uint32_t visb = 0;                 // which of res[] are visible scores (lanes with g == 0)
#pragma unroll
    for (int st = 0; st < IX_STEPS; ++st) res[st] = -__builtin_inff();
    // ring of IX_DEPTH key blocks per wave: the one being computed and the
    // next IX_DEPTH - 1 in flight (the loop is unrolled, so the ring indices
    // are constants and the blocks stay in registers)
    const int key_base = blockIdx.x * IX_KEYS_PER_WG + wave * 32;
    v4i ring[IX_DEPTH][KS];
#pragma unroll
    for (int p = 0; p < IX_DEPTH - 1; ++p) load_keys(key_base + p * IX_KEYS_PER_STEP, ring[p]);
    // (blocks at or past L_cap load zeros and store nothing; no early exit, so
    // the loop unrolls fully)
#pragma unroll
    for (int step = 0; step < IX_STEPS; ++step) {
        const int s0 = key_base + step * IX_KEYS_PER_STEP;
        if (step + IX_DEPTH - 1 < IX_STEPS)
            load_keys(s0 + (IX_DEPTH - 1) * IX_KEYS_PER_STEP, ring[(step + IX_DEPTH - 1) % IX_DEPTH]);
        const v4i* bk = ring[step % IX_DEPTH];
        const int s = s0 + j;
        // positions on an unallocated page score -inf
        const bool page_ok = pm.table == nullptr || key_block_row(pm, b, L_cap, s0) >= 0;
        float sum[NQL];
#pragma unroll
        for (int q = 0; q < NQL; ++q) sum[q] = 0.0f;
        if (s0 <= pos_max) {
            v16i acc[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                acc[rb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rb][ks], bk[ks], acc[rb], 0, 0, 0);
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int sl = H_I >= 8 ? (32 * rb + 8 * (r / 4)) / H_I : 4 * rb + r / 4;
                    const int dot = acc[rb][r];
                    sum[sl] += wr[rb][r] * (float)(dot > 0 ? dot : 0);
                }
            }
            if (H_I >= 8) {
#pragma unroll
                for (int q = 0; q < NQL; ++q) sum[q] = xor32_sum(sum[q]);
            }
        }
        if (s < L_cap) {
#pragma unroll
            for (int q = 0; q < NQL; ++q) {
                int qt;
                if (H_I >= 8) {
                    if (g != 0) continue;        // both halves hold the total; one writes
                    qt = q;
                } else {
                    qt = 2 * q + g;
                }
                const int t = t0 + qt;
                if (t >= Tq) continue;
                const int pos = len - Tq + t;
                if constexpr (NQL == 1) {
                    const bool vis = s <= pos && page_ok;
                    res[step] = vis ? sum[q] : -__builtin_inff();
                    visb |= (uint32_t)vis << step;
                } else {
                    S[((size_t)b * Tq + t) * L_cap + s] =
                        s <= pos && page_ok ? sum[q] : -__builtin_inff();
                }
            }
        }
    }
    if constexpr (NQL == 1) {
        // the top-k summary of this wave's 256 keys (wave chunk 4 * blockIdx.x
        // + wave of the query's row; step st of key j is position code
        // 32 * st + j): their M largest score keys with their codes,
        // invisible positions counting as none.  The lanes with g = 1 take
        // steps 4-7 of key j from lane j (one lane swap each), so every lane
        // holds four keys.
        if (summary.keys != nullptr) {
            static_assert(IX_STEPS == 8 && IX_STEPS * 32 == TOPK_WAVE_CHUNK &&
                              IX_KEYS_PER_STEP == 128,
                          "a wave's keys are one summary wave chunk");
            uint32_t key[4], code[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (visb >> i) & 1u ? score_key(res[i]) : 0u;
                const uint32_t hi = (visb >> (4 + i)) & 1u ? score_key(res[4 + i]) : 0u;
                const auto r = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
                key[i] = g == 0 ? lo : r[0];             // r[0]: lane j's value
                code[i] = (uint32_t)(32 * (4 * g + i) + j);
            }
            const int M = summary.M;
            const size_t off = (((size_t)b * Tq + t0) * (gridDim.x * 4) + blockIdx.x * 4 + wave) * M;
            wave_top_m<4>(key, code, M, summary.keys + off, summary.codes + off);
        }
        // the workgroup's IX_KEYS_PER_WG scores are contiguous in S: stage them
        // in LDS in key order, then one 16-byte streaming store per thread
        static_assert(IX_KEYS_PER_WG % (4 * IX_THREADS) == 0, "whole 16-byte stores");
        __shared__ __attribute__((aligned(16))) float sres[IX_KEYS_PER_WG];
        if (g == 0) {
#pragma unroll
            for (int step = 0; step < IX_STEPS; ++step)
                sres[step * IX_KEYS_PER_STEP + wave * 32 + j] = res[step];
        }
        __syncthreads();
        const int t = t0;
        const int k0 = blockIdx.x * IX_KEYS_PER_WG;
        float* srow = S + ((size_t)b * Tq + t) * L_cap + k0;
        const bool a16 = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
#pragma unroll
        for (int c = 0; c < IX_KEYS_PER_WG / (4 * IX_THREADS); ++c) {
            const int e = (c * IX_THREADS + threadIdx.x) * 4;
            const v4f v = *reinterpret_cast<const v4f*>(&sres[e]);
            if (t < Tq) {
                if (k0 + e + 3 < L_cap && a16) {
                    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(srow + e));
                } else {
                    for (int u = 0; u < 4; ++u)
                        if (k0 + e + u < L_cap) srow[e + u] = v[u];
                }
            }
        }
    }
}

// Two or more queries per sequence (prefill, multi-query decode): every wave
// owns two queries (their 2 x 64 head rows, four 32-row MFMA blocks, stay in
// registers) and streams the key blocks of its workgroup's key range up to
// its last visible key; the four waves of a workgroup read the same key
// blocks at about the same time, so each key block comes from HBM / L2 once
// per workgroup and from L1 for the other waves.  The keys are split across
// workgroups too (blockIdx.z takes keys [z * chunk, (z+1) * chunk)), so few
// queries still fill the chip while every key block serves all the queries
// of its workgroup; waves without a query return at once.  The epilogue
// (ReLU, head weight, head sum) is the same as above.
constexpr int PF_QPWAVE = 2;
constexpr int PF_QPW = 4 * PF_QPWAVE;     // queries per workgroup
constexpr int PF_MIN_TQ = 2;              // from this many queries per sequence on
// key splits aim at this many workgroups: the ones that fit at once (two per
// CU), so a few queries per sequence run in one round of long workgroups
constexpr int PF_TARGET_WGS = 512;

template <int D_I>
__global__ __launch_bounds__(IX_THREADS, 2) void indexer_prefill_kernel(
    const int8_t* __restrict__ qI, const float* __restrict__ w, const int8_t* __restrict__ kI,
    const int32_t* __restrict__ kv_len, int Tq, int L_cap, int chunk, float* __restrict__ S,
    uint32_t* __restrict__ zero, uint32_t zero_n, PageMap pm) {
    grid_clear(zero, zero_n);
    constexpr int H_I = 64;
    constexpr int KS = D_I / 32;
    constexpr int RB = 2 * PF_QPWAVE;                 // 32-row blocks per wave
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 31;
    const int g = lane >> 5;
    const int b = blockIdx.y;
    const int tw = blockIdx.x * PF_QPW + wave * PF_QPWAVE;   // first query of this wave
    if (tw >= Tq) return;                  // no query here (no workgroup barrier follows)
    const int s_lo = blockIdx.z * chunk;                      // this workgroup's keys
    const int s_hi = min(s_lo + chunk, L_cap);
    const int len = clamp_len(kv_len[b], L_cap);

    // A operands: block rb holds heads 32*(rb%2) .. +32 of query tw + rb/2.
    // The head weights of the wave's queries sit in LDS (read only by the
    // fp32 epilogue; the wave writes and reads its own rows, in order), which
    // keeps 64 registers per lane free for occupancy.
    __shared__ __attribute__((aligned(16))) float sw[PF_QPW * H_I];
    v4i a[RB][KS];
    int pos[PF_QPWAVE];
#pragma unroll
    for (int q = 0; q < PF_QPWAVE; ++q) pos[q] = tw + q < Tq ? len - Tq + tw + q : -1;
    const int pos_max = max(pos[0], pos[PF_QPWAVE - 1]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int t = tw + rb / 2;
        const bool tv = t < Tq;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            a[rb][ks] = tv ? *reinterpret_cast<const v4i*>(
                                 qI + (((size_t)b * Tq + t) * H_I + 32 * (rb % 2) + j) * D_I +
                                 32 * ks + 16 * g)
                           : v4i{0, 0, 0, 0};
        }
    }
    float* const wq = sw + wave * PF_QPWAVE * H_I;     // this wave's queries' weights
#pragma unroll
    for (int q = 0; q < PF_QPWAVE; ++q)
        wq[q * H_I + lane] = tw + q < Tq ? w[((size_t)b * Tq + tw + q) * H_I + lane] : 0.0f;

    // Folded weights: when every head weight of the wave's queries is a power
    // of two 2^e with e in [-2, 1] and every query byte q keeps 4 * 2^e * q
    // inside int8, the A operands become q' = 4w * q (a left shift by e + 2),
    // and w * ReLU(q . k) = ReLU(q' . k) / 4 (w > 0): the head sum is then an
    // integer sum of ReLUs, converted to fp32 once and scaled by 1/4 (both
    // exact steps after the one rounding of the conversion, which is the
    // rounding of the exact score).  The check is per wave; a wave that fails
    // it takes the fp32 epilogue.
    bool lane_ok = true;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int t = tw + rb / 2;
        if (t >= Tq) continue;                     // zero operands: nothing to scale
        const uint32_t wb = __float_as_uint(w[((size_t)b * Tq + t) * H_I + 32 * (rb % 2) + j]);
        // 0.25, 0.5, 1, 2 are exponents 125..128 with a zero mantissa
        const uint32_t ex = (wb >> 23) & 0xFFu;
        const bool pow2 = (wb & 0x807FFFFFu) == 0u && ex >= 125u && ex <= 128u;
        const int sh = (int)ex - 125;
        // a byte times 2^sh fits int8 iff its top sh + 1 bits are equal
        const uint32_t m = (((0xFFu << (8 - sh)) & 0xFFu) * 0x01010101u) & (pow2 ? ~0u : 0u);
        uint32_t bad = 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t x = (uint32_t)a[rb][ks][c];
                bad |= (x ^ (x << 1)) & m;
            }
        lane_ok = lane_ok && pow2 && bad == 0u;
    }
    const bool fast = __ballot(!lane_ok) == 0ull;
    if (fast) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int t = tw + rb / 2;
            if (t >= Tq) continue;
            const uint32_t wb = __float_as_uint(w[((size_t)b * Tq + t) * H_I + 32 * (rb % 2) + j]);
            const int sh = (int)((wb >> 23) & 0xFFu) - 125;
            const uint32_t keep = ((0xFFu << sh) & 0xFFu) * 0x01010101u;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    a[rb][ks][c] = (int)(((uint32_t)a[rb][ks][c] << sh) & keep);
        }
    }

    // as in the decode kernel: unconditional loads, dead lanes read the zero row
    const uintptr_t zero_row = reinterpret_cast<uintptr_t>(g_zero_keys);
    auto load_keys = [&](int s0, v4i* bk) {
        const int s = s0 + j;
        const long long r0 =
            s0 <= pos_max && s0 < s_hi && s0 < L_cap ? key_block_row(pm, b, L_cap, s0) : -1;
        const bool live = r0 >= 0 && s < L_cap;
        const uintptr_t src =
            (live ? reinterpret_cast<uintptr_t>(kI + (size_t)(r0 + j) * D_I) : zero_row) + 16 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bk[ks] = *(global_v4i_ptr)(src + 32 * ks);
    };

    auto run = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        // the 16 products of one 32-key block (four accumulator chains, one per
        // row block, interleaved)
        auto products = [&](const v4i* bk, v16i (&acc)[RB]) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rb][ks], bk[ks], acc[rb], 0, 0, 0);
        };
        // the two queries' scores of a block from its products (lane j: key j)
        auto scores = [&](const v16i (&acc)[RB], float (&sum)[PF_QPWAVE]) {
            if constexpr (FAST) {
                // integer ReLU sums; pairs of ReLUs go into one three-input add
                int tot[PF_QPWAVE];
#pragma unroll
                for (int q = 0; q < PF_QPWAVE; ++q) tot[q] = 0;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2)
                        tot[rb / 2] += max(acc[rb][r], 0) + max(acc[rb][r + 1], 0);
#pragma unroll
                for (int q = 0; q < PF_QPWAVE; ++q) {
                    // the other half of the heads sits in lane j ^ 32
                    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)tot[q],
                                                                    (uint32_t)tot[q], false, false);
                    sum[q] = (float)((int)r[0] + (int)r[1]) * 0.25f;
                }
            } else {
#pragma unroll
                for (int q = 0; q < PF_QPWAVE; ++q) sum[q] = 0.0f;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        // heads 32*(rb%2) + 8*r4 + 4g .. +4 of query rb/2
                        const v4f wv = *reinterpret_cast<const v4f*>(
                            wq + (rb / 2) * H_I + 32 * (rb % 2) + 8 * r4 + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int dot = acc[rb][4 * r4 + i];
                            sum[rb / 2] += wv[i] * (float)(dot > 0 ? dot : 0);
                        }
                    }
#pragma unroll
                for (int q = 0; q < PF_QPWAVE; ++q) sum[q] = xor32_sum(sum[q]);
            }
        };
        // the block's scores, -inf past each query's position or on an
        // unallocated page (sum is not read for a block no query of the wave sees)
        auto store = [&](int s0, const float (&sum)[PF_QPWAVE]) {
            const int s = s0 + j;
            if (g == 0 && s < L_cap) {
                const bool page_ok = pm.table == nullptr || key_block_row(pm, b, L_cap, s0) >= 0;
#pragma unroll
                for (int q = 0; q < PF_QPWAVE; ++q) {
                    if (tw + q >= Tq) continue;                   // past the last query
                    S[((size_t)b * Tq + tw + q) * L_cap + s] =
                        s <= pos[q] && page_ok ? sum[q] : -__builtin_inff();
                }
            }
        };
        // one block's products issued together with another block's scores:
        // the MFMA chains run under the VALU work (one MFMA per six VALU ops)
        auto overlapped = [&](const v4i* bk, v16i (&acc_next)[RB], const v16i (&acc)[RB],
                              float (&sum)[PF_QPWAVE]) {
            products(bk, acc_next);
            scores(acc, sum);
#pragma unroll
            for (int i = 0; i < RB * KS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
        };

        // Software pipeline over the 32-key blocks the wave's queries see
        // ([s_lo, s_end)): block i's products are issued with block i-1's
        // scores (two accumulator sets) while block i+1's keys are in flight
        // (two key buffers); the blocks past them only get -inf.  Scheduling
        // barriers keep each block's key loads where they stand, ahead of the
        // products (left to the scheduler, half of them sank to the end of
        // the previous block and their latency showed).
        const int s_vis = pos_max >= s_lo ? ((pos_max - s_lo) / 32 + 1) * 32 + s_lo : s_lo;
        const int s_end = min(s_hi, s_vis);
        v4i kb0[KS], kb1[KS];
        v16i acc0[RB], acc1[RB];
        float sum[PF_QPWAVE];
        if (s_lo < s_end) {
            load_keys(s_lo, kb0);
            load_keys(s_lo + 32, kb1);
            products(kb0, acc0);
            for (int s0 = s_lo;; s0 += 64) {
                // block s0 (acc0, issued) | block s0 + 32 (kb1) | block s0 + 64 (into kb0)
                __builtin_amdgcn_sched_barrier(0);
                load_keys(s0 + 64, kb0);
                __builtin_amdgcn_sched_barrier(0);
                if (s0 + 32 >= s_end) {
                    scores(acc0, sum);
                    store(s0, sum);
                    break;
                }
                overlapped(kb1, acc1, acc0, sum);
                store(s0, sum);
                __builtin_amdgcn_sched_barrier(0);
                load_keys(s0 + 96, kb1);
                __builtin_amdgcn_sched_barrier(0);
                if (s0 + 64 >= s_end) {
                    scores(acc1, sum);
                    store(s0 + 32, sum);
                    break;
                }
                overlapped(kb0, acc0, acc1, sum);
                store(s0 + 32, sum);
            }
        }
#pragma unroll
        for (int q = 0; q < PF_QPWAVE; ++q) sum[q] = 0.0f;
        for (int s0 = s_end; s0 < s_hi; s0 += 32) store(s0, sum);
    };
    if (fast) run(std::true_type{});
    else run(std::false_type{});
}

template <int H_I, int D_I>
hipError_t launch_ix(const int8_t* qI, const float* w, const int8_t* kI, const int32_t* kv_len,
                     int B, int Tq, int L_cap, float* S, uint32_t* zero, uint32_t zero_n,
                     hipStream_t stream, PageMap pm, SummaryOut summary) {
    constexpr int QPW = IX_ROWS / H_I;
    dim3 grid((L_cap + IX_KEYS_PER_WG - 1) / IX_KEYS_PER_WG, (Tq + QPW - 1) / QPW, B);
    if constexpr (H_I == 64) {
        if (Tq >= PF_MIN_TQ) {
            // key splits: enough workgroups to fill the chip, chunks of whole
            // 64-key steps
            const int rows = (Tq + PF_QPW - 1) / PF_QPW * B;
            const int steps = (L_cap + 63) / 64;
            int splits = (PF_TARGET_WGS + rows - 1) / rows;
            if (splits > steps) splits = steps;
            if (splits < 1) splits = 1;
            const int chunk = (steps + splits - 1) / splits * 64;
            splits = (L_cap + chunk - 1) / chunk;
            dim3 pgrid((Tq + PF_QPW - 1) / PF_QPW, B, splits);
            hipLaunchKernelGGL((indexer_prefill_kernel<D_I>), pgrid, dim3(IX_THREADS), 0, stream, qI,
                               w, kI, kv_len, Tq, L_cap, chunk, S, zero, zero_n, pm);
            return hipGetLastError();
        }
    }
    if (QPW != 1) summary.keys = nullptr;  // only the one-query workgroups write it
    hipLaunchKernelGGL((indexer_scores_kernel<H_I, D_I>), grid, dim3(IX_THREADS), 0, stream,
                       qI, w, kI, kv_len, Tq, L_cap, S, zero, zero_n, pm, summary);
    return hipGetLastError();
}

}  // namespace

bool indexer_writes_summary(int Tq, int H_I) { return H_I == 64 && Tq < PF_MIN_TQ; }

bool indexer_shape_supported(int H_I, int D_I) {
    const bool h_ok = H_I == 4 || H_I == 8 || H_I == 16 || H_I == 32 || H_I == 64;
    const bool d_ok = D_I == 32 || D_I == 64 || D_I == 128;
    return h_ok && d_ok;
}

#define ISA_IX_CASE(HH, DD)                                                              \
    if (H_I == HH && D_I == DD)                                                          \
        return launch_ix<HH, DD>(qI, w, kI, kv_len, B, Tq, L_cap, S, zero, zero_n, stream, pm, \
                                 summary);

hipError_t launch_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                                 const int32_t* kv_len, int B, int Tq, int H_I, int D_I,
                                 int L_cap, float* S, uint32_t* zero, uint32_t zero_n,
                                 hipStream_t stream, PageMap pm, SummaryOut summary) {
    ISA_IX_CASE(64, 128) ISA_IX_CASE(64, 64) ISA_IX_CASE(64, 32)
    ISA_IX_CASE(32, 128) ISA_IX_CASE(32, 64) ISA_IX_CASE(32, 32)
    ISA_IX_CASE(16, 128) ISA_IX_CASE(16, 64) ISA_IX_CASE(16, 32)
    ISA_IX_CASE(8, 128) ISA_IX_CASE(8, 64) ISA_IX_CASE(8, 32)
    ISA_IX_CASE(4, 128) ISA_IX_CASE(4, 64) ISA_IX_CASE(4, 32)
    return hipErrorInvalidValue;
}
#undef ISA_IX_CASE

}  // namespace isa
