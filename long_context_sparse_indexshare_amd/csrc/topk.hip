// Top-k position select over fp32 scores (gfx950).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1: keep the top-K positions; K = index_topk = 2048 in the config fragment
// of "GLM-5.2核心技术解析"): for each query, the min(k, pos+1) visible positions
// that come first under (score descending, position ascending), listed in
// ascending position and padded with -1.
//
// Scores are compared as order-preserving 32-bit keys.  The selection starts
// from a summary: for every wave chunk of 256 positions, its M largest keys
// with their positions (written by the indexer's epilogue in a decode group
// call, else by a summary kernel).  Rows of at most 262144 positions whose
// summary holds at least 2k keys (decode rows and long prefill rows alike)
// then take one workgroup per row (topk_direct_kernel, described there): the
// candidates come from the summary, and only chunks whose summary may miss a
// candidate are read again.  Longer rows (up to 2^21 positions) are spread
// over many workgroups per row, with M chosen so the summary holds about 2k
// keys:
//   1. filter:   every workgroup derives from the row's summary a threshold L
//                with at least k summary keys >= L (the summary's keys are
//                scores of distinct visible positions, so at least k scores
//                are >= L: the k-th largest is >= L), then keeps its chunk's
//                scores >= L as one run of (key, position) entries in
//                ascending position, in slots of its own.  L lies within
//                1/4096 of the summary's key range below its k-th largest
//                key, so a row keeps little more than k entries.
//   2. finish:   one workgroup per row holds the candidates in ascending
//                position (in registers when the runs are short, else staged
//                in LDS), finds the exact k-th key T and how many keys equal
//                to T are taken (the lowest positions) by radix passes over
//                the candidates' key range and a direct ranking of the cut
//                bin, and writes every selected position straight to its
//                place after one block scan of (above T, equal to T) counts.
// Shorter rows (whose summary would hold fewer than 2k keys), when there are
// at least 256 of them (a prefill chunk), take a first-digit histogram
// kernel and one workgroup per row (topk_select_kernel) instead.
// Workgroups never wait on each other inside a kernel: on gfx950 a device-
// scope fence writes back and invalidates the whole L2 of the XCD, so each
// hand-over between workgroups goes through a kernel boundary instead.
#include <type_traits>

#include "isa_internal.h"

namespace isa {

namespace {

__device__ __forceinline__ int visible_count(const int32_t* kv_len, int row, int Tq, int L_cap) {
    const int b = row / Tq;
    const int t = row - b * Tq;
    int len = kv_len[b];
    len = len < 0 ? 0 : (len > L_cap ? L_cap : len);
    const int n = len - Tq + t + 1;
    return n > 0 ? n : 0;
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active), in
// registers: DPP row shifts by 1, 2, 4 and 8 scan each 16-lane row, then
// row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds the total of lanes 0-31 to rows 2 and 3.  (A __shfl_up
// ladder goes through the LDS crossbar, six dependent round trips.)
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    uint32_t v = x;
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

// Exclusive prefix sum over the NT threads of the workgroup; *total gets the sum.
template <int NT = TOPK_THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* sh_waves) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t inc = wave_inclusive_scan(v);
    __syncthreads();
    if (lane == 63) sh_waves[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t x = sh_waves[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    *total = all;
    return before + inc - v;
}

// Over bins h[0..nbins) (nbins = NT * per): the largest bin B with
// sum_{b >= B} h[b] >= need (descending) or the smallest bin B with
// sum_{b <= B} h[b] >= need (ascending).  Returns (B, the count strictly
// beyond it: above for descending, below for ascending) to every thread.
// Thread t owns bins [PER*t, PER*t + PER) ascending, or the mirrored range
// descending, and keeps them in registers (16-byte loads where PER allows):
// find_bin_load requests them, find_bin_regs does the rest, so a caller can
// have them in flight across other waits.
template <int PER, bool DESC, int NT = TOPK_THREADS>
__device__ __forceinline__ void find_bin_load(const uint32_t* h, uint32_t (&hv)[PER]) {
    const int first = DESC ? (NT - 1 - (int)threadIdx.x) * PER : (int)threadIdx.x * PER;
    if constexpr (PER % 4 == 0) {
#pragma unroll
        for (int i = 0; i < PER; i += 4) {
            const uint4 q = *reinterpret_cast<const uint4*>(h + first + i);
            hv[i] = q.x; hv[i + 1] = q.y; hv[i + 2] = q.z; hv[i + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) hv[i] = h[first + i];
    }
}

template <int PER, bool DESC, int NT = TOPK_THREADS>
__device__ __forceinline__ uint2 find_bin_regs(const uint32_t (&hv)[PER], uint32_t need,
                                               uint32_t* sh_waves, uint32_t* sh_res) {
    const int first = DESC ? (NT - 1 - (int)threadIdx.x) * PER : (int)threadIdx.x * PER;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += hv[i];
    uint32_t total;
    const uint32_t before = block_exclusive_scan<NT>(local, &total, sh_waves);
    if (before < need && before + local >= need) {
        // the bin where the running count (in this thread's direction) reaches need
        uint32_t acc = before;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int o = DESC ? PER - 1 - i : i;
            const uint32_t c = hv[o];
            if (!found && acc + c >= need) {
                sh_res[0] = (uint32_t)(first + o);
                sh_res[1] = acc;
                found = true;
            }
            acc += c;
        }
    }
    __syncthreads();
    const uint2 r = make_uint2(sh_res[0], sh_res[1]);
    __syncthreads();
    return r;
}

template <int PER, bool DESC, int NT = TOPK_THREADS>
__device__ __forceinline__ uint2 find_bin(const uint32_t* h, uint32_t need, uint32_t* sh_waves,
                                          uint32_t* sh_res) {
    uint32_t hv[PER];
    find_bin_load<PER, DESC, NT>(h, hv);
    return find_bin_regs<PER, DESC, NT>(hv, need, sh_waves, sh_res);
}

// Zeroes counters (histograms, candidate counts, tickets) at the start of a
// call, so workspaces need no initialisation.  A fill kernel rather than a
// memset keeps calls capturable in a HIP graph.
__global__ __launch_bounds__(256) void clear_u32_kernel(uint32_t* __restrict__ p, size_t n) {
    const size_t n4 = n / 4;
    uint4* p4 = reinterpret_cast<uint4*>(p);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
        p4[i] = make_uint4(0, 0, 0, 0);
    for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = 0u;
}

// The histogram kernel takes HIST_PER scores per thread.  With many rows it
// takes larger chunks than the classify kernel (16 per thread): fewer
// workgroups per row add their bins into the row's histogram, so a bin that
// many scores share takes fewer contending global atomics.  With few rows
// (decode) it takes the classify kernel's 4096-score chunks (4 per thread),
// so that enough workgroups stream the scores, as long as a row's hot bins
// do not collect the atomics of too many workgroups.
constexpr int HIST_THREADS = 1024;
constexpr int HIST_PER_MANY = 16;
constexpr int HIST_PER_FEW = 4;
constexpr int HIST_MIN_WGS = 256;          // below this many 16-per-thread chunks: 4 per thread,
constexpr int HIST_MAX_FEW_CHUNKS = 64;    // unless a row would take more chunks than this

template <int HIST_PER>
__global__ __launch_bounds__(HIST_THREADS) void topk_hist_kernel(const float* __restrict__ S,
                                                                 const int32_t* __restrict__ kv_len,
                                                                 int Tq, int L_cap, int k,
                                                                 uint32_t* __restrict__ hist) {
    constexpr int HIST_CHUNK = HIST_THREADS * HIST_PER;
    const int row = blockIdx.y;
    const int start = blockIdx.x * HIST_CHUNK;
    // every score of the thread in flight before the first is used, and before
    // the row's visible length arrives (the loads stay inside the row; those
    // past the length are not counted)
    const float* rowp = S + (size_t)row * L_cap;
    float v[HIST_PER];
#pragma unroll
    for (int e = 0; e < HIST_PER; ++e) {
        const int s = start + e * HIST_THREADS + threadIdx.x;
        v[e] = s < L_cap ? rowp[s] : 0.0f;
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    if (start >= n) return;
    __shared__ uint32_t lh[TOPK_HIST_BINS];
    for (int i = threadIdx.x; i < TOPK_HIST_BINS; i += HIST_THREADS) lh[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < HIST_PER; ++e) {
        const int s = start + e * HIST_THREADS + threadIdx.x;
        if (s < n) atomicAdd(&lh[score_key(v[e]) >> (32 - TOPK_HIST_BITS)], 1u);
    }
    __syncthreads();
    uint32_t* gh = hist + (size_t)row * TOPK_HIST_BINS;
    for (int i = threadIdx.x; i < TOPK_HIST_BINS; i += HIST_THREADS) {
        const uint32_t c = lh[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// Entries the finishing workgroup stages in LDS (more are read from global).
constexpr int ENT_LDS = 12288;
constexpr int HIST2_BINS = 1024;          // prefill select path: second digit, key bits [19:10]
constexpr int COL_MAX = 512;              // entries ranked directly for the exact cut

// ---------------------------------------------------------------------------
// Summary, for calls whose indexer did not write it: wave w of workgroup c
// covers wave chunk 4c + w (positions 1024c + 32w + 128q + j, code 32q + j;
// lane l takes q = 2e + l / 32 and j = l % 32 for e < 4) and writes its M
// largest keys with their codes; invisible positions take key 0.
constexpr int SUM_THREADS = 256;
__global__ __launch_bounds__(SUM_THREADS) void topk_summary_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int M,
    int nwchunks, uint32_t* __restrict__ summary, uint8_t* __restrict__ codes) {
    const int row = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int base = blockIdx.x * (4 * TOPK_WAVE_CHUNK) + wave * 32 + (lane & 31);
    const int qh = lane >> 5;
    const float* rowp = S + (size_t)row * L_cap;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int s = base + (2 * e + qh) * 128;
        v[e] = s < L_cap ? rowp[s] : 0.0f;
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    uint32_t key[4], code[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        key[e] = base + (2 * e + qh) * 128 < n ? score_key(v[e]) : 0u;
        code[e] = (uint32_t)((2 * e + qh) * 32 + (lane & 31));
    }
    const size_t off = ((size_t)row * nwchunks + blockIdx.x * 4 + wave) * M;
    wave_top_m<4>(key, code, M, summary + off, codes + off);
}

// Radix bins over a key range [lo, hi]: bin = (key - lo) >> sh, with sh the
// smallest shift that leaves at most RB_BINS bins.  Histograms are stored in
// descending key order (LDS index RB_BINS - 1 - bin), so the keys at or above
// a bin are counted by a prefix of the array.
constexpr int RB_BITS = 12;
constexpr int RB_BINS = 1 << RB_BITS;

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
    const uint32_t r = hi - lo;
    const int bits = r ? 32 - __builtin_clz(r) : 0;
    return bits > RB_BITS ? bits - RB_BITS : 0;
}

// Over a descending histogram h[RB_BINS] (NT threads, four bins each): the
// first index whose running count reaches need, the count before it and the
// count in it, returned to every thread (.x, .y, .z).  Two barriers.  The
// running count must reach need.  tot (NT / 64 words) and res (3 words) are
// rewritten: every thread must be past its reads of the previous call's
// values, which a barrier between the calls ensures.
template <int NT>
__device__ __forceinline__ uint3 find_cut(const uint32_t* h, uint32_t need, uint32_t* tot,
                                          uint32_t* res) {
    static_assert(RB_BINS == 4 * NT, "four bins per thread");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint4 q = *reinterpret_cast<const uint4*>(h + 4 * threadIdx.x);
    const uint32_t local = q.x + q.y + q.z + q.w;
    const uint32_t inc = wave_inclusive_scan(local);
    if (lane == 63) tot[wave] = inc;
    __syncthreads();
    uint32_t before = inc - local;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) before += w < wave ? tot[w] : 0u;
    if (before < need && before + local >= need) {
        const uint32_t hv[4] = {q.x, q.y, q.z, q.w};
        uint32_t acc = before;
        bool found = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!found && acc + hv[i] >= need) {
                res[0] = 4u * threadIdx.x + i;
                res[1] = acc;
                res[2] = hv[i];
                found = true;
            }
            acc += hv[i];
        }
    }
    __syncthreads();
    return make_uint3(res[0], res[1], res[2]);
}

// Filter: every workgroup (4096 positions of one row) derives the row's
// threshold L from the summary and keeps its chunk's visible keys >= L as one
// run of (key, position) entries in ascending position, in the chunk's own
// entry slots (one per position of the chunk, so no atomics and no
// overflow), and writes the run's length.  L: with the summary's keys in [MN, MX] histogrammed into RB_BINS
// bins, the lower edge of the highest bin at which the summary keys at or
// above it reach k.  The summary keys are scores of distinct visible
// positions, so at least k scores are >= L, and L lies within one bin width
// (1/4096 of the summary's key range) below the k-th largest summary key.  A
// summary with fewer than k keys gives L = 0: every visible position.
constexpr int SUM_PER = TOPK_MAX_SUMMARY / TOPK_THREADS;
struct FilterShared {
    uint32_t h[RB_BINS];
    uint32_t red[3][TOPK_THREADS / 64];   // per wave: summary key count, max, ~min
    uint32_t tot[TOPK_THREADS / 64];
    uint32_t res[3];
    uint32_t cnt[TOPK_PER_THREAD * (TOPK_THREADS / 64)];   // kept keys per (e, wave)
};

__global__ __launch_bounds__(TOPK_THREADS) void topk_filter_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ summary, int nsum, uint32_t* __restrict__ counts,
    uint2* __restrict__ ent, int nchunks_max) {
    const int row = blockIdx.y;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NW = TOPK_THREADS / 64;
    static_assert(TOPK_PER_THREAD * NW == 64, "one lane per (e, wave) count");
    __shared__ FilterShared f;

    // this chunk's scores and the row's summary, requested before the row's
    // visible length arrives (they stay inside the row and its summary; the
    // scores past the length are masked below)
    // (position = start + e * TOPK_THREADS + tid: ascending order is (e, wave, lane))
    const float* rowp = S + (size_t)row * L_cap;
    const int start = c * TOPK_CHUNK;
    float sc[TOPK_PER_THREAD];
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        sc[e] = s < L_cap ? rowp[s] : 0.0f;
    }
    const uint32_t* su = summary + (size_t)row * nsum;
    uint32_t u[SUM_PER];
#pragma unroll
    for (int i = 0; i < SUM_PER; ++i) {
        const int j = i * TOPK_THREADS + tid;
        u[i] = j < nsum ? su[j] : 0u;
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    if (c >= nch) return;

    *reinterpret_cast<uint4*>(&f.h[4 * tid]) = make_uint4(0u, 0u, 0u, 0u);
    uint32_t cnt = 0, mx = 0, nmn = 0;                  // nmn = ~(minimum nonzero key)
#pragma unroll
    for (int i = 0; i < SUM_PER; ++i) {
        cnt += u[i] != 0u;
        mx = max(mx, u[i]);
        nmn = max(nmn, u[i] ? ~u[i] : 0u);
    }
    cnt = __builtin_amdgcn_readlane(wave_inclusive_scan(cnt), 63);
    mx = wave_max_u32(mx);
    nmn = wave_max_u32(nmn);
    if (lane == 0) {
        f.red[0][wave] = cnt;
        f.red[1][wave] = mx;
        f.red[2][wave] = nmn;
    }
    __syncthreads();
    uint32_t C = 0, MX = 0, NMN = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        C += f.red[0][w];
        MX = max(MX, f.red[1][w]);
        NMN = max(NMN, f.red[2][w]);
    }
    const uint32_t MN = ~NMN;
    uint32_t L;
    if (C < (uint32_t)k) {
        L = 0u;
    } else if (MX == MN) {
        L = MN;
    } else {
        const int sh = range_shift(MN, MX);
#pragma unroll
        for (int i = 0; i < SUM_PER; ++i)
            if (u[i]) atomicAdd(&f.h[RB_BINS - 1 - ((u[i] - MN) >> sh)], 1u);
        __syncthreads();
        if (wave == 0) {
            // one wave finds the bin (one barrier instead of a block scan's
            // two): lane l sums bins [64l, 64l + 64), then the crossing
            // lane's 64 bins one per lane
            uint32_t local = 0;
            const uint4* hb = reinterpret_cast<const uint4*>(f.h) + 16 * lane;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint4 x = hb[q];
                local += x.x + x.y + x.z + x.w;
            }
            const uint32_t need = (uint32_t)k;
            const uint32_t inc = wave_inclusive_scan(local);
            const int cl = (int)__builtin_ctzll(__ballot(inc >= need && inc - local < need));
            const uint32_t base = __builtin_amdgcn_readlane(inc - local, cl);
            const uint32_t cb = f.h[64 * cl + lane];
            const uint32_t inc2 = base + wave_inclusive_scan(cb);
            const int bl = (int)__builtin_ctzll(__ballot(inc2 >= need && inc2 - cb < need));
            if (lane == 0) f.res[0] = MN + ((uint32_t)(RB_BINS - 1 - (64 * cl + bl)) << sh);
        }
        __syncthreads();
        L = f.res[0];
    }

    uint32_t keys[TOPK_PER_THREAD];
    uint64_t kept[TOPK_PER_THREAD];
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        const bool valid = s < n;
        keys[e] = valid ? score_key(sc[e]) : 0u;
        kept[e] = __ballot(valid && keys[e] >= L);
        if (lane == 0) f.cnt[e * NW + wave] = (uint32_t)__popcll(kept[e]);
    }
    __syncthreads();
    // every wave scans the 64 (e, wave) counts itself, in ascending-position order
    const uint32_t v = f.cnt[lane];
    const uint32_t inc = wave_inclusive_scan(v);
    const uint32_t total = __builtin_amdgcn_readlane(inc, 63);
    const uint32_t excl = inc - v;
    uint2* re = ent + ((size_t)row * nchunks_max + c) * TOPK_SLOT_CAP;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const uint32_t base = __builtin_amdgcn_readlane(excl, e * NW + wave);
        if ((kept[e] >> lane) & 1ull) {
            const uint32_t slot = base + (uint32_t)__popcll(kept[e] & below);
            if (slot < (uint32_t)TOPK_SLOT_CAP)
                re[slot] = make_uint2(keys[e], (uint32_t)(start + e * TOPK_THREADS + tid));
        }
    }
    if (tid == 0) counts[(size_t)row * nchunks_max + c] = total;
}

// ---------------------------------------------------------------------------
// Finish: one workgroup per row.  The candidates are the row's keys >= L (at
// least k of them), listed chunk by chunk, each chunk's run in ascending
// position.  Thread t takes chunk t / TPC (TPC = threads per chunk, a power of
// two) and slots [8 * (t % TPC), +8) of it, so the candidates in thread order
// are in ascending position; the common case (every run within the slots the
// threads cover) keeps them in registers from a single round of loads.
// Otherwise they are staged in LDS in that order, or, past the LDS, read from
// the entry slots through the runs' starts.
//   * the exact cut: radix passes over [min, max] of the candidates (4096
//     bins each, the range of the cut bin next) find the bin holding the k-th
//     largest key; once that bin holds at most COL_MAX candidates they are
//     ranked directly under (key desc, position asc), giving the k-th key T
//     and how many candidates equal to T are taken (needT, the lowest
//     positions); a bin of width one is the key T itself;
//   * the output: one block scan over the per-thread counts of candidates
//     above T and equal to T gives each candidate the number selected before
//     it (above before + min(equal before, needT)), so it is written straight
//     to its place in the ascending-position list.
constexpr int FIN_THREADS = 1024;
constexpr int FIN_WAVES = FIN_THREADS / 64;
constexpr int FIN_REG = 8;                          // candidates per thread per tile
constexpr int FIN_TILE = FIN_THREADS * FIN_REG;
static_assert(TOPK_MAX_CHUNKS <= FIN_THREADS / 2, "at least two threads per chunk");
static_assert(FIN_TILE < 65536, "per-tile counts fit 16 bits");
struct FinishShared {
    uint32_t h[RB_BINS];
    uint2 lent[ENT_LDS];                  // staged candidates, ascending position
    uint2 col[COL_MAX];                   // candidates of the cut bin, ranked directly
    uint32_t cstart[TOPK_MAX_CHUNKS + 1]; // chunk -> first candidate in position order
    uint32_t red[3][FIN_WAVES];
    uint32_t tot[FIN_WAVES];
    uint32_t tot2[2][FIN_WAVES];
    uint32_t res[3];
    uint32_t cut[2];
    uint32_t ncol;
};

// Candidate sources of the finish.  Each gives the thread's candidates of a
// tile in ascending position (tile(T, fn): fn(j, valid, key, pos) for
// j < FIN_REG) and visits all of its candidates in any order (each(fn)).
struct SrcRegs {
    const uint2 (&e)[FIN_REG];
    uint32_t nvalid;                      // the first nvalid are candidates
    __device__ int ntiles() const { return 1; }
    template <class F> __device__ __forceinline__ void tile(int, F fn) const {
#pragma unroll
        for (int j = 0; j < FIN_REG; ++j) fn(j, (uint32_t)j < nvalid, e[j].x, e[j].y);
    }
    template <class F> __device__ __forceinline__ void each(F fn) const {
#pragma unroll
        for (int j = 0; j < FIN_REG; ++j)
            if ((uint32_t)j < nvalid) fn(e[j].x, e[j].y);
    }
};
struct SrcLds {
    const uint2* lent;
    uint32_t ntot;
    __device__ int ntiles() const { return (int)((ntot + FIN_TILE - 1) / FIN_TILE); }
    template <class F> __device__ __forceinline__ void tile(int T, F fn) const {
        const uint32_t i0 = (uint32_t)T * FIN_TILE + threadIdx.x * FIN_REG;
#pragma unroll
        for (int j = 0; j < FIN_REG; ++j) {
            const uint32_t i = i0 + j;
            const uint2 v = i < ntot ? lent[i] : make_uint2(0u, 0u);
            fn(j, i < ntot, v.x, v.y);
        }
    }
    template <class F> __device__ __forceinline__ void each(F fn) const {
        for (uint32_t i = threadIdx.x; i < ntot; i += FIN_THREADS) {
            const uint2 v = lent[i];
            fn(v.x, v.y);
        }
    }
};
struct SrcGlobal {                        // the entry buffer, through the chunk starts
    const uint2* re;                      // the row's slots
    const uint32_t* cstart;               // LDS, nch + 1 entries
    int nch;
    uint32_t ntot;
    __device__ int ntiles() const { return (int)((ntot + FIN_TILE - 1) / FIN_TILE); }
    __device__ __forceinline__ uint2 at(uint32_t i) const {
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cstart[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        return re[(size_t)lo * TOPK_SLOT_CAP + (i - cstart[lo])];
    }
    template <class F> __device__ __forceinline__ void tile(int T, F fn) const {
        const uint32_t i0 = (uint32_t)T * FIN_TILE + threadIdx.x * FIN_REG;
#pragma unroll
        for (int j = 0; j < FIN_REG; ++j) {
            const uint32_t i = i0 + j;
            const uint2 v = i < ntot ? at(i) : make_uint2(0u, 0u);
            fn(j, i < ntot, v.x, v.y);
        }
    }
    template <class F> __device__ __forceinline__ void each(F fn) const {
        for (uint32_t i = threadIdx.x; i < ntot; i += FIN_THREADS) {
            const uint2 v = at(i);
            fn(v.x, v.y);
        }
    }
};
// The exact cut and the ordered output over one source.  On entry the
// histogram is zero, ncol is 0, and every thread has passed a barrier after
// which [MN, MX] is the candidates' key range.
template <class Src>
__device__ __forceinline__ void finish_select(const Src& src, int k, uint32_t MN, uint32_t MX,
                                              FinishShared& f, int32_t* __restrict__ out) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    uint32_t lo = MN, hi = MX, need = (uint32_t)k;
    uint32_t T, needT;
    for (bool first = true;; first = false) {
        if (lo == hi) {
            T = lo;
            needT = need;
            break;
        }
        const int sh = range_shift(lo, hi);
        if (!first) {
            // every thread is past its reads of the previous pass's histogram
            *reinterpret_cast<uint4*>(&f.h[4 * tid]) = make_uint4(0u, 0u, 0u, 0u);
            if (tid == 0) f.ncol = 0u;
            __syncthreads();
        }
        src.each([&](uint32_t key, uint32_t) {
            if (key >= lo && key <= hi) atomicAdd(&f.h[RB_BINS - 1 - ((key - lo) >> sh)], 1u);
        });
        __syncthreads();
        const uint3 r = find_cut<FIN_THREADS>(f.h, need, f.tot, f.res);
        const uint32_t b = (uint32_t)(RB_BINS - 1) - r.x;
        need -= r.y;                                    // >= 1 keys to take from bin b
        const uint32_t blo = lo + (b << sh);
        const uint32_t width = (1u << sh) - 1u;
        const uint32_t bhi = hi - blo < width ? hi : blo + width;
        if (sh == 0) {
            T = blo;
            needT = need;
            break;
        }
        if (r.z <= (uint32_t)COL_MAX) {
            src.each([&](uint32_t key, uint32_t pos) {
                if (key >= blo && key <= bhi) {
                    const uint32_t slot = atomicAdd(&f.ncol, 1u);
                    if (slot < (uint32_t)COL_MAX) f.col[slot] = make_uint2(key, pos);
                }
            });
            __syncthreads();
            const uint32_t m = r.z;
            for (uint32_t t = tid; t < m; t += FIN_THREADS) {
                const uint2 e = f.col[t];
                uint32_t rank = 0, eq = 0;
                for (uint32_t j = 0; j < m; ++j) {
                    const uint2 o = f.col[j];
                    rank += (uint32_t)(o.x > e.x) | ((uint32_t)(o.x == e.x) & (uint32_t)(o.y < e.y));
                    eq += (uint32_t)(o.x == e.x) & (uint32_t)(o.y <= e.y);
                }
                if (rank == need - 1) {
                    f.cut[0] = e.x;
                    f.cut[1] = eq;                      // keys equal to T taken
                }
            }
            __syncthreads();
            T = f.cut[0];
            needT = f.cut[1];
            break;
        }
        lo = blo;
        hi = bhi;
    }

    // ordered output: per tile, one block scan over (above T, equal to T)
    // counts packed in 16-bit halves
    uint32_t a_run = 0, e_run = 0;
    const int nt = src.ntiles();
    for (int t = 0; t < nt; ++t) {
        uint32_t am = 0, em = 0;
        uint32_t pos[FIN_REG];
        src.tile(t, [&](int j, bool valid, uint32_t key, uint32_t p) {
            pos[j] = p;
            am |= (uint32_t)(valid && key > T) << j;
            em |= (uint32_t)(valid && key == T) << j;
        });
        const uint32_t packed = ((uint32_t)__popc(am) << 16) | (uint32_t)__popc(em);
        const uint32_t inc = wave_inclusive_scan(packed);
        if (lane == 63) f.tot2[t & 1][wave] = inc;
        __syncthreads();
        uint32_t before = inc - packed, all = 0;
#pragma unroll
        for (int w = 0; w < FIN_WAVES; ++w) {
            const uint32_t x = f.tot2[t & 1][w];
            before += w < wave ? x : 0u;
            all += x;
        }
        uint32_t a0 = a_run + (before >> 16), e0 = e_run + (before & 0xFFFFu);
#pragma unroll
        for (int j = 0; j < FIN_REG; ++j) {
            if ((am >> j) & 1u) {
                const uint32_t o = a0 + (e0 < needT ? e0 : needT);
                if (o < (uint32_t)k) out[o] = (int32_t)pos[j];   // exactly k are selected
                ++a0;
            } else if ((em >> j) & 1u) {
                if (e0 < needT && a0 + e0 < (uint32_t)k) out[a0 + e0] = (int32_t)pos[j];
                ++e0;
            }
        }
        a_run += all >> 16;
        e_run += all & 0xFFFFu;
    }
}

__global__ __launch_bounds__(FIN_THREADS) void topk_finish_kernel(
    const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k, const uint32_t* __restrict__ counts,
    const uint2* __restrict__ ent, int nchunks_max, int tpc_log2, int32_t* __restrict__ idx) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    __shared__ FinishShared f;
    const int tpc = 1 << tpc_log2;
    const int c = tid >> tpc_log2;
    const int sub = tid & (tpc - 1);
    const uint32_t slot0 = (uint32_t)sub * FIN_REG;
    // slots a chunk's threads cover (within the chunk's slots)
    const uint32_t cover = (uint32_t)tpc * FIN_REG < (uint32_t)TOPK_SLOT_CAP
                               ? (uint32_t)tpc * FIN_REG : (uint32_t)TOPK_SLOT_CAP;
    // every load is issued before the row's visible length arrives: the
    // chunk's run length, the thread's slots (all inside the row's slots;
    // those past the run are loaded but not used) and the threshold
    const bool cin = c < nchunks_max;
    const uint32_t cnt_raw = cin ? counts[(size_t)row * nchunks_max + c] : 0u;
    const uint2* re = ent + (size_t)row * nchunks_max * TOPK_SLOT_CAP;
    const uint2* ce = re + (size_t)(cin ? c : 0) * TOPK_SLOT_CAP;
    uint2 e[FIN_REG];
#pragma unroll
    for (int j = 0; j < FIN_REG; j += 2) {
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (cin && slot0 + j < cover) q = *reinterpret_cast<const uint4*>(ce + slot0 + j);
        e[j] = make_uint2(q.x, q.y);
        e[j + 1] = make_uint2(q.z, q.w);
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    int32_t* out = idx + (size_t)row * k;
    if (n <= k) {
        // every visible position, then -1 padding
        for (int j = tid; j < k; j += FIN_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const bool mine = c < nch;
    const uint32_t cnt = mine ? cnt_raw : 0u;
    const uint32_t capped = cnt;                        // a run never exceeds its slots
    const uint32_t nvalid = capped > slot0 ? (capped - slot0 < (uint32_t)FIN_REG ? capped - slot0 : FIN_REG) : 0u;
    const bool slow = mine && cnt > cover;              // a run longer than the slots loaded
    uint32_t mx = 0u, nmn = 0u;
#pragma unroll
    for (int j = 0; j < FIN_REG; ++j) {
        if ((uint32_t)j < nvalid) {
            mx = max(mx, e[j].x);
            nmn = max(nmn, ~e[j].x);
        }
    }
    mx = wave_max_u32(mx);
    nmn = wave_max_u32(nmn);
    const uint64_t slow_w = __ballot(slow);
    *reinterpret_cast<uint4*>(&f.h[4 * tid]) = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) f.ncol = 0u;
    if (lane == 0) {
        f.red[0][wave] = mx;
        f.red[1][wave] = nmn;
        f.red[2][wave] = slow_w != 0ull;
    }
    __syncthreads();
    uint32_t MX = 0u, NMN = 0u, SLOW = 0u;
#pragma unroll
    for (int w = 0; w < FIN_WAVES; ++w) {
        MX = max(MX, f.red[0][w]);
        NMN = max(NMN, f.red[1][w]);
        SLOW |= f.red[2][w];
    }
    if (!SLOW) {
        finish_select(SrcRegs{e, nvalid}, k, ~NMN, MX, f, out);
        return;
    }

    // a run longer than the slots loaded: stage the candidates in LDS, or
    // read them from the entry slots; first the key range over all of them
    auto range_of = [&](const auto& src) {
        uint32_t a = 0u, b = 0u;
        src.each([&](uint32_t key, uint32_t) {
            a = max(a, key);
            b = max(b, ~key);
        });
        a = wave_max_u32(a);
        b = wave_max_u32(b);
        __syncthreads();                                // red is free again
        if (lane == 0) {
            f.red[0][wave] = a;
            f.red[1][wave] = b;
        }
        __syncthreads();
        uint32_t A = 0u, B = 0u;
#pragma unroll
        for (int w = 0; w < FIN_WAVES; ++w) {
            A = max(A, f.red[0][w]);
            B = max(B, f.red[1][w]);
        }
        return make_uint2(~B, A);
    };
    uint32_t ntot;
    const uint32_t cs = block_exclusive_scan<FIN_THREADS>(sub == 0 ? capped : 0u, &ntot, f.tot);
    if (mine && sub == 0) f.cstart[c] = cs;
    if (tid == 0) f.cstart[nch] = ntot;
    __syncthreads();
    if (ntot <= (uint32_t)ENT_LDS) {
        if (mine)
            for (uint32_t s = sub; s < capped; s += (uint32_t)tpc) f.lent[f.cstart[c] + s] = ce[s];
        __syncthreads();
        const SrcLds src{f.lent, ntot};
        const uint2 r = range_of(src);
        finish_select(src, k, r.x, r.y, f, out);
    } else {
        const SrcGlobal src{re, f.cstart, nch, ntot};
        const uint2 r = range_of(src);
        finish_select(src, k, r.x, r.y, f, out);
    }
}
// ---------------------------------------------------------------------------
// Direct select (decode rows of at most DIR_MAX_N positions whose summary
// holds at least 2k keys; topk_layout decides): one workgroup per row takes
// its candidates from the summary, so no kernel runs between the summary and
// the output.  A wave chunk is "saturated" when its M-th summary key is at
// least the candidate threshold Lc: an unsaturated chunk's keys >= Lc are
// exactly its summary keys >= Lc (any other key of the chunk is at most its
// M-th summary key), so only saturated chunks are read from the scores again.
//   1. L from the summary as in the filter kernel (Lc = max(L, 1), key 0
//      being no value): at least k summary keys are >= L, so the row's k-th
//      key is >= L and every selected position is a candidate;
//   2. candidates: the summary entries >= Lc of unsaturated chunks (held in
//      registers) and the keys >= Lc of saturated chunks, read from the
//      scores and staged in LDS (more than DIR_STAGE: read again in every
//      pass);
//   3. the exact cut (T, P), selecting the keys > T and the keys equal to T
//      at positions <= P: radix passes over the candidates' key range as in
//      the finish kernel, the cut bin ranked directly once it holds at most
//      COL_MAX candidates; a bin of one key holding more takes P from a
//      position bitmap of the candidates equal to T.  With no saturated
//      chunk the summary's histogram from step 1 is the first pass;
//   4. the selected positions set bits of an LDS bitmap of the row; a block
//      scan of the per-thread bit counts gives each thread its first output
//      slot, and each thread writes the positions of its bits in order.
constexpr int DIR_THREADS = 1024;
constexpr int DIR_WAVES = DIR_THREADS / 64;
constexpr int DIR_PER = 8;                                  // summary entries per thread
constexpr int DIR_MAX_N = 262144;
constexpr int DIR_WORDS = DIR_MAX_N / 32;                   // bitmap words
constexpr int DIR_MAX_WCHUNKS = DIR_MAX_N / TOPK_WAVE_CHUNK;
constexpr int DIR_STAGE = 8192;                             // staged candidates of saturated chunks
constexpr int DIR_UNROLL = 8;                               // score loads in flight per thread
static_assert(DIR_THREADS * DIR_PER == TOPK_MAX_SUMMARY, "one thread per 8 summary entries");
static_assert(RB_BINS == 4 * DIR_THREADS, "four histogram bins per thread");

struct __attribute__((aligned(16))) DirectShared {
    uint32_t h[RB_BINS];
    uint32_t bits[DIR_WORDS];
    uint2 stage[DIR_STAGE];
    uint2 col[COL_MAX];
    uint32_t sat[DIR_MAX_WCHUNKS];        // saturated wave chunks, any order
    uint32_t red[3][DIR_WAVES];
    uint32_t tot[DIR_WAVES];
    uint32_t otot[DIR_WAVES];             // the output scan's wave totals
    uint32_t res[3];
    uint32_t cut[2];
    uint32_t nsat, nstage, ncol;
};

// Position of code c in wave chunk b.
__device__ __forceinline__ uint32_t wchunk_pos(uint32_t b, uint32_t c) {
    return (b >> 2) * 1024u + (b & 3u) * 32u + (c >> 5) * 128u + (c & 31u);
}

// WPT: bitmap words per thread (4 covers rows of up to 131072 positions, 8 up
// to DIR_MAX_N).
template <int WPT>
__global__ __launch_bounds__(DIR_THREADS) void topk_direct_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ skeys, const uint8_t* __restrict__ scodes, int nw, int M,
    int32_t* __restrict__ idx) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
    __shared__ DirectShared f;

    // the thread's summary entries (wave chunk blk, entries [8 sub, +8)) and
    // the chunk's M-th key, requested before the row's visible length arrives
    const int tpb_log2 = M == 32 ? 2 : (M == 16 ? 1 : 0);   // M / 8 threads per chunk
    const int blk = tid >> tpb_log2;
    const int sub = tid & ((1 << tpb_log2) - 1);
    const bool has = blk < nw;
    const size_t cbase = ((size_t)row * nw + (has ? blk : 0)) * M;
    uint4 ka = make_uint4(0u, 0u, 0u, 0u), kb = ka;
    uint2 cc = make_uint2(0u, 0u);
    uint32_t Kb = 0u;
    if (has) {
        ka = *reinterpret_cast<const uint4*>(skeys + cbase + sub * DIR_PER);
        kb = *reinterpret_cast<const uint4*>(skeys + cbase + sub * DIR_PER + 4);
        cc = *reinterpret_cast<const uint2*>(scodes + cbase + sub * DIR_PER);
        Kb = skeys[cbase + M - 1];
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    int32_t* out = idx + (size_t)row * k;
    if (n <= k) {
        // every visible position, then -1 padding
        for (int j = tid; j < k; j += DIR_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    const uint32_t key[DIR_PER] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
    uint32_t pos[DIR_PER];
#pragma unroll
    for (int i = 0; i < DIR_PER; ++i)
        pos[i] = wchunk_pos((uint32_t)blk, ((i < 4 ? cc.x : cc.y) >> (8 * (i & 3))) & 0xFFu);

    *reinterpret_cast<uint4*>(&f.h[4 * tid]) = make_uint4(0u, 0u, 0u, 0u);
    static_assert(WPT == 4 || WPT == 8, "one or two 16-byte bitmap accesses per thread");
#pragma unroll
    for (int u = 0; u < WPT; u += 4)
        *reinterpret_cast<uint4*>(&f.bits[WPT * tid + u]) = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) {
        f.nsat = 0u;
        f.nstage = 0u;
        f.ncol = 0u;
    }
    // 1. the summary's nonzero key count and range, then L
    uint32_t cnt = 0u, mx = 0u, nmn = 0u;                // nmn = ~(minimum nonzero key)
#pragma unroll
    for (int i = 0; i < DIR_PER; ++i) {
        cnt += key[i] != 0u;
        mx = max(mx, key[i]);
        nmn = max(nmn, key[i] ? ~key[i] : 0u);
    }
    cnt = __builtin_amdgcn_readlane(wave_inclusive_scan(cnt), 63);
    mx = wave_max_u32(mx);
    nmn = wave_max_u32(nmn);
    if (lane == 0) {
        f.red[0][wave] = cnt;
        f.red[1][wave] = mx;
        f.red[2][wave] = nmn;
    }
    __syncthreads();
    uint32_t C = 0u, MX = 0u, NMN = 0u;
#pragma unroll
    for (int w = 0; w < DIR_WAVES; ++w) {
        C += f.red[0][w];
        MX = max(MX, f.red[1][w]);
        NMN = max(NMN, f.red[2][w]);
    }
    const uint32_t MN = ~NMN;
    uint32_t L;
    int sh0 = 0;
    bool have_cut = false;                               // h holds the summary's histogram
    uint3 r0 = make_uint3(0u, 0u, 0u);
    if (C < (uint32_t)k) {
        L = 0u;
    } else if (MX == MN) {
        L = MN;
    } else {
        sh0 = range_shift(MN, MX);
#pragma unroll
        for (int i = 0; i < DIR_PER; ++i)
            if (key[i]) atomicAdd(&f.h[RB_BINS - 1 - ((key[i] - MN) >> sh0)], 1u);
        __syncthreads();
        if (wave == 0) {
            // lane l sums bins [64l, 64l + 64), then the crossing lane's 64
            // bins one per lane: the bin, the count above it, the count in it
            uint32_t local = 0u;
            const uint4* hb = reinterpret_cast<const uint4*>(f.h) + 16 * lane;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint4 x = hb[q];
                local += x.x + x.y + x.z + x.w;
            }
            const uint32_t need = (uint32_t)k;
            const uint32_t inc = wave_inclusive_scan(local);
            const int cl = (int)__builtin_ctzll(__ballot(inc >= need && inc - local < need));
            const uint32_t base = __builtin_amdgcn_readlane(inc - local, cl);
            const uint32_t cbv = f.h[64 * cl + lane];
            const uint32_t inc2 = base + wave_inclusive_scan(cbv);
            const int bl = (int)__builtin_ctzll(__ballot(inc2 >= need && inc2 - cbv < need));
            if (lane == bl) {
                f.res[0] = (uint32_t)(64 * cl + bl);
                f.res[1] = inc2 - cbv;
                f.res[2] = cbv;
            }
        }
        __syncthreads();
        r0 = make_uint3(f.res[0], f.res[1], f.res[2]);
        L = MN + ((uint32_t)(RB_BINS - 1 - (int)r0.x) << sh0);
        have_cut = true;
    }
    const uint32_t Lc = L ? L : 1u;

    // 2. saturated chunks into the list; candidates of the others stay in
    // registers.  When the summary's cut bin is small its entries also go to
    // the cut list now (used only if no chunk turns out saturated: then the
    // candidates are the summary entries >= L and the summary's histogram
    // is theirs).
    const bool sat = has && Kb >= Lc;
    uint32_t cmask = 0u;
#pragma unroll
    for (int i = 0; i < DIR_PER; ++i) cmask |= (uint32_t)(!sat && key[i] >= Lc) << i;
    const bool spec = have_cut && r0.z <= (uint32_t)COL_MAX;
    const uint32_t width0 = (1u << sh0) - 1u;
    const uint32_t bhi0 = MX - L < width0 ? MX : L + width0;    // the summary's cut bin is [L, bhi0]
    {
        const bool lead = sat && sub == 0;
        const uint64_t lm = __ballot(lead);
        if (lm) {
            uint32_t b0 = 0u;
            if (lane == 0) b0 = atomicAdd(&f.nsat, (uint32_t)__popcll(lm));
            b0 = __builtin_amdgcn_readfirstlane(b0);
            if (lead) f.sat[b0 + (uint32_t)__popcll(lm & below)] = (uint32_t)blk;
        }
        if (spec) {
            // one LDS atomic per wave and entry index for the list's slots
#pragma unroll
            for (int i = 0; i < DIR_PER; ++i) {
                const bool in = ((cmask >> i) & 1u) && key[i] <= bhi0;
                const uint64_t im = __ballot(in);
                if (im) {
                    uint32_t b0 = 0u;
                    if (lane == 0) b0 = atomicAdd(&f.ncol, (uint32_t)__popcll(im));
                    b0 = __builtin_amdgcn_readfirstlane(b0);
                    const uint32_t slot = b0 + (uint32_t)__popcll(im & below);
                    if (in && slot < (uint32_t)COL_MAX) f.col[slot] = make_uint2(key[i], pos[i]);
                }
            }
        }
    }
    __syncthreads();
    const uint32_t nsat = f.nsat;

    uint32_t* const myw = &f.bits[WPT * tid];
    auto load_words = [&](uint32_t (&wv)[WPT]) {
#pragma unroll
        for (int u = 0; u < WPT; u += 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(myw + u);
            wv[u] = x.x; wv[u + 1] = x.y; wv[u + 2] = x.z; wv[u + 3] = x.w;
        }
    };
    auto set_bit = [&](uint32_t p) { atomicOr(&f.bits[p >> 5], 1u << (p & 31u)); };
    // the cut list's m entries ranked under (key desc, position asc): the
    // first need are selected
    auto mark_ranked = [&](uint32_t m, uint32_t need) {
        for (uint32_t t = tid; t < m; t += DIR_THREADS) {
            const uint2 e = f.col[t];
            uint32_t rank = 0u;
            for (uint32_t q = 0; q < m; ++q) {
                const uint2 o = f.col[q];
                rank += (uint32_t)(o.x > e.x) | ((uint32_t)(o.x == e.x) & (uint32_t)(o.y < e.y));
            }
            if (rank < need) set_bit(e.y);
        }
    };
    // 4. once the bitmap holds the k selected positions: each thread's bit
    // count, one wave scan and the waves' totals give its first output slot
    auto write_output = [&]() {
        uint32_t wv[WPT];
        load_words(wv);
        uint32_t local = 0u;
#pragma unroll
        for (int w = 0; w < WPT; ++w) local += (uint32_t)__popc(wv[w]);
        const uint32_t inc = wave_inclusive_scan(local);
        if (lane == 63) f.otot[wave] = inc;
        __syncthreads();
        uint32_t o = inc - local;
#pragma unroll
        for (int w = 0; w < DIR_WAVES; ++w) o += w < wave ? f.otot[w] : 0u;
#pragma unroll
        for (int w = 0; w < WPT; ++w) {
            uint32_t x = wv[w];
            while (x) {
                const uint32_t bit = (uint32_t)__builtin_ctz(x);
                x &= x - 1u;
                if (o < (uint32_t)k) out[o] = (int32_t)((uint32_t)(WPT * tid + w) * 32u + bit);
                ++o;
            }
        }
    };

    if (nsat == 0u && spec) {
        // the common case: the cut bin ranked directly, the entries above it
        // all selected
        mark_ranked(r0.z, (uint32_t)k - r0.y);
#pragma unroll
        for (int i = 0; i < DIR_PER; ++i)
            if (((cmask >> i) & 1u) && key[i] > bhi0) set_bit(pos[i]);
        __syncthreads();
        write_output();
        return;
    }
    if (tid == 0) f.ncol = 0u;              // the cut list starts again (next filled after barriers)

    const uint32_t total = nsat * TOPK_WAVE_CHUNK;
    const float* rowp = S + (size_t)row * L_cap;
    // the scores of the saturated chunks, DIR_UNROLL loads in flight per
    // thread (addresses clamped inside the visible row): fn(keep, key,
    // position), keep for the keys >= Lc
    auto scan_saturated = [&](auto fn) {
        for (uint32_t j0 = 0; j0 < total; j0 += DIR_UNROLL * DIR_THREADS) {
            float v[DIR_UNROLL];
            uint32_t sp[DIR_UNROLL];
#pragma unroll
            for (int u = 0; u < DIR_UNROLL; ++u) {
                const uint32_t j = j0 + (uint32_t)(u * DIR_THREADS + tid);
                const uint32_t jj = j < total ? j : total - 1u;
                sp[u] = wchunk_pos(f.sat[jj >> 8], jj & 255u);
                v[u] = rowp[sp[u] < (uint32_t)n ? sp[u] : (uint32_t)n - 1u];
            }
#pragma unroll
            for (int u = 0; u < DIR_UNROLL; ++u) {
                const uint32_t j = j0 + (uint32_t)(u * DIR_THREADS + tid);
                const uint32_t kk = j < total && sp[u] < (uint32_t)n ? score_key(v[u]) : 0u;
                fn(kk >= Lc, kk, sp[u]);
            }
        }
    };
    if (nsat > 0u) {
        scan_saturated([&](bool keep, uint32_t kk, uint32_t sp) {
            const uint64_t km = __ballot(keep);
            if (km) {
                uint32_t b0 = 0u;
                if (lane == 0) b0 = atomicAdd(&f.nstage, (uint32_t)__popcll(km));
                b0 = __builtin_amdgcn_readfirstlane(b0);
                if (keep) {
                    const uint32_t slot = b0 + (uint32_t)__popcll(km & below);
                    if (slot < (uint32_t)DIR_STAGE) f.stage[slot] = make_uint2(kk, sp);
                }
            }
        });
        __syncthreads();
    }
    const uint32_t nst = f.nstage;
    const bool overflow = nst > (uint32_t)DIR_STAGE;
    // every candidate once: fn(key, position)
    auto each = [&](auto fn) {
#pragma unroll
        for (int i = 0; i < DIR_PER; ++i)
            if ((cmask >> i) & 1u) fn(key[i], pos[i]);
        if (!overflow) {
            for (uint32_t j = tid; j < nst; j += DIR_THREADS) {
                const uint2 e = f.stage[j];
                fn(e.x, e.y);
            }
        } else {
            scan_saturated([&](bool keep, uint32_t kk, uint32_t sp) {
                if (keep) fn(kk, sp);
            });
        }
    };

    // 3. the exact cut
    uint32_t lo, hi, need = (uint32_t)k;
    const bool pre = nsat == 0u && have_cut;            // the summary's histogram is the first pass
    if (pre) {
        lo = MN;
        hi = MX;
    } else {
        uint32_t a = 0u, b = 0u;
        each([&](uint32_t kk, uint32_t) {
            a = max(a, kk);
            b = max(b, ~kk);
        });
        a = wave_max_u32(a);
        b = wave_max_u32(b);
        if (lane == 0) {                                 // red was last read before a barrier
            f.red[0][wave] = a;
            f.red[1][wave] = b;
        }
        __syncthreads();
        uint32_t A = 0u, B = 0u;
#pragma unroll
        for (int w = 0; w < DIR_WAVES; ++w) {
            A = max(A, f.red[0][w]);
            B = max(B, f.red[1][w]);
        }
        lo = ~B;
        hi = A;
    }
    uint32_t T;
    bool h_dirty = have_cut;
    for (bool first = true;; first = false) {
        int sh;
        uint3 r;
        if (first && pre) {
            sh = sh0;
            r = r0;
        } else {
            if (lo == hi) {
                T = lo;
                break;
            }
            sh = range_shift(lo, hi);
            if (h_dirty) {
                // every thread is past its reads of the previous histogram
                *reinterpret_cast<uint4*>(&f.h[4 * tid]) = make_uint4(0u, 0u, 0u, 0u);
                __syncthreads();
            }
            each([&](uint32_t kk, uint32_t) {
                if (kk >= lo && kk <= hi) atomicAdd(&f.h[RB_BINS - 1 - ((kk - lo) >> sh)], 1u);
            });
            __syncthreads();
            r = find_cut<DIR_THREADS>(f.h, need, f.tot, f.res);
            h_dirty = true;
        }
        const uint32_t b = (uint32_t)(RB_BINS - 1) - r.x;
        need -= r.y;                                     // >= 1 keys to take from bin b
        const uint32_t blo = lo + (b << sh);
        const uint32_t width = (1u << sh) - 1u;
        const uint32_t bhi = hi - blo < width ? hi : blo + width;
        if (r.z <= (uint32_t)COL_MAX) {
            // the bin's candidates to the cut list, the ones above it selected
            each([&](uint32_t kk, uint32_t p) {
                if (kk > bhi) {
                    set_bit(p);
                } else if (kk >= blo) {
                    const uint32_t slot = atomicAdd(&f.ncol, 1u);
                    if (slot < (uint32_t)COL_MAX) f.col[slot] = make_uint2(kk, p);
                }
            });
            __syncthreads();
            mark_ranked(r.z, need);
            __syncthreads();
            write_output();
            return;
        }
        if (sh == 0) {
            T = blo;
            break;
        }
        lo = blo;
        hi = bhi;
    }

    // a single key T holds the cut: P is the need-th lowest position among
    // the candidates equal to T (a bitmap of them, scanned)
    each([&](uint32_t kk, uint32_t p) {
        if (kk == T) set_bit(p);
    });
    __syncthreads();
    {
        uint32_t wv[WPT];
        load_words(wv);
        uint32_t local = 0u;
#pragma unroll
        for (int w = 0; w < WPT; ++w) local += (uint32_t)__popc(wv[w]);
        uint32_t all;
        const uint32_t before = block_exclusive_scan<DIR_THREADS>(local, &all, f.tot);
        if (before < need && before + local >= need) {
            uint32_t rem = need - before;
#pragma unroll
            for (int w = 0; w < WPT; ++w) {
                const uint32_t c = (uint32_t)__popc(wv[w]);
                if (rem > 0u && rem <= c) {
                    uint32_t x = wv[w];
                    for (uint32_t i = 1; i < rem; ++i) x &= x - 1u;
                    f.cut[1] = (uint32_t)(WPT * tid + w) * 32u + (uint32_t)__builtin_ctz(x);
                    rem = 0u;
                } else if (rem > 0u) {
                    rem -= c;
                }
            }
        }
        *reinterpret_cast<uint4*>(myw) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(myw + 4) = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
    }
    const uint32_t P = f.cut[1];
    each([&](uint32_t kk, uint32_t p) {
        if (kk > T || (kk == T && p <= P)) set_bit(p);
    });
    __syncthreads();
    write_output();
}

// ---------------------------------------------------------------------------
// Many rows of at most SEL_MAX_N positions (prefill): after the histogram
// kernel, one workgroup of 1024 threads per row does the rest in LDS.  With
// fewer rows than the chip has compute units (decode) the classify/finish
// pair spreads each row over many workgroups instead: one workgroup streams
// one row at only a fraction of the HBM rate.
//   1. the threshold bin from the row's histogram;
//   2. every wave streams its contiguous segment of the row in steps of 256
//      positions and appends the keys at or above the threshold bin to an LDS
//      entry list, one ordered run per step (recorded per wave and step), and
//      builds the candidates' second-digit histogram;
//   3. the exact k-th key T and position cut s_cut as in the finish kernel;
//   4. each wave counts the selected entries of its runs, the waves' counts
//      are scanned, and each wave writes its selected positions in order.
// If the entry list overflows, steps 3-4 read the row's scores again.
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_STEP = 256;                                    // positions per wave step
constexpr int SEL_MAX_N = 262144;
constexpr int SEL_MIN_ROWS = 256;
constexpr int SEL_MAX_STEPS = SEL_MAX_N / SEL_WAVES / SEL_STEP;  // 64
constexpr int SEL_UNROLL = 8;                                    // steps in flight per wave
constexpr int SEL_ENT = 12288;

struct SelectShared {
    uint2 ent[SEL_ENT];                          // (key, position) of the kept keys
    uint2 rec[SEL_WAVES][SEL_MAX_STEPS];         // (first entry, count) of every step's run
    uint32_t h2[HIST2_BINS];                     // candidates' second digit
    uint32_t sh[2048];                           // radix passes when many keys share the prefix
    uint2 col[COL_MAX];
    uint32_t wsum[SEL_WAVES];
    uint32_t alloc, ncol;
    uint32_t waves[SEL_WAVES];
    uint32_t res[4];
};

__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ hist, int32_t* __restrict__ idx) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = visible_count(kv_len, row, Tq, L_cap);
    int32_t* out = idx + (size_t)row * k;
    if (n <= k) {
        for (int j = tid; j < k; j += SEL_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    __shared__ SelectShared f;
    const float* rowp = S + (size_t)row * L_cap;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // 1. threshold bin
    for (int i = tid; i < HIST2_BINS; i += SEL_THREADS) f.h2[i] = 0;
    if (tid == 0) { f.alloc = 0; f.ncol = 0; }
    const uint2 th = find_bin<TOPK_HIST_BINS / SEL_THREADS, true, SEL_THREADS>(
        hist + (size_t)row * TOPK_HIST_BINS, (uint32_t)k, f.waves, f.res);   // barriers inside
    const uint32_t bin1 = th.x;

    // 2. stream the row: wave w owns [w * seg, (w + 1) * seg); position of
    // (step s, key e, lane) = w * seg + s * 256 + e * 64 + lane, so the order of
    // a step's keys is (e, lane)
    const int seg = ((n + SEL_WAVES * SEL_STEP - 1) / (SEL_WAVES * SEL_STEP)) * SEL_STEP;
    const int p0 = wave * seg;
    const int nsteps = p0 >= n ? 0 : (min(seg, n - p0) + SEL_STEP - 1) / SEL_STEP;
    for (int s0 = 0; s0 < nsteps; s0 += SEL_UNROLL) {
        float sc[SEL_UNROLL][4];
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = p0 + (s0 + u) * SEL_STEP + e * 64 + lane;
                sc[u][e] = (s0 + u < nsteps && pos < n) ? rowp[pos] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            if (s0 + u >= nsteps) break;
            const int sbase = p0 + (s0 + u) * SEL_STEP;
            uint32_t key[4];
            uint64_t b[4];
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = sbase + e * 64 + lane;
                const bool valid = pos < n;
                key[e] = valid ? score_key(sc[u][e]) : 0u;
                const uint32_t d = key[e] >> (32 - TOPK_HIST_BITS);
                if (valid && d == bin1) atomicAdd(&f.h2[(key[e] >> 10) & (HIST2_BINS - 1)], 1u);
                b[e] = __ballot(valid && d >= bin1);
                c[e] = (uint32_t)__popcll(b[e]);
            }
            const uint32_t cnt = c[0] + c[1] + c[2] + c[3];
            uint32_t base = 0;
            if (lane == 0 && cnt) base = atomicAdd(&f.alloc, cnt);
            base = __builtin_amdgcn_readfirstlane(base);
            if (lane == 0) f.rec[wave][s0 + u] = make_uint2(base, cnt);
            uint32_t before = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if ((b[e] >> lane) & 1ull) {
                    const uint32_t slot = base + before + (uint32_t)__popcll(b[e] & below);
                    if (slot < (uint32_t)SEL_ENT) f.ent[slot] = make_uint2(key[e], (uint32_t)(sbase + e * 64 + lane));
                }
                before += c[e];
            }
        }
    }
    __syncthreads();
    const uint32_t total = f.alloc;
    const bool overflow = total > (uint32_t)SEL_ENT;

    // f(key, pos) for every candidate of the threshold bin
    auto for_each_cand = [&](auto fn) {
        if (!overflow) {
            for (uint32_t i = tid; i < total; i += SEL_THREADS) {
                const uint2 e = f.ent[i];
                if ((e.x >> (32 - TOPK_HIST_BITS)) == bin1) fn(e.x, (int)e.y);
            }
        } else {
            for (int s = tid; s < n; s += SEL_THREADS) {
                const uint32_t key = score_key(rowp[s]);
                if ((key >> (32 - TOPK_HIST_BITS)) == bin1) fn(key, s);
            }
        }
    };

    // 3. exact cut
    uint32_t need = (uint32_t)k - th.y;          // >= 1 keys still to take from the bin
    const uint2 r2 = find_bin<HIST2_BINS / SEL_THREADS, true, SEL_THREADS>(f.h2, need, f.waves, f.res);
    need -= r2.y;                                // >= 1 keys to take among the prefix group
    const uint32_t pre22 = (bin1 << 10) | r2.x;
    for_each_cand([&](uint32_t key, int s) {
        if ((key >> 10) == pre22) {
            const uint32_t slot = atomicAdd(&f.ncol, 1u);
            if (slot < (uint32_t)COL_MAX) f.col[slot] = make_uint2(key, (uint32_t)s);
        }
    });
    __syncthreads();
    const uint32_t m = f.ncol;
    uint32_t T;
    int s_cut;
    if (m <= (uint32_t)COL_MAX) {
        for (uint32_t t = tid; t < m; t += SEL_THREADS) {
            const uint2 e = f.col[t];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < m; ++j) {
                const uint2 o = f.col[j];
                rank += (uint32_t)(o.x > e.x) | ((uint32_t)(o.x == e.x) & (uint32_t)(o.y < e.y));
            }
            if (rank == need - 1) { f.res[2] = e.x; f.res[3] = e.y; }
        }
        __syncthreads();
        T = f.res[2];
        s_cut = (int)f.res[3];
    } else {
        uint32_t* sh = f.sh;
        for (int i = tid; i < 1024; i += SEL_THREADS) sh[i] = 0;
        __syncthreads();
        for_each_cand([&](uint32_t key, int) {
            if ((key >> 10) == pre22) atomicAdd(&sh[key & 1023u], 1u);
        });
        __syncthreads();
        const uint2 r3 = find_bin<1024 / SEL_THREADS, true, SEL_THREADS>(sh, need, f.waves, f.res);
        need -= r3.y;
        T = (pre22 << 10) | r3.x;
        for (int i = tid; i < 2048; i += SEL_THREADS) sh[i] = 0;
        __syncthreads();
        for_each_cand([&](uint32_t key, int s) {
            if (key == T) atomicAdd(&sh[(uint32_t)s >> 10], 1u);
        });
        __syncthreads();
        const uint2 q2 = find_bin<2048 / SEL_THREADS, false, SEL_THREADS>(sh, need, f.waves, f.res);
        const uint32_t p2 = q2.x;
        need -= q2.y;
        for (int i = tid; i < 1024; i += SEL_THREADS) sh[i] = 0;
        __syncthreads();
        for_each_cand([&](uint32_t key, int s) {
            if (key == T && ((uint32_t)s >> 10) == p2) atomicAdd(&sh[(uint32_t)s & 1023u], 1u);
        });
        __syncthreads();
        const uint32_t p3 = find_bin<1024 / SEL_THREADS, false, SEL_THREADS>(sh, need, f.waves, f.res).x;
        s_cut = (int)((p2 << 10) | p3);
    }
    __syncthreads();
    // branch-free selection test (see the finish kernel)
    auto sel_of = [&](uint32_t key, uint32_t s) -> uint32_t {
        return (uint32_t)(key > T) | ((uint32_t)(key == T) & (uint32_t)(s <= (uint32_t)s_cut));
    };

    // 4. ordered output: per wave, its runs (or, after an overflow, its segment
    // of the row) in order
    auto walk = [&](auto emit) {
        if (!overflow) {
            for (int s = 0; s < nsteps; ++s) {
                const uint2 r = f.rec[wave][s];
                for (uint32_t j0 = 0; j0 < r.y; j0 += 64) {
                    const uint32_t jj = j0 + lane;
                    const uint2 e = f.ent[r.x + (jj < r.y ? jj : 0u)];
                    emit((uint32_t)(jj < r.y) & sel_of(e.x, e.y), e.y);
                }
            }
        } else {
            for (int s = 0; s < nsteps; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pos = p0 + s * SEL_STEP + e * 64 + lane;
                    const uint32_t in = pos < n ? 1u : 0u;
                    const uint32_t key = in ? score_key(rowp[pos]) : 0u;
                    emit(in & sel_of(key, (uint32_t)pos), (uint32_t)pos);
                }
        }
    };
    uint32_t cnt_w = 0;
    walk([&](uint32_t sel, uint32_t) { cnt_w += (uint32_t)__popcll(__ballot(sel)); });
    if (lane == 0) f.wsum[wave] = cnt_w;
    __syncthreads();
    uint32_t o = 0;
    for (int w = 0; w < wave; ++w) o += f.wsum[w];
    walk([&](uint32_t sel, uint32_t pos) {
        const uint64_t bb = __ballot(sel);
        const uint32_t at = o + (uint32_t)__popcll(bb & below);
        if (sel && at < (uint32_t)k) out[at] = (int32_t)pos;   // exactly k are selected
        o += (uint32_t)__popcll(bb);
    });
}

}  // namespace

bool topk_uses_select(int rows, int L_cap) {
    return L_cap <= SEL_MAX_N && rows >= SEL_MIN_ROWS;
}

TopkLayout topk_layout(int rows, int L_cap, int k, bool fused) {
    TopkLayout L;
    L.rows = rows;
    L.nchunks = (L_cap + TOPK_CHUNK - 1) / TOPK_CHUNK;
    // wave chunks of 256 positions (4 per 1024-position indexer workgroup)
    L.nwchunks = (L_cap + 4 * TOPK_WAVE_CHUNK - 1) / (4 * TOPK_WAVE_CHUNK) * 4;
    // the one-workgroup-per-row select kernel needs only the first-digit
    // histograms; the direct kernel the summary (8 or 16 keys per wave chunk,
    // up to TOPK_MAX_SUMMARY per row, at least 2k); the filter/finish pair
    // the summary (about 2k keys per row), the run lengths and the entry slots
    // direct path: Mmin, the smallest of 8, 16, 32 keys per wave chunk that
    // gives the row at least 2k summary keys within TOPK_MAX_SUMMARY, or twice
    // that (up to 32), with which few chunks saturate (a saturated chunk costs
    // the direct kernel a second read and more passes).  Twice Mmin when the
    // indexer's epilogue writes the summary or the rows are few; Mmin when a
    // summary kernel over many rows pays for every key of M (its rounds are
    // bound by VALU issue)
    int Mmin = 0;
    for (int m = 8; m <= TOPK_DIRECT_MAX_M && Mmin == 0; m *= 2)
        if ((long long)L.nwchunks * m >= 2LL * k && L.nwchunks * m <= TOPK_MAX_SUMMARY) Mmin = m;
    int Md = fused || rows <= TOPK_FEW_ROWS ? 2 * Mmin : Mmin;
    while (Md > TOPK_DIRECT_MAX_M || L.nwchunks * Md > TOPK_MAX_SUMMARY) Md /= 2;
    L.direct = Mmin != 0 && L_cap <= DIR_MAX_N;
    L.select = !L.direct && topk_uses_select(rows, L_cap);
    const bool sel = L.select;
    int M = (int)((2LL * k * TOPK_WAVE_CHUNK + L_cap - 1) / L_cap);
    M = M < 1 ? 1 : (M > TOPK_MAX_M ? TOPK_MAX_M : M);
    L.M = L.direct ? Md : M;
    const bool runs = !sel && !L.direct;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    // counters zeroed at the start of every call come first
    L.hist = take(sel ? (size_t)rows * TOPK_HIST_BINS * 4 : 0);
    L.zero_bytes = off;
    // scratch overwritten by every call
    L.summary = take(sel ? 0 : (size_t)rows * L.nwchunks * L.M * 4);
    L.codes = take(sel ? 0 : (size_t)rows * L.nwchunks * L.M);
    L.counts = take(runs ? (size_t)rows * L.nchunks * 4 : 0);
    L.ent = take(runs ? (size_t)rows * L.nchunks * TOPK_SLOT_CAP * 8 : 0);
    L.total = off;
    return L;
}

hipError_t launch_clear_u32(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n / 4 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(clear_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                              int k, int32_t* idx, void* ws, bool counters_clear,
                              hipStream_t stream, bool summary_ready) {
    const int rows = B * Tq;
    const TopkLayout L = topk_layout(rows, L_cap, k, summary_ready);
    char* base = static_cast<char*>(ws);
    if (L.select) {
        uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
        if (!counters_clear) {
            hipError_t e = launch_clear_u32(reinterpret_cast<uint32_t*>(base), L.zero_bytes / 4, stream);
            if (e != hipSuccess) return e;
        }
        constexpr int CH_MANY = HIST_THREADS * HIST_PER_MANY, CH_FEW = HIST_THREADS * HIST_PER_FEW;
        const size_t wgs_many = (size_t)rows * ((L_cap + CH_MANY - 1) / CH_MANY);
        if (wgs_many >= (size_t)HIST_MIN_WGS || (L_cap + CH_FEW - 1) / CH_FEW > HIST_MAX_FEW_CHUNKS)
            hipLaunchKernelGGL(topk_hist_kernel<HIST_PER_MANY>, dim3((L_cap + CH_MANY - 1) / CH_MANY, rows),
                               dim3(HIST_THREADS), 0, stream, S, kv_len, Tq, L_cap, k, hist);
        else
            hipLaunchKernelGGL(topk_hist_kernel<HIST_PER_FEW>, dim3((L_cap + CH_FEW - 1) / CH_FEW, rows),
                               dim3(HIST_THREADS), 0, stream, S, kv_len, Tq, L_cap, k, hist);
        hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(SEL_THREADS), 0, stream, S,
                           kv_len, Tq, L_cap, k, hist, idx);
        return hipGetLastError();
    }
    uint32_t* summary = reinterpret_cast<uint32_t*>(base + L.summary);
    uint8_t* codes = reinterpret_cast<uint8_t*>(base + L.codes);
    uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.counts);
    uint2* ent = reinterpret_cast<uint2*>(base + L.ent);
    if (!summary_ready)
        hipLaunchKernelGGL(topk_summary_kernel, dim3(L.nwchunks / 4, rows), dim3(SUM_THREADS), 0,
                           stream, S, kv_len, Tq, L_cap, L.M, L.nwchunks, summary, codes);
    if (L.direct) {
        if (L_cap <= DIR_MAX_N / 2)
            hipLaunchKernelGGL(topk_direct_kernel<4>, dim3(rows), dim3(DIR_THREADS), 0, stream, S,
                               kv_len, Tq, L_cap, k, summary, codes, L.nwchunks, L.M, idx);
        else
            hipLaunchKernelGGL(topk_direct_kernel<8>, dim3(rows), dim3(DIR_THREADS), 0, stream, S,
                               kv_len, Tq, L_cap, k, summary, codes, L.nwchunks, L.M, idx);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_filter_kernel, dim3(L.nchunks, rows), dim3(TOPK_THREADS), 0, stream, S,
                       kv_len, Tq, L_cap, k, summary, L.nwchunks * L.M, counts, ent, L.nchunks);
    // threads per chunk in the finish: FIN_THREADS over the chunk count rounded up to a power of two
    int tpc_log2 = 10;
    while ((1 << (10 - tpc_log2)) < L.nchunks) --tpc_log2;
    hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(FIN_THREADS), 0, stream, kv_len, Tq,
                       L_cap, k, counts, ent, L.nchunks, tpc_log2, idx);
    return hipGetLastError();
}

}  // namespace isa
