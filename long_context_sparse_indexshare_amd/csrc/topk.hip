// Top-k position select over fp32 scores (gfx950).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1: keep the top-K positions; K = index_topk = 2048 in the config fragment
// of "GLM-5.2核心技术解析"): for each query, the min(k, pos+1) visible positions
// that come first under (score descending, position ascending), listed in
// ascending position and padded with -1.
//
// Scores are compared as order-preserving 32-bit keys.  Few rows of up to
// 2^21 positions (decode) are spread over many workgroups per row:
//   0. summary:  for every run of 256 positions, its M largest keys (written
//                by the indexer's epilogue in the group call, else by a
//                summary kernel).  M is chosen so the row's summary holds
//                about 2k keys.
//   1. filter:   every workgroup derives from the row's summary a threshold L
//                with at least k summary keys >= L (the summary's keys are
//                scores of distinct visible positions, so at least k scores
//                are >= L: the k-th largest is >= L), then keeps its chunk's
//                scores >= L as one run of (key, position) entries in
//                ascending position.  On random scores L sits a few percent
//                below the k-th largest, so a row keeps little more than k
//                entries.
//   2. finish:   one workgroup per row finds the exact k-th key T and the
//                position cut among keys equal to T by radix passes over the
//                bits the candidates do not share, then writes the selected
//                positions as the ordered stream compaction of the runs taken
//                chunk by chunk.  If the entry buffer overflowed (a very flat
//                score distribution) the row's scores are read again.
// With at least 256 rows of at most 262144 positions (a prefill chunk) a
// first-digit histogram kernel and one workgroup per row
// (topk_select_kernel) do the work instead.
// Workgroups never wait on each other inside a kernel: on gfx950 a device-
// scope fence writes back and invalidates the whole L2 of the XCD, so each
// hand-over between workgroups goes through a kernel boundary instead.
#include <type_traits>

#include "isa_internal.h"

namespace isa {

namespace {

constexpr int CAND_MIN = 16384;

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
// covers positions c*1024 + w*256 + e*64 + lane (e < 4), wave chunk c*4 + w,
// and writes that chunk's M largest keys; invisible positions take key 0.
// Chunk 0 also zeroes the row's entry counter for the filter that follows.
constexpr int SUM_THREADS = 256;
__global__ __launch_bounds__(SUM_THREADS) void topk_summary_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int M,
    int nwchunks, uint32_t* __restrict__ summary, uint32_t* __restrict__ alloc) {
    const int row = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int base = blockIdx.x * (4 * TOPK_WAVE_CHUNK) + wave * TOPK_WAVE_CHUNK;
    const float* rowp = S + (size_t)row * L_cap;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int s = base + e * 64 + lane;
        v[e] = s < L_cap ? rowp[s] : 0.0f;
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    uint32_t key[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) key[e] = base + e * 64 + lane < n ? score_key(v[e]) : 0u;
    wave_top_m<4>(key, M, summary + ((size_t)row * nwchunks + blockIdx.x * 4 + wave) * M);
    if (blockIdx.x == 0 && threadIdx.x == 0) alloc[row] = 0u;
}

// Threshold of a row from its summary (nsum keys, SUM_PER per thread, key 0
// = none): with P the bits every summary key shares, two 8-bit digits of the
// bits below them are fixed in turn, each the largest digit that still has
// at least k summary keys at or above it; the threshold is P with those two
// digits and zeros below (0 when the summary holds fewer than k keys).  The
// summary keys are scores of distinct visible positions, so at least k of
// the row's scores are >= the threshold.  Every thread returns the same value.
constexpr int SUM_PER = TOPK_MAX_SUMMARY / TOPK_THREADS;
struct ThresholdShared {
    uint32_t red[3][TOPK_THREADS / 64];   // per wave: count, max, ~min
    uint32_t h[256];
    uint32_t res[2];                      // digit, count in the bins above it
};

__device__ __forceinline__ uint32_t summary_threshold(const uint32_t (&u)[SUM_PER], uint32_t k,
                                                      ThresholdShared& t) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
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
        t.red[0][wave] = cnt;
        t.red[1][wave] = mx;
        t.red[2][wave] = nmn;
    }
    __syncthreads();
    uint32_t C = 0, MX = 0, NMN = 0;
#pragma unroll
    for (int w = 0; w < TOPK_THREADS / 64; ++w) {
        C += t.red[0][w];
        MX = max(MX, t.red[1][w]);
        NMN = max(NMN, t.red[2][w]);
    }
    if (C < k) return 0u;
    const uint32_t MN = ~NMN;
    const uint32_t x = MX ^ MN;
    if (x == 0u) return MN;                             // every summary key equal
    int hb = 31 - __builtin_clz(x);                     // highest bit the keys differ in
    uint32_t fval = hb >= 31 ? 0u : (MX >> (hb + 1)) << (hb + 1);
    uint32_t fmask = hb >= 31 ? 0u : ~((1u << (hb + 1)) - 1u);
    uint32_t need = k;
    for (int pass = 0; pass < 2 && hb >= 0; ++pass) {
        const int nb = hb + 1 < 8 ? hb + 1 : 8;
        const int sh = hb - nb + 1;
        const uint32_t bm = (1u << nb) - 1u;
        if (threadIdx.x < 256) t.h[threadIdx.x] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SUM_PER; ++i)
            if (u[i] && (u[i] & fmask) == fval) atomicAdd(&t.h[(u[i] >> sh) & bm], 1u);
        __syncthreads();
        if (wave == 0) {
            // bins in descending order: lane l holds bins 255-4l .. 252-4l
            uint32_t hv[4], local = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hv[j] = t.h[255 - 4 * lane - j];
                local += hv[j];
            }
            const uint32_t inc = wave_inclusive_scan(local);
            const uint32_t before = inc - local;
            if (before < need && inc >= need) {
                uint32_t acc = before;
                int d = 0;
                uint32_t above = 0;
                bool found = false;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (!found && acc + hv[j] >= need) {
                        d = 255 - 4 * lane - j;
                        above = acc;
                        found = true;
                    }
                    acc += hv[j];
                }
                t.res[0] = (uint32_t)d;
                t.res[1] = above;
            }
        }
        __syncthreads();
        fval |= t.res[0] << sh;
        fmask |= bm << sh;
        need -= t.res[1];
        hb = sh - 1;
        __syncthreads();                                // t.h and t.res read before the next pass
    }
    return fval;
}

// Filter: every workgroup (4096 positions of one row) derives the row's
// threshold L from the summary and keeps its chunk's visible keys >= L as one
// run of (key, position) entries in ascending position.  One atomic per
// workgroup reserves the run in the row's entry buffer; the runs of a row
// tile [0, total) with no gaps, and runs[row][chunk] records where each
// chunk's run starts and how long it is.  Chunk 0 records L for the finish.
__global__ __launch_bounds__(TOPK_THREADS) void topk_filter_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ summary, int nsum, uint32_t* __restrict__ alloc,
    uint32_t* __restrict__ row_L, uint2* __restrict__ runs, uint2* __restrict__ ent, uint32_t cap,
    int nchunks_max) {
    const int row = blockIdx.y;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int NW = TOPK_THREADS / 64;
    static_assert(TOPK_PER_THREAD * NW == 64, "one wave scans the (e, wave) counts");
    __shared__ ThresholdShared ts;
    __shared__ uint32_t sh_cnt[TOPK_PER_THREAD][NW];   // then the exclusive offsets
    __shared__ uint32_t sh_base;

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
    const uint32_t L = summary_threshold(u, (uint32_t)k, ts);
    if (c == 0 && tid == 0) row_L[row] = L;

    uint32_t keys[TOPK_PER_THREAD];
    uint64_t kept[TOPK_PER_THREAD];
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        const bool valid = s < n;
        keys[e] = valid ? score_key(sc[e]) : 0u;
        kept[e] = __ballot(valid && keys[e] >= L);
        if (lane == 0) sh_cnt[e][wave] = (uint32_t)__popcll(kept[e]);
    }
    __syncthreads();
    if (wave == 0) {
        // exclusive scan of the 64 (e, wave) counts in ascending-position order
        const uint32_t v = sh_cnt[lane / NW][lane % NW];
        const uint32_t inc = wave_inclusive_scan(v);
        const uint32_t total = __builtin_amdgcn_readlane(inc, 63);
        sh_cnt[lane / NW][lane % NW] = inc - v;
        if (lane == 0) {
            const uint32_t base = total ? atomicAdd(&alloc[row], total) : 0u;
            sh_base = base;
            runs[(size_t)row * nchunks_max + c] = make_uint2(base, total);
        }
    }
    __syncthreads();
    const uint32_t base = sh_base;
    uint2* re = ent + (size_t)row * cap;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        if ((kept[e] >> lane) & 1ull) {
            const uint32_t slot = base + sh_cnt[e][wave] + (uint32_t)__popcll(kept[e] & below);
            if (slot < cap) re[slot] = make_uint2(keys[e], (uint32_t)(start + e * TOPK_THREADS + tid));
        }
    }
}

// LDS of the finishing step.
constexpr int FIN_THREADS = 1024;
constexpr int FIN_WAVES = FIN_THREADS / 64;
constexpr int FIN_SPEC = 6;               // entries per thread requested before the total is known
constexpr int FIN_LDS_PER = ENT_LDS / FIN_THREADS;
constexpr int FIN_PER = 8;                // entries per thread per compaction tile
constexpr int FIN_DIGIT = 12;             // bits per radix pass of the exact cut
constexpr int FIN_BINS = 1 << FIN_DIGIT;
static_assert(TOPK_MAX_CHUNKS <= FIN_THREADS, "one chunk per thread");
static_assert(ENT_LDS % FIN_THREADS == 0 && FIN_SPEC <= FIN_LDS_PER, "staging geometry");
static_assert(FIN_BINS % FIN_THREADS == 0, "digit bins per thread");
struct FinishShared {
    uint32_t sh[FIN_BINS];                // digit histograms
    uint32_t cbase[TOPK_MAX_CHUNKS];      // chunk -> first entry of its run
    uint32_t cstart[TOPK_MAX_CHUNKS + 1]; // chunk -> index of its run's first entry in chunk order
    uint2 lent[ENT_LDS];                  // the row's entries, in allocation order
    uint2 col[COL_MAX];                   // entries of the cut's bin, ranked directly
    uint32_t ncol;
    uint32_t waves[FIN_WAVES];
    uint32_t red[2][FIN_WAVES];
    uint32_t res[4];
};

// Finish: one workgroup per row.  The candidates are the row's keys >= L (at
// least k of them).  The exact k-th key T and the last selected position
// s_cut among keys equal to T follow from radix passes over the bits the
// candidates do not all share (12 bits per pass, highest first): each pass
// histograms the candidates that match the bits fixed so far and fixes the
// digit holding the k-th key; once that digit's bin holds at most COL_MAX
// entries they are ranked directly under (key desc, position asc), and if
// every key bit gets fixed first, two passes over the position bits of the
// keys equal to T give s_cut.  The runs, taken in chunk order, list the
// candidates in ascending position, so one flattened pass (eight consecutive
// entries per thread, the bounds of the thread's run and of the next one read
// together, and one block scan of the selected counts) writes the selected
// positions in order.  If the entry buffer overflowed, the row's scores are
// read instead of the entries.
__global__ __launch_bounds__(FIN_THREADS) void topk_finish_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ alloc, const uint32_t* __restrict__ row_L,
    const uint2* __restrict__ runs, const uint2* __restrict__ ent, uint32_t cap, int nchunks_max,
    int32_t* __restrict__ idx) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint2* re = ent + (size_t)row * cap;
    // every load of this phase is issued before any is used, and before the
    // row's visible length arrives: the entry count, the threshold, the chunk
    // table and the first entries (all inside the row's workspace; entries
    // past the row's total, chunks past its length and the whole lot for a
    // row that needs no selection are loaded but never used)
    const uint32_t total = alloc[row];
    const uint32_t Lr = row_L[row];
    const uint2 rr_all = tid < nchunks_max ? runs[(size_t)row * nchunks_max + tid] : make_uint2(0u, 0u);
    const uint32_t nspec = cap < (uint32_t)(FIN_SPEC * FIN_THREADS) ? cap : (uint32_t)(FIN_SPEC * FIN_THREADS);
    uint2 v[FIN_SPEC];
#pragma unroll
    for (int u = 0; u < FIN_SPEC; ++u) {
        const uint32_t i = u * FIN_THREADS + tid;
        v[u] = i < nspec ? re[i] : make_uint2(0u, 0u);
    }
    const int n = visible_count(kv_len, row, Tq, L_cap);
    int32_t* out = idx + (size_t)row * k;
    if (n <= k) {
        // every visible position, then -1 padding
        for (int j = tid; j < k; j += FIN_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    __shared__ FinishShared f;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const float* rowp = S + (size_t)row * L_cap;
    const uint2 rr = tid < nch ? rr_all : make_uint2(0u, 0u);
    // 0: entries staged in LDS; 1: read from the entry buffer; 2: buffer overflowed, re-read S
    const int mode = total <= (uint32_t)ENT_LDS ? 0 : (total <= cap ? 1 : 2);
    if (mode == 0) {
#pragma unroll
        for (int u = 0; u < FIN_SPEC; ++u) {
            const uint32_t i = u * FIN_THREADS + tid;
            if (i < total) f.lent[i] = v[u];
        }
        if (total > (uint32_t)(FIN_SPEC * FIN_THREADS)) {
            uint2 w[FIN_LDS_PER - FIN_SPEC];
#pragma unroll
            for (int u = 0; u < FIN_LDS_PER - FIN_SPEC; ++u) {
                const uint32_t i = (FIN_SPEC + u) * FIN_THREADS + tid;
                w[u] = i < total ? re[i] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < FIN_LDS_PER - FIN_SPEC; ++u) {
                const uint32_t i = (FIN_SPEC + u) * FIN_THREADS + tid;
                if (i < total) f.lent[i] = w[u];
            }
        }
    }
    if (tid < nch) f.cbase[tid] = rr.x;
    uint32_t ntot;
    const uint32_t cs = block_exclusive_scan<FIN_THREADS>(tid < nch ? rr.y : 0u, &ntot, f.waves);
    if (tid < nch) f.cstart[tid] = cs;
    if (tid == 0) f.cstart[nch] = ntot;
    __syncthreads();

    // f(key, pos) for every candidate
    auto for_each_cand = [&](auto fn) {
        if (mode == 0) {
            for (uint32_t i = tid; i < total; i += FIN_THREADS) {
                const uint2 e = f.lent[i];
                fn(e.x, (int)e.y);
            }
        } else if (mode == 1) {
            for (uint32_t i = tid; i < total; i += FIN_THREADS) {
                const uint2 e = re[i];
                fn(e.x, (int)e.y);
            }
        } else {
            for (int s = tid; s < n; s += FIN_THREADS) {
                const uint32_t key = score_key(rowp[s]);
                if (key >= Lr) fn(key, s);
            }
        }
    };

    // largest and smallest candidate key: the bits above the highest bit
    // they differ in are common to every candidate
    uint32_t mx = 0u, nmn = 0u;
    for_each_cand([&](uint32_t key, int) {
        mx = max(mx, key);
        nmn = max(nmn, ~key);
    });
    mx = wave_max_u32(mx);
    nmn = wave_max_u32(nmn);
    if (lane == 0) {
        f.red[0][wave] = mx;
        f.red[1][wave] = nmn;
    }
    __syncthreads();
    uint32_t MX = 0u, NMN = 0u;
#pragma unroll
    for (int w = 0; w < FIN_WAVES; ++w) {
        MX = max(MX, f.red[0][w]);
        NMN = max(NMN, f.red[1][w]);
    }
    const uint32_t diff = MX ^ ~NMN;
    int hb = diff ? 31 - __builtin_clz(diff) : -1;      // bits above hb are fixed
    uint32_t fval = hb >= 31 ? 0u : (hb < 0 ? MX : (MX >> (hb + 1)) << (hb + 1));
    uint32_t fmask = hb >= 31 ? 0u : (hb < 0 ? ~0u : ~((1u << (hb + 1)) - 1u));
    uint32_t need = (uint32_t)k;                        // keys still to take among the matches
    uint32_t T = 0u;
    int s_cut = -1;
    bool ranked = false;
    for (;;) {
        if (hb < 0) break;
        const int nb = hb + 1 < FIN_DIGIT ? hb + 1 : FIN_DIGIT;
        const int sh = hb - nb + 1;
        const uint32_t bm = (1u << nb) - 1u;
        __syncthreads();                                // previous readers of f.sh are done
        for (int i = tid; i < FIN_BINS; i += FIN_THREADS) f.sh[i] = 0u;
        if (tid == 0) f.ncol = 0u;
        __syncthreads();
        for_each_cand([&](uint32_t key, int) {
            if ((key & fmask) == fval) atomicAdd(&f.sh[(key >> sh) & bm], 1u);
        });
        __syncthreads();
        const uint2 r = find_bin<FIN_BINS / FIN_THREADS, true, FIN_THREADS>(f.sh, need, f.waves,
                                                                             f.res);
        const uint32_t m = f.sh[r.x];                   // entries of the cut's bin
        need -= r.y;                                    // >= 1 keys to take from that bin
        fval |= r.x << sh;
        fmask |= bm << sh;
        hb = sh - 1;
        if (m <= (uint32_t)COL_MAX) {
            // rank the bin's entries directly under (key desc, position asc);
            // the one of rank need-1 is the last selected
            for_each_cand([&](uint32_t key, int s) {
                if ((key & fmask) == fval) {
                    const uint32_t slot = atomicAdd(&f.ncol, 1u);
                    f.col[slot] = make_uint2(key, (uint32_t)s);
                }
            });
            __syncthreads();
            for (uint32_t t = tid; t < m; t += FIN_THREADS) {
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
            ranked = true;
            break;
        }
    }
    if (!ranked) {
        // every key bit is fixed: T = fval, and among the keys equal to T the
        // need lowest positions are selected (position bits [20:10], then [9:0])
        T = fval;
        __syncthreads();
        for (int i = tid; i < 2048; i += FIN_THREADS) f.sh[i] = 0u;
        __syncthreads();
        for_each_cand([&](uint32_t key, int s) {
            if (key == T) atomicAdd(&f.sh[(uint32_t)s >> 10], 1u);
        });
        __syncthreads();
        const uint2 q2 = find_bin<2048 / FIN_THREADS, false, FIN_THREADS>(f.sh, need, f.waves, f.res);
        const uint32_t p2 = q2.x;
        need -= q2.y;
        for (int i = tid; i < 1024; i += FIN_THREADS) f.sh[i] = 0u;
        __syncthreads();
        for_each_cand([&](uint32_t key, int s) {
            if (key == T && ((uint32_t)s >> 10) == p2) atomicAdd(&f.sh[(uint32_t)s & 1023u], 1u);
        });
        __syncthreads();
        const uint32_t p3 = find_bin<1024 / FIN_THREADS, false, FIN_THREADS>(f.sh, need, f.waves, f.res).x;
        s_cut = (int)((p2 << 10) | p3);
    }
    __syncthreads();

    // selected: a key above T, or equal to T at a position <= s_cut.
    // Evaluated without branches: the compiler lost the value of a
    // conditionally written position on the short-circuit form of this test.
    auto sel_of = [&](uint32_t key, uint32_t s) -> uint32_t {
        return (uint32_t)(key > T) | ((uint32_t)(key == T) & (uint32_t)(s <= (uint32_t)s_cut));
    };

    if (mode == 2) {
        // overflow: ordered stream compaction over the row's scores
        constexpr int PER = 8;
        constexpr int TILE = PER * FIN_THREADS;
        uint32_t written = 0;
        for (uint32_t t0 = 0; t0 < (uint32_t)n; t0 += TILE) {
            const uint32_t v0 = t0 + (uint32_t)tid * PER;
            uint32_t selmask = 0;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const uint32_t vv = v0 + u;
                const uint32_t in = vv < (uint32_t)n ? 1u : 0u;
                const uint32_t key = in ? score_key(rowp[vv]) : 0u;
                selmask |= (in & sel_of(key, vv)) << u;
            }
            uint32_t tile_total;
            uint32_t o = written + block_exclusive_scan<FIN_THREADS>((uint32_t)__popc(selmask),
                                                                     &tile_total, f.waves);
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                if ((selmask >> u) & 1u) {
                    if (o < (uint32_t)k) out[o] = (int32_t)(v0 + u);   // exactly k are selected
                    ++o;
                }
            }
            written += tile_total;
        }
        return;
    }

    // ordered compaction over the runs in chunk order; the LDS and global
    // entry sources are separate instantiations so that no load goes through
    // a generic pointer
    auto compact = [&](auto source) {
        constexpr bool LDS = decltype(source)::value;
        auto get = [&](uint32_t a) -> uint2 {
            if constexpr (LDS) return f.lent[a];
            else return re[a];
        };
        uint32_t written = 0;
        for (uint32_t t0 = 0; t0 < ntot; t0 += FIN_PER * FIN_THREADS) {
            const uint32_t i0 = t0 + (uint32_t)tid * FIN_PER;
            // the run holding entry i0: the last chunk whose run starts at or
            // before it (past the end: the last entry, whose result is masked)
            const uint32_t a0 = i0 < ntot ? i0 : ntot - 1;
            int lo = 0, hi = nch - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (f.cstart[mid] <= a0) lo = mid;
                else hi = mid - 1;
            }
            const int c = lo;
            // The thread's entries lie in run c and, past one boundary, in run
            // c + 1: both runs' bounds are read at once (clamped indices; run
            // c + 1 is only used when it exists).  The 64 lanes of a wave span
            // several boundaries, so a per-entry walk would cost a dependent
            // LDS read at nearly every step.  Entries past run c + 1 (runs
            // shorter than FIN_PER entries) take the walk.
            const int c1 = c + 1 < nch ? c + 1 : nch - 1;
            const int c2 = c + 2 <= nch ? c + 2 : nch;
            const uint32_t run_s = f.cstart[c], run_e = f.cstart[c + 1], run_b = f.cbase[c];
            const uint32_t run_e2 = f.cstart[c2], run_b2 = f.cbase[c1];
            uint32_t pos[FIN_PER];
            uint32_t selmask = 0;
#pragma unroll
            for (int u = 0; u < FIN_PER; ++u) {
                const uint32_t i = i0 + u;
                const uint32_t a = i < ntot ? i : ntot - 1;
                uint32_t slot;
                if (a < run_e) {
                    slot = run_b + (a - run_s);
                } else if (a < run_e2) {
                    slot = run_b2 + (a - run_e);
                } else {
                    int cc = c + 1;
                    while (f.cstart[cc + 1] <= a) ++cc;
                    slot = f.cbase[cc] + (a - f.cstart[cc]);
                }
                const uint2 e = get(slot);
                pos[u] = e.y;
                selmask |= ((uint32_t)(i < ntot) & sel_of(e.x, e.y)) << u;
            }
            uint32_t tile_total;
            uint32_t o = written + block_exclusive_scan<FIN_THREADS>((uint32_t)__popc(selmask),
                                                                     &tile_total, f.waves);
#pragma unroll
            for (int u = 0; u < FIN_PER; ++u) {
                if ((selmask >> u) & 1u) {
                    if (o < (uint32_t)k) out[o] = (int32_t)pos[u];   // exactly k are selected
                    ++o;
                }
            }
            written += tile_total;
        }
    };
    if (mode == 0) compact(std::true_type{});
    else compact(std::false_type{});
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

TopkLayout topk_layout(int rows, int L_cap, int k) {
    TopkLayout L;
    L.rows = rows;
    L.nchunks = (L_cap + TOPK_CHUNK - 1) / TOPK_CHUNK;
    // wave chunks of 256 positions (4 per 1024-position indexer workgroup)
    L.nwchunks = (L_cap + 4 * TOPK_WAVE_CHUNK - 1) / (4 * TOPK_WAVE_CHUNK) * 4;
    // summary keys per wave chunk: about 2k per row in all
    int M = (int)((2LL * k * TOPK_WAVE_CHUNK + L_cap - 1) / L_cap);
    L.M = M < 1 ? 1 : (M > TOPK_MAX_M ? TOPK_MAX_M : M);
    uint32_t cap = (uint32_t)(L_cap / 8);
    const uint32_t lo = (uint32_t)(L_cap < 2 * CAND_MIN ? L_cap : 2 * CAND_MIN);
    if (cap < lo) cap = lo;
    cap = (cap + 63u) & ~63u;
    L.cap = cap;
    // the one-workgroup-per-row select kernel needs only the first-digit
    // histograms; the filter/finish pair needs the entry counters, the
    // thresholds, the summary and its entry buffer
    L.select = topk_uses_select(rows, L_cap);
    const bool sel = L.select;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    // counters zeroed at the start of every call come first
    L.alloc = take(sel ? 0 : (size_t)rows * 4);
    L.hist = take(sel ? (size_t)rows * TOPK_HIST_BINS * 4 : 0);
    L.zero_bytes = off;
    // scratch overwritten by every call
    L.row_state = take(sel ? 0 : (size_t)rows * 4);
    L.summary = take(sel ? 0 : (size_t)rows * L.nwchunks * L.M * 4);
    L.runs = take(sel ? 0 : (size_t)rows * L.nchunks * 8);
    L.ent = take(sel ? 0 : (size_t)rows * cap * 8);
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
    const TopkLayout L = topk_layout(rows, L_cap, k);
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
    uint32_t* alloc = reinterpret_cast<uint32_t*>(base + L.alloc);
    uint32_t* row_L = reinterpret_cast<uint32_t*>(base + L.row_state);
    uint32_t* summary = reinterpret_cast<uint32_t*>(base + L.summary);
    uint2* runs = reinterpret_cast<uint2*>(base + L.runs);
    uint2* ent = reinterpret_cast<uint2*>(base + L.ent);
    if (!summary_ready) {
        // the summary kernel also zeroes the entry counters
        hipLaunchKernelGGL(topk_summary_kernel, dim3(L.nwchunks / 4, rows), dim3(SUM_THREADS), 0,
                           stream, S, kv_len, Tq, L_cap, L.M, L.nwchunks, summary, alloc);
    } else if (!counters_clear) {
        hipError_t e = launch_clear_u32(reinterpret_cast<uint32_t*>(base), L.zero_bytes / 4, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_filter_kernel, dim3(L.nchunks, rows), dim3(TOPK_THREADS), 0, stream, S,
                       kv_len, Tq, L_cap, k, summary, L.nwchunks * L.M, alloc, row_L, runs, ent,
                       L.cap, L.nchunks);
    hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(FIN_THREADS), 0, stream, S, kv_len,
                       Tq, L_cap, k, alloc, row_L, runs, ent, L.cap, L.nchunks, idx);
    return hipGetLastError();
}

}  // namespace isa
