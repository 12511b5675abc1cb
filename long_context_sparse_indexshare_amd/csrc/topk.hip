// Top-k position select over fp32 scores (gfx950).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1: keep the top-K positions; K = index_topk = 2048 in the config fragment
// of "GLM-5.2核心技术解析"): for each query, the min(k, pos+1) visible positions
// that come first under (score descending, position ascending), listed in
// ascending position and padded with -1.
//
// Radix select on the order-preserving 32-bit image of each score, spread
// over many workgroups per query so one long row (up to 2^21 positions) uses
// the whole chip:
//   0. clear:   zero the row counters in the workspace.
//   1. hist:    every workgroup histograms the top 12 key bits of a 4096-score
//               chunk in LDS and adds its non-zero bins to the row's global
//               histogram.
//   2. classify: every workgroup finds the bin that holds the k-th key, counts
//               its keys above that bin, and appends the keys that fall in the
//               bin to a per-row candidate list (one atomic per workgroup).
//   3. finish:  the exact threshold key T and the position cut-off among keys
//               equal to T (two radix passes over the low 20 key bits, two over
//               the position bits, on the candidates staged in LDS), and the
//               output offset of every chunk.  With few rows every compact
//               workgroup does this itself; with many, one workgroup per row.
//               If the candidate list overflowed the row is re-read instead.
//   4. compact: every workgroup re-reads its chunk and writes the selected
//               positions, in order, at its offset.
// Workgroups never wait on each other inside a kernel: on gfx950 a device-
// scope fence writes back and invalidates the whole L2 of the XCD, so each
// hand-over between workgroups goes through a kernel boundary instead.
#include "isa_internal.h"

namespace isa {

namespace {

constexpr int CAND_MIN = 16384;

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                       // -0.0 ranks as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // monotone in the float order
}

__device__ __forceinline__ int visible_count(const int32_t* kv_len, int row, int Tq, int L_cap) {
    const int b = row / Tq;
    const int t = row - b * Tq;
    int len = kv_len[b];
    len = len < 0 ? 0 : (len > L_cap ? L_cap : len);
    const int n = len - Tq + t + 1;
    return n > 0 ? n : 0;
}

// Exclusive prefix sum over the 256 threads of the workgroup; *total gets the sum.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total, uint32_t* sh_waves) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    __syncthreads();
    if (lane == 63) sh_waves[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < TOPK_THREADS / 64; ++w) {
        const uint32_t x = sh_waves[w];
        before += w < wave ? x : 0u;
        all += x;
    }
    *total = all;
    return before + inc - v;
}

// Over bins h[0..nbins) (nbins = 256 * per): the largest bin B with
// sum_{b >= B} h[b] >= need (descending) or the smallest bin B with
// sum_{b <= B} h[b] >= need (ascending).  Returns B and the count strictly
// beyond it (above for descending, below for ascending) to every thread.
template <int PER, bool DESC>
__device__ void find_bin(const uint32_t* h, uint32_t need, uint32_t* bin_out, uint32_t* beyond_out,
                         uint32_t* sh_waves, uint32_t* sh_res) {
    const int tid = threadIdx.x;
    // thread t owns bins [PER*t, PER*t + PER) ascending, or the mirrored range descending
    const int first = DESC ? (TOPK_THREADS - 1 - tid) * PER : tid * PER;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += h[first + i];
    uint32_t total;
    const uint32_t before = block_exclusive_scan(local, &total, sh_waves);
    if (before < need && before + local >= need) {
        uint32_t acc = before;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bin = DESC ? first + PER - 1 - i : first + i;
            const uint32_t c = h[bin];
            if (acc + c >= need) {
                sh_res[0] = (uint32_t)bin;
                sh_res[1] = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    *bin_out = sh_res[0];
    *beyond_out = sh_res[1];
    __syncthreads();
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

__global__ __launch_bounds__(TOPK_THREADS) void topk_hist_kernel(const float* __restrict__ S,
                                                                 const int32_t* __restrict__ kv_len,
                                                                 int Tq, int L_cap, int k,
                                                                 uint32_t* __restrict__ hist) {
    const int row = blockIdx.y;
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    const int start = blockIdx.x * TOPK_CHUNK;
    if (start >= n) return;
    __shared__ uint32_t lh[TOPK_HIST_BINS];
    for (int i = threadIdx.x; i < TOPK_HIST_BINS; i += TOPK_THREADS) lh[i] = 0;
    __syncthreads();
    const float* rowp = S + (size_t)row * L_cap;
#pragma unroll 4
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + threadIdx.x;
        if (s < n) atomicAdd(&lh[score_key(rowp[s]) >> (32 - TOPK_HIST_BITS)], 1u);
    }
    __syncthreads();
    uint32_t* gh = hist + (size_t)row * TOPK_HIST_BINS;
    for (int i = threadIdx.x; i < TOPK_HIST_BINS; i += TOPK_THREADS) {
        const uint32_t c = lh[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

struct RowState {
    uint32_t bin;     // first-digit bin of the k-th key
    uint32_t T;       // exact k-th key
    int32_t s_cut;    // last selected position among keys equal to T
    uint32_t pad;
};

// Candidates the finishing workgroup stages in LDS (more fall back to global).
constexpr int CAND_LDS = 6144;

// Calls f(key, pos) for every key in the threshold bin: from the copy of the
// candidate list staged in LDS, from the list in global memory, or by
// re-reading the row when the list overflowed.
template <class F>
__device__ __forceinline__ void for_each_candidate(int mode, const uint2* lcand, const uint2* cand,
                                                   uint32_t nc, const float* rowp, int n,
                                                   uint32_t bin, F f) {
    if (mode == 0) {
        for (uint32_t i = threadIdx.x; i < nc; i += TOPK_THREADS) {
            const uint2 c = lcand[i];
            f(c.x, (int)c.y);
        }
    } else if (mode == 1) {
        for (uint32_t i = threadIdx.x; i < nc; i += TOPK_THREADS) {
            const uint2 c = cand[i];
            f(c.x, (int)c.y);
        }
    } else {
        for (int s = threadIdx.x; s < n; s += TOPK_THREADS) {
            const uint32_t key = score_key(rowp[s]);
            if ((key >> (32 - TOPK_HIST_BITS)) == bin) f(key, s);
        }
    }
}

// The bin of the first digit that holds the k-th key, and the number of
// keys in the bins above it, from the row's global histogram.
__device__ void threshold_bin(const uint32_t* gh, int k, uint32_t* sh, uint32_t* sh_waves,
                              uint32_t* sh_res, uint32_t* bin1, uint32_t* above1) {
    const int tid = threadIdx.x;
    // the histogram has 4096 bins; scan it in two halves of 2048 through LDS
    // (each half: 8 independent loads in flight per thread)
    auto stage_half = [&](const uint32_t* src) {
        uint32_t v[2048 / TOPK_THREADS];
#pragma unroll
        for (int u = 0; u < 2048 / TOPK_THREADS; ++u) v[u] = src[u * TOPK_THREADS + tid];
#pragma unroll
        for (int u = 0; u < 2048 / TOPK_THREADS; ++u) sh[u * TOPK_THREADS + tid] = v[u];
    };
    stage_half(gh + 2048);
    __syncthreads();
    uint32_t hi_local = 0;
    for (int i = tid; i < 2048; i += TOPK_THREADS) hi_local += sh[i];
    uint32_t hi_total;
    block_exclusive_scan(hi_local, &hi_total, sh_waves);
    if (hi_total >= (uint32_t)k) {
        find_bin<8, true>(sh, (uint32_t)k, bin1, above1, sh_waves, sh_res);
        *bin1 += 2048;
    } else {
        __syncthreads();
        stage_half(gh);
        __syncthreads();
        find_bin<8, true>(sh, (uint32_t)k - hi_total, bin1, above1, sh_waves, sh_res);
        *above1 += hi_total;
    }
}

// Classify: every workgroup counts its chunk's keys above the threshold bin
// and appends the keys inside it to the row's candidate list (one atomic per
// workgroup reserves its slots).
__global__ __launch_bounds__(TOPK_THREADS) void topk_classify_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ cand_cnt,
    uint32_t* __restrict__ count_above, uint2* __restrict__ cand, uint32_t cap, int nchunks_max) {
    const int row = blockIdx.y;
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const int c = blockIdx.x;
    if (c >= nch) return;
    const int tid = threadIdx.x;
    __shared__ uint32_t sh[2048];
    __shared__ uint32_t sh_waves[TOPK_THREADS / 64];
    __shared__ uint32_t sh_res[4];
    __shared__ uint32_t sh_base;

    uint32_t bin1, above1;
    threshold_bin(hist + (size_t)row * TOPK_HIST_BINS, k, sh, sh_waves, sh_res, &bin1, &above1);

    const float* rowp = S + (size_t)row * L_cap;
    const int start = c * TOPK_CHUNK;
    uint32_t keys[TOPK_PER_THREAD];
    uint32_t n_above = 0, n_cand = 0;
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        const bool valid = s < n;
        const uint32_t key = valid ? score_key(rowp[s]) : 0u;
        keys[e] = key;
        const uint32_t d = key >> (32 - TOPK_HIST_BITS);
        n_above += (valid && d > bin1) ? 1u : 0u;
        n_cand += (valid && d == bin1) ? 1u : 0u;
    }
    uint32_t above_total;
    block_exclusive_scan(n_above, &above_total, sh_waves);
    uint32_t cand_total;
    const uint32_t cand_before = block_exclusive_scan(n_cand, &cand_total, sh_waves);
    if (tid == 0) {
        count_above[(size_t)row * nchunks_max + c] = above_total;
        sh_base = cand_total ? atomicAdd(&cand_cnt[row], cand_total) : 0u;
    }
    __syncthreads();
    uint32_t slot = sh_base + cand_before;
    uint2* rc = cand + (size_t)row * cap;
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        if (s < n && (keys[e] >> (32 - TOPK_HIST_BITS)) == bin1) {
            if (slot < cap) rc[slot] = make_uint2(keys[e], (uint32_t)s);
            ++slot;
        }
    }
}

// LDS of the finishing step.
struct FinishShared {
    uint32_t sh[2048 + 512];          // digit histograms, then per-chunk counts / offsets
    uint2 lcand[CAND_LDS];            // the row's candidates
    uint32_t waves[TOPK_THREADS / 64];
    uint32_t res[4];
};

// Finish a row: the exact k-th key T, the last selected position s_cut
// among keys equal to T, and the output offset of every chunk, left in
// f.sh[0..nch).  Needs the histogram, the candidate list and count_above of
// the classify step.
__device__ void finish_row(int row, int n, int k, int L_cap, const float* S,
                           const uint32_t* hist, const uint32_t* cand_cnt, const uint2* cand,
                           uint32_t cap, const uint32_t* count_above, int nchunks_max,
                           FinishShared& f, RowState* st_out) {
    const int tid = threadIdx.x;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const float* rowp = S + (size_t)row * L_cap;
    uint32_t bin1, above1;
    threshold_bin(hist + (size_t)row * TOPK_HIST_BINS, k, f.sh, f.waves, f.res, &bin1, &above1);
    const uint32_t nc = cand_cnt[row];
    const uint2* rc = cand + (size_t)row * cap;
    const int mode = nc <= (uint32_t)CAND_LDS ? 0 : (nc <= cap ? 1 : 2);
    if (mode == 0) {
        // stage the candidates: 8 independent loads in flight per thread
        for (uint32_t base = 0; base < nc; base += 8 * TOPK_THREADS) {
            uint2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t i = base + u * TOPK_THREADS + tid;
                v[u] = i < nc ? rc[i] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t i = base + u * TOPK_THREADS + tid;
                if (i < nc) f.lcand[i] = v[u];
            }
        }
        __syncthreads();
    }
    uint32_t* sh = f.sh;
    uint32_t need = (uint32_t)k - above1;       // >= 1 keys still to take from the bin

    // key bits [19:10]
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(mode, f.lcand, rc, nc, rowp, n, bin1,
                       [&](uint32_t key, int) { atomicAdd(&sh[(key >> 10) & 1023u], 1u); });
    __syncthreads();
    uint32_t d2, above2;
    find_bin<4, true>(sh, need, &d2, &above2, f.waves, f.res);
    need -= above2;
    const uint32_t pre22 = (bin1 << 10) | d2;
    // key bits [9:0]
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(mode, f.lcand, rc, nc, rowp, n, bin1, [&](uint32_t key, int) {
        if ((key >> 10) == pre22) atomicAdd(&sh[key & 1023u], 1u);
    });
    __syncthreads();
    uint32_t d3, above3;
    find_bin<4, true>(sh, need, &d3, &above3, f.waves, f.res);
    need -= above3;                              // keys equal to T still to take (>= 1)
    const uint32_t T = (pre22 << 10) | d3;
    // among keys equal to T, the need-th lowest position: position bits [20:10], then [9:0]
    for (int i = tid; i < 2048; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(mode, f.lcand, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key == T) atomicAdd(&sh[(uint32_t)s >> 10], 1u);
    });
    __syncthreads();
    uint32_t p2, below2;
    find_bin<8, false>(sh, need, &p2, &below2, f.waves, f.res);
    need -= below2;
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(mode, f.lcand, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key == T && ((uint32_t)s >> 10) == p2) atomicAdd(&sh[(uint32_t)s & 1023u], 1u);
    });
    __syncthreads();
    uint32_t p3, below3;
    find_bin<4, false>(sh, need, &p3, &below3, f.waves, f.res);
    const int s_cut = (int)((p2 << 10) | p3);

    // selected keys of the bin per chunk, plus the keys above it: exclusive
    // prefix over the chunks = each chunk's output offset (nch <= 512)
    for (int i = tid; i < nch; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(mode, f.lcand, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key > T || (key == T && s <= s_cut)) atomicAdd(&sh[s / TOPK_CHUNK], 1u);
    });
    __syncthreads();
    {
        const uint32_t* ca = count_above + (size_t)row * nchunks_max;
        const int c0 = 2 * tid, c1 = 2 * tid + 1;
        const uint32_t v0 = c0 < nch ? sh[c0] + ca[c0] : 0u;
        const uint32_t v1 = c1 < nch ? sh[c1] + ca[c1] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v0 + v1, &tot, f.waves);   // barriers inside
        if (c0 < nch) sh[c0] = ex;
        if (c1 < nch) sh[c1] = ex + v0;
    }
    __syncthreads();
    st_out->bin = bin1;
    st_out->T = T;
    st_out->s_cut = s_cut;
    st_out->pad = 0;
}

// Finish kernel (many rows): one workgroup per row writes the row's state and
// chunk offsets for the compact step.
__global__ __launch_bounds__(TOPK_THREADS) void topk_finish_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ cand_cnt,
    const uint32_t* __restrict__ count_above, const uint2* __restrict__ cand, uint32_t cap,
    int nchunks_max, RowState* __restrict__ row_state, uint32_t* __restrict__ chunk_off) {
    const int row = blockIdx.x;
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    __shared__ FinishShared f;
    RowState st;
    finish_row(row, n, k, L_cap, S, hist, cand_cnt, cand, cap, count_above, nchunks_max, f, &st);
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    for (int i = threadIdx.x; i < nch; i += TOPK_THREADS)
        chunk_off[(size_t)row * nchunks_max + i] = f.sh[i];
    if (threadIdx.x == 0) row_state[row] = st;
}

// Compact: every workgroup re-reads its chunk and writes the selected
// positions, in order, at the chunk's offset.  With SELF_FINISH (few rows)
// each workgroup first finishes the row itself instead of reading the finish
// kernel's results, which saves a launch.
template <bool SELF_FINISH>
__global__ __launch_bounds__(TOPK_THREADS) void topk_compact_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ cand_cnt,
    const uint32_t* __restrict__ count_above, const uint2* __restrict__ cand, uint32_t cap,
    const RowState* __restrict__ row_state, const uint32_t* __restrict__ chunk_off,
    int nchunks_max, int32_t* __restrict__ idx) {
    const int row = blockIdx.y;
    const int n = visible_count(kv_len, row, Tq, L_cap);
    int32_t* out = idx + (size_t)row * k;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    if (n <= k) {
        // every visible position, then -1 padding (k <= 2048 < one chunk)
        if (c == 0)
            for (int j = tid; j < k; j += TOPK_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    if (c >= nch) return;
    __shared__ uint32_t sh_waves[TOPK_THREADS / 64];
    RowState st;
    uint32_t off;
    if constexpr (SELF_FINISH) {
        __shared__ FinishShared f;
        finish_row(row, n, k, L_cap, S, hist, cand_cnt, cand, cap, count_above, nchunks_max, f, &st);
        off = f.sh[c];
    } else {
        st = row_state[row];
        off = chunk_off[(size_t)row * nchunks_max + c];
    }
    const float* rowp = S + (size_t)row * L_cap;
    const int first = c * TOPK_CHUNK + tid * TOPK_PER_THREAD;   // thread-contiguous run
    uint32_t selmask = 0, cnt = 0;
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = first + e;
        if (s < n) {
            const uint32_t key = score_key(rowp[s]);
            const uint32_t d = key >> (32 - TOPK_HIST_BITS);
            const bool sel = d > st.bin ||
                             (d == st.bin && (key > st.T || (key == st.T && s <= st.s_cut)));
            if (sel) {
                selmask |= 1u << e;
                ++cnt;
            }
        }
    }
    uint32_t total;
    uint32_t pos = block_exclusive_scan(cnt, &total, sh_waves) + off;
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        if (selmask & (1u << e)) {
            if (pos < (uint32_t)k) out[pos] = first + e;   // the offsets sum to exactly k
            ++pos;
        }
    }
}

}  // namespace

TopkLayout topk_layout(int rows, int L_cap) {
    TopkLayout L;
    L.rows = rows;
    L.nchunks = (L_cap + TOPK_CHUNK - 1) / TOPK_CHUNK;
    uint32_t cap = (uint32_t)(L_cap / 8);
    const uint32_t lo = (uint32_t)(L_cap < CAND_MIN ? L_cap : CAND_MIN);
    if (cap < lo) cap = lo;
    cap = (cap + 63u) & ~63u;
    L.cap = cap;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    // counters zeroed at the start of every call come first
    L.hist = take((size_t)rows * TOPK_HIST_BINS * 4);
    L.cand_cnt = take((size_t)rows * 4);
    // scratch overwritten by every call
    L.row_state = take((size_t)rows * sizeof(RowState));
    L.count_above = take((size_t)rows * L.nchunks * 4);
    L.chunk_off = take((size_t)rows * L.nchunks * 4);
    L.cand = take((size_t)rows * cap * 8);
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
                              int k, int32_t* idx, void* ws, bool counters_clear, bool hist_ready,
                              hipStream_t stream) {
    const int rows = B * Tq;
    const TopkLayout L = topk_layout(rows, L_cap);
    char* base = static_cast<char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
    uint32_t* cand_cnt = reinterpret_cast<uint32_t*>(base + L.cand_cnt);
    RowState* row_state = reinterpret_cast<RowState*>(base + L.row_state);
    uint32_t* count_above = reinterpret_cast<uint32_t*>(base + L.count_above);
    uint32_t* chunk_off = reinterpret_cast<uint32_t*>(base + L.chunk_off);
    uint2* cand = reinterpret_cast<uint2*>(base + L.cand);
    if (!counters_clear) {                      // hist and cand_cnt precede row_state
        hipError_t e = launch_clear_u32(reinterpret_cast<uint32_t*>(base), L.row_state / 4, stream);
        if (e != hipSuccess) return e;
    }
    dim3 grid(L.nchunks, rows);
    if (!hist_ready)
        hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len, Tq,
                           L_cap, k, hist);
    hipLaunchKernelGGL(topk_classify_kernel, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len, Tq,
                       L_cap, k, hist, cand_cnt, count_above, cand, L.cap, L.nchunks);
    // few rows: every compact workgroup finishes its row itself (one launch
    // fewer); many rows: one finish workgroup per row
    if ((size_t)rows * L.nchunks <= 2048) {
        hipLaunchKernelGGL(topk_compact_kernel<true>, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len,
                           Tq, L_cap, k, hist, cand_cnt, count_above, cand, L.cap, row_state,
                           chunk_off, L.nchunks, idx);
    } else {
        hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(TOPK_THREADS), 0, stream, S,
                           kv_len, Tq, L_cap, k, hist, cand_cnt, count_above, cand, L.cap,
                           L.nchunks, row_state, chunk_off);
        hipLaunchKernelGGL(topk_compact_kernel<false>, grid, dim3(TOPK_THREADS), 0, stream, S,
                           kv_len, Tq, L_cap, k, hist, cand_cnt, count_above, cand, L.cap,
                           row_state, chunk_off, L.nchunks, idx);
    }
    return hipGetLastError();
}

}  // namespace isa
