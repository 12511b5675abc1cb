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
//   2. refine:  every workgroup finds the bin that holds the k-th key, counts
//               its keys above that bin, and appends the keys that fall in the
//               bin to a per-row candidate list (one atomic per workgroup).  The
//               last workgroup of the row (ticket counter) resolves the exact
//               threshold key T and the position cut-off among keys equal to T
//               (two radix passes over the low 20 key bits, two over the
//               position bits), then turns per-chunk selected counts into
//               output offsets.  If the candidate list overflowed it re-reads
//               the row instead.
//   3. compact: every workgroup re-reads its chunk and writes the selected
//               positions, in order, at its offset.
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

// Zeroes the per-row counters (histograms, candidate counts, tickets) at the
// start of every call, so the workspace needs no initialisation.  A fill
// kernel rather than a memset keeps the call capturable in a HIP graph.
__global__ __launch_bounds__(256) void topk_clear_kernel(uint4* __restrict__ p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
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

// Calls f(key, pos) for every key in the threshold bin: from the candidate
// list, or by re-reading the row when the list overflowed.
template <class F>
__device__ __forceinline__ void for_each_candidate(bool overflow, const uint2* cand, uint32_t nc,
                                                   const float* rowp, int n, uint32_t bin, F f) {
    if (!overflow) {
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

__global__ __launch_bounds__(TOPK_THREADS) void topk_refine_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
    uint32_t* __restrict__ hist, uint32_t* __restrict__ cand_cnt, uint32_t* __restrict__ ticket,
    RowState* __restrict__ row_state, uint32_t* __restrict__ count_above,
    uint32_t* __restrict__ chunk_off, uint2* __restrict__ cand, uint32_t cap, int nchunks_max) {
    const int row = blockIdx.y;
    const int n = visible_count(kv_len, row, Tq, L_cap);
    if (n <= k) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const int c = blockIdx.x;
    if (c >= nch) return;
    const int tid = threadIdx.x;

    __shared__ uint32_t sh[2048 + 512];          // histograms, then chunk counts
    __shared__ uint32_t sh_waves[TOPK_THREADS / 64];
    __shared__ uint32_t sh_res[4];
    __shared__ uint32_t sh_base;
    __shared__ int sh_last;

    uint32_t* gh = hist + (size_t)row * TOPK_HIST_BINS;
    // the row histogram has 4096 bins; reduce it in two halves of 2048 through LDS
    uint32_t bin1, above1;
    {
        // upper half first: bins 2048..4095
        for (int i = tid; i < 2048; i += TOPK_THREADS) sh[i] = gh[2048 + i];
        __syncthreads();
        uint32_t hi_total_local = 0;
        for (int i = tid; i < 2048; i += TOPK_THREADS) hi_total_local += sh[i];
        uint32_t hi_total;
        block_exclusive_scan(hi_total_local, &hi_total, sh_waves);
        if (hi_total >= (uint32_t)k) {
            find_bin<8, true>(sh, (uint32_t)k, &bin1, &above1, sh_waves, sh_res);
            bin1 += 2048;
        } else {
            __syncthreads();
            for (int i = tid; i < 2048; i += TOPK_THREADS) sh[i] = gh[i];
            __syncthreads();
            find_bin<8, true>(sh, (uint32_t)k - hi_total, &bin1, &above1, sh_waves, sh_res);
            above1 += hi_total;
        }
    }

    // classify this chunk's keys
    const float* rowp = S + (size_t)row * L_cap;
    const int start = c * TOPK_CHUNK;
    uint32_t keys[TOPK_PER_THREAD];
    uint32_t n_above = 0, n_cand = 0;
#pragma unroll
    for (int e = 0; e < TOPK_PER_THREAD; ++e) {
        const int s = start + e * TOPK_THREADS + tid;
        const uint32_t key = s < n ? score_key(rowp[s]) : 0u;
        keys[e] = key;
        const uint32_t d = key >> (32 - TOPK_HIST_BITS);
        const bool valid = s < n;
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
    {
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
    // publish, then let the last workgroup of the row finish it
    __threadfence();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&ticket[row], 1u) == (uint32_t)(nch - 1);
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    const uint32_t nc = __hip_atomic_load(&cand_cnt[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool overflow = nc > cap;
    const uint2* rc = cand + (size_t)row * cap;
    uint32_t need = (uint32_t)k - above1;       // >= 1 keys still to take from the bin

    // key bits [19:10]
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(overflow, rc, nc, rowp, n, bin1,
                       [&](uint32_t key, int) { atomicAdd(&sh[(key >> 10) & 1023u], 1u); });
    __syncthreads();
    uint32_t d2, above2;
    find_bin<4, true>(sh, need, &d2, &above2, sh_waves, sh_res);
    need -= above2;
    const uint32_t pre22 = (bin1 << 10) | d2;
    // key bits [9:0]
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(overflow, rc, nc, rowp, n, bin1, [&](uint32_t key, int) {
        if ((key >> 10) == pre22) atomicAdd(&sh[key & 1023u], 1u);
    });
    __syncthreads();
    uint32_t d3, above3;
    find_bin<4, true>(sh, need, &d3, &above3, sh_waves, sh_res);
    need -= above3;                              // keys equal to T still to take (>= 1)
    const uint32_t T = (pre22 << 10) | d3;
    // among keys equal to T, the need-th lowest position: position bits [20:10], then [9:0]
    for (int i = tid; i < 2048; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(overflow, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key == T) atomicAdd(&sh[(uint32_t)s >> 10], 1u);
    });
    __syncthreads();
    uint32_t p2, below2;
    find_bin<8, false>(sh, need, &p2, &below2, sh_waves, sh_res);
    need -= below2;
    for (int i = tid; i < 1024; i += TOPK_THREADS) sh[i] = 0;
    __syncthreads();
    for_each_candidate(overflow, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key == T && ((uint32_t)s >> 10) == p2) atomicAdd(&sh[(uint32_t)s & 1023u], 1u);
    });
    __syncthreads();
    uint32_t p3, below3;
    find_bin<4, false>(sh, need, &p3, &below3, sh_waves, sh_res);
    const int s_cut = (int)((p2 << 10) | p3);

    // selected keys of the bin per chunk, then output offsets of every chunk
    uint32_t* cc = sh;                          // nch <= 512 counters
    for (int i = tid; i < nch; i += TOPK_THREADS) cc[i] = 0;
    __syncthreads();
    for_each_candidate(overflow, rc, nc, rowp, n, bin1, [&](uint32_t key, int s) {
        if (key > T || (key == T && s <= s_cut)) atomicAdd(&cc[s / TOPK_CHUNK], 1u);
    });
    __syncthreads();
    {
        const uint32_t* ca = count_above + (size_t)row * nchunks_max;
        // each thread owns two consecutive chunks (nch <= 512)
        const int c0 = 2 * tid, c1 = 2 * tid + 1;
        const uint32_t v0 = c0 < nch ? cc[c0] + ca[c0] : 0u;
        const uint32_t v1 = c1 < nch ? cc[c1] + ca[c1] : 0u;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan(v0 + v1, &tot, sh_waves);
        uint32_t* co = chunk_off + (size_t)row * nchunks_max;
        if (c0 < nch) co[c0] = ex;
        if (c1 < nch) co[c1] = ex + v0;
    }
    if (tid == 0) {
        RowState st;
        st.bin = bin1;
        st.T = T;
        st.s_cut = s_cut;
        st.pad = 0;
        row_state[row] = st;
    }
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_compact_kernel(
    const float* __restrict__ S, const int32_t* __restrict__ kv_len, int Tq, int L_cap, int k,
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
    const RowState st = row_state[row];
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
    uint32_t pos = block_exclusive_scan(cnt, &total, sh_waves) + chunk_off[(size_t)row * nchunks_max + c];
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
    L.ticket = take((size_t)rows * 4);
    // scratch overwritten by every call
    L.row_state = take((size_t)rows * sizeof(RowState));
    L.count_above = take((size_t)rows * L.nchunks * 4);
    L.chunk_off = take((size_t)rows * L.nchunks * 4);
    L.cand = take((size_t)rows * cap * 8);
    L.total = off;
    return L;
}

hipError_t launch_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap,
                              int k, int32_t* idx, void* ws, hipStream_t stream) {
    const int rows = B * Tq;
    const TopkLayout L = topk_layout(rows, L_cap);
    char* base = static_cast<char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
    uint32_t* cand_cnt = reinterpret_cast<uint32_t*>(base + L.cand_cnt);
    uint32_t* ticket = reinterpret_cast<uint32_t*>(base + L.ticket);
    RowState* row_state = reinterpret_cast<RowState*>(base + L.row_state);
    uint32_t* count_above = reinterpret_cast<uint32_t*>(base + L.count_above);
    uint32_t* chunk_off = reinterpret_cast<uint32_t*>(base + L.chunk_off);
    uint2* cand = reinterpret_cast<uint2*>(base + L.cand);
    const size_t n16 = L.row_state / 16;         // hist, cand_cnt and ticket precede row_state
    const int clear_blocks = (int)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(topk_clear_kernel, dim3(clear_blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(base), n16);
    dim3 grid(L.nchunks, rows);
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len, Tq, L_cap,
                       k, hist);
    hipLaunchKernelGGL(topk_refine_kernel, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len, Tq,
                       L_cap, k, hist, cand_cnt, ticket, row_state, count_above, chunk_off, cand,
                       L.cap, L.nchunks);
    hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(TOPK_THREADS), 0, stream, S, kv_len, Tq,
                       L_cap, k, row_state, chunk_off, L.nchunks, idx);
    return hipGetLastError();
}

}  // namespace isa
