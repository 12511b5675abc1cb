// Access counts of an index set (gfx950).
//
// Definition ("GLM-5.2 深度技术解析：智谱百万上下文旗舰模型的架构创新与工程实践",
// HiSparse memory-management section: after every attention step each
// position the indexer's top-k selected gains one access, and the access
// frequencies decide which cache entries are hot or cold):
//   counts[b, s] += |{ (t, j) : idx[b, t, j] == s }|   for 0 <= s < L_cap,
// other slot values (-1 padding, out of range) are ignored.
//
// One thread per four slots (one 16-byte load when a row of k slots is a
// multiple of four), one device-scope atomic add per valid slot.  The counts
// are integers, so the result does not depend on the order of the adds.
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int HIST_THREADS = 256;

template <bool VEC>
__global__ __launch_bounds__(HIST_THREADS) void index_histogram_kernel(
    const int32_t* __restrict__ idx, int Tq, int k, int L_cap, uint32_t* __restrict__ counts,
    size_t n_slots) {
    const size_t per_seq = (size_t)Tq * k;
    for (size_t i0 = ((size_t)blockIdx.x * HIST_THREADS + threadIdx.x) * 4; i0 < n_slots;
         i0 += (size_t)gridDim.x * HIST_THREADS * 4) {
        int v[4];
        if constexpr (VEC) {
            const int4 x = *reinterpret_cast<const int4*>(idx + i0);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = i0 + u < n_slots ? idx[i0 + u] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = v[u];
            if (s < 0 || s >= L_cap) continue;
            const size_t b = (i0 + u) / per_seq;      // a sequence's slots are contiguous
            atomicAdd(&counts[b * (size_t)L_cap + s], 1u);
        }
    }
}

}  // namespace

hipError_t launch_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                                  uint32_t* counts, hipStream_t stream) {
    const size_t n_slots = (size_t)B * Tq * k;
    size_t blocks = (n_slots + HIST_THREADS * 4 - 1) / (HIST_THREADS * 4);
    if (blocks > 4096) blocks = 4096;
    if (k % 4 == 0)
        hipLaunchKernelGGL(index_histogram_kernel<true>, dim3((unsigned)blocks), dim3(HIST_THREADS),
                           0, stream, idx, Tq, k, L_cap, counts, n_slots);
    else
        hipLaunchKernelGGL(index_histogram_kernel<false>, dim3((unsigned)blocks),
                           dim3(HIST_THREADS), 0, stream, idx, Tq, k, L_cap, counts, n_slots);
    return hipGetLastError();
}

}  // namespace isa
