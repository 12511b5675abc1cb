// Sparse latent attention over the selected positions (gfx950, bf16 MFMA).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1: attention loads keys and values only at the top-K positions; the
// latent row is kv_lora_rank = 512 wide, "GLM-5.2核心技术解析" config
// fragment, plus the RoPE slice; read in absorbed-MLA form, where the key is
// the whole latent row and the value its first D_v entries):
//   z_j = sm_scale * Q[h] . C[idx_j];  out[h] = sum_j softmax(z)_j * C[idx_j, :D_v].
//
// One workgroup = one query x a range of its k slots (a split), all heads.
// Per tile of T gathered latent rows (each row is read from HBM once and
// shared by every head):
//   * the rows are gathered into LDS (row pitch D*2+16 bytes, so that the
//     32 rows read by one ds_read_b128 land on distinct banks);
//   * wave (rb, hb) computes S^T = C_rows(rb) . Q(hb)^T with
//     v_mfma_f32_32x32x16_bf16: a 32-row x 32-head block, Q^T held in
//     registers for the whole kernel;
//   * online softmax in the exp2 domain; a head's 32 rows sit in one lane
//     pair, so its max and sum need one cross-lane swap plus one LDS exchange
//     between the row-block waves;
//   * the accumulator layout of S^T is exactly the k-permuted B-operand layout
//     of the next product, so P^T goes to the PV MFMA straight from registers
//     (bf16) -- the other row blocks' P^T comes through the LDS bytes that held
//     the RoPE slice, which only the QK product reads;
//   * O^T[cols x heads] += V^T . P^T, where the V^T operand comes from the
//     row-major tile through ds_read_b64_tr_b16 (two transposing reads per
//     operand, in the same k order as P^T).
// With several splits per query, partial (O, max, sum) go to the workspace
// and a merge kernel combines them in split order.
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int AT_THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) v4bf* lds_v4bf_ptr;

__device__ __forceinline__ v4bf lds_read_tr(const char* lds_base, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf_ptr)(lds_base + byte_off));
}

__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 h = (__bf16)x;                    // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

template <int HB, int D, int DV>
struct AttendGeom {
    static constexpr int NRB = 4 / HB;              // 32-row blocks per tile
    static constexpr int T = 32 * NRB;              // tile rows
    static constexpr int KS = D / 16;               // k-steps of the QK product
    static constexpr int CH = D * 2 / 16;           // 16-byte chunks per latent row
    static constexpr int PITCH = D * 2 + 16;        // LDS row pitch (bytes)
    static constexpr int DVW = DV / NRB;            // value columns per wave
    static constexpr int NB = DVW / 32;             // 32-column blocks per wave
    static constexpr int XSLOTS = (D - DV) * 2 / 32;                    // 32-byte exchange slots per row
    static constexpr int LDS_BYTES = T * PITCH;
    static_assert(D % 16 == 0 && DV % (32 * NRB) == 0, "tile shape");
    static_assert(T * (D - DV) * 2 >= 4 * 64 * 32, "P exchange must fit the RoPE bytes");
};

template <int HB, int D, int DV>
__global__ __launch_bounds__(AT_THREADS) void sparse_attend_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ C, const int32_t* __restrict__ idx,
    int Tq, int H, int L_cap, int k, float scale_log2, int slots_per_split, int splits,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
    using G = AttendGeom<HB, D, DV>;
    constexpr int T = G::T;
    constexpr int NRB = G::NRB;
    constexpr int PITCH = G::PITCH;

    __shared__ __attribute__((aligned(16))) char tile[G::LDS_BYTES];
    __shared__ int svalid[T];
    __shared__ float red_max[4][32];
    __shared__ float red_sum[4][32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;
    const int g = lane >> 5;
    const int rb = wave / HB;
    const int hb = wave % HB;
    const int q = blockIdx.y;              // b * Tq + t
    const int sp = blockIdx.x;
    const int b = q / Tq;
    const int head = hb * 32 + j;
    const bool head_ok = head < H;
    const int slot0 = sp * slots_per_split;
    const int slot1 = min(slot0 + slots_per_split, k);
    const int32_t* qidx = idx + (size_t)q * k;
    const uint16_t* Cb = C + (size_t)b * L_cap * D;

    // Q^T operand of this wave's heads: lane (head j, half g) holds dims 16*ks + 8*g .. +8
    v8bf qb[G::KS];
    {
        const uint16_t* qrow = Q + ((size_t)q * H + (head_ok ? head : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const uint4 v = head_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * g)
                                    : make_uint4(0, 0, 0, 0);
            qb[ks] = __builtin_bit_cast(v8bf, v);
        }
    }

    v16f o[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
        for (int r = 0; r < 16; ++r) o[nb][r] = 0.0f;
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    // gather one tile of latent rows into LDS (rows past the split or with an
    // invalid position are zero, so their value rows contribute nothing)
    auto gather = [&](int tile_start) {
        for (int c = tid; c < T * G::CH; c += AT_THREADS) {
            const int r = c / G::CH;
            const int ch = c - r * G::CH;
            const int slot = tile_start + r;
            const int s = slot < slot1 ? qidx[slot] : -1;
            const bool valid = s >= 0 && s < L_cap;
            const uint4 v = valid ? *reinterpret_cast<const uint4*>(Cb + (size_t)s * D + ch * 8)
                                  : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(tile + r * PITCH + ch * 16) = v;
            if (ch == 0) svalid[r] = valid;
        }
    };

    for (int tile_start = slot0; tile_start < slot1; tile_start += T) {
        __syncthreads();                   // previous tile fully consumed
        gather(tile_start);
        __syncthreads();

        // ---- S^T block: rows 32*rb .. +32 of the tile, heads of block hb
        v16f st;
        for (int r = 0; r < 16; ++r) st[r] = 0.0f;
        const char* arow = tile + (32 * rb + j) * PITCH + 16 * g;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const v8bf a = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(arow + 32 * ks));
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], st, 0, 0, 0);
        }
        // register r holds tile row 32*rb + 8*(r/4) + 4*g + r%4, head j
        float mloc = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * rb + 8 * (r / 4) + 4 * g + (r % 4);
            const float x = svalid[row] ? st[r] * scale_log2 : -__builtin_inff();
            st[r] = x;
            mloc = fmaxf(mloc, x);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        if (g == 0) red_max[wave][j] = mloc;
        __syncthreads();                   // also: every wave finished reading the RoPE bytes
        float mt = -__builtin_inff();
#pragma unroll
        for (int r2 = 0; r2 < NRB; ++r2) mt = fmaxf(mt, red_max[r2 * HB + hb][j]);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
        v8bf pk[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2f(st[r] - m_use);
            psum += p;
            pk[r / 8][r % 8] = (__bf16)p;
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;

        // ---- publish P^T through the RoPE bytes of the tile
        {
            const int e = wave * 64 + lane;
            char* xs = tile + (e / G::XSLOTS) * PITCH + DV * 2 + (e % G::XSLOTS) * 32;
            *reinterpret_cast<v8bf*>(xs) = pk[0];
            *reinterpret_cast<v8bf*>(xs + 16) = pk[1];
        }
        __syncthreads();

        // ---- O^T[cols of this wave x heads of hb] += V^T . P^T over all T rows
        const int col0 = rb * G::DVW;
        const int G16 = lane >> 4;
        const int i16 = lane & 15;
#pragma unroll
        for (int r2 = 0; r2 < NRB; ++r2) {
            v8bf pb[2];
            if (r2 == rb) {
                pb[0] = pk[0];
                pb[1] = pk[1];
            } else {
                const int e = (r2 * HB + hb) * 64 + lane;
                const char* xs = tile + (e / G::XSLOTS) * PITCH + DV * 2 + (e % G::XSLOTS) * 32;
                pb[0] = *reinterpret_cast<const v8bf*>(xs);
                pb[1] = *reinterpret_cast<const v8bf*>(xs + 16);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int row = 32 * r2 + 16 * kk + 4 * (G16 >> 1) + (i16 >> 2);
#pragma unroll
                for (int nb = 0; nb < G::NB; ++nb) {
                    const int col = col0 + 32 * nb + 16 * (G16 & 1) + 4 * (i16 & 3);
                    const int off = row * PITCH + col * 2;
                    const v4bf lo = lds_read_tr(tile, off);
                    const v4bf hi = lds_read_tr(tile, off + 8 * PITCH);
                    const v8bf a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], o[nb], 0, 0, 0);
                }
            }
        }
    }

    // ---- finish: total softmax denominator of each head over all row blocks
    float lsum = l_run + __shfl_xor(l_run, 32);
    __syncthreads();
    if (g == 0) red_sum[wave][j] = lsum;
    __syncthreads();
    float l_tot = 0.0f;
#pragma unroll
    for (int r2 = 0; r2 < NRB; ++r2) l_tot += red_sum[r2 * HB + hb][j];

    // o[nb] register r holds value column col0 + 32*nb + 8*(r/4) + 4*g + r%4 of head j
    const int col0 = rb * G::DVW;
    if (splits == 1) {
        if (!head_ok) return;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = out + ((size_t)q * H + head) * DV;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int col = col0 + 32 * nb + 8 * r4 + 4 * g;
                ushort4 v;
                v.x = f2bf(o[nb][4 * r4 + 0] * inv);
                v.y = f2bf(o[nb][4 * r4 + 1] * inv);
                v.z = f2bf(o[nb][4 * r4 + 2] * inv);
                v.w = f2bf(o[nb][4 * r4 + 3] * inv);
                *reinterpret_cast<ushort4*>(orow + col) = v;
            }
        }
        if (lse && rb == 0 && g == 0) {
            lse[(size_t)q * H + head] =
                l_tot > 0.0f ? (m_run + log2f(l_tot)) * LN2 : -__builtin_inff();
        }
    } else {
        if (!head_ok) return;
        const size_t pbase = ((size_t)q * splits + sp) * H + head;
        float* po = part_o + pbase * DV;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int col = col0 + 32 * nb + 8 * r4 + 4 * g;
                *reinterpret_cast<float4*>(po + col) =
                    make_float4(o[nb][4 * r4], o[nb][4 * r4 + 1], o[nb][4 * r4 + 2], o[nb][4 * r4 + 3]);
            }
        }
        if (rb == 0 && g == 0) part_ml[pbase] = make_float2(m_run, l_tot);
    }
}

// Combines the splits of one (query, head): out = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s.
template <int DV>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           int H, int splits,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
    const int qh = blockIdx.x;             // q * H + h
    const int q = qh / H;
    const int h = qh - q * H;
    __shared__ float wts[64];
    __shared__ float sh_norm[2];
    if (threadIdx.x < 64) {
        float M = -__builtin_inff();
        for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[((size_t)q * splits + s) * H + h].x);
        const float Mu = M == -__builtin_inff() ? 0.0f : M;
        if (threadIdx.x == 0) {
            float L = 0.0f;
            for (int s = 0; s < splits; ++s) {
                const float2 ml = part_ml[((size_t)q * splits + s) * H + h];
                L += exp2f(ml.x - Mu) * ml.y;
            }
            sh_norm[0] = L > 0.0f ? 1.0f / L : 0.0f;
            sh_norm[1] = L > 0.0f ? (M + log2f(L)) * LN2 : -__builtin_inff();
        }
        for (int s = threadIdx.x; s < splits; s += 64)
            wts[s] = exp2f(part_ml[((size_t)q * splits + s) * H + h].x - Mu);
    }
    __syncthreads();
    const float inv = sh_norm[0];
    for (int col = threadIdx.x; col < DV; col += 256) {
        float acc = 0.0f;
        for (int s = 0; s < splits; ++s)
            acc += wts[s] * part_o[(((size_t)q * splits + s) * H + h) * DV + col];
        out[(size_t)qh * DV + col] = f2bf(acc * inv);
    }
    if (lse && threadIdx.x == 0) lse[qh] = sh_norm[1];
}

template <int HB, int D, int DV>
hipError_t launch_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx, int B, int Tq,
                         int H, int L_cap, int k, float sm_scale, uint16_t* out, float* lse,
                         void* ws, hipStream_t stream) {
    const AttendPlan plan = attend_plan(B, Tq, H, DV, k);
    const int nq = B * Tq;
    float* part_o = static_cast<float*>(ws);
    float2* part_ml = nullptr;
    if (plan.splits > 1)
        part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                            (size_t)nq * plan.splits * H * DV * sizeof(float));
    dim3 grid(plan.splits, nq);
    hipLaunchKernelGGL((sparse_attend_kernel<HB, D, DV>), grid, dim3(AT_THREADS), 0, stream, Q, C,
                       idx, Tq, H, L_cap, k, sm_scale * LOG2E, plan.slots_per_split, plan.splits,
                       out, lse, part_o, part_ml);
    if (plan.splits > 1) {
        hipLaunchKernelGGL((merge_splits_kernel<DV>), dim3(nq * H), dim3(256), 0, stream, part_o,
                           part_ml, H, plan.splits, out, lse);
    }
    return hipGetLastError();
}

}  // namespace

AttendPlan attend_plan(int B, int Tq, int H, int D_v, int k) {
    AttendPlan p;
    p.head_blocks = D_v == 512 ? 2 : 1;
    const int T = 32 * (4 / p.head_blocks);
    const int nq = B * Tq;
    const int tiles = (k + T - 1) / T;
    int splits = (512 + nq - 1) / nq;          // aim for >= 512 workgroups
    if (splits > tiles) splits = tiles;
    if (splits > 64) splits = 64;
    if (splits < 1) splits = 1;
    const int tiles_per_split = (tiles + splits - 1) / splits;
    splits = (tiles + tiles_per_split - 1) / tiles_per_split;
    p.splits = splits;
    p.slots_per_split = tiles_per_split * T;
    p.partial_bytes = splits > 1 ? (size_t)nq * splits * H * ((size_t)D_v + 2) * sizeof(float) : 0;
    return p;
}

bool attend_shape_supported(int H, int D, int D_v) {
    if (D == 576 && D_v == 512) return H >= 1 && H <= 64;
    if (D == 160 && D_v == 128) return H >= 1 && H <= 32;
    return false;
}

hipError_t launch_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                                    int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                                    float sm_scale, uint16_t* out, float* lse, void* ws,
                                    hipStream_t stream) {
    // 576-wide rows: two 32-head blocks per workgroup (heads past H are zero);
    // 160-wide rows: one 32-head block and 128-row tiles.
    if (D == 576 && D_v == 512)
        return launch_attend<2, 576, 512>(Q, C, idx, B, Tq, H, L_cap, k, sm_scale, out, lse, ws, stream);
    if (D == 160 && D_v == 128)
        return launch_attend<1, 160, 128>(Q, C, idx, B, Tq, H, L_cap, k, sm_scale, out, lse, ws, stream);
    return hipErrorInvalidValue;
}

}  // namespace isa
