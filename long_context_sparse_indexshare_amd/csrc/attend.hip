// Sparse latent attention over the selected positions (gfx950, bf16 MFMA).
//
// Definition ("GLM-5.2 Explained: 1M Token Context AI Agent Model", section
// 2.1: attention loads keys and values only at the top-K positions; the
// latent row is kv_lora_rank = 512 wide, "GLM-5.2核心技术解析" config
// fragment, plus the RoPE slice; read in absorbed-MLA form, where the key is
// the whole latent row and the value its first D_v entries):
//   z_j = sm_scale * Q[h] . C[idx_j];  out[h] = sum_j softmax(z)_j * C[idx_j, :D_v].
//
// A group of 4 waves owns one query, HB blocks of 32 heads, 1/VS of the
// value columns, and a range (split) of the query's k slots; a workgroup
// holds GR such groups on alternate tiles of the same range.  Per tile of 32
// gathered latent rows (each row is read from HBM once and shared by all the
// workgroup's heads):
//   * gather: eight threads per tile row load its 16-byte chunks straight
//     into registers (thread (row, sub) owns chunks sub, sub + 8, ...) and
//     store them to LDS once they land; each group has its next tile in
//     flight in registers while it computes the current one from LDS (the
//     direct-to-LDS load path measured ~3x slower for this pattern); slots
//     that are -1 or out of range load a zero row;
//   * LDS rows carry one 16-byte pad and each 16-row half of a tile is
//     stored as a 4 x 4 transpose of its rows (tile_slot), so both the QK
//     operand reads and the transposing PV reads hit distinct banks;
//   * S^T = C_rows . Q^T on v_mfma_f32_32x32x16_bf16, a 32-row x 32-head
//     block per head block, with the contraction over the latent dims split
//     between the 4/HB waves of the head block (each holds only its share of
//     Q^T in registers); the partial blocks are summed through LDS in a fixed
//     order, so every wave of the block holds identical bits;
//   * online softmax in the exp2 domain; a head's 32 rows sit in one lane
//     pair (16 registers each), so max and sum need one cross-lane swap;
//   * the accumulator layout of S^T is exactly the k-permuted B-operand
//     layout of the next product, so P^T feeds the PV MFMA from registers;
//     O^T[cols x heads] += V^T . P^T, with V^T read from the row-major tile by
//     ds_read_b64_tr_b16 (two transposing reads per operand, same k order).
// With several splits per query the partial (O, max, sum) go to the
// workspace and a merge kernel combines them in split order (workgroups never
// hand data to each other inside a kernel: on gfx950 a device-scope fence
// writes back and invalidates the whole L2 of the XCD).
#include "isa_internal.h"

namespace isa {
namespace {

constexpr int AT_THREADS = 256;
constexpr int TILE_ROWS = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// The running softmax reference max moves only when a tile's max exceeds it
// by more than this (log2 units): P stays <= 2^8, and most tiles skip the
// rescale of the output accumulators.
constexpr float RESCALE_SLACK = 8.0f;

typedef __attribute__((address_space(3))) v4bf* lds_v4bf_ptr;
// Gathers go through global-address-space pointers: a generic (flat) load
// also counts against the LDS wait counter, so every LDS wait would stall on
// the gathers still in flight.
typedef const __attribute__((address_space(1))) v4u* global_v4u_ptr;

// Largest slot range one workgroup takes (the whole set when not split).
constexpr int MAX_SPLIT_SLOTS = 2048;
constexpr int MAX_SPLITS = 16;

// Source of the zero rows that stand in for -1 / out-of-range slots.
__device__ __attribute__((aligned(16))) uint4 g_zero_row[576 * 2 / 16];

__device__ __forceinline__ v4bf lds_read_tr(const char* lds_base, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf_ptr)(lds_base + byte_off));
}

// Barrier that waits only for this wave's LDS operations, not for the
// direct-to-LDS loads still in flight into the other buffer.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 h = (__bf16)x;                    // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Workgroup blockIdx.x runs on XCD blockIdx.x % 8 (the dispatcher deals
// workgroups round robin over the 8 XCDs).  Work items are numbered so that a
// query's items are consecutive; giving every XCD one contiguous range of
// per_xcd items keeps a query's splits and head blocks (and, in the merge, its
// partials) on as few XCDs as the balance allows, sharing their L2.  Items
// past the end belong to no work.
__device__ __forceinline__ int xcd_item(int wg, int per_xcd) {
    return (wg % 8) * per_xcd + wg / 8;
}

// LDS slot of tile row r: within each 16-row half the rows are stored as a
// 4 x 4 transpose (slot 4*(r%4) + (r/4)%4).  With an odd number of 16-byte
// bank groups per row stride (stride = 4 mod 8 words, 64 banks), both read
// patterns of a tile hit distinct banks: the QK operand reads (16
// consecutive rows, one 16-byte chunk: any 16 distinct slots of a half) and
// the transposing PV reads (rows 4i..4i+3, 64 contiguous bytes each, whose
// slots 4*(r%4) + i start 64 bytes apart in bank order).  Rows keep their
// tile order everywhere else.
__device__ __forceinline__ int tile_slot(int r) {
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

// Two E4M3 codes (the low or high 16 bits of w) times the row scale, as two
// bf16 in one word.  The scale is a power of two, so the products are exact
// in bf16 while they stay in its normal range.
template <bool HI>
__device__ __forceinline__ uint32_t kv8_dequant_pair(uint32_t w, float scale) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    return __builtin_bit_cast(uint32_t, v);
}

template <int HB, int VS, int D, int DV, int GR>
struct AttendGeom {
    static constexpr int KSP = 4 / HB;              // waves sharing a head block (K split)
    static constexpr int KS = D / 16;               // k-steps of the QK product
    static constexpr int KSW = KS / KSP;            // k-steps per wave
    static constexpr int CH = D * 2 / 16;           // 16-byte chunks per latent row
    static constexpr int CROWB = D * 2;             // latent row bytes in HBM
    // LDS row stride: one 16-byte pad per row puts the 16 rows a quarter-wave
    // reads (same chunk, consecutive rows) in distinct 4-bank groups, and the
    // transposing reads (4 rows x 32 bytes) in distinct banks too
    static constexpr int ROWB = D * 2 + 16;
    static_assert((ROWB / 4) % 8 == 4, "pad keeps row starts spread over the banks");
    static constexpr int COLS = DV / VS;            // value columns of the workgroup
    static constexpr int CW = COLS / KSP;           // value columns per wave
    static constexpr int NB = CW / 32;              // 32-column MFMA blocks per wave
    static constexpr int TILE_BYTES = TILE_ROWS * ROWB;
    static constexpr int TILE_CHUNKS = TILE_ROWS * CH;
    // gather: 8 threads per row, thread (row, sub) takes chunks sub, sub + 8, ...
    static constexpr int TPR = AT_THREADS / TILE_ROWS;
    static constexpr int GPT = (CH + TPR - 1) / TPR;     // chunks per thread
    // GR groups of 4 waves per workgroup, each on its own tiles; waves per
    // SIMD: 2 where the accumulators fit 256 registers per lane (two groups
    // in one workgroup, or two workgroups), else 1
    static constexpr int THREADS = AT_THREADS * GR;
    static constexpr int WAVES_PER_SIMD = NB <= 4 ? 2 : 1;
    static constexpr int WG_PER_CU = WAVES_PER_SIMD / GR > 0 ? WAVES_PER_SIMD / GR : 1;
    // QK accumulators per wave (two halve the dependent MFMA chain where
    // registers allow)
    static constexpr int QK_ACC = (WAVES_PER_SIMD == 2 && NB == 4) ? 1 : 2;
    static_assert(GR == 1 || WAVES_PER_SIMD == 2, "two groups need the 256-register budget");
    static_assert(KS % KSP == 0, "the K split must divide the k-steps");
    static_assert(CW % 32 == 0, "value columns per wave");
};

// KV8: the latent cache is FP8 (see kv8_dequant_pair): the gather reads the
// E4M3 codes, the row's exponent byte and the bf16 RoPE slice, and the tile
// store writes the dequantized bf16 row, so the LDS tile and everything that
// reads it are the same as for a bf16 cache.
template <int HB, int VS, int D, int DV, int GR, bool KV8>
__global__ __launch_bounds__((AttendGeom<HB, VS, D, DV, GR>::THREADS),
                             (AttendGeom<HB, VS, D, DV, GR>::WG_PER_CU)) void sparse_attend_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ C, const uint8_t* __restrict__ C8,
    const uint8_t* __restrict__ Ce, const uint16_t* __restrict__ Cr,
    const int32_t* __restrict__ idx, int Tq, int H, int L_cap, int k, float scale_log2,
    int slots_per_split, int splits, int nq, int nz, int per_xcd, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float2* __restrict__ part_ml,
    PageMap pm) {
    using G = AttendGeom<HB, VS, D, DV, GR>;
    constexpr int ROWB = G::ROWB;
    // FP8 row: DV code bytes, the exponent byte, D - DV bf16 RoPE dims
    constexpr int F8CH = DV / 16;                  // 16-byte code chunks per row
    constexpr int F8PT = F8CH / G::TPR;            // code chunks per gather thread
    constexpr int RCH = (D - DV) * 2 / 16;         // 16-byte RoPE chunks per row
    static_assert(!KV8 || (F8CH % G::TPR == 0 && RCH <= G::TPR), "FP8 gather geometry");

    __shared__ __attribute__((aligned(16))) char tiles[GR][G::TILE_BYTES];
    // per group: partial S^T blocks of the reduce-scatter ([owner wave][slot][lane]),
    // the waves' row maxima or softmax sums ([wave][lane]), their P rows in bf16
    __shared__ __attribute__((aligned(16))) float4 xbufs[GR][4][4][64];
    __shared__ float mbufs[GR][4][64];
    __shared__ uint32_t pbufs[GR][4][4][64];
    __shared__ uint32_t s_bad;
    __shared__ int sidx[MAX_SPLIT_SLOTS + TILE_ROWS * GR];
    __shared__ uint32_t tmask[(MAX_SPLIT_SLOTS + TILE_ROWS * GR) / TILE_ROWS + 2];   // valid rows per tile

    // group and wave indices are wave-uniform: keep them in scalar registers
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / AT_THREADS);   // group of 4 waves
    const int tid = threadIdx.x % AT_THREADS;  // index within the group
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int g = lane >> 5;
    const int hbl = wave % HB;              // head block within the workgroup
    const int kp = wave / HB;               // this wave's share of the K and column split
    // work item (query, split, head-block group x column part), numbered in
    // that order, from the workgroup's place in the XCD round robin (see
    // xcd_item)
    const int item = xcd_item(blockIdx.x, per_xcd);
    if (item >= nq * splits * nz) return;
    const int q = item / (splits * nz);     // b * Tq + t
    const int sp = (item / nz) % splits;
    const int zz = item % nz;
    const int hbg = zz / VS;                // head-block group of the workgroup
    const int vh = zz - hbg * VS;           // column part
    const int b = q / Tq;
    const int head = (hbg * HB + hbl) * 32 + j;
    const bool head_ok = head < H;
    const int slot0 = sp * slots_per_split;
    const int slot1 = min(slot0 + slots_per_split, k);
    const int32_t* qidx = idx + (size_t)q * k;
    // cache rows of this sequence: [b*L_cap, (b+1)*L_cap) of a contiguous
    // cache, or the page pool (slots are translated to pool rows below)
    const size_t row0 = pm.table ? 0 : (size_t)b * L_cap;
    const char* Cb = KV8 ? nullptr : reinterpret_cast<const char*>(C + row0 * D);
    const char* C8b = KV8 ? reinterpret_cast<const char*>(C8 + row0 * DV) : nullptr;
    const uint8_t* Ceb = KV8 ? Ce + row0 : nullptr;
    const char* Crb = KV8 ? reinterpret_cast<const char*>(Cr + row0 * (D - DV)) : nullptr;
    const int col0 = vh * G::COLS + kp * G::CW;   // first value column of this wave
    char* tile = tiles[grp];
    float4 (*xb)[4][64] = xbufs[grp];
    float (*mbuf)[64] = mbufs[grp];
    uint32_t (*pbuf)[4][64] = pbufs[grp];

    // tiles of the split; group grp takes tiles grp, grp + GR, ...  Every group
    // runs the same number of iterations (a group past the last tile computes
    // an all-invalid tile, which changes nothing), so the workgroup barriers
    // stay uniform.
    const int ntiles = (slot1 - slot0 + TILE_ROWS - 1) / TILE_ROWS;
    const int iters = (ntiles + GR - 1) / GR;
    // this split's positions, once, into LDS; invalid ones and the padding up
    // to a whole number of tiles per group become -1
    const int padded = iters * GR * TILE_ROWS;
    for (int i = threadIdx.x; i < padded; i += G::THREADS) {
        int s = slot0 + i < slot1 ? qidx[slot0 + i] : -1;
        bool ok = s >= 0 && s < L_cap;
        if (pm.table != nullptr && ok) {
            // logical position -> row of the page pool; unallocated pages are skipped
            const int page = pm.table[(size_t)b * pm.max_blocks + (s >> pm.shift)];
            ok = page >= 0 && page < pm.n_pages;
            s = (page << pm.shift) + (s & ((1 << pm.shift) - 1));
        }
        sidx[i] = ok ? s : -1;
        // a wave covers 64 consecutive slots = two tiles: one bit per row
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {
            tmask[i / TILE_ROWS] = (uint32_t)bits;
            tmask[i / TILE_ROWS + 1] = (uint32_t)(bits >> 32);
        }
    }

    v8bf qb[G::KSW];   // this wave's share of Q^T (loaded after the first gather is issued)
    v16f o[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nb][r] = 0.0f;
    float m_run = -__builtin_inff();   // running reference max (log2 units), same in every wave of a head block

    // gather: thread (row tid / 8, sub tid % 8) owns chunks sub, sub + 8, ... of
    // one tile row, so one base address and immediate offsets serve all its
    // loads and LDS stores; rows of -1 / out-of-range slots read a zero row.
    // (Macros rather than lambdas keep the register arrays out of memory.)
    const uintptr_t zero_row = reinterpret_cast<uintptr_t>(g_zero_row);
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(Cb);
    const int grow = tid / G::TPR;
    const int gsub = tid % G::TPR;
    char* const lrow = tile + tile_slot(grow) * ROWB + gsub * 16;
#define ISA_LOAD_TILE(R, TS)                                                                   \
    {                                                                                          \
        const int s_ = sidx[(TS) - slot0 + grow];   /* -1 past the split (padded) */           \
        const uintptr_t ra_ = (s_ >= 0 ? cbase + (size_t)s_ * G::CROWB : zero_row) + gsub * 16; \
        _Pragma("unroll") for (int i_ = 0; i_ < G::GPT; ++i_) {                               \
            if (G::CH % G::TPR == 0 || gsub + G::TPR * i_ < G::CH)                             \
                R[i_] = *(global_v4u_ptr)(ra_ + i_ * G::TPR * 16);                             \
        }                                                                                      \
    }
#define ISA_STORE_TILE(R)                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < G::GPT; ++i_) {                                   \
        if (G::CH % G::TPR == 0 || gsub + G::TPR * i_ < G::CH)                                 \
            *reinterpret_cast<v4u*>(lrow + i_ * G::TPR * 16) = R[i_];                          \
    }
    // FP8 rows: thread (row, sub) takes code chunks sub, sub + 8, ... (each is
    // 16 dims, 32 bytes of the bf16 tile row), RoPE chunk sub (if any) and the
    // row's exponent byte; an invalid slot reads zero codes with exponent 0.
    const uintptr_t c8base = reinterpret_cast<uintptr_t>(C8b);
    const uintptr_t crbase = reinterpret_cast<uintptr_t>(Crb);
    char* const lrow8 = tile + tile_slot(grow) * ROWB;
#define ISA_LOAD_TILE8(R8, RR, SE, TS)                                                         \
    {                                                                                          \
        const int s_ = sidx[(TS) - slot0 + grow];                                              \
        const uintptr_t ca_ = (s_ >= 0 ? c8base + (size_t)s_ * DV : zero_row) + gsub * 16;     \
        _Pragma("unroll") for (int i_ = 0; i_ < F8PT; ++i_)                                    \
            R8[i_] = *(global_v4u_ptr)(ca_ + i_ * G::TPR * 16);                                \
        if (gsub < RCH)                                                                        \
            RR = *(global_v4u_ptr)((s_ >= 0 ? crbase + (size_t)s_ * ((D - DV) * 2) : zero_row) \
                                   + gsub * 16);                                               \
        SE = s_ >= 0 ? (uint32_t)Ceb[s_] : 0u;                                                 \
    }
#define ISA_STORE_TILE8(R8, RR, SE)                                                            \
    {                                                                                          \
        const float sc_ = __uint_as_float((SE) << 23);                                         \
        _Pragma("unroll") for (int i_ = 0; i_ < F8PT; ++i_) {                                  \
            char* d_ = lrow8 + (gsub + i_ * G::TPR) * 32;                                      \
            *reinterpret_cast<v4u*>(d_) = v4u{kv8_dequant_pair<false>(R8[i_][0], sc_),         \
                                              kv8_dequant_pair<true>(R8[i_][0], sc_),          \
                                              kv8_dequant_pair<false>(R8[i_][1], sc_),         \
                                              kv8_dequant_pair<true>(R8[i_][1], sc_)};         \
            *reinterpret_cast<v4u*>(d_ + 16) = v4u{kv8_dequant_pair<false>(R8[i_][2], sc_),    \
                                                   kv8_dequant_pair<true>(R8[i_][2], sc_),     \
                                                   kv8_dequant_pair<false>(R8[i_][3], sc_),    \
                                                   kv8_dequant_pair<true>(R8[i_][3], sc_)};    \
        }                                                                                      \
        if (gsub < RCH) *reinterpret_cast<v4u*>(lrow8 + DV * 2 + gsub * 16) = RR;              \
    }

    // one tile of the online softmax attention, from the LDS tile.  The K
    // split leaves each of the KSP waves of a head block a partial S^T; a
    // reduce-scatter through LDS gives wave kp the sums of registers
    // [kp*RG, (kp+1)*RG) (RG = 16/KSP registers: 32/KSP tile rows for both
    // lane halves), added in kp order, and each wave turns only its own rows
    // into softmax weights P; the bf16 P rows are then exchanged so every
    // wave feeds the whole P^T to its PV product.  The reference max: on the
    // first tile with a valid row it is the tile's max (one more exchange);
    // afterwards P is computed against the running reference and only when
    // some wave's rows exceed it by more than RESCALE_SLACK (all waves see the
    // same maxima, so the decision is the same in each) is the reference
    // moved, the accumulators rescaled and P computed again.
    static_assert(G::KSP == 2 || G::KSP == 4, "the K split spans two or four waves");
    constexpr int RG = 16 / G::KSP;          // registers (of 16) this wave finalizes
    constexpr int RQ = RG / 4;               // float4 slots per (owner, source) pair
    float l_own = 0.0f;                      // softmax sum over this wave's rows
    bool bad = false;                        // a row of this wave exceeded the reference by > RESCALE_SLACK
    auto compute_tile = [&](int tile_start, bool exact) {
        // ---- partial S^T (32 rows x 32 heads) over this wave's k-steps: every
        // A operand is requested from LDS first, then the MFMAs run in two
        // independent accumulator chains (even and odd k-steps)
        const char* arow = tile + tile_slot(j) * ROWB;
        v8bf a[G::KSW];
#pragma unroll
        for (int i = 0; i < G::KSW; ++i) {
            const int ch = 2 * (kp * G::KSW + i) + g;
            a[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(arow + ch * 16));
        }
        // keep the scheduler from sinking the reads between the MFMAs (where
        // the registers allow: the wide variant holds twice the accumulators)
        if constexpr (G::NB <= 4) __builtin_amdgcn_sched_barrier(0);
        v16f st, st2;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = st2[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < G::KSW; ++i) {
            if (i & 1)
                st2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qb[i], st2, 0, 0, 0);
            else
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qb[i], st, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] += st2[r];
        // ---- reduce-scatter: every wave posts all its partial registers
        // (its own share included, so the sum below needs no branch on kp)
#pragma unroll
        for (int o = 0; o < G::KSP; ++o)
#pragma unroll
            for (int q4 = 0; q4 < RQ; ++q4) {
                const int r0 = o * RG + 4 * q4;
                xb[o * HB + hbl][kp * RQ + q4][lane] = make_float4(st[r0], st[r0 + 1], st[r0 + 2], st[r0 + 3]);
            }
        lds_barrier();
        float so[RG];                        // this wave's rows: registers kp*RG + i
#pragma unroll
        for (int q4 = 0; q4 < RQ; ++q4) {
            float4 acc = xb[wave][q4][lane];
#pragma unroll
            for (int src = 1; src < G::KSP; ++src) {
                const float4 v = xb[wave][src * RQ + q4][lane];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            so[4 * q4] = acc.x; so[4 * q4 + 1] = acc.y; so[4 * q4 + 2] = acc.z; so[4 * q4 + 3] = acc.w;
        }
        // register r holds tile row 8*(r/4) + 4*g + r%4, head j; rows of -1
        // slots get -inf (tiles without such rows, the usual case, skip this)
        const uint32_t tm = tmask[(tile_start - slot0) / TILE_ROWS];
        if (tm != 0xFFFFFFFFu) {
#pragma unroll
            for (int i = 0; i < RG; ++i) {
                const int r = kp * RG + i;
                if (!((tm >> (8 * (r / 4) + 4 * g + (r % 4))) & 1u)) so[i] = -__builtin_inff();
            }
        }
        float mloc = so[0];
#pragma unroll
        for (int i = 1; i < RG; ++i) mloc = fmaxf(mloc, so[i]);
        mloc = xor32_max(mloc) * scale_log2;   // scale > 0 keeps the order
        // the reference: exact (the tile's max over every wave's rows, one more
        // exchange) on the workgroup's first tile, otherwise the running one,
        // with P bounded by 2^RESCALE_SLACK unless a row exceeds it (then the
        // workgroup's tiles are computed again with exact references)
        if (exact) {
            mbuf[wave][lane] = mloc;
            lds_barrier();
            float m_t = mbuf[hbl][lane];
#pragma unroll
            for (int src = 1; src < G::KSP; ++src) m_t = fmaxf(m_t, mbuf[src * HB + hbl][lane]);
            const bool move = m_t > m_run + RESCALE_SLACK;
            if (__ballot(move)) {
                const float m_new = move ? m_t : m_run;
                const bool had = m_run != -__builtin_inff();
                const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                m_run = m_new;
                if (__ballot(had)) {
                    l_own *= alpha;
#pragma unroll
                    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
                }
            }
        } else {
            bad = bad || __ballot(mloc > m_run + RESCALE_SLACK) != 0ull;
        }
        // P of this wave's rows, posted in bf16
        {
            const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
            float psum = 0.0f;
#pragma unroll
            for (int d = 0; d < RG / 2; ++d) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(so[2 * d], scale_log2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(so[2 * d + 1], scale_log2, -m_use));
                psum += p0;
                psum += p1;
                pbuf[wave][d][lane] = (uint32_t)f2bf(p0) | ((uint32_t)f2bf(p1) << 16);
            }
            l_own += psum;
        }
        // ---- the V^T operands of the PV product (read transposed from the
        // row-major tile, two reads per operand): with few value blocks they are
        // requested before the exchange completes, so their LDS latency
        // overlaps it
        const int G16 = lane >> 4;
        const int i16 = lane & 15;
        constexpr bool PRE_V = G::NB <= 4;
        v4bf vlo[2][G::NB], vhi[2][G::NB];
        auto read_v = [&](int kk, int nb) {
            const int row = 16 * kk + 4 * (G16 >> 1) + (i16 >> 2);
            const int col = col0 + 32 * nb + 16 * (G16 & 1) + 4 * (i16 & 3);
            vlo[kk][nb] = lds_read_tr(tile, tile_slot(row) * ROWB + col * 2);
            vhi[kk][nb] = lds_read_tr(tile, tile_slot(row + 8) * ROWB + col * 2);
        };
        if constexpr (PRE_V) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int nb = 0; nb < G::NB; ++nb) read_v(kk, nb);
        }
        lds_barrier();
        // ---- all of P^T as the PV B operand: register r of the tile is owned
        // by wave r / RG, which posted it as dword (r % RG) / 2
        v8bf pk[2];
#pragma unroll
        for (int r2 = 0; r2 < 8; ++r2) {
            const int r = 2 * r2;
            const uint32_t w2 = pbuf[(r / RG) * HB + hbl][(r % RG) / 2][lane];
            pk[r / 8][r % 8] = __builtin_bit_cast(__bf16, (uint16_t)(w2 & 0xFFFFu));
            pk[r / 8][r % 8 + 1] = __builtin_bit_cast(__bf16, (uint16_t)(w2 >> 16));
        }

        // ---- O^T[this wave's columns x heads] += V^T . P^T over the tile's 32 rows
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int nb = 0; nb < G::NB; ++nb) {
                if constexpr (!PRE_V) read_v(kk, nb);
                const v4bf lo = vlo[kk][nb], hi = vhi[kk][nb];
                const v8bf av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[kk], o[nb], 0, 0, 0);
            }
        }
    };

    // software pipeline: the next tile of the group is in flight in registers
    // while the current one is computed from LDS
    auto tile_start = [&](int it) { return slot0 + (it * GR + grp) * TILE_ROWS; };
    if (threadIdx.x == 0) s_bad = 0u;
    lds_barrier();                          // sidx visible
    v4u rA[KV8 ? 1 : G::GPT];   // native vectors: HIP's uint4 class defeats register promotion
    v4u r8A[KV8 ? F8PT : 1], rrA = v4u{0u, 0u, 0u, 0u};
    uint32_t seA = 0;
#define ISA_LOAD_ANY(TS)                                                                        \
    if constexpr (KV8) { ISA_LOAD_TILE8(r8A, rrA, seA, TS) } else { ISA_LOAD_TILE(rA, TS) }
#define ISA_STORE_ANY()                                                                         \
    if constexpr (KV8) { ISA_STORE_TILE8(r8A, rrA, seA) } else { ISA_STORE_TILE(rA) }
    if (iters > 0) { ISA_LOAD_ANY(tile_start(0)) }
    // this wave's share of Q^T, requested after the first tile's gather (which
    // gates everything): lane (head j, half g) holds dims 16*ks + 8*g .. +8 for
    // ks in [kp*KSW, (kp+1)*KSW).  Heads past H read head 0; their results are
    // never stored.
    if constexpr (GR == 2) {
        // both groups need the same Q: the workgroup's 64 head rows (contiguous
        // in HBM) are staged once in the still unused tile LDS, 64 rows of ROWB
        // bytes, and every wave reads its share from there
        constexpr int QROWS = HB * 32;
        constexpr int QCH = QROWS * G::CH;
        constexpr int QPT = (QCH + G::THREADS - 1) / G::THREADS;
        static_assert(QROWS * ROWB <= GR * G::TILE_BYTES, "Q rows fit the tile buffers");
        char* const qlds = &tiles[0][0];
        const int h0 = hbg * QROWS;
        v4u qt[QPT];
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int c = u * G::THREADS + (int)threadIdx.x;
            if (QCH % G::THREADS == 0 || c < QCH) {
                const int hr = c / G::CH, ch = c - (c / G::CH) * G::CH;
                const int hh = h0 + hr < H ? h0 + hr : 0;
                qt[u] = *(global_v4u_ptr)(Q + ((size_t)q * H + hh) * D + ch * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int c = u * G::THREADS + (int)threadIdx.x;
            if (QCH % G::THREADS == 0 || c < QCH) {
                const int hr = c / G::CH, ch = c - (c / G::CH) * G::CH;
                *reinterpret_cast<v4u*>(qlds + hr * ROWB + ch * 16) = qt[u];
            }
        }
        lds_barrier();
        const char* qr = qlds + (hbl * 32 + j) * ROWB;
#pragma unroll
        for (int i = 0; i < G::KSW; ++i)
            qb[i] = __builtin_bit_cast(
                v8bf, *reinterpret_cast<const v4u*>(qr + (16 * (kp * G::KSW + i) + 8 * g) * 2));
        lds_barrier();                      // Q read out before the tiles are written
    } else {
        const uint16_t* qrow = Q + ((size_t)q * H + (head_ok ? head : 0)) * D;
#pragma unroll
        for (int i = 0; i < G::KSW; ++i)
            qb[i] = __builtin_bit_cast(
                v8bf, *reinterpret_cast<const uint4*>(qrow + 16 * (kp * G::KSW + i) + 8 * g));
    }
    if (iters > 0) { ISA_STORE_ANY() }
    if (iters > 1) { ISA_LOAD_ANY(tile_start(1)) }
    lds_barrier();
    auto tile_loop = [&](bool exact_all) {
        for (int it = 0; it < iters; ++it) {
            compute_tile(tile_start(it), exact_all || it == 0);   // in flight: tile it+1
            if (it + 1 >= iters) break;
            lds_barrier();
            ISA_STORE_ANY()
            if (it + 2 < iters) { ISA_LOAD_ANY(tile_start(it + 2)) }
            lds_barrier();
        }
    };
    tile_loop(false);
    // a row above the running reference by more than RESCALE_SLACK (possible
    // when a group's first tile holds no valid row, or with very uneven
    // scores): the whole split again, with an exact reference on every tile
    if (bad) atomicOr(&s_bad, 1u);
    lds_barrier();
    if (s_bad) {
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[nb][r] = 0.0f;
        m_run = -__builtin_inff();
        l_own = 0.0f;
        if (iters > 0) { ISA_LOAD_ANY(tile_start(0)) ISA_STORE_ANY() }
        if (iters > 1) { ISA_LOAD_ANY(tile_start(1)) }
        lds_barrier();
        tile_loop(true);
        lds_barrier();
    }
#undef ISA_LOAD_ANY
#undef ISA_STORE_ANY
#undef ISA_LOAD_TILE8
#undef ISA_STORE_TILE8
#undef ISA_LOAD_TILE
#undef ISA_STORE_TILE

    // the softmax sum of every head over the group's rows: both lane halves,
    // then the head block's waves in kp order
    float l_run;
    {
        mbuf[wave][lane] = xor32_sum(l_own);
        lds_barrier();
        l_run = mbuf[hbl][lane];
#pragma unroll
        for (int src = 1; src < G::KSP; ++src) l_run += mbuf[src * HB + hbl][lane];
    }

    // With two groups, group g finishes value blocks [g*NB/2, (g+1)*NB/2): each
    // group hands the other the blocks it does not finish, with its (max, sum),
    // through the (now free) tile LDS, and both combine the two online-softmax
    // states in the same order (group 0's term first), so both hold the same
    // sum and maximum.
    constexpr int HALF = GR == 2 ? G::NB / 2 : G::NB;
    auto mine_block = [&](int nb) { return GR == 1 || nb / HALF == grp; };
    if constexpr (GR == 2) {
        static_assert(G::NB % 2 == 0, "value blocks split between the groups");
        constexpr int PER_LANE = HALF * 16 + 2;
        static_assert(GR * 4 * 64 * PER_LANE * 4 <= GR * G::TILE_BYTES, "hand-off fits the tiles");
        float* const mb = reinterpret_cast<float*>(&tiles[0][0]);
        float* const give = mb + (size_t)((grp * 4 + wave) * PER_LANE) * 64;
        const float* const take = mb + (size_t)(((1 - grp) * 4 + wave) * PER_LANE) * 64;
        lds_barrier();                      // every wave is done with the tiles
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            if (!mine_block(nb)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) give[((nb % HALF) * 16 + r) * 64 + lane] = o[nb][r];
            }
        }
        give[(HALF * 16) * 64 + lane] = m_run;
        give[(HALF * 16 + 1) * 64 + lane] = l_run;
        lds_barrier();
        const float m_t = take[(HALF * 16) * 64 + lane];
        const float l_t = take[(HALF * 16 + 1) * 64 + lane];
        const float m0 = grp == 0 ? m_run : m_t, m1 = grp == 0 ? m_t : m_run;
        const float l0 = grp == 0 ? l_run : l_t, l1 = grp == 0 ? l_t : l_run;
        const float M = fmaxf(m0, m1);
        const float Mu = M == -__builtin_inff() ? 0.0f : M;
        const float a0 = __builtin_amdgcn_exp2f(m0 - Mu);
        const float a1 = __builtin_amdgcn_exp2f(m1 - Mu);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            if (mine_block(nb)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float own = o[nb][r];
                    const float oth = take[((nb % HALF) * 16 + r) * 64 + lane];
                    o[nb][r] = (grp == 0 ? own : oth) * a0 + (grp == 0 ? oth : own) * a1;
                }
            }
        }
        l_run = l0 * a0 + l1 * a1;
        m_run = M;
    }

    // softmax denominator of head j over all the workgroup's rows
    const float l_tot = l_run;

    // o[nb] register r holds value column col0 + 32*nb + 8*(r/4) + 4*g + r%4 of head j
    if (splits == 1) {
        if (!head_ok) return;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = out + ((size_t)q * H + head) * DV;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            if (!mine_block(nb)) continue;
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
        if (lse && grp == 0 && kp == 0 && vh == 0 && g == 0)
            lse[(size_t)q * H + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * LN2 : -__builtin_inff();
        return;
    }

    // ---- split: publish this split's output normalised by its own sum (bf16;
    // the merge re-weights it by the split's (max, sum), kept in fp32).  The
    // partial keeps the register layout, [..][wave][nb][r4][lane] x 4 bf16, so
    // every store instruction writes 512 contiguous bytes; the merge kernel
    // reads it in that layout.
    {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int n_hbg = nz / VS;
        v2u* po = reinterpret_cast<v2u*>(part_o) +
                  (((((size_t)q * splits + sp) * n_hbg + hbg) * VS + vh) * 4 + wave) *
                      (G::NB * 4 * 64);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            if (!mine_block(nb)) continue;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const uint32_t lo = (uint32_t)f2bf(o[nb][4 * r4] * inv) |
                                    ((uint32_t)f2bf(o[nb][4 * r4 + 1] * inv) << 16);
                const uint32_t hi = (uint32_t)f2bf(o[nb][4 * r4 + 2] * inv) |
                                    ((uint32_t)f2bf(o[nb][4 * r4 + 3] * inv) << 16);
                // streaming stores: the merge fetches the partials back from
                // beyond L2 whatever the store policy (its counted reads hold
                // them whole), and non-temporal writes cost the layer less
                __builtin_nontemporal_store(v2u{lo, hi}, &po[(nb * 4 + r4) * 64 + lane]);
            }
        }
        if (head_ok && grp == 0 && kp == 0 && g == 0)
            part_ml[(((size_t)q * splits + sp) * VS + vh) * H + head] = make_float2(m_run, l_tot);
    }
}

// Combines the splits of every (query, head): with each split's output O_s
// normalised by its own sum l_s, out = sum_s w_s O_s / sum_s w_s where
// w_s = 2^(m_s - M) l_s, in split order; column part p uses the (max, sum)
// its own workgroups wrote.  The partials are in the attention kernel's
// register layout (per query, split, head-block group and column part:
// [wave][nb][r4][lane] x 4 bf16), and a merge thread takes one lane position
// of that layout (4 columns of one head), so its loads are contiguous across
// threads.  Every split's partial is requested before any is used.
constexpr int MERGE_THREADS = 256;
template <int DV, int VS, int HB, int NB, int CW, int MS>
__global__ __launch_bounds__(MERGE_THREADS) void merge_splits_kernel(
    const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml, int nq, int H,
    int n_hbg, int splits, int per_xcd, uint16_t* __restrict__ out, float* __restrict__ lse) {
    constexpr int COLS = DV / VS;
    constexpr int BLOCK = 4 * NB * 4 * 64;         // v2u per (query, split, hbg, column part)
    static_assert(MERGE_THREADS == 4 * 64, "a workgroup covers the 4 r4 rows of one (wave, nb)");
    // The workgroup's 256 threads are lane x r4 of one (query, head-block
    // group, column part, wave, nb) of the layout: those are uniform, and a
    // split's partials are one contiguous 2 KiB run at a uniform address.
    int rest = __builtin_amdgcn_readfirstlane(xcd_item(blockIdx.x, per_xcd));
    const int nb = rest % NB; rest /= NB;
    const int wave = rest % 4; rest /= 4;
    const int vh = rest % VS; rest /= VS;
    const int hbg = rest % n_hbg; rest /= n_hbg;
    const int q = rest;
    if (q >= nq) return;
    const int lane = threadIdx.x & 63;
    const int r4 = threadIdx.x >> 6;
    const int hbl = wave % HB, kp = wave / HB;
    const int head = (hbg * HB + hbl) * 32 + (lane & 31);
    const int head_c = head < H ? head : H - 1;     // heads past H load head H-1, store nothing
    const int col = vh * COLS + kp * CW + 32 * nb + 8 * r4 + 4 * (lane >> 5);
    const v2u* pb = reinterpret_cast<const v2u*>(part_o) +
                    ((((size_t)q * splits) * n_hbg + hbg) * VS + vh) * BLOCK +
                    ((size_t)wave * NB + nb) * 4 * 64;
    const size_t pstride = (size_t)n_hbg * VS * BLOCK;       // v2u between splits
    const float2* mb = part_ml + ((size_t)q * splits * VS + vh) * H;
    const size_t mstride = (size_t)VS * H;                   // float2 between splits
    // every load is issued before any is used, unconditionally: splits past
    // the last one (up to MS, the smallest of 2, 4, 8, 16 that holds them)
    // read the last one again and get weight 0 below
    float2 ml[MS];
    v2u v[MS];
#pragma unroll
    for (int sj = 0; sj < MS; ++sj) {
        const int sc = sj < splits ? sj : splits - 1;
        ml[sj] = mb[sc * mstride + head_c];
        v[sj] = pb[sc * pstride + threadIdx.x];
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int sj = 0; sj < MS; ++sj) M = fmaxf(M, ml[sj].x);
    const float Mu = M == -__builtin_inff() ? 0.0f : M;
    float L = 0.0f;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sj = 0; sj < MS; ++sj) {
        // 0 for an empty split or one past the last; weights below 2^-126
        // (flushed by v_exp_f32) are far below the fp32 resolution of the
        // sum, whose largest term has weight 1
        const float wgt = sj < splits ? __builtin_amdgcn_exp2f(ml[sj].x - Mu) * ml[sj].y : 0.0f;
        L += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w32 = v[sj][e / 2];
            acc[e] += wgt * __uint_as_float((e & 1) ? (w32 & 0xFFFF0000u) : (w32 << 16));
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const v2u r = {(uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16),
                   (uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16)};
    if (head >= H) return;
    *reinterpret_cast<v2u*>(out + ((size_t)q * H + head) * DV + col) = r;
    if (lse && vh == 0 && kp == 0 && nb == 0 && r4 == 0 && lane < 32)
        lse[(size_t)q * H + head] = L > 0.0f ? (M + log2f(L)) * LN2 : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// Many queries (prefill): one workgroup of four waves per query, wave w
// owning heads [16w, 16w + 16) whole.  Per tile of 32 gathered latent rows
// (two LDS tile buffers; during each tile's QK products the next tile goes
// from registers into the other buffer, then the one after it is requested;
// one barrier per tile):
//   * S^T (32 rows x 16 heads) = C_rows . Q^T on v_mfma_f32_16x16x32_bf16
//     over all D dims (the wave's Q^T stays in registers): two 16-row blocks,
//     each summed in two accumulator chains;
//   * the 16x16 accumulator layout gives lane (g, j) rows 4g..4g+3 and
//     16+4g..16+4g+3 of head j, which are the B-operand rows of the next
//     product when its contraction pairs lane group g with those rows: P^T
//     feeds PV from registers, and a head's tile max takes two lane swaps;
//   * O^T (DV columns x 16 heads) += V^T . P^T in DV/16 blocks, V^T read
//     transposed (ds_read_b64_tr_b16) from the row-major tile in the same row
//     order; rows sit in LDS in the order heads_slot gives, which keeps both
//     read patterns free of bank conflicts.
// No wave waits for another except at the tile barrier: there is no K split,
// so no exchange of partial scores or of P, at the price of every wave
// reading the whole tile from LDS.  The reference max of a head moves only
// when its exact tile max exceeds it by more than RESCALE_SLACK.
constexpr int HW_THREADS = 256;
// LDS slot of tile row r in the per-query kernel: within each 16-row half,
// rows 0-7 take the even slots and rows 8-15 the odd ones.  With a row stride
// of 4 mod 8 words (64 banks), the QK operand reads (16 rows, one 16-byte
// chunk) touch 16 distinct 4-bank groups for any 16 slots of a half, and each
// 32-lane half of a transposing V^T read (8 rows, 32 bytes each: rows 0-7 or
// 8-15 of a half) starts its rows on 8 distinct multiples of 8 banks.
__device__ __forceinline__ int heads_slot(int r) {
    return (r & 16) | ((r & 7) << 1) | ((r >> 3) & 1);
}
// log2 of the largest P the per-query kernel keeps without moving the reference
constexpr float HW_HEADROOM = 64.0f;

__device__ __forceinline__ float xor16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int DV, bool KV8>
__global__ __launch_bounds__(HW_THREADS, 1) void attend_heads_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ C, const uint8_t* __restrict__ C8,
    const uint8_t* __restrict__ Ce, const uint16_t* __restrict__ Cr,
    const int32_t* __restrict__ idx, int Tq, int H, int L_cap, int k, float scale_log2, int nq,
    int per_xcd, uint16_t* __restrict__ out, float* __restrict__ lse, PageMap pm) {
    constexpr int ROWB = D * 2 + 16;              // one 16-byte pad per row (see heads_slot)
    static_assert((ROWB / 4) % 8 == 4, "pad keeps row starts spread over the banks");
    constexpr int CH = D * 2 / 16;                // 16-byte chunks per latent row
    constexpr int CROWB = D * 2;
    constexpr int TPR = HW_THREADS / TILE_ROWS;   // gather threads per tile row
    constexpr int GPT = (CH + TPR - 1) / TPR;
    constexpr int KS = D / 32;                    // k-steps of the QK product
    constexpr int NBV = DV / 16;                  // 16-column value blocks
    constexpr int TILE_BYTES = TILE_ROWS * ROWB;
    constexpr int F8CH = DV / 16;                 // FP8 rows: code chunks,
    constexpr int F8PT = F8CH / TPR;              //   per gather thread,
    constexpr int RCH = (D - DV) * 2 / 16;        //   RoPE chunks
    static_assert(D % 32 == 0 && DV % 16 == 0 && KS % 2 == 0, "k-steps and value blocks");
    static_assert(!KV8 || (F8CH % TPR == 0 && RCH <= TPR), "FP8 gather geometry");

    __shared__ __attribute__((aligned(16))) char tiles[2][TILE_BYTES];
    __shared__ int sidx[MAX_SPLIT_SLOTS + TILE_ROWS];
    __shared__ uint32_t tmask[MAX_SPLIT_SLOTS / TILE_ROWS + 2];   // valid rows per tile
    __shared__ uint32_t s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;
    const int q = xcd_item(blockIdx.x, per_xcd);   // b * Tq + t
    if (q >= nq) return;
    const int b = q / Tq;
    const int head = 16 * wave + j;
    const bool head_ok = head < H;
    const int32_t* qidx = idx + (size_t)q * k;
    const size_t row0 = pm.table ? 0 : (size_t)b * L_cap;
    const char* Cb = KV8 ? nullptr : reinterpret_cast<const char*>(C + row0 * D);
    const char* C8b = KV8 ? reinterpret_cast<const char*>(C8 + row0 * DV) : nullptr;
    const uint8_t* Ceb = KV8 ? Ce + row0 : nullptr;
    const char* Crb = KV8 ? reinterpret_cast<const char*>(Cr + row0 * (D - DV)) : nullptr;

    // the query's positions into LDS; invalid ones and the padding up to a
    // whole tile become -1
    const int ntiles = (k + TILE_ROWS - 1) / TILE_ROWS;
    const int padded = ntiles * TILE_ROWS;
    for (int i = tid; i < padded; i += HW_THREADS) {
        int s = i < k ? qidx[i] : -1;
        bool ok = s >= 0 && s < L_cap;
        if (pm.table != nullptr && ok) {
            // logical position -> row of the page pool; unallocated pages are skipped
            const int page = pm.table[(size_t)b * pm.max_blocks + (s >> pm.shift)];
            ok = page >= 0 && page < pm.n_pages;
            s = (page << pm.shift) + (s & ((1 << pm.shift) - 1));
        }
        sidx[i] = ok ? s : -1;
        // a wave covers 64 consecutive slots = two tiles: one bit per row
        const uint64_t bits = __ballot(ok);
        if (lane == 0) {
            tmask[i / TILE_ROWS] = (uint32_t)bits;
            tmask[i / TILE_ROWS + 1] = (uint32_t)(bits >> 32);
        }
    }

    // gather: thread (row tid / TPR, sub tid % TPR) owns chunks sub, sub + TPR,
    // ... of one tile row; rows of -1 slots read a zero row
    const uintptr_t zero_row = reinterpret_cast<uintptr_t>(g_zero_row);
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(Cb);
    const uintptr_t c8base = reinterpret_cast<uintptr_t>(C8b);
    const uintptr_t crbase = reinterpret_cast<uintptr_t>(Crb);
    const int grow = tid / TPR;
    const int gsub = tid % TPR;
    const int lrow_off = heads_slot(grow) * ROWB;
#define ISA_HW_LOAD(T)                                                                         \
    {                                                                                          \
        const int s_ = sidx[(T) * TILE_ROWS + grow];                                           \
        if constexpr (KV8) {                                                                   \
            const uintptr_t ca_ = (s_ >= 0 ? c8base + (size_t)s_ * DV : zero_row) + gsub * 16; \
            _Pragma("unroll") for (int i_ = 0; i_ < F8PT; ++i_)                                \
                r8[i_] = *(global_v4u_ptr)(ca_ + i_ * TPR * 16);                               \
            if (gsub < RCH)                                                                    \
                rr = *(global_v4u_ptr)((s_ >= 0 ? crbase + (size_t)s_ * ((D - DV) * 2)         \
                                                : zero_row) + gsub * 16);                      \
            se = s_ >= 0 ? (uint32_t)Ceb[s_] : 0u;                                             \
        } else {                                                                               \
            const uintptr_t ra_ = (s_ >= 0 ? cbase + (size_t)s_ * CROWB : zero_row) + gsub * 16; \
            _Pragma("unroll") for (int i_ = 0; i_ < GPT; ++i_) {                               \
                if (CH % TPR == 0 || gsub + TPR * i_ < CH)                                     \
                    r[i_] = *(global_v4u_ptr)(ra_ + i_ * TPR * 16);                            \
            }                                                                                  \
        }                                                                                      \
    }
#define ISA_HW_STORE(BUF)                                                                      \
    {                                                                                          \
        char* const l_ = &tiles[BUF][0] + lrow_off;                                            \
        if constexpr (KV8) {                                                                   \
            const float sc_ = __uint_as_float(se << 23);                                       \
            _Pragma("unroll") for (int i_ = 0; i_ < F8PT; ++i_) {                              \
                char* d_ = l_ + (gsub + i_ * TPR) * 32;                                        \
                *reinterpret_cast<v4u*>(d_) = v4u{kv8_dequant_pair<false>(r8[i_][0], sc_),     \
                                                  kv8_dequant_pair<true>(r8[i_][0], sc_),      \
                                                  kv8_dequant_pair<false>(r8[i_][1], sc_),     \
                                                  kv8_dequant_pair<true>(r8[i_][1], sc_)};     \
                *reinterpret_cast<v4u*>(d_ + 16) = v4u{kv8_dequant_pair<false>(r8[i_][2], sc_), \
                                                       kv8_dequant_pair<true>(r8[i_][2], sc_),  \
                                                       kv8_dequant_pair<false>(r8[i_][3], sc_), \
                                                       kv8_dequant_pair<true>(r8[i_][3], sc_)}; \
            }                                                                                  \
            if (gsub < RCH) *reinterpret_cast<v4u*>(l_ + DV * 2 + gsub * 16) = rr;             \
        } else {                                                                               \
            _Pragma("unroll") for (int i_ = 0; i_ < GPT; ++i_) {                               \
                if (CH % TPR == 0 || gsub + TPR * i_ < CH)                                     \
                    *reinterpret_cast<v4u*>(l_ + gsub * 16 + i_ * TPR * 16) = r[i_];           \
            }                                                                                  \
        }                                                                                      \
    }

    v4u r[KV8 ? 1 : GPT];        // native vectors: HIP's uint4 class defeats register promotion
    v4u r8[KV8 ? F8PT : 1], rr = v4u{0u, 0u, 0u, 0u};
    uint32_t se = 0;
    if (tid == 0) s_bad = 0u;
    lds_barrier();                                 // sidx and the flag visible
    // the wave's Q^T: lane (g, j) holds dims 32ks + 8g .. +8 of head j; heads
    // past H read head 0 (never stored)
    v8bf qb[KS];
    {
        const uint16_t* qrow = Q + ((size_t)q * H + (head_ok ? head : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = __builtin_bit_cast(v8bf, *(global_v4u_ptr)(qrow + 32 * ks + 8 * g));
    }

    v4f o[NBV];
    float m_run = -__builtin_inff();     // the head's reference max (log2 units), same in its 4 lanes
    float l_own = 0.0f;                  // softmax sum over this lane's rows
    bool bad = false;                    // a tile max above the reference by more than HW_HEADROOM
    // One pass over the tiles.  EXACT = false: a head's reference is the max
    // of its first tile with a valid row and stays there (P = 2^(s - ref) is
    // kept in bf16, whose range holds any P up to 2^HW_HEADROOM); a tile
    // whose max exceeds the reference by more than that sets `bad`, and the
    // pass is run again with EXACT = true, which moves the reference to every
    // tile's max that exceeds it and rescales the accumulators.
    auto pass = [&](auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) o[nb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        m_run = -__builtin_inff();
        l_own = 0.0f;
        if (ntiles > 0) ISA_HW_LOAD(0)
        if (ntiles > 0) ISA_HW_STORE(0)
        if (ntiles > 1) ISA_HW_LOAD(1)
        lds_barrier();
        for (int it = 0; it < ntiles; ++it) {
            // tile it + 1 (in registers since the previous iteration) goes into
            // the other buffer during this tile's QK products, so its LDS
            // writes overlap them: a bf16 tile one 16-byte piece per k-step
            // pair, an FP8 tile (dequantized here) before the products; then
            // tile it + 2 is requested.  The other buffer was last read in the
            // previous iteration, which every wave finished before that
            // iteration's barrier
            if constexpr (KV8) {
                if (it + 1 < ntiles) {
                    ISA_HW_STORE((it + 1) & 1)
                    if (it + 2 < ntiles) ISA_HW_LOAD(it + 2)
                }
            }
            char* const lnext = &tiles[(it + 1) & 1][0] + lrow_off + gsub * 16;
            const char* tb = &tiles[it & 1][0];
            // ---- S^T: rows j (block 0) and 16 + j (block 1), dims 32ks + 8g ..;
            // the A operands of k-step pair p + 2 are requested before the
            // products of pair p
            const char* a0p = tb + heads_slot(j) * ROWB + 16 * g;
            const char* a1p = tb + heads_slot(16 + j) * ROWB + 16 * g;
            v4f s00 = {0.0f, 0.0f, 0.0f, 0.0f}, s01 = s00, s10 = s00, s11 = s00;
            v8bf A[3][4];
            auto lda = [&](int p, v8bf (&d)[4]) {
                d[0] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(a0p + 128 * p));
                d[1] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(a1p + 128 * p));
                d[2] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(a0p + 128 * p + 64));
                d[3] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(a1p + 128 * p + 64));
            };
            lda(0, A[0]);
            lda(1, A[1]);
#pragma unroll
            for (int p = 0; p < KS / 2; ++p) {
                if (p + 2 < KS / 2) lda(p + 2, A[(p + 2) % 3]);
                __builtin_amdgcn_sched_barrier(0);
                const v8bf(&c)[4] = A[p % 3];
                s00 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c[0], qb[2 * p], s00, 0, 0, 0);
                s10 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c[1], qb[2 * p], s10, 0, 0, 0);
                s01 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c[2], qb[2 * p + 1], s01, 0, 0, 0);
                s11 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c[3], qb[2 * p + 1], s11, 0, 0, 0);
                if constexpr (!KV8) {
                    static_assert(KV8 || GPT == KS / 2, "one tile piece per k-step pair");
                    if (it + 1 < ntiles && (CH % TPR == 0 || gsub + TPR * p < CH))
                        *reinterpret_cast<v4u*>(lnext + p * TPR * 16) = r[p];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (!KV8) {
                if (it + 2 < ntiles) ISA_HW_LOAD(it + 2)
            }
            // the V^T operands of the first value blocks, requested while the
            // scores finish: lane (g, j) supplies row 4g + j/4 (and 16 + 4g +
            // j/4), columns 16nb + 4(j%4) .. +4, and receives column 16nb + j of
            // rows 4g .. 4g+3 (and 16 + 4g ..)
            const char* vlo = tb + heads_slot(4 * g + (j >> 2)) * ROWB + 8 * (j & 3);
            const char* vhi = tb + heads_slot(16 + 4 * g + (j >> 2)) * ROWB + 8 * (j & 3);
            constexpr int VD = 4;                      // value blocks requested ahead
            v4bf VL[VD], VH[VD];
#pragma unroll
            for (int nb = 0; nb < VD; ++nb) {
                VL[nb] = lds_read_tr(vlo, 32 * nb);
                VH[nb] = lds_read_tr(vhi, 32 * nb);
            }
            v4f s0 = s00 + s01, s1 = s10 + s11;        // rows 4g + i and 16 + 4g + i of head j
            const uint32_t tm = tmask[it];
            if (tm != 0xFFFFFFFFu) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!((tm >> (4 * g + i)) & 1u)) s0[i] = -__builtin_inff();
                    if (!((tm >> (16 + 4 * g + i)) & 1u)) s1[i] = -__builtin_inff();
                }
            }
            float mloc = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                               fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
            mloc = xor32_max(xor16_max(mloc)) * scale_log2;   // scale > 0 keeps the order
            if constexpr (EXACT) {
                const bool move = mloc > m_run + RESCALE_SLACK;
                if (__ballot(move)) {
                    const float m_new = move ? mloc : m_run;
                    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                    m_run = m_new;
                    l_own *= alpha;
#pragma unroll
                    for (int nb = 0; nb < NBV; ++nb) o[nb] *= alpha;
                }
            } else {
                // the accumulators are still zero when the reference is first set
                if (m_run == -__builtin_inff()) m_run = mloc;
                bad = bad || mloc > m_run + HW_HEADROOM;
            }
            const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
            v8bf pk;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[i], scale_log2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s1[i], scale_log2, -m_use));
                psum += p0;
                psum += p1;
                pk[i] = (__bf16)p0;
                pk[4 + i] = (__bf16)p1;
            }
            l_own += psum;
            // ---- O^T += V^T . P^T, the operands of block nb + VD requested
            // before the product of block nb
#pragma unroll
            for (int nb = 0; nb < NBV; ++nb) {
                const v4bf lo = VL[nb % VD], hi = VH[nb % VD];
                if (nb + VD < NBV) {
                    VL[nb % VD] = lds_read_tr(vlo, 32 * (nb + VD));
                    VH[nb % VD] = lds_read_tr(vhi, 32 * (nb + VD));
                }
                __builtin_amdgcn_sched_barrier(0);
                const v8bf av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pk, o[nb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (it + 1 < ntiles) lds_barrier();   // tile it + 1 visible, tile it read
        }
    };
    pass(std::false_type{});
    // a head whose scores rose far above its first tile's: every wave runs the
    // query again with exact references (the tile barriers need all of them)
    if (bad) atomicOr(&s_bad, 1u);
    lds_barrier();
    if (s_bad) {
        lds_barrier();                 // every wave has read the flag and left the tiles
        pass(std::true_type{});
    }
#undef ISA_HW_LOAD
#undef ISA_HW_STORE

    // the softmax sum of head j over all rows: the four lane groups
    const float l_tot = xor32_sum(xor16_sum(l_own));
    if (!head_ok) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    // o[nb] lane (g, j) element i: column 16nb + 4g + i of head j
    uint16_t* orow = out + ((size_t)q * H + head) * DV + 4 * g;
#pragma unroll
    for (int nb = 0; nb < NBV; ++nb) {
        ushort4 v;
        v.x = f2bf(o[nb][0] * inv);
        v.y = f2bf(o[nb][1] * inv);
        v.z = f2bf(o[nb][2] * inv);
        v.w = f2bf(o[nb][3] * inv);
        *reinterpret_cast<ushort4*>(orow + 16 * nb) = v;
    }
    if (lse && g == 0)
        lse[(size_t)q * H + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * LN2 : -__builtin_inff();
}

// The latent cache: bf16 rows (C), or FP8 codes, exponents and bf16 RoPE
// slices (C8, Ce, Cr).
struct KvSrc {
    const uint16_t* C;
    const uint8_t* C8;
    const uint8_t* Ce;
    const uint16_t* Cr;
};

template <int HB, int VS, int D, int DV, int GR, bool KV8>
hipError_t launch_attend(const uint16_t* Q, KvSrc kv, const int32_t* idx, int B, int Tq,
                         int H, int L_cap, int k, float sm_scale, uint16_t* out, float* lse,
                         void* partials, hipStream_t stream, PageMap pm) {
    const AttendPlan plan = attend_plan(B, Tq, H, D, DV, k);
    const int nq = B * Tq;
    char* base = static_cast<char*>(partials);
    uint16_t* part_o = reinterpret_cast<uint16_t*>(base + plan.part_o_off);
    float2* part_ml = reinterpret_cast<float2*>(base + plan.part_ml_off);
    const int n_hbg = (H + 32 * HB - 1) / (32 * HB);
    const int nz = n_hbg * VS;
    const int items = nq * plan.splits * nz;
    const int per_xcd = (items + 7) / 8;
    hipLaunchKernelGGL((sparse_attend_kernel<HB, VS, D, DV, GR, KV8>), dim3(8 * per_xcd),
                       dim3(AT_THREADS * GR), 0, stream, Q, kv.C, kv.C8, kv.Ce, kv.Cr, idx, Tq, H,
                       L_cap, k, sm_scale * LOG2E, plan.slots_per_split, plan.splits, nq, nz,
                       per_xcd, out, lse, part_o, part_ml, pm);
    if (plan.splits > 1)
    {
        using Gm = AttendGeom<HB, VS, D, DV, GR>;
        const size_t threads = (size_t)nq * n_hbg * VS * 4 * Gm::NB * 4 * 64;
        const int mwg = (int)((threads + MERGE_THREADS - 1) / MERGE_THREADS);
        const int mper = (mwg + 7) / 8;
        // the merge issues one load per split it may combine: as few as the
        // call has
        auto merge = [&](auto ms_tag) {
            constexpr int MS = decltype(ms_tag)::value;
            hipLaunchKernelGGL((merge_splits_kernel<DV, VS, HB, Gm::NB, Gm::CW, MS>),
                               dim3(8 * mper), dim3(MERGE_THREADS), 0, stream, part_o, part_ml,
                               nq, H, n_hbg, plan.splits, mper, out, lse);
        };
        static_assert(MAX_SPLITS == 16, "merge variants for up to 16 splits");
        if (plan.splits <= 2) merge(std::integral_constant<int, 2>{});
        else if (plan.splits <= 4) merge(std::integral_constant<int, 4>{});
        else if (plan.splits <= 8) merge(std::integral_constant<int, 8>{});
        else merge(std::integral_constant<int, 16>{});
    }
    return hipGetLastError();
}

}  // namespace

AttendPlan attend_plan(int B, int Tq, int H, int D, int D_v, int k) {
    AttendPlan p;
    const int nq = B * Tq;
    // many queries: one workgroup per query holds both 32-head blocks and
    // every value column; few queries (decode): one 32-head block per
    // workgroup, two groups of 4 waves on alternate tiles (the two blocks'
    // gathers of a row meet in L2), and the k slots split across workgroups
    const bool wide = nq >= 256 || D != 576;
    p.head_blocks = wide ? 2 : 1;
    p.col_parts = 1;
    const int n_hbg = (H + 32 * p.head_blocks - 1) / (32 * p.head_blocks);
    const int units = nq * n_hbg * p.col_parts;
    const int tiles = (k + TILE_ROWS - 1) / TILE_ROWS;
    // one workgroup per CU (256 CUs): the decode variant's workgroup holds two
    // groups of 4 waves
    const int target = 256;
    int splits = units >= target ? 1 : (target + units - 1) / units;
    if (splits > MAX_SPLITS) splits = MAX_SPLITS;
    if (splits > tiles) splits = tiles;
    const int tiles_per_split = (tiles + splits - 1) / splits;
    splits = (tiles + tiles_per_split - 1) / tiles_per_split;
    p.splits = splits;
    p.slots_per_split = tiles_per_split * TILE_ROWS;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    // partial outputs cover every head slot of the workgroups (32 * head_blocks
    // per head-block group), bf16
    p.part_o_off = take(splits > 1 ? (size_t)nq * splits * n_hbg * 32 * p.head_blocks * D_v * 2 : 0);
    p.part_ml_off = take(splits > 1 ? (size_t)nq * splits * p.col_parts * H * 8 : 0);
    p.partial_bytes = off;
    return p;
}

bool attend_shape_supported(int H, int D, int D_v) {
    if (D == 576 && D_v == 512) return H >= 1 && H <= 64;
    if (D == 160 && D_v == 128) return H >= 1 && H <= 64;
    return false;
}

namespace {

template <bool KV8>
hipError_t dispatch_attend(const uint16_t* Q, KvSrc kv, const int32_t* idx, int B, int Tq, int H,
                           int D, int D_v, int L_cap, int k, float sm_scale, uint16_t* out,
                           float* lse, void* partials, hipStream_t stream, PageMap pm) {
    const AttendPlan plan = attend_plan(B, Tq, H, D, D_v, k);
    if (D == 576 && D_v == 512) {
        if (plan.head_blocks == 2 && plan.splits == 1 && k <= MAX_SPLIT_SLOTS) {
            // many queries: one four-wave workgroup per query, 16 heads per wave
            const int nq = B * Tq;
            const int per_xcd = (nq + 7) / 8;
            hipLaunchKernelGGL((attend_heads_kernel<576, 512, KV8>), dim3(8 * per_xcd),
                               dim3(HW_THREADS), 0, stream, Q, kv.C, kv.C8, kv.Ce, kv.Cr, idx, Tq,
                               H, L_cap, k, sm_scale * LOG2E, nq, per_xcd, out, lse, pm);
            return hipGetLastError();
        }
        if (plan.head_blocks == 2)
            return launch_attend<2, 1, 576, 512, 1, KV8>(Q, kv, idx, B, Tq, H, L_cap, k, sm_scale,
                                                         out, lse, partials, stream, pm);
        return launch_attend<1, 1, 576, 512, 2, KV8>(Q, kv, idx, B, Tq, H, L_cap, k, sm_scale, out,
                                                     lse, partials, stream, pm);
    }
    if (D == 160 && D_v == 128)
        return launch_attend<2, 1, 160, 128, 1, KV8>(Q, kv, idx, B, Tq, H, L_cap, k, sm_scale, out,
                                                     lse, partials, stream, pm);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx,
                                    int B, int Tq, int H, int D, int D_v, int L_cap, int k,
                                    float sm_scale, uint16_t* out, float* lse, void* partials,
                                    hipStream_t stream, PageMap pm) {
    return dispatch_attend<false>(Q, KvSrc{C, nullptr, nullptr, nullptr}, idx, B, Tq, H, D, D_v,
                                  L_cap, k, sm_scale, out, lse, partials, stream, pm);
}

hipError_t launch_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                        const uint16_t* Cr, const int32_t* idx, int B, int Tq,
                                        int H, int D, int D_v, int L_cap, int k, float sm_scale,
                                        uint16_t* out, float* lse, void* partials,
                                        hipStream_t stream, PageMap pm) {
    return dispatch_attend<true>(Q, KvSrc{nullptr, C8, Ce, Cr}, idx, B, Tq, H, D, D_v, L_cap, k,
                                 sm_scale, out, lse, partials, stream, pm);
}

}  // namespace isa
