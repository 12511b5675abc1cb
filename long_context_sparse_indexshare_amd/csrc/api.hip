// C ABI of libisa: host-side argument checks, workspace carving, and the
// IndexShare group driver.  The group rule follows "GLM-5.2 技术报告解读"
// section 1 (training-strategy table: the indexer runs in the first of every
// four sparse layers and the other three reuse its top-k) and "GLM-5.2
// Explained: 1M Token Context AI Agent Model" section 2.1 (compute the index
// set, or reuse the previous one) and 2.2.1 (later MTP draft steps reuse the
// first step's set).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/isa.h"
#include "isa_internal.h"

namespace {

thread_local std::string g_last_error;

isa_status fail(isa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
isa_status fail(isa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

isa_status ok() {
    g_last_error.clear();
    return ISA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define ISA_CHECK(cond, st, ...) \
    do {                         \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

isa_status check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ISA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

isa_status check_indexer(const int8_t* qI, const float* w, const int8_t* kI, const int32_t* kv_len,
                         int B, int Tq, int H_I, int D_I, int L_cap, const float* S) {
    ISA_CHECK(qI && w && kI && kv_len && S, ISA_ERR_INVALID_ARG, "indexer: NULL tensor pointer");
    ISA_CHECK(B > 0 && Tq > 0 && H_I > 0 && D_I > 0 && L_cap > 0, ISA_ERR_INVALID_ARG,
              "indexer: sizes must be positive (B=%d Tq=%d H_I=%d D_I=%d L_cap=%d)", B, Tq, H_I,
              D_I, L_cap);
    ISA_CHECK(L_cap <= ISA_MAX_LCAP, ISA_ERR_INVALID_ARG, "indexer: L_cap=%d exceeds %d", L_cap,
              ISA_MAX_LCAP);
    ISA_CHECK(isa::indexer_shape_supported(H_I, D_I), ISA_ERR_UNSUPPORTED,
              "indexer: (H_I=%d, D_I=%d) not compiled; H_I in {4,8,16,32,64}, D_I in {32,64,128}",
              H_I, D_I);
    ISA_CHECK(aligned(qI, 16) && aligned(kI, 16) && aligned(w, 4) && aligned(S, 4) &&
                  aligned(kv_len, 4),
              ISA_ERR_INVALID_ARG, "indexer: qI and kI need 16-byte alignment");
    return ISA_OK;
}

isa_status check_topk(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap, int k,
                      const int32_t* idx) {
    ISA_CHECK(S && kv_len && idx, ISA_ERR_INVALID_ARG, "topk: NULL tensor pointer");
    ISA_CHECK(B > 0 && Tq > 0 && L_cap > 0, ISA_ERR_INVALID_ARG,
              "topk: sizes must be positive (B=%d Tq=%d L_cap=%d)", B, Tq, L_cap);
    ISA_CHECK(k >= 1 && k <= ISA_MAX_TOPK, ISA_ERR_INVALID_ARG, "topk: k=%d outside [1, %d]", k,
              ISA_MAX_TOPK);
    ISA_CHECK(L_cap <= ISA_MAX_LCAP, ISA_ERR_INVALID_ARG, "topk: L_cap=%d exceeds %d", L_cap,
              ISA_MAX_LCAP);
    ISA_CHECK((long long)B * Tq <= 65535, ISA_ERR_UNSUPPORTED, "topk: B*Tq=%lld exceeds 65535",
              (long long)B * Tq);
    ISA_CHECK(aligned(S, 4) && aligned(idx, 4) && aligned(kv_len, 4), ISA_ERR_INVALID_ARG,
              "topk: misaligned pointer");
    return ISA_OK;
}

// C: the bf16 cache, or (fp8) any non-NULL stand-in when the FP8 arrays are
// checked separately by check_kv8
isa_status check_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx, int B, int Tq,
                        int H, int D, int D_v, int L_cap, int k, float sm_scale,
                        const uint16_t* out) {
    ISA_CHECK(Q && C && idx && out, ISA_ERR_INVALID_ARG, "attend: NULL tensor pointer");
    ISA_CHECK(B > 0 && Tq > 0 && H > 0 && D > 0 && D_v > 0 && L_cap > 0, ISA_ERR_INVALID_ARG,
              "attend: sizes must be positive (B=%d Tq=%d H=%d D=%d D_v=%d L_cap=%d)", B, Tq, H, D,
              D_v, L_cap);
    ISA_CHECK(k >= 1 && k <= ISA_MAX_TOPK, ISA_ERR_INVALID_ARG, "attend: k=%d outside [1, %d]", k,
              ISA_MAX_TOPK);
    ISA_CHECK(L_cap <= ISA_MAX_LCAP, ISA_ERR_INVALID_ARG, "attend: L_cap=%d exceeds %d", L_cap,
              ISA_MAX_LCAP);
    ISA_CHECK(std::isfinite(sm_scale) && sm_scale > 0.0f, ISA_ERR_INVALID_ARG,
              "attend: sm_scale must be finite and positive (got %g)", (double)sm_scale);
    ISA_CHECK(isa::attend_shape_supported(H, D, D_v), ISA_ERR_UNSUPPORTED,
              "attend: (H=%d, D=%d, D_v=%d) not compiled; (D, D_v) in {(576,512), (160,128)}, "
              "H <= 64",
              H, D, D_v);
    ISA_CHECK((long long)B * Tq <= 65535, ISA_ERR_UNSUPPORTED, "attend: B*Tq=%lld exceeds 65535",
              (long long)B * Tq);
    ISA_CHECK(aligned(Q, 16) && aligned(C, 16) && aligned(out, 16) && aligned(idx, 4),
              ISA_ERR_INVALID_ARG, "attend: Q, C and out need 16-byte alignment");
    return ISA_OK;
}

isa_status check_kv8(const uint8_t* C8, const uint8_t* Ce, const uint16_t* Cr) {
    ISA_CHECK(C8 && Ce && Cr, ISA_ERR_INVALID_ARG, "attend fp8: NULL cache pointer");
    ISA_CHECK(aligned(C8, 16) && aligned(Cr, 16), ISA_ERR_INVALID_ARG,
              "attend fp8: C8 and Cr need 16-byte alignment");
    return ISA_OK;
}

// Shapes of the FP8 variant, as (D, D_v) of the bf16 one.
bool kv8_shape_supported(int D_c, int D_r) {
    return (D_c == 512 && D_r == 64) || (D_c == 128 && D_r == 32);
}

// Page geometry of the paged calls; on success *pm describes it.
isa_status check_pages(const int32_t* table, int max_blocks, int block_size, int n_pages,
                       isa::PageMap* pm) {
    ISA_CHECK(table && aligned(table, 4), ISA_ERR_INVALID_ARG, "paged: NULL or misaligned table");
    ISA_CHECK(max_blocks > 0 && n_pages > 0, ISA_ERR_INVALID_ARG,
              "paged: max_blocks=%d and n_pages=%d must be positive", max_blocks, n_pages);
    int shift = 5;
    while (shift < 16 && (1 << shift) < block_size) ++shift;
    ISA_CHECK(block_size == (1 << shift), ISA_ERR_INVALID_ARG,
              "paged: block_size=%d is not a power of two in [32, 65536]", block_size);
    ISA_CHECK((long long)n_pages * block_size < (1LL << 31), ISA_ERR_INVALID_ARG,
              "paged: n_pages * block_size must stay below 2^31");
    ISA_CHECK((long long)max_blocks * block_size <= ISA_MAX_LCAP, ISA_ERR_INVALID_ARG,
              "paged: max_blocks * block_size exceeds %d", ISA_MAX_LCAP);
    *pm = isa::PageMap{table, max_blocks, shift, n_pages};
    return ISA_OK;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Group workspace: [top-k counters | top-k scratch | scores S | attention
// partials]; the counters are zeroed by one fill kernel at the start of a call.
struct GroupLayout {
    size_t topk, topk_zero_bytes, scores, attend, total;
    bool need_index;
};

GroupLayout group_layout(const isa_group_args* a) {
    GroupLayout L;
    L.need_index = !a->reuse_idx || a->per_layer_indexer;
    const size_t rows = (size_t)a->B * a->Tq;
    const isa::AttendPlan ap = isa::attend_plan(a->B, a->Tq, a->H, a->D, a->D_v, a->k);
    size_t off = 0;
    L.topk = off;
    L.topk_zero_bytes = 0;
    if (L.need_index) {
        const isa::TopkLayout tl = isa::topk_layout((int)rows, a->L_cap, a->k,
                                                    isa::indexer_writes_summary(a->Tq, a->H_I));
        L.topk_zero_bytes = tl.zero_bytes;           // the counters come first
        off += round_up(tl.total);
    }
    L.scores = off;
    off += L.need_index ? round_up(rows * (size_t)a->L_cap * sizeof(float)) : 0;
    L.attend = off;
    off += round_up(ap.partial_bytes);
    L.total = off;
    return L;
}

}  // namespace

// Scratch memory of isa_group_forward_noalloc: one fixed array in the code
// object, so the call allocates nothing.  Every GPU the library runs on holds
// its own copy of it (until the process ends), at its own address.  In host
// code the name `scratch` is only a host-side stand-in: the device address of
// the current GPU's copy comes from hipGetSymbolAddress, once per device, and
// only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[ISA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device), or an error status.
isa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ISA_ERR_HIP, "noalloc: hipGetDevice: %s", hipGetErrorString(e));
    ISA_CHECK(dev >= 0 && dev < MAX_DEVICES, ISA_ERR_UNSUPPORTED, "noalloc: device %d beyond %d",
              dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(ISA_ERR_HIP, "noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ISA_OK;
}

}  // namespace

extern "C" {

int isa_abi_version(void) { return ISA_ABI_VERSION; }

const char* isa_last_error(void) { return g_last_error.c_str(); }

isa_status isa_indexer_scores(const int8_t* qI, const float* w, const int8_t* kI,
                              const int32_t* kv_len, int B, int Tq, int H_I, int D_I, int L_cap,
                              float* S, void* stream) {
    isa_status st = check_indexer(qI, w, kI, kv_len, B, Tq, H_I, D_I, L_cap, S);
    if (st != ISA_OK) return st;
    return check_hip(isa::launch_indexer_scores(qI, w, kI, kv_len, B, Tq, H_I, D_I, L_cap, S,
                                                nullptr, 0, static_cast<hipStream_t>(stream)),
                     "indexer launch");
}

isa_status isa_indexer_scores_paged(const int8_t* qI, const float* w, const int8_t* kI_pages,
                                    const int32_t* block_table, int max_blocks, int block_size,
                                    int n_pages, const int32_t* kv_len, int B, int Tq, int H_I,
                                    int D_I, float* S, void* stream) {
    isa::PageMap pm;
    isa_status st = check_pages(block_table, max_blocks, block_size, n_pages, &pm);
    if (st != ISA_OK) return st;
    const int L_cap = max_blocks * block_size;
    st = check_indexer(qI, w, kI_pages, kv_len, B, Tq, H_I, D_I, L_cap, S);
    if (st != ISA_OK) return st;
    return check_hip(isa::launch_indexer_scores(qI, w, kI_pages, kv_len, B, Tq, H_I, D_I, L_cap, S,
                                                nullptr, 0, static_cast<hipStream_t>(stream), pm),
                     "indexer launch");
}

size_t isa_topk_workspace_bytes(int B, int Tq, int L_cap, int k) {
    if (B <= 0 || Tq <= 0 || L_cap <= 0 || k <= 0) return 0;
    return isa::topk_layout(B * Tq, L_cap, k).total;
}

isa_status isa_topk_select(const float* S, const int32_t* kv_len, int B, int Tq, int L_cap, int k,
                           int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    isa_status st = check_topk(S, kv_len, B, Tq, L_cap, k, idx);
    if (st != ISA_OK) return st;
    const size_t need = isa_topk_workspace_bytes(B, Tq, L_cap, k);
    ISA_CHECK(need == 0 || (ws && ws_bytes >= need && aligned(ws, 256)), ISA_ERR_WORKSPACE,
              "topk: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
    return check_hip(isa::launch_topk_select(S, kv_len, B, Tq, L_cap, k, idx, ws, false,
                                             static_cast<hipStream_t>(stream)),
                     "topk launch");
}

size_t isa_attend_workspace_bytes(int B, int Tq, int H, int D, int D_v, int k) {
    if (B <= 0 || Tq <= 0 || H <= 0 || D <= 0 || D_v <= 0 || k <= 0) return 0;
    return isa::attend_plan(B, Tq, H, D, D_v, k).partial_bytes;
}

isa_status isa_sparse_mla_attend(const uint16_t* Q, const uint16_t* C, const int32_t* idx, int B,
                                 int Tq, int H, int D, int D_v, int L_cap, int k, float sm_scale,
                                 uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                 void* stream) {
    isa_status st = check_attend(Q, C, idx, B, Tq, H, D, D_v, L_cap, k, sm_scale, out);
    if (st != ISA_OK) return st;
    ISA_CHECK(!lse || aligned(lse, 4), ISA_ERR_INVALID_ARG, "attend: misaligned lse");
    const size_t need = isa_attend_workspace_bytes(B, Tq, H, D, D_v, k);
    if (need) {
        ISA_CHECK(ws && ws_bytes >= need && aligned(ws, 256), ISA_ERR_WORKSPACE,
                  "attend: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
    }
    return check_hip(isa::launch_sparse_mla_attend(Q, C, idx, B, Tq, H, D, D_v, L_cap, k, sm_scale,
                                                   out, lse, ws, static_cast<hipStream_t>(stream)),
                     "attend launch");
}

isa_status isa_sparse_mla_attend_paged(const uint16_t* Q, const uint16_t* C_pages,
                                       const int32_t* block_table, int max_blocks,
                                       int block_size, int n_pages, const int32_t* idx, int B,
                                       int Tq, int H, int D, int D_v, int k, float sm_scale,
                                       uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                       void* stream) {
    isa::PageMap pm;
    isa_status st = check_pages(block_table, max_blocks, block_size, n_pages, &pm);
    if (st != ISA_OK) return st;
    const int L_cap = max_blocks * block_size;
    st = check_attend(Q, C_pages, idx, B, Tq, H, D, D_v, L_cap, k, sm_scale, out);
    if (st != ISA_OK) return st;
    ISA_CHECK(!lse || aligned(lse, 4), ISA_ERR_INVALID_ARG, "attend: misaligned lse");
    const size_t need = isa_attend_workspace_bytes(B, Tq, H, D, D_v, k);
    if (need) {
        ISA_CHECK(ws && ws_bytes >= need && aligned(ws, 256), ISA_ERR_WORKSPACE,
                  "attend: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
    }
    return check_hip(isa::launch_sparse_mla_attend(Q, C_pages, idx, B, Tq, H, D, D_v, L_cap, k,
                                                   sm_scale, out, lse, ws,
                                                   static_cast<hipStream_t>(stream), pm),
                     "attend launch");
}

size_t isa_attend_fp8_workspace_bytes(int B, int Tq, int H, int D_c, int D_r, int k) {
    if (D_c <= 0 || D_r <= 0) return 0;
    return isa_attend_workspace_bytes(B, Tq, H, D_c + D_r, D_c, k);
}

isa_status isa_sparse_mla_attend_fp8(const uint16_t* Q, const uint8_t* C8, const uint8_t* Ce,
                                     const uint16_t* Cr, const int32_t* idx, int B, int Tq, int H,
                                     int D_c, int D_r, int L_cap, int k, float sm_scale,
                                     uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream) {
    ISA_CHECK(kv8_shape_supported(D_c, D_r), ISA_ERR_UNSUPPORTED,
              "attend fp8: (D_c=%d, D_r=%d) not compiled; (512, 64) or (128, 32)", D_c, D_r);
    isa_status st = check_kv8(C8, Ce, Cr);
    if (st != ISA_OK) return st;
    st = check_attend(Q, Cr, idx, B, Tq, H, D_c + D_r, D_c, L_cap, k, sm_scale, out);
    if (st != ISA_OK) return st;
    ISA_CHECK(!lse || aligned(lse, 4), ISA_ERR_INVALID_ARG, "attend fp8: misaligned lse");
    const size_t need = isa_attend_fp8_workspace_bytes(B, Tq, H, D_c, D_r, k);
    if (need) {
        ISA_CHECK(ws && ws_bytes >= need && aligned(ws, 256), ISA_ERR_WORKSPACE,
                  "attend fp8: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                  ws_bytes);
    }
    return check_hip(isa::launch_sparse_mla_attend_fp8(Q, C8, Ce, Cr, idx, B, Tq, H, D_c + D_r,
                                                       D_c, L_cap, k, sm_scale, out, lse, ws,
                                                       static_cast<hipStream_t>(stream)),
                     "attend fp8 launch");
}

isa_status isa_index_histogram(const int32_t* idx, int B, int Tq, int k, int L_cap,
                               uint32_t* counts, void* stream) {
    ISA_CHECK(idx && counts, ISA_ERR_INVALID_ARG, "histogram: NULL tensor pointer");
    ISA_CHECK(B > 0 && Tq > 0 && L_cap > 0, ISA_ERR_INVALID_ARG,
              "histogram: sizes must be positive (B=%d Tq=%d L_cap=%d)", B, Tq, L_cap);
    ISA_CHECK(k >= 1 && k <= ISA_MAX_TOPK, ISA_ERR_INVALID_ARG, "histogram: k=%d outside [1, %d]",
              k, ISA_MAX_TOPK);
    ISA_CHECK(L_cap <= ISA_MAX_LCAP, ISA_ERR_INVALID_ARG, "histogram: L_cap=%d exceeds %d", L_cap,
              ISA_MAX_LCAP);
    ISA_CHECK(aligned(idx, 16) && aligned(counts, 4), ISA_ERR_INVALID_ARG,
              "histogram: idx needs 16-byte alignment, counts 4-byte");
    return check_hip(isa::launch_index_histogram(idx, B, Tq, k, L_cap, counts,
                                                 static_cast<hipStream_t>(stream)),
                     "histogram launch");
}

size_t isa_group_workspace_bytes(const isa_group_args* a) {
    if (!a || a->B <= 0 || a->Tq <= 0 || a->L_cap <= 0 || a->H <= 0 || a->D_v <= 0 || a->k <= 0)
        return 0;
    return group_layout(a).total;
}

// Checks every argument of a group call except the workspace; on success
// *pm describes the page geometry (or none) and *L the workspace layout.
static isa_status check_group(const isa_group_args* a, isa::PageMap* pm, GroupLayout* L) {
    ISA_CHECK(a, ISA_ERR_INVALID_ARG, "group: NULL args");
    ISA_CHECK(a->n_layers >= 1 && a->n_layers <= 64, ISA_ERR_INVALID_ARG,
              "group: n_layers=%d outside [1, 64]", a->n_layers);
    const bool kv8 = a->kv_fp8 != 0;
    ISA_CHECK(a->Q && (kv8 ? (a->C8 && a->Ce && a->Cr) : a->C != nullptr) && a->out && a->idx &&
                  a->kv_len,
              ISA_ERR_INVALID_ARG, "group: NULL pointer array or tensor");
    if (kv8) {
        ISA_CHECK(kv8_shape_supported(a->D_v, a->D - a->D_v), ISA_ERR_UNSUPPORTED,
                  "group: FP8 cache with (D=%d, D_v=%d) not compiled", a->D, a->D_v);
    }
    *pm = isa::PageMap{nullptr, 0, 0, 0};
    if (a->paged) {
        isa_status st = check_pages(a->block_table, a->max_blocks, a->block_size, a->n_pages, pm);
        if (st != ISA_OK) return st;
        ISA_CHECK((long long)a->max_blocks * a->block_size == a->L_cap, ISA_ERR_INVALID_ARG,
                  "group: paged caches need L_cap = max_blocks * block_size (%d != %d * %d)",
                  a->L_cap, a->max_blocks, a->block_size);
    }
    const bool per_layer = a->per_layer_indexer != 0;
    const bool need_index = !a->reuse_idx || per_layer;
    const int n_ix = per_layer ? a->n_layers : (need_index ? 1 : 0);
    if (n_ix) {
        ISA_CHECK(a->qI && a->w && a->kI, ISA_ERR_INVALID_ARG, "group: NULL indexer arrays");
    }
    // the score buffer lives in the workspace: stand in an aligned non-NULL
    // address for it while checking the caller's tensors
    const float* ws_scores = reinterpret_cast<const float*>(256);
    for (int l = 0; l < n_ix; ++l) {
        isa_status st = check_indexer(a->qI[l], a->w[l], a->kI[l], a->kv_len, a->B, a->Tq, a->H_I,
                                      a->D_I, a->L_cap, ws_scores);
        if (st != ISA_OK) return st;
    }
    if (need_index) {
        isa_status st = check_topk(ws_scores, a->kv_len, a->B, a->Tq,
                                   a->L_cap, a->k, a->idx);
        if (st != ISA_OK) return st;
    }
    for (int l = 0; l < a->n_layers; ++l) {
        if (kv8) {
            isa_status st = check_kv8(a->C8[l], a->Ce[l], a->Cr[l]);
            if (st != ISA_OK) return st;
        }
        isa_status st = check_attend(a->Q[l], kv8 ? a->Cr[l] : a->C[l], a->idx, a->B, a->Tq, a->H,
                                     a->D, a->D_v, a->L_cap, a->k, a->sm_scale, a->out[l]);
        if (st != ISA_OK) return st;
        if (a->lse && a->lse[l]) {
            ISA_CHECK(aligned(a->lse[l], 4), ISA_ERR_INVALID_ARG, "group: misaligned lse[%d]", l);
        }
    }
    *L = group_layout(a);
    return ISA_OK;
}

// The launches of one group call on `stream`, with scratch memory at ws
// (L.total bytes, 256-byte aligned).
static isa_status launch_group(const isa_group_args* a, const isa::PageMap& pm,
                               const GroupLayout& L, char* ws, hipStream_t stream) {
    const bool kv8 = a->kv_fp8 != 0;
    const bool per_layer = a->per_layer_indexer != 0;
    float* S = reinterpret_cast<float*>(ws + L.scores);
    char* topk_ws = ws + L.topk;
    void* attend_ws = ws + L.attend;
    // with one query per sequence the indexer also writes the top-k summary
    const bool ix_summary = isa::indexer_writes_summary(a->Tq, a->H_I);
    const isa::TopkLayout tl = isa::topk_layout(a->B * a->Tq, a->L_cap, a->k, ix_summary);
    const bool fused_summary = L.need_index && !tl.select && ix_summary;
    const isa::SummaryOut summary =
        fused_summary ? isa::SummaryOut{reinterpret_cast<uint32_t*>(topk_ws + tl.summary),
                                        reinterpret_cast<uint8_t*>(topk_ws + tl.codes), tl.M}
                      : isa::SummaryOut{nullptr, nullptr, 0};
    // each index set: the indexer grid also zeroes the top-k counters
    // (histograms, entry counts), then the top-k runs
    auto index = [&](int l) -> isa_status {
        isa_status st = check_hip(isa::launch_indexer_scores(a->qI[l], a->w[l], a->kI[l], a->kv_len,
                                                             a->B, a->Tq, a->H_I, a->D_I, a->L_cap,
                                                             S, reinterpret_cast<uint32_t*>(topk_ws),
                                                             (uint32_t)(L.topk_zero_bytes / 4),
                                                             stream, pm, summary),
                                  "group: indexer launch");
        if (st != ISA_OK) return st;
        return check_hip(isa::launch_topk_select(S, a->kv_len, a->B, a->Tq, a->L_cap, a->k, a->idx,
                                                 topk_ws, true, stream, fused_summary),
                         "group: topk launch");
    };
    if (L.need_index && !per_layer) {
        isa_status st = index(0);
        if (st != ISA_OK) return st;
    }
    for (int l = 0; l < a->n_layers; ++l) {
        if (per_layer) {
            isa_status st = index(l);
            if (st != ISA_OK) return st;
        }
        float* lse = a->lse ? a->lse[l] : nullptr;
        const hipError_t e =
            kv8 ? isa::launch_sparse_mla_attend_fp8(a->Q[l], a->C8[l], a->Ce[l], a->Cr[l], a->idx,
                                                    a->B, a->Tq, a->H, a->D, a->D_v, a->L_cap,
                                                    a->k, a->sm_scale, a->out[l], lse, attend_ws,
                                                    stream, pm)
                : isa::launch_sparse_mla_attend(a->Q[l], a->C[l], a->idx, a->B, a->Tq, a->H, a->D,
                                                a->D_v, a->L_cap, a->k, a->sm_scale, a->out[l],
                                                lse, attend_ws, stream, pm);
        isa_status st = check_hip(e, "group: attend launch");
        if (st != ISA_OK) return st;
    }
    return ok();
}

isa_status isa_group_forward(const isa_group_args* a, void* stream_v) {
    isa::PageMap pm;
    GroupLayout L;
    isa_status st = check_group(a, &pm, &L);
    if (st != ISA_OK) return st;
    ISA_CHECK(a->ws && a->ws_bytes >= L.total && aligned(a->ws, 256), ISA_ERR_WORKSPACE,
              "group: workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total, a->ws_bytes);
    return launch_group(a, pm, L, static_cast<char*>(a->ws), static_cast<hipStream_t>(stream_v));
}

size_t isa_group_noalloc_max_bytes(void) { return ISA_NOALLOC_SCRATCH_BYTES; }

isa_status isa_group_forward_noalloc(const isa_group_args* a, void* stream_v) {
    isa::PageMap pm;
    GroupLayout L;
    isa_status st = check_group(a, &pm, &L);
    if (st != ISA_OK) return st;
    ISA_CHECK(L.total <= (size_t)ISA_NOALLOC_SCRATCH_BYTES, ISA_ERR_WORKSPACE,
              "group noalloc: the call needs %zu bytes of scratch, above the fixed %zu",
              L.total, (size_t)ISA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != ISA_OK) return st;
    return launch_group(a, pm, L, static_cast<char*>(ws), static_cast<hipStream_t>(stream_v));
}

}  // extern "C"
