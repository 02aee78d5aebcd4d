// C ABI of libfa2mi: argument validation, then one launch on the caller's
// stream. Validation never touches the HIP runtime, so a rejected call has no
// side effect at all.
#include <atomic>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fa2mi.h"
#include "fa2_launch.h"

namespace {

thread_local char g_last_error[256] = "";

fa2_status fail(fa2_status st, const char *fn, const char *what) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", fn, what);
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool good_dtype(fa2_dtype dt) { return dt == FA2_F32 || dt == FA2_F16 || dt == FA2_BF16; }

bool good_dim(int64_t d) { return d == 32 || d == 64 || d == 128; }

#define REQUIRE_PTR(fn, p)                                                          \
    do {                                                                            \
        if ((p) == nullptr) return fail(FA2_ERR_INVALID_ARG, fn, #p " is NULL");    \
        if (!aligned16(p)) return fail(FA2_ERR_INVALID_ARG, fn, #p " is not 16-byte aligned"); \
    } while (0)

// Common checks of the attention entry points.
fa2_status check_attn(const char *fn, fa2_dtype dt, int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim,
                      float scale, int rows_per_block, int64_t grid_rows) {
    if (!good_dtype(dt)) return fail(FA2_ERR_INVALID_ARG, fn, "unknown dtype");
    if (bh <= 0 || n_q <= 0 || n_k <= 0 || head_dim <= 0)
        return fail(FA2_ERR_INVALID_ARG, fn, "bh, n_q, n_k and head_dim must all be > 0");
    if (!good_dim(head_dim)) return fail(FA2_ERR_UNSUPPORTED, fn, "head_dim must be 32, 64 or 128");
    // the kernels take the lengths as int; bounding them first also keeps
    // the byte count below within int64
    if (n_q > INT_MAX || n_k > INT_MAX) return fail(FA2_ERR_INVALID_ARG, fn, "n_q and n_k must be below 2^31");
    // One head's [n, head_dim] rows stay within 2 GiB, so the kernels' 32-bit
    // byte offsets (including a tile read past the last row) cannot wrap.
    const int64_t es = dt == FA2_F32 ? 4 : 2;
    if ((n_q > n_k ? n_q : n_k) * head_dim * es > (int64_t(1) << 31))
        return fail(FA2_ERR_INVALID_ARG, fn, "one head's rows exceed 2 GiB (n * head_dim * element size)");
    if (!(scale > 0.f) || scale == __builtin_inff())
        return fail(FA2_ERR_INVALID_ARG, fn, "scale must be positive and finite");
    const int64_t blocks = (grid_rows + rows_per_block - 1) / rows_per_block;
    if (bh > INT_MAX / blocks) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    return FA2_OK;
}

fa2_status launched(const char *fn, hipError_t e) {
    if (e != hipSuccess) return fail(FA2_ERR_LAUNCH, fn, hipGetErrorString(e));
    g_last_error[0] = '\0';
    return FA2_OK;
}

fa2_status check_psa(const char *fn, fa2_dtype dt, int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h,
                     int32_t w) {
    if (!good_dtype(dt)) return fail(FA2_ERR_INVALID_ARG, fn, "unknown dtype");
    if (batch <= 0 || num_heads <= 0 || key_dim <= 0 || h <= 0 || w <= 0)
        return fail(FA2_ERR_INVALID_ARG, fn, "batch, num_heads, key_dim, h and w must all be > 0");
    if (!good_dim(key_dim)) return fail(FA2_ERR_UNSUPPORTED, fn, "key_dim must be 32, 64 or 128");
    const int64_t hw = (int64_t)h * w;
    const int64_t slice_elems = hw * key_dim;
    if (slice_elems > INT_MAX) return fail(FA2_ERR_INVALID_ARG, fn, "h * w * key_dim exceeds 2^31 - 1");
    // generous bound on the workgroup count (tiles of >= 8 pixels)
    const int64_t tiles = (int64_t)batch * num_heads * 4 * ((hw + 7) / 8);
    if (tiles > INT_MAX) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    return FA2_OK;
}

}  // namespace

// Scratch of the allocation-free key-split forward: the float32 partial
// outputs and log2-sum-exps that fa2_fwd_splitkv keeps in a caller workspace.
// Every device the library runs on holds its own copy from the time the code
// object is loaded until the process ends. In host code `scratch` only names
// the symbol: its device address on the current device comes from
// hipGetSymbolAddress (taken once per device, then cached).
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev`, which must be current.
hipError_t scratch_ptr(int dev, void **out) {
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

namespace fa2mi {

SplitPlan plan_splitkv(int64_t bh, int64_t n_q, int64_t n_k, int head_dim, int requested) {
    SplitPlan p{};
    p.waves = n_q <= 64 ? 2 : n_q <= 128 ? 4 : 8;
    const int64_t rows = 32 * p.waves;
    const int64_t blocks = bh * ((n_q + rows - 1) / rows);
    const int64_t tiles = (n_k + kSplitKeyAlign - 1) / kSplitKeyAlign;
    int64_t want = requested;
    if (want <= 0) {
        // one workgroup per CU measured fastest (more ranges add prologue,
        // epilogue and combine work without more bandwidth)
        constexpr int64_t kTargetBlocks = 256, kMinKeys = 256;
        want = (kTargetBlocks + blocks - 1) / blocks;
        const int64_t cap = (n_k + kMinKeys - 1) / kMinKeys;
        if (want > cap) want = cap;
    }
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const int64_t per = (n_k + want - 1) / want;
    const int64_t len = (per + kSplitKeyAlign - 1) / kSplitKeyAlign * kSplitKeyAlign;
    p.split_len = (int)len;
    p.nsplit = (int)((n_k + len - 1) / len);
    if (p.nsplit == 1) {
        p.ws_bytes = 0;
    } else if (p.nsplit > INT_MAX / blocks || bh * n_q / 8 > INT_MAX) {
        p.ws_bytes = -1;  // the partial or the combine grid does not fit
    } else {
        p.ws_bytes = (int64_t)p.nsplit * bh * n_q * (head_dim + 1) * (int64_t)sizeof(float);
    }
    return p;
}

}  // namespace fa2mi

extern "C" {

int32_t fa2_abi_version(void) { return 1; }

const char *fa2_status_str(fa2_status s) {
    switch (s) {
        case FA2_OK: return "ok";
        case FA2_ERR_INVALID_ARG: return "invalid argument";
        case FA2_ERR_UNSUPPORTED: return "unsupported size";
        case FA2_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

const char *fa2_last_error(void) { return g_last_error; }

fa2_status fa2_fwd(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse, int64_t bh,
                   int64_t n_q, int64_t n_k, int32_t head_dim, float scale, void *stream) {
    static const char fn[] = "fa2_fwd";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, scale, fa2mi::kFwdRowsPerBlock, n_q);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, q);
    REQUIRE_PTR(fn, k);
    REQUIRE_PTR(fn, v);
    REQUIRE_PTR(fn, o);
    REQUIRE_PTR(fn, lse);
    const fa2mi::AttnShape s{bh, (int)n_q, (int)n_k, head_dim, scale};
    return launched(fn, fa2mi::launch_fwd((int)dt, q, k, v, o, lse, s, (hipStream_t)stream));
}

fa2_status fa2_fwd_splitkv_plan(fa2_dtype dt, int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim,
                                int32_t num_splits, int32_t *splits_used, int64_t *workspace_bytes) {
    static const char fn[] = "fa2_fwd_splitkv_plan";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, 1.f, fa2mi::kFwdRowsPerBlock, n_q);
    if (st != FA2_OK) return st;
    if (num_splits < 0) return fail(FA2_ERR_INVALID_ARG, fn, "num_splits must be >= 0 (0 picks it)");
    if (splits_used == nullptr || workspace_bytes == nullptr)
        return fail(FA2_ERR_INVALID_ARG, fn, "splits_used and workspace_bytes must not be NULL");
    const fa2mi::SplitPlan p = fa2mi::plan_splitkv(bh, n_q, n_k, head_dim, num_splits);
    if (p.ws_bytes < 0) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    *splits_used = p.nsplit;
    *workspace_bytes = p.ws_bytes;
    g_last_error[0] = '\0';
    return FA2_OK;
}

fa2_status fa2_fwd_splitkv(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse,
                           void *workspace, int64_t workspace_bytes, int64_t bh, int64_t n_q, int64_t n_k,
                           int32_t head_dim, float scale, int32_t num_splits, void *stream) {
    static const char fn[] = "fa2_fwd_splitkv";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, scale, fa2mi::kFwdRowsPerBlock, n_q);
    if (st != FA2_OK) return st;
    if (num_splits < 0) return fail(FA2_ERR_INVALID_ARG, fn, "num_splits must be >= 0 (0 picks it)");
    REQUIRE_PTR(fn, q);
    REQUIRE_PTR(fn, k);
    REQUIRE_PTR(fn, v);
    REQUIRE_PTR(fn, o);
    REQUIRE_PTR(fn, lse);
    const fa2mi::SplitPlan p = fa2mi::plan_splitkv(bh, n_q, n_k, head_dim, num_splits);
    if (p.ws_bytes < 0) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    if (p.ws_bytes > 0) {
        REQUIRE_PTR(fn, workspace);
        if (workspace_bytes < p.ws_bytes)
            return fail(FA2_ERR_INVALID_ARG, fn, "workspace_bytes is below the size fa2_fwd_splitkv_plan reports");
    }
    const fa2mi::AttnShape s{bh, (int)n_q, (int)n_k, head_dim, scale};
    return launched(fn, fa2mi::launch_fwd_splitkv((int)dt, q, k, v, o, lse, static_cast<float *>(workspace), s, p,
                                                  (hipStream_t)stream));
}

int64_t fa2_fwd_splitkv_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

fa2_status fa2_fwd_splitkv_noalloc(fa2_dtype dt, const void *q, const void *k, const void *v, void *o, float *lse,
                                   int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim, float scale,
                                   int32_t num_splits, void *stream) {
    static const char fn[] = "fa2_fwd_splitkv_noalloc";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, scale, fa2mi::kFwdRowsPerBlock, n_q);
    if (st != FA2_OK) return st;
    if (num_splits < 0) return fail(FA2_ERR_INVALID_ARG, fn, "num_splits must be >= 0 (0 picks it)");
    REQUIRE_PTR(fn, q);
    REQUIRE_PTR(fn, k);
    REQUIRE_PTR(fn, v);
    REQUIRE_PTR(fn, o);
    REQUIRE_PTR(fn, lse);
    const fa2mi::SplitPlan p = fa2mi::plan_splitkv(bh, n_q, n_k, head_dim, num_splits);
    if (p.ws_bytes < 0) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    if (p.ws_bytes > kNoAllocScratchBytes)
        return fail(FA2_ERR_INVALID_ARG, fn,
                    "partials exceed the 32 MiB static scratch (splits * bh * n_q * (head_dim + 1) * 4 bytes); "
                    "use fa2_fwd_splitkv with a workspace");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA2_ERR_LAUNCH, fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FA2_ERR_UNSUPPORTED, fn, "device index above 63");
    if (stream != nullptr) {
        int sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return fail(FA2_ERR_INVALID_ARG, fn, hipGetErrorString(e));
        if (sdev != dev) return fail(FA2_ERR_INVALID_ARG, fn, "stream does not belong to the current device");
    }
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        e = scratch_ptr(dev, &ws);
        if (e != hipSuccess) return fail(FA2_ERR_LAUNCH, fn, hipGetErrorString(e));
    }
    const fa2mi::AttnShape s{bh, (int)n_q, (int)n_k, head_dim, scale};
    return launched(fn, fa2mi::launch_fwd_splitkv((int)dt, q, k, v, o, lse, static_cast<float *>(ws), s, p,
                                                  (hipStream_t)stream));
}

fa2_status fa2_bwd_delta(fa2_dtype dt, const void *o, const void *d_o, float *delta, int64_t bh, int64_t n_q,
                         int32_t head_dim, void *stream) {
    static const char fn[] = "fa2_bwd_delta";
    fa2_status st = check_attn(fn, dt, bh, n_q, 1, head_dim, 1.f, 1 << 30, n_q);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, o);
    REQUIRE_PTR(fn, d_o);
    REQUIRE_PTR(fn, delta);
    const int64_t rows = bh * n_q;
    if (rows / 8 > INT_MAX) return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    return launched(fn, fa2mi::launch_bwd_delta((int)dt, o, d_o, delta, rows, head_dim, (hipStream_t)stream));
}

fa2_status fa2_bwd_dq(fa2_dtype dt, const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                      const float *delta, void *dq, int64_t bh, int64_t n_q, int64_t n_k, int32_t head_dim,
                      float scale, void *stream) {
    static const char fn[] = "fa2_bwd_dq";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, scale, fa2mi::kFwdRowsPerBlock, n_q);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, q);
    REQUIRE_PTR(fn, k);
    REQUIRE_PTR(fn, v);
    REQUIRE_PTR(fn, d_o);
    REQUIRE_PTR(fn, lse);
    REQUIRE_PTR(fn, delta);
    REQUIRE_PTR(fn, dq);
    const fa2mi::AttnShape s{bh, (int)n_q, (int)n_k, head_dim, scale};
    return launched(fn, fa2mi::launch_bwd_dq((int)dt, q, k, v, d_o, lse, delta, dq, s, (hipStream_t)stream));
}

fa2_status fa2_bwd_dkdv(fa2_dtype dt, const void *q, const void *k, const void *v, const void *d_o,
                        const float *lse, const float *delta, void *dk, void *dv, int64_t bh, int64_t n_q,
                        int64_t n_k, int32_t head_dim, float scale, void *stream) {
    static const char fn[] = "fa2_bwd_dkdv";
    fa2_status st = check_attn(fn, dt, bh, n_q, n_k, head_dim, scale, fa2mi::kDkdvKeysPerBlock, n_k);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, q);
    REQUIRE_PTR(fn, k);
    REQUIRE_PTR(fn, v);
    REQUIRE_PTR(fn, d_o);
    REQUIRE_PTR(fn, lse);
    REQUIRE_PTR(fn, delta);
    REQUIRE_PTR(fn, dk);
    REQUIRE_PTR(fn, dv);
    const fa2mi::AttnShape s{bh, (int)n_q, (int)n_k, head_dim, scale};
    return launched(fn, fa2mi::launch_bwd_dkdv((int)dt, q, k, v, d_o, lse, delta, dk, dv, s, (hipStream_t)stream));
}

fa2_status fa2_pad_cols(fa2_dtype dt, const void *src, void *dst, int64_t rows, int32_t d_src, int32_t d_dst,
                        void *stream) {
    static const char fn[] = "fa2_pad_cols";
    if (!good_dtype(dt)) return fail(FA2_ERR_INVALID_ARG, fn, "unknown dtype");
    if (rows <= 0 || d_src <= 0 || d_dst <= 0) return fail(FA2_ERR_INVALID_ARG, fn, "rows, d_src and d_dst must be > 0");
    if ((rows + fa2mi::kPadColsRowsPerBlock - 1) / fa2mi::kPadColsRowsPerBlock > INT_MAX)
        return fail(FA2_ERR_INVALID_ARG, fn, "grid exceeds 2^31 - 1 workgroups");
    if ((int64_t)fa2mi::kPadColsRowsPerBlock * (d_src > d_dst ? d_src : d_dst) > INT_MAX)
        return fail(FA2_ERR_INVALID_ARG, fn, "row width too large");
    REQUIRE_PTR(fn, src);
    REQUIRE_PTR(fn, dst);
    return launched(fn, fa2mi::launch_pad_cols((int)dt, src, dst, rows, d_src, d_dst, (hipStream_t)stream));
}

fa2_status psa_pack_qkv(fa2_dtype dt, const void *qkv, void *packed, int32_t batch, int32_t num_heads,
                        int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_pack_qkv";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, qkv);
    REQUIRE_PTR(fn, packed);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_pack((int)dt, qkv, packed, s, (hipStream_t)stream));
}

fa2_status psa_merge_attn(fa2_dtype dt, const void *o_lo, const void *o_hi, void *out, int32_t batch,
                          int32_t num_heads, int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_merge_attn";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, o_lo);
    REQUIRE_PTR(fn, o_hi);
    REQUIRE_PTR(fn, out);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_merge((int)dt, o_lo, o_hi, out, s, (hipStream_t)stream));
}

fa2_status psa_merge_attn_backward(fa2_dtype dt, const void *d_out, void *d_o_lo, void *d_o_hi, int32_t batch,
                                   int32_t num_heads, int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_merge_attn_backward";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, d_out);
    REQUIRE_PTR(fn, d_o_lo);
    REQUIRE_PTR(fn, d_o_hi);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_merge_backward((int)dt, d_out, d_o_lo, d_o_hi, s, (hipStream_t)stream));
}

fa2_status psa_pack_qkv_backward(fa2_dtype dt, const void *d_packed, const void *d_qk_extra, void *d_qkv,
                                 int32_t batch, int32_t num_heads, int32_t key_dim, int32_t h, int32_t w,
                                 void *stream) {
    static const char fn[] = "psa_pack_qkv_backward";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, d_packed);
    if (d_qk_extra != nullptr) REQUIRE_PTR(fn, d_qk_extra);
    REQUIRE_PTR(fn, d_qkv);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_pack_backward((int)dt, d_packed, d_qk_extra, d_qkv, s,
                                                         (hipStream_t)stream));
}

fa2_status psa_extract_v_nchw(fa2_dtype dt, const void *qkv, void *v, int32_t batch, int32_t num_heads,
                              int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_extract_v_nchw";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, qkv);
    REQUIRE_PTR(fn, v);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_extract_v((int)dt, qkv, v, s, (hipStream_t)stream));
}

fa2_status psa_extract_v_backward(fa2_dtype dt, const void *d_v, void *d_qkv, int32_t batch, int32_t num_heads,
                                  int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_extract_v_backward";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    REQUIRE_PTR(fn, d_v);
    REQUIRE_PTR(fn, d_qkv);
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_extract_v_backward((int)dt, d_v, d_qkv, s, (hipStream_t)stream));
}

fa2_status psa_attn_fused(fa2_dtype dt, const void *qkv, void *out, float *lse, int32_t batch,
                          int32_t num_heads, int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_attn_fused";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    if (dt == FA2_F32) return fail(FA2_ERR_UNSUPPORTED, fn, "dtype must be F16 or BF16");
    if (key_dim != 32 && key_dim != 64) return fail(FA2_ERR_UNSUPPORTED, fn, "key_dim must be 32 or 64");
    REQUIRE_PTR(fn, qkv);
    REQUIRE_PTR(fn, out);
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return fail(FA2_ERR_INVALID_ARG, fn, "lse is not 4-byte aligned");
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_fused((int)dt, qkv, out, lse, s, (hipStream_t)stream));
}

fa2_status psa_attn_fused_backward(fa2_dtype dt, const void *qkv, const void *out, const float *lse,
                                   const void *d_out, void *d_qkv, float *delta, int32_t batch, int32_t num_heads,
                                   int32_t key_dim, int32_t h, int32_t w, void *stream) {
    static const char fn[] = "psa_attn_fused_backward";
    fa2_status st = check_psa(fn, dt, batch, num_heads, key_dim, h, w);
    if (st != FA2_OK) return st;
    if (dt == FA2_F32) return fail(FA2_ERR_UNSUPPORTED, fn, "dtype must be F16 or BF16");
    if (key_dim != 32 && key_dim != 64) return fail(FA2_ERR_UNSUPPORTED, fn, "key_dim must be 32 or 64");
    if ((int64_t)h * w > fa2mi::psa_fused_bwd_max_pixels(key_dim))
        return fail(FA2_ERR_UNSUPPORTED, fn,
                    key_dim == 32 ? "h * w must be <= 512 at key_dim 32" : "h * w must be <= 128 at key_dim 64");
    REQUIRE_PTR(fn, qkv);
    REQUIRE_PTR(fn, out);
    REQUIRE_PTR(fn, d_out);
    REQUIRE_PTR(fn, d_qkv);
    if (lse == nullptr || delta == nullptr) return fail(FA2_ERR_INVALID_ARG, fn, "lse and delta must not be NULL");
    if (((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(delta)) & 3u) != 0)
        return fail(FA2_ERR_INVALID_ARG, fn, "lse and delta must be 4-byte aligned");
    const fa2mi::PsaShape s{batch, num_heads, key_dim, h * w};
    return launched(fn, fa2mi::launch_psa_fused_backward((int)dt, qkv, out, lse, d_out, d_qkv, delta, s,
                                                         (hipStream_t)stream));
}

}  // extern "C"
