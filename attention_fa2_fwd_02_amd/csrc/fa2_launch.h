// Host-side launch interface between the C ABI (fa2_abi.hip) and the kernel
// translation units. Arguments are already validated when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2mi {

struct AttnShape {
    int64_t bh;
    int n_q;
    int n_k;
    int head_dim;
    float scale;
};

// dt: 0 f32, 1 f16, 2 bf16 (the fa2_dtype values).
hipError_t launch_fwd(int dt, const void *q, const void *k, const void *v, void *o, float *lse,
                      const AttnShape &s, hipStream_t stream);

// Key-split forward plan: nsplit key ranges of split_len rows (the last may
// be shorter), workgroups of `waves` wavefronts (32 query rows each).
// nsplit == 1 runs the plain forward and needs no workspace.
struct SplitPlan {
    int nsplit;
    int split_len;
    int waves;
    int64_t ws_bytes;  // float32 partial outputs and log2-sum-exps
};
// Key ranges start on multiples of this many rows (the forward's key tile).
constexpr int kSplitKeyAlign = 64;
// Host-only (no HIP call). requested <= 0 picks the split count from the
// sizes: enough workgroups for one per CU of a 256-CU device, ranges of at
// least 256 keys.
SplitPlan plan_splitkv(int64_t bh, int64_t n_q, int64_t n_k, int head_dim, int requested);
hipError_t launch_fwd_splitkv(int dt, const void *q, const void *k, const void *v, void *o, float *lse, float *ws,
                              const AttnShape &s, const SplitPlan &sp, hipStream_t stream);
hipError_t launch_bwd_delta(int dt, const void *o, const void *d_o, float *delta, int64_t rows,
                            int head_dim, hipStream_t stream);
hipError_t launch_bwd_dq(int dt, const void *q, const void *k, const void *v, const void *d_o,
                         const float *lse, const float *delta, void *dq, const AttnShape &s,
                         hipStream_t stream);
hipError_t launch_bwd_dkdv(int dt, const void *q, const void *k, const void *v, const void *d_o,
                           const float *lse, const float *delta, void *dk, void *dv,
                           const AttnShape &s, hipStream_t stream);

// Row-major [rows, d_src] -> [rows, d_dst]: copy the first min(d_src, d_dst)
// columns, zero the rest (d_dst > d_src pads, d_dst < d_src crops).
hipError_t launch_pad_cols(int dt, const void *src, void *dst, int64_t rows, int d_src, int d_dst,
                           hipStream_t stream);
// Rows moved per workgroup of the column copy (the ABI bounds its grid).
constexpr int kPadColsRowsPerBlock = 16;

struct PsaShape {
    int batch;
    int num_heads;
    int key_dim;
    int hw;
};

hipError_t launch_psa_pack(int dt, const void *qkv, void *packed, const PsaShape &s, hipStream_t stream);
hipError_t launch_psa_merge(int dt, const void *lo, const void *hi, void *out, const PsaShape &s,
                            hipStream_t stream);
hipError_t launch_psa_fused(int dt, const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream);
hipError_t launch_psa_merge_backward(int dt, const void *d_out, void *d_lo, void *d_hi, const PsaShape &s,
                                     hipStream_t stream);
hipError_t launch_psa_pack_backward(int dt, const void *d_packed, const void *d_qk_extra, void *d_qkv,
                                    const PsaShape &s, hipStream_t stream);
// Fused block backward (key_dim 32 or 64, maps of at most
// psa_fused_bwd_max_pixels(key_dim) pixels): delta, then dQ, then dK/dV, all
// written into d_qkv. 0 for other key dims.
constexpr int psa_fused_bwd_max_pixels(int key_dim) { return key_dim == 32 ? 512 : key_dim == 64 ? 128 : 0; }
hipError_t launch_psa_fused_backward(int dt, const void *qkv, const void *out, const float *lse, const void *d_out,
                                     void *d_qkv, float *delta, const PsaShape &s, hipStream_t stream);
hipError_t launch_psa_extract_v(int dt, const void *qkv, void *v, const PsaShape &s, hipStream_t stream);
hipError_t launch_psa_extract_v_backward(int dt, const void *d_v, void *d_qkv, const PsaShape &s,
                                         hipStream_t stream);

// Smallest query rows per forward / dq workgroup and key rows per dkdv
// workgroup (the ABI checks that the 1-D grids fit in int32).
constexpr int kFwdRowsPerBlock = 64;
constexpr int kDkdvKeysPerBlock = 64;

}  // namespace fa2mi
