// PSA rearrangements around the attention of a C2PSA block (vision_rs
// psa.rs, "psa_pack_qkv", "psa_merge_attn_nchw" and their backward kernels
// "psa_pack_qkv_backward", "psa_merge_attn_backward"). The first four are
// batched transposes between a channel-major NCHW slice [kd channels][hw pixels] and
// a pixel-major attention operand [hw rows][kd]:
//   pack : slice (b, head, s) of qkv = channels head*4kd + s*kd .. +kd of
//          batch b, i.e. the contiguous [kd][hw] block ((b*nh+head)*4+s)*kd*hw,
//          goes to packed section s, head row b*nh+head: the contiguous
//          [hw][kd] block (s*BH + b*nh + head)*hw*kd;
//   merge: o_lo / o_hi head bh ([hw][kd] at bh*hw*kd) go to out channels
//          head*2kd (+kd for hi) of batch b: the contiguous [kd][hw] block
//          (2*bh + half)*kd*hw;
//   merge backward: the inverse of merge (d_out slices to d_o_lo / d_o_hi);
//   pack backward : the inverse of pack (d_packed sections to d_qkv slices),
//          optionally adding a second Q/K gradient pair;
// and, without a transpose, "psa_extract_v_nchw" and "psa_extract_v_backward"
// (the V channels of each head as one contiguous block).
// One workgroup moves a kd x P tile (P pixels) through LDS so that global
// reads and writes are both contiguous 16-byte vectors; the merge of 16-bit
// maps whose h*w is a multiple of 8 uses a register transpose instead (below).
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2mi {

// Reads VEC elements at src[0..VEC) (fewer at the end of a row when the row
// length is not a multiple of VEC; missing ones are left as zero bits).
template <typename elem, int VEC, bool ALIGNED>
__device__ __forceinline__ uint4 ld_vec(const elem *src, int avail) {
    if constexpr (ALIGNED) {
        return *reinterpret_cast<const uint4 *>(src);
    } else {
        uint4 r = make_uint4(0, 0, 0, 0);
        elem *e = reinterpret_cast<elem *>(&r);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (i < avail) e[i] = src[i];
        return r;
    }
}

template <typename elem, int VEC, bool ALIGNED>
__device__ __forceinline__ void st_vec(elem *dst, const uint4 &v, int avail) {
    if constexpr (ALIGNED) {
        *reinterpret_cast<uint4 *>(dst) = v;
    } else {
        const elem *e = reinterpret_cast<const elem *>(&v);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (i < avail) dst[i] = e[i];
    }
}

// Up to four section pointers, passed by value.
struct SecPtrs {
    const void *p[4];
};

// [KD][hw] channel slices -> [hw][KD] row slices, tile of P pixels per
// workgroup. Source slice `slice` (the contiguous [KD][hw] block `slice` of
// src) is (head row bhh, section s) with slice = bhh * NSEC + s; it goes to
// dst[s] + bhh * hw * KD. pack: NSEC = 4 (Q, K, V_lo, V_hi sections of the
// packed buffer); merge backward: NSEC = 2 (d_o_lo, d_o_hi).
// ALIGNED: hw is a multiple of VEC, so pixel vectors never straddle a row end.
template <typename elem, int KD, int NSEC, bool ALIGNED>
__global__ __launch_bounds__(256) void to_rows_kernel(const elem *__restrict__ src_all, SecPtrs dst_sec, int hw,
                                                      int tiles_per_slice) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;  // pixels per tile
    constexpr int LD = P + VEC;        // LDS row stride (channel rows)
    __shared__ __attribute__((aligned(16))) elem tile[KD * LD];

    const int tid = threadIdx.x;
    // neighbouring tiles of a slice share cache lines at their edges (a
    // channel row is rarely a multiple of 128 bytes): keep them on one XCD
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = b / tiles_per_slice;
    const int p0 = (b % tiles_per_slice) * P;
    const int s = slice % NSEC, bhh = slice / NSEC;
    const elem *src = src_all + (int64_t)slice * KD * hw;
    elem *dst = const_cast<elem *>(static_cast<const elem *>(dst_sec.p[s])) + (int64_t)bhh * hw * KD;

    {   // read: channel row c, pixel vector pv
        const int c = tid / (P / VEC), pv = tid % (P / VEC);
        const int p = p0 + pv * VEC;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (p < hw) v = ld_vec<elem, VEC, ALIGNED>(src + (int64_t)c * hw + p, hw - p);
        *reinterpret_cast<uint4 *>(tile + c * LD + pv * VEC) = v;
    }
    __syncthreads();
    {   // write: pixel p, channel vector cv; the P x KD block of dst is contiguous
        const int p = tid / (KD / VEC), cv = tid % (KD / VEC);
        if (p0 + p < hw) {
            uint4 v;
            elem *e = reinterpret_cast<elem *>(&v);
#pragma unroll
            for (int i = 0; i < VEC; ++i) e[i] = tile[(cv * VEC + i) * LD + p];
            *reinterpret_cast<uint4 *>(dst + (int64_t)(p0 + p) * KD + cv * VEC) = v;
        }
    }
}

// [hw][KD] row slices -> [KD][hw] channel slices. Destination slice
// slice = bhh * NSEC + s (the contiguous [KD][hw] block `slice` of out) is
// read from src[s] + bhh * hw * KD. merge: NSEC = 2 (o_lo, o_hi); pack
// backward: NSEC = 4 (the sections of d_packed). ADD: sections 0 and 1 also
// add add_sec[s] + bhh * hw * KD (the second V-split call's dQ and dK) in
// fp32 before rounding; T is then the element type, else any type of the
// element's size (the copy moves bits).
template <typename T, int KD, int NSEC, bool ADD, bool ALIGNED>
__global__ __launch_bounds__(256) void to_channels_kernel(SecPtrs src_sec, SecPtrs add_sec, T *__restrict__ out,
                                                          int hw, int tiles_per_slice) {
    using elem = T;
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;
    constexpr int LD = KD + VEC;  // LDS row stride (pixel rows)
    __shared__ __attribute__((aligned(16))) elem tile[P * LD];

    const int tid = threadIdx.x;
    // neighbouring tiles of a slice share cache lines at their edges (a
    // channel row is rarely a multiple of 128 bytes): keep them on one XCD
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = b / tiles_per_slice;
    const int p0 = (b % tiles_per_slice) * P;
    const int s = slice % NSEC, bhh = slice / NSEC;
    const elem *src = static_cast<const elem *>(src_sec.p[s]) + (int64_t)bhh * hw * KD;
    elem *dst = out + (int64_t)slice * KD * hw;

    {   // read: pixel p, channel vector cv (contiguous P x KD block)
        const int p = tid / (KD / VEC), cv = tid % (KD / VEC);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (p0 + p < hw) {
            const int64_t off = (int64_t)(p0 + p) * KD + cv * VEC;
            v = *reinterpret_cast<const uint4 *>(src + off);
            if constexpr (ADD) {
                if (s < 2) {
                    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const elem *>(add_sec.p[s]) +
                                                                     (int64_t)bhh * hw * KD + off);
                    elem *ev = reinterpret_cast<elem *>(&v);
                    const elem *ew = reinterpret_cast<const elem *>(&w);
#pragma unroll
                    for (int i = 0; i < VEC; ++i)
                        ev[i] = static_cast<elem>(static_cast<float>(ev[i]) + static_cast<float>(ew[i]));
                }
            }
        }
        *reinterpret_cast<uint4 *>(tile + p * LD + cv * VEC) = v;
    }
    __syncthreads();
    {   // write: channel c, pixel vector pv
        const int c = tid / (P / VEC), pv = tid % (P / VEC);
        const int p = p0 + pv * VEC;
        if (p < hw) {
            uint4 v;
            elem *e = reinterpret_cast<elem *>(&v);
#pragma unroll
            for (int i = 0; i < VEC; ++i) e[i] = tile[(pv * VEC + i) * LD + c];
            st_vec<elem, VEC, ALIGNED>(dst + (int64_t)c * hw + p, v, hw - p);
        }
    }
}

// 16-bit elements with h*w a multiple of 8 (every channel row 16-byte
// aligned), row slices to channel slices without LDS. Thread task (slice,
// pixel group pg of 8 pixels, channel group cg of 8 channels), cg fastest: it
// loads eight 16-byte pieces (8 channels of 8 consecutive pixel rows),
// transposes the 8 x 8 block in registers and stores eight 16-byte pieces of
// channel rows. No barrier, and 128 bytes per thread in flight at once. On the
// merge of a 16 x 4 head, key_dim 32, 20 x 20 f16 block this takes 3.4 us
// against 3.8 us for the LDS kernel; for the opposite direction (the pack) the LDS kernel
// stays the faster one, so only this direction has a register form.
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t a = reinterpret_cast<const uint32_t *>(&in[2 * k])[j >> 1];
            const uint32_t b = reinterpret_cast<const uint32_t *>(&in[2 * k + 1])[j >> 1];
            // element j of rows 2k (low half) and 2k+1 (high half)
            o[k] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// [hw][KD] row slices -> [KD][hw] channel slices (as to_channels_kernel
// without ADD)
template <int KD, int NSEC>
__global__ __launch_bounds__(128) void to_channels_reg_kernel(SecPtrs src_sec, uint16_t *__restrict__ out_all,
                                                              int hw, int npg, int64_t ntasks) {
    constexpr int NCG = KD / 8;
    const int64_t t = (int64_t)blockIdx.x * 128 + threadIdx.x;
    if (t >= ntasks) return;
    const int cg = (int)(t % NCG);
    const int64_t r = t / NCG;
    const int pg = (int)(r % npg);
    const int64_t slice = r / npg;
    const int s = (int)(slice % NSEC);
    const int64_t bhh = slice / NSEC;
    const uint16_t *src = static_cast<const uint16_t *>(src_sec.p[s]) + bhh * hw * KD + (int64_t)pg * 8 * KD + cg * 8;
    uint4 in[8], out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) in[j] = *reinterpret_cast<const uint4 *>(src + j * KD);
    transpose8x8_b16(in, out);
    uint16_t *dst = out_all + slice * KD * hw + (int64_t)cg * 8 * hw + pg * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4 *>(dst + (int64_t)c * hw) = out[c];
}

template <int KD, int NSEC>
static hipError_t to_channels_reg_launch(const SecPtrs &src, void *out, const PsaShape &s, hipStream_t stream) {
    const int npg = s.hw / 8;
    const int64_t ntasks = (int64_t)s.batch * s.num_heads * NSEC * npg * (KD / 8);
    hipLaunchKernelGGL((to_channels_reg_kernel<KD, NSEC>), dim3((unsigned)((ntasks + 127) / 128)), dim3(128), 0,
                       stream, src, (uint16_t *)out, s.hw, npg, ntasks);
    return hipGetLastError();
}

template <typename elem, int KD, int NSEC>
static hipError_t to_rows_dispatch(const void *src, const SecPtrs &dst, const PsaShape &s, hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;
    const int tps = (s.hw + P - 1) / P;
    const int grid = s.batch * s.num_heads * NSEC * tps;
    if (s.hw % VEC == 0)
        hipLaunchKernelGGL((to_rows_kernel<elem, KD, NSEC, true>), dim3(grid), dim3(256), 0, stream,
                           (const elem *)src, dst, s.hw, tps);
    else
        hipLaunchKernelGGL((to_rows_kernel<elem, KD, NSEC, false>), dim3(grid), dim3(256), 0, stream,
                           (const elem *)src, dst, s.hw, tps);
    return hipGetLastError();
}

template <typename T, int KD, int NSEC, bool ADD>
static hipError_t to_channels_dispatch(const SecPtrs &src, const SecPtrs &add, void *out, const PsaShape &s,
                                       hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int P = 256 * VEC / KD;
    const int tps = (s.hw + P - 1) / P;
    const int grid = s.batch * s.num_heads * NSEC * tps;
    if (s.hw % VEC == 0)
        hipLaunchKernelGGL((to_channels_kernel<T, KD, NSEC, ADD, true>), dim3(grid), dim3(256), 0, stream, src, add,
                           (T *)out, s.hw, tps);
    else
        hipLaunchKernelGGL((to_channels_kernel<T, KD, NSEC, ADD, false>), dim3(grid), dim3(256), 0, stream, src,
                           add, (T *)out, s.hw, tps);
    return hipGetLastError();
}

template <typename elem, int NSEC>
static hipError_t to_rows_by_kd(const void *src, const SecPtrs &dst, const PsaShape &s, hipStream_t st) {
    switch (s.key_dim) {
        case 32: return to_rows_dispatch<elem, 32, NSEC>(src, dst, s, st);
        case 64: return to_rows_dispatch<elem, 64, NSEC>(src, dst, s, st);
        case 128: return to_rows_dispatch<elem, 128, NSEC>(src, dst, s, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int NSEC, bool ADD>
static hipError_t to_channels_by_kd(const SecPtrs &src, const SecPtrs &add, void *out, const PsaShape &s,
                                    hipStream_t st) {
    if (sizeof(T) == 2 && !ADD && s.hw % 8 == 0) {
        switch (s.key_dim) {
            case 32: return to_channels_reg_launch<32, NSEC>(src, out, s, st);
            case 64: return to_channels_reg_launch<64, NSEC>(src, out, s, st);
            case 128: return to_channels_reg_launch<128, NSEC>(src, out, s, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (s.key_dim) {
        case 32: return to_channels_dispatch<T, 32, NSEC, ADD>(src, add, out, s, st);
        case 64: return to_channels_dispatch<T, 64, NSEC, ADD>(src, add, out, s, st);
        case 128: return to_channels_dispatch<T, 128, NSEC, ADD>(src, add, out, s, st);
        default: return hipErrorInvalidValue;
    }
}

// psa_extract_v_nchw and its backward: per head, the V_lo and V_hi channels
// are one contiguous block of 2 kd rows of hw pixels both in qkv (channels
// head*4kd + 2kd ..) and in v (channels head*2kd ..). Block j of src
// (src + j*src_stride + src_off) is copied to, or with ADD added in fp32 to,
// block j of dst (dst + j*dst_stride + dst_off); block_vecs 16-byte vectors
// per block (2 kd hw elements is always a whole number of vectors, and every
// block starts 16-byte aligned).
template <typename T, bool ADD>
__global__ __launch_bounds__(256) void vblock_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                     int64_t src_stride, int64_t src_off, int64_t dst_stride,
                                                     int64_t dst_off, int block_vecs, int chunks) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const int j = blockIdx.x / chunks;
    const int v = (blockIdx.x % chunks) * 256 + threadIdx.x;
    if (v >= block_vecs) return;
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src + j * src_stride + src_off) + v;
    uint4 *d4 = reinterpret_cast<uint4 *>(dst + j * dst_stride + dst_off) + v;
    uint4 x = *s4;
    if constexpr (ADD) {
        const uint4 y = *d4;
        T *ex = reinterpret_cast<T *>(&x);
        const T *ey = reinterpret_cast<const T *>(&y);
#pragma unroll
        for (int i = 0; i < VEC; ++i) ex[i] = static_cast<T>(static_cast<float>(ey[i]) + static_cast<float>(ex[i]));
    }
    *d4 = x;
}

template <typename T, bool ADD>
static hipError_t vblock_launch(const void *src, void *dst, int64_t src_stride, int64_t src_off, int64_t dst_stride,
                                int64_t dst_off, const PsaShape &s, hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const int64_t block_elems = (int64_t)2 * s.key_dim * s.hw;
    const int block_vecs = (int)(block_elems / VEC);
    const int chunks = (block_vecs + 255) / 256;
    const int grid = s.batch * s.num_heads * chunks;
    hipLaunchKernelGGL((vblock_kernel<T, ADD>), dim3(grid), dim3(256), 0, stream, (const T *)src, (T *)dst,
                       src_stride, src_off, dst_stride, dst_off, block_vecs, chunks);
    return hipGetLastError();
}

hipError_t launch_psa_extract_v(int dt, const void *qkv, void *v, const PsaShape &s, hipStream_t stream) {
    const int64_t kh = (int64_t)s.key_dim * s.hw;
    if (dt == 0) return vblock_launch<uint32_t, false>(qkv, v, 4 * kh, 2 * kh, 2 * kh, 0, s, stream);
    return vblock_launch<uint16_t, false>(qkv, v, 4 * kh, 2 * kh, 2 * kh, 0, s, stream);
}

hipError_t launch_psa_extract_v_backward(int dt, const void *d_v, void *d_qkv, const PsaShape &s,
                                         hipStream_t stream) {
    const int64_t kh = (int64_t)s.key_dim * s.hw;
    switch (dt) {
        case 0: return vblock_launch<float, true>(d_v, d_qkv, 2 * kh, 0, 4 * kh, 2 * kh, s, stream);
        case 1: return vblock_launch<_Float16, true>(d_v, d_qkv, 2 * kh, 0, 4 * kh, 2 * kh, s, stream);
        case 2: return vblock_launch<__bf16, true>(d_v, d_qkv, 2 * kh, 0, 4 * kh, 2 * kh, s, stream);
        default: return hipErrorInvalidValue;
    }
}

// Section pointers of a section-major buffer [n][B*nh][hw][kd].
static SecPtrs sections(const void *base, int n, const PsaShape &s, int esize) {
    SecPtrs r{};
    const int64_t sec_bytes = (int64_t)s.batch * s.num_heads * s.hw * s.key_dim * esize;
    for (int i = 0; i < n; ++i) r.p[i] = static_cast<const char *>(base) + i * sec_bytes;
    return r;
}

hipError_t launch_psa_pack(int dt, const void *qkv, void *packed, const PsaShape &s, hipStream_t stream) {
    if (dt == 0) return to_rows_by_kd<uint32_t, 4>(qkv, sections(packed, 4, s, 4), s, stream);
    return to_rows_by_kd<uint16_t, 4>(qkv, sections(packed, 4, s, 2), s, stream);
}

hipError_t launch_psa_merge(int dt, const void *lo, const void *hi, void *out, const PsaShape &s,
                            hipStream_t stream) {
    const SecPtrs src{{lo, hi, nullptr, nullptr}}, none{};
    if (dt == 0) return to_channels_by_kd<uint32_t, 2, false>(src, none, out, s, stream);
    return to_channels_by_kd<uint16_t, 2, false>(src, none, out, s, stream);
}

hipError_t launch_psa_merge_backward(int dt, const void *d_out, void *d_lo, void *d_hi, const PsaShape &s,
                                     hipStream_t stream) {
    const SecPtrs dst{{d_lo, d_hi, nullptr, nullptr}};
    if (dt == 0) return to_rows_by_kd<uint32_t, 2>(d_out, dst, s, stream);
    return to_rows_by_kd<uint16_t, 2>(d_out, dst, s, stream);
}

hipError_t launch_psa_pack_backward(int dt, const void *d_packed, const void *d_qk_extra, void *d_qkv,
                                    const PsaShape &s, hipStream_t stream) {
    const int es = dt == 0 ? 4 : 2;
    const SecPtrs src = sections(d_packed, 4, s, es);
    if (d_qk_extra == nullptr) {
        const SecPtrs none{};
        if (dt == 0) return to_channels_by_kd<uint32_t, 4, false>(src, none, d_qkv, s, stream);
        return to_channels_by_kd<uint16_t, 4, false>(src, none, d_qkv, s, stream);
    }
    const SecPtrs add = sections(d_qk_extra, 2, s, es);
    switch (dt) {
        case 0: return to_channels_by_kd<float, 4, true>(src, add, d_qkv, s, stream);
        case 1: return to_channels_by_kd<_Float16, 4, true>(src, add, d_qkv, s, stream);
        case 2: return to_channels_by_kd<__bf16, 4, true>(src, add, d_qkv, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa2mi
