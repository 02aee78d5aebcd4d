// PSA rearrangements around the attention of a C2PSA block (vision_rs
// psa.rs, "psa_pack_qkv" and "psa_merge_attn_nchw"). Both are batched
// transposes between a channel-major NCHW slice [kd channels][hw pixels] and
// a pixel-major attention operand [hw rows][kd]:
//   pack : slice (b, head, s) of qkv = channels head*4kd + s*kd .. +kd of
//          batch b, i.e. the contiguous [kd][hw] block ((b*nh+head)*4+s)*kd*hw,
//          goes to packed section s, head row b*nh+head: the contiguous
//          [hw][kd] block (s*BH + b*nh + head)*hw*kd;
//   merge: o_lo / o_hi head bh ([hw][kd] at bh*hw*kd) go to out channels
//          head*2kd (+kd for hi) of batch b: the contiguous [kd][hw] block
//          (2*bh + half)*kd*hw.
// One workgroup moves a kd x P tile (P pixels) through LDS so that global
// reads and writes are both contiguous 16-byte vectors.
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

// [KD][hw] slice -> [hw][KD] slice, tile of P pixels per workgroup.
// ALIGNED: hw is a multiple of VEC, so pixel vectors never straddle a row end.
template <typename elem, int KD, bool ALIGNED>
__global__ __launch_bounds__(256) void pack_kernel(const elem *__restrict__ qkv, elem *__restrict__ packed,
                                                   int nh, int bh, int hw, int tiles_per_slice) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;  // pixels per tile
    constexpr int LD = P + VEC;        // LDS row stride (channel rows)
    __shared__ __attribute__((aligned(16))) elem tile[KD * LD];

    const int tid = threadIdx.x;
    const int slice = blockIdx.x / tiles_per_slice;  // (b*nh + head)*4 + s
    const int p0 = (blockIdx.x % tiles_per_slice) * P;
    const int s = slice % 4, bhh = slice / 4;
    const elem *src = qkv + (int64_t)slice * KD * hw;
    elem *dst = packed + ((int64_t)s * bh + bhh) * hw * KD;

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
    (void)nh;
}

// [hw][KD] slice -> [KD][hw] slice.
template <typename elem, int KD, bool ALIGNED>
__global__ __launch_bounds__(256) void merge_kernel(const elem *__restrict__ lo, const elem *__restrict__ hi,
                                                    elem *__restrict__ out, int hw, int tiles_per_slice) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;
    constexpr int LD = KD + VEC;  // LDS row stride (pixel rows)
    __shared__ __attribute__((aligned(16))) elem tile[P * LD];

    const int tid = threadIdx.x;
    const int slice = blockIdx.x / tiles_per_slice;  // 2*bh + half
    const int p0 = (blockIdx.x % tiles_per_slice) * P;
    const int half = slice & 1, bhh = slice >> 1;
    const elem *src = (half ? hi : lo) + (int64_t)bhh * hw * KD;
    elem *dst = out + (int64_t)slice * KD * hw;

    {   // read: pixel p, channel vector cv (contiguous P x KD block)
        const int p = tid / (KD / VEC), cv = tid % (KD / VEC);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (p0 + p < hw) v = *reinterpret_cast<const uint4 *>(src + (int64_t)(p0 + p) * KD + cv * VEC);
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

template <typename elem, int KD>
static hipError_t pack_dispatch(const void *qkv, void *packed, const PsaShape &s, hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;
    const int tps = (s.hw + P - 1) / P;
    const int bh = s.batch * s.num_heads;
    const int grid = bh * 4 * tps;
    if (s.hw % VEC == 0)
        hipLaunchKernelGGL((pack_kernel<elem, KD, true>), dim3(grid), dim3(256), 0, stream, (const elem *)qkv,
                           (elem *)packed, s.num_heads, bh, s.hw, tps);
    else
        hipLaunchKernelGGL((pack_kernel<elem, KD, false>), dim3(grid), dim3(256), 0, stream, (const elem *)qkv,
                           (elem *)packed, s.num_heads, bh, s.hw, tps);
    return hipGetLastError();
}

template <typename elem, int KD>
static hipError_t merge_dispatch(const void *lo, const void *hi, void *out, const PsaShape &s, hipStream_t stream) {
    constexpr int VEC = 16 / (int)sizeof(elem);
    constexpr int P = 256 * VEC / KD;
    const int tps = (s.hw + P - 1) / P;
    const int bh = s.batch * s.num_heads;
    const int grid = bh * 2 * tps;
    if (s.hw % VEC == 0)
        hipLaunchKernelGGL((merge_kernel<elem, KD, true>), dim3(grid), dim3(256), 0, stream, (const elem *)lo,
                           (const elem *)hi, (elem *)out, s.hw, tps);
    else
        hipLaunchKernelGGL((merge_kernel<elem, KD, false>), dim3(grid), dim3(256), 0, stream, (const elem *)lo,
                           (const elem *)hi, (elem *)out, s.hw, tps);
    return hipGetLastError();
}

// The rearrangements copy bits, so only the element size matters.
template <typename elem>
static hipError_t pack_by_kd(const void *qkv, void *packed, const PsaShape &s, hipStream_t st) {
    switch (s.key_dim) {
        case 32: return pack_dispatch<elem, 32>(qkv, packed, s, st);
        case 64: return pack_dispatch<elem, 64>(qkv, packed, s, st);
        case 128: return pack_dispatch<elem, 128>(qkv, packed, s, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename elem>
static hipError_t merge_by_kd(const void *lo, const void *hi, void *out, const PsaShape &s, hipStream_t st) {
    switch (s.key_dim) {
        case 32: return merge_dispatch<elem, 32>(lo, hi, out, s, st);
        case 64: return merge_dispatch<elem, 64>(lo, hi, out, s, st);
        case 128: return merge_dispatch<elem, 128>(lo, hi, out, s, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_psa_pack(int dt, const void *qkv, void *packed, const PsaShape &s, hipStream_t stream) {
    return dt == 0 ? pack_by_kd<uint32_t>(qkv, packed, s, stream) : pack_by_kd<uint16_t>(qkv, packed, s, stream);
}

hipError_t launch_psa_merge(int dt, const void *lo, const void *hi, void *out, const PsaShape &s,
                            hipStream_t stream) {
    return dt == 0 ? merge_by_kd<uint32_t>(lo, hi, out, s, stream) : merge_by_kd<uint16_t>(lo, hi, out, s, stream);
}

}  // namespace fa2mi
