// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// MFMA tiling. Every kernel works on 32x32 output blocks with the CDNA
// matrix instructions v_mfma_f32_32x32x16_{bf16,f16} (8 operand elements per
// lane, 16-deep contraction) and v_mfma_f32_32x32x2_f32 (1 element per lane,
// 2-deep). For both:
//   A operand (M x K):  lane l holds row (l % 32), k-slots h*KPL .. h*KPL+KPL-1
//   B operand (K x N):  lane l holds column (l % 32), the same k-slots
//   C (32 x 32 fp32):   lane l holds column (l % 32); its register c holds
//                       row 8*(c/4) + 4*h + (c%4)
// with h = l / 32 and KPL the per-lane operand width.
//
// Because a C block keeps one column per lane, a C block of probabilities
// (rows = keys, column = query) can be fed straight back as the B operand of
// the next product that contracts over keys: register c of lane half h is
// k-slot (c mod KPL) of step c / KPL, standing for key 8*(c/4) + 4*h + c%4.
// The matching A operand (e.g. V^T) is read from an LDS tile stored
// transposed so that those keys are contiguous (see ld_t_frag).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2mi {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum class Dt { F32 = 0, F16 = 1, BF16 = 2 };

template <Dt DT> struct Traits;

template <> struct Traits<Dt::BF16> {
    using elem = __bf16;
    using frag = bf16x8;
    using half_frag = bf16x4;
    static constexpr int KPL = 8;
    __device__ static inline f32x16 mfma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Traits<Dt::F16> {
    using elem = _Float16;
    using frag = f16x8;
    using half_frag = f16x4;
    static constexpr int KPL = 8;
    __device__ static inline f32x16 mfma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <> struct Traits<Dt::F32> {
    using elem = float;
    using frag = float;
    using half_frag = float;
    static constexpr int KPL = 1;
    __device__ static inline f32x16 mfma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Row of C-block register c for lane half h.
__device__ __forceinline__ constexpr int crow(int c, int h) { return 8 * (c >> 2) + 4 * h + (c & 3); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Element count of one 16-byte vector.
template <Dt DT> constexpr int vec_elems() { return 16 / (int)sizeof(typename Traits<DT>::elem); }

// ---------------------------------------------------------------------------
// Operand fragments

// A/B fragment from a row-major tile (global or LDS): row pointer `row`,
// contraction step t, lane half h. Slots are h*KPL .. h*KPL+KPL-1 of step t,
// i.e. columns t*2*KPL + h*KPL + m.
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag ld_row_frag(const typename Traits<DT>::elem *row, int t, int h) {
    using Tr = Traits<DT>;
    return *reinterpret_cast<const typename Tr::frag *>(row + t * 2 * Tr::KPL + h * Tr::KPL);
}

// A fragment from a transposed LDS tile (one LDS row per output row d, keys
// contiguous): slots of contraction step t of 32-key block kb, lane half h,
// in the key order of a C block fed back as a B operand (see file comment).
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag ld_t_frag(const typename Traits<DT>::elem *trow, int kb, int t, int h) {
    using Tr = Traits<DT>;
    if constexpr (Tr::KPL == 8) {
        const typename Tr::elem *p = trow + 32 * kb + 16 * t + 4 * h;
        typename Tr::half_frag lo = *reinterpret_cast<const typename Tr::half_frag *>(p);
        typename Tr::half_frag hi = *reinterpret_cast<const typename Tr::half_frag *>(p + 8);
        typename Tr::frag f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f[m] = lo[m];
            f[m + 4] = hi[m];
        }
        return f;
    } else {
        return trow[32 * kb + crow(t, h)];
    }
}

// B fragment made from registers of a C block (probabilities or dS): step t.
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag c_to_frag(const f32x16 &c, int t) {
    using Tr = Traits<DT>;
    if constexpr (Tr::KPL == 8) {
        typename Tr::frag f;
#pragma unroll
        for (int m = 0; m < 8; ++m) f[m] = static_cast<typename Tr::elem>(c[8 * t + m]);
        return f;
    } else {
        return c[t];
    }
}

// ---------------------------------------------------------------------------
// Cooperative tile staging: an R x D row-major global tile is moved by the
// workgroup in 4-row x VEC-column blocks (VEC = one 16-byte vector), each
// thread owning whole blocks. Rows at or beyond `valid` are zero-filled.
// COL_FAST numbers blocks along a row first (neighbouring lanes read
// neighbouring 16-byte pieces of one row: best for tiles kept row-major in
// LDS); otherwise down a column first (neighbouring lanes write neighbouring
// 4-row runs of one transposed LDS row: conflict-free transposed stores).

template <Dt DT, int R, int D, int NT, bool COL_FAST = true>
struct TileStage {
    using elem = typename Traits<DT>::elem;
    static constexpr int VEC = vec_elems<DT>();
    static constexpr int BLOCKS = (R / 4) * (D / VEC);
    static constexpr int PER_THREAD = (BLOCKS + NT - 1) / NT;
    static_assert(R % 4 == 0 && D % VEC == 0, "tile shape");
    uint4 v[PER_THREAD][4];

    __device__ static constexpr int row_block(int blk) { return COL_FAST ? blk / (D / VEC) : blk % (R / 4); }
    __device__ static constexpr int col_block(int blk) { return COL_FAST ? blk % (D / VEC) : blk / (R / 4); }

    // Global -> registers. `base` points at row 0 of the tile; row stride D.
    __device__ __forceinline__ void load(const elem *__restrict__ base, int valid, int tid) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int blk = tid + i * NT;
            const int rb = row_block(blk), cb = col_block(blk);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rb * 4 + r;
                if (blk < BLOCKS && row < valid)
                    v[i][r] = *reinterpret_cast<const uint4 *>(base + (int64_t)row * D + cb * VEC);
                else
                    v[i][r] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    // Registers -> LDS, row-major with row stride LD (elements).
    template <int LD>
    __device__ __forceinline__ void store_rows(elem *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int blk = tid + i * NT;
            if (blk >= BLOCKS) break;
            const int rb = row_block(blk), cb = col_block(blk);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint4 *>(lds + (rb * 4 + r) * LD + cb * VEC) = v[i][r];
        }
    }

    // Registers -> LDS transposed: element (row, col) goes to lds[col*LD + row],
    // so each 4-row block column becomes one 4-element run.
    template <int LD>
    __device__ __forceinline__ void store_transposed(elem *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int blk = tid + i * NT;
            if (blk >= BLOCKS) break;
            const int rb = row_block(blk), cb = col_block(blk);
            if constexpr (sizeof(elem) == 2) {
                const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&v[i][0]);
                const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&v[i][1]);
                const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&v[i][2]);
                const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&v[i][3]);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    // columns 2p (low halves) and 2p+1 (high halves)
                    uint2 even, odd;
                    even.x = (r0[p] & 0xffffu) | (r1[p] << 16);
                    even.y = (r2[p] & 0xffffu) | (r3[p] << 16);
                    odd.x = (r0[p] >> 16) | (r1[p] & 0xffff0000u);
                    odd.y = (r2[p] >> 16) | (r3[p] & 0xffff0000u);
                    const int col = cb * VEC + 2 * p;
                    *reinterpret_cast<uint2 *>(lds + col * LD + rb * 4) = even;
                    *reinterpret_cast<uint2 *>(lds + (col + 1) * LD + rb * 4) = odd;
                }
            } else {
                const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&v[i][0]);
                const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&v[i][1]);
                const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&v[i][2]);
                const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&v[i][3]);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int col = cb * VEC + p;
                    *reinterpret_cast<uint4 *>(lds + col * LD + rb * 4) = make_uint4(r0[p], r1[p], r2[p], r3[p]);
                }
            }
        }
    }
};

// Maps the hardware workgroup id to a logical tile id so that the tiles one
// XCD runs are contiguous in logical order (same heads -> shared K/V in that
// XCD's L2). Workgroups are dealt round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
    constexpr int kXcd = 8;
    const int x = hw_id % kXcd, slot = hw_id / kXcd;
    const int q = total / kXcd, r = total % kXcd;
    return x * q + min(x, r) + slot;
}

// Max / sum with the lane 32 apart (the other half of a C block column).
__device__ __forceinline__ float xhalf_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float xhalf_sum(float x) { return x + __shfl_xor(x, 32); }

}  // namespace fa2mi
