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
// Largest log2 gap allowed between a score and the reference max before the
// forward rescales (keeps probabilities <= 2^8 = 256).
constexpr float kRescaleLog2 = 8.f;

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
    __device__ static inline float sum_frag(frag f, float acc) { return acc + f; }
};

// Sum of the 16 values of a C block, as a balanced tree so that the adds
// overlap. Row sums of probabilities use plain float adds: on gfx950 a packed
// dot (v_dot2c_f32_bf16 / _f16, the other way to sum 16-bit pairs) does not
// issue while the matrix pipe runs, and each one was measured to add about
// 7.5 cycles to a wave's MFMA stream, where independent float adds hide
// under it.
__device__ __forceinline__ float sum16(const f32x16 &c) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = c[2 * i] + c[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    return (a[0] + a[1]) + (a[2] + a[3]);
}

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

// Shifted LDS rows: row r of a tile with row stride LD (an odd multiple of
// 64 bytes) starts at r * LD + row_shift(r) elements (16-bit types), a
// 16-byte shift that cycles every 4 rows. ds_read_b64_tr_b16 takes 4
// consecutive rows at a time: one shift, rows 64 bytes apart modulo 256, no
// bank conflict. Row reads of 16 (ds_read_b128) or 32 (8-byte reads)
// consecutive rows at one column land 64 (r mod 4) + 16 ((r / 4) mod 4) bytes
// apart modulo 256: 16 distinct 16-byte slots instead of 4. The shift only
// depends on bits 2-3 of the row, so for rows 16k + lane terms it is a
// per-lane constant. LD must leave 24 elements of room past the data.
__device__ __forceinline__ constexpr int row_shift(int r) { return 8 * ((r >> 2) & 3); }

// ld_vt_frag_tr on a tile with shifted rows.
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag ld_vt_frag_tr_sh(const typename Traits<DT>::elem *vtile, int LD,
                                                                       int key0, int d0, int lane) {
    static_assert(Traits<DT>::KPL == 8, "16-bit element types only");
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    using lds_i16x4 = __attribute__((address_space(3))) i16x4;
    const int l = lane & 15, g = lane >> 4, hh = g >> 1;
    const int r = key0 + 4 * hh + (l >> 2);
    const int c = d0 + 16 * (g & 1) + 4 * (l & 3);
    const typename Traits<DT>::elem *p0 = vtile + r * LD + row_shift(r) + c;
    const typename Traits<DT>::elem *p1 = vtile + (r + 8) * LD + row_shift(r + 8) + c;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p1));
    return __builtin_bit_cast(typename Traits<DT>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// Cooperative tile staging: an R x D row-major global tile is moved by the
// workgroup in RB-row x VEC-column blocks (VEC = one 16-byte vector), each
// thread owning whole blocks. Loads are buffer loads: rows past the end of
// the buffer read as zero, with no lane-dependent branch.
// COL_FAST numbers blocks along a row first (neighbouring lanes read
// neighbouring 16-byte pieces of one row: best for tiles kept row-major in
// LDS); otherwise down a column first (neighbouring lanes write neighbouring
// RB-row runs of one transposed LDS row: conflict-free transposed stores).

template <Dt DT, int R, int D, int NT, bool COL_FAST = true, int RB = 4>
struct TileStage {
    using elem = typename Traits<DT>::elem;
    static constexpr int VEC = vec_elems<DT>();
    static constexpr int BLOCKS = (R / RB) * (D / VEC);
    static constexpr int PER_THREAD = (BLOCKS + NT - 1) / NT;
    static_assert(R % RB == 0 && D % VEC == 0, "tile shape");
    static_assert(RB == 1 || RB == 2 || RB == 4, "block height");
    uint4 v[PER_THREAD][RB];

    __device__ static constexpr int row_block(int blk) { return COL_FAST ? blk / (D / VEC) : blk % (R / RB); }
    __device__ static constexpr int col_block(int blk) { return COL_FAST ? blk % (D / VEC) : blk / (R / RB); }

    // Global -> registers: rows row0 .. row0 + R - 1 of the buffer `rsrc`
    // covers (row stride D; rows past its end read as zero, so there is no
    // lane-dependent branch). Byte offsets are 32-bit, as for RowStage.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int row0, int tid);

    // Registers -> LDS, row-major with row stride LD (elements).
    template <int LD>
    __device__ __forceinline__ void store_rows(elem *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int blk = tid + i * NT;
            if (BLOCKS % NT != 0 && blk >= BLOCKS) break;
            const int rb = row_block(blk), cb = col_block(blk);
#pragma unroll
            for (int r = 0; r < RB; ++r)
                *reinterpret_cast<uint4 *>(lds + (rb * RB + r) * LD + cb * VEC) = v[i][r];
        }
    }

    // Registers -> LDS transposed: element (row, col) goes to lds[col*LD + row],
    // so each RB-row block column becomes one RB-element run.
    template <int LD>
    __device__ __forceinline__ void store_transposed(elem *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int blk = tid + i * NT;
            if (BLOCKS % NT != 0 && blk >= BLOCKS) break;
            const int rb = row_block(blk), cb = col_block(blk);
            const uint32_t *w[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) w[r] = reinterpret_cast<const uint32_t *>(&v[i][r]);
            if constexpr (sizeof(elem) == 2) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    // columns 2p (low halves) and 2p+1 (high halves)
                    const int col = cb * VEC + 2 * p;
                    elem *e0 = lds + col * LD + rb * RB;
                    elem *e1 = lds + (col + 1) * LD + rb * RB;
                    if constexpr (RB == 4) {
                        uint2 even, odd;
                        even.x = (w[0][p] & 0xffffu) | (w[1][p] << 16);
                        even.y = (w[2][p] & 0xffffu) | (w[3][p] << 16);
                        odd.x = (w[0][p] >> 16) | (w[1][p] & 0xffff0000u);
                        odd.y = (w[2][p] >> 16) | (w[3][p] & 0xffff0000u);
                        *reinterpret_cast<uint2 *>(e0) = even;
                        *reinterpret_cast<uint2 *>(e1) = odd;
                    } else if constexpr (RB == 2) {
                        *reinterpret_cast<uint32_t *>(e0) = (w[0][p] & 0xffffu) | (w[1][p] << 16);
                        *reinterpret_cast<uint32_t *>(e1) = (w[0][p] >> 16) | (w[1][p] & 0xffff0000u);
                    } else {
                        *reinterpret_cast<uint16_t *>(e0) = (uint16_t)(w[0][p] & 0xffffu);
                        *reinterpret_cast<uint16_t *>(e1) = (uint16_t)(w[0][p] >> 16);
                    }
                }
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    elem *e = lds + (cb * VEC + p) * LD + rb * RB;
                    if constexpr (RB == 4)
                        *reinterpret_cast<uint4 *>(e) = make_uint4(w[0][p], w[1][p], w[2][p], w[3][p]);
                    else if constexpr (RB == 2)
                        *reinterpret_cast<uint2 *>(e) = make_uint2(w[0][p], w[1][p]);
                    else
                        *reinterpret_cast<uint32_t *>(e) = w[0][p];
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Buffer resources: a raw buffer over one head's rows. Loads at byte offsets
// at or past `bytes` return zero (hardware range check), which zero-fills the
// rows of a ragged last tile without branches.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

template <Dt DT, int R, int D, int NT, bool COL_FAST, int RB>
__device__ __forceinline__ void TileStage<DT, R, D, NT, COL_FAST, RB>::load(__amdgpu_buffer_rsrc_t rsrc, int row0,
                                                                             int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
        const int blk = tid + i * NT;
        const int rb = row_block(blk), cb = col_block(blk);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int row = rb * RB + r;
            if (BLOCKS % NT == 0 || blk < BLOCKS)
                v[i][r] = buffer_load16(rsrc, ((uint32_t)(row0 + row) * D + cb * VEC) * (uint32_t)sizeof(elem));
            else
                v[i][r] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Row-major R x D tile staging through registers with buffer loads: thread
// tid owns PER_THREAD 16-byte pieces, numbered along rows first.
template <Dt DT, int R, int D, int NT>
struct RowStage {
    using elem = typename Traits<DT>::elem;
    static constexpr int VEC = vec_elems<DT>();
    static constexpr int PIECES = R * (D / VEC);
    static constexpr int PER_THREAD = (PIECES + NT - 1) / NT;
    uint4 v[PER_THREAD];

    // rows row0 .. row0+R-1 of the buffer (row stride D elements); byte
    // offsets are 32-bit, so the buffer plus one tile must stay below 4 GiB
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int row0, int tid) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int pc = tid + i * NT;
            const int row = pc / (D / VEC), cv = pc % (D / VEC);
            if (PIECES % NT == 0 || pc < PIECES)
                v[i] = buffer_load16(rsrc, ((uint32_t)(row0 + row) * D + cv * VEC) * (uint32_t)sizeof(elem));
        }
    }

    template <int LD>
    __device__ __forceinline__ void store(elem *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int pc = tid + i * NT;
            const int row = pc / (D / VEC), cv = pc % (D / VEC);
            if (PIECES % NT == 0 || pc < PIECES)
                *reinterpret_cast<uint4 *>(lds + row * LD + cv * VEC) = v[i];
        }
    }
};

// A fragment (32 rows d x 16 keys) of V^T read from a ROW-MAJOR V tile in LDS
// (row = key, stride LD elements) with the gfx950 transposing LDS read
// ds_read_b64_tr_b16. Within each 16-lane group that instruction returns to
// lane j, as element r, element (j % 4) of the 4-element chunk addressed by
// lane 4r + j/4 of the group. Lane l of group g therefore points at
//   V[key0 + 4H + l/4][d0 + 16(g%2) + 4(l%4)]   (H = g/2 = lane half)
// so that lane j receives V[key0 + 4H + r][d0 + 16(g%2) + j], r = 0..3: the
// keys of C-block registers fed back as a B operand (see crow). Two reads
// cover the slots of keys +0..3 and +8..11 of the 16-key step.
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag ld_vt_frag_tr(const typename Traits<DT>::elem *vtile, int LD,
                                                                   int key0, int d0, int lane) {
    static_assert(Traits<DT>::KPL == 8, "16-bit element types only");
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const int l = lane & 15, g = lane >> 4, hh = g >> 1;
    const typename Traits<DT>::elem *p = vtile + (key0 + 4 * hh + (l >> 2)) * LD + d0 + 16 * (g & 1) + 4 * (l & 3);
    using lds_i16x4 = __attribute__((address_space(3))) i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 8 * LD));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Traits<DT>::frag, both);
}

// ---------------------------------------------------------------------------
// Unpadded tiles (64 or 32 rows) of 16-bit elements filled by buffer -> LDS DMA
// (gfx950 buffer_load_dwordx4 ... lds: lane i of a wave instruction writes its
// 16 bytes at LDS base + 16 i, so one instruction fills 1 KiB of consecutive
// rows). Bank conflicts are avoided by an XOR swizzle of the 16-byte chunks
// of each row instead of padding: logical chunk c of row r sits at physical
// chunk c ^ swz(r). The LDS behaves as 64 four-byte banks (256 bytes per bank
// cycle); ds_read_b128 serves 16 lanes at a time (16 consecutive rows, one
// chunk each) and ds_read_b64_tr_b16 32 lanes (4 consecutive rows from a
// multiple of 4, 64 bytes each). swz makes both patterns touch every bank
// once:
//   D = 128 (one row per 256 bytes): 4 (r % 4) + (r / 4) % 4
//   D = 64  (two rows):              4 ((r / 2) % 2) + (r / 4) % 4
//   D = 32  (four rows):             (r / 4) % 4
// For the rows a wave reads (32 kb + lane for K; 32 kb + 16 t + 4 hh + l / 4
// (+ 8) for V) the swizzle does not depend on kb or t, so every fragment
// address is a per-lane constant plus an immediate offset.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (D == 64) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else return (r >> 2) & 3;
}

template <Dt DT, int D, int ROWS_ = 64>
struct SwzTile {
    static_assert(sizeof(typename Traits<DT>::elem) == 2, "16-bit element types only");
    using frag = typename Traits<DT>::frag;
    static constexpr int RB = 2 * D;                    // row bytes
    static constexpr int NC = RB / 16;                  // 16-byte chunks per row
    static constexpr int ROWS = ROWS_;                  // a multiple of 32
    static constexpr int BYTES = ROWS * RB;             // one tile
    static constexpr int PIECES = BYTES / 1024;         // DMA instructions per tile
    static constexpr int TS = D / 16;                   // contraction steps of a K fragment
    static constexpr int NDB = D / 32;
    uint32_t koff[TS];         // K fragment t of row lane % 32 (kb = 0)
    uint32_t voff[NDB][2];     // V^T read pair (db, lower / upper 8 keys) (kb = t = 0)

    __device__ __forceinline__ void init(int lane) {
        const int h = lane >> 5, col = lane & 31;
#pragma unroll
        for (int t = 0; t < TS; ++t) koff[t] = (uint32_t)(col * RB + (((2 * t + h) ^ swz<D>(col)) << 4));
        const int l = lane & 15, g = lane >> 4, hh = g >> 1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const int r = 4 * hh + (l >> 2) + 8 * hi;
                const int cb = (32 * db + 16 * (g & 1)) * 2 + 8 * (l & 3);  // logical byte in the row
                voff[db][hi] = (uint32_t)(r * RB + (((cb >> 4) ^ swz<D>(r)) << 4) + (cb & 15));
            }
    }
    // A/B fragment of K rows 32 kb + lane % 32, contraction step t
    __device__ __forceinline__ frag k(const char *tile, int kb, int t) const {
        return *reinterpret_cast<const frag *>(tile + kb * 32 * RB + koff[t]);
    }
    // A fragment of V^T (as ld_vt_frag_tr): d block db, keys 32 kb + 16 t ..
    __device__ __forceinline__ frag vt(const char *tile, int kb, int t, int db) const {
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        using lds_i16x4 = __attribute__((address_space(3))) i16x4;
        const char *base = tile + (32 * kb + 16 * t) * RB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + voff[db][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + voff[db][1]));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // voff[db][hi] from voff[0][hi]: the chunk index of d block db is that of
    // block 0 XOR 4 db, and the XOR only touches the chunk bits of the
    // offset, so a caller can keep two base registers (passed through
    // opaque() once per tile) instead of 2 NDB loop-invariant offsets.
    __device__ static __forceinline__ uint32_t vt_off(uint32_t v0, int db) { return v0 ^ (uint32_t)(db << 6); }
    // vt() with the pair of offsets given: kb = 0, keys 16 t ..
    __device__ static __forceinline__ frag vt_pair(const char *tile, uint32_t lo_off, uint32_t hi_off, int t) {
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        using lds_i16x4 = __attribute__((address_space(3))) i16x4;
        const char *base = tile + 16 * t * RB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + lo_off));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + hi_off));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // Global byte offset (within a tile) that lane `lane` loads in DMA piece J:
    // rows J * 1024 / RB .., physical chunk lane % NC, logical chunk
    // (lane % NC) ^ swz(row).
    __device__ static __forceinline__ uint32_t piece_off(int J, int lane) {
        const int row = J * (1024 / RB) + lane / NC, p = lane % NC;
        return (uint32_t)(row * RB + ((p ^ swz<D>(row)) << 4));
    }
};

// One 16-byte-per-lane buffer -> LDS DMA: lane i loads the 16 bytes at
// byte `voffset` of the buffer `rsrc` and writes them at lds + 16 i (`lds`
// wave-uniform). Bytes at or past the buffer's end read as zero (hardware
// range check), so a ragged last tile is zero-filled.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0,
                                             0);
}

// Wait for this wave's outstanding buffer loads (the DMA pieces) only:
// s_waitcnt vmcnt(0), leaving expcnt and lgkmcnt at their maxima.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// After the barrier that publishes DMA-filled LDS: the compiler does not see
// the DMA as a store to the LDS arrays, so make it assume LDS has changed.
__device__ __forceinline__ void lds_changed() { __asm__ volatile("" ::: "memory"); }

// Hides a register's value from the optimiser (no instruction is emitted), so
// that values derived from it inside a loop are not hoisted out of the loop
// and kept live across it.
__device__ __forceinline__ void opaque(uint32_t &x) { __asm__ volatile("" : "+v"(x)); }

// Block height that gives each of NT threads one staging block of an R x D
// tile when possible (4 rows at most).
template <Dt DT, int R, int D, int NT>
constexpr int stage_rows() {
    constexpr int r = (R * (D / vec_elems<DT>())) / NT;
    return r >= 4 ? 4 : (r >= 2 ? 2 : 1);
}

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
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with x in both, the two results hold, in every
// lane, x of that lane and x of the lane 32 apart (in some order).
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace fa2mi
