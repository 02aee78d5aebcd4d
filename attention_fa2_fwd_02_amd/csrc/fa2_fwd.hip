// Attention forward (vision-rs flash_attn2.rs, "Forward"; vyre-libs
// flash_attention_2.rs, tiled builder): O = softmax(scale Q K^T) V and the
// natural-log LSE per query row, by the online-softmax recurrence over key
// tiles so the score matrix never leaves registers.
//
// Workgroup: WAVES wavefronts, each owning 32 query rows (BR = 32*WAVES rows
// per workgroup). Per key tile of BC rows:
//   1. K (row-major) and V (transposed) tiles are staged in LDS; the next
//      tile is fetched into registers while the current one is computed.
//   2. S^T = K Q^T on MFMA: one C block per 32 keys; each lane owns one query
//      (the C column), so a row's max needs one exchange between lane halves.
//   3. Online softmax in the log2 domain (scale*log2(e) folded into one FMA
//      before exp2): P = 2^(S - m), l += rowsum(P) in float32 over P before
//      it is rounded to the element type for the product (lane-partial
//      sums, combined at the end). The reference m is the first tile's row max; later tiles use
//      it as it is unless l leaves range, in which case the workgroup redoes
//      the rows with the max taken on every tile and m raised lazily (only
//      when a row max exceeds it by more than kRescaleLog2, O and l then
//      rescaled by 2^(m - m') as in the online-softmax recurrence).
//   4. O^T += V^T P^T on MFMA, P fed from registers as the B operand.
// Epilogue: O = O^T / l rounded to the element type; LSE = ln2 * (m + log2 l).
// 16-bit inputs at head_dim 128 with key lengths in whole 256-key groups and
// at least two 256-row query blocks per CU run the persistent form
// (fwd_stream_kernel): one 8-wave workgroup per CU walks the query blocks,
// its K/V ring and Q loads running on from one block into the next.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2mi {

template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag zero_frag() {
    typename Traits<DT>::frag f;
    if constexpr (Traits<DT>::KPL == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<typename Traits<DT>::elem>(0.f);
    } else {
        f = 0.f;
    }
    return f;
}

// Stores the 4 consecutive values c = 4g .. 4g+3 of a C block, scaled by mul,
// at dst[0..3] in the element type.
template <Dt DT>
__device__ __forceinline__ void store4(typename Traits<DT>::elem *dst, const f32x16 &c, int g, float mul) {
    using elem = typename Traits<DT>::elem;
    if constexpr (sizeof(elem) == 2) {
        typename Traits<DT>::half_frag v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = static_cast<elem>(c[4 * g + i] * mul);
        *reinterpret_cast<typename Traits<DT>::half_frag *>(dst) = v;
    } else {
        *reinterpret_cast<float4 *>(dst) =
            make_float4(c[4 * g] * mul, c[4 * g + 1] * mul, c[4 * g + 2] * mul, c[4 * g + 3] * mul);
    }
}

// V tile row stride. 16-bit types: row-major, read only by
// ds_read_b64_tr_b16, which serves 4 rows x 64 bytes per cycle; rows whose
// starts are 64 bytes apart modulo 256 keep those in distinct banks (64-byte
// pad from D = 64 up; D = 32 rows are 64 bytes already). float32: the tile
// is stored transposed (keys contiguous).
template <Dt DT, int D, int BC>
constexpr int fwd_ldv() {
    if constexpr (sizeof(typename Traits<DT>::elem) == 2) return D >= 64 ? D + 32 : D;
    else return BC + 4;
}

// One key tile of the forward for one wave: scores, online softmax with lazy
// rescaling, and the P V accumulation. MASK: the tile is the ragged last one
// and keys at or beyond kvalid do not exist (probability 0). FAST: the row
// max is taken only on the FIRST tile; later tiles use the current reference
// as it is (see fwd_kernel). FIRST is a template parameter so that the
// steady-state loop body has no branch between the score products and the
// softmax: the exponentials of the first key block can then be scheduled
// among the products of the second (5% faster at head_dim 64, the same at
// 128).
template <Dt DT, int D, int BC, bool MASK, bool FAST = false, bool FIRST = true>
__device__ __forceinline__ void fwd_tile(const typename Traits<DT>::elem *kt, const typename Traits<DT>::elem *vt,
                                         const typename Traits<DT>::frag (&qf)[D / (2 * Traits<DT>::KPL)],
                                         f32x16 (&acc)[D / 32], float &m_ref, float &l_run, float scale_log2,
                                         int kvalid, int lane) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr bool TR = sizeof(elem) == 2;
    constexpr int KPL = Tr::KPL;
    constexpr int KSTEP = 2 * KPL;
    constexpr int VEC = vec_elems<DT>();
    constexpr int LDK = D + VEC;
    constexpr int LDV = fwd_ldv<DT, D, BC>();
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int TS = D / KSTEP;
    constexpr int TP = 32 / KSTEP;
    const int h = lane >> 5, col = lane & 31;
    // S^T = K Q^T (raw dot products), one 32x32 block per 32 keys. 16-bit
    // types: block by block, so the first block is complete while the
    // second's products still run; float32: the blocks' chains interleaved
    // (the layout its tests verify).
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
    if constexpr (TR) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < TS; ++t)
                s[kb] = Tr::mfma(ld_row_frag<DT>(kt + (32 * kb + col) * LDK, t, h), qf[t], s[kb]);
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                s[kb] = Tr::mfma(ld_row_frag<DT>(kt + (32 * kb + col) * LDK, t, h), qf[t], s[kb]);
    }

    // ragged last tile: keys >= kvalid do not exist (probability 0)
    if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (32 * kb + crow(c, h) >= kvalid) s[kb][c] = -INFINITY;
    }
    if constexpr (!FAST || FIRST) {
        // lane-partial max of the raw scores (scale > 0, so the max commutes
        // with scaling)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c) mx = fmaxf(mx, s[kb][c]);
        // Lazy rescaling: the reference max only moves when some row's max
        // exceeds it by more than kRescaleLog2 (probabilities then stay
        // <= 2^kRescaleLog2). Moving it rescales O and l by 2^(m_ref - m_new),
        // the online-softmax correction; the final O = acc / l is unchanged.
        const float mx2 = mx * scale_log2;
        if (__any(mx2 > m_ref + kRescaleLog2)) {
            __asm__ volatile("" ::: "memory");
            const float m_new = fmaxf(m_ref, xhalf_max(mx2));
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[db][c] *= alpha;
            l_run *= alpha;
            m_ref = m_new;
        }
    }
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 16; ++c) s[kb][c] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][c], scale_log2, neg_m));
    // O^T += V^T P^T: per 16-key step, one P fragment feeds all d blocks;
    // l sums the probabilities.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < TP; ++t) {
            const frag pf = c_to_frag<DT>(s[kb], t);
            l_run = Tr::sum_frag(pf, l_run);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                frag vf;
                if constexpr (TR)
                    vf = ld_vt_frag_tr<DT>(vt, LDV, 32 * kb + 16 * t, 32 * db, lane);
                else
                    vf = ld_t_frag<DT>(vt + (32 * db + col) * LDV, kb, t, h);
                acc[db] = Tr::mfma(vf, pf, acc[db]);
            }
        }

}

// One 64-key tile of the 16-bit forward on DMA-filled swizzled tiles (see
// SwzTile): the same steps as fwd_tile, with fragment addresses precomputed
// per lane; the fast pass's steady tile (no mask, no max) has its own
// phase-ordered schedule.
struct NoMid {
    __device__ __forceinline__ void operator()() const {}
};

template <Dt DT, int D, bool MASK, bool FAST, bool FIRST, class Mid = NoMid>
__device__ __forceinline__ void fwd_tile_dma(const char *kt, const char *vt, const SwzTile<DT, D> &sw,
                                             const typename Traits<DT>::frag (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                             float &m_ref, float &l_run, float scale_log2, int kvalid, int lane,
                                             const Mid &mid = Mid{}) {
    using Tr = Traits<DT>;
    using frag = typename Tr::frag;
    constexpr int NKB = 2, NDB = D / 32, TS = D / 16, TP = 2;
    const int h = lane >> 5;
    f32x16 s[NKB];
    if constexpr (FAST && !FIRST && !MASK) {
        // The steady tile of the fast pass in three phases of one kind each,
        // their order pinned by scheduling barriers: the score products back
        // to back with each K fragment read two products ahead; the softmax
        // as VALU work only; the P V products back to back with each V^T
        // fragment read two products ahead (the first two before the
        // softmax). VALU work between a wave's own products slows its matrix
        // stream, while the other wave of the SIMD fills the softmax phase
        // with its products (4% fewer cycles at N 4096, D 128 than the
        // compiler's interleaved schedule).
        constexpr int AK = 2, AV = 2, NP = NKB * TP * NDB;
        frag kq[NKB * TS], vq[NP];
        auto read_k = [&](int j) { kq[j] = sw.k(kt, j / TS, j % TS); };
        auto read_v = [&](int i) { vq[i] = sw.vt(vt, i / (TP * NDB), (i / NDB) % TP, i % NDB); };
#pragma unroll
        for (int j = 0; j < AK; ++j) read_k(j);
        s[0] = zero16();
        s[1] = zero16();
#pragma unroll
        for (int j = 0; j < NKB * TS; ++j) {
            if (j + AK < NKB * TS) read_k(j + AK);
            __builtin_amdgcn_sched_barrier(0);
            s[j / TS] = Tr::mfma(kq[j], qf[j % TS], s[j / TS]);
            __builtin_amdgcn_sched_barrier(0);
        }
        mid();
#pragma unroll
        for (int i = 0; i < AV; ++i) read_v(i);
        __builtin_amdgcn_sched_barrier(0);
        const float neg_m = -m_ref;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c) s[kb][c] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][c], scale_log2, neg_m));
        l_run += sum16(s[0]) + sum16(s[1]);
        frag pf[NKB][TP];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < TP; ++t) pf[kb][t] = c_to_frag<DT>(s[kb], t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i + AV < NP) read_v(i + AV);
            __builtin_amdgcn_sched_barrier(0);
            acc[i % NDB] = Tr::mfma(vq[i], pf[i / (TP * NDB)][(i / NDB) % TP], acc[i % NDB]);
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = zero16();
#pragma unroll
        for (int t = 0; t < TS; ++t) s[kb] = Tr::mfma(sw.k(kt, kb, t), qf[t], s[kb]);
    }
    mid();
    if constexpr (MASK) {
        // key row of register c: 32 kb + crow(c, h) = 32 kb + 8 (c / 4) + c % 4
        // + 4 h; one per-lane bound against constant offsets (no per-register
        // row index to keep live)
        const int kv = kvalid - 4 * h;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (32 * kb + 8 * (c >> 2) + (c & 3) >= kv) s[kb][c] = -INFINITY;
    }
    if constexpr (!FAST || FIRST) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c) mx = fmaxf(mx, s[kb][c]);
        const float mx2 = mx * scale_log2;
        if (__any(mx2 > m_ref + kRescaleLog2)) {
            __asm__ volatile("" ::: "memory");
            const float m_new = fmaxf(m_ref, xhalf_max(mx2));
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[db][c] *= alpha;
            l_run *= alpha;
            m_ref = m_new;
        }
    }
    const float neg_m = -m_ref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 16; ++c) s[kb][c] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][c], scale_log2, neg_m));
    // l: float32 sum of the probabilities before they are rounded for the
    // product
    l_run += sum16(s[0]) + sum16(s[1]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < TP; ++t) {
            const frag pf = c_to_frag<DT>(s[kb], t);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = Tr::mfma(sw.vt(vt, kb, t, db), pf, acc[db]);
        }
}

// Issues this wave's share of the DMA of K/V tile `tile` of a head (64 rows,
// PIECES 1 KiB pieces per tile and tensor, piece J to wave J % WAVES) into
// the stage arrays kd / vd. Bytes past the buffer's range read as zero.
template <Dt DT, int D, int WAVES>
__device__ __forceinline__ void fwd_dma_tile(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, int tile,
                                             char *kd, char *vd, int wv, int lane) {
    using Sw = SwzTile<DT, D>;
    constexpr int BYTES = Sw::BYTES, PIECES = Sw::PIECES;
    const uint32_t t0 = (uint32_t)tile * (uint32_t)BYTES;
#pragma unroll
    for (int j = 0; j < (PIECES + WAVES - 1) / WAVES; ++j) {
        const int J = wv + WAVES * j;
        if (PIECES % WAVES == 0 || J < PIECES) {
            const uint32_t off = t0 + Sw::piece_off(J, lane);
            dma16(krs, off, kd + 1024 * J);
            dma16(vrs, off, vd + 1024 * J);
        }
    }
}

// One pass of the 16-bit forward over the key tiles of one head on two DMA
// stages (tile it in K0/V0 for even it, K1/V1 for odd it), each stage its own
// LDS array so that the compiler can tell a stage being filled from the
// stage being read (it then keeps the DMA in flight across the reads instead
// of waiting for it). Step it issues the DMA of tile it + 1 into the other
// stage (last read in step it - 1, before that step's barrier), computes
// tile it, then waits for its own DMA pieces and meets the other waves at
// the tile's one barrier, which publishes tile it + 1. Past the last tile the
// DMA reads zeros (buffer range check) into a stage no later step reads.
// FASTP: pass 0 (reference max from the first tile); else the exact pass.
template <Dt DT, int D, int WAVES, bool FASTP>
__device__ __forceinline__ void fwd_pass2(char *K0, char *K1, char *V0, char *V1, __amdgpu_buffer_rsrc_t krs,
                                          __amdgpu_buffer_rsrc_t vrs, const SwzTile<DT, D> &sw,
                                          const typename Traits<DT>::frag (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                          float &m_ref, float &l_run, float scale_log2, int klen, int lane,
                                          int wv) {
    constexpr int BC = 64, NDB = D / 32;
    const int ntiles = (klen + BC - 1) / BC;
    const int nfull = klen / BC;
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = zero16();
    m_ref = -INFINITY;
    l_run = 0.f;
    fwd_dma_tile<DT, D, WAVES>(krs, vrs, 0, K0, V0, wv, lane);
    wait_dma();
    __syncthreads();
    lds_changed();
    auto step = [&](auto first_tag, auto odd_tag, int it) {
        constexpr bool FIRSTP = decltype(first_tag)::value;
        constexpr bool ODD = decltype(odd_tag)::value;
        // The scheduling barriers keep the DMA issue ahead of the tile and
        // the wait for it behind the tile's last products (left to itself
        // the compiler may sink the issue and hoist the wait, which then
        // stalls on the DMA right away).
        fwd_dma_tile<DT, D, WAVES>(krs, vrs, it + 1, ODD ? K0 : K1, ODD ? V0 : V1, wv, lane);
        __builtin_amdgcn_sched_barrier(0);
        fwd_tile_dma<DT, D, false, FASTP, FIRSTP>(ODD ? K1 : K0, ODD ? V1 : V0, sw, qf, acc, m_ref, l_run,
                                                   scale_log2, BC, lane);
        __builtin_amdgcn_sched_barrier(0);
        wait_dma();
        __syncthreads();
        lds_changed();
    };
    int it = 0;
    if (nfull > 0) {
        step(std::true_type{}, std::false_type{}, 0);
        it = 1;
    }
    for (; it + 1 < nfull; it += 2) {
        step(std::false_type{}, std::true_type{}, it);
        step(std::false_type{}, std::false_type{}, it + 1);
    }
    if (it < nfull) step(std::false_type{}, std::true_type{}, it++);
    // ragged last tile: the first and only one sets the reference max;
    // after full tiles pass 0 keeps the reference (no rescaling, which
    // could shrink an l that already exceeded the limit back under it)
    if (nfull < ntiles) {
        const int kv = klen - nfull * BC;
        if (FASTP && nfull > 0) {
            if (nfull & 1) fwd_tile_dma<DT, D, true, true, false>(K1, V1, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
            else fwd_tile_dma<DT, D, true, true, false>(K0, V0, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
        } else {
            if (nfull & 1) fwd_tile_dma<DT, D, true, false, true>(K1, V1, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
            else fwd_tile_dma<DT, D, true, false, true>(K0, V0, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
        }
    }
}

// Both passes of the 16-bit forward (see fwd_kernel) on DMA-filled tiles
// (buffer -> LDS DMA, no register staging): fwd_pass2 on two stages, or for
// 8-wave workgroups pass 0 on three stages with tiles fetched two ahead.
template <Dt DT, int D, int WAVES>
__device__ __forceinline__ void fwd_pass_dma(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                             const typename Traits<DT>::frag (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                             float &m_ref, float &l_run, float scale_log2, int klen, int lane,
                                             int wave) {
    using Sw = SwzTile<DT, D>;
    constexpr int BC = Sw::ROWS, BYTES = Sw::BYTES, PIECES = Sw::PIECES, NDB = D / 32;
    __shared__ __attribute__((aligned(1024))) char K0[BYTES];
    __shared__ __attribute__((aligned(1024))) char K1[BYTES];
    __shared__ __attribute__((aligned(1024))) char V0[BYTES];
    __shared__ __attribute__((aligned(1024))) char V1[BYTES];
    Sw sw;
    sw.init(lane);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ntiles = (klen + BC - 1) / BC;
    const int nfull = klen / BC;
    auto dma_tile = [&](int tile, char *kd, char *vd) { fwd_dma_tile<DT, D, WAVES>(krs, vrs, tile, kd, vd, wv, lane); };
    if constexpr (WAVES == 8 || (WAVES == 4 && D == 64)) {
        // Pass 0 of 8-wave workgroups (and of the 4-wave ones at head_dim 64,
        // two per CU: 48 KiB of LDS each) with tiles fetched two ahead: three
        // LDS stages (tile t in stage t % 3); step t issues the DMA of tile t + 2
        // into the stage of tile t - 1 (last read before the previous
        // barrier), computes tile t, then waits for tile t + 1's pieces only
        // (loads complete in order) and meets the others at the barrier.
        __shared__ __attribute__((aligned(1024))) char K2[BYTES];
        __shared__ __attribute__((aligned(1024))) char V2[BYTES];
        using F = std::false_type;
        using T = std::true_type;
        // DMA instructions per wave and tile (a wave with no piece has none
        // outstanding, so the count holds for every wave)
        constexpr int NPW = 2 * ((PIECES + WAVES - 1) / WAVES);
        static_assert((PIECES % WAVES == 0 || PIECES < WAVES) && NPW < 16, "pieces per wave");
        auto kst = [&](auto st) -> char * {
            constexpr int S = decltype(st)::value;
            if constexpr (S == 0) return K0;
            else if constexpr (S == 1) return K1;
            else return K2;
        };
        auto vst = [&](auto st) -> char * {
            constexpr int S = decltype(st)::value;
            if constexpr (S == 0) return V0;
            else if constexpr (S == 1) return V1;
            else return V2;
        };
#pragma unroll
        for (int i = 0; i < NDB; ++i) acc[i] = zero16();
        m_ref = -INFINITY;
        l_run = 0.f;
        dma_tile(0, K0, V0);
        dma_tile(1, K1, V1);
        __builtin_amdgcn_s_waitcnt(0x0f70 | NPW);  // tile 0 landed
        lds_changed();
        __builtin_amdgcn_s_barrier();
        lds_changed();
        auto step = [&](auto first_tag, auto stage_tag, int it) {
            constexpr int S = decltype(stage_tag)::value;
            using S2N = std::integral_constant<int, (S + 2) % 3>;
            dma_tile(it + 2, kst(S2N{}), vst(S2N{}));
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile_dma<DT, D, false, true, decltype(first_tag)::value>(kst(stage_tag), vst(stage_tag), sw, qf, acc,
                                                                         m_ref, l_run, scale_log2, BC, lane);
            __builtin_amdgcn_sched_barrier(0);
            // tile it + 1 landed (this wave's pieces; tile it + 2 stays in
            // flight), then a bare barrier: __syncthreads' release fence
            // would drain every outstanding DMA, tile it + 2's included. LDS
            // is written here only by the DMA, so no other store needs it.
            __builtin_amdgcn_s_waitcnt(0x0f70 | NPW);
            lds_changed();
            __builtin_amdgcn_s_barrier();
            lds_changed();
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        int it = 0;
        if (nfull > 0) step(T{}, S0{}, it++);
        for (; it + 2 < nfull; it += 3) {
            step(F{}, S1{}, it);
            step(F{}, S2{}, it + 1);
            step(F{}, S0{}, it + 2);
        }
        if (it < nfull) step(F{}, S1{}, it++);
        if (it < nfull) step(F{}, S2{}, it++);
        if (nfull < ntiles) {
            const int st = nfull % 3;
            const int kv = klen - nfull * BC;
            if (nfull == 0) fwd_tile_dma<DT, D, true, false, true>(K0, V0, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
            else if (st == 0) fwd_tile_dma<DT, D, true, true, false>(K0, V0, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
            else if (st == 1) fwd_tile_dma<DT, D, true, true, false>(K1, V1, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
            else fwd_tile_dma<DT, D, true, true, false>(K2, V2, sw, qf, acc, m_ref, l_run, scale_log2, kv, lane);
        }
        wait_dma();  // nothing left in flight past the pass
    } else {
        fwd_pass2<DT, D, WAVES, true>(K0, K1, V0, V1, krs, vrs, sw, qf, acc, m_ref, l_run, scale_log2, klen, lane, wv);
    }
    // a barrier for the whole workgroup either way: pass 1 refills the stages
    // l sums the float32 probabilities, so it bounds every one of them: at
    // or below the limit none overflowed the element type when rounded for
    // the product (f16 tops out at 65504, bf16 near 2^128)
    constexpr float kLim = DT == Dt::F16 ? 65504.f : 0x1p100f;
    const bool bad = !(l_run <= kLim);  // also true for inf and NaN
    if (__syncthreads_or(bad))
        fwd_pass2<DT, D, WAVES, false>(K0, K1, V0, V1, krs, vrs, sw, qf, acc, m_ref, l_run, scale_log2, klen, lane,
                                       wv);
}

// The float32 forward: padded tiles staged through registers (K row-major,
// V transposed so keys are contiguous) in two LDS stages, the exact
// recurrence (row max on every tile, lazy rescaling) in one pass. After each
// tile the next tile, already in registers, is stored into the other stage
// and the one after is fetched; one barrier per tile orders this tile's reads
// of a stage before that stage is refilled two tiles later. (float32 does
// not take the two-pass form of the 16-bit types: compiled that way, the
// first P V product of a pass read its accumulator input from a separate
// register block that the next LDS load and VALU results overwrote within
// 0-15 issue slots while the 16-pass f32 MFMA was still reading it, which
// corrupted output channels 16-23; tests/test_isa_srcc_war.py scans every
// kernel for that pattern.)
template <int D, int WAVES>
__device__ __forceinline__ void fwd_pass_f32(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                             const float (&qf)[D / 2], f32x16 (&acc)[D / 32], float &m_ref,
                                             float &l_run, float scale_log2, int klen, int lane, int tid) {
    constexpr Dt DT = Dt::F32;
    constexpr int BC = 64, NT = WAVES * 64, NDB = D / 32;
    constexpr int LDK = D + vec_elems<DT>();
    constexpr int LDV = fwd_ldv<DT, D, BC>();
    constexpr int KS = BC * LDK, VS = D * LDV;
    __shared__ __attribute__((aligned(16))) float Ks[2 * KS];
    __shared__ __attribute__((aligned(16))) float Vs[2 * VS];
    RowStage<DT, BC, D, NT> kst;
    TileStage<DT, BC, D, NT, false, stage_rows<DT, BC, D, NT>()> vst;
    const int ntiles = (klen + BC - 1) / BC;
    const int nfull = klen / BC;
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = zero16();
    m_ref = -INFINITY;
    l_run = 0.f;
    kst.load(krs, 0, tid);
    vst.load(vrs, 0, tid);
    kst.template store<LDK>(Ks, tid);
    vst.template store_transposed<LDV>(Vs, tid);
    if (ntiles > 1) {
        kst.load(krs, BC, tid);
        vst.load(vrs, BC, tid);
    }
    __syncthreads();
    for (int it = 0; it < nfull; ++it) {
        fwd_tile<DT, D, BC, false>(Ks + (it & 1) * KS, Vs + (it & 1) * VS, qf, acc, m_ref, l_run, scale_log2, BC,
                                   lane);
        if (it + 1 < ntiles) {
            kst.template store<LDK>(Ks + ((it + 1) & 1) * KS, tid);
            vst.template store_transposed<LDV>(Vs + ((it + 1) & 1) * VS, tid);
            if (it + 2 < ntiles) {
                kst.load(krs, (it + 2) * BC, tid);
                vst.load(vrs, (it + 2) * BC, tid);
            }
        }
        __syncthreads();
    }
    if (nfull < ntiles)
        fwd_tile<DT, D, BC, true>(Ks + (nfull & 1) * KS, Vs + (nfull & 1) * VS, qf, acc, m_ref, l_run, scale_log2,
                                  klen - nfull * BC, lane);
}

// PARTIAL: key-split mode. The key rows of a head are cut into nsplit
// consecutive ranges of split_len rows (a multiple of BC; the last range may
// be shorter); workgroup (bh, split, query block) runs the recurrence over
// its range only and writes the range's normalised output in float32 to
// O = Opart[nsplit][bh][n_q][D] and its log2-sum-exp, m + log2 l, to
// LSE = Lpart[nsplit][bh][n_q]. splitkv_combine_kernel merges the ranges.
template <Dt DT, int D, int BC, int WAVES, bool PARTIAL>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, void *__restrict__ O, float *__restrict__ LSE, int n_q,
    int n_k, int n_qblocks, int total_blocks, float scale_log2, int nsplit, int split_len) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr bool TR = sizeof(elem) == 2;  // 16-bit types: DMA-filled tiles
    constexpr int BR = 32 * WAVES;
    constexpr int NDB = D / 32;             // 32-row blocks of O^T
    constexpr int TS = D / (2 * Tr::KPL);   // contraction steps over head_dim
    static_assert(BC == 64 && D % 32 == 0, "tile shape");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    // Block order: query block fastest, then split, then head, so the
    // workgroups that share one key range sit next to each other (same XCD,
    // same L2).
    int bh, qb, split = 0, kbeg = 0, klen = n_k;
    if constexpr (PARTIAL) {
        qb = blk % n_qblocks;
        const int rest = blk / n_qblocks;
        split = rest % nsplit;
        bh = rest / nsplit;
        kbeg = split * split_len;
        klen = min(split_len, n_k - kbeg);
    } else {
        bh = blk / n_qblocks;
        qb = blk % n_qblocks;
    }
    const int qrow = qb * BR + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = ((int64_t)bh * n_k + kbeg) * D;

    frag qf[TS];
    if (qrow < n_q) {
        const elem *qp = Q + qoff + (int64_t)qrow * D;
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = ld_row_frag<DT>(qp, t, h);
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = zero_frag<DT>();
    }

    f32x16 acc[NDB];
    // m_ref: the reference max (log2 units) the probabilities of this row are
    // taken against; l_run: lane-partial sum of those probabilities.
    float m_ref, l_run;

    // K/V tiles: buffer loads over this head's rows (rows past n_k read as
    // zero).
    const uint32_t head_bytes = (uint32_t)klen * D * (uint32_t)sizeof(elem);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + koff, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + koff, head_bytes);
    // Pass 0 (16-bit types) takes the row max on the first tile only: later
    // probabilities (a ragged last tile's included) are 2^(s - m_ref) against
    // that reference as they are. The reference only scales every
    // probability of a row by the same power of two, which O = acc / l
    // cancels, so this is the same softmax as long as the values stay in
    // range. If some row of the workgroup ends with l above 2^100 (bf16) or
    // 65504 (f16, where a probability above it would not fit the element
    // type of the product) or not finite (a score about 100, or for f16 16,
    // or more above the first tile's max, in log2 units), the workgroup runs
    // pass 1: the recurrence with the max taken on every tile (lazy
    // rescaling). float32 runs that exact recurrence only.
    if constexpr (TR)
        fwd_pass_dma<DT, D, WAVES>(krs, vrs, qf, acc, m_ref, l_run, scale_log2, klen, lane, wave);
    else
        fwd_pass_f32<D, WAVES>(krs, vrs, qf, acc, m_ref, l_run, scale_log2, klen, lane, tid);

    const float l_tot = xhalf_sum(l_run);
    if (qrow < n_q) {
        const float inv = 1.f / l_tot;
        if constexpr (PARTIAL) {
            const int bh_count = total_blocks / (n_qblocks * nsplit);
            const int64_t prow = ((int64_t)split * bh_count + bh) * n_q + qrow;
            float *op = static_cast<float *>(O) + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) store4<Dt::F32>(op + 32 * db + 8 * g + 4 * h, acc[db], g, inv);
            if (h == 0) LSE[prow] = m_ref + __log2f(l_tot);
        } else {
            elem *op = static_cast<elem *>(O) + qoff + (int64_t)qrow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) store4<DT>(op + 32 * db + 8 * g + 4 * h, acc[db], g, inv);
            if (h == 0) LSE[(int64_t)bh * n_q + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
        }
    }
}

// Persistent form of the 8-wave 16-bit forward for key lengths that are a
// multiple of 256: one workgroup per CU (gridDim.x, a multiple of 8) walks
// query blocks, so that a block's start and end overlap the neighbouring
// blocks' work instead of leaving the CU idle. Four LDS stages: tile t of
// every block sits in stage t % 4, and the ring runs on across blocks: the
// block's last two steps fetch the next block's tiles 0 and 1, and the next
// block's Q rows are loaded into the Q registers right after the last tile's
// score products (their last use). The pass is pass 0 of fwd_kernel (row
// max on the first tile only); a block whose l leaves range is redone with
// the exact recurrence (fwd_pass2), after which the next block starts from
// scratch. Block order: workgroup g on XCD g % 8 takes blocks
// i * gridDim.x + (g % 8) * gridDim.x / 8 + g / 8, so that the workgroups of
// one XCD work on neighbouring blocks (one head's K/V in that XCD's L2).
constexpr int kStreamGrid = 256;  // one workgroup per CU

template <Dt DT, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_stream_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, typename Traits<DT>::elem *__restrict__ O,
    float *__restrict__ LSE, int n_q, int n_k, int n_qblocks, int total_blocks, float scale_log2) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using Sw = SwzTile<DT, D>;
    constexpr int WAVES = 8, BR = 32 * WAVES, BC = Sw::ROWS, NDB = D / 32, TS = D / 16;
    constexpr int BYTES = Sw::BYTES, PIECES = Sw::PIECES;
    constexpr int NPW = 2 * (PIECES / WAVES);  // DMA instructions per wave and tile
    static_assert(PIECES % WAVES == 0 && NPW + TS < 16, "pieces per wave");
    // 128 KiB of stages: the K tiles (declared first) land in the low 64 KiB
    // and the V tiles above, and the V^T read offsets carry the 64 KiB as a
    // bias (read address = (V stage - bias) + (offset + bias)), so every
    // fragment read is a base register plus a constant that fits the 16-bit
    // LDS offset field. With the stages in one 32 KiB block each, reads of
    // the upper two took a VALU add per read between the products (+3% cycles
    // at N 4096, D 128). The sums are the same under any placement; only the
    // add per read depends on it.
    __shared__ __attribute__((aligned(1024))) char K0[BYTES];
    __shared__ __attribute__((aligned(1024))) char K1[BYTES];
    __shared__ __attribute__((aligned(1024))) char K2[BYTES];
    __shared__ __attribute__((aligned(1024))) char K3[BYTES];
    __shared__ __attribute__((aligned(1024))) char V0[BYTES];
    __shared__ __attribute__((aligned(1024))) char V1[BYTES];
    __shared__ __attribute__((aligned(1024))) char V2[BYTES];
    __shared__ __attribute__((aligned(1024))) char V3[BYTES];
    __shared__ int bad_at;
    constexpr uint32_t kVBias = 4 * BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    Sw sw;
    sw.init(lane);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            sw.voff[db][hi] += kVBias;
            opaque(sw.voff[db][hi]);
        }
    const int ntiles = n_k / BC;
    const int G = gridDim.x;
    int L = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
    if (L >= total_blocks) return;

    const uint32_t kv_bytes = (uint32_t)n_k * D * (uint32_t)sizeof(elem);
    auto k_rsrc = [&](int blk) { return make_rsrc(K + (int64_t)(blk / n_qblocks) * n_k * D, kv_bytes); };
    auto v_rsrc = [&](int blk) { return make_rsrc(V + (int64_t)(blk / n_qblocks) * n_k * D, kv_bytes); };
    // Q rows of block blk (rows at or past n_q read as zero)
    auto q_rsrc = [&](int blk) {
        const int bh = blk / n_qblocks, q0 = (blk % n_qblocks) * BR;
        return make_rsrc(Q + ((int64_t)bh * n_q + q0) * D, (uint32_t)min(BR, n_q - q0) * D * (uint32_t)sizeof(elem));
    };
    // this lane's Q fragment t: row wave * 32 + col, columns 16 t + 8 h ..
    const uint32_t q_lane = (uint32_t)(((wave * 32 + col) * D + h * Tr::KPL) * (int)sizeof(elem));
    frag qf[TS];
    auto load_q = [&](__amdgpu_buffer_rsrc_t qr) {
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = __builtin_bit_cast(frag, buffer_load16(qr, q_lane + 32 * t));
    };
    auto dma_tile = [&](__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int tile, char *kd, char *vd) {
        fwd_dma_tile<DT, D, WAVES>(kr, vr, tile, kd, vd, wv, lane);
    };

    __amdgpu_buffer_rsrc_t krs = k_rsrc(L), vrs = v_rsrc(L);
    // start of the first block (and of any block after a redone one)
    auto restart = [&](bool publish_flag) {
        load_q(q_rsrc(L));
        dma_tile(krs, vrs, 0, K0, V0);
        dma_tile(krs, vrs, 1, K1, V1);
        if (publish_flag && tid == 0) bad_at = -1;
        // Q and tile 0 landed (loads complete in order), the flag written
        __builtin_amdgcn_s_waitcnt(0x0070 | NPW);
        lds_changed();
        __builtin_amdgcn_s_barrier();
        lds_changed();
    };
    restart(true);

    using F = std::false_type;
    using T = std::true_type;
    constexpr float kLim = DT == Dt::F16 ? 65504.f : 0x1p100f;
    f32x16 acc[NDB];
    float m_ref, l_run;
    for (int i = 0;; ++i) {
        const int Ln = L + G;
        const bool has_next = Ln < total_blocks;
        // past the last block the look-ahead reads zeros: tiles past this
        // head's end, and Q rows of an empty range
        const __amdgpu_buffer_rsrc_t nkrs = has_next ? k_rsrc(Ln) : krs;
        const __amdgpu_buffer_rsrc_t nvrs = has_next ? v_rsrc(Ln) : vrs;
        const int ntile0 = has_next ? 0 : ntiles;
        const __amdgpu_buffer_rsrc_t nqrs = has_next ? q_rsrc(Ln) : make_rsrc(Q, 0);

#pragma unroll
        for (int d = 0; d < NDB; ++d) acc[d] = zero16();
        m_ref = -INFINITY;
        l_run = 0.f;
        // step t: DMA of tile t + 2 (of this block, or tile t + 2 - ntiles of
        // the next) into stage (t + 2) % 4, last read in step t - 2; tile t;
        // wait for tile t + 1's pieces (WAITN: the loads issued after them,
        // tile t + 2's and, in the last step, the next block's Q); barrier
        auto step = [&](auto first_tag, auto stage_tag, auto waitn_tag, __amdgpu_buffer_rsrc_t kr,
                        __amdgpu_buffer_rsrc_t vr, int dtile, const auto &mid) {
            constexpr int S = decltype(stage_tag)::value;
            constexpr int WAITN = decltype(waitn_tag)::value;
            char *const kc = S == 0 ? K0 : S == 1 ? K1 : S == 2 ? K2 : K3;
            char *const vc = S == 0 ? V0 : S == 1 ? V1 : S == 2 ? V2 : V3;
            char *const kn = S == 0 ? K2 : S == 1 ? K3 : S == 2 ? K0 : K1;
            char *const vn = S == 0 ? V2 : S == 1 ? V3 : S == 2 ? V0 : V1;
            dma_tile(kr, vr, dtile, kn, vn);
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile_dma<DT, D, false, true, decltype(first_tag)::value>(kc, vc - kVBias, sw, qf, acc, m_ref, l_run,
                                                                         scale_log2, BC, lane, mid);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x0f70 | WAITN);
            lds_changed();
            __builtin_amdgcn_s_barrier();
            lds_changed();
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        using C3 = std::integral_constant<int, 3>;
        using WN = std::integral_constant<int, NPW>;
        using WQ = std::integral_constant<int, NPW + TS>;
        const NoMid none;
        step(T{}, C0{}, WN{}, krs, vrs, 2, none);
        int t = 1;
        for (; t + 6 < ntiles; t += 4) {
            step(F{}, C1{}, WN{}, krs, vrs, t + 2, none);
            step(F{}, C2{}, WN{}, krs, vrs, t + 3, none);
            step(F{}, C3{}, WN{}, krs, vrs, t + 4, none);
            step(F{}, C0{}, WN{}, krs, vrs, t + 5, none);
        }
        step(F{}, C1{}, WN{}, krs, vrs, ntiles - 1, none);
        step(F{}, C2{}, WN{}, nkrs, nvrs, ntile0, none);
        step(F{}, C3{}, WQ{}, nkrs, nvrs, ntile0 + 1, [&]() { load_q(nqrs); });

        // l sums the float32 probabilities: at or below the limit none of
        // them overflowed the element type when rounded for the product
        if (__any(!(l_run <= kLim)) && lane == 0) bad_at = i;
        lds_changed();
        __builtin_amdgcn_s_waitcnt(0xc07f);  // the flag written (lgkmcnt 0)
        __builtin_amdgcn_s_barrier();
        lds_changed();
        const bool redo = __builtin_amdgcn_readfirstlane(bad_at) == i;
        if (redo) {
            wait_dma();
            load_q(q_rsrc(L));
            Sw sw0;  // unbiased offsets
            sw0.init(lane);
            fwd_pass2<DT, D, WAVES, false>(K0, K1, V0, V1, krs, vrs, sw0, qf, acc, m_ref, l_run, scale_log2, n_k,
                                           lane, wv);
        }

        // the next block's Q rows and tile 1 landed (issued during the last
        // tile): waiting here, before the stores, keeps the next block's
        // first products from waiting on the stores as well
        wait_dma();
        const float l_tot = xhalf_sum(l_run);
        const int qrow = (L % n_qblocks) * BR + wave * 32 + col;
        if (qrow < n_q) {
            const int64_t row = (int64_t)(L / n_qblocks) * n_q + qrow;
            const float inv = 1.f / l_tot;
            elem *op = O + row * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) store4<DT>(op + 32 * db + 8 * g + 4 * h, acc[db], g, inv);
            if (h == 0) LSE[row] = (m_ref + __log2f(l_tot)) * kLn2;
        }
        if (!has_next) break;
        L = Ln;
        krs = nkrs;
        vrs = nvrs;
        if (redo) restart(false);
    }
    wait_dma();  // nothing left in flight at the end
}

// Merge of a key-split forward's ranges (the log-sum-exp combination of
// partial softmax results; exact up to rounding). Per query row, with L_s the
// log2-sum-exp of range s and O_s its normalised output:
//   L = log2 sum_s 2^(L_s),  O = sum_s 2^(L_s - L) O_s,  lse = ln2 * L.
// D/4 threads per row, 4 consecutive columns each.
template <Dt DT, int D>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(const float *__restrict__ Opart,
                                                              const float *__restrict__ Lpart,
                                                              typename Traits<DT>::elem *__restrict__ O,
                                                              float *__restrict__ LSE, int64_t rows, int nsplit) {
    constexpr int TPR = D / 4;
    constexpr int RPB = 256 / TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * 4;
    if (row >= rows) return;
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, Lpart[s * rows + row]);
    float sum = 0.f;
    f32x16 acc = zero16();  // only entries 0..3 are used (store4 group 0)
    for (int s = 0; s < nsplit; ++s) {
        const float w = exp2f(Lpart[s * rows + row] - mx);
        const float4 o = *reinterpret_cast<const float4 *>(Opart + (s * rows + row) * D + c0);
        sum += w;
        acc[0] = __builtin_fmaf(w, o.x, acc[0]);
        acc[1] = __builtin_fmaf(w, o.y, acc[1]);
        acc[2] = __builtin_fmaf(w, o.z, acc[2]);
        acc[3] = __builtin_fmaf(w, o.w, acc[3]);
    }
    store4<DT>(O + row * D + c0, acc, 0, 1.f / sum);
    if (c0 == 0) LSE[row] = (mx + log2f(sum)) * kLn2;
}

template <Dt DT, int D, int WAVES>
static hipError_t fwd_launch(const void *q, const void *k, const void *v, void *o, float *lse, const AttnShape &s,
                             hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BC = 64, BR = 32 * WAVES;
    const int nqb = (s.n_q + BR - 1) / BR;
    const int total = (int)(s.bh * nqb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((fwd_kernel<DT, D, BC, WAVES, false>), dim3(total), dim3(WAVES * 64), 0, stream,
                       (const elem *)q, (const elem *)k, (const elem *)v, o, lse, s.n_q, s.n_k, nqb, total,
                       scale_log2, 1, s.n_k);
    return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t fwd_stream_launch(const void *q, const void *k, const void *v, void *o, float *lse,
                                    const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    const int nqb = (s.n_q + 255) / 256;
    const int total = (int)(s.bh * nqb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((fwd_stream_kernel<DT, D>), dim3(kStreamGrid), dim3(512), 0, stream, (const elem *)q,
                       (const elem *)k, (const elem *)v, (elem *)o, lse, s.n_q, s.n_k, nqb, total, scale_log2);
    return hipGetLastError();
}

// Workgroup size by problem size: 8 waves (256 query rows, K/V tiles shared by
// the most rows) when that still gives every CU at least two workgroups,
// else 4 or 2 waves so that small problems still spread over the chip.
template <Dt DT, int D>
static hipError_t fwd_dispatch(const void *q, const void *k, const void *v, void *o, float *lse,
                               const AttnShape &s, hipStream_t stream) {
    constexpr int64_t kCus = 256;
    // head_dim 64 keeps two 4-wave workgroups per CU instead of one 8-wave
    // one: its tile is softmax-bound (half the products of head_dim 128 per
    // exponential), and waves of two workgroups, which meet at different
    // barriers, fill each other's softmax phases better (cross-attention,
    // 1024 x 8192 keys: 9% fewer kernel cycles, 2% less time; at head_dim
    // 128 the 4-wave launch is 5% slower)
    if constexpr (D == 128 && DT != Dt::F32) {
        // key lengths in whole groups of four tiles and at least two query
        // blocks per CU: the persistent launch, which overlaps each block's
        // start and end with its neighbours' tiles (BH 512, N 4096, D 128:
        // 5% fewer kernel cycles, 3% less time than one workgroup per block)
        if (s.n_k >= 256 && s.n_k % 256 == 0 && s.bh * ((s.n_q + 255) / 256) >= 2 * kStreamGrid)
            return fwd_stream_launch<DT, D>(q, k, v, o, lse, s, stream);
    }
    if (D != 64 && s.bh * ((s.n_q + 255) / 256) >= 2 * kCus) return fwd_launch<DT, D, 8>(q, k, v, o, lse, s, stream);
    if (s.bh * ((s.n_q + 127) / 128) >= kCus) return fwd_launch<DT, D, 4>(q, k, v, o, lse, s, stream);
    return fwd_launch<DT, D, 2>(q, k, v, o, lse, s, stream);
}

// Key-split forward: partial pass over sp.nsplit key ranges into the
// workspace, then the combine pass into o and lse.
template <Dt DT, int D, int WAVES>
static hipError_t splitkv_launch(const void *q, const void *k, const void *v, void *o, float *lse, float *ws,
                                 const AttnShape &s, const SplitPlan &sp, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BC = 64, BR = 32 * WAVES;
    static_assert(BC == kSplitKeyAlign, "key ranges must start on tile boundaries");
    const int nqb = (s.n_q + BR - 1) / BR;
    const int total = (int)(s.bh * nqb * sp.nsplit);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    const int64_t rows = s.bh * s.n_q;
    float *opart = ws;
    float *lpart = ws + (int64_t)sp.nsplit * rows * D;
    hipLaunchKernelGGL((fwd_kernel<DT, D, BC, WAVES, true>), dim3(total), dim3(WAVES * 64), 0, stream,
                       (const elem *)q, (const elem *)k, (const elem *)v, (void *)opart, lpart, s.n_q, s.n_k, nqb,
                       total, scale_log2, sp.nsplit, sp.split_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int RPB = 256 / (D / 4);
    hipLaunchKernelGGL((splitkv_combine_kernel<DT, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       stream, (const float *)opart, (const float *)lpart, (elem *)o, lse, rows, sp.nsplit);
    return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t splitkv_dispatch(const void *q, const void *k, const void *v, void *o, float *lse, float *ws,
                                   const AttnShape &s, const SplitPlan &sp, hipStream_t stream) {
    if (sp.nsplit == 1) return fwd_dispatch<DT, D>(q, k, v, o, lse, s, stream);
    switch (sp.waves) {
        case 2: return splitkv_launch<DT, D, 2>(q, k, v, o, lse, ws, s, sp, stream);
        case 4: return splitkv_launch<DT, D, 4>(q, k, v, o, lse, ws, s, sp, stream);
        case 8: return splitkv_launch<DT, D, 8>(q, k, v, o, lse, ws, s, sp, stream);
        default: return hipErrorInvalidValue;
    }
}

template <Dt DT>
static hipError_t splitkv_by_dim(const void *q, const void *k, const void *v, void *o, float *lse, float *ws,
                                 const AttnShape &s, const SplitPlan &sp, hipStream_t stream) {
    switch (s.head_dim) {
        case 32: return splitkv_dispatch<DT, 32>(q, k, v, o, lse, ws, s, sp, stream);
        case 64: return splitkv_dispatch<DT, 64>(q, k, v, o, lse, ws, s, sp, stream);
        case 128: return splitkv_dispatch<DT, 128>(q, k, v, o, lse, ws, s, sp, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd_splitkv(int dt, const void *q, const void *k, const void *v, void *o, float *lse, float *ws,
                              const AttnShape &s, const SplitPlan &sp, hipStream_t stream) {
    switch (dt) {
        case 0: return splitkv_by_dim<Dt::F32>(q, k, v, o, lse, ws, s, sp, stream);
        case 1: return splitkv_by_dim<Dt::F16>(q, k, v, o, lse, ws, s, sp, stream);
        case 2: return splitkv_by_dim<Dt::BF16>(q, k, v, o, lse, ws, s, sp, stream);
        default: return hipErrorInvalidValue;
    }
}

template <Dt DT>
static hipError_t fwd_by_dim(const void *q, const void *k, const void *v, void *o, float *lse,
                             const AttnShape &s, hipStream_t stream) {
    switch (s.head_dim) {
        case 32: return fwd_dispatch<DT, 32>(q, k, v, o, lse, s, stream);
        case 64: return fwd_dispatch<DT, 64>(q, k, v, o, lse, s, stream);
        case 128: return fwd_dispatch<DT, 128>(q, k, v, o, lse, s, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd(int dt, const void *q, const void *k, const void *v, void *o, float *lse,
                      const AttnShape &s, hipStream_t stream) {
    switch (dt) {
        case 0: return fwd_by_dim<Dt::F32>(q, k, v, o, lse, s, stream);
        case 1: return fwd_by_dim<Dt::F16>(q, k, v, o, lse, s, stream);
        case 2: return fwd_by_dim<Dt::BF16>(q, k, v, o, lse, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa2mi
