// Attention backward (vision-rs flash_attn2.rs, "Backward - dQ" and
// "Backward - dK / dV"), recomputing the probabilities from the saved LSE:
//   p_ij  = exp(scale q_i.k_j - lse_i)
//   dS_ij = p_ij (dO_i.v_j - delta_i),     delta_i = O_i.dO_i
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_i dS_ij q_i,         dV_j = sum_i p_ij dO_i
// Three deterministic passes, no atomics:
//   delta_kernel - delta_i = rowsum(O * dO) (fp32), read by both others;
//   dq_kernel    - one workgroup per 32*WAVES query rows, looping over key
//                  tiles (the forward's structure with dS in place of P);
//                  dq_stream_kernel, its persistent form at head_dim 128,
//                  walks query blocks with one workgroup per CU;
//   dkdv_kernel  - one workgroup per 32*WAVES key rows, looping over query
//                  tiles; K and V of the wave's 32 keys stay in registers.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2mi {

template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag zero_frag_b() {
    typename Traits<DT>::frag f;
    if constexpr (Traits<DT>::KPL == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<typename Traits<DT>::elem>(0.f);
    } else {
        f = 0.f;
    }
    return f;
}

template <Dt DT>
__device__ __forceinline__ void store4_b(typename Traits<DT>::elem *dst, const f32x16 &c, int g, float mul) {
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

// ---------------------------------------------------------------------------
// delta_i = sum_d O_id dO_id. TPR lanes share one row, one 16-byte vector each.
template <Dt DT, int D>
__global__ __launch_bounds__(256) void delta_kernel(const typename Traits<DT>::elem *__restrict__ O,
                                                    const typename Traits<DT>::elem *__restrict__ dO,
                                                    float *__restrict__ delta, int64_t rows) {
    using elem = typename Traits<DT>::elem;
    constexpr int VEC = vec_elems<DT>();
    constexpr int TPR = D / VEC;  // lanes per row (<= 32)
    constexpr int RPB = 256 / TPR;
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
    const int sub = tid % TPR;
    float acc = 0.f;
    if (row < rows) {
        const uint4 a = *reinterpret_cast<const uint4 *>(O + row * D + sub * VEC);
        const uint4 b = *reinterpret_cast<const uint4 *>(dO + row * D + sub * VEC);
        const elem *ea = reinterpret_cast<const elem *>(&a);
        const elem *eb = reinterpret_cast<const elem *>(&b);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc += static_cast<float>(ea[i]) * static_cast<float>(eb[i]);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && sub == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// Shared pieces of the two gradient kernels. Tiles come in through raw
// buffer loads over one head's rows (rows past the end read as zero) and sit
// row-major in LDS in two stages; transposed MFMA operands are read from the
// row-major tiles with ds_read_b64_tr_b16 (16-bit types) or, for float32,
// from a transposed copy. No masking is needed: a key past n_k has zero K
// and V rows and so adds nothing to dQ; a query past n_q has zero Q and dO
// rows and so adds nothing to dK or dV.

// Tile access for the gradient kernels. 16-bit types: padded row-major tiles
// read as rows (ds_read_b128) and, for transposed operands, with
// ds_read_b64_tr_b16. The gfx950 LDS behaves as 64 four-byte banks;
// ds_read_b128 serves 16 lanes per cycle (16 consecutive rows, one 16-byte
// chunk each) and ds_read_b64_tr_b16 32 lanes per cycle (4 consecutive rows,
// 64 bytes each). Two layouts:
//  SHIFT: the row stride is an odd multiple of 64 bytes (the transposing
//    reads' 4 rows fill 256 bytes) and rows are shifted by row_shift (the 16
//    rows of a row read fill 16 distinct 16-byte slots): no bank conflict
//    for either pattern (dkdv, 1.8% faster at N 4096, D 128);
//  plain: a row stride of an odd number of 16-byte chunks (19 at D = 128,
//    9 at 64, 5 at 32): row reads conflict-free, transposing reads at most
//    2-way, less address arithmetic (dq, 0.8% faster than shifted).
// float32: padded row-major tiles plus a transposed copy (stride LDT).
template <Dt DT, int D, bool SHIFT>
struct BwdTile {
    using elem = typename Traits<DT>::elem;
    using frag = typename Traits<DT>::frag;
    static constexpr bool TR = sizeof(elem) == 2;
    static constexpr bool SH = TR && SHIFT;
    static constexpr int VEC = vec_elems<DT>();
    // shifted: the smallest odd multiple of 64 bytes that holds a row plus
    // the largest shift (48 bytes)
    static constexpr int LD_UNITS = (2 * D + 48 + 63) / 64;
    static constexpr int LD =
        SH ? 32 * (LD_UNITS | 1) : (TR ? (D == 128 ? D + 3 * VEC : D + VEC) : D + VEC);  // row stride

    __device__ static __forceinline__ const elem *row_ptr(const elem *tile, int row) {
        if constexpr (SH)
            return tile + row * LD + row_shift(row);
        else
            return tile + row * LD;
    }

    // row fragment (contraction step t over head_dim) of tile row `row`
    __device__ static __forceinline__ frag row(const elem *tile, int row, int t, int h) {
        return ld_row_frag<DT>(row_ptr(tile, row), t, h);
    }

    // A fragment of T^T: columns 32db.. of the tile x its rows 32kb + 16t ..
    // in the row order of C-block registers fed back as B operands
    template <int LDT>
    __device__ static __forceinline__ frag trans(const elem *tile, const elem *ttile, int kb, int t, int db,
                                                 int lane) {
        if constexpr (SH) {
            (void)ttile;
            return ld_vt_frag_tr_sh<DT>(tile, LD, 32 * kb + 16 * t, 32 * db, lane);
        } else if constexpr (TR) {
            (void)ttile;
            return ld_vt_frag_tr<DT>(tile, LD, 32 * kb + 16 * t, 32 * db, lane);
        } else {
            (void)tile;
            return ld_t_frag<DT>(ttile + (32 * db + (lane & 31)) * LDT, kb, t, lane >> 5);
        }
    }

    template <int R, int NT>
    __device__ static __forceinline__ void store(const RowStage<DT, R, D, NT> &st, elem *tile, int tid) {
        using St = RowStage<DT, R, D, NT>;
        if constexpr (SH) {
#pragma unroll
            for (int i = 0; i < St::PER_THREAD; ++i) {
                const int pc = tid + i * NT;
                const int row = pc / (D / VEC), cv = pc % (D / VEC);
                if (St::PIECES % NT == 0 || pc < St::PIECES)
                    *reinterpret_cast<uint4 *>(tile + row * LD + row_shift(row) + cv * VEC) = st.v[i];
            }
        } else {
            st.template store<LD>(tile, tid);
        }
    }
};

// dQ over DMA-filled tiles (16-bit types): K and V tiles of 64 keys go
// straight from memory into unpadded swizzled LDS tiles (SwzTile), one LDS
// array per stage, with the forward's step structure (fwd_pass_dma): step it
// issues the DMA of tile it + 1 into the other stage, computes tile it, waits
// for its own DMA pieces and meets the other waves at the tile's one barrier.
// Keys past n_k read as zero rows and add nothing to dQ.
template <Dt DT, int D, int WAVES>
__device__ __forceinline__ void dq_pass_dma(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                            const typename Traits<DT>::frag (&qf)[D / 16],
                                            const typename Traits<DT>::frag (&df)[D / 16], float lse2, float dl,
                                            f32x16 (&acc)[D / 32], float scale_log2, int n_k, int lane, int wave) {
    using Tr = Traits<DT>;
    using frag = typename Tr::frag;
    using Sw = SwzTile<DT, D>;
    constexpr int BC = Sw::ROWS, BYTES = Sw::BYTES, PIECES = Sw::PIECES, NDB = D / 32, TS = D / 16;
    __shared__ __attribute__((aligned(1024))) char K0[BYTES];
    __shared__ __attribute__((aligned(1024))) char K1[BYTES];
    __shared__ __attribute__((aligned(1024))) char V0[BYTES];
    __shared__ __attribute__((aligned(1024))) char V1[BYTES];
    Sw sw;
    sw.init(lane);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ntiles = (n_k + BC - 1) / BC;
    auto dma_tile = [&](int tile, char *kd, char *vd) {
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
    };
    // One 64-key tile, per 32-key block kb in phases of one kind each, their
    // order pinned by scheduling barriers: the S products, the dP products,
    // the softmax and dS as VALU work only, the dQ products. Every LDS
    // operand is read two products ahead, the next block's first ones
    // during the current block's last products, from the precomputed
    // per-lane offsets. VALU work between a wave's own products (an
    // interleaved exponential, or an address XOR) slows its matrix stream;
    // the other wave of the SIMD fills the softmax phase (12% fewer cycles
    // at N 4096, D 128 than the compiler's interleaved schedule).
    auto tile_fn = [&](const char *kt, const char *vt) {
        constexpr int AHEAD = 2;
        constexpr int OPK = 2 * TS + 2 * NDB, NOP = 2 * OPK;  // operands per key block / per tile
        frag op[NOP];
        // operand j: key block j / OPK; then K (S), V (dP), transposed K (dQ)
        auto read = [&](int j) {
            const int kb = j / OPK, r = j % OPK;
            if (r < TS)
                op[j] = sw.k(kt, kb, r);
            else if (r < 2 * TS)
                op[j] = sw.k(vt, kb, r - TS);
            else
                op[j] = sw.vt(kt, kb, (r - 2 * TS) / NDB, (r - 2 * TS) % NDB);
        };
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) read(j);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int base = kb * OPK;
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                if (base + t + AHEAD < NOP) read(base + t + AHEAD);
                __builtin_amdgcn_sched_barrier(0);
                s = Tr::mfma(op[base + t], qf[t], s);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const int j = base + TS + t;
                if (j + AHEAD < NOP) read(j + AHEAD);
                __builtin_amdgcn_sched_barrier(0);
                dp = Tr::mfma(op[j], df[t], dp);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lse2));
                s[c] = p * (dp[c] - dl);
            }
            const frag dsf[2] = {c_to_frag<DT>(s, 0), c_to_frag<DT>(s, 1)};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 2 * NDB; ++i) {
                const int j = base + 2 * TS + i;
                if (j + AHEAD < NOP) read(j + AHEAD);
                __builtin_amdgcn_sched_barrier(0);
                acc[i % NDB] = Tr::mfma(op[j], dsf[i / NDB], acc[i % NDB]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    dma_tile(0, K0, V0);
    wait_dma();
    __syncthreads();
    lds_changed();
    // stage of tile it: K0/V0 for even it, K1/V1 for odd it
    auto step = [&](auto odd_tag, int it) {
        constexpr bool ODD = decltype(odd_tag)::value;
        dma_tile(it + 1, ODD ? K0 : K1, ODD ? V0 : V1);
        __builtin_amdgcn_sched_barrier(0);
        tile_fn(ODD ? K1 : K0, ODD ? V1 : V0);
        __builtin_amdgcn_sched_barrier(0);
        wait_dma();
        __syncthreads();
        lds_changed();
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        step(std::false_type{}, it);
        step(std::true_type{}, it + 1);
    }
    if (it < ntiles) step(std::false_type{}, it);
}

// dQ for float32: padded K and V tiles staged through registers plus a
// transposed K copy (BwdTile), two LDS stages, one barrier per tile.
template <int D, int BC, int WAVES>
__device__ __forceinline__ void dq_pass_f32(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                            const float (&qf)[D / 2], const float (&df)[D / 2], float lse2, float dl,
                                            f32x16 (&acc)[D / 32], float scale_log2, int n_k, int lane, int tid) {
    constexpr Dt DT = Dt::F32;
    using Tr = Traits<DT>;
    constexpr int NT = WAVES * 64;
    using Tl = BwdTile<DT, D, false>;
    constexpr int LDT = BC + 4;          // transposed K copy
    constexpr int KS = BC * Tl::LD;
    constexpr int TSZ = D * LDT;
    constexpr int NKB = BC / 32, NDB = D / 32, TS = D / 2, TP = 16;
    __shared__ __attribute__((aligned(16))) float Ks[2 * KS];
    __shared__ __attribute__((aligned(16))) float Vs[2 * KS];
    __shared__ __attribute__((aligned(16))) float Kt[2 * TSZ];
    const int h = lane >> 5, col = lane & 31;
    RowStage<DT, BC, D, NT> kst, vst;
    TileStage<DT, BC, D, NT, false, stage_rows<DT, BC, D, NT>()> ktst;
    auto load = [&](int row0) {
        kst.load(krs, row0, tid);
        vst.load(vrs, row0, tid);
        ktst.load(krs, row0, tid);
    };
    auto store = [&](int stage) {
        Tl::store(kst, Ks + stage * KS, tid);
        Tl::store(vst, Vs + stage * KS, tid);
        ktst.template store_transposed<LDT>(Kt + stage * TSZ, tid);
    };
    const int ntiles = (n_k + BC - 1) / BC;
    load(0);
    store(0);
    if (ntiles > 1) load(BC);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int st = it & 1;
        const float *kt = Ks + st * KS, *vt = Vs + st * KS, *ktt = Kt + st * TSZ;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                s = Tr::mfma(Tl::row(kt, 32 * kb + col, t, h), qf[t], s);
                dp = Tr::mfma(Tl::row(vt, 32 * kb + col, t, h), df[t], dp);
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lse2));
                s[c] = p * (dp[c] - dl);
            }
#pragma unroll
            for (int t = 0; t < TP; ++t) {
                const float dsf = c_to_frag<DT>(s, t);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = Tr::mfma(Tl::template trans<LDT>(kt, ktt, kb, t, db, lane), dsf, acc[db]);
            }
        }
        if (it + 1 < ntiles) {
            store((it + 1) & 1);
            if (it + 2 < ntiles) load((it + 2) * BC);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// dQ: per workgroup BR = 32*WAVES query rows (one 32-row block per wave, each
// lane owning one query column), looping over key tiles of BC rows:
//   S^T = K Q^T, dP^T = V dO^T (K, V row-major A operands from LDS; Q, dO
//   B operands from registers), P = 2^(S*scale*log2e - lse*log2e),
//   dS = P (dP - delta), dQ^T += K^T dS^T (K^T via transposing reads).
template <Dt DT, int D, int BC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, const typename Traits<DT>::elem *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Delta, typename Traits<DT>::elem *__restrict__ dQ,
    int n_q, int n_k, int n_qblocks, int total_blocks, float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr bool TR = sizeof(elem) == 2;
    constexpr int BR = 32 * WAVES;
    constexpr int NDB = D / 32;
    constexpr int TS = D / (2 * Tr::KPL);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_qblocks, qb = blk % n_qblocks;
    const int qrow = qb * BR + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = (int64_t)bh * n_k * D;
    const bool qvalid = qrow < n_q;

    frag qf[TS], df[TS];
    // invalid rows: zero operands and lse = +inf, so every P is 0
    float lse2 = INFINITY, dl = 0.f;
    if (qvalid) {
        const elem *qp = Q + qoff + (int64_t)qrow * D;
        const elem *dp = dO + qoff + (int64_t)qrow * D;
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            qf[t] = ld_row_frag<DT>(qp, t, h);
            df[t] = ld_row_frag<DT>(dp, t, h);
        }
        lse2 = LSE[(int64_t)bh * n_q + qrow] * kLog2e;
        dl = Delta[(int64_t)bh * n_q + qrow];
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = df[t] = zero_frag_b<DT>();
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = zero16();

    const uint32_t head_bytes = (uint32_t)n_k * D * (uint32_t)sizeof(elem);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + koff, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + koff, head_bytes);
    if constexpr (TR) {
        static_assert(BC == 64, "DMA tiles hold 64 keys");
        dq_pass_dma<DT, D, WAVES>(krs, vrs, qf, df, lse2, dl, acc, scale_log2, n_k, lane, wave);
    } else {
        dq_pass_f32<D, BC, WAVES>(krs, vrs, qf, df, lse2, dl, acc, scale_log2, n_k, lane, tid);
    }

    if (qvalid) {
        elem *op = dQ + qoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) store4_b<DT>(op + 32 * db + 8 * g + 4 * h, acc[db], g, scale);
    }
}

// ---------------------------------------------------------------------------
// Persistent form of the 8-wave 16-bit dQ at head_dim 128 (as the forward's
// fwd_stream_kernel), for key lengths that are a multiple of 256 with at
// least two 256-row query blocks per CU: one workgroup per CU walks query
// blocks i * gridDim.x + (g % 8) * gridDim.x / 8 + g / 8, so a block's start
// and end overlap the neighbouring blocks' tiles. Four LDS stages (tile t of
// every block in stage t % 4, fetched two ahead, one barrier per tile); a
// block's last two steps fetch the next block's tiles 0 and 1, and the next
// block's Q, dO, lse and delta are loaded into their registers during the
// last tile, each right after its last use (Q after the second key block's
// score products, dO after its dP products, lse and delta after its dS).
// K stages sit in the low 64 KiB and V stages above; V is read with row
// offsets that carry the 64 KiB as a bias, so every LDS read folds its
// constant into the 16-bit offset field.
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// One 64-key tile of dQ (as dq_pass_dma's tile): swk reads K (rows and
// transposed), swv the V rows of a tile addressed vt - bias. Hooks run after
// the second key block's S products (hq), dP products (hd) and dS (hl).
template <Dt DT, int D, class HQ, class HD, class HL>
__device__ __forceinline__ void dq_tile_stream(const char *kt, const char *vt, const SwzTile<DT, D> &swk,
                                               const SwzTile<DT, D> &swv,
                                               const typename Traits<DT>::frag (&qf)[D / 16],
                                               const typename Traits<DT>::frag (&df)[D / 16], float lse2, float dl,
                                               f32x16 (&acc)[D / 32], float scale_log2, const HQ &hq, const HD &hd,
                                               const HL &hl) {
    using Tr = Traits<DT>;
    using frag = typename Tr::frag;
    constexpr int NDB = D / 32, TS = D / 16, AHEAD = 2;
    constexpr int OPK = 2 * TS + 2 * NDB, NOP = 2 * OPK;  // operands per key block / per tile
    frag op[NOP];
    // operand j: key block j / OPK; then K (S), V (dP), transposed K (dQ)
    auto read = [&](int j) {
        const int kb = j / OPK, r = j % OPK;
        if (r < TS)
            op[j] = swk.k(kt, kb, r);
        else if (r < 2 * TS)
            op[j] = swv.k(vt, kb, r - TS);
        else
            op[j] = swk.vt(kt, kb, (r - 2 * TS) / NDB, (r - 2 * TS) % NDB);
    };
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) read(j);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int base = kb * OPK;
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            if (base + t + AHEAD < NOP) read(base + t + AHEAD);
            __builtin_amdgcn_sched_barrier(0);
            s = Tr::mfma(op[base + t], qf[t], s);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kb == 1) {
            hq();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            const int j = base + TS + t;
            if (j + AHEAD < NOP) read(j + AHEAD);
            __builtin_amdgcn_sched_barrier(0);
            dp = Tr::mfma(op[j], df[t], dp);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kb == 1) {
            hd();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lse2));
            s[c] = p * (dp[c] - dl);
        }
        const frag dsf[2] = {c_to_frag<DT>(s, 0), c_to_frag<DT>(s, 1)};
        if (kb == 1) hl();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * NDB; ++i) {
            const int j = base + 2 * TS + i;
            if (j + AHEAD < NOP) read(j + AHEAD);
            __builtin_amdgcn_sched_barrier(0);
            acc[i % NDB] = Tr::mfma(op[j], dsf[i / NDB], acc[i % NDB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

constexpr int kDqStreamGrid = 256;  // one workgroup per CU

template <Dt DT, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_stream_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, const typename Traits<DT>::elem *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Delta, typename Traits<DT>::elem *__restrict__ dQ,
    int n_q, int n_k, int n_qblocks, int total_blocks, float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using Sw = SwzTile<DT, D>;
    constexpr int WAVES = 8, BR = 32 * WAVES, BC = Sw::ROWS, NDB = D / 32, TS = D / 16;
    constexpr int BYTES = Sw::BYTES, PIECES = Sw::PIECES;
    constexpr int NPW = 2 * (PIECES / WAVES);  // DMA instructions per wave and tile
    constexpr int NQ = 2 * TS + 2;             // loads of a block's Q, dO, lse and delta per lane
    static_assert(PIECES % WAVES == 0 && NPW + NQ < 64 && NPW < 16, "pieces per wave");
    __shared__ __attribute__((aligned(1024))) char K0[BYTES];
    __shared__ __attribute__((aligned(1024))) char K1[BYTES];
    __shared__ __attribute__((aligned(1024))) char K2[BYTES];
    __shared__ __attribute__((aligned(1024))) char K3[BYTES];
    __shared__ __attribute__((aligned(1024))) char V0[BYTES];
    __shared__ __attribute__((aligned(1024))) char V1[BYTES];
    __shared__ __attribute__((aligned(1024))) char V2[BYTES];
    __shared__ __attribute__((aligned(1024))) char V3[BYTES];
    constexpr uint32_t kVBias = 4 * BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    Sw swk;
    swk.init(lane);
    Sw swv = swk;
#pragma unroll
    for (int t = 0; t < TS; ++t) {
        swv.koff[t] += kVBias;
        opaque(swv.koff[t]);
    }
    const int ntiles = n_k / BC;
    const int G = gridDim.x;
    int L = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
    if (L >= total_blocks) return;

    const uint32_t kv_bytes = (uint32_t)n_k * D * (uint32_t)sizeof(elem);
    auto k_rsrc = [&](int blk) { return make_rsrc(K + (int64_t)(blk / n_qblocks) * n_k * D, kv_bytes); };
    auto v_rsrc = [&](int blk) { return make_rsrc(V + (int64_t)(blk / n_qblocks) * n_k * D, kv_bytes); };
    // rows of block blk (rows at or past n_q read as zero)
    auto row_rsrc = [&](const void *base, int blk, int row_bytes) {
        const int bh = blk / n_qblocks, q0 = (blk % n_qblocks) * BR;
        return make_rsrc(static_cast<const char *>(base) + ((int64_t)bh * n_q + q0) * row_bytes,
                         (uint32_t)min(BR, n_q - q0) * (uint32_t)row_bytes);
    };
    constexpr int RB = D * (int)sizeof(elem);
    // this lane's fragment t: row wave * 32 + col, columns 16 t + 8 h ..
    const uint32_t q_lane = (uint32_t)((wave * 32 + col) * RB + h * Tr::KPL * (int)sizeof(elem));
    const uint32_t l_lane = (uint32_t)((wave * 32 + col) * 4);
    frag qf[TS], df[TS];
    float lse_raw, dl;
    auto load_q = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = __builtin_bit_cast(frag, buffer_load16(r, q_lane + 32 * t));
    };
    auto load_do = [&](__amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int t = 0; t < TS; ++t) df[t] = __builtin_bit_cast(frag, buffer_load16(r, q_lane + 32 * t));
    };
    auto load_ld = [&](__amdgpu_buffer_rsrc_t lr, __amdgpu_buffer_rsrc_t er) {
        lse_raw = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, l_lane, 0, 0));
        dl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(er, l_lane, 0, 0));
    };
    // this wave's DMA pieces of tile `tile` (piece J to wave J % WAVES)
    auto dma_tile = [&](__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int tile, char *kd, char *vd) {
        const uint32_t t0 = (uint32_t)tile * (uint32_t)BYTES;
#pragma unroll
        for (int j = 0; j < PIECES / WAVES; ++j) {
            const int J = wv + WAVES * j;
            const uint32_t off = t0 + Sw::piece_off(J, lane);
            dma16(kr, off, kd + 1024 * J);
            dma16(vr, off, vd + 1024 * J);
        }
    };

    __amdgpu_buffer_rsrc_t krs = k_rsrc(L), vrs = v_rsrc(L);
    load_q(row_rsrc(Q, L, RB));
    load_do(row_rsrc(dO, L, RB));
    load_ld(row_rsrc(LSE, L, 4), row_rsrc(Delta, L, 4));
    dma_tile(krs, vrs, 0, K0, V0);
    dma_tile(krs, vrs, 1, K1, V1);
    // Q, dO, lse, delta and tile 0 landed (loads complete in order)
    __builtin_amdgcn_s_waitcnt(0x0f70 | NPW);
    lds_changed();
    __builtin_amdgcn_s_barrier();
    lds_changed();

    f32x16 acc[NDB];
    for (;;) {
        const int Ln = L + G;
        const bool has_next = Ln < total_blocks;
        // past the last block the look-ahead reads zeros: tiles past this
        // head's end, and rows of an empty range
        const __amdgpu_buffer_rsrc_t nkrs = has_next ? k_rsrc(Ln) : krs;
        const __amdgpu_buffer_rsrc_t nvrs = has_next ? v_rsrc(Ln) : vrs;
        const int ntile0 = has_next ? 0 : ntiles;
        const int qrow = (L % n_qblocks) * BR + wave * 32 + col;
        // rows past n_q: lse = +inf, so every P is 0 (their Q and dO are zero)
        const float lse2 = qrow < n_q ? lse_raw * kLog2e : INFINITY;
#pragma unroll
        for (int d = 0; d < NDB; ++d) acc[d] = zero16();
        // step t: DMA of tile t + 2 (of this block, or tile t + 2 - ntiles of
        // the next) into stage (t + 2) % 4, last read in step t - 2; tile t;
        // wait for tile t + 1's pieces (WAITN: the loads issued after them,
        // tile t + 2's and, in the last step, the next block's rows); barrier
        auto step = [&](auto stage_tag, auto waitn_tag, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                        int dtile, const auto &hq, const auto &hd, const auto &hl) {
            constexpr int S = decltype(stage_tag)::value;
            constexpr int WAITN = decltype(waitn_tag)::value;
            char *const kc = S == 0 ? K0 : S == 1 ? K1 : S == 2 ? K2 : K3;
            char *const vc = S == 0 ? V0 : S == 1 ? V1 : S == 2 ? V2 : V3;
            char *const kn = S == 0 ? K2 : S == 1 ? K3 : S == 2 ? K0 : K1;
            char *const vn = S == 0 ? V2 : S == 1 ? V3 : S == 2 ? V0 : V1;
            dma_tile(kr, vr, dtile, kn, vn);
            __builtin_amdgcn_sched_barrier(0);
            dq_tile_stream<DT, D>(kc, vc - kVBias, swk, swv, qf, df, lse2, dl, acc, scale_log2, hq, hd, hl);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x0f70 | (WAITN & 15) | ((WAITN >> 4) << 14));
            lds_changed();
            __builtin_amdgcn_s_barrier();
            lds_changed();
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        using C3 = std::integral_constant<int, 3>;
        using WN = std::integral_constant<int, NPW>;
        using WQ = std::integral_constant<int, NPW + NQ>;
        const NoHook none;
        int t = 0;
        for (; t + 8 <= ntiles; t += 4) {
            step(C0{}, WN{}, krs, vrs, t + 2, none, none, none);
            step(C1{}, WN{}, krs, vrs, t + 3, none, none, none);
            step(C2{}, WN{}, krs, vrs, t + 4, none, none, none);
            step(C3{}, WN{}, krs, vrs, t + 5, none, none, none);
        }
        const __amdgpu_buffer_rsrc_t nq = has_next ? row_rsrc(Q, Ln, RB) : make_rsrc(Q, 0);
        const __amdgpu_buffer_rsrc_t nd = has_next ? row_rsrc(dO, Ln, RB) : make_rsrc(dO, 0);
        const __amdgpu_buffer_rsrc_t nl = has_next ? row_rsrc(LSE, Ln, 4) : make_rsrc(LSE, 0);
        const __amdgpu_buffer_rsrc_t ne = has_next ? row_rsrc(Delta, Ln, 4) : make_rsrc(Delta, 0);
        step(C0{}, WN{}, krs, vrs, ntiles - 2, none, none, none);
        step(C1{}, WN{}, krs, vrs, ntiles - 1, none, none, none);
        step(C2{}, WN{}, nkrs, nvrs, ntile0, none, none, none);
        step(C3{}, WQ{}, nkrs, nvrs, ntile0 + 1, [&]() { load_q(nq); }, [&]() { load_do(nd); },
             [&]() { load_ld(nl, ne); });

        // the next block's rows and tile 1 landed (issued during the last
        // tile): waiting here, before the stores, keeps the next block's
        // first products from waiting on the stores as well
        wait_dma();
        if (qrow < n_q) {
            elem *op = dQ + ((int64_t)(L / n_qblocks) * n_q + qrow) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) store4_b<DT>(op + 32 * db + 8 * g + 4 * h, acc[db], g, scale);
        }
        if (!has_next) break;
        L = Ln;
        krs = nkrs;
        vrs = nvrs;
    }
}

// ---------------------------------------------------------------------------
// dK, dV over DMA-filled tiles (16-bit types). Each wave's own 32 V rows go
// once into a wave-private swizzled LDS tile (B operand of dP = dO V^T, read
// again for every query tile; in registers they would take the wave past 256
// VGPRs); query tiles of 32 rows of Q and dO go by DMA into swizzled tiles,
// one LDS array per stage, with the forward's step structure (fwd_pass_dma).
// lse (times log2 e) and delta of a tile come through registers of the first
// 32 lanes, one tile ahead. Queries past n_q read as zero Q and dO rows and
// add nothing. At the end each wave stages its dK and dV rows through its
// own V tile and writes whole 16-byte pieces of full rows.
template <Dt DT, int D, int WAVES>
__device__ __forceinline__ void dkdv_pass_dma(__amdgpu_buffer_rsrc_t qrs, __amdgpu_buffer_rsrc_t drs,
                                              __amdgpu_buffer_rsrc_t vrs, __amdgpu_buffer_rsrc_t lrs,
                                              __amdgpu_buffer_rsrc_t ers,
                                              const typename Traits<DT>::frag (&kf)[D / 16],
                                              typename Traits<DT>::elem *__restrict__ dk_rows,
                                              typename Traits<DT>::elem *__restrict__ dv_rows, int krow0, int n_k,
                                              int n_q, float scale_log2, float scale, int lane, int wave, int tid) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using Sw = SwzTile<DT, D, 32>;
    constexpr int BQ = Sw::ROWS, BYTES = Sw::BYTES, PIECES = Sw::PIECES, NDB = D / 32, TS = D / 16;
    constexpr int RB = Sw::RB, NC = Sw::NC;
    __shared__ __attribute__((aligned(1024))) char Q0[BYTES];
    __shared__ __attribute__((aligned(1024))) char Q1[BYTES];
    __shared__ __attribute__((aligned(1024))) char D0[BYTES];
    __shared__ __attribute__((aligned(1024))) char D1[BYTES];
    // 16-byte aligned (the DMA needs no more), so that the LDS layout puts
    // the 1024-aligned per-tile arrays first, within reach of the 16-bit
    // immediate offsets of the LDS reads
    __shared__ __attribute__((aligned(16))) char Vw[WAVES * BYTES];
    __shared__ __attribute__((aligned(16))) float L0[BQ];
    __shared__ __attribute__((aligned(16))) float L1[BQ];
    __shared__ __attribute__((aligned(16))) float E0[BQ];
    __shared__ __attribute__((aligned(16))) float E1[BQ];
    const int h = lane >> 5;
    Sw sw;
    sw.init(lane);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    char *vown = Vw + wv * BYTES;
    const int ntiles = (n_q + BQ - 1) / BQ;

    auto dma_tile = [&](int tile, char *qd, char *dd) {
        const uint32_t t0 = (uint32_t)tile * (uint32_t)BYTES;
#pragma unroll
        for (int j = 0; j < (PIECES + WAVES - 1) / WAVES; ++j) {
            const int J = wv + WAVES * j;
            if (PIECES % WAVES == 0 || J < PIECES) {
                const uint32_t off = t0 + Sw::piece_off(J, lane);
                dma16(qrs, off, qd + 1024 * J);
                dma16(drs, off, dd + 1024 * J);
            }
        }
    };
    // lse * log2e and delta of query tile `tile` (rows past n_q read as 0: their
    // Q and dO rows are zero, so their terms vanish whatever P is)
    float lreg = 0.f, dreg = 0.f;
    auto load_ld = [&](int tile) {
        if (tid < BQ) {
            lreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (tile * BQ + tid) * 4, 0, 0));
            dreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ers, (tile * BQ + tid) * 4, 0, 0));
        }
    };
    auto store_ld = [&](float *ld, float *ed) {
        if (tid < BQ) {
            ld[tid] = lreg * kLog2e;
            ed[tid] = dreg;
        }
    };

    f32x16 accK[NDB], accV[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) accK[i] = accV[i] = zero16();

    // One query tile in phases of one kind each, their order pinned by
    // scheduling barriers: the S and dP products, the softmax and dS as VALU
    // work only, the dV and dK products. The operands come from LDS ahead of
    // their products: the Q, dO and V fragments of step t + 1 before the S
    // and dP products of step t, the transposed dO / Q fragment of dV / dK
    // product i + 2 before product i (left to itself at 256 registers, the
    // compiler read each operand just before its product and waited for it,
    // which left the matrix pipe idle about 40% of the time). The S / dP
    // reads use the precomputed per-lane offsets; the eight transposed-read
    // offsets are rebuilt per tile from two base registers (the XOR of a
    // constant) between the products and the softmax, which leaves room for
    // the operands in flight and keeps address arithmetic out of the product
    // phases (VALU work between a wave's own products slows its matrix
    // stream).
    auto tile_fn = [&](const char *qt, const char *dt, const float *ls, const float *es) {
        constexpr int AHEAD1 = 1, AHEAD2 = 2;
        uint32_t v0 = sw.voff[0][0], v1 = sw.voff[0][1];
        opaque(v0);
        opaque(v1);
        f32x16 s = zero16(), dp = zero16();
        frag qa[TS], da[TS], va[TS];
        auto read1 = [&](int t) {
            qa[t] = sw.k(qt, 0, t);
            da[t] = sw.k(dt, 0, t);
            va[t] = sw.k(vown, 0, t);
        };
#pragma unroll
        for (int t = 0; t < AHEAD1; ++t) read1(t);
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            if (t + AHEAD1 < TS) read1(t + AHEAD1);
            __builtin_amdgcn_sched_barrier(0);
            s = Tr::mfma(qa[t], kf[t], s);
            dp = Tr::mfma(da[t], va[t], dp);
            __builtin_amdgcn_sched_barrier(0);
        }
        // A operands of the 4 NDB dV / dK products, i = 2 (NDB t + db) + (0: dV, 1: dK)
        constexpr int NP = 4 * NDB;
        frag ob[NP];
        uint32_t vo[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            vo[db][0] = Sw::vt_off(v0, db);
            vo[db][1] = Sw::vt_off(v1, db);
        }
        auto read2 = [&](int i) {
            const int t = i / (2 * NDB), db = (i >> 1) % NDB;
            ob[i] = Sw::vt_pair((i & 1) ? qt : dt, vo[db][0], vo[db][1], t);
        };
#pragma unroll
        for (int i = 0; i < AHEAD2; ++i) read2(i);
        __builtin_amdgcn_sched_barrier(0);
        // p into s, dS into dp (rows = queries along a lane's registers)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 l4 = *reinterpret_cast<const float4 *>(ls + 8 * g + 4 * h);
            const float4 d4 = *reinterpret_cast<const float4 *>(es + 8 * g + 4 * h);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * g + i;
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lv[i]));
                s[c] = pv;
                dp[c] = pv * (dp[c] - dv[i]);
            }
        }
        const frag pf[2] = {c_to_frag<DT>(s, 0), c_to_frag<DT>(s, 1)};
        const frag dsf[2] = {c_to_frag<DT>(dp, 0), c_to_frag<DT>(dp, 1)};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i + AHEAD2 < NP) read2(i + AHEAD2);
            __builtin_amdgcn_sched_barrier(0);
            const int t = i / (2 * NDB), db = (i >> 1) % NDB;
            if (i & 1)
                accK[db] = Tr::mfma(ob[i], dsf[t], accK[db]);
            else
                accV[db] = Tr::mfma(ob[i], pf[t], accV[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: the wave's V rows, query tile 0 and its lse / delta; tile 1's
    // lse / delta into registers
#pragma unroll
    for (int J = 0; J < PIECES; ++J) dma16(vrs, (uint32_t)(krow0 + 32 * wv) * RB + Sw::piece_off(J, lane), vown + 1024 * J);
    dma_tile(0, Q0, D0);
    load_ld(0);
    wait_dma();
    store_ld(L0, E0);
    load_ld(1);
    wait_dma();
    __syncthreads();
    lds_changed();
    // stage of tile it: Q0/D0/L0/E0 for even it, the others for odd it
    auto step = [&](auto odd_tag, int it) {
        constexpr bool ODD = decltype(odd_tag)::value;
        dma_tile(it + 1, ODD ? Q0 : Q1, ODD ? D0 : D1);
        store_ld(ODD ? L0 : L1, ODD ? E0 : E1);
        load_ld(it + 2);
        __builtin_amdgcn_sched_barrier(0);
        tile_fn(ODD ? Q1 : Q0, ODD ? D1 : D0, ODD ? L1 : L0, ODD ? E1 : E0);
        __builtin_amdgcn_sched_barrier(0);
        wait_dma();
        __syncthreads();
        lds_changed();
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        step(std::false_type{}, it);
        step(std::true_type{}, it + 1);
    }
    if (it < ntiles) step(std::false_type{}, it);

    // Epilogue through the wave's own V tile (no other wave reads it): lane
    // `col` holds dK / dV of key col, d = 32 db + 8 g + 4 h + 0..3; it writes
    // those 8 bytes at the swizzled place of row col, then the wave reads
    // back whole 16-byte chunks, 16 lanes per 256-byte row, and stores them.
    // Its lane-derived offsets are computed from a copy of the lane index
    // the optimiser cannot match with the prologue's (it would otherwise keep
    // the prologue's across the loop in spilled registers: 44 bytes per lane
    // stored and reloaded once per wave, 16% more HBM writes than dK + dV).
    uint32_t lane_e = (uint32_t)lane;
    opaque(lane_e);
    const int col = lane_e & 31, he = lane_e >> 5;
    auto emit = [&](const f32x16 (&acc)[NDB], float mul, elem *rows) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                typename Tr::half_frag v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = static_cast<elem>(acc[db][4 * g + i] * mul);
                const int c = 4 * db + g;  // logical chunk of d = 32 db + 8 g
                *reinterpret_cast<typename Tr::half_frag *>(vown + col * RB + ((c ^ swz<D>(col)) << 4) + 8 * he) = v;
            }
        constexpr int PER = 32 * NC / 64;  // chunks per lane
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = (int)lane_e + 64 * i, r = idx / NC, p = idx % NC;
            const uint4 w = *reinterpret_cast<const uint4 *>(vown + r * RB + (p << 4));
            const int c = p ^ swz<D>(r);
            if (krow0 + 32 * wv + r < n_k)
                *reinterpret_cast<uint4 *>(rows + (int64_t)(32 * wv + r) * D + c * 8) = w;
        }
    };
    emit(accK, scale, dk_rows);
    emit(accV, 1.f, dv_rows);
}

// dK, dV for float32: K and V rows of the wave's keys in registers; query
// tiles of BQ rows of Q and dO staged through registers into padded tiles plus
// transposed copies, with lse * log2e and delta, two LDS stages.
template <int D, int BQ, int WAVES>
__device__ __forceinline__ void dkdv_pass_f32(__amdgpu_buffer_rsrc_t qrs, __amdgpu_buffer_rsrc_t drs,
                                              __amdgpu_buffer_rsrc_t lrs, __amdgpu_buffer_rsrc_t ers,
                                              const float (&kf)[D / 2], const float (&vf)[D / 2],
                                              f32x16 (&accK)[D / 32], f32x16 (&accV)[D / 32], int n_q,
                                              float scale_log2, int lane, int tid) {
    constexpr Dt DT = Dt::F32;
    using Tr = Traits<DT>;
    constexpr int NT = WAVES * 64;
    using Tl = BwdTile<DT, D, true>;
    constexpr int LDT = BQ + 4;
    constexpr int QS = BQ * Tl::LD;
    constexpr int TSZ = D * LDT;
    constexpr int NQB = BQ / 32, NDB = D / 32, TS = D / 2, TP = 16;
    static_assert(BQ <= NT, "lse staging");
    __shared__ __attribute__((aligned(16))) float Qs[2 * QS];
    __shared__ __attribute__((aligned(16))) float Ds[2 * QS];
    __shared__ __attribute__((aligned(16))) float Qt[2 * TSZ];
    __shared__ __attribute__((aligned(16))) float Dt_[2 * TSZ];
    __shared__ __attribute__((aligned(16))) float Ls[2 * BQ];
    __shared__ __attribute__((aligned(16))) float Dl[2 * BQ];
    const int h = lane >> 5, col = lane & 31;
    RowStage<DT, BQ, D, NT> qst, dst;
    constexpr int RBS = stage_rows<DT, BQ, D, NT>();
    TileStage<DT, BQ, D, NT, false, RBS> qtst, dtst;
    float lreg = 0.f, dreg = 0.f;
    auto load = [&](int row0) {
        qst.load(qrs, row0, tid);
        dst.load(drs, row0, tid);
        if (tid < BQ) {
            lreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (row0 + tid) * 4, 0, 0));
            dreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ers, (row0 + tid) * 4, 0, 0));
        }
        qtst.load(qrs, row0, tid);
        dtst.load(drs, row0, tid);
    };
    auto store = [&](int stage) {
        Tl::store(qst, Qs + stage * QS, tid);
        Tl::store(dst, Ds + stage * QS, tid);
        if (tid < BQ) {
            Ls[stage * BQ + tid] = lreg * kLog2e;
            Dl[stage * BQ + tid] = dreg;
        }
        qtst.template store_transposed<LDT>(Qt + stage * TSZ, tid);
        dtst.template store_transposed<LDT>(Dt_ + stage * TSZ, tid);
    };
    const int ntiles = (n_q + BQ - 1) / BQ;
    load(0);
    store(0);
    if (ntiles > 1) load(BQ);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int st = it & 1;
        const float *qt = Qs + st * QS, *dt = Ds + st * QS, *qtt = Qt + st * TSZ, *dtt = Dt_ + st * TSZ;
        const float *ls = Ls + st * BQ, *dls = Dl + st * BQ;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                s = Tr::mfma(Tl::row(qt, 32 * qb + col, t, h), kf[t], s);
                dp = Tr::mfma(Tl::row(dt, 32 * qb + col, t, h), vf[t], dp);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4 *>(ls + 32 * qb + 8 * g + 4 * h);
                const float4 d4 = *reinterpret_cast<const float4 *>(dls + 32 * qb + 8 * g + 4 * h);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * g + i;
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lv[i]));
                    s[c] = pv;
                    dp[c] = pv * (dp[c] - dv[i]);
                }
            }
#pragma unroll
            for (int t = 0; t < TP; ++t) {
                const float pf = c_to_frag<DT>(s, t);
                const float dsf = c_to_frag<DT>(dp, t);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    accV[db] = Tr::mfma(Tl::template trans<LDT>(dt, dtt, qb, t, db, lane), pf, accV[db]);
                    accK[db] = Tr::mfma(Tl::template trans<LDT>(qt, qtt, qb, t, db, lane), dsf, accK[db]);
                }
            }
        }
        if (it + 1 < ntiles) {
            store((it + 1) & 1);
            if (it + 2 < ntiles) load((it + 2) * BQ);
        }
        __syncthreads();
    }
}

// dK, dV: per workgroup BKV = 32*WAVES key rows, wave w owning keys
// 32w..32w+31 as B operands (K rows in registers). Query tiles of BQ rows:
// Q and dO as A operands of S = Q K^T and dP = dO V^T, and via transposing
// reads of dK^T += Q^T dS and dV^T += dO^T P, plus lse*log2e and delta.
// C blocks: rows = queries, column = key; lse and delta vary along a lane's
// registers.
template <Dt DT, int D, int BQ, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, const typename Traits<DT>::elem *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Delta, typename Traits<DT>::elem *__restrict__ dK,
    typename Traits<DT>::elem *__restrict__ dV, int n_q, int n_k, int n_kblocks, int total_blocks,
    float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr bool TR = sizeof(elem) == 2;
    constexpr int BKV = 32 * WAVES;
    constexpr int NDB = D / 32;
    constexpr int TS = D / (2 * Tr::KPL);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_kblocks, kblk = blk % n_kblocks;
    const int krow = kblk * BKV + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = (int64_t)bh * n_k * D;
    const int64_t loff = (int64_t)bh * n_q;

    frag kf[TS];
    if (krow < n_k) {
        const elem *kp = K + koff + (int64_t)krow * D;
#pragma unroll
        for (int t = 0; t < TS; ++t) kf[t] = ld_row_frag<DT>(kp, t, h);
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t) kf[t] = zero_frag_b<DT>();
    }

    const uint32_t head_bytes = (uint32_t)n_q * D * (uint32_t)sizeof(elem);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dO + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(LSE + loff, (uint32_t)n_q * 4u);
    const __amdgpu_buffer_rsrc_t ers = make_rsrc(Delta + loff, (uint32_t)n_q * 4u);

    if constexpr (TR) {
        static_assert(BQ == 32, "DMA query tiles hold 32 rows");
        // V rows past n_k read as zero
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + koff, (uint32_t)n_k * D * (uint32_t)sizeof(elem));
        const int krow0 = kblk * BKV;
        dkdv_pass_dma<DT, D, WAVES>(qrs, drs, vrs, lrs, ers, kf, dK + koff + (int64_t)krow0 * D,
                                    dV + koff + (int64_t)krow0 * D, krow0, n_k, n_q, scale_log2, scale, lane, wave,
                                    tid);
    } else {
        frag vf[TS];
        if (krow < n_k) {
            const elem *vp = V + koff + (int64_t)krow * D;
#pragma unroll
            for (int t = 0; t < TS; ++t) vf[t] = ld_row_frag<DT>(vp, t, h);
        } else {
#pragma unroll
            for (int t = 0; t < TS; ++t) vf[t] = zero_frag_b<DT>();
        }
        f32x16 accK[NDB], accV[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) accK[i] = accV[i] = zero16();
        dkdv_pass_f32<D, BQ, WAVES>(qrs, drs, lrs, ers, kf, vf, accK, accV, n_q, scale_log2, lane, tid);
        if (krow < n_k) {
            elem *kp = dK + koff + (int64_t)krow * D;
            elem *vp = dV + koff + (int64_t)krow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    store4_b<DT>(kp + 32 * db + 8 * g + 4 * h, accK[db], g, scale);
                    store4_b<DT>(vp + 32 * db + 8 * g + 4 * h, accV[db], g, 1.f);
                }
        }
    }
}

// ---------------------------------------------------------------------------

template <Dt DT, int D>
static hipError_t delta_dispatch(const void *o, const void *d_o, float *delta, int64_t rows, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int RPB = 256 / (D / vec_elems<DT>());
    const int64_t grid = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((delta_kernel<DT, D>), dim3((unsigned)grid), dim3(256), 0, stream, (const elem *)o,
                       (const elem *)d_o, delta, rows);
    return hipGetLastError();
}

template <Dt DT, int D, int WAVES>
static hipError_t dq_launch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                            const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    // float32 at head_dim 128 halves the key tile to fit two LDS stages
    constexpr int BC = (sizeof(elem) == 4 && D == 128) ? 32 : 64, BR = 32 * WAVES;
    const int nqb = (s.n_q + BR - 1) / BR;
    const int total = (int)(s.bh * nqb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((dq_kernel<DT, D, BC, WAVES>), dim3(total), dim3(WAVES * 64), 0, stream, (const elem *)q,
                       (const elem *)k, (const elem *)v, (const elem *)d_o, lse, delta, (elem *)dq, s.n_q, s.n_k,
                       nqb, total, scale_log2, s.scale);
    return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t dq_stream_launch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                                   const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    const int nqb = (s.n_q + 255) / 256;
    const int total = (int)(s.bh * nqb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((dq_stream_kernel<DT, D>), dim3(kDqStreamGrid), dim3(512), 0, stream, (const elem *)q,
                       (const elem *)k, (const elem *)v, (const elem *)d_o, lse, delta, (elem *)dq, s.n_q, s.n_k,
                       nqb, total, scale_log2, s.scale);
    return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t dq_dispatch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                              const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    constexpr int64_t kCus = 256;
    if constexpr (D == 128 && DT != Dt::F32) {
        // key lengths in whole groups of four tiles and at least two query
        // blocks per CU: the persistent launch
        if (s.n_k >= 256 && s.n_k % 256 == 0 && s.bh * ((s.n_q + 255) / 256) >= 2 * kDqStreamGrid)
            return dq_stream_launch<DT, D>(q, k, v, d_o, lse, delta, dq, s, stream);
    }
    if (s.bh * ((s.n_q + 255) / 256) >= 2 * kCus) return dq_launch<DT, D, 8>(q, k, v, d_o, lse, delta, dq, s, stream);
    if (s.bh * ((s.n_q + 127) / 128) >= kCus) return dq_launch<DT, D, 4>(q, k, v, d_o, lse, delta, dq, s, stream);
    return dq_launch<DT, D, 2>(q, k, v, d_o, lse, delta, dq, s, stream);
}

template <Dt DT, int D, int WAVES>
static hipError_t dkdv_launch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                              const float *delta, void *dk, void *dv, const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BKV = 32 * WAVES;
    constexpr int BQ = 32;  // one 32-query block per tile keeps a wave within 256 VGPRs
    const int nkb = (s.n_k + BKV - 1) / BKV;
    const int total = (int)(s.bh * nkb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((dkdv_kernel<DT, D, BQ, WAVES>), dim3(total), dim3(WAVES * 64), 0, stream,
                       (const elem *)q, (const elem *)k, (const elem *)v, (const elem *)d_o, lse, delta,
                       (elem *)dk, (elem *)dv, s.n_q, s.n_k, nkb, total, scale_log2, s.scale);
    return hipGetLastError();
}

// Workgroup size by problem size, as for the forward (key rows here).
template <Dt DT, int D>
static hipError_t dkdv_dispatch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                                const float *delta, void *dk, void *dv, const AttnShape &s, hipStream_t stream) {
    constexpr int64_t kCus = 256;
    if (s.bh * ((s.n_k + 255) / 256) >= 2 * kCus)
        return dkdv_launch<DT, D, 8>(q, k, v, d_o, lse, delta, dk, dv, s, stream);
    if (s.bh * ((s.n_k + 127) / 128) >= kCus) return dkdv_launch<DT, D, 4>(q, k, v, d_o, lse, delta, dk, dv, s, stream);
    return dkdv_launch<DT, D, 2>(q, k, v, d_o, lse, delta, dk, dv, s, stream);
}

#define FA2_DISPATCH_DIM(FN, DT, HD, ...)                         \
    switch (HD) {                                                 \
        case 32: return FN<DT, 32>(__VA_ARGS__);                  \
        case 64: return FN<DT, 64>(__VA_ARGS__);                  \
        case 128: return FN<DT, 128>(__VA_ARGS__);                \
        default: return hipErrorInvalidValue;                     \
    }

#define FA2_DISPATCH(FN, DTI, HD, ...)                                         \
    switch (DTI) {                                                             \
        case 0: { FA2_DISPATCH_DIM(FN, Dt::F32, HD, __VA_ARGS__) }             \
        case 1: { FA2_DISPATCH_DIM(FN, Dt::F16, HD, __VA_ARGS__) }             \
        case 2: { FA2_DISPATCH_DIM(FN, Dt::BF16, HD, __VA_ARGS__) }            \
        default: return hipErrorInvalidValue;                                  \
    }

hipError_t launch_bwd_delta(int dt, const void *o, const void *d_o, float *delta, int64_t rows, int head_dim,
                            hipStream_t stream) {
    FA2_DISPATCH(delta_dispatch, dt, head_dim, o, d_o, delta, rows, stream)
}

hipError_t launch_bwd_dq(int dt, const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                         const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    FA2_DISPATCH(dq_dispatch, dt, s.head_dim, q, k, v, d_o, lse, delta, dq, s, stream)
}

hipError_t launch_bwd_dkdv(int dt, const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                           const float *delta, void *dk, void *dv, const AttnShape &s, hipStream_t stream) {
    FA2_DISPATCH(dkdv_dispatch, dt, s.head_dim, q, k, v, d_o, lse, delta, dk, dv, s, stream)
}

}  // namespace fa2mi
