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
//   dkdv_kernel  - one workgroup per 32*WAVES key rows, looping over query
//                  tiles; K and V of the wave's 32 keys stay in registers.
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
    constexpr int NT = WAVES * 64;
    constexpr int BR = 32 * WAVES;
    constexpr int KPL = Tr::KPL;
    constexpr int KSTEP = 2 * KPL;
    using Tl = BwdTile<DT, D, false>;
    constexpr int LDT = BC + 4;          // float32 transposed K copy
    constexpr int KS = BC * Tl::LD;
    constexpr int TSZ = TR ? 1 : D * LDT;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int TS = D / KSTEP;
    constexpr int TP = 32 / KSTEP;

    __shared__ __attribute__((aligned(16))) elem Ks[2 * KS];
    __shared__ __attribute__((aligned(16))) elem Vs[2 * KS];
    __shared__ __attribute__((aligned(16))) elem Kt[2 * TSZ];

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
    RowStage<DT, BC, D, NT> kst, vst;
    constexpr int RBS = stage_rows<DT, BC, D, NT>();
    TileStage<DT, BC, D, NT, false, RBS> ktst;  // float32 only: transposed K
    auto load = [&](int row0) {
        kst.load(krs, row0, tid);
        vst.load(vrs, row0, tid);
        if constexpr (!TR) ktst.load(krs, row0, tid);
    };
    auto store = [&](int stage) {
        Tl::store(kst, Ks + stage * KS, tid);
        Tl::store(vst, Vs + stage * KS, tid);
        if constexpr (!TR) ktst.template store_transposed<LDT>(Kt + stage * TSZ, tid);
    };

    const int ntiles = (n_k + BC - 1) / BC;
    load(0);
    store(0);
    if (ntiles > 1) load(BC);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int st = it & 1;
        const elem *kt = Ks + st * KS;
        const elem *vt = Vs + st * KS;
        const elem *ktt = Kt + st * TSZ;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 s = zero16(), dp = zero16();
            if constexpr (TR) {
                // 16-bit types: the S chain first, so that its exponentials
                // can be scheduled among the dP products (1% faster at the
                // LLM shape, same results)
#pragma unroll
                for (int t = 0; t < TS; ++t) s = Tr::mfma(Tl::row(kt, 32 * kb + col, t, h), qf[t], s);
#pragma unroll
                for (int t = 0; t < TS; ++t) dp = Tr::mfma(Tl::row(vt, 32 * kb + col, t, h), df[t], dp);
            } else {
#pragma unroll
                for (int t = 0; t < TS; ++t) {
                    s = Tr::mfma(Tl::row(kt, 32 * kb + col, t, h), qf[t], s);
                    dp = Tr::mfma(Tl::row(vt, 32 * kb + col, t, h), df[t], dp);
                }
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lse2));
                s[c] = p * (dp[c] - dl);
            }
#pragma unroll
            for (int t = 0; t < TP; ++t) {
                const frag dsf = c_to_frag<DT>(s, t);
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

    if (qvalid) {
        elem *op = dQ + qoff + (int64_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) store4_b<DT>(op + 32 * db + 8 * g + 4 * h, acc[db], g, scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: per workgroup BKV = 32*WAVES key rows, wave w owning keys
// 32w..32w+31 as B operands: K rows in registers, V rows in LDS for 16-bit
// types (read once per 32-query block; that keeps a wave within 256 VGPRs,
// i.e. two waves per SIMD) and in registers for float32. Query tiles
// of BQ rows: Q and dO row-major in LDS (A operands of S = Q K^T and
// dP = dO V^T, and via transposing reads of dK^T += Q^T dS and
// dV^T += dO^T P), plus lse*log2e and delta. C blocks: rows = queries,
// column = key; lse and delta vary along a lane's registers.
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
    constexpr int NT = WAVES * 64;
    constexpr int BKV = 32 * WAVES;
    constexpr int KPL = Tr::KPL;
    constexpr int KSTEP = 2 * KPL;
    using Tl = BwdTile<DT, D, true>;
    constexpr int LDT = BQ + 4;          // float32 transposed copies
    constexpr int QS = BQ * Tl::LD;
    constexpr int TSZ = TR ? 1 : D * LDT;
    constexpr int NQB = BQ / 32;
    constexpr int NDB = D / 32;
    constexpr int TS = D / KSTEP;
    constexpr int TP = 32 / KSTEP;
    static_assert(BQ <= NT, "lse staging");

    __shared__ __attribute__((aligned(16))) elem Qs[2 * QS];
    __shared__ __attribute__((aligned(16))) elem Ds[2 * QS];
    __shared__ __attribute__((aligned(16))) elem Qt[2 * TSZ];
    __shared__ __attribute__((aligned(16))) elem Dt_[2 * TSZ];
    __shared__ __attribute__((aligned(16))) float Ls[2 * BQ];
    __shared__ __attribute__((aligned(16))) float Dl[2 * BQ];
    constexpr bool VLDS = TR;
    __shared__ __attribute__((aligned(16))) elem Vk[VLDS ? BKV * Tl::LD : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_kblocks, kblk = blk % n_kblocks;
    const int krow = kblk * BKV + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = (int64_t)bh * n_k * D;
    const int64_t loff = (int64_t)bh * n_q;

    frag kf[TS], vf[VLDS ? 1 : TS];
    if (krow < n_k) {
        const elem *kp = K + koff + (int64_t)krow * D;
#pragma unroll
        for (int t = 0; t < TS; ++t) kf[t] = ld_row_frag<DT>(kp, t, h);
        if constexpr (!VLDS) {
            const elem *vp = V + koff + (int64_t)krow * D;
#pragma unroll
            for (int t = 0; t < TS; ++t) vf[t] = ld_row_frag<DT>(vp, t, h);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t) kf[t] = zero_frag_b<DT>();
        if constexpr (!VLDS) {
#pragma unroll
            for (int t = 0; t < TS; ++t) vf[t] = zero_frag_b<DT>();
        }
    }
    if constexpr (VLDS) {
        // this workgroup's V rows (rows past n_k read as zero)
        const __amdgpu_buffer_rsrc_t vrs =
            make_rsrc(V + koff, (uint32_t)n_k * D * (uint32_t)sizeof(elem));
        RowStage<DT, BKV, D, NT> vst;
        vst.load(vrs, kblk * BKV, tid);
        Tl::store(vst, Vk, tid);
        // made visible by the barrier after the first query tile is staged
    }
    const elem *vkrow = Tl::row_ptr(Vk, wave * 32 + col);

    f32x16 accK[NDB], accV[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) accK[i] = accV[i] = zero16();

    const uint32_t head_bytes = (uint32_t)n_q * D * (uint32_t)sizeof(elem);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dO + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(LSE + loff, (uint32_t)n_q * 4u);
    const __amdgpu_buffer_rsrc_t ers = make_rsrc(Delta + loff, (uint32_t)n_q * 4u);
    RowStage<DT, BQ, D, NT> qst, dst;
    constexpr int RBS = stage_rows<DT, BQ, D, NT>();
    TileStage<DT, BQ, D, NT, false, RBS> qtst, dtst;  // float32 only: transposed copies
    float lreg = 0.f, dreg = 0.f;
    auto load = [&](int row0) {
        qst.load(qrs, row0, tid);
        dst.load(drs, row0, tid);
        if (tid < BQ) {
            // rows past n_q read as 0: their Q and dO rows are zero, so their
            // terms vanish whatever P is
            lreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (row0 + tid) * 4, 0, 0));
            dreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ers, (row0 + tid) * 4, 0, 0));
        }
        if constexpr (!TR) {
            qtst.load(qrs, row0, tid);
            dtst.load(drs, row0, tid);
        }
    };
    auto store = [&](int stage) {
        Tl::store(qst, Qs + stage * QS, tid);
        Tl::store(dst, Ds + stage * QS, tid);
        if (tid < BQ) {
            Ls[stage * BQ + tid] = lreg * kLog2e;
            Dl[stage * BQ + tid] = dreg;
        }
        if constexpr (!TR) {
            qtst.template store_transposed<LDT>(Qt + stage * TSZ, tid);
            dtst.template store_transposed<LDT>(Dt_ + stage * TSZ, tid);
        }
    };

    const int ntiles = (n_q + BQ - 1) / BQ;
    load(0);
    store(0);
    if (ntiles > 1) load(BQ);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int st = it & 1;
        const elem *qt = Qs + st * QS;
        const elem *dt = Ds + st * QS;
        const elem *qtt = Qt + st * TSZ;
        const elem *dtt = Dt_ + st * TSZ;
        const float *ls = Ls + st * BQ;
        const float *dls = Dl + st * BQ;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                s = Tr::mfma(Tl::row(qt, 32 * qb + col, t, h), kf[t], s);
                if constexpr (VLDS)
                    dp = Tr::mfma(Tl::row(dt, 32 * qb + col, t, h), ld_row_frag<DT>(vkrow, t, h), dp);
                else
                    dp = Tr::mfma(Tl::row(dt, 32 * qb + col, t, h), vf[t], dp);
            }
            // p into s, dS into dp
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
                const frag pf = c_to_frag<DT>(s, t);
                const frag dsf = c_to_frag<DT>(dp, t);
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
static hipError_t dq_dispatch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                              const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    constexpr int64_t kCus = 256;
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
