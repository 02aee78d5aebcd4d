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
// dQ: per workgroup BR = 32*WAVES query rows; key tiles of BC rows staged as
// K row-major (for S^T = K Q^T), K transposed (for dQ^T = K^T dS^T) and V
// row-major (for dP^T = V dO^T). Each lane owns one query column.
template <Dt DT, int D, int BC, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void dq_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, const typename Traits<DT>::elem *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Delta, typename Traits<DT>::elem *__restrict__ dQ,
    int n_q, int n_k, int n_qblocks, int total_blocks, float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int NT = WAVES * 64;
    constexpr int BR = 32 * WAVES;
    constexpr int KPL = Tr::KPL;
    constexpr int KSTEP = 2 * KPL;
    constexpr int VEC = vec_elems<DT>();
    constexpr int LDK = D + VEC;
    constexpr int LDT = BC + 4;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int TS = D / KSTEP;
    constexpr int TP = 32 / KSTEP;

    __shared__ __attribute__((aligned(16))) elem Ks[BC * LDK];
    __shared__ __attribute__((aligned(16))) elem Vs[BC * LDK];
    __shared__ __attribute__((aligned(16))) elem Kt[D * LDT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_qblocks, qb = blk % n_qblocks;
    const int qrow = qb * BR + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = (int64_t)bh * n_k * D;
    const bool qvalid = qrow < n_q;

    frag qf[TS], df[TS];
    float lse2 = 0.f, dl = 0.f;
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

    TileStage<DT, BC, D, NT, true> kst, vst;
    const int ntiles = (n_k + BC - 1) / BC;
    kst.load(K + koff, n_k, tid);
    vst.load(V + koff, n_k, tid);
    kst.template store_rows<LDK>(Ks, tid);
    kst.template store_transposed<LDT>(Kt, tid);
    vst.template store_rows<LDK>(Vs, tid);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int j0 = it * BC;
        const bool more = it + 1 < ntiles;
        if (more) {
            kst.load(K + koff + (int64_t)(j0 + BC) * D, n_k - j0 - BC, tid);
            vst.load(V + koff + (int64_t)(j0 + BC) * D, n_k - j0 - BC, tid);
        }
        const int kvalid = n_k - j0;
        f32x16 ds[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 s = zero16(), dp = zero16();
            const elem *krow = Ks + (32 * kb + col) * LDK;
            const elem *vrow = Vs + (32 * kb + col) * LDK;
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                s = Tr::mfma(ld_row_frag<DT>(krow, t, h), qf[t], s);
                dp = Tr::mfma(ld_row_frag<DT>(vrow, t, h), df[t], dp);
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                float x = s[c] * scale_log2 - lse2;
                if (kvalid < BC && 32 * kb + crow(c, h) >= kvalid) x = -INFINITY;
                const float p = qvalid ? __builtin_amdgcn_exp2f(x) : 0.f;
                ds[kb][c] = p * (dp[c] - dl);
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const elem *trow = Kt + (32 * db + col) * LDT;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < TP; ++t)
                    acc[db] = Tr::mfma(ld_t_frag<DT>(trow, kb, t, h), c_to_frag<DT>(ds[kb], t), acc[db]);
        }
        __syncthreads();
        if (more) {
            kst.template store_rows<LDK>(Ks, tid);
            kst.template store_transposed<LDT>(Kt, tid);
            vst.template store_rows<LDK>(Vs, tid);
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
// 32w..32w+31 with their K and V rows in registers (B operands). Query tiles
// of BQ rows are staged as Q and dO row-major (A operands of S = Q K^T and
// dP = dO V^T) and transposed (A operands of dK^T = Q^T dS, dV^T = dO^T P),
// plus log2-scaled LSE and delta. C blocks: rows = queries, column = key.
template <Dt DT, int D, int BQ, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void dkdv_kernel(
    const typename Traits<DT>::elem *__restrict__ Q, const typename Traits<DT>::elem *__restrict__ K,
    const typename Traits<DT>::elem *__restrict__ V, const typename Traits<DT>::elem *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Delta, typename Traits<DT>::elem *__restrict__ dK,
    typename Traits<DT>::elem *__restrict__ dV, int n_q, int n_k, int n_kblocks, int total_blocks,
    float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int NT = WAVES * 64;
    constexpr int BKV = 32 * WAVES;
    constexpr int KPL = Tr::KPL;
    constexpr int KSTEP = 2 * KPL;
    constexpr int VEC = vec_elems<DT>();
    constexpr int LDQ = D + VEC;
    constexpr int LDT = BQ + 4;
    constexpr int NQB = BQ / 32;
    constexpr int NDB = D / 32;
    constexpr int TS = D / KSTEP;
    constexpr int TP = 32 / KSTEP;
    static_assert(BQ <= NT, "lse staging");

    __shared__ __attribute__((aligned(16))) elem Qs[BQ * LDQ];
    __shared__ __attribute__((aligned(16))) elem Ds[BQ * LDQ];
    __shared__ __attribute__((aligned(16))) elem Qt[D * LDT];
    __shared__ __attribute__((aligned(16))) elem Dt_[D * LDT];
    __shared__ __attribute__((aligned(16))) float Ls[BQ];
    __shared__ __attribute__((aligned(16))) float Dl[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_kblocks, kblk = blk % n_kblocks;
    const int krow = kblk * BKV + wave * 32 + col;
    const int64_t qoff = (int64_t)bh * n_q * D;
    const int64_t koff = (int64_t)bh * n_k * D;
    const int64_t loff = (int64_t)bh * n_q;

    frag kf[TS], vf[TS];
    if (krow < n_k) {
        const elem *kp = K + koff + (int64_t)krow * D;
        const elem *vp = V + koff + (int64_t)krow * D;
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            kf[t] = ld_row_frag<DT>(kp, t, h);
            vf[t] = ld_row_frag<DT>(vp, t, h);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TS; ++t) kf[t] = vf[t] = zero_frag_b<DT>();
    }

    f32x16 accK[NDB], accV[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) accK[i] = accV[i] = zero16();

    TileStage<DT, BQ, D, NT, true> qst, dst;
    const int ntiles = (n_q + BQ - 1) / BQ;
    float lreg = INFINITY, dreg = 0.f;
    qst.load(Q + qoff, n_q, tid);
    dst.load(dO + qoff, n_q, tid);
    if (tid < BQ && tid < n_q) {
        lreg = LSE[loff + tid] * kLog2e;
        dreg = Delta[loff + tid];
    }
    qst.template store_rows<LDQ>(Qs, tid);
    qst.template store_transposed<LDT>(Qt, tid);
    dst.template store_rows<LDQ>(Ds, tid);
    dst.template store_transposed<LDT>(Dt_, tid);
    if (tid < BQ) {
        Ls[tid] = lreg;
        Dl[tid] = dreg;
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int i0 = it * BQ;
        const bool more = it + 1 < ntiles;
        if (more) {
            qst.load(Q + qoff + (int64_t)(i0 + BQ) * D, n_q - i0 - BQ, tid);
            dst.load(dO + qoff + (int64_t)(i0 + BQ) * D, n_q - i0 - BQ, tid);
            lreg = INFINITY;
            dreg = 0.f;
            if (tid < BQ && i0 + BQ + tid < n_q) {
                lreg = LSE[loff + i0 + BQ + tid] * kLog2e;
                dreg = Delta[loff + i0 + BQ + tid];
            }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x16 s = zero16(), dp = zero16();
            const elem *qrow = Qs + (32 * qb + col) * LDQ;
            const elem *drow = Ds + (32 * qb + col) * LDQ;
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                s = Tr::mfma(ld_row_frag<DT>(qrow, t, h), kf[t], s);
                dp = Tr::mfma(ld_row_frag<DT>(drow, t, h), vf[t], dp);
            }
            f32x16 p, ds;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4 *>(Ls + 32 * qb + 8 * g + 4 * h);
                const float4 d4 = *reinterpret_cast<const float4 *>(Dl + 32 * qb + 8 * g + 4 * h);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * g + i;
                    const float pv = __builtin_amdgcn_exp2f(s[c] * scale_log2 - lv[i]);
                    p[c] = pv;
                    ds[c] = pv * (dp[c] - dv[i]);
                }
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const elem *dtr = Dt_ + (32 * db + col) * LDT;
                const elem *qtr = Qt + (32 * db + col) * LDT;
#pragma unroll
                for (int t = 0; t < TP; ++t) {
                    accV[db] = Tr::mfma(ld_t_frag<DT>(dtr, qb, t, h), c_to_frag<DT>(p, t), accV[db]);
                    accK[db] = Tr::mfma(ld_t_frag<DT>(qtr, qb, t, h), c_to_frag<DT>(ds, t), accK[db]);
                }
            }
        }
        __syncthreads();
        if (more) {
            qst.template store_rows<LDQ>(Qs, tid);
            qst.template store_transposed<LDT>(Qt, tid);
            dst.template store_rows<LDQ>(Ds, tid);
            dst.template store_transposed<LDT>(Dt_, tid);
            if (tid < BQ) {
                Ls[tid] = lreg;
                Dl[tid] = dreg;
            }
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

template <Dt DT, int D>
static hipError_t dq_dispatch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                              const float *delta, void *dq, const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int WAVES = 4, BC = 64, BR = 32 * WAVES;
    const int nqb = (s.n_q + BR - 1) / BR;
    const int total = (int)(s.bh * nqb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((dq_kernel<DT, D, BC, WAVES>), dim3(total), dim3(WAVES * 64), 0, stream, (const elem *)q,
                       (const elem *)k, (const elem *)v, (const elem *)d_o, lse, delta, (elem *)dq, s.n_q, s.n_k,
                       nqb, total, scale_log2, s.scale);
    return hipGetLastError();
}

template <Dt DT, int D>
static hipError_t dkdv_dispatch(const void *q, const void *k, const void *v, const void *d_o, const float *lse,
                                const float *delta, void *dk, void *dv, const AttnShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int WAVES = 4, BQ = 64, BKV = 32 * WAVES;
    static_assert(BKV == kDkdvKeysPerBlock, "key block");
    const int nkb = (s.n_k + BKV - 1) / BKV;
    const int total = (int)(s.bh * nkb);
    const float scale_log2 = (float)((double)s.scale * 1.4426950408889634);
    hipLaunchKernelGGL((dkdv_kernel<DT, D, BQ, WAVES>), dim3(total), dim3(WAVES * 64), 0, stream,
                       (const elem *)q, (const elem *)k, (const elem *)v, (const elem *)d_o, lse, delta,
                       (elem *)dk, (elem *)dv, s.n_q, s.n_k, nkb, total, scale_log2, s.scale);
    return hipGetLastError();
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
