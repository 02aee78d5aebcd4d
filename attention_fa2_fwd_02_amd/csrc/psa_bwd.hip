// Fused backward of the C2PSA attention block for small maps (key_dim 32 up
// to 512 pixels, key_dim 64 up to 128) (vision_rs
// psa.rs: the block's backward hooks psa_merge_attn_backward,
// psa_fa2_backward for both value halves, psa_pack_qkv_backward; vision-rs
// flash_attn2.rs "Backward - dQ" and "Backward - dK / dV" for the algebra).
//
// One probability matrix serves both value halves (value width 2 kd), so the
// block's gradient is that of a single attention with D_qk = kd, D_v = 2 kd:
//   p_ij  = exp(scale q_i.k_j - lse_i)             (lse from the forward)
//   delta_i = sum_c out_ic d_out_ic                  (c over the 2 kd channels)
//   dS_ij = p_ij (d_out_i.v_j - delta_i)
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i p_ij d_out_i
// Everything is read straight from the NCHW activations (qkv, out, d_out) and
// written straight into d_qkv (its Q, K, V_lo, V_hi channels, overwritten),
// in three launches and without atomics:
//   psa_delta_kernel     - delta per pixel from out and d_out;
//   psa_bwd_dq_kernel    - one workgroup per (head, 128 queries), the head's
//                          whole K^T and V^T in LDS (the forward's layout);
//   psa_bwd_dkdv_kernel  - one workgroup per (head, 128 keys), the head's
//                          whole Q^T and d_out^T in LDS.
// Operands sit channel-major in LDS as they come from NCHW: products that
// contract over channels read them with ds_read_b64_tr_b16, products that
// contract over pixels read them row-wise. Pixels past h*w load as zero:
// a zero key (k, v) only changes its own dk, dv, which are not stored; a
// zero query (q, d_out) with lse = +inf has p = 0.
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2mi {

namespace {

constexpr int kPsaBwdBlock = 128; // pixels per workgroup block

// delta[bh][n] = sum over the head's 2 kd output channels of out * d_out.
// One workgroup per (head, 256 pixels), one pixel per thread.
template <typename T, int DV>
__global__ __launch_bounds__(256) void psa_delta_kernel(const T *__restrict__ out, const T *__restrict__ d_out,
                                                        float *__restrict__ delta, int num_heads, int hw,
                                                        int blocks_per_head) {
    const int bh = blockIdx.x / blocks_per_head;
    const int p = (blockIdx.x % blocks_per_head) * 256 + threadIdx.x;
    if (p >= hw) return;
    const int b = bh / num_heads, hd = bh % num_heads;
    const int64_t base = ((int64_t)b * num_heads * DV + (int64_t)hd * DV) * hw + p;
    float acc = 0.f;
#pragma unroll 8
    for (int c = 0; c < DV; ++c) acc += static_cast<float>(out[base + (int64_t)c * hw]) *
                                        static_cast<float>(d_out[base + (int64_t)c * hw]);
    delta[(int64_t)bh * hw + p] = acc;
}

// The channel-major operand arrays use shifted rows (row_shift): the
// transposing reads take 4 consecutive rows at a time, the row reads 32
// consecutive rows at once, and both stay free of bank conflicts (without
// the shift the row reads on these 64-byte-odd strides are 8-way).

// Row fragment (as ld_t_frag) of row `row` of a shifted array.
template <Dt DT>
__device__ __forceinline__ typename Traits<DT>::frag ld_row_sh(const typename Traits<DT>::elem *tile, int LD, int row,
                                                                int kb, int t, int h) {
    return ld_t_frag<DT>(tile + row * LD + row_shift(row), kb, t, h);
}

// ROWS channel rows x CAP pixels (pixels p0 .. p0 + CAP - 1, zero at or past
// hw) of one head's NCHW channel group, staged through registers into LDS
// rows of stride LD. Thread tid owns the 16-byte column tid % VPR of rows
// tid / VPR + RPP * i, so its offsets only step by whole rows.
template <Dt DT, int ROWS, int CAP, int NT>
struct ChanStage {
    using elem = typename Traits<DT>::elem;
    static constexpr int VEC = 8, VPR = CAP / VEC, RPP = NT / VPR;
    static constexpr int PER = (ROWS + RPP - 1) / RPP;
    static_assert(NT % VPR == 0 && (ROWS % RPP == 0 || RPP % ROWS == 0), "load mapping");
    uint4 v[PER];

    // rows row0 .. row0 + ROWS - 1 of the buffer that `rs` / `base` cover
    template <bool ALIGNED>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, const elem *base, int row0, int p0, int hw,
                                         int tid) {
        const int cv = tid % VPR, r0 = tid / VPR;
        const int p = p0 + cv * VEC;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int row = r0 + RPP * i;
            if (!(ROWS % RPP == 0 || row < ROWS)) continue;
            if constexpr (ALIGNED) {
                const uint32_t off =
                    p < hw ? ((uint32_t)(row0 + row) * hw + p) * (uint32_t)sizeof(elem) : 0xfffffff0u;
                v[i] = buffer_load16(rs, off);
            } else {
                uint4 x = make_uint4(0, 0, 0, 0);
                elem *e = reinterpret_cast<elem *>(&x);
                const elem *rp = base + (int64_t)(row0 + row) * hw;
#pragma unroll
                for (int k = 0; k < VEC; ++k)
                    if (p + k < hw) e[k] = rp[p + k];
                v[i] = x;
            }
        }
    }

    template <int LD>
    __device__ __forceinline__ void store(elem *lds, int tid) const {
        const int cv = tid % VPR, r0 = tid / VPR;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int row = r0 + RPP * i;
            if (!(ROWS % RPP == 0 || row < ROWS)) continue;
            // LD and the shifts are multiples of 8 elements: 16-byte aligned
            *reinterpret_cast<uint4 *>(lds + row * LD + row_shift(row) + cv * VEC) = v[i];
        }
    }
};

// Shared geometry: W = whole-map operand pair ([KD][CAP], [DV][CAP]), B =
// 128-pixel block pair ([KD][128], [DV][128]). Row strides are an odd number
// of 64-byte units (conflict-free transposing reads), rows shifted as above.
template <int KD_, int CAP>
struct PsaBwdCfg {
    static constexpr int KD = KD_, DV = 2 * KD, BR = kPsaBwdBlock, NT = 512;
    static constexpr int LDW = CAP + 32, LDB = BR + 32;
    static constexpr int W_K = KD * LDW, W_V = DV * LDW, B_K = KD * LDB, B_V = DV * LDB;
    static constexpr int NBH = CAP / 64;  // most 32-pixel blocks of one half of the map
    static constexpr int OPS_BYTES = 2 * (W_K + W_V + B_K + B_V);
    static_assert(OPS_BYTES + 2 * CAP * 4 <= 160 * 1024, "LDS");
    // partial results exchanged through the operand space afterwards
    // (floats per lane): dQ^T blocks; dK^T and dV^T blocks
    static constexpr int XQ = 16 * (KD / 32), XKV = 16 * (KD / 32 + DV / 32);
    static_assert(4 * 64 * XQ * 4 <= OPS_BYTES && 4 * 64 * XKV * 4 <= OPS_BYTES, "exchange");
};

}  // namespace

// ---------------------------------------------------------------------------
// dQ: workgroup (head, 128 queries); wave (qs, ks) = query slice qs (32
// queries, lane = query), key half ks of the map's 32-key blocks:
//   S^T = K Q^T, dP^T = V d_out^T (A from the whole-map K^T / V^T with
//   transposing reads, B from the block's Q^T / d_out^T likewise),
//   dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (K^T rows, dS^T as B);
// the two key halves' partial dQ^T are added through LDS.
template <Dt DT, int KD_, int CAP, bool ALIGNED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void psa_bwd_dq_kernel(
    const typename Traits<DT>::elem *__restrict__ qkv, const typename Traits<DT>::elem *__restrict__ d_out,
    const float *__restrict__ lse, const float *__restrict__ delta, typename Traits<DT>::elem *__restrict__ d_qkv,
    int num_heads, int hw, int n_blocks, int total_blocks, float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using C = PsaBwdCfg<KD_, CAP>;
    constexpr int KD = C::KD, DV = C::DV, BR = C::BR, NT = C::NT, LDW = C::LDW, LDB = C::LDB;
    constexpr int NCB = KD / 32;  // 32-channel blocks of dQ^T
    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[C::OPS_BYTES];
    elem *Kt = reinterpret_cast<elem *>(lds_raw);
    elem *Vt = Kt + C::W_K;
    elem *Qt = Vt + C::W_V;
    elem *Dt_ = Qt + C::B_K;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qs = wave & 3, ks = wave >> 2;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_blocks, qblk = blk % n_blocks;
    const int b = bh / num_heads, hd = bh % num_heads;
    const int q0 = qblk * BR;
    const elem *qbase = qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * hw;
    const elem *dbase = d_out + ((int64_t)b * num_heads * DV + (int64_t)hd * DV) * hw;
    elem *gbase = d_qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * hw;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, (uint32_t)(4 * KD * hw) * (uint32_t)sizeof(elem));
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dbase, (uint32_t)(DV * hw) * (uint32_t)sizeof(elem));

    {
        ChanStage<DT, KD, CAP, NT> sk;
        ChanStage<DT, DV, CAP, NT> sv;
        ChanStage<DT, KD, BR, NT> sq;
        ChanStage<DT, DV, BR, NT> sd;
        sq.template load<ALIGNED>(rq, qbase, 0, q0, hw, tid);
        sd.template load<ALIGNED>(rd, dbase, 0, q0, hw, tid);
        sk.template load<ALIGNED>(rq, qbase, KD, 0, hw, tid);
        sv.template load<ALIGNED>(rq, qbase, 2 * KD, 0, hw, tid);
        sq.template store<LDB>(Qt, tid);
        sd.template store<LDB>(Dt_, tid);
        sk.template store<LDW>(Kt, tid);
        sv.template store<LDW>(Vt, tid);
    }
    const int qrow = q0 + 32 * qs + col;
    // invalid query rows: zero operands and lse = +inf, so every p is 0
    const float lse2 = qrow < hw ? lse[(int64_t)bh * hw + qrow] * kLog2e : INFINITY;
    const float dl = qrow < hw ? delta[(int64_t)bh * hw + qrow] : 0.f;
    __syncthreads();

    const int nblk = (hw + 31) / 32, nb_lo = (nblk + 1) / 2;
    const int kb0 = ks ? nb_lo : 0;
    const int nb = ks ? nblk - nb_lo : nb_lo;
    const bool active = q0 + 32 * qs < hw && nb > 0;
    f32x16 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();
    if (active) {
        frag qf[KD / 16], df[DV / 16];
#pragma unroll
        for (int t = 0; t < KD / 16; ++t) qf[t] = ld_vt_frag_tr_sh<DT>(Qt, LDB, 16 * t, 32 * qs, lane);
#pragma unroll
        for (int t = 0; t < DV / 16; ++t) df[t] = ld_vt_frag_tr_sh<DT>(Dt_, LDB, 16 * t, 32 * qs, lane);
#pragma unroll
        for (int kb = 0; kb < C::NBH; ++kb) {
            if (kb >= nb) break;
            const int key0 = 32 * (kb0 + kb);
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < KD / 16; ++t) s = Tr::mfma(ld_vt_frag_tr_sh<DT>(Kt, LDW, 16 * t, key0, lane), qf[t], s);
#pragma unroll
            for (int t = 0; t < DV / 16; ++t) dp = Tr::mfma(ld_vt_frag_tr_sh<DT>(Vt, LDW, 16 * t, key0, lane), df[t], dp);
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lse2));
                s[c] = p * (dp[c] - dl);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const frag dsf = c_to_frag<DT>(s, t);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[cb] = Tr::mfma(ld_row_sh<DT>(Kt, LDW, 32 * cb + col, kb0 + kb, t, h), dsf, acc[cb]);
            }
        }
    }
    __syncthreads();  // K^T / V^T no longer read: reuse the space

    // key half 1 hands its partial dQ^T (registers c of lane (col, h) in
    // each channel block) to half 0 of the same query slice
    constexpr int XQ = C::XQ;
    float *xch = reinterpret_cast<float *>(lds_raw);  // [qs][64 lanes][XQ]
    if (ks == 1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4 *>(xch + (qs * 64 + lane) * XQ + 16 * cb + 4 * g) =
                    make_float4(acc[cb][4 * g], acc[cb][4 * g + 1], acc[cb][4 * g + 2], acc[cb][4 * g + 3]);
    }
    __syncthreads();
    if (ks == 0 && qrow < hw) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 o = *reinterpret_cast<const float4 *>(xch + (qs * 64 + lane) * XQ + 16 * cb + 4 * g);
                const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int chn = 32 * cb + crow(4 * g + i, h);  // Q channel
                    gbase[(int64_t)chn * hw + qrow] = static_cast<elem>((acc[cb][4 * g + i] + ov[i]) * scale);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup (head, 128 keys); wave (ks, qh) = key slice ks (32 keys,
// lane = key), query half qh of the map's 32-query blocks:
//   S = Q K^T, dP = d_out V^T (A from the whole-map Q^T / d_out^T with
//   transposing reads, B = the slice's K / V, read once),
//   P = exp2(S scale log2e - lse log2e), dS = P (dP - delta),
//   dV^T += d_out^T P, dK^T += Q^T dS (A = rows of d_out^T / Q^T);
// the two query halves' partial dK^T, dV^T are added through LDS.
template <Dt DT, int KD_, int CAP, bool ALIGNED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void psa_bwd_dkdv_kernel(
    const typename Traits<DT>::elem *__restrict__ qkv, const typename Traits<DT>::elem *__restrict__ d_out,
    const float *__restrict__ lse, const float *__restrict__ delta, typename Traits<DT>::elem *__restrict__ d_qkv,
    int num_heads, int hw, int n_blocks, int total_blocks, float scale_log2, float scale) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using C = PsaBwdCfg<KD_, CAP>;
    constexpr int KD = C::KD, DV = C::DV, BR = C::BR, NT = C::NT, LDW = C::LDW, LDB = C::LDB;
    constexpr int NCB = KD / 32;  // 32-channel blocks of dK^T
    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[C::OPS_BYTES];
    __shared__ __attribute__((aligned(16))) float Ls[CAP];
    __shared__ __attribute__((aligned(16))) float Dl[CAP];
    elem *Qt = reinterpret_cast<elem *>(lds_raw);
    elem *Dt_ = Qt + C::W_K;
    elem *Kt = Dt_ + C::W_V;
    elem *Vt = Kt + C::B_K;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ks = wave & 3, qh = wave >> 2;
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_blocks, kblk = blk % n_blocks;
    const int b = bh / num_heads, hd = bh % num_heads;
    const int k0 = kblk * BR;
    const elem *qbase = qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * hw;
    const elem *dbase = d_out + ((int64_t)b * num_heads * DV + (int64_t)hd * DV) * hw;
    elem *gbase = d_qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * hw;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, (uint32_t)(4 * KD * hw) * (uint32_t)sizeof(elem));
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dbase, (uint32_t)(DV * hw) * (uint32_t)sizeof(elem));

    {
        ChanStage<DT, KD, BR, NT> sk;
        ChanStage<DT, DV, BR, NT> sv;
        ChanStage<DT, KD, CAP, NT> sq;
        ChanStage<DT, DV, CAP, NT> sd;
        sk.template load<ALIGNED>(rq, qbase, KD, k0, hw, tid);
        sv.template load<ALIGNED>(rq, qbase, 2 * KD, k0, hw, tid);
        sq.template load<ALIGNED>(rq, qbase, 0, 0, hw, tid);
        sd.template load<ALIGNED>(rd, dbase, 0, 0, hw, tid);
        sk.template store<LDB>(Kt, tid);
        sv.template store<LDB>(Vt, tid);
        sq.template store<LDW>(Qt, tid);
        sd.template store<LDW>(Dt_, tid);
    }
    static_assert(CAP <= NT, "lse staging");
    if (tid < CAP) {
        // pixels past hw: lse = +inf, so their p is 0
        Ls[tid] = tid < hw ? lse[(int64_t)bh * hw + tid] * kLog2e : INFINITY;
        Dl[tid] = tid < hw ? delta[(int64_t)bh * hw + tid] : 0.f;
    }
    __syncthreads();

    const int nblk = (hw + 31) / 32, nb_lo = (nblk + 1) / 2;
    const int qb0 = qh ? nb_lo : 0;
    const int nb = qh ? nblk - nb_lo : nb_lo;
    const bool active = k0 + 32 * ks < hw && nb > 0;
    f32x16 accK[NCB], accV[DV / 32];
#pragma unroll
    for (int i = 0; i < NCB; ++i) accK[i] = zero16();
#pragma unroll
    for (int i = 0; i < DV / 32; ++i) accV[i] = zero16();
    if (active) {
        frag kf[KD / 16], vf[DV / 16];
#pragma unroll
        for (int t = 0; t < KD / 16; ++t) kf[t] = ld_vt_frag_tr_sh<DT>(Kt, LDB, 16 * t, 32 * ks, lane);
#pragma unroll
        for (int t = 0; t < DV / 16; ++t) vf[t] = ld_vt_frag_tr_sh<DT>(Vt, LDB, 16 * t, 32 * ks, lane);
#pragma unroll
        for (int qb = 0; qb < C::NBH; ++qb) {
            if (qb >= nb) break;
            const int qblock = qb0 + qb;
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < KD / 16; ++t)
                s = Tr::mfma(ld_vt_frag_tr_sh<DT>(Qt, LDW, 16 * t, 32 * qblock, lane), kf[t], s);
#pragma unroll
            for (int t = 0; t < DV / 16; ++t) dp = Tr::mfma(ld_vt_frag_tr_sh<DT>(Dt_, LDW, 16 * t, 32 * qblock, lane), vf[t], dp);
            // register c of lane half h is query 32 qblock + crow(c, h)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4 *>(Ls + 32 * qblock + 8 * g + 4 * h);
                const float4 d4 = *reinterpret_cast<const float4 *>(Dl + 32 * qblock + 8 * g + 4 * h);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * g + i;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c], scale_log2, -lv[i]));
                    s[c] = p;
                    dp[c] = p * (dp[c] - dv[i]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const frag pf = c_to_frag<DT>(s, t);
                const frag dsf = c_to_frag<DT>(dp, t);
#pragma unroll
                for (int db = 0; db < DV / 32; ++db)
                    accV[db] = Tr::mfma(ld_row_sh<DT>(Dt_, LDW, 32 * db + col, qblock, t, h), pf, accV[db]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    accK[cb] = Tr::mfma(ld_row_sh<DT>(Qt, LDW, 32 * cb + col, qblock, t, h), dsf, accK[cb]);
            }
        }
    }
    __syncthreads();  // Q^T / d_out^T no longer read: reuse the space

    // query half 1 hands its partial dK^T, dV^T to half 0 of the same key slice
    constexpr int XF = C::XKV;  // floats per lane: dK^T blocks, then dV^T blocks
    float *xch = reinterpret_cast<float *>(lds_raw);  // [ks][64 lanes][XF]
    if (qh == 1) {
        float *dst = xch + (ks * 64 + lane) * XF;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                *reinterpret_cast<float4 *>(dst + 16 * cb + 4 * g) =
                    make_float4(accK[cb][4 * g], accK[cb][4 * g + 1], accK[cb][4 * g + 2], accK[cb][4 * g + 3]);
#pragma unroll
            for (int db = 0; db < DV / 32; ++db)
                *reinterpret_cast<float4 *>(dst + 16 * (NCB + db) + 4 * g) =
                    make_float4(accV[db][4 * g], accV[db][4 * g + 1], accV[db][4 * g + 2], accV[db][4 * g + 3]);
        }
    }
    __syncthreads();
    const int krow = k0 + 32 * ks + col;
    if (qh == 0 && krow < hw) {
        const float *src = xch + (ks * 64 + lane) * XF;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const float4 ok = *reinterpret_cast<const float4 *>(src + 16 * cb + 4 * g);
                const float okv[4] = {ok.x, ok.y, ok.z, ok.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * g + i;
                    gbase[(int64_t)(KD + 32 * cb + crow(c, h)) * hw + krow] =
                        static_cast<elem>((accK[cb][c] + okv[i]) * scale);
                }
            }
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) {
                const float4 ov = *reinterpret_cast<const float4 *>(src + 16 * (NCB + db) + 4 * g);
                const float ovv[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * g + i;
                    gbase[(int64_t)(2 * KD + 32 * db + crow(c, h)) * hw + krow] =
                        static_cast<elem>(accV[db][c] + ovv[i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------

namespace {

template <Dt DT, int KD, int CAP, bool ALIGNED>
hipError_t psa_bwd_launch(const void *qkv, const void *out, const float *lse, const void *d_out, void *d_qkv,
                          float *delta, const PsaShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BR = kPsaBwdBlock;
    const int bhn = s.batch * s.num_heads;
    const int nblocks = (s.hw + BR - 1) / BR;
    const int grid = bhn * nblocks;
    const float scale = (float)(1.0 / __builtin_sqrt((double)KD));
    const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)KD));
    const int bph = (s.hw + 255) / 256;
    hipLaunchKernelGGL((psa_delta_kernel<elem, 2 * KD>), dim3(bhn * bph), dim3(256), 0, stream, (const elem *)out,
                       (const elem *)d_out, delta, s.num_heads, s.hw, bph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((psa_bwd_dq_kernel<DT, KD, CAP, ALIGNED>), dim3(grid), dim3(512), 0, stream, (const elem *)qkv,
                       (const elem *)d_out, lse, (const float *)delta, (elem *)d_qkv, s.num_heads, s.hw, nblocks,
                       grid, scale_log2, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((psa_bwd_dkdv_kernel<DT, KD, CAP, ALIGNED>), dim3(grid), dim3(512), 0, stream,
                       (const elem *)qkv, (const elem *)d_out, lse, (const float *)delta, (elem *)d_qkv,
                       s.num_heads, s.hw, nblocks, grid, scale_log2, scale);
    return hipGetLastError();
}

template <Dt DT, int KD, int CAP>
hipError_t psa_bwd_aligned(const void *qkv, const void *out, const float *lse, const void *d_out, void *d_qkv,
                           float *delta, const PsaShape &s, hipStream_t stream) {
    if (s.hw % 8 == 0) return psa_bwd_launch<DT, KD, CAP, true>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    return psa_bwd_launch<DT, KD, CAP, false>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
}

// Smallest whole-map capacity that holds the map: 64, 128, 256 or 512
// pixels at key_dim 32; 64 or 128 at key_dim 64 (the LDS holds the map's
// Q^T, d_out^T or K^T, V^T plus a block of the other pair; capacities are
// powers of two for the load mapping).
template <Dt DT, int KD>
hipError_t psa_bwd_dispatch(const void *qkv, const void *out, const float *lse, const void *d_out, void *d_qkv,
                            float *delta, const PsaShape &s, hipStream_t stream) {
    if (s.hw <= 64) return psa_bwd_aligned<DT, KD, 64>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    if (s.hw <= 128) return psa_bwd_aligned<DT, KD, 128>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    if constexpr (KD == 32) {
        if (s.hw <= 256) return psa_bwd_aligned<DT, KD, 256>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
        return psa_bwd_aligned<DT, KD, 512>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_psa_fused_backward(int dt, const void *qkv, const void *out, const float *lse, const void *d_out,
                                     void *d_qkv, float *delta, const PsaShape &s, hipStream_t stream) {
    if (s.hw > psa_fused_bwd_max_pixels(s.key_dim)) return hipErrorInvalidValue;
    if (s.key_dim == 32) {
        if (dt == 1) return psa_bwd_dispatch<Dt::F16, 32>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
        if (dt == 2) return psa_bwd_dispatch<Dt::BF16, 32>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    } else if (s.key_dim == 64) {
        if (dt == 1) return psa_bwd_dispatch<Dt::F16, 64>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
        if (dt == 2) return psa_bwd_dispatch<Dt::BF16, 64>(qkv, out, lse, d_out, d_qkv, delta, s, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa2mi
