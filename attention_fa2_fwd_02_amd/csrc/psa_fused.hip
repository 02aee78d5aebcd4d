// Fused PSA attention forward: the pack -> attention(V_lo) -> attention(V_hi)
// -> merge sequence of a C2PSA block (vision_rs psa.rs, module doc and
// "psa_pack_qkv", "psa_merge_attn_nchw") in one kernel that reads the NCHW
// qkv activation directly and writes the NCHW output directly.
//
// For head (b, hd) the channels of qkv are Q = hd*4kd + [0, kd),
// K = +[kd, 2kd), V = [V_lo | V_hi] = +[2kd, 4kd); each channel is a row of
// h*w pixels. So Q^T [kd][N], K^T [kd][N] and V^T [2kd][N] are row blocks of
// the activation, and the output O^T [2kd][N] is the row block of channels
// hd*2kd + [0, 2kd) of `out`. Both value halves share one probability matrix
// (the split into V_lo and V_hi of the pages only exists because of their
// power-of-two head_dim; P is the same for both), so attention runs once
// with value width 2kd.
//
// MFMA mapping (16-bit types): S^T = K Q^T with the A operand K and the B
// operand Q both read from their channel-major LDS tiles with the
// transposing LDS read (the contraction order over channels is the same
// permutation on both sides); O^T += V^T P^T with V^T read directly from its
// channel-major (key-contiguous) tile. O^T keeps one query per lane, so the
// epilogue stages it through LDS and writes pixel-contiguous rows.
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2mi {

// One key tile of the fused PSA forward for one wave (K^T and V^T tiles in
// LDS): scores, online softmax with lazy rescaling, P V. MASK: the tile is
// the ragged last one (keys at or beyond kvalid get probability 0).
template <Dt DT, int KD, int LDKT, int LDVT, bool MASK>
__device__ __forceinline__ void psa_tile(const typename Traits<DT>::elem *kt, const typename Traits<DT>::elem *vt,
                                         const typename Traits<DT>::frag (&qf)[KD / 16], f32x16 (&acc)[KD / 16],
                                         float &m_ref, float &l_run, float scale_log2, int kvalid, int lane) {
    using Tr = Traits<DT>;
    using frag = typename Tr::frag;
    constexpr int TS = KD / 16, NKB = 2, NDB = 2 * KD / 32;
    const int h = lane >> 5, col = lane & 31;
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            s[kb] = Tr::mfma(ld_vt_frag_tr<DT>(kt, LDKT, 16 * t, 32 * kb, lane), qf[t], s[kb]);
    if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < 16; ++c)
                if (32 * kb + crow(c, h) >= kvalid) s[kb][c] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 16; ++c) mx = fmaxf(mx, s[kb][c]);
    const float mx2 = mx * scale_log2;
    if (__any(mx2 > m_ref + kRescaleLog2)) {
        const float m_new = fmaxf(m_ref, xhalf_max(mx2));
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[db][c] *= alpha;
        l_run *= alpha;
        m_ref = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][c], scale_log2, -m_ref));
            s[kb][c] = p;
            l_run += p;
        }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const frag pf = c_to_frag<DT>(s[kb], t);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = Tr::mfma(ld_t_frag<DT>(vt + (32 * db + col) * LDVT, kb, t, h), pf, acc[db]);
        }
}

template <Dt DT, int KD, int WAVES, bool ALIGNED>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void psa_fused_kernel(const typename Traits<DT>::elem *__restrict__ qkv,
                                                               typename Traits<DT>::elem *__restrict__ out,
                                                               float *__restrict__ lse, int num_heads, int hw,
                                                               int n_qblocks, float scale_log2) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    static_assert(Tr::KPL == 8, "16-bit element types");
    constexpr int NT = WAVES * 64;
    constexpr int BR = 32 * WAVES;     // queries per workgroup
    constexpr int BC = 64;             // keys per tile
    constexpr int DV = 2 * KD;         // value width (V_lo | V_hi)
    constexpr int VEC = 8;             // elements per 16-byte vector
    constexpr int TS = KD / 16;        // contraction steps over channels
    constexpr int NKB = BC / 32;
    constexpr int NDB = DV / 32;
    // LDS strides (elements). Transposing reads serve 4 rows x 64 bytes per
    // cycle: Q^T rows (BR queries) and K^T rows (BC keys) start 64 bytes apart
    // modulo 256. V^T rows are read 8 bytes per lane down 32 rows.
    constexpr int LDQ = BR + 32;
    constexpr int LDKT = BC + 32;
    constexpr int LDVT = BC + 4;
    constexpr int LDO = BR + 8;        // output staging rows
    constexpr int KSZ = KD * LDKT, VSZ = DV * LDVT;
    constexpr int QSZ = KD * LDQ;
    constexpr int OSZ = DV * LDO;
    constexpr int STAGE = KSZ + VSZ;
    constexpr int LDS_ELEMS = QSZ + (2 * STAGE > OSZ ? 2 * STAGE : OSZ);
    __shared__ __attribute__((aligned(16))) elem lds[LDS_ELEMS];
    elem *Qt = lds;
    elem *stage0 = lds + QSZ;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    const int bh = blockIdx.x / n_qblocks, qb = blockIdx.x % n_qblocks;
    const int b = bh / num_heads, hd = bh % num_heads;
    const int q0 = qb * BR;
    const int64_t plane = (int64_t)hw;
    const elem *qbase = qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * plane;
    const elem *kbase = qbase + (int64_t)KD * plane;
    const elem *vbase = qbase + (int64_t)2 * KD * plane;
    elem *obase = out + ((int64_t)b * num_heads * DV + (int64_t)hd * DV) * plane;

    // one row-vector of a channel-major block: rows x cols pixels starting
    // at pixel p0; pixels past hw read as zero
    auto ldrow = [&](const elem *rowp, int p) -> uint4 {
        uint4 v = make_uint4(0, 0, 0, 0);
        if constexpr (ALIGNED) {
            if (p < hw) v = *reinterpret_cast<const uint4 *>(rowp + p);
        } else {
            elem *e = reinterpret_cast<elem *>(&v);
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                if (p + i < hw) e[i] = rowp[p + i];
        }
        return v;
    };

    // Q^T block [KD][BR]
    for (int i = tid; i < KD * (BR / VEC); i += NT) {
        const int r = i / (BR / VEC), cv = i % (BR / VEC);
        *reinterpret_cast<uint4 *>(Qt + r * LDQ + cv * VEC) = ldrow(qbase + r * plane, q0 + cv * VEC);
    }
    // K^T [KD][BC] and V^T [DV][BC] tiles through registers into one stage
    constexpr int KV_VECS = (KD + DV) * (BC / VEC);
    constexpr int PER = (KV_VECS + NT - 1) / NT;
    uint4 reg[PER];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * NT;
            if (KV_VECS % NT == 0 || v < KV_VECS) {
                const int r = v / (BC / VEC), cv = v % (BC / VEC);
                const elem *rowp = r < KD ? kbase + r * plane : vbase + (r - KD) * plane;
                reg[i] = ldrow(rowp, j0 + cv * VEC);
            }
        }
    };
    auto store_tile = [&](elem *st) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = tid + i * NT;
            if (KV_VECS % NT == 0 || v < KV_VECS) {
                const int r = v / (BC / VEC), cv = v % (BC / VEC);
                elem *dst = r < KD ? st + r * LDKT + cv * VEC : st + KSZ + (r - KD) * LDVT + cv * VEC;
                if (r < KD)
                    *reinterpret_cast<uint4 *>(dst) = reg[i];
                else {  // V^T rows are 8-byte aligned (LDVT = BC + 4)
                    reinterpret_cast<uint2 *>(dst)[0] = make_uint2(reg[i].x, reg[i].y);
                    reinterpret_cast<uint2 *>(dst)[1] = make_uint2(reg[i].z, reg[i].w);
                }
            }
        }
    };

    const int ntiles = (hw + BC - 1) / BC;
    load_tile(0);
    store_tile(stage0);
    if (ntiles > 1) load_tile(BC);
    __syncthreads();

    // Q fragments (B operand of S^T): channel order of the transposing read
    frag qf[TS];
#pragma unroll
    for (int t = 0; t < TS; ++t) qf[t] = ld_vt_frag_tr<DT>(Qt, LDQ, 16 * t, 32 * wave, lane);

    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = zero16();
    float m_ref = -INFINITY, l_run = 0.f;

    const int nfull = hw / BC;
    for (int it = 0; it < nfull; ++it) {
        const elem *kt = stage0 + (it & 1) * STAGE;
        psa_tile<DT, KD, LDKT, LDVT, false>(kt, kt + KSZ, qf, acc, m_ref, l_run, scale_log2, BC, lane);
        if (it + 1 < ntiles) {
            store_tile(stage0 + ((it + 1) & 1) * STAGE);
            if (it + 2 < ntiles) load_tile((it + 2) * BC);
        }
        __syncthreads();
    }
    if (nfull < ntiles) {
        const elem *kt = stage0 + (nfull & 1) * STAGE;
        psa_tile<DT, KD, LDKT, LDVT, true>(kt, kt + KSZ, qf, acc, m_ref, l_run, scale_log2, hw - nfull * BC, lane);
        __syncthreads();
    }

    // epilogue: O^T / l into LDS (rows = output channels; the K/V stages are
    // free after the last barrier), then pixel-contiguous 16-byte stores
    const float l_tot = xhalf_sum(l_run);
    const float inv = 1.f / l_tot;
    const int qrow = q0 + wave * 32 + col;
    if (lse != nullptr && h == 0 && qrow < hw) lse[(int64_t)bh * hw + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
    elem *Os = stage0;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 16; ++c) Os[(32 * db + crow(c, h)) * LDO + wave * 32 + col] = static_cast<elem>(acc[db][c] * inv);
    __syncthreads();
    for (int i = tid; i < DV * (BR / VEC); i += NT) {
        const int r = i / (BR / VEC), cv = i % (BR / VEC);
        const int p = q0 + cv * VEC;
        if (p >= hw) continue;
        uint4 v;
        elem *e = reinterpret_cast<elem *>(&v);
#pragma unroll
        for (int k = 0; k < VEC; ++k) e[k] = Os[r * LDO + cv * VEC + k];
        elem *dst = obase + r * plane + p;
        if constexpr (ALIGNED) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                if (p + k < hw) dst[k] = e[k];
        }
    }
}


template <Dt DT, int KD, int WAVES>
static hipError_t psa_fused_launch(const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BR = 32 * WAVES;
    const int nqb = (s.hw + BR - 1) / BR;
    const int grid = s.batch * s.num_heads * nqb;
    const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)KD));
    if (s.hw % 8 == 0)
        hipLaunchKernelGGL((psa_fused_kernel<DT, KD, WAVES, true>), dim3(grid), dim3(WAVES * 64), 0, stream,
                           (const elem *)qkv, (elem *)out, lse, s.num_heads, s.hw, nqb, scale_log2);
    else
        hipLaunchKernelGGL((psa_fused_kernel<DT, KD, WAVES, false>), dim3(grid), dim3(WAVES * 64), 0, stream,
                           (const elem *)qkv, (elem *)out, lse, s.num_heads, s.hw, nqb, scale_log2);
    return hipGetLastError();
}

// Query rows per workgroup: 128 (4 waves) for long sequences with many
// workgroups, else 64 (short sequences leave few waves per CU, and each
// wave's serial work, not K/V staging, sets the time).
template <Dt DT, int KD>
static hipError_t psa_fused_dispatch(const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream) {
    const int64_t bh = (int64_t)s.batch * s.num_heads;
    if (bh * ((s.hw + 127) / 128) >= 4 * 256) return psa_fused_launch<DT, KD, 4>(qkv, out, lse, s, stream);
    return psa_fused_launch<DT, KD, 2>(qkv, out, lse, s, stream);
}

hipError_t launch_psa_fused(int dt, const void *qkv, void *out, float *lse, const PsaShape &s,
                            hipStream_t stream) {
    if (dt == 1) {
        if (s.key_dim == 32) return psa_fused_dispatch<Dt::F16, 32>(qkv, out, lse, s, stream);
        if (s.key_dim == 64) return psa_fused_dispatch<Dt::F16, 64>(qkv, out, lse, s, stream);
    } else if (dt == 2) {
        if (s.key_dim == 32) return psa_fused_dispatch<Dt::BF16, 32>(qkv, out, lse, s, stream);
        if (s.key_dim == 64) return psa_fused_dispatch<Dt::BF16, 64>(qkv, out, lse, s, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa2mi
