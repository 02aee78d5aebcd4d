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


// Calls f(std::integral_constant<int, v>) for a wave-uniform 0 <= v < N, so
// that register arrays can be indexed with v at compile time.
template <int N, typename F>
__device__ __forceinline__ void uniform_switch(int v, F &&f) {
    if constexpr (N > 1) {
        if (v == N - 1) {
            f(std::integral_constant<int, N - 1>{});
            return;
        }
        uniform_switch<N - 1>(v, f);
    } else {
        f(std::integral_constant<int, 0>{});
    }
}

// Small feature maps (the usual C2PSA case: h*w of a few hundred pixels).
// One workgroup per (head, 128 queries) with 4 KS waves = 4 query sub-blocks
// of 32 x KS key slices (the map's ceil(h*w / 32) blocks of 32 keys split
// evenly; a ragged last block is masked). Wave w runs on SIMD w % 4, so the
// KS slices of one query sub-block share a SIMD. The head's whole K^T and
// V^T (zero past h*w) and the Q^T block are fetched with 16-byte loads:
// Q^T and K^T first, written to LDS, then V^T, whose loads are issued once
// Q^T and K^T have landed and arrive while the score products run;
// each wave keeps the scores of its key slice in registers, so its softmax
// needs one exact row max and one exp2 pass, no online rescaling; its block
// loops have wave-uniform trip counts. The KS slices of a query sub-block
// are merged through LDS with the online-softmax combination (max, rescaled
// sums), each wave finishing DV / KS of the value channels and storing them
// straight to the pixel rows. KS = 4 (16 waves, four per SIMD, at most 128
// VGPRs each) gives each SIMD more waves to hide latency with.
template <int KD, int NB, int KS = 2>
struct PsaSmallCfg {
    static constexpr int KC = 2 * NB * 32;       // key capacity (h*w <= KC)
    static constexpr int NBS = (2 * NB + KS - 1) / KS;  // 32-key blocks per slice, at most
    // LDS rows hold KCL >= KC keys, a power of two, so that the loads map
    // threads to (row, 16-byte column) with shifts
    static constexpr int KCL = KC <= 64 ? 64 : KC <= 128 ? 128 : KC <= 256 ? 256 : 512;
    static constexpr int DV = 2 * KD;            // value width (V_lo | V_hi)
    static constexpr int BR = 128;               // queries per workgroup
    static constexpr int NW = 4 * KS;            // waves
    static constexpr int CPS = DV / KS;          // value channels each wave finishes
    // LDS strides (elements): transposed reads of K^T and Q^T want rows an
    // odd number of 64-byte units apart; V^T rows (8-byte reads down 32 rows)
    // KCL + 4 elements apart.
    static constexpr int LDKT = KCL + 32;
    static constexpr int LDVT = KCL + 4;
    static constexpr int LDQ = BR + 32;
    static constexpr int KT_SZ = KD * LDKT, VT_SZ = DV * LDVT, QT_SZ = KD * LDQ;
    // after the products the LDS holds the merge exchange (float): per wave
    // and per other slice, 32 queries x CPS channels (+4 pad), then m and l
    static constexpr int LDX = CPS + 4;
    static constexpr int XCH_FLOATS = NW * (KS - 1) * 32 * LDX + NW * 2 * 32;
    static constexpr int MAIN_BYTES = 2 * (KT_SZ + VT_SZ + QT_SZ);
    // the exchange sits past the operands when both fit (no barrier before
    // it), else it reuses their space
    static constexpr bool SEPX = MAIN_BYTES + 4 * XCH_FLOATS <= 160 * 1024;
    static constexpr int LDS_BYTES = SEPX ? MAIN_BYTES + 4 * XCH_FLOATS
                                          : (MAIN_BYTES > 4 * XCH_FLOATS ? MAIN_BYTES : 4 * XCH_FLOATS);
    static_assert(LDS_BYTES <= 160 * 1024 && MAIN_BYTES % 16 == 0, "LDS");
    static_assert(CPS == 16 || CPS == 32 || CPS == 64, "channel slices of whole C-block halves");
};

// Largest map each key_dim handles with this kernel (32-key blocks per half).
template <int KD> constexpr int psa_small_max_nb() { return KD == 32 ? 7 : 4; }

template <Dt DT, int KD, int NB, bool ALIGNED, int KS = 2>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(KS, KS))) void psa_small_kernel(
    const typename Traits<DT>::elem *__restrict__ qkv, typename Traits<DT>::elem *__restrict__ out,
    float *__restrict__ lse, int num_heads, int hw, int n_qblocks, int total_blocks, float scale_log2) {
    using Tr = Traits<DT>;
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using C = PsaSmallCfg<KD, NB, KS>;
    static_assert(Tr::KPL == 8, "16-bit element types");
    constexpr int NT = 64 * C::NW, VEC = 8, TS = KD / 16, DV = C::DV, BR = C::BR, NDB = DV / 32;
    constexpr int NBS = C::NBS;
    constexpr int LDKT = C::LDKT, LDVT = C::LDVT, LDQ = C::LDQ;
    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[C::LDS_BYTES];
    elem *Kt = reinterpret_cast<elem *>(lds_raw);
    elem *Vt = Kt + C::KT_SZ;
    elem *Qt = Vt + C::VT_SZ;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qs = wave & 3, ks = wave >> 2;  // waves w, w+4, ... share a SIMD
    const int h = lane >> 5, col = lane & 31;
    const int blk = xcd_remap(blockIdx.x, total_blocks);
    const int bh = blk / n_qblocks, qb = blk % n_qblocks;
    const int b = bh / num_heads, hd = bh % num_heads;
    const int q0 = qb * BR;
    const int64_t plane = (int64_t)hw;
    // the head's 4*KD channel rows (Q, K, V_lo, V_hi) are contiguous
    const elem *qbase = qkv + ((int64_t)b * num_heads * 4 * KD + (int64_t)hd * 4 * KD) * plane;
    elem *obase = out + ((int64_t)b * num_heads * DV + (int64_t)hd * DV) * plane;

    // Loads: Q^T [KD][BR], K^T [KD][KCL] and V^T [DV][KCL] (all zero past
    // hw). Thread tid owns 16-byte column tid % VPR of rows tid / VPR + RPP * i
    // (VPR vectors per row, RPP rows per pass), so its offsets only step by
    // whole rows.
    constexpr int VPR = C::KCL / VEC, RPP = NT / VPR;
    constexpr int K_PER = (KD + RPP - 1) / RPP, V_PER = (DV + RPP - 1) / RPP;
    constexpr int QPR = BR / VEC;                        // Q^T: 16 vectors per row
    constexpr int QRP = NT / QPR;                        // Q^T rows per pass
    constexpr int Q_PER = (KD + QRP - 1) / QRP;
    static_assert((KD % RPP == 0 || RPP % KD == 0) && (DV % RPP == 0 || RPP % DV == 0), "load mapping");
    static_assert(KD % QRP == 0 || QRP % KD == 0, "load mapping");
    // buffer over the head's channel rows (Q, K, V_lo, V_hi are contiguous);
    // vectors past a row's hw pixels get an offset beyond the range and read
    // as zero
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(qbase, (uint32_t)(4 * KD * hw) * (uint32_t)sizeof(elem));
    const int cvec = tid % VPR, rbase = tid / VPR;
    const int pk = cvec * VEC;                          // this thread's key column
    const int qr = tid / QPR, qc = (tid % QPR) * VEC;   // its Q^T vectors
    auto load_vec = [&](int row, int p) -> uint4 {
        if constexpr (ALIGNED) {
            const uint32_t off = p < hw ? ((uint32_t)row * hw + p) * (uint32_t)sizeof(elem) : 0xfffffff0u;
            return buffer_load16(rs, off);
        } else {
            uint4 x = make_uint4(0, 0, 0, 0);
            elem *e = reinterpret_cast<elem *>(&x);
            const elem *rowp = qbase + (int64_t)row * plane;
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                if (p + k < hw) e[k] = rowp[p + k];
            return x;
        }
    };
    uint4 rq[Q_PER], rk[K_PER], rv[V_PER];
#pragma unroll
    for (int i = 0; i < Q_PER; ++i)
        if (KD % QRP == 0 || qr + QRP * i < KD) rq[i] = load_vec(qr + QRP * i, q0 + qc);
#pragma unroll
    for (int i = 0; i < K_PER; ++i)
        if (KD % RPP == 0 || rbase + RPP * i < KD) rk[i] = load_vec(KD + rbase + RPP * i, pk);
#pragma unroll
    for (int i = 0; i < Q_PER; ++i)
        if (KD % QRP == 0 || qr + QRP * i < KD) *reinterpret_cast<uint4 *>(Qt + (qr + QRP * i) * LDQ + qc) = rq[i];
#pragma unroll
    for (int i = 0; i < K_PER; ++i)
        if (KD % RPP == 0 || rbase + RPP * i < KD)
            *reinterpret_cast<uint4 *>(Kt + (rbase + RPP * i) * LDKT + pk) = rk[i];
    __syncthreads();
    // V^T (two thirds of the bytes) is requested only now, so that Q^T and
    // K^T, which the score products need first, do not share the memory
    // system with it; it streams in during those products
#pragma unroll
    for (int i = 0; i < V_PER; ++i)
        if (DV % RPP == 0 || rbase + RPP * i < DV) rv[i] = load_vec(2 * KD + rbase + RPP * i, pk);

    // this wave: queries q0 + 32 qs + [0, 32), key blocks kb0 + [0, nb): the
    // map's ceil(hw / 32) key blocks split evenly over the KS slices (the
    // first nblk % KS slices take one more; nb <= NBS since hw <= 64 NB);
    // blocks past nb are not computed
    const int nblk = (hw + 31) / 32, nbase = nblk / KS, nrem = nblk % KS;
    const int kb0 = ks * nbase + min(ks, nrem);
    const int nb = nbase + (ks < nrem ? 1 : 0);
    const bool active = q0 + 32 * qs < hw && nb > 0;
    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = zero16();
    float m = -INFINITY, l_run = 0.f;
    f32x16 s[NBS];
    if (active) {
        frag qf[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) qf[t] = ld_vt_frag_tr<DT>(Qt, LDQ, 16 * t, 32 * qs, lane);
#pragma unroll
        for (int kb = 0; kb < NBS; ++kb) {
            if (kb >= nb) break;
            s[kb] = zero16();
#pragma unroll
            for (int t = 0; t < TS; ++t)
                s[kb] = Tr::mfma(ld_vt_frag_tr<DT>(Kt, LDKT, 16 * t, 32 * (kb0 + kb), lane), qf[t], s[kb]);
        }
        // keys past hw do not exist (probability 0); only blocks that reach
        // past hw need the per-element test
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NBS; ++kb) {
            if (kb >= nb) break;
            if (32 * (kb0 + kb + 1) > hw) {
                const int limit = hw - 32 * (kb0 + kb) - 4 * h;  // first invalid crow - 4h
#pragma unroll
                for (int c = 0; c < 16; ++c) s[kb][c] = crow(c, 0) >= limit ? -INFINITY : s[kb][c];
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) mx = fmaxf(mx, s[kb][c]);
        }
        m = xhalf_max(mx) * scale_log2;  // exact max of this slice, log2 units
    }
    // V^T goes to LDS only now: its loads were issued after Q^T and K^T had
    // landed and streamed in during the products above
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
        if (DV % RPP == 0 || rbase + RPP * i < DV) {  // V^T rows are 8-byte aligned
            elem *dst = Vt + (rbase + RPP * i) * LDVT + pk;
            reinterpret_cast<uint2 *>(dst)[0] = make_uint2(rv[i].x, rv[i].y);
            reinterpret_cast<uint2 *>(dst)[1] = make_uint2(rv[i].z, rv[i].w);
        }
    }
    __syncthreads();
    if (active) {
        // probabilities block by block, so that the exp2 of a block overlaps
        // the P V products of the one before; the row sum is taken in float32
        // over the probabilities before they are rounded for the products
        // (a slice with no keys keeps m = -inf and contributes nothing)
        const float neg_m = m == -INFINITY ? 0.f : -m;
#pragma unroll
        for (int kb = 0; kb < NBS; ++kb) {
            if (kb >= nb) break;
#pragma unroll
            for (int c = 0; c < 16; ++c) s[kb][c] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][c], scale_log2, neg_m));
            l_run += sum16(s[kb]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const frag pf = c_to_frag<DT>(s[kb], t);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = Tr::mfma(ld_t_frag<DT>(Vt + (32 * db + col) * LDVT, kb0 + kb, t, h), pf, acc[db]);
            }
        }
    }
    const float l_slice = xhalf_sum(l_run);
    if constexpr (!C::SEPX) __syncthreads();  // K^T / V^T no longer read: reuse the space

    // Merge the KS slices. Wave (qs, ks) finishes channels [ks CPS, (ks+1)
    // CPS) and hands every other slice's channels to that slice's wave. A
    // slice j covers registers [RL(j), RL(j) + RN) of C block j CPS / 32 (RN =
    // 16 for whole blocks, 8 for half blocks: registers 8..15 hold channels
    // 16..31 of the block in both lane halves); registers 4g..4g+3 are 4
    // consecutive channels, moved as one 16-byte vector. Exchange layout:
    // [source wave][other-slice index][query][LDX] floats, then m and l.
    // NSB whole blocks per slice when CPS >= 32.
    constexpr int CPS = C::CPS, LDX = C::LDX, RN = CPS >= 32 ? 16 : 8, NSB = CPS >= 32 ? CPS / 32 : 1;
    float *xch = reinterpret_cast<float *>(lds_raw + (C::SEPX ? C::MAIN_BYTES : 0));
    float *ml = xch + C::NW * (KS - 1) * 32 * LDX;  // [wave][2][32]
    constexpr auto slice_db = [](int j) { return (j * CPS) / 32; };
    constexpr auto slice_rl = [](int j) { return CPS >= 32 ? 0 : ((j * CPS) % 32) / 2; };
    uniform_switch<KS>(ks, [&](auto ks_c) {
        constexpr int KSV = decltype(ks_c)::value;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            if (j == KSV) continue;
            const int jj = j < KSV ? j : j - 1;
            float *dst = xch + ((wave * (KS - 1) + jj) * 32 + col) * LDX;
            const int rl = slice_rl(j);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const f32x16 &a = acc[slice_db(j) + sb];
#pragma unroll
                for (int g = 0; g < RN / 4; ++g) {
                    const int c = rl + 4 * g;
                    *reinterpret_cast<float4 *>(dst + 32 * sb + crow(c, h) - 2 * rl) =
                        make_float4(a[c], a[c + 1], a[c + 2], a[c + 3]);
                }
            }
        }
    });
    if (h == 0) {
        ml[wave * 64 + col] = m;
        ml[wave * 64 + 32 + col] = l_slice;
    }
    __syncthreads();
    float mj[KS], lj[KS];
    float m_max = -INFINITY;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int w = qs + 4 * j;
        mj[j] = ml[w * 64 + col];
        lj[j] = ml[w * 64 + 32 + col];
        m_max = fmaxf(m_max, mj[j]);
    }
    float aj[KS];
    float l_tot = 0.f;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        aj[j] = mj[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj[j] - m_max);
        l_tot += lj[j] * aj[j];
    }
    const float inv = 1.f / l_tot;
    const int qrow = q0 + 32 * qs + col;
    if (lse != nullptr && ks == 0 && h == 0 && qrow < hw) lse[(int64_t)bh * hw + qrow] = (m_max + __log2f(l_tot)) * kLn2;
    if (qrow < hw) uniform_switch<KS>(ks, [&](auto ks_c) {
        // channel 32 db + crow(c, h), pixel qrow: each store instruction
        // writes 32 consecutive pixels of two channel rows
        constexpr int KSV = decltype(ks_c)::value;
        constexpr int rl = slice_rl(KSV);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const int db = slice_db(KSV) + sb;
            const f32x16 &a = acc[db];
#pragma unroll
            for (int g = 0; g < RN / 4; ++g) {
                const int c = rl + 4 * g;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = 0.f;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    float x[4];
                    if (j == KSV) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] = a[c + i];
                    } else {
                        const int jj = KSV < j ? KSV : KSV - 1;  // this slice's index in wave j's list
                        const float *src = xch + (((qs + 4 * j) * (KS - 1) + jj) * 32 + col) * LDX;
                        const float4 y = *reinterpret_cast<const float4 *>(src + 32 * sb + crow(c, h) - 2 * rl);
                        x[0] = y.x;
                        x[1] = y.y;
                        x[2] = y.z;
                        x[3] = y.w;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] += x[i] * aj[j];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int chn = 32 * db + crow(c + i, h);
                    obase[(int64_t)chn * plane + qrow] = static_cast<elem>(v[i] * inv);
                }
            }
        }
    });
}

template <Dt DT, int KD, int NB, int KS = 2>
static hipError_t psa_small_launch(const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream) {
    using elem = typename Traits<DT>::elem;
    constexpr int BR = PsaSmallCfg<KD, NB, KS>::BR;
    constexpr int NT = 64 * PsaSmallCfg<KD, NB, KS>::NW;
    const int nqb = (s.hw + BR - 1) / BR;
    const int grid = s.batch * s.num_heads * nqb;
    const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)KD));
    if (s.hw % 8 == 0)
        hipLaunchKernelGGL((psa_small_kernel<DT, KD, NB, true, KS>), dim3(grid), dim3(NT), 0, stream,
                           (const elem *)qkv, (elem *)out, lse, s.num_heads, s.hw, nqb, grid, scale_log2);
    else
        hipLaunchKernelGGL((psa_small_kernel<DT, KD, NB, false, KS>), dim3(grid), dim3(NT), 0, stream,
                           (const elem *)qkv, (elem *)out, lse, s.num_heads, s.hw, nqb, grid, scale_log2);
    return hipGetLastError();
}

// Smallest key capacity (64, 128, 256 or 448 keys) that holds the map.
template <Dt DT, int KD>
static hipError_t psa_small_dispatch(const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream) {
    if (s.hw <= 64) return psa_small_launch<DT, KD, 1>(qkv, out, lse, s, stream);
    if (s.hw <= 128) return psa_small_launch<DT, KD, 2>(qkv, out, lse, s, stream);
    if constexpr (psa_small_max_nb<KD>() == 7) {
        if (s.hw > 256) return psa_small_launch<DT, KD, 7>(qkv, out, lse, s, stream);
    }
    return psa_small_launch<DT, KD, 4>(qkv, out, lse, s, stream);
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

// Maps of at most 64 * psa_small_max_nb pixels take the whole-head kernel above.
// Larger ones use the tiled kernel with 128 query rows per workgroup (4
// waves) when there are many workgroups, else 64.
template <Dt DT, int KD>
static hipError_t psa_fused_dispatch(const void *qkv, void *out, float *lse, const PsaShape &s, hipStream_t stream) {
    if (s.hw <= 64 * psa_small_max_nb<KD>()) return psa_small_dispatch<DT, KD>(qkv, out, lse, s, stream);
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
