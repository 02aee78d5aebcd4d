/*
 * CPU oracle for exact scaled dot-product attention and the PSA
 * rearrangements. TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the library's compute path never does.
 * It shares no code, header or constant with the HIP kernels.
 *
 * Everything is the plain definition, materialised one score row at a time in
 * fp64 (no tiling, no online recurrence, no fusion):
 *
 *   s_ij  = scale * sum_d q_id k_jd                  (vision-rs flash_attn2.rs,
 *   m_i   = max_j s_ij                                 "Forward": scaled dot
 *   P_ij  = exp(s_ij - m_i) / sum_j exp(s_ij - m_i)    product, softmax, P V)
 *   O_ic  = sum_j P_ij v_jc
 *   LSE_i = m_i + ln(sum_j exp(s_ij - m_i))          (same page, "Forward":
 *                                                     log-sum-exp saved for
 *                                                     the backward pass)
 *
 * Backward, given dO (same page, "Backward - dQ" and "Backward - dK / dV"):
 *   dP_ij = sum_c dO_ic v_jc
 *   D_i   = sum_j P_ij dP_ij          (equal to sum_c O_ic dO_ic)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
 *   dV_j  = sum_i P_ij dO_i
 *
 * PSA rearrangements (vision_rs psa.rs, "psa_pack_qkv" and
 * "psa_merge_attn_nchw", and their backward kernels "psa_pack_qkv_backward"
 * and "psa_merge_attn_backward"): pure index maps, copied element by element.
 * The gradient of a permutation is the inverse permutation of the gradient.
 *
 * The query/key head dim (d) and the value head dim (dv) are separate so that
 * one attention with dv = 2*key_dim can be compared with two at dv = key_dim.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One query row of one head: fills s[0..nk) with the scaled scores, returns
 * m = max_j s_j and writes l = sum_j exp(s_j - m). */
static double score_row(const double *qi, const double *k, int64_t nk, int64_t d,
                        double scale, double *s, double *l_out) {
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        const double *kj = k + j * d;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += qi[c] * kj[c];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) l += exp(s[j] - m);
    *l_out = l;
    return m;
}

/* Forward over bh heads. q [bh,nq,d], k [bh,nk,d], v [bh,nk,dv],
 * o [bh,nq,dv], lse [bh,nq]. Rows are independent, so the (head, row) pairs
 * are spread over threads. Returns 0, or -1 on bad sizes / no memory. */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t dv, double scale,
                    int nthreads) {
    if (bh <= 0 || nq <= 0 || nk <= 0 || d <= 0 || dv <= 0) return -1;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)nk * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < bh * nq; ++r) {
            if (!s) continue;
            int64_t b = r / nq, i = r % nq;
            const double *qi = q + (b * nq + i) * d;
            const double *kb = k + b * nk * d;
            const double *vb = v + b * nk * dv;
            double l;
            double m = score_row(qi, kb, nk, d, scale, s, &l);
            double *oi = o + (b * nq + i) * dv;
            for (int64_t c = 0; c < dv; ++c) oi[c] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                double p = exp(s[j] - m) / l;
                const double *vj = vb + j * dv;
                for (int64_t c = 0; c < dv; ++c) oi[c] += p * vj[c];
            }
            lse[b * nq + i] = m + log(l);
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/* Backward over bh heads. dout [bh,nq,dv]; dq [bh,nq,d], dk [bh,nk,d],
 * dv_out [bh,nk,dv]. dK and dV sum over every query row of a head, so each
 * thread owns whole heads. */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv_out,
                    int64_t bh, int64_t nq, int64_t nk, int64_t d, int64_t dv, double scale,
                    int nthreads) {
    if (bh <= 0 || nq <= 0 || nk <= 0 || d <= 0 || dv <= 0) return -1;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)nk * sizeof(double));
        double *p = (double *)malloc((size_t)nk * sizeof(double));
        double *dp = (double *)malloc((size_t)nk * sizeof(double));
        if (!s || !p || !dp) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < bh; ++b) {
            if (!s || !p || !dp) continue;
            const double *qb = q + b * nq * d, *kb = k + b * nk * d;
            const double *vb = v + b * nk * dv, *dob = dout + b * nq * dv;
            double *dqb = dq + b * nq * d, *dkb = dk + b * nk * d, *dvb = dv_out + b * nk * dv;
            memset(dkb, 0, (size_t)(nk * d) * sizeof(double));
            memset(dvb, 0, (size_t)(nk * dv) * sizeof(double));
            for (int64_t i = 0; i < nq; ++i) {
                const double *qi = qb + i * d, *doi = dob + i * dv;
                double l;
                double m = score_row(qi, kb, nk, d, scale, s, &l);
                double delta = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    p[j] = exp(s[j] - m) / l;
                    const double *vj = vb + j * dv;
                    double acc = 0.0;
                    for (int64_t c = 0; c < dv; ++c) acc += doi[c] * vj[c];
                    dp[j] = acc;
                    delta += p[j] * dp[j];
                }
                double *dqi = dqb + i * d;
                for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    double ds = p[j] * (dp[j] - delta);
                    const double *kj = kb + j * d;
                    double *dkj = dkb + j * d, *dvj = dvb + j * dv;
                    for (int64_t c = 0; c < d; ++c) {
                        dqi[c] += scale * ds * kj[c];
                        dkj[c] += scale * ds * qi[c];
                    }
                    for (int64_t c = 0; c < dv; ++c) dvj[c] += p[j] * doi[c];
                }
            }
        }
        free(s);
        free(p);
        free(dp);
    }
    return failed ? -1 : 0;
}

/* psa_pack_qkv: qkv NCHW [B, nh*4*kd, H*W] -> packed [4, B*nh, H*W, kd].
 * For section s (0 Q, 1 K, 2 V_lo, 3 V_hi), head h of batch b, pixel n and
 * channel d within the section:
 *   packed[s][b*nh+h][n][d] = qkv[b][h*4*kd + s*kd + d][n]
 * Elements are copied as raw bytes of size esize. */
int oracle_psa_pack(const void *qkv, void *packed, int esize,
                    int64_t batch, int64_t nh, int64_t kd, int64_t hw) {
    if (batch <= 0 || nh <= 0 || kd <= 0 || hw <= 0 || esize <= 0) return -1;
    const char *src = (const char *)qkv;
    char *dst = (char *)packed;
    int64_t bh = batch * nh, qkv_ch = nh * 4 * kd;
    for (int64_t s = 0; s < 4; ++s)
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t h = 0; h < nh; ++h)
                for (int64_t n = 0; n < hw; ++n)
                    for (int64_t d = 0; d < kd; ++d) {
                        int64_t so = (b * qkv_ch + h * 4 * kd + s * kd + d) * hw + n;
                        int64_t dof = ((s * bh + b * nh + h) * hw + n) * kd + d;
                        memcpy(dst + dof * esize, src + so * esize, (size_t)esize);
                    }
    return 0;
}

/* psa_merge_attn_nchw: lo, hi [B*nh, H*W, kd] -> out NCHW [B, nh*2*kd, H*W]:
 *   out[b][h*2*kd + d][n]      = lo[b*nh+h][n][d]
 *   out[b][h*2*kd + kd + d][n] = hi[b*nh+h][n][d] */
int oracle_psa_merge(const void *lo, const void *hi, void *out, int esize,
                     int64_t batch, int64_t nh, int64_t kd, int64_t hw) {
    if (batch <= 0 || nh <= 0 || kd <= 0 || hw <= 0 || esize <= 0) return -1;
    const char *a = (const char *)lo, *bsrc = (const char *)hi;
    char *dst = (char *)out;
    int64_t c = nh * 2 * kd;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < nh; ++h)
            for (int64_t n = 0; n < hw; ++n)
                for (int64_t d = 0; d < kd; ++d) {
                    int64_t so = ((b * nh + h) * hw + n) * kd + d;
                    int64_t d_lo = (b * c + h * 2 * kd + d) * hw + n;
                    int64_t d_hi = (b * c + h * 2 * kd + kd + d) * hw + n;
                    memcpy(dst + d_lo * esize, a + so * esize, (size_t)esize);
                    memcpy(dst + d_hi * esize, bsrc + so * esize, (size_t)esize);
                }
    return 0;
}

/* psa_merge_attn_backward: d_out NCHW [B, nh*2*kd, H*W] -> d_lo, d_hi
 * [B*nh, H*W, kd], the inverse of psa_merge_attn_nchw:
 *   d_lo[b*nh+h][n][d] = d_out[b][h*2*kd + d][n]
 *   d_hi[b*nh+h][n][d] = d_out[b][h*2*kd + kd + d][n] */
int oracle_psa_merge_backward(const void *d_out, void *d_lo, void *d_hi, int esize,
                              int64_t batch, int64_t nh, int64_t kd, int64_t hw) {
    if (batch <= 0 || nh <= 0 || kd <= 0 || hw <= 0 || esize <= 0) return -1;
    const char *src = (const char *)d_out;
    char *lo = (char *)d_lo, *hi = (char *)d_hi;
    int64_t c = nh * 2 * kd;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < nh; ++h)
            for (int64_t n = 0; n < hw; ++n)
                for (int64_t d = 0; d < kd; ++d) {
                    int64_t dof = ((b * nh + h) * hw + n) * kd + d;
                    int64_t s_lo = (b * c + h * 2 * kd + d) * hw + n;
                    int64_t s_hi = (b * c + h * 2 * kd + kd + d) * hw + n;
                    memcpy(lo + dof * esize, src + s_lo * esize, (size_t)esize);
                    memcpy(hi + dof * esize, src + s_hi * esize, (size_t)esize);
                }
    return 0;
}

/* psa_pack_qkv_backward: d_packed [4, B*nh, H*W, kd] -> d_qkv NCHW
 * [B, nh*4*kd, H*W], the inverse of psa_pack_qkv:
 *   d_qkv[b][h*4*kd + s*kd + d][n] = d_packed[s][b*nh+h][n][d] */
int oracle_psa_pack_backward(const void *d_packed, void *d_qkv, int esize,
                             int64_t batch, int64_t nh, int64_t kd, int64_t hw) {
    if (batch <= 0 || nh <= 0 || kd <= 0 || hw <= 0 || esize <= 0) return -1;
    const char *src = (const char *)d_packed;
    char *dst = (char *)d_qkv;
    int64_t bh = batch * nh, qkv_ch = nh * 4 * kd;
    for (int64_t s = 0; s < 4; ++s)
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t h = 0; h < nh; ++h)
                for (int64_t n = 0; n < hw; ++n)
                    for (int64_t d = 0; d < kd; ++d) {
                        int64_t so = ((s * bh + b * nh + h) * hw + n) * kd + d;
                        int64_t dof = (b * qkv_ch + h * 4 * kd + s * kd + d) * hw + n;
                        memcpy(dst + dof * esize, src + so * esize, (size_t)esize);
                    }
    return 0;
}

/* psa_extract_v_nchw: qkv NCHW [B, nh*4*kd, H*W] -> v NCHW [B, nh*2*kd, H*W]:
 *   v[b][h*2*kd + d][n] = qkv[b][h*4*kd + 2*kd + d][n],  d < 2*kd */
int oracle_psa_extract_v(const void *qkv, void *v, int esize,
                         int64_t batch, int64_t nh, int64_t kd, int64_t hw) {
    if (batch <= 0 || nh <= 0 || kd <= 0 || hw <= 0 || esize <= 0) return -1;
    const char *src = (const char *)qkv;
    char *dst = (char *)v;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < nh; ++h)
            for (int64_t d = 0; d < 2 * kd; ++d)
                for (int64_t n = 0; n < hw; ++n) {
                    int64_t so = (b * nh * 4 * kd + h * 4 * kd + 2 * kd + d) * hw + n;
                    int64_t dof = (b * nh * 2 * kd + h * 2 * kd + d) * hw + n;
                    memcpy(dst + dof * esize, src + so * esize, (size_t)esize);
                }
    return 0;
}
