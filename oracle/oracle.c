/*
 * oracle.c -- plain fp64 CPU reference for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no online state):
 *
 *   For each (batch b, head h, query i), with a scale s,
 *     S_ij   = s * (q_i . k_j)                        for every valid key j
 *     m_i    = max_j S_ij                             (pass 1)
 *     l_i    = sum_j exp(S_ij - m_i)                  (pass 2)
 *     O_i    = sum_j exp(S_ij - m_i) * v_j / l_i      (pass 3)
 *     LSE_i  = m_i + ln(l_i)
 *
 *   - "Flash Attention 4" (mlc.ai, section "algorithm structure"): the
 *     definitions of s_ij, the per-row maximum, p_ij, l_i, o_i and O_i = o_i/l_i;
 *     FlashAttention returns the same result as standard attention.
 *   - "Flash Attention记录" (zhen8838), section "SoftMax": the safe softmax
 *     that subtracts the row maximum before exponentiating, in three passes.
 *   - "FlashAttention：一次前向计算" (qingsen), section "what attention
 *     computes": S = QK^T, P = rowwise softmax(sS), O = PV with an explicit
 *     scale s; section "general update": L_i = s*m_i + log(l_i) where m_i is
 *     the maximum of the unscaled scores (same value as m_i + ln l_i here,
 *     because this file keeps the scores already scaled).
 *
 * Valid keys (causal masking): "Flash Attention 4", section "Causal Mask":
 * with Nq queries and Nk keys the mask is aligned to the bottom-right corner,
 * so query i may use keys j <= i + Nk - Nq (clamped to Nk - 1).  A row with
 * no valid key has O = 0 ("algorithm structure": O is 0 when the row sum is
 * 0) and LSE = -inf ("rescale and write-back": rows without a valid key).
 *
 * Grouped K/V heads: "Flash Attention 4", section "GQA support": with H
 * query heads and Hkv K/V heads (Hkv divides H), G = H / Hkv consecutive
 * query heads share one K/V head, query head h = kv * G + offset, so query
 * head h reads K/V head h / G.  Hkv = H is plain multi-head attention.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   fixed length : q [B, Nq, H, d]; k, v [B, Nk, Hkv, d]; o [B, Nq, H, d];
 *                  lse [B, H, Nq]
 *   packed varlen: q, o [T, H, d]; k, v [T, Hkv, d] with sequence b occupying
 *                  tokens offsets[b] .. offsets[b+1]-1 (self attention,
 *                  Nq = Nk = L_b); lse [H, T]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads an OpenMP region of this library uses (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of keys query i may use. */
static int64_t valid_keys(int64_t i, int64_t Nq, int64_t Nk, int causal)
{
    if (!causal) return Nk;
    int64_t last = i + Nk - Nq;          /* largest usable key index */
    if (last < 0) return 0;
    if (last >= Nk) return Nk;
    return last + 1;
}

/*
 * One query row.  qi points at d values; key j starts at k + j*stride,
 * value j at v + j*stride.  s_buf must hold nvalid doubles.
 */
static void attention_row(const double *qi, const double *k, const double *v,
                          int64_t stride, int64_t nvalid, int64_t d,
                          double scale, double *s_buf, double *out, double *lse)
{
    if (nvalid <= 0) {
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    /* pass 1: scaled scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < nvalid; ++j) {
        const double *kj = k + j * stride;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
        s_buf[j] = scale * dot;
        if (s_buf[j] > m) m = s_buf[j];
    }
    /* pass 2: denominator relative to the maximum */
    double l = 0.0;
    for (int64_t j = 0; j < nvalid; ++j) l += exp(s_buf[j] - m);
    /* pass 3: normalised weighted sum of the value rows */
    for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t j = 0; j < nvalid; ++j) {
        double p = exp(s_buf[j] - m) / l;
        const double *vj = v + j * stride;
        for (int64_t c = 0; c < d; ++c) out[c] += p * vj[c];
    }
    *lse = m + log(l);
}

/* Fixed-length batch, every row.  Returns 0, or -1 on bad arguments. */
int oracle_attn_fwd(const double *q, const double *k, const double *v,
                    double *o, double *lse,
                    int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                    double scale, int causal)
{
    if (!q || !k || !v || !o || !lse || B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0 ||
        Hkv <= 0 || H % Hkv != 0)
        return -1;
    const int64_t group = H / Hkv;      /* query heads per K/V head */
    const int64_t stride = Hkv * d;     /* between consecutive keys */
    const int64_t nrows = B * H * Nq;
    int bad = 0;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = r % Nq;
                int64_t h = (r / Nq) % H;
                int64_t b = r / (Nq * H);
                const double *qi = q + ((b * Nq + i) * H + h) * d;
                const double *kb = k + (b * Nk * Hkv + h / group) * d;
                const double *vb = v + (b * Nk * Hkv + h / group) * d;
                attention_row(qi, kb, vb, stride, valid_keys(i, Nq, Nk, causal), d, scale,
                              s_buf, o + ((b * Nq + i) * H + h) * d,
                              lse + (b * H + h) * Nq + i);
            }
            free(s_buf);
        }
    }
    return bad ? -1 : 0;
}

/* Packed variable-length batch of nseq sequences, every row. */
int oracle_attn_fwd_varlen(const double *q, const double *k, const double *v,
                           double *o, double *lse,
                           int64_t nseq, const int64_t *offsets, int64_t H, int64_t Hkv,
                           int64_t d, double scale, int causal)
{
    if (!q || !k || !v || !o || !lse || !offsets || nseq < 0 || H < 0 || d <= 0 ||
        Hkv <= 0 || H % Hkv != 0)
        return -1;
    const int64_t T = offsets[nseq];
    int64_t maxlen = 0;
    for (int64_t b = 0; b < nseq; ++b) {
        int64_t L = offsets[b + 1] - offsets[b];
        if (L < 0) return -1;
        if (L > maxlen) maxlen = L;
    }
    const int64_t group = H / Hkv;
    const int64_t stride = Hkv * d;
    int bad = 0;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        if (!s_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < T * H; ++r) {
                int64_t h = r % H;
                int64_t t = r / H;
                int64_t b = 0;
                while (offsets[b + 1] <= t) ++b;
                int64_t start = offsets[b];
                int64_t L = offsets[b + 1] - start;
                int64_t i = t - start;
                attention_row(q + (t * H + h) * d, k + (start * Hkv + h / group) * d,
                              v + (start * Hkv + h / group) * d, stride,
                              valid_keys(i, L, L, causal), d, scale, s_buf,
                              o + (t * H + h) * d, lse + h * T + t);
            }
            free(s_buf);
        }
    }
    return bad ? -1 : 0;
}

/*
 * A chosen subset of rows.  rows holds nrows triples (b, h, i).  Without
 * offsets the layout is the fixed-length one with sizes Nq, Nk; with offsets
 * (nseq+1 entries) the layout is the packed one and b names a sequence, i a
 * position inside it.  Results go to o_out [nrows, d] and lse_out [nrows].
 */
int oracle_attn_fwd_rows(const double *q, const double *k, const double *v,
                         int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                         double scale, int causal,
                         const int64_t *offsets, int64_t nseq,
                         int64_t nrows, const int64_t *rows,
                         double *o_out, double *lse_out)
{
    if (!q || !k || !v || !rows || !o_out || !lse_out || H <= 0 || d <= 0 || nrows < 0 ||
        Hkv <= 0 || H % Hkv != 0)
        return -1;
    int64_t maxkeys = Nk;
    if (offsets) {
        maxkeys = 0;
        for (int64_t b = 0; b < nseq; ++b) {
            int64_t L = offsets[b + 1] - offsets[b];
            if (L > maxkeys) maxkeys = L;
        }
    }
    const int64_t group = H / Hkv;
    const int64_t stride = Hkv * d;
    int bad = 0;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(maxkeys > 0 ? maxkeys : 1));
        if (!s_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
                const double *qi, *kb, *vb;
                int64_t nvalid;
                if (offsets) {
                    if (b < 0 || b >= nseq) {
#pragma omp atomic write
                        bad = 1;
                        continue;
                    }
                    int64_t start = offsets[b], L = offsets[b + 1] - offsets[b];
                    if (h < 0 || h >= H || i < 0 || i >= L) {
#pragma omp atomic write
                        bad = 1;
                        continue;
                    }
                    qi = q + ((start + i) * H + h) * d;
                    kb = k + (start * Hkv + h / group) * d;
                    vb = v + (start * Hkv + h / group) * d;
                    nvalid = valid_keys(i, L, L, causal);
                } else {
                    if (h < 0 || h >= H || i < 0 || i >= Nq || b < 0) {
#pragma omp atomic write
                        bad = 1;
                        continue;
                    }
                    qi = q + ((b * Nq + i) * H + h) * d;
                    kb = k + (b * Nk * Hkv + h / group) * d;
                    vb = v + (b * Nk * Hkv + h / group) * d;
                    nvalid = valid_keys(i, Nq, Nk, causal);
                }
                attention_row(qi, kb, vb, stride, nvalid, d, scale, s_buf,
                              o_out + r * d, lse_out + r);
            }
            free(s_buf);
        }
    }
    return bad ? -1 : 0;
}

/*
 * Backward pass (gradients of O with respect to Q, K, V).
 *
 * "FlashAttention-4（下）" (argus-lessons), section 1: the backward recomputes
 * S and P and takes the gradients of the two products, dP and dV for O = PV,
 * dQ = dS K and dK = dS^T Q for S = Q K^T (scaled), with dS the gradient of
 * the row softmax.  Written out for one (batch, head), valid keys j of row i:
 *
 *   s_ij  = scale * (q_i . k_j),  LSE_i = ln sum_j exp(s_ij),  P_ij = exp(s_ij - LSE_i)
 *   dV_j  = sum_i P_ij dO_i                      (gradient of O = P V in V)
 *   dP_ij = dO_i . v_j                           (... in P)
 *   D_i   = sum_j P_ij dP_ij                     (= dO_i . O_i)
 *   dS_ij = P_ij (dP_ij - D_i)                   (row-softmax Jacobian applied to dP)
 *   dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
 *
 * With grouped K/V heads the G query heads of a K/V head add into its dK, dV.
 * Rows without a valid key contribute nothing.  Everything is recomputed here
 * in fp64 from q, k, v, dO (the forward's O and LSE are not inputs).
 * Layouts as for the forward; dq like q, dk and dv like k.
 */
static void bwd_head(const double *q, const double *k, const double *v, const double *dout,
                     double *dq, double *dk, double *dv,
                     int64_t qstride, int64_t kstride, int64_t Nq, int64_t Nk, int64_t d,
                     double scale, int causal, double *p_buf, double *dp_buf)
{
    /* q, dout, dq: query rows at qstride; k, v, dk, dv: key rows at kstride */
    for (int64_t i = 0; i < Nq; ++i) {
        const int64_t nvalid = valid_keys(i, Nq, Nk, causal);
        if (nvalid <= 0) continue;
        const double *qi = q + i * qstride;
        const double *doi = dout + i * qstride;
        double m = -INFINITY;
        for (int64_t j = 0; j < nvalid; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += qi[c] * k[j * kstride + c];
            p_buf[j] = scale * dot;
            if (p_buf[j] > m) m = p_buf[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nvalid; ++j) l += exp(p_buf[j] - m);
        const double lse = m + log(l);
        double D = 0.0;
        for (int64_t j = 0; j < nvalid; ++j) {
            p_buf[j] = exp(p_buf[j] - lse);
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c) dot += doi[c] * v[j * kstride + c];
            dp_buf[j] = dot;
            D += p_buf[j] * dot;
        }
        double *dqi = dq + i * qstride;
        for (int64_t j = 0; j < nvalid; ++j) {
            const double ds = p_buf[j] * (dp_buf[j] - D);
            for (int64_t c = 0; c < d; ++c) {
                dqi[c] += scale * ds * k[j * kstride + c];
                dk[j * kstride + c] += scale * ds * qi[c];
                dv[j * kstride + c] += p_buf[j] * doi[c];
            }
        }
    }
}

/* Fixed length, every gradient.  dq, dk, dv are overwritten. */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv,
                    int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                    double scale, int causal)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || H < 0 || Nq < 0 || Nk < 0 ||
        d <= 0 || Hkv <= 0 || H % Hkv != 0)
        return -1;
    const int64_t group = H / Hkv;
    memset(dq, 0, sizeof(double) * (size_t)(B * Nq * H * d));
    memset(dk, 0, sizeof(double) * (size_t)(B * Nk * Hkv * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * Nk * Hkv * d));
    int bad = 0;
    /* one (batch, K/V head) per iteration: its query heads are the only writers of its dK, dV */
#pragma omp parallel
    {
        double *p_buf = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *dp_buf = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!p_buf || !dp_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < B * Hkv; ++u) {
                const int64_t b = u / Hkv, kvh = u % Hkv;
                for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h)
                    bwd_head(q + (b * Nq * H + h) * d, k + (b * Nk * Hkv + kvh) * d,
                             v + (b * Nk * Hkv + kvh) * d, dout + (b * Nq * H + h) * d,
                             dq + (b * Nq * H + h) * d, dk + (b * Nk * Hkv + kvh) * d,
                             dv + (b * Nk * Hkv + kvh) * d, H * d, Hkv * d, Nq, Nk, d,
                             scale, causal, p_buf, dp_buf);
            }
        }
        free(p_buf);
        free(dp_buf);
    }
    return bad ? -1 : 0;
}

/* Packed variable length (self attention per sequence), every gradient. */
int oracle_attn_bwd_varlen(const double *q, const double *k, const double *v, const double *dout,
                           double *dq, double *dk, double *dv,
                           int64_t nseq, const int64_t *offsets, int64_t H, int64_t Hkv,
                           int64_t d, double scale, int causal)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !offsets || nseq < 0 || H < 0 ||
        d <= 0 || Hkv <= 0 || H % Hkv != 0)
        return -1;
    const int64_t T = offsets[nseq];
    int64_t maxlen = 0;
    for (int64_t b = 0; b < nseq; ++b) {
        int64_t L = offsets[b + 1] - offsets[b];
        if (L < 0) return -1;
        if (L > maxlen) maxlen = L;
    }
    const int64_t group = H / Hkv;
    memset(dq, 0, sizeof(double) * (size_t)(T * H * d));
    memset(dk, 0, sizeof(double) * (size_t)(T * Hkv * d));
    memset(dv, 0, sizeof(double) * (size_t)(T * Hkv * d));
    int bad = 0;
#pragma omp parallel
    {
        double *p_buf = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        double *dp_buf = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        if (!p_buf || !dp_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < nseq * Hkv; ++u) {
                const int64_t b = u / Hkv, kvh = u % Hkv;
                const int64_t start = offsets[b], L = offsets[b + 1] - start;
                for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h)
                    bwd_head(q + (start * H + h) * d, k + (start * Hkv + kvh) * d,
                             v + (start * Hkv + kvh) * d, dout + (start * H + h) * d,
                             dq + (start * H + h) * d, dk + (start * Hkv + kvh) * d,
                             dv + (start * Hkv + kvh) * d, H * d, Hkv * d, L, L, d,
                             scale, causal, p_buf, dp_buf);
            }
        }
        free(p_buf);
        free(dp_buf);
    }
    return bad ? -1 : 0;
}

/*
 * Selected rows of the gradients, for checks at sizes where the full
 * gradients are too slow here.  One (batch or sequence, K/V head) with its G
 * query heads: q, dout [Nq, G, d]; k, v [Nk, d] (contiguous slices).  Same
 * definitions as above ("FlashAttention-4（下）", section 1), taken in order:
 *
 *   1. for every query row (g, i): LSE_gi = ln sum_j exp(s_gij) and
 *      D_gi = sum_j P_gij dP_gij over its valid keys;
 *   2. dQ for the requested rows (g, i): scale * sum_j P_gij (dP_gij - D_gi) k_j;
 *   3. dK, dV for the requested key rows j, summed over the G query heads and
 *      the queries that see key j: dV_j = sum P_gij dO_gi,
 *      dK_j = scale * sum P_gij (dP_gij - D_gi) q_gi.
 *
 * qrows holds nq pairs (g, i); krows holds nk key indices; dq_out [nq, d],
 * dk_out, dv_out [nk, d].  Returns -1 on a bad argument or allocation failure.
 */
int oracle_attn_bwd_rows(const double *q, const double *k, const double *v, const double *dout,
                         int64_t G, int64_t Nq, int64_t Nk, int64_t d, double scale, int causal,
                         int64_t nq, const int64_t *qrows, double *dq_out,
                         int64_t nk, const int64_t *krows, double *dk_out, double *dv_out)
{
    if (!q || !k || !v || !dout || G <= 0 || Nq < 0 || Nk < 0 || d <= 0 || nq < 0 || nk < 0 ||
        (nq > 0 && (!qrows || !dq_out)) || (nk > 0 && (!krows || !dk_out || !dv_out)))
        return -1;
    for (int64_t r = 0; r < nq; ++r)
        if (qrows[2 * r] < 0 || qrows[2 * r] >= G || qrows[2 * r + 1] < 0 || qrows[2 * r + 1] >= Nq)
            return -1;
    for (int64_t r = 0; r < nk; ++r)
        if (krows[r] < 0 || krows[r] >= Nk) return -1;
    const int64_t rs = G * d;                       /* token stride of q and dout */
    double *lse = (double *)malloc(sizeof(double) * (size_t)(G * Nq > 0 ? G * Nq : 1));
    double *dsum = (double *)malloc(sizeof(double) * (size_t)(G * Nq > 0 ? G * Nq : 1));
    if (!lse || !dsum) {
        free(lse);
        free(dsum);
        return -1;
    }
    int bad = 0;
    /* 1. per query row: LSE and D */
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s_buf) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t u = 0; u < G * Nq; ++u) {
                const int64_t g = u / Nq, i = u % Nq;
                const double *qi = q + i * rs + g * d, *doi = dout + i * rs + g * d;
                const int64_t nvalid = valid_keys(i, Nq, Nk, causal);
                double mrow = -INFINITY;
                for (int64_t j = 0; j < nvalid; ++j) {
                    double qk = 0.0;
                    for (int64_t c = 0; c < d; ++c) qk += qi[c] * k[j * d + c];
                    s_buf[j] = scale * qk;
                    if (s_buf[j] > mrow) mrow = s_buf[j];
                }
                double lrow = 0.0;
                for (int64_t j = 0; j < nvalid; ++j) lrow += exp(s_buf[j] - mrow);
                const double L = nvalid > 0 ? mrow + log(lrow) : -INFINITY;
                double D = 0.0;
                for (int64_t j = 0; j < nvalid; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c) dot += doi[c] * v[j * d + c];
                    D += exp(s_buf[j] - L) * dot;
                }
                lse[u] = L;
                dsum[u] = D;
            }
        }
        free(s_buf);
    }
    if (bad) {
        free(lse);
        free(dsum);
        return -1;
    }
    /* 2. dQ rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nq; ++r) {
        const int64_t g = qrows[2 * r], i = qrows[2 * r + 1];
        const double *qi = q + i * rs + g * d, *doi = dout + i * rs + g * d;
        double *out = dq_out + r * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        const int64_t nvalid = valid_keys(i, Nq, Nk, causal);
        for (int64_t j = 0; j < nvalid; ++j) {
            double sd = 0.0, pd = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                sd += qi[c] * k[j * d + c];
                pd += doi[c] * v[j * d + c];
            }
            const double p = exp(scale * sd - lse[g * Nq + i]);
            const double ds = p * (pd - dsum[g * Nq + i]);
            for (int64_t c = 0; c < d; ++c) out[c] += scale * ds * k[j * d + c];
        }
    }
    /* 3. dK, dV rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nk; ++r) {
        const int64_t j = krows[r];
        double *ok = dk_out + r * d, *ov = dv_out + r * d;
        for (int64_t c = 0; c < d; ++c) ok[c] = ov[c] = 0.0;
        for (int64_t g = 0; g < G; ++g)
            for (int64_t i = 0; i < Nq; ++i) {
                if (j >= valid_keys(i, Nq, Nk, causal)) continue;
                const double *qi = q + i * rs + g * d, *doi = dout + i * rs + g * d;
                double sd = 0.0, pd = 0.0;
                for (int64_t c = 0; c < d; ++c) {
                    sd += qi[c] * k[j * d + c];
                    pd += doi[c] * v[j * d + c];
                }
                const double p = exp(scale * sd - lse[g * Nq + i]);
                const double ds = p * (pd - dsum[g * Nq + i]);
                for (int64_t c = 0; c < d; ++c) {
                    ov[c] += p * doi[c];
                    ok[c] += scale * ds * qi[c];
                }
            }
    }
    free(lse);
    free(dsum);
    return 0;
}
