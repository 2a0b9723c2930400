/*
 * attn_oracle.c -- plain fp64 CPU oracle for causal RoPE attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library in attention_attn_fwd_04_amd/csrc.
 *
 * What it computes (each step cites the page that defines it):
 *
 *  1. bf16 inputs are widened to fp64 exactly (a bf16 value is the top half
 *     of an IEEE binary32 word).
 *  2. RoPE, NeoX convention ("AttnFuse: A Composable DSL for Compiling
 *     Attentions to Fused GPU Kernels", section 2 "Rotary Position
 *     Embeddings" and section 4.1 "Fused RoPE"): dimension pair r is
 *     (r, r + D/2); at position p it is rotated by the angle
 *     p * theta^(-2r/D):
 *        x'[r]       = x[r] cos - x[r+D/2] sin
 *        x'[r+D/2]   = x[r+D/2] cos + x[r] sin
 *     theta == 0 means "no rotation".
 *  3. Scores ("Attention block decomposition", "Three shapes, two
 *     reductions"): s(n,m) = scale * sum over pairs of the pair terms
 *     q'[r]k'[r] + q'[r+D/2]k'[r+D/2], contracted over D.
 *  4. Optional per-pair distance window ("ATFlash -- Per-RoPE-Wavelength
 *     Attention Windows", "The idea"): pair r contributes to s(n,m) only when
 *     n - m <= w[r].  The table is w[r] = floor(k * lambda_r) with the pair's
 *     wavelength lambda_r = 2*pi*theta^(2r/D).
 *  5. Causal mask: keys m > n are excluded ("Flash Attention: Causal Prefill
 *     D=128", "Reverse traversal isolates the causal mask").
 *  6. Row softmax over the materialised score row, then O = P V, contracted
 *     over the key axis ("Attention block decomposition").  No intermediate
 *     rounding: everything stays fp64.  The online-softmax recurrence the
 *     kernels use is exact ("AttnFuse", section 2 "FlashAttention and online
 *     softmax"), so the plain definition is the reference.
 *  7. Grouped-query attention: query head hq reads KV head hq / (Hq/Hkv).
 *
 * Layout of every tensor: [B, S, H, D] contiguous ("BSHD"), bf16 bits as
 * uint16_t.  Positions are 0..S-1 plus an optional common offset, which the
 * invariance tests use (scores depend only on n - m).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Step 2 for one row: x (D values, fp64) at position pos -> out. */
static void rotate_row(const double *x, int D, double theta, double pos,
                       double *out)
{
    int half = D / 2;
    if (theta == 0.0) {
        memcpy(out, x, sizeof(double) * (size_t)D);
        return;
    }
    for (int r = 0; r < half; ++r) {
        double freq = pow(theta, -2.0 * (double)r / (double)D);
        double ang = pos * freq;
        double c = cos(ang), s = sin(ang);
        out[r] = x[r] * c - x[r + half] * s;
        out[r + half] = x[r + half] * c + x[r] * s;
    }
}

/* Exported: rotate one bf16 row (used by the convention tests). */
void oracle_rope_row(const uint16_t *x, int D, double theta, double pos,
                     double *out)
{
    double tmp[1024];
    for (int d = 0; d < D; ++d)
        tmp[d] = widen_bf16(x[d]);
    rotate_row(tmp, D, theta, pos, out);
}

/* Step 3 + 4 for one (query, key) pair of rotated rows. */
static double score(const double *qr, const double *kr, int D, double scale,
                    const int32_t *window, long long dist)
{
    int half = D / 2;
    double acc = 0.0;
    for (int r = 0; r < half; ++r) {
        if (window != NULL && dist > (long long)window[r])
            continue;
        acc += qr[r] * kr[r] + qr[r + half] * kr[r + half];
    }
    return scale * acc;
}

static const uint16_t *row_ptr(const uint16_t *t, int S, int H, int D, int b,
                               int s, int h)
{
    return t + (((size_t)b * S + s) * H + h) * (size_t)D;
}

/* Rotated K for every position of one (b, hk) head: S x D fp64. */
static double *rotated_keys(const uint16_t *k, int S, int Hkv, int D, int b,
                            int hk, double theta, long long pos_offset)
{
    double *kr = (double *)malloc(sizeof(double) * (size_t)S * D);
    if (!kr)
        return NULL;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < S; ++m) {
        double raw[1024];
        const uint16_t *src = row_ptr(k, S, Hkv, D, b, m, hk);
        for (int d = 0; d < D; ++d)
            raw[d] = widen_bf16(src[d]);
        rotate_row(raw, D, theta, (double)(m + pos_offset), kr + (size_t)m * D);
    }
    return kr;
}

/*
 * Attention output for a list of query rows.
 *   rows: n_rows triples (b, n, hq)
 *   out:  n_rows x D fp64
 *   lse:  optional n_rows natural-log log-sum-exp of the row's scores
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int B, int S, int Hq, int Hkv, int D, double rope_theta,
                     int causal, double scale, const int32_t *window,
                     long long pos_offset, const int32_t *rows,
                     long long n_rows, double *out, double *lse)
{
    if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 ||
        (D % 2) != 0 || (Hq % Hkv) != 0)
        return -1;
    int group = Hq / Hkv;
    for (long long i = 0; i < n_rows; ++i) {
        int b = rows[3 * i], n = rows[3 * i + 1], hq = rows[3 * i + 2];
        if (b < 0 || b >= B || n < 0 || n >= S || hq < 0 || hq >= Hq)
            return -1;
    }
    int status = 0;
    for (int b = 0; b < B && status == 0; ++b) {
        for (int hk = 0; hk < Hkv && status == 0; ++hk) {
            /* Does any requested row read this KV head? */
            long long any = 0;
            for (long long i = 0; i < n_rows; ++i)
                if (rows[3 * i] == b && rows[3 * i + 2] / group == hk)
                    ++any;
            if (!any)
                continue;
            double *kr = rotated_keys(k, S, Hkv, D, b, hk, rope_theta, pos_offset);
            if (!kr) {
                status = -1;
                break;
            }
#pragma omp parallel for schedule(dynamic, 1)
            for (long long i = 0; i < n_rows; ++i) {
                if (rows[3 * i] != b || rows[3 * i + 2] / group != hk)
                    continue;
                int n = rows[3 * i + 1], hq = rows[3 * i + 2];
                double qraw[1024], qr[1024];
                const uint16_t *qs = row_ptr(q, S, Hq, D, b, n, hq);
                for (int d = 0; d < D; ++d)
                    qraw[d] = widen_bf16(qs[d]);
                rotate_row(qraw, D, rope_theta, (double)(n + pos_offset), qr);

                int m_end = causal ? n + 1 : S; /* keys 0..m_end-1 */
                double *srow = (double *)malloc(sizeof(double) * (size_t)(m_end > 0 ? m_end : 1));
                double mu = -INFINITY;
                for (int m = 0; m < m_end; ++m) {
                    srow[m] = score(qr, kr + (size_t)m * D, D, scale, window,
                                    (long long)n - (long long)m);
                    if (srow[m] > mu)
                        mu = srow[m];
                }
                double z = 0.0;
                for (int m = 0; m < m_end; ++m) {
                    srow[m] = exp(srow[m] - mu);
                    z += srow[m];
                }
                double *o = out + (size_t)i * D;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int m = 0; m < m_end; ++m) {
                    double p = srow[m] / z;
                    const uint16_t *vs = row_ptr(v, S, Hkv, D, b, m, hk);
                    for (int d = 0; d < D; ++d)
                        o[d] += p * widen_bf16(vs[d]);
                }
                if (lse)
                    lse[i] = mu + log(z);
                free(srow);
            }
            free(kr);
        }
    }
    return status;
}

/*
 * Decode ("AttnFuse", section 4.2 "Flash Decoding"): one new query per
 * sequence, at position L-1 (+ pos_offset), against a cache of L keys and
 * values.  The cache holds keys as they were stored (rotated when they were
 * appended); only the query is rotated here.  Every key 0..L-1 is visible;
 * with a window, pair r counts for key m only when (L-1) - m <= w[r].
 *   q: [B, Hq, D]; k, v: [B, L, Hkv, D]; out: [B, Hq, D] fp64;
 *   lse: optional [B, Hq] natural-log log-sum-exp of the scaled scores.
 */
int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  int B, int L, int Hq, int Hkv, int D, double rope_theta,
                  double scale, const int32_t *window, long long pos_offset,
                  double *out, double *lse)
{
    if (B < 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 ||
        (D % 2) != 0 || (Hq % Hkv) != 0)
        return -1;
    int group = Hq / Hkv;
    long long n = (long long)L - 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < (long long)B * Hq; ++bh) {
        int b = (int)(bh / Hq), hq = (int)(bh % Hq), hk = hq / group;
        double qraw[1024], qr[1024], kr[1024];
        const uint16_t *qs = q + ((size_t)b * Hq + hq) * (size_t)D;
        for (int d = 0; d < D; ++d)
            qraw[d] = widen_bf16(qs[d]);
        rotate_row(qraw, D, rope_theta, (double)(n + pos_offset), qr);
        double *srow = (double *)malloc(sizeof(double) * (size_t)L);
        double mu = -INFINITY;
        for (int m = 0; m < L; ++m) {
            const uint16_t *ks = row_ptr(k, L, Hkv, D, b, m, hk);
            for (int d = 0; d < D; ++d)
                kr[d] = widen_bf16(ks[d]);
            srow[m] = score(qr, kr, D, scale, window, n - (long long)m);
            if (srow[m] > mu)
                mu = srow[m];
        }
        double z = 0.0;
        for (int m = 0; m < L; ++m) {
            srow[m] = exp(srow[m] - mu);
            z += srow[m];
        }
        double *o = out + (size_t)bh * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int m = 0; m < L; ++m) {
            double p = srow[m] / z;
            const uint16_t *vs = row_ptr(v, L, Hkv, D, b, m, hk);
            for (int d = 0; d < D; ++d)
                o[d] += p * widen_bf16(vs[d]);
        }
        if (lse)
            lse[bh] = mu + log(z);
        free(srow);
    }
    return 0;
}

/* Inverse rotation (by -angle) of one fp64 row, in place. */
static void unrotate_row(double *x, int D, double theta, double pos)
{
    int half = D / 2;
    if (theta == 0.0)
        return;
    for (int r = 0; r < half; ++r) {
        double freq = pow(theta, -2.0 * (double)r / (double)D);
        double ang = pos * freq;
        double c = cos(ang), s = sin(ang);
        double a = x[r], b = x[r + half];
        x[r] = a * c + b * s;
        x[r + half] = b * c - a * s;
    }
}

/*
 * Backward of the attention above ("AttnFuse", section 4.4 "Backward Pass":
 * the gradients with respect to Q, K and V), from the plain definition:
 *   P = softmax(S), S = scale Q'K'^T (masked), O = P V, upstream dO:
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(P o dP)),
 *   dQ' = scale dS K',  dK' = scale dS^T Q',
 * then dQ = R(n)^T dQ' and dK = R(m)^T dK' (the rotation is orthogonal).
 * With grouped heads, dK and dV of a KV head sum over its query heads.
 * q, do: [B,S,Hq,D]; k, v: [B,S,Hkv,D] bf16 bits; dq [B,S,Hq,D],
 * dk, dv [B,S,Hkv,D] fp64 outputs.  No window.
 */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const uint16_t *dout, int B, int S, int Hq, int Hkv, int D,
                    double rope_theta, int causal, double scale, double *dq,
                    double *dk, double *dv)
{
    if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 ||
        (D % 2) != 0 || (Hq % Hkv) != 0)
        return -1;
    int group = Hq / Hkv;
    size_t nq = (size_t)B * S * Hq * D, nkv = (size_t)B * S * Hkv * D;
    memset(dq, 0, sizeof(double) * nq);
    memset(dk, 0, sizeof(double) * nkv);
    memset(dv, 0, sizeof(double) * nkv);
    for (int b = 0; b < B; ++b) {
        for (int hk = 0; hk < Hkv; ++hk) {
            double *kr = rotated_keys(k, S, Hkv, D, b, hk, rope_theta, 0);
            double *dkr = (double *)calloc((size_t)S * D, sizeof(double));
            if (!kr || !dkr) {
                free(kr);
                free(dkr);
                return -1;
            }
            for (int g = 0; g < group; ++g) {
                int hq = hk * group + g;
#pragma omp parallel
                {
                    double *dkr_t = (double *)calloc((size_t)S * D, sizeof(double));
                    double *dv_t = (double *)calloc((size_t)S * D, sizeof(double));
                    double *p = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
                    double *dp = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 4)
                    for (int n = 0; n < S; ++n) {
                        double qraw[1024], qr[1024], dor[1024], dqr[1024];
                        const uint16_t *qs = row_ptr(q, S, Hq, D, b, n, hq);
                        const uint16_t *ds = row_ptr(dout, S, Hq, D, b, n, hq);
                        for (int d = 0; d < D; ++d) {
                            qraw[d] = widen_bf16(qs[d]);
                            dor[d] = widen_bf16(ds[d]);
                            dqr[d] = 0.0;
                        }
                        rotate_row(qraw, D, rope_theta, (double)n, qr);
                        int m_end = causal ? n + 1 : S;
                        double mu = -INFINITY;
                        for (int m = 0; m < m_end; ++m) {
                            p[m] = score(qr, kr + (size_t)m * D, D, scale, NULL, 0);
                            if (p[m] > mu)
                                mu = p[m];
                        }
                        double z = 0.0;
                        for (int m = 0; m < m_end; ++m) {
                            p[m] = exp(p[m] - mu);
                            z += p[m];
                        }
                        double delta = 0.0;
                        for (int m = 0; m < m_end; ++m) {
                            p[m] /= z;
                            const uint16_t *vs = row_ptr(v, S, Hkv, D, b, m, hk);
                            double acc = 0.0;
                            for (int d = 0; d < D; ++d)
                                acc += dor[d] * widen_bf16(vs[d]);
                            dp[m] = acc;
                            delta += p[m] * acc;
                        }
                        for (int m = 0; m < m_end; ++m) {
                            double dsm = p[m] * (dp[m] - delta);
                            const double *km = kr + (size_t)m * D;
                            double *dkm = dkr_t + (size_t)m * D, *dvm = dv_t + (size_t)m * D;
                            for (int d = 0; d < D; ++d) {
                                dqr[d] += scale * dsm * km[d];
                                dkm[d] += scale * dsm * qr[d];
                                dvm[d] += p[m] * dor[d];
                            }
                        }
                        unrotate_row(dqr, D, rope_theta, (double)n);
                        double *dqo = dq + (((size_t)b * S + n) * Hq + hq) * (size_t)D;
                        for (int d = 0; d < D; ++d)
                            dqo[d] = dqr[d];
                    }
#pragma omp critical
                    {
                        for (size_t i = 0; i < (size_t)S * D; ++i)
                            dkr[i] += dkr_t[i];
                        for (int m = 0; m < S; ++m) {
                            double *dvo = dv + (((size_t)b * S + m) * Hkv + hk) * (size_t)D;
                            for (int d = 0; d < D; ++d)
                                dvo[d] += dv_t[(size_t)m * D + d];
                        }
                    }
                    free(dkr_t);
                    free(dv_t);
                    free(p);
                    free(dp);
                }
            }
            for (int m = 0; m < S; ++m) {
                unrotate_row(dkr + (size_t)m * D, D, rope_theta, (double)m);
                double *dko = dk + (((size_t)b * S + m) * Hkv + hk) * (size_t)D;
                for (int d = 0; d < D; ++d)
                    dko[d] = dkr[(size_t)m * D + d];
            }
            free(kr);
            free(dkr);
        }
    }
    return 0;
}

/*
 * The per-row terms of the backward above for one query row (b, n, hq),
 * given the rotated keys kr of its KV head: the rotated query qr, the
 * upstream row dor, the probabilities p[m] and dS[m] = p[m] (dP[m] - Delta)
 * over the visible keys m < m_end, which is returned.
 */
static int bwd_row_terms(const uint16_t *q, const uint16_t *v,
                         const uint16_t *dout, int S, int Hq, int Hkv, int D,
                         double theta, int causal, double scale, int b, int n,
                         int hq, int hk, const double *kr, double *qr,
                         double *dor, double *p, double *ds)
{
    double qraw[1024];
    const uint16_t *qs = row_ptr(q, S, Hq, D, b, n, hq);
    const uint16_t *dsrc = row_ptr(dout, S, Hq, D, b, n, hq);
    for (int d = 0; d < D; ++d) {
        qraw[d] = widen_bf16(qs[d]);
        dor[d] = widen_bf16(dsrc[d]);
    }
    rotate_row(qraw, D, theta, (double)n, qr);
    int m_end = causal ? n + 1 : S;
    double mu = -INFINITY;
    for (int m = 0; m < m_end; ++m) {
        p[m] = score(qr, kr + (size_t)m * D, D, scale, NULL, 0);
        if (p[m] > mu)
            mu = p[m];
    }
    double z = 0.0;
    for (int m = 0; m < m_end; ++m) {
        p[m] = exp(p[m] - mu);
        z += p[m];
    }
    double delta = 0.0;
    for (int m = 0; m < m_end; ++m) {
        p[m] /= z;
        const uint16_t *vs = row_ptr(v, S, Hkv, D, b, m, hk);
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += dor[d] * widen_bf16(vs[d]);
        ds[m] = acc;
        delta += p[m] * acc;
    }
    for (int m = 0; m < m_end; ++m)
        ds[m] = p[m] * (ds[m] - delta);
    return m_end;
}

/*
 * Entries of the backward above at full size, one at a time: dq of the
 * query rows qrows (n_q triples b, n, hq) and dk, dv of the key rows kcols
 * (n_k triples b, m, hk).  A query row costs one score row; a key row costs
 * one score row per query that sees it (S - m of them per query head under
 * the causal mask).  dq_out: n_q x D, dk_out, dv_out: n_k x D (fp64).
 */
int oracle_attn_bwd_sampled(const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const uint16_t *dout, int B,
                            int S, int Hq, int Hkv, int D, double rope_theta,
                            int causal, double scale, const int32_t *qrows,
                            int n_q, double *dq_out, const int32_t *kcols,
                            int n_k, double *dk_out, double *dv_out)
{
    if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 ||
        (D % 2) != 0 || (Hq % Hkv) != 0 || n_q < 0 || n_k < 0)
        return -1;
    int group = Hq / Hkv;
    for (int i = 0; i < n_q + n_k; ++i) {
        const int32_t *t = i < n_q ? qrows + 3 * i : kcols + 3 * (i - n_q);
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= S || t[2] < 0 ||
            t[2] >= (i < n_q ? Hq : Hkv))
            return -1;
    }
    for (int i = 0; i < n_q; ++i) {
        int b = qrows[3 * i], n = qrows[3 * i + 1], hq = qrows[3 * i + 2];
        int hk = hq / group;
        double *kr = rotated_keys(k, S, Hkv, D, b, hk, rope_theta, 0);
        double *p = (double *)malloc(sizeof(double) * (size_t)S);
        double *ds = (double *)malloc(sizeof(double) * (size_t)S);
        if (!kr || !p || !ds) {
            free(kr);
            free(p);
            free(ds);
            return -1;
        }
        double qr[1024], dor[1024], dqr[1024];
        int m_end = bwd_row_terms(q, v, dout, S, Hq, Hkv, D, rope_theta, causal,
                                  scale, b, n, hq, hk, kr, qr, dor, p, ds);
        for (int d = 0; d < D; ++d)
            dqr[d] = 0.0;
        for (int m = 0; m < m_end; ++m)
            for (int d = 0; d < D; ++d)
                dqr[d] += scale * ds[m] * kr[(size_t)m * D + d];
        unrotate_row(dqr, D, rope_theta, (double)n);
        memcpy(dq_out + (size_t)i * D, dqr, sizeof(double) * (size_t)D);
        free(kr);
        free(p);
        free(ds);
    }
    for (int j = 0; j < n_k; ++j) {
        int b = kcols[3 * j], m = kcols[3 * j + 1], hk = kcols[3 * j + 2];
        double *kr = rotated_keys(k, S, Hkv, D, b, hk, rope_theta, 0);
        if (!kr)
            return -1;
        double dkr[1024], dvr[1024];
        for (int d = 0; d < D; ++d)
            dkr[d] = dvr[d] = 0.0;
        int fail = 0;
        for (int g = 0; g < group; ++g) {
            int hq = hk * group + g;
#pragma omp parallel
            {
                double dk_t[1024], dv_t[1024], qr[1024], dor[1024];
                double *p = (double *)malloc(sizeof(double) * (size_t)S);
                double *ds = (double *)malloc(sizeof(double) * (size_t)S);
                for (int d = 0; d < D; ++d)
                    dk_t[d] = dv_t[d] = 0.0;
                if (p && ds) {
#pragma omp for schedule(dynamic, 1)
                    for (int n = causal ? m : 0; n < S; ++n) {
                        bwd_row_terms(q, v, dout, S, Hq, Hkv, D, rope_theta,
                                      causal, scale, b, n, hq, hk, kr, qr, dor,
                                      p, ds);
                        for (int d = 0; d < D; ++d) {
                            dv_t[d] += p[m] * dor[d];
                            dk_t[d] += scale * ds[m] * qr[d];
                        }
                    }
                }
#pragma omp critical
                {
                    if (!p || !ds)
                        fail = 1;
                    for (int d = 0; d < D; ++d) {
                        dkr[d] += dk_t[d];
                        dvr[d] += dv_t[d];
                    }
                }
                free(p);
                free(ds);
            }
        }
        free(kr);
        if (fail)
            return -1;
        unrotate_row(dkr, D, rope_theta, (double)m);
        memcpy(dk_out + (size_t)j * D, dkr, sizeof(double) * (size_t)D);
        memcpy(dv_out + (size_t)j * D, dvr, sizeof(double) * (size_t)D);
    }
    return 0;
}

/*
 * The scaled score row s(n, m) for m = 0..S-1 of one query (b, n, hq), with
 * masked keys (m > n under the causal mask) set to -inf.  Used by the
 * invariance and window tests.
 */
int oracle_scores_row(const uint16_t *q, const uint16_t *k, int B, int S,
                      int Hq, int Hkv, int D, double rope_theta, int causal,
                      double scale, const int32_t *window, long long pos_offset,
                      int b, int n, int hq, double *scores)
{
    if (b < 0 || b >= B || n < 0 || n >= S || hq < 0 || hq >= Hq ||
        D <= 0 || D > 1024 || (Hq % Hkv) != 0)
        return -1;
    int hk = hq / (Hq / Hkv);
    double raw[1024], qr[1024], kr[1024];
    const uint16_t *qs = row_ptr(q, S, Hq, D, b, n, hq);
    for (int d = 0; d < D; ++d)
        raw[d] = widen_bf16(qs[d]);
    rotate_row(raw, D, rope_theta, (double)(n + pos_offset), qr);
    for (int m = 0; m < S; ++m) {
        if (causal && m > n) {
            scores[m] = -INFINITY;
            continue;
        }
        const uint16_t *ks = row_ptr(k, S, Hkv, D, b, m, hk);
        for (int d = 0; d < D; ++d)
            raw[d] = widen_bf16(ks[d]);
        rotate_row(raw, D, rope_theta, (double)(m + pos_offset), kr);
        scores[m] = score(qr, kr, D, scale, window, (long long)n - (long long)m);
    }
    return 0;
}

/*
 * Window table ("ATFlash", "The idea"): w[r] = floor(k_turns * lambda_r),
 * lambda_r = 2*pi*theta^(2r/D), for r = 0..D/2-1, evaluated in fp64.
 */
int oracle_window_table(double rope_theta, int D, double k_turns, int32_t *w)
{
    if (D <= 0 || (D % 2) != 0 || !(rope_theta > 1.0) || !(k_turns > 0.0))
        return -1;
    const double two_pi = 6.283185307179586476925286766559;
    for (int r = 0; r < D / 2; ++r) {
        double lam = two_pi * pow(rope_theta, 2.0 * (double)r / (double)D);
        double wr = floor(k_turns * lam);
        w[r] = wr > 2147483647.0 ? 2147483647 : (int32_t)wr;
    }
    return 0;
}

/*
 * Pair terms removed by the window over one head's causal triangle
 * (0 <= m <= n < S): for each pair r, the cells with distance
 * delta = n - m > w[r].  Distance delta occurs S - delta times, so pair r
 * removes sum_{delta = max(w[r]+1, 0)}^{S-1} (S - delta) cells, which is the
 * triangular number T(S - lo) with lo = max(w[r]+1, 0).
 */
long long oracle_pruned_terms(const int32_t *w, int D, int S)
{
    long long total = 0;
    for (int r = 0; r < D / 2; ++r) {
        long long lo = (long long)w[r] + 1;
        if (lo < 0)
            lo = 0;
        if (lo > S - 1)
            continue;
        long long cnt = (long long)S - lo; /* number of distances lo..S-1 */
        total += cnt * (cnt + 1) / 2;
    }
    return total;
}
