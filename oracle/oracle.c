/*
 * Float64 CPU oracle for the scaled-dot-product attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP path.
 *
 * What it computes is the plain definition, not the tiled online-softmax
 * algorithm the GPU kernel uses:
 *
 *   s_j    = scale * sum_{d ascending} q[i,d] * k[j,d]   (float64)
 *   m      = max over visible j of s_j
 *   p_j    = exp(s_j - m),  l = sum_{j ascending} p_j
 *   O[i,:] = (sum_{j ascending} p_j * v[j,:]) / l
 *   LSE[i] = m + log(l)                                    (natural log)
 *
 * Sources: "An Optimal Mapper Meets a Real GPU", section "Ground rules" (FP16
 * in, FP32 accumulate, gated against PyTorch SDPA) and "Experiment one" (query
 * length equals key length; the causal column of the case table); the STAGE_D.md
 * notes on the head-dim-512 kernel (LSE as an output; S = S_0 + S_1 summed in
 * logit space before the softmax).  Readings where the pages are silent:
 * causal means key j is visible to query i iff j <= i; the scale multiplies the
 * dot product; LSE is the natural log over the scaled logits; inputs are the
 * exact fp16 values widened to double and the scale is the float32 value the
 * GPU receives, widened exactly.
 *
 * Decode (query length Sq different from key length Sk, a few queries against
 * a long key/value cache; the decode kernel of "Validating Memory-Optimal
 * Transformer Kernels on Real Hardware", section 5): the same definition with
 * q, o of shape [B, H, Sq, D] and k, v of shape [B, H, Sk, D].  The pages fix
 * no alignment for the causal mask when Sq != Sk; the reading taken here is
 * bottom-right alignment, the one a cache of past keys implies: query i is the
 * (Sk - Sq + i)-th position, so key j is visible iff j <= i + (Sk - Sq).  With
 * Sq = Sk this is the j <= i rule above.
 *
 * Engineering: build with -O2 -ffp-contract=off and no fast-math, so every sum
 * is evaluated in the written order.  Rows are independent; OpenMP splits over
 * rows only, so results do not depend on the thread count.  Per-row scratch is
 * heap-allocated (a fixed-size stack array would cap S).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE-754 binary16 bit pattern -> double, exactly (every fp16 value is a
 * double).  sign | 5-bit exponent (bias 15) | 10-bit fraction. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

static double *widen(const uint16_t *x, size_t n)
{
    double *y = (double *)malloc(n * sizeof(double));
    if (!y)
        return NULL;
    for (size_t t = 0; t < n; ++t)
        y[t] = oracle_half_to_double(x[t]);
    return y;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Planted mistakes, used only by the oracle's own power tests to show that
 * its pins catch an error of each kind.  0 = the oracle as specified.
 *   1: causal mask off by one (key j visible iff j < i + 2)
 *   2: scale dropped from the logits
 *   3: LSE without the max term (log l only)
 *   4: O not divided by l
 *   5: key and query roles swapped in the dot product (q[j] . k[i])
 *   6: last head-dim element dropped from the dot product
 *   7: causal mask aligned top-left (key j visible iff j <= i) when Sq != Sk
 */
static int visible(int causal, int mistake, int i, int j, int off)
{
    if (!causal)
        return 1;
    if (mistake == 1)
        return j < i + off + 2;
    if (mistake == 7)
        return j <= i;
    return j <= i + off;
}

/* Sq query rows against Sk keys; off = Sk - Sq is the causal alignment. */
static int run(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16,
               double *o, double *lse, int B, int H, int Sq, int Sk, int D, int causal,
               float scale, int nthreads, int mistake)
{
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1)
        return -1;
    if (causal && Sq > Sk)
        return -3; /* the first Sq - Sk rows would see no key */
    const int off = Sk - Sq;
    size_t nq = (size_t)B * H * Sq * D, nk = (size_t)B * H * Sk * D;
    double *q = widen(q16, nq), *k = widen(k16, nk), *v = widen(v16, nk);
    if (!q || !k || !v) {
        free(q);
        free(k);
        free(v);
        return -2;
    }
    const double sc = (mistake == 2) ? 1.0 : (double)scale;
    const int dlen = (mistake == 6 && D > 1) ? D - 1 : D;
    const long rows = (long)B * H * Sq;
    int err = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Sk * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < rows; ++r) {
                const long bh = r / Sq;
                const int i = (int)(r % Sq);
                const double *Q = q + (size_t)bh * Sq * D;
                const double *K = k + (size_t)bh * Sk * D;
                const double *V = v + (size_t)bh * Sk * D;
                /* logits over visible keys; -inf marks a masked key */
                double m = -INFINITY;
                for (int j = 0; j < Sk; ++j) {
                    if (!visible(causal, mistake, i, j, off)) {
                        s[j] = -INFINITY;
                        continue;
                    }
                    const double *qa = (mistake == 5) ? Q + (size_t)j * D : Q + (size_t)i * D;
                    const double *kb = (mistake == 5) ? K + (size_t)i * D : K + (size_t)j * D;
                    double dot = 0.0;
                    for (int d = 0; d < dlen; ++d)
                        dot += qa[d] * kb[d];
                    s[j] = sc * dot;
                    if (s[j] > m)
                        m = s[j];
                }
                /* weights and their sum, keys ascending */
                double l = 0.0;
                for (int j = 0; j < Sk; ++j) {
                    s[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
                    l += s[j];
                }
                for (int d = 0; d < D; ++d)
                    acc[d] = 0.0;
                for (int j = 0; j < Sk; ++j) {
                    if (!visible(causal, mistake, i, j, off))
                        continue; /* weight exactly 0 */
                    const double *vj = V + (size_t)j * D;
                    for (int d = 0; d < D; ++d)
                        acc[d] += s[j] * vj[d];
                }
                double *orow = o + (size_t)r * D;
                for (int d = 0; d < D; ++d)
                    orow[d] = (mistake == 4) ? acc[d] : acc[d] / l;
                lse[r] = (mistake == 3) ? log(l) : m + log(l);
            }
        }
        free(s);
        free(acc);
    }
    free(q);
    free(k);
    free(v);
    return err;
}

/*
 * O = softmax(scale * Q K^T + causal mask) V and LSE, in float64.
 * q, k, v: fp16 bit patterns, contiguous [B, H, S, D].
 * o: float64 [B, H, S, D]; lse: float64 [B, H, S].  The caller owns all.
 * nthreads <= 0 keeps the OpenMP default.  Returns 0, -1 (bad shape) or
 * -2 (out of memory).
 */
int oracle_attn_fwd_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        double *o, double *lse, int B, int H, int S, int D,
                        int causal, float scale, int nthreads)
{
    return run(q, k, v, o, lse, B, H, S, S, D, causal, scale, nthreads, 0);
}

/* The same computation with one planted mistake (see the list above). */
int oracle_attn_fwd_f64_planted(const uint16_t *q, const uint16_t *k,
                                const uint16_t *v, double *o, double *lse,
                                int B, int H, int S, int D, int causal,
                                float scale, int nthreads, int mistake)
{
    return run(q, k, v, o, lse, B, H, S, S, D, causal, scale, nthreads, mistake);
}

/*
 * Decode form: q, o [B, H, Sq, D]; k, v [B, H, Sk, D]; lse [B, H, Sq].
 * Causal: key j visible to query i iff j <= i + (Sk - Sq) (bottom-right);
 * returns -3 when causal and Sq > Sk.  `mistake` as above (0 = as specified).
 */
int oracle_attn_fwd_kv_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           double *o, double *lse, int B, int H, int Sq, int Sk, int D,
                           int causal, float scale, int nthreads, int mistake)
{
    return run(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, nthreads, mistake);
}

/*
 * Scaled partial logits over the head-dim range [d0, d1):
 *   out[b,h,i,j] = scale * sum_{d0 <= d < d1} q[i,d] k[j,d]   (-inf if masked)
 * out is float64 [B, H, S, S].  With [0, D) this is the full logit matrix; two
 * ranges [0, D/2) and [D/2, D) are the S_0 / S_1 sub-tiles of the notes on the
 * head-dim-512 kernel, which add to S in logit space.
 */
int oracle_logits_f64(const uint16_t *q16, const uint16_t *k16, double *out,
                      int B, int H, int S, int D, int d0, int d1, int causal,
                      float scale, int nthreads)
{
    if (B < 1 || H < 1 || S < 1 || D < 1 || d0 < 0 || d1 > D || d0 > d1)
        return -1;
    size_t n = (size_t)B * H * S * D;
    double *q = widen(q16, n), *k = widen(k16, n);
    if (!q || !k) {
        free(q);
        free(k);
        return -2;
    }
    const long rows = (long)B * H * S;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const long bh = r / S;
        const int i = (int)(r % S);
        const double *qi = q + ((size_t)bh * S + i) * D;
        for (int j = 0; j < S; ++j) {
            double *dst = out + (size_t)r * S + j;
            if (causal && j > i) {
                *dst = -INFINITY;
                continue;
            }
            const double *kj = k + ((size_t)bh * S + j) * D;
            double dot = 0.0;
            for (int d = d0; d < d1; ++d)
                dot += qi[d] * kj[d];
            *dst = (double)scale * dot;
        }
    }
    free(q);
    free(k);
    return 0;
}

/*
 * Softmax over given logits and the weighted sum of V:
 *   O[i,:] = sum_j exp(s_ij - m_i) v[j,:] / l_i,  LSE[i] = m_i + log(l_i)
 * logits: float64 [B, H, S, S] with -inf for masked keys (every row needs at
 * least one finite logit); v: fp16 bits [B, H, S, D].
 */
int oracle_softmax_av_f64(const double *logits, const uint16_t *v16, double *o,
                          double *lse, int B, int H, int S, int D, int nthreads)
{
    if (B < 1 || H < 1 || S < 1 || D < 1)
        return -1;
    size_t n = (size_t)B * H * S * D;
    double *v = widen(v16, n);
    if (!v)
        return -2;
    const long rows = (long)B * H * S;
    int err = 0;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < rows; ++r) {
                const long bh = r / S;
                const double *s = logits + (size_t)r * S;
                const double *V = v + (size_t)bh * S * D;
                double m = -INFINITY;
                for (int j = 0; j < S; ++j)
                    if (s[j] > m)
                        m = s[j];
                double l = 0.0;
                for (int d = 0; d < D; ++d)
                    acc[d] = 0.0;
                for (int j = 0; j < S; ++j) {
                    if (s[j] == -INFINITY)
                        continue;
                    double p = exp(s[j] - m);
                    l += p;
                    for (int d = 0; d < D; ++d)
                        acc[d] += p * V[(size_t)j * D + d];
                }
                for (int d = 0; d < D; ++d)
                    o[(size_t)r * D + d] = acc[d] / l;
                lse[r] = m + log(l);
            }
        }
        free(acc);
    }
    free(v);
    return err;
}

/*
 * Backward pass of the forward above, in float64, for L = sum(dO * O):
 *   P[i,j]  = softmax_j(scale q_i.k_j + mask)        (the forward's weights)
 *   dV[j]   = sum_i P[i,j] dO[i]
 *   dP[i,j] = dO[i] . v[j]
 *   Dlt[i]  = dO[i] . O[i]          (= sum_j P[i,j] dP[i,j])
 *   dS[i,j] = P[i,j] (dP[i,j] - Dlt[i])
 *   dQ[i]   = scale sum_j dS[i,j] k[j],   dK[j] = scale sum_i dS[i,j] q[i]
 * The step after the forward ("Validating Memory-Optimal Transformer Kernels
 * on Real Hardware", abstract and section 4: the backward kernel and the
 * fused forward+backward that avoid the O(n^2) intermediate); the chain rule
 * of the softmax is the plain one.  q, k, v, dO: fp16 bits [B, H, S, D];
 * dq, dk, dv: float64 [B, H, S, D], overwritten.  Sums run in index order;
 * heads are independent and OpenMP splits over heads only.
 * `mistake` (0 = as specified) plants one error for the pins' power tests:
 *   1: Dlt dropped (dS = P dP)   2: scale dropped from dQ and dK
 *   3: dV from unnormalised weights   4: causal mask off by one
 */
int oracle_attn_bwd_f64(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16,
                        const uint16_t *do16, double *dq, double *dk, double *dv,
                        int B, int H, int S, int D, int causal, float scale, int nthreads,
                        int mistake)
{
    if (B < 1 || H < 1 || S < 1 || D < 1)
        return -1;
    size_t n = (size_t)B * H * S * D;
    double *q = widen(q16, n), *k = widen(k16, n), *v = widen(v16, n), *g = widen(do16, n);
    if (!q || !k || !v || !g) {
        free(q);
        free(k);
        free(v);
        free(g);
        return -2;
    }
    const double sc = (double)scale;
    const long heads = (long)B * H;
    int err = 0;
    memset(dk, 0, n * sizeof(double));
    memset(dv, 0, n * sizeof(double));
    set_threads(nthreads);
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)S * sizeof(double));
        double *dp = (double *)malloc((size_t)S * sizeof(double));
        double *o = (double *)malloc((size_t)D * sizeof(double));
        if (!p || !dp || !o) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (long bh = 0; bh < heads; ++bh) {
                const double *Q = q + (size_t)bh * S * D, *K = k + (size_t)bh * S * D;
                const double *V = v + (size_t)bh * S * D, *G = g + (size_t)bh * S * D;
                double *dQ = dq + (size_t)bh * S * D, *dK = dk + (size_t)bh * S * D;
                double *dV = dv + (size_t)bh * S * D;
                for (int i = 0; i < S; ++i) {
                    const int last = !causal ? S - 1 : (mistake == 4 ? (i + 1 < S ? i + 1 : S - 1) : i);
                    double m = -INFINITY;
                    for (int j = 0; j <= last; ++j) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += Q[(size_t)i * D + d] * K[(size_t)j * D + d];
                        p[j] = sc * dot;
                        if (p[j] > m)
                            m = p[j];
                    }
                    double l = 0.0;
                    for (int j = 0; j <= last; ++j) {
                        p[j] = exp(p[j] - m);
                        l += p[j];
                    }
                    /* O[i] and Dlt[i] */
                    for (int d = 0; d < D; ++d)
                        o[d] = 0.0;
                    for (int j = 0; j <= last; ++j)
                        for (int d = 0; d < D; ++d)
                            o[d] += p[j] * V[(size_t)j * D + d];
                    double dlt = 0.0;
                    for (int d = 0; d < D; ++d)
                        dlt += G[(size_t)i * D + d] * (o[d] / l);
                    for (int j = 0; j <= last; ++j) {
                        double t = 0.0;
                        for (int d = 0; d < D; ++d)
                            t += G[(size_t)i * D + d] * V[(size_t)j * D + d];
                        dp[j] = t;
                    }
                    for (int d = 0; d < D; ++d)
                        dQ[(size_t)i * D + d] = 0.0;
                    const double gs = (mistake == 2) ? 1.0 : sc;
                    for (int j = 0; j <= last; ++j) {
                        const double pn = p[j] / l;
                        const double ds = (mistake == 1) ? pn * dp[j] : pn * (dp[j] - dlt);
                        const double pv = (mistake == 3) ? p[j] : pn;
                        for (int d = 0; d < D; ++d) {
                            dQ[(size_t)i * D + d] += gs * ds * K[(size_t)j * D + d];
                            dK[(size_t)j * D + d] += gs * ds * Q[(size_t)i * D + d];
                            dV[(size_t)j * D + d] += pv * G[(size_t)i * D + d];
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
        free(o);
    }
    free(q);
    free(k);
    free(v);
    free(g);
    return err;
}
