/*
 * ja_oracle.c -- plain, slow, obviously-correct CPU oracle for the join-agg
 * hot path.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the product library never does.
 * It shares no code, header or constant with the HIP path.
 *
 * Everything here computes in IEEE double precision.  Rounding to bfloat16
 * (or IEEE half) happens only where a relation is materialised, via
 * orc_f64_to_bf16() (orc_f64_to_f16()).
 *
 * Sources (the pages: "Every Kernel Is a Join: Automatic Multi-GPU Parallelism
 * for AI Computations in Einsummable", paperpeel full text):
 *   - section 1 (Introduction): every operation is a join followed by an
 *     aggregation; a matrix multiply is a join on the shared inner index
 *     followed by SUM.  orc_einsum2 is that result written out as the plain
 *     loop nest (the contraction's definition).
 *   - section 3.2, Example 3.4: matrix multiply [i,j] x [j,k] -> [i,k].
 *   - attention, RMSNorm and SwiGLU: the pages name these operators without
 *     formulas; the textbook definitions are used (scaled dot-product
 *     attention of Vaswani et al., cited in section 1; root-mean-square
 *     normalisation; SiLU-gated linear unit).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> double                                                       */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits
 * (bias 127), 7 stored mantissa bits.  Decoding is exact. */
static double bf16_decode(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int m = h & 0x7F;
    double v;
    if (e == 0xFF) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -126 - 7); /* subnormal: m * 2^-133 */
    } else {
        v = ldexp((double)(128 + m), e - 127 - 7);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even mantissa. The value is
 * rounded once, directly from double. */
static uint16_t bf16_encode(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int E;
    double f = frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
    /* normal bf16 numbers have a = (1.m) * 2^(E-1) with E-1 >= -126 */
    if (E - 1 >= -126) {
        double r = nearbyint(ldexp(f, 8)); /* 8 significant bits, RNE */
        if (r == 256.0) { r = 128.0; E += 1; }
        int be = (E - 1) + 127;
        if (be >= 255) return sign | 0x7F80; /* overflow to infinity */
        return sign | (uint16_t)(be << 7) | (uint16_t)((int)r - 128);
    }
    /* subnormal range: multiples of 2^-133 */
    double q = nearbyint(ldexp(a, 133));
    if (q >= 128.0) return sign | (uint16_t)(1 << 7); /* rounds up to min normal */
    return sign | (uint16_t)q;
}

/* IEEE binary16 (half): 1 sign bit, 5 exponent bits (bias 15), 10 stored
 * mantissa bits.  Decoding is exact. */
static double f16_decode(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -14 - 10); /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(1024 + m), e - 15 - 10);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even mantissa, once,
 * directly from double; magnitudes that round past 65504 become infinity. */
static uint16_t f16_encode(double x) {
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int E;
    double f = frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
    if (E - 1 >= -14) {        /* normal: a = (1.m) * 2^(E-1) */
        double r = nearbyint(ldexp(f, 11)); /* 11 significant bits, RNE */
        if (r == 2048.0) { r = 1024.0; E += 1; }
        int he = (E - 1) + 15;
        if (he >= 31) return sign | 0x7C00;
        return sign | (uint16_t)(he << 10) | (uint16_t)((int)r - 1024);
    }
    double q = nearbyint(ldexp(a, 24)); /* subnormal range: multiples of 2^-24 */
    if (q >= 1024.0) return sign | (uint16_t)(1 << 10);
    return sign | (uint16_t)q;
}

void orc_f16_to_f64(const uint16_t* in, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f16_decode(in[i]);
}

void orc_f64_to_f16(const double* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = f16_encode(in[i]);
}

void orc_bf16_to_f64(const uint16_t* in, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_decode(in[i]);
}

void orc_f64_to_bf16(const double* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_encode(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Two-operand einsum as a loop nest                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    int na, nb, nc;
    char a[27], b[27], c[27];
    int nsum;          /* letters summed over: in an input, not in the output */
    char sum[27];
    int64_t ext[26];
    int64_t sa[26], sb[26]; /* stride of each letter in A and B (0 if absent) */
} esum_t;

static int parse_einsum(const char* spec, const int64_t* ext26, esum_t* e) {
    memset(e, 0, sizeof(*e));
    const char* comma = strchr(spec, ',');
    const char* arrow = strstr(spec, "->");
    if (!comma || !arrow || comma > arrow) return -1;
    e->na = (int)(comma - spec);
    e->nb = (int)(arrow - comma - 1);
    e->nc = (int)strlen(arrow + 2);
    if (e->na > 26 || e->nb > 26 || e->nc > 26) return -1;
    memcpy(e->a, spec, e->na);
    memcpy(e->b, comma + 1, e->nb);
    memcpy(e->c, arrow + 2, e->nc);
    int seen_a[26] = {0}, seen_b[26] = {0}, seen_c[26] = {0};
    for (int i = 0; i < e->na; ++i) { int l = e->a[i] - 'a'; if (l < 0 || l > 25 || seen_a[l]++) return -1; }
    for (int i = 0; i < e->nb; ++i) { int l = e->b[i] - 'a'; if (l < 0 || l > 25 || seen_b[l]++) return -1; }
    for (int i = 0; i < e->nc; ++i) {
        int l = e->c[i] - 'a';
        if (l < 0 || l > 25 || seen_c[l]++) return -1;
        if (!seen_a[l] && !seen_b[l]) return -1;
    }
    for (int l = 0; l < 26; ++l) {
        e->ext[l] = ext26[l];
        if ((seen_a[l] || seen_b[l]) && !seen_c[l]) e->sum[e->nsum++] = (char)('a' + l);
    }
    int64_t s = 1;
    for (int i = e->na - 1; i >= 0; --i) { e->sa[e->a[i] - 'a'] = s; s *= e->ext[e->a[i] - 'a']; }
    s = 1;
    for (int i = e->nb - 1; i >= 0; --i) { e->sb[e->b[i] - 'a'] = s; s *= e->ext[e->b[i] - 'a']; }
    return 0;
}

/* One output element: sum over all summed-letter index combinations of A*B. */
static double esum_point(const esum_t* e, const double* A, const double* B, int64_t o) {
    int64_t idx[26] = {0};
    for (int i = e->nc - 1; i >= 0; --i) {
        int l = e->c[i] - 'a';
        idx[l] = o % e->ext[l];
        o /= e->ext[l];
    }
    int64_t nsum = 1;
    for (int i = 0; i < e->nsum; ++i) nsum *= e->ext[e->sum[i] - 'a'];
    double acc = 0.0;
    for (int64_t c = 0; c < nsum; ++c) {
        int64_t r = c;
        for (int i = e->nsum - 1; i >= 0; --i) {
            int l = e->sum[i] - 'a';
            idx[l] = r % e->ext[l];
            r /= e->ext[l];
        }
        int64_t oa = 0, ob = 0;
        for (int l = 0; l < 26; ++l) { oa += idx[l] * e->sa[l]; ob += idx[l] * e->sb[l]; }
        acc += A[oa] * B[ob];
    }
    return acc;
}

/* C = einsum(spec, A, B), all dense row-major over their letter strings.
 * ext26[l] is the extent of letter 'a'+l.  Returns 0, or -1 on a bad spec. */
int orc_einsum2(const char* spec, const int64_t* ext26, const double* A, const double* B, double* C) {
    esum_t e;
    if (parse_einsum(spec, ext26, &e)) return -1;
    int64_t nout = 1;
    for (int i = 0; i < e.nc; ++i) nout *= e.ext[e.c[i] - 'a'];
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t o = 0; o < nout; ++o) C[o] = esum_point(&e, A, B, o);
    return 0;
}

/* The same contraction evaluated only at the listed output linear indices. */
int orc_einsum2_points(const char* spec, const int64_t* ext26, const double* A, const double* B,
                       int64_t npts, const int64_t* pts, double* vals) {
    esum_t e;
    if (parse_einsum(spec, ext26, &e)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) vals[p] = esum_point(&e, A, B, pts[p]);
    return 0;
}

/* Plain row-major matrix product C[M,N] = A[M,K] B[K,N] (i-k-j loop order),
 * used where a chain of large products makes the generic loop nest too slow.
 * Same definition as orc_einsum2("ik,kj->ij"). */
void orc_matmul(const double* A, const double* B, double* C, int64_t M, int64_t K, int64_t N) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * K + k];
            const double* b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Scaled dot-product attention, textbook two-pass softmax per query row     */
/* ------------------------------------------------------------------------ */

/* Q [B,H,S,D], K and V [B,HK,T,D] with HK dividing H, dense row-major
 * doubles.  Query head h reads key-value head h / (H / HK): with HK < H this
 * is grouped-query attention, query heads g*(H/HK) .. (g+1)*(H/HK)-1 sharing
 * key-value head g (the pages' section 3.3, Shardable Indices); HK = H is
 * ordinary multi-head attention.  For each listed row (b,h,s):
 * score_t = scale * <Q[b,h,s,:], K[b,kv(h),t,:]>, keys t > s are excluded
 * when causal; p_t = exp(score_t - max_t score_t);
 * out = sum_t p_t V[b,kv(h),t,:] / sum_t p_t.  rows holds 3 int64 per row.
 * Packed sequences (the pages' section 3.3: independent sequences packed end
 * to end along the sequence index; attention never crosses a sequence
 * boundary): with nseq > 0, seq_ends holds the ascending end positions of the
 * sequences (the last equal to S = T), and key t is visible to query s only
 * if both lie in the same sequence [start, end). */
void orc_attention_rows(const double* Q, const double* K, const double* V, int64_t B, int64_t H, int64_t HK,
                        int64_t S, int64_t T, int64_t D, double scale, int causal, int64_t nseq,
                        const int64_t* seq_ends, int64_t nrows, const int64_t* rows, double* out) {
    (void)B;
    const int64_t rep = H / HK;
#pragma omp parallel
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t b = rows[3 * r], h = rows[3 * r + 1], s = rows[3 * r + 2];
            const double* q = Q + ((b * H + h) * S + s) * D;
            const double* kb = K + (b * HK + h / rep) * T * D;
            const double* vb = V + (b * HK + h / rep) * T * D;
            int64_t tmin = 0, tmax = causal ? (s + 1 < T ? s + 1 : T) : T;
            for (int64_t k = 0; k < nseq; ++k)
                if (s < seq_ends[k]) {  /* the query's sequence is [tmin, seq_ends[k]) */
                    if (seq_ends[k] < tmax) tmax = seq_ends[k];
                    break;
                } else {
                    tmin = seq_ends[k];
                }
            double m = -INFINITY;
            for (int64_t t = tmin; t < tmax; ++t) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += q[d] * kb[t * D + d];
                sc[t] = scale * acc;
                if (sc[t] > m) m = sc[t];
            }
            double l = 0.0;
            for (int64_t t = tmin; t < tmax; ++t) { sc[t] = exp(sc[t] - m); l += sc[t]; }
            double* o = out + r * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t t = tmin; t < tmax; ++t)
                for (int64_t d = 0; d < D; ++d) o[d] += sc[t] * vb[t * D + d];
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
        }
        free(sc);
    }
}

/* ------------------------------------------------------------------------ */
/* Row-wise and elementwise operators                                        */
/* ------------------------------------------------------------------------ */

/* y[r,d] = x[r,d] / sqrt(mean_d x[r,:]^2 + eps) * g[d]  (mean over all D). */
void orc_rmsnorm(const double* x, const double* g, int64_t R, int64_t D, double eps, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const double* xr = x + r * D;
        double ss = 0.0;
        for (int64_t d = 0; d < D; ++d) ss += xr[d] * xr[d];
        double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t d = 0; d < D; ++d) y[r * D + d] = xr[d] * inv * g[d];
    }
}

/* h = silu(g) * u with silu(g) = g / (1 + exp(-g)). */
void orc_swiglu(const double* g, const double* u, int64_t n, double* h) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

void orc_add(const double* a, const double* b, int64_t n, double* c) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) c[i] = a[i] + b[i];
}
