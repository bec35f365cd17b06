/*
 * fairy_oracle.c -- plain, slow, obviously correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (see fairy_oracle.h).  Written from the pages'
 * definitions; double precision throughout, exact integers where the method
 * decides integers.  No blocking, fusion or reordering beyond the
 * definitions: every output row is an ordered sum over its columns.
 */
#include "fairy_oracle.h"

#include <complex.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int32_t orc_version(void) { return 1; }

int32_t orc_set_threads(int32_t nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return (int32_t)omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Phase code  [Fairy2i article §3.1]                                        */
/* ------------------------------------------------------------------------ */
/* The page computes k = floor(2*theta/pi + 1/2) mod 4 with theta = arg(w) and
 * returns [1, i, -1, -i][k].  Exact comparison form of the same rule:
 *   |Re| > |Im|  -> real axis: k = 0 if Re > 0 else 2
 *   |Im| > |Re|  -> imag axis: k = 1 if Im > 0 else 3
 *   |Re| == |Im| -> theta is exactly +-45 or +-135 degrees; the floor sends the
 *                   boundary to the counter-clockwise neighbour:
 *                   +45 -> 1, +135 -> 2, -135 -> 3, -45 -> 0.
 * Reading: w == 0 (any signed zeros) -> code 0 (theta taken as 0). */
int32_t orc_phase_code(float re, float im)
{
    double a = re, b = im;
    double A = fabs(a), B = fabs(b);
    if (A == 0.0 && B == 0.0) return 0;
    if (A > B) return a > 0.0 ? 0 : 2;
    if (B > A) return b > 0.0 ? 1 : 3;
    if (a > 0.0 && b > 0.0) return 1;  /* theta = +45  */
    if (a < 0.0 && b > 0.0) return 2;  /* theta = +135 */
    if (a < 0.0 && b < 0.0) return 3;  /* theta = -135 */
    return 0;                          /* theta = -45  */
}

/* ------------------------------------------------------------------------ */
/* Widely-linear conversion  [Fairy2i article §2.1]                          */
/* ------------------------------------------------------------------------ */
void orc_real_to_complex(const float* R, int64_t n, int64_t m,
                         double* u_re, double* u_im, double* w_re, double* w_im)
{
    const int64_t ld = 2 * m;
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j < m; ++j) {
            double r11 = R[i * ld + j];
            double r12 = R[i * ld + m + j];
            double r21 = R[(n + i) * ld + j];
            double r22 = R[(n + i) * ld + m + j];
            u_re[i * m + j] = 0.5 * (r11 + r22);
            u_im[i * m + j] = 0.5 * (r21 - r12);
            w_re[i * m + j] = 0.5 * (r11 - r22);
            w_im[i * m + j] = 0.5 * (r12 + r21);
        }
    }
}

void orc_real_to_complex_f32(const float* R, int64_t n, int64_t m,
                             float* u_re, float* u_im, float* w_re, float* w_im)
{
    /* Round the exact half-sums once to fp32.  A sum of two fp32 values
     * formed in double and then rounded to fp32 equals the directly rounded
     * fp32 result (53 >= 2*24+2), and halving is exact in double. */
    const int64_t ld = 2 * m;
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j < m; ++j) {
            double r11 = R[i * ld + j];
            double r12 = R[i * ld + m + j];
            double r21 = R[(n + i) * ld + j];
            double r22 = R[(n + i) * ld + m + j];
            u_re[i * m + j] = (float)(0.5 * (r11 + r22));
            u_im[i * m + j] = (float)(0.5 * (r21 - r12));
            w_re[i * m + j] = (float)(0.5 * (r11 - r22));
            w_im[i * m + j] = (float)(0.5 * (r12 + r21));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Exact mean of |v|  [Fairy2i article §3.2]                                 */
/* ------------------------------------------------------------------------ */
/* Every fp32 magnitude is sig * 2^(eb-150) with a 24-bit integer sig and
 * eb in 1..254 (eb = 1 for subnormals).  The sum of all selected magnitudes is
 * therefore N * 2^-149 with the integer N = sum sig * 2^(eb-1), kept here in a
 * plain multi-word integer (little-endian 32-bit words).  The mean is
 * N / (count * 2^149); the fp32 result is the representable value closest to
 * it (ties to even), found by measuring the exact distance of the candidates. */
#define ORC_WORDS 16

typedef struct { uint32_t w[ORC_WORDS]; } orc_big;

static void big_zero(orc_big* a) { memset(a, 0, sizeof(*a)); }

/* a += v * 2^pos, v < 2^64 */
static void big_add_shifted(orc_big* a, uint64_t v, int pos)
{
    int word = pos / 32, sh = pos % 32;
    /* v << sh spans at most three 32-bit words */
    uint64_t lo = (v << sh) & 0xffffffffull;
    uint64_t mid = (sh == 0) ? (v >> 32) : ((v >> (32 - sh)) & 0xffffffffull);
    uint64_t hi = (sh == 0) ? 0 : (v >> (64 - sh));
    uint64_t parts[3] = {lo, mid, hi};
    uint64_t carry = 0;
    for (int k = word; k < ORC_WORDS; ++k) {
        uint64_t add = (k - word < 3) ? parts[k - word] : 0;
        uint64_t s = (uint64_t)a->w[k] + add + carry;
        a->w[k] = (uint32_t)s;
        carry = s >> 32;
        if (k - word >= 2 && carry == 0) break;
    }
}

static int big_cmp(const orc_big* a, const orc_big* b)
{
    for (int k = ORC_WORDS - 1; k >= 0; --k) {
        if (a->w[k] != b->w[k]) return a->w[k] < b->w[k] ? -1 : 1;
    }
    return 0;
}

/* r = |a - b| */
static void big_absdiff(const orc_big* a, const orc_big* b, orc_big* r)
{
    const orc_big* x = a; const orc_big* y = b;
    if (big_cmp(a, b) < 0) { x = b; y = a; }
    int64_t borrow = 0;
    for (int k = 0; k < ORC_WORDS; ++k) {
        int64_t d = (int64_t)x->w[k] - (int64_t)y->w[k] - borrow;
        borrow = d < 0;
        r->w[k] = (uint32_t)(d + (borrow ? ((int64_t)1 << 32) : 0));
    }
}

static double big_to_double(const orc_big* a)
{
    double s = 0.0;
    for (int k = ORC_WORDS - 1; k >= 0; --k) s = s * 4294967296.0 + (double)a->w[k];
    return s;
}

/* exact value of a non-negative finite float f as k * 2^e */
static void float_parts(float f, uint64_t* k, int* e)
{
    uint32_t bits; memcpy(&bits, &f, 4);
    uint32_t ex = (bits >> 23) & 0xff, man = bits & 0x7fffff;
    if (ex == 0) { *k = man; *e = -149; }
    else { *k = man | 0x800000u; *e = (int)ex - 150; }
}

static float round_ratio_to_f32(const orc_big* N, uint64_t count)
{
    orc_big zero; big_zero(&zero);
    if (count == 0 || big_cmp(N, &zero) == 0) return 0.0f;
    /* approximate, then settle between neighbours exactly */
    double approx = ldexp(big_to_double(N) / (double)count, -149);
    float c0 = (float)approx;
    float cand[3] = { nextafterf(c0, 0.0f), c0, nextafterf(c0, INFINITY) };
    float best = 0.0f; orc_big bestd; int have = 0;
    for (int i = 0; i < 3; ++i) {
        float f = cand[i];
        if (!(f >= 0.0f) || isinf(f)) continue;
        uint64_t k; int e; float_parts(f, &k, &e);
        /* f * count * 2^149 = (k*count) * 2^(e+149), e+149 >= 0 */
        orc_big X; big_zero(&X);
        unsigned __int128 kc = (unsigned __int128)k * count;
        big_add_shifted(&X, (uint64_t)kc, e + 149);
        if ((uint64_t)(kc >> 64)) big_add_shifted(&X, (uint64_t)(kc >> 64), e + 149 + 64);
        orc_big d; big_absdiff(&X, N, &d);
        int better = 0;
        if (!have) better = 1;
        else {
            int c = big_cmp(&d, &bestd);
            if (c < 0) better = 1;
            else if (c == 0) {          /* tie: even significand wins */
                uint64_t kb; int eb; float_parts(best, &kb, &eb);
                if ((kb & 1u) && !(k & 1u)) better = 1;
            }
        }
        if (better) { best = f; bestd = d; have = 1; }
    }
    return best;
}

static void big_add_abs_float(orc_big* N, float v)
{
    uint32_t bits; memcpy(&bits, &v, 4);
    bits &= 0x7fffffffu;
    uint32_t ex = bits >> 23, man = bits & 0x7fffff;
    uint64_t sig = ex ? (man | 0x800000u) : man;
    int eb = ex ? (int)ex : 1;
    if (sig) big_add_shifted(N, sig, eb - 1);
}

float orc_abs_mean(const float* v, const uint8_t* sel, int64_t count)
{
    orc_big N; big_zero(&N);
    uint64_t c = 0;
    for (int64_t i = 0; i < count; ++i) {
        if (!sel[i]) continue;
        big_add_abs_float(&N, v[i]);
        ++c;
    }
    return round_ratio_to_f32(&N, c);
}

/* ------------------------------------------------------------------------ */
/* PhaseQuant with recursive residual stages                                 */
/* [Fairy2i article §3.1, §3.2, §4.1]                                        */
/* ------------------------------------------------------------------------ */
/* Reading of the garbled §4.1 steps: R_1 = W; stage k quantises R_k with its
 * own scales; R_{k+1} = R_k - Q_k(R_k), one fp32 subtraction per element on
 * the axis the code selects (the other axis is unchanged). */
void orc_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                    uint8_t* codes, float* scales, float* resid_re, float* resid_im)
{
    float* r_re = (float*)malloc(sizeof(float) * (size_t)count);
    float* r_im = (float*)malloc(sizeof(float) * (size_t)count);
    uint8_t* sel_re = (uint8_t*)malloc((size_t)count);
    uint8_t* sel_im = (uint8_t*)malloc((size_t)count);
    memcpy(r_re, w_re, sizeof(float) * (size_t)count);
    memcpy(r_im, w_im, sizeof(float) * (size_t)count);

    for (int32_t k = 0; k < stages; ++k) {
        uint8_t* ck = codes + (int64_t)k * count;
        for (int64_t i = 0; i < count; ++i) {
            int32_t c = orc_phase_code(r_re[i], r_im[i]);
            ck[i] = (uint8_t)c;
            sel_re[i] = (c == 0 || c == 2);   /* codeword +-1 */
            sel_im[i] = (c == 1 || c == 3);   /* codeword +-i */
        }
        float s_re = orc_abs_mean(r_re, sel_re, count);
        float s_im = orc_abs_mean(r_im, sel_im, count);
        scales[2 * k + 0] = s_re;
        scales[2 * k + 1] = s_im;
        /* R_{k+1} = R_k - (s_re*Re(i^c) + i*s_im*Im(i^c)) */
        for (int64_t i = 0; i < count; ++i) {
            switch (ck[i]) {
            case 0: r_re[i] = (float)((double)r_re[i] - (double)s_re); break;
            case 1: r_im[i] = (float)((double)r_im[i] - (double)s_im); break;
            case 2: r_re[i] = (float)((double)r_re[i] + (double)s_re); break;
            default: r_im[i] = (float)((double)r_im[i] + (double)s_im); break;
            }
        }
    }
    if (resid_re) memcpy(resid_re, r_re, sizeof(float) * (size_t)count);
    if (resid_im) memcpy(resid_im, r_im, sizeof(float) * (size_t)count);
    free(r_re); free(r_im); free(sel_re); free(sel_im);
}

/* ------------------------------------------------------------------------ */
/* Packing: 16 two-bit codes per uint32                                      */
/* ------------------------------------------------------------------------ */
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t orc_packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout)
{
    if (layout == 0) return (int64_t)planes * rows * (m / 16);
    return rows * ceil_div(m, 64) * planes * 4;
}

/* word index and bit offset of (plane, row, column) */
static void orc_locate(int32_t planes, int64_t rows, int64_t m, int32_t layout,
                       int32_t p, int64_t r, int64_t c, int64_t* word, int* bit)
{
    if (layout == 0) {
        *word = ((int64_t)p * rows + r) * (m / 16) + c / 16;
        *bit = (int)(2 * (c % 16));
    } else {
        int64_t groups = ceil_div(m, 64);
        int64_t g = c / 64, u = (c % 64) / 16;
        int t = (int)(c % 16);
        *word = ((r * groups + g) * planes + p) * 4 + u;
        *bit = (t % 2 == 0) ? 14 - t : 31 - t;
    }
}

void orc_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m,
              int32_t layout, uint32_t* out)
{
    int64_t nw = orc_packed_words(rows, m, planes, layout);
    memset(out, 0, sizeof(uint32_t) * (size_t)nw);   /* padding columns: code 0 */
    for (int32_t p = 0; p < planes; ++p)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < m; ++c) {
                int64_t w; int bit;
                orc_locate(planes, rows, m, layout, p, r, c, &w, &bit);
                out[w] |= (uint32_t)(codes[((int64_t)p * rows + r) * m + c] & 3u) << bit;
            }
}

void orc_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m,
                int32_t layout, uint8_t* codes)
{
    for (int32_t p = 0; p < planes; ++p)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < m; ++c) {
                int64_t w; int bit;
                orc_locate(planes, rows, m, layout, p, r, c, &w, &bit);
                codes[((int64_t)p * rows + r) * m + c] = (uint8_t)((packed[w] >> bit) & 3u);
            }
}

/* ------------------------------------------------------------------------ */
/* Complex linear layer                                                      */
/* ------------------------------------------------------------------------ */
/* codeword i^c, in the order the page's phase_quant returns them */
static const double complex ORC_CODEWORD[4] = { 1.0, I, -1.0, -I };

void orc_cgemv_dense(const uint8_t* codes, const float* scales, int32_t stages, int32_t has_conj,
                     int64_t n, int64_t m, const double* x_re, const double* x_im,
                     int32_t batch, int64_t ldx, double* y_re, double* y_im, int64_t ldy)
{
    const int32_t planes = stages * (has_conj ? 2 : 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int32_t b = 0; b < batch; ++b) {
            double complex y = 0.0;
            for (int32_t p = 0; p < planes; ++p) {
                const int conj_plane = (p >= stages);      /* W_k multiplies conj(x) */
                const double s_re = scales[2 * p], s_im = scales[2 * p + 1];
                const uint8_t* row = codes + ((int64_t)p * n + r) * m;
                for (int64_t j = 0; j < m; ++j) {
                    double complex q = ORC_CODEWORD[row[j] & 3];
                    double complex w = s_re * creal(q) + I * (s_im * cimag(q));
                    double complex x = x_re[b * ldx + j] + I * x_im[b * ldx + j];
                    y += w * (conj_plane ? conj(x) : x);
                }
            }
            y_re[b * ldy + r] = creal(y);
            y_im[b * ldy + r] = cimag(y);
        }
    }
}

void orc_cgemv_acc(const uint8_t* codes, const float* scales, int32_t stages, int32_t has_conj,
                   int64_t n, int64_t m, const double* x_re, const double* x_im,
                   int32_t batch, int64_t ldx, double* acc, double* y_re, double* y_im, int64_t ldy)
{
    const int32_t planes = stages * (has_conj ? 2 : 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int32_t b = 0; b < batch; ++b) {
            double yr = 0.0, yi = 0.0;
            for (int32_t p = 0; p < planes; ++p) {
                const uint8_t* row = codes + ((int64_t)p * n + r) * m;
                double A1 = 0, A2 = 0, A3 = 0, A4 = 0;
                for (int64_t j = 0; j < m; ++j) {
                    double complex q = ORC_CODEWORD[row[j] & 3];
                    double reB = creal(q), imB = cimag(q);
                    double xr = x_re[b * ldx + j], xi = x_im[b * ldx + j];
                    A1 += reB * xr;
                    A2 += imB * xi;
                    A3 += reB * xi;
                    A4 += imB * xr;
                }
                if (acc) {
                    acc[(((int64_t)p * 4 + 0) * batch + b) * n + r] = A1;
                    acc[(((int64_t)p * 4 + 1) * batch + b) * n + r] = A2;
                    acc[(((int64_t)p * 4 + 2) * batch + b) * n + r] = A3;
                    acc[(((int64_t)p * 4 + 3) * batch + b) * n + r] = A4;
                }
                const double s_re = scales[2 * p], s_im = scales[2 * p + 1];
                if (p < stages) {
                    /* (s_re ReB + i s_im ImB)(xr + i xi) */
                    yr += s_re * A1 - s_im * A2;
                    yi += s_re * A3 + s_im * A4;
                } else {
                    /* (s_re ReB + i s_im ImB)(xr - i xi) */
                    yr += s_re * A1 + s_im * A2;
                    yi += -s_re * A3 + s_im * A4;
                }
            }
            y_re[b * ldy + r] = yr;
            y_im[b * ldy + r] = yi;
        }
    }
}

void orc_cgemv_acc_i64(const uint8_t* codes, int32_t planes, int64_t n, int64_t m,
                       const int8_t* x_re, const int8_t* x_im, int32_t batch, int64_t ldx,
                       int64_t* acc)
{
    /* ReB, ImB of the codeword i^c */
    static const int RE[4] = { 1, 0, -1, 0 };
    static const int IM[4] = { 0, 1, 0, -1 };
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int32_t b = 0; b < batch; ++b) {
            for (int32_t p = 0; p < planes; ++p) {
                const uint8_t* row = codes + ((int64_t)p * n + r) * m;
                int64_t A1 = 0, A2 = 0, A3 = 0, A4 = 0;
                for (int64_t j = 0; j < m; ++j) {
                    int c = row[j] & 3;
                    int64_t xr = x_re[b * ldx + j], xi = x_im[b * ldx + j];
                    A1 += RE[c] * xr;
                    A2 += IM[c] * xi;
                    A3 += RE[c] * xi;
                    A4 += IM[c] * xr;
                }
                acc[(((int64_t)p * 4 + 0) * batch + b) * n + r] = A1;
                acc[(((int64_t)p * 4 + 1) * batch + b) * n + r] = A2;
                acc[(((int64_t)p * 4 + 2) * batch + b) * n + r] = A3;
                acc[(((int64_t)p * 4 + 3) * batch + b) * n + r] = A4;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Complex attention  [iFairy press article §三; Fairy2i article §2.2]      */
/* ------------------------------------------------------------------------ */
/* score(i, j) = scale * Re( sum_d q[i][d] * conj(k[j][d]) ), written with
 * complex arithmetic exactly as the definition reads; the softmax is the
 * textbook one (subtract the row maximum, exponentiate, normalise). */
static int orc_masked(int32_t causal, int64_t i, int64_t j, int64_t sq, int64_t sk)
{
    return causal && j > i + (sk - sq);
}

void orc_cattn_scores(const float* q_re, const float* q_im, const float* k_re, const float* k_im,
                      int32_t heads, int64_t sq, int64_t sk, int32_t d, double scale, int32_t causal,
                      double* s)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < sq; ++i) {
            const int64_t qo = ((int64_t)h * sq + i) * d;
            for (int64_t j = 0; j < sk; ++j) {
                double* out = s + ((int64_t)h * sq + i) * sk + j;
                if (orc_masked(causal, i, j, sq, sk)) {
                    *out = -INFINITY;
                    continue;
                }
                const int64_t ko = ((int64_t)h * sk + j) * d;
                double complex acc = 0.0;
                for (int32_t t = 0; t < d; ++t) {
                    const double complex q = (double)q_re[qo + t] + I * (double)q_im[qo + t];
                    const double complex k = (double)k_re[ko + t] + I * (double)k_im[ko + t];
                    acc += q * conj(k);
                }
                *out = scale * creal(acc);
            }
        }
}

void orc_cattention(const float* q_re, const float* q_im, const float* k_re, const float* k_im,
                    const float* v_re, const float* v_im, int32_t heads, int64_t sq, int64_t sk, int32_t d,
                    double scale, int32_t causal, double* o_re, double* o_im)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)heads * (size_t)sq * (size_t)sk);
    if (!s) abort();
    orc_cattn_scores(q_re, q_im, k_re, k_im, heads, sq, sk, d, scale, causal, s);
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < sq; ++i) {
            const double* row = s + ((int64_t)h * sq + i) * sk;
            double mx = -INFINITY;
            for (int64_t j = 0; j < sk; ++j)
                if (row[j] > mx) mx = row[j];
            double den = 0.0;
            for (int64_t j = 0; j < sk; ++j) den += (row[j] == -INFINITY) ? 0.0 : exp(row[j] - mx);
            for (int32_t t = 0; t < d; ++t) {
                double ar = 0.0, ai = 0.0;
                for (int64_t j = 0; j < sk; ++j) {
                    if (row[j] == -INFINITY) continue;
                    const double p = exp(row[j] - mx) / den;
                    const int64_t vo = ((int64_t)h * sk + j) * d + t;
                    ar += p * (double)v_re[vo];   /* real and imaginary parts weighted separately */
                    ai += p * (double)v_im[vo];
                }
                o_re[((int64_t)h * sq + i) * d + t] = ar;
                o_im[((int64_t)h * sq + i) * d + t] = ai;
            }
        }
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Complex rotary position encoding  [iFairy press article §三]             */
/* ------------------------------------------------------------------------ */
void orc_rope(double* y_re, double* y_im, int64_t rows, int64_t n, int64_t ld, const int32_t* pos,
              int32_t head_dim, double base)
{
    for (int64_t b = 0; b < rows; ++b)
        for (int64_t r = 0; r < n; ++r) {
            const int64_t j = r % head_dim;
            const double theta = pow(base, -(double)j / (double)head_dim);
            const double complex rot = cexp(I * ((double)pos[b] * theta));
            const double complex y = (y_re[b * ld + r] + I * y_im[b * ld + r]) * rot;
            y_re[b * ld + r] = creal(y);
            y_im[b * ld + r] = cimag(y);
        }
}
