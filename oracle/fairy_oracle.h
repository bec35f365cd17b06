/*
 * fairy_oracle.h -- plain, slow CPU oracle for the 2-bit PhaseQuant complex
 * linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Everything is computed the obvious way, in double precision (exact integer
 * arithmetic where the method decides integers), straight from the
 * definitions on the pages:
 *
 *   [Fairy2i article]  hotelren.com/news/3072820, "复数域低比特量化框架Fairy2i":
 *       §2.1 real-to-complex widely-linear conversion,
 *       §3.1 unit-circle codebook {1, i, -1, -i} and the phase rule,
 *       §3.2 axis-aligned scales s_re, s_im,
 *       §4.1 recursive residual quantisation,
 *       §4.2 multiplication-free matmul (four real partial products).
 *   [iFairy talk]      news.43b.com.cn/a/865699.html, minutes of the iFairy talk:
 *       §2.3.1 multiplying by i is a real/imag swap plus a negation.
 *   [iFairy abstract]  arXiv 2508.05571 record: every code has exactly one
 *       non-zero axis, so inference needs only additions and swaps.
 *   [iFairy press article] bestcxt.com, §三: attention scores are the real
 *       part of the Hermitian inner product (a real number for the softmax).
 *
 * Readings taken where the pages are silent are stated next to the
 * function they affect.
 *
 * Parity pins (the tests that tie this oracle to something other than
 * itself) live in tests/test_oracle_*.py.
 */
#ifndef FAIRY_ORACLE_H
#define FAIRY_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t orc_version(void);

/* Number of OpenMP threads used by the row-parallel GEMV/GEMM loops
 * (each output row is still summed sequentially, so results do not depend
 * on it).  Returns the count actually in effect. */
int32_t orc_set_threads(int32_t nthreads);

/* PhaseQuant code of one complex weight re + i*im:
 * the quadrant k = floor(2*theta/pi + 1/2) mod 4 of theta = arg(w),
 * codeword i^k (0 <-> 1, 1 <-> i, 2 <-> -1, 3 <-> -i).
 * [Fairy2i article §3.1]  Evaluated by exact comparisons. */
int32_t orc_phase_code(float re, float im);

/* Widely-linear conversion [Fairy2i article §2.1]:
 * R is row-major [2n][2m]; outputs are [n][m] in double, exact:
 *   ReU = (R11+R22)/2, ImU = (R21-R12)/2, ReW = (R11-R22)/2, ImW = (R12+R21)/2. */
void orc_real_to_complex(const float* R, int64_t n, int64_t m,
                         double* u_re, double* u_im, double* w_re, double* w_im);

/* Same conversion rounded once to fp32 (round to nearest even). */
void orc_real_to_complex_f32(const float* R, int64_t n, int64_t m,
                             float* u_re, float* u_im, float* w_re, float* w_im);

/* Exact mean of |v[i]| over the i with sel[i] != 0, rounded once to the
 * nearest fp32 (ties to even).  Empty selection -> 0.  count < 2^32. */
float orc_abs_mean(const float* v, const uint8_t* sel, int64_t count);

/* PhaseQuant with S recursive residual stages over `count` complex weights.
 *   codes  : [stages][count] uint8 (values 0..3)
 *   scales : [stages][2] = {s_re, s_im}
 *   resid  : R_{S+1} (nullable)
 * [Fairy2i article §3.1, §3.2, §4.1] */
void orc_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                    uint8_t* codes, float* scales, float* resid_re, float* resid_im);

/* Packed layouts (16 codes per uint32).
 *   0 = ROW16  : words [planes][rows][m/16]; column 16w+t at bits 2t..2t+1.
 *   1 = TILED64: words [rows][ceil(m/64)][planes][4]; word u of group g holds
 *                column 64g+16u+t at bit offset (t even ? 14-t : 31-t);
 *                columns >= m hold code 0. */
int64_t orc_packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout);
void orc_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m,
              int32_t layout, uint32_t* out);
void orc_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m,
                int32_t layout, uint8_t* codes);

/* Complex linear layer with dequantised weights, dense complex arithmetic:
 *   y[b] = sum_{k<S} What(U_k) x[b] + has_conj * sum_{k<S} What(W_k) conj(x[b])
 * with What(c) = s_re*Re(i^c) + i*s_im*Im(i^c).
 * codes: [P][n][m] with P = S*(1+has_conj), planes ordered U_1..U_S, W_1..W_S;
 * scales: [P][2]; x_re/x_im: [batch][ldx]; y_re/y_im: [batch][ldy]. */
void orc_cgemv_dense(const uint8_t* codes, const float* scales, int32_t stages, int32_t has_conj,
                     int64_t n, int64_t m, const double* x_re, const double* x_im,
                     int32_t batch, int64_t ldx, double* y_re, double* y_im, int64_t ldy);

/* The same layer in the four-accumulator form [Fairy2i article §4.2]:
 * per plane p, row r, column b:
 *   A1 = sum ReB*x_re, A2 = sum ImB*x_im, A3 = sum ReB*x_im, A4 = sum ImB*x_re
 * (ReB, ImB in {-1,0,1}), then the per-axis scales once at the end.
 * acc (nullable): [P][4][batch][n]. */
void orc_cgemv_acc(const uint8_t* codes, const float* scales, int32_t stages, int32_t has_conj,
                   int64_t n, int64_t m, const double* x_re, const double* x_im,
                   int32_t batch, int64_t ldx, double* acc, double* y_re, double* y_im, int64_t ldy);

/* Integer activations: exact int64 four-accumulator sums, acc [P][4][batch][n]. */
void orc_cgemv_acc_i64(const uint8_t* codes, int32_t planes, int64_t n, int64_t m,
                       const int8_t* x_re, const int8_t* x_im, int32_t batch, int64_t ldx,
                       int64_t* acc);

/* Complex attention  [iFairy press article §三; Fairy2i article §2.2;
 * iFairy talk §2.1.4]: the similarity of query q and key k is the real part
 * of their Hermitian inner product, Re(sum_d q_d conj(k_d)); a softmax over
 * the keys turns the (scaled) scores into real weights, and the value
 * vectors' real and imaginary parts are averaged with those weights.
 *   q: [heads][sq][d], k, v: [heads][sk][d], split re/im planes (float);
 *   causal != 0: query i sees keys j <= i + (sk - sq) only (sk >= sq).
 * Scores: s [heads][sq][sk] = scale * Re(q . conj(k)), masked entries -inf.
 * Output: o [heads][sq][d] (double). */
void orc_cattn_scores(const float* q_re, const float* q_im, const float* k_re, const float* k_im,
                      int32_t heads, int64_t sq, int64_t sk, int32_t d, double scale, int32_t causal,
                      double* s);
void orc_cattention(const float* q_re, const float* q_im, const float* k_re, const float* k_im,
                    const float* v_re, const float* v_im, int32_t heads, int64_t sq, int64_t sk, int32_t d,
                    double scale, int32_t causal, double* o_re, double* o_im);

/* Complex rotary position encoding  [iFairy press article §三; iFairy talk
 * §2.1.3]: on the complex plane the rotation is one complex multiplication.
 * y[b][r] <- y[b][r] * exp(i * pos[b] * theta_j), j = r % head_dim,
 * theta_j = base^(-j / head_dim); y is [rows][ld] (double, in place). */
void orc_rope(double* y_re, double* y_im, int64_t rows, int64_t n, int64_t ld, const int32_t* pos,
              int32_t head_dim, double base);

#ifdef __cplusplus
}
#endif
#endif
