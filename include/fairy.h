/*
 * fairy.h -- libfairy: the multiplication-free 2-bit complex linear layer
 * (iFairy / Fairy±i, Fairy2i) on AMD MI355X (gfx950).
 *
 *   y = sum_k [ Q(U_k) x + Q(W_k) conj(x) ]
 *
 * Each weight is a 2-bit PhaseQuant code c in {0,1,2,3} standing for the
 * codeword i^c in {1, i, -1, -i}; each (matrix, stage) carries two per-axis
 * scales (s_re, s_im).  Products reduce to sign flips and real/imag swaps
 * feeding four fp32 accumulators; the scales are applied once at the end.
 *
 * Sources (web pages; cited by page title and section):
 *   [Fairy2i article]  "复数域低比特量化框架Fairy2i" (hotelren.com/news/3072820):
 *                      §2.1 widely-linear conversion, §3.1 codebook and phase
 *                      rule, §3.2 axis scales, §4.1 recursive residual,
 *                      §4.2 multiplication-free matmul, §5.2 (troubleshooting)
 *                      item 3: check that real and imaginary parts are kept
 *                      and handled apart.
 *   [iFairy press article] bestcxt.com article on iFairy, §一: two bits per
 *                      weight, one eighth of the storage of fp16.
 *   [iFairy talk]      minutes of the talk "iFairy: 2-bit复数基座大模型"
 *                      (news.43b.com.cn/a/865699.html), §2.3.1: times i is a
 *                      real/imag swap with a negation.
 *   [iFairy abstract]  arXiv 2508.05571 record: one non-zero axis per code,
 *                      inference with additions and swaps only.
 *   [Fairy2i abstract] chatpaper.ai record of Fairy2i: widely-linear form,
 *                      recursive residual quantisation, multiplication-free
 *                      accumulation.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - All data pointers are DEVICE pointers unless stated otherwise.  The
 *    fairy_clinear descriptor itself is read on the host.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is asynchronous on that stream; the caller keeps every buffer alive
 *    until the stream has synchronised.
 *  - The caller allocates and owns every buffer.  The library allocates no
 *    device memory, keeps no pointer after a call returns and has no mutable
 *    global state; calls on different streams may overlap.
 *  - Arguments are validated on the host before any launch.  A call that
 *    returns an error launches nothing and writes nothing.  Calls never
 *    throw, abort or print.
 *  - Complex data is always split into separate real and imaginary planes
 *    (structure of arrays), as [Fairy2i article §5.2, item 3] asks.
 *  - Inputs must be finite.  NaN/Inf inputs are undefined behaviour (not
 *    checked).
 */
#ifndef FAIRY_H
#define FAIRY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FAIRY_ABI_VERSION 1

typedef enum {
    FAIRY_OK = 0,
    FAIRY_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad enum, misalignment */
    FAIRY_ERR_UNSUPPORTED = 2,  /* valid request outside what v1 implements */
    FAIRY_ERR_HIP = 3,          /* a HIP runtime call or launch failed */
    FAIRY_ERR_WORKSPACE = 4     /* workspace missing or too small */
} fairy_status;

/* Packed code layouts.  Both hold 16 two-bit codes per uint32.
 *  ROW16   : words [planes][rows][m/16]; column 16w+t of a row sits at
 *            bits 2t..2t+1 of its word w.  Canonical interchange layout.
 *  TILED64 : words [rows][ceil(m/64)][planes][4]; the 64 columns of group g
 *            of every plane of a row are contiguous (planes interleaved), and
 *            word u of the group holds column 64g+16u+t at bit offset
 *            (t even ? 14-t : 31-t).  Columns >= m hold code 0.  This is the
 *            layout the GEMV/GEMM kernels read: one 128-bit load per lane per
 *            plane, and after a left shift by 2k the codes of columns 2k and
 *            2k+1 sit in the sign and top exponent bits of a bf16 pair.
 * Inside a word, a code's bit 1 is the sign of its codeword and bit 0 its
 * axis (0 = real, 1 = imaginary): code c <-> i^c. */
typedef enum {
    FAIRY_LAYOUT_ROW16 = 0,
    FAIRY_LAYOUT_TILED64 = 1
} fairy_layout;

/* Activation element types (SoA planes, row-major [batch][ldx]). */
typedef enum {
    FAIRY_F32 = 0,
    FAIRY_BF16 = 1,  /* raw bfloat16 bit patterns */
    FAIRY_I8 = 2     /* plain integers, scale 1 */
} fairy_dtype;

/* Prefill GEMM algorithm. */
typedef enum {
    FAIRY_ALGO_AUTO = 0,
    FAIRY_ALGO_VALU = 1,  /* direct decode on the vector ALUs */
    FAIRY_ALGO_MFMA = 2   /* codes expanded to ternary planes, matrix cores */
} fairy_algo;

/* A quantised complex linear layer.
 *  n, m      : complex output and input sizes (rows x columns).
 *  stages    : S, number of recursive residual stages (1..8).
 *  has_conj  : 1 for the widely-linear form U x + W conj(x), 0 for U x only.
 *  Planes    : P = S * (1 + has_conj), ordered U_1..U_S, W_1..W_S.
 *  layout    : FAIRY_LAYOUT_TILED64 for fairy_cgemv / fairy_cgemm.
 *  packed    : device, fairy_packed_words(n, m, P, layout) uint32 words,
 *              16-byte aligned.
 *  scales    : device float [P][2] = {s_re, s_im} per plane. */
typedef struct {
    int64_t n, m;
    int32_t stages, has_conj;
    int32_t layout;
    const uint32_t* packed;
    const float* scales;
} fairy_clinear;

int32_t fairy_abi_version(void);

/* Static, human-readable name of a status code; never NULL. */
const char* fairy_status_string(fairy_status status);

/* Widely-linear conversion of a real layer [Fairy2i article §2.1]:
 * R (row-major [2n][2m] fp32) is split into blocks R11 = R[:n,:m],
 * R12 = R[:n,m:], R21 = R[n:,:m], R22 = R[n:,m:] and
 *   ReU = (R11+R22)/2, ImU = (R21-R12)/2, ReW = (R11-R22)/2, ImW = (R12+R21)/2,
 * each rounded once to fp32 (nearest even).  Then R x equals U x_c + W conj(x_c)
 * under x_c = x[:m] + i x[m:], y_c = y[:n] + i y[n:].
 * Outputs u_re, u_im, w_re, w_im are [n][m].  n, m >= 1. */
fairy_status fairy_real_to_complex(const float* R, int64_t n, int64_t m,
                                   float* u_re, float* u_im, float* w_re, float* w_im,
                                   void* stream);

/* Workspace for fairy_phasequant: per stage, 16 copies of 512 uint64
 * exponent buckets plus 2 counts (65,792 bytes per stage; the copies spread
 * the integer atomics of the launch).  Returns 0 for invalid arguments. */
size_t fairy_phasequant_workspace_bytes(int64_t count, int32_t stages);

/* PhaseQuant with S recursive residual stages [Fairy2i article §3.1, §3.2,
 * §4.1; iFairy abstract].
 *   Stage k (k = 1..S) quantises R_k (R_1 = W):
 *     code  = quadrant of arg(R_k): floor(2 theta/pi + 1/2) mod 4, evaluated by
 *             exact comparisons; |Re| == |Im| goes to the counter-clockwise
 *             neighbour; 0 (any signed zeros) -> code 0;
 *     s_re  = mean |Re R_k| over entries coded +-1, s_im = mean |Im R_k| over
 *             entries coded +-i: the exact mean rounded once to fp32 (nearest
 *             even); an empty set gives 0.  Reduction is in exact integers,
 *             so the result does not depend on launch shape or order;
 *     R_{k+1} = R_k - (s_re Re(i^c) + i s_im Im(i^c)): one fp32 subtraction
 *             on the code's axis.
 *   w_re, w_im : [count] fp32 (a matrix is passed flattened, row-major).
 *   codes      : [stages][count] uint8 (0..3).
 *   scales     : [stages][2] fp32 {s_re, s_im}, written on the device.
 *   resid_re/im: nullable, R_{S+1}.
 *   workspace  : device, >= fairy_phasequant_workspace_bytes(count, stages),
 *                8-byte aligned; contents on entry are ignored.
 * 1 <= count < 2^32, 1 <= stages <= 8. */
fairy_status fairy_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                              uint8_t* codes, float* scales, float* resid_re, float* resid_im,
                              void* workspace, size_t workspace_bytes, void* stream);

/* PhaseQuant for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): fairy_phasequant
 * with the same arguments except the workspace, and the same kernels and
 * results bit for bit.  The exponent buckets live in a static device array
 * inside the library, 526,336 bytes (8 stages x 65,792), which each GPU the
 * library runs on holds until the process ends; every valid stage count
 * fits (otherwise UNSUPPORTED).  The call allocates nothing (no hipMalloc,
 * no allocating library routine); its first call on a device looks up the
 * array's address there.  All calls on one GPU share that array: calls that
 * overlap on one GPU (on different streams) race and must not be issued. */
fairy_status fairy_phasequant_noalloc(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                                      uint8_t* codes, float* scales, float* resid_re, float* resid_im,
                                      void* stream);

/* ---- Packed storage ------------------------------------------------------------
 * [iFairy press article §一: a weight takes two bits, so a model takes one
 * eighth of its fp16 storage; Fairy2i article §5.2 item 3: the device must
 * support the complex storage format, real and imaginary parts kept apart]
 * The pages fix no word layout: ROW16 and TILED64 above are this library's.
 *
 * Number of uint32 words of a packed buffer; -1 for invalid arguments. */
int64_t fairy_packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout);

/* Pack codes [planes][rows][m] (uint8, values 0..3; higher bits ignored)
 * into `layout`, 16 codes per uint32.  m % 16 == 0 (else UNSUPPORTED);
 * codes and packed 16-byte aligned. */
fairy_status fairy_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m,
                        int32_t layout, uint32_t* packed, void* stream);

/* Inverse of fairy_pack (padding columns are not written). */
fairy_status fairy_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m,
                          int32_t layout, uint8_t* codes, void* stream);

/* Workspace bytes fairy_cgemv needs for this layer and batch (0 in v1). */
size_t fairy_cgemv_workspace_bytes(const fairy_clinear* L, int32_t batch, int32_t xdtype);

/* Decode-time complex GEMV [Fairy2i article §4.2, §2.1; iFairy talk §2.3.1]:
 *   y[b] = sum_{k<S} What(U_k) x[b] + has_conj * sum_{k<S} What(W_k) conj(x[b]),
 *   What(c) = s_re Re(i^c) + i s_im Im(i^c),
 * computed as four accumulators per plane and batch column,
 *   A1 = sum ReB x_re, A2 = sum ImB x_im, A3 = sum ReB x_im, A4 = sum ImB x_re,
 * and the epilogue  U plane: y_re += s_re A1 - s_im A2, y_im += s_re A3 + s_im A4;
 *                   W plane: y_re += s_re A1 + s_im A2, y_im += s_im A4 - s_re A3.
 *   x_re, x_im : [batch][ldx] of xdtype (F32, BF16 or I8), 16-byte aligned,
 *                ldx >= m and ldx a multiple of 16 elements.
 *   y_re, y_im : [batch][ldy] fp32, ldy >= n.  Overwritten.
 *   acc        : nullable; I8 only: int32 [P][4][batch][n], the exact integer
 *                accumulators A1..A4 per plane (planes U_1..U_S, W_1..W_S).
 *   batch      : 1..64.
 *   workspace  : may be NULL when fairy_cgemv_workspace_bytes() is 0.
 * The layer must be TILED64 with m % 16 == 0 and m <= 7680 (F32), 14528
 * (BF16) or 26112 (I8): one batch column of activations is staged whole in
 * 64 KiB of LDS.  Otherwise UNSUPPORTED.
 * float outputs are within 1e-5 relative L2 of the exact result on the same
 * inputs; integer accumulators are exact. */
fairy_status fairy_cgemv(const fairy_clinear* L, const void* x_re, const void* x_im,
                         int32_t xdtype, int32_t batch, int64_t ldx,
                         float* y_re, float* y_im, int64_t ldy, int32_t* acc,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- Several layers on one input ------------------------------------------------
 * [Fairy2i article §2.2, item 1: every projection matrix of an attention
 * layer (Q, K and V) gets its own widely-linear form, and all of them are
 * applied to the same input]  fairy_cgemv for `count` layers that read the
 * same activations, in one launch where the shape allows (the q, k and v
 * projections, or gate and up of an MLP), else layer by layer.  Each output
 * equals what fairy_cgemv gives for that layer alone (same kernels and
 * summation order).
 *   layers     : host array [count] (1 <= count <= 8) of descriptors, each
 *                valid for fairy_cgemv; all with the same m, stages and
 *                has_conj (else INVALID_ARG); n may differ.
 *   x_re, x_im : as fairy_cgemv, shared by every layer.
 *   y_re, y_im : host arrays [count] of device pointers, layer l writes
 *                [batch][ldy[l]] fp32 there; ldy: host array [count].
 *   batch      : 1..64.  No raw accumulators.
 * Same float bound as fairy_cgemv. */
fairy_status fairy_cgemv_group(const fairy_clinear* layers, int32_t count, const void* x_re, const void* x_im,
                               int32_t xdtype, int32_t batch, int64_t ldx, float* const* y_re, float* const* y_im,
                               const int64_t* ldy, void* stream);

/* ---- Table-lookup GEMV (batch 1) ----------------------------------------------
 * [iFairy talk §2.3.2: table-lookup inference precomputes the results of the
 * 16 input combinations of a pair of codes]  Same result as fairy_cgemv with
 * batch = 1, computed another way: for every pair of same-parity columns held
 * in one 4-bit field of a TILED64 word and every plane, a 16-entry table of
 * (y_re, y_im) contributions is built from x and the plane's scales, and each
 * pair of codes costs one table read and two adds.  Kept as a measured
 * alternative to the direct bit decode of fairy_cgemv.
 *   x_re, x_im : [m] of xdtype (F32 or BF16; I8 is UNSUPPORTED), 16-byte aligned.
 *   y_re, y_im : [n] fp32, overwritten.
 *   workspace  : device, 16-byte aligned, at least
 *                fairy_cgemv_lut_workspace_bytes(L) bytes (partial sums of
 *                the column chunks); may be NULL when that is 0.
 * The layer must be TILED64 with m % 16 == 0 (no limit on m from LDS).
 * Float outputs are within 1e-5 relative L2 of the exact result; the chunk
 * partials are added in a fixed order, so repeated calls are bitwise equal.
 * fairy_cgemv_lut_workspace_bytes returns 0 for an invalid layer as well. */
size_t fairy_cgemv_lut_workspace_bytes(const fairy_clinear* L);
fairy_status fairy_cgemv_lut(const fairy_clinear* L, const void* x_re, const void* x_im,
                             int32_t xdtype, float* y_re, float* y_im,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the optional fairy_cgemm workspace for these arguments, 0 when
 * no path uses one.  The matrix-core path at token counts whose 64-row x
 * 64-token blocks would leave compute units idle (P of 1, 2 or 4 and no acc
 * requested) splits the K range and keeps fp32 partial sums there:
 * splits x 2 x M x n floats, added in split order by a second kernel. */
size_t fairy_cgemm_workspace_bytes(const fairy_clinear* L, int64_t M, int32_t xdtype, int32_t algo);

/* Prefill GEMM: fairy_cgemv over M >= 1 token rows (same semantics, same
 * argument rules with batch replaced by M; acc is [P][4][M][n] for I8).
 * algo: AUTO, VALU (any dtype) or MFMA (BF16 or I8; codes expanded to
 * ternary {-1,0,1} planes feeding the matrix cores).  AUTO takes MFMA for
 * BF16 and I8 from M = 16.  The m limit of fairy_cgemv applies to the VALU
 * path only: the matrix-core path streams the activations in chunks.
 * workspace: NULL (the call runs without a K split) or at least
 *   fairy_cgemm_workspace_bytes() bytes, 16-byte aligned, owned by the
 *   caller and not read before being written (ERR_WORKSPACE if smaller or
 *   misaligned).  Calls sharing one workspace must not overlap. */
fairy_status fairy_cgemm(const fairy_clinear* L, const void* x_re, const void* x_im,
                         int32_t xdtype, int64_t M, int64_t ldx,
                         float* y_re, float* y_im, int64_t ldy, int32_t* acc, int32_t algo,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- Rotary position encoding fused into the output ---------------------------
 * [iFairy press article §三 and iFairy talk §2.1.3: on the complex plane the
 * rotary position encoding is one complex multiplication per output]
 * Same as fairy_cgemv / fairy_cgemm (no raw accumulators), then every output
 *   y[b][r] <- y[b][r] * exp(i * positions[b] * theta_j),
 *   j = r % head_dim,  theta_j = base^(-j / head_dim),
 * i.e. the rotate-half real RoPE of a real head of 2*head_dim dimensions
 * whose dimension pairs (j, j + head_dim) are the complex dimension j.
 * Angles and the rotation are evaluated in fp64 and rounded once to fp32.
 *   positions : device int32 [batch] (or [M]), 4-byte aligned
 *   head_dim  : complex dimensions per head, >= 1;  base : finite, > 0. */
fairy_status fairy_cgemv_rope(const fairy_clinear* L, const void* x_re, const void* x_im,
                              int32_t xdtype, int32_t batch, int64_t ldx,
                              float* y_re, float* y_im, int64_t ldy,
                              const int32_t* positions, int32_t head_dim, float base, void* stream);
fairy_status fairy_cgemm_rope(const fairy_clinear* L, const void* x_re, const void* x_im,
                              int32_t xdtype, int64_t M, int64_t ldx,
                              float* y_re, float* y_im, int64_t ldy, int32_t algo,
                              const int32_t* positions, int32_t head_dim, float base, void* stream);

/* ---- Whole-layer conversion on the device ----------------------------------
 * [Fairy2i article §2.1 (widely-linear split), §3.1-§3.2 (PhaseQuant codes and
 * axis scales), §4.1 (recursive residual stages)]: the steps above chained on
 * `stream` with every intermediate in `workspace`, ending in TILED64 words.
 * For a real layer the PhaseQuant stages read R and form U and W themselves
 * (the same rounding as fairy_real_to_complex), so the U, W planes never
 * reach memory; the workspace holds the byte codes and the buckets.
 *
 * Workspace bytes for a conversion (0 for invalid arguments): has_conj = 1
 * for fairy_quantize_real, 0 for fairy_quantize_complex. */
size_t fairy_quantize_workspace_bytes(int64_t n, int64_t m, int32_t stages, int32_t has_conj);

/* R: device fp32 [2n][2m], row-major.  Output: a widely-linear layer with
 * P = 2S planes U_1..U_S, W_1..W_S,
 *   packed : device, fairy_packed_words(n, m, 2S, TILED64) words, 16-byte aligned;
 *   scales : device float [2S][2].
 * Bit-identical to fairy_real_to_complex, fairy_phasequant on U and on W,
 * and fairy_pack(TILED64) called in turn.  n*m < 2^32, 1 <= S <= 8;
 * m % 16 == 0 (else UNSUPPORTED); workspace 256-byte aligned, at least
 * fairy_quantize_workspace_bytes(n, m, S, 1) (else ERR_WORKSPACE). */
fairy_status fairy_quantize_real(const float* R, int64_t n, int64_t m, int32_t stages,
                                 uint32_t* packed, float* scales,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* w_re, w_im: device fp32 [n][m] of a complex layer; output P = S planes
 * (no conjugate branch).  Same rules, workspace from
 * fairy_quantize_workspace_bytes(n, m, S, 0). */
fairy_status fairy_quantize_complex(const float* w_re, const float* w_im, int64_t n, int64_t m,
                                    int32_t stages, uint32_t* packed, float* scales,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---- Serialised quantised layer ------------------------------------------------
 * This library's own format (the pages define none), little-endian:
 *   offset  bytes  field
 *        0      8  magic, the ASCII bytes "FAIRYQL1"
 *        8      4  uint32 format version (1)
 *       12      4  uint32 header bytes H = 64 + 8P rounded up to a multiple of 64
 *       16      8  int64 n          24  8  int64 m
 *       32      4  int32 stages S   36  4  int32 has_conj
 *       40      4  int32 layout (FAIRY_LAYOUT_TILED64)
 *       44      4  int32 planes P = S (1 + has_conj)
 *       48      8  uint64 packed bytes (4 * fairy_packed_words(n, m, P, layout))
 *       56      8  zero
 *       64     8P  float scales [P][2]; zero up to H
 *        H         the packed words, exactly as the kernels read them.
 * Buffers are host memory owned by the caller. */
typedef struct {
    int64_t n, m;
    int32_t stages, has_conj, layout, planes;
    uint64_t packed_bytes;
    uint32_t header_bytes;
} fairy_layer_info;

/* Size of the file of a TILED64 layer (0 for invalid arguments or m % 16 != 0). */
size_t fairy_layer_file_bytes(int64_t n, int64_t m, int32_t stages, int32_t has_conj);

/* Writes the file of layer L (device data) into host buffer `buf` of
 * `bytes` (ERR_WORKSPACE if too small).  Copies on `stream` and waits for it. */
fairy_status fairy_layer_save(const fairy_clinear* L, void* buf, size_t bytes, void* stream);

/* Reads and checks a header: magic, version (other versions: UNSUPPORTED),
 * sizes consistent with each other and with `bytes`.  Host only; touches no
 * device. */
fairy_status fairy_layer_read_info(const void* buf, size_t bytes, fairy_layer_info* info);

/* Copies the scales and packed words of a checked file into device buffers
 * (packed 16-byte aligned, fairy_layer_info.packed_bytes; scales [P][2]);
 * copies on `stream` and waits for it. */
fairy_status fairy_layer_load(const void* buf, size_t bytes, uint32_t* packed, float* scales,
                              void* stream);

/* ---- Complex attention -------------------------------------------------------
 * [iFairy press article §三; Fairy2i article §2.2; iFairy talk §2.1.4]
 *   score(i, j) = scale * Re(sum_t q[i][t] conj(k[j][t]))
 *              (= scale * (q_re . k_re + q_im . k_im), the real dot product of
 *                 the concatenated [re | im] vectors)
 *   w(i, .)    = softmax over the keys j (causal: only j <= i + sk - sq)
 *   o[i][t]    = sum_j w(i, j) v[j][t], real and imaginary parts separately.
 *   q_re, q_im       : device bf16 [heads][sq][d];  k_*, v_* : bf16 [heads][sk][d]
 *   o_re, o_im       : device fp32 [heads][sq][d], overwritten
 *   dtype            : FAIRY_BF16 (others UNSUPPORTED); d in {32, 64, 128}
 *                      (else UNSUPPORTED); all pointers 16-byte aligned
 *   causal           : 0 or 1; causal needs sk >= sq (INVALID_ARG otherwise)
 * One fused pass on the matrix cores (online softmax, nothing of size
 * sq x sk in memory).  Scores are exact fp32 sums of the bf16 products;
 * the weights are carried to ~2^-17 relative precision (each weight's
 * error is at most 2^-17 of it, so o is off by at most 2^-17 of the
 * weighted sum of |v|), and o is within 1e-5 relative L2 of the exact
 * result on the same bf16 inputs for values that do not cancel. */
fairy_status fairy_cattention(const void* q_re, const void* q_im, const void* k_re, const void* k_im,
                              const void* v_re, const void* v_im, int32_t dtype, int32_t heads,
                              int64_t sq, int64_t sk, int32_t d, float scale, int32_t causal,
                              float* o_re, float* o_im, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FAIRY_H */
