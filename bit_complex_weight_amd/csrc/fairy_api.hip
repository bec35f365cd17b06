// fairy_api.hip -- the C ABI of libfairy (include/fairy.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime; an invalid call launches nothing and writes nothing.  Errors
// are reported as fairy_status codes, never by exceptions or printing.
#include "fairy_gemv_impl.h"

#include <cmath>

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

fairy_status from_hip(hipError_t e) { return e == hipSuccess ? FAIRY_OK : FAIRY_ERR_HIP; }

// Launch errors are read with hipGetLastError() after each launch.  Another
// component on this thread (for example an event query that returned
// hipErrorNotReady) may have left a stale error behind; drop it once the
// arguments have been validated and just before the first launch.
void clear_stale_error() { (void)hipGetLastError(); }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool valid_layout(int32_t l) { return l == FAIRY_LAYOUT_ROW16 || l == FAIRY_LAYOUT_TILED64; }

bool valid_dtype(int32_t d) { return d == FAIRY_F32 || d == FAIRY_BF16 || d == FAIRY_I8; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Largest m whose staged activations (one batch column, re and im, 64-column
// groups padded by 16 bytes, after the scale prefix) fit in 64 KiB of LDS:
// 7680 (F32), 14528 (BF16), 26112 (I8).
int64_t max_m_for(int32_t xdtype)
{
    const int64_t groups = (64 * 1024 - fairy::gemv::kScaleBytes) / (2 * fairy::gemv::x_group_bytes(xdtype));
    return 64 * groups;
}

// Checks shared by fairy_cgemv and fairy_cgemm.  Returns FAIRY_OK and fills
// the launcher's view of the layer on success.
fairy_status check_layer_call(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype,
                              int64_t rows, int64_t ldx, const float* y_re, const float* y_im, int64_t ldy,
                              const int32_t* acc, fairy::LayerArgs* out, bool staged_x = true)
{
    if (!L || !x_re || !x_im || !y_re || !y_im) return FAIRY_ERR_INVALID_ARG;
    if (L->n < 1 || L->m < 1 || L->n > kMaxDim || L->m > kMaxDim) return FAIRY_ERR_INVALID_ARG;
    if (L->stages < 1 || L->stages > 8) return FAIRY_ERR_INVALID_ARG;
    if (L->has_conj != 0 && L->has_conj != 1) return FAIRY_ERR_INVALID_ARG;
    if (!valid_layout(L->layout)) return FAIRY_ERR_INVALID_ARG;
    if (!L->packed || !L->scales) return FAIRY_ERR_INVALID_ARG;
    if (!valid_dtype(xdtype)) return FAIRY_ERR_INVALID_ARG;
    if (rows < 1) return FAIRY_ERR_INVALID_ARG;
    if (ldx < L->m || ldy < L->n) return FAIRY_ERR_INVALID_ARG;
    if (acc && xdtype != FAIRY_I8) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(L->packed, 16) || !aligned(x_re, 16) || !aligned(x_im, 16) || !aligned(L->scales, 4) ||
        !aligned(y_re, 4) || !aligned(y_im, 4) || (acc && !aligned(acc, 4)))
        return FAIRY_ERR_INVALID_ARG;
    if (ldx % 16 != 0) return FAIRY_ERR_INVALID_ARG;
    if (L->layout != FAIRY_LAYOUT_TILED64) return FAIRY_ERR_UNSUPPORTED;
    if (L->m % 16 != 0) return FAIRY_ERR_UNSUPPORTED;
    if (staged_x && L->m > max_m_for(xdtype)) return FAIRY_ERR_UNSUPPORTED;
    out->packed = L->packed;
    out->scales = L->scales;
    out->n = L->n;
    out->m = L->m;
    out->stages = L->stages;
    out->planes = L->stages * (1 + L->has_conj);
    return FAIRY_OK;
}

}  // namespace

extern "C" {

int32_t fairy_abi_version(void) { return FAIRY_ABI_VERSION; }

const char* fairy_status_string(fairy_status status)
{
    switch (status) {
    case FAIRY_OK: return "FAIRY_OK";
    case FAIRY_ERR_INVALID_ARG: return "FAIRY_ERR_INVALID_ARG: null pointer, bad size, bad enum or misalignment";
    case FAIRY_ERR_UNSUPPORTED: return "FAIRY_ERR_UNSUPPORTED: valid request outside what this version implements";
    case FAIRY_ERR_HIP: return "FAIRY_ERR_HIP: a HIP runtime call or kernel launch failed";
    case FAIRY_ERR_WORKSPACE: return "FAIRY_ERR_WORKSPACE: workspace missing or too small";
    }
    return "FAIRY_ERR_UNKNOWN: not a fairy_status value";
}

fairy_status fairy_real_to_complex(const float* R, int64_t n, int64_t m, float* u_re, float* u_im,
                                   float* w_re, float* w_im, void* stream)
{
    if (!R || !u_re || !u_im || !w_re || !w_im) return FAIRY_ERR_INVALID_ARG;
    if (n < 1 || m < 1 || n > kMaxDim || m > kMaxDim) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(R, 4) || !aligned(u_re, 4) || !aligned(u_im, 4) || !aligned(w_re, 4) || !aligned(w_im, 4))
        return FAIRY_ERR_INVALID_ARG;
    clear_stale_error();
    return from_hip(fairy::launch_real_to_complex(R, n, m, u_re, u_im, w_re, w_im, as_stream(stream)));
}

size_t fairy_phasequant_workspace_bytes(int64_t count, int32_t stages)
{
    if (count < 1 || count >= ((int64_t)1 << 32) || stages < 1 || stages > 8) return 0;
    return fairy::phasequant_workspace_bytes(stages);
}

fairy_status fairy_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                              uint8_t* codes, float* scales, float* resid_re, float* resid_im, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    if (!w_re || !w_im || !codes || !scales) return FAIRY_ERR_INVALID_ARG;
    if (count < 1 || count >= ((int64_t)1 << 32)) return FAIRY_ERR_INVALID_ARG;
    if (stages < 1 || stages > 8) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(w_re, 4) || !aligned(w_im, 4) || !aligned(scales, 4) || (resid_re && !aligned(resid_re, 4)) ||
        (resid_im && !aligned(resid_im, 4)))
        return FAIRY_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < fairy::phasequant_workspace_bytes(stages) || !aligned(workspace, 8))
        return FAIRY_ERR_WORKSPACE;
    clear_stale_error();
    return from_hip(fairy::launch_phasequant(w_re, w_im, count, stages, codes, scales, resid_re, resid_im,
                                             workspace, as_stream(stream)));
}

fairy_status fairy_phasequant_noalloc(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                                      uint8_t* codes, float* scales, float* resid_re, float* resid_im, void* stream)
{
    if (!w_re || !w_im || !codes || !scales) return FAIRY_ERR_INVALID_ARG;
    if (count < 1 || count >= ((int64_t)1 << 32)) return FAIRY_ERR_INVALID_ARG;
    if (stages < 1 || stages > 8) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(w_re, 4) || !aligned(w_im, 4) || !aligned(scales, 4) || (resid_re && !aligned(resid_re, 4)) ||
        (resid_im && !aligned(resid_im, 4)))
        return FAIRY_ERR_INVALID_ARG;
    if (fairy::phasequant_workspace_bytes(stages) > fairy::phasequant_scratch_bytes()) return FAIRY_ERR_UNSUPPORTED;
    clear_stale_error();
    void* ws = nullptr;
    hipError_t e = fairy::phasequant_scratch(&ws);
    if (e != hipSuccess) return FAIRY_ERR_HIP;
    return from_hip(fairy::launch_phasequant(w_re, w_im, count, stages, codes, scales, resid_re, resid_im, ws,
                                             as_stream(stream)));
}

int64_t fairy_packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout)
{
    if (rows < 1 || m < 1 || planes < 1 || planes > 16 || !valid_layout(layout)) return -1;
    if (rows > kMaxDim || m > kMaxDim) return -1;
    if (layout == FAIRY_LAYOUT_ROW16 && m % 16 != 0) return -1;
    return fairy::packed_words(rows, m, planes, layout);
}

static fairy_status check_pack(const void* codes, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                               const void* packed)
{
    if (!codes || !packed) return FAIRY_ERR_INVALID_ARG;
    if (planes < 1 || planes > 16 || rows < 1 || m < 1 || rows > kMaxDim || m > kMaxDim)
        return FAIRY_ERR_INVALID_ARG;
    if (!valid_layout(layout)) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return FAIRY_ERR_INVALID_ARG;
    if (m % 16 != 0) return FAIRY_ERR_UNSUPPORTED;
    return FAIRY_OK;
}

fairy_status fairy_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                        uint32_t* packed, void* stream)
{
    fairy_status st = check_pack(codes, planes, rows, m, layout, packed);
    if (st != FAIRY_OK) return st;
    clear_stale_error();
    return from_hip(fairy::launch_pack(codes, planes, rows, m, layout, packed, as_stream(stream)));
}

fairy_status fairy_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                          uint8_t* codes, void* stream)
{
    fairy_status st = check_pack(codes, planes, rows, m, layout, packed);
    if (st != FAIRY_OK) return st;
    clear_stale_error();
    return from_hip(fairy::launch_unpack(packed, planes, rows, m, layout, codes, as_stream(stream)));
}

size_t fairy_cgemv_workspace_bytes(const fairy_clinear* L, int32_t batch, int32_t xdtype)
{
    (void)L;
    (void)batch;
    (void)xdtype;
    return 0;
}

fairy_status fairy_cgemv(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype,
                         int32_t batch, int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (batch < 1 || batch > 64) return FAIRY_ERR_INVALID_ARG;
    fairy::LayerArgs la;
    fairy_status st = check_layer_call(L, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, acc, &la);
    if (st != FAIRY_OK) return st;
    clear_stale_error();
    return from_hip(fairy::launch_cgemv(la, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, acc, as_stream(stream)));
}

fairy_status fairy_cgemv_group(const fairy_clinear* layers, int32_t count, const void* x_re, const void* x_im,
                               int32_t xdtype, int32_t batch, int64_t ldx, float* const* y_re, float* const* y_im,
                               const int64_t* ldy, void* stream)
{
    if (!layers || !y_re || !y_im || !ldy) return FAIRY_ERR_INVALID_ARG;
    if (count < 1 || count > fairy::gemv::kMaxGroup) return FAIRY_ERR_INVALID_ARG;
    if (batch < 1 || batch > 64) return FAIRY_ERR_INVALID_ARG;
    fairy::LayerArgs la[fairy::gemv::kMaxGroup];
    for (int32_t l = 0; l < count; ++l) {
        fairy_status st = check_layer_call(&layers[l], x_re, x_im, xdtype, batch, ldx, y_re[l], y_im[l], ldy[l],
                                           nullptr, &la[l]);
        if (st != FAIRY_OK) return st;
        if (layers[l].m != layers[0].m || layers[l].stages != layers[0].stages ||
            layers[l].has_conj != layers[0].has_conj)
            return FAIRY_ERR_INVALID_ARG;
    }
    clear_stale_error();
    return from_hip(fairy::launch_cgemv_group(la, y_re, y_im, ldy, count, x_re, x_im, xdtype, batch, ldx,
                                              as_stream(stream)));
}

// Layer view and block shape of a table-lookup GEMV call; false when the
// layer is invalid or its chunk grid exceeds the launch limits.
static bool lut_plan(const fairy_clinear* L, fairy::LayerArgs* la, fairy::LutConfig* c)
{
    if (!L || L->n < 1 || L->m < 1 || L->n > kMaxDim || L->m > kMaxDim) return false;
    if (L->stages < 1 || L->stages > 8 || (L->has_conj != 0 && L->has_conj != 1)) return false;
    la->packed = L->packed;
    la->scales = L->scales;
    la->n = L->n;
    la->m = L->m;
    la->stages = L->stages;
    la->planes = L->stages * (1 + L->has_conj);
    *c = fairy::cgemv_lut_config(*la);
    const int64_t units = ((L->m + 63) / 64) * (int64_t)la->planes;
    return (units + c->JB - 1) / c->JB <= 65535;
}

size_t fairy_cgemv_lut_workspace_bytes(const fairy_clinear* L)
{
    fairy::LayerArgs la;
    fairy::LutConfig c;
    if (!lut_plan(L, &la, &c)) return 0;
    return fairy::cgemv_lut_workspace_bytes(la, c);
}

fairy_status fairy_cgemv_lut(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype,
                             float* y_re, float* y_im, void* workspace, size_t workspace_bytes, void* stream)
{
    fairy::LayerArgs la;
    fairy_status st = check_layer_call(L, x_re, x_im, xdtype, 1, L ? (L->m + 15) / 16 * 16 : 0, y_re, y_im, L ? L->n : 0,
                                       nullptr, &la, false);
    if (st != FAIRY_OK) return st;
    if (xdtype != FAIRY_BF16 && xdtype != FAIRY_F32) return FAIRY_ERR_UNSUPPORTED;
    fairy::LutConfig c;
    if (!lut_plan(L, &la, &c)) return FAIRY_ERR_UNSUPPORTED;
    const size_t need = fairy::cgemv_lut_workspace_bytes(la, c);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return FAIRY_ERR_WORKSPACE;
    clear_stale_error();
    return from_hip(fairy::launch_cgemv_lut(la, c, x_re, x_im, xdtype, y_re, y_im, workspace, as_stream(stream)));
}

size_t fairy_cgemm_workspace_bytes(const fairy_clinear* L, int64_t M, int32_t xdtype, int32_t algo)
{
    fairy::LayerArgs la;
    if (!L || M < 1) return 0;
    la.packed = L->packed;
    la.scales = L->scales;
    la.n = L->n;
    la.m = L->m;
    la.stages = L->stages;
    la.planes = L->stages * (1 + (L->has_conj ? 1 : 0));
    return fairy::cgemm_workspace_bytes(la, M, xdtype, algo);
}

fairy_status fairy_cgemm(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype, int64_t M,
                         int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc, int32_t algo,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 1 || M > kMaxDim) return FAIRY_ERR_INVALID_ARG;
    if (algo != FAIRY_ALGO_AUTO && algo != FAIRY_ALGO_VALU && algo != FAIRY_ALGO_MFMA) return FAIRY_ERR_INVALID_ARG;
    fairy::LayerArgs la;
    fairy_status st = check_layer_call(L, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, acc, &la, false);
    if (st != FAIRY_OK) return st;
    if (algo == FAIRY_ALGO_MFMA && xdtype == FAIRY_F32) return FAIRY_ERR_UNSUPPORTED;
    if (!fairy::cgemm_uses_mfma(M, xdtype, algo) && L->m > max_m_for(xdtype)) return FAIRY_ERR_UNSUPPORTED;
    // the workspace is optional: without one the call runs unsplit
    const size_t need = fairy::cgemm_workspace_bytes(la, M, xdtype, algo);
    if (workspace && need && (workspace_bytes < need || !aligned(workspace, 16))) return FAIRY_ERR_WORKSPACE;
    clear_stale_error();
    hipError_t e = fairy::launch_cgemm(la, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, acc, algo,
                                       need ? workspace : nullptr, as_stream(stream));
    if (e == hipErrorNotSupported) return FAIRY_ERR_UNSUPPORTED;
    return from_hip(e);
}

// Rotary position arguments: positions device int32 [rows], 4-byte aligned;
// head_dim >= 1; base finite and > 0.
static fairy_status check_rope(const int32_t* positions, int32_t head_dim, float base, fairy::LayerArgs* la)
{
    if (!positions || !aligned(positions, 4) || head_dim < 1) return FAIRY_ERR_INVALID_ARG;
    if (!(base > 0.0f) || base > 3.0e38f) return FAIRY_ERR_INVALID_ARG;
    la->rope_pos = positions;
    la->rope_d = head_dim;
    la->rope_log2_base = std::log2((double)base);
    return FAIRY_OK;
}

fairy_status fairy_cgemv_rope(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype,
                              int32_t batch, int64_t ldx, float* y_re, float* y_im, int64_t ldy,
                              const int32_t* positions, int32_t head_dim, float base, void* stream)
{
    if (batch < 1 || batch > 64) return FAIRY_ERR_INVALID_ARG;
    fairy::LayerArgs la;
    fairy_status st = check_layer_call(L, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, nullptr, &la);
    if (st != FAIRY_OK) return st;
    if ((st = check_rope(positions, head_dim, base, &la)) != FAIRY_OK) return st;
    clear_stale_error();
    return from_hip(fairy::launch_cgemv(la, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, nullptr,
                                        as_stream(stream)));
}

fairy_status fairy_cgemm_rope(const fairy_clinear* L, const void* x_re, const void* x_im, int32_t xdtype,
                              int64_t M, int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t algo,
                              const int32_t* positions, int32_t head_dim, float base, void* stream)
{
    if (M < 1 || M > kMaxDim) return FAIRY_ERR_INVALID_ARG;
    if (algo != FAIRY_ALGO_AUTO && algo != FAIRY_ALGO_VALU && algo != FAIRY_ALGO_MFMA) return FAIRY_ERR_INVALID_ARG;
    fairy::LayerArgs la;
    fairy_status st = check_layer_call(L, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, nullptr, &la, false);
    if (st != FAIRY_OK) return st;
    if (algo == FAIRY_ALGO_MFMA && xdtype == FAIRY_F32) return FAIRY_ERR_UNSUPPORTED;
    if (!fairy::cgemm_uses_mfma(M, xdtype, algo) && L->m > max_m_for(xdtype)) return FAIRY_ERR_UNSUPPORTED;
    if ((st = check_rope(positions, head_dim, base, &la)) != FAIRY_OK) return st;
    clear_stale_error();
    hipError_t e = fairy::launch_cgemm(la, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, nullptr, algo, nullptr,
                                       as_stream(stream));
    if (e == hipErrorNotSupported) return FAIRY_ERR_UNSUPPORTED;
    return from_hip(e);
}

fairy_status fairy_cattention(const void* q_re, const void* q_im, const void* k_re, const void* k_im,
                              const void* v_re, const void* v_im, int32_t dtype, int32_t heads, int64_t sq,
                              int64_t sk, int32_t d, float scale, int32_t causal, float* o_re, float* o_im,
                              void* stream)
{
    const void* ptrs[8] = {q_re, q_im, k_re, k_im, v_re, v_im, o_re, o_im};
    for (const void* p : ptrs)
        if (!p || !aligned(p, 16)) return FAIRY_ERR_INVALID_ARG;
    if (heads < 1 || heads > 65535 || sq < 1 || sk < 1 || sq > kMaxDim || sk > kMaxDim) return FAIRY_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FAIRY_ERR_INVALID_ARG;
    if (causal && sk < sq) return FAIRY_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return FAIRY_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return FAIRY_ERR_INVALID_ARG;
    if (dtype != FAIRY_BF16) return FAIRY_ERR_UNSUPPORTED;
    if (d != 32 && d != 64 && d != 128) return FAIRY_ERR_UNSUPPORTED;
    clear_stale_error();
    return from_hip(fairy::launch_cattention(q_re, q_im, k_re, k_im, v_re, v_im, heads, sq, sk, d, scale, causal,
                                             o_re, o_im, as_stream(stream)));
}

}  // extern "C"
