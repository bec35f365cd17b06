// fairy_gemm.hip -- prefill complex GEMM on gfx950.
//
// The prefill layer is the decode layer applied to M token rows at once
// [Fairy2i article §4.2]; at M in the thousands it is a dense contraction.
#include "fairy_gemv_impl.h"

namespace fairy {

// token count from which the VALU path maps lanes to tokens
constexpr int64_t kValuTokensMin = 64;

// AUTO: the matrix cores from 16 tokens (measured without a workspace: at
// M = 16 they beat the VALU kernels on the 2048x2048, 5504x2048 and
// 2048x5504 S=2 layers, at M = 8 they lose on two of the three)
bool cgemm_uses_mfma(int64_t M, int32_t xdtype, int32_t algo)
{
    const bool mfma_ok = xdtype == FAIRY_BF16 || xdtype == FAIRY_I8;
    return (algo == FAIRY_ALGO_MFMA) || (algo == FAIRY_ALGO_AUTO && mfma_ok && M >= 16);
}

// The matrix-core path at token counts that leave CUs idle splits K and
// keeps the partial sums here; every other path needs none.
size_t cgemm_workspace_bytes(const LayerArgs& L, int64_t M, int32_t xdtype, int32_t algo)
{
    if (!cgemm_uses_mfma(M, xdtype, algo) || (xdtype != FAIRY_BF16 && xdtype != FAIRY_I8)) return 0;
    return cgemm_mfma_workspace_bytes(L.n, L.m, M, L.planes, xdtype);
}

hipError_t launch_cgemm(const LayerArgs& L, const void* x_re, const void* x_im, int32_t xdtype, int64_t M,
                        int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc, int32_t algo,
                        void* workspace, hipStream_t s)
{
    if (cgemm_uses_mfma(M, xdtype, algo)) {
        if (xdtype != FAIRY_BF16 && xdtype != FAIRY_I8) return hipErrorNotSupported;
        const gemv::GemvArgs a = gemv::make_args(L, x_re, x_im, M, ldx, y_re, y_im, ldy, acc);
        return launch_cgemm_mfma(a, xdtype, workspace, s);
    }
    // VALU path.  From a wave's worth of tokens: lanes are tokens, the code
    // words are decoded once per wave on the scalar unit.  Otherwise (and
    // for fp32 activations) the decode kernel streams the token rows
    // through LDS in chunks, re-reading the (L2-resident) codes per chunk.
    if (M >= kValuTokensMin && cgemm_valu_tokens_supported(xdtype, L.m, L.planes)) {
        const gemv::GemvArgs a = gemv::make_args(L, x_re, x_im, M, ldx, y_re, y_im, ldy, acc);
        return launch_cgemm_valu(a, xdtype, s);
    }
    return launch_cgemv(L, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, acc, s);
}

}  // namespace fairy
