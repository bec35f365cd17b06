// fairy_internal.h -- shared declarations of the HIP library (not installed).
//
// Device helpers common to the kernels: the 2-bit code decode and the
// cross-lane (DPP / row-swap) reductions.  Host launchers are declared at
// the bottom; fairy_api.hip validates arguments and calls them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fairy.h"

namespace fairy {

// ---------------------------------------------------------------------------
// Code decode
// ---------------------------------------------------------------------------
// A code c = 2*s + a holds the sign s of its codeword i^c and its axis a
// (0 = real, 1 = imaginary).  [Fairy2i article §3.1; iFairy abstract: every
// codeword has exactly one non-zero axis.]
//
// TILED64 words store column t of a 16-column word at bit (t even ? 14-t : 31-t),
// so after `w << 2k` the codes of columns 2k (low half) and 2k+1 (high half)
// occupy bits 15:14 and 31:30.  Read as a bfloat16 pair, masking with
// 0xC000C000 leaves the sign bit and the top exponent bit: the value is
// +-2 when that exponent bit is set and +-0 otherwise.  Hence
//   ImB pair (x2) = ws & 0xC000C000                  (axis bit set  -> +-2)
//   ReB pair (x2) = (ws ^ 0x40004000) & 0xC000C000   (axis bit clear -> +-2)
// Two bit operations per two codes and no multiplies; the factor 2 is
// removed once in the epilogue.
__device__ __forceinline__ void decode_bf16_pair(uint32_t w, int k, uint32_t& re2, uint32_t& im2)
{
    const uint32_t ws = w << (2 * k);
    im2 = ws & 0xC000C000u;
    re2 = (ws ^ 0x40004000u) & 0xC000C000u;
}

// Column t of a TILED64 word -> the shift that moves its code to bits 31:30,
// where, read as fp32, the same masks give +-2 / +-0.
__device__ __forceinline__ int f32_shift(int t) { return (t & 1) ? (t - 1) : (16 + t); }

// int8 ternary planes for dot4: the four columns whose codes share bit offset
// 2s inside each byte of a word are, by byte b = 0..3,
//   t = 14-2s, 6-2s, 15-2s, 7-2s.
// v_perm turns four 2-bit selectors into four {-1,0,1} bytes.
__device__ __forceinline__ int i8_group_col(int s, int b)
{
    return (b == 0) ? 14 - 2 * s : (b == 1) ? 6 - 2 * s : (b == 2) ? 15 - 2 * s : 7 - 2 * s;
}

// ---------------------------------------------------------------------------
// Cross-lane sums over aligned groups of W lanes (W = 2..64), result in every
// lane of the group, all in VALU instructions (no LDS round trips):
//   distance 1, 2: DPP quad_perm (xor 1, xor 2);
//   8-lane halves: DPP row_half_mirror (lane i <-> 7 - i: after the quad
//     steps every lane of a quad holds the quad's sum, so this adds the
//     other quad of the half);
//   16-lane rows: DPP row_mirror (lane i <-> 15 - i, the other half);
//   32 and 64: v_permlane16_swap / v_permlane32_swap (rows 0 <-> 1 and
//     2 <-> 3; the two halves of the wave).
// At every step the two lanes of a pair add the same two values (in either
// order: addition is commutative), so all lanes of a group hold
// bit-identical results.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_half_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); }

// x + (the value of the lane 16 or 32 away), identical in both lanes
__device__ __forceinline__ float swap16_add(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_add(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int swap16_add(int v)
{
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(r[0] + r[1]);
}
__device__ __forceinline__ int swap32_add(int v)
{
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(r[0] + r[1]);
}

template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    v += __int_as_float(dpp_xor1(__float_as_int(v)));
    if (W >= 4) v += __int_as_float(dpp_xor2(__float_as_int(v)));
    if (W >= 8) v += __int_as_float(dpp_half_mirror(__float_as_int(v)));
    if (W >= 16) v += __int_as_float(dpp_mirror(__float_as_int(v)));
    if (W >= 32) v = swap16_add(v);
    if (W >= 64) v = swap32_add(v);
    return v;
}

template <int W>
__device__ __forceinline__ int group_sum_i(int v)
{
    v += dpp_xor1(v);
    if (W >= 4) v += dpp_xor2(v);
    if (W >= 8) v += dpp_half_mirror(v);
    if (W >= 16) v += dpp_mirror(v);
    if (W >= 32) v = swap16_add(v);
    if (W >= 64) v = swap32_add(v);
    return v;
}

// ---------------------------------------------------------------------------
// Host launchers (arguments already validated)
// ---------------------------------------------------------------------------
hipError_t launch_real_to_complex(const float* R, int64_t n, int64_t m, float* u_re, float* u_im,
                                  float* w_re, float* w_im, hipStream_t s);

size_t phasequant_workspace_bytes(int32_t stages);
hipError_t launch_phasequant(const float* w_re, const float* w_im, int64_t count, int32_t stages,
                             uint8_t* codes, float* scales, float* resid_re, float* resid_im,
                             void* workspace, hipStream_t s);

// PhaseQuant of both matrices of a real layer R [2n][2m], U and W formed
// inside the stage kernels (no planes in memory): codes [2S][n*m] (U_1..U_S,
// W_1..W_S), scales [2S][2] in the same order; bit-identical to the
// conversion followed by launch_phasequant on U and on W.
size_t phasequant_real_workspace_bytes(int32_t stages);
hipError_t launch_phasequant_real(const float* R, int64_t n, int64_t m, int32_t stages, uint8_t* codes,
                                  float* scales, void* workspace, hipStream_t s);

// Device address (current device) and size of the static PhaseQuant bucket
// array used by fairy_phasequant_noalloc.
hipError_t phasequant_scratch(void** out);
size_t phasequant_scratch_bytes();

int64_t packed_words(int64_t rows, int64_t m, int32_t planes, int32_t layout);
hipError_t launch_pack(const uint8_t* codes, int32_t planes, int64_t rows, int64_t m, int32_t layout,
                       uint32_t* packed, hipStream_t s);
hipError_t launch_unpack(const uint32_t* packed, int32_t planes, int64_t rows, int64_t m,
                         int32_t layout, uint8_t* codes, hipStream_t s);

struct LayerArgs {
    const uint32_t* packed;
    const float* scales;
    int64_t n, m;
    int32_t stages, planes;
    // optional rotary position encoding of the outputs (rope_pos == nullptr: none)
    const int32_t* rope_pos = nullptr;
    int32_t rope_d = 1;
    double rope_log2_base = 0.0;
};

hipError_t launch_cgemv(const LayerArgs& L, const void* x_re, const void* x_im, int32_t xdtype,
                        int64_t batch, int64_t ldx, float* y_re, float* y_im, int64_t ldy,
                        int32_t* acc, hipStream_t s);

// Decode GEMV of up to 8 layers (same m, stages and conjugate branch) that
// read the same activations: one launch when the shape allows, else one per
// layer.  No raw accumulators, no rotary encoding.
hipError_t launch_cgemv_group(const LayerArgs* L, const float* const* y_re, const float* const* y_im,
                              const int64_t* ldy, int32_t count, const void* x_re, const void* x_im, int32_t xdtype,
                              int64_t batch, int64_t ldx, hipStream_t s);

// Whether fairy_cgemm takes the matrix-core path for these arguments (it
// streams the activations in chunks, so any m; the VALU path stages whole
// activation rows in LDS).
bool cgemm_uses_mfma(int64_t M, int32_t xdtype, int32_t algo);
size_t cgemm_workspace_bytes(const LayerArgs& L, int64_t M, int32_t xdtype, int32_t algo);
hipError_t launch_cgemm(const LayerArgs& L, const void* x_re, const void* x_im, int32_t xdtype,
                        int64_t M, int64_t ldx, float* y_re, float* y_im, int64_t ldy, int32_t* acc,
                        int32_t algo, void* workspace, hipStream_t s);

// table-lookup GEMV, batch 1 (fairy_gemv_lut.hip): W waves of rows and JB
// 16-byte units per block
struct LutConfig {
    int W, JB;
};
LutConfig cgemv_lut_config(const LayerArgs& L);
size_t cgemv_lut_workspace_bytes(const LayerArgs& L, const LutConfig& c);
hipError_t launch_cgemv_lut(const LayerArgs& L, const LutConfig& c, const void* x_re, const void* x_im,
                            int32_t xdtype, float* y_re, float* y_im, void* workspace, hipStream_t s);

// complex attention forward (fairy_attention.hip); bf16 inputs, d in {32, 64, 128}
hipError_t launch_cattention(const void* q_re, const void* q_im, const void* k_re, const void* k_im,
                             const void* v_re, const void* v_im, int32_t heads, int64_t sq, int64_t sk, int32_t d,
                             float scale, int32_t causal, float* o_re, float* o_im, hipStream_t s);

}  // namespace fairy
