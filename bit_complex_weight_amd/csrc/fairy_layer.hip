// fairy_layer.hip -- whole-layer conversion on the device and the serialised
// quantised-layer format (include/fairy.h).
//
// Conversion chains the steps of the path in the pages' order [Fairy2i
// article §2.1, §3.1-§3.2, §4.1]: widely-linear split of a real matrix,
// PhaseQuant of U and of W with S recursive residual stages each, and packing
// into TILED64; every intermediate lives in the caller's workspace and
// nothing touches the host.  The file format is this library's own (the
// pages name none; their deployment notes only ask that the device support
// the complex storage format and keep real and imaginary parts apart): a
// fixed little-endian header, the scales, then the packed words exactly as
// the kernels read them.
#include "fairy_internal.h"

#include <cstring>

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
fairy_status from_hip(hipError_t e) { return e == hipSuccess ? FAIRY_OK : FAIRY_ERR_HIP; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace carve-up for a conversion: [codes P x n x m] [PhaseQuant
// buckets: one matrix's for complex input, U's and W's for real input, whose
// U and W are formed inside the PhaseQuant stages], each 256-byte aligned.
struct Carve {
    size_t codes, pq, total;
};

bool carve(int64_t n, int64_t m, int32_t stages, int32_t has_conj, Carve* c)
{
    if (n < 1 || m < 1 || n > kMaxDim || m > kMaxDim || stages < 1 || stages > 8) return false;
    if (has_conj != 0 && has_conj != 1) return false;
    if (n * m >= ((int64_t)1 << 32)) return false;  // PhaseQuant element count
    const size_t count = (size_t)(n * m);
    const int32_t P = stages * (1 + has_conj);
    c->codes = round_up((size_t)P * count, kAlign);
    c->pq = round_up(has_conj ? fairy::phasequant_real_workspace_bytes(stages) : fairy::phasequant_workspace_bytes(stages),
                     kAlign);
    c->total = c->codes + c->pq;
    return true;
}

// ---- file format ----------------------------------------------------------
constexpr char kMagic[8] = {'F', 'A', 'I', 'R', 'Y', 'Q', 'L', '1'};
constexpr uint32_t kFormatVersion = 1;
constexpr size_t kFixedHeader = 64;

size_t header_bytes(int32_t planes) { return round_up(kFixedHeader + 8 * (size_t)planes, 64); }

template <typename T>
void put(uint8_t* base, size_t off, T v)
{
    std::memcpy(base + off, &v, sizeof(T));
}
template <typename T>
T get(const uint8_t* base, size_t off)
{
    T v;
    std::memcpy(&v, base + off, sizeof(T));
    return v;
}

}  // namespace

extern "C" {

size_t fairy_quantize_workspace_bytes(int64_t n, int64_t m, int32_t stages, int32_t has_conj)
{
    Carve c;
    return carve(n, m, stages, has_conj, &c) ? c.total : 0;
}

static fairy_status quantize(const float* R, const float* w_re, const float* w_im, int64_t n, int64_t m,
                             int32_t stages, int32_t has_conj, uint32_t* packed, float* scales, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    Carve c;
    if (!carve(n, m, stages, has_conj, &c)) return FAIRY_ERR_INVALID_ARG;
    if (!packed || !scales) return FAIRY_ERR_INVALID_ARG;
    if (!aligned(packed, 16) || !aligned(scales, 4)) return FAIRY_ERR_INVALID_ARG;
    if (m % 16 != 0) return FAIRY_ERR_UNSUPPORTED;
    if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < c.total) return FAIRY_ERR_WORKSPACE;
    const hipStream_t s = as_stream(stream);
    const int64_t count = n * m;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* codes = ws;
    void* pq = ws + c.codes;
    (void)hipGetLastError();
    hipError_t e = hipSuccess;
    if (has_conj) {
        // planes U_1..U_S, then W_1..W_S; scales follow the same order
        if ((e = fairy::launch_phasequant_real(R, n, m, stages, codes, scales, pq, s)) != hipSuccess)
            return from_hip(e);
    } else {
        if ((e = fairy::launch_phasequant(w_re, w_im, count, stages, codes, scales, nullptr, nullptr, pq, s)) !=
            hipSuccess)
            return from_hip(e);
    }
    const int32_t P = stages * (1 + has_conj);
    return from_hip(fairy::launch_pack(codes, P, n, m, FAIRY_LAYOUT_TILED64, packed, s));
}

fairy_status fairy_quantize_real(const float* R, int64_t n, int64_t m, int32_t stages, uint32_t* packed,
                                 float* scales, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!R || !aligned(R, 4)) return FAIRY_ERR_INVALID_ARG;
    return quantize(R, nullptr, nullptr, n, m, stages, 1, packed, scales, workspace, workspace_bytes, stream);
}

fairy_status fairy_quantize_complex(const float* w_re, const float* w_im, int64_t n, int64_t m, int32_t stages,
                                    uint32_t* packed, float* scales, void* workspace, size_t workspace_bytes,
                                    void* stream)
{
    if (!w_re || !w_im || !aligned(w_re, 4) || !aligned(w_im, 4)) return FAIRY_ERR_INVALID_ARG;
    return quantize(nullptr, w_re, w_im, n, m, stages, 0, packed, scales, workspace, workspace_bytes, stream);
}

size_t fairy_layer_file_bytes(int64_t n, int64_t m, int32_t stages, int32_t has_conj)
{
    if (n < 1 || m < 1 || n > kMaxDim || m > kMaxDim || stages < 1 || stages > 8) return 0;
    if ((has_conj != 0 && has_conj != 1) || m % 16 != 0) return 0;
    const int32_t P = stages * (1 + has_conj);
    return header_bytes(P) + 4 * (size_t)fairy::packed_words(n, m, P, FAIRY_LAYOUT_TILED64);
}

fairy_status fairy_layer_save(const fairy_clinear* L, void* buf, size_t bytes, void* stream)
{
    if (!L || !buf || !L->packed || !L->scales) return FAIRY_ERR_INVALID_ARG;
    if (L->layout != FAIRY_LAYOUT_TILED64) return FAIRY_ERR_UNSUPPORTED;
    const size_t total = fairy_layer_file_bytes(L->n, L->m, L->stages, L->has_conj);
    if (total == 0) return FAIRY_ERR_INVALID_ARG;
    if (bytes < total) return FAIRY_ERR_WORKSPACE;
    const int32_t P = L->stages * (1 + L->has_conj);
    const size_t hb = header_bytes(P);
    const size_t packed_bytes = total - hb;
    uint8_t* b = static_cast<uint8_t*>(buf);
    std::memset(b, 0, hb);
    std::memcpy(b, kMagic, 8);
    put<uint32_t>(b, 8, kFormatVersion);
    put<uint32_t>(b, 12, (uint32_t)hb);
    put<int64_t>(b, 16, L->n);
    put<int64_t>(b, 24, L->m);
    put<int32_t>(b, 32, L->stages);
    put<int32_t>(b, 36, L->has_conj);
    put<int32_t>(b, 40, L->layout);
    put<int32_t>(b, 44, P);
    put<uint64_t>(b, 48, (uint64_t)packed_bytes);
    const hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    hipError_t e = hipMemcpyAsync(b + kFixedHeader, L->scales, 8 * (size_t)P, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(b + hb, L->packed, packed_bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return from_hip(e);
}

fairy_status fairy_layer_read_info(const void* buf, size_t bytes, fairy_layer_info* info)
{
    if (!buf || !info) return FAIRY_ERR_INVALID_ARG;
    if (bytes < kFixedHeader) return FAIRY_ERR_INVALID_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(buf);
    if (std::memcmp(b, kMagic, 8) != 0) return FAIRY_ERR_INVALID_ARG;
    if (get<uint32_t>(b, 8) != kFormatVersion) return FAIRY_ERR_UNSUPPORTED;
    fairy_layer_info v;
    v.n = get<int64_t>(b, 16);
    v.m = get<int64_t>(b, 24);
    v.stages = get<int32_t>(b, 32);
    v.has_conj = get<int32_t>(b, 36);
    v.layout = get<int32_t>(b, 40);
    v.planes = get<int32_t>(b, 44);
    v.packed_bytes = get<uint64_t>(b, 48);
    const uint32_t hb = get<uint32_t>(b, 12);
    if (v.layout != FAIRY_LAYOUT_TILED64) return FAIRY_ERR_UNSUPPORTED;
    const size_t total = fairy_layer_file_bytes(v.n, v.m, v.stages, v.has_conj);
    if (total == 0 || v.planes != v.stages * (1 + v.has_conj) || hb != header_bytes(v.planes) ||
        v.packed_bytes != total - hb)
        return FAIRY_ERR_INVALID_ARG;
    if (bytes < total) return FAIRY_ERR_INVALID_ARG;
    v.header_bytes = hb;
    *info = v;
    return FAIRY_OK;
}

fairy_status fairy_layer_load(const void* buf, size_t bytes, uint32_t* packed, float* scales, void* stream)
{
    fairy_layer_info v;
    fairy_status st = fairy_layer_read_info(buf, bytes, &v);
    if (st != FAIRY_OK) return st;
    if (!packed || !scales || !aligned(packed, 16) || !aligned(scales, 4)) return FAIRY_ERR_INVALID_ARG;
    const uint8_t* b = static_cast<const uint8_t*>(buf);
    const hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    hipError_t e = hipMemcpyAsync(scales, b + kFixedHeader, 8 * (size_t)v.planes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(packed, b + v.header_bytes, v.packed_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return from_hip(e);
}

}  // extern "C"
