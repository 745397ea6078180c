// pn_quant.hip -- weight quantizers on gfx950: the PN reference quantizer and the NVFP4 clip
// search. These write the blocks the GEMVs read; their results are fixed bit for bit by the
// definitions below, so every floating-point step is a single IEEE operation in a fixed order
// (no contraction into fused multiply-adds in this file).
//
// PN: "PN weight format", section "Reference quantizer".
// NVFP4: "Quantisation and profiles", sections "NVFP4" and "The clip search"; NInfer "tensor
// formats" section 3.3 for the E2M1 / E4M3FN words.
#include <algorithm>

#include "pn_common.h"

#pragma clang fp contract(off)

namespace pn {

// ---- binary16 <-> double ---------------------------------------------------------------------

__device__ __forceinline__ double f16_to_f64(uint32_t h)
{
    const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    double v;
    if (e == 0)
        v = (double)m * 0x1p-24;
    else if (e == 31)
        v = m ? __builtin_nan("") : __builtin_inf();
    else
        v = __longlong_as_double((int64_t)((uint64_t)(e - 15 + 1023) << 52 | (uint64_t)m << 42));
    return (h & 0x8000u) ? -v : v;
}

// double -> binary16, round to nearest even on the integer significand, subnormals kept,
// overflow to infinity.
__device__ __forceinline__ uint32_t f64_to_f16(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull)
        return sign | 0x7E00u;  // NaN
    const int e = (int)(a >> 52) - 1023;
    if (e >= 16)
        return sign | 0x7C00u;  // also infinity
    const uint64_t sig = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    if (e >= -14) {
        uint64_t q = sig >> 42;
        const uint64_t rem = sig & ((1ull << 42) - 1), half = 1ull << 41;
        if (rem > half || (rem == half && (q & 1)))
            q++;
        int ee = e;
        if (q == 2048) {
            q = 1024;
            ee++;
        }
        if (ee >= 16)
            return sign | 0x7C00u;
        return sign | (uint32_t)((ee + 15) << 10) | (uint32_t)(q - 1024);
    }
    // subnormal: quantum 2^-24; value = sig * 2^(e - 52), so q = sig >> (28 - e)
    if (a == 0)
        return sign;
    const int shift = 28 - e;  // >= 43
    if (shift > 54)
        return sign;  // below 2^-25: rounds to zero (2^-25 itself is a tie to even zero)
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1)))
        q++;
    return sign | (uint32_t)q;  // q == 1024 is the smallest normal
}

// ---- PN reference quantizer -------------------------------------------------------------------

template <int TYPE>
__global__ void __launch_bounds__(256) pn_quantize_kernel(const float *__restrict__ w,
                                                          int64_t nrows, int nb, int64_t K,
                                                          uint8_t *__restrict__ W,
                                                          int32_t *__restrict__ status)
{
    using F = Fmt<TYPE>;
    constexpr int G = F::G, Z = F::Z, BITS = F::BITS, CPW = F::CPW;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nrows * nb)
        return;
    const int64_t row = q / nb;
    const int b = (int)(q - row * nb);
    const float *wg = w + row * K + (int64_t)b * G;

    double amax = 0.0, mx = -__builtin_inf(), mn = __builtin_inf();
    bool nonfinite = false;
    for (int k = 0; k < G; k++) {
        const double v = (double)wg[k];
        nonfinite |= !__builtin_isfinite(v);
        const double av = __builtin_fabs(v);
        amax = av > amax ? av : amax;
        mx = v > mx ? v : mx;
        mn = v < mn ? v : mn;
    }
    uint8_t best_codes[G];
    uint32_t dbest = 0;
    int st = 0;
    for (int k = 0; k < G; k++)
        best_codes[k] = (uint8_t)Z;
    if (nonfinite) {
        st = 1;
    } else if (amax != 0.0) {
        const double sigma = (__builtin_fabs(mn) > mx) ? 1.0 : -1.0;
        double best = __builtin_inf();
        bool found = false, overflowed = false;
        for (int i = 0; i < 36; i++) {
            const double m = (double)(50 + 2 * i) / 100.0;
            const uint32_t s16 = f64_to_f16(sigma * m * amax / (double)Z);
            const double s = f16_to_f64(s16);
            if (s == 0.0)
                continue;
            if (!__builtin_isfinite(s)) {
                overflowed = true;
                continue;
            }
            double err = 0.0;
            uint8_t trial[G];
            for (int k = 0; k < G; k++) {
                const double wv = (double)wg[k];
                double qv = __builtin_rint(wv / s) + (double)Z;
                qv = qv < 0.0 ? 0.0 : qv;
                qv = qv > (double)(2 * Z - 1) ? (double)(2 * Z - 1) : qv;
                const int n = (int)qv;
                trial[k] = (uint8_t)n;
                const double e = wv - s * (double)(n - Z);
                err += e * e;
            }
            if (err <= best) {
                best = err;
                dbest = s16;
                for (int k = 0; k < G; k++)
                    best_codes[k] = trial[k];
                found = true;
            }
        }
        if (!found) {
            dbest = 0;
            for (int k = 0; k < G; k++)
                best_codes[k] = (uint8_t)Z;
            if (overflowed)
                st = 2;
        }
    }
    // pack: d, then word i holds codes i*CPW + t at BITS*(t>>1) + 16*(t&1)
    uint16_t *out = reinterpret_cast<uint16_t *>(W + row * (int64_t)nb * kBlockBytes +
                                                 (int64_t)b * kBlockBytes);
    out[0] = (uint16_t)dbest;
    for (int i = 0; i < 8; i++) {
        uint32_t word = 0;
        for (int t = 0; t < CPW; t++)
            word |= (uint32_t)best_codes[i * CPW + t] << (BITS * (t >> 1) + 16 * (t & 1));
        out[1 + 2 * i] = (uint16_t)word;
        out[2 + 2 * i] = (uint16_t)(word >> 16);
    }
    if (st && status)
        atomicOr(status + row, st);
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

}  // namespace pn

using namespace pn;

extern "C" {

int pn_quantize_rows(int type, const float *w, int64_t nrows, int64_t K, void *W, int32_t *status,
                     void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (nrows < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (nrows == 0)
        return PN_OK;
    if (!w || !W)
        return PN_ERR_NULL;
    if (!aligned(w, 4) || !aligned(W, 2) || (status && !aligned(status, 4)))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (status) {
        hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, s,
                           status, nrows, 0);
        if ((st = launch_status()) != PN_OK)
            return st;
    }
    const int nb = (int)(K / pn_group(type));
    const int64_t total = nrows * nb;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (type == PN_TYPE_PN3T)
        hipLaunchKernelGGL(pn_quantize_kernel<PN_TYPE_PN3T>, grid, block, 0, s, w, nrows, nb, K,
                           (uint8_t *)W, status);
    else
        hipLaunchKernelGGL(pn_quantize_kernel<PN_TYPE_PN4T>, grid, block, 0, s, w, nrows, nb, K,
                           (uint8_t *)W, status);
    return launch_status();
}

}  // extern "C"
