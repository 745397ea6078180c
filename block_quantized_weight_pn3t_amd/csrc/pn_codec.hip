// pn_codec.hip -- PN and NVFP4 row validation and bit-exact decode on gfx950, plus the host
// helpers shared by every entry point of libpn.so.
//
// PN: "PN weight format", sections "Block layout", "Value", "Validation".
// NVFP4: "Quantisation and profiles", section "NVFP4"; NInfer "tensor formats" section 3.3.
#include <string.h>

#include <atomic>

#include "pn_common.h"

namespace pn {

// Per-device facts, looked up once per device and kept for the process (atomics: entry points
// may be called from several host threads, on different devices).
constexpr int kMaxDevices = 64;
static std::atomic<int> g_dev_status[kMaxDevices];  // 0 unknown, else status + 1000
static std::atomic<int> g_dev_cus[kMaxDevices];     // 0 unknown

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return PN_ERR_HIP;
    if (dev < kMaxDevices) {
        const int c = g_dev_status[dev].load(std::memory_order_relaxed);
        if (c != 0)
            return c - 1000;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return PN_ERR_HIP;
    const int st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? PN_OK : PN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        g_dev_status[dev].store(st + 1000, std::memory_order_relaxed);
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    }
    return st;
}

int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        const int c = g_dev_cus[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0) {
            g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
            return prop.multiProcessorCount;
        }
    }
    return 256;  // MI355X; entry points have passed check_device() before they size a grid
}

int launch_status()
{
    return hipGetLastError() == hipSuccess ? PN_OK : PN_ERR_HIP;
}

// ---- PN validation ------------------------------------------------------------------------------
// One wave per row; lane l checks blocks l, l+64, ... . A row is invalid when some block's d has an
// all-ones exponent (fp16 NaN or infinity) or, for pn3t, some word has bit 15 or bit 31 set.
template <int TYPE>
__global__ void __launch_bounds__(256) validate_kernel(const uint8_t *__restrict__ W, int64_t nrows,
                                                      int nb, int64_t row_bytes,
                                                      int32_t *__restrict__ verdict)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= nrows)
        return;
    const uint8_t *base = W + row * row_bytes;
    bool bad = false;
    for (int b = lane; b < nb; b += 64) {
        RawBlock rb;
        load_block(base + (int64_t)kBlockBytes * b, rb);
        bad |= (block_d_bits(rb) & 0x7C00u) == 0x7C00u;
        if (TYPE == PN_TYPE_PN3T) {
            uint32_t any = 0;
#pragma unroll
            for (int i = 0; i < 8; i++)
                any |= block_word(rb, i);
            bad |= (any & 0x80008000u) != 0;
        }
    }
    const bool row_bad = __any(bad);
    if (lane == 0)
        verdict[row] = row_bad ? 0 : 1;
}

// ---- PN decode -----------------------------------------------------------------------------------
// One thread per u32 word: decodes the word's 10 (pn3t) or 8 (pn4t) codes as fp32(d) * (n - z),
// a single IEEE multiply (exact: d has 11 significant bits and n - z at most 4).
template <int TYPE>
__global__ void __launch_bounds__(256) dequantize_kernel(const uint8_t *__restrict__ W,
                                                         int64_t nrows, int nb, int64_t row_bytes,
                                                         float *__restrict__ out)
{
    using F = Fmt<TYPE>;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t words_per_row = (int64_t)nb * 8;
    if (q >= nrows * words_per_row)
        return;
    const int64_t row = q / words_per_row;
    const int rem = (int)(q - row * words_per_row);
    const int b = rem >> 3, i = rem & 7;
    const uint8_t *blk = W + row * row_bytes + (int64_t)kBlockBytes * b;
    // 2-byte loads only: the word sits at a 2-byte aligned address
    const uint16_t *h = reinterpret_cast<const uint16_t *>(blk);
    const float d = f16_bits_to_f32(h[0]);
    const uint32_t word = (uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16);
    float *o = out + row * (int64_t)nb * F::G + (int64_t)b * F::G + i * F::CPW;
#pragma unroll
    for (int t = 0; t < F::CPW; t++) {
        const int shift = F::BITS * (t >> 1) + 16 * (t & 1);
        const int n = (int)((word >> shift) & ((1u << F::BITS) - 1));
        o[t] = d * (float)(n - F::Z);
    }
}

// ---- NVFP4 validation and decode ------------------------------------------------------------------

__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    // E4M3FN: sign bit 7, exponent bits 6:3 (bias 7), fraction bits 2:0; e = 0 is m * 2^-9;
    // e = 15, m = 7 is NaN. Built from bits: normal values are re-biased into binary32.
    const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, m = c & 7u;
    float v;
    if (e == 0)
        v = (float)m * 0x1p-9f;
    else if (e == 15 && m == 7)
        v = __builtin_nanf("");
    else
        v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | s);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c)
{
    // E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 for words 0..7; bit 3 is the sign.
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const uint32_t bits = (e == 0) ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
    return __builtin_bit_cast(float, bits | ((c & 8u) << 28));
}

__global__ void __launch_bounds__(256) nvfp4_validate_kernel(const uint8_t *__restrict__ scales,
                                                             int gok, int64_t N, int groups,
                                                             int32_t *__restrict__ verdict)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= N)
        return;
    bool bad = false;
    for (int j = lane; j < groups; j += 64) {
        const uint32_t s = scales[row * groups + j];
        bad |= (s & 0x80u) != 0 || s == 0x7Fu;
    }
    const bool row_bad = __any(bad);
    if (lane == 0)
        verdict[row] = (gok && !row_bad) ? 1 : 0;
}

// One thread per code byte (two weights).
__global__ void __launch_bounds__(256) nvfp4_dequantize_kernel(const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales,
                                                               float g, int64_t N, int64_t K,
                                                               float *__restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t half_k = K >> 1;
    if (q >= N * half_k)
        return;
    const int64_t row = q / half_k;
    const int64_t kk = (q - row * half_k) * 2;
    const uint32_t byte = codes[q];
    const float S = e4m3_to_f32(scales[row * (K >> 4) + (kk >> 4)]);
    const float p0 = e2m1_to_f32(byte & 0xFu) * S;  // exact
    const float p1 = e2m1_to_f32(byte >> 4) * S;
    out[row * K + kk] = p0 * g;
    out[row * K + kk + 1] = p1 * g;
}

}  // namespace pn

using namespace pn;

extern "C" {

int64_t pn_row_bytes(int type, int64_t K)
{
    const int G = pn_group(type);
    if (G == 0 || K <= 0 || K % G)
        return 0;
    return (K / G) * kBlockBytes;
}

const char *pn_status_string(int status)
{
    switch (status) {
    case PN_OK: return "ok";
    case PN_ERR_TYPE: return "unknown PN type";
    case PN_ERR_SHAPE: return "K is not a positive whole number of blocks (or a size is negative)";
    case PN_ERR_TOKENS: return "token count M out of range (0..16 for PN, 0..4 for NVFP4 and row-scaled E4M3)";
    case PN_ERR_NULL: return "required pointer is NULL";
    case PN_ERR_ALIGN: return "pointer misaligned";
    case PN_ERR_HIP: return "HIP runtime error";
    case PN_ERR_DEVICE: return "current device is not gfx950";
    case PN_ERR_HADAMARD: return "Hadamard slice size is not a power of two in 2..16384 dividing K";
    default: return "unknown status";
    }
}

static int pn_rows_common(int type, const void *W, int64_t nrows, int64_t K, const void *out)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (nrows < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (nrows == 0)
        return PN_OK;
    if (!W || !out)
        return PN_ERR_NULL;
    if (!aligned(W, 2) || !aligned(out, 4))
        return PN_ERR_ALIGN;
    return check_device();
}

int pn_validate_rows(int type, const void *W, int64_t nrows, int64_t K, int32_t *verdict,
                     void *stream)
{
    int st = pn_rows_common(type, W, nrows, K, verdict);
    if (st != PN_OK || nrows == 0)
        return st;
    const int nb = (int)(K / pn_group(type));
    const int64_t rb = pn_row_bytes(type, K);
    const dim3 grid((unsigned)((nrows + 3) / 4)), block(256);
    hipStream_t s = (hipStream_t)stream;
    if (type == PN_TYPE_PN3T)
        hipLaunchKernelGGL(validate_kernel<PN_TYPE_PN3T>, grid, block, 0, s,
                           (const uint8_t *)W, nrows, nb, rb, verdict);
    else
        hipLaunchKernelGGL(validate_kernel<PN_TYPE_PN4T>, grid, block, 0, s,
                           (const uint8_t *)W, nrows, nb, rb, verdict);
    return launch_status();
}

int pn_validate_row(int type, const void *row, int64_t K, int32_t *verdict, void *stream)
{
    return pn_validate_rows(type, row, 1, K, verdict, stream);
}

int pn_dequantize_rows(int type, const void *W, int64_t nrows, int64_t K, float *out, void *stream)
{
    int st = pn_rows_common(type, W, nrows, K, out);
    if (st != PN_OK || nrows == 0)
        return st;
    const int nb = (int)(K / pn_group(type));
    const int64_t rb = pn_row_bytes(type, K);
    const int64_t total = nrows * nb * 8;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    hipStream_t s = (hipStream_t)stream;
    if (type == PN_TYPE_PN3T)
        hipLaunchKernelGGL(dequantize_kernel<PN_TYPE_PN3T>, grid, block, 0, s,
                           (const uint8_t *)W, nrows, nb, rb, out);
    else
        hipLaunchKernelGGL(dequantize_kernel<PN_TYPE_PN4T>, grid, block, 0, s,
                           (const uint8_t *)W, nrows, nb, rb, out);
    return launch_status();
}

int pn_dequantize_row(int type, const void *row, int64_t K, float *out, void *stream)
{
    return pn_dequantize_rows(type, row, 1, K, out, stream);
}

static int nvfp4_common(int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % 16)
        return PN_ERR_SHAPE;
    return PN_OK;
}

int pn_nvfp4_validate_rows(const uint8_t *scales, float g, int64_t N, int64_t K, int32_t *verdict,
                           void *stream)
{
    int st = nvfp4_common(N, K);
    if (st != PN_OK || N == 0)
        return st;
    if (!scales || !verdict)
        return PN_ERR_NULL;
    if (!aligned(verdict, 4))
        return PN_ERR_ALIGN;
    if ((st = check_device()) != PN_OK)
        return st;
    const int gok = (g > 0.0f && g <= 3.402823466e38f) ? 1 : 0;  // finite and positive
    hipLaunchKernelGGL(nvfp4_validate_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, scales, gok, N, (int)(K / 16), verdict);
    return launch_status();
}

int pn_nvfp4_dequantize_rows(const uint8_t *codes, const uint8_t *scales, float g, int64_t N,
                             int64_t K, float *out, void *stream)
{
    int st = nvfp4_common(N, K);
    if (st != PN_OK || N == 0)
        return st;
    if (!codes || !scales || !out)
        return PN_ERR_NULL;
    if (!aligned(out, 4))
        return PN_ERR_ALIGN;
    if ((st = check_device()) != PN_OK)
        return st;
    const int64_t total = N * (K / 2);
    hipLaunchKernelGGL(nvfp4_dequantize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, (hipStream_t)stream, codes, scales, g, N, K, out);
    return launch_status();
}

}  // extern "C"
