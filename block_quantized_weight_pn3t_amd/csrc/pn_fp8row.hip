// pn_fp8row.hip -- row-scaled E4M3FN weights on gfx950: validation, decode, the GEMV y = W.x for
// M = 1..4 fp32 tokens, and the FP8-head quantizer.
//
// Format: NInfer "tensor formats", section 3.4 (FP8_E4M3FN_ROW_BF16S): codes [N, K] E4M3FN words
// (section 3.3), one bfloat16 multiplier per row (section 3.1); w = binary32(e4m3(c) * s).
// Quantizer: "Quantisation and profiles", "The FP8 head" (multipliers 1.0, 0.95, 0.90 of the row's
// largest weight), with the scale stored as the bfloat16 multiplier.
//
// GEMV design (HBM-bound at 1 byte per weight; no MFMA: a matrix-vector product):
//  * Persistent: one workgroup of 8 waves per CU; rows split into contiguous ranges per SIMD slot,
//    the older wave of a SIMD taking the larger share (the instruction arbiter favours it).
//  * x is staged once per workgroup in LDS, in K-phases when it does not fit: chunk j of 16 floats
//    at a stride of 20 floats (80 bytes), so 8 consecutive lanes reading 16-byte pieces of
//    consecutive chunks hit 8 distinct bank groups. Its loads are issued before the first weight
//    loads (the memory counter retires loads in order, so waiting for x never waits for weights).
//  * A wave takes its rows R at a time; lane l owns the 16-byte code chunks l, l + 64, ... of the
//    phase ("items" of 64 chunks), streamed through a ring of D items with non-temporal loads
//    (every chunk is read once: 6.7 TB/s against 5.6 with ordinary loads on the head at M = 1). Per chunk and row: 8
//    v_cvt_pk_f32_fp8 (two exact E4M3FN values each) and 16 FMA per token, x read from LDS once
//    for the R rows.
//  * Per group: a transposed permlane/DPP reduction of the R x M partial sums, times the row's
//    multiplier, stored (phases after the first add into y). One fixed order per output.
#include <stdlib.h>

#include <algorithm>

#include "pn_common.h"

namespace pn {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b)
{
    return __builtin_bit_cast(float, b << 16);
}

// ---- validation: one wave per row ----------------------------------------------------------------

// Section 3.4 validity: the multiplier has sign bit 0 and is finite; no code is a NaN word (0x7F,
// 0xFF); a positive-zero multiplier requires every code to be a signed zero.
__global__ void fp8row_validate_kernel(const uint8_t *__restrict__ codes,
                                       const uint16_t *__restrict__ scales, int64_t N, int64_t K,
                                       int32_t *__restrict__ verdict, int vec16)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= N)
        return;  // the whole wave
    const uint32_t s = scales[row];
    const uint8_t *r = codes + row * K;
    uint32_t nan7 = 0, nz = 0;  // per byte lane: low 7 bits all ones / not all zero
    if (vec16) {  // K a multiple of 16, rows 16-byte aligned: SWAR over 16 codes
        for (int64_t k = 16 * (int64_t)lane; k < K; k += 16 * 64) {
            const uint4 v = *reinterpret_cast<const uint4 *>(r + k);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t low = w[i] & 0x7F7F7F7Fu;
                nan7 |= (low + 0x01010101u) & 0x80808080u;  // no carry leaves a byte
                nz |= low;
            }
        }
    } else {
        for (int64_t k = lane; k < K; k += 64) {
            const uint32_t low = r[k] & 0x7Fu;
            nan7 |= (low == 0x7Fu);
            nz |= low;
        }
    }
    const bool bad = (s & 0x8000u) || (s & 0x7F80u) == 0x7F80u || nan7 != 0 || (s == 0 && nz != 0);
    const bool any_bad = __any(bad);
    if (lane == 0)
        verdict[row] = any_bad ? 0 : 1;
}

// ---- decode: one thread per code -------------------------------------------------------------------

__global__ void fp8row_dequantize_kernel(const uint8_t *__restrict__ codes,
                                         const uint16_t *__restrict__ scales, int64_t N, int64_t K,
                                         float *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * K)
        return;
    const int64_t row = i / K;
    const float c32 = __builtin_amdgcn_cvt_f32_fp8((int)codes[i], 0);  // exact E4M3FN value
    out[i] = c32 * bf16_bits_to_f32(scales[row]);
}

// ---- GEMV -------------------------------------------------------------------------------------------

constexpr int kChunkStride = 20;  // floats per staged chunk of 16 x (80 bytes)
constexpr int kFp8MaxLds = 160 * 1024;

// Product of one 16-code chunk with x: two chains of 8.
__device__ __forceinline__ void chunk_fma(uint4 c, const float *xv, float &a0, float &a1)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);  // bytes 0, 1
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);   // bytes 2, 3
        float &a = q < 2 ? a0 : a1;
        a = __builtin_fmaf(lo.x, xv[4 * q + 0], a);
        a = __builtin_fmaf(lo.y, xv[4 * q + 1], a);
        a = __builtin_fmaf(hi.x, xv[4 * q + 2], a);
        a = __builtin_fmaf(hi.y, xv[4 * q + 3], a);
    }
}

template <int M, int R, int D, int QX>
__global__ void __launch_bounds__(512) fp8row_gemv_kernel(const uint8_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ scales,
                                                          int64_t N, int64_t K,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y, RowSplit sp,
                                                          int fnum, int phase_ch, int x_vec4)
{
    constexpr int V = ((M * R + 3) / 4) * 4;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t r_begin;
    int nrows;
    wave_rows(N, sp, wave, 8, fnum, r_begin, nrows);
    const int ngroups = (nrows + R - 1) / R;
    const int64_t nch = K >> 4;
    const uint8_t *wbase = codes + r_begin * K;

    for (int64_t c0 = 0; c0 < nch; c0 += phase_ch) {
        const int pch = (int)min((int64_t)phase_ch, nch - c0);
        const int iters = (pch + 63) >> 6;
        const int nitems = ngroups * iters;

        // 1. x loads of this phase: float4 q of token m, chunk j = q / 4 (uniform branch past the
        // needed count; the weight loads issued next are unconditional)
        const int total = M * pch * 4;
        const int nq = (total + 511) >> 9;
        float4 xv[QX];
#pragma unroll
        for (int u = 0; u < QX; u++) {
            if (u < nq) {
                const int q = min((int)threadIdx.x + u * 512, total - 1);
                const int m = q / (pch * 4), c = q - m * pch * 4;
                const float *src = x + (int64_t)m * K + 16 * c0 + 4 * c;
                xv[u] = x_vec4 ? *reinterpret_cast<const float4 *>(src)
                               : make_float4(src[0], src[1], src[2], src[3]);
            }
        }

        // 2. first weight loads (clamped: no load inside a branch, none outside the matrix)
        auto load_item = [&](uint4 (&buf)[R], int it) {
            it = min(it, max(nitems - 1, 0));
            const int g = it / iters, i = it - g * iters;
            const int64_t j = c0 + min(lane + 64 * i, pch - 1);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = min(g * R + r, max(nrows - 1, 0));
                buf[r] = load_nt16(wbase + (int64_t)row * K + 16 * j);
            }
        };
        uint4 buf[D][R];
#pragma unroll
        for (int p = 0; p < D - 1; p++)
            load_item(buf[p], p);

        // 3. stage x
        if (c0)
            __syncthreads();  // the previous phase's readers are done
#pragma unroll
        for (int u = 0; u < QX; u++) {
            const int q = (int)threadIdx.x + u * 512;
            if (u < nq && q < total) {
                const int m = q / (pch * 4), c = q - m * pch * 4;
                const int j = c >> 2, e = c & 3;
                *reinterpret_cast<float4 *>(lds + (m * pch + j) * kChunkStride + 4 * e) = xv[u];
            }
        }
        __syncthreads();

        // 4. stream
        float acc[M][R];
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int r = 0; r < R; r++)
                acc[m][r] = 0.0f;

        auto compute_item = [&](const uint4 (&cb)[R], int it) {
            const int g = it / iters, i = it - g * iters;
            const int jl = lane + 64 * i;
            const bool valid = jl < pch;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float4 *xq = reinterpret_cast<const float4 *>(
                    lds + (m * pch + min(jl, pch - 1)) * kChunkStride);
                float xw[16];
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const float4 t = xq[c];
                    xw[4 * c + 0] = t.x;
                    xw[4 * c + 1] = t.y;
                    xw[4 * c + 2] = t.z;
                    xw[4 * c + 3] = t.w;
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float a0 = 0.0f, a1 = 0.0f;
                    chunk_fma(cb[r], xw, a0, a1);
                    // selected, not multiplied by a mask: a NaN code of a clamped lane stays out
                    acc[m][r] += valid ? a0 + a1 : 0.0f;
                }
            }
            if (i == iters - 1) {  // the group's rows are complete for this phase
                float v[V], tot[V / 4];
#pragma unroll
                for (int o = 0; o < V; o++)
                    v[o] = (o < M * R) ? acc[(o < M * R ? o : 0) / R][o % R] : 0.0f;
                transpose_reduce<V>(v, tot);
                if ((lane & 15) == 0) {
                    const int qq = lane >> 4;
#pragma unroll
                    for (int t = 0; t < V / 4; t++) {
                        const int o = t + qq * (V / 4);
                        const int m = o / R, r = o - m * R;
                        const int row = g * R + r;
                        if (o < M * R && row < nrows) {
                            const float sc = bf16_bits_to_f32(scales[r_begin + row]);
                            float *dst = y + (int64_t)m * N + r_begin + row;
                            *dst = c0 ? __builtin_fmaf(sc, tot[t], *dst) : sc * tot[t];
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < M; m++)
#pragma unroll
                    for (int r = 0; r < R; r++)
                        acc[m][r] = 0.0f;
            }
        };

        for (int it0 = 0; it0 < nitems; it0 += D) {
#pragma unroll
            for (int s = 0; s < D; s++) {
                const int it = it0 + s;
                load_item(buf[(s + D - 1) % D], it + D - 1);
                if (it < nitems)
                    compute_item(buf[s], it);
            }
        }
    }
}

// One token, rows of at most 1024*CPL codes (CPL <= 5: registers): x in registers. Lane l owns chunks l, l + 64, ...,
// l + 64*(CPL-1) of every row (its 16*CPL x values live in VGPRs: no LDS, no barrier), and each
// wave streams its contiguous row range front to back (the access pattern of a plain copy) through
// a ring of D rows; partial sums of 4 rows are reduced together (transposed reduction), times
// each row's multiplier.
template <int CPL, int D>
__global__ void __launch_bounds__(512) fp8row_gemv_xreg_kernel(const uint8_t *__restrict__ codes,
                                                               const uint16_t *__restrict__ scales,
                                                               int64_t N, int64_t K,
                                                               const float *__restrict__ x,
                                                               float *__restrict__ y, RowSplit sp,
                                                               int fnum)
{
    static_assert(D % 4 == 0, "ring size must be a multiple of the rows per reduction");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t r_begin;
    int nrows;
    wave_rows(N, sp, wave, 8, fnum, r_begin, nrows);
    const int last = max(nrows - 1, 0);
    const int nch = (int)(K >> 4);

    // x of this lane's chunks (clamped past the row's end; their products are dropped)
    float xr[CPL][16];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int j = min(lane + 64 * i, nch - 1);
        const float4 *src = reinterpret_cast<const float4 *>(x + 16 * (int64_t)j);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 t = src[q];
            xr[i][4 * q + 0] = t.x;
            xr[i][4 * q + 1] = t.y;
            xr[i][4 * q + 2] = t.z;
            xr[i][4 * q + 3] = t.w;
        }
    }

    const uint8_t *wbase = codes + r_begin * K;
    auto load_row = [&](uint4 (&rb)[CPL], int it) {
        const uint8_t *rp = wbase + (int64_t)min(it, last) * K;
#pragma unroll
        for (int i = 0; i < CPL; i++)
            rb[i] = load_nt16(rp + 16 * (int64_t)min(lane + 64 * i, nch - 1));
    };
    uint4 buf[D][CPL];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        load_row(buf[p], p);

    float vals[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int it0 = 0; it0 < nrows; it0 += D) {
#pragma unroll
        for (int s = 0; s < D; s++) {
            const int it = it0 + s;
            load_row(buf[(s + D - 1) % D], it + D - 1);
            if (it < nrows) {
                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; i++) {
                    float c0 = 0.0f, c1 = 0.0f;
                    chunk_fma(buf[s][i], xr[i], c0, c1);
                    // selected, not multiplied by a mask: clamped chunks stay out
                    const bool ok = lane + 64 * i < nch;
                    a0 += ok ? c0 : 0.0f;
                    a1 += ok ? c1 : 0.0f;
                }
                const int slot = s & 3;
                vals[slot] = a0 + a1;
                if (slot == 3 || it == nrows - 1) {
                    float tot[1];
                    transpose_reduce<4>(vals, tot);
                    if ((lane & 15) == 0) {
                        const int jr = lane >> 4;
                        if (jr <= slot) {
                            const int64_t row = r_begin + it - slot + jr;
                            y[row] = bf16_bits_to_f32(scales[row]) * tot[0];
                        }
                    }
                    vals[0] = vals[1] = vals[2] = vals[3] = 0.0f;
                }
            }
        }
    }
}

// ---- host ---------------------------------------------------------------------------------------

static int fp8row_common(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K)
{
    if (N < 0 || K <= 0)
        return PN_ERR_SHAPE;
    if (N > 0 && (!codes || !scales))
        return PN_ERR_NULL;
    if (!aligned(scales, 2))
        return PN_ERR_ALIGN;
    return PN_OK;
}

static int fp8_num_cus() { return device_cus(); }

template <int M, int QX, int D>
static int launch_fp8row_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                              const float *x, float *y, hipStream_t s)
{
    // rows per item: x is read from LDS once per chunk for R rows (4 at 2-4 tokens: 198 / 230 /
    // 266 us on the head at 2 / 3 / 4 tokens against 203 / 256 / 294 us with 2)
    constexpr int R = M == 1 ? 2 : 4;
    constexpr auto kern = fp8row_gemv_kernel<M, R, D, QX>;
    if (!lds_limit_once<kern>(kFp8MaxLds))
        return PN_ERR_HIP;
    const int64_t nch = K >> 4;
    // a phase holds at most 512 chunks (8192 weights) and fits LDS at 4 tokens; 16 float4 x loads
    // per thread at most
    const int phase_ch = (int)std::min<int64_t>(nch, 512);
    const size_t lds = (size_t)M * phase_ch * kChunkStride * sizeof(float);
    const int grid = (int)std::min<int64_t>(fp8_num_cus(), (N + 3) / 4);
    const char *e = getenv("PN_GEMV_SPLIT");
    // the older wave's share of a SIMD's rows, in sixteenths (measured on the head: 8 at 1-2
    // tokens; 9 at 3-4 tokens, 227 / 265 us against 234 / 280 us with 8)
    const int fnum = e ? std::max(4, std::min(15, atoi(e))) : (M >= 3 ? 9 : 8);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, codes, scales, N, K, x, y,
                       row_split(N, grid), fnum, phase_ch, aligned(x, 16) ? 1 : 0);
    return launch_status();
}

template <int CPL>
static int launch_fp8row_xreg(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                              const float *x, float *y, hipStream_t s)
{
    const int grid = (int)std::min<int64_t>(fp8_num_cus(), (N + 3) / 4);
    const char *e = getenv("PN_GEMV_SPLIT");
    const int fnum = e ? std::max(4, std::min(15, atoi(e))) : 12;
    const char *d = getenv("PN_FP8ROW_DEPTH");  // ring of 8 rows (registers allow it up to CPL 4)
    if (CPL <= 4 && d && atoi(d) >= 8)
        hipLaunchKernelGGL((fp8row_gemv_xreg_kernel<CPL, 8>), dim3((unsigned)grid), dim3(512), 0, s,
                           codes, scales, N, K, x, y, row_split(N, grid), fnum);
    else
        hipLaunchKernelGGL((fp8row_gemv_xreg_kernel<CPL, 4>), dim3((unsigned)grid), dim3(512), 0, s,
                           codes, scales, N, K, x, y, row_split(N, grid), fnum);
    return launch_status();
}

}  // namespace pn

using namespace pn;

extern "C" int pn_fp8row_validate_rows(const uint8_t *codes, const uint16_t *scales, int64_t N,
                                       int64_t K, int32_t *verdict, void *stream)
{
    int st = fp8row_common(codes, scales, N, K);
    if (st != PN_OK || N == 0)
        return st;
    if (!verdict)
        return PN_ERR_NULL;
    if (!aligned(verdict, 4))
        return PN_ERR_ALIGN;
    if ((st = check_device()) != PN_OK)
        return st;
    const int vec16 = (K % 16 == 0 && aligned(codes, 16)) ? 1 : 0;
    hipLaunchKernelGGL(fp8row_validate_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0,
                       (hipStream_t)stream, codes, scales, N, K, verdict, vec16);
    return launch_status();
}

extern "C" int pn_fp8row_dequantize_rows(const uint8_t *codes, const uint16_t *scales, int64_t N,
                                         int64_t K, float *out, void *stream)
{
    int st = fp8row_common(codes, scales, N, K);
    if (st != PN_OK || N == 0)
        return st;
    if (!out)
        return PN_ERR_NULL;
    if (!aligned(out, 4))
        return PN_ERR_ALIGN;
    if ((st = check_device()) != PN_OK)
        return st;
    const int64_t n = N * K;
    hipLaunchKernelGGL(fp8row_dequantize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, codes, scales, N, K, out);
    return launch_status();
}

extern "C" int pn_gemv_fp8row(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                              const float *x, int64_t M, float *y, void *stream)
{
    if (N < 0 || K <= 0 || K % 16)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (N == 0 || M == 0)
        return PN_OK;
    if (!codes || !scales || !x || !y)
        return PN_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(x, 4) || !aligned(y, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // float4 x loads per thread for one phase: M * min(K/16, 512) * 4 / 512
    // one token, K <= 5120, x 16-byte aligned: x in registers (PN_GEMV_NO_XREG selects the LDS
    // kernel, for tests)
    const int64_t nch = K >> 4;
    if (M == 1 && nch <= 64 * 5 && aligned(x, 16) && !getenv("PN_GEMV_NO_XREG")) {
        return nch <= 64 * 2   ? launch_fp8row_xreg<2>(codes, scales, N, K, x, y, s)
               : nch <= 64 * 4 ? launch_fp8row_xreg<4>(codes, scales, N, K, x, y, s)
                               : launch_fp8row_xreg<5>(codes, scales, N, K, x, y, s);
    }
    switch (M) {
    case 1: return launch_fp8row_gemv<1, 4, 4>(codes, scales, N, K, x, y, s);
    case 2: return launch_fp8row_gemv<2, 8, 4>(codes, scales, N, K, x, y, s);
    case 3: return launch_fp8row_gemv<3, 12, 4>(codes, scales, N, K, x, y, s);
    default: return launch_fp8row_gemv<4, 16, 4>(codes, scales, N, K, x, y, s);
    }
}
