// pn_nvfp4_gemv.hip -- W4A16 decode-step GEMV over NVFP4 weights, M = 1..4 bf16 tokens, gfx950.
//
// Format: "Quantisation and profiles", section "NVFP4": w = e2m1(code) * weight_scale[n, k/16] *
// weight_scale_2; NInfer "tensor formats" section 3.3 for the E2M1 / E4M3FN words. Layout: codes
// [N, K/2] with even k in the low nibble, scales [N, K/16], one fp32 global multiplier g.
//
// Design: like the PN GEMV, a workgroup stages x (bf16 pairs) in LDS and each wave streams R rows;
// lane l takes groups of 16 weights l, l+64, ... (8 code bytes and 1 scale byte, coalesced).
// v_cvt_scalef32_pk_bf16_fp4 turns one code byte into a pair of bf16 weights (exact: E2M1 values
// have 2 significant bits) and v_dot2_f32_bf16 multiplies the pair with the matching bf16 x pair
// into an fp32 sum: one instruction per weight. The group's E4M3 scale multiplies the group sum
// once; g multiplies the row total once.
#include <stdlib.h>

#include <algorithm>

#include "pn_common.h"

namespace pn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGroupLdsWords = 12;  // 8 bf16 pairs of a group + 4 words of bank padding

__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float v;
    if (e == 0)
        v = (float)m * 0x1p-9f;
    else if (e == 15 && m == 7)
        v = __builtin_nanf("");
    else
        v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

template <int M>
__device__ __forceinline__ void stage_x_bf16(uint32_t *lds, const uint16_t *__restrict__ x,
                                             int64_t K, int pg0, int pg)
{
    const int pairs = pg * 8;
    for (int q = threadIdx.x; q < M * pairs; q += blockDim.x) {
        const int m = q / pairs, rem = q - m * pairs;
        const int j = rem >> 3, i = rem & 7;
        const int64_t k = (int64_t)pg0 * 16 + 2 * rem;
        const uint32_t v = (uint32_t)x[(int64_t)m * K + k] | ((uint32_t)x[(int64_t)m * K + k + 1] << 16);
        lds[(m * pg + j) * kGroupLdsWords + i] = v;
    }
}

template <int M, int R>
__global__ void __launch_bounds__(256) nvfp4_gemv_kernel(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         float g, int64_t N, int64_t K,
                                                         const uint16_t *__restrict__ x,
                                                         float *__restrict__ y, int phase_groups)
{
    extern __shared__ uint32_t xl[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * R;
    const int ngroups = (int)(K >> 4);

    float acc[M][R];
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int r = 0; r < R; r++)
            acc[m][r] = 0.0f;

    for (int pg0 = 0; pg0 < ngroups; pg0 += phase_groups) {
        const int pg = min(phase_groups, ngroups - pg0);
        if (pg0)
            __syncthreads();
        stage_x_bf16<M>(xl, x, K, pg0, pg);
        __syncthreads();
        if (row0 >= N)
            continue;
        const uint8_t *cp[R];
        const uint8_t *sp[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = min(row0 + r, N - 1);
            cp[r] = codes + row * (K >> 1) + (int64_t)pg0 * 8;
            sp[r] = scales + row * ngroups + pg0;
        }
        for (int j = lane; j < pg; j += 64) {
            uint2 cw[R];
            uint32_t sw[R];
#pragma unroll
            for (int r = 0; r < R; r++) {
                cw[r] = *reinterpret_cast<const uint2 *>(cp[r] + 8 * j);
                sw[r] = sp[r][j];
            }
            float part[M][R];
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int r = 0; r < R; r++)
                    part[m][r] = 0.0f;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const uint32_t *xg = xl + (m * pg + j) * kGroupLdsWords;
                uint32_t xp[8];
#pragma unroll
                for (int i = 0; i < 8; i++)
                    xp[i] = xg[i];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float s = part[m][r];
#define PN_FP4_PAIR(word, sel, xi)                                                                 \
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, sel), \
                                        __builtin_bit_cast(bf16x2_t, xp[xi]), s, false)
                    PN_FP4_PAIR(cw[r].x, 0, 0);
                    PN_FP4_PAIR(cw[r].x, 1, 1);
                    PN_FP4_PAIR(cw[r].x, 2, 2);
                    PN_FP4_PAIR(cw[r].x, 3, 3);
                    PN_FP4_PAIR(cw[r].y, 0, 4);
                    PN_FP4_PAIR(cw[r].y, 1, 5);
                    PN_FP4_PAIR(cw[r].y, 2, 6);
                    PN_FP4_PAIR(cw[r].y, 3, 7);
#undef PN_FP4_PAIR
                    part[m][r] = s;
                }
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float S = e4m3_value(sw[r]);
#pragma unroll
                for (int m = 0; m < M; m++)
                    acc[m][r] = __builtin_fmaf(S, part[m][r], acc[m][r]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float s = wave_sum(acc[m][r]);
            if (lane == 0 && row0 + r < N)
                y[(int64_t)m * N + row0 + r] = s * g;
        }
}

// ---- rows of at most 64*GPL groups: x in registers ------------------------------------------------
//
// Persistent: one workgroup of 8 waves per CU; rows split into contiguous ranges per SIMD slot
// (quotient and remainder from the host). Lane l owns groups l, l + 64, ..., l + 64*(GPL-1) of every
// row: its x (8 bf16 pairs per group and token) is loaded once, straight into registers (bf16
// pairs are what v_dot2_f32_bf16 takes: no staging arithmetic, no LDS, no barrier). The x loads
// are issued before the first weight loads, so waiting for x never waits for weights. Each row
// then costs per lane GPL 8-byte code loads and GPL scale-byte loads, streamed through a ring of D
// rows; per group: 8 conversions + 8 DOT2 + one E4M3 conversion (v_cvt_f32_fp8 reads the OCP
// E4M3FN word) + one FMA. Partial sums of 4 / M rows are reduced together (transposed reduction).
struct NvRowSplit {
    int64_t rq;  // N / (gridDim.x * 4)
    int rr;      // N % (gridDim.x * 4)
};

__device__ __forceinline__ float nv_dot8(uint2 cw, const uint32_t *xp, float s)
{
#define PN_FP4_PAIR(word, sel, xi)                                                                 \
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, sel), \
                                        __builtin_bit_cast(bf16x2_t, xp[xi]), s, false)
    PN_FP4_PAIR(cw.x, 0, 0);
    PN_FP4_PAIR(cw.x, 1, 1);
    PN_FP4_PAIR(cw.x, 2, 2);
    PN_FP4_PAIR(cw.x, 3, 3);
    PN_FP4_PAIR(cw.y, 0, 4);
    PN_FP4_PAIR(cw.y, 1, 5);
    PN_FP4_PAIR(cw.y, 2, 6);
    PN_FP4_PAIR(cw.y, 3, 7);
#undef PN_FP4_PAIR
    return s;
}

template <int GPL>
struct NvRow {
    uint2 c[GPL];
    uint32_t s[GPL];
};

template <int M, int GPL, int D>
__global__ void __launch_bounds__(512) nvfp4_gemv_xreg_kernel(const uint8_t *__restrict__ codes,
                                                              const uint8_t *__restrict__ scales,
                                                              float g, int64_t N, int64_t K,
                                                              const uint16_t *__restrict__ x,
                                                              float *__restrict__ y, NvRowSplit sp,
                                                              int fnum)
{
    constexpr int RPR = 4 / M;  // rows per reduction
    static_assert(D % RPR == 0, "ring size must be a multiple of the rows per reduction");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ng = (int)(K >> 4);  // groups per row (<= 64 * GPL)

    // rows of this wave: slot = (workgroup, SIMD); the two waves of a SIMD split its range, the
    // older one (favoured by the instruction arbiter) taking fnum/16 of it
    const int slot = blockIdx.x * 4 + (wave & 3);
    const int64_t s0 = (int64_t)slot * sp.rq + min(slot, sp.rr);
    const int64_t cnt = sp.rq + (slot < sp.rr ? 1 : 0);
    const int64_t mid = (cnt * fnum + 8) >> 4;
    const int64_t r_begin = min(s0 + ((wave >> 2) ? mid : 0), N - 1);
    const int nrows = (int)((wave >> 2) ? cnt - mid : mid);
    const int last = max(nrows - 1, 0);

    // x of this lane's groups, bf16 pairs in registers (clamped for groups past the row's end)
    uint32_t xr[M][GPL][8];
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int i = 0; i < GPL; i++) {
            const int j = min(lane + 64 * i, ng - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)m * K + 16 * (int64_t)j);
            const uint4 a = src[0], b = src[1];
            xr[m][i][0] = a.x; xr[m][i][1] = a.y; xr[m][i][2] = a.z; xr[m][i][3] = a.w;
            xr[m][i][4] = b.x; xr[m][i][5] = b.y; xr[m][i][6] = b.z; xr[m][i][7] = b.w;
        }

    const int64_t cbytes = K >> 1;
    auto load_row = [&](NvRow<GPL> &rw, int it) {
        const int64_t row = r_begin + min(it, last);
        const uint8_t *cp = codes + row * cbytes;
        const uint8_t *sc = scales + row * ng;
#pragma unroll
        for (int i = 0; i < GPL; i++) {
            const int j = min(lane + 64 * i, ng - 1);
            rw.c[i] = load_nt8(cp + 8 * (int64_t)j);  // each 8-byte piece is read once
            rw.s[i] = sc[j];
        }
    };
    NvRow<GPL> buf[D];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        load_row(buf[p], p);

    float vals[4];
#pragma unroll
    for (int o = 0; o < 4; o++)
        vals[o] = 0.0f;
    for (int it0 = 0; it0 < nrows; it0 += D) {
#pragma unroll
        for (int sidx = 0; sidx < D; sidx++) {
            const int it = it0 + sidx;
            load_row(buf[(sidx + D - 1) % D], it + D - 1);
            if (it < nrows) {
                const int rs = sidx % RPR;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float acc = 0.0f;
#pragma unroll
                    for (int i = 0; i < GPL; i++) {
                        // groups past the row's end (clamped loads) get a zero scale
                        const float S = (lane + 64 * i < ng)
                                            ? __builtin_amdgcn_cvt_f32_fp8((int)buf[sidx].s[i], 0)
                                            : 0.0f;
                        acc = __builtin_fmaf(S, nv_dot8(buf[sidx].c[i], xr[m][i], 0.0f), acc);
                    }
                    vals[rs * M + m] = acc;
                }
                if (rs == RPR - 1 || it == nrows - 1) {
                    float tot[1];
                    transpose_reduce<4>(vals, tot);
                    if ((lane & 15) == 0) {
                        const int o = lane >> 4;  // value o = rs * M + m
                        const int jr = o / M, m = o - jr * M;
                        if (jr <= rs)
                            y[(int64_t)m * N + r_begin + (it - rs + jr)] = tot[0] * g;
                    }
#pragma unroll
                    for (int o = 0; o < 4; o++)
                        vals[o] = 0.0f;
                }
            }
        }
    }
}

// Older-wave share in sixteenths (PN_GEMV_NV_SPLIT overrides; 4..15); 10/16 measured best.
static int nv_older_share()
{
    const char *e = getenv("PN_GEMV_NV_SPLIT");
    const int v = e ? atoi(e) : 10;
    return v < 4 ? 4 : v > 15 ? 15 : v;
}

template <int M, int GPL>
static int launch_nv_xreg(const uint8_t *codes, const uint8_t *scales, float g, int64_t N, int64_t K,
                          const uint16_t *x, float *y, hipStream_t s)
{
    const int cus = device_cus();
    const int grid = (int)std::min<int64_t>(cus, (N + 3) / 4);
    const int64_t S = (int64_t)grid * 4;
    // ring of 4 rows at 1-2 tokens, 2 at 3-4 (registers: x takes 8*GPL per token)
    hipLaunchKernelGGL((nvfp4_gemv_xreg_kernel<M, GPL, M <= 2 ? 4 : 2>), dim3((unsigned)grid),
                       dim3(512), 0, s, codes, scales, g, N, K, x, y, NvRowSplit{N / S, (int)(N % S)},
                       nv_older_share());
    return launch_status();
}

constexpr int kNvLdsBudget = 80 * 1024;

template <int M, int R>
static int launch_nv(const uint8_t *codes, const uint8_t *scales, float g, int64_t N, int64_t K,
                     const uint16_t *x, float *y, hipStream_t s)
{
    const int ngroups = (int)(K >> 4);
    const int per_group = M * kGroupLdsWords * 4;
    const int phase_groups = min(ngroups, kNvLdsBudget / per_group);
    constexpr auto kern = nvfp4_gemv_kernel<M, R>;
    if (!lds_limit_once<kern>(kNvLdsBudget))
        return PN_ERR_HIP;
    const int64_t rows_per_wg = 4 * R;
    hipLaunchKernelGGL(kern, dim3((unsigned)((N + rows_per_wg - 1) / rows_per_wg)), dim3(256),
                       (size_t)phase_groups * per_group, s, codes, scales, g, N, K, x, y,
                       phase_groups);
    return launch_status();
}

}  // namespace pn

using namespace pn;

extern "C" int pn_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, float g, int64_t N,
                             int64_t K, const uint16_t *x_bf16, int64_t M, float *y, void *stream)
{
    if (N < 0 || K <= 0 || K % 16)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (N == 0 || M == 0)
        return PN_OK;
    if (!codes || !scales || !x_bf16 || !y)
        return PN_ERR_NULL;
    if (!aligned(codes, 8) || !aligned(x_bf16, 2) || !aligned(y, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    // x in registers: at most 64*GPL groups per row (GPL = 6 at 1-2 tokens, 5 at 3-4), x 16-byte
    // aligned (PN_GEMV_NO_XREG selects the LDS kernel, for tests)
    const int64_t ng = K >> 4;
    if (ng <= 64 * (M <= 2 ? 6 : 5) && aligned(x_bf16, 16) && !getenv("PN_GEMV_NO_XREG")) {
        switch (M) {
        case 1:
            return ng <= 64 * 4   ? launch_nv_xreg<1, 4>(codes, scales, g, N, K, x_bf16, y, s)
                   : ng <= 64 * 5 ? launch_nv_xreg<1, 5>(codes, scales, g, N, K, x_bf16, y, s)
                                  : launch_nv_xreg<1, 6>(codes, scales, g, N, K, x_bf16, y, s);
        case 2:
            return ng <= 64 * 4   ? launch_nv_xreg<2, 4>(codes, scales, g, N, K, x_bf16, y, s)
                   : ng <= 64 * 5 ? launch_nv_xreg<2, 5>(codes, scales, g, N, K, x_bf16, y, s)
                                  : launch_nv_xreg<2, 6>(codes, scales, g, N, K, x_bf16, y, s);
        case 3:
            return ng <= 64 * 4 ? launch_nv_xreg<3, 4>(codes, scales, g, N, K, x_bf16, y, s)
                                : launch_nv_xreg<3, 5>(codes, scales, g, N, K, x_bf16, y, s);
        default:
            return ng <= 64 * 4 ? launch_nv_xreg<4, 4>(codes, scales, g, N, K, x_bf16, y, s)
                                : launch_nv_xreg<4, 5>(codes, scales, g, N, K, x_bf16, y, s);
        }
    }
    switch (M) {
    case 1: return launch_nv<1, 2>(codes, scales, g, N, K, x_bf16, y, s);
    case 2: return launch_nv<2, 2>(codes, scales, g, N, K, x_bf16, y, s);
    case 3: return launch_nv<3, 2>(codes, scales, g, N, K, x_bf16, y, s);
    default: return launch_nv<4, 2>(codes, scales, g, N, K, x_bf16, y, s);
    }
}
