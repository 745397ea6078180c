// pn_gemv.hip -- decode-step GEMV y = W.x over PN blocks (pn3t, pn4t), M = 1..4 tokens, gfx950.
//
// Format: "PN weight format" (PNX-FORMAT-v0): "Block layout" (34-byte blocks, the shift rule
// BITS*(t>>1) + 16*(t&1), no code crosses a 16-bit half), "Value" (w = d * (n - z)).
//
// Design (HBM-bound; no MFMA: this is a matrix-vector product, not a dense contraction):
//  * Persistent: one workgroup per CU. Rows are split into contiguous, balanced ranges, one per
//    wave. A wave streams its rows through a ring of register buffers so several rows of loads
//    are in flight while one is decoded. Loads are never inside a branch (indices are clamped),
//    which keeps the hardware wait counts exact. Weight loads are 2 x 16 bytes from
//    a 4-byte aligned address plus 2 bytes, exactly the block's 34 bytes at either alignment
//    parity, re-aligned with v_alignbit.
//  * Decode uses the pairing of the layout: one AND with a mask like 0x00070007 leaves two codes,
//    one per 16-bit half, at bit position p of the half. As fp16 words those halves are the exact
//    subnormals n * 2^(p-24), i.e. a ready-made fp16 pair for v_dot2_f32_f16 (full rate on gfx950;
//    the mixed-precision FMA v_fma_mix_f32 and v_cvt_f32_f16 issue at half rate). x is staged per
//    block as fp16 pairs: x' = x * 2^(24-p) * 2^-s (s puts the block's largest |x'| in
//    [2^14, 2^15)), split into hi = fp16(x') and lo = fp16(x' - hi), so each pair of weights costs
//    two dot2 (hi, lo) and x keeps ~22 significant bits:
//      pn3t word: 1 shift + 5 AND + 10 DOT2 for 10 weights; pn4t: 1 shift + 4 AND + 8 DOT2 for 8.
//  * The zero point is folded per block: sum_k (n_k - z) x_k = sum_k n_k x_k - z * sum_k x_k, with
//    the block's plain sum of x staged next to the pairs; d * 2^s multiplies once per block.
//  * fp32 accumulation; the R rows x M tokens of partial sums are reduced together by a
//    transposed permlane/DPP reduction. Each output is produced by one wave in a fixed order:
//    results are deterministic (no atomics).
//  * Rows of at most 64 blocks keep the staged x of their block in registers (lane l owns block l);
//    longer rows stage x in LDS once per workgroup (in K-phases when it does not fit).
#include <stdlib.h>

#include "pn_common.h"

namespace pn {

typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));

// Bit position p, inside its 16-bit half after the masking below, of code t of a word: pn3t t = 0,1
// and 6,7 sit at p = 0; t = 2,3 and 8,9 at p = 3; t = 4,5 at p = 6 (t = 6..9 after a >> 9).
// pn4t: t = 0,1 and 4,5 at p = 0; t = 2,3 and 6,7 at p = 4 (t = 4..7 after a >> 8).
template <int TYPE> __device__ __forceinline__ int code_pos(int t);
template <> __device__ __forceinline__ int code_pos<PN_TYPE_PN3T>(int t) { return 3 * ((t >> 1) % 3); }
template <> __device__ __forceinline__ int code_pos<PN_TYPE_PN4T>(int t) { return 4 * ((t >> 1) & 1); }

__device__ __forceinline__ float dot2(uint32_t codes, uint32_t xpair, float acc)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2_t, codes),
                                  __builtin_bit_cast(h16x2_t, xpair), acc, false);
}

// ah += sum over the word's codes of n_t * x'hi_t, al the same with the lo parts. xp holds the
// word's CPW/2 pairs as (hi, lo) dwords: xp[2j] = hi pair j, xp[2j+1] = lo pair j.
template <int TYPE>
__device__ __forceinline__ void word_dot(uint32_t w, const uint32_t *xp, float &ah, float &al);

template <>
__device__ __forceinline__ void word_dot<PN_TYPE_PN3T>(uint32_t w, const uint32_t *xp, float &ah,
                                                       float &al)
{
    const uint32_t a0 = w & 0x00070007u;  // t = 0 | t = 1   (p = 0)
    const uint32_t a1 = w & 0x00380038u;  // t = 2 | t = 3   (p = 3)
    const uint32_t a2 = w & 0x01C001C0u;  // t = 4 | t = 5   (p = 6)
    const uint32_t ws = w >> 9;
    const uint32_t a3 = ws & 0x00070007u; // t = 6 | t = 7   (p = 0)
    const uint32_t a4 = ws & 0x00380038u; // t = 8 | t = 9   (p = 3)
    ah = dot2(a0, xp[0], ah);
    al = dot2(a0, xp[1], al);
    ah = dot2(a1, xp[2], ah);
    al = dot2(a1, xp[3], al);
    ah = dot2(a2, xp[4], ah);
    al = dot2(a2, xp[5], al);
    ah = dot2(a3, xp[6], ah);
    al = dot2(a3, xp[7], al);
    ah = dot2(a4, xp[8], ah);
    al = dot2(a4, xp[9], al);
}

template <>
__device__ __forceinline__ void word_dot<PN_TYPE_PN4T>(uint32_t w, const uint32_t *xp, float &ah,
                                                       float &al)
{
    const uint32_t a0 = w & 0x000F000Fu;  // t = 0 | t = 1   (p = 0)
    const uint32_t a1 = w & 0x00F000F0u;  // t = 2 | t = 3   (p = 4)
    const uint32_t ws = w >> 8;
    const uint32_t a2 = ws & 0x000F000Fu; // t = 4 | t = 5   (p = 0)
    const uint32_t a3 = ws & 0x00F000F0u; // t = 6 | t = 7   (p = 4)
    ah = dot2(a0, xp[0], ah);
    al = dot2(a0, xp[1], al);
    ah = dot2(a1, xp[2], ah);
    al = dot2(a1, xp[3], al);
    ah = dot2(a2, xp[4], ah);
    al = dot2(a2, xp[5], al);
    ah = dot2(a3, xp[6], ah);
    al = dot2(a3, xp[7], al);
}

// ---- x staging ----------------------------------------------------------------------------------
// One staged block of x (G consecutive values of one token) is G + 2 dwords: the G/2 pairs as
// (hi, lo) dwords, then sxs = (sum of the block's x) * 2^-s and scl = 2^s.

// Scale exponent of a block: s such that max_e |x_e| * 2^(24 - p_e - s) lies in [2^14, 2^15).
__device__ __forceinline__ int block_shift(float amax_scaled)
{
    if (!(amax_scaled > 0.0f) || !(amax_scaled < __builtin_inff()))
        return 0;  // all zero, or non-finite input (the result is then non-finite too)
    return __builtin_amdgcn_frexp_expf(amax_scaled) - 15;
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// hi and lo fp16 pairs of two staged values (x' already scaled)
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    hi = pack_h2(ha, hb);
    lo = pack_h2((_Float16)(a - (float)ha), (_Float16)(b - (float)hb));
}

// Pass 1: 16-byte global loads of x, plain fp32 values written to their block slots in LDS.
// Unrolled so that every thread has its loads in flight together.
template <int TYPE, int M>
__device__ __forceinline__ void stage_x_raw(float *lds, const float *__restrict__ x, int64_t K,
                                            int pb, int pn, bool vec4)
{
    using F = Fmt<TYPE>;
    constexpr int U = 8;
    const int per_tok = pn * (F::G / 4);
    const int total = M * per_tok;
    for (int q0 = threadIdx.x; q0 < total; q0 += U * blockDim.x) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int q = q0 + u * blockDim.x;
            if (q < total) {
                const int m = q / per_tok, c = q - m * per_tok;
                const float *src = x + (int64_t)m * K + (int64_t)pb * F::G + 4 * c;
                if (vec4)
                    v[u] = *reinterpret_cast<const float4 *>(src);
                else
                    v[u] = make_float4(src[0], src[1], src[2], src[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int q = q0 + u * blockDim.x;
            if (q < total) {
                const int m = q / per_tok, c = q - m * per_tok;
                const int b = (4 * c) / F::G, e = 4 * c - b * F::G;
                *reinterpret_cast<float4 *>(lds + (m * pn + b) * F::LDS_STRIDE + e) = v[u];
            }
        }
    }
}

// Pass 2 (after a barrier), one thread per (token, block): sum and scale exponent, then the pairs
// rewritten in place (pair q occupies exactly the dwords of values 2q and 2q+1).
template <int TYPE, int M>
__device__ __forceinline__ void stage_x_pairs(float *lds, int pn)
{
    using F = Fmt<TYPE>;
    for (int q = threadIdx.x; q < M * pn; q += blockDim.x) {
        float *blk = lds + q * F::LDS_STRIDE;
        const float4 *src = reinterpret_cast<const float4 *>(blk);
        float sum = 0.0f, amax = 0.0f;
#pragma unroll
        for (int c = 0; c < F::G / 4; c++) {
            const float4 v = src[c];
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                sum += vv[i];
                amax = fmaxf(amax, __builtin_ldexpf(__builtin_fabsf(vv[i]),
                                                    24 - code_pos<TYPE>((4 * c + i) % F::CPW)));
            }
        }
        const int s = block_shift(amax);
        uint32_t *bw = reinterpret_cast<uint32_t *>(blk);
#pragma unroll
        for (int c = 0; c < F::G / 4; c++) {
            const float4 v = src[c];
            const int t0 = (4 * c) % F::CPW, t2 = (4 * c + 2) % F::CPW;
            uint32_t h0, l0, h1, l1;
            split_pair(__builtin_ldexpf(v.x, 24 - code_pos<TYPE>(t0) - s),
                       __builtin_ldexpf(v.y, 24 - code_pos<TYPE>(t0) - s), h0, l0);
            split_pair(__builtin_ldexpf(v.z, 24 - code_pos<TYPE>(t2) - s),
                       __builtin_ldexpf(v.w, 24 - code_pos<TYPE>(t2) - s), h1, l1);
            *reinterpret_cast<uint4 *>(bw + 4 * c) = make_uint4(h0, l0, h1, l1);
        }
        blk[F::G] = __builtin_ldexpf(sum, -s);
        blk[F::G + 1] = __builtin_ldexpf(1.0f, s);
    }
}

// ---- cross-lane reduction ---------------------------------------------------------------------

#define PN_DPP(v, ctrl)                                                                            \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF,  \
                                                       0xF, false))

// Sum over the 16 lanes of each DPP row; every lane of the row receives the row's sum.
__device__ __forceinline__ float row16_sum(float v)
{
    v += PN_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
    v += PN_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
    v += PN_DPP(v, 0x141);  // row_half_mirror
    v += PN_DPP(v, 0x140);  // row_mirror
    return v;
}

__device__ __forceinline__ void swap32(float &a, float &b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    a = __builtin_bit_cast(float, (unsigned)p[0]);
    b = __builtin_bit_cast(float, (unsigned)p[1]);
}

__device__ __forceinline__ void swap16(float &a, float &b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    a = __builtin_bit_cast(float, (unsigned)p[0]);
    b = __builtin_bit_cast(float, (unsigned)p[1]);
}

// Transposed reduction of V per-lane partial sums (V a multiple of 4) over the wave. Afterwards
// out[i] (i < V/4) holds, in every lane of DPP row q = lane / 16, the wave total of value
// i + q * V/4. Cost: 3V/4 swaps + 3V/4 adds + V DPP adds, i.e. 2.5 instructions per value.
template <int V>
__device__ __forceinline__ void transpose_reduce(float (&v)[V], float (&out)[V / 4])
{
    float a[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; i++) {
        float lo = v[i], hi = v[i + V / 2];
        swap32(lo, hi);  // lo = [v_i lanes 0-31 | v_(i+V/2) lanes 0-31], hi = the upper halves
        a[i] = lo + hi;  // lanes 0-31: value i, lanes 32-63: value i + V/2
    }
#pragma unroll
    for (int i = 0; i < V / 4; i++) {
        float lo = a[i], hi = a[i + V / 4];
        swap16(lo, hi);
        out[i] = row16_sum(lo + hi);
    }
}

// ---- the kernel -------------------------------------------------------------------------------

template <int R>
struct Item {
    RawBlock blk[R];
};

// Balanced contiguous row range of wave gw out of T: [begin, begin + count).
__device__ __forceinline__ void wave_rows(int64_t N, int64_t T, int64_t gw, int64_t &begin, int &count)
{
    begin = gw * N / T;
    count = (int)((gw + 1) * N / T - begin);
}

// ---- general kernel: x staged in LDS --------------------------------------------------------
// Rows are split into T = gridDim.x * waves contiguous, balanced ranges, one per wave. A wave walks
// its range R rows at a time; for each group, lane l takes blocks l, l+64, ... of the R rows (an
// "item" is one 64-block slice of R rows). Items go through a ring of D register buffers: the loads
// of item i + D - 1 are issued before item i is decoded. Each group ends with one transposed
// reduction and a store. K-phases (x larger than LDS) run as an outer loop; phases after the first
// add into y.
template <int TYPE, int M, int R, int D>
__global__ void __launch_bounds__(512) pn_gemv_kernel(const uint8_t *__restrict__ W, int64_t N,
                                                       int nb, int64_t row_bytes,
                                                       const float *__restrict__ x, int64_t K,
                                                       float *__restrict__ y, int phase_nb,
                                                       int x_vec4)
{
    using F = Fmt<TYPE>;
    constexpr int V = ((M * R + 3) / 4) * 4;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const int nwaves = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    int64_t r_begin;
    int nrows;
    wave_rows(N, (int64_t)gridDim.x * nwaves, (int64_t)blockIdx.x * nwaves + wave, r_begin, nrows);
    const int ngroups = (nrows + R - 1) / R;
    const uint8_t *wbase = W + r_begin * row_bytes;

    for (int pb = 0; pb < nb; pb += phase_nb) {
        const int pn = min(phase_nb, nb - pb);
        const int iters = (pn + 63) >> 6;
        const int nitems = ngroups * iters;

        auto load_item = [&](Item<R> &it_buf, int it) {
            it = min(it, max(nitems - 1, 0));
            const int g = it / iters, i = it - g * iters;
            const int b = min(lane + 64 * i, pn - 1);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = min(g * R + r, max(nrows - 1, 0));  // a wave may own no rows
                load_block(wbase + (int64_t)row * row_bytes + (int64_t)kBlockBytes * (pb + b),
                           it_buf.blk[r]);
            }
        };

        // Loads are never inside a branch (item indices are clamped; a clamped load re-reads a
        // block already requested, and its result is unused): the wait counts then stay exact.
        Item<R> buf[D];
#pragma unroll
        for (int p = 0; p < D - 1; p++)
            load_item(buf[p], p);  // first weights in flight while x is staged
        if (pb)
            __syncthreads();
        stage_x_raw<TYPE, M>(lds, x, K, pb, pn, x_vec4 != 0);
        __syncthreads();
        stage_x_pairs<TYPE, M>(lds, pn);
        __syncthreads();

        float acc[M][R];
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int r = 0; r < R; r++)
                acc[m][r] = 0.0f;

        auto compute_item = [&](const Item<R> &it_buf, int it) {
            const int g = it / iters, i = it - g * iters;
            const int b = lane + 64 * i;
            const bool valid = b < pn;
            const float *xb = lds + min(b, pn - 1) * F::LDS_STRIDE;
            float ah[M][R], al[M][R];
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int r = 0; r < R; r++)
                    ah[m][r] = al[m][r] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {  // word pairs (2j, 2j+1): 2 * CPW dwords of x pairs
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const uint4 *xq = reinterpret_cast<const uint4 *>(xb + m * pn * F::LDS_STRIDE +
                                                                      j * 2 * F::CPW);
                    uint32_t xv[2 * F::CPW];
#pragma unroll
                    for (int c = 0; c < 2 * F::CPW / 4; c++) {
                        const uint4 t = xq[c];
                        xv[4 * c + 0] = t.x;
                        xv[4 * c + 1] = t.y;
                        xv[4 * c + 2] = t.z;
                        xv[4 * c + 3] = t.w;
                    }
#pragma unroll
                    for (int r = 0; r < R; r++) {
                        word_dot<TYPE>(block_word(it_buf.blk[r], 2 * j), xv, ah[m][r], al[m][r]);
                        word_dot<TYPE>(block_word(it_buf.blk[r], 2 * j + 1), xv + F::CPW, ah[m][r],
                                       al[m][r]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float2 ss = *reinterpret_cast<const float2 *>(xb + m * pn * F::LDS_STRIDE + F::G);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float d = valid ? f16_bits_to_f32(block_d_bits(it_buf.blk[r])) : 0.0f;
                    const float t = __builtin_fmaf(-(float)F::Z, ss.x, ah[m][r] + al[m][r]);
                    acc[m][r] = __builtin_fmaf(d * ss.y, t, acc[m][r]);
                }
            }
            if (i == iters - 1) {  // the group's rows are complete: reduce and store
                float v[V], tot[V / 4];
#pragma unroll
                for (int o = 0; o < V; o++)
                    v[o] = (o < M * R) ? acc[(o < M * R ? o : 0) / R][o % R] : 0.0f;
                transpose_reduce<V>(v, tot);
                if ((lane & 15) == 0) {
                    const int q = lane >> 4;
#pragma unroll
                    for (int t = 0; t < V / 4; t++) {
                        const int o = t + q * (V / 4);
                        const int m = o / R, r = o - m * R;
                        const int row = g * R + r;
                        if (o < M * R && row < nrows) {
                            float *dst = y + (int64_t)m * N + r_begin + row;
                            *dst = pb ? *dst + tot[t] : tot[t];
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

        if constexpr (D == 2) {
            for (int it = 0; it < nitems; it += 2) {
                load_item(buf[1], it + 1);
                compute_item(buf[0], it);
                if (it + 1 >= nitems)
                    break;
                load_item(buf[0], it + 2);
                compute_item(buf[1], it + 1);
            }
        } else {
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
}

// ---- short rows: x in registers -----------------------------------------------------------------
// For rows of at most 64 blocks (K <= 5120 for pn3t, 4096 for pn4t) lane l always owns block l, so
// its staged x (M x G/2 hi/lo pairs, the block sum and scale) stays in registers: no LDS, no
// barrier. A wave streams its rows one at a time through a ring of D row buffers (D - 1 rows of
// loads in flight), and reduces 4 / M rows at once with the transposed reduction.
template <int TYPE, int M, int D>
__global__ void __launch_bounds__(512) pn_gemv_xreg_kernel(const uint8_t *__restrict__ W, int64_t N,
                                                            int nb, int64_t row_bytes,
                                                            const float *__restrict__ x, int64_t K,
                                                            float *__restrict__ y, int x_vec4)
{
    using F = Fmt<TYPE>;
    constexpr int RPR = 4 / M;  // rows per reduction
    static_assert(D % RPR == 0, "ring size must be a multiple of the rows per reduction");
    const int nwaves = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    int64_t r_begin;
    int nrows;
    wave_rows(N, (int64_t)gridDim.x * nwaves, (int64_t)blockIdx.x * nwaves + wave, r_begin, nrows);
    const bool active = lane < nb;
    const int b = min(lane, nb - 1);
    const uint8_t *wbase = W + r_begin * row_bytes + (int64_t)kBlockBytes * b;

    // Loads are never inside a branch (row indices are clamped to the wave's last row; a clamped
    // load re-reads a row already requested and is unused): the wait counts then stay exact.
    const int last = max(nrows - 1, 0);
    RawBlock buf[D];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        load_block(wbase + (int64_t)min(p, last) * row_bytes, buf[p]);

    uint32_t xq[M][F::G];  // (hi, lo) pair dwords of the lane's block
    float sxs[M], scl[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float *src = x + (int64_t)m * K + (int64_t)b * F::G;
        float xv[F::G];
#pragma unroll
        for (int c = 0; c < F::G / 4; c++) {
            const float4 v = x_vec4 ? reinterpret_cast<const float4 *>(src)[c]
                                    : make_float4(src[4 * c], src[4 * c + 1], src[4 * c + 2],
                                                  src[4 * c + 3]);
            xv[4 * c + 0] = v.x;
            xv[4 * c + 1] = v.y;
            xv[4 * c + 2] = v.z;
            xv[4 * c + 3] = v.w;
        }
        float sum = 0.0f, amax = 0.0f;
#pragma unroll
        for (int e = 0; e < F::G; e++) {
            sum += xv[e];
            amax = fmaxf(amax, __builtin_ldexpf(__builtin_fabsf(xv[e]), 24 - code_pos<TYPE>(e % F::CPW)));
        }
        const int s = block_shift(amax);
#pragma unroll
        for (int e = 0; e < F::G; e += 2) {
            const int sh = 24 - code_pos<TYPE>(e % F::CPW) - s;
            split_pair(__builtin_ldexpf(xv[e], sh), __builtin_ldexpf(xv[e + 1], sh), xq[m][e],
                       xq[m][e + 1]);
        }
        sxs[m] = __builtin_ldexpf(sum, -s);
        scl[m] = __builtin_ldexpf(1.0f, s);
    }

    float vals[4];
#pragma unroll
    for (int o = 0; o < 4; o++)
        vals[o] = 0.0f;

    for (int it0 = 0; it0 < nrows; it0 += D) {
#pragma unroll
        for (int s = 0; s < D; s++) {
            const int it = it0 + s;
            load_block(wbase + (int64_t)min(it + D - 1, last) * row_bytes, buf[(s + D - 1) % D]);
            if (it < nrows) {
                const float d = active ? f16_bits_to_f32(block_d_bits(buf[s])) : 0.0f;
                const int slot = s % RPR;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float ah = 0.0f, al = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        word_dot<TYPE>(block_word(buf[s], i), &xq[m][i * F::CPW], ah, al);
                    vals[slot * M + m] = (d * scl[m]) * __builtin_fmaf(-(float)F::Z, sxs[m], ah + al);
                }
                if (slot == RPR - 1 || it == nrows - 1) {
                    float tot[1];
                    transpose_reduce<4>(vals, tot);
                    if ((lane & 15) == 0) {
                        const int o = lane >> 4;  // value o = slot * M + m
                        const int j = o / M, m = o - j * M;
                        const int row = it - slot + j;
                        if (j <= slot)
                            y[(int64_t)m * N + r_begin + row] = tot[0];
                    }
#pragma unroll
                    for (int o = 0; o < 4; o++)
                        vals[o] = 0.0f;
                }
            }
        }
    }
}

constexpr int kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

struct LaunchCfg {
    int waves;  // waves per workgroup
    int grid;   // workgroups (one per CU)
};

static int num_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return 256;
        cus = prop.multiProcessorCount;
    }
    return cus;
}

// Waves per workgroup (one workgroup per CU): the count in [4, 8] whose split of the rows over all
// waves, in groups of R rows, has the smallest largest-range / mean ratio (the largest count wins
// ties). PN_GEMV_WAVES overrides it.
static LaunchCfg choose_cfg(int64_t N, int R)
{
    const int cus = num_cus();
    LaunchCfg c{8, cus};
    if (const char *e = getenv("PN_GEMV_WAVES")) {
        c.waves = atoi(e);
    } else {
        double best = 1e30;
        for (int w = 8; w >= 4; w--) {
            const int64_t T = (int64_t)cus * w;
            const double mean = (double)N / T;
            const int64_t most = (N + T - 1) / T;
            const double worst = (double)(((most + R - 1) / R) * R);
            const double ratio = worst / (mean > 0 ? mean : 1);
            if (ratio < best - 1e-9) {
                best = ratio;
                c.waves = w;
            }
        }
    }
    c.waves = c.waves < 1 ? 1 : (c.waves > 8 ? 8 : c.waves);
    return c;
}

template <int TYPE, int M, int R, int D>
static int launch_lds(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y,
                      hipStream_t s)
{
    using F = Fmt<TYPE>;
    const int nb = (int)(K / F::G);
    const int per_block = M * F::LDS_STRIDE * (int)sizeof(float);
    const int phase_nb = min(nb, kMaxLds / per_block);
    const size_t lds = (size_t)phase_nb * per_block;
    auto kern = pn_gemv_kernel<TYPE, M, R, D>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kMaxLds) != hipSuccess)
            return PN_ERR_HIP;
        attr_set = true;
    }
    const LaunchCfg c = choose_cfg(N, R);
    const int64_t T = (int64_t)c.grid * c.waves;
    const int grid = (int)(N < T ? (N + c.waves - 1) / c.waves : c.grid);
    const int vec4 = aligned(x, 16) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * c.waves), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, y, phase_nb, vec4);
    return launch_status();
}

template <int TYPE, int M, int D>
static int launch_xreg(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y,
                       hipStream_t s)
{
    using F = Fmt<TYPE>;
    const int nb = (int)(K / F::G);
    const LaunchCfg c = choose_cfg(N, 1);
    const int64_t T = (int64_t)c.grid * c.waves;
    const int grid = (int)(N < T ? (N + c.waves - 1) / c.waves : c.grid);
    const int vec4 = aligned(x, 16) ? 1 : 0;
    hipLaunchKernelGGL((pn_gemv_xreg_kernel<TYPE, M, D>), dim3((unsigned)grid), dim3(64 * c.waves),
                       0, s, W, N, nb, (int64_t)nb * kBlockBytes, x, K, y, vec4);
    return launch_status();
}

template <int TYPE>
static int dispatch_m(const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
                      hipStream_t s)
{
    const bool short_rows = K / Fmt<TYPE>::G <= 64 && !getenv("PN_GEMV_NO_XREG");
    switch (M) {
    case 1:
        return short_rows ? launch_xreg<TYPE, 1, 8>(W, N, K, x, y, s)
                          : launch_lds<TYPE, 1, 2, 4>(W, N, K, x, y, s);
    case 2:
        return short_rows ? launch_xreg<TYPE, 2, 2>(W, N, K, x, y, s)
                          : launch_lds<TYPE, 2, 2, 2>(W, N, K, x, y, s);
    case 3: return launch_lds<TYPE, 3, 1, 2>(W, N, K, x, y, s);
    default: return launch_lds<TYPE, 4, 2, 2>(W, N, K, x, y, s);
    }
}

}  // namespace pn

using namespace pn;

extern "C" int pn_gemv(int type, const void *W, int64_t N, int64_t K, const float *x, int64_t M,
                       float *y, void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (N < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (N == 0 || M == 0)
        return PN_OK;
    if (!W || !x || !y)
        return PN_ERR_NULL;
    if (!aligned(W, 2) || !aligned(x, 4) || !aligned(y, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (type == PN_TYPE_PN3T)
        return dispatch_m<PN_TYPE_PN3T>((const uint8_t *)W, N, K, x, M, y, s);
    return dispatch_m<PN_TYPE_PN4T>((const uint8_t *)W, N, K, x, M, y, s);
}
