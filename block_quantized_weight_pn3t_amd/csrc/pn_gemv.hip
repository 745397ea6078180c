// pn_gemv.hip -- decode-step GEMV y = W.x over PN blocks (pn3t, pn4t), M = 1..4 tokens, gfx950.
//
// Format: "PN weight format" (PNX-FORMAT-v0): "Block layout" (34-byte blocks, the shift rule
// BITS*(t>>1) + 16*(t&1), no code crosses a 16-bit half), "Value" (w = d * (n - z)).
//
// Design (HBM-bound; no MFMA: this is a matrix-vector product, not a dense contraction):
//  * Persistent: one workgroup of 4 or 8 waves per CU (a multiple of the CU's 4 SIMDs). Rows are
//    split into contiguous, balanced ranges, one per wave. A wave streams its rows through a ring
//    of register buffers so several rows of loads are in flight while one is decoded. Loads are
//    never inside a branch (indices are clamped), which keeps the hardware wait counts exact.
//    A block is read as 2 x 16 bytes from a 4-byte aligned address plus 2 bytes -- exactly its 34
//    bytes at either alignment parity -- and re-aligned with v_alignbit.
//  * Code extraction uses the pairing of the layout: one AND with a mask like 0x00070007 (pn3t) or
//    0x0F0F0F0F (pn4t) isolates several codes at once; the decode then uses only full-rate
//    instructions where it can (on gfx950 v_fma_mix_f32 and v_cvt_f32_f16 issue at half rate):
//    - pn4t: the masked bytes 0..15 read as E4M3 are exactly n * 2^-9, so v_cvt_pk_f32_fp8 turns
//      two codes into two fp32 values; x is staged as fp32 * 2^9 in the matching byte order.
//      Per word: 3 bit ops + 4 conversions + 8 FMA for 8 weights.
//    - pn3t, rows of <= 64 blocks (K <= 5120): a masked 16-bit half holding n << p reads as the
//      exact fp16 subnormal n * 2^(p-24), so the two codes one mask leaves form an fp16 pair for
//      v_dot2_f32_f16. x is staged as fp16 pairs x' = x * 2^(24-p-s) (s per block puts the largest
//      |x'| near 2^15), split into hi and lo halves (lo = the exact remainder), ~20 significant
//      bits. Per word: 1 shift + 5 AND + 10 DOT2 for 10 weights.
//    - pn3t, longer rows or 3-4 tokens: fp32 x staged as x * 2^(24-p) and v_fma_mix_f32 on the
//      same fp16 subnormal codes (half rate, but the staging stays a plain copy).
//  * The zero point is folded per block: sum_k (n_k - z) x_k = sum_k n_k x_k - z * sum_k x_k, with
//    the block's plain sum of x staged next to x; d (times the block's 2^s) multiplies once.
//  * fp32 accumulation; R rows x M tokens of partial sums are reduced together by a transposed
//    permlane/DPP reduction. Each output is produced by one wave in a fixed order: results are
//    deterministic (no atomics).
//  * Rows of at most 64 blocks keep the staged x of their block in registers (lane l owns block l);
//    longer rows stage x in LDS once per workgroup (in K-phases when it does not fit).
#include <stdlib.h>

#include <algorithm>

#include "pn_common.h"
#include "pn_hadamard.h"

namespace pn {

typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));

// Bit position p, inside its 16-bit half after the masking used below, of code t of a word: pn3t
// t = 0,1 and 6,7 sit at p = 0; t = 2,3 and 8,9 at p = 3; t = 4,5 at p = 6 (t = 6..9 after >> 9).
__device__ __forceinline__ int pn3t_code_pos(int t) { return 3 * ((t >> 1) % 3); }

// pn4t staging slot of code t inside its word: the conversion order (t0,t4), (t1,t5), (t2,t6),
// (t3,t7) of the bytes of w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F.
__device__ __forceinline__ int pn4t_slot(int t) { return (t < 4) ? 2 * t : 2 * (t - 4) + 1; }

__device__ __forceinline__ float dot2(uint32_t codes, uint32_t xpair, float acc)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2_t, codes),
                                  __builtin_bit_cast(h16x2_t, xpair), acc, false);
}

__device__ __forceinline__ float h_lo(uint32_t a) { return (float)__builtin_bit_cast(_Float16, (uint16_t)a); }
__device__ __forceinline__ float h_hi(uint32_t a) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(a >> 16)); }

// ---- per-word decode + multiply-accumulate ----------------------------------------------------

// pn4t, fp32 x staged * 2^9 in slot order: acc0/acc1 += sum_t n_t * x_t.
__device__ __forceinline__ void word_fp8(uint32_t w, const float *xs, float &acc0, float &acc1)
{
    const uint32_t a = w & 0x0F0F0F0Fu;         // bytes: t0 t4 t1 t5
    const uint32_t b = (w >> 4) & 0x0F0F0F0Fu;  // bytes: t2 t6 t3 t7
    const f32x2_t c0 = __builtin_amdgcn_cvt_pk_f32_fp8(a, false);
    const f32x2_t c1 = __builtin_amdgcn_cvt_pk_f32_fp8(a, true);
    const f32x2_t c2 = __builtin_amdgcn_cvt_pk_f32_fp8(b, false);
    const f32x2_t c3 = __builtin_amdgcn_cvt_pk_f32_fp8(b, true);
    acc0 = __builtin_fmaf(c0.x, xs[0], acc0);
    acc1 = __builtin_fmaf(c0.y, xs[1], acc1);
    acc0 = __builtin_fmaf(c1.x, xs[2], acc0);
    acc1 = __builtin_fmaf(c1.y, xs[3], acc1);
    acc0 = __builtin_fmaf(c2.x, xs[4], acc0);
    acc1 = __builtin_fmaf(c2.y, xs[5], acc1);
    acc0 = __builtin_fmaf(c3.x, xs[6], acc0);
    acc1 = __builtin_fmaf(c3.y, xs[7], acc1);
}

// pn3t, fp16 x pairs as (hi, lo) dwords (held in float registers): ah/al += sum_t n_t * x'hi_t /
// x'lo_t.
__device__ __forceinline__ float dot2f(uint32_t codes, float xpair, float acc)
{
    return dot2(codes, __builtin_bit_cast(uint32_t, xpair), acc);
}

__device__ __forceinline__ void word_dot2(uint32_t w, const float *xp, float &ah, float &al)
{
    const uint32_t a0 = w & 0x00070007u;  // t = 0 | t = 1   (p = 0)
    const uint32_t a1 = w & 0x00380038u;  // t = 2 | t = 3   (p = 3)
    const uint32_t a2 = w & 0x01C001C0u;  // t = 4 | t = 5   (p = 6)
    const uint32_t ws = w >> 9;
    const uint32_t a3 = ws & 0x00070007u; // t = 6 | t = 7   (p = 0)
    const uint32_t a4 = ws & 0x00380038u; // t = 8 | t = 9   (p = 3)
    ah = dot2f(a0, xp[0], ah);
    al = dot2f(a0, xp[1], al);
    ah = dot2f(a1, xp[2], ah);
    al = dot2f(a1, xp[3], al);
    ah = dot2f(a2, xp[4], ah);
    al = dot2f(a2, xp[5], al);
    ah = dot2f(a3, xp[6], ah);
    al = dot2f(a3, xp[7], al);
    ah = dot2f(a4, xp[8], ah);
    al = dot2f(a4, xp[9], al);
}

// pn3t, fp32 x staged * 2^(24-p): acc0/acc1 += sum_t n_t * x_t (mixed-precision FMA).
__device__ __forceinline__ void word_mix(uint32_t w, const float *xs, float &acc0, float &acc1)
{
    const uint32_t a0 = w & 0x00070007u;
    const uint32_t a1 = w & 0x00380038u;
    const uint32_t a2 = w & 0x01C001C0u;
    const uint32_t ws = w >> 9;
    const uint32_t a3 = ws & 0x00070007u;
    const uint32_t a4 = ws & 0x00380038u;
    acc0 = __builtin_fmaf(h_lo(a0), xs[0], acc0);
    acc1 = __builtin_fmaf(h_hi(a0), xs[1], acc1);
    acc0 = __builtin_fmaf(h_lo(a1), xs[2], acc0);
    acc1 = __builtin_fmaf(h_hi(a1), xs[3], acc1);
    acc0 = __builtin_fmaf(h_lo(a2), xs[4], acc0);
    acc1 = __builtin_fmaf(h_hi(a2), xs[5], acc1);
    acc0 = __builtin_fmaf(h_lo(a3), xs[6], acc0);
    acc1 = __builtin_fmaf(h_hi(a3), xs[7], acc1);
    acc0 = __builtin_fmaf(h_lo(a4), xs[8], acc0);
    acc1 = __builtin_fmaf(h_hi(a4), xs[9], acc1);
}

// ---- fp32 x staging in LDS (general kernel) ----------------------------------------------------
// Token m, block b of a K-phase at float offset (m*pn + b)*LDS_STRIDE: the G staged values (pn4t:
// x * 2^9 in slot order; pn3t: x * 2^(24-p) in k order), then at offset G the block's plain sum.

template <int TYPE> __device__ __forceinline__ float stage_factor(int t);
template <> __device__ __forceinline__ float stage_factor<PN_TYPE_PN3T>(int t)
{
    return __builtin_bit_cast(float, (uint32_t)(127 + 24 - pn3t_code_pos(t)) << 23);
}
template <> __device__ __forceinline__ float stage_factor<PN_TYPE_PN4T>(int)
{
    return 512.0f;
}

// 2^(p - 24): the exact inverse of the pn3t staging factor.
__device__ __forceinline__ float pn3t_unstage(int t)
{
    return __builtin_bit_cast(float, (uint32_t)(127 - 24 + pn3t_code_pos(t)) << 23);
}

template <int TYPE> __device__ __forceinline__ int stage_slot(int e)
{
    if (TYPE == PN_TYPE_PN4T)
        return (e & ~7) + pn4t_slot(e & 7);
    return e;
}

// Pass 1: coalesced 16-byte loads of four consecutive x of one block, scaled and written to their
// slots. pn4t: the 16 quads of a block are the 16 lanes of one DPP row, which also produce the
// block's plain sum (quad sums, then a fixed butterfly). pn3t (20 quads per block): see pass 2.
template <int TYPE, int M>
__device__ __forceinline__ void stage_x(float *lds, const float *__restrict__ x, int64_t K, int pb,
                                        int pn, bool vec4)
{
    using F = Fmt<TYPE>;
    constexpr int U = 8;
    const int per_tok = pn * (F::G / 4);
    const int total = M * per_tok;  // a multiple of 16
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
            if (q < total) {  // whole DPP rows are in or out (total and the row base are multiples of 16)
                const int m = q / per_tok, c = q - m * per_tok;
                const int b = (4 * c) / F::G, e = 4 * c - b * F::G;
                float *blk = lds + (m * pn + b) * F::LDS_STRIDE;
                const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; i++)
                    blk[stage_slot<TYPE>(e + i)] = vv[i] * stage_factor<TYPE>((e + i) % F::CPW);
                if (TYPE == PN_TYPE_PN4T) {
                    float s = ((vv[0] + vv[1]) + vv[2]) + vv[3];
                    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
                    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
                    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x141, 0xF, 0xF, false));
                    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x140, 0xF, 0xF, false));
                    if (e == 0)
                        blk[F::G] = s;
                }
            }
        }
    }
}

// Pass 2 (pn3t only, after a barrier): thread per (token, block) sums the block's x in k order,
// recovering each value exactly from its power-of-two-scaled copy.
template <int TYPE, int M>
__device__ __forceinline__ void stage_block_sums(float *lds, int pn)
{
    using F = Fmt<TYPE>;
    for (int q = threadIdx.x; q < M * pn; q += blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(lds + q * F::LDS_STRIDE);
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < F::G / 4; c++) {
            const float4 v = src[c];
            s += v.x * pn3t_unstage((4 * c + 0) % F::CPW);
            s += v.y * pn3t_unstage((4 * c + 1) % F::CPW);
            s += v.z * pn3t_unstage((4 * c + 2) % F::CPW);
            s += v.w * pn3t_unstage((4 * c + 3) % F::CPW);
        }
        lds[q * F::LDS_STRIDE + F::G] = s;
    }
}

// ---- kernels -------------------------------------------------------------------------------------

template <int R>
struct Item {
    RawBlock blk[R];
};


// General kernel, fp32 x staged in LDS. A wave walks its rows R at a time; for each group, lane l
// takes blocks l, l+64, ... of the R rows (an "item" is one 64-block slice of R rows). Items go
// through a ring of D register buffers: the loads of item i + D - 1 are issued before item i is
// decoded. Each group ends with one transposed reduction and a store. K-phases (x larger than LDS)
// run as an outer loop; phases after the first add into y.
template <int TYPE, int M, int R, int D>
__global__ void __launch_bounds__(512) pn_gemv_kernel(const uint8_t *__restrict__ W, int64_t N,
                                                       int nb, int64_t row_bytes,
                                                       const float *__restrict__ x, int64_t K,
                                                       float *__restrict__ y, RowSplit sp,
                                                       int phase_nb, int x_vec4, int fnum)
{
    using F = Fmt<TYPE>;
    constexpr int V = ((M * R + 3) / 4) * 4;
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const int nwaves = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    int64_t r_begin;
    int nrows;
    wave_rows(N, sp, wave, nwaves, fnum, r_begin, nrows);
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
        stage_x<TYPE, M>(lds, x, K, pb, pn, x_vec4 != 0);
        __syncthreads();
        if (TYPE == PN_TYPE_PN3T) {
            stage_block_sums<TYPE, M>(lds, pn);
            __syncthreads();
        }

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
            const int live = min(R, nrows - g * R);  // rows of the group that exist (uniform)
            const float *xb = lds + min(b, pn - 1) * F::LDS_STRIDE;
            // accumulator chains per output: NC = 8 (two words each) at M <= 2, 4 at M >= 3 (registers);
            // the codes are unsigned, so a chain's rounding error scales with sum n|x|
            constexpr int NC = M <= 2 ? 8 : 4;
            float a[NC][M][R];
#pragma unroll
            for (int c = 0; c < NC; c++)
#pragma unroll
                for (int m = 0; m < M; m++)
#pragma unroll
                    for (int r = 0; r < R; r++)
                        a[c][m][r] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {  // word pairs (2j, 2j+1)
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float4 *xq = reinterpret_cast<const float4 *>(xb + m * pn * F::LDS_STRIDE +
                                                                        j * 2 * F::CPW);
                    float xv[2 * F::CPW];
#pragma unroll
                    for (int c = 0; c < 2 * F::CPW / 4; c++) {
                        const float4 t = xq[c];
                        xv[4 * c + 0] = t.x;
                        xv[4 * c + 1] = t.y;
                        xv[4 * c + 2] = t.z;
                        xv[4 * c + 3] = t.w;
                    }
#pragma unroll
                    for (int r = 0; r < R; r++) {
                        if (r < live) {
                            const uint32_t w0 = block_word(it_buf.blk[r], 2 * j);
                            const uint32_t w1 = block_word(it_buf.blk[r], 2 * j + 1);
                            const int c0 = (2 * j) % NC, c1 = (2 * j + 2) % NC;  // chain pairs
                            if (TYPE == PN_TYPE_PN4T) {
                                word_fp8(w0, xv, a[c0][m][r], a[c0 + 1][m][r]);
                                word_fp8(w1, xv + F::CPW, a[c1][m][r], a[c1 + 1][m][r]);
                            } else {
                                word_mix(w0, xv, a[c0][m][r], a[c0 + 1][m][r]);
                                word_mix(w1, xv + F::CPW, a[c1][m][r], a[c1 + 1][m][r]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float sx = xb[m * pn * F::LDS_STRIDE + F::G];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const float d = valid ? f16_bits_to_f32(block_d_bits(it_buf.blk[r])) : 0.0f;
                    float t = 0.0f;
#pragma unroll
                    for (int c = 0; c < NC; c += 2)
                        t += a[c][m][r] + a[c + 1][m][r];
                    acc[m][r] = __builtin_fmaf(d, __builtin_fmaf(-(float)F::Z, sx, t), acc[m][r]);
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

// ---- x as fp16 hi/lo pairs ------------------------------------------------------------------

// fp16 hi/lo pair of two staged values. hi is x' with its fp32 significand cut to fp16 width
// (exactly an fp16 value in fp16's normal range; below it, 0); lo = x' - hi is exact in fp32 and
// is converted with truncation. Relative error of hi + lo: below 2^-20 for |x'| >= 2^-14.
__device__ __forceinline__ void split_pair(float a, float b, float &hi, float &lo)
{
    const float ha = (__builtin_fabsf(a) >= 0x1p-14f)
                         ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFFE000u)
                         : 0.0f;
    const float hb = (__builtin_fabsf(b) >= 0x1p-14f)
                         ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) & 0xFFFFE000u)
                         : 0.0f;
    hi = __builtin_bit_cast(float, __builtin_amdgcn_cvt_pkrtz(ha, hb));
    lo = __builtin_bit_cast(float, __builtin_amdgcn_cvt_pkrtz(a - ha, b - hb));
}

// Scale exponent of a block: s such that max_e |x_e| * 2^(24 - p_e - s) lies in [2^14, 2^15).
__device__ __forceinline__ int block_shift(float amax_scaled)
{
    if (!(amax_scaled > 0.0f) || !(amax_scaled < __builtin_inff()))
        return 0;  // all zero, or non-finite input (the result is then non-finite too)
    return __builtin_amdgcn_frexp_expf(amax_scaled) - 15;
}

// ---- long rows: flat partition over (row group, block) ------------------------------------------

// pn4t with x in natural k order (x * 2^9): the conversions yield the codes in the order (t0,t4),
// (t1,t5), (t2,t6), (t3,t7), and each is paired with its own x.
__device__ __forceinline__ void word_fp8n(uint32_t w, const float *xn, float &acc0, float &acc1)
{
    const uint32_t a = w & 0x0F0F0F0Fu;         // bytes: t0 t4 t1 t5
    const uint32_t b = (w >> 4) & 0x0F0F0F0Fu;  // bytes: t2 t6 t3 t7
    const f32x2_t c0 = __builtin_amdgcn_cvt_pk_f32_fp8(a, false);
    const f32x2_t c1 = __builtin_amdgcn_cvt_pk_f32_fp8(a, true);
    const f32x2_t c2 = __builtin_amdgcn_cvt_pk_f32_fp8(b, false);
    const f32x2_t c3 = __builtin_amdgcn_cvt_pk_f32_fp8(b, true);
    acc0 = __builtin_fmaf(c0.x, xn[0], acc0);
    acc1 = __builtin_fmaf(c0.y, xn[4], acc1);
    acc0 = __builtin_fmaf(c1.x, xn[1], acc0);
    acc1 = __builtin_fmaf(c1.y, xn[5], acc1);
    acc0 = __builtin_fmaf(c2.x, xn[2], acc0);
    acc1 = __builtin_fmaf(c2.y, xn[6], acc1);
    acc0 = __builtin_fmaf(c3.x, xn[3], acc0);
    acc1 = __builtin_fmaf(c3.y, xn[7], acc1);
}

constexpr int kFlatWaves = 8;  // waves per workgroup of the flat kernel (two per SIMD)

// Rows of more than 64 blocks, x fully resident in LDS (one K-phase), M = 1..2.
//
// Work split: the rows are taken R at a time ("groups"); a workgroup owns a balanced, contiguous
// range of groups, and the (group, block) pairs of that range, in row-major order, are cut into
// kFlatWaves contiguous pieces, one per wave. Each SIMD gets a quarter; the instruction arbiter
// favours the older of the two waves on a SIMD, so that wave takes the larger part (fnum/16; 10/16
// measured best), the younger one the rest. A wave walks its piece 64 blocks at a time
// (lane l takes the l-th block of each "item"); since a group has at least 64 blocks an item spans
// at most two groups, so each lane keeps two accumulator sets, for the item's first group and the
// next one. When the walk leaves a group, the group's sums are reduced across the wave: a group
// that lies wholly inside the piece is stored to y; the (at most two) groups at the piece's ends
// are written to LDS and, after a barrier, summed over the waves that share them, lowest wave
// first. Every output thus has one fixed summation order (deterministic), and only the last item
// of a piece is partly idle.
//
// Staging: all x loads of the workgroup are issued before the first weight loads, so waiting for
// x never waits for weights (the memory counter retires loads in order).
// ROT: x is first rotated, x' = H_B x / sqrt(B) on slices of B = 2^hL elements (the Hadamard
// rotation of "Files that use PN", as read in pn_hadamard.h), in the registers that hold it
// (stages 0-7) and through the x area of LDS (stages 8 and up), before it is staged.
template <int TYPE, int M, int R, int D, int QPT, bool ROT>
__device__ __forceinline__ void flat_body(const uint8_t *__restrict__ W, int64_t N,
                                                            int nb, int64_t row_bytes,
                                                            const float *__restrict__ x, int64_t K,
                                                            float *__restrict__ y, int64_t gq,
                                                            int gr, int x_vec4, int fnum, int hL,
                                                            float hscale, int blk_id)
{
    using F = Fmt<TYPE>;
    constexpr int V = ((M * R + 3) / 4) * 4;
    constexpr int QB = F::G / 4;  // 16-byte pieces of x per block
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);  // staged x: [M][nb][LDS_STRIDE]
    float *part = lds + M * nb * F::LDS_STRIDE;    // partial sums: [kFlatWaves][2][V]
    int *meta = reinterpret_cast<int *>(part + kFlatWaves * 2 * V);  // [kFlatWaves][4]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // this workgroup's groups [P0, P1) and this wave's piece [F0, F1) of its (group, block) pairs
    // (gq, gr: quotient and remainder of the group count by the grid, from the host)
    const int blk = blk_id;
    const int64_t P0 = (int64_t)blk * gq + min(blk, gr);
    const int T = (int)(gq + (blk < gr ? 1 : 0)) * nb;  // < 2^30 (checked on the host)
    // SIMD j = wave & 3 takes the quarter [q0, q1) of the range; its older wave (h = 0) the first
    // fnum/16 of it, the younger wave (h = 1) the rest.
    const int sj = wave & 3, sh = wave >> 2;
    const int q0 = (int)(((int64_t)sj * T) >> 2), q1 = (int)(((int64_t)(sj + 1) * T) >> 2);
    const int qm = q0 + (int)(((int64_t)(q1 - q0) * fnum) >> 4);
    const int F0 = sh ? qm : q0;
    const int F1 = sh ? q1 : qm;
    const int L = F1 - F0;
    const int nitems = (L + 63) >> 6;
    const int pf = (int)((uint32_t)F0 / (uint32_t)nb);  // first group of the piece (relative to P0)
    const int pl = L > 0 ? (int)((uint32_t)(F1 - 1) / (uint32_t)nb) : pf;  // last group
    const int be = L > 0 ? (F1 - 1) - pl * nb : 0;  // block of the piece's last pair

    // 1. x loads: nq = ceil(total / 512) per thread (at most QPT), under a uniform branch so that
    // no load is issued past the last round. The weight loads issued next are unconditional, so
    // waiting for x never waits for them.
    const int per_tok = nb * QB;
    const int total = M * per_tok;
    // ROT: thread (wave w, lane l) takes, for u = 4 g + j, the float4 at
    // 256 (w + 8 g) + 64 j + l: a wave holds whole 1024-element pieces of x, 4 float4 per lane
    // 256 elements apart, so the rotation's stages 8-9 stay in registers. Otherwise l + 512 u.
    const int nq = ROT ? 4 * ((total + 256 * kFlatWaves - 1) / (256 * kFlatWaves))
                       : (total + kFlatWaves * 64 - 1) / (kFlatWaves * 64);
    auto qpos = [&](int u) {
        return ROT ? 256 * (wave + kFlatWaves * (u >> 2)) + 64 * (u & 3) + lane
                   : (int)threadIdx.x + u * kFlatWaves * 64;
    };
    // Each workgroup walks x from its own starting block (rotated by the workgroup index) so that
    // the CUs of an XCD do not all request the same lines of x, i.e. the same L2 channel, at once.
    // (with ROT by whole 1024-element pieces, which its waves transform: 256 float4 units, where
    // x holds a whole number of them)
    const int rot = !ROT ? (int)(((uint32_t)blk_id * 17u) % (uint32_t)(M * nb)) * QB
                    : (total & 255) ? 0
                                    : (int)(((uint32_t)blk_id * 17u) % (uint32_t)(total >> 8)) * 256;
    auto rotq = [&](int q) { q += rot; return q >= total ? q - total : q; };
    auto token_of = [](int q, int per) {  // q / per for q < M * per, without a division
        int m = 0;
#pragma unroll
        for (int i = 1; i < M; i++)
            m += q >= i * per ? 1 : 0;
        return m;
    };
    float4 xv[QPT];
#pragma unroll
    for (int u = 0; u < QPT; u++) {
        if (u < nq) {
            const int q = rotq(min(qpos(u), total - 1));
            const int m = token_of(q, per_tok);
            const float *src = x + (int64_t)m * K + 4 * (q - m * per_tok);
            xv[u] = x_vec4 ? *reinterpret_cast<const float4 *>(src)
                           : make_float4(src[0], src[1], src[2], src[3]);
        } else if (ROT) {
            xv[u] = make_float4(0.f, 0.f, 0.f, 0.f);  // transformed with the rest, never staged
        }
    }

    // 2. first weight loads. Item positions come from uniform cursors (group, block of the item's
    // first pair); a lane past the piece's end re-reads the piece's last pair (the result is
    // unused), and item indices past the last item are clamped, so no load is ever inside a
    // branch and no load leaves the matrix.
    auto load_item = [&](Item<R> &buf, int itc, int pu, int bu) {
        int b = bu + lane, p = pu;
        if (b >= nb) {
            b -= nb;
            p += 1;
        }
        if (64 * itc + lane >= L) {
            p = pl;
            b = be;
        }
        const int64_t row0 = R * (P0 + p);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = min(row0 + r, N - 1);
            load_block(W + row * row_bytes + (int64_t)kBlockBytes * b, buf.blk[r]);
        }
    };
    int lp = pf, lb = F0 - pf * nb, lit = 0;  // load cursor, at item lit
    auto load_next = [&](Item<R> &buf, int it) {
        const int itc = min(it, max(nitems - 1, 0));
        if (lit < itc) {  // uniform; advances by at most one item per call
            lb += 64;
            if (lb >= nb) {
                lb -= nb;
                lp += 1;
            }
            lit += 1;
        }
        load_item(buf, itc, lp, lb);
    };
    Item<R> buf[D];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        load_next(buf[p], p);

    // 2b. the rotation (ROT), while those loads are in flight: lanes hold consecutive float4 of x,
    // so a wave holds 256 consecutive elements at a multiple of 256, and slices never straddle
    // tokens (B divides K). Lanes past the end hold a clamped copy, in slices of their own.
    if constexpr (ROT) {
        // four float4 at a time (their lane exchanges in flight together), only as many as hold x
#pragma unroll
        for (int g0 = 0; g0 < QPT; g0 += 4)
            if (g0 < nq) {  // uniform
                float4(&v4)[4] = *reinterpret_cast<float4(*)[4]>(&xv[g0]);
                hadamard_wave_n<4>(v4, hL, hscale);
                hadamard_regs_8_9(v4, hL, hscale);
            }
        if (hL > 10) {  // uniform
            lds_f32 *hb = (lds_f32 *)lds;
#pragma unroll
            for (int u = 0; u < QPT; u++) {
                const int q0 = qpos(u);
                if (u < nq && q0 < total) {
                    const int q = rotq(q0);
                    hb[4 * q + 0] = xv[u].x;
                    hb[4 * q + 1] = xv[u].y;
                    hb[4 * q + 2] = xv[u].z;
                    hb[4 * q + 3] = xv[u].w;
                }
            }
            hadamard_lds_stages<kFlatWaves * 64>(hb, 4 * total, hL, hscale, 10);
#pragma unroll
            for (int u = 0; u < QPT; u++) {
                const int q = rotq(min(qpos(u), total - 1));
                if (u < nq)
                    xv[u] = make_float4(hb[4 * q], hb[4 * q + 1], hb[4 * q + 2], hb[4 * q + 3]);
            }
            __syncthreads();  // step 3 writes the same area
        }
    }

    // 3. stage x: pn4t x * 2^9 in k order, the block's plain sum at offset G (a DPP row of 16
    // lanes holds one block); pn3t x * 2^(24-p), sums in a second pass.
#pragma unroll
    for (int u = 0; u < QPT; u++) {
        const int q0 = qpos(u);
        if (u < nq && q0 < total) {  // pn4t: whole DPP rows are in or out (total and row bases are multiples of 16)
            const int q = rotq(q0);  // a whole-block rotation keeps each DPP row on one block
            const int m = token_of(q, per_tok);
            const int c = q - m * per_tok;
            const int b = c / QB, e = 4 * (c - b * QB);
            float *blk = lds + (m * nb + b) * F::LDS_STRIDE;
            const float4 v = xv[u];
            if (TYPE == PN_TYPE_PN4T) {
                *reinterpret_cast<float4 *>(blk + e) =
                    make_float4(v.x * 512.0f, v.y * 512.0f, v.z * 512.0f, v.w * 512.0f);
                float s = ((v.x + v.y) + v.z) + v.w;
                s += PN_DPP(s, 0xB1);
                s += PN_DPP(s, 0x4E);
                s += PN_DPP(s, 0x141);
                s += PN_DPP(s, 0x140);
                if (e == 0)
                    blk[F::G] = s;
            } else {
                *reinterpret_cast<float4 *>(blk + e) =
                    make_float4(v.x * stage_factor<TYPE>((e + 0) % F::CPW),
                                v.y * stage_factor<TYPE>((e + 1) % F::CPW),
                                v.z * stage_factor<TYPE>((e + 2) % F::CPW),
                                v.w * stage_factor<TYPE>((e + 3) % F::CPW));
            }
        }
    }
    if (lane == 0) {
        meta[wave * 4 + 0] = F0;
        meta[wave * 4 + 1] = F1;
        meta[wave * 4 + 2] = pf;
        meta[wave * 4 + 3] = pl;
    }
    __syncthreads();
    if (TYPE == PN_TYPE_PN3T) {
        stage_block_sums<TYPE, M>(lds, nb);
        __syncthreads();
    }

    // 4. stream the piece
    float accA[M][R], accB[M][R];
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int r = 0; r < R; r++)
            accA[m][r] = accB[m][r] = 0.0f;
    int pc = pf, bc = F0 - pf * nb;  // compute cursor

    auto flush = [&](int p) {  // group p is done in this wave: reduce accA and store it
        float v[V], tot[V / 4];
#pragma unroll
        for (int o = 0; o < V; o++)
            v[o] = (o < M * R) ? accA[(o < M * R ? o : 0) / R][o % R] : 0.0f;
        transpose_reduce<V>(v, tot);
        const bool complete = F0 <= p * nb && (p + 1) * nb <= F1;
        if ((lane & 15) == 0) {
            const int q = lane >> 4;
#pragma unroll
            for (int t = 0; t < V / 4; t++) {
                const int o = t + q * (V / 4);
                if (o < M * R) {
                    const int m = o / R, r = o - m * R;
                    if (complete) {
                        const int64_t row = R * (P0 + p) + r;
                        if (row < N)
                            y[(int64_t)m * N + row] = tot[t];
                    } else {
                        part[(wave * 2 + (p == pf ? 0 : 1)) * V + o] = tot[t];
                    }
                }
            }
        }
    };

    auto compute_item = [&](const Item<R> &it_buf, int it) {
        int b = bc + lane;
        const bool second = b >= nb;
        if (second)
            b -= nb;
        const bool valid = 64 * it + lane < L;
        const float *xb = lds + (valid ? b : 0) * F::LDS_STRIDE;
        // eight accumulator chains per output (two words each): the codes are unsigned, so a
        // chain's rounding error scales with sum n|x|, not sum |n - z||x|
        float a[8][M][R];
#pragma unroll
        for (int c = 0; c < 8; c++)
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int r = 0; r < R; r++)
                    a[c][m][r] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {  // word pairs (2j, 2j+1)
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float4 *xq = reinterpret_cast<const float4 *>(xb + m * nb * F::LDS_STRIDE +
                                                                    j * 2 * F::CPW);
                float xw[2 * F::CPW];
#pragma unroll
                for (int c = 0; c < 2 * F::CPW / 4; c++) {
                    const float4 t = xq[c];
                    xw[4 * c + 0] = t.x;
                    xw[4 * c + 1] = t.y;
                    xw[4 * c + 2] = t.z;
                    xw[4 * c + 3] = t.w;
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const uint32_t w0 = block_word(it_buf.blk[r], 2 * j);
                    const uint32_t w1 = block_word(it_buf.blk[r], 2 * j + 1);
                    const int c0 = (4 * j) % 8, c1 = (4 * j + 2) % 8;  // chain pairs of words 2j, 2j+1
                    if (TYPE == PN_TYPE_PN4T) {
                        word_fp8n(w0, xw, a[c0][m][r], a[c0 + 1][m][r]);
                        word_fp8n(w1, xw + F::CPW, a[c1][m][r], a[c1 + 1][m][r]);
                    } else {
                        word_mix(w0, xw, a[c0][m][r], a[c0 + 1][m][r]);
                        word_mix(w1, xw + F::CPW, a[c1][m][r], a[c1 + 1][m][r]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float sx = xb[m * nb * F::LDS_STRIDE + F::G];  // the block's plain sum of x
#pragma unroll
            for (int r = 0; r < R; r++) {
                // d is selected, not multiplied by a mask, so a non-finite d stays in its own row
                const float d = f16_bits_to_f32(block_d_bits(it_buf.blk[r]));
                const float dA = (valid && !second) ? d : 0.0f;
                const float dB = (valid && second) ? d : 0.0f;
                const float sn = ((a[0][m][r] + a[1][m][r]) + (a[2][m][r] + a[3][m][r])) +
                                 ((a[4][m][r] + a[5][m][r]) + (a[6][m][r] + a[7][m][r]));
                const float t = __builtin_fmaf(-(float)F::Z, sx, sn);
                accA[m][r] = __builtin_fmaf(dA, t, accA[m][r]);
                accB[m][r] = __builtin_fmaf(dB, t, accB[m][r]);
            }
        }
        bc += 64;  // advance the compute cursor; leaving group pc completes it
        if (bc >= nb) {
            bc -= nb;
            flush(pc);
#pragma unroll
            for (int m = 0; m < M; m++)
#pragma unroll
                for (int r = 0; r < R; r++) {
                    accA[m][r] = accB[m][r];
                    accB[m][r] = 0.0f;
                }
            pc += 1;
        }
    };

    if constexpr (D == 2) {
        for (int it = 0; it < nitems; it += 2) {
            load_next(buf[1], it + 1);
            compute_item(buf[0], it);
            if (it + 1 >= nitems)
                break;
            load_next(buf[0], it + 2);
            compute_item(buf[1], it + 1);
        }
    } else {
        for (int it0 = 0; it0 < nitems; it0 += D) {
#pragma unroll
            for (int s = 0; s < D; s++) {
                const int it = it0 + s;
                load_next(buf[(s + D - 1) % D], it + D - 1);
                if (it < nitems)
                    compute_item(buf[s], it);
            }
        }
    }
    if (nitems > 0 && pc <= pl)
        flush(pc);
    __syncthreads();

    // 5. groups shared by several waves: the lowest wave that touches one sums the partials of
    // every wave that touches it, in wave order. meta[w] = (F0, F1, first group, last group).
    if (threadIdx.x < 2 * kFlatWaves) {
        const int w = threadIdx.x >> 1, s = threadIdx.x & 1;
        const int4 *m4 = reinterpret_cast<const int4 *>(meta);
        int4 mm[kFlatWaves];
#pragma unroll
        for (int w2 = 0; w2 < kFlatWaves; w2++)
            mm[w2] = m4[w2];
        const int4 me = m4[w];
        const int p = s ? me.w : me.z;
        auto touches = [&](const int4 &q) { return q.y > q.x && q.z <= p && p <= q.w; };
        bool own = me.y > me.x && !(s == 1 && me.w == me.z);
        own = own && !(me.x <= p * nb && (p + 1) * nb <= me.y);  // complete: already stored
#pragma unroll
        for (int w2 = 0; w2 < kFlatWaves; w2++)
            if (w2 < w && touches(mm[w2]))
                own = false;
        if (own) {
            float tot[M * R];
#pragma unroll
            for (int o = 0; o < M * R; o++)
                tot[o] = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < kFlatWaves; w2++) {
                if (w2 >= w && touches(mm[w2])) {
                    const float *src = part + (w2 * 2 + (p == mm[w2].z ? 0 : 1)) * V;
#pragma unroll
                    for (int o = 0; o < M * R; o++)
                        tot[o] += src[o];
                }
            }
#pragma unroll
            for (int o = 0; o < M * R; o++) {
                const int m = o / R, r = o - m * R;
                const int64_t row = R * (P0 + p) + r;
                if (row < N)
                    y[(int64_t)m * N + row] = tot[o];
            }
        }
    }
}
template <int TYPE, int M, int R, int D, int QPT, bool ROT>
__global__ void __launch_bounds__(512) pn_gemv_flat_kernel(const uint8_t *__restrict__ W, int64_t N,
                                                            int nb, int64_t row_bytes,
                                                            const float *__restrict__ x, int64_t K,
                                                            float *__restrict__ y, int64_t gq,
                                                            int gr, int x_vec4, int fnum, int hL,
                                                            float hscale)
{
    flat_body<TYPE, M, R, D, QPT, ROT>(W, N, nb, row_bytes, x, K, y, gq, gr, x_vec4, fnum, hL,
                                       hscale, (int)blockIdx.x);
}

// ---- short rows: staged x in registers ----------------------------------------------------------

// Rows of at most 64 blocks (K <= 5120 for pn3t, 4096 for pn4t): lane l always owns block l, so
// its staged x stays in registers: no LDS, no barrier. pn3t keeps fp16 hi/lo pairs (dot2 decode);
// pn4t keeps fp32 * 2^9 in slot order (fp8-conversion decode). A wave streams its rows one at a
// time through a ring of D row buffers (D - 1 rows of loads in flight) and reduces 4 / M rows at
// once with the transposed reduction.
// ROT: x is first rotated into LDS, x' = H_B x / sqrt(B) on slices of B = 2^hL elements (the
// Hadamard rotation of "Files that use PN", as read in pn_hadamard.h); the staging then reads x'.
template <int TYPE, int M, int D, bool ROT>
__device__ __forceinline__ void xreg_body(const uint8_t *__restrict__ W, int64_t N,
                                                            int nb, int64_t row_bytes,
                                                            const float *__restrict__ x, int64_t K,
                                                            float *__restrict__ y, RowSplit sp,
                                                            int x_vec4, int fnum, int hL,
                                                            float hscale, int blk_id)
{
    using F = Fmt<TYPE>;
    constexpr int RPR = 4 / M;  // rows per reduction
    static_assert(D % RPR == 0, "ring size must be a multiple of the rows per reduction");
    const int nwaves = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t r_begin;
    int nrows;
    wave_rows(N, sp, wave, nwaves, fnum, r_begin, nrows, blk_id);
    const bool active = lane < nb;
    const int b = min(lane, nb - 1);
    const uint8_t *wbase = W + r_begin * row_bytes + (int64_t)kBlockBytes * b;

    // Cooperative staging, 512 threads: thread t takes word t & 7 of block t >> 3 of every token.
    // The x loads are issued before the first weight loads, so waiting for x never waits for
    // weights (the memory counter retires loads in order).
    // (blocks taken in an order rotated by the workgroup index, as in the long-row kernel)
    const int bb = ((threadIdx.x >> 3) + blk_id * 5) & 63, i = threadIdx.x & 7;
    const bool have = bb < nb;
    float xv[M][F::CPW];
    auto load_x = [&](const float *xs, int vec) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float *src = xs + (int64_t)m * K + (int64_t)min(bb, nb - 1) * F::G + i * F::CPW;
#pragma unroll
            for (int t = 0; t < F::CPW; t += 2) {
                const float2 p = vec ? *reinterpret_cast<const float2 *>(src + t)
                                     : make_float2(src[t], src[t + 1]);
                xv[m][t] = have ? p.x : 0.0f;
                xv[m][t + 1] = have ? p.y : 0.0f;
            }
        }
    };
    // ROT: x as float4 per lane, thread (wave w, lane l) taking for u = 4 g + j the float4 at
    // 256 (w + 8 g) + 64 j + l: a wave holds whole 1024-element pieces, 4 float4 per lane 256
    // elements apart, so the rotation's stages 0-9 stay in registers (at most 64 blocks of M
    // tokens over 8 waves)
    constexpr int HQ = ROT ? 4 * ((M * 64 * F::G / 4 + 2047) / 2048) : 1;
    const int total4 = (int)(M * K / 4), nh = 4 * ((total4 + 2047) >> 11);
    auto hpos = [&](int u) { return 256 * (wave + 8 * (u >> 2)) + 64 * (u & 3) + lane; };
    // workgroups start at different 1024-element pieces of x (as the plain staging rotates its
    // blocks), so that the CUs of an XCD do not request the same lines at once
    const int hrot = (!ROT || (total4 & 255)) ? 0
                     : (int)(((uint32_t)blk_id * 5u) % (uint32_t)(total4 >> 8)) * 256;
    auto hq = [&](int q) { q += hrot; return q >= total4 ? q - total4 : q; };
    float4 hv[HQ];
    if constexpr (ROT) {
#pragma unroll
        for (int u = 0; u < HQ; u++) {
            const float *src = x + 4 * hq(min(hpos(u), total4 - 1));
            if (u < nh)
                hv[u] = x_vec4 ? *reinterpret_cast<const float4 *>(src)
                               : make_float4(src[0], src[1], src[2], src[3]);
            else
                hv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        load_x(x, x_vec4);
    }

    // Loads are never inside a branch (row indices are clamped to the wave's last row; a clamped
    // load re-reads a row already requested and is unused): the wait counts then stay exact.
    const int last = max(nrows - 1, 0);
    RawBlock buf[D];
#pragma unroll
    for (int p = 0; p < D - 1; p++)
        load_block(wbase + (int64_t)min(p, last) * row_bytes, buf[p]);

    if constexpr (ROT) {  // the rotation, while the weight loads are in flight
        extern __shared__ float4 hx_dyn[];  // M * K floats
        lds_f32 *hb = (lds_f32 *)(float *)hx_dyn;
#pragma unroll
        for (int g0 = 0; g0 < HQ; g0 += 4)
            if (g0 < nh) {  // uniform
                float4(&v4)[4] = *reinterpret_cast<float4(*)[4]>(&hv[g0]);
                hadamard_wave_n<4>(v4, hL, hscale);
                hadamard_regs_8_9(v4, hL, hscale);
            }
#pragma unroll
        for (int u = 0; u < HQ; u++) {
            const int q0 = hpos(u);
            if (u < nh) {
                if (q0 < total4) {
                    const int q = hq(q0);
                    hb[4 * q + 0] = hv[u].x;
                    hb[4 * q + 1] = hv[u].y;
                    hb[4 * q + 2] = hv[u].z;
                    hb[4 * q + 3] = hv[u].w;
                }
            }
        }
        if (hL > 10)
            hadamard_lds_stages<512>(hb, 4 * total4, hL, hscale, 10);
        else
            __syncthreads();
        load_x((const float *)hx_dyn, 1);
    }

    // The block's amax and sum by a DPP butterfly over its 8 lanes; the staged words go to LDS,
    // then every lane lifts its own block into registers.
    __shared__ float4 stage4[M * 64 * F::LDS_STRIDE / 4];
    float *stage = reinterpret_cast<float *>(stage4);
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float *v = xv[m];
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < F::CPW; t++)
            sum += v[t];
        sum += PN_DPP(sum, 0xB1);   // lanes xor 1
        sum += PN_DPP(sum, 0x4E);   // lanes xor 2
        sum += PN_DPP(sum, 0x141);  // the mirror half of the 8-lane group
        float *blk = stage + (m * 64 + bb) * F::LDS_STRIDE;
        if (TYPE == PN_TYPE_PN3T) {
            float amax = 0.0f;
#pragma unroll
            for (int t = 0; t < F::CPW; t++)
                amax = fmaxf(amax, __builtin_fabsf(v[t]) * stage_factor<PN_TYPE_PN3T>(t));
            amax = fmaxf(amax, PN_DPP(amax, 0xB1));
            amax = fmaxf(amax, PN_DPP(amax, 0x4E));
            amax = fmaxf(amax, PN_DPP(amax, 0x141));
            const int sh = block_shift(amax);
            const float down = __builtin_ldexpf(1.0f, -sh);
            float4 o[3];
            float *of = reinterpret_cast<float *>(o);
#pragma unroll
            for (int t = 0; t < F::CPW; t += 2) {
                const float f = stage_factor<PN_TYPE_PN3T>(t) * down;
                split_pair(v[t] * f, v[t + 1] * f, of[t], of[t + 1]);
            }
            float *dst = blk + i * F::CPW;  // 10 dwords at an 8-byte aligned offset
#pragma unroll
            for (int t = 0; t < F::CPW; t += 2)
                *reinterpret_cast<float2 *>(dst + t) = make_float2(of[t], of[t + 1]);
            if (i == 0)
                *reinterpret_cast<float2 *>(blk + F::G) =
                    make_float2(sum * down, __builtin_ldexpf(1.0f, sh));
        } else {
            float4 o[2];
            float *of = reinterpret_cast<float *>(o);
#pragma unroll
            for (int t = 0; t < F::CPW; t++)
                of[pn4t_slot(t)] = v[t] * 512.0f;
            float4 *dst = reinterpret_cast<float4 *>(blk + i * F::CPW);
            dst[0] = o[0];
            dst[1] = o[1];
            if (i == 0)
                *reinterpret_cast<float2 *>(blk + F::G) = make_float2(sum, 1.0f);
        }
    }
    __syncthreads();

    float xq[M][F::G];  // pn3t: (hi, lo) fp16 pair dwords; pn4t: fp32 * 2^9 in slot order
    float sxs[M], scl[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float4 *blk = reinterpret_cast<const float4 *>(stage + (m * 64 + lane) * F::LDS_STRIDE);
#pragma unroll
        for (int c = 0; c < F::G / 4; c++) {
            const float4 t = blk[c];
            xq[m][4 * c + 0] = t.x;
            xq[m][4 * c + 1] = t.y;
            xq[m][4 * c + 2] = t.z;
            xq[m][4 * c + 3] = t.w;
        }
        const float2 ss = *reinterpret_cast<const float2 *>(stage + (m * 64 + lane) * F::LDS_STRIDE + F::G);
        sxs[m] = ss.x;
        scl[m] = ss.y;
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
                    // Eight accumulator chains of two words each: the codes are unsigned (the
                    // zero point is folded in below), so a chain's rounding error scales with
                    // sum n|x|, not sum |n - z||x|; short chains keep it well inside the bound.
                    float a[8];
#pragma unroll
                    for (int c = 0; c < 8; c++)
                        a[c] = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const uint32_t w = block_word(buf[s], i);
                        const int c = 2 * (i & 3);
                        if (TYPE == PN_TYPE_PN3T)
                            word_dot2(w, &xq[m][i * F::CPW], a[c], a[c + 1]);
                        else
                            word_fp8(w, &xq[m][i * F::CPW], a[c], a[c + 1]);
                    }
                    const float t = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
                    vals[slot * M + m] = (d * scl[m]) * __builtin_fmaf(-(float)F::Z, sxs[m], t);
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
template <int TYPE, int M, int D, bool ROT>
__global__ void __launch_bounds__(512) pn_gemv_xreg_kernel(const uint8_t *__restrict__ W, int64_t N,
                                                            int nb, int64_t row_bytes,
                                                            const float *__restrict__ x, int64_t K,
                                                            float *__restrict__ y, RowSplit sp,
                                                            int x_vec4, int fnum, int hL,
                                                            float hscale)
{
    xreg_body<TYPE, M, D, ROT>(W, N, nb, row_bytes, x, K, y, sp, x_vec4, fnum, hL, hscale,
                               (int)blockIdx.x);
}

// ---- host side ----------------------------------------------------------------------------------

constexpr int kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

struct LaunchCfg {
    int waves;  // waves per workgroup
    int grid;   // workgroups (one per CU)
};

// Share of a SIMD's work given to the older of its two waves, in sixteenths (PN_GEMV_SPLIT).
// Measured best: 12/16 for the short-row kernel, 10/16 for the long-row kernel.
static int older_share(int dflt)
{
    const char *e = getenv("PN_GEMV_SPLIT");
    const int v = e ? atoi(e) : dflt;
    return v < 4 ? 4 : v > 15 ? 15 : v;
}

static int num_cus() { return device_cus(); }

// Waves per workgroup (one workgroup per CU): 8 (two per SIMD, so one wave's memory waits overlap
// the other's arithmetic) unless the rows are too few to give every wave a group of R. Rows are
// split per SIMD (see wave_rows), so either count keeps the SIMDs balanced. PN_GEMV_WAVES (4 or 8)
// overrides it.
static LaunchCfg choose_cfg(int64_t N, int R)
{
    const int cus = num_cus();
    LaunchCfg c{8, cus};
    if (const char *e = getenv("PN_GEMV_WAVES"))
        c.waves = atoi(e) <= 4 ? 4 : 8;
    else if (N < (int64_t)cus * 8 * R)
        c.waves = 4;
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
    constexpr auto kern = pn_gemv_kernel<TYPE, M, R, D>;
    if (!lds_limit_once<kern>(kMaxLds))
        return PN_ERR_HIP;
    const LaunchCfg c = choose_cfg(N, R);
    const int grid = (int)std::min<int64_t>(c.grid, (N + 3) / 4);
    const int vec4 = aligned(x, 16) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * c.waves), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, y, row_split(N, grid), phase_nb, vec4, 8);
    return launch_status();
}

template <int TYPE, int M, int D, bool ROT = false>
static int launch_xreg(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y,
                       hipStream_t s, int hL = 0, float hscale = 1.0f)
{
    using F = Fmt<TYPE>;
    const int nb = (int)(K / F::G);
    const int grid = (int)std::min<int64_t>(num_cus(), (N + 3) / 4);
    const int vec4 = aligned(x, 16) ? 1 : 0;
    constexpr auto kern = pn_gemv_xreg_kernel<TYPE, M, D, ROT>;
    const size_t lds = ROT ? (size_t)M * K * sizeof(float) : 0;  // the rotated x
    if (ROT && !lds_limit_once<kern>((int)((size_t)M * 64 * F::G * sizeof(float))))
        return PN_ERR_HIP;
    // 512 threads: the cooperative staging gives each thread one word of one block
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, y, row_split(N, grid), vec4,
                       older_share(12), hL, hscale);
    return launch_status();
}

constexpr int kNotApplicable = 1;  // internal: the flat kernel does not take this shape

template <int TYPE, int M, int QPT, bool ROT>
static int launch_flat_q(const uint8_t *W, int64_t N, int nb, const float *x, int64_t K, float *y,
                         int grid, int64_t NP, size_t lds, hipStream_t s, int hL, float hscale)
{
    constexpr auto kern = pn_gemv_flat_kernel<TYPE, M, 2, 4, QPT, ROT>;
    if (!lds_limit_once<kern>(kMaxLds))
        return PN_ERR_HIP;
    const int vec4 = aligned(x, 16) ? 1 : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kFlatWaves), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, y, NP / grid, (int)(NP % grid), vec4,
                       older_share(10), hL, hscale);
    return launch_status();
}

// The flat kernel takes rows of at least 64 blocks whose x (M tokens) fits in LDS at once and
// whose staging needs at most 32 16-byte loads per thread; otherwise kNotApplicable.
template <int TYPE, int M, bool ROT = false>
static int launch_flat(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y,
                       hipStream_t s, int hL = 0, float hscale = 1.0f)
{
    using F = Fmt<TYPE>;
    constexpr int R = 2, V = ((M * R + 3) / 4) * 4;
    const int64_t nb = K / F::G;
    const int64_t NP = (N + R - 1) / R;
    const int grid = (int)std::min<int64_t>(num_cus(), NP);
    const size_t lds = (size_t)M * nb * F::LDS_STRIDE * sizeof(float) +
                       (size_t)kFlatWaves * 2 * V * sizeof(float) + kFlatWaves * 4 * sizeof(int);
    const int64_t need = (M * nb * (F::G / 4) + 64 * kFlatWaves - 1) / (64 * kFlatWaves);
    const int64_t per_wg = (NP + grid - 1) / grid;  // groups per workgroup, at most
    if (nb < 64 || lds > (size_t)kMaxLds || need > 32 || per_wg * nb >= (int64_t(1) << 30))
        return kNotApplicable;
    if (need <= 8)
        return launch_flat_q<TYPE, M, 8, ROT>(W, N, (int)nb, x, K, y, grid, NP, lds, s, hL, hscale);
    if (need <= 16)
        return launch_flat_q<TYPE, M, 16, ROT>(W, N, (int)nb, x, K, y, grid, NP, lds, s, hL, hscale);
    if (need <= 24)  // two tokens of down (17 per thread): fewer registers than 32
        return launch_flat_q<TYPE, M, 24, ROT>(W, N, (int)nb, x, K, y, grid, NP, lds, s, hL, hscale);
    return launch_flat_q<TYPE, M, 32, ROT>(W, N, (int)nb, x, K, y, grid, NP, lds, s, hL, hscale);
}

// Rows in flight per wave in the short-row kernel at M = 1 (ring size 4 or 8); PN_GEMV_DEPTH
// overrides the default.
static int ring_depth()
{
    const char *e = getenv("PN_GEMV_DEPTH");
    return (e && atoi(e) >= 8) ? 8 : 4;
}

int launch_mfma(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int M, float *y,
                int cus, hipStream_t s);
bool mfma_stages_weights(int type, const void *W, int64_t N, int64_t K);
int launch_mfma_group(const pn_gemv_part *parts, int count, int64_t K, const float *x, int M,
                      int cus, hipStream_t s);

template <int TYPE>
static int dispatch_m(const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
                      hipStream_t s)
{
    const bool short_rows = K / Fmt<TYPE>::G <= 64 && !getenv("PN_GEMV_NO_XREG");
    const bool flat = !getenv("PN_GEMV_NO_FLAT");
    int st;
    switch (M) {
    case 1:
        if (short_rows)
            return ring_depth() == 8 ? launch_xreg<TYPE, 1, 8>(W, N, K, x, y, s)
                                     : launch_xreg<TYPE, 1, 4>(W, N, K, x, y, s);
        if (flat && (st = launch_flat<TYPE, 1>(W, N, K, x, y, s)) != kNotApplicable)
            return st;
        return launch_lds<TYPE, 1, 2, 4>(W, N, K, x, y, s);
    case 2:
        if (short_rows)
            return launch_xreg<TYPE, 2, 2>(W, N, K, x, y, s);
        // rows of 65-128 blocks: the matrix cores, where they stage the weights, beat the
        // long-row kernel at two tokens (0.3-2 us per launch at 5120 rows); longer rows and
        // one token stay on the vector units (PN_GEMV_NO_MFMA keeps them there)
        if (K / Fmt<TYPE>::G > 64 && K / Fmt<TYPE>::G <= 128 && !getenv("PN_GEMV_NO_MFMA") &&
            mfma_stages_weights(TYPE, W, N, K))
            return launch_mfma(TYPE, W, N, K, x, 2, y, num_cus(), s);
        if (flat && (st = launch_flat<TYPE, 2>(W, N, K, x, y, s)) != kNotApplicable)
            return st;
        return launch_lds<TYPE, 2, 2, 2>(W, N, K, x, y, s);
    default: break;
    }
    // three or more tokens: the matrix cores. At three and four tokens only the kernel that stages
    // the weights through LDS beats the vector-unit kernel; other shapes keep the latter
    // (PN_GEMV_MFMA forces the matrix cores, PN_GEMV_NO_MFMA the vector units: tests, timing).
    if (M > 4 || getenv("PN_GEMV_MFMA") ||
        (!getenv("PN_GEMV_NO_MFMA") && mfma_stages_weights(TYPE, W, N, K)))
        return launch_mfma(TYPE, W, N, K, x, (int)M, y, num_cus(), s);
    if (M == 3)
        return launch_lds<TYPE, 3, 1, 2>(W, N, K, x, y, s);
    return launch_lds<TYPE, 4, 2, 2>(W, N, K, x, y, s);
}

// The GEMV over Hadamard-rotated x, with the rotation fused into the x staging of the register
// kernel (rows of at most 64 blocks) and the long-row kernel (x of the call fits its LDS area).
template <int TYPE>
static int dispatch_hadamard(const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
                             float *y, int hL, float hscale, hipStream_t s)
{
    const bool short_rows = K / Fmt<TYPE>::G <= 64;
    int st;
    if (M == 1) {
        if (short_rows)
            return launch_xreg<TYPE, 1, 4, true>(W, N, K, x, y, s, hL, hscale);
        if ((st = launch_flat<TYPE, 1, true>(W, N, K, x, y, s, hL, hscale)) != kNotApplicable)
            return st;
        return PN_ERR_SHAPE;
    }
    if (short_rows)
        return launch_xreg<TYPE, 2, 2, true>(W, N, K, x, y, s, hL, hscale);
    if ((st = launch_flat<TYPE, 2, true>(W, N, K, x, y, s, hL, hscale)) != kNotApplicable)
        return st;
    return PN_ERR_SHAPE;
}

// ---- several GEMVs that share x, in one launch -----------------------------------------------
// One grid serves up to 4 matrices (parts) that read the same x: part i owns the workgroups
// [start_i, start_{i+1}), and within them runs the register kernel's body (rows of at most 64
// blocks) or the long-row kernel's body (longer rows whose x fits, 8 float4 of x per thread),
// exactly as its own launch of that many workgroups would. The parts' fixed costs (x staging,
// the first weight latency, drain) then run side by side instead of one launch after another.
constexpr int kGroupMax = 4;
enum { kGroupXreg3 = 0, kGroupXreg4 = 1, kGroupFlat3 = 2, kGroupFlat4 = 3 };

struct GroupPart {
    const uint8_t *W;
    float *y;
    int64_t N, row_bytes, gq;
    RowSplit sp;
    int nb, kind, start, gr, fnum;
};

struct GroupArgs {
    GroupPart p[kGroupMax];
    const float *x;
    int64_t K;
    int count, x_vec4, hL;
    float hscale;
};

// ROT: every part reads x rotated in slices of 2^hL (the fused staging of the two bodies).
template <int M, bool ROT>
__global__ void __launch_bounds__(512) pn_gemv_group_kernel(GroupArgs ga)
{
    constexpr int D = M == 1 ? 4 : 2;  // the register kernel's ring, as its own launch uses
    int i = 0;
#pragma unroll
    for (int j = 1; j < kGroupMax; j++)
        if (j < ga.count && (int)blockIdx.x >= ga.p[j].start)
            i = j;
    const GroupPart &p = ga.p[i];
    const int blk = (int)blockIdx.x - p.start;
    switch (p.kind) {
    case kGroupXreg3:
        xreg_body<PN_TYPE_PN3T, M, D, ROT>(p.W, p.N, p.nb, p.row_bytes, ga.x, ga.K, p.y, p.sp,
                                           ga.x_vec4, p.fnum, ga.hL, ga.hscale, blk);
        break;
    case kGroupXreg4:
        xreg_body<PN_TYPE_PN4T, M, D, ROT>(p.W, p.N, p.nb, p.row_bytes, ga.x, ga.K, p.y, p.sp,
                                           ga.x_vec4, p.fnum, ga.hL, ga.hscale, blk);
        break;
    case kGroupFlat3:
        flat_body<PN_TYPE_PN3T, M, 2, 4, 8, ROT>(p.W, p.N, p.nb, p.row_bytes, ga.x, ga.K, p.y,
                                                 p.gq, p.gr, ga.x_vec4, p.fnum, ga.hL, ga.hscale,
                                                 blk);
        break;
    default:
        flat_body<PN_TYPE_PN4T, M, 2, 4, 8, ROT>(p.W, p.N, p.nb, p.row_bytes, ga.x, ga.K, p.y,
                                                 p.gq, p.gr, ga.x_vec4, p.fnum, ga.hL, ga.hscale,
                                                 blk);
        break;
    }
}

// Static LDS of the group kernel: the register kernel's staging area for both types.
template <int M> constexpr int group_static_lds()
{
    return M * 64 * (Fmt<PN_TYPE_PN3T>::LDS_STRIDE + Fmt<PN_TYPE_PN4T>::LDS_STRIDE) * 4;
}

// The part's kind and its dynamic LDS need, or -1 where neither body takes the shape.
template <int M, bool ROT>
static int group_kind(int type, int64_t N, int64_t K, int grid_max, size_t &lds)
{
    const int G = type == PN_TYPE_PN3T ? Fmt<PN_TYPE_PN3T>::G : Fmt<PN_TYPE_PN4T>::G;
    const int stride =
        type == PN_TYPE_PN3T ? Fmt<PN_TYPE_PN3T>::LDS_STRIDE : Fmt<PN_TYPE_PN4T>::LDS_STRIDE;
    const int64_t nb = K / G;
    lds = ROT ? (size_t)M * K * sizeof(float) : 0;  // the register body's rotated x
    if (nb <= 64)
        return type == PN_TYPE_PN3T ? kGroupXreg3 : kGroupXreg4;
    constexpr int V = ((M * 2 + 3) / 4) * 4;
    lds = (size_t)M * nb * stride * sizeof(float) + (size_t)kFlatWaves * 2 * V * sizeof(float) +
          kFlatWaves * 4 * sizeof(int);
    const int64_t need = (M * nb * (G / 4) + 64 * kFlatWaves - 1) / (64 * kFlatWaves);
    const int64_t NP = (N + 1) / 2;
    const int64_t nq_rot = 4 * ((M * nb * (G / 4) + 256 * kFlatWaves - 1) / (256 * kFlatWaves));
    if (need > 8 || (ROT && nq_rot > 8) || lds + group_static_lds<M>() > (size_t)kMaxLds ||
        ((NP + grid_max - 1) / grid_max) * nb >= (int64_t(1) << 30))
        return -1;
    return type == PN_TYPE_PN3T ? kGroupFlat3 : kGroupFlat4;
}

// Launches the group, or returns kNotApplicable where a part's shape is not taken.
template <int M, bool ROT = false>
static int launch_group(const pn_gemv_part *parts, int count, int64_t K, const float *x,
                        hipStream_t s, int hL = 0, float hscale = 1.0f)
{
    const int cus = num_cus();
    GroupArgs ga{};
    int n = 0;
    size_t lds = 0;
    double bytes[kGroupMax], total = 0.0;
    int cap[kGroupMax];
    for (int i = 0; i < count; i++) {
        if (parts[i].N == 0)
            continue;
        size_t l = 0;
        const int kind = group_kind<M, ROT>(parts[i].type, parts[i].N, K, cus, l);
        if (kind < 0)
            return kNotApplicable;
        GroupPart &g = ga.p[n];
        g.W = (const uint8_t *)parts[i].W;
        g.y = parts[i].y;
        g.N = parts[i].N;
        g.row_bytes = pn_row_bytes(parts[i].type, K);
        g.nb = (int)(g.row_bytes / kBlockBytes);
        g.kind = kind;
        g.fnum = kind <= kGroupXreg4 ? older_share(12) : older_share(10);
        bytes[n] = (double)g.N * (double)g.row_bytes;
        total += bytes[n];
        // workgroups beyond these would get no rows (register body: 4 rows per workgroup at
        // least; long-row body: one row pair)
        cap[n] = (int)std::min<int64_t>(cus, kind <= kGroupXreg4 ? (g.N + 3) / 4 : (g.N + 1) / 2);
        lds = std::max(lds, l);
        n++;
    }
    if (n == 0)
        return PN_OK;
    // workgroups in proportion to bytes (at least one each), the rest to the most loaded part
    int grid[kGroupMax], used = 0;
    for (int j = 0; j < n; j++) {
        grid[j] = std::max(1, std::min(cap[j], (int)(cus * bytes[j] / total)));
        used += grid[j];
    }
    while (used < cus) {
        int best = -1;
        double load = 0.0;
        for (int j = 0; j < n; j++)
            if (grid[j] < cap[j] && bytes[j] / grid[j] > load) {
                load = bytes[j] / grid[j];
                best = j;
            }
        if (best < 0)
            break;
        grid[best]++;
        used++;
    }
    int start = 0;
    for (int j = 0; j < n; j++) {
        GroupPart &g = ga.p[j];
        g.start = start;
        start += grid[j];
        g.sp = row_split(g.N, grid[j]);
        const int64_t NP = (g.N + 1) / 2;
        g.gq = NP / grid[j];
        g.gr = (int)(NP % grid[j]);
        if (g.kind >= kGroupFlat3 && (g.gq + 1) * g.nb >= (int64_t(1) << 30))
            return kNotApplicable;  // the long-row body's (row pair, block) index must fit 30 bits
    }
    ga.count = n;
    ga.x = x;
    ga.K = K;
    ga.x_vec4 = aligned(x, 16) ? 1 : 0;
    ga.hL = hL;
    ga.hscale = hscale;
    if (lds + group_static_lds<M>() > (size_t)kMaxLds)
        return kNotApplicable;
    constexpr auto kern = pn_gemv_group_kernel<M, ROT>;
    if (!lds_limit_once<kern>(kMaxLds - group_static_lds<M>()))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)start), dim3(512), lds, s, ga);
    return launch_status();
}

int hadamard_log(int64_t B, int64_t K);
float hadamard_scale(int L);
int launch_mfma_hadamard(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int M,
                         float *y, int cus, int hL, float hscale, hipStream_t s);

}  // namespace pn

using namespace pn;

extern "C" int pn_gemv_hadamard(int type, const void *W, int64_t N, int64_t K, const float *x,
                                int64_t M, int64_t B, float *y, void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (N < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_GEMV_HADAMARD_MAX_TOKENS)
        return PN_ERR_TOKENS;
    const int L = hadamard_log(B, K);
    if (L < 0)
        return PN_ERR_HADAMARD;
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
    const float hs = hadamard_scale(L);
    // three or four tokens: one launch of the matrix-core kernel where it stages x in one pass
    if (M >= 3 && (st = launch_mfma_hadamard(type, (const uint8_t *)W, N, K, x, (int)M, y,
                                             num_cus(), L, hs, s)) != 1)
        return st;
    // else tokens two at a time (the fused staging serves one or two; W read once per pair)
    for (int64_t m0 = 0; m0 < M; m0 += 2) {
        const int64_t mc = std::min<int64_t>(2, M - m0);
        st = type == PN_TYPE_PN3T
                 ? dispatch_hadamard<PN_TYPE_PN3T>((const uint8_t *)W, N, K, x + m0 * K, mc,
                                                   y + m0 * N, L, hs, s)
                 : dispatch_hadamard<PN_TYPE_PN4T>((const uint8_t *)W, N, K, x + m0 * K, mc,
                                                   y + m0 * N, L, hs, s);
        if (st != PN_OK)
            return st;
    }
    return PN_OK;
}

extern "C" int pn_gemv_group(const pn_gemv_part *parts, int count, int64_t K, const float *x,
                             int64_t M, void *stream)
{
    if (count < 1 || count > PN_GEMV_GROUP_MAX_PARTS)
        return PN_ERR_SHAPE;
    if (!parts)
        return PN_ERR_NULL;
    if (M < 0 || M > PN_GEMV_MAX_TOKENS)
        return PN_ERR_TOKENS;
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.type != PN_TYPE_PN3T && p.type != PN_TYPE_PN4T)
            return PN_ERR_TYPE;
        if (p.N < 0 || pn_row_bytes(p.type, K) == 0)
            return PN_ERR_SHAPE;
    }
    if (M == 0)
        return PN_OK;
    bool any = false;
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.N == 0)
            continue;
        any = true;
        if (!p.W || !p.y)
            return PN_ERR_NULL;
        if (!aligned(p.W, 2) || !aligned(p.y, 4))
            return PN_ERR_ALIGN;
    }
    if (!any)
        return PN_OK;
    if (!x)
        return PN_ERR_NULL;
    if (!aligned(x, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (count > 1 && M <= 4 && !getenv("PN_GEMV_NO_GROUP")) {
        st = M == 1   ? launch_group<1>(parts, count, K, x, s)
             : M == 2 ? launch_group<2>(parts, count, K, x, s)
                      : launch_mfma_group(parts, count, K, x, (int)M, num_cus(), s);
        if (st != kNotApplicable)
            return st;
    }
    // one launch per part (three or more tokens, or a shape the group does not take)
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.N == 0)
            continue;
        st = p.type == PN_TYPE_PN3T
                 ? dispatch_m<PN_TYPE_PN3T>((const uint8_t *)p.W, p.N, K, x, M, p.y, s)
                 : dispatch_m<PN_TYPE_PN4T>((const uint8_t *)p.W, p.N, K, x, M, p.y, s);
        if (st != PN_OK)
            return st;
    }
    return PN_OK;
}

extern "C" int pn_gemv_group_hadamard(const pn_gemv_part *parts, int count, int64_t K,
                                      const float *x, int64_t M, int64_t B, void *stream)
{
    if (count < 1 || count > PN_GEMV_GROUP_MAX_PARTS)
        return PN_ERR_SHAPE;
    if (!parts)
        return PN_ERR_NULL;
    if (M < 0 || M > PN_GEMV_HADAMARD_MAX_TOKENS)
        return PN_ERR_TOKENS;
    for (int i = 0; i < count; i++) {
        if (parts[i].type != PN_TYPE_PN3T && parts[i].type != PN_TYPE_PN4T)
            return PN_ERR_TYPE;
        if (parts[i].N < 0 || pn_row_bytes(parts[i].type, K) == 0)
            return PN_ERR_SHAPE;
    }
    const int L = hadamard_log(B, K);
    if (L < 0)
        return PN_ERR_HADAMARD;
    if (M == 0)
        return PN_OK;
    bool any = false;
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.N == 0)
            continue;
        any = true;
        if (!p.W || !p.y)
            return PN_ERR_NULL;
        if (!aligned(p.W, 2) || !aligned(p.y, 4))
            return PN_ERR_ALIGN;
    }
    if (!any)
        return PN_OK;
    if (!x)
        return PN_ERR_NULL;
    if (!aligned(x, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (count > 1 && M <= 2 && !getenv("PN_GEMV_NO_GROUP")) {
        const float hs = hadamard_scale(L);
        st = M == 1 ? launch_group<1, true>(parts, count, K, x, s, L, hs)
                    : launch_group<2, true>(parts, count, K, x, s, L, hs);
        if (st != kNotApplicable)
            return st;
    }
    // one fused launch per part (three or four tokens, or a shape the group does not take)
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.N == 0)
            continue;
        st = pn_gemv_hadamard(p.type, p.W, p.N, K, x, M, B, p.y, stream);
        if (st != PN_OK)
            return st;
    }
    return PN_OK;
}

extern "C" int pn_gemv(int type, const void *W, int64_t N, int64_t K, const float *x, int64_t M,
                       float *y, void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (N < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_GEMV_MAX_TOKENS)
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
