// pn_gemv_mfma.hip -- PN decode-step GEMV for 3..16 tokens on the gfx950 matrix cores.
//
// Format: "PN weight format", sections "Block layout" and "Value": a 34-byte block holds an fp16
// scale d and eight little-endian words; code t of a word sits at bit BITS*(t>>1) + 16*(t&1), and
// the weight is d * (n - z). The sum computed is y[m, r] = sum_k w[r, k] x[m, k].
//
// Why the matrix cores here: at one or two tokens the multiply-adds are a small share of the
// arithmetic and the vector units keep up with HBM; from three tokens on they are not (one FMA
// per weight per token on top of the decode). The decode itself stays on the vector units and
// feeds the matrix cores directly:
//
//  * A masked 16-bit half that holds a code n at bit p (p <= 6 for pn3t, <= 4 for pn4t) reads as
//    the fp16 subnormal n * 2^(p-24), exactly. So `word & 0x00070007` (and its shifted masks) is a
//    pair of fp16 operands with no conversion: one AND per two weights. These are the B operand
//    of v_mfma_f32_16x16x32_f16 (k = code position, n = output row), 16 rows per tile.
//  * x is the A operand (rows = tokens). It is staged in LDS once per workgroup as an fp16 (hi, lo)
//    pair x * 2^(E + 24 - p) per code position; hi and lo are fed as two MFMAs on the same codes,
//    so the sum of both is ~22-bit exact x. E is one exponent per token (and phase) chosen from
//    the largest |x| so that hi stays below 2^15.
//  * Each block's MFMA chain starts from C = -z * 2^E * sum(x of the block), so the chain ends at
//    2^E * sum (n - z) x for the block's 16 rows x 16 token slots, and one FMA per token adds
//    d * chain into the row's sum. The block's scale d therefore never meets a code in fp16.
//
// Operand layout (measured on gfx950 with a one-wave probe): for 16x16x32, lane l holds
// A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16] for j < 8, and the result
// D[4 (l / 16) + j][l % 16], j < 4. With k-groups g = l / 16, lane (n = l % 16, g) decodes words
// 2g and 2g+1 of its row's block: codes 20g..20g+19 (pn3t: steps of 8, 8 and 4 codes, the last
// one zero-padded) or 16g..16g+15 (pn4t: 8 and 8) of the block, in element order, and holds y for
// tokens 4g..4g+3 of row n.
//
// Work split: one workgroup of 8 waves per CU owns a contiguous range of rows (tiles of 16, the
// last one masked). The 8 waves split the blocks of every tile; a wave walks its blocks in order
// and, for each block, all tiles of its group, so each x operand is read from LDS once per block.
// Partial sums meet in LDS at the end and are added in wave order: deterministic. x larger than
// LDS is staged in phases of blocks; a later phase may only lower the exponent (the running sums
// are rescaled by a power of two), so nothing overflows.
#include "pn_common.h"

namespace pn {

typedef float mf_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u2a4 __attribute__((ext_vector_type(2), aligned(4)));

template <int TYPE> struct MTile;
template <> struct MTile<PN_TYPE_PN3T> {
    static constexpr int G = 80, PERG = 20, CHUNKS = 6, Z = 4;
    // bit position (after the decode's one shift) of code kl of a lane's 20: pairs t = 0..9 of a
    // word sit at 0, 3, 6 and, after >> 9, at 0, 3
    static constexpr int pe(int kl) { return 3 * ((((kl % 10) >> 1)) % 3); }
};
template <> struct MTile<PN_TYPE_PN4T> {
    static constexpr int G = 64, PERG = 16, CHUNKS = 4, Z = 8;
    // pairs t = 0..7 of a word sit at 0, 4 and, after >> 8, at 0, 4
    static constexpr int pe(int kl) { return ((kl >> 1) & 1) * 4; }
};

constexpr int kMfmaThreads = 512;
constexpr int kMfmaWaves = kMfmaThreads / 64;
constexpr int kMfmaMaxTG = 9;   // tiles of 16 rows per group (accumulators per lane: 4 per tile)
constexpr int kMfmaUnits = 2;   // staging units (one token, one k-group of a block) per thread and pass

struct MfmaRaw {
    mf_u2a4 w;       // the aligned dwords covering the lane's two words
    uint32_t tail;   // the 16 bits after them (used when the words are not 4-byte aligned)
    uint32_t dbits;  // the block's fp16 scale
    uint32_t sh;     // 0 or 16: realignment shift
};

// Loads of lane (row, g) for block b: exactly the block's bytes that the lane uses (the words of
// a block are 4-byte aligned in every other block, so the lane reads the 8 aligned bytes at or
// before its words and, when misaligned, the 2 bytes after).
__device__ __forceinline__ void mfma_issue(const uint8_t *rowp, int b, int g, MfmaRaw &r)
{
    const uint8_t *blk = rowp + 34 * b;
    const uint8_t *wo = blk + 2 + 8 * g;
    const uint32_t mis = (uint32_t)reinterpret_cast<uintptr_t>(wo) & 2u;
    const uint8_t *a0 = wo - mis;  // pointer arithmetic keeps the global address space
    r.w = *reinterpret_cast<const mf_u2a4 *>(a0);
    r.tail = *reinterpret_cast<const uint16_t *>(a0 + (mis ? 8 : 6));
    r.dbits = *reinterpret_cast<const uint16_t *>(blk);
    r.sh = mis << 3;
}

// The lane's two words as MFMA B operands (fp16 subnormal code pairs, see the file comment).
template <int TYPE> struct MfmaB;
template <> struct MfmaB<PN_TYPE_PN3T> {
    u32x4v b0, b1, b2;
    __device__ __forceinline__ void decode(const MfmaRaw &r)
    {
        const uint32_t w0 = __builtin_amdgcn_alignbit(r.w.y, r.w.x, r.sh);
        const uint32_t w1 = __builtin_amdgcn_alignbit(r.tail, r.w.y, r.sh);
        const uint32_t s0 = w0 >> 9, s1 = w1 >> 9;
        b0 = u32x4v{w0 & 0x00070007u, w0 & 0x00380038u, w0 & 0x01C001C0u, s0 & 0x00070007u};
        b1 = u32x4v{s0 & 0x00380038u, w1 & 0x00070007u, w1 & 0x00380038u, w1 & 0x01C001C0u};
        // the last four codes fill half of a 16x16x32 step; the other half meets zero x (any
        // finite code words do), here a copy of the same two
        const uint32_t v8 = s1 & 0x00070007u, v9 = s1 & 0x00380038u;
        b2 = u32x4v{v8, v9, v8, v9};
    }
};
template <> struct MfmaB<PN_TYPE_PN4T> {
    u32x4v b0, b1;
    __device__ __forceinline__ void decode(const MfmaRaw &r)
    {
        const uint32_t w0 = __builtin_amdgcn_alignbit(r.w.y, r.w.x, r.sh);
        const uint32_t w1 = __builtin_amdgcn_alignbit(r.tail, r.w.y, r.sh);
        const uint32_t s0 = w0 >> 8, s1 = w1 >> 8;
        b0 = u32x4v{w0 & 0x000F000Fu, w0 & 0x00F000F0u, s0 & 0x000F000Fu, s0 & 0x00F000F0u};
        b1 = u32x4v{w1 & 0x000F000Fu, w1 & 0x00F000F0u, s1 & 0x000F000Fu, s1 & 0x00F000F0u};
    }
};

// x operands of one block for lane (token, g): CHUNKS x 16 bytes (hi and lo halves).
struct MfmaA {
    u32x4v c[6];
};

// One block of one 16-row tile: c <- c + codes . x over the block, hi and lo passes. The chain is
// one asm block so that the accumulator stays in place (destination = C operand) from step to
// step, and the independent cycles around it are explicit: 3 before (operands just written by
// vector instructions) and 16 after (the result is read, and the sources may be rewritten, by
// vector instructions). Left to the compiler, a vector write to a register still being read as
// the C operand of an in-flight 16x16x32 step was scheduled too close on gfx950 and corrupted
// the sum.
template <int TYPE>
__device__ __forceinline__ mf_f4 mfma_block(const MfmaA &a, const MfmaB<TYPE> &b, mf_f4 c);
template <>
__device__ __forceinline__ mf_f4 mfma_block<PN_TYPE_PN3T>(const MfmaA &a,
                                                          const MfmaB<PN_TYPE_PN3T> &b, mf_f4 c)
{
    asm volatile("s_nop 2\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %1, %7, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %2, %7, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %3, %8, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %4, %8, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %5, %9, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %6, %9, %0\n\t"
                 "s_nop 7\n\t"
                 "s_nop 7"
                 : "+v"(c)
                 : "v"(a.c[0]), "v"(a.c[1]), "v"(a.c[2]), "v"(a.c[3]), "v"(a.c[4]), "v"(a.c[5]),
                   "v"(b.b0), "v"(b.b1), "v"(b.b2));
    return c;
}
template <>
__device__ __forceinline__ mf_f4 mfma_block<PN_TYPE_PN4T>(const MfmaA &a,
                                                          const MfmaB<PN_TYPE_PN4T> &b, mf_f4 c)
{
    asm volatile("s_nop 2\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %1, %5, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %2, %5, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %3, %6, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %4, %6, %0\n\t"
                 "s_nop 7\n\t"
                 "s_nop 7"
                 : "+v"(c)
                 : "v"(a.c[0]), "v"(a.c[1]), "v"(a.c[2]), "v"(a.c[3]), "v"(b.b0), "v"(b.b1));
    return c;
}

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi)
{
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// One staging unit: token m, block brel of the phase, k-group g (PERG consecutive x values).
template <int TYPE>
__device__ __forceinline__ void mfma_load_unit(const float *__restrict__ x, int64_t K, int m,
                                               int64_t k0, int xvec4, float (&v)[MTile<TYPE>::PERG])
{
    constexpr int PERG = MTile<TYPE>::PERG;
    const float *src = x + (int64_t)m * K + k0;
    if (xvec4) {
#pragma unroll
        for (int q = 0; q < PERG / 4; q++) {
            const float4 f = reinterpret_cast<const float4 *>(src)[q];
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < PERG; e++)
            v[e] = src[e];
    }
}

template <int TYPE, int TG>
__global__ void __launch_bounds__(kMfmaThreads)
pn_gemv_mfma_kernel(const uint8_t *__restrict__ W, int64_t N, int nb, int64_t row_bytes,
                    const float *__restrict__ x, int64_t K, int M, float *__restrict__ y,
                    int64_t rq, int rr, int Pb, int nph, int xvec4)
{
    using T = MTile<TYPE>;
    constexpr int P = (8 + TG - 1) / TG;  // block steps of loads in flight (about 8 tiles' worth)
    constexpr int PERG = T::PERG, CH = T::CHUNKS;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ uint32_t smax[2][16];
    __shared__ int sexp[2][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int per_block = 64 * (CH * M + 1);
    const int zs_off = CH * 64 * M;

    const int64_t wg = blockIdx.x;
    const int64_t r0 = wg * rq + (wg < rr ? wg : rr);
    const int64_t r1 = r0 + rq + (wg < rr ? 1 : 0);
    const int ntiles = (int)((r1 - r0 + 15) >> 4);
    const int ngroups = (ntiles + TG - 1) / TG;

    if (tid < 32)
        (&smax[0][0])[tid] = 0u;

    for (int grp = 0; grp < ngroups; grp++) {
        const int t0 = grp * TG;
        const int gt = min(TG, ntiles - t0);
        const uint8_t *rowp[TG];
#pragma unroll
        for (int t = 0; t < TG; t++) {
            int64_t r = r0 + 16 * (int64_t)(t0 + t) + n16;
            r = r < r1 ? r : r1 - 1;
            rowp[t] = W + r * row_bytes;
        }
        mf_f4 acc[TG];
#pragma unroll
        for (int t = 0; t < TG; t++)
            acc[t] = mf_f4{0.f, 0.f, 0.f, 0.f};

        for (int p = 0; p < nph; p++) {
            const int q = grp * nph + p;
            const int pb0 = p * Pb, npb = min(nb, pb0 + Pb) - pb0;
            const int U = npb * M * 4;
            const int nch = (U + kMfmaThreads * kMfmaUnits - 1) / (kMfmaThreads * kMfmaUnits);

            // ---- stage x for blocks [pb0, pb0 + npb) ----
            __syncthreads();  // earlier readers of the x area, sexp and smax are done
            if (tid < 16)
                smax[(q + 1) & 1][tid] = 0u;
            float xr[kMfmaUnits][PERG];
            for (int c = 0; c < nch; c++) {
#pragma unroll
                for (int ub = 0; ub < kMfmaUnits; ub++) {
                    const int u = (c * kMfmaUnits + ub) * kMfmaThreads + tid;
                    if (u < U) {
                        const int gg = u & 3, m = (u >> 2) % M, brel = (u >> 2) / M;
                        mfma_load_unit<TYPE>(x, K, m, (int64_t)(pb0 + brel) * T::G + PERG * gg,
                                             xvec4, xr[ub]);
                        float mx = 0.f;
#pragma unroll
                        for (int e = 0; e < PERG; e++)
                            mx = fmaxf(mx, fabsf(xr[ub][e]));
                        atomicMax(&smax[q & 1][m], __float_as_uint(mx));
                    }
                }
            }
            __syncthreads();
            if (tid < 16) {
                const uint32_t mb = smax[q & 1][tid];
                int E = 1 << 20;  // an all-zero token keeps the previous exponent
                if (mb != 0u) {
                    int ex;
                    frexpf(__uint_as_float(mb), &ex);
                    E = -9 - ex;  // largest |x| * 2^(E + 24) < 2^15
                }
                if (p > 0)
                    E = min(E, sexp[(q - 1) & 1][tid]);
                sexp[q & 1][tid] = E;
            }
            __syncthreads();
            for (int c = 0; c < nch; c++) {
#pragma unroll
                for (int ub = 0; ub < kMfmaUnits; ub++) {
                    const int u = (c * kMfmaUnits + ub) * kMfmaThreads + tid;
                    if (u < U) {  // U is a multiple of 4: whole quads take this branch
                        const int gg = u & 3, m = (u >> 2) % M, brel = (u >> 2) / M;
                        if (nch > 1)
                            mfma_load_unit<TYPE>(x, K, m, (int64_t)(pb0 + brel) * T::G + PERG * gg,
                                                 xvec4, xr[ub]);
                        const int eb = sexp[q & 1][m] + 24;
                        uint32_t hw[PERG / 2], lw[PERG / 2];
                        float s = 0.f;
#pragma unroll
                        for (int e = 0; e < PERG; e += 2) {
                            s += xr[ub][e];
                            s += xr[ub][e + 1];
                            const float v0 = ldexpf(xr[ub][e], eb - T::pe(e));
                            const float v1 = ldexpf(xr[ub][e + 1], eb - T::pe(e + 1));
                            const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                            hw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                            lw[e / 2] = pack_h2(v0 - (float)h0, v1 - (float)h1);
                        }
                        uint8_t *blk = lds + brel * per_block;
                        auto chunk = [&](int ch) {
                            return reinterpret_cast<u32x4v *>(blk + ((ch * 4 + gg) * M + m) * 16);
                        };
                        *chunk(0) = u32x4v{hw[0], hw[1], hw[2], hw[3]};
                        *chunk(1) = u32x4v{lw[0], lw[1], lw[2], lw[3]};
                        *chunk(2) = u32x4v{hw[4], hw[5], hw[6], hw[7]};
                        *chunk(3) = u32x4v{lw[4], lw[5], lw[6], lw[7]};
                        if constexpr (CH == 6) {  // the last 4 codes, zero-padded to a full step
                            *chunk(4) = u32x4v{hw[8], hw[9], 0u, 0u};
                            *chunk(5) = u32x4v{lw[8], lw[9], 0u, 0u};
                        }
                        // sum of the block's x for the zero point: k-groups 0+1, 2+3, then both
                        s += PN_DPP(s, 0xB1);  // quad_perm [1,0,3,2]
                        s += PN_DPP(s, 0x4E);  // quad_perm [2,3,0,1]
                        if (gg == 0)
                            reinterpret_cast<float *>(blk + zs_off)[m] =
                                -(float)T::Z * ldexpf(s, sexp[q & 1][m]);
                    }
                }
            }
            for (int i = tid; i < npb * 16; i += kMfmaThreads)
                if ((i & 15) >= M)
                    reinterpret_cast<float *>(lds + (i >> 4) * per_block + zs_off)[i & 15] = 0.f;
            __syncthreads();

            if (p > 0) {  // the running sums move to this phase's (lower or equal) exponent
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int dE = sexp[q & 1][4 * g + j] - sexp[(q - 1) & 1][4 * g + j];
#pragma unroll
                    for (int t = 0; t < TG; t++)
                        acc[t][j] = ldexpf(acc[t][j], dE);
                }
            }

            // ---- this wave's blocks of the phase, every tile of the group ----
            const int kb0 = pb0 + (wave * npb) / kMfmaWaves;
            const int ns = pb0 + ((wave + 1) * npb) / kMfmaWaves - kb0;
            if (ns > 0) {
                MfmaRaw raw[P][TG];
                // The ring's loads are issued in the order they are consumed, and kept in that
                // order (scheduling barriers), so every wait leaves the later loads in flight.
#pragma unroll
                for (int s = 0; s < P; s++)
#pragma unroll
                    for (int t = 0; t < TG; t++) {
                        mfma_issue(rowp[t], kb0 + min(s, ns - 1), g, raw[s][t]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                MfmaA a;
#pragma unroll
                for (int ch = 0; ch < 6; ch++)
                    a.c[ch] = u32x4v{0u, 0u, 0u, 0u};
                for (int i = 0; i < ns; i += P) {
#pragma unroll
                    for (int s = 0; s < P; s++) {
                        const int st = i + s;
                        const int brel = min(st, ns - 1) + kb0 - pb0;
                        const uint8_t *blk = lds + brel * per_block;
                        if (n16 < M) {
#pragma unroll
                            for (int ch = 0; ch < CH; ch++)
                                a.c[ch] = *reinterpret_cast<const u32x4v *>(
                                    blk + ((ch * 4 + g) * M + n16) * 16);
                        }
                        const mf_f4 c0 = *reinterpret_cast<const mf_f4 *>(blk + zs_off + 16 * g);
                        const int nxt = kb0 + min(st + P, ns - 1);
                        // No branch around the use of a ring slot: a step past the wave's last
                        // block or a tile past the group's last one is computed on clamped (valid)
                        // data and added with d = 0. A branch here lets the decode sink below the
                        // slot's refill and the load waits lose the ring's depth.
                        const bool live = st < ns;
#pragma unroll
                        for (int t = 0; t < TG; t++) {
                            MfmaB<TYPE> bop;
                            bop.decode(raw[s][t]);
                            const float dv =
                                (live && t < gt) ? f16_bits_to_f32(raw[s][t].dbits) : 0.f;
                            mfma_issue(rowp[t], nxt, g, raw[s][t]);
                            __builtin_amdgcn_sched_barrier(0);
                            const mf_f4 dd = mfma_block<TYPE>(a, bop, c0);
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                acc[t][j] = fmaf(dv, dd[j], acc[t][j]);
                        }
                    }
                }
            }
        }

        // ---- partial sums of the 8 waves, added in wave order ----
        __syncthreads();
        mf_f4 *red = reinterpret_cast<mf_f4 *>(lds);
#pragma unroll
        for (int t = 0; t < TG; t++)
            red[(t * kMfmaWaves + wave) * 64 + lane] = acc[t];
        __syncthreads();
        const int ql = (grp * nph + nph - 1) & 1;
        for (int i = tid; i < gt * 64; i += kMfmaThreads) {
            const int t = i >> 6, l = i & 63;
            mf_f4 s = red[(t * kMfmaWaves) * 64 + l];
#pragma unroll
            for (int w = 1; w < kMfmaWaves; w++)
                s += red[(t * kMfmaWaves + w) * 64 + l];
            const int64_t row = r0 + 16 * (int64_t)(t0 + t) + (l & 15);
            if (row < r1) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int m = 4 * (l >> 4) + j;
                    if (m < M)
                        y[(int64_t)m * N + row] = ldexpf(s[j], -sexp[ql][m]);
                }
            }
        }
    }
}

// LDS for the x of a phase and, aliased, the 8 waves' partial sums (8 KB per tile of the group).
constexpr int kMfmaLds = 160 * 1024 - 1024;

template <int TYPE, int TG>
static int launch_mfma_tg(const uint8_t *W, int64_t N, int nb, const float *x, int64_t K, int M,
                          float *y, int64_t rq, int rr, int grid, int Pb, int nph, hipStream_t s)
{
    using T = MTile<TYPE>;
    const size_t lds = std::max<size_t>((size_t)Pb * 64 * (T::CHUNKS * M + 1),
                                        (size_t)TG * kMfmaWaves * 64 * 16);
    auto kern = pn_gemv_mfma_kernel<TYPE, TG>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kMfmaLds) != hipSuccess)
            return PN_ERR_HIP;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMfmaThreads), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, M, y, rq, rr, Pb, nph,
                       aligned(x, 16) ? 1 : 0);
    return launch_status();
}

template <int TYPE>
static int launch_mfma_t(const uint8_t *W, int64_t N, int64_t K, const float *x, int M, float *y,
                         int cus, hipStream_t s)
{
    using T = MTile<TYPE>;
    const int nb = (int)(K / T::G);
    const int grid = (int)std::min<int64_t>(cus, (N + 15) / 16);
    const int64_t rq = N / grid;
    const int rr = (int)(N % grid);
    const int64_t tiles_max = (rq + (rr ? 1 : 0) + 15) / 16;
    const int64_t ng = (tiles_max + kMfmaMaxTG - 1) / kMfmaMaxTG;
    const int TG = (int)((tiles_max + ng - 1) / ng);
    const int per_block = 64 * (T::CHUNKS * M + 1);
    const int pb_max = kMfmaLds / per_block;
    const int nph = (nb + pb_max - 1) / pb_max;
    const int Pb = (nb + nph - 1) / nph;
    switch (TG) {
#define PN_MFMA_CASE(tg)                                                                           \
    case tg: return launch_mfma_tg<TYPE, tg>(W, N, nb, x, K, M, y, rq, rr, grid, Pb, nph, s);
    PN_MFMA_CASE(1) PN_MFMA_CASE(2) PN_MFMA_CASE(3) PN_MFMA_CASE(4) PN_MFMA_CASE(5)
    PN_MFMA_CASE(6) PN_MFMA_CASE(7) PN_MFMA_CASE(8) PN_MFMA_CASE(9)
#undef PN_MFMA_CASE
    default: return PN_ERR_SHAPE;
    }
}

int launch_mfma(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int M, float *y,
                int cus, hipStream_t s)
{
    if (type == PN_TYPE_PN3T)
        return launch_mfma_t<PN_TYPE_PN3T>(W, N, K, x, M, y, cus, s);
    return launch_mfma_t<PN_TYPE_PN4T>(W, N, K, x, M, y, cus, s);
}

}  // namespace pn
