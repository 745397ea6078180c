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
//    pair of fp16 operands with no conversion, and one packed fp16 add of -z * 2^(p-24) makes it
//    (n - z) * 2^(p-24), still exact: two instructions per two weights. These are the B operand
//    of v_mfma_f32_16x16x32_f16 (k = code position, n = output row), 16 rows per tile. Taking z
//    off each code (instead of folding d * (sum n x - z sum x)) leaves no cancellation for the
//    matrix cores' accumulation to round.
//  * x is the A operand (rows = tokens), staged in LDS once per workgroup as an fp16 (hi, lo) pair
//    x * 2^(E + 24 - p) per code position, E one exponent per token and group of blocks (one
//    block in the direct-load kernel, four in the LDS-staged one) chosen from the group's largest
//    |x| so that hi stays below 2^15: the sum of hi and lo is ~22-bit exact x. Up to 8 tokens, hi
//    and lo are two token slots of one operand; up to 16, two operands.
//  * Each block's chain gives 2^E * sum (n - z) x for 16 rows x 16 token slots; one multiply by
//    d per block and one exact 2^-E scaling per token and group add it into the row's sum. The
//    block's scale d never meets a code in fp16.
//
// Operand layout (measured on gfx950 with a one-wave probe): for 16x16x32, lane l holds
// A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16] for j < 8, and the result
// D[4 (l / 16) + j][l % 16], j < 4. With k-groups g = l / 16, lane (n = l % 16, g) decodes words
// 2g and 2g+1 of its row's block: codes 20g..20g+19 (pn3t: steps of 8, 8 and 4 codes, the last
// one zero-padded) or 16g..16g+15 (pn4t: 8 and 8) of the block, in element order, and holds y for
// tokens 4g..4g+3 of row n.
//
// Work split: one workgroup of 8 waves per CU owns a contiguous range of rows (tiles of 16, the
// last one masked). Its 8 waves split the (tile, block) work of each phase of x; partial sums
// meet in LDS at the end and are added in wave order: deterministic. x larger than LDS is staged
// in phases of blocks. Two kernels: one stages the weights through LDS with whole-line copies
// (W 4-byte aligned, rows of a multiple of 4 blocks), the other reads each lane's bytes directly
// (any 2-byte aligned W and block count).
#include "pn_common.h"

namespace pn {

typedef float mf_f4 __attribute__((ext_vector_type(4)));

bool mfma_stages_weights(int type, const void *W, int64_t N, int64_t K);
typedef uint32_t mf_u2a4 __attribute__((ext_vector_type(2), aligned(4)));

template <int TYPE> struct MTile;
template <> struct MTile<PN_TYPE_PN3T> {
    static constexpr int G = 80, PERG = 20, KSTEPS = 3, Z = 4;
    // bit position (after the decode's one shift) of code kl of a lane's 20: pairs t = 0..9 of a
    // word sit at 0, 3, 6 and, after >> 9, at 0, 3
    static constexpr int pe(int kl) { return 3 * ((((kl % 10) >> 1)) % 3); }
};
template <> struct MTile<PN_TYPE_PN4T> {
    static constexpr int G = 64, PERG = 16, KSTEPS = 2, Z = 8;
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

// A masked pair of codes n at bit p (fp16 subnormals n 2^(p-24)) plus the pair (-z 2^(p-24)):
// (n - z) 2^(p-24), exactly (every value stays on the subnormal grid). The zero point is thus
// taken off each code before the matrix cores, and no sum of large terms cancels afterwards.
typedef _Float16 mf_h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t minus_z(uint32_t pair, uint32_t negz)
{
    return __builtin_bit_cast(uint32_t,
                              __builtin_bit_cast(mf_h2, pair) + __builtin_bit_cast(mf_h2, negz));
}

// The lane's two words as MFMA B operands: fp16 subnormal pairs (n - z) 2^(p-24).
template <int TYPE> struct MfmaB;
template <> struct MfmaB<PN_TYPE_PN3T> {
    u32x4v b0, b1, b2;
    __device__ __forceinline__ void decode(const MfmaRaw &r)
    {
        words(__builtin_amdgcn_alignbit(r.w.y, r.w.x, r.sh),
              __builtin_amdgcn_alignbit(r.tail, r.w.y, r.sh));
    }
    __device__ __forceinline__ void words(uint32_t w0, uint32_t w1)
    {
        // -z 2^(p-24) for z = 4 at p = 0, 3, 6: fp16 words 0x8004, 0x8020, 0x8100
        constexpr uint32_t z0 = 0x80048004u, z3 = 0x80208020u, z6 = 0x81008100u;
        const uint32_t s0 = w0 >> 9, s1 = w1 >> 9;
        b0 = u32x4v{minus_z(w0 & 0x00070007u, z0), minus_z(w0 & 0x00380038u, z3),
                    minus_z(w0 & 0x01C001C0u, z6), minus_z(s0 & 0x00070007u, z0)};
        b1 = u32x4v{minus_z(s0 & 0x00380038u, z3), minus_z(w1 & 0x00070007u, z0),
                    minus_z(w1 & 0x00380038u, z3), minus_z(w1 & 0x01C001C0u, z6)};
        // the last four codes fill half of a 16x16x32 step; the other half meets zero x (any
        // finite words do): the same codes before the zero point comes off
        const uint32_t m8 = s1 & 0x00070007u, m9 = s1 & 0x00380038u;
        b2 = u32x4v{minus_z(m8, z0), minus_z(m9, z3), m8, m9};
    }
};
template <> struct MfmaB<PN_TYPE_PN4T> {
    u32x4v b0, b1;
    __device__ __forceinline__ void decode(const MfmaRaw &r)
    {
        words(__builtin_amdgcn_alignbit(r.w.y, r.w.x, r.sh),
              __builtin_amdgcn_alignbit(r.tail, r.w.y, r.sh));
    }
    __device__ __forceinline__ void words(uint32_t w0, uint32_t w1)
    {
        // -z 2^(p-24) for z = 8 at p = 0, 4: fp16 words 0x8008, 0x8080
        constexpr uint32_t z0 = 0x80088008u, z4 = 0x80808080u;
        const uint32_t s0 = w0 >> 8, s1 = w1 >> 8;
        b0 = u32x4v{minus_z(w0 & 0x000F000Fu, z0), minus_z(w0 & 0x00F000F0u, z4),
                    minus_z(s0 & 0x000F000Fu, z0), minus_z(s0 & 0x00F000F0u, z4)};
        b1 = u32x4v{minus_z(w1 & 0x000F000Fu, z0), minus_z(w1 & 0x00F000F0u, z4),
                    minus_z(s1 & 0x000F000Fu, z0), minus_z(s1 & 0x00F000F0u, z4)};
    }
};

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));

// x operands of one block for one lane: SLOT, c[ks] (slot = the lane's token row); K-split,
// c[2 ks + h]. The upper half of pn3t's last step stays zero.
struct MfmaA {
    u32x4v c[6];
};

// One block of one 16-row tile: codes . x over the block, hi and lo passes, from C = 0. The chain
// is one asm block so that the accumulator stays in place (destination = C operand) from step to
// step, and the independent cycles around it are explicit: 3 before (operands just written by
// vector instructions) and 16 after (the result is read, and the sources may be rewritten, by
// vector instructions). Left to the compiler, a vector write to a register still being read as
// the C operand of an in-flight 16x16x32 step was scheduled too close on gfx950 and corrupted
// the sum.
template <int TYPE>
__device__ __forceinline__ mf_f4 mfma_block(const MfmaA &a, const MfmaB<TYPE> &b);
template <>
__device__ __forceinline__ mf_f4 mfma_block<PN_TYPE_PN3T>(const MfmaA &a,
                                                          const MfmaB<PN_TYPE_PN3T> &b)
{
    mf_f4 c;
    asm volatile("s_nop 2\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %1, %7, 0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %2, %7, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %3, %8, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %4, %8, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %5, %9, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %6, %9, %0\n\t"
                 "s_nop 7\n\t"
                 "s_nop 7"
                 : "=&v"(c)
                 : "v"(a.c[0]), "v"(a.c[1]), "v"(a.c[2]), "v"(a.c[3]), "v"(a.c[4]), "v"(a.c[5]),
                   "v"(b.b0), "v"(b.b1), "v"(b.b2));
    return c;
}
template <>
__device__ __forceinline__ mf_f4 mfma_block<PN_TYPE_PN4T>(const MfmaA &a,
                                                          const MfmaB<PN_TYPE_PN4T> &b)
{
    mf_f4 c;
    asm volatile("s_nop 2\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %1, %5, 0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %2, %5, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %3, %6, %0\n\t"
                 "v_mfma_f32_16x16x32_f16 %0, %4, %6, %0\n\t"
                 "s_nop 7\n\t"
                 "s_nop 7"
                 : "=&v"(c)
                 : "v"(a.c[0]), "v"(a.c[1]), "v"(a.c[2]), "v"(a.c[3]), "v"(b.b0), "v"(b.b1));
    return c;
}

// Two blocks of one 16-row tile at once: two independent chains interleaved (each step depends
// on the one two steps back), in place, with the same explicit independent cycles as mfma_block.
// SLOT: one A operand per k-step (hi and lo in token slots). K-split: hi and lo A operands.
template <int TYPE, bool SLOT> struct MfmaPair;
template <> struct MfmaPair<PN_TYPE_PN3T, true> {
    static __device__ __forceinline__ void run(mf_f4 &c0, mf_f4 &c1, const MfmaA &a0,
                                               const MfmaA &a1, const MfmaB<PN_TYPE_PN3T> &b0,
                                               const MfmaB<PN_TYPE_PN3T> &b1)
    {
        asm volatile("s_nop 2\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %2, %8, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %5, %11, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %3, %9, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %6, %12, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %4, %10, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %7, %13, %1\n\t"
                     "s_nop 7\n\t"
                     "s_nop 7"
                     : "=&v"(c0), "=&v"(c1)
                     : "v"(a0.c[0]), "v"(a0.c[1]), "v"(a0.c[2]), "v"(a1.c[0]), "v"(a1.c[1]),
                       "v"(a1.c[2]), "v"(b0.b0), "v"(b0.b1), "v"(b0.b2), "v"(b1.b0), "v"(b1.b1),
                       "v"(b1.b2));
    }
};
template <> struct MfmaPair<PN_TYPE_PN4T, true> {
    static __device__ __forceinline__ void run(mf_f4 &c0, mf_f4 &c1, const MfmaA &a0,
                                               const MfmaA &a1, const MfmaB<PN_TYPE_PN4T> &b0,
                                               const MfmaB<PN_TYPE_PN4T> &b1)
    {
        asm volatile("s_nop 2\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %2, %6, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %4, %8, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %3, %7, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %5, %9, %1\n\t"
                     "s_nop 7\n\t"
                     "s_nop 7"
                     : "=&v"(c0), "=&v"(c1)
                     : "v"(a0.c[0]), "v"(a0.c[1]), "v"(a1.c[0]), "v"(a1.c[1]), "v"(b0.b0),
                       "v"(b0.b1), "v"(b1.b0), "v"(b1.b1));
    }
};
template <> struct MfmaPair<PN_TYPE_PN3T, false> {
    static __device__ __forceinline__ void run(mf_f4 &c0, mf_f4 &c1, const MfmaA &a0,
                                               const MfmaA &a1, const MfmaB<PN_TYPE_PN3T> &b0,
                                               const MfmaB<PN_TYPE_PN3T> &b1)
    {
        asm volatile("s_nop 2\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %2, %14, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %8, %17, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %3, %14, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %9, %17, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %4, %15, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %10, %18, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %5, %15, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %11, %18, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %6, %16, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %12, %19, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %7, %16, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %13, %19, %1\n\t"
                     "s_nop 7\n\t"
                     "s_nop 7"
                     : "=&v"(c0), "=&v"(c1)
                     : "v"(a0.c[0]), "v"(a0.c[1]), "v"(a0.c[2]), "v"(a0.c[3]), "v"(a0.c[4]),
                       "v"(a0.c[5]), "v"(a1.c[0]), "v"(a1.c[1]), "v"(a1.c[2]), "v"(a1.c[3]),
                       "v"(a1.c[4]), "v"(a1.c[5]), "v"(b0.b0), "v"(b0.b1), "v"(b0.b2),
                       "v"(b1.b0), "v"(b1.b1), "v"(b1.b2));
    }
};
template <> struct MfmaPair<PN_TYPE_PN4T, false> {
    static __device__ __forceinline__ void run(mf_f4 &c0, mf_f4 &c1, const MfmaA &a0,
                                               const MfmaA &a1, const MfmaB<PN_TYPE_PN4T> &b0,
                                               const MfmaB<PN_TYPE_PN4T> &b1)
    {
        asm volatile("s_nop 2\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %2, %10, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %6, %12, 0\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %3, %10, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %7, %12, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %4, %11, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %8, %13, %1\n\t"
                     "v_mfma_f32_16x16x32_f16 %0, %5, %11, %0\n\t"
                     "v_mfma_f32_16x16x32_f16 %1, %9, %13, %1\n\t"
                     "s_nop 7\n\t"
                     "s_nop 7"
                     : "=&v"(c0), "=&v"(c1)
                     : "v"(a0.c[0]), "v"(a0.c[1]), "v"(a0.c[2]), "v"(a0.c[3]), "v"(a1.c[0]),
                       "v"(a1.c[1]), "v"(a1.c[2]), "v"(a1.c[3]), "v"(b0.b0), "v"(b0.b1),
                       "v"(b1.b0), "v"(b1.b1));
    }
};

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi)
{
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

typedef __attribute__((address_space(1))) const float gfloat_t;
typedef float mf_x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const mf_x4 gfloat4_t;

// One staging unit: token m, block brel of the phase, k-group g (PERG consecutive x values).
template <int TYPE>
__device__ __forceinline__ void mfma_load_unit(gfloat_t *x, int64_t K, int m,
                                               int64_t k0, int xvec4, float (&v)[MTile<TYPE>::PERG])
{
    constexpr int PERG = MTile<TYPE>::PERG;
    gfloat_t *src = x + (int64_t)m * K + k0;
    if (xvec4) {
#pragma unroll
        for (int q = 0; q < PERG / 4; q++) {
            const mf_x4 f = reinterpret_cast<gfloat4_t *>(src)[q];
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < PERG; e++)
            v[e] = src[e];
    }
}

// Bytes of one block's x operands in LDS: 16 bytes per (k-step of 8 codes, k-group, slot) for
// full steps; pn3t's last step of 4 codes takes 8 bytes (its other half is zero in registers).
// Then 16 exponents (one per token slot).
template <int TYPE> __host__ __device__ constexpr int mfma_a_bytes(int M)
{
    return TYPE == PN_TYPE_PN3T ? 320 * M : 256 * M;
}
template <int TYPE> __host__ __device__ constexpr int mfma_block_bytes(int M)
{
    return mfma_a_bytes<TYPE>(M) + 64;
}

// LDS byte offset of the A operand (k-step ks, hi or lo h) of token m in k-group g.
template <int TYPE, bool SLOT>
__device__ __forceinline__ int mfma_a_off(int ks, int h, int g, int m, int M)
{
    if (ks < 2)
        return SLOT ? ((ks * 4 + g) * 2 * M + 2 * m + h) * 16
                    : (((2 * ks + h) * 4 + g) * M + m) * 16;
    return 256 * M + (SLOT ? (g * 2 * M + 2 * m + h) * 8 : ((h * 4 + g) * M + m) * 8);
}

// A operands of one block for lane (n16, g) from the x area: SLOT, slot n16 (token n16 / 2, hi or
// lo by parity); K-split, token n16, hi and lo.
template <int TYPE, bool SLOT>
__device__ __forceinline__ void mfma_read_a(MfmaA &a, const uint8_t *blk, int g, int n16, int M)
{
    const int m = SLOT ? n16 >> 1 : n16;
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int h = 0; h < (SLOT ? 1 : 2); h++)
            a.c[SLOT ? ks : 2 * ks + h] = *reinterpret_cast<const u32x4v *>(
                blk + mfma_a_off<TYPE, SLOT>(ks, SLOT ? (n16 & 1) : h, g, m, M));
    if constexpr (MTile<TYPE>::KSTEPS == 3) {
#pragma unroll
        for (int h = 0; h < (SLOT ? 1 : 2); h++) {
            const u32x2v v = *reinterpret_cast<const u32x2v *>(
                blk + mfma_a_off<TYPE, SLOT>(2, SLOT ? (n16 & 1) : h, g, m, M));
            a.c[SLOT ? 2 : 4 + h].x = v.x;
            a.c[SLOT ? 2 : 4 + h].y = v.y;
        }
    }
}

// Stages x for the blocks [pb0, pb0 + npb) of a phase into the x area xa (mfma_block_bytes per
// block). Every thread of the workgroup calls it; it holds two barriers. One unit = one token m,
// one block, one k-group g: PERG consecutive x values; the 4 EG units of a group of EG blocks
// and one token sit in adjacent lanes. Per group and token, the exponent E is chosen from the
// group's largest |x| (so that |x| * 2^(E + 24) < 2^15) and x * 2^(E + 24 - p) is split into fp16
// hi + lo; -E is stored beside each block's operands and applied after the MFMA chains.
// Layout SLOT (up to 8 tokens): hi and lo are token slots 2m, 2m+1 of one A operand, so one MFMA
// per k-step covers both; K-split (up to 16 tokens): hi and lo are two A operands on the same
// codes. `after_loads` runs once the first x loads are issued (a caller's weight prefetch: loads
// retire in order, so waiting for x then leaves the prefetch in flight).
template <int TYPE, bool SLOT, int EG, class F>
__device__ __forceinline__ void mfma_stage(uint8_t *xa, const float *x, int64_t K, int M,
                                           int ML, int pb0, int npb, int xvec4, F after_loads)
{
    using T = MTile<TYPE>;
    constexpr int PERG = T::PERG;
    const int tid = threadIdx.x;
    const int per_block = mfma_block_bytes<TYPE>(ML), e_off = mfma_a_bytes<TYPE>(ML);
    constexpr int UNITS = kMfmaUnits;  // units per thread and pass
    const int U = npb * M * 4;
    const int nch = (U + kMfmaThreads * UNITS - 1) / (kMfmaThreads * UNITS);
    // unit u: k-group u % 4, then the block within its group of EG, then the token, then the group
    auto unit_coords = [&](int u, int &gg, int &m, int &brel) {
        gg = u & 3;
        const int v = u >> 2, bi = v % EG, w = v / EG;
        m = w % M;
        brel = EG * (w / M) + bi;
    };
    __syncthreads();  // earlier readers of the x area are done
    // x is a restrict kernel argument, so its loads may otherwise move past the prefetch below;
    // through an opaque copy of the address they stay in program order
    uint64_t xaddr = reinterpret_cast<uint64_t>(x);
    asm volatile("" : "+s"(xaddr));
    gfloat_t *xg = reinterpret_cast<gfloat_t *>(xaddr);
    float xr[UNITS][PERG];
    // loads outside any branch (a unit past the end loads the last one again), so the waits for
    // them can leave the weight prefetch issued after them in flight
    auto load = [&](int c) {
#pragma unroll
        for (int ub = 0; ub < UNITS; ub++) {
            const int u = min((c * UNITS + ub) * kMfmaThreads + tid, U - 1);
            int gg, m, brel;
            unit_coords(u, gg, m, brel);
            mfma_load_unit<TYPE>(xg, K, m, (int64_t)(pb0 + brel) * T::G + PERG * gg, xvec4, xr[ub]);
        }
    };
    auto convert = [&](int c) {
    #pragma unroll
            for (int ub = 0; ub < UNITS; ub++) {
                const int u = (c * UNITS + ub) * kMfmaThreads + tid;
                if (u < U) {  // U is a multiple of 4 EG: whole lane groups take this branch
                    int gg, m, brel;
                    unit_coords(u, gg, m, brel);
                    float mx = 0.f;
    #pragma unroll
                    for (int e = 0; e < PERG; e++)
                        mx = fmaxf(mx, fabsf(xr[ub][e]));
                    mx = fmaxf(mx, PN_DPP(mx, 0xB1));      // quad_perm [1,0,3,2]
                    mx = fmaxf(mx, PN_DPP(mx, 0x4E));      // quad_perm [2,3,0,1]
                    if (EG == 4) {
                        mx = fmaxf(mx, PN_DPP(mx, 0x124));  // row_ror:4
                        mx = fmaxf(mx, PN_DPP(mx, 0x128));  // row_ror:8
                    }
                    int ex = 0;
                    frexpf(mx, &ex);
                    const int E = mx > 0.f ? -9 - ex : 0;
                    const int eb = E + 24;
                    uint32_t hw[PERG / 2], lw[PERG / 2];
    #pragma unroll
                    for (int e = 0; e < PERG; e += 2) {
                        const float v0 = ldexpf(xr[ub][e], eb - T::pe(e));
                        const float v1 = ldexpf(xr[ub][e + 1], eb - T::pe(e + 1));
                        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                        hw[e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                        lw[e / 2] = pack_h2(v0 - (float)h0, v1 - (float)h1);
                    }
                    uint8_t *blk = xa + brel * per_block;
                    auto put16 = [&](int ks, int h, u32x4v v) {
                        *reinterpret_cast<u32x4v *>(blk + mfma_a_off<TYPE, SLOT>(ks, h, gg, m, ML)) = v;
                    };
                    put16(0, 0, u32x4v{hw[0], hw[1], hw[2], hw[3]});
                    put16(0, 1, u32x4v{lw[0], lw[1], lw[2], lw[3]});
                    put16(1, 0, u32x4v{hw[4], hw[5], hw[6], hw[7]});
                    put16(1, 1, u32x4v{lw[4], lw[5], lw[6], lw[7]});
                    if constexpr (T::KSTEPS == 3) {  // the last 4 codes
                        *reinterpret_cast<u32x2v *>(blk + mfma_a_off<TYPE, SLOT>(2, 0, gg, m, ML)) =
                            u32x2v{hw[8], hw[9]};
                        *reinterpret_cast<u32x2v *>(blk + mfma_a_off<TYPE, SLOT>(2, 1, gg, m, ML)) =
                            u32x2v{lw[8], lw[9]};
                    }
                    if (gg == 0) {
                        int *es = reinterpret_cast<int *>(blk + e_off);
                        if (SLOT)
                            es[2 * m] = es[2 * m + 1] = -E;
                        else
                            es[m] = -E;
                    }
                }
            }
    };
    load(0);
    asm volatile("" ::: "memory");  // the x loads are issued before the prefetch
    after_loads();
    asm volatile("" ::: "memory");
    convert(0);
    for (int c = 1; c < nch; c++) {
        load(c);
        convert(c);
    }
    const int used = SLOT ? 2 * M : M;
    for (int i = tid; i < npb * 16; i += kMfmaThreads)
        if ((i & 15) >= used)
            reinterpret_cast<int *>(xa + (i >> 4) * per_block + e_off)[i & 15] = 0;
    __syncthreads();
}

template <int TYPE, int TG>
__global__ void __launch_bounds__(kMfmaThreads)
pn_gemv_mfma_kernel(const uint8_t *__restrict__ W, int64_t N, int nb, int64_t row_bytes,
                    const float *__restrict__ x, int64_t K, int M, float *__restrict__ y,
                    int64_t rq, int rr, int Pb, int nph, int xvec4)
{
    constexpr int P = (8 + TG - 1) / TG;  // block steps of loads in flight (about 8 tiles' worth)
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int per_block = mfma_block_bytes<TYPE>(M);
    const int e_off = mfma_a_bytes<TYPE>(M);

    const int64_t wg = blockIdx.x;
    const int64_t r0 = wg * rq + (wg < rr ? wg : rr);
    const int64_t r1 = r0 + rq + (wg < rr ? 1 : 0);
    const int ntiles = (int)((r1 - r0 + 15) >> 4);
    const int ngroups = (ntiles + TG - 1) / TG;

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
            const int pb0 = p * Pb, npb = min(nb, pb0 + Pb) - pb0;
            mfma_stage<TYPE, false, 1>(lds, x, K, M, M, pb0, npb, xvec4, [] {});

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
                        if (n16 < M)
                            mfma_read_a<TYPE, false>(a, blk, g, n16, M);
                        const i32x4v ex = *reinterpret_cast<const i32x4v *>(blk + e_off + 16 * g);
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
                            const mf_f4 dd = mfma_block<TYPE>(a, bop);
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                acc[t][j] += ldexpf(dv * dd[j], ex[j]);
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
                        y[(int64_t)m * N + row] = s[j];
                }
            }
        }
    }
}

// ---- weights staged through LDS: 16 rows x 4 blocks per wave and step ------------------------
//
// A wave copies 16 rows x 4 blocks (16 segments of 136 contiguous bytes, 2176 bytes) straight from
// HBM into a private LDS slot with 9 buffer loads of one dword per lane (each covers 256
// contiguous bytes; the 9th, bytes 1920..2175 of the step, rewrites 128 of them with the same
// values), and each lane reads its two words per block from there. The direct loads of the
// other kernel touch 16-20 cache lines for 512 bytes per instruction; these, 2-3 per 256. Each
// wave keeps 3 steps in flight in a ring of 4 slots. The offsets within a step are constant per
// lane; the step's position is one scalar offset, and the buffer's bounds check reads rows past
// the matrix end as zero. Past its last step a wave re-issues its last one, so that exactly
// kWaitAfter loads follow every step it waits for. The waits are explicit (the compiler does not order LDS
// reads after these copies).
constexpr int kChunkBlocks = 4;
constexpr int kChunkBytes = 16 * kChunkBlocks * kBlockBytes;  // 2176
constexpr int kLdsRing = 4;                                    // slots per wave (a power of 2)
constexpr int kStepLoads = 9;                                  // buffer loads per step
// Steps in flight ahead of the one being read: every slot but that one. The wait for a step's copy
// therefore leaves exactly kWaitAfter loads (the later steps') in flight.
constexpr int kStepsAhead = kLdsRing - 1;
constexpr int kWaitAfter = kStepsAhead * kStepLoads;
static_assert(kWaitAfter <= 63, "vmcnt holds at most 63 loads");
static_assert(kStepLoads == 8 + 1, "issue(): 8 loads of 64 dwords and one of the last 64");

typedef __attribute__((address_space(3))) void lds_void_t;

// MC: the token capacity of the x layout (2, 4, 8 or 16; M <= MC), so that every LDS offset of
// the loop is a constant. Up to 8, hi and lo are token slots.
template <int TYPE, int TG, int MC>
__device__ __forceinline__ void
mfma_lds_body(const uint8_t *__restrict__ W, int64_t N, int nb, int64_t row_bytes,
              const float *__restrict__ x, int64_t K, int M, float *__restrict__ y, int64_t rq,
              int rr, int Pb, int nph, int xvec4, int blk_id){
    constexpr bool SLOT = MC <= 8;
    constexpr int ACC = SLOT ? 2 : 4;       // tokens per lane
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    constexpr int per_block = mfma_block_bytes<TYPE>(MC);
    constexpr int e_off = mfma_a_bytes<TYPE>(MC);
    const int alim = SLOT ? 2 * M : M;  // lanes (by n16) that hold A operands
    // x area first (its offsets fit the 16-bit immediates of LDS instructions), then the slots
    uint8_t *const xa = lds;
    uint8_t *const ring = lds + Pb * per_block + wave * kLdsRing * kChunkBytes;

    const int64_t wg = blk_id;
    const int64_t r0 = wg * rq + (wg < rr ? wg : rr);
    const int64_t r1 = r0 + rq + (wg < rr ? 1 : 0);
    const int ntiles = (int)((r1 - r0 + 15) >> 4);
    const int ngroups = (ntiles + TG - 1) / TG;

    // dword k of a step (row k / 34, byte 4 (k % 34) of its segment): k = 64 j + lane for
    // j < 8, k = 480 + lane for the 9th load
    const __amdgpu_buffer_rsrc_t wres =
        __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, (int)(N * row_bytes), 0x00020000);
    uint32_t voff[kStepLoads];
#pragma unroll
    for (int j = 0; j < kStepLoads; j++) {
        const int k = j < 8 ? 64 * j + lane : 480 + lane;
        voff[j] = (uint32_t)((k / 34) * row_bytes + 4 * (k % 34));
    }
    auto issue = [&](int tile, int c4, int slot) {  // tile: index within the workgroup
        uint8_t *dst = ring + slot * kChunkBytes;
        const uint32_t soff = (uint32_t)((r0 + 16 * (int64_t)tile) * row_bytes) +
                              (uint32_t)(c4 * kChunkBlocks * kBlockBytes);
#pragma unroll
        for (int j = 0; j < kStepLoads; j++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t *)(dst + (j < 8 ? 256 * j : 1920)),
                                                     4, voff[j], soff, 0, 0);
    };

    MfmaA a0, a1;
#pragma unroll
    for (int ch = 0; ch < 6; ch++)
        a0.c[ch] = a1.c[ch] = u32x4v{0u, 0u, 0u, 0u};

    for (int grp = 0; grp < ngroups; grp++) {
        const int t0 = grp * TG;
        const int gt = min(TG, ntiles - t0);
        float acc[TG][ACC];
#pragma unroll
        for (int t = 0; t < TG; t++)
#pragma unroll
            for (int j = 0; j < ACC; j++)
                acc[t][j] = 0.f;

        for (int p = 0; p < nph; p++) {
            const int pb0 = p * Pb, npb = min(nb, pb0 + Pb) - pb0;  // both multiples of 4
            const int n4 = npb >> 2, c40 = pb0 >> 2;
            // items (tile, 4-block step), tile-major, split evenly over the 8 waves
            const int items = gt * n4;
            const int i0 = (wave * items) / kMfmaWaves, i1 = ((wave + 1) * items) / kMfmaWaves;
            // prefetch cursor: item pf (slot pf % 4) is (tile pt, step pc); past the wave's last
            // item it stays on that item (the copy is re-issued, nothing reads it)
            int pf = i0, pt = i0 / n4, pc = i0 % n4;
            auto issue_next = [&]() {
                issue(t0 + pt, c40 + pc, pf & (kLdsRing - 1));
                if (pf + 1 < i1 && ++pc == n4) {
                    pc = 0;
                    ++pt;
                }
                ++pf;
            };
            mfma_stage<TYPE, SLOT, kChunkBlocks>(xa, x, K, M, MC, pb0, npb, xvec4, [&] {
#pragma unroll
                for (int s = 0; s < kStepsAhead; s++)
                    issue_next();
            });
#pragma unroll
            for (int t = 0; t < TG; t++) {
                const int lo = max(i0, t * n4), hi = min(i1, (t + 1) * n4);
                for (int it = lo; it < hi; it++) {
                    // refill the slot read one step ago, then wait for this step's copy: loads
                    // retire in order and exactly kStepsAhead steps (kWaitAfter loads) were
                    // issued after it
                    asm volatile("" ::: "memory");  // that slot's reads stay before
                    issue_next();
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitAfter) : "memory");
                    const uint8_t *cr = ring + (it & (kLdsRing - 1)) * kChunkBytes + 136 * n16;
                    const uint8_t *cw = cr + 8 * g;
                    const uint8_t *xb = xa + ((it - t * n4) * kChunkBlocks) * per_block;
                    // the step's 4 blocks share one exponent per token (-E stored per block)
                    const i32x4v nE = *reinterpret_cast<const i32x4v *>(xb + e_off + 16 * g);
                    float sacc[ACC];
#pragma unroll
                    for (int j = 0; j < ACC; j++)
                        sacc[j] = 0.f;
#pragma unroll
                    for (int jp = 0; jp < 2; jp++) {
                        // block 2jp: words 2 mod 4 aligned (read 12 bytes from 2 before);
                        // block 2jp+1: words 4-byte aligned
                        const int j0 = 2 * jp, j1 = 2 * jp + 1;
                        const uint32_t *e = reinterpret_cast<const uint32_t *>(cw + 34 * j0);
                        const uint32_t *o = reinterpret_cast<const uint32_t *>(cw + 34 * j1 + 2);
                        const uint32_t e0 = e[0], e1 = e[1], e2 = e[2], o0 = o[0], o1 = o[1];
                        const float d0 = f16_bits_to_f32(
                            *reinterpret_cast<const uint16_t *>(cr + 34 * j0));
                        const float d1 = f16_bits_to_f32(
                            *reinterpret_cast<const uint16_t *>(cr + 34 * j1));
                        const uint8_t *x0 = xb + j0 * per_block, *x1 = xb + j1 * per_block;
                        if (n16 < alim) {
                            mfma_read_a<TYPE, SLOT>(a0, x0, g, n16, MC);
                            mfma_read_a<TYPE, SLOT>(a1, x1, g, n16, MC);
                        }
                        mf_f4 c0, c1;
                        MfmaB<TYPE> b0, b1;
                        b0.words(__builtin_amdgcn_alignbit(e1, e0, 16),
                                 __builtin_amdgcn_alignbit(e2, e1, 16));
                        b1.words(o0, o1);
                        MfmaPair<TYPE, SLOT>::run(c0, c1, a0, a1, b0, b1);
                        if (SLOT) {  // hi + lo slots, times d
                            sacc[0] = fmaf(d0, c0[0] + c0[1], sacc[0]);
                            sacc[1] = fmaf(d0, c0[2] + c0[3], sacc[1]);
                            sacc[0] = fmaf(d1, c1[0] + c1[1], sacc[0]);
                            sacc[1] = fmaf(d1, c1[2] + c1[3], sacc[1]);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; j++) {
                                sacc[j] = fmaf(d0, c0[j], sacc[j]);
                                sacc[j] = fmaf(d1, c1[j], sacc[j]);
                            }
                        }
                    }
                    // undo the step's exponent: an exact scaling of the step's sum
#pragma unroll
                    for (int j = 0; j < ACC; j++)
                        acc[t][j] += ldexpf(sacc[j], nE[SLOT ? 2 * j : j]);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the re-issued steps too
        }

        // ---- partial sums of the 8 waves, added in wave order ----
        __syncthreads();  // every wave is done with its slots and the x area
        mf_f4 *red = reinterpret_cast<mf_f4 *>(lds);
#pragma unroll
        for (int t = 0; t < TG; t++) {
            mf_f4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < ACC; j++)
                v[j] = acc[t][j];
            red[(t * kMfmaWaves + wave) * 64 + lane] = v;
        }
        __syncthreads();
        for (int i = tid; i < gt * 64; i += kMfmaThreads) {
            const int t = i >> 6, l = i & 63;
            mf_f4 sm = red[(t * kMfmaWaves) * 64 + l];
#pragma unroll
            for (int w = 1; w < kMfmaWaves; w++)
                sm += red[(t * kMfmaWaves + w) * 64 + l];
            const int64_t row = r0 + 16 * (int64_t)(t0 + t) + (l & 15);
            if (row < r1) {
#pragma unroll
                for (int j = 0; j < ACC; j++) {
                    const int m = ACC * (l >> 4) + j;
                    if (m < M)
                        y[(int64_t)m * N + row] = sm[j];
                }
            }
        }
    }
}
template <int TYPE, int TG, int MC>
__global__ void __launch_bounds__(kMfmaThreads)
pn_gemv_mfma_lds_kernel(const uint8_t *__restrict__ W, int64_t N, int nb, int64_t row_bytes,
                        const float *__restrict__ x, int64_t K, int M, float *__restrict__ y,
                        int64_t rq, int rr, int Pb, int nph, int xvec4)
{
    mfma_lds_body<TYPE, TG, MC>(W, N, nb, row_bytes, x, K, M, y, rq, rr, Pb, nph, xvec4,
                                (int)blockIdx.x);
}

// LDS for the x of a phase and, aliased, the 8 waves' partial sums (8 KB per tile of the group).
constexpr int kMfmaLds = 160 * 1024 - 1024;

template <int TYPE, int TG>
static int launch_mfma_tg(const uint8_t *W, int64_t N, int nb, const float *x, int64_t K, int M,
                          float *y, int64_t rq, int rr, int grid, int Pb, int nph, hipStream_t s)
{
    const size_t lds = std::max<size_t>((size_t)Pb * mfma_block_bytes<TYPE>(M),
                                        (size_t)TG * kMfmaWaves * 64 * 16);
    constexpr auto kern = pn_gemv_mfma_kernel<TYPE, TG>;
    if (!lds_limit_once<kern>(kMfmaLds))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMfmaThreads), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, M, y, rq, rr, Pb, nph,
                       aligned(x, 16) ? 1 : 0);
    return launch_status();
}

template <int TYPE, int TG, int MC>
static int launch_mfma_lds_tg(const uint8_t *W, int64_t N, int nb, const float *x, int64_t K,
                              int M, float *y, int64_t rq, int rr, int grid, int Pb, int nph,
                              size_t lds, hipStream_t s)
{
    constexpr auto kern = pn_gemv_mfma_lds_kernel<TYPE, TG, MC>;
    if (!lds_limit_once<kern>(kMfmaLds))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMfmaThreads), lds, s, W, N, nb,
                       (int64_t)nb * kBlockBytes, x, K, M, y, rq, rr, Pb, nph,
                       aligned(x, 16) ? 1 : 0);
    return launch_status();
}

template <int TYPE, int MC>
static int launch_mfma_lds_t(const uint8_t *W, int64_t N, int nb, const float *x, int64_t K, int M,
                             float *y, int grid, int64_t rq, int rr, hipStream_t s)
{
    // tiles of 16 rows per group
    constexpr int max_tg = kMfmaMaxTG;
    const int64_t tiles_max = (rq + (rr ? 1 : 0) + 15) / 16;
    const int64_t ng = (tiles_max + max_tg - 1) / max_tg;
    const int TG = (int)((tiles_max + ng - 1) / ng);
    const int ring = kMfmaWaves * kLdsRing * kChunkBytes;
    const int per_block = mfma_block_bytes<TYPE>(MC);
    const int pb_max = ((kMfmaLds - ring) / per_block) & ~(kChunkBlocks - 1);
    const int nph = (nb + pb_max - 1) / pb_max;
    const int Pb = ((nb + nph - 1) / nph + kChunkBlocks - 1) & ~(kChunkBlocks - 1);
    // x area (Pb blocks), then the slots; the partial sums at the end alias the start
    const size_t lds = std::max<size_t>((size_t)Pb * per_block + ring, (size_t)TG * 8192);
    switch (TG) {
#define PN_MFMA_CASE(tg)                                                                           \
    case tg:                                                                                       \
        if constexpr (tg <= max_tg)                                                                \
            return launch_mfma_lds_tg<TYPE, tg, MC>(W, N, nb, x, K, M, y, rq, rr, grid, Pb, nph, \
                                                      lds, s);                                 \
        else                                                                                       \
            return PN_ERR_SHAPE;
    PN_MFMA_CASE(1) PN_MFMA_CASE(2) PN_MFMA_CASE(3) PN_MFMA_CASE(4) PN_MFMA_CASE(5)
    PN_MFMA_CASE(6) PN_MFMA_CASE(7) PN_MFMA_CASE(8) PN_MFMA_CASE(9)
#undef PN_MFMA_CASE
    default: return PN_ERR_SHAPE;
    }
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
    // weights staged through LDS (4-byte aligned W, rows of a multiple of 4 blocks);
    // PN_GEMV_MFMA_DIRECT keeps the direct-load kernel (tests, timing)
    if (mfma_stages_weights(TYPE, W, N, K))
        return M == 2   ? launch_mfma_lds_t<TYPE, 2>(W, N, nb, x, K, M, y, grid, rq, rr, s)
               : M <= 4 ? launch_mfma_lds_t<TYPE, 4>(W, N, nb, x, K, M, y, grid, rq, rr, s)
               : M <= 8 ? launch_mfma_lds_t<TYPE, 8>(W, N, nb, x, K, M, y, grid, rq, rr, s)
                        : launch_mfma_lds_t<TYPE, 16>(W, N, nb, x, K, M, y, grid, rq, rr, s);
    const int per_block = mfma_block_bytes<TYPE>(M);
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

// Whether the matrix-core path stages these weights through LDS: 4-byte aligned, rows of a
// multiple of 4 blocks, offsets (rows + a tile) within 31 bits.
bool mfma_stages_weights(int type, const void *W, int64_t N, int64_t K)
{
    const int64_t nb = K / (type == PN_TYPE_PN3T ? 80 : 64);
    return aligned(W, 4) && nb % kChunkBlocks == 0 && (N + 16) * nb * kBlockBytes < (int64_t(1) << 31) &&
           !getenv("PN_GEMV_MFMA_DIRECT");
}

int launch_mfma(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int M, float *y,
                int cus, hipStream_t s)
{
    if (type == PN_TYPE_PN3T)
        return launch_mfma_t<PN_TYPE_PN3T>(W, N, K, x, M, y, cus, s);
    return launch_mfma_t<PN_TYPE_PN4T>(W, N, K, x, M, y, cus, s);
}

}  // namespace pn
