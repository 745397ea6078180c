// pn_gemv_rows.hip -- PN decode-step GEMV y = W.x at 1-4 tokens on the vector units of gfx950.
//
// Format: "PN weight format" (PNX-FORMAT-v0): "Block layout" (34-byte blocks: fp16 d, then eight
// little-endian u32 words; code t of a word at bit BITS*(t>>1) + 16*(t&1), so no code crosses a
// 16-bit half), "Value" (w = d * (n - z), exact in fp32).
//
// Arithmetic (exact decode, x as given in fp32):
//  * Every 16-bit half of a word holds PAIRS codes at bits BITS*r (r < PAIRS). One and-or keeps
//    the codes at bit p = BITS*r of both halves of a dword and writes the fp16 exponent of
//    2^(10-p) over them: each half becomes the fp16 number 2^(10-p) + n, exactly. One packed fp16
//    add of -(2^(10-p) + z) leaves the integer n - z in each half, exactly (code z gives +0): no
//    zero-point fold and no cancellation. Positions past the fp16 mantissa are reached after one
//    shift of the dword (by 9 for pn3t, 8 for pn4t).
//  * Each weight then takes one v_fma_mix_f32 per token: the fp16 n - z widens exactly and its
//    product with the fp32 x is exact inside the fma, so the only roundings are fp32 sums: four
//    chains per lane and item, one multiply by the block's d, a 64-lane tree and the in-order sum
//    over a row's chunks (and K slices).
//  * At 2-4 tokens each code goes to fp32 instead (an and-or under an fp32 exponent, one exact
//    subtraction), and each token takes a plain v_fma_f32: the same values, products and sums.
//
// Reading blocks whose words are not 4-byte aligned. Take a block that starts at a 4-byte aligned
// address p (its words straddle dwords): the aligned dwords D_i = bytes [p + 4i, p + 4i + 4) hold
// (d | w0.lo), (w0.hi | w1.lo), ..., (w6.hi | w7.lo), (w7.hi | next block's d). Every half of
// these still has its codes at bits BITS*r, so each of D_1..D_7 decodes as it stands (low half:
// the odd codes of word i-1, high half: the even codes of word i), and one v_bfi joins D_0's high
// half and D_8's low half into a ninth. A block at 2 mod 4 is read from p - 2: D_0 = (previous
// block's last half | d), D_1..D_8 = its eight aligned words. Either way a lane reads P + 1 aligned
// dwords and decodes P of them; only the x each half meets differs, and that is fixed per lane.
//
// Work split: a lane owns a "piece" of P consecutive words of one block (P = 8, 4 or 2); a wave
// covers a chunk of 64 pieces (8P blocks) of a row per item and keeps that chunk's x in registers
// (read from the workgroup's copy of x in LDS when its chunk changes). A workgroup (one per CU,
// 8 or 12 waves) owns a contiguous range of rows; its items (chunk, row), chunk-major, form groups
// of up to D rows of one chunk. Where a row is one chunk its waves take the groups one at a time
// from a counter in LDS as they free up; otherwise each wave owns a contiguous run of them. Each
// lane's words come straight from HBM into registers through buffer loads, one group ahead of the
// decode. Per group the 64 lane sums of its items are added by DPP and permlane
// swaps; one lane writes each item's partial to LDS, and at the end the workgroup adds each row's
// chunk partials in chunk order and writes y. The partial of an item does not depend on the wave
// that computes it, and nothing is added in arrival order: the same inputs and launch shape give
// the same bits.
#include <stdlib.h>

#include <algorithm>

#include "pn_common.h"

namespace pn {
namespace rows {

// Dynamic LDS every launch requests at least: more than half of the CU's 160 KB, so that no CU
// ever holds two of these workgroups while another holds none.
constexpr int kLdsFloor = 82 * 1024;
constexpr int kLdsMax = 160 * 1024;
// x a workgroup can always stage (more where the partials leave room; the host cuts K into
// slices beyond that).
constexpr int kXLdsMax = 128 * 1024;

template <int TYPE> struct Dec;
template <> struct Dec<PN_TYPE_PN3T> {
    // NPOS code positions per half are decoded in place (bit BITS*r, r < NPOS), the rest after a
    // shift of the dword by SHIFT bits
    static constexpr int BITS = 3, CPW = 10, PAIRS = 5, Z = 4, G = 80, NPOS = 3, SHIFT = 9;
    // fp32 decode (3-4 tokens): codes whose bit in the dword lies past bit 20 are read after a
    // shift by SH32
    static constexpr int SH32 = 8;
    // floats a block of x takes in LDS: 20 mod 32 words, so that the 16-byte reads of 8
    // consecutive lanes (blocks 84 words apart) fall on 8 disjoint groups of 4 banks
    static constexpr int GS = 84;
};
template <> struct Dec<PN_TYPE_PN4T> {
    static constexpr int BITS = 4, CPW = 8, PAIRS = 4, Z = 8, G = 64, NPOS = 2, SHIFT = 8;
    static constexpr int SH32 = 12;
    static constexpr int GS = 68;  // 4 mod 32 words
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// One matrix of a grouped launch (several matrices of one type and K that read the same x): its
// workgroups are [g0, next part's g0), and it replaces base, nbytes, par, N, y and ystride.
struct Part {
    const uint8_t *base;
    uint32_t nbytes;
    uint32_t par;
    int N;
    int g0;
    float *y;
    int64_t ystride;
    int type;             // a launch of mixed types: the part's type and its row shape
    uint32_t row_stride;
    int nb;
    int NC;
    int rows_max;
};
constexpr int kMaxParts = 4;

struct Args {
    const uint8_t *base;  // 4-byte aligned start of the bytes this launch reads
    uint32_t nbytes;      // bytes from base the launch may read (a multiple of 4)
    uint32_t par;         // the first block of row 0 starts at base + par (0 or 2)
    uint32_t row_stride;  // bytes from one row of the launch to the next (a multiple of 4)
    int N;                // rows of the launch
    int nb;               // blocks per row in this slice of K
    int NC;               // chunks of 8P blocks per row (the last may be partial)
    int rows_max;         // rows of the workgroup with the most rows
    const float *x;       // x of this slice: x[m * xstride + k], k < nb * G
    int64_t xstride;
    float *y;             // y[m * ystride + n * yinc] for launch row n
    int64_t ystride;
    int64_t yinc;
    int accumulate;       // add to y (later slices of K) instead of overwriting it
    int nparts;           // 0: one matrix (the fields above); else parts[0..nparts)
    Part parts[kMaxParts];
};

// One item's registers: the P + 1 aligned dwords of the lane's piece and (P < 8) the dword that
// holds the block's d.
template <int P> struct Slot {
    uint32_t s[P + 1];
    uint32_t dw;
};

template <int P>
__device__ __forceinline__ void load_slot(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t dvoff,
                                          uint32_t soff, Slot<P> &sl)
{
    if constexpr (P == 8) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16u, soff, 0);
        sl.s[8] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 32u, soff, 0);
        sl.s[0] = a[0]; sl.s[1] = a[1]; sl.s[2] = a[2]; sl.s[3] = a[3];
        sl.s[4] = b[0]; sl.s[5] = b[1]; sl.s[6] = b[2]; sl.s[7] = b[3];
        sl.dw = 0;
    } else if constexpr (P == 4) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        sl.s[4] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 16u, soff, 0);
        sl.dw = __builtin_amdgcn_raw_buffer_load_b32(rs, dvoff, soff, 0);
        sl.s[0] = a[0]; sl.s[1] = a[1]; sl.s[2] = a[2]; sl.s[3] = a[3];
    } else {
        static_assert(P == 2, "pieces of 2, 4 or 8 words");
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
        sl.s[2] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 8u, soff, 0);
        sl.dw = __builtin_amdgcn_raw_buffer_load_b32(rs, dvoff, soff, 0);
        sl.s[0] = a[0]; sl.s[1] = a[1];
    }
}

// Decode constants kept in registers (the and-or is a VOP3 instruction: no literal operands).
// Position u (bit p = BITS * u of each half): the code mask in both halves, the fp16 exponent field
// 25 - p in both halves (the code n becomes the fp16 number 2^(10 - p) + n), and
// -(2^(10 - p) + z) in both halves.
template <int TYPE> struct Consts {
    uint32_t mask[Dec<TYPE>::NPOS];
    uint32_t magic[Dec<TYPE>::NPOS];
    h2 bias[Dec<TYPE>::NPOS];
};

template <int TYPE>
__device__ __forceinline__ Consts<TYPE> make_consts()
{
    using D = Dec<TYPE>;
    Consts<TYPE> c;
#pragma unroll
    for (int u = 0; u < D::NPOS; u++) {
        const int p = D::BITS * u;
        uint32_t mk = (((1u << D::BITS) - 1u) << p) * 0x00010001u;
        uint32_t mg = ((uint32_t)(25 - p) << 10) * 0x00010001u;
        const _Float16 bz = (_Float16)(-(float)((1 << (10 - p)) + D::Z));
        uint32_t bb = __builtin_bit_cast(uint32_t, h2{bz, bz});
        asm volatile("" : "+v"(mk));
        asm volatile("" : "+v"(mg));
        asm volatile("" : "+v"(bb));
        c.mask[u] = mk;
        c.magic[u] = mg;
        c.bias[u] = __builtin_bit_cast(h2, bb);
    }
    return c;
}

// The fp32 decode of 2-4 tokens: code r of half h sits at bit q = BITS*r + 16*h of the dword (or of
// the dword shifted right by SH32, where q + BITS > 23); one and-or keeps it under the fp32
// exponent of 2^(23-q), so the float is 2^(23-q) + n exactly, and one fp32 subtraction of
// 2^(23-q) + z leaves n - z exactly. Each weight then takes plain fp32 fmas, one per token, where
// the fp16 decode takes a mixed-precision fma per token: the same products and sums, bit for bit.
template <int TYPE> struct Consts32 {
    uint32_t mask[Dec<TYPE>::PAIRS][2];
    uint32_t magic[Dec<TYPE>::PAIRS][2];
};

template <int TYPE> __host__ __device__ constexpr int q32(int r, int h)
{
    using D = Dec<TYPE>;
    const int q = D::BITS * r + 16 * h;
    return q + D::BITS > 23 ? q - D::SH32 : q;
}

template <int TYPE>
__device__ __forceinline__ Consts32<TYPE> make_consts32()
{
    using D = Dec<TYPE>;
    Consts32<TYPE> c;
#pragma unroll
    for (int r = 0; r < D::PAIRS; r++)
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int q = q32<TYPE>(r, h);
            uint32_t mk = ((1u << D::BITS) - 1u) << q, mg = (uint32_t)(127 + 23 - q) << 23;
            asm volatile("" : "+v"(mk));
            asm volatile("" : "+v"(mg));
            c.mask[r][h] = mk;
            c.magic[r][h] = mg;
        }
    return c;
}

// Per-lane constants of the piece: offsets of its dwords from a row chunk's start, and how its
// halves pair with x.
struct Lane {
    uint32_t voff;   // the first of the P + 1 dwords
    uint32_t dvoff;  // the dword holding d (D_0 of the block)
    uint32_t voffl;  // voff in the last chunk of a row: past every buffer for a lane past the
    uint32_t dvoffl; // row's end, so that its loads read nothing (dvoff likewise)
    uint32_t bmask;  // v_bfi mask joining dword 0 and dword P into the last decoded dword
    uint32_t dsh;    // bit of d in its dword (0 or 16)
    bool straddle;   // the block starts at 0 mod 4 (its words straddle dwords)
    int bl;          // block of the piece within a chunk
    int xoff;        // LDS offset (floats) of the piece's x within a chunk
};

// x of the piece for one token, in decode order: xs[j][h][r] multiplies the code at pair r of half
// h of decoded dword j. Words 4-byte aligned (block at 2 mod 4): dword j is word j of the piece,
// low half = even codes, high half = odd codes. Words at 2 mod 4 (block at 0 mod 4): dword j
// (j < P-1) holds the odd codes of word j (low half) and the even codes of word j+1 (high half);
// the joined last dword holds the odd codes of word P-1 and the even codes of word 0. xp: the
// piece's CPW * P consecutive x values in LDS (16-byte aligned).
template <int TYPE, int P>
__device__ __forceinline__ void read_x(const float *xp, bool straddle,
                                       float (&xs)[P][2][Dec<TYPE>::PAIRS])
{
    using D = Dec<TYPE>;
    constexpr int XN = D::CPW * P;
    // the aligned order first, read straight into place: x[CPW j + 2r + h] -> xs[j][h][r]
#pragma unroll
    for (int i = 0; i < XN; i += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(xp + i);
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int e = i + u, j = e / D::CPW, c = e - j * D::CPW;
            xs[j][c & 1][c >> 1] = f[u];
        }
    }
    // then, where the words straddle dwords, the cyclic shift in place: (e_j, o_j) -> (o_j, e_j+1)
    float e0[D::PAIRS];
#pragma unroll
    for (int r = 0; r < D::PAIRS; r++)
        e0[r] = xs[0][0][r];
#pragma unroll
    for (int j = 0; j < P; j++)
#pragma unroll
        for (int r = 0; r < D::PAIRS; r++) {
            const float o = xs[j][1][r];
            const float en = j < P - 1 ? xs[j + 1][0][r] : e0[r];
            xs[j][0][r] = straddle ? o : xs[j][0][r];
            xs[j][1][r] = straddle ? en : o;
        }
}

// One item: out[m] = d * sum over the piece of (n - z) * x[m, k]. Software-pipelined: the codes of
// dword j + 1 are decoded while dword j's products accumulate, into eight chains per token, so
// that no instruction waits on the one just before it.
template <int TYPE, int P>
__device__ __forceinline__ void decode_dword(uint32_t v, const Consts<TYPE> &c,
                                             h2 (&n)[Dec<TYPE>::PAIRS])
{
    using D = Dec<TYPE>;
    const uint32_t vs = v >> D::SHIFT;
#pragma unroll
    for (int r = 0; r < D::PAIRS; r++) {
        const int u = r < D::NPOS ? r : r - D::NPOS;
        const uint32_t src = r < D::NPOS ? v : vs;
        n[r] = __builtin_bit_cast(h2, (src & c.mask[u]) | c.magic[u]) + c.bias[u];
    }
}

template <int TYPE, int M, int P>
__device__ __forceinline__ void item_mac(const Slot<P> &sl, const Lane &ln, uint32_t dwid,
                                         const float (&xs)[M][P][2][Dec<TYPE>::PAIRS],
                                         const Consts<TYPE> &c, const Consts32<TYPE> &c32,
                                         float (&out)[M])
{
    using D = Dec<TYPE>;
    constexpr int CH = 4;  // chains per token and half
    float acc[M][CH][2];
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int k = 0; k < CH; k++)
            acc[m][k][0] = acc[m][k][1] = 0.0f;
    const uint32_t last = (ln.bmask & sl.s[0]) | (~ln.bmask & sl.s[P]);
    if constexpr (M >= 2) {
#pragma unroll
        for (int j = 0; j < P; j++) {
            const uint32_t v = j < P - 1 ? sl.s[j + 1] : last;
            const uint32_t vs = v >> D::SH32;
#pragma unroll
            for (int r = 0; r < D::PAIRS; r++) {
                const int k = (j * D::PAIRS + r) % CH;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int q = D::BITS * r + 16 * h;
                    const uint32_t src = q + D::BITS > 23 ? vs : v;
                    const float w =
                        __builtin_bit_cast(float, (src & c32.mask[r][h]) | c32.magic[r][h]) -
                        (float)((1u << (23 - q32<TYPE>(r, h))) + (uint32_t)D::Z);
#pragma unroll
                    for (int m = 0; m < M; m++)
                        acc[m][k][h] = __builtin_fmaf(w, xs[m][j][h][r], acc[m][k][h]);
                }
            }
        }
    } else {
    h2 n[2][D::PAIRS];
    decode_dword<TYPE, P>(P > 1 ? sl.s[1] : last, c, n[0]);
#pragma unroll
    for (int j = 0; j < P; j++) {
        if (j + 1 < P)
            decode_dword<TYPE, P>(j + 1 < P - 1 ? sl.s[j + 2] : last, c, n[(j + 1) & 1]);
#pragma unroll
        for (int r = 0; r < D::PAIRS; r++) {
            const h2 nn = n[j & 1][r];
            const float wlo = (float)nn.x, whi = (float)nn.y;
            const int k = (j * D::PAIRS + r) % CH;
#pragma unroll
            for (int m = 0; m < M; m++) {
                acc[m][k][0] = __builtin_fmaf(wlo, xs[m][j][0][r], acc[m][k][0]);
                acc[m][k][1] = __builtin_fmaf(whi, xs[m][j][1][r], acc[m][k][1]);
            }
        }
    }
    }
    // d of the block; zero width for lanes past the end of the row (their x is zero too)
    const uint32_t dbits = __builtin_amdgcn_ubfe(P == 8 ? sl.s[0] : sl.dw, ln.dsh, dwid);
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)dbits);
#pragma unroll
    for (int m = 0; m < M; m++) {
        float t[CH];
#pragma unroll
        for (int k = 0; k < CH; k++)
            t[k] = acc[m][k][0] + acc[m][k][1];
        out[m] = d * ((t[0] + t[1]) + (t[2] + t[3]));
    }
}

typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// The matrix a workgroup works on: the launch's (one matrix) or, in a grouped launch, its part's,
// found from the part table (uniform; no indexing of the argument array), with g and G made
// part-local. Scalars only, so that nothing of the argument goes to private memory.
struct View {
    const uint8_t *base;
    uint32_t nbytes, par, row_stride;
    int N, nb, NC, rows_max;
    float *y;
    int64_t ystride;
    int g, G, type;
};

__device__ __forceinline__ View make_view(const Args &a0, int type, bool mixed)
{
    View v;
    v.base = a0.base;
    v.nbytes = a0.nbytes;
    v.par = a0.par;
    v.row_stride = a0.row_stride;
    v.N = a0.N;
    v.nb = a0.nb;
    v.NC = a0.NC;
    v.rows_max = a0.rows_max;
    v.y = a0.y;
    v.ystride = a0.ystride;
    v.g = blockIdx.x;
    v.G = gridDim.x;
    v.type = type;
    if (a0.nparts > 0) {
        int pi = 0;
#pragma unroll
        for (int i = 1; i < kMaxParts; i++)
            pi = i < a0.nparts && v.g >= a0.parts[i].g0 ? i : pi;
#pragma unroll
        for (int i = 0; i < kMaxParts; i++)
            if (i == pi) {
                const Part &pt = a0.parts[i];
                const int gend = i + 1 < a0.nparts ? a0.parts[i + 1 < kMaxParts ? i + 1 : i].g0 : v.G;
                v.base = pt.base;
                v.nbytes = pt.nbytes;
                v.par = pt.par;
                v.N = pt.N;
                v.y = pt.y;
                v.ystride = pt.ystride;
                if (mixed) {
                    v.type = pt.type;
                    v.row_stride = pt.row_stride;
                    v.nb = pt.nb;
                    v.NC = pt.NC;
                    v.rows_max = pt.rows_max;
                }
                v.g -= pt.g0;
                v.G = gend - pt.g0;
            }
    }
    return v;
}

template <int TYPE, int M, int P, int DEPTH, int NW, int PRE, bool DYN>
__device__ __forceinline__ void rows_body(const Args &a, const View &v)
{
    const int g = v.g, G = v.G;
    using D = Dec<TYPE>;
    constexpr int PPB = 8 / P;   // pieces per block
    constexpr int CB = 8 * P;    // blocks per chunk
    constexpr uint32_t CBYTES = 34u * CB;
    constexpr int LOADS = 3;     // load instructions per item
    static_assert(DEPTH * LOADS <= 63, "vmcnt range");
    extern __shared__ float lds[];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = (int)((int64_t)v.N * g / G), r1 = (int)((int64_t)v.N * (g + 1) / G);
    const int nr = r1 - r0;
    const int NC = v.NC;
    // x staged per token: whole chunks, each block of x in GS floats (zero past the slice)
    const int XT = NC * CB * D::GS;
    float *xl = lds;
    float *part = lds + M * XT;                    // [rows_max][NC][M]
    const int dummy = v.rows_max * NC * M;         // then 64 dummy slots
    int *tickets = reinterpret_cast<int *>(part + dummy + 64);  // then the group counter

    // ---- lane constants
    Lane ln;
    {
        ln.bl = lane / PPB;
        const int q = lane - ln.bl * PPB;
        const uint32_t bstart = v.par + 34u * (uint32_t)ln.bl;
        const bool straddle = (bstart & 2u) == 0;  // block at 0 mod 4: words straddle dwords
        const uint32_t s0 = straddle ? bstart : bstart - 2u;
        ln.voff = s0 + 4u * P * (uint32_t)q;
        ln.dvoff = s0;
        ln.bmask = straddle ? 0xFFFF0000u : 0u;
        ln.dsh = straddle ? 0u : 16u;
        ln.straddle = straddle;
        ln.xoff = D::GS * ln.bl + D::CPW * P * q;
        const bool act_last = (NC - 1) * CB + ln.bl < v.nb;
        ln.voffl = act_last ? ln.voff : 0x80000000u;
        ln.dvoffl = act_last ? ln.dvoff : 0x80000000u;
    }
    const Consts<TYPE> cst = make_consts<TYPE>();
    Consts32<TYPE> cst32;
    if constexpr (M >= 2)
        cst32 = make_consts32<TYPE>();
    const uint32_t rstride = v.row_stride;

    // ---- groups: the items (row, chunk) of the workgroup, chunk-major, in groups of at most DEPTH
    // rows of one chunk, so that x changes only between groups. Two ways to share them out:
    //  * DYN (one token, rows of one chunk, at least three groups per wave): groups of DEPTH
    //    rows; wave w takes group w first, and every further group goes to the wave that asks
    //    next (a ticket counter in LDS), one group ahead of its decode. The SIMD's arbiter favours its older waves, so a fixed split would leave
    //    the younger ones finishing alone; taking groups as they free up ends the waves of a
    //    workgroup together.
    //  * otherwise: each wave owns a contiguous run of the items, cut into one segment per chunk
    //    and each segment into groups of DEPTH (the last may hold fewer), so that its x changes at
    //    most a few times; a cursor walks it one group at a time, a group ahead of the decode.
    // Either way the result of a group does not depend on the wave that takes it.
    const int gpc = (nr + DEPTH - 1) / DEPTH;  // groups per chunk
    const int NG = NC * gpc;
    auto group_of = [&](int gi, int &c, int &r, int &cnt) {
        c = gi < NG ? gi / gpc : 0;
        r = gi < NG ? (gi - c * gpc) * DEPTH : 0;
        cnt = gi < NG ? min(DEPTH, nr - r) : 0;
    };
    if (DYN && threadIdx.x == 0)
        *tickets = 0;  // read only after the staging barrier
    struct Cur {
        int c, r;  // chunk and row (within the workgroup) of the next item
        int rem;   // items left in the current segment
        int left;  // items left in the wave's run
    };
    Cur lcur;
    {
        const int I = NC * nr;
        const int it0 = (int)((int64_t)I * w / NW), it1 = (int)((int64_t)I * (w + 1) / NW);
        lcur.left = it1 - it0;
        lcur.c = nr > 0 ? it0 / nr : 0;
        lcur.r = it0 - lcur.c * nr;
        lcur.rem = min(nr - lcur.r, lcur.left);
    }
    int tk = w;  // the next ticket (DYN)
    // the next group: chunk, first row and number of items (0 past the end)
    auto next_group = [&](int &c, int &r, int &cnt) {
        if constexpr (DYN) {
            group_of(tk, c, r, cnt);
            return;
        }
        if (lcur.rem == 0 && lcur.left > 0) {
            lcur.c++;
            lcur.r = 0;
            lcur.rem = min(nr, lcur.left);
        }
        c = lcur.c;
        r = lcur.r;
        cnt = min(DEPTH, lcur.rem);
        lcur.r += cnt;
        lcur.rem -= cnt;
        lcur.left -= cnt;
    };

    // ---- weight loads. Every slot is refilled unconditionally right after its item (a refill
    // that may or may not happen would make the compiler copy the slot, and the copy would wait
    // for the load in flight); the load of an empty item goes through a buffer of size 0, which
    // reads no memory. Lanes past the end of a row load nothing in the row's last chunk.
    auto load_item = [&](Slot<P> &sl, int c, int r, bool real) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(v.base), (short)0, real ? (int)v.nbytes : 0, 0x00020000);
        const bool lastc = c == NC - 1;
        load_slot<P>(rs, lastc ? ln.voffl : ln.voff, lastc ? ln.dvoffl : ln.dvoff,
                     (uint32_t)(r0 + r) * rstride + CBYTES * (uint32_t)c, sl);
    };
    int lgc = 0, lgr = 0, lgn = 0;  // the group being loaded
    // ---- x staging: the first pass of x loads goes out before the weight loads, so that waiting
    // for it waits for no weights; further passes (large M * K) wait for everything in flight
    constexpr int G4 = D::G / 4;       // 16-byte pieces of x per block
    constexpr int XPT = 8;             // pieces per thread and pass
    const int nvalid = v.nb * G4;      // pieces per token inside the slice
    const int ntot = NC * CB * G4;     // pieces per token, whole chunks
    const int npieces = M * ntot;
    auto stage_load = [&](int pass, float4 (&v)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int f = (pass * XPT + i) * 64 * NW + (int)threadIdx.x;
            const int m = f / ntot, e = f - m * ntot;
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (f < npieces && e < nvalid) {
                const f32x4a4 t = *reinterpret_cast<const f32x4a4 *>(a.x + (int64_t)m * a.xstride + 4 * e);
                v[i] = make_float4(t.x, t.y, t.z, t.w);
            }
        }
    };
    auto stage_store = [&](int pass, const float4 (&v)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int f = (pass * XPT + i) * 64 * NW + (int)threadIdx.x;
            const int m = f / ntot, e = f - m * ntot;
            const int b = e / G4, c4 = e - b * G4;
            if (f < npieces)
                *reinterpret_cast<float4 *>(xl + m * XT + b * D::GS + 4 * c4) = v[i];
        }
    };
    const int npass = (npieces + XPT * 64 * NW - 1) / (XPT * 64 * NW);
    float4 xv0[XPT];
    stage_load(0, xv0);

    // The first PRE items' weights go out before x is staged, the rest after: at 1-2 tokens the
    // x of a workgroup would otherwise queue behind every wave's first group of weights in the
    // memory system, and the barrier waits for the slowest wave's x.
    Slot<P> ring[DEPTH];
    next_group(lgc, lgr, lgn);
#pragma unroll
    for (int s = 0; s < PRE; s++)
        load_item(ring[s], lgc, lgr + s, s < lgn);

    stage_store(0, xv0);
    for (int pass = 1; pass < npass; pass++) {
        float4 v[XPT];
        stage_load(pass, v);
        stage_store(pass, v);
    }
    // a plain barrier: __syncthreads() would also wait for the weight loads in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int s = PRE; s < DEPTH; s++)
        load_item(ring[s], lgc, lgr + s, s < lgn);

    // ---- items: x of the current chunk in registers, DEPTH items in flight. The partials of a
    // group are summed over the wave together (one transposed reduction), and the first lane of
    // each DPP row stores its share of them.
    static_assert(DEPTH % 4 == 0, "groups of 4k items");
    constexpr int V = DEPTH * M;
    float xs[M][P][2][D::PAIRS];
    int xc = -1;             // chunk whose x is in xs
    uint32_t dwid = 16;      // d field width: 0 for lanes past the end of the row
    const int q = lane >> 4;
    for (;;) {
        const int gc = lgc, gr = lgr, gn = lgn;  // this group (already loaded)
        if (gn == 0)
            break;
        // the next group, loaded as this one is decoded. A ticket: all 64 lanes add one (one
        // wave's adds are one LDS instruction), so the counter moves by 64 per ticket and the
        // first lane's old value over 64 is the ticket; no branch around the atomic
        if constexpr (DYN) {
            const int t = __hip_atomic_fetch_add(tickets, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP);
            tk = NW + (__builtin_amdgcn_readfirstlane(t) >> 6);
        }
        next_group(lgc, lgr, lgn);
        if (gc != xc) {
            xc = gc;
            dwid = xc * CB + ln.bl < v.nb ? 16u : 0u;
#pragma unroll
            for (int m = 0; m < M; m++)
                read_x<TYPE, P>(xl + m * XT + xc * CB * D::GS + ln.xoff, ln.straddle, xs[m]);
        }
        float pv[V];
#pragma unroll
        for (int s = 0; s < DEPTH; s++) {
#pragma unroll
            for (int m = 0; m < M; m++)
                pv[s * M + m] = 0.0f;
            if (s < gn) {  // uniform
                float o[M];
                item_mac<TYPE, M, P>(ring[s], ln, dwid, xs, cst, cst32, o);
#pragma unroll
                for (int m = 0; m < M; m++)
                    pv[s * M + m] = o[m];
            }
            __builtin_amdgcn_sched_barrier(0);
            load_item(ring[s], lgc, lgr + s, s < lgn);
            __builtin_amdgcn_sched_barrier(0);
        }
        // tot[i] in DPP row q = the wave total of value i + q * V/4: item i/M + q * DEPTH/4,
        // token i % M. Every lane stores (the row's first lane to the partial, the others to
        // their dummy slots): a divergent branch would make the compiler wait for the loads.
        float tot[V / 4];
        transpose_reduce<V>(pv, tot);
#pragma unroll
        for (int i = 0; i < V / 4; i++) {
            const int si = i / M + q * (DEPTH / 4);
            const bool real = si < gn && (lane & 15) == 0;
            part[real ? ((gr + si) * NC + gc) * M + i % M : dummy + lane] = tot[i];
        }
    }

    __syncthreads();
    for (int i = threadIdx.x; i < nr * M; i += 64 * NW) {
        const int k = i / M, m = i - k * M;
        float acc = 0.0f;
        for (int c = 0; c < NC; c++)
            acc += part[(k * NC + c) * M + m];
        float *yp = v.y + (int64_t)m * v.ystride + (int64_t)(r0 + k) * a.yinc;
        *yp = a.accumulate ? *yp + acc : acc;
    }
}

template <int TYPE, int M, int P, int DEPTH, int NW, int PRE, bool DYN>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
pn_gemv_rows_kernel(const Args a)
{
    const View v = make_view(a, TYPE, false);
    rows_body<TYPE, M, P, DEPTH, NW, PRE, DYN>(a, v);
}

// Matrices of both types in one launch: each workgroup runs its part's decode, with that type's
// own piece size, ring depth and early-weight count (those a launch of the type alone takes, so
// that every row gets the same bits), under one launch shape.
template <int M, int P3, int DEPTH3, int PRE3, int P4, int DEPTH4, int PRE4, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
pn_gemv_rows_mixed_kernel(const Args a)
{
    const View v = make_view(a, PN_TYPE_PN3T, true);
    if (v.type == PN_TYPE_PN3T)
        rows_body<PN_TYPE_PN3T, M, P3, DEPTH3, NW, PRE3, false>(a, v);
    else
        rows_body<PN_TYPE_PN4T, M, P4, DEPTH4, NW, PRE4, false>(a, v);
}

}  // namespace rows

// ---- host -----------------------------------------------------------------------------------------

namespace {

// Launch shape per piece size: items in flight per wave (DEPTH) and waves per workgroup (NW, one
// workgroup per CU; the register budget is 512 / (NW / 4) per lane).
template <int TYPE, int M, int P> struct Cfg {
    static constexpr int DEPTH = P == 2 && M <= 2 ? 8 : 4;
    // pn3t 8-word pieces hold 80 x per lane, and 2-4 tokens hold M x per code plus the fp32
    // decode's masks: two waves per SIMD keep them without spills
    static constexpr int NW = (TYPE == PN_TYPE_PN3T && P == 8) || M >= 2 ? 8 : 12;
    // items whose weights are requested before x is staged
    static constexpr int PRE = M <= 2 ? 1 : DEPTH;
};

template <int TYPE, int M, int P>
int launch_one(const rows::Args &a, int grid, size_t lds, hipStream_t s)
{
    using C = Cfg<TYPE, M, P>;
    // A counter hands out the groups at one token where rows are one chunk and every wave can
    // expect at least three groups; otherwise each wave keeps its own run of items (with several
    // chunks, so that it re-reads x only a few times; with few groups, so that no wave stands
    // idle).
    if constexpr (M == 1) {
        if (a.NC == 1 && (a.rows_max + C::DEPTH - 1) / C::DEPTH >= 3 * C::NW) {
            constexpr auto kd = rows::pn_gemv_rows_kernel<TYPE, M, P, C::DEPTH, C::NW, C::PRE, true>;
            if (!lds_limit_once<kd>(rows::kLdsMax))
                return PN_ERR_HIP;
            hipLaunchKernelGGL(kd, dim3((unsigned)grid), dim3(64 * C::NW), lds, s, a);
            return launch_status();
        }
    }
    constexpr auto kern = rows::pn_gemv_rows_kernel<TYPE, M, P, C::DEPTH, C::NW, C::PRE, false>;
    if (!lds_limit_once<kern>(rows::kLdsMax))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * C::NW), lds, s, a);
    return launch_status();
}

template <int TYPE, int M>
int launch_p(int P, const rows::Args &a, int grid, size_t lds, hipStream_t s)
{
    if constexpr (M == 1) {
        if (P == 8)
            return launch_one<TYPE, M, 8>(a, grid, lds, s);
    }
    if constexpr (M <= 3) {
        if (P == 4)
            return launch_one<TYPE, M, 4>(a, grid, lds, s);
    }
    return launch_one<TYPE, M, 2>(a, grid, lds, s);
}

// Piece size for a row of nb blocks at M tokens: among the sizes whose x fits the registers without
// spills (8 words at one token, 4 up to three tokens: 120 x floats and 218 VGPRs for pn3t at
// three; 2 always), the fewest VALU operations per weight, counting the lanes of a partial last
// chunk as spent. Each item also pays a fixed cost whatever its piece size: the reduction of
// its partial across the wave, the partial's LDS write and the item's scheduling. Its weight,
// kItemOps, is fitted to launches timed at every piece size (rows of 40-272 blocks, 1024-17408
// rows, 1-2 tokens): at 18 the model kept 2-word pieces where 4 or 8 words ran 0.3-2 us faster.
constexpr double kItemOps = 70.0;

template <int TYPE, int M>
int choose_p(int64_t nb)
{
    using D = rows::Dec<TYPE>;
    int best = 2;
    double best_cost = 1e30;
    for (int P : {8, 4, 2}) {
        if ((M > 1 && P == 8) || (M > 3 && P == 4))
            continue;
        const int64_t cb = 8 * P, nc = (nb + cb - 1) / cb;
        const double eff = (double)nb / (double)(nc * cb);
        const double ops = P * (1 + D::PAIRS * (2 + 2 * M)) + kItemOps;  // per item and lane
        const double cost = ops / (eff * D::CPW * P);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = P;
        }
    }
    return best;
}

// The piece size a launch takes for a matrix of N rows of nb blocks: the model's, or
// PN_GEMV_PIECE=8|4|2 where the registers allow it (tests reach every variant with it; the results
// stay within the same bound). At three tokens 4-word pieces are kept only where the ceil(N / CUs)
// rows of a workgroup give its 8 waves at least 8 groups of 4 items: on fewer rows (k and v,
// 1024x5120: 3 groups) the waves sit idle and 2-word pieces run 5.8 against 7.9 us. It depends on
// the matrix alone, never on how a group deals its workgroups, so a group keeps the bits of
// separate calls; every launcher takes the piece size from here.
template <int TYPE, int M>
int piece_for(int64_t nb, int64_t N)
{
    int P = choose_p<TYPE, M>(nb);
    if (M == 3 && P == 4) {
        const int64_t rows_wg = (N + device_cus() - 1) / device_cus();
        if ((rows_wg + 3) / 4 * ((nb + 31) / 32) < 8)
            P = 2;
    }
    if (const char *e = getenv("PN_GEMV_PIECE")) {
        const int f = atoi(e);
        if ((f == 8 && M == 1) || (f == 4 && M <= 3) || f == 2)
            P = f;
    }
    return P;
}

// rows [0, N) of one parity class (row_stride a multiple of 4), blocks [b0, b0 + nb) of each
template <int TYPE, int M>
int launch_rows(const uint8_t *row0, int64_t N, int64_t row_stride, int64_t nb, int64_t b0,
                const float *x, int64_t K, float *y, int64_t ystride, int64_t yinc,
                bool accumulate, int P, hipStream_t s)
{
    using D = rows::Dec<TYPE>;
    const int64_t cb = 8 * P, NC = (nb + cb - 1) / cb;
    const size_t x_bytes = (size_t)M * NC * cb * D::GS * sizeof(float);
    const int cus = device_cus();
    // partials of a workgroup beside the staged x
    const int64_t part_cap = ((int64_t)rows::kLdsMax - (int64_t)x_bytes) / (int64_t)sizeof(float) - 65;
    const int64_t rows_cap = part_cap / (NC * M);
    if (rows_cap < 1)
        return PN_ERR_SHAPE;
    const int64_t slice_bytes = nb * kBlockBytes;
    int64_t done = 0;
    while (done < N) {
        // byte offsets of a launch fit 32 bits
        int64_t n = std::min<int64_t>(N - done, rows_cap * cus);
        n = std::min<int64_t>(n, ((int64_t)0x7FFF0000 - slice_bytes) / row_stride + 1);
        const int grid = (int)std::min<int64_t>(cus, n);
        const uint8_t *first = row0 + done * row_stride + b0 * kBlockBytes;
        const uintptr_t fa = reinterpret_cast<uintptr_t>(first);
        rows::Args a;
        a.par = (uint32_t)(fa & 3u);
        a.base = first - a.par;
        const int64_t end = (int64_t)a.par + (n - 1) * row_stride + slice_bytes;
        a.nbytes = (uint32_t)((end + 3) & ~(int64_t)3);
        a.row_stride = (uint32_t)row_stride;
        a.N = (int)n;
        a.nb = (int)nb;
        a.NC = (int)NC;
        a.rows_max = (int)((n + grid - 1) / grid);
        a.x = x + b0 * D::G;
        a.xstride = K;
        a.y = y + done * yinc;
        a.ystride = ystride;
        a.yinc = yinc;
        a.accumulate = accumulate ? 1 : 0;
        a.nparts = 0;
        const size_t lds = std::max<size_t>(
            rows::kLdsFloor, x_bytes + ((size_t)a.rows_max * NC * M + 65) * sizeof(float));
        const int st = launch_p<TYPE, M>(P, a, grid, lds, s);
        if (st != PN_OK)
            return st;
        done += n;
    }
    return PN_OK;
}

template <int TYPE, int M>
int launch_typed(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    using D = rows::Dec<TYPE>;
    const int64_t nb = K / D::G;
    const int64_t rb = nb * kBlockBytes;
    const int P = piece_for<TYPE, M>(nb, N);
    const int64_t cb = 8 * P;
    // K slices of whole chunks, each slice after the first adding to y: as few as fit the LDS
    // beside the partials of ceil(N / CUs) rows per workgroup (never fewer chunks per slice than
    // kXLdsMax of x holds; taller matrices then split their rows over launches), and of balanced
    // length, so that no launch is a short tail
    const int64_t nc_all = (nb + cb - 1) / cb;
    const int64_t cbytes = (int64_t)M * cb * D::GS * (int64_t)sizeof(float);
    const int64_t rows_wg = (N + device_cus() - 1) / device_cus();
    const int64_t fit_rows = ((int64_t)rows::kLdsMax - 65 * (int64_t)sizeof(float)) /
                             (cbytes + rows_wg * M * (int64_t)sizeof(float));
    const int64_t fit = std::max<int64_t>(1, std::max<int64_t>(fit_rows, rows::kXLdsMax / cbytes));
    const int64_t nslices = (nc_all + fit - 1) / fit;
    const int64_t slice_nb = (nc_all + nslices - 1) / nslices * cb;
    // rows of an odd block count alternate between two alignments: each class is its own launch
    const bool two = (rb & 2) != 0;
    for (int64_t b0 = 0; b0 < nb; b0 += slice_nb) {
        const int64_t n = std::min(slice_nb, nb - b0);
        for (int cls = 0; cls < (two ? 2 : 1); cls++) {
            const int64_t Nc = two ? (N - cls + 1) / 2 : N;
            if (Nc == 0)
                continue;
            const int st = launch_rows<TYPE, M>(W + cls * rb, Nc, two ? 2 * rb : rb, n, b0, x, K,
                                                y + cls, N, two ? 2 : 1, b0 > 0, P, s);
            if (st != PN_OK)
                return st;
        }
    }
    return PN_OK;
}

template <int TYPE>
int launch_m(const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M, float *y,
             hipStream_t s)
{
    switch (M) {
    case 1: return launch_typed<TYPE, 1>(W, N, K, x, y, s);
    case 2: return launch_typed<TYPE, 2>(W, N, K, x, y, s);
    case 3: return launch_typed<TYPE, 3>(W, N, K, x, y, s);
    default: return launch_typed<TYPE, 4>(W, N, K, x, y, s);
    }
}

// Several matrices of one type and K that read the same x, as one launch: the workgroups are dealt
// to the parts in proportion to their rows (at least one each), each part's rows split over its
// own workgroups as in a launch of its own. Only where every part is one launch of one alignment
// class (whole rows of x fit the LDS, row bytes a multiple of 4, 31-bit offsets) and the rows of a
// workgroup fit its partials; otherwise returns 1 and the caller launches the parts one by one.
template <int TYPE, int M>
int launch_group_typed(const GroupPart *gp, int count, int64_t K, const float *x, hipStream_t s)
{
    using D = rows::Dec<TYPE>;
    const int64_t nb = K / D::G;
    const int64_t rb = nb * kBlockBytes;
    if (count < 2 || count > rows::kMaxParts || (rb & 2))
        return 1;
    // one piece size for all parts: the one each would take alone, else separate launches
    const int P = piece_for<TYPE, M>(nb, gp[0].N);
    for (int i = 1; i < count; i++)
        if (piece_for<TYPE, M>(nb, gp[i].N) != P)
            return 1;
    const int64_t cb = 8 * P, NC = (nb + cb - 1) / cb;
    const size_t x_bytes = (size_t)M * NC * cb * D::GS * sizeof(float);
    if (x_bytes > (size_t)rows::kXLdsMax)
        return 1;
    int64_t total = 0;
    for (int i = 0; i < count; i++) {
        if (gp[i].N <= 0 || gp[i].N * rb > (int64_t)0x7FFF0000)
            return 1;
        total += gp[i].N;
    }
    const int cus = device_cus();
    const int grid = (int)std::min<int64_t>(cus, total);
    if (grid < count)
        return 1;
    // workgroups per part: proportional to rows, at least one, at most the part's rows
    int gcount[rows::kMaxParts];
    int used = 0;
    for (int i = 0; i < count; i++) {
        gcount[i] = (int)std::max<int64_t>(1, std::min<int64_t>(gp[i].N, gp[i].N * grid / total));
        used += gcount[i];
    }
    for (int i = 0; used < grid; i = (i + 1) % count)
        if (gcount[i] < gp[i].N) {
            gcount[i]++;
            used++;
        }
    for (int i = 0; used > grid; i = (i + 1) % count)
        if (gcount[i] > 1) {
            gcount[i]--;
            used--;
        }
    const int64_t part_cap = ((int64_t)rows::kLdsMax - (int64_t)x_bytes) / (int64_t)sizeof(float) - 65;
    rows::Args a{};
    int64_t rows_max = 0;
    int g0 = 0;
    for (int i = 0; i < count; i++) {
        const uintptr_t fa = reinterpret_cast<uintptr_t>(gp[i].W);
        rows::Part &pt = a.parts[i];
        pt.par = (uint32_t)(fa & 3u);
        pt.base = gp[i].W - pt.par;
        pt.nbytes = (uint32_t)(((int64_t)pt.par + gp[i].N * rb + 3) & ~(int64_t)3);
        pt.N = (int)gp[i].N;
        pt.g0 = g0;
        pt.y = gp[i].y;
        pt.ystride = gp[i].N;
        g0 += gcount[i];
        rows_max = std::max<int64_t>(rows_max, (gp[i].N + gcount[i] - 1) / gcount[i]);
    }
    if (rows_max * NC * M > part_cap)
        return 1;
    a.nparts = count;
    a.base = a.parts[0].base;
    a.nbytes = a.parts[0].nbytes;
    a.par = a.parts[0].par;
    a.N = a.parts[0].N;
    a.y = a.parts[0].y;
    a.ystride = a.parts[0].ystride;
    a.row_stride = (uint32_t)rb;
    a.nb = (int)nb;
    a.NC = (int)NC;
    a.rows_max = (int)rows_max;
    a.x = x;
    a.xstride = K;
    a.yinc = 1;
    a.accumulate = 0;
    const size_t lds = std::max<size_t>(
        rows::kLdsFloor, x_bytes + ((size_t)rows_max * NC * M + 65) * sizeof(float));
    return launch_p<TYPE, M>(P, a, grid, lds, s);
}

template <int TYPE>
int launch_group_m(const GroupPart *gp, int count, int64_t K, const float *x, int64_t M,
                   hipStream_t s)
{
    switch (M) {
    case 1: return launch_group_typed<TYPE, 1>(gp, count, K, x, s);
    case 2: return launch_group_typed<TYPE, 2>(gp, count, K, x, s);
    case 3: return launch_group_typed<TYPE, 3>(gp, count, K, x, s);
    default: return launch_group_typed<TYPE, 4>(gp, count, K, x, s);
    }
}

template <int M, int P3, int P4>
int launch_mixed_one(const rows::Args &a, int grid, size_t lds, hipStream_t s)
{
    using C3 = Cfg<PN_TYPE_PN3T, M, P3>;
    using C4 = Cfg<PN_TYPE_PN4T, M, P4>;
    constexpr auto kern = rows::pn_gemv_rows_mixed_kernel<M, P3, C3::DEPTH, C3::PRE, P4, C4::DEPTH,
                                                          C4::PRE, 8>;
    if (!lds_limit_once<kern>(rows::kLdsMax))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * 8), lds, s, a);
    return launch_status();
}

// piece sizes a launch can take: 8, 4 and 2 at one token, 4 and 2 at two and three, 2 at four
template <int M, int P3>
int launch_mixed_p4(const rows::Args &a, int grid, size_t lds, int P4, hipStream_t s)
{
    if constexpr (M == 1) {
        if (P4 == 8)
            return launch_mixed_one<M, P3, 8>(a, grid, lds, s);
    }
    if constexpr (M <= 3) {
        if (P4 == 4)
            return launch_mixed_one<M, P3, 4>(a, grid, lds, s);
    }
    return launch_mixed_one<M, P3, 2>(a, grid, lds, s);
}

template <int M>
int launch_mixed_p3(const rows::Args &a, int grid, size_t lds, int P3, int P4, hipStream_t s)
{
    if constexpr (M == 1) {
        if (P3 == 8)
            return launch_mixed_p4<M, 8>(a, grid, lds, P4, s);
    }
    if constexpr (M <= 3) {
        if (P3 == 4)
            return launch_mixed_p4<M, 4>(a, grid, lds, P4, s);
    }
    return launch_mixed_p4<M, 2>(a, grid, lds, P4, s);
}

// Matrices of both types (and one K) as one launch: each type with the piece size a launch of its
// own would take, 8 waves per CU, each part with its own row shape, x layout and share of the
// workgroups. The shares follow the cost model of choose_p (rows x chunks x operations per item),
// not the bytes: a pn4t row of 80 blocks is two items, the second a quarter full, against one
// for a pn3t row of 64. Returns 1 where the shapes do not allow it (as launch_group_typed).
template <int M>
int launch_group_mixed(const GroupPart *gp, int count, int64_t K, const float *x, hipStream_t s)
{
    using D3 = rows::Dec<PN_TYPE_PN3T>;
    using D4 = rows::Dec<PN_TYPE_PN4T>;
    if (count < 2 || count > rows::kMaxParts || K % D3::G || K % D4::G)
        return 1;
    const int64_t nb3 = K / D3::G, nb4 = K / D4::G;
    if (((nb3 * kBlockBytes) & 2) || ((nb4 * kBlockBytes) & 2))
        return 1;
    // one piece size per type: the one each part would take alone, else no mixed launch
    int P3 = 0, P4 = 0;
    for (int i = 0; i < count; i++) {
        const bool p3 = gp[i].type == PN_TYPE_PN3T;
        const int Pi = p3 ? piece_for<PN_TYPE_PN3T, M>(nb3, gp[i].N)
                          : piece_for<PN_TYPE_PN4T, M>(nb4, gp[i].N);
        int &Pt = p3 ? P3 : P4;
        if (Pt && Pt != Pi)
            return 1;
        Pt = Pi;
    }
    if (!P3)
        P3 = 2;
    if (!P4)
        P4 = 2;
    // per-item operations of each type (the cost model of choose_p)
    const int64_t ops3 = (int64_t)(P3 * (1 + D3::PAIRS * (2 + 2 * M)) + kItemOps);
    const int64_t ops4 = (int64_t)(P4 * (1 + D4::PAIRS * (2 + 2 * M)) + kItemOps);
    const int64_t nc3 = (nb3 + 8 * P3 - 1) / (8 * P3), nc4 = (nb4 + 8 * P4 - 1) / (8 * P4);
    int64_t cost[rows::kMaxParts], total_cost = 0, total_rows = 0;
    for (int i = 0; i < count; i++) {
        const bool p3 = gp[i].type == PN_TYPE_PN3T;
        const int64_t rb = (p3 ? nb3 : nb4) * kBlockBytes;
        if (gp[i].N <= 0 || gp[i].N * rb > (int64_t)0x7FFF0000)
            return 1;
        cost[i] = gp[i].N * (p3 ? nc3 * ops3 : nc4 * ops4);
        total_cost += cost[i];
        total_rows += gp[i].N;
    }
    const int grid = (int)std::min<int64_t>(device_cus(), total_rows);
    if (grid < count)
        return 1;
    int gcount[rows::kMaxParts];
    int used = 0;
    for (int i = 0; i < count; i++) {
        gcount[i] = (int)std::max<int64_t>(1, std::min<int64_t>(gp[i].N, cost[i] * grid / total_cost));
        used += gcount[i];
    }
    for (int i = 0; used < grid; i = (i + 1) % count)
        if (gcount[i] < gp[i].N) {
            gcount[i]++;
            used++;
        }
    for (int i = 0; used > grid; i = (i + 1) % count)
        if (gcount[i] > 1) {
            gcount[i]--;
            used--;
        }
    rows::Args a{};
    size_t lds = rows::kLdsFloor;
    int g0 = 0;
    for (int i = 0; i < count; i++) {
        const bool p3 = gp[i].type == PN_TYPE_PN3T;
        const int64_t nb = p3 ? nb3 : nb4, rb = nb * kBlockBytes, cb = 8 * (p3 ? P3 : P4);
        const int64_t NC = (nb + cb - 1) / cb;
        const size_t x_bytes = (size_t)M * NC * cb * (p3 ? D3::GS : D4::GS) * sizeof(float);
        if (x_bytes > (size_t)rows::kXLdsMax)
            return 1;
        const int64_t rows_max = (gp[i].N + gcount[i] - 1) / gcount[i];
        const int64_t part_cap =
            ((int64_t)rows::kLdsMax - (int64_t)x_bytes) / (int64_t)sizeof(float) - 65;
        if (rows_max * NC * M > part_cap)
            return 1;
        lds = std::max(lds, x_bytes + ((size_t)rows_max * NC * M + 65) * sizeof(float));
        const uintptr_t fa = reinterpret_cast<uintptr_t>(gp[i].W);
        rows::Part &pt = a.parts[i];
        pt.par = (uint32_t)(fa & 3u);
        pt.base = gp[i].W - pt.par;
        pt.nbytes = (uint32_t)(((int64_t)pt.par + gp[i].N * rb + 3) & ~(int64_t)3);
        pt.N = (int)gp[i].N;
        pt.g0 = g0;
        pt.y = gp[i].y;
        pt.ystride = gp[i].N;
        pt.type = gp[i].type;
        pt.row_stride = (uint32_t)rb;
        pt.nb = (int)nb;
        pt.NC = (int)NC;
        pt.rows_max = (int)rows_max;
        g0 += gcount[i];
    }
    a.nparts = count;
    a.x = x;
    a.xstride = K;
    a.yinc = 1;
    a.accumulate = 0;
    return launch_mixed_p3<M>(a, grid, lds, P3, P4, s);
}

int launch_group_mixed_m(const GroupPart *gp, int count, int64_t K, const float *x, int64_t M,
                         hipStream_t s)
{
    switch (M) {
    case 1: return launch_group_mixed<1>(gp, count, K, x, s);
    case 2: return launch_group_mixed<2>(gp, count, K, x, s);
    case 3: return launch_group_mixed<3>(gp, count, K, x, s);
    default: return launch_group_mixed<4>(gp, count, K, x, s);
    }
}

}  // namespace

// Several PN GEMVs of one type (type < 0: parts of both types, each part's own type in gp) and K
// over the same x at 1 <= M <= 4 as one launch (arguments already checked): PN_OK, an error, or 1
// where the parts must run as launches of their own.
int launch_vec_group(int type, const GroupPart *gp, int count, int64_t K, const float *x,
                     int64_t M, hipStream_t s)
{
    if (type < 0)  // both types
        return launch_group_mixed_m(gp, count, K, x, M, s);
    return type == PN_TYPE_PN3T ? launch_group_m<PN_TYPE_PN3T>(gp, count, K, x, M, s)
                                : launch_group_m<PN_TYPE_PN4T>(gp, count, K, x, M, s);
}

// The vector-unit PN GEMV for 1 <= M <= 4 (arguments already checked by the entry point).
int launch_vec(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
               float *y, hipStream_t s)
{
    return type == PN_TYPE_PN3T ? launch_m<PN_TYPE_PN3T>(W, N, K, x, M, y, s)
                                : launch_m<PN_TYPE_PN4T>(W, N, K, x, M, y, s);
}

}  // namespace pn
