// pn_gemv_vec.hip -- PN decode-step GEMV y = W.x at 1-4 tokens on the vector units of gfx950.
//
// Format: "PN weight format" (PNX-FORMAT-v0): "Block layout" (34-byte blocks: fp16 d, then eight
// little-endian u32 words; code t of a word at bit BITS*(t>>1) + 16*(t&1); no code crosses a 16-bit
// half), "Value" (w = d * (n - z), exact in fp32).
//
// Arithmetic (exact decode, fp32 x as given):
//  * Codes t = 2j and 2j + 1 of a word sit at the same bit p = BITS*j of its two 16-bit halves. One
//    and-or keeps both and sets the fp16 exponent of 2^(10-p) in each half: the pair becomes the
//    fp16 numbers (2^(10-p) + n_lo, 2^(10-p) + n_hi), exactly. One packed fp16 add of
//    -(2^(10-p) + z) then gives the integers n - z in both halves, exactly (code z gives +0): no
//    zero-point fold, no cancellation. Positions past the fp16 mantissa take a shift of the word
//    first (by 9 for pn3t, 8 for pn4t).
//  * Each weight is one v_fma_mix_f32: its fp16 n - z widens exactly and the product with the fp32
//    x is exact inside the fma, so the only roundings are fp32 sums: four chains per lane and item
//    (dword parity x half), one multiply by the block's d, a 64-lane tree and the in-order sum of a
//    row's chunks. Per pair of weights: 1 and-or + 1 packed add + 2 fma.
//  * Any 16-bit halves whose codes share bit positions pair up, so an item may read its words as
//    they sit in memory: 4-byte aligned words directly, words at 2 mod 4 as the aligned dwords
//    around them (each holding the high half of one word and the low half of the next), with one
//    v_bfi to close the piece. x follows the pairing in registers.
//
// Work split (one workgroup of up to 16 waves per CU, 4 per SIMD):
//  * A lane owns a "piece" of P consecutive words of one block; a wave covers a chunk of 64
//    pieces (8P blocks) of K and keeps that chunk's x in registers for every row it processes.
//  * CU g owns rows g, g + G, g + 2G, ...; within it, wave w takes chunk w % NC of every
//    (W/NC)-th row, or, with 17 chunks, chunk w of every row plus a share of the 17th chunk.
//  * The streaming kernel (rows of a multiple of 8 blocks from a 4-byte aligned W) copies each item
//    -- one row's chunk, 272P contiguous bytes -- into its own LDS ring slot with 16-byte loads
//    straight to LDS (every load instruction reads one contiguous span), then every lane reads its
//    piece from LDS. The lane kernel (any alignment, and the last blocks of a row past a multiple
//    of 8) reads its piece from global memory directly: P dwords, a 16-bit half-word and d.
//  * Per item, the 64 lane partials are summed by a transposed permlane/DPP reduction over a batch
//    of items; the wave writes one partial per (row, chunk, token) to LDS; after a barrier the
//    workgroup adds each row's chunk partials in chunk order and writes y. No atomics: the same
//    inputs and launch shape give the same bits, and both kernels give the same bits on the
//    shapes they share.
#include <stdlib.h>

#include <algorithm>

#include "pn_common.h"

namespace pn {
namespace vec {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
// Dynamic LDS every launch requests at least: more than half of the CU's 160 KB, so that no CU
// ever holds two of these persistent workgroups while another holds none.
constexpr int kLdsFloor = 82 * 1024;
constexpr int kLdsMax = 160 * 1024;
// Two workgroups per CU (8 waves per SIMD, at most 64 registers): each takes more than a third of
// the LDS and at most half.
constexpr int kLdsFloor2 = 54 * 1024;
constexpr int kLdsMax2 = 80 * 1024;

template <int TYPE> struct Dec;
template <> struct Dec<PN_TYPE_PN3T> {
    // NPOS code positions per 16-bit half are decoded in place (BITS * u, u < NPOS); the rest
    // after a shift of the dword by SHIFT bits
    static constexpr int BITS = 3, CPW = 10, PAIRS = 5, Z = 4, G = 80, NPOS = 3, SHIFT = 9;
};
template <> struct Dec<PN_TYPE_PN4T> {
    static constexpr int BITS = 4, CPW = 8, PAIRS = 4, Z = 8, G = 64, NPOS = 2, SHIFT = 8;
};

typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Registers of one item in flight: P 4-byte aligned dwords, the 16-bit half-word that completes
// the piece when its words are not 4-byte aligned, and the block's d.
template <int P> struct Slot {
    uint32_t dw[P];
    uint16_t ext;  // kept 16-bit (never widened: only its low half is merged in)
    uint16_t d;    // kept 16-bit: only its fp16 value is used
};

// One lane's loads within its chunk. A chunk spans 8P blocks (272P bytes, a multiple of 4), so
// every chunk of a row has the same offsets and alignment; the chunk and the row enter through the
// (uniform) row pointer.
//  * Words 4-byte aligned (block start 2 mod 4): the P words are read as they are; dword i holds
//    word Pq + i: even codes in its low half, odd codes in its high half.
//  * Words 2 mod 4 (block start 0 mod 4): the P aligned dwords from the piece's first word back by
//    two bytes are read; dword i holds the high half of word Pq + i - 1 (low half) and the low half
//    of word Pq + i (high half). Dword 0's low half is then replaced by the high half of the piece's
//    last word (the 16-bit ext read just past the dwords), so dword 0 pairs word Pq + P - 1's odd
//    codes with word Pq's even codes. No byte is read twice and none is skipped.
// In both cases every dword holds two 16-bit halves whose codes sit at the same in-half bit
// positions, which is what the paired decode needs; the lane's x registers follow the pairing.
struct LaneMap {
    uint32_t main;  // P dwords, 4-byte aligned
    uint32_t ext;   // the 16-bit half-word (the block's d when unused: in bounds)
    uint32_t d;     // the block's d
    uint32_t keep;  // bits of dword 0 kept when ext is merged in (all of them when aligned)
    bool aligned;
    int elem;       // first element of K this lane's piece covers, in chunk 0
};

// par2: bit 1 of the address of the first block of the chunk's row segment.
template <int TYPE, int P>
__device__ __forceinline__ LaneMap lane_map(int lane, uint32_t par2)
{
    using D = Dec<TYPE>;
    constexpr int PPB = 8 / P;
    const int b = lane / PPB, q = lane - b * PPB;
    const uint32_t s = 34u * (uint32_t)b;
    const bool aligned = ((par2 + s) & 2u) != 0;
    LaneMap m;
    m.main = s + 4u * P * q + (aligned ? 2u : 0u);
    m.ext = aligned ? s : s + 4u * P * q + 4u * P;
    m.d = s;
    m.keep = aligned ? 0xFFFFFFFFu : 0xFFFF0000u;
    m.aligned = aligned;
    m.elem = D::G * b + D::CPW * P * q;
    return m;
}

// One item's loads through the buffer resource of the launch's weights: soff = byte offset of the
// (row, chunk) segment, the lane offsets from its LaneMap.
template <int P>
__device__ __forceinline__ void load_slot(__amdgpu_buffer_rsrc_t rs, uint32_t soff,
                                          const LaneMap &lm, Slot<P> &sl)
{
    if constexpr (P == 1) {
        sl.dw[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, lm.main, soff, 0);
    } else if constexpr (P == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, lm.main, soff, 0);
        sl.dw[0] = v[0];
        sl.dw[1] = v[1];
    } else {
        static_assert(P == 4, "pieces of 1, 2 or 4 words");
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lm.main, soff, 0);
        sl.dw[0] = v[0];
        sl.dw[1] = v[1];
        sl.dw[2] = v[2];
        sl.dw[3] = v[3];
    }
    sl.ext = __builtin_amdgcn_raw_buffer_load_b16(rs, lm.ext, soff, 0);
    sl.d = __builtin_amdgcn_raw_buffer_load_b16(rs, lm.d, soff, 0);
}

// N consecutive floats from a 4-byte aligned address.
template <int N>
__device__ __forceinline__ void load_x(const float *__restrict__ x, float (&xs)[N])
{
    static_assert(N % 2 == 0, "");
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f32x4a4 v = *reinterpret_cast<const f32x4a4 *>(x + i);
            xs[i] = v.x;
            xs[i + 1] = v.y;
            xs[i + 2] = v.z;
            xs[i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const f32x2a4 v = *reinterpret_cast<const f32x2a4 *>(x + i);
            xs[i] = v.x;
            xs[i + 1] = v.y;
        }
    }
}

// x of one lane's piece, in pairing order: xs[i][h][r] multiplies the code at pair position r of
// the half h of dword i. xv[e] = x[elem + e] (CPW * P contiguous values).
template <int TYPE, int P>
__device__ __forceinline__ void pair_x(const float (&xv)[Dec<TYPE>::CPW * P], bool aligned,
                                       float (&xs)[P][2][Dec<TYPE>::PAIRS])
{
    using D = Dec<TYPE>;
#pragma unroll
    for (int i = 0; i < P; i++)
#pragma unroll
        for (int r = 0; r < D::PAIRS; r++) {
            // aligned: word Pq + i, code 2r (low half) and 2r + 1 (high half)
            // unaligned: high half = word Pq + i, code 2r; low half = word Pq + i - 1 (cyclic
            // within the piece), code 2r + 1
            const float lo_a = xv[D::CPW * i + 2 * r], hi_a = xv[D::CPW * i + 2 * r + 1];
            const float lo_u = xv[D::CPW * ((i + P - 1) % P) + 2 * r + 1];
            xs[i][0][r] = aligned ? lo_a : lo_u;
            xs[i][1][r] = aligned ? hi_a : lo_a;
        }
}

// Decode constants kept in registers (the and-or is a VOP3 instruction: no literal operands).
// Position u (bit p = BITS * u of each 16-bit half): the mask of the code in both halves, the
// fp16 exponent field 25 - p in both halves (so that the code n becomes the fp16 number
// 2^(10 - p) + n, exactly), and -(2^(10 - p) + z) in both halves.
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

// Q items (ring slots S0 .. S0 + Q - 1): the lane's P dwords of one row each, M tokens.
// out[q][m] = d * sum_k (n_k - z) x[m, k]. The items are decoded in lockstep, so that the
// instruction stream carries 2Q independent fma chains.
// Per pair of codes (one per half, same bit position): one and-or builds the fp16 pair
// (2^(10-p) + n_lo, 2^(10-p) + n_hi), one packed fp16 add subtracts 2^(10-p) + z from both --
// exact, giving the integers n - z (code z gives +0) -- and each code takes one fp32 fma whose
// fp16 operand widens exactly (v_fma_mix_f32): the product with x is exact inside the fma.
template <int TYPE, int M, int P, int Q, int S0, int NS>
__device__ __forceinline__ void items_mac(const Slot<P> (&sl)[NS], uint32_t keep,
                                          const float (&xs)[M][P][2][Dec<TYPE>::PAIRS],
                                          const Consts<TYPE> &c, float (&out)[Q][M])
{
    using D = Dec<TYPE>;
    static_assert(S0 + Q <= NS, "");
    // four fma chains per item and token: dword parity x half
    constexpr int CH = P >= 2 ? 2 : 1;
    float acc[Q][M][CH][2];
#pragma unroll
    for (int q = 0; q < Q; q++)
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int h = 0; h < CH; h++)
                acc[q][m][h][0] = acc[q][m][h][1] = 0.0f;
#pragma unroll
    for (int i = 0; i < P; i++) {
        uint32_t v[Q], vs[Q];
#pragma unroll
        for (int q = 0; q < Q; q++) {
            v[q] = sl[S0 + q].dw[i];
            // (dw0 & keep) | (ext & ~keep); ext goes in as a 16-bit operand (bits 16-31 of its
            // register are never selected), so no zero-extension is emitted
            if (i == 0)
                asm("v_bfi_b32 %0, %1, %2, %3"
                    : "=v"(v[q])
                    : "v"(keep), "v"(sl[S0 + q].dw[0]),
                      "v"(__builtin_bit_cast(_Float16, sl[S0 + q].ext)));
            vs[q] = v[q] >> D::SHIFT;
        }
#pragma unroll
        for (int r = 0; r < D::PAIRS; r++) {
            const int u = r % D::NPOS;
#pragma unroll
            for (int q = 0; q < Q; q++) {
                const uint32_t src = r < D::NPOS ? v[q] : vs[q];
                const h2 n = __builtin_bit_cast(h2, (src & c.mask[u]) | c.magic[u]) + c.bias[u];
                const float wlo = (float)n.x, whi = (float)n.y;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float *a = acc[q][m][i % CH];
                    a[0] = __builtin_fmaf(wlo, xs[m][i][0][r], a[0]);
                    a[1] = __builtin_fmaf(whi, xs[m][i][1][r], a[1]);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; q++) {
        const float d = (float)__builtin_bit_cast(_Float16, sl[S0 + q].d);
#pragma unroll
        for (int m = 0; m < M; m++) {
            float t = acc[q][m][0][0] + acc[q][m][0][1];
            if constexpr (CH == 2)
                t += acc[q][m][1][0] + acc[q][m][1][1];
            out[q][m] = d * t;
        }
    }
}

// Sum over the wave; the total lands in every lane (DPP rows, then the permlane swaps).
__device__ __forceinline__ float wave_total(float v)
{
    v = row16_sum(v);
    float lo = v, hi = v;
    swap16(lo, hi);
    v = lo + hi;
    lo = v;
    hi = v;
    swap32(lo, hi);
    return lo + hi;
}

struct Args {
    const uint8_t *W;  // row 0 of this launch
    int64_t N;         // rows of this launch
    int64_t rb;        // bytes per row
    const float *x;    // x[m * xstride + k], k < K
    int64_t K;         // elements of this launch's slice of K
    int64_t xstride;
    float *y;          // y[m * ystride + n]
    int64_t ystride;
    int accumulate;    // add to y (later slices of a long K) instead of overwriting it
    int NP, NC;        // pieces per row, chunks per row (NC divides the wave count, or is one more)
    int Rc_max;        // rows of the CU with the most rows
};

constexpr int kTailMax = 4;  // tail items per wave at most (the host splits taller launches)

// Dynamic LDS: partials [Rc_max][NC][M] floats and 64 dummy slots; then the staged x: with XLDS
// the whole x of the launch [M][NC * 64 * XN] (zero past K), else only the tail chunk
// [M][64 * XN] (17-chunk rows).
// XLDS: x staged in LDS by the workgroup (coalesced loads, once per CU); otherwise every lane
// loads its own x from global memory (for x too large for LDS).
// The grid is even or the rows' byte length a multiple of 4, so all rows of a CU start at the
// same address modulo 4 and every lane keeps one alignment case.
template <int TYPE, int M, int P, int R, bool XLDS>
__global__ void __launch_bounds__(kThreads) pn_gemv_vec_kernel(Args a)
{
    using D = Dec<TYPE>;
    constexpr int XN = D::CPW * P;  // x values per lane and token
    constexpr int V = R * M;        // partials per lane and batch
    constexpr uint32_t kChunkBytes = 272u * P;
    static_assert(V % 4 == 0, "a batch of R items times M tokens must be a multiple of 4");
    extern __shared__ float lds[];

    const int lane = threadIdx.x & 63;
    const int W = blockDim.x >> 6;  // waves: NC * (16 / NC), or 16 when NC = 17
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x, cu = blockIdx.x;
    const int Rc = (int)((a.N - cu + G - 1) / G);  // rows cu, cu + G, ...
    float *part = lds;                                // [Rc_max][NC][M], then 64 dummy slots
    const int dummy = a.Rc_max * a.NC * M;
    float *xl = lds + dummy + 64;                     // staged x
    const uint32_t par2 =
        (uint32_t)(reinterpret_cast<uintptr_t>(a.W) + (uint64_t)cu * (uint64_t)a.rb) & 2u;
    const bool tail = a.NC > W;  // 17 chunks: chunk W is shared out as tail items

    // main items: chunk c for rows k = j, j + S, ... (S = W / NC waves per chunk)
    const int NCm = tail ? W : a.NC;
    const int S = W / NCm;
    const int c = w % NCm, j = w / NCm;
    const int n_items = Rc > j ? (Rc - j + S - 1) / S : 0;
    // tail items: rows [tb0, tb1) of chunk W
    const int tb0 = tail ? Rc * w / W : 0, tb1 = tail ? Rc * (w + 1) / W : 0;
    const int n_tail = tb1 - tb0;

    // lanes past the end of a partial last chunk read lane 0's piece (in bounds) and get zero x
    const bool active = c * 64 + lane < a.NP;
    const bool active_t = W * 64 + lane < a.NP;
    const LaneMap lm = lane_map<TYPE, P>(active ? lane : 0, par2);
    LaneMap lt = lm;  // the tail chunk
    if (tail)
        lt = lane_map<TYPE, P>(active_t ? lane : 0, par2);

    // ---- x staging, part 1: the workgroup's coalesced loads (global -> registers), issued before
    // the weight loads so that waiting for them never waits for weights
    constexpr int kStage = 8;  // float4 per thread per staging pass
    const int xs_chunk0 = XLDS ? 0 : (tail ? W : 0);
    const int xs_chunks = XLDS ? a.NC : (tail ? 1 : 0);
    const int xs_per_tok = xs_chunks * 64 * XN;  // floats per token (a multiple of 4)
    const int xs_n4 = M * xs_per_tok / 4;         // float4 to stage
    f32x4a4 stage[kStage];
    auto stage_load = [&](int pass) {
#pragma unroll
        for (int h = 0; h < kStage; h++) {
            const int i4 = (pass * kStage + h) * (int)blockDim.x + (int)threadIdx.x;
            f32x4a4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (i4 < xs_n4) {
                const int f = 4 * i4, m = f / xs_per_tok, r = f - m * xs_per_tok;
                const int64_t e = (int64_t)xs_chunk0 * 64 * XN + r;
                const float *src = a.x + (int64_t)m * a.xstride + e;
                if (e + 4 <= a.K) {
                    v = *reinterpret_cast<const f32x4a4 *>(src);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        v[q] = (e + q < a.K) ? src[q] : 0.0f;
                }
            }
            stage[h] = v;
        }
    };
    auto stage_store = [&](int pass) {
#pragma unroll
        for (int h = 0; h < kStage; h++) {
            const int i4 = (pass * kStage + h) * (int)blockDim.x + (int)threadIdx.x;
            if (i4 < xs_n4)
                *reinterpret_cast<f32x4a4 *>(xl + 4 * i4) = stage[h];
        }
    };
    const int stage_passes = (xs_n4 + kStage * (int)blockDim.x - 1) / (kStage * (int)blockDim.x);
    if (stage_passes > 0)
        stage_load(0);

    // ---- x of this wave's chunk when it is not staged: straight from global memory
    float xs[M][P][2][D::PAIRS];
    if constexpr (!XLDS) {
        const int e = c * 64 * XN + lm.elem;
#pragma unroll
        for (int m = 0; m < M; m++) {
            float xv[XN];
#pragma unroll
            for (int i = 0; i < XN; i++)
                xv[i] = 0.0f;
            if (active)
                load_x(a.x + (int64_t)m * a.xstride + e, xv);
            pair_x<TYPE, P>(xv, lm.aligned, xs[m]);
        }
    }
    const Consts<TYPE> cst = make_consts<TYPE>();

    // the launch's weights as a buffer: byte offsets fit 32 bits (the host keeps a launch's rows
    // under 2 GiB); every offset used below lies inside the rows
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.W), (short)0, (int)(a.N * a.rb), 0x00020000);
    const uint32_t rb32 = (uint32_t)a.rb;
    // main item t: row cu + G (j + S t), chunk c
    const uint32_t main_base = ((uint32_t)cu + (uint32_t)(G * j)) * rb32 + kChunkBytes * c;
    const uint32_t main_step = (uint32_t)(G * S) * rb32;
    auto main_off = [&](int t) -> uint32_t {
        t = min(t, n_items - 1);  // past the end: re-read the last item (a cache hit, discarded)
        return main_base + (uint32_t)t * main_step;
    };
    // ---- weight loads: tail items first (the oldest in flight), then the ring of main items
    Slot<P> tslot[kTailMax][1];
    if (tail) {
#pragma unroll
        for (int i = 0; i < kTailMax; i++) {
            const int k = n_tail > 0 ? tb0 + min(i, n_tail - 1) : 0;
            load_slot<P>(rs, ((uint32_t)cu + (uint32_t)(G * k)) * rb32 + kChunkBytes * W, lt,
                         tslot[i][0]);
        }
    }
    Slot<P> ring[R];
    if (n_items > 0) {
#pragma unroll
        for (int s = 0; s < R; s++)
            load_slot<P>(rs, main_off(s), lm, ring[s]);
    }

    // ---- x staging, part 2: registers -> LDS (more passes for a large x), then every lane
    // reads its piece's x
    if (stage_passes > 0) {
        stage_store(0);
        for (int pass = 1; pass < stage_passes; pass++) {
            stage_load(pass);
            stage_store(pass);
        }
        __syncthreads();
    }
    if constexpr (XLDS) {
        const int off = c * 64 * XN + lm.elem;
#pragma unroll
        for (int m = 0; m < M; m++) {
            float xv[XN];
#pragma unroll
            for (int i = 0; i < XN; i++) {
                const float v = xl[m * xs_per_tok + off + i];
                xv[i] = active ? v : 0.0f;
            }
            pair_x<TYPE, P>(xv, lm.aligned, xs[m]);
        }
    }

    // ---- tail items (17-chunk rows): x of chunk W from LDS
    if (tail) {
        const int toff = (W - xs_chunk0) * 64 * XN + lt.elem;
#pragma unroll
        for (int i = 0; i < kTailMax; i++) {
            if (i < n_tail) {
                float xt[M][P][2][D::PAIRS];
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float xv[XN];
#pragma unroll
                    for (int q = 0; q < XN; q++) {
                        const float v = xl[m * xs_per_tok + toff + q];
                        xv[q] = active_t ? v : 0.0f;
                    }
                    pair_x<TYPE, P>(xv, lt.aligned, xt[m]);
                }
                const int k = tb0 + i;
                float o[1][M];
                items_mac<TYPE, M, P, 1, 0, 1>(tslot[i], lt.keep, xt, cst, o);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float tot = wave_total(o[0][m]);
                    part[lane == 0 ? (k * a.NC + W) * M + m : dummy + lane] = tot;
                }
            }
        }
    }

    // ---- main items in whole batches of R, computed in groups of Q (interleaved by the
    // compiler), each group's slots refilled right after the group
    constexpr int Q = R >= 4 ? 2 : 1;
    auto group_mac = [&](int g, float (&o)[Q][M]) {
        // g is a compile-time constant after unrolling; the switch folds away
        static_assert(R <= 8, "");
        switch (g) {
        case 0: items_mac<TYPE, M, P, Q, 0, R>(ring, lm.keep, xs, cst, o); break;
        case 1: if constexpr (Q == 1) items_mac<TYPE, M, P, Q, 1, R>(ring, lm.keep, xs, cst, o); break;
        case 2: if constexpr (2 + Q <= R) items_mac<TYPE, M, P, Q, 2, R>(ring, lm.keep, xs, cst, o); break;
        case 3: if constexpr (Q == 1 && 4 <= R) items_mac<TYPE, M, P, Q, 3, R>(ring, lm.keep, xs, cst, o); break;
        case 4: if constexpr (4 + Q <= R) items_mac<TYPE, M, P, Q, 4, R>(ring, lm.keep, xs, cst, o); break;
        case 5: if constexpr (Q == 1 && 6 <= R) items_mac<TYPE, M, P, Q, 5, R>(ring, lm.keep, xs, cst, o); break;
        case 6: if constexpr (6 + Q <= R) items_mac<TYPE, M, P, Q, 6, R>(ring, lm.keep, xs, cst, o); break;
        default: if constexpr (Q == 1 && 8 <= R) items_mac<TYPE, M, P, Q, 7, R>(ring, lm.keep, xs, cst, o); break;
        }
    };
    int t0 = 0;
    for (; t0 + R <= n_items; t0 += R) {
        float pv[V];
#pragma unroll
        for (int g = 0; g < R; g += Q) {
            float o[Q][M];
            group_mac(g, o);
#pragma unroll
            for (int q = 0; q < Q; q++)
#pragma unroll
                for (int m = 0; m < M; m++)
                    pv[(g + q) * M + m] = o[q][m];
            // refill the slots only after their last use, so that the refills land in the slots'
            // own registers (a refill hoisted above the use would need a copy at the loop edge,
            // which waits for the load)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = g; s < g + Q; s++)
                load_slot<P>(rs, main_off(t0 + s + R), lm, ring[s]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // reduce the batch over the wave: tot[i] in DPP row q = total of value i + q * V/4.
        // Every lane stores (the first lane of each DPP row to its partial, the others to their own
        // dummy slot): a divergent branch here would make the compiler drain the loads in flight.
        float tot[V / 4];
        transpose_reduce<V>(pv, tot);
        {
            const int q = lane >> 4;
#pragma unroll
            for (int i = 0; i < V / 4; i++) {
                const int v = i + q * (V / 4);
                const int s = v / M, m = v - s * M;
                const int t = t0 + s;
                const int idx = (lane & 15) == 0 ? ((j + S * t) * a.NC + c) * M + m : dummy + lane;
                part[idx] = tot[i];
            }
        }
    }
    // ---- the last n_items - t0 < R items, one at a time (they sit in ring slots 0, 1, ...)
#pragma unroll
    for (int s = 0; s < R - 1; s++) {
        if (t0 + s < n_items) {
            float o[1][M];
            items_mac<TYPE, M, P, 1, 0, 1>(*reinterpret_cast<const Slot<P>(*)[1]>(&ring[s]), lm.keep, xs,
                                           cst, o);
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float tot = wave_total(o[0][m]);
                part[lane == 0 ? ((j + S * (t0 + s)) * a.NC + c) * M + m : dummy + lane] = tot;
            }
        }
    }

    __syncthreads();
    for (int i = threadIdx.x; i < Rc * M; i += blockDim.x) {
        const int k = i / M, m = i - k * M;
        float acc = 0.0f;
        for (int cc = 0; cc < a.NC; cc++)
            acc += part[((size_t)k * a.NC + cc) * M + m];
        float *yp = a.y + (int64_t)m * a.ystride + cu + (int64_t)G * k;
        *yp = a.accumulate ? *yp + acc : acc;
    }
}

// ---- the streaming kernel: coalesced 16-byte loads straight into LDS ----------------------------
//
// For rows whose segments are 4-byte aligned and a whole number of 16-byte pieces (W 4-byte
// aligned, an even block count per row, chunks of 8P blocks = 17P pieces). An item (row, chunk)
// is copied by the wave into its own LDS ring slot with 17P consecutive 16-byte loads
// (buffer_load ... lds: lane i copies bytes [16i, 16i + 16) of the segment), so every load
// instruction reads one contiguous span and every byte of the matrix is read once. The lanes
// then read their pieces (the same LaneMap as above, within the slot) from LDS.
// The compiler does not track the copies into LDS: the waits for them are explicit
// (s_waitcnt vmcnt, counting the copies issued after the awaited one), and a slot is refilled only
// after the reads of its previous item have returned (s_waitcnt lgkmcnt(0)).

typedef __attribute__((address_space(3))) void lds_void;

// Copy instructions per item: 17P pieces over 64 lanes.
template <int P> constexpr int copy_instrs() { return (17 * P + 63) / 64; }

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

// The LDS byte address of a shared-memory pointer (what M0 takes).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const void *)p);
}

// pieces: 16-byte pieces of this chunk (17P, or fewer for the last chunk of a row: 17 per 8 blocks).
// Every instruction is issued with at least lane 0 active (a lane with no piece of its own copies
// piece 0 again, into the slot's unused tail), so that each item adds exactly copy_instrs<P>() to
// the wave's vmcnt, whatever its length.
// The copy is written as assembly on purpose: the compiler would otherwise make every later LDS read
// wait for all copies in flight (it cannot tell the ring slots apart), which empties the ring.
template <int P>
__device__ __forceinline__ void copy_item(u32x4s rs, uint32_t soff, uint32_t dst, int lane,
                                          int pieces)
{
#pragma unroll
    for (int k = 0; k < copy_instrs<P>(); k++) {
        const bool mine = lane + 64 * k < pieces;
        if (mine || lane == 0) {
            const uint32_t vo = mine ? 1024u * k + 16u * lane : 0u;
            asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                         :
                         : "v"(vo), "s"(rs), "s"(dst + 1024u * k), "s"(soff)
                         : "memory", "m0");
        }
    }
}

// A lane's piece from its LDS slot: P + 1 dwords from its first aligned dword (one vector read;
// the last dword carries ext in its low half for unaligned words, and is unused otherwise), and d.
typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x5a4 __attribute__((ext_vector_type(5), aligned(4)));
template <int P>
__device__ __forceinline__ void read_piece(const uint8_t *sb, const LaneMap &lm, Slot<P> &sl)
{
    if constexpr (P == 1) {
        const u32x2a4 v = *reinterpret_cast<const u32x2a4 *>(sb + lm.main);
        sl.dw[0] = v[0];
        sl.ext = (uint16_t)v[1];
    } else if constexpr (P == 2) {
        const u32x3a4 v = *reinterpret_cast<const u32x3a4 *>(sb + lm.main);
        sl.dw[0] = v[0];
        sl.dw[1] = v[1];
        sl.ext = (uint16_t)v[2];
    } else {
        static_assert(P == 4, "pieces of 1, 2 or 4 words");
        const u32x4a4 v = *reinterpret_cast<const u32x4a4 *>(sb + lm.main);
        const uint32_t e = *reinterpret_cast<const uint32_t *>(sb + lm.main + 16);
        sl.dw[0] = v[0];
        sl.dw[1] = v[1];
        sl.dw[2] = v[2];
        sl.dw[3] = v[3];
        sl.ext = (uint16_t)e;
    }
    sl.d = *reinterpret_cast<const uint16_t *>(sb + lm.d);
}

#define PN_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory")

// Wait until at most `newer` (0 <= newer <= MAXN, uniform) memory operations are in flight: for
// the copy issued just before the last `newer` ones. The immediate is chosen by a uniform branch.
template <int MAXN>
__device__ __forceinline__ void wait_newer(int newer)
{
    if constexpr (MAXN > 0) {
        if (newer >= MAXN) {
            PN_WAIT_VM(MAXN);
            return;
        }
        wait_newer<MAXN - 1>(newer);
    } else {
        PN_WAIT_VM(0);
    }
}
#define PN_WAIT_LGKM0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")

// LDS: partials [Rc_max][NC][M] and 64 dummy slots, the staged x (as above), then per wave a ring
// of R slots of 272P bytes, then (17-chunk rows) per wave kTailMax tail slots.
// WPE: waves per SIMD the kernel is built for (8: two workgroups per CU, 64 registers).
template <int TYPE, int M, int P, int R, int B, bool XLDS, int WPE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
pn_gemv_stream_kernel(Args a)
{
    using D = Dec<TYPE>;
    constexpr int XN = D::CPW * P;
    constexpr int V = B * M;
    constexpr uint32_t L = 272u * P;
    constexpr int I = copy_instrs<P>();
    // items decoded per step (two in lockstep where the registers allow)
    constexpr int Q = WPE <= 4 && M <= 2 && R % 2 == 0 && B % 4 == 0 ? 2 : 1;
    static_assert(B % R == 0 && B % (2 * Q) == 0 && R % Q == 0 && V % 4 == 0, "");
    static_assert((R - 1) * I <= 63, "vmcnt range");
    extern __shared__ float lds[];

    const int lane = threadIdx.x & 63;
    const int W = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x, cu = blockIdx.x;
    const int Rc = (int)((a.N - cu + G - 1) / G);
    float *part = lds;
    const int dummy = a.Rc_max * a.NC * M;
    float *xl = lds + dummy + 64;
    const bool tail = a.NC > W;
    const int NCm = tail ? W : a.NC;
    const int S = W / NCm;
    const int c = w % NCm, j = w / NCm;
    const int n_items = Rc > j ? (Rc - j + S - 1) / S : 0;
    const int tb0 = tail ? Rc * w / W : 0, tb1 = tail ? Rc * (w + 1) / W : 0;
    const int n_tail = tb1 - tb0;
    const bool active = c * 64 + lane < a.NP;
    const bool active_t = W * 64 + lane < a.NP;
    // rows start 4-byte aligned: block b of a chunk starts at 34b, aligned words for odd b. The
    // piece is read from LDS as P + 1 dwords from lm.main (ext in the last one's low half)
    const LaneMap lm = lane_map<TYPE, P>(active ? lane : 0, 0u);
    const LaneMap lt = lane_map<TYPE, P>(active_t ? lane : 0, 0u);

    const int xs_chunk0 = XLDS ? 0 : (tail ? W : 0);
    const int xs_chunks = XLDS ? a.NC : (tail ? 1 : 0);
    const int xs_per_tok = xs_chunks * 64 * XN;
    const int xs_n4 = M * xs_per_tok / 4;
    // ring slots 16-byte aligned
    uint8_t *ring_all = reinterpret_cast<uint8_t *>(lds) +
                        ((((uint32_t)(dummy + 64 + M * xs_per_tok)) * 4u + 15u) & ~15u);
    constexpr uint32_t SL = L + 16;  // slot stride: a piece read may run 4 bytes past the chunk
    uint8_t *ring = ring_all + (uint32_t)w * (R * SL);
    uint8_t *tslots = ring_all + (uint32_t)W * (R * SL) + (uint32_t)w * (kTailMax * SL);
    const uint32_t ring_a = lds_addr(ring), tslots_a = lds_addr(tslots);

    // buffer resource of the launch's weights: base, stride 0, byte count, dword 3 of a raw buffer
    const uint64_t wb = reinterpret_cast<uint64_t>(a.W);
    const u32x4s rs = {(uint32_t)wb, (uint32_t)(wb >> 32) & 0xFFFFu, (uint32_t)(a.N * a.rb),
                       0x00020000u};
    const uint32_t rb32 = (uint32_t)a.rb;
    const uint32_t main_base = ((uint32_t)cu + (uint32_t)(G * j)) * rb32 + L * c;
    // 16-byte pieces of this wave's chunk and of the tail chunk (the last chunk of a row may be
    // short: the row holds a multiple of 8 blocks, 17 pieces per 8 blocks)
    const int row_pieces = (int)(rb32 / 16u);
    const int pc = min(17 * P, row_pieces - 17 * P * c);
    const int pt = min(17 * P, row_pieces - 17 * P * W);
    const uint32_t main_step = (uint32_t)(G * S) * rb32;
    auto main_off = [&](int t) -> uint32_t {
        t = min(t, n_items - 1);
        return main_base + (uint32_t)t * main_step;
    };

    // ---- x staging: straight from global memory into LDS (copies of 64 consecutive 16-byte
    // pieces of one token per instruction, shared out over the waves), issued before the weight
    // copies, so that waiting for them waits for no weights. K * 4 bytes is a multiple of 16.
    {
        const uint64_t xb = reinterpret_cast<uint64_t>(a.x);
        const u32x4s rx = {(uint32_t)xb, (uint32_t)(xb >> 32) & 0xFFFFu,
                           (uint32_t)((M - 1) * a.xstride + a.K) * 4u, 0x00020000u};
        const int e0 = xs_chunk0 * 64 * XN;                                 // first element
        const int ppt = (int)(min((int64_t)xs_per_tok, a.K - e0) / 4);       // pieces per token
        const int ipt = (ppt + 63) / 64;                                    // instructions per token
        const uint32_t xl_a = lds_addr(xl);
        for (int q = w; q < M * ipt; q += W) {
            const int m = q / ipt, k = q - m * ipt;
            const int pi = 64 * k + lane;  // this lane's piece of token m
            if (pi < ppt) {
                const uint32_t vo = (uint32_t)((int64_t)m * a.xstride + e0) * 4u + 16u * pi;
                asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                             :
                             : "v"(vo), "s"(rx), "s"(xl_a + 4u * (m * xs_per_tok + 64 * 4 * k))
                             : "memory", "m0");
            }
        }
    }

    // x of this wave's chunk when it is not staged: per lane, XN consecutive floats per token,
    // loaded (and waited for) before any weight copy is issued -- an ordinary load, whose wait
    // the compiler places itself (lanes past the end of a partial last chunk get zero x)
    float xs[M][P][2][D::PAIRS];
    if constexpr (!XLDS) {
        const int e = c * 64 * XN + lm.elem;
#pragma unroll
        for (int m = 0; m < M; m++) {
            float xv[XN];
#pragma unroll
            for (int i = 0; i < XN; i++)
                xv[i] = 0.0f;
            if (active)
                load_x(a.x + (int64_t)m * a.xstride + e, xv);
            pair_x<TYPE, P>(xv, lm.aligned, xs[m]);
        }
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int i = 0; i < P; i++)
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int r = 0; r < D::PAIRS; r++)
                        asm volatile("" ::"v"(xs[m][i][h][r]));  // loaded before the copies start
    }
    const Consts<TYPE> cst = make_consts<TYPE>();

    // ---- copies: the tail items (kTailMax, clamped), then the first R main items
    if (tail) {
#pragma unroll
        for (int i = 0; i < kTailMax; i++) {
            const int k = n_tail > 0 ? tb0 + min(i, n_tail - 1) : 0;
            copy_item<P>(rs, ((uint32_t)cu + (uint32_t)(G * k)) * rb32 + L * W, tslots_a + i * SL,
                         lane, pt);
        }
    }
#pragma unroll
    for (int s = 0; s < R; s++)
        if (s < n_items)
            copy_item<P>(rs, main_off(s), ring_a + s * SL, lane, pc);

    // ---- x: wait for this wave's x copies (the weight copies issued after them may still fly),
    // then the workgroup's, then every lane reads its pairing order
    wait_newer<R * I + kTailMax * I>(((tail ? kTailMax : 0) + min(R, n_items)) * I);
    __syncthreads();
    if constexpr (XLDS) {
        const int off = c * 64 * XN + lm.elem;
#pragma unroll
        for (int m = 0; m < M; m++) {
            float xv[XN];
#pragma unroll
            for (int i = 0; i < XN; i++) {
                const float v = xl[m * xs_per_tok + off + i];
                xv[i] = active ? v : 0.0f;
            }
            pair_x<TYPE, P>(xv, lm.aligned, xs[m]);
        }
    }

    // ---- tail items: wait for all of their copies (the R main copies may still fly)
    if (tail) {
        wait_newer<R * I>(min(R, n_items) * I);
        const int toff = (W - xs_chunk0) * 64 * XN + lt.elem;
#pragma unroll
        for (int i = 0; i < kTailMax; i++) {
            if (i < n_tail) {
                float xt[M][P][2][D::PAIRS];
#pragma unroll
                for (int m = 0; m < M; m++) {
                    float xv[XN];
#pragma unroll
                    for (int q = 0; q < XN; q++) {
                        const float v = xl[m * xs_per_tok + toff + q];
                        xv[q] = active_t ? v : 0.0f;
                    }
                    pair_x<TYPE, P>(xv, lt.aligned, xt[m]);
                }
                Slot<P> ts[1];
                read_piece<P>(tslots + i * SL, lt, ts[0]);
                float o[1][M];
                items_mac<TYPE, M, P, 1, 0, 1>(ts, lt.keep, xt, cst, o);
                const int k = tb0 + i;
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float tot = wave_total(o[0][m]);
                    part[lane == 0 ? (k * a.NC + W) * M + m : dummy + lane] = tot;
                }
            }
        }
    }

    if (n_items > 0) {
        // pipeline in steps of Q items: D[par] holds items t .. t + Q - 1 (read from LDS one step
        // ahead); a step refills their slots with items t + R .., starts reading the next Q items
        // and decodes its own in lockstep
        Slot<P> Dq[2][Q];
        wait_newer<(R - Q) * I>((min(R, n_items) - Q) * I);
#pragma unroll
        for (int q = 0; q < Q; q++)
            read_piece<P>(ring + q * SL, lm, Dq[0][q]);
        auto step = [&](int t, int par, float (&o)[Q][M]) {
            PN_WAIT_LGKM0();
            // refills only for items that exist, so that the last wait drains no useless copy;
            // then wait for items t + Q .. t + 2Q - 1, with the copies issued after them in flight
#pragma unroll
            for (int q = 0; q < Q; q++)
                if (t + q + R < n_items)
                    copy_item<P>(rs, main_off(t + q + R), ring_a + ((t + q) % R) * SL, lane, pc);
            wait_newer<(R - Q) * I>(min(n_items - (t + 2 * Q), R - Q) * I);
#pragma unroll
            for (int q = 0; q < Q; q++)
                read_piece<P>(ring + ((t + Q + q) % R) * SL, lm, Dq[par ^ 1][q]);
            items_mac<TYPE, M, P, Q, 0, Q>(Dq[par], lm.keep, xs, cst, o);
            // keep the decode ahead of the next step's wait for these reads: its results are
            // inputs of an (empty) volatile statement, which stays in program order
#pragma unroll
            for (int q = 0; q < Q; q++)
#pragma unroll
                for (int m = 0; m < M; m++)
                    asm volatile("" ::"v"(o[q][m]));
        };
        int t0 = 0;
        for (; t0 + B <= n_items; t0 += B) {
            float pv[V];
#pragma unroll
            for (int s = 0; s < B; s += Q) {
                float o[Q][M];
                step(t0 + s, (s / Q) & 1, o);
#pragma unroll
                for (int q = 0; q < Q; q++)
#pragma unroll
                    for (int m = 0; m < M; m++)
                        pv[(s + q) * M + m] = o[q][m];
            }
            float tot[V / 4];
            transpose_reduce<V>(pv, tot);
            const int q = lane >> 4;
#pragma unroll
            for (int i = 0; i < V / 4; i++) {
                const int v = i + q * (V / 4);
                const int s = v / M, m = v - s * M;
                const int idx =
                    (lane & 15) == 0 ? ((j + S * (t0 + s)) * a.NC + c) * M + m : dummy + lane;
                part[idx] = tot[i];
            }
        }
        // the last n_items - t0 < B items: t0 is a multiple of B, so the pipeline state is that of
        // a batch start (items past n_items are decoded from re-read slots and dropped)
#pragma unroll
        for (int s = 0; s < B; s += Q) {
            if (t0 + s < n_items) {
                float o[Q][M];
                step(t0 + s, (s / Q) & 1, o);
#pragma unroll
                for (int q = 0; q < Q; q++) {
                    const int t = t0 + s + q;
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        const float tot = wave_total(o[q][m]);
                        part[lane == 0 && t < n_items ? ((j + S * t) * a.NC + c) * M + m
                                                      : dummy + lane] = tot;
                    }
                }
            }
        }
        // drain the copies still in flight before the workgroup may exit
        PN_WAIT_VM(0);
    }

    __syncthreads();
    for (int i = threadIdx.x; i < Rc * M; i += blockDim.x) {
        const int k = i / M, m = i - k * M;
        float acc = 0.0f;
        for (int cc = 0; cc < a.NC; cc++)
            acc += part[((size_t)k * a.NC + cc) * M + m];
        float *yp = a.y + (int64_t)m * a.ystride + cu + (int64_t)G * k;
        *yp = a.accumulate ? *yp + acc : acc;
    }
}

}  // namespace vec

// ---- host -----------------------------------------------------------------------------------------

namespace {

template <int TYPE, int M, int P, int R, bool XLDS>
int launch_one(const vec::Args &a, int grid, int waves, size_t lds, hipStream_t s)
{
    constexpr auto kern = vec::pn_gemv_vec_kernel<TYPE, M, P, R, XLDS>;
    if (!lds_limit_once<kern>(vec::kLdsMax))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * waves), lds, s, a);
    return launch_status();
}

template <int TYPE, int M, int P, int R>
int launch_x(const vec::Args &a, bool xlds, int grid, int waves, size_t lds, hipStream_t s)
{
    return xlds ? launch_one<TYPE, M, P, R, true>(a, grid, waves, lds, s)
                : launch_one<TYPE, M, P, R, false>(a, grid, waves, lds, s);
}

template <int TYPE, int M, int P, int R, int B, bool XLDS, int WPE>
int launch_stream_one(const vec::Args &a, int grid, int waves, size_t lds, hipStream_t s)
{
    constexpr auto kern = vec::pn_gemv_stream_kernel<TYPE, M, P, R, B, XLDS, WPE>;
    if (!lds_limit_once<kern>(vec::kLdsMax))
        return PN_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * waves), lds, s, a);
    return launch_status();
}

// Items in flight per wave (a batch of R items times M tokens must be a multiple of 4).
template <int M> constexpr int ring_items() { return M == 1 ? 8 : M == 2 ? 4 : M == 3 ? 4 : 2; }
// Streaming kernel: LDS ring slots per wave, and items per reduction batch.
// Streaming kernel: LDS ring slots per wave, and items per reduction batch. One token on a tall
// matrix runs two workgroups per CU (8 waves per SIMD, 64 registers, batches of 4 items);
// otherwise one workgroup of up to 16 waves per CU.
template <int M> constexpr int stream_ring() { return M == 4 ? 2 : 4; }
template <int M, int WPE> constexpr int stream_batch() { return WPE == 8 ? 4 : M == 1 ? 8 : M == 4 ? 2 : 4; }

template <int TYPE, int M, int P, int WPE>
int launch_stream_w(const vec::Args &a, bool xlds, int grid, int waves, size_t lds, hipStream_t s)
{
    constexpr int R = stream_ring<M>(), B = stream_batch<M, WPE>();
    return xlds ? launch_stream_one<TYPE, M, P, R, B, true, WPE>(a, grid, waves, lds, s)
                : launch_stream_one<TYPE, M, P, R, B, false, WPE>(a, grid, waves, lds, s);
}

template <int TYPE, int M, int P>
int launch_stream_x(const vec::Args &a, bool xlds, bool two, int grid, int waves, size_t lds,
                    hipStream_t s)
{
    if constexpr (M == 1)
        if (two)
            return launch_stream_w<TYPE, M, P, 8>(a, xlds, grid, waves, lds, s);
    return launch_stream_w<TYPE, M, P, 4>(a, xlds, grid, waves, lds, s);
}

// One launch group over a slice of K of nb blocks starting at block b0 (rows of rb bytes).
// stream: the slice's rows are 4-byte aligned and hold a multiple of 8 blocks (streaming kernel);
// otherwise the lane kernel, which assumes no alignment.
template <int TYPE, int M>
int launch_slice(const uint8_t *W, int64_t N, int64_t rb, int64_t b0, int64_t nb, const float *x,
                 int64_t K, float *y, bool accumulate, bool stream, hipStream_t s)
{
    using D = vec::Dec<TYPE>;
    // rows of an odd block count alternate between 0 and 2 mod 4: an even grid keeps all rows of a
    // CU (cu, cu + G, ...) at one alignment
    const bool odd_rows = (rb & 2) != 0;
    const int cus = device_cus();
    // workgroups per CU and the LDS each may take
    const int per_cu = stream && M == 1 && N >= 16 * (int64_t)cus ? 2 : 1;
    const int64_t lds_max = per_cu == 2 ? vec::kLdsMax2 : vec::kLdsMax;
    const size_t lds_floor = per_cu == 2 ? vec::kLdsFloor2 : vec::kLdsFloor;
    // words per lane piece: 1 at 3-4 tokens (their x fills the registers), else 2; 4 where a row
    // would need more than 17 chunks of 2-word pieces
    const int P = M >= 3 && (nb + 7) / 8 <= vec::kWaves + 1           ? 1
                  : (nb * 8 / 2 + 63) / 64 > vec::kWaves + 1 ? 4
                                                             : 2;
    const int64_t NP = nb * 8 / P, NC = (NP + 63) / 64;
    if (NC > vec::kWaves + 1)
        return PN_ERR_SHAPE;  // the caller slices K so that this does not happen
    const bool tail = NC == vec::kWaves + 1;
    const int waves = tail ? vec::kWaves : (int)(NC * (vec::kWaves / NC));
    const int XN = D::CPW * P;
    // the streaming kernel's LDS rings (and tail slots)
    const int ring = stream_ring<M>();
    const size_t ring_bytes =
        stream ? (size_t)waves * (272 * P + 16) * (ring + (tail ? vec::kTailMax : 0)) + 16 : 0;
    // x staged in LDS by each workgroup when the whole x (M tokens, padded to whole chunks)
    // leaves room for the partials; otherwise each lane loads its own x (and only the tail chunk
    // is staged)
    const size_t xall_bytes = (size_t)M * NC * 64 * XN * sizeof(float);
    // the streaming kernel stages x whenever the partials of its rows still fit beside it
    const int64_t rows_hint = std::min<int64_t>((N + per_cu * cus - 1) / (per_cu * cus), 64);
    const bool xlds =
        stream ? xall_bytes + ring_bytes + 64 * sizeof(float) +
                         (size_t)(rows_hint * NC * M) * sizeof(float) <=
                     (size_t)lds_max
               : xall_bytes <= 128 * 1024;
    const size_t x_bytes = xlds ? xall_bytes : tail ? (size_t)M * 64 * XN * sizeof(float) : 0;
    // rows per launch: the partials must fit the LDS beside the staged x, and a wave takes at most
    // kTailMax tail items
    int64_t rows_per_cu = (lds_max - (int64_t)(x_bytes + ring_bytes) -
                           64 * (int64_t)sizeof(float)) /
                          (NC * M * (int64_t)sizeof(float));
    if (tail)
        rows_per_cu = std::min<int64_t>(rows_per_cu, (int64_t)vec::kTailMax * vec::kWaves);
    if (rows_per_cu < 1)
        return PN_ERR_SHAPE;
    const int grid_cap = odd_rows && cus > 1 && (cus & 1) ? cus - 1 : per_cu * cus;
    int64_t done = 0;
    while (done < N) {
        // a launch's rows stay under 2 GiB: the kernel addresses them with 32-bit byte offsets
        int64_t n = std::min<int64_t>(N - done, rows_per_cu * grid_cap);
        n = std::min<int64_t>(n, (int64_t)0x7FFFFFFF / rb);
        int grid = (int)std::min<int64_t>(grid_cap, n);
        if (odd_rows && grid > 1 && (grid & 1)) {
            grid -= 1;
            n = std::min<int64_t>(n, rows_per_cu * grid);
        }
        vec::Args a;
        a.W = W + done * rb + b0 * kBlockBytes;
        a.N = n;
        a.rb = rb;
        a.x = x + b0 * D::G;
        a.K = nb * D::G;
        a.xstride = K;
        a.y = y + done;
        a.ystride = N;
        a.accumulate = accumulate ? 1 : 0;
        a.NP = (int)NP;
        a.NC = (int)NC;
        a.Rc_max = (int)((n + grid - 1) / grid);
        const size_t lds =
            std::max<size_t>(lds_floor,
                             ((size_t)a.Rc_max * NC * M + 64) * sizeof(float) + x_bytes + ring_bytes);
        int st;
        constexpr int R = ring_items<M>();
        if constexpr (M >= 3) {
            if (P == 1) {
                st = stream ? launch_stream_x<TYPE, M, 1>(a, xlds, false, grid, waves, lds, s)
                            : launch_x<TYPE, M, 1, R>(a, xlds, grid, waves, lds, s);
                if (st != PN_OK)
                    return st;
                done += n;
                continue;
            }
        }
        if (stream) {
            st = P == 2 ? launch_stream_x<TYPE, M, 2>(a, xlds, per_cu == 2, grid, waves, lds, s)
                        : launch_stream_x<TYPE, M, 4>(a, xlds, per_cu == 2, grid, waves, lds, s);
        } else {
            st = P == 2 ? launch_x<TYPE, M, 2, R>(a, xlds, grid, waves, lds, s)
                        : launch_x<TYPE, M, 4, R>(a, xlds, grid, waves, lds, s);
        }
        if (st != PN_OK)
            return st;
        done += n;
    }
    return PN_OK;
}

// Blocks [b0, b0 + nb) of every row: with W 4-byte aligned (and b0 a multiple of 8), the first
// multiple of 8 blocks on the streaming kernel and the rest on the lane kernel, adding to y.
template <int TYPE, int M>
int launch_range(const uint8_t *W, int64_t N, int64_t rb, int64_t b0, int64_t nb, const float *x,
                 int64_t K, float *y, bool accumulate, hipStream_t s)
{
    const bool aligned = (reinterpret_cast<uintptr_t>(W) & 3) == 0 && (b0 & 7) == 0;
    const int64_t nb8 = aligned && !getenv("PN_GEMV_LANE") ? nb & ~(int64_t)7 : 0;
    if (nb8 > 0) {
        const int st = launch_slice<TYPE, M>(W, N, rb, b0, nb8, x, K, y, accumulate, true, s);
        if (st != PN_OK || nb8 == nb)
            return st;
        accumulate = true;
    }
    return launch_slice<TYPE, M>(W, N, rb, b0 + nb8, nb - nb8, x, K, y, accumulate, false, s);
}

// K is cut into slices of at most 17 chunks of 2-word pieces (272 blocks; 544 with 4-word pieces
// once a row needs them; 136 blocks of 1-word pieces at 3-4 tokens); each slice after the first
// adds its sums to y, in slice order.
template <int TYPE, int M>
int launch_typed(const uint8_t *W, int64_t N, int64_t K, const float *x, float *y, hipStream_t s)
{
    using D = vec::Dec<TYPE>;
    const int64_t nb = K / D::G;
    const int64_t rb = nb * kBlockBytes;
    // 16 chunks of 4-word pieces (17 chunks of 1-word pieces at 3-4 tokens); a multiple of 8
    // keeps every slice's alignment that of the row
    constexpr int64_t kSliceBlocks = M >= 3 ? 136 : 512;
    if (nb <= (M >= 3 ? 136 : 544))
        return launch_range<TYPE, M>(W, N, rb, 0, nb, x, K, y, false, s);
    for (int64_t b0 = 0; b0 < nb; b0 += kSliceBlocks) {
        const int st = launch_range<TYPE, M>(W, N, rb, b0, std::min(kSliceBlocks, nb - b0), x, K,
                                             y, b0 > 0, s);
        if (st != PN_OK)
            return st;
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

}  // namespace

// The vector-unit PN GEMV for 1 <= M <= 4 (arguments already checked by the entry point).
int launch_vec(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
               float *y, hipStream_t s)
{
    return type == PN_TYPE_PN3T ? launch_m<PN_TYPE_PN3T>(W, N, K, x, M, y, s)
                                : launch_m<PN_TYPE_PN4T>(W, N, K, x, M, y, s);
}

}  // namespace pn
