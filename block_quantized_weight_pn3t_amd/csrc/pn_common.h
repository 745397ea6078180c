// pn_common.h -- shared pieces of the gfx950 kernels and the host entry points of libpn.so.
//
// Formats: "PN weight format" (PNX-FORMAT-v0), sections "Types", "Block layout", "Value";
// NVFP4 per "Quantisation and profiles", section "NVFP4", and NInfer "tensor formats" 3.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pn.h"

namespace pn {

// Per-type constants ("Types"): code width, weights per block, codes per u32 word, zero point.
// LDS_STRIDE is the number of floats a staged block of x occupies in LDS: the G scaled values,
// the block's plain sum of x at offset G, and padding so that consecutive lanes reading 16-byte
// pieces of consecutive blocks hit disjoint LDS banks (stride = 4 mod 32 words for pn4t,
// 20 mod 32 for pn3t: both give 8 (and 16) distinct 16-byte bank groups).
template <int TYPE> struct Fmt;
template <> struct Fmt<PN_TYPE_PN3T> {
    static constexpr int BITS = 3, G = 80, CPW = 10, Z = 4, LDS_STRIDE = 84;
};
template <> struct Fmt<PN_TYPE_PN4T> {
    static constexpr int BITS = 4, G = 64, CPW = 8, Z = 8, LDS_STRIDE = 68;
};

constexpr int kBlockBytes = 34;

// One matrix of a group of PN GEMVs that read the same x (host side).
struct GroupPart {
    const uint8_t *W;
    int64_t N;
    float *y;
    int type;
};

// One PN block brought into registers without assuming 4-byte alignment of its words.
// A block at byte address p (2-byte aligned) is read as 32 bytes from the 4-byte aligned address
// q4 plus one 16-bit piece at q2:
//   p = 0 mod 4: q4 = p (d and words 0..6 straddle dwords), q2 = p + 32 (upper half of word 7);
//   p = 2 mod 4: q4 = p + 2 (the eight words, aligned), q2 = p (d).
// Exactly the block's 34 bytes are read, never a byte past it.
struct RawBlock {
    uint32_t dw[8];
    uint32_t piece;  // the 16-bit piece, zero-extended
    uint32_t shift;  // 16 when p = 0 mod 4, 0 when p = 2 mod 4 (funnel-shift amount)
};

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_block(const uint8_t *p, RawBlock &rb)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const bool odd = (a & 2u) != 0;  // p = 2 mod 4
    const uint8_t *q4 = odd ? p + 2 : p;
    const uint8_t *q2 = odd ? p : p + 32;
    // Ordinary (temporal) loads: the three loads of a block, and neighbouring lanes' blocks, share
    // cache lines; non-temporal loads measured slower here.
    const u32x4a4 v0 = *reinterpret_cast<const u32x4a4 *>(q4);
    const u32x4a4 v1 = *reinterpret_cast<const u32x4a4 *>(q4 + 16);
    rb.piece = *reinterpret_cast<const uint16_t *>(q2);
    rb.dw[0] = v0.x; rb.dw[1] = v0.y; rb.dw[2] = v0.z; rb.dw[3] = v0.w;
    rb.dw[4] = v1.x; rb.dw[5] = v1.y; rb.dw[6] = v1.z; rb.dw[7] = v1.w;
    rb.shift = odd ? 0u : 16u;
}

// Word i (0..7) of the block, as the little-endian u32 at byte 2 + 4i of the block.
__device__ __forceinline__ uint32_t block_word(const RawBlock &rb, int i)
{
    const uint32_t hi = (i < 7) ? rb.dw[i + 1] : rb.piece;
    return __builtin_amdgcn_alignbit(hi, rb.dw[i], rb.shift);
}

// Non-temporal (streaming) loads, for data that one load instruction consumes whole: each cache line
// is requested once, so marking it for early eviction loses nothing and keeps the caches for x.
// (The PN block reader does not use them: its three loads per block share cache lines.)
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt16(const void *p)
{
    const u32x4v t = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 load_nt8(const void *p)
{
    const u32x2v t = __builtin_nontemporal_load(reinterpret_cast<const u32x2v *>(p));
    return make_uint2(t.x, t.y);
}

// The fp16 scale d of the block in the low 16 bits (upper bits undefined).
__device__ __forceinline__ uint32_t block_d_bits(const RawBlock &rb)
{
    return rb.shift ? rb.dw[0] : rb.piece;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// ---- cross-lane reduction -----------------------------------------------------------------------

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

// Row range of a wave. The rows are split into balanced contiguous ranges over the SIMD slots
// (4 per workgroup: a CU's SIMDs, which take the workgroup's waves round-robin), and each slot's
// range over the waves that share that SIMD (wave w and w + 4 of an 8-wave group). Every SIMD thus
// gets the same number of rows, +-1, whichever wave count divides it. The instruction arbiter
// favours the older wave of a SIMD, so it may be given the larger part (fnum/16). The quotient
// and remainder of N by the slot count come from the host (rq, rr): no division runs on the
// device.
struct RowSplit {
    int64_t rq;  // N / (gridDim.x * 4)
    int rr;      // N % (gridDim.x * 4)
};

// (blk: the workgroup's index among those that share the rows)
__device__ __forceinline__ void wave_rows(int64_t N, RowSplit sp, int wave, int nwaves, int fnum,
                                          int64_t &begin, int &count, int blk)
{
    const int slot = blk * 4 + (wave & 3);
    const int h = wave >> 2;
    const int64_t s0 = (int64_t)slot * sp.rq + min(slot, sp.rr);
    const int64_t cnt = sp.rq + (slot < sp.rr ? 1 : 0);
    // two waves per SIMD: the older one (h = 0) takes the first fnum/16 of the slot's rows
    const int64_t mid = nwaves == 8 ? (cnt * fnum + 8) >> 4 : cnt;
    const int64_t b0 = h ? mid : 0;
    const int64_t b1 = h ? cnt : mid;
    count = (int)(b1 - b0);
    // an empty range may start at N; its (unused, clamped) prefetch must still address a real row
    begin = min(s0 + b0, N - 1);
}
__device__ __forceinline__ void wave_rows(int64_t N, RowSplit sp, int wave, int nwaves, int fnum,
                                          int64_t &begin, int &count)
{
    wave_rows(N, sp, wave, nwaves, fnum, begin, count, (int)blockIdx.x);
}

inline RowSplit row_split(int64_t N, int grid)
{
    const int64_t S = (int64_t)grid * 4;
    return RowSplit{N / S, (int)(N % S)};
}

// Host side --------------------------------------------------------------------------------------

// Checks that the current device is gfx950 (cached per device). Returns PN_OK, PN_ERR_HIP or
// PN_ERR_DEVICE.
int check_device();
// Compute units of the current device (cached per device).
int device_cus();

// Raises kernel KERN's limit of dynamic LDS to `bytes`, once per process: a function-local static
// (one per kernel) is initialised exactly once even when several host threads launch at once.
// false if the runtime refused (the caller reports PN_ERR_HIP). The library serves the current
// device of a single-GPU process; the attribute is not set again per device.
template <auto KERN>
inline bool lds_limit_once(int bytes)
{
    static const bool ok = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               bytes) == hipSuccess;
    return ok;
}

// Maps the launch status of the last kernel to PN_OK / PN_ERR_HIP.
int launch_status();

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int pn_group(int type)
{
    return type == PN_TYPE_PN3T ? 80 : type == PN_TYPE_PN4T ? 64 : 0;
}

}  // namespace pn
