// pn_hadamard.h -- Hadamard rotation of the activations: the device code of the rotation kernel.
//
// "PN weight format", section "Files that use PN": the model rotates the activations that reach the
// PN weights with a Hadamard transform, performed by the engine; the page gives neither the order
// nor the normalisation. Reading used here: K is cut into consecutive slices of B = 2^L elements
// (B divides K), and each slice is multiplied by the orthonormal Sylvester-ordered Walsh-Hadamard
// matrix H_B / sqrt(B), H_B[i][j] = (-1)^popcount(i & j).
//
// Computed as the fast transform: L butterfly stages (a, b) -> (a + b, a - b) on element pairs
// that differ in bit s of their index, s = 0 .. L-1 in order, then one multiply by fp32(1/sqrt B)
// (exact when L is even). Every stage adds two values of the previous one, so each output is a
// sum of B terms +-x taken pairwise in L levels: its error is at most
// ((L + 2) 2^-24 + O(2^-48)) * sum_j |x_j| / sqrt(B) over the slice (L additions and the scaling,
// whose constant carries one more rounding when L is odd).
//
// Layout: a lane holds 4 consecutive elements (one float4), so stages 0-1 run in its registers;
// the 64 lanes of a wave hold 256 consecutive elements, so stages 2-7 pair lanes lane ^ 2^(s-2),
// all on the vector ALU: DPP moves for lane xor 1, 2, 4 (a half-row mirror, i -> i ^ 7, then a
// quad reverse, i -> i ^ 3) and 8 (a row rotation by 8); gfx950's permlane16/32 swaps for xor 16
// and 32, two registers at a time (swap, add and subtract, swap back). Stages 8 and up pair
// elements held by other waves and go through LDS, 1-3 stages per pass.
#pragma once
#include <hip/hip_runtime.h>

#include "pn_common.h"

namespace pn {

typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kHadamardMaxLog = 14;  // B <= 16384

// The value of lane ^ MASK (MASK 1, 2, 4 or 8), by DPP within rows of 16 lanes.
template <int MASK>
__device__ __forceinline__ float hx_partner(float v)
{
    if constexpr (MASK == 1)
        return PN_DPP(v, 0xB1);  // quad_perm [1,0,3,2]
    else if constexpr (MASK == 2)
        return PN_DPP(v, 0x4E);  // quad_perm [2,3,0,1]
    else if constexpr (MASK == 4)
        return PN_DPP(PN_DPP(v, 0x141), 0x1B);  // row_half_mirror, then quad_perm [3,2,1,0]
    else
        return PN_DPP(v, 0x128);  // row_ror:8
}

// One butterfly stage across lanes lane ^ MASK: the lower lane of a pair takes a + b, the upper
// a - b (a held by the lower lane). For MASK 16 and 32 two registers go together: after a swap
// of rows (16) or halves (32) between them, one holds the lower halves of both and the other the
// upper halves; their sum and difference, swapped back, are the two results.
template <int MASK>
__device__ __forceinline__ void hx_swap_bfly(float &a, float &b)
{
    if constexpr (MASK == 32)
        swap32(a, b);
    else
        swap16(a, b);
    const float s = a + b, d = a - b;
    a = s;
    b = d;
    if constexpr (MASK == 32)
        swap32(a, b);
    else
        swap16(a, b);
}

template <int MASK>
__device__ __forceinline__ void hx_lane_stage(float4 &v, bool upper)
{
    if constexpr (MASK >= 16) {
        hx_swap_bfly<MASK>(v.x, v.y);
        hx_swap_bfly<MASK>(v.z, v.w);
    } else {
        // partner + (+-1) * own: the product is exact, so this is the same rounding as
        // partner - own / partner + own, and the DPP move can fold into the add
        const float sgn = upper ? -1.0f : 1.0f;
        v.x = hx_partner<MASK>(v.x) + sgn * v.x;
        v.y = hx_partner<MASK>(v.y) + sgn * v.y;
        v.z = hx_partner<MASK>(v.z) + sgn * v.z;
        v.w = hx_partner<MASK>(v.w) + sgn * v.w;
    }
}

// Stages 0 .. min(L, 8) - 1 on the float4 of this lane: elements 4 * lane .. 4 * lane + 3 of the
// wave's 256 (the wave must be converged, and its 256 elements a whole number of slices or a
// piece of one slice starting at a multiple of 256). Where L <= 8 the scaling follows.
__device__ __forceinline__ void hadamard_wave(float4 &v, int L, float scale)
{
    const unsigned lane = __lane_id();
    float a, b;
    if (L >= 1) {
        a = v.x + v.y;
        b = v.x - v.y;
        v.x = a;
        v.y = b;
        a = v.z + v.w;
        b = v.z - v.w;
        v.z = a;
        v.w = b;
    }
    if (L >= 2) {
        a = v.x + v.z;
        b = v.x - v.z;
        v.x = a;
        v.z = b;
        a = v.y + v.w;
        b = v.y - v.w;
        v.y = a;
        v.w = b;
    }
    if (L >= 3)
        hx_lane_stage<1>(v, lane & 1);
    if (L >= 4)
        hx_lane_stage<2>(v, lane & 2);
    if (L >= 5)
        hx_lane_stage<4>(v, lane & 4);
    if (L >= 6)
        hx_lane_stage<8>(v, lane & 8);
    if (L >= 7)
        hx_lane_stage<16>(v, lane & 16);
    if (L >= 8)
        hx_lane_stage<32>(v, lane & 32);
    if (L <= 8) {
        v.x *= scale;
        v.y *= scale;
        v.z *= scale;
        v.w *= scale;
    }
}

// R stages s .. s+R-1 over buf[0, total) in LDS: groups of 2^R elements at stride 2^s. A thread
// takes 2 groups at a time (NT apart): all their reads, then the butterflies, then the writes of
// the groups that exist (a clamped group past the end is read, never written).
template <int NT, int R>
__device__ __forceinline__ void hx_lds_pass(lds_f32 *buf, int total, int s, bool last, float scale)
{
    constexpr int E = 1 << R, G4 = 2;
    const int ng = total >> R;
    const int low = (1 << s) - 1;
    for (int q0 = (int)threadIdx.x; q0 < ng; q0 += G4 * NT) {
        float v[G4][E];
        int base[G4];
#pragma unroll
        for (int g = 0; g < G4; g++) {
            const int q = min(q0 + g * NT, ng - 1);
            base[g] = ((q >> s) << (s + R)) | (q & low);
#pragma unroll
            for (int j = 0; j < E; j++)
                v[g][j] = buf[base[g] + (j << s)];
        }
#pragma unroll
        for (int g = 0; g < G4; g++) {
#pragma unroll
            for (int b = 0; b < R; b++) {
#pragma unroll
                for (int j = 0; j < E; j++) {
                    if (!(j & (1 << b))) {
                        const float lo = v[g][j], hi = v[g][j | (1 << b)];
                        v[g][j] = lo + hi;
                        v[g][j | (1 << b)] = lo - hi;
                    }
                }
            }
            if (last) {
#pragma unroll
                for (int j = 0; j < E; j++)
                    v[g][j] *= scale;
            }
        }
#pragma unroll
        for (int g = 0; g < G4; g++) {
            if (q0 + g * NT < ng) {
#pragma unroll
                for (int j = 0; j < E; j++)
                    buf[base[g] + (j << s)] = v[g][j];
            }
        }
    }
}

// Stages s0 .. L-1 (L > s0) over buf[0, total) in LDS, total a multiple of 2^L, then the scaling.
// Every thread of the workgroup (NT of them) calls it; it starts and ends with a barrier.
template <int NT>
__device__ void hadamard_lds_stages(lds_f32 *buf, int total, int L, float scale, int s0 = 8)
{
    int s = s0;
    while (s < L) {  // uniform
        const int left = L - s, passes = (left + 2) / 3, r = (left + passes - 1) / passes;
        const bool last = s + r == L;
        __syncthreads();
        switch (r) {
        case 1: hx_lds_pass<NT, 1>(buf, total, s, last, scale); break;
        case 2: hx_lds_pass<NT, 2>(buf, total, s, last, scale); break;
        default: hx_lds_pass<NT, 3>(buf, total, s, last, scale); break;
        }
        s += r;
    }
    __syncthreads();
}

}  // namespace pn
