// pn_hadamard.h -- Hadamard rotation of the activations, as device code shared by the standalone
// rotation kernel and the GEMV kernels that fuse it into their x staging.
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
// the 64 lanes of a wave hold 256 consecutive elements, so stages 2-7 pair lanes lane ^ 2^(s-2)
// (ds_swizzle within 32 lanes, ds_bpermute across the halves); stages 8 and up pair elements
// held by other waves and go through LDS, 1-4 stages per pass.
#pragma once
#include <hip/hip_runtime.h>

namespace pn {

typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kHadamardMaxLog = 14;  // B <= 16384

template <int MASK>
__device__ __forceinline__ float hx_partner(float v)
{
    if constexpr (MASK == 32)
        return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32u) << 2),
                                                           __float_as_int(v)));
    else  // bit-mask swizzle: and 0x1F, or 0, xor MASK
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (MASK << 10) | 0x1F));
}

// The lower element of a pair takes a + b, the upper a - b (its partner holds a).
template <int MASK>
__device__ __forceinline__ void hx_lane_stage(float4 &v, bool upper)
{
    float p;
    p = hx_partner<MASK>(v.x);
    v.x = upper ? p - v.x : p + v.x;
    p = hx_partner<MASK>(v.y);
    v.y = upper ? p - v.y : p + v.y;
    p = hx_partner<MASK>(v.z);
    v.z = upper ? p - v.z : p + v.z;
    p = hx_partner<MASK>(v.w);
    v.w = upper ? p - v.w : p + v.w;
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

// R stages s .. s+R-1 over buf[0, total) in LDS: groups of 2^R elements at stride 2^s.
template <int NT, int R>
__device__ __forceinline__ void hx_lds_pass(lds_f32 *buf, int total, int s, bool last, float scale)
{
    constexpr int E = 1 << R;
    const int ng = total >> R;
    const int low = (1 << s) - 1;
    for (int q = (int)threadIdx.x; q < ng; q += NT) {
        const int base = ((q >> s) << (s + R)) | (q & low);
        float v[E];
#pragma unroll
        for (int j = 0; j < E; j++)
            v[j] = buf[base + (j << s)];
#pragma unroll
        for (int b = 0; b < R; b++) {
#pragma unroll
            for (int j = 0; j < E; j++) {
                if (!(j & (1 << b))) {
                    const float lo = v[j], hi = v[j | (1 << b)];
                    v[j] = lo + hi;
                    v[j | (1 << b)] = lo - hi;
                }
            }
        }
        if (last) {
#pragma unroll
            for (int j = 0; j < E; j++)
                v[j] *= scale;
        }
#pragma unroll
        for (int j = 0; j < E; j++)
            buf[base + (j << s)] = v[j];
    }
}

// Stages 8 .. L-1 (L > 8) over buf[0, total) in LDS, total a multiple of 2^L, then the scaling.
// Every thread of the workgroup (NT of them) calls it; it starts and ends with a barrier.
template <int NT>
__device__ void hadamard_lds_stages(lds_f32 *buf, int total, int L, float scale)
{
    int s = 8;
    while (s < L) {  // uniform
        const int left = L - s, passes = (left + 3) >> 2, r = (left + passes - 1) / passes;
        const bool last = s + r == L;
        __syncthreads();
        switch (r) {
        case 1: hx_lds_pass<NT, 1>(buf, total, s, last, scale); break;
        case 2: hx_lds_pass<NT, 2>(buf, total, s, last, scale); break;
        case 3: hx_lds_pass<NT, 3>(buf, total, s, last, scale); break;
        default: hx_lds_pass<NT, 4>(buf, total, s, last, scale); break;
        }
        s += r;
    }
    __syncthreads();
}

}  // namespace pn
