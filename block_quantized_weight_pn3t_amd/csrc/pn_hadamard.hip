// pn_hadamard.hip -- the Hadamard rotation of the activations as its own launch
// ("PN weight format", "Files that use PN"; the reading and the arithmetic are stated in
// pn_hadamard.h). pn_gemv_hadamard and pn_gemv_group_hadamard run it into a per-stream
// workspace ahead of the GEMV, and pn_gemv_hadamard_noalloc into a static device array.
#include "pn_common.h"
#include "pn_hadamard.h"

namespace pn {

constexpr int kHxThreads = 256;
constexpr int kHxChunk = 1024;  // elements per workgroup step when slices exceed one wave's 256

__device__ __forceinline__ float4 hx_load4(const float *p, int vec4)
{
    if (vec4)
        return *reinterpret_cast<const float4 *>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ void hx_store4(float *p, float4 v, int vec4)
{
    if (vec4) {
        *reinterpret_cast<float4 *>(p) = v;
    } else {
        p[0] = v.x;
        p[1] = v.y;
        p[2] = v.z;
        p[3] = v.w;
    }
}

// Slices of at most 256 elements: each wave transforms its own 256 elements in registers.
// Starts are multiples of 256 float4 per workgroup step, so every wave covers whole slices.
__global__ void __launch_bounds__(kHxThreads)
hadamard_wave_kernel(const float *x, float *out, int64_t nq, int L, float scale, int vin, int vout)
{
    const int64_t stride = (int64_t)gridDim.x * kHxThreads;
    for (int64_t q0 = (int64_t)blockIdx.x * kHxThreads; q0 < nq; q0 += stride) {
        const int64_t q = q0 + threadIdx.x;
        float4 v = hx_load4(x + 4 * min(q, nq - 1), vin);
        hadamard_wave(v, L, scale);
        if (q < nq)
            hx_store4(out + 4 * q, v, vout);
    }
}

// Slices of 512 or more elements: a workgroup takes chunks of C elements (C a multiple of the
// slice, at most 16384), runs stages 0-7 per wave into LDS and the rest in LDS, then writes the
// chunk back. The whole chunk is read before any of it is written, so out may equal x.
__global__ void __launch_bounds__(kHxThreads)
hadamard_lds_kernel(const float *x, float *out, int64_t total, int C, int L, float scale, int vin,
                    int vout)
{
    extern __shared__ float4 hx_smem[];
    lds_f32 *buf = (lds_f32 *)(float *)hx_smem;
    for (int64_t c0 = (int64_t)blockIdx.x * C; c0 < total; c0 += (int64_t)gridDim.x * C) {
        const int n = (int)min<int64_t>(C, total - c0);  // a multiple of the slice (>= 512)
        const int nq = n >> 2;                           // a multiple of 128
        for (int q0 = 0; q0 < nq; q0 += kHxThreads) {
            const int q = q0 + (int)threadIdx.x;
            float4 v = hx_load4(x + c0 + 4 * min(q, nq - 1), vin);
            hadamard_wave(v, L, scale);
            if (q < nq) {
                buf[4 * q + 0] = v.x;
                buf[4 * q + 1] = v.y;
                buf[4 * q + 2] = v.z;
                buf[4 * q + 3] = v.w;
            }
        }
        hadamard_lds_stages<kHxThreads>(buf, n, L, scale);
        for (int q = (int)threadIdx.x; q < nq; q += kHxThreads)
            hx_store4(out + c0 + 4 * q,
                      make_float4(buf[4 * q], buf[4 * q + 1], buf[4 * q + 2], buf[4 * q + 3]), vout);
        __syncthreads();  // the next chunk overwrites buf
    }
}

// log2 of a valid slice size (a power of two, 2 <= B <= 16384, dividing K), else -1.
int hadamard_log(int64_t B, int64_t K)
{
    if (B < 2 || B > (int64_t(1) << kHadamardMaxLog) || (B & (B - 1)) || K <= 0 || K % B)
        return -1;
    int L = 0;
    while ((int64_t(1) << L) < B)
        L++;
    return L;
}

float hadamard_scale(int L)
{
    return (float)(1.0 / sqrt((double)(int64_t(1) << L)));
}

static int num_cus_hx() { return device_cus(); }

}  // namespace pn

using namespace pn;

extern "C" int pn_hadamard_rows(const float *x, int64_t M, int64_t K, int64_t B, float *out,
                                void *stream)
{
    if (M < 0 || K <= 0 || K % 4)
        return PN_ERR_SHAPE;
    const int L = hadamard_log(B, K);
    if (L < 0)
        return PN_ERR_HADAMARD;
    if (M == 0)
        return PN_OK;
    if (!x || !out)
        return PN_ERR_NULL;
    if (!aligned(x, 4) || !aligned(out, 4))
        return PN_ERR_ALIGN;
    if (M * K / 4 >= (int64_t(1) << 40))
        return PN_ERR_SHAPE;
    int st = check_device();
    if (st != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const float scale = hadamard_scale(L);
    const int vin = aligned(x, 16) ? 1 : 0, vout = aligned(out, 16) ? 1 : 0;
    const int64_t total = M * K;  // a multiple of B and of 4
    if (L <= 8) {
        const int64_t nq = total / 4;
        const int grid = (int)std::min<int64_t>((nq + kHxThreads - 1) / kHxThreads,
                                                (int64_t)num_cus_hx() * 8);
        hipLaunchKernelGGL(hadamard_wave_kernel, dim3((unsigned)grid), dim3(kHxThreads), 0, s, x,
                           out, nq, L, scale, vin, vout);
    } else {
        const int C = (int)std::max<int64_t>(B, kHxChunk);
        const int64_t chunks = (total + C - 1) / C;
        const int grid = (int)std::min<int64_t>(chunks, (int64_t)num_cus_hx() * 4);
        const size_t lds = (size_t)C * sizeof(float);
        if (!lds_limit_once<hadamard_lds_kernel>((int)((size_t(1) << kHadamardMaxLog) * sizeof(float))))
            return PN_ERR_HIP;
        hipLaunchKernelGGL(hadamard_lds_kernel, dim3((unsigned)grid), dim3(kHxThreads), lds, s, x,
                           out, total, C, L, scale, vin, vout);
    }
    return launch_status();
}
