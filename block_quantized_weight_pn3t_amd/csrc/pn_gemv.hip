// pn_gemv.hip -- the PN GEMV entry points of the C ABI: argument checks and dispatch.
//
// "PN weight format" (PNX-FORMAT-v0), "Value": y[m, n] = sum_k d * (n_k - z) * x[m, k].
//  * 1-4 tokens: the row-stream kernel of pn_gemv_rows.hip (exact decode of every weight to the
//    integer n - z, one fp32 fma per weight and token; no matrix cores: a matrix-vector product is
//    not a dense contraction).
//  * 5-16 tokens: the matrix-core kernels of pn_gemv_mfma.hip.
//  * Hadamard-rotated activations ("Files that use PN"): the rotation of pn_hadamard_rows into a
//    stream-ordered temporary, then the GEMV above on it -- the same bits as the two calls made by
//    hand. The group variants rotate x once for all their matrices.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "pn_common.h"

namespace pn {

int launch_vec_group(int type, const GroupPart *gp, int count, int64_t K, const float *x,
                     int64_t M, hipStream_t s);
int launch_vec(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
               float *y, hipStream_t s);
int launch_mfma(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int M, float *y,
                int cus, hipStream_t s);
int hadamard_log(int64_t B, int64_t K);

static int dispatch(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
                    float *y, hipStream_t s)
{
    if (M <= 4)
        return launch_vec(type, W, N, K, x, M, y, s);
    return launch_mfma(type, W, N, K, x, (int)M, y, device_cus(), s);
}

static int check_part(const pn_gemv_part &p, int64_t K)
{
    if (p.type != PN_TYPE_PN3T && p.type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (p.N < 0 || pn_row_bytes(p.type, K) == 0)
        return PN_ERR_SHAPE;
    return PN_OK;
}

// Arguments of a group call: every part's type and shape, then (for parts with rows) pointers and
// alignment, then x. any = some part has rows.
static int check_group(const pn_gemv_part *parts, int count, int64_t K, const float *x,
                       bool &any)
{
    any = false;
    for (int i = 0; i < count; i++) {
        const int st = check_part(parts[i], K);
        if (st != PN_OK)
            return st;
    }
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
    if (any && !x)
        return PN_ERR_NULL;
    if (any && !aligned(x, 4))
        return PN_ERR_ALIGN;
    return PN_OK;
}

static int run_group(const pn_gemv_part *parts, int count, int64_t K, const float *x, int64_t M,
                     hipStream_t s)
{
    // at 1-4 tokens the parts of each type run as one launch where the shapes allow it (the
    // parts' outputs are independent, so the order of the launches does not matter)
    bool done[PN_GEMV_GROUP_MAX_PARTS] = {};
    if (M <= 4) {
        // parts of both types: one launch over all of them where the shapes allow it
        GroupPart all[PN_GEMV_GROUP_MAX_PARTS];
        int n = 0;
        bool t3 = false, t4 = false;
        for (int i = 0; i < count; i++)
            if (parts[i].N > 0) {
                t3 = t3 || parts[i].type == PN_TYPE_PN3T;
                t4 = t4 || parts[i].type == PN_TYPE_PN4T;
                all[n++] = GroupPart{(const uint8_t *)parts[i].W, parts[i].N, parts[i].y,
                                     parts[i].type};
            }
        if (t3 && t4) {
            const int st = launch_vec_group(-1, all, n, K, x, M, s);
            if (st != 1)
                return st;
        }
        for (int type : {PN_TYPE_PN3T, PN_TYPE_PN4T}) {
            GroupPart gp[PN_GEMV_GROUP_MAX_PARTS];
            int idx[PN_GEMV_GROUP_MAX_PARTS];
            int n = 0;
            for (int i = 0; i < count; i++)
                if (parts[i].N > 0 && parts[i].type == type) {
                    idx[n] = i;
                    gp[n++] = GroupPart{(const uint8_t *)parts[i].W, parts[i].N, parts[i].y, type};
                }
            if (n < 2)
                continue;
            const int st = launch_vec_group(type, gp, n, K, x, M, s);
            if (st == 1)
                continue;  // shapes it cannot group: one launch per part below
            if (st != PN_OK)
                return st;
            for (int j = 0; j < n; j++)
                done[idx[j]] = true;
        }
    }
    for (int i = 0; i < count; i++) {
        const pn_gemv_part &p = parts[i];
        if (p.N == 0 || done[i])
            continue;
        const int st = dispatch(p.type, (const uint8_t *)p.W, p.N, K, x, M, p.y, s);
        if (st != PN_OK)
            return st;
    }
    return PN_OK;
}

// The stream-ordered temporaries of the rotated-x calls come from a memory pool of the library's
// own per device that keeps what is freed (release threshold at its maximum): after the first
// call the allocation is a reuse inside the pool, not a trip to the system, which the device's
// default pool (threshold 0) makes on every call. Each device keeps up to its largest temporary
// for the life of the process. Under stream capture the default pool's allocation is used, which
// a graph records as its own allocation node.
constexpr int kMaxPoolDevices = 64;
static std::atomic<hipMemPool_t> g_pool[kMaxPoolDevices];
static std::mutex g_pool_mu;

static hipMemPool_t temp_pool()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxPoolDevices)
        return nullptr;
    hipMemPool_t p = g_pool[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lk(g_pool_mu);
    p = g_pool[dev].load(std::memory_order_relaxed);
    if (!p) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        uint64_t keep = ~0ull;
        if (hipMemPoolCreate(&p, &props) != hipSuccess || !p ||
            hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_pool[dev].store(p, std::memory_order_release);
    }
    return p;
}

// x' = the rotation of x[M, K] in a stream-ordered temporary, then f(x'); the temporary is
// released on the same stream after f's launches.
template <typename F>
static int with_rotated(const float *x, int64_t M, int64_t K, int64_t B, hipStream_t s, F f)
{
    const size_t bytes = (size_t)(M * K) * sizeof(float);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
        (void)hipGetLastError();
        return PN_ERR_HIP;
    }
    hipMemPool_t pool = nullptr;
    if (cap == hipStreamCaptureStatusNone && !(pool = temp_pool()))
        return PN_ERR_HIP;
    float *xr = nullptr;
    const hipError_t e = pool ? hipMallocFromPoolAsync(reinterpret_cast<void **>(&xr), bytes, pool, s)
                              : hipMallocAsync(reinterpret_cast<void **>(&xr), bytes, s);
    if (e != hipSuccess || !xr) {
        (void)hipGetLastError();
        return PN_ERR_HIP;
    }
    int st = pn_hadamard_rows(x, M, K, B, xr, s);
    if (st == PN_OK)
        st = f(xr);
    if (hipFreeAsync(xr, s) != hipSuccess && st == PN_OK)
        st = PN_ERR_HIP;
    return st;
}

// ---- the rotated x of pn_gemv_hadamard_noalloc: a file-scope device array --------------------
// Each GPU the library runs on holds its own copy for the life of the process. In host code the
// array's name is a host-side stand-in, not a device address: the address is looked up once per
// device (with that device current) and only that address is handed to kernels.
__device__ __align__(256) float scratch[PN_NOALLOC_MAX_FLOATS];

constexpr int kMaxScratchDevices = 64;
static std::atomic<float *> g_scratch[kMaxScratchDevices];
static std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, or nullptr (the caller reports
// PN_ERR_HIP).
static float *scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return nullptr;
    float *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return nullptr;
        }
        p = static_cast<float *>(q);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
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
    if (M < 0 || M > PN_GEMV_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (N == 0 || M == 0)
        return PN_OK;
    if (!W || !x || !y)
        return PN_ERR_NULL;
    if (!aligned(W, 2) || !aligned(x, 4) || !aligned(y, 4))
        return PN_ERR_ALIGN;
    const int st = check_device();
    if (st != PN_OK)
        return st;
    return dispatch(type, (const uint8_t *)W, N, K, x, M, y, (hipStream_t)stream);
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
    bool any = false;
    int st = check_group(parts, count, K, x, any);
    if (st != PN_OK || M == 0 || !any)
        return st;
    if ((st = check_device()) != PN_OK)
        return st;
    return run_group(parts, count, K, x, M, (hipStream_t)stream);
}

extern "C" int pn_gemv_hadamard(int type, const void *W, int64_t N, int64_t K, const float *x,
                                int64_t M, int64_t B, float *y, void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (N < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_GEMV_HADAMARD_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (hadamard_log(B, K) < 0)
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
    return with_rotated(x, M, K, B, s, [&](const float *xr) {
        return dispatch(type, (const uint8_t *)W, N, K, xr, M, y, s);
    });
}

extern "C" int pn_gemv_hadamard_noalloc(int type, const void *W, int64_t N, int64_t K,
                                        const float *x, int64_t M, int64_t B, float *y,
                                        void *stream)
{
    if (type != PN_TYPE_PN3T && type != PN_TYPE_PN4T)
        return PN_ERR_TYPE;
    if (N < 0 || pn_row_bytes(type, K) == 0)
        return PN_ERR_SHAPE;
    if (M < 0 || M > PN_GEMV_HADAMARD_MAX_TOKENS)
        return PN_ERR_TOKENS;
    if (hadamard_log(B, K) < 0)
        return PN_ERR_HADAMARD;
    if (M * K > PN_NOALLOC_MAX_FLOATS)
        return PN_ERR_SHAPE;
    if (N == 0 || M == 0)
        return PN_OK;
    if (!W || !x || !y)
        return PN_ERR_NULL;
    if (!aligned(W, 2) || !aligned(x, 4) || !aligned(y, 4))
        return PN_ERR_ALIGN;
    int st = check_device();
    if (st != PN_OK)
        return st;
    float *xr = scratch_ptr();
    if (!xr)
        return PN_ERR_HIP;
    hipStream_t s = (hipStream_t)stream;
    st = pn_hadamard_rows(x, M, K, B, xr, s);
    if (st != PN_OK)
        return st;
    return dispatch(type, (const uint8_t *)W, N, K, xr, M, y, s);
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
        const int st = check_part(parts[i], K);
        if (st != PN_OK)
            return st;
    }
    if (hadamard_log(B, K) < 0)
        return PN_ERR_HADAMARD;
    bool any = false;
    int st = check_group(parts, count, K, x, any);
    if (st != PN_OK || M == 0 || !any)
        return st;
    if ((st = check_device()) != PN_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    return with_rotated(x, M, K, B, s,
                        [&](const float *xr) { return run_group(parts, count, K, xr, M, s); });
}
