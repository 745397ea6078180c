// pn_gemv.hip -- the PN GEMV entry points of the C ABI: argument checks and dispatch.
//
// "PN weight format" (PNX-FORMAT-v0), "Value": y[m, n] = sum_k d * (n_k - z) * x[m, k].
//  * 1-4 tokens: the row-stream kernel of pn_gemv_rows.hip (exact decode of every weight to the
//    integer n - z, one fp32 fma per weight and token; no matrix cores: a matrix-vector product is
//    not a dense contraction).
//  * 5-16 tokens: the matrix-core kernels of pn_gemv_mfma.hip.
//  * Hadamard-rotated activations ("Files that use PN"): the rotation of pn_hadamard_rows into a
//    workspace of the call's stream, then the GEMV above on it -- the same bits as the two calls
//    made by hand. The group variants rotate x once for all their matrices.
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

// The rotated x of the rotated-x calls lives in a workspace per stream: each device keeps a table
// of up to kStreamSlots streams, each with a buffer grown on that stream when a call needs more
// and held for the life of the process. Work on one stream runs in order, so a call reuses its
// stream's buffer with no event and no allocation (a stream-ordered allocation and free per call
// cost about 14 us of host time, and an event recorded per call about 2-4 us of GPU time, more
// than the rotation); different streams never share a buffer. The device's lock is held while a
// call enqueues its launches, so that calls from several host threads on one stream do not
// interleave. A stream's handle names its slot: a destroyed stream's handle is not handed out
// again before the work on it has ended, so a new stream with the same handle may take the slot
// over. When the table is full, on hipStreamPerThread (one handle for a different stream in each
// host thread) and under stream capture (so that the graph records an allocation node of its
// own), a call allocates a temporary on its stream (hipMallocAsync) and frees it there after its
// launches.
constexpr int kStreamSlots = 16;
struct StreamSlot {
    hipStream_t stream = nullptr;
    float *buf = nullptr;
    size_t cap = 0;
    bool used = false;
};
struct Workspace {
    std::mutex mu;
    StreamSlot slot[kStreamSlots];
};
constexpr int kMaxWorkspaceDevices = 64;
static Workspace g_ws[kMaxWorkspaceDevices];

template <typename F>
static int rotate_then(float *xr, const float *x, int64_t M, int64_t K, int64_t B, hipStream_t s,
                       F f)
{
    const int st = pn_hadamard_rows(x, M, K, B, xr, s);
    return st == PN_OK ? f(xr) : st;
}

static int hip_failed()
{
    (void)hipGetLastError();
    return PN_ERR_HIP;
}

// x' = the rotation of x[M, K] in the stream's workspace (else a temporary), then f(x').
template <typename F>
static int with_rotated(const float *x, int64_t M, int64_t K, int64_t B, hipStream_t s, F f)
{
    const size_t bytes = (size_t)(M * K) * sizeof(float);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess)
        return hip_failed();
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxWorkspaceDevices)
        return hip_failed();
    Workspace &w = g_ws[dev];
    std::lock_guard<std::mutex> lk(w.mu);
    StreamSlot *sl = nullptr;
    if (cap == hipStreamCaptureStatusNone && s != hipStreamPerThread) {
        for (StreamSlot &c : w.slot)
            if (c.used && c.stream == s) {
                sl = &c;
                break;
            }
        if (!sl)
            for (StreamSlot &c : w.slot)
                if (!c.used) {
                    c.used = true;
                    c.stream = s;
                    sl = &c;
                    break;
                }
    }
    if (!sl) {
        float *xr = nullptr;
        if (hipMallocAsync(reinterpret_cast<void **>(&xr), bytes, s) != hipSuccess || !xr)
            return hip_failed();
        int st = rotate_then(xr, x, M, K, B, s, f);
        if (hipFreeAsync(xr, s) != hipSuccess && st == PN_OK)
            st = hip_failed();
        return st;
    }
    if (bytes > sl->cap) {
        // every earlier use of the old buffer is on this stream, so it is released after them
        if (sl->buf && hipFreeAsync(sl->buf, s) != hipSuccess)
            return hip_failed();
        sl->buf = nullptr;
        sl->cap = 0;
        const size_t want = (bytes + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
        if (hipMallocAsync(reinterpret_cast<void **>(&sl->buf), want, s) != hipSuccess || !sl->buf) {
            sl->buf = nullptr;
            return hip_failed();
        }
        sl->cap = want;
    }
    return rotate_then(sl->buf, x, M, K, B, s, f);
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
