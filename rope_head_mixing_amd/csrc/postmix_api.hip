// postmix_api.hip -- the C ABI declared in include/postmix.h: argument
// validation (done before any HIP call), device checks and kernel launches on
// the caller's stream.  The library never allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/postmix.h"
#include "postmix_launch.h"
#include "postmix_testing.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_last_error[0] = '\0';
    return PM_OK;
}

// ---- per-device facts (queried once per device) ---------------------------

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];
// test hook (postmix_testing.h): per calling thread, so it never changes
// another thread's results
thread_local int g_force_general = 0;

int check_device(int* n_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PM_ERR_DEVICE, "device index %d out of range", dev);
    int state = g_dev_state[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(PM_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        const bool is950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_dev_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                             std::memory_order_relaxed);
        state = is950 ? 1 : 2;
        g_dev_state[dev].store(state, std::memory_order_release);
        if (!is950)
            return fail(PM_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                        prop.gcnArchName);
    }
    if (state != 1) return fail(PM_ERR_DEVICE, "device %d is not gfx950", dev);
    *n_cu = g_dev_cus[dev].load(std::memory_order_relaxed);
    return PM_OK;
}

// ---- argument checks --------------------------------------------------------

int check_shape(int64_t sq, int32_t nh, int32_t nope, int32_t pe) {
    if (sq < 0) return fail(PM_ERR_SHAPE, "sq must be >= 0 (got %lld)", (long long)sq);
    if (nh < 1 || nh > 128) return fail(PM_ERR_SHAPE, "nh must be in [1, 128] (got %d)", nh);
    if (nope < 0 || nope % 8 != 0)
        return fail(PM_ERR_SHAPE, "nope must be >= 0 and a multiple of 8 (got %d)", nope);
    if (pe < 0 || pe % 16 != 0)
        return fail(PM_ERR_SHAPE, "pe must be >= 0 and a multiple of 16 (got %d)", pe);
    const int64_t d = (int64_t)nope + pe;
    if (d <= 0) return fail(PM_ERR_SHAPE, "nope + pe must be > 0");
    // offsets within a token (head * d + channel, head < 128) fit 31 bits
    if (d > ((int64_t)1 << 24))
        return fail(PM_ERR_SHAPE, "nope + pe must be at most 2^24 (got %lld)", (long long)d);
    // element offsets stay well inside int64 (data-sized grids are split over x and y)
    if (sq > ((int64_t)1 << 40) / ((int64_t)nh * d))
        return fail(PM_ERR_SHAPE, "sq=%lld too large for nh=%d, d=%d", (long long)sq, nh, nope + pe);
    return PM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    const char* name;
    const void* p;
    size_t bytes;
};

bool overlaps(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
    const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
    return a0 < b1 && b0 < a1;
}

int check_no_overlap(const Range* outs, int n_out, const Range* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(PM_ERR_OVERLAP, "output %s overlaps input %s (in-place is not supported)",
                            outs[i].name, ins[j].name);
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(PM_ERR_OVERLAP, "output %s overlaps %s", outs[i].name, outs[j].name);
    }
    return PM_OK;
}

// Checks shared by the forward and the input gradient.
int check_rope_args(const float* rope_cos, const float* rope_sin, int64_t table_rows,
                    const int32_t* positions, int32_t pe) {
    if (pe == 0) return PM_OK;
    if (!rope_cos) return fail(PM_ERR_NULL, "rope_cos is NULL");
    if (!rope_sin) return fail(PM_ERR_NULL, "rope_sin is NULL");
    if (!positions) return fail(PM_ERR_NULL, "positions is NULL");
    if (table_rows < 1) return fail(PM_ERR_SHAPE, "table_rows must be >= 1 when pe > 0");
    if (!aligned16(rope_cos)) return fail(PM_ERR_ALIGN, "rope_cos is not 16-byte aligned");
    if (!aligned16(rope_sin)) return fail(PM_ERR_ALIGN, "rope_sin is not 16-byte aligned");
    if (((uintptr_t)positions & 3u) != 0) return fail(PM_ERR_ALIGN, "positions is not 4-byte aligned");
    return PM_OK;
}

int mix_common(const char* xname, const pm_bf16* X, const pm_bf16* W, const float* rope_cos,
               const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
               int32_t nh, int32_t nope, int32_t pe, const char* oname, pm_bf16* Out, void* stream,
               bool dx) {
    int rc = check_shape(sq, nh, nope, pe);
    if (rc) return rc;
    if (sq == 0) return ok();
    if (!X) return fail(PM_ERR_NULL, "%s is NULL", xname);
    if (!W) return fail(PM_ERR_NULL, "W is NULL");
    if (!Out) return fail(PM_ERR_NULL, "%s is NULL", oname);
    rc = check_rope_args(rope_cos, rope_sin, table_rows, positions, pe);
    if (rc) return rc;
    if (!aligned16(X)) return fail(PM_ERR_ALIGN, "%s is not 16-byte aligned", xname);
    if (!aligned16(Out)) return fail(PM_ERR_ALIGN, "%s is not 16-byte aligned", oname);
    if (((uintptr_t)W & 1u) != 0) return fail(PM_ERR_ALIGN, "W is not 2-byte aligned");
    const size_t act = (size_t)sq * nh * (nope + pe) * sizeof(pm_bf16);
    const size_t tab = pe ? (size_t)table_rows * (pe / 2) * sizeof(float) : 0;
    const Range outs[1] = {{oname, Out, act}};
    const Range ins[5] = {{xname, X, act},
                          {"W", W, (size_t)nh * nh * sizeof(pm_bf16)},
                          {"rope_cos", pe ? rope_cos : nullptr, tab},
                          {"rope_sin", pe ? rope_sin : nullptr, tab},
                          {"positions", pe ? positions : nullptr, (size_t)sq * sizeof(int32_t)}};
    rc = check_no_overlap(outs, 1, ins, 5);
    if (rc) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc) return rc;
    pm::MixArgs a;
    a.X = X;
    a.W = W;
    a.rcos = rope_cos;
    a.rsin = rope_sin;
    a.table_rows = table_rows;
    a.positions = positions;
    a.sq = sq;
    a.nh = nh;
    a.nope = nope;
    a.pe = pe;
    a.Out = Out;
    a.n_cu = n_cu;
    a.waves_per_cu = 16;
    a.force_general = g_force_general != 0;
    hipError_t e = pm::launch_mix(a, dx, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

__global__ void zero_fill_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

}  // namespace

extern "C" {

int postmix_fwd(const pm_bf16* O, const pm_bf16* W, const float* rope_cos, const float* rope_sin,
                int64_t table_rows, const int32_t* positions, int64_t sq, int32_t nh, int32_t nope,
                int32_t pe, pm_bf16* Y, void* stream) {
    return mix_common("O", O, W, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe, "Y",
                      Y, stream, false);
}

int postmix_bwd_dx(const pm_bf16* dY, const pm_bf16* W, const float* rope_cos,
                   const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
                   int32_t nh, int32_t nope, int32_t pe, pm_bf16* dO, void* stream) {
    return mix_common("dY", dY, W, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe,
                      "dO", dO, stream, true);
}

size_t postmix_bwd_dw_workspace_bytes(int64_t sq, int32_t nh, int32_t nope, int32_t pe) {
    char saved[sizeof g_last_error];
    memcpy(saved, g_last_error, sizeof saved);
    const int rc = check_shape(sq, nh, nope, pe);
    memcpy(g_last_error, saved, sizeof saved);  // a size query leaves the message alone
    if (rc || sq == 0) return 0;
    int64_t blocks = pm::dw_plan(sq, nh, nope, pe).partials();
    if (pm::bwd_fused_applies(nh, nope, pe)) {  // postmix_bwd's single pass has its own blocks
        const int64_t fb = pm::bwd_fused_plan(sq, nh, nope, pe).partials();
        if (fb > blocks) blocks = fb;
    }
    const size_t bytes = (size_t)blocks * nh * nh * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

int postmix_bwd_dw(const pm_bf16* dY, const pm_bf16* O, const float* rope_cos,
                   const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
                   int32_t nh, int32_t nope, int32_t pe, float* dW, void* workspace,
                   size_t workspace_bytes, void* stream) {
    int rc = check_shape(sq, nh, nope, pe);
    if (rc) return rc;
    if (!dW) return fail(PM_ERR_NULL, "dW is NULL");
    if (((uintptr_t)dW & 3u) != 0) return fail(PM_ERR_ALIGN, "dW is not 4-byte aligned");
    const size_t wbytes = (size_t)nh * nh * sizeof(float);
    if (sq == 0) {
        // an empty sum: dW = 0
        int n_cu = 0;
        rc = check_device(&n_cu);
        if (rc) return rc;
        const int64_t n = (int64_t)nh * nh;
        hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           (hipStream_t)stream, dW, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    if (!dY) return fail(PM_ERR_NULL, "dY is NULL");
    if (!O) return fail(PM_ERR_NULL, "O is NULL");
    rc = check_rope_args(rope_cos, rope_sin, table_rows, positions, pe);
    if (rc) return rc;
    if (!aligned16(dY)) return fail(PM_ERR_ALIGN, "dY is not 16-byte aligned");
    if (!aligned16(O)) return fail(PM_ERR_ALIGN, "O is not 16-byte aligned");
    const size_t need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe);
    if (need > 0 && !workspace) return fail(PM_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(PM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PM_ERR_ALIGN, "workspace is not 16-byte aligned");
    const size_t act = (size_t)sq * nh * (nope + pe) * sizeof(pm_bf16);
    const size_t tab = pe ? (size_t)table_rows * (pe / 2) * sizeof(float) : 0;
    const Range outs[2] = {{"dW", dW, wbytes}, {"workspace", workspace, need}};
    const Range ins[5] = {{"dY", dY, act},
                          {"O", O, act},
                          {"rope_cos", pe ? rope_cos : nullptr, tab},
                          {"rope_sin", pe ? rope_sin : nullptr, tab},
                          {"positions", pe ? positions : nullptr, (size_t)sq * sizeof(int32_t)}};
    rc = check_no_overlap(outs, 2, ins, 5);
    if (rc) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc) return rc;
    pm::DwArgs a;
    a.dY = dY;
    a.O = O;
    a.rcos = rope_cos;
    a.rsin = rope_sin;
    a.table_rows = table_rows;
    a.positions = positions;
    a.sq = sq;
    a.nh = nh;
    a.nope = nope;
    a.pe = pe;
    a.dW = dW;
    a.partials = (float*)workspace;
    a.force_general = g_force_general != 0;
    hipError_t e = pm::launch_dw(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// ---- the static scratch of postmix_bwd_noalloc -------------------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device (with
// that device current) by hipGetSymbolAddress, and only that address is
// passed to kernels.
static constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on that device).
int scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PM_ERR_DEVICE, "device index %d out of range", dev);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PM_OK;
}

// postmix_bwd, with the partials either in the caller's workspace or
// (use_scratch) in the library's static scratch.
int bwd_common(const pm_bf16* dY, const pm_bf16* O, const pm_bf16* W, const float* rope_cos,
               const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
               int32_t nh, int32_t nope, int32_t pe, pm_bf16* dO, float* dW, void* workspace,
               size_t workspace_bytes, void* stream, bool use_scratch) {
    int rc = check_shape(sq, nh, nope, pe);
    if (rc) return rc;
    if (!dW) return fail(PM_ERR_NULL, "dW is NULL");
    if (((uintptr_t)dW & 3u) != 0) return fail(PM_ERR_ALIGN, "dW is not 4-byte aligned");
    if (sq == 0) {
        // no tokens: dO is empty and dW is an empty sum (no partials)
        return postmix_bwd_dw(dY, O, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe, dW,
                              nullptr, 0, stream);
    }
    if (!dY) return fail(PM_ERR_NULL, "dY is NULL");
    if (!O) return fail(PM_ERR_NULL, "O is NULL");
    if (!W) return fail(PM_ERR_NULL, "W is NULL");
    if (!dO) return fail(PM_ERR_NULL, "dO is NULL");
    rc = check_rope_args(rope_cos, rope_sin, table_rows, positions, pe);
    if (rc) return rc;
    if (!aligned16(dY)) return fail(PM_ERR_ALIGN, "dY is not 16-byte aligned");
    if (!aligned16(O)) return fail(PM_ERR_ALIGN, "O is not 16-byte aligned");
    if (!aligned16(dO)) return fail(PM_ERR_ALIGN, "dO is not 16-byte aligned");
    if (((uintptr_t)W & 1u) != 0) return fail(PM_ERR_ALIGN, "W is not 2-byte aligned");
    const size_t need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe);
    if (use_scratch) {
        if (need > kScratchBytes)
            return fail(PM_ERR_WORKSPACE,
                        "the weight-gradient partials of this shape need %zu bytes, more than the %zu "
                        "bytes of postmix_bwd_noalloc's static scratch; call postmix_bwd with a workspace",
                        need, kScratchBytes);
    } else {
        if (need > 0 && !workspace) return fail(PM_ERR_NULL, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(PM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (!aligned16(workspace)) return fail(PM_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    const size_t act = (size_t)sq * nh * (nope + pe) * sizeof(pm_bf16);
    const size_t tab = pe ? (size_t)table_rows * (pe / 2) * sizeof(float) : 0;
    const Range outs[3] = {{"dO", dO, act}, {"dW", dW, (size_t)nh * nh * sizeof(float)},
                           {"workspace", use_scratch ? nullptr : workspace, need}};
    const Range ins[6] = {{"dY", dY, act},
                          {"O", O, act},
                          {"W", W, (size_t)nh * nh * sizeof(pm_bf16)},
                          {"rope_cos", pe ? rope_cos : nullptr, tab},
                          {"rope_sin", pe ? rope_sin : nullptr, tab},
                          {"positions", pe ? positions : nullptr, (size_t)sq * sizeof(int32_t)}};
    rc = check_no_overlap(outs, 3, ins, 6);
    if (rc) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc) return rc;
    if (use_scratch) {
        rc = scratch_for_current_device(&workspace);
        if (rc) return rc;
    }
    pm::MixArgs mx;
    mx.X = dY;
    mx.W = W;
    mx.rcos = rope_cos;
    mx.rsin = rope_sin;
    mx.table_rows = table_rows;
    mx.positions = positions;
    mx.sq = sq;
    mx.nh = nh;
    mx.nope = nope;
    mx.pe = pe;
    mx.Out = dO;
    mx.n_cu = n_cu;
    mx.waves_per_cu = 16;
    mx.force_general = g_force_general != 0;
    pm::DwArgs a;
    a.dY = dY;
    a.O = O;
    a.rcos = rope_cos;
    a.rsin = rope_sin;
    a.table_rows = table_rows;
    a.positions = positions;
    a.sq = sq;
    a.nh = nh;
    a.nope = nope;
    a.pe = pe;
    a.dW = dW;
    a.partials = (float*)workspace;
    a.force_general = mx.force_general;
    hipError_t e;
    // with nh = 64 or 128 and a W that is not 16-byte aligned, postmix_bwd_dx
    // runs the general kernel (the tiled one reads W with 16-byte loads), so
    // the fused pass, whose dO is the tiled kernel's, is not used there
    const bool w_ok = ((uintptr_t)W & 15u) == 0 || (nh != 64 && nh != 128);
    if (!mx.force_general && w_ok && pm::bwd_fused_applies(nh, nope, pe)) {
        e = pm::launch_bwd_fused(mx, a, (hipStream_t)stream);
    } else {
        e = pm::launch_mix(mx, true, (hipStream_t)stream);
        if (e == hipSuccess) e = pm::launch_dw(a, (hipStream_t)stream);
    }
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int postmix_bwd(const pm_bf16* dY, const pm_bf16* O, const pm_bf16* W, const float* rope_cos,
                const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
                int32_t nh, int32_t nope, int32_t pe, pm_bf16* dO, float* dW, void* workspace,
                size_t workspace_bytes, void* stream) {
    return bwd_common(dY, O, W, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe, dO, dW,
                      workspace, workspace_bytes, stream, false);
}

int postmix_bwd_noalloc(const pm_bf16* dY, const pm_bf16* O, const pm_bf16* W, const float* rope_cos,
                        const float* rope_sin, int64_t table_rows, const int32_t* positions, int64_t sq,
                        int32_t nh, int32_t nope, int32_t pe, pm_bf16* dO, float* dW, void* stream) {
    return bwd_common(dY, O, W, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe, dO, dW,
                      nullptr, 0, stream, true);
}

int postmix_rope_apply(const pm_bf16* X, const float* rope_cos, const float* rope_sin,
                       int64_t table_rows, const int32_t* positions, int64_t sq, int32_t nh,
                       int32_t nope, int32_t pe, int32_t direction, pm_bf16* Out, void* stream) {
    int rc = check_shape(sq, nh, nope, pe);
    if (rc) return rc;
    if (direction != 1 && direction != -1) return fail(PM_ERR_SHAPE, "direction must be +1 or -1");
    if (sq == 0) return ok();
    if (!X) return fail(PM_ERR_NULL, "X is NULL");
    if (!Out) return fail(PM_ERR_NULL, "Out is NULL");
    rc = check_rope_args(rope_cos, rope_sin, table_rows, positions, pe);
    if (rc) return rc;
    if (!aligned16(X)) return fail(PM_ERR_ALIGN, "X is not 16-byte aligned");
    if (!aligned16(Out)) return fail(PM_ERR_ALIGN, "Out is not 16-byte aligned");
    const size_t act = (size_t)sq * nh * (nope + pe) * sizeof(pm_bf16);
    const size_t tab = pe ? (size_t)table_rows * (pe / 2) * sizeof(float) : 0;
    const Range outs[1] = {{"Out", Out, act}};
    const Range ins[4] = {{"X", X, act},
                          {"rope_cos", pe ? rope_cos : nullptr, tab},
                          {"rope_sin", pe ? rope_sin : nullptr, tab},
                          {"positions", pe ? positions : nullptr, (size_t)sq * sizeof(int32_t)}};
    rc = check_no_overlap(outs, 1, ins, 4);
    if (rc) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc) return rc;
    hipError_t e = pm::launch_rope_apply(X, rope_cos, rope_sin, table_rows, positions, sq, nh, nope, pe,
                                         direction, Out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int postmix_kv_index_remap(const int32_t* idx, int64_t rows, int64_t sq, int64_t topk,
                           int64_t seqlen_kv, int32_t pad_value, int32_t* out, void* stream) {
    if (rows < 0) return fail(PM_ERR_SHAPE, "rows must be >= 0");
    if (sq < 1) return fail(PM_ERR_SHAPE, "sq must be >= 1");
    if (rows % sq != 0) return fail(PM_ERR_SHAPE, "rows (%lld) must be a multiple of sq (%lld)",
                                    (long long)rows, (long long)sq);
    if (topk < 0) return fail(PM_ERR_SHAPE, "topk must be >= 0");
    if (seqlen_kv < 0) return fail(PM_ERR_SHAPE, "seqlen_kv must be >= 0");
    const int64_t batches = rows / sq;
    if (batches > 0 && seqlen_kv > (int64_t)INT32_MAX / batches)
        return fail(PM_ERR_SHAPE, "batches * seqlen_kv = %lld * %lld exceeds the int32 index range",
                    (long long)batches, (long long)seqlen_kv);
    if (rows > ((int64_t)1 << 40) / (topk > 0 ? topk : 1))
        return fail(PM_ERR_SHAPE, "table of %lld x %lld entries is too large", (long long)rows, (long long)topk);
    if (rows == 0 || topk == 0) return ok();
    if (!idx) return fail(PM_ERR_NULL, "idx is NULL");
    if (!out) return fail(PM_ERR_NULL, "out is NULL");
    if (((uintptr_t)idx & 3u) != 0) return fail(PM_ERR_ALIGN, "idx is not 4-byte aligned");
    if (((uintptr_t)out & 3u) != 0) return fail(PM_ERR_ALIGN, "out is not 4-byte aligned");
    const size_t bytes = (size_t)rows * topk * sizeof(int32_t);
    if (out != idx) {  // in place is fine (each element is read, then written, by one thread)
        const Range outs[1] = {{"out", out, bytes}};
        const Range ins[1] = {{"idx", idx, bytes}};
        int rc = check_no_overlap(outs, 1, ins, 1);
        if (rc) return rc;
    }
    int n_cu = 0;
    int rc = check_device(&n_cu);
    if (rc) return rc;
    hipError_t e = pm::launch_kv_remap(idx, rows, sq, topk, seqlen_kv, pad_value, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int postmix_rope_table(double theta, int32_t pe, int64_t table_rows, float* cos_out,
                       float* sin_out, void* stream) {
    if (!(theta > 0.0)) return fail(PM_ERR_SHAPE, "theta must be > 0");
    if (pe <= 0 || pe % 16 != 0) return fail(PM_ERR_SHAPE, "pe must be a positive multiple of 16 (got %d)", pe);
    if (table_rows < 0) return fail(PM_ERR_SHAPE, "table_rows must be >= 0");
    if (table_rows == 0) return ok();
    if (!cos_out) return fail(PM_ERR_NULL, "cos_out is NULL");
    if (!sin_out) return fail(PM_ERR_NULL, "sin_out is NULL");
    if (!aligned16(cos_out)) return fail(PM_ERR_ALIGN, "cos_out is not 16-byte aligned");
    if (!aligned16(sin_out)) return fail(PM_ERR_ALIGN, "sin_out is not 16-byte aligned");
    const size_t tab = (size_t)table_rows * (pe / 2) * sizeof(float);
    const Range outs[2] = {{"cos_out", cos_out, tab}, {"sin_out", sin_out, tab}};
    int rc = check_no_overlap(outs, 2, nullptr, 0);
    if (rc) return rc;
    int n_cu = 0;
    rc = check_device(&n_cu);
    if (rc) return rc;
    hipError_t e = pm::launch_rope_table(theta, pe, table_rows, cos_out, sin_out, n_cu,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return fail(PM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char* postmix_status_string(int status) {
    switch (status) {
        case PM_OK: return "ok";
        case PM_ERR_NULL: return "null pointer";
        case PM_ERR_SHAPE: return "bad shape";
        case PM_ERR_ALIGN: return "misaligned pointer";
        case PM_ERR_OVERLAP: return "output overlaps input";
        case PM_ERR_WORKSPACE: return "workspace too small";
        case PM_ERR_DEVICE: return "device is not gfx950";
        case PM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* postmix_last_error(void) { return g_last_error; }

int pm_testing_set_general_kernels(int enable) {
    const int prev = g_force_general;
    g_force_general = enable ? 1 : 0;
    return prev;
}

}  // extern "C"
