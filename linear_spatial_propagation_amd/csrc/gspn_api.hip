// gspn_api.hip -- C ABI of libgspn: argument validation and kernel dispatch.
//
// The operator and every convention are specified in include/gspn.h.
#include <hip/hip_runtime.h>

#include <rocblas/rocblas.h>

#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gspn_kernels.h"
#include "../../include/gspn.h"

namespace {

thread_local char g_last_error[512] = "";

void set_error(const char* what, hipError_t e) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}
void set_error_text(const char* text) { snprintf(g_last_error, sizeof(g_last_error), "%s", text); }

int popcount4(uint32_t d) { return (int)((d & 1u) + ((d >> 1) & 1u) + ((d >> 2) & 1u) + ((d >> 3) & 1u)); }

// Host-side checks of sizes and options (no pointers).
int check_sizes(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                int32_t cpw, int32_t dtype) {
    if (B <= 0 || C <= 0 || H <= 0 || W <= 0) return GSPN_ERR_SHAPE;
    if (H > GSPN_MAX_SIDE || W > GSPN_MAX_SIDE) return GSPN_ERR_SHAPE;
    // one workgroup per slice (or per slice and direction) of 256 threads:
    // the launch must stay below 2^32 work-items
    if (B > (1LL << 22) / C) return GSPN_ERR_SHAPE;                     // B*C <= 2^22
    if (B * C > (int64_t)(1LL << 62) / (H * W * 4 * 4)) return GSPN_ERR_SHAPE;
    if (dirs == 0 || (dirs & ~15u)) return GSPN_ERR_DIRS;
    if (groups < 1) return GSPN_ERR_GROUPS;
    if ((dirs & 3u) && H % groups) return GSPN_ERR_GROUPS;
    if ((dirs & 12u) && W % groups) return GSPN_ERR_GROUPS;
    if (cpw < 1 || C % cpw) return GSPN_ERR_CPW;
    if (dtype != GSPN_F32 && dtype != GSPN_BF16) return GSPN_ERR_DTYPE;
    return GSPN_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

int auto_path(int64_t H, int64_t W) {
    return (H <= gspn::kFusedMaxSide && W <= gspn::kFusedMaxSide) ? GSPN_PATH_FUSED : GSPN_PATH_GENERAL;
}

}  // namespace

extern "C" {

int gspn_version(void) { return GSPN_VERSION; }

const char* gspn_last_error(void) { return g_last_error; }

const char* gspn_status_string(int status) {
    switch (status) {
        case GSPN_OK: return "GSPN_OK";
        case GSPN_ERR_NULL: return "GSPN_ERR_NULL: a pointer is null";
        case GSPN_ERR_SHAPE: return "GSPN_ERR_SHAPE: a size is <= 0, above GSPN_MAX_SIDE, or overflows";
        case GSPN_ERR_DIRS: return "GSPN_ERR_DIRS: dirs must be a non-zero mask of bits 0..3";
        case GSPN_ERR_GROUPS: return "GSPN_ERR_GROUPS: groups must be >= 1 and divide each scanned side";
        case GSPN_ERR_CPW: return "GSPN_ERR_CPW: ch_per_weight must be >= 1 and divide C";
        case GSPN_ERR_DTYPE: return "GSPN_ERR_DTYPE: unknown dtype";
        case GSPN_ERR_ALIGN: return "GSPN_ERR_ALIGN: a base pointer is not 16-byte aligned";
        case GSPN_ERR_ALIAS: return "GSPN_ERR_ALIAS: an output overlaps an input or another output";
        case GSPN_ERR_HIP: return "GSPN_ERR_HIP: a HIP call failed (see gspn_last_error)";
        case GSPN_ERR_PATH: return "GSPN_ERR_PATH: unknown path, or the path cannot run this shape";
        case GSPN_ERR_FLAGS: return "GSPN_ERR_FLAGS: unknown bit in flags";
        case GSPN_ERR_SCRATCH: return "GSPN_ERR_SCRATCH: the shape's workspace exceeds the static scratch";
        default: return "unknown GSPN status";
    }
}

int gspn_select_path(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                     int32_t ch_per_weight, int32_t dtype) {
    const int rc = check_sizes(B, C, H, W, dirs, groups, ch_per_weight, dtype);
    if (rc) return rc;
    const int path = auto_path(H, W);
    if (path == GSPN_PATH_GENERAL) {
        gspn::ScanArgs a{};
        a.B = (int)B; a.C = (int)C; a.H = (int)H; a.W = (int)W;
        a.dirs = dirs; a.groups = groups; a.cpw = ch_per_weight; a.bf16 = dtype == GSPN_BF16;
        if (gspn::slice_supported(a)) return GSPN_PATH_SLICE;
    }
    return path;
}

}  // extern "C"

namespace {

// The backward of gspn_scan_fwd (flags = 0) and of its per-direction
// variants (gspn_scan_fwd_ex's flags; line kernels only).
int scan_bwd_impl(const void* x, const void* w_raw, const void* lam, const void* u, const void* gy, void* gx,
                  void* gw_raw, void* glam, void* gu, int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs,
                  int32_t groups, int32_t ch_per_weight, uint32_t flags, int32_t dtype, int32_t path,
                  hipStream_t stream) {
    g_last_error[0] = '\0';
    int rc = check_sizes(B, C, H, W, dirs, groups, ch_per_weight, dtype);
    if (rc) return rc;
    if (flags & ~(uint32_t)(GSPN_LAM_PER_DIR | GSPN_U_PER_DIR)) return GSPN_ERR_FLAGS;
    if (!x || !w_raw || !lam || !u || !gy || !gx || !gw_raw || !glam || !gu) return GSPN_ERR_NULL;
    const void* ptrs[9] = {x, w_raw, lam, u, gy, gx, gw_raw, glam, gu};
    for (const void* q : ptrs)
        if ((uintptr_t)q & 15u) return GSPN_ERR_ALIGN;
    const size_t es = dtype == GSPN_BF16 ? 2 : 4;
    const size_t nbytes = (size_t)B * C * H * W * es;
    const size_t wbytes = (size_t)popcount4(dirs) * B * (C / ch_per_weight) * 3 * H * W * es;
    const size_t lbytes = (flags & GSPN_LAM_PER_DIR) ? popcount4(dirs) * nbytes : nbytes;
    const size_t ubytes = (flags & GSPN_U_PER_DIR) ? popcount4(dirs) * nbytes : nbytes;
    // every output is disjoint from every input and from the other outputs
    const void* outs[4] = {gx, gw_raw, glam, gu};
    const size_t out_bytes[4] = {nbytes, wbytes, lbytes, ubytes};
    const void* ins[5] = {x, w_raw, lam, u, gy};
    const size_t in_bytes[5] = {nbytes, wbytes, lbytes, ubytes, nbytes};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return GSPN_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return GSPN_ERR_ALIAS;
    }
    // per-direction lambda / u run on the line kernels only
    if (path == GSPN_PATH_AUTO) path = flags ? GSPN_PATH_GENERAL : auto_path(H, W);
    if (path != GSPN_PATH_FUSED && path != GSPN_PATH_GENERAL) return GSPN_ERR_PATH;
    if (path == GSPN_PATH_FUSED && (auto_path(H, W) != GSPN_PATH_FUSED || flags)) return GSPN_ERR_PATH;
    if (path == GSPN_PATH_GENERAL && !gspn::lines_supported((int)H, (int)W)) {
        set_error_text("the backward runs on the line kernels: H, W <= 512 and multiples of K");
        return GSPN_ERR_PATH;
    }

    gspn::GradArgs g;
    g.fwd.x = x; g.fwd.w = w_raw; g.fwd.lam = lam; g.fwd.u = u; g.fwd.y = nullptr;
    g.fwd.B = (int)B; g.fwd.C = (int)C; g.fwd.H = (int)H; g.fwd.W = (int)W;
    g.fwd.dirs = dirs; g.fwd.groups = groups; g.fwd.cpw = ch_per_weight; g.fwd.bf16 = dtype == GSPN_BF16;
    g.fwd.lam_dir = (flags & GSPN_LAM_PER_DIR) != 0;
    g.fwd.u_dir = (flags & GSPN_U_PER_DIR) != 0;
    g.gy = gy; g.gx = gx; g.gw = gw_raw; g.glam = glam; g.gu = gu;
    if (path == GSPN_PATH_FUSED) {
        const hipError_t e = gspn::launch_fused_bwd(g, stream);
        if (e != hipSuccess) { set_error("fused backward launch", e); return GSPN_ERR_HIP; }
        return GSPN_OK;
    }
    void* work = nullptr;
    hipError_t e = hipMallocAsync(&work, gspn::lines_bwd_workspace_bytes(g), stream);
    if (e != hipSuccess) { set_error("hipMallocAsync(workspace)", e); return GSPN_ERR_HIP; }
    e = gspn::launch_lines_bwd(g, work, stream);
    const hipError_t ef = hipFreeAsync(work, stream);
    if (e != hipSuccess) { set_error("backward kernel launch", e); return GSPN_ERR_HIP; }
    if (ef != hipSuccess) { set_error("hipFreeAsync(workspace)", ef); return GSPN_ERR_HIP; }
    return GSPN_OK;
}


// `scratch` (may be null): a device buffer of GSPN_NOALLOC_SCRATCH_BYTES that
// serves as the workspace instead of a stream-ordered allocation; shapes whose
// workspace is larger are rejected with GSPN_ERR_SCRATCH before any launch.
int scan_fwd_impl(const void* x, const void* w_raw, const void* lam, const void* u, void* y, int64_t B,
                  int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight,
                  uint32_t flags, int32_t dtype, int32_t path, hipStream_t stream, void* scratch = nullptr) {
    g_last_error[0] = '\0';
    int rc = check_sizes(B, C, H, W, dirs, groups, ch_per_weight, dtype);
    if (rc) return rc;
    if (flags & ~(uint32_t)(GSPN_LAM_PER_DIR | GSPN_U_PER_DIR)) return GSPN_ERR_FLAGS;
    if (!x || !w_raw || !lam || !u || !y) return GSPN_ERR_NULL;
    const void* ptrs[5] = {x, w_raw, lam, u, y};
    for (const void* q : ptrs)
        if ((uintptr_t)q & 15u) return GSPN_ERR_ALIGN;
    const size_t es = dtype == GSPN_BF16 ? 2 : 4;
    const size_t E = (size_t)B * C * H * W;
    const size_t nbytes = E * es;
    const size_t wbytes = (size_t)popcount4(dirs) * B * (C / ch_per_weight) * 3 * H * W * es;
    const size_t lbytes = (flags & GSPN_LAM_PER_DIR) ? popcount4(dirs) * nbytes : nbytes;
    const size_t ubytes = (flags & GSPN_U_PER_DIR) ? popcount4(dirs) * nbytes : nbytes;
    if (overlaps(y, nbytes, x, nbytes) || overlaps(y, nbytes, lam, lbytes) ||
        overlaps(y, nbytes, u, ubytes) || overlaps(y, nbytes, w_raw, wbytes))
        return GSPN_ERR_ALIAS;
    gspn::ScanArgs a;
    a.x = x; a.w = w_raw; a.lam = lam; a.u = u; a.y = y;
    a.B = (int)B; a.C = (int)C; a.H = (int)H; a.W = (int)W;
    a.dirs = dirs; a.groups = groups; a.cpw = ch_per_weight; a.bf16 = dtype == GSPN_BF16;
    a.lam_dir = (flags & GSPN_LAM_PER_DIR) != 0;
    a.u_dir = (flags & GSPN_U_PER_DIR) != 0;

    // per-direction lambda / u run on the line kernels only
    if (path == GSPN_PATH_AUTO) {
        path = flags ? GSPN_PATH_GENERAL : auto_path(H, W);
        if (path == GSPN_PATH_GENERAL && gspn::slice_supported(a)) path = GSPN_PATH_SLICE;
    }
    if (path != GSPN_PATH_FUSED && path != GSPN_PATH_GENERAL && path != GSPN_PATH_SLICE) return GSPN_ERR_PATH;
    if (path == GSPN_PATH_FUSED && (auto_path(H, W) != GSPN_PATH_FUSED || flags)) return GSPN_ERR_PATH;
    if (path == GSPN_PATH_SLICE && !gspn::slice_supported(a)) return GSPN_ERR_PATH;
    if (flags && !gspn::lines_supported((int)H, (int)W)) {
        set_error_text("per-direction lambda / u run on the line kernels: H, W <= 512 and multiples of K");
        return GSPN_ERR_PATH;
    }

    if (path == GSPN_PATH_SLICE) {
        const hipError_t e = gspn::launch_slice(a, stream);
        if (e != hipSuccess) { set_error("slice kernel launch", e); return GSPN_ERR_HIP; }
        return GSPN_OK;
    }
    if (path == GSPN_PATH_FUSED) {
        const hipError_t e = gspn::launch_fused(a, stream);
        if (e != hipSuccess) { set_error("fused kernel launch", e); return GSPN_ERR_HIP; }
        return GSPN_OK;
    }
    // general path: stream-ordered workspace (line kernels when the sides
    // allow, else the per-line fallback)
    const bool lines = gspn::lines_supported(a.H, a.W);
    const size_t pbytes = lines ? gspn::lines_workspace_bytes(a) : (size_t)popcount4(dirs) * E * sizeof(float);
    if (scratch) {
        if (pbytes > (size_t)GSPN_NOALLOC_SCRATCH_BYTES) {
            snprintf(g_last_error, sizeof(g_last_error),
                     "the workspace of this shape (%zu bytes) exceeds the static scratch (%zu bytes)", pbytes,
                     (size_t)GSPN_NOALLOC_SCRATCH_BYTES);
            return GSPN_ERR_SCRATCH;
        }
        const hipError_t el = lines ? gspn::launch_lines(a, scratch, stream)
                                    : gspn::launch_general(a, static_cast<float*>(scratch), stream);
        if (el != hipSuccess) { set_error("general kernel launch", el); return GSPN_ERR_HIP; }
        return GSPN_OK;
    }
    void* work = nullptr;
    hipError_t e = hipMallocAsync(&work, pbytes, stream);
    if (e != hipSuccess) { set_error("hipMallocAsync(workspace)", e); return GSPN_ERR_HIP; }
    e = lines ? gspn::launch_lines(a, work, stream) : gspn::launch_general(a, static_cast<float*>(work), stream);
    const hipError_t ef = hipFreeAsync(work, stream);
    if (e != hipSuccess) { set_error("general kernel launch", e); return GSPN_ERR_HIP; }
    if (ef != hipSuccess) { set_error("hipFreeAsync(workspace)", ef); return GSPN_ERR_HIP; }
    return GSPN_OK;
}

}  // namespace

extern "C" {

int gspn_scan_fwd_path(const void* x, const void* w_raw, const void* lam, const void* u, void* y,
                       int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                       int32_t ch_per_weight, int32_t dtype, int32_t path, hipStream_t stream) {
    return scan_fwd_impl(x, w_raw, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, 0u, dtype, path,
                         stream);
}

int gspn_scan_fwd_ex(const void* x, const void* w_raw, const void* lam, const void* u, void* y, int64_t B,
                     int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight,
                     uint32_t flags, int32_t dtype, hipStream_t stream) {
    return scan_fwd_impl(x, w_raw, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, flags, dtype,
                         GSPN_PATH_AUTO, stream);
}

int gspn_scan_fwd_batched(const gspn_problem* problems, int32_t count, int32_t dtype, hipStream_t stream) {
    g_last_error[0] = '\0';
    if (!problems) return GSPN_ERR_NULL;
    if (count < 1 || count > GSPN_MAX_BATCH) return GSPN_ERR_SHAPE;
    if (dtype != GSPN_F32 && dtype != GSPN_BF16) return GSPN_ERR_DTYPE;
    const size_t es = dtype == GSPN_BF16 ? 2 : 4;
    gspn::ScanArgs args[GSPN_MAX_BATCH];
    for (int i = 0; i < count; ++i) {
        const gspn_problem& q = problems[i];
        const int rc = check_sizes(q.B, q.C, q.H, q.W, q.dirs, q.groups, q.ch_per_weight, dtype);
        if (rc) return rc;
        if (!q.x || !q.w_raw || !q.lam || !q.u || !q.y) return GSPN_ERR_NULL;
        const void* ptrs[5] = {q.x, q.w_raw, q.lam, q.u, q.y};
        for (const void* v : ptrs)
            if ((uintptr_t)v & 15u) return GSPN_ERR_ALIGN;
        if (auto_path(q.H, q.W) != GSPN_PATH_FUSED) {
            set_error_text("every problem of a batch must take the fused path (H, W <= 64)");
            return GSPN_ERR_PATH;
        }
        gspn::ScanArgs& a = args[i];
        a.x = q.x; a.w = q.w_raw; a.lam = q.lam; a.u = q.u; a.y = q.y;
        a.B = (int)q.B; a.C = (int)q.C; a.H = (int)q.H; a.W = (int)q.W;
        a.dirs = q.dirs; a.groups = q.groups; a.cpw = q.ch_per_weight; a.bf16 = dtype == GSPN_BF16;
        a.lam_dir = 0; a.u_dir = 0;
    }
    // no output overlaps an input of any problem or another output
    for (int i = 0; i < count; ++i) {
        const gspn_problem& q = problems[i];
        const size_t ny = (size_t)q.B * q.C * q.H * q.W * es;
        for (int j = 0; j < count; ++j) {
            const gspn_problem& r = problems[j];
            const size_t n = (size_t)r.B * r.C * r.H * r.W * es;
            const size_t nw = (size_t)popcount4(r.dirs) * r.B * (r.C / r.ch_per_weight) * 3 * r.H * r.W * es;
            if (overlaps(q.y, ny, r.x, n) || overlaps(q.y, ny, r.lam, n) || overlaps(q.y, ny, r.u, n) ||
                overlaps(q.y, ny, r.w_raw, nw))
                return GSPN_ERR_ALIAS;
            if (j != i && overlaps(q.y, ny, r.y, n)) return GSPN_ERR_ALIAS;
        }
    }
    const hipError_t e = gspn::launch_fused_batched(args, count, stream);
    if (e != hipSuccess) { set_error("batched fused kernel launch", e); return GSPN_ERR_HIP; }
    return GSPN_OK;
}

int gspn_scan_fwd(const void* x, const void* w_raw, const void* lam, const void* u, void* y,
                  int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                  int32_t ch_per_weight, int32_t dtype, hipStream_t stream) {
    return gspn_scan_fwd_path(x, w_raw, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, dtype,
                              GSPN_PATH_AUTO, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation entry point
// The workspace of gspn_scan_fwd_noalloc: one static array per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, looked up once per device on the
// first call made with that device current.
static __device__ __align__(256) unsigned char scratch[GSPN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { set_error("hipGetDevice", e); return GSPN_ERR_HIP; }
    if (dev < 0 || dev >= kMaxDevices) { set_error_text("device index out of range"); return GSPN_ERR_HIP; }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("hipGetSymbolAddress(scratch)", e != hipSuccess ? e : hipErrorInvalidSymbol);
            return GSPN_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GSPN_OK;
}

}  // namespace

extern "C" {

int gspn_scan_fwd_noalloc(const void* x, const void* w_raw, const void* lam, const void* u, void* y,
                          int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                          int32_t ch_per_weight, int32_t dtype, hipStream_t stream) {
    g_last_error[0] = '\0';
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return scan_fwd_impl(x, w_raw, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, 0u, dtype,
                         GSPN_PATH_AUTO, stream, ws);
}

int gspn_bwd_supported(int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dirs, int32_t groups,
                       int32_t ch_per_weight, int32_t dtype) {
    const int rc = check_sizes(B, C, H, W, dirs, groups, ch_per_weight, dtype);
    if (rc) return rc;
    return gspn::lines_supported((int)H, (int)W) ? GSPN_OK : GSPN_ERR_PATH;
}

int gspn_scan_bwd(const void* x, const void* w_raw, const void* lam, const void* u, const void* gy,
                  void* gx, void* gw_raw, void* glam, void* gu, int64_t B, int64_t C, int64_t H,
                  int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight, int32_t dtype,
                  hipStream_t stream) {
    return gspn_scan_bwd_path(x, w_raw, lam, u, gy, gx, gw_raw, glam, gu, B, C, H, W, dirs, groups,
                              ch_per_weight, dtype, GSPN_PATH_AUTO, stream);
}

int gspn_scan_bwd_path(const void* x, const void* w_raw, const void* lam, const void* u, const void* gy,
                       void* gx, void* gw_raw, void* glam, void* gu, int64_t B, int64_t C, int64_t H,
                       int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight, int32_t dtype,
                       int32_t path, hipStream_t stream) {
    return scan_bwd_impl(x, w_raw, lam, u, gy, gx, gw_raw, glam, gu, B, C, H, W, dirs, groups, ch_per_weight, 0u,
                         dtype, path, stream);
}

int gspn_scan_bwd_ex(const void* x, const void* w_raw, const void* lam, const void* u, const void* gy,
                     void* gx, void* gw_raw, void* glam, void* gu, int64_t B, int64_t C, int64_t H, int64_t W,
                     uint32_t dirs, int32_t groups, int32_t ch_per_weight, uint32_t flags, int32_t dtype,
                     hipStream_t stream) {
    return scan_bwd_impl(x, w_raw, lam, u, gy, gx, gw_raw, glam, gu, B, C, H, W, dirs, groups, ch_per_weight,
                         flags, dtype, GSPN_PATH_AUTO, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- block
namespace {

std::mutex g_blas_mutex;
rocblas_handle g_blas[64];   // per device, created on first use

int blas_handle(rocblas_handle* h) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { set_error("hipGetDevice", e); return GSPN_ERR_HIP; }
    if (dev < 0 || dev >= 64) { set_error_text("device index out of range"); return GSPN_ERR_HIP; }
    if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
        g_blas[dev] = nullptr;
        set_error_text("rocblas_create_handle failed");
        return GSPN_ERR_HIP;
    }
    *h = g_blas[dev];
    return GSPN_OK;
}

// For each batch b: Out_b (N x P, row-major, batch stride so) = Wt (N x K,
// row-major) * In_b (K x P, row-major, batch stride si).  In rocBLAS's
// column-major terms Out_b^T = In_b^T * Wt^T, with no transposes.
// out_f32: the output is fp32 whatever the input dtype.
int gemm_rows(rocblas_handle h, int64_t N, int64_t K, int64_t P, const void* Wt, const void* in, int64_t si,
              void* out, int64_t so, int64_t batch, bool bf16, bool out_f32 = false) {
    const rocblas_datatype t = bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    const rocblas_datatype to = out_f32 ? rocblas_datatype_f32_r : t;
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)P, (rocblas_int)N, (rocblas_int)K, &alpha,
        in, t, (rocblas_int)P, si, Wt, t, (rocblas_int)K, 0, &beta, out, to, (rocblas_int)P, so, out, to,
        (rocblas_int)P, so, (rocblas_int)batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) {
        snprintf(g_last_error, sizeof(g_last_error), "rocblas_gemm_strided_batched_ex: %s",
                 rocblas_status_to_string(st));
        return GSPN_ERR_HIP;
    }
    return GSPN_OK;
}

int64_t block_rows(int64_t Cp, uint32_t dirs, int32_t cpw) {
    return 3 * Cp + 3 * (int64_t)popcount4(dirs) * (Cp / cpw);
}

}  // namespace

extern "C" {

int64_t gspn_block_rows(int64_t C_proxy, uint32_t dirs, int32_t ch_per_weight) {
    if (C_proxy <= 0) return GSPN_ERR_SHAPE;
    if (dirs == 0 || (dirs & ~15u)) return GSPN_ERR_DIRS;
    if (ch_per_weight < 1 || C_proxy % ch_per_weight) return GSPN_ERR_CPW;
    return block_rows(C_proxy, dirs, ch_per_weight);
}

int gspn_block_fwd(const void* x, const void* w_in, const void* w_out, void* z, int64_t B, int64_t C,
                   int64_t C_proxy, int64_t H, int64_t W, uint32_t dirs, int32_t groups, int32_t ch_per_weight,
                   uint32_t flags, int32_t dtype, hipStream_t stream) {
    g_last_error[0] = '\0';
    if (flags & ~(uint32_t)GSPN_BLOCK_RMSNORM) return GSPN_ERR_FLAGS;
    const bool norm = (flags & GSPN_BLOCK_RMSNORM) != 0;
    if (C <= 0 || C > (1LL << 22)) return GSPN_ERR_SHAPE;
    int rc = check_sizes(B, C_proxy, H, W, dirs, groups, ch_per_weight, dtype);
    if (rc) return rc;
    if (B * C > (1LL << 22)) return GSPN_ERR_SHAPE;
    if (!x || !w_in || !w_out || !z) return GSPN_ERR_NULL;
    const void* ptrs[4] = {x, w_in, w_out, z};
    for (const void* q : ptrs)
        if ((uintptr_t)q & 15u) return GSPN_ERR_ALIGN;
    const bool bf16 = dtype == GSPN_BF16;
    const size_t es = bf16 ? 2 : 4;
    const int64_t HW = H * W, Cp = C_proxy, Cw = C_proxy / ch_per_weight;
    const int64_t nd = popcount4(dirs), rows = block_rows(Cp, dirs, ch_per_weight);
    const size_t xbytes = (size_t)B * C * HW * es;
    if (overlaps(z, xbytes, x, xbytes) || overlaps(z, xbytes, w_in, (size_t)rows * C * es) ||
        overlaps(z, xbytes, w_out, (size_t)C * Cp * es))
        return GSPN_ERR_ALIAS;
    // the GEMM sizes are 32-bit in rocBLAS
    if (HW > INT32_MAX || rows > INT32_MAX || C > INT32_MAX) return GSPN_ERR_SHAPE;

    // workspace: g (the input projection, [B][rows][HW]) | y | and, unless
    // the fused scan reads g in place, x_proxy | taps (nd slabs) | lam | u;
    // then, when the normalisation follows a library GEMM, that GEMM's fp32
    // output (rounded once, by the scaling pass); each 256-byte aligned
    const bool in_place = auto_path(H, W) == GSPN_PATH_FUSED;
    const bool mfma_out = gspn::outproj_supported((int)Cp, (int)C, (int)HW, bf16);
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t ep = (size_t)B * Cp * HW * es, et = (size_t)nd * B * Cw * 3 * HW * es;
    const size_t o_g = 0, o_y = al((size_t)B * rows * HW * es), o_x = o_y + al(ep), o_t = o_x + al(ep),
                 o_l = o_t + al(et), o_u = o_l + al(ep);
    const size_t o_zf = in_place ? o_x : o_u + al(ep);
    const size_t total = o_zf + (norm && !mfma_out ? al((size_t)B * C * HW * sizeof(float)) : 0);
    char* work = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&work), total, stream);
    if (e != hipSuccess) { set_error("hipMallocAsync(workspace)", e); return GSPN_ERR_HIP; }

    rc = GSPN_OK;
    {
        std::lock_guard<std::mutex> lock(g_blas_mutex);
        rocblas_handle h = nullptr;
        rc = blas_handle(&h);
        if (rc == GSPN_OK && rocblas_set_stream(h, stream) != rocblas_status_success) {
            set_error_text("rocblas_set_stream failed");
            rc = GSPN_ERR_HIP;
        }
        // one GEMM reads x once: g_b = w_in x_b, [B][rows][HW]
        if (rc == GSPN_OK) rc = gemm_rows(h, rows, C, HW, w_in, x, C * HW, work + o_g, rows * HW, B, bf16);
        // The fused scan reads g in place: x_proxy, lam and u are row blocks of
        // g with a batch stride of `rows` planes, and the taps of slab s start
        // at row C_proxy + s*Cw*3.  The other paths take contiguous tensors:
        // g's row blocks are copied into x_proxy, lam, u [B][C_proxy][HW] and
        // the taps [nd][B][Cw*3][HW] (strided 2D copies).
        if (in_place && rc == GSPN_OK) {
            gspn::ScanArgs a;
            const size_t plane = (size_t)HW * es;
            a.x = work + o_g;
            a.w = work + o_g + (size_t)Cp * plane;
            a.lam = work + o_g + (size_t)(Cp + nd * Cw * 3) * plane;
            a.u = work + o_g + (size_t)(2 * Cp + nd * Cw * 3) * plane;
            a.y = work + o_y;
            a.B = (int)B; a.C = (int)Cp; a.H = (int)H; a.W = (int)W;
            a.dirs = dirs; a.groups = groups; a.cpw = ch_per_weight; a.bf16 = bf16;
            a.lam_dir = a.u_dir = 0;
            a.x_bplanes = (int)rows; a.w_bplanes = (int)rows; a.w_splanes = (int)(Cw * 3);
            const hipError_t el = gspn::launch_fused(a, stream);
            if (el != hipSuccess) { set_error("fused kernel launch", el); rc = GSPN_ERR_HIP; }
        }
        const size_t pitch = (size_t)rows * HW * es;
        auto rows_to = [&](char* dst, int64_t r0, int64_t nr, size_t dst_pitch) {
            if (rc != GSPN_OK) return;
            const hipError_t ec = hipMemcpy2DAsync(dst, dst_pitch, work + o_g + (size_t)r0 * HW * es, pitch,
                                                   (size_t)nr * HW * es, (size_t)B, hipMemcpyDeviceToDevice, stream);
            if (ec != hipSuccess) { set_error("hipMemcpy2DAsync", ec); rc = GSPN_ERR_HIP; }
        };
        if (!in_place) {
            rows_to(work + o_x, 0, Cp, (size_t)Cp * HW * es);
            for (int64_t sl = 0; sl < nd; ++sl)
                rows_to(work + o_t + (size_t)sl * B * Cw * 3 * HW * es, Cp + sl * Cw * 3, Cw * 3,
                        (size_t)Cw * 3 * HW * es);
            rows_to(work + o_l, Cp + nd * Cw * 3, Cp, (size_t)Cp * HW * es);
            rows_to(work + o_u, 2 * Cp + nd * Cw * 3, Cp, (size_t)Cp * HW * es);
        }
        if (rc == GSPN_OK && !in_place)
            rc = scan_fwd_impl(work + o_x, work + o_t, work + o_l, work + o_u, work + o_y, B, Cp, H, W, dirs,
                               groups, ch_per_weight, 0u, dtype, GSPN_PATH_AUTO, stream);
        // z: [B][C][HW] = w_out (C x C_proxy) * y_b, each pixel scaled by the
        // 1 / rms of its C_proxy scan outputs when normalising: one
        // hand-written MFMA kernel when the shape allows, else the library
        // GEMM followed by the scaling
        if (rc == GSPN_OK) {
            if (mfma_out) {
                const hipError_t el = gspn::launch_outproj(work + o_y, w_out, z, (int)B, (int)Cp, (int)C, (int)HW,
                                                           norm, GSPN_BLOCK_NORM_EPS, stream);
                if (el != hipSuccess) { set_error("output projection launch", el); rc = GSPN_ERR_HIP; }
            } else if (!norm) {
                rc = gemm_rows(h, C, Cp, HW, w_out, work + o_y, Cp * HW, z, C * HW, B, bf16);
            } else {
                // fp32 GEMM output, scaled and rounded to the dtype once
                rc = gemm_rows(h, C, Cp, HW, w_out, work + o_y, Cp * HW, work + o_zf, C * HW, B, bf16, true);
                if (rc == GSPN_OK) {
                    const hipError_t el = gspn::launch_rms_scale(work + o_y, reinterpret_cast<const float*>(work + o_zf), z,
                                                                 (int)B, (int)Cp, (int)C,
                                                                 (int)HW, bf16, GSPN_BLOCK_NORM_EPS, stream);
                    if (el != hipSuccess) { set_error("normalisation launch", el); rc = GSPN_ERR_HIP; }
                }
            }
        }
    }
    const hipError_t ef = hipFreeAsync(work, stream);
    if (rc != GSPN_OK) return rc;
    if (ef != hipSuccess) { set_error("hipFreeAsync(workspace)", ef); return GSPN_ERR_HIP; }
    return GSPN_OK;
}

}  // extern "C"
