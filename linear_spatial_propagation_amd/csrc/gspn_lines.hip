// gspn_lines.hip -- GSPN line scan for grids with sides up to 512 that do not
// fit the fused kernel (forward).
//
// Organisation (three launches on the caller's stream, kernels in
// gspn_lines.h):
//  1. transpose_kernel: x, lambda and the LR/RL raw taps are copied to a
//     [W][H] (column-major) layout, so that every direction reads its lines
//     as contiguous rows.  64 x 64 tiles through LDS, 16-byte accesses.
//  2. line_scan_kernel<K>: one wave per (direction, b, c) scan; lane l owns
//     K consecutive positions of the line (K * 64 >= line length), so a line
//     is one wave (lines longer than 256: four waves of 2 positions per lane
//     that exchange their end states once per line), the state lives in K
//     VGPRs per lane, and the neighbours across lanes come from DPP wave
//     shifts.  The inputs of the next kDepth
//     lines are prefetched into registers with 16-byte (or K-element) loads;
//     taps are normalised as they are consumed (3 exp + 1 rcp per pixel).
//     Each direction writes h, line-major, to its own fp32 plane.
//  3. merge_kernel: y = u * (h_TB + h_BT + h_LR + h_RL) per 64 x 64 tile; the
//     LR/RL planes are read along their lines and transposed through LDS.
#include "gspn_lines.h"

namespace gspn {
namespace {

template <typename T>
hipError_t launch_lines_t(const ScanArgs& a, const LinesWorkspace& ws, hipStream_t stream) {
    const int H = a.H, W = a.W;
    const int Cw = a.C / a.cpw;
    LineParams p;
    p.x = a.x; p.lam = a.lam; p.w = a.w;
    p.xT = ws.xT; p.lamT = ws.lamT; p.wT = ws.wT;
    p.planes = ws.planes;
    p.sink = ws.sink;
    const size_t E = (size_t)a.B * a.C * H * W;
    p.lam_ds = a.lam_dir ? E : 0;
    p.lamT_ds = a.lam_dir ? E : 0;
    p.B = a.B; p.C = a.C; p.H = H; p.W = W; p.Cw = Cw; p.cpw = a.cpw; p.groups = a.groups;
    int ncol = 0;
    p.nd = enabled_slots(a.dirs, p.dir_of_slot, p.col_index, &ncol);

    // 1. column-major copies for LR / RL
    if (ncol > 0) {
        const size_t planes_xl = (size_t)a.B * a.C;
        launch_transpose(static_cast<const T*>(a.x), static_cast<T*>(ws.xT), planes_xl, H, W, stream);
        if (a.lam_dir) {
            for (int s = 0; s < p.nd; ++s) {
                if (p.dir_of_slot[s] < 2) continue;
                launch_transpose(static_cast<const T*>(a.lam) + (size_t)s * E,
                                 static_cast<T*>(ws.lamT) + (size_t)p.col_index[s] * E, planes_xl, H, W, stream);
            }
        } else {
            launch_transpose(static_cast<const T*>(a.lam), static_cast<T*>(ws.lamT), planes_xl, H, W, stream);
        }
        const size_t wslab = (size_t)a.B * Cw * 3;
        for (int s = 0; s < p.nd; ++s) {
            if (p.dir_of_slot[s] < 2) continue;
            launch_transpose(static_cast<const T*>(a.w) + (size_t)s * wslab * H * W,
                             static_cast<T*>(ws.wT) + (size_t)p.col_index[s] * wslab * H * W, wslab, H, W, stream);
        }
    }
    // 2. scans
    launch_line_scan<T>(p, stream);
    // 3. merge
    MergeParams q;
    q.in[0] = a.u; q.out[0] = a.y; q.in[1] = nullptr; q.out[1] = nullptr;
    q.planes = ws.planes;
    q.B = a.B; q.C = a.C; q.H = H; q.W = W; q.nd = p.nd;
    for (int s = 0; s < 4; ++s) q.dir_of_slot[s] = p.dir_of_slot[s];
    if (a.u_dir) launch_merge_dirs<T>(q, stream);
    else launch_merge<T, 1>(q, stream);
    return hipGetLastError();
}

}  // namespace

int lines_positions_per_lane(int H, int W) {
    const int m = std::max(H, W);
    return m <= 64 ? 1 : m <= 128 ? 2 : m <= 256 ? 4 : 8;
}

bool lines_supported(int H, int W) {
    if (std::max(H, W) > kLinesMaxSide) return false;
    // every line is a whole number of K-element vectors
    const int K = lines_positions_per_lane(H, W);
    return H % K == 0 && W % K == 0;
}

size_t lines_workspace_bytes(const ScanArgs& a) {
    const size_t E = (size_t)a.B * a.C * a.H * a.W;
    const size_t es = a.bf16 ? 2 : 4;
    int nd = 0, ncol = 0;
    for (int d = 0; d < 4; ++d)
        if ((a.dirs >> d) & 1u) { ++nd; if (d >= 2) ++ncol; }
    const size_t Ew = (size_t)a.B * (a.C / a.cpw) * 3 * a.H * a.W;
    size_t bytes = (size_t)nd * E * sizeof(float) + kSinkBytes;
    if (ncol) bytes += E * es + (a.lam_dir ? ncol : 1) * E * es + (size_t)ncol * Ew * es;
    return bytes;
}

hipError_t launch_lines(const ScanArgs& a, void* workspace, hipStream_t stream) {
    const size_t E = (size_t)a.B * a.C * a.H * a.W;
    const size_t es = a.bf16 ? 2 : 4;
    int nd = 0, ncol = 0;
    for (int d = 0; d < 4; ++d)
        if ((a.dirs >> d) & 1u) { ++nd; if (d >= 2) ++ncol; }
    LinesWorkspace ws;
    char* base = static_cast<char*>(workspace);
    ws.planes = reinterpret_cast<float*>(base);
    base += (size_t)nd * E * sizeof(float);
    ws.sink = reinterpret_cast<float*>(base);
    base += kSinkBytes;
    ws.xT = ncol ? base : nullptr;
    base += ncol ? E * es : 0;
    ws.lamT = ncol ? base : nullptr;
    base += ncol ? (a.lam_dir ? ncol : 1) * E * es : 0;
    ws.wT = ncol ? base : nullptr;
    return a.bf16 ? launch_lines_t<uint16_t>(a, ws, stream) : launch_lines_t<float>(a, ws, stream);
}

}  // namespace gspn
