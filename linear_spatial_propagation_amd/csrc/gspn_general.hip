// gspn_general.hip -- GSPN line scan for any grid up to 4096 x 4096.
//
// Same operator as the fused kernel (GSPN CVPR 2025 paper notes, "Key
// design 1/2/3"; GSPN-2 compact channel sharing), organised for lines longer
// than one wavefront:
//  * kernel 1: one workgroup (256 threads) per (enabled direction, b, c).
//    Thread t owns positions t, t+256, ... of the line; the previous line
//    lives in a double-buffered LDS array, one barrier per line step.  Taps
//    are normalised as they are consumed.  Each direction writes its h into
//    its own fp32 plane of the workspace.
//  * kernel 2: y = u * sum of the planes, in the fixed order TB, BT, LR, RL.
// This path is the general fallback: it moves popcount(dirs) * 8 extra bytes
// per element through the workspace.
#include "gspn_device.h"
#include "gspn_kernels.h"

namespace gspn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSide = 4096;
constexpr int kMaxPerThread = kMaxSide / kThreads;

struct GeneralParams {
    const void* x;
    const void* w;
    const void* lam;
    const void* u;
    void* y;
    float* planes;
    int B, C, H, W, Cw, cpw, groups;
    uint32_t dirs;
    int nd;
    int dir_of_slot[4];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void direction_kernel(GeneralParams prm) {
    __shared__ float hbuf[2][kMaxSide];
    const T* __restrict__ gx = static_cast<const T*>(prm.x);
    const T* __restrict__ gw = static_cast<const T*>(prm.w);
    const T* __restrict__ glam = static_cast<const T*>(prm.lam);

    const int H = prm.H, W = prm.W, C = prm.C;
    const size_t HW = (size_t)H * W;
    const int blk = blockIdx.x;                 // (slot, b, c), c fastest
    const int c = blk % C;
    const int b = (blk / C) % prm.B;
    const int slot = blk / (C * prm.B);
    const int d = prm.dir_of_slot[slot];
    const int k = c / prm.cpw;
    const bool is_row = d < 2;
    const int n = is_row ? H : W;
    const int m = is_row ? W : H;
    const int L = n / prm.groups;

    const size_t sbase = ((size_t)b * C + c) * HW;
    const T* __restrict__ xs = gx + sbase;
    const T* __restrict__ ls = glam + sbase;
    const T* __restrict__ ws = gw + ((size_t)(slot * prm.B + b) * prm.Cw + k) * 3 * HW;
    float* __restrict__ plane = prm.planes + (size_t)slot * prm.B * C * HW + sbase;

    int gl = 0;  // lines since the group started
    for (int i = 0; i < n; ++i) {
        float* hn = hbuf[i & 1];
        const float* hp = hbuf[(i & 1) ^ 1];
        for (int j = 0; j < kMaxPerThread; ++j) {
            const int p = threadIdx.x + j * kThreads;
            if (p >= m) break;
            int r, q;
            switch (d) {
                case 0: r = i; q = p; break;
                case 1: r = H - 1 - i; q = p; break;
                case 2: r = p; q = i; break;
                default: r = p; q = W - 1 - i; break;
            }
            const size_t e = (size_t)r * W + q;
            const float xl = to_f32(ls[e]) * to_f32(xs[e]);
            float v;
            if (gl == 0) {
                v = xl;
            } else {
                const bool has0 = p >= 1, has2 = p + 1 < m;
                const float a0 = has0 ? to_f32(ws[e]) : 0.0f;
                const float a1 = to_f32(ws[HW + e]);
                const float a2 = has2 ? to_f32(ws[2 * HW + e]) : 0.0f;
                const Taps tp = normalise_taps(a0, a1, a2, has0, has2);
                // difference form: the weights sum to exactly 1 (w1 = 1 - w0 -
                // w2 implicitly), so rounding in the normalisation cannot add a
                // drift that compounds over thousands of lines
                const float hc = hp[p];
                const float hl = has0 ? hp[p - 1] : hc;
                const float hr = has2 ? hp[p + 1] : hc;
                v = hc + xl;
                v = fmaf(tp.w0, hl - hc, v);
                v = fmaf(tp.w2, hr - hc, v);
            }
            hn[p] = v;
            plane[e] = v;
        }
        gl = (gl + 1 == L) ? 0 : gl + 1;
        __syncthreads();
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(GeneralParams prm, size_t E) {
    const T* __restrict__ gu = static_cast<const T*>(prm.u);
    T* __restrict__ gy = static_cast<T*>(prm.y);
    for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < E; e += (size_t)gridDim.x * kThreads) {
        float acc = 0.0f;
        for (int s = 0; s < prm.nd; ++s) acc += prm.planes[(size_t)s * E + e];
        // y is not read again: non-temporal store
        __builtin_nontemporal_store(from_f32(to_f32(gu[e]) * acc, (T*)nullptr), gy + e);
    }
}

}  // namespace

hipError_t launch_general(const ScanArgs& a, float* planes, hipStream_t stream) {
    GeneralParams p;
    p.x = a.x; p.w = a.w; p.lam = a.lam; p.u = a.u; p.y = a.y; p.planes = planes;
    p.B = a.B; p.C = a.C; p.H = a.H; p.W = a.W;
    p.cpw = a.cpw; p.Cw = a.C / a.cpw; p.groups = a.groups; p.dirs = a.dirs;
    p.nd = 0;
    for (int d = 0; d < 4; ++d)
        if ((a.dirs >> d) & 1u) p.dir_of_slot[p.nd++] = d;
    for (int s = p.nd; s < 4; ++s) p.dir_of_slot[s] = 0;
    const unsigned grid1 = (unsigned)((long)p.nd * a.B * a.C);
    const size_t E = (size_t)a.B * a.C * a.H * a.W;
    const unsigned grid2 = (unsigned)std::min<size_t>((E + kThreads - 1) / kThreads, 4096);
    if (a.bf16) {
        hipLaunchKernelGGL(direction_kernel<uint16_t>, dim3(grid1), dim3(kThreads), 0, stream, p);
        hipLaunchKernelGGL(merge_kernel<uint16_t>, dim3(grid2), dim3(kThreads), 0, stream, p, E);
    } else {
        hipLaunchKernelGGL(direction_kernel<float>, dim3(grid1), dim3(kThreads), 0, stream, p);
        hipLaunchKernelGGL(merge_kernel<float>, dim3(grid2), dim3(kThreads), 0, stream, p, E);
    }
    return hipGetLastError();
}

}  // namespace gspn
