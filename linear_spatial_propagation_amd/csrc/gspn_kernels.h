// gspn_kernels.h -- host-side launchers of the GSPN HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

// One validated call.  Sizes fit in int (checked by the C ABI layer).
struct ScanArgs {
    const void* x;
    const void* w;
    const void* lam;
    const void* u;
    void* y;
    int B, C, H, W;
    uint32_t dirs;
    int groups;
    int cpw;
    int bf16;     // 1: bf16 storage, 0: fp32 storage
    int lam_dir;  // 1: lam holds one [B][C][H][W] slab per enabled direction (line path only)
    int u_dir;    // 1: u holds one slab per enabled direction, y = sum_d u_d h_d (line path only)
    // Fused path only: strides in H*W planes, 0 for the contiguous layout.
    // x, lam and u: planes between batch items (default C); w: planes
    // between batch items (default (C/cpw)*3) and between direction slabs
    // (default B*(C/cpw)*3).  y is always contiguous.
    int x_bplanes = 0, w_bplanes = 0, w_splanes = 0;
};

// Fused 4-direction kernel: H <= 64 and W <= 64.
constexpr int kFusedMaxSide = 64;
hipError_t launch_fused(const ScanArgs& a, hipStream_t stream);
// Up to 32 validated fused-path problems of one dtype in one launch.
hipError_t launch_fused_batched(const ScanArgs* probs, int count, hipStream_t stream);

// Line path: H, W <= kLinesMaxSide with both sides multiples of K (the
// positions per lane, lines_positions_per_lane).  Workspace layout, in
// order: fp32 planes [nd][B][C][H*W], a 2 KiB sink for idle lanes' stores;
// if LR or RL is enabled, x and lambda
// transposed ([B][C][W][H], I/O dtype; lambda once per column direction when
// it is per direction) and the enabled column directions'
// raw taps transposed ([ncol][B][C/cpw][3][W][H]).
constexpr int kLinesMaxSide = 512;
struct LinesWorkspace {
    float* planes;
    float* sink;
    void* xT;
    void* lamT;
    void* wT;
};
int lines_positions_per_lane(int H, int W);
bool lines_supported(int H, int W);
size_t lines_workspace_bytes(const ScanArgs& a);
hipError_t launch_lines(const ScanArgs& a, void* workspace, hipStream_t stream);

// Backward on the line kernels (same shapes as lines_supported): the
// forward's ScanArgs (y unused) plus dL/dy and the four gradients.
struct GradArgs {
    ScanArgs fwd;
    const void* gy;
    void* gx;
    void* gw;      // dL/d raw taps, layout of w
    void* glam;
    void* gu;
};
// Fused backward: H <= 64 and W <= 64, no workspace.
hipError_t launch_fused_bwd(const GradArgs& g, hipStream_t stream);
size_t lines_bwd_workspace_bytes(const GradArgs& g);
hipError_t launch_lines_bwd(const GradArgs& g, void* workspace, hipStream_t stream);

// Compressed block: the output projection with the block's RMS
// normalisation fused (bf16; C_proxy in {16, 32, 64, 128, 256}, C % 32 == 0,
// H*W % 8 == 0), and the normalisation alone for the other shapes: it
// scales the fp32 z a library GEMM computed and rounds it into the output.
bool outproj_supported(int Cp, int C, int HW, bool bf16);
hipError_t launch_outproj(const void* y, const void* w_out, void* z, int B, int Cp, int C, int HW, bool norm,
                          float eps, hipStream_t stream);
hipError_t launch_rms_scale(const void* y, const float* zf, void* z, int B, int Cp, int C, int HW, bool bf16,
                            float eps, hipStream_t stream);

// One workgroup per (b, c) slice with the slice's sum in LDS: bf16, shared
// lambda and u, H, W <= 128, W % 8 == 0, H even, groups >= 8 and, with LR or
// RL enabled, (W / groups) % 8 == 0.  No workspace.
bool slice_supported(const ScanArgs& a);
hipError_t launch_slice(const ScanArgs& a, hipStream_t stream);

// Per-line fallback: any H, W <= 4096.  `planes` is an fp32 workspace of
// popcount(dirs) * B*C*H*W floats.
hipError_t launch_general(const ScanArgs& a, float* planes, hipStream_t stream);

}  // namespace gspn
