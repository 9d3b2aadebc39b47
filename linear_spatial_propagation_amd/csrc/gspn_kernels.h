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
    int bf16;  // 1: bf16 storage, 0: fp32 storage
};

// Fused 4-direction kernel: H <= 64 and W <= 64.
constexpr int kFusedMaxSide = 64;
hipError_t launch_fused(const ScanArgs& a, hipStream_t stream);

// General path: any H, W <= 4096.  `planes` is an fp32 workspace of
// popcount(dirs) * B*C*H*W floats.
hipError_t launch_general(const ScanArgs& a, float* planes, hipStream_t stream);

}  // namespace gspn
