// gspn_block.hip -- output projection of the compressed propagation block,
// with the block's normalisation fused into it.
//
// The block ("GSPN-2: Efficient Parallel Sequence Modeling", author response,
// "Relate Compressive Proxy Dimension to Low-rank Approximation"; C-GSPN
// abstract: a compressed latent-space propagation block with fused
// normalisation) projects x to C_proxy channels, runs the scan there and
// projects the result back to C channels.  The normalisation is read as an
// RMS normalisation of the scan output y of each pixel over its C_proxy
// channels, y / sqrt(mean_q y_q^2 + eps), with no learned gain (w_out
// absorbs a per-channel gain).  It is fused into the output projection:
//
//   z[b][c][p] = inv_rms[b][p] * sum_q w_out[c][q] * y[b][q][p]
//
// Design (gfx950, bf16 in and out, fp32 accumulation):
//  * One workgroup of four waves owns 256 consecutive pixels of one batch
//    item; wave w owns 64 of them, as two 32-pixel blocks.  The workgroup
//    stages y[b][:, pixels] (C_proxy x 256, coalesced 16-byte rows) in LDS
//    once.
//  * MFMA v_mfma_f32_32x32x16_bf16 with D (32 pixels x 32 output channels)
//    = A (32 pixels x 16 proxy channels) * B (16 x 32): A is a wave's pixel
//    block read from the staged tile (kept in registers for the whole
//    kernel); B is 32 rows of w_out, copied once per workgroup into an LDS
//    stage (double-buffered: the next block is copied while the current one
//    is multiplied) and shared by the four waves and both pixel blocks.  The
//    loop runs over the C output channels in blocks of 32; a workgroup
//    reads y once and w_out once.
//  * The RMS of each pixel comes from the A operand itself: each lane holds
//    half of its pixel's C_proxy values; the two halves are added across
//    the lane pair (l, l ^ 32), so the normalisation costs no extra pass
//    over y.
//  * Each wave's 32 x 64 result block goes through LDS so that z is written
//    as whole 128-byte row segments, 16 bytes per lane, not as scattered
//    pieces of rows.
#include "gspn_device.h"
#include "gspn_kernels.h"

namespace gspn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPix = 256;    // pixels per workgroup, 64 per wave (two 32-pixel blocks)
constexpr int kThreadsP = 256;

// Layout of v_mfma_f32_32x32x16_bf16 (lane l of the wave, e = 0..7,
// r = 0..15): A[m][k] with m = l % 32, k = 8 (l / 32) + e; B[k][n] with
// k = 8 (l / 32) + e, n = l % 32; D[m][n] = acc[r] with
// m = 8 (r / 4) + 4 (l / 32) + r % 4, n = l % 32.
template <int KQ, bool NORM>
__global__ __launch_bounds__(kThreadsP, KQ <= 128 ? 2 : 1) void outproj_kernel(const uint16_t* __restrict__ y,
                                                               const uint16_t* __restrict__ w_out,
                                                               uint16_t* __restrict__ z, int C, int HW, int tiles,
                                                               float eps) {
    constexpr int kSteps = KQ / 16;      // MFMA k-steps
    constexpr int kRowVecs = kPix / 8;   // 16-byte vectors per staged y row
    constexpr int kWPitch = KQ + 8;      // bf16 per staged w_out row (16 bytes of padding)
    constexpr int kWBlock = 32 * kWPitch;   // one staged block of 32 w_out rows
    constexpr int kOPitch = 64 + 8;      // bf16 per row of a wave's 32 x 64 output block
    constexpr int kTileElems = KQ * kPix;
    constexpr int kLoopElems = 2 * kWBlock + 4 * 32 * kOPitch;
    constexpr int kLdsElems = kTileElems > kLoopElems ? kTileElems : kLoopElems;
    constexpr int kWVecs = 32 * KQ / 8;     // 16-byte pieces of a w_out block
    // LDS: the y tile while the A operand is built; then two w_out stages
    // and the four waves' output blocks
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, col = lane & 31;
    const int b = blockIdx.x / tiles;
    const int p_base = (blockIdx.x - b * tiles) * kPix;
    const uint16_t* __restrict__ yb = y + (size_t)b * KQ * HW;

    // ---- stage y[b][q][p_base .. p_base + 256) as tile[q][p] (pixels past
    // HW read the last whole vector; their results are not stored)
    for (int i = tid; i < KQ * kRowVecs; i += kThreadsP) {
        const int q = i / kRowVecs, v = i - q * kRowVecs;
        const int p = min(p_base + v * 8, HW - 8);
        *reinterpret_cast<uint4*>(&lds[q * kPix + v * 8]) = *reinterpret_cast<const uint4*>(yb + (size_t)q * HW + p);
    }
    __syncthreads();

    // ---- A operand, two 32-pixel blocks per wave: pixel wave*64 + 32 h + col,
    // proxy channels 16 s + 8 half + e; and the sum of squares of each pixel
    bf16x8 a[2][kSteps];
    float ss[2] = {0.0f, 0.0f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t v = lds[(16 * s + 8 * half + e) * kPix + wave * 64 + 32 * h + col];
                a[h][s][e] = __builtin_bit_cast(__bf16, v);
                const float f = to_f32(v);
                ss[h] = fmaf(f, f, ss[h]);
            }
        }
    }
    // 1 / rms of the 16 pixels of each block whose results this lane holds
    // (rows 8 (r / 4) + 4 half + r % 4): the two halves of each pixel's sum
    // sit in lanes l and l ^ 32
    float inv[2][16];
    if constexpr (NORM) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float tot = ss[h] + __shfl_xor(ss[h], 32);
            const float my_inv = 1.0f / sqrtf(tot * (1.0f / KQ) + eps);
#pragma unroll
            for (int r = 0; r < 16; ++r) inv[h][r] = __shfl(my_inv, 8 * (r / 4) + 4 * half + (r % 4));
        }
    }
    __syncthreads();   // the y tile is no longer read: its space becomes the stages

    uint16_t* wst = lds;                                  // 2 x [32][kWPitch]
    uint16_t* ost = lds + 2 * kWBlock + wave * 32 * kOPitch;   // this wave's [32][kOPitch]
    // w_out rows c0 .. c0 + 32 as whole 16-byte pieces: loaded into
    // registers early, written into a stage late, so the load's latency is
    // covered by a block's multiplications
    constexpr int kWPer = (kWVecs + kThreadsP - 1) / kThreadsP;
    uint4 wreg[kWPer];
    auto load_w = [&](int c0) {
#pragma unroll
        for (int k = 0; k < kWPer; ++k) {
            const int i = min(tid + k * kThreadsP, kWVecs - 1);
            const int r = i / (KQ / 8), v = i - r * (KQ / 8);
            wreg[k] = *reinterpret_cast<const uint4*>(w_out + (size_t)(c0 + r) * KQ + v * 8);
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int k = 0; k < kWPer; ++k) {
            const int i = tid + k * kThreadsP;
            const int r = i / (KQ / 8), v = i - r * (KQ / 8);
            if (i < kWVecs) *reinterpret_cast<uint4*>(&wst[buf * kWBlock + r * kWPitch + v * 8]) = wreg[k];
        }
    };
    const int px0 = p_base + wave * 64;
    uint16_t* __restrict__ zb = z + (size_t)b * C * HW;
    load_w(0);
    store_w(0);
    __syncthreads();
    int buf = 0;
    for (int c0 = 0; c0 < C; c0 += 32, buf ^= 1) {
        // the next block goes to the other stage (last read two blocks ago;
        // the barrier at the end of the previous block ordered those reads)
        const bool more = c0 + 32 < C;
        if (more) load_w(c0 + 32);
        // B operand: w_out row c0 + col, proxy channels 16 s + 8 half + e
        f32x16 acc[2] = {{}, {}};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&wst[buf * kWBlock + col * kWPitch + 16 * s + 8 * half]);
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][s], bv, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][s], bv, acc[1], 0, 0, 0);
        }
        // results -> this wave's LDS block as [channel][pixel] bf16: lane holds
        // channel col, pixels 32 h + 8 g + 4 half + j (one 8-byte write per g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = NORM ? acc[h][4 * g + j] * inv[h][4 * g + j] : acc[h][4 * g + j];
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2*>(ost + col * kOPitch + 32 * h + 8 * g + 4 * half) = o;
            }
        }
        // -> global as whole 128-byte rows: lane takes channel row lane / 8
        // (+ 8 k), pixels 8 (lane % 8) .. + 8 (a wave's LDS accesses complete
        // in order, so its own block needs no barrier)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = lane / 8 + 8 * k, px = 8 * (lane & 7);
            const uint4 v = *reinterpret_cast<const uint4*>(ost + r * kOPitch + px);
            if (px0 + px < HW) {
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 o = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(zb + (size_t)(c0 + r) * HW + px0 + px));
            }
        }
        if (more) store_w(buf ^ 1);
        __syncthreads();   // stage buf ^ 1 is complete; stage buf may be overwritten next
    }
}

// Fallback for the shapes the MFMA kernel does not take (and fp32): a
// library GEMM has written zf = w_out y in fp32; scale each pixel by 1 / rms
// of its scan output and round once into z.  One thread per pixel; both
// loops read and write consecutive pixels across threads.
template <typename T>
__global__ __launch_bounds__(256) void rms_scale_kernel(const T* __restrict__ y, const float* __restrict__ zf,
                                                        T* __restrict__ z, int Cp, int C, int HW, long npix,
                                                        float eps) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= npix) return;
    const long b = i / HW, p = i - b * HW;
    const T* yb = y + (size_t)b * Cp * HW + p;
    float ss = 0.0f;
    for (int q = 0; q < Cp; ++q) {
        const float f = to_f32(yb[(size_t)q * HW]);
        ss = fmaf(f, f, ss);
    }
    const float s = 1.0f / sqrtf(ss / (float)Cp + eps);
    const float* zfb = zf + (size_t)b * C * HW + p;
    T* zb = z + (size_t)b * C * HW + p;
    for (int c = 0; c < C; ++c) zb[(size_t)c * HW] = from_f32(zfb[(size_t)c * HW] * s, (T*)nullptr);
}

template <int KQ>
hipError_t launch_outproj_kq(const void* y, const void* w_out, void* z, int B, int C, int HW, bool norm,
                             float eps, hipStream_t stream) {
    const int tiles = (HW + kPix - 1) / kPix;
    const dim3 grid((unsigned)(B * tiles));
    const uint16_t* yy = static_cast<const uint16_t*>(y);
    const uint16_t* ww = static_cast<const uint16_t*>(w_out);
    uint16_t* zz = static_cast<uint16_t*>(z);
    if (norm) hipLaunchKernelGGL((outproj_kernel<KQ, true>), grid, dim3(kThreadsP), 0, stream, yy, ww, zz, C, HW, tiles, eps);
    else hipLaunchKernelGGL((outproj_kernel<KQ, false>), grid, dim3(kThreadsP), 0, stream, yy, ww, zz, C, HW, tiles, eps);
    return hipGetLastError();
}

}  // namespace

bool outproj_supported(int Cp, int C, int HW, bool bf16) {
    return bf16 && (Cp == 16 || Cp == 32 || Cp == 64 || Cp == 128 || Cp == 256) && C % 32 == 0 && HW % 8 == 0;
}

hipError_t launch_outproj(const void* y, const void* w_out, void* z, int B, int Cp, int C, int HW, bool norm,
                          float eps, hipStream_t stream) {
    switch (Cp) {
        case 16: return launch_outproj_kq<16>(y, w_out, z, B, C, HW, norm, eps, stream);
        case 32: return launch_outproj_kq<32>(y, w_out, z, B, C, HW, norm, eps, stream);
        case 64: return launch_outproj_kq<64>(y, w_out, z, B, C, HW, norm, eps, stream);
        case 128: return launch_outproj_kq<128>(y, w_out, z, B, C, HW, norm, eps, stream);
        case 256: return launch_outproj_kq<256>(y, w_out, z, B, C, HW, norm, eps, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rms_scale(const void* y, const float* zf, void* z, int B, int Cp, int C, int HW, bool bf16,
                            float eps, hipStream_t stream) {
    const long npix = (long)B * HW;
    const dim3 grid((unsigned)((npix + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL((rms_scale_kernel<uint16_t>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(y),
                           zf, static_cast<uint16_t*>(z), Cp, C, HW, npix, eps);
    else
        hipLaunchKernelGGL((rms_scale_kernel<float>), grid, dim3(256), 0, stream, static_cast<const float*>(y), zf,
                           static_cast<float*>(z), Cp, C, HW, npix, eps);
    return hipGetLastError();
}

}  // namespace gspn
