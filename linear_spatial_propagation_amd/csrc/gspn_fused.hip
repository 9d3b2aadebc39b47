// gspn_fused.hip -- fused 4-direction GSPN line scan for grids up to 64 x 64.
//
// What it computes: the line recurrence h_i = w_i h_{i-1} + lambda_i x_i of
// "Parallel Sequence Modeling via Generalized Spatial Propagation Network"
// (CVPR 2025 paper notes, "Key design 1"), with tridiagonal row-stochastic
// w_i ("Key design 2"), in the four scan directions, merged as
// y = u * sum_dir h_dir, with optional local groups ("Key design 3") and one
// weight map shared by ch_per_weight consecutive channels (GSPN-2 author
// response, "How Channel-shared Weight Mitigates the Concurrency
// Bottleneck?").
//
// Design (gfx950, wave64):
//  * One workgroup of four waves per (batch b, weight set k[, channel
//    chunk]).  Wave d owns scan direction d (TB, BT, LR, RL); lane p owns
//    position p of the line, so a whole line is one wave and the state h
//    lives in one VGPR per lane.  Neighbours p-1 / p+1 come from the
//    adjacent lanes through DPP wave shifts -- no LDS traffic, no barrier in
//    the recurrence.
//  * Each wave normalises its direction's taps once per workgroup (3 exp + 1
//    rcp per pixel) into registers (64 lines x 3 taps) and reuses them for
//    every channel of the weight set: the sigmoid work is shared by the
//    channel group instead of being repeated per channel.
//  * lambda * x of the current channel is staged once in LDS as fp32
//    (row pitch 65 floats), with 16-byte coalesced loads, and read by all
//    four waves: row directions read LDS rows, column directions read LDS
//    columns; the odd pitch makes both conflict-free.  The next channel's
//    x and lambda are loaded while the current channel is scanned.
//  * TB/BT accumulate into one fp32 LDS plane and LR/RL into another: in
//    the first half of its lines each wave stores, after one workgroup
//    barrier it adds onto the partner direction's stores.  The summation
//    order is fixed, so results are deterministic.
//  * The merge reads both planes, multiplies by u and writes y once, rounded
//    to bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
//  * HBM traffic is the algorithmic minimum: x, lambda, u and the taps are
//    read once and y is written once.
#include "gspn_device.h"
#include "gspn_kernels.h"

namespace gspn {
namespace {

constexpr int kS = kFusedMaxSide;    // max lines and max positions
constexpr int kPitch = kS + 1;       // LDS row pitch (floats) of a 64 x 64 plane
constexpr int kPlane = kS * kPitch;  // floats per LDS plane
constexpr int kThreads = 256;

struct FusedParams {
    const void* x;
    const void* w;
    const void* lam;
    const void* u;
    void* y;
    int B, C, H, W;
    int Cw, cpw, groups;
    uint32_t dirs;
    int nchunk;     // channel chunks per weight set
    int chunk_len;  // channels per chunk
};

// 16-byte access = N elements.
template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {
    static constexpr int N = 8;
};
template <>
struct Vec<float> {
    static constexpr int N = 4;
};

// Load up to N consecutive elements into a 16-byte register image.
// `vec`: the address is 16-byte aligned and all N elements exist.
__device__ __forceinline__ uint4 load_raw(const uint16_t* __restrict__ p, int nvalid, bool vec) {
    if (vec) return *reinterpret_cast<const uint4*>(p);
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 8; ++j)
        if (j < nvalid) v[j >> 1] |= (uint32_t)p[j] << ((j & 1) * 16);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 load_raw(const float* __restrict__ p, int nvalid, bool vec) {
    if (vec) return *reinterpret_cast<const uint4*>(p);
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 4; ++j)
        if (j < nvalid) v[j] = __float_as_uint(p[j]);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void unpack(uint4 r, float (&o)[8]) {
    o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x);
    o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
    o[4] = bf16_lo(r.z); o[5] = bf16_hi(r.z);
    o[6] = bf16_lo(r.w); o[7] = bf16_hi(r.w);
}
__device__ __forceinline__ void unpack(uint4 r, float (&o)[4]) {
    o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y);
    o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
}

__device__ __forceinline__ void store_out(uint16_t* __restrict__ p, const float (&v)[8], int nvalid, bool vec) {
    if (vec) {
        uint4 r = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        *reinterpret_cast<uint4*>(p) = r;
    } else {
        for (int j = 0; j < 8; ++j)
            if (j < nvalid) p[j] = from_f32(v[j], (uint16_t*)nullptr);
    }
}
__device__ __forceinline__ void store_out(float* __restrict__ p, const float (&v)[4], int nvalid, bool vec) {
    if (vec) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        for (int j = 0; j < 4; ++j)
            if (j < nvalid) p[j] = v[j];
    }
}

template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fused_scan_kernel(FusedParams prm) {
    constexpr int N = Vec<T>::N;         // elements per 16-byte access
    constexpr int kMaxIt = kS * kS / (kThreads * N);
    __shared__ float lds[4 * kPlane];    // XL[2] | P_row | P_col

    const T* __restrict__ gx = static_cast<const T*>(prm.x);
    const T* __restrict__ gw = static_cast<const T*>(prm.w);
    const T* __restrict__ glam = static_cast<const T*>(prm.lam);
    const T* __restrict__ gu = static_cast<const T*>(prm.u);
    T* __restrict__ gy = static_cast<T*>(prm.y);

    const int H = prm.H, W = prm.W, B = prm.B, C = prm.C, Cw = prm.Cw;
    const int HW = H * W;
    const uint32_t dirs = prm.dirs;

    // ---- which (b, k, chunk) this workgroup owns
    const int wg = blockIdx.x;
    const int chunk = wg % prm.nchunk;
    const int bk = wg / prm.nchunk;
    const int k = bk % Cw;
    const int b = bk / Cw;
    const int c_begin = k * prm.cpw + chunk * prm.chunk_len;
    const int c_end = min(c_begin + prm.chunk_len, (k + 1) * prm.cpw);

    // ---- this wave's direction
    const int tid = threadIdx.x;
    const int d = uniform(tid >> 6);
    const int p = tid & 63;
    const bool is_row = d < 2;
    const bool on = (dirs >> d) & 1u;
    const bool partner_on = (dirs >> (d ^ 1)) & 1u;
    const int n = is_row ? H : W;      // lines
    const int m = is_row ? W : H;      // positions per line
    const int L = n / prm.groups;      // lines per group
    const bool has0 = p >= 1;
    const bool has2 = p + 1 < m;
    uint64_t start_mask = 0;           // bit s: line s starts a group
    for (int s = 0; s < n; s += L) start_mask |= 1ull << s;

    // ---- prologue: normalised taps of this direction, one line per step s.
    // Taps are staged through LDS in chunks of 16 lines for all four
    // directions, transposed for the column directions so that every wave
    // then reads its taps as [line][position] rows (conflict-free).  Entries
    // outside the grid are staged as 0 so idle lanes stay finite.
    float w0[kS], w1[kS], w2[kS];
    {
        constexpr int kChunk = 16;
        constexpr int kSP = kPitch;                 // staging row pitch (floats)
        float* S = lds;                             // [4][3][kChunk][kSP]
#pragma unroll
        for (int ch = 0; ch < kS / kChunk; ++ch) {
            const int s0 = ch * kChunk;
            for (int dd = 0; dd < 4; ++dd) {
                if (!((dirs >> dd) & 1u)) continue;
                const int slab = __builtin_popcount(dirs & ((1u << dd) - 1u));
                const T* __restrict__ src = gw + ((size_t)(slab * B + b) * Cw + k) * 3 * (size_t)HW;
                const int nd_ = dd < 2 ? H : W;
                const int md_ = dd < 2 ? W : H;
                float* Sd = S + dd * 3 * kChunk * kSP;
                if (dd < 2) {
                    // lines are memory rows: threads run along the row
                    const int pp = tid & 63;
                    for (int ii = tid >> 6; ii < kChunk; ii += kThreads / 64) {
                        const int s = s0 + ii;
                        const bool ok = s < nd_ && pp < md_;
                        const int r = dd == 0 ? s : H - 1 - s;
                        for (int t = 0; t < 3; ++t)
                            Sd[(t * kChunk + ii) * kSP + pp] = ok ? to_f32(src[(size_t)t * HW + r * W + pp]) : 0.0f;
                    }
                } else {
                    // lines are memory columns: threads run along the row
                    // (across lines) and the tile is written transposed
                    const int ii = tid & (kChunk - 1);
                    const int s = s0 + ii;
                    const int q = dd == 2 ? s : W - 1 - s;
                    for (int pp = tid / kChunk; pp < kS; pp += kThreads / kChunk) {
                        const bool ok = s < nd_ && pp < md_;
                        for (int t = 0; t < 3; ++t)
                            Sd[(t * kChunk + ii) * kSP + pp] = ok ? to_f32(src[(size_t)t * HW + pp * W + q]) : 0.0f;
                    }
                }
            }
            __syncthreads();
            const float* Sw = S + d * 3 * kChunk * kSP + p;
#pragma unroll
            for (int ii = 0; ii < kChunk; ++ii) {
                const Taps tp = normalise_taps(Sw[ii * kSP], Sw[(kChunk + ii) * kSP],
                                               Sw[(2 * kChunk + ii) * kSP], has0, has2);
                w0[s0 + ii] = tp.w0;
                w1[s0 + ii] = tp.w1;
                w2[s0 + ii] = tp.w2;
            }
            __syncthreads();
        }
    }

    // ---- staging / merge thread mapping: rows of W, N elements per thread
    const int tpr = (W + N - 1) / N;         // threads per row
    const int rpi = kThreads / tpr;          // rows per iteration
    const int tr = tid / tpr;
    const int tc = tid - tr * tpr;
    const int col0 = tc * N;
    const int nvalid = min(N, W - col0);
    const bool t_active = tr < rpi;
    const bool vec = (W % N) == 0;
    const bool row_any = (dirs & 3u) != 0;
    const bool col_any = (dirs & 12u) != 0;

    // padding rows/columns of XL must read as zero
    {
        float4* z = reinterpret_cast<float4*>(lds);
        for (int i = tid; i < (2 * kPlane) / 4; i += kThreads) z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();

    uint4 xr[kMaxIt], lr[kMaxIt];
    auto load_xl = [&](int c) {
        const size_t base = ((size_t)b * C + c) * (size_t)HW;
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int r = tr + it * rpi;
            if (t_active && r < H) {
                xr[it] = load_raw(gx + base + r * W + col0, nvalid, vec);
                lr[it] = load_raw(glam + base + r * W + col0, nvalid, vec);
            }
        }
    };
    auto write_xl = [&](float* X) {
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int r = tr + it * rpi;
            if (t_active && r < H) {
                float xv[N], lv[N];
                unpack(xr[it], xv);
                unpack(lr[it], lv);
#pragma unroll
                for (int j = 0; j < N; ++j)
                    if (j < nvalid) X[r * kPitch + col0 + j] = xv[j] * lv[j];
            }
        }
    };

    load_xl(c_begin);
    write_xl(lds);
    __syncthreads();

    float* const Pl = lds + (is_row ? 2 : 3) * kPlane;
    const int nstore = partner_on ? ((d & 1) ? n / 2 : (n + 1) / 2) : n;
    int off0, delta;
    switch (d) {
        case 0: off0 = p; delta = kPitch; break;                    // TB
        case 1: off0 = (H - 1) * kPitch + p; delta = -kPitch; break;  // BT
        case 2: off0 = p * kPitch; delta = 1; break;                // LR
        default: off0 = p * kPitch + W - 1; delta = -1; break;      // RL
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int buf = (c - c_begin) & 1;
        const float* const X = lds + buf * kPlane;
        const bool has_next = c + 1 < c_end;
        if (has_next) load_xl(c + 1);

        // ---- scan: first part stores, second part adds onto the partner
        float h = 0.0f;
        int off = off0;
        if (on) {
#pragma unroll
            for (int s = 0; s < kS; ++s) {
                if (s < nstore) {
                    const float xl = X[off];
                    if ((start_mask >> s) & 1u) {
                        h = xl;
                    } else {
                        const float hl = from_left(h), hr = from_right(h);
                        float v = fmaf(w1[s], h, xl);
                        v = fmaf(w0[s], hl, v);
                        h = fmaf(w2[s], hr, v);
                    }
                    Pl[off] = h;
                    off += delta;
                }
            }
        }
        __syncthreads();
        if (on) {
#pragma unroll
            for (int s = 0; s < kS; ++s) {
                if (s >= nstore && s < n) {
                    const float xl = X[off];
                    if ((start_mask >> s) & 1u) {
                        h = xl;
                    } else {
                        const float hl = from_left(h), hr = from_right(h);
                        float v = fmaf(w1[s], h, xl);
                        v = fmaf(w0[s], hl, v);
                        h = fmaf(w2[s], hr, v);
                    }
                    Pl[off] += h;
                    off += delta;
                }
            }
        }
        if (has_next) write_xl(lds + (buf ^ 1) * kPlane);
        __syncthreads();

        // ---- merge: y = u * (P_row + P_col)
        {
            const size_t base = ((size_t)b * C + c) * (size_t)HW;
            const float* PR = lds + 2 * kPlane;
            const float* PC = lds + 3 * kPlane;
#pragma unroll
            for (int it = 0; it < kMaxIt; ++it) {
                const int r = tr + it * rpi;
                if (t_active && r < H) {
                    float uv[N], yv[N];
                    unpack(load_raw(gu + base + r * W + col0, nvalid, vec), uv);
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        const int o = r * kPitch + col0 + j;
                        float acc = 0.0f;
                        if (j < nvalid) {
                            if (row_any) acc = PR[o];
                            if (col_any) acc += PC[o];
                        }
                        yv[j] = uv[j] * acc;
                    }
                    store_out(gy + base + r * W + col0, yv, nvalid, vec);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_fused(const ScanArgs& a, hipStream_t stream) {
    FusedParams p;
    p.x = a.x; p.w = a.w; p.lam = a.lam; p.u = a.u; p.y = a.y;
    p.B = a.B; p.C = a.C; p.H = a.H; p.W = a.W;
    p.cpw = a.cpw; p.Cw = a.C / a.cpw; p.groups = a.groups; p.dirs = a.dirs;
    // Split a weight set's channels over several workgroups only when there
    // are too few (b, k) pairs to occupy the GPU (two workgroups per CU).
    const long sets = (long)a.B * p.Cw;
    const long want = 512;
    int nchunk = 1;
    if (sets < want) nchunk = (int)std::min<long>(a.cpw, (want + sets - 1) / sets);
    p.chunk_len = (a.cpw + nchunk - 1) / nchunk;
    p.nchunk = (a.cpw + p.chunk_len - 1) / p.chunk_len;
    const unsigned grid = (unsigned)(sets * p.nchunk);
    if (a.bf16)
        hipLaunchKernelGGL(fused_scan_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(fused_scan_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gspn
