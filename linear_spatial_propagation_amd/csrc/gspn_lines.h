// gspn_lines.h -- kernels of the line path (transpose, line scan, merge),
// shared by the forward launcher (gspn_lines.hip) and the backward one
// (gspn_lines_bwd.hip).  Internal header: every definition has internal
// linkage, so each translation unit instantiates its own copies.
//
// Same operator as the fused kernel: the line recurrence of "Parallel
// Sequence Modeling via Generalized Spatial Propagation Network" (CVPR 2025
// paper notes, "Key design 1"), tridiagonal row-stochastic weights ("Key
// design 2"), four scan directions merged as y = u * sum_dir h_dir, local
// groups ("Key design 3"), channel-shared weights (GSPN-2 author response,
// "How Channel-shared Weight Mitigates the Concurrency Bottleneck?").
#pragma once

#include "gspn_device.h"
#include "gspn_kernels.h"

namespace gspn {
namespace {

constexpr int kDepth = 4;   // lines prefetched ahead
constexpr int kDepthK4 = 8; // the line scan with 4 positions per lane (sides 129..256), whose
                            // waves are memory-latency bound; with 8 per lane they are not
constexpr size_t kSinkBytes = 64 * 8 * sizeof(float);

// 16-byte vector <-> floats
__device__ __forceinline__ void unpack(uint4 r, float (&o)[8]) {
    o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x); o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
    o[4] = bf16_lo(r.z); o[5] = bf16_hi(r.z); o[6] = bf16_lo(r.w); o[7] = bf16_hi(r.w);
}
__device__ __forceinline__ void unpack(uint4 r, float (&o)[4]) {
    o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y); o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
}
// 16-byte store of 8 bf16 (rounded to nearest even) or 4 fp32.  Outputs use
// these ordinary stores too, not non-temporal ones: a wave's pieces of a
// 128-byte line may come from two instructions (or two waves) and combine
// in the L2, where non-temporal partial-line stores each reach HBM as a
// write of their own.
__device__ __forceinline__ void store16(uint16_t* p, const float (&v)[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ void store16(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- transpose
// src [P][R][Cc] -> dst [P][Cc][R], one 64 x 64 tile per workgroup, values
// converted from TS to TD on the way (fp32 -> bf16 rounds to nearest even).
// Whole tiles move as 16-byte vectors; a tile that crosses the edge of the
// plane goes element by element.
constexpr int kTile = 64;

__device__ __forceinline__ uint4 pack16(const float (&v)[8]) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4]) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}

template <typename TS, typename TD>
__global__ __launch_bounds__(256) void transpose_kernel(const TS* __restrict__ src, TD* __restrict__ dst, int R,
                                                        int Cc, int tiles_r, int tiles_c) {
    constexpr int NS = 16 / sizeof(TS);             // elements per 16-byte load
    constexpr int ND = 16 / sizeof(TD);             // elements per 16-byte store
    constexpr int NV = NS > ND ? NS : ND;
    __shared__ float tile[kTile][kTile + 1];        // values widened to fp32 (exact for bf16)
    const int t = blockIdx.x;
    const int tc = t % tiles_c;
    const int tr = (t / tiles_c) % tiles_r;
    const size_t plane = (size_t)(t / (tiles_c * tiles_r));
    const TS* s = src + plane * (size_t)R * Cc;
    TD* o = dst + plane * (size_t)R * Cc;
    const int r0 = tr * kTile, c0 = tc * kTile;
    const bool whole = r0 + kTile <= R && c0 + kTile <= Cc && Cc % NV == 0 && R % NV == 0;
    if (whole) {
        // thread -> (row, vector) of the tile; then (column, vector of rows)
        constexpr int kLV = kTile / NS, kLI = kTile * kLV / 256;
#pragma unroll
        for (int it = 0; it < kLI; ++it) {
            const int v = threadIdx.x + 256 * it;
            const int i = v / kLV, cv = (v % kLV) * NS;
            float f[NS];
            unpack(*reinterpret_cast<const uint4*>(s + (size_t)(r0 + i) * Cc + c0 + cv), f);
#pragma unroll
            for (int e = 0; e < NS; ++e) tile[i][cv + e] = f[e];
        }
        __syncthreads();
        constexpr int kSV = kTile / ND, kSI = kTile * kSV / 256;
#pragma unroll
        for (int it = 0; it < kSI; ++it) {
            const int v = threadIdx.x + 256 * it;
            const int cc = v / kSV, rv = (v % kSV) * ND;    // output row cc, rows rv.. of the input
            float f[ND];
#pragma unroll
            for (int e = 0; e < ND; ++e) f[e] = tile[rv + e][cc];
            *reinterpret_cast<uint4*>(o + (size_t)(c0 + cc) * R + r0 + rv) = pack16(f);
        }
        return;
    }
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < kTile; i += 4) {
        const int r = r0 + i, c = c0 + tx;
        tile[i][tx] = (r < R && c < Cc) ? to_f32(s[(size_t)r * Cc + c]) : 0.0f;
    }
    __syncthreads();
    for (int i = ty; i < kTile; i += 4) {
        const int c = c0 + i, r = r0 + tx;
        if (c < Cc && r < R) o[(size_t)c * R + r] = from_f32(tile[tx][i], (TD*)nullptr);
    }
}

// ---------------------------------------------------------------- scan
struct LineParams {
    const void* x;      // [B][C][H][W]
    const void* lam;
    const void* w;      // [nd][B][Cw][3][H][W]
    const void* xT;     // [B][C][W][H] (when LR or RL is enabled)
    const void* lamT;
    const void* wT;     // [ncol][B][Cw][3][W][H]
    float* planes;      // [nd][B][C][n_d][m_d], line-major per direction
    float* sink;        // 64 * 8 floats that absorb the stores of idle lanes
    size_t lam_ds;      // elements between directions' lambda slabs (0: shared)
    size_t lamT_ds;     // elements between column directions' transposed slabs (0: shared)
    int B, C, H, W, Cw, cpw, groups;
    int nd;
    int dir_of_slot[4];
    int col_index[4];   // slot -> index among the enabled column directions
};

// K consecutive elements of one line for one lane, as raw storage.
template <typename T, int K>
struct LineVec {
    static constexpr int kBytes = K * (int)sizeof(T);
    static constexpr int kWords = (kBytes + 3) / 4;
    uint32_t v[kWords];
    // aligned whole-vector load (m % K == 0)
    __device__ __forceinline__ void load(const T* p) {
        if constexpr (kBytes == 2) {
            v[0] = *reinterpret_cast<const uint16_t*>(p);
        } else if constexpr (kBytes == 4) {
            v[0] = *reinterpret_cast<const uint32_t*>(p);
        } else if constexpr (kBytes == 8) {
            const uint2 a = *reinterpret_cast<const uint2*>(p);
            v[0] = a.x; v[1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < kBytes / 16; ++i) {
                const uint4 a = reinterpret_cast<const uint4*>(p)[i];
                v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
            }
        }
    }
    __device__ __forceinline__ float get(int e) const {
        if constexpr (sizeof(T) == 2) {
            const uint32_t w = v[e >> 1];
            return (e & 1) ? bf16_hi(w) : bf16_lo(w);
        } else {
            return __uint_as_float(v[e]);
        }
    }
};

// The inputs of one line for one lane: three raw taps, and x and lambda of
// each of the G channels that share the taps.
template <typename T, int K, int G>
struct LineData {
    LineVec<T, K> a[3], x[G], l[G];
};

// D: lines loaded ahead (deeper for long lines: fewer waves share the GPU
// then, so each must keep more bytes in flight).
// SPLIT > 1: a line is held by the SPLIT waves of a workgroup, each owning
// 64 K consecutive positions; after every line each wave publishes the
// states at both of its ends through LDS and takes its neighbours' (one
// barrier per line).  Splitting the unit of work balances launches whose
// scans barely exceed one wave per SIMD: hires512's 1280 scans as 2560 waves
// of 4 positions per lane left half the SIMDs with a third wave; as 5120
// waves of 2 positions (5 per SIMD) its scan is about 1% faster (same bits).
// G: channels per wave, G consecutive channels of one weight set (cpw a
// multiple of G): the taps are loaded and normalised once per pixel and
// drive the G channels' scans (the channel-shared weights of the GSPN-2
// author response, "How Channel-shared Weight Mitigates the Concurrency
// Bottleneck?").  SPLIT = 2 takes G = 1.
template <typename T, int K, int D, int SPLIT, int G>
__global__ __launch_bounds__(256) void line_scan_kernel(LineParams prm) {
    static_assert(SPLIT == 1 || G == 1, "split lines scan one channel per wave");
    const int lane = threadIdx.x & 63;
    const int half = SPLIT >= 2 ? uniform(threadIdx.x >> 6) : 0;   // which part of the line
    const int unit = SPLIT >= 2 ? (int)blockIdx.x : (int)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
    const int C = prm.C, B = prm.B;
    const int CG = C / G;   // channel groups
    if (unit >= prm.nd * B * CG) return;   // whole wave
    // (b, channel group, slot), slot fastest: the directions of one slice run
    // side by side, so the pair that reads the same x and lambda shares them
    // in cache
    const int slot = unit % prm.nd;
    const int c = ((unit / prm.nd) % CG) * G;   // first channel of the group
    const int b = unit / (prm.nd * CG);
    const int d = prm.dir_of_slot[slot];
    const int k = c / prm.cpw;
    const bool is_row = d < 2;
    const bool asc = d == 0 || d == 2;
    const int H = prm.H, W = prm.W;
    const size_t HW = (size_t)H * W;
    const int n = is_row ? H : W;   // lines
    const int m = is_row ? W : H;   // positions per line
    const int L = n / prm.groups;

    // every tensor is read as [n][m], line-major; channel g of the group is
    // g * HW further on
    const T* xs = static_cast<const T*>(is_row ? prm.x : prm.xT) + ((size_t)b * C + c) * HW;
    const T* ls = (is_row ? static_cast<const T*>(prm.lam) + slot * prm.lam_ds
                          : static_cast<const T*>(prm.lamT) + prm.col_index[slot] * prm.lamT_ds) +
                  ((size_t)b * C + c) * HW;
    const T* ws = is_row
        ? static_cast<const T*>(prm.w) + ((size_t)(slot * B + b) * prm.Cw + k) * 3 * HW
        : static_cast<const T*>(prm.wT) + ((size_t)(prm.col_index[slot] * B + b) * prm.Cw + k) * 3 * HW;
    float* plane = prm.planes + ((size_t)slot * B * C + (size_t)b * C + c) * HW;

    // lane's positions p0 .. p0+K-1; lanes past the line read a clamped
    // vector and keep h = 0.  Masking is done on the bits with masks the
    // compiler cannot see through, so that it stays branch-free (a select
    // on loaded data turned into exec-masked branches with conservative
    // memory-counter waits).
    const int p0 = half * 64 * K + K * lane;
    const bool lane_on = p0 < m;
    const int pl = lane_on ? p0 : m - K;   // clamped (m % K == 0, m >= K)
    auto opaque = [](bool on) {
        uint32_t v = on ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(v));
        return v;
    };
    const uint32_t ml = opaque(lane_on);                   // the lane's positions exist
    const uint32_t m0 = opaque(lane_on && p0 >= 1);        // position p0 has tap 0
    const uint32_t m2 = opaque(lane_on && p0 + K < m);     // position p0+K-1 has tap 2
    const float f0 = lane_on && p0 >= 1 ? 1.0f : 0.0f;     // same, as factors of the
    const float f2 = lane_on && p0 + K < m ? 1.0f : 0.0f;  // dropped product terms
    const float fl = lane_on ? 1.0f : 0.0f;
    auto masked = [](float v, uint32_t msk) { return __uint_as_float(__float_as_uint(v) & msk); };

    auto load_line = [&](LineData<T, K, G>& q, int i) {
        const int j = asc ? i : n - 1 - i;
        const size_t o = (size_t)j * m + pl;
        q.a[0].load(ws + o);
        q.a[1].load(ws + HW + o);
        q.a[2].load(ws + 2 * HW + o);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            q.x[g].load(xs + g * HW + o);
            q.l[g].load(ls + g * HW + o);
        }
    };

    LineData<T, K, G> buf[D];
#pragma unroll
    for (int s = 0; s < D; ++s) load_line(buf[s], min(s, n - 1));

    float h[G][K];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < K; ++e) h[g][e] = 0.0f;
    // SPLIT: the neighbour part's state at the common edge (position
    // 64K - 1 or 64K of the line), from the previous line
    __shared__ float edge[2][SPLIT > 1 ? SPLIT : 1][2];   // [line parity][part][first, last position]
    float bndl = 0.0f, bndr = 0.0f;
    const bool takes_left = SPLIT >= 2 && half > 0 && lane == 0;
    const bool takes_right = SPLIT >= 2 && half < SPLIT - 1 && lane == 63;

    // D lines per iteration; steps past the last line (when D does not
    // divide n) compute on clamped data and store nothing
    for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            const LineData<T, K, G>& q = buf[s];
            float xl[G][K], a0[K], a1[K], a2[K];
            float amin = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < K; ++e) xl[g][e] = masked(q.x[g].get(e), ml) * masked(q.l[g].get(e), ml);
#pragma unroll
            for (int e = 0; e < K; ++e) {
                a0[e] = masked(q.a[0].get(e), e == 0 ? m0 : ml);   // missing taps -> 0
                a1[e] = masked(q.a[1].get(e), ml);
                a2[e] = masked(q.a[2].get(e), e == K - 1 ? m2 : ml);
                amin = fminf(amin, fminf(fminf(a0[e], a1[e]), a2[e]));
            }
            float hn[G][K];
            if (i % L == 0) {   // group start: h = lambda x, the taps are unused
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int e = 0; e < K; ++e) hn[g][e] = xl[g][e];
            } else {
                float w0[K], w2[K];
                // the rational form is safe when every tap is >= -40
                if (__builtin_amdgcn_ballot_w64(amin < -40.0f) == 0) {
                    const float kNegLog2e = -1.44269504088896340736f;
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const float q0 = 1.0f + __builtin_amdgcn_exp2f(a0[e] * kNegLog2e);
                        const float q1 = 1.0f + __builtin_amdgcn_exp2f(a1[e] * kNegLog2e);
                        const float q2 = 1.0f + __builtin_amdgcn_exp2f(a2[e] * kNegLog2e);
                        const float p12 = q1 * q2 * (e == 0 ? f0 : fl);
                        const float p01 = q0 * q1 * (e == K - 1 ? f2 : fl);
                        const float inv = __builtin_amdgcn_rcpf(fmaf(q0, q2, p12) + p01);
                        w0[e] = p12 * inv;
                        w2[e] = p01 * inv;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const bool h0 = lane_on && p0 + e >= 1, h2 = lane_on && p0 + e + 1 < m;
                        const Taps tp = normalise_taps(a0[e], a1[e], a2[e], h0, h2);
                        w0[e] = tp.w0;
                        w2[e] = tp.w2;
                    }
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float left = from_left(h[g][K - 1]);
                    float right = from_right(h[g][0]);
                    if constexpr (SPLIT >= 2) {
                        // the lane exchange runs in every lane before the edge
                        // lanes take the other part's value: sunk into a branch
                        // it would read the masked-off edge lanes as 0
                        asm volatile("" : "+v"(left), "+v"(right));
                        left = takes_left ? bndl : left;
                        right = takes_right ? bndr : right;
                    }
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const float hl = e == 0 ? left : h[g][e - 1];
                        const float hr = e == K - 1 ? right : h[g][e + 1];
                        float v = h[g][e] + xl[g][e];
                        v = fmaf(w0[e], hl - h[g][e], v);
                        hn[g][e] = fmaf(w2[e], hr - h[g][e], v);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < K; ++e) h[g][e] = hn[g][e];
            if constexpr (SPLIT >= 2) {
                // swap the edge states; the parity double-buffers the slots so
                // that one barrier per line suffices
                const int par = i & 1;
                if (lane == 0) edge[par][half][0] = h[0][0];
                if (lane == 63) edge[par][half][1] = h[0][K - 1];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                bndl = half > 0 ? edge[par][half > 0 ? half - 1 : 0][1] : 0.0f;
                bndr = half < SPLIT - 1 ? edge[par][half < SPLIT - 1 ? half + 1 : 0][0] : 0.0f;
            }
            {
                // unconditional store (a store under a divergent branch also
                // makes the counter waits conservative): lanes past the line
                // and steps past the last line write to a per-lane sink
                const int j = asc ? i : n - 1 - i;
                const bool real = i < n && lane_on;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float* dst = real ? plane + (size_t)g * HW + (size_t)j * m + p0 : prm.sink + K * lane;
                    if constexpr (K == 1) {
                        dst[0] = h[g][0];
                    } else if constexpr (K == 2) {
                        *reinterpret_cast<float2*>(dst) = make_float2(h[g][0], h[g][1]);
                    } else {
#pragma unroll
                        for (int e = 0; e < K; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(h[g][e], h[g][e + 1], h[g][e + 2], h[g][e + 3]);
                    }
                }
            }
            // refill the slot with the line D ahead (clamped: no
            // condition), after its data has been used
            load_line(buf[s], min(i + D, n - 1));
        }
    }
}

// ---------------------------------------------------------------- merge
// out_j = in_j * (sum of the planes) for NP (in, out) pairs: the forward's
// y = u * sum_dir h_dir (NP = 1), and in the backward gu = gy * sum_dir h_dir
// (NP = 1) and gx = lam * G, glam = x * G with G the summed adjoints (NP = 2).
struct MergeParams {
    const void* in[2];
    void* out[2];
    const float* planes;
    int B, C, H, W;
    int nd;
    int dir_of_slot[4];
    int tiles_r, tiles_c;
};

// One 64 x 64 tile of one (b, c) slice; the planes are summed in slot order
// (TB, BT, LR, RL).  Row planes are [H][W]; column planes [W][H] are read
// along their lines and transposed through LDS.  Thread -> (row, 16
// consecutive columns): 16-byte accesses throughout; a tile that crosses the
// edge of the slice goes element by element.
template <typename T, int NP>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams prm) {
    __shared__ float tile[kTile][kTile + 1];
    const int t = blockIdx.x;
    const int tc = t % prm.tiles_c;
    const int tr = (t / prm.tiles_c) % prm.tiles_r;
    const size_t bc = (size_t)(t / (prm.tiles_c * prm.tiles_r));
    const int H = prm.H, W = prm.W;
    const size_t HW = (size_t)H * W;
    const size_t E = (size_t)prm.B * prm.C * HW;
    const int r0 = tr * kTile, c0 = tc * kTile;
    const T* __restrict__ gin[NP];
    T* __restrict__ gout[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        gin[j] = static_cast<const T*>(prm.in[j]) + bc * HW;
        gout[j] = static_cast<T*>(prm.out[j]) + bc * HW;
    }
    bool any_col = false;
    for (int slot = 0; slot < prm.nd; ++slot) any_col |= prm.dir_of_slot[slot] >= 2;

    if (r0 + kTile <= H && c0 + kTile <= W && W % 16 == 0 && H % 16 == 0) {
        const int i = threadIdx.x >> 2, j0 = (threadIdx.x & 3) * 16;   // tile row i, columns j0..j0+15
        const size_t o = (size_t)(r0 + i) * W + c0 + j0;
        constexpr int N = 16 / (int)sizeof(T);
        // the multipliers are loaded first: their latency overlaps the
        // plane reads and the transpose instead of following the barrier
        uint4 gv[NP][16 / N];
#pragma unroll
        for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int e = 0; e < 16; e += N) gv[j][e / N] = *reinterpret_cast<const uint4*>(gin[j] + o + e);
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
        // column planes: tile[q][r] = sum over LR, RL (slot order) at
        // (row r0 + r, column c0 + q); this thread reads line c0 + i
        if (any_col) {
            float cs[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) cs[e] = 0.0f;
            for (int slot = 0; slot < prm.nd; ++slot) {
                if (prm.dir_of_slot[slot] < 2) continue;
                const float* P = prm.planes + slot * E + bc * HW + (size_t)(c0 + i) * H + r0 + j0;
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(P + e);
                    cs[e] += v.x; cs[e + 1] += v.y; cs[e + 2] += v.z; cs[e + 3] += v.w;
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) tile[i][j0 + e] = cs[e];
        }
        // row planes, in slot order (TB before BT)
        for (int slot = 0; slot < prm.nd; ++slot) {
            if (prm.dir_of_slot[slot] >= 2) continue;
            const float* P = prm.planes + slot * E + bc * HW + (size_t)(r0 + i) * W + c0 + j0;
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const float4 v = *reinterpret_cast<const float4*>(P + e);
                acc[e] += v.x; acc[e + 1] += v.y; acc[e + 2] += v.z; acc[e + 3] += v.w;
            }
        }
        __syncthreads();
        float sum[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[e] = any_col ? acc[e] + tile[j0 + e][i] : acc[e];
#pragma unroll
        for (int j = 0; j < NP; ++j) {
#pragma unroll
            for (int e = 0; e < 16; e += N) {
                float f[N];
                unpack(gv[j][e / N], f);
#pragma unroll
                for (int q = 0; q < N; ++q) f[q] *= sum[e + q];
                store16(gout[j] + o + e, f);
            }
        }
        return;
    }

    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    float acc[kTile / 4];
#pragma unroll
    for (int s = 0; s < kTile / 4; ++s) acc[s] = 0.0f;
    for (int slot = 0; slot < prm.nd; ++slot) {
        if (prm.dir_of_slot[slot] >= 2) continue;
        const float* P = prm.planes + slot * E + bc * HW;
#pragma unroll
        for (int s = 0; s < kTile / 4; ++s) {
            const int r = r0 + ty + 4 * s, q = c0 + tx;
            if (r < H && q < W) acc[s] += P[(size_t)r * W + q];
        }
    }
    bool first = true;
    for (int slot = 0; slot < prm.nd; ++slot) {
        if (prm.dir_of_slot[slot] < 2) continue;
        const float* P = prm.planes + slot * E + bc * HW;
#pragma unroll
        for (int s = 0; s < kTile / 4; ++s) {
            const int q = c0 + ty + 4 * s, r = r0 + tx;
            const float v = (q < W && r < H) ? P[(size_t)q * H + r] : 0.0f;
            if (first) tile[ty + 4 * s][tx] = v;
            else tile[ty + 4 * s][tx] += v;
        }
        first = false;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTile / 4; ++s) {
        const int r = r0 + ty + 4 * s, q = c0 + tx;
        if (r < H && q < W) {
            const float sum = any_col ? acc[s] + tile[tx][ty + 4 * s] : acc[s];
            const size_t e = (size_t)r * W + q;
#pragma unroll
            for (int j = 0; j < NP; ++j)
                gout[j][e] = from_f32(to_f32(gin[j][e]) * sum, (T*)nullptr);
        }
    }
}

// y = sum_d u_d * h_d (per-direction gates: the elementwise learnable merger).
// Same tiling as merge_kernel; u holds one [B][C][H][W] slab per enabled
// direction (slot order).  The sum runs in slot order (TB, BT, LR, RL); each
// column plane is transposed through LDS on its own, so that its gate
// multiplies it at the right pixel.
template <typename T>
__global__ __launch_bounds__(256) void merge_dirs_kernel(MergeParams prm) {
    __shared__ float tile[kTile][kTile + 1];
    const int t = blockIdx.x;
    const int tc = t % prm.tiles_c;
    const int tr = (t / prm.tiles_c) % prm.tiles_r;
    const size_t bc = (size_t)(t / (prm.tiles_c * prm.tiles_r));
    const int H = prm.H, W = prm.W;
    const size_t HW = (size_t)H * W;
    const size_t E = (size_t)prm.B * prm.C * HW;
    const int r0 = tr * kTile, c0 = tc * kTile;
    const T* __restrict__ gu = static_cast<const T*>(prm.in[0]) + bc * HW;
    T* __restrict__ gy = static_cast<T*>(prm.out[0]) + bc * HW;

    if (r0 + kTile <= H && c0 + kTile <= W && W % 16 == 0 && H % 16 == 0) {
        const int i = threadIdx.x >> 2, j0 = (threadIdx.x & 3) * 16;   // tile row i, columns j0..j0+15
        const size_t o = (size_t)(r0 + i) * W + c0 + j0;
        constexpr int N = 16 / (int)sizeof(T);
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
        for (int slot = 0; slot < prm.nd; ++slot) {
            float pv[16];
            if (prm.dir_of_slot[slot] < 2) {
                const float* P = prm.planes + slot * E + bc * HW + o;
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(P + e);
                    pv[e] = v.x; pv[e + 1] = v.y; pv[e + 2] = v.z; pv[e + 3] = v.w;
                }
            } else {
                // this thread reads line c0 + i (rows r0+j0 ..) and takes
                // back row r0 + i, columns c0+j0 .. from the tile
                const float* P = prm.planes + slot * E + bc * HW + (size_t)(c0 + i) * H + r0 + j0;
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(P + e);
                    tile[i][j0 + e] = v.x; tile[i][j0 + e + 1] = v.y;
                    tile[i][j0 + e + 2] = v.z; tile[i][j0 + e + 3] = v.w;
                }
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 16; ++e) pv[e] = tile[j0 + e][i];
                __syncthreads();
            }
            const T* us = gu + slot * E + o;
#pragma unroll
            for (int e = 0; e < 16; e += N) {
                float f[N];
                unpack(*reinterpret_cast<const uint4*>(us + e), f);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[e + q] = fmaf(f[q], pv[e + q], acc[e + q]);
            }
        }
#pragma unroll
        for (int e = 0; e < 16; e += N) {
            float f[N];
#pragma unroll
            for (int q = 0; q < N; ++q) f[q] = acc[e + q];
            store16(gy + o + e, f);
        }
        return;
    }

    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    float acc[kTile / 4];
#pragma unroll
    for (int s = 0; s < kTile / 4; ++s) acc[s] = 0.0f;
    for (int slot = 0; slot < prm.nd; ++slot) {
        const float* P = prm.planes + slot * E + bc * HW;
        const T* us = gu + slot * E;
        if (prm.dir_of_slot[slot] < 2) {
#pragma unroll
            for (int s = 0; s < kTile / 4; ++s) {
                const int r = r0 + ty + 4 * s, q = c0 + tx;
                if (r < H && q < W) acc[s] = fmaf(to_f32(us[(size_t)r * W + q]), P[(size_t)r * W + q], acc[s]);
            }
        } else {
#pragma unroll
            for (int s = 0; s < kTile / 4; ++s) {
                const int q = c0 + ty + 4 * s, r = r0 + tx;
                tile[ty + 4 * s][tx] = (q < W && r < H) ? P[(size_t)q * H + r] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < kTile / 4; ++s) {
                const int r = r0 + ty + 4 * s, q = c0 + tx;
                if (r < H && q < W) acc[s] = fmaf(to_f32(us[(size_t)r * W + q]), tile[tx][ty + 4 * s], acc[s]);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int s = 0; s < kTile / 4; ++s) {
        const int r = r0 + ty + 4 * s, q = c0 + tx;
        if (r < H && q < W) gy[(size_t)r * W + q] = from_f32(acc[s], (T*)nullptr);
    }
}

}  // namespace
}  // namespace gspn

namespace gspn {
namespace {

// ---------------------------------------------------------------- host side
// Enabled directions -> slots (ascending bit order), and each slot's index
// among the enabled column directions.  Returns the number of slots.
inline int enabled_slots(uint32_t dirs, int (&dir_of_slot)[4], int (&col_index)[4], int* ncol) {
    int nd = 0, nc = 0;
    for (int d = 0; d < 4; ++d) {
        if (!((dirs >> d) & 1u)) continue;
        dir_of_slot[nd] = d;
        col_index[nd] = d >= 2 ? nc++ : 0;
        ++nd;
    }
    for (int s = nd; s < 4; ++s) { dir_of_slot[s] = 0; col_index[s] = 0; }
    if (ncol) *ncol = nc;
    return nd;
}

// planes x [R][Cc] -> [Cc][R]
template <typename TS, typename TD>
void launch_transpose(const TS* src, TD* dst, size_t planes, int R, int Cc, hipStream_t stream) {
    const int tiles_r = (R + kTile - 1) / kTile, tiles_c = (Cc + kTile - 1) / kTile;
    hipLaunchKernelGGL((transpose_kernel<TS, TD>), dim3((unsigned)(planes * tiles_r * tiles_c)), dim3(256), 0, stream,
                       src, dst, R, Cc, tiles_r, tiles_c);
}

// Channels per wave of the line scan: 2 when the weight sets have an even
// number of channels and the halved launch still has at least 8 waves per
// SIMD (8192 on the 1024 SIMDs of the GPU), else 1.
inline int line_scan_channels(const LineParams& p) {
    const long units = (long)p.nd * p.B * p.C;
    const int m = p.H > p.W ? p.H : p.W;
    return m <= 256 && p.cpw % 2 == 0 && units / 2 >= 8192 ? 2 : 1;
}

// one wave per (slot, b, group of G channels)
template <typename T>
void launch_line_scan(const LineParams& p, hipStream_t stream) {
    const long units = (long)p.nd * p.B * p.C;
    const int m = p.H > p.W ? p.H : p.W;
    if (m > 256) {   // sides above 256: four waves of 2 positions per lane hold a line
        hipLaunchKernelGGL((line_scan_kernel<T, 2, kDepthK4, 4, 1>), dim3((unsigned)units), dim3(256), 0, stream, p);
        return;
    }
    const int G = line_scan_channels(p);
    const dim3 grid((unsigned)((units / G + 3) / 4));
    if (G == 2) {
        if (m <= 64) hipLaunchKernelGGL((line_scan_kernel<T, 1, kDepth, 1, 2>), grid, dim3(256), 0, stream, p);
        else if (m <= 128) hipLaunchKernelGGL((line_scan_kernel<T, 2, kDepth, 1, 2>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((line_scan_kernel<T, 4, kDepthK4, 1, 2>), grid, dim3(256), 0, stream, p);
    } else {
        if (m <= 64) hipLaunchKernelGGL((line_scan_kernel<T, 1, kDepth, 1, 1>), grid, dim3(256), 0, stream, p);
        else if (m <= 128) hipLaunchKernelGGL((line_scan_kernel<T, 2, kDepth, 1, 1>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((line_scan_kernel<T, 4, kDepthK4, 1, 1>), grid, dim3(256), 0, stream, p);
    }
}

template <typename T>
void launch_merge_dirs(MergeParams q, hipStream_t stream) {
    q.tiles_r = (q.H + kTile - 1) / kTile;
    q.tiles_c = (q.W + kTile - 1) / kTile;
    hipLaunchKernelGGL((merge_dirs_kernel<T>), dim3((unsigned)((size_t)q.B * q.C * q.tiles_r * q.tiles_c)),
                       dim3(256), 0, stream, q);
}

template <typename T, int NP>
void launch_merge(MergeParams q, hipStream_t stream) {
    q.tiles_r = (q.H + kTile - 1) / kTile;
    q.tiles_c = (q.W + kTile - 1) / kTile;
    hipLaunchKernelGGL((merge_kernel<T, NP>), dim3((unsigned)((size_t)q.B * q.C * q.tiles_r * q.tiles_c)), dim3(256),
                       0, stream, q);
}

}  // namespace
}  // namespace gspn
