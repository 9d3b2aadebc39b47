// gspn_lines_bwd.hip -- backward of the GSPN line scan (sides up to 512).
//
// The gradients are the exact vector-Jacobian product of the forward
// operator ("Parallel Sequence Modeling via Generalized Spatial Propagation
// Network", CVPR 2025 paper notes, "Key design 1-3"; the GSPN-2 author
// response notes that the backward runs with the same speed-up as the
// forward, "Backward Benchmark").  With S = sum_dir h_dir and G = sum_dir g_dir:
//   gu = gy * S;   gx = lam * G;   glam = x * G
//   g_i = gy*u (at line i) + w_{i+1}^T g_{i+1}   (adjoint, last line first;
//         the second term is cut at the first line of a group)
//   dL/dw_t[i][p] = sum over the channels of a weight set of
//                   g_i[p] * h_{i-1}[p+t-1]
//   dL/da_t = w_t (1 - sigmoid(a_t)) (dL/dw_t - sum_v dL/dw_v w_v)
//         (sigmoid-then-normalise; 0 on the taps the forward never reads),
//         evaluated from E0 = D0 - D1, E2 = D2 - D1 without cancellation.
// With per-direction lambda_d / u_d (the variants y = sum_d u_d h_d, h_d
// driven by lambda_d x) the adjoint of direction d takes gy * u_d as its
// source, gu_d = gy * h_d, glam_d = x * g_d and gx = sum_d lambda_d g_d.
//
// Launches, in order, on the caller's stream:
//  1. transpose_kernel: x, lambda, gy, u and the LR/RL raw taps to [W][H];
//  2. line_scan_kernel: the forward again, h of every direction into fp32
//     planes;
//  3. merge_kernel: gu = gy * sum of the planes;
//  4. adjoint_scan_kernel: one wave per (direction, b, weight set), two for
//     lines longer than 256; the CH
//     channels of a chunk of the set run in lockstep, so each pixel's taps
//     are normalised once for all of them and their tap gradients are summed
//     in registers.  g overwrites h in the planes (line i's slot is free once
//     line i+1 has used h_i).  When a set's channels fit one chunk, dL/da
//     is rounded to the storage dtype in this kernel: the row directions
//     write the caller's tensor, the column directions a line-major copy.
//     Otherwise it goes to an fp32 workspace, line-major, one launch per
//     chunk, the later ones adding to it;
//  5. merge_kernel: gx = lam * G, glam = x * G;
//  6. the tap gradients to the caller's layout and dtype: a transpose of the
//     column directions' copies (and, from the fp32 workspace, a conversion
//     of the row directions').
#include "gspn_lines.h"

namespace gspn {
namespace {

struct AdjointParams {
    const void* gy;     // [B][C][H][W]
    const void* u;      // [B][C][H][W], or one slab per enabled direction (u_ds apart)
    const void* gyT;    // [B][C][W][H] (when LR or RL is enabled)
    const void* uT;     // transposed u, one slab per column direction when per direction
    size_t u_ds, uT_ds; // elements between u slabs (0: shared)
    const void* w;      // raw taps [nd][B][Cw][3][H][W]
    const void* wT;     // [ncol][B][Cw][3][W][H]
    float* planes;      // [nd][B][C][n][m]: h on entry, the adjoint g on exit
    float* ga;          // [nd][B][Cw][3][n][m]: dL/d raw taps, line-major
    void* gw_out;       // DIRECT: the caller's tap gradients, written by the row directions
    float* sink;        // absorbs the stores of idle lanes and finished steps
    int B, C, H, W, Cw, cpw, groups, nd;
    int chunk;          // this launch runs channels chunk*CH .. chunk*CH+CH-1 of every set
    int dir_of_slot[4];
    int col_index[4];
};

template <int K>
__device__ __forceinline__ void load_f32(float (&dst)[K], const float* p) {
    if constexpr (K == 1) {
        dst[0] = p[0];
    } else if constexpr (K == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        dst[0] = v.x; dst[1] = v.y;
    } else {
#pragma unroll
        for (int e = 0; e < K; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + e);
            dst[e] = v.x; dst[e + 1] = v.y; dst[e + 2] = v.z; dst[e + 3] = v.w;
        }
    }
}

template <int K>
__device__ __forceinline__ void store_f32(float* p, const float (&v)[K]);

// K values rounded to the storage dtype (round to nearest even) and stored.
template <typename T, int K>
__device__ __forceinline__ void store_t(T* p, const float (&v)[K]) {
    if constexpr (sizeof(T) == 4) {
        store_f32<K>(reinterpret_cast<float*>(p), v);
    } else if constexpr (K == 1) {
        *p = from_f32(v[0], (T*)nullptr);
    } else if constexpr (K == 2) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
    } else if constexpr (K == 4) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
}

template <int K>
__device__ __forceinline__ void store_f32(float* p, const float (&v)[K]) {
    if constexpr (K == 1) {
        p[0] = v[0];
    } else if constexpr (K == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
        for (int e = 0; e < K; e += 4) *reinterpret_cast<float4*>(p + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
}

// Everything one reverse step reads, for one lane.
template <typename T, int K, int CH, bool ACC, int SPLIT>
struct AdjointStep {
    LineVec<T, K> a[3];          // raw taps of line i
    LineVec<T, K> gy[CH], u[CH]; // at line i
    float hp[CH][K];             // h_{i-1}
    float gp[ACC ? 3 : 1][K];    // earlier chunks' dL/da at line i (ACC only)
    float hx[SPLIT == 2 ? CH : 1];   // SPLIT: h_{i-1} of the other part at the common edge
};

// DIRECT (a set's channels in one chunk, so nothing accumulates across
// launches): the tap gradients are rounded to the storage dtype here; row
// directions write the caller's layout, column directions a line-major
// workspace that one transpose puts in place.
// SPLIT = 2 (CH = 1): a line is held by the two waves of a 128-thread
// workgroup, each owning 64 K consecutive positions, as in the forward line
// scan.  Each part reads the other's h_{i-1} at the common edge from the
// planes, and after every step the two swap w0 g / w2 g at that edge through
// LDS (one barrier per step).
template <typename T, int K, int CH, bool ACC, bool DIRECT, int SPLIT>
__global__ __launch_bounds__(256) void adjoint_scan_kernel(AdjointParams prm) {
    static_assert(SPLIT == 1 || CH == 1, "split lines carry one channel");
    const int lane = threadIdx.x & 63;
    const int half = SPLIT == 2 ? uniform(threadIdx.x >> 6) : 0;   // which part of the line
    // (b, k, slot), slot fastest: the directions of one set run side by side,
    // so the pair that reads the same gy and u shares them in cache
    const int unit = SPLIT == 2 ? (int)blockIdx.x : (int)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
    const int B = prm.B, C = prm.C, Cw = prm.Cw;
    if (unit >= prm.nd * B * Cw) return;   // whole wave
    const int slot = unit % prm.nd;
    const int k = (unit / prm.nd) % Cw;
    const int b = unit / (prm.nd * Cw);
    const int d = prm.dir_of_slot[slot];
    const bool is_row = d < 2;
    const bool asc = d == 0 || d == 2;
    const int H = prm.H, W = prm.W;
    const size_t HW = (size_t)H * W;
    const int n = is_row ? H : W;   // lines
    const int m = is_row ? W : H;   // positions per line
    const int L = n / prm.groups;
    const int cbase = k * prm.cpw + prm.chunk * CH;

    // every tensor is read as [n][m], line-major; channel ch at + ch * HW
    const T* gys = static_cast<const T*>(is_row ? prm.gy : prm.gyT) + ((size_t)b * C + cbase) * HW;
    const T* us = (is_row ? static_cast<const T*>(prm.u) + slot * prm.u_ds
                          : static_cast<const T*>(prm.uT) + prm.col_index[slot] * prm.uT_ds) +
                  ((size_t)b * C + cbase) * HW;
    const T* ws = is_row
        ? static_cast<const T*>(prm.w) + ((size_t)(slot * B + b) * Cw + k) * 3 * HW
        : static_cast<const T*>(prm.wT) + ((size_t)(prm.col_index[slot] * B + b) * Cw + k) * 3 * HW;
    float* pl = prm.planes + ((size_t)slot * B * C + (size_t)b * C + cbase) * HW;
    float* gas = prm.ga + ((size_t)(slot * B + b) * Cw + k) * 3 * HW;

    // lane's positions p0 .. p0+K-1; lanes past the line read a clamped
    // vector and hold g = 0 (masks the compiler cannot see through keep the
    // code branch-free, as in the forward scan)
    const int p0 = half * 64 * K + K * lane;
    const bool lane_on = p0 < m;
    const int pc = lane_on ? p0 : m - K;
    auto opaque = [](bool on) {
        uint32_t v = on ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(v));
        return v;
    };
    const uint32_t ml = opaque(lane_on);
    const uint32_t m0 = opaque(lane_on && p0 >= 1);
    const uint32_t m2 = opaque(lane_on && p0 + K < m);
    const float f0 = lane_on && p0 >= 1 ? 1.0f : 0.0f;
    const float f2 = lane_on && p0 + K < m ? 1.0f : 0.0f;
    const float fl = lane_on ? 1.0f : 0.0f;
    auto masked = [](float v, uint32_t msk) { return __uint_as_float(__float_as_uint(v) & msk); };

    using Step = AdjointStep<T, K, CH, ACC, SPLIT>;
    // SPLIT: the lanes at the common edge and the other part's edge position
    const bool takes_left = SPLIT == 2 && half == 1 && lane == 0;
    const bool takes_right = SPLIT == 2 && half == 0 && lane == 63;
    const int pe = min(half == 0 ? 64 * K : 64 * K - 1, m - 1);
    __shared__ float xch[2][2];   // [step parity][part]: w2 g (part 0) / w0 g (part 1) at the edge
    auto load_step = [&](Step& q, int i) {   // 0 <= i < n
        const int j = asc ? i : n - 1 - i;
        const size_t o = (size_t)j * m + pc;
        q.a[0].load(ws + o);
        q.a[1].load(ws + HW + o);
        q.a[2].load(ws + 2 * HW + o);
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            q.gy[ch].load(gys + ch * HW + o);
            q.u[ch].load(us + ch * HW + o);
        }
        const int ip = i > 0 ? i - 1 : 0;
        const size_t lp = (size_t)(asc ? ip : n - 1 - ip) * m;
        const size_t op = lp + pc;
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) load_f32<K>(q.hp[ch], pl + ch * HW + op);
        if constexpr (SPLIT == 2) {
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) q.hx[ch] = pl[ch * HW + lp + pe];
        }
        if constexpr (ACC) {
#pragma unroll
            for (int t = 0; t < 3; ++t) load_f32<K>(q.gp[t], gas + t * HW + o);
        }
    };

    Step buf[kDepth];
#pragma unroll
    for (int s = 0; s < kDepth; ++s) load_step(buf[s], max(n - 1 - s, 0));

    float carry[CH][K];   // w_{i+1}^T g_{i+1}
#pragma unroll
    for (int ch = 0; ch < CH; ++ch)
#pragma unroll
        for (int e = 0; e < K; ++e) carry[ch][e] = 0.0f;

    for (int s0 = 0; s0 < n; s0 += kDepth) {
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            const int i = n - 1 - (s0 + s);            // < 0: past the last step
            const Step& q = buf[s];
            const bool live = i >= 0;
            const bool coupled = live && i % L != 0;   // line i reads line i-1 (uniform)
            const int j = asc ? i : n - 1 - i;
            const bool put = live && lane_on;

            float g[CH][K];
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
#pragma unroll
                for (int e = 0; e < K; ++e)
                    g[ch][e] = fmaf(masked(q.gy[ch].get(e), ml), masked(q.u[ch].get(e), ml), carry[ch][e]);
                store_f32<K>(put ? pl + ch * HW + (size_t)j * m + p0 : prm.sink + K * lane, g[ch]);
            }

            float ga[3][K];
            float cs0[SPLIT == 2 ? K : 1], cs2[SPLIT == 2 ? K : 1];   // SPLIT: w0 g, w2 g of line i
            if (coupled) {
                // tap-gradient differences summed over the chunk's channels:
                // E0 = sum g (h[p-1] - h[p]), E2 = sum g (h[p+1] - h[p])
                float ed[2][K];
#pragma unroll
                for (int e = 0; e < K; ++e) { ed[0][e] = 0.0f; ed[1][e] = 0.0f; }
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) {
                    float left = from_left(q.hp[ch][K - 1]);
                    float right = from_right(q.hp[ch][0]);
                    if constexpr (SPLIT == 2) {
                        // the lane exchange runs in every lane before the edge
                        // lanes take the other part's value (sunk into a
                        // branch it would read the masked-off lanes as 0)
                        asm volatile("" : "+v"(left), "+v"(right));
                        left = takes_left ? q.hx[ch] : left;
                        right = takes_right ? q.hx[ch] : right;
                    }
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const float hl = e == 0 ? left : q.hp[ch][e - 1];
                        const float hr = e == K - 1 ? right : q.hp[ch][e + 1];
                        ed[0][e] = fmaf(g[ch][e], hl - q.hp[ch][e], ed[0][e]);
                        ed[1][e] = fmaf(g[ch][e], hr - q.hp[ch][e], ed[1][e]);
                    }
                }
                // weights of line i and 1 - sigmoid of its taps
                float a0[K], a1[K], a2[K], w0[K], w1[K], w2[K], o0[K], o1[K], o2[K];
                float amin = 0.0f;
#pragma unroll
                for (int e = 0; e < K; ++e) {
                    a0[e] = masked(q.a[0].get(e), e == 0 ? m0 : ml);   // missing taps -> 0
                    a1[e] = masked(q.a[1].get(e), ml);
                    a2[e] = masked(q.a[2].get(e), e == K - 1 ? m2 : ml);
                    amin = fminf(amin, fminf(fminf(a0[e], a1[e]), a2[e]));
                }
                const float kNegLog2e = -1.44269504088896340736f;
                if (__builtin_amdgcn_ballot_w64(amin < -40.0f) == 0) {
                    // exp(-a) <= e^40: no overflow; 1 - sigmoid(a) = e * sigmoid(a)
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const float e0 = fast_exp2(a0[e] * kNegLog2e);
                        const float e1 = fast_exp2(a1[e] * kNegLog2e);
                        const float e2 = fast_exp2(a2[e] * kNegLog2e);
                        const float s0 = fast_rcp(1.0f + e0) * (e == 0 ? f0 : fl);
                        const float s1 = fast_rcp(1.0f + e1);
                        const float s2 = fast_rcp(1.0f + e2) * (e == K - 1 ? f2 : fl);
                        const float inv = fast_rcp(s0 + s1 + s2);
                        w0[e] = s0 * inv; w1[e] = s1 * inv; w2[e] = s2 * inv;
                        o0[e] = e0 * s0; o1[e] = e1 * s1; o2[e] = e2 * s2;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        const bool h0 = lane_on && p0 + e >= 1, h2 = lane_on && p0 + e + 1 < m;
                        const Taps tp = normalise_taps(a0[e], a1[e], a2[e], h0, h2);
                        w0[e] = tp.w0; w1[e] = tp.w1; w2[e] = tp.w2;
                        const float av[3] = {a0[e], a1[e], a2[e]};
                        float om[3];
#pragma unroll
                        for (int t = 0; t < 3; ++t) {
                            const float ex = fast_exp2(av[t] * kNegLog2e);   // may be inf
                            const float sg = fast_rcp(1.0f + ex);
                            om[t] = av[t] >= 0.0f ? ex * sg : 1.0f - sg;
                        }
                        o0[e] = om[0]; o1[e] = om[1]; o2[e] = om[2];
                    }
                }
                // D_t - sum_v w_v D_v without cancellation (weights sum to 1):
                //   t = 0: w1 E0 + w2 (E0 - E2); t = 1: -(w0 E0 + w2 E2);
                //   t = 2: w1 E2 + w0 (E2 - E0)
#pragma unroll
                for (int e = 0; e < K; ++e) {
                    const float E0 = ed[0][e], E2 = ed[1][e];
                    ga[0][e] = w0[e] * o0[e] * fmaf(w1[e], E0, w2[e] * (E0 - E2));
                    ga[1][e] = -(w1[e] * o1[e] * fmaf(w0[e], E0, w2[e] * E2));
                    ga[2][e] = w2[e] * o2[e] * fmaf(w1[e], E2, w0[e] * (E2 - E0));
                }
                // carry into line i-1: (w_i^T g_i)[p] = w1 g[p] + w0[p+1] g[p+1]
                // + w2[p-1] g[p-1], with w1 = 1 - w0 - w2 (SPLIT: after the
                // edge exchange below)
                if constexpr (SPLIT == 2) {
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        cs0[e] = w0[e] * g[0][e];
                        cs2[e] = w2[e] * g[0][e];
                    }
                } else
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) {
                    float c0[K], c2[K];
#pragma unroll
                    for (int e = 0; e < K; ++e) {
                        c0[e] = w0[e] * g[ch][e];
                        c2[e] = w2[e] * g[ch][e];
                    }
                    const float r0 = from_right(c0[0]);
                    const float l2 = from_left(c2[K - 1]);
#pragma unroll
                    for (int e = 0; e < K; ++e)
                        carry[ch][e] = (g[ch][e] - c0[e] - c2[e]) + (e == K - 1 ? r0 : c0[e + 1]) +
                                       (e == 0 ? l2 : c2[e - 1]);
                }
            } else {
                // first line of a group: its taps are unused, nothing flows on
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int e = 0; e < K; ++e) ga[t][e] = 0.0f;
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
#pragma unroll
                    for (int e = 0; e < K; ++e) carry[ch][e] = 0.0f;
                if constexpr (SPLIT == 2) {
#pragma unroll
                    for (int e = 0; e < K; ++e) { cs0[e] = 0.0f; cs2[e] = 0.0f; }
                }
            }
            if constexpr (SPLIT == 2) {
                // swap w2 g / w0 g at the common edge; the step parity
                // double-buffers the slots, so one barrier per step suffices
                const int par = (s0 + s) & 1;
                if (lane == (half == 0 ? 63 : 0)) xch[par][half] = half == 0 ? cs2[K - 1] : cs0[0];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                const float xo = xch[par][half ^ 1];
                float r0 = from_right(cs0[0]);
                float l2 = from_left(cs2[K - 1]);
                asm volatile("" : "+v"(r0), "+v"(l2));
                r0 = takes_right ? xo : r0;
                l2 = takes_left ? xo : l2;
                if (coupled) {
#pragma unroll
                    for (int e = 0; e < K; ++e)
                        carry[0][e] = (g[0][e] - cs0[e] - cs2[e]) + (e == K - 1 ? r0 : cs0[e + 1]) +
                                      (e == 0 ? l2 : cs2[e - 1]);
                }
            }
            if constexpr (ACC) {
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int e = 0; e < K; ++e) ga[t][e] += q.gp[t][e];
            }
            if constexpr (DIRECT) {
                T* gt = (is_row ? static_cast<T*>(prm.gw_out) : reinterpret_cast<T*>(prm.ga)) +
                        ((size_t)(slot * B + b) * Cw + k) * 3 * HW;
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    store_t<T, K>(put ? gt + t * HW + (size_t)j * m + p0 : reinterpret_cast<T*>(prm.sink) + K * lane,
                                  ga[t]);
            } else {
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    store_f32<K>(put ? gas + t * HW + (size_t)j * m + p0 : prm.sink + K * lane, ga[t]);
            }
            // refill the slot with the step kDepth ahead (clamped), after use
            load_step(buf[s], max(i - kDepth, 0));
        }
    }
}

// fp32 -> storage dtype, 8 elements per thread when `vec` (16-byte aligned,
// count % 8 == 0), else one.
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, size_t count,
                                                      int vec) {
    const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (vec) {
        const size_t e = tid * 8;
        if (e >= count) return;
        float f[8];
        const float4 v0 = *reinterpret_cast<const float4*>(src + e);
        const float4 v1 = *reinterpret_cast<const float4*>(src + e + 4);
        f[0] = v0.x; f[1] = v0.y; f[2] = v0.z; f[3] = v0.w; f[4] = v1.x; f[5] = v1.y; f[6] = v1.z; f[7] = v1.w;
        if constexpr (sizeof(T) == 2) {
            store16(dst + e, f);
        } else {
            const float a[4] = {f[0], f[1], f[2], f[3]}, c[4] = {f[4], f[5], f[6], f[7]};
            store16(dst + e, a);
            store16(dst + e + 4, c);
        }
        return;
    }
    if (tid < count) dst[tid] = from_f32(src[tid], (T*)nullptr);
}

// Lines longer than 256 (K = 8) are split over two waves with 4 positions
// each (the launch then has twice the waves, which balances scans that
// barely exceed one wave per SIMD, as in the forward).
template <typename T>
void launch_adjoint(const AdjointParams& p, int K, int CH, bool acc, bool direct, hipStream_t stream) {
    const long units = (long)p.nd * p.B * p.Cw;
    if (K == 8 && CH == 1) {
        const dim3 grid((unsigned)units), block(128);
        if (acc) hipLaunchKernelGGL((adjoint_scan_kernel<T, 4, 1, true, false, 2>), grid, block, 0, stream, p);
        else if (direct) hipLaunchKernelGGL((adjoint_scan_kernel<T, 4, 1, false, true, 2>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((adjoint_scan_kernel<T, 4, 1, false, false, 2>), grid, block, 0, stream, p);
        return;
    }
    const dim3 grid((unsigned)((units + 3) / 4)), block(256);
#define GSPN_ADJ(KK, CC)                                                                                          \
    if (K == KK && CH == CC) {                                                                                    \
        if (acc) hipLaunchKernelGGL((adjoint_scan_kernel<T, KK, CC, true, false, 1>), grid, block, 0, stream, p); \
        else if (direct)                                                                                          \
            hipLaunchKernelGGL((adjoint_scan_kernel<T, KK, CC, false, true, 1>), grid, block, 0, stream, p);      \
        else hipLaunchKernelGGL((adjoint_scan_kernel<T, KK, CC, false, false, 1>), grid, block, 0, stream, p);    \
        return;                                                                                                   \
    }
    GSPN_ADJ(1, 1) GSPN_ADJ(1, 2) GSPN_ADJ(1, 4) GSPN_ADJ(1, 8)
    GSPN_ADJ(2, 1) GSPN_ADJ(2, 2) GSPN_ADJ(2, 4)
    GSPN_ADJ(4, 1) GSPN_ADJ(4, 2)
#undef GSPN_ADJ
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BwdLayout {
    size_t planes, sink, xT, lamT, gyT, uT, wT, ga, total;
};

BwdLayout bwd_layout(const GradArgs& g) {
    const ScanArgs& a = g.fwd;
    const size_t E = (size_t)a.B * a.C * a.H * a.W;
    const size_t es = a.bf16 ? 2 : 4;
    int dos[4], ci[4], ncol = 0;
    const int nd = enabled_slots(a.dirs, dos, ci, &ncol);
    const size_t Ew = (size_t)a.B * (a.C / a.cpw) * 3 * a.H * a.W;
    BwdLayout l;
    size_t o = 0;
    l.planes = o; o += align256((size_t)nd * E * sizeof(float));
    l.sink = o;   o += align256(kSinkBytes);
    l.xT = l.lamT = l.gyT = l.uT = l.wT = 0;
    if (ncol) {
        l.xT = o;   o += align256(E * es);
        l.lamT = o; o += align256((a.lam_dir ? ncol : 1) * E * es);
        l.gyT = o;  o += align256(E * es);
        l.uT = o;   o += align256((a.u_dir ? ncol : 1) * E * es);
        l.wT = o;   o += align256((size_t)ncol * Ew * es);
    }
    l.ga = o; o += align256((size_t)nd * Ew * sizeof(float));
    l.total = o;
    return l;
}

template <typename T>
hipError_t launch_lines_bwd_t(const GradArgs& g, void* workspace, hipStream_t stream) {
    const ScanArgs& a = g.fwd;
    const int H = a.H, W = a.W;
    const int Cw = a.C / a.cpw;
    const BwdLayout l = bwd_layout(g);
    char* base = static_cast<char*>(workspace);
    float* planes = reinterpret_cast<float*>(base + l.planes);
    float* sink = reinterpret_cast<float*>(base + l.sink);
    T* xT = reinterpret_cast<T*>(base + l.xT);
    T* lamT = reinterpret_cast<T*>(base + l.lamT);
    T* gyT = reinterpret_cast<T*>(base + l.gyT);
    T* uT = reinterpret_cast<T*>(base + l.uT);
    T* wT = reinterpret_cast<T*>(base + l.wT);
    float* ga = reinterpret_cast<float*>(base + l.ga);

    LineParams p;
    p.x = a.x; p.lam = a.lam; p.w = a.w;
    p.xT = xT; p.lamT = lamT; p.wT = wT;
    p.planes = planes;
    p.sink = sink;
    const size_t E = (size_t)a.B * a.C * H * W;
    p.lam_ds = a.lam_dir ? E : 0;    // per-direction lambda: one slab per slot
    p.lamT_ds = a.lam_dir ? E : 0;   // and one transposed slab per column direction
    p.B = a.B; p.C = a.C; p.H = H; p.W = W; p.Cw = Cw; p.cpw = a.cpw; p.groups = a.groups;
    int ncol = 0;
    p.nd = enabled_slots(a.dirs, p.dir_of_slot, p.col_index, &ncol);
    const size_t slices = (size_t)a.B * a.C;
    const size_t wslab = (size_t)a.B * Cw * 3;          // [H][W] planes per slab
    const size_t HW = (size_t)H * W;

    // 1. column-major copies for LR / RL
    if (ncol > 0) {
        launch_transpose(static_cast<const T*>(a.x), xT, slices, H, W, stream);
        launch_transpose(static_cast<const T*>(g.gy), gyT, slices, H, W, stream);
        if (!a.lam_dir) launch_transpose(static_cast<const T*>(a.lam), lamT, slices, H, W, stream);
        if (!a.u_dir) launch_transpose(static_cast<const T*>(a.u), uT, slices, H, W, stream);
        for (int s = 0; s < p.nd; ++s) {
            if (p.dir_of_slot[s] < 2) continue;
            if (a.lam_dir)
                launch_transpose(static_cast<const T*>(a.lam) + (size_t)s * E, lamT + (size_t)p.col_index[s] * E,
                                 slices, H, W, stream);
            if (a.u_dir)
                launch_transpose(static_cast<const T*>(a.u) + (size_t)s * E, uT + (size_t)p.col_index[s] * E,
                                 slices, H, W, stream);
            launch_transpose(static_cast<const T*>(a.w) + (size_t)s * wslab * HW,
                             wT + (size_t)p.col_index[s] * wslab * HW, wslab, H, W, stream);
        }
    }
    // 2. forward states
    launch_line_scan<T>(p, stream);
    // 3. gu = gy * sum_dir h_dir, or gu_d = gy * h_d per direction
    MergeParams q;
    q.planes = planes;
    q.B = a.B; q.C = a.C; q.H = H; q.W = W; q.nd = p.nd;
    for (int s = 0; s < 4; ++s) q.dir_of_slot[s] = p.dir_of_slot[s];
    q.in[0] = g.gy; q.out[0] = g.gu; q.in[1] = nullptr; q.out[1] = nullptr;
    // one direction's plane: the merge of a single slot
    auto one_slot = [&](MergeParams m, int s) {
        m.planes = planes + (size_t)s * E;
        m.nd = 1;
        m.dir_of_slot[0] = p.dir_of_slot[s];
        return m;
    };
    if (a.u_dir) {
        for (int s = 0; s < p.nd; ++s) {
            MergeParams m = one_slot(q, s);
            m.out[0] = static_cast<T*>(g.gu) + (size_t)s * E;
            launch_merge<T, 1>(m, stream);
        }
    } else {
        launch_merge<T, 1>(q, stream);
    }
    // 4. adjoint scans, one launch per chunk of channels
    AdjointParams r;
    r.gy = g.gy; r.u = a.u; r.gyT = gyT; r.uT = uT; r.w = a.w; r.wT = wT;
    r.u_ds = a.u_dir ? E : 0;
    r.uT_ds = a.u_dir ? E : 0;
    r.planes = planes; r.ga = ga; r.sink = sink; r.gw_out = g.gw;
    r.B = a.B; r.C = a.C; r.H = H; r.W = W; r.Cw = Cw; r.cpw = a.cpw; r.groups = a.groups; r.nd = p.nd;
    for (int s = 0; s < 4; ++s) { r.dir_of_slot[s] = p.dir_of_slot[s]; r.col_index[s] = p.col_index[s]; }
    const int K = lines_positions_per_lane(H, W);
    int CH = 8 / K;
    while (a.cpw % CH) CH /= 2;
    const bool direct = a.cpw / CH == 1;   // one chunk: tap gradients rounded in the adjoint kernel
    for (int c = 0; c < a.cpw / CH; ++c) {
        r.chunk = c;
        launch_adjoint<T>(r, K, CH, c > 0, direct, stream);
    }
    // 5. gx = lam * G, glam = x * G; per-direction lambda:
    //    gx = sum_d lam_d * g_d, glam_d = x * g_d
    if (a.lam_dir) {
        q.in[0] = a.lam; q.out[0] = g.gx; q.in[1] = nullptr; q.out[1] = nullptr;
        launch_merge_dirs<T>(q, stream);
        for (int s = 0; s < p.nd; ++s) {
            MergeParams m = one_slot(q, s);
            m.in[0] = a.x;
            m.out[0] = static_cast<T*>(g.glam) + (size_t)s * E;
            launch_merge<T, 1>(m, stream);
        }
    } else {
        q.in[0] = a.lam; q.out[0] = g.gx; q.in[1] = a.x; q.out[1] = g.glam;
        launch_merge<T, 2>(q, stream);
    }
    // 6. tap gradients in the caller's layout and dtype (direct: only the
    //    column directions' line-major copies remain to be transposed)
    const size_t slab = wslab * HW;
    for (int s = 0; s < p.nd; ++s) {
        if (direct) {
            if (p.dir_of_slot[s] >= 2)
                launch_transpose(reinterpret_cast<const T*>(ga) + (size_t)s * slab, static_cast<T*>(g.gw) + (size_t)s * slab,
                                 wslab, W, H, stream);
            continue;
        }
        const float* src = ga + (size_t)s * slab;
        T* dst = static_cast<T*>(g.gw) + (size_t)s * slab;
        if (p.dir_of_slot[s] >= 2) {
            launch_transpose(src, dst, wslab, W, H, stream);   // [W][H] -> [H][W]
        } else {
            const int vec = slab % 8 == 0 && ((uintptr_t)dst & 15u) == 0;
            const size_t threads = vec ? slab / 8 : slab;
            hipLaunchKernelGGL(convert_kernel<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                               src, dst, slab, vec);
        }
    }
    return hipGetLastError();
}

}  // namespace

size_t lines_bwd_workspace_bytes(const GradArgs& g) { return bwd_layout(g).total; }

hipError_t launch_lines_bwd(const GradArgs& g, void* workspace, hipStream_t stream) {
    return g.fwd.bf16 ? launch_lines_bwd_t<uint16_t>(g, workspace, stream)
                      : launch_lines_bwd_t<float>(g, workspace, stream);
}

}  // namespace gspn
