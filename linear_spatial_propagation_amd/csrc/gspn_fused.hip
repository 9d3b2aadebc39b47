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
//    rcp per pixel) into registers (64 lines x 2 taps; the middle tap is
//    implied by the unit row sum) and reuses them for
//    every channel of the weight set: the sigmoid work is shared by the
//    channel group instead of being repeated per channel.  Row directions
//    stage their taps in chunks of 16 rows; column directions of bf16 grids
//    copy their whole tap block (whole 128-byte rows) straight into LDS and
//    normalise it from there, so no 128-byte line is fetched in pieces.
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
constexpr int kPitch = kS + 4;       // LDS row pitch (floats): rows 16-byte aligned; row
                                     // and 4-wide column accesses are conflict-free
constexpr int kPlane = kS * kPitch;  // floats per LDS plane
constexpr int kThreads = 256;
constexpr int kMaxBatch = 32;        // problems per batched launch (kernel-argument space)

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
    // layout strides in H*W planes: x / lam / u between batch items; w
    // between batch items and between direction slabs
    int x_bplanes, w_bplanes, w_splanes;
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

// y is written once and not read again by the kernel: stores are
// non-temporal (streamed out of the L2 instead of left dirty in it, which
// the end of the kernel would otherwise have to write back).
__device__ __forceinline__ void store_out(uint16_t* __restrict__ p, const float (&v)[8], int nvalid, bool vec) {
    if (vec) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 r = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
    } else {
        for (int j = 0; j < 8; ++j)
            if (j < nvalid) p[j] = from_f32(v[j], (uint16_t*)nullptr);
    }
}
__device__ __forceinline__ void store_out(float* __restrict__ p, const float (&v)[4], int nvalid, bool vec) {
    if (vec) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 r = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
    } else {
        for (int j = 0; j < 4; ++j)
            if (j < nvalid) p[j] = v[j];
    }
}

// 16-byte loads (16-byte aligned).  The kernel reads every input line once,
// as whole 128-byte lines.  Taps are loaded non-temporally (streamed through
// the caches instead of kept).  x, lambda and u rows are too when a weight set
// has several channels: measured on one GPU, non-temporal taps took cls56
// (cpw = 1) from 163.4 to 158.0 us and cgspn1k (cpw = 8) from 41.9 to 41.2 us;
// non-temporal rows as well took cgspn1k to 40.5 us but cls56 to 164.7 us.
template <typename T>
__device__ __forceinline__ uint4 load16(const T* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool NT, typename T>
__device__ __forceinline__ uint4 load16_rows(const T* p) {
    if constexpr (NT) return load16(p);
    else return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------- scan
// One part of one direction's scan of the channel held in X, on lane p.
//  ASC: lines are visited in increasing line coordinate j (TB: row j, LR:
//  column j); otherwise decreasing (BT, RL).  STRIDE: floats between
//  consecutive line coordinates in an LDS plane (65 for rows, 1 for
//  columns); X and P point at this lane's float at j = 0.  ADD: add h onto
//  the partner direction's stores instead of storing.  X (and P when
//  adding) are prefetched kDepth lines ahead.
//  The middle tap's weight is 1 - w0 - w2 (rows are stochastic), so one
//  step is h' = (h + xl) + w0 (h[p-1] - h) + w2 (h[p+1] - h): the lane
//  exchange fuses into the two subtractions (v_sub_f32 with a DPP source)
//  and only w0 and w2 occupy registers (64 lines x 2 per lane).
constexpr int kDepth = 4;

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ float line_step(float h, float xl, float w0, float w2) {
    const float dl = from_left(h) - h;
    const float dr = from_right(h) - h;
    float v = h + xl;
    v = fmaf(w0, dl, v);
    return fmaf(w2, dr, v);
}

// Static form: a global scan over exactly kS lines, scan steps [S0, S1).
template <bool ASC, int STRIDE, bool ADD, int S0, int S1>
__device__ __forceinline__ void scan_static(const float* __restrict__ X, float* __restrict__ P,
                                            const float (&w0)[kS], const float (&w2)[kS], float& h) {
    float xp[kDepth], pp[kDepth];
#pragma unroll
    for (int t = 0; t < kDepth; ++t) {
        const int j = ASC ? S0 + t : kS - 1 - (S0 + t);
        xp[t] = X[j * STRIDE];
        if (ADD) pp[t] = P[j * STRIDE];
    }
#pragma unroll
    for (int st = S0; st < S1; ++st) {
        const int j = ASC ? st : kS - 1 - st;
        const int slot = (st - S0) % kDepth;
        const float xl = xp[slot];
        const float pv = ADD ? pp[slot] : 0.0f;
        if (st + kDepth < S1) {
            const int jn = ASC ? j + kDepth : j - kDepth;
            xp[slot] = X[jn * STRIDE];
            if (ADD) pp[slot] = P[jn * STRIDE];
        }
        h = st == 0 ? xl : line_step(h, xl, w0[j], w2[j]);
        P[j * STRIDE] = ADD ? pv + h : h;
    }
}

// Static form for column directions (stride 1): the line coordinates of a
// lane are contiguous, so X and P move 4 lines per 16-byte LDS access; the
// next block is read while the current one is scanned.
template <bool ASC, bool ADD, int S0, int S1>
__device__ __forceinline__ void scan_static_cols(const float* __restrict__ X, float* __restrict__ P,
                                                 const float (&w0)[kS], const float (&w2)[kS],
                                                 float& h) {
    static_assert(S0 % 4 == 0 && S1 % 4 == 0, "blocks of 4 lines");
    constexpr int kBlocks = (S1 - S0) / 4;
    const float4* X4 = reinterpret_cast<const float4*>(X);
    float4* P4 = reinterpret_cast<float4*>(P);
    // block of the i-th group of 4 scan steps
#define GSPN_BLK(i) (ASC ? (S0 / 4 + (i)) : (kS / 4 - 1 - (S0 / 4 + (i))))
    float4 xc = X4[GSPN_BLK(0)], xn = xc;
    float4 pc = ADD ? P4[GSPN_BLK(0)] : xc, pn = pc;
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
        if (i + 1 < kBlocks) {
            xn = X4[GSPN_BLK(i + 1)];
            if (ADD) pn = P4[GSPN_BLK(i + 1)];
        }
        const float xs[4] = {xc.x, xc.y, xc.z, xc.w};
        const float ps[4] = {pc.x, pc.y, pc.z, pc.w};
        float hs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = ASC ? q : 3 - q;          // element of the block, in scan order
            const int st = S0 + 4 * i + q;          // scan step
            const int j = GSPN_BLK(i) * 4 + e;      // line coordinate
            h = st == 0 ? xs[e] : line_step(h, xs[e], w0[j], w2[j]);
            hs[e] = ADD ? ps[e] + h : h;
        }
        P4[GSPN_BLK(i)] = make_float4(hs[0], hs[1], hs[2], hs[3]);
        xc = xn;
        pc = pn;
    }
#undef GSPN_BLK
}

// General form: any line count n <= kS and group length L.  The loop is
// unrolled over all kS line coordinates so the weight registers and LDS
// offsets stay static; `skip` and `cnt` (uniform) select which of them this
// part processes and `gpos` is the scan step's position in its group.  They
// are kept opaque to the optimiser so the per-line conditions are evaluated
// in the loop with scalar instructions instead of being precomputed.
template <bool ASC, int STRIDE, bool ADD>
__device__ __forceinline__ void scan_general(const float* __restrict__ X, float* __restrict__ P,
                                             const float (&w0)[kS], const float (&w2)[kS], int L,
                                             int skip, int cnt, int& gpos, float& h) {
    float xp[kDepth], pp[kDepth];
#pragma unroll
    for (int t = 0; t < kDepth; ++t) {
        const int j = ASC ? t : kS - 1 - t;
        xp[t] = X[j * STRIDE];
        if (ADD) pp[t] = P[j * STRIDE];
    }
#pragma unroll
    for (int t = 0; t < kS; ++t) {
        const int j = ASC ? t : kS - 1 - t;
        const float xl = xp[t % kDepth];
        const float pv = ADD ? pp[t % kDepth] : 0.0f;
        if (t + kDepth < kS) {
            const int jn = ASC ? j + kDepth : j - kDepth;
            xp[t % kDepth] = X[jn * STRIDE];
            if (ADD) pp[t % kDepth] = P[jn * STRIDE];
        }
        asm volatile("" : "+s"(skip), "+s"(cnt), "+s"(gpos));
        if (skip > 0) {
            --skip;
        } else if (cnt > 0) {
            --cnt;
            h = gpos == 0 ? xl : line_step(h, xl, w0[j], w2[j]);
            gpos = gpos + 1 == L ? 0 : gpos + 1;
            P[j * STRIDE] = ADD ? pv + h : h;
        }
    }
}

struct ScanCtl {
    int d;          // direction 0..3 (TB, BT, LR, RL)
    int p;          // lane = position on the line
    bool fast;      // global scan (one group) with both directions of the pair on
    int L;          // lines per group
    int skip1, cnt1, skip2, cnt2;  // general form: store part, add part
};

template <int D, bool ADD>
__device__ __forceinline__ void scan_dir(const ScanCtl& k, const float* X, float* P, const float (&w0)[kS],
                                         const float (&w2)[kS], int& gpos, float& h) {
    constexpr bool kAsc = (D == 0 || D == 2);
    constexpr int kStride = D < 2 ? kPitch : 1;
    const int base = D < 2 ? k.p : k.p * kPitch;
    if (k.fast) {
        if (D >= 2) {
            if (ADD) scan_static_cols<kAsc, true, kS / 2, kS>(X + base, P + base, w0, w2, h);
            else scan_static_cols<kAsc, false, 0, kS / 2>(X + base, P + base, w0, w2, h);
        } else {
            if (ADD) scan_static<kAsc, kStride, true, kS / 2, kS>(X + base, P + base, w0, w2, h);
            else scan_static<kAsc, kStride, false, 0, kS / 2>(X + base, P + base, w0, w2, h);
        }
    } else {
        scan_general<kAsc, kStride, ADD>(X + base, P + base, w0, w2, k.L, ADD ? k.skip2 : k.skip1,
                                         ADD ? k.cnt2 : k.cnt1, gpos, h);
    }
}

template <bool ADD>
__device__ __forceinline__ void scan_any(const ScanCtl& k, const float* X, float* P, const float (&w0)[kS],
                                         const float (&w2)[kS], int& gpos, float& h) {
    switch (k.d) {
        case 0: scan_dir<0, ADD>(k, X, P, w0, w2, gpos, h); break;
        case 1: scan_dir<1, ADD>(k, X, P, w0, w2, gpos, h); break;
        case 2: scan_dir<2, ADD>(k, X, P, w0, w2, gpos, h); break;
        default: scan_dir<3, ADD>(k, X, P, w0, w2, gpos, h); break;
    }
}

// ---------------------------------------------------------------- staging
// Raw taps of one (b, k).  Direction dd's [3][H][W] block is found by
// arithmetic from the global base pointer (no table of pointers), so the
// compiler keeps the accesses global loads, which only the vector-memory
// counter tracks (loads through a generic pointer would also hold the LDS
// counter and serialise every LDS wait behind them).
__device__ __forceinline__ int first_dir(uint32_t dirs) { return __builtin_ctz(dirs); }

template <typename T>
struct TapSrc {
    const T* w;
    uint32_t dirs;
    int splanes, bplanes, b, k, HW;   // planes between direction slabs / batch items
    __device__ __forceinline__ const T* dir(int dd) const {
        const int slab = __builtin_popcount(dirs & ((1u << dd) - 1u));
        return w + ((size_t)slab * splanes + (size_t)b * bplanes + (size_t)k * 3) * (size_t)HW;
    }
};

// Raw taps of 16 line coordinates [j0, j0+16) of the calling wave's own
// direction d, loaded as 16-byte vectors (rows that are whole vectors
// only) and staged in the wave's own LDS region S[d][tap][jj][position]
// (fp32, pitch kPitch).  Since every wave stages and reads only its own
// direction, the prologue needs no workgroup barrier between chunks.
//   Row directions: lane -> (line jj, vector along the row), 8 lanes per
//   128-byte row.  Column directions: lane -> (row r, vector along the 16
//   columns), written transposed.
template <typename T>
struct TapChunk {
    static constexpr int N = Vec<T>::N;
    static constexpr int kChunk = 16;
    static constexpr int kVPR = kS / N;                 // vectors per 64-wide row
    static constexpr int kPerTap = kChunk * kVPR;       // vectors per tap and chunk
    static constexpr int kLoads = 3 * kPerTap / 64;     // per lane
    uint4 v[kLoads];

    struct Slot {
        int t, r, c;
        bool ok;   // direction enabled and the vector inside the grid
    };
    __device__ __forceinline__ static Slot slot(int i, int d, uint32_t dirs, int j0, int H, int W, int lane) {
        const int u = lane + 64 * i;
        Slot q;
        q.t = u / kPerTap;
        const int e = u % kPerTap;
        if (d < 2) { q.r = j0 + e / kVPR; q.c = (e % kVPR) * N; }
        else { q.r = e / (kChunk / N); q.c = j0 + (e % (kChunk / N)) * N; }
        q.ok = ((dirs >> d) & 1u) && q.r < H && q.c + N <= W;
        return q;
    }
    // Staged values are sanitised for normalise_fast: besides everything
    // outside the grid, the taps that are never used -- a missing tap (tap
    // 0 at position 0, tap 2 at position m-1) and all taps of the scan's
    // first line -- are staged as 0.  Row directions: line = row, position
    // = column; column directions: the other way round.
    __device__ __forceinline__ static bool vector_used(const Slot& q, int d, int first_line, int H) {
        if (d < 2) return q.r != first_line;
        return !((q.t == 0 && q.r == 0) || (q.t == 2 && q.r == H - 1));
    }
    // The load is unconditional, from an address clamped into the tensor;
    // store() zeroes what lies outside.  (A load under a divergent branch
    // makes the compiler's memory-counter waits conservative.)
    __device__ __forceinline__ void load_one(int i, const TapSrc<T>& wsrc, int d, uint32_t dirs, int j0, int H,
                                             int W, int HW, int lane) {
        const Slot q = slot(i, d, dirs, j0, H, W, lane);
        const int dd = ((dirs >> d) & 1u) ? d : first_dir(dirs);
        const T* src = wsrc.dir(dd) + (size_t)q.t * HW + min(q.r, H - 1) * W + min(q.c, W - N);
        v[i] = load16(src);
    }
    __device__ __forceinline__ void load(const TapSrc<T>& wsrc, int d, uint32_t dirs, int j0, int H, int W,
                                         int HW, int lane) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) load_one(i, wsrc, d, dirs, j0, H, W, HW, lane);
    }
    // Write as fp32 into the wave's region Sd = S[d] ([tap][jj][position]).
    __device__ __forceinline__ void store(float* Sd, int d, uint32_t dirs, int j0, int H, int W, int first_line,
                                          int lane) const {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const Slot q = slot(i, d, dirs, j0, H, W, lane);
            uint32_t m = q.ok && vector_used(q, d, first_line, H) ? 0xffffffffu : 0u;
            asm volatile("" : "+v"(m));   // opaque, so the load above stays unconditional
            float f[N];
            unpack(make_uint4(v[i].x & m, v[i].y & m, v[i].z & m, v[i].w & m), f);
            // unused elements at the vector's ends
            if (d < 2) {
                if (q.t == 0 && q.c == 0) f[0] = 0.0f;               // position 0 has no tap 0
                if (q.t == 2 && q.c + N == W) f[N - 1] = 0.0f;       // position W-1 has no tap 2
            } else {
                if (q.c == first_line) f[0] = 0.0f;                  // first line (column)
                if (q.c + N - 1 == first_line) f[N - 1] = 0.0f;
            }
            float* St = Sd + q.t * kChunk * kPitch;
            if (d < 2) {
                const int jj = q.r - j0;
#pragma unroll
                for (int e = 0; e < N; ++e) St[jj * kPitch + q.c + e] = f[e];
            } else {
                const int jj0 = q.c - j0;
#pragma unroll
                for (int e = 0; e < N; ++e) St[(jj0 + e) * kPitch + q.r] = f[e];
            }
        }
    }
};

// Element-wise staging of the same chunk into the wave's own region (rows
// that are not whole vectors).
template <typename T>
__device__ __forceinline__ void stage_taps_scalar(float* Sd, const TapSrc<T>& wsrc, int d, uint32_t dirs, int j0,
                                                  int H, int W, int HW, int first_line, int lane) {
    constexpr int kChunk = 16;
    if (!((dirs >> d) & 1u)) return;
    const T* src = wsrc.dir(d);
    for (int jj = 0; jj < kChunk; ++jj) {
        // row directions: line = row j0+jj, lane = column; column
        // directions: line = column j0+jj, lane = row
        const int r = d < 2 ? j0 + jj : lane;
        const int q = d < 2 ? lane : j0 + jj;
        const int line = d < 2 ? r : q, pos = d < 2 ? q : r, m = d < 2 ? W : H;
        const bool ok = r < H && q < W && line != first_line;
        for (int t = 0; t < 3; ++t) {
            // unused taps are staged as 0 (see TapChunk::vector_used)
            const bool used = ok && !(t == 0 && pos == 0) && !(t == 2 && pos == m - 1);
            Sd[(t * kChunk + jj) * kPitch + lane] = used ? to_f32(src[(size_t)t * HW + r * W + q]) : 0.0f;
        }
    }
}

// ---------------------------------------------------------------- kernel
// The work of workgroup `wg` of one problem.  VEC: every row is a whole
// number of 16-byte vectors (W % N == 0).  NTR: x, lambda and u rows are
// loaded non-temporally.
template <typename T, bool VEC, bool NTR>
__device__ __forceinline__ void fused_scan_body(const FusedParams& prm, const int wg) {
    constexpr int N = Vec<T>::N;                     // elements per 16-byte access
    constexpr int kMaxIt = kS * kS / (kThreads * N); // merge/staging iterations
    constexpr int kChunk = 16;
    // bf16 rows of whole vectors: the column directions copy their raw taps
    // straight into LDS in the prologue (see column_prologue below)
    constexpr bool kColDirect = VEC && sizeof(T) == 2;
    // that copy: 3 taps x 64 rows of 144 bytes (a 128-byte bf16 row + 16
    // bytes of padding) per column direction, after the two row waves'
    // fp32 staging regions
    constexpr int kRowStageBytes = 2 * 3 * kChunk * kPitch * 4;
    constexpr int kColRowBytes = 144;
    constexpr int kColRegionBytes = 3 * kS * kColRowBytes;
    constexpr int kLdsFloats = kColDirect ? (kRowStageBytes + 2 * kColRegionBytes) / 4 : 3 * kPlane;
    static_assert(kLdsFloats >= 3 * kPlane, "the prologue's LDS also holds the three planes");
    // LDS: XL (lambda*x of the current channel, fp32) | P_row | P_col; the
    // tap staging of the prologue reuses the same space.
    __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];

    const T* __restrict__ gx = static_cast<const T*>(prm.x);
    const T* __restrict__ gw = static_cast<const T*>(prm.w);
    const T* __restrict__ glam = static_cast<const T*>(prm.lam);
    const T* __restrict__ gu = static_cast<const T*>(prm.u);
    T* __restrict__ gy = static_cast<T*>(prm.y);

    const int H = prm.H, W = prm.W, C = prm.C, Cw = prm.Cw;
    const int HW = H * W;
    const uint32_t dirs = prm.dirs;
    constexpr bool vec = VEC;

    // ---- which (b, k, chunk) this workgroup owns
    const int chunk = wg % prm.nchunk;
    const int bk = wg / prm.nchunk;
    const int k = bk % Cw;
    const int b = bk / Cw;
    const int c_begin = k * prm.cpw + chunk * prm.chunk_len;
    const int c_end = min(c_begin + prm.chunk_len, (k + 1) * prm.cpw);

    // ---- this wave's direction; lane p = position on the line
    const int tid = threadIdx.x;
    const int d = uniform(tid >> 6);
    const int p = tid & 63;
    const bool is_row = d < 2;
    const bool asc = (d == 0 || d == 2);
    const bool on = (dirs >> d) & 1u;
    const bool partner_on = (dirs >> (d ^ 1)) & 1u;
    const int n = is_row ? H : W;      // lines
    const int m = is_row ? W : H;      // positions per line
    const int L = n / prm.groups;      // lines per group
    // Taps toward p-1 / p+1 exist.  Lanes past the line (p >= m) get
    // neither, so their weights are w0 = w2 = 0 and their state stays 0.
    const bool has0 = p >= 1 && p < m;
    const bool has2 = p + 1 < m;

    // ---- x / lambda / u rows: N elements per thread
    const int tpr = (W + N - 1) / N;         // threads per row
    const int rpi = kThreads / tpr;          // rows per iteration
    const int tr = tid / tpr;
    const int tc = tid - tr * tpr;
    const int col0 = tc * N;
    const int nvalid = min(N, W - col0);
    const bool t_active = tr < rpi;
    const bool row_any = (dirs & 3u) != 0;
    const bool col_any = (dirs & 12u) != 0;
    auto load_rows = [&](const T* __restrict__ g, int c, uint4 (&dst)[kMaxIt]) {
        const T* __restrict__ sl = g + ((size_t)b * prm.x_bplanes + c) * (size_t)HW;
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int r = tr + it * rpi;
            if constexpr (VEC) {
                // unconditional, row clamped (see TapChunk::load_one)
                dst[it] = load16_rows<NTR>(sl + min(r, H - 1) * W + col0);
            } else {
                if (t_active && r < H) dst[it] = load_raw(sl + r * W + col0, nvalid, vec);
            }
        }
    };
    // XL <- lambda * x (fp32, pitch kPitch)
    auto write_xl = [&](const uint4 (&xs)[kMaxIt], const uint4 (&ls)[kMaxIt]) {
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int r = tr + it * rpi;
            if (t_active && r < H) {
                float xv[N], lv[N];
                unpack(xs[it], xv);
                unpack(ls[it], lv);
                if (vec) {
                    float4* dst = reinterpret_cast<float4*>(lds + r * kPitch + col0);
#pragma unroll
                    for (int j = 0; j < N; j += 4)
                        dst[j / 4] = make_float4(xv[j] * lv[j], xv[j + 1] * lv[j + 1], xv[j + 2] * lv[j + 2],
                                                 xv[j + 3] * lv[j + 3]);
                } else {
#pragma unroll
                    for (int j = 0; j < N; ++j)
                        if (j < nvalid) lds[r * kPitch + col0 + j] = xv[j] * lv[j];
                }
            }
        }
    };

    // x / lambda of the next channel and u of the current one travel in
    // registers; the first channel's loads are in flight during the prologue
    uint4 x1[kMaxIt], l1[kMaxIt], u0[kMaxIt];

    // ---- prologue: normalised taps of this direction, indexed by line
    // coordinate j (row for TB/BT, column for LR/RL).  Each wave stages the
    // taps of 16 line coordinates of its own direction in its own LDS
    // region as fp32 [tap][j][position] (pitch kPitch), transposed for
    // LR/RL, and reads them along its lanes: no workgroup barrier is needed
    // between chunks, so waves do not wait on each other's loads.  Entries
    // outside the grid are staged as 0, which keeps idle lanes finite.
    //
    // Load schedule (whole-vector rows): chunk 0 is loaded up front; the
    // loads of chunks 1.. and then of the first channel's x / lambda / u
    // rows are issued one at a time between normalised lines, kSlots per
    // chunk, so that the memory pipe stays busy while the VALU normalises
    // and no wave stalls on a long burst of loads.
    float w0[kS], w2[kS];
    const int first_line = asc ? 0 : n - 1;
    {
        float* S = lds;   // [4][3][kChunk][kPitch]
        const TapSrc<T> wsrc{gw, dirs, prm.w_splanes, prm.w_bplanes, b, k, HW};
        constexpr int kNCh = kS / kChunk;
        constexpr int kLd = TapChunk<T>::kLoads;
#ifndef GSPN_TAP_AHEAD
#define GSPN_TAP_AHEAD 3
#endif
#ifndef GSPN_SLOTS
#define GSPN_SLOTS 8
#endif
        // Chunks loaded up front: three, or two when a weight set has one
        // channel (the instantiation without non-temporal rows, NTR false):
        // there the taps are three quarters of the bytes and the first chunk
        // arrives sooner when fewer compete with it (cls56 155.5-156.0 ->
        // 153.4-153.9 us in steady state on one GPU, same bits; cgspn1k is
        // best with three).
        constexpr int kAhead = NTR ? GSPN_TAP_AHEAD : 2;
        constexpr int kTapItems = (kNCh - kAhead) * kLd;     // items [0, kTapItems): tap loads of chunks kAhead..
        constexpr int kItems = kTapItems + 3 * kMaxIt;       // then x, lambda, u rows
        constexpr int kSlots = (kItems + kNCh - 1) / kNCh > GSPN_SLOTS ? (kItems + kNCh - 1) / kNCh : GSPN_SLOTS;
        constexpr int kSlotStep = kSlots <= kChunk / 2 ? 2 : 1;   // odd lines when they fit
        static_assert(kSlots <= kChunk && kItems <= kSlots * kNCh, "issue slots");
        static_assert(kAhead > 1 || kSlots >= kLd, "chunk c + 1 is issued while chunk c is normalised");
        // Column directions of bf16 rows (whole vectors): the wave copies all
        // of its direction's raw taps (3 x 64 rows of 128 bytes) into LDS
        // with direct global-to-LDS loads, 16 bytes per lane, whole 128-byte
        // rows -- the chunks of 16 columns the row path uses would read each
        // 128-byte line in four 32-byte pieces, at different times -- and
        // then normalises 8 line coordinates (columns) per 16-byte LDS read
        // of its own row (lane p = row p; the 144-byte row pitch keeps those
        // reads free of bank conflicts).  Taps that are never used (outside
        // the grid, a missing border tap, the scan's first line) are zeroed
        // on the way into normalise_fast, as the row path's staging does.
        auto column_prologue = [&]() {
            constexpr int kBlocks = kColRegionBytes / 1024;   // 1 KB per wave-wide copy
            static_assert(kColRegionBytes % 1024 == 0, "whole 1 KB blocks");
            char* region = reinterpret_cast<char*>(lds) + kRowStageBytes + (d - 2) * kColRegionBytes;
            // The first channel's x / lambda / u rows are requested before the
            // copies, so that they travel with them.  Requested after the
            // copies, they started only once a wait for the copies (which the
            // compiler places before it reuses the copies' address registers)
            // had passed, and the wait below then took a second memory round
            // trip: per-wave timestamps showed the column waves ending the
            // prologue last in every workgroup.  cls56 166-168 -> 161-165 us
            // on one GPU, same bits; cgspn1k unchanged.
            load_rows(gx, c_begin, x1);
            load_rows(glam, c_begin, l1);
            load_rows(gu, c_begin, u0);
            if (on) {
                const T* src = wsrc.dir(d);
                const int vpr = W / N;   // 16-byte pieces per row
#pragma unroll
                for (int i = 0; i < kBlocks; ++i) {
                    // 16-byte slot i*64 + p of the region: LDS row lr (tap
                    // lr / 64, grid row lr % 64), piece kk of 9 (piece 8 is
                    // padding and repeats piece 7); rows and pieces outside
                    // the grid read clamped addresses and are masked below
                    const int sl = i * 64 + p;
                    const int lr = sl / 9, kk = sl - lr * 9;
                    const T* g = src + (size_t)(lr >> 6) * HW + min(lr & 63, H - 1) * W + min(kk, vpr - 1) * N;
#if defined(__HIP_DEVICE_COMPILE__)
                    __builtin_amdgcn_global_load_lds(g, region + i * 1024, 16, 0, 0);
#endif
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies have landed in LDS
            const bool has1 = p < m;
            static_for<0, kS / 8>([&](auto gc) {
                constexpr int g8 = decltype(gc)::value;
                __builtin_amdgcn_sched_barrier(0);
                float a0[8], a1[8], a2[8];
                unpack(*reinterpret_cast<const uint4*>(region + (0 * kS + p) * kColRowBytes + g8 * 16), a0);
                unpack(*reinterpret_cast<const uint4*>(region + (1 * kS + p) * kColRowBytes + g8 * 16), a1);
                unpack(*reinterpret_cast<const uint4*>(region + (2 * kS + p) * kColRowBytes + g8 * 16), a2);
                float amin = 0.0f;
                static_for<0, 8>([&](auto ec) {
                    constexpr int e = decltype(ec)::value;
                    constexpr int j = g8 * 8 + e;   // line coordinate (column)
                    const bool used = on && j < W && j != first_line;
                    a0[e] = used && has0 ? a0[e] : 0.0f;
                    a1[e] = used && has1 ? a1[e] : 0.0f;
                    a2[e] = used && has2 ? a2[e] : 0.0f;
                    amin = fminf(amin, fminf(fminf(a0[e], a1[e]), a2[e]));
                    const float2 w = normalise_fast(a0[e], a1[e], a2[e], has0, has2);
                    w0[j] = w.x;
                    w2[j] = w.y;
                });
                // a tap below -40 in these 8 columns: the exact-form branches
                if (__builtin_amdgcn_ballot_w64(amin < -40.0f) != 0) {
                    static_for<0, 8>([&](auto ec) {
                        constexpr int e = decltype(ec)::value;
                        const Taps tp = normalise_taps(a0[e], a1[e], a2[e], has0, has2);
                        w0[g8 * 8 + e] = tp.w0;
                        w2[g8 * 8 + e] = tp.w2;
                    });
                }
            });
        };
        // Row directions (and every direction of other instantiations):
        // chunks of 16 line coordinates staged as fp32 in the wave's region.
        auto chunked_prologue = [&]() {
        TapChunk<T> tapv[kNCh];
        if constexpr (VEC) {
#pragma unroll
            for (int ch = 0; ch < kAhead; ++ch) tapv[ch].load(wsrc, d, dirs, ch * kChunk, H, W, HW, p);
        } else {
            load_rows(gx, c_begin, x1);
            load_rows(glam, c_begin, l1);
            load_rows(gu, c_begin, u0);
        }
        static_for<0, kNCh>([&](auto chc) {
            constexpr int ch = decltype(chc)::value;
            constexpr int j0 = ch * kChunk;
            float* const Sd = S + d * 3 * kChunk * kPitch;   // this wave's region
            if constexpr (VEC) tapv[ch].store(Sd, d, dirs, j0, H, W, first_line, p);
            else stage_taps_scalar<T>(Sd, wsrc, d, dirs, j0, H, W, HW, first_line, p);
            const float* Sw = Sd + p;
            float amin = 0.0f;   // smallest staged tap of this chunk (staged unused taps are 0)
            static_for<0, kChunk>([&](auto jjc) {
                constexpr int jj = decltype(jjc)::value;
                constexpr int g = kSlots * ch + jj / kSlotStep;   // item issued before this line
                if constexpr (VEC && jj % kSlotStep == kSlotStep - 1 && jj / kSlotStep < kSlots && g < kItems) {
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (g < kTapItems) {
                        constexpr int cn = kAhead + g / kLd;
                        tapv[cn].load_one(g % kLd, wsrc, d, dirs, cn * kChunk, H, W, HW, p);
                    } else {
                        constexpr int q = g - kTapItems;
                        constexpr int it = q % kMaxIt;
                        const int r = min(tr + it * rpi, H - 1);
                        const size_t o = ((size_t)b * prm.x_bplanes + c_begin) * (size_t)HW + r * W + col0;
                        if constexpr (q / kMaxIt == 0) x1[it] = load16_rows<NTR>(gx + o);
                        else if constexpr (q / kMaxIt == 1) l1[it] = load16_rows<NTR>(glam + o);
                        else u0[it] = load16_rows<NTR>(gu + o);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                const float a0 = Sw[jj * kPitch], a1 = Sw[(kChunk + jj) * kPitch], a2 = Sw[(2 * kChunk + jj) * kPitch];
                amin = fminf(amin, fminf(fminf(a0, a1), a2));
                const float2 w = normalise_fast(a0, a1, a2, has0, has2);
                w0[j0 + jj] = w.x;
                w2[j0 + jj] = w.y;
            });
            // a tap below -40 anywhere in the wave's chunk: redo the chunk
            // with the exact-form branches (rare: N(0,1) taps never get there)
            if (__builtin_amdgcn_ballot_w64(amin < -40.0f) != 0) {
                static_for<0, kChunk>([&](auto jjc) {
                    constexpr int jj = decltype(jjc)::value;
                    const Taps tp = normalise_taps(Sw[jj * kPitch], Sw[(kChunk + jj) * kPitch],
                                                   Sw[(2 * kChunk + jj) * kPitch], has0, has2);
                    w0[j0 + jj] = tp.w0;
                    w2[j0 + jj] = tp.w2;
                });
            }
        });
        };
        if (kColDirect && d >= 2) column_prologue();
        else chunked_prologue();
        __syncthreads();   // every wave is done with the staging area (it becomes XL)
    }

    // padding rows/columns of XL must read as zero
    {
        float4* z = reinterpret_cast<float4*>(lds);
        for (int i = tid; i < kPlane / 4; i += kThreads) z[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    write_xl(x1, l1);
    __syncthreads();

    float* const Pl = lds + (is_row ? 1 : 2) * kPlane;
    const int nstore = partner_on ? ((d & 1) ? n / 2 : (n + 1) / 2) : n;
    ScanCtl ctl;
    ctl.d = d;
    ctl.p = p;
    // The static form runs all kS lines of the padded 64 x 64 planes.  With
    // fewer lines or positions it is still exact: padded XL is zero, padded
    // lanes keep h = 0 (w0 = w2 = 0), and a descending scan meets its first
    // real line with h = 0, so that line gets h = lambda x, the restart.
    ctl.fast = L == n && partner_on;
    ctl.L = L;
    ctl.skip1 = asc ? 0 : kS - n;          // general form: first visited
    ctl.cnt1 = nstore;                     // line coordinate is 0 (asc)
    ctl.skip2 = ctl.skip1 + nstore;        // or n-1 (desc)
    ctl.cnt2 = n - nstore;

    for (int c = c_begin; c < c_end; ++c) {
        // Next channel's x / lambda (and below u) are loaded without a
        // condition: the last channel reloads itself (a cache hit) and the
        // XL it writes is never read.  Loads and their use under separate
        // conditions would make the compiler's counter waits at the loop
        // head conservative (waiting for u in flight).
        const int cn = min(c + 1, c_end - 1);
        load_rows(gx, cn, x1);
        load_rows(glam, cn, l1);

        // ---- scan: the first part stores, the second adds onto the partner
        float h = 0.0f;
        int gpos = 0;
        if (on) scan_any<false>(ctl, lds, Pl, w0, w2, gpos, h);
        __syncthreads();
        if (on) scan_any<true>(ctl, lds, Pl, w0, w2, gpos, h);
        __syncthreads();

        // ---- merge: y = u * (P_row + P_col); then XL <- next channel
        {
            T* __restrict__ ys = gy + ((size_t)b * C + c) * (size_t)HW;
            const float* PR = lds + kPlane;
            const float* PC = lds + 2 * kPlane;
            if (vec && row_any && col_any) {
#pragma unroll
                for (int it = 0; it < kMaxIt; ++it) {
                    const int r = tr + it * rpi;
                    const int o = min(r, H - 1) * kPitch + col0;   // rows past H are read, not stored
                    float uv[N], yv[N];
                    unpack(u0[it], uv);
#pragma unroll
                    for (int j = 0; j < N; j += 4) {
                        const float4 a = *reinterpret_cast<const float4*>(PR + o + j);
                        const float4 e = *reinterpret_cast<const float4*>(PC + o + j);
                        yv[j] = uv[j] * (a.x + e.x);
                        yv[j + 1] = uv[j + 1] * (a.y + e.y);
                        yv[j + 2] = uv[j + 2] * (a.z + e.z);
                        yv[j + 3] = uv[j + 3] * (a.w + e.w);
                    }
                    if (t_active && r < H) store_out(ys + r * W + col0, yv, N, true);
                }
            } else {
#pragma unroll
                for (int it = 0; it < kMaxIt; ++it) {
                    const int r = tr + it * rpi;
                    if (t_active && r < H) {
                        float uv[N], yv[N];
                        unpack(u0[it], uv);
#pragma unroll
                        for (int j = 0; j < N; ++j) {
                            const int o = r * kPitch + col0 + j;
                            float acc = 0.0f;
                            if (vec || j < nvalid) {
                                if (row_any) acc = PR[o];
                                if (col_any) acc += PC[o];
                            }
                            yv[j] = uv[j] * acc;
                        }
                        store_out(ys + r * W + col0, yv, nvalid, vec);
                    }
                }
            }
        }
        write_xl(x1, l1);
        load_rows(gu, cn, u0);
        __syncthreads();
    }
}

template <typename T, bool VEC, bool NTR>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fused_scan_kernel(FusedParams prm) {
    fused_scan_body<T, VEC, NTR>(prm, blockIdx.x);
}

// Several independent problems in one launch: problem i owns workgroups
// [wg_begin[i], wg_begin[i+1]).  Small problems then share the GPU instead
// of each leaving most of it idle.
struct FusedBatch {
    FusedParams p[kMaxBatch];
    int wg_begin[kMaxBatch + 1];
    int count;
};

template <typename T, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fused_scan_batched_kernel(FusedBatch bat) {
    const int wg = blockIdx.x;
    int i = 0;
    while (i + 1 < bat.count && wg >= bat.wg_begin[i + 1]) ++i;   // uniform
    fused_scan_body<T, VEC, false>(bat.p[i], wg - bat.wg_begin[i]);
}

// Channel chunks per weight set: split a set's channels over several
// workgroups only when there are too few (b, k) pairs in the launch to
// occupy the GPU (two workgroups per CU).
void set_chunks(FusedParams& p, long sets_in_launch) {
    const long want = 512;
    int nchunk = 1;
    if (sets_in_launch < want) nchunk = (int)std::min<long>(p.cpw, (want + sets_in_launch - 1) / sets_in_launch);
    p.chunk_len = (p.cpw + nchunk - 1) / nchunk;
    p.nchunk = (p.cpw + p.chunk_len - 1) / p.chunk_len;
}

FusedParams fused_params(const ScanArgs& a) {
    FusedParams p;
    p.x = a.x; p.w = a.w; p.lam = a.lam; p.u = a.u; p.y = a.y;
    p.B = a.B; p.C = a.C; p.H = a.H; p.W = a.W;
    p.cpw = a.cpw; p.Cw = a.C / a.cpw; p.groups = a.groups; p.dirs = a.dirs;
    p.x_bplanes = a.x_bplanes ? a.x_bplanes : a.C;
    p.w_bplanes = a.w_bplanes ? a.w_bplanes : p.Cw * 3;
    p.w_splanes = a.w_splanes ? a.w_splanes : a.B * p.Cw * 3;
    return p;
}

}  // namespace

hipError_t launch_fused_batched(const ScanArgs* probs, int count, hipStream_t stream) {
    if (count < 1 || count > kMaxBatch) return hipErrorInvalidValue;
    FusedBatch bat;
    long sets = 0;
    bool vec = true;
    for (int i = 0; i < count; ++i) {
        sets += (long)probs[i].B * (probs[i].C / probs[i].cpw);
        vec = vec && probs[i].W % (probs[0].bf16 ? Vec<uint16_t>::N : Vec<float>::N) == 0;
    }
    int wg = 0;
    for (int i = 0; i < count; ++i) {
        bat.p[i] = fused_params(probs[i]);
        set_chunks(bat.p[i], sets);
        bat.wg_begin[i] = wg;
        wg += bat.p[i].B * bat.p[i].Cw * bat.p[i].nchunk;
    }
    for (int i = count; i <= kMaxBatch; ++i) bat.wg_begin[i] = wg;
    for (int i = count; i < kMaxBatch; ++i) bat.p[i] = bat.p[0];
    bat.count = count;
    const unsigned grid = (unsigned)wg;
    if (probs[0].bf16) {
        if (vec) hipLaunchKernelGGL((fused_scan_batched_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, stream, bat);
        else hipLaunchKernelGGL((fused_scan_batched_kernel<uint16_t, false>), dim3(grid), dim3(kThreads), 0, stream, bat);
    } else {
        if (vec) hipLaunchKernelGGL((fused_scan_batched_kernel<float, true>), dim3(grid), dim3(kThreads), 0, stream, bat);
        else hipLaunchKernelGGL((fused_scan_batched_kernel<float, false>), dim3(grid), dim3(kThreads), 0, stream, bat);
    }
    return hipGetLastError();
}

hipError_t launch_fused(const ScanArgs& a, hipStream_t stream) {
    FusedParams p = fused_params(a);
    const long sets = (long)a.B * p.Cw;
    set_chunks(p, sets);
    const unsigned grid = (unsigned)(sets * p.nchunk);
    const bool vec = a.W % (a.bf16 ? Vec<uint16_t>::N : Vec<float>::N) == 0;
    const bool ntr = a.cpw > 1;   // non-temporal x / lambda / u rows (see load16)
    if (a.bf16) {
        if (vec && ntr) hipLaunchKernelGGL((fused_scan_kernel<uint16_t, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        else if (vec) hipLaunchKernelGGL((fused_scan_kernel<uint16_t, true, false>), dim3(grid), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fused_scan_kernel<uint16_t, false, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    } else {
        if (vec && ntr) hipLaunchKernelGGL((fused_scan_kernel<float, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        else if (vec) hipLaunchKernelGGL((fused_scan_kernel<float, true, false>), dim3(grid), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fused_scan_kernel<float, false, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gspn
