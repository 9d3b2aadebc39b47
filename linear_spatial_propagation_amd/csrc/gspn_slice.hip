// gspn_slice.hip -- the four-direction GSPN scan with one workgroup per
// (b, c) slice, for local-group grids with sides up to 128 (bf16).
//
// Same operator as the other kernels: the line recurrence of "Parallel
// Sequence Modeling via Generalized Spatial Propagation Network" (CVPR 2025
// paper notes, "Key design 1"), tridiagonal row-stochastic weights ("Key
// design 2"), four scan directions merged as y = u * sum_dir h_dir, and the
// local variant ("Key design 3": each direction's scan axis split into g
// groups that restart the state).
//
// Design (gfx950, wave64), for H, W <= 128 and at least 8 groups:
//  * One workgroup of 8 waves owns a whole (b, c) slice.  The sum of the
//    four directions is held in LDS as fp32 (H x 129 floats), so no
//    per-direction plane goes through HBM and there is no separate merge
//    pass: every input is read once and y is written once.
//  * The directions run one after the other (TB, BT, LR, RL: the fixed
//    summation order; the loop over them is unrolled at compile time so each
//    direction's registers live only in its own code); within a direction,
//    wave w scans groups w, w + 8, ...  The first enabled direction reads x
//    and lambda and leaves lambda x in a second fp32 LDS plane; the others
//    take it from there, so x and lambda leave HBM once per slice.
//    Lane l owns positions 2l and 2l + 1 of a line, the state is two VGPRs
//    and the neighbours across lanes come from DPP wave shifts.  The first
//    enabled direction stores into the LDS sum, the others add.  Directions
//    of one kind give each wave the same lines, so a barrier is needed only
//    between the row and the column directions and before the output pass.
//  * Row directions read each line (a row) as 4-byte pieces per lane,
//    loaded four lines ahead (a group's first line without its taps, which
//    the recurrence does not use).  Column directions read, for each of the
//    lane's two rows, the group's columns as 16-byte pieces of 8 columns:
//    the eight waves own the groups side by side, so between them they read
//    whole 128-byte lines at the same time, with no transposed copy.  Two
//    pieces are in flight ahead of the scan.
//  * With 8- or 16-column groups LR and RL run back to back per group in one
//    wave, all their pieces (and u's) requested at once; RL, the last
//    direction, writes y = u * (sum + h) itself as 16-byte pieces, so
//    there is no output pass and no final barrier.  These are ordinary
//    stores: the four waves' pieces of a 128-byte line combine in the L2,
//    where non-temporal ones would reach HBM as partial-line writes (4.5x
//    the bytes of y).  Otherwise u
//    is requested after the last direction's scans and a separate pass
//    writes y.
//  * Taps are normalised as they are consumed (3 exp + 1 rcp per pixel and
//    direction, the rational form; rows with a tap below -40 take the exact
//    form).
//  * 8 waves and 129 KB of LDS per workgroup, one workgroup per CU at two
//    waves per SIMD (the column directions' pieces in flight need the
//    registers).
#include "gspn_device.h"
#include "gspn_kernels.h"

namespace gspn {
namespace {

constexpr int kSliceMax = 128;            // largest side
constexpr int kAccPitch = kSliceMax + 1;  // floats per LDS row of the sum (odd: column accesses spread over banks)
constexpr int kWaves = 8;
constexpr int kSliceThreads = 64 * kWaves;
constexpr int kRowDepth = 4;              // lines loaded ahead by the row directions
constexpr int kColChunk = 8;              // columns per 16-byte piece read by the column directions
constexpr int kUVecs = kSliceMax * kSliceMax / 8 / kSliceThreads;   // u vectors per thread

struct SliceParams {
    const uint16_t* x;
    const uint16_t* w;
    const uint16_t* lam;
    const uint16_t* u;
    uint16_t* y;
    int B, C, H, W, Cw, cpw, groups;
    uint32_t dirs;
};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ float bf16_at(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Weights of the lane's two positions.  Raw taps that are missing or
// belong to an idle position are 0 here (finite), as normalise_fast needs.
__device__ __forceinline__ void weights2(const float (&a0)[2], const float (&a1)[2], const float (&a2)[2],
                                         const bool (&h0)[2], const bool (&h2)[2], float (&w0)[2], float (&w2)[2]) {
    const float amin = fminf(fminf(fminf(a0[0], a1[0]), a2[0]), fminf(fminf(a0[1], a1[1]), a2[1]));
    if (__builtin_amdgcn_ballot_w64(amin < -40.0f) == 0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float2 w = normalise_fast(a0[e], a1[e], a2[e], h0[e], h2[e]);
            w0[e] = w.x;
            w2[e] = w.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const Taps t = normalise_taps(a0[e], a1[e], a2[e], h0[e], h2[e]);
            w0[e] = t.w0;
            w2[e] = t.w2;
        }
    }
}

// One line step of the lane's two positions (the middle weight is
// 1 - w0 - w2: h' = (h + xl) + w0 (h[p-1] - h) + w2 (h[p+1] - h)).
__device__ __forceinline__ void step2(float (&h)[2], const float (&xl)[2], const float (&w0)[2],
                                      const float (&w2)[2]) {
    const float left = from_left(h[1]);    // position 2l - 1 (lane l - 1)
    const float right = from_right(h[0]);  // position 2l + 2 (lane l + 1)
    const float n0 = fmaf(w2[0], h[1] - h[0], fmaf(w0[0], left - h[0], h[0] + xl[0]));
    const float n1 = fmaf(w2[1], right - h[1], fmaf(w0[1], h[0] - h[1], h[1] + xl[1]));
    h[0] = n0;
    h[1] = n1;
}

// Two waves per SIMD (one workgroup per CU): the column directions keep
// two 8-column pieces of each input in flight per lane.
// PNCH: 8-column pieces per group of the LR/RL pair this instantiation
// holds (1 or 2; one per kernel keeps each kernel's code to its own pair).
template <int PNCH>
__global__ __attribute__((amdgpu_flat_work_group_size(kSliceThreads, kSliceThreads), amdgpu_waves_per_eu(2, 2)))
void slice_scan_kernel(SliceParams prm) {
    __shared__ float acc[kSliceMax * kAccPitch];
    __shared__ float xlp[kSliceMax * kAccPitch];   // lambda * x, written by the first direction
    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63;
    // Waves w and w + 4 share a SIMD and get the same work; at equal priority
    // the SIMD favours the older wave, and per-wave timestamps showed waves
    // 4-7 finishing the column pair about 6 us after waves 0-3.  Raising the
    // younger waves' issue priority evens that out: local2k 265.6-266.6 ->
    // 262.4-263.0 us on one GPU (waves 0-3 raised instead: 264.3-265.0),
    // same bits.
    if (wave >= 4) __builtin_amdgcn_s_setprio(1);
    const int H = prm.H, W = prm.W, C = prm.C, B = prm.B;
    const size_t HW = (size_t)H * W;
    const int slice = blockIdx.x;
    const int c = slice % C, b = slice / C;
    const int k = c / prm.cpw;
    const uint16_t* __restrict__ xs = prm.x + (size_t)slice * HW;
    const uint16_t* __restrict__ ls = prm.lam + (size_t)slice * HW;
    const uint16_t* __restrict__ us = prm.u + (size_t)slice * HW;
    uint16_t* __restrict__ ys = prm.y + (size_t)slice * HW;
    const int nvec = (int)(HW / 8);

    const uint32_t dirs = prm.dirs;
    const int last = 31 - __builtin_clz(dirs);
    uint4 uu[kUVecs];   // u of the slice, requested when the last direction's scans are done
    const int first = __builtin_ctz(dirs);
    // LR and RL over 8- or 16-column groups run back to back per group (one
    // wave, its own columns: no barrier between them), sharing the x and
    // lambda pieces and with all pieces of both in flight at once
    const bool both_cols = (dirs & 12u) == 12u && W / prm.groups == PNCH * kColChunk;
    // with the pair, RL is the last direction and writes y = u * sum itself;
    // otherwise u is requested after the last direction's scans and a
    // separate pass writes y
    const bool fused_out = both_cols;
    const int u_dir = fused_out ? -1 : last;
    // the pair's pieces of a group of PNCH 8-column pieces: taps of LR and RL,
    // and u
    typedef uint4 Taps3[PNCH][2][3];   // [piece][row 2l, 2l + 1][tap]
    const int prc = 2 * lane < H ? 2 * lane : H - 2;
    const uint16_t* __restrict__ ws_lr =
        prm.w + ((size_t)(__builtin_popcount(dirs & 3u) * B + b) * prm.Cw + k) * 3 * HW;
    const uint16_t* __restrict__ ws_rl = ws_lr + (size_t)B * prm.Cw * 3 * HW;   // the next slab
    auto load_pair = [&](int gi, Taps3& ta, Taps3& tb, uint4 (&tu)[PNCH][2]) {
#pragma unroll
        for (int ch = 0; ch < PNCH; ++ch)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const size_t o = (size_t)(prc + e) * W + gi * PNCH * kColChunk + kColChunk * ch;
#pragma unroll
                for (int t = 0; t < 3; ++t) ta[ch][e][t] = *reinterpret_cast<const uint4*>(ws_lr + t * HW + o);
            }
#pragma unroll
        for (int ch = 0; ch < PNCH; ++ch)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const size_t o = (size_t)(prc + e) * W + gi * PNCH * kColChunk + kColChunk * ch;
#pragma unroll
                for (int t = 0; t < 3; ++t) tb[ch][e][t] = *reinterpret_cast<const uint4*>(ws_rl + t * HW + o);
            }
#pragma unroll
        for (int ch = 0; ch < PNCH; ++ch)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                tu[ch][e] = *reinterpret_cast<const uint4*>(us + (size_t)(prc + e) * W + gi * PNCH * kColChunk +
                                                            kColChunk * ch);
    };
    int slot = 0;
    static_for<0, 4>([&](auto dc) {   // unrolled: each direction's registers live only in its own code
        constexpr int d = decltype(dc)::value;
        if (!((dirs >> d) & 1u)) return;
        const bool store = d == first;
        const uint16_t* __restrict__ ws = prm.w + ((size_t)(slot * B + b) * prm.Cw + k) * 3 * HW;
        ++slot;
        if (d == 3 && both_cols) return;   // done with LR
        if (d == 2 && both_cols) {
            const int r0 = 2 * lane;
            const bool on = r0 < H;
            const int rc = on ? r0 : H - 2;
            const bool h0[2] = {on && r0 >= 1, on};
            const bool h2[2] = {on, on && r0 + 2 < H};
            const int L = PNCH * kColChunk;
            constexpr int NCH = PNCH;
            auto pair = [&](auto first_c) {
                constexpr bool kFirst = decltype(first_c)::value;   // x and lambda from memory (LR is the first direction)
                constexpr int kQ = kFirst ? 5 : 3;
                for (int gi = wave; gi < prm.groups; gi += kWaves) {
                    const int c_base = gi * L;
                    uint4 qa[NCH][2][kQ];   // [piece][row][tap 0, 1, 2 of LR (, x, lambda)]
                    uint4 qb[NCH][2][3];    // [piece][row][tap 0, 1, 2 of RL]
                    uint4 uq[NCH][2];       // [piece][row] u, for RL's output
                    if constexpr (kFirst) {
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const size_t o = (size_t)(rc + e) * W + c_base + kColChunk * ch;
                                qa[ch][e][3] = *reinterpret_cast<const uint4*>(xs + o);
                                qa[ch][e][4] = *reinterpret_cast<const uint4*>(ls + o);
                            }
                        Taps3 ta3;
                        load_pair(gi, ta3, qb, uq);
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                            for (int e = 0; e < 2; ++e)
#pragma unroll
                                for (int t = 0; t < 3; ++t) qa[ch][e][t] = ta3[ch][e][t];
                    } else {
                        load_pair(gi, qa, qb, uq);
                    }
                    float ov[NCH][2][kColChunk];   // [piece][row][column] y of RL's current piece
                    // one line of either direction: column index cl in 0 .. L - 1
                    // of the group, taps from tp
                    // mode: 0 stores h into the sum, 1 adds it, 2 writes y = u * (sum + h)
                    auto line = [&](float (&h)[2], const uint4 (&tp)[NCH][2][3], auto clc, bool first_line,
                                    auto mode_c) {
                        constexpr int cl = decltype(clc)::value;
                        constexpr int kMode = decltype(mode_c)::value;
                        constexpr int ch = cl / kColChunk, j = cl % kColChunk;
                        float xl[2];
                        if constexpr (kFirst) {
#pragma unroll
                            for (int e = 0; e < 2; ++e)
                                xl[e] = on ? bf16_at(qa[ch][e][3], j) * bf16_at(qa[ch][e][4], j) : 0.0f;
                        } else {
#pragma unroll
                            for (int e = 0; e < 2; ++e) xl[e] = on ? xlp[(r0 + e) * kAccPitch + c_base + cl] : 0.0f;
                        }
                        if (first_line) {
                            h[0] = xl[0];
                            h[1] = xl[1];
                        } else {
                            float a0[2], a1[2], a2[2], w0[2], w2[2];
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                a0[e] = h0[e] ? bf16_at(tp[ch][e][0], j) : 0.0f;
                                a1[e] = on ? bf16_at(tp[ch][e][1], j) : 0.0f;
                                a2[e] = h2[e] ? bf16_at(tp[ch][e][2], j) : 0.0f;
                            }
                            weights2(a0, a1, a2, h0, h2, w0, w2);
                            step2(h, xl, w0, w2);
                        }
                        float* dst = acc + r0 * kAccPitch + c_base + cl;
                        if constexpr (kMode == 2) {
#pragma unroll
                            for (int e = 0; e < 2; ++e) ov[ch][e][j] = bf16_at(uq[ch][e], j) * (dst[e * kAccPitch] + h[e]);
                            if (j == 0 && on) {   // the piece is complete (RL runs its columns descending)
                                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
                                for (int e = 0; e < 2; ++e) {
                                    const u32x4 r4 = {pack_bf16x2(ov[ch][e][0], ov[ch][e][1]),
                                                      pack_bf16x2(ov[ch][e][2], ov[ch][e][3]),
                                                      pack_bf16x2(ov[ch][e][4], ov[ch][e][5]),
                                                      pack_bf16x2(ov[ch][e][6], ov[ch][e][7])};
                                    // an ordinary store: the pieces of one 128-byte line come from
                                    // four waves and merge in the L2 (non-temporal ones would
                                    // each reach HBM as a partial-line write)
                                    *reinterpret_cast<u32x4*>(ys + (size_t)(r0 + e) * W + c_base + kColChunk * ch) = r4;
                                }
                            }
                        } else if (on) {
                            if constexpr (kMode == 0) {
                                dst[0] = h[0];
                                dst[kAccPitch] = h[1];
                            } else {
                                dst[0] += h[0];
                                dst[kAccPitch] += h[1];
                            }
                        }
                    };
                    uint4 ta[NCH][2][3];
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                        for (int e = 0; e < 2; ++e)
#pragma unroll
                            for (int t = 0; t < 3; ++t) ta[ch][e][t] = qa[ch][e][t];
                    float h[2] = {0.0f, 0.0f};
                    static_for<0, PNCH * kColChunk>([&](auto ic) {            // LR: columns ascending
                        constexpr int i = decltype(ic)::value;
                        line(h, ta, std::integral_constant<int, i>{}, i == 0, std::integral_constant<int, kFirst ? 0 : 1>{});
                    });
                    static_for<0, PNCH * kColChunk>([&](auto ic) {            // RL: columns descending
                        constexpr int i = decltype(ic)::value;
                        line(h, qb, std::integral_constant<int, PNCH * kColChunk - 1 - i>{}, i == 0,
                             std::integral_constant<int, 2>{});
                    });
                }
            };
            if (store) pair(std::true_type{});
            else pair(std::false_type{});
        } else if (d < 2) {
            // ---- row direction: line = row, position = column (lane: 2l, 2l + 1)
            const int L = H / prm.groups;
            const int q0 = 2 * lane;
            const bool on = q0 < W;
            const int qc = on ? q0 : W - 2;
            const bool h0[2] = {on && q0 >= 1, on};
            const bool h2[2] = {on, on && q0 + 2 < W};
            auto rows = [&](auto asc_c, auto first_c) {
                constexpr bool kAsc = decltype(asc_c)::value;
                // the first direction reads x and lambda and leaves lambda x in
                // LDS for the others
                constexpr bool kFirst = decltype(first_c)::value;
                constexpr int kQ = kFirst ? 5 : 3;
                for (int gi = wave; gi < prm.groups; gi += kWaves) {
                    const int r_base = gi * L;
                    auto row_of = [&](int i) { return r_base + (kAsc ? i : L - 1 - i); };
                    uint32_t ring[kRowDepth][kQ];   // 3 taps (, x, lambda): two bf16 each
                    auto load = [&](uint32_t (&q)[kQ], int i, bool taps = true) {
                        const size_t o = (size_t)row_of(min(i, L - 1)) * W + qc;
                        if (taps) {
                            q[0] = *reinterpret_cast<const uint32_t*>(ws + o);
                            q[1] = *reinterpret_cast<const uint32_t*>(ws + HW + o);
                            q[2] = *reinterpret_cast<const uint32_t*>(ws + 2 * HW + o);
                        }
                        if constexpr (kFirst) {
                            q[3] = *reinterpret_cast<const uint32_t*>(xs + o);
                            q[4] = *reinterpret_cast<const uint32_t*>(ls + o);
                        }
                    };
                    // the group's first line has no taps (h = lambda x there)
                    load(ring[0], 0, false);
#pragma unroll
                    for (int s = 1; s < kRowDepth; ++s) load(ring[s], s);
                    float h[2] = {0.0f, 0.0f};
                    // kRowDepth lines per iteration; steps past the group's last
                    // line compute on clamped data and store nothing
                    for (int i0 = 0; i0 < L; i0 += kRowDepth) {
#pragma unroll
                        for (int s = 0; s < kRowDepth; ++s) {
                            const int i = i0 + s;
                            const uint32_t* q = ring[s];
                            float* xd = xlp + row_of(min(i, L - 1)) * kAccPitch + q0;
                            float xl[2];
                            if constexpr (kFirst) {
                                xl[0] = on ? bf16_lo(q[3]) * bf16_lo(q[4]) : 0.0f;
                                xl[1] = on ? bf16_hi(q[3]) * bf16_hi(q[4]) : 0.0f;
                                if (i < L && on) {
                                    xd[0] = xl[0];
                                    xd[1] = xl[1];
                                }
                            } else {
                                xl[0] = on ? xd[0] : 0.0f;
                                xl[1] = on ? xd[1] : 0.0f;
                            }
                            if (i == 0) {   // the group's first line: h = lambda x
                                h[0] = xl[0];
                                h[1] = xl[1];
                            } else {
                                const float a0[2] = {h0[0] ? bf16_lo(q[0]) : 0.0f, h0[1] ? bf16_hi(q[0]) : 0.0f};
                                const float a1[2] = {on ? bf16_lo(q[1]) : 0.0f, on ? bf16_hi(q[1]) : 0.0f};
                                const float a2[2] = {h2[0] ? bf16_lo(q[2]) : 0.0f, h2[1] ? bf16_hi(q[2]) : 0.0f};
                                float w0[2], w2[2];
                                weights2(a0, a1, a2, h0, h2, w0, w2);
                                step2(h, xl, w0, w2);
                            }
                            if (i < L && on) {
                                float* dst = acc + row_of(i) * kAccPitch + q0;
                                if (kFirst) {
                                    dst[0] = h[0];
                                    dst[1] = h[1];
                                } else {
                                    dst[0] += h[0];
                                    dst[1] += h[1];
                                }
                            }
                            load(ring[s], i + kRowDepth);
                        }
                    }
                }
            };
            if (d == 0) rows(std::true_type{}, std::true_type{});   // TB is the first direction when enabled
            else if (store) rows(std::false_type{}, std::true_type{});
            else rows(std::false_type{}, std::false_type{});
        } else {
            // ---- column direction: line = column, position = row (lane: 2l, 2l + 1)
            const int L = W / prm.groups;   // a multiple of 4
            const int nch = L / kColChunk;  // chunks of kColChunk columns
            const int r0 = 2 * lane;
            const bool on = r0 < H;
            const int rc = on ? r0 : H - 2;
            const bool h0[2] = {on && r0 >= 1, on};
            const bool h2[2] = {on, on && r0 + 2 < H};
            auto cols = [&](auto asc_c, auto first_c) {
                constexpr bool kAsc = decltype(asc_c)::value;
                constexpr bool kFirst = decltype(first_c)::value;   // x and lambda from memory, lambda x to LDS
                constexpr int kQ = kFirst ? 5 : 3;
                for (int gi = wave; gi < prm.groups; gi += kWaves) {
                    const int c_base = gi * L;
                    // chunk ch (in scan order) covers columns cols_of(ch) .. + kColChunk
                    auto cols_of = [&](int ch) { return c_base + kColChunk * (kAsc ? ch : nch - 1 - ch); };
                    typedef uint4 Chunk[2][kQ];   // [row 2l, 2l + 1][tap 0, 1, 2 (, x, lambda)]
                    auto load = [&](Chunk& q, int ch) {
                        const int cc = cols_of(min(ch, nch - 1));
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const size_t o = (size_t)(rc + e) * W + cc;
                            q[e][0] = *reinterpret_cast<const uint4*>(ws + o);
                            q[e][1] = *reinterpret_cast<const uint4*>(ws + HW + o);
                            q[e][2] = *reinterpret_cast<const uint4*>(ws + 2 * HW + o);
                            if constexpr (kFirst) {
                                q[e][3] = *reinterpret_cast<const uint4*>(xs + o);
                                q[e][4] = *reinterpret_cast<const uint4*>(ls + o);
                            }
                        }
                    };
                    float h[2] = {0.0f, 0.0f};
                    auto scan = [&](const Chunk& q, int ch) {
                        const int cc = cols_of(ch);
#pragma unroll
                        for (int t = 0; t < kColChunk; ++t) {
                            const int j = kAsc ? t : kColChunk - 1 - t;   // column cc + j (compile-time)
                            float xl[2];
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                float* xd = xlp + (r0 + e) * kAccPitch + cc + j;
                                if constexpr (kFirst) {
                                    xl[e] = on ? bf16_at(q[e][3], j) * bf16_at(q[e][4], j) : 0.0f;
                                    if (on) *xd = xl[e];
                                } else {
                                    xl[e] = on ? *xd : 0.0f;
                                }
                            }
                            if (ch == 0 && t == 0) {   // the group's first line
                                h[0] = xl[0];
                                h[1] = xl[1];
                            } else {
                                float a0[2], a1[2], a2[2], w0[2], w2[2];
#pragma unroll
                                for (int e = 0; e < 2; ++e) {
                                    a0[e] = h0[e] ? bf16_at(q[e][0], j) : 0.0f;
                                    a1[e] = on ? bf16_at(q[e][1], j) : 0.0f;
                                    a2[e] = h2[e] ? bf16_at(q[e][2], j) : 0.0f;
                                }
                                weights2(a0, a1, a2, h0, h2, w0, w2);
                                step2(h, xl, w0, w2);
                            }
                            if (on) {
                                float* dst = acc + r0 * kAccPitch + cc + j;
                                if (kFirst) {
                                    dst[0] = h[0];
                                    dst[kAccPitch] = h[1];
                                } else {
                                    dst[0] += h[0];
                                    dst[kAccPitch] += h[1];
                                }
                            }
                        }
                    };
                    // two chunks in flight: each buffer is refilled after use
                    Chunk qa, qb;
                    load(qa, 0);
                    load(qb, 1);
                    for (int ch = 0; ch < nch; ch += 2) {
                        scan(qa, ch);
                        load(qa, ch + 2);
                        if (ch + 1 < nch) {
                            scan(qb, ch + 1);
                            load(qb, ch + 3);
                        }
                    }
                }
            };
            if (d == 2) {
                if (store) cols(std::true_type{}, std::true_type{});
                else cols(std::true_type{}, std::false_type{});
            } else {
                if (store) cols(std::false_type{}, std::true_type{});
                else cols(std::false_type{}, std::false_type{});
            }
        }
        if (d == u_dir) {
#pragma unroll
            for (int i = 0; i < kUVecs; ++i) {
                const int v = min(tid + i * kSliceThreads, nvec - 1);
                uu[i] = *reinterpret_cast<const uint4*>(us + (size_t)v * 8);
            }
        }
        // a barrier where the next direction reads what other waves wrote:
        // between row and column directions and before the output pass.
        // Directions of one kind give each wave the same lines, so between
        // TB and BT (or LR and RL) a wave only reads its own LDS writes.

        const uint32_t later = d == 2 && both_cols ? 0u : dirs & ~((2u << d) - 1u);   // the pair ran RL too
        const bool next_col = later != 0 && __builtin_ctz(later) >= 2;
        if (later == 0 ? !fused_out : (d >= 2) != next_col) __syncthreads();
    });
    if (fused_out) return;   // RL wrote y

    // ---- y = u * sum
#pragma unroll
    for (int i = 0; i < kUVecs; ++i) {
        const int v = tid + i * kSliceThreads;
        if (v < nvec) {
            const int p = v * 8;
            const int r = p / W, q = p - r * W;
            const float* s = acc + r * kAccPitch + q;
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = bf16_at(uu[i], e) * s[e];
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 r4 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])};
            __builtin_nontemporal_store(r4, reinterpret_cast<u32x4*>(ys + p));
        }
    }
}

}  // namespace

bool slice_supported(const ScanArgs& a) {
    if (!a.bf16 || a.lam_dir || a.u_dir) return false;
    if (a.H > kSliceMax || a.W > kSliceMax || a.H < 2 || a.W < 8) return false;
    if (a.W % 8 || a.H % 2) return false;
    if (a.groups < kWaves) return false;                   // every wave owns a group
    if ((a.dirs & 12u) && (a.W / a.groups) % kColChunk) return false;   // column groups in 16-byte pieces
    return true;
}

hipError_t launch_slice(const ScanArgs& a, hipStream_t stream) {
    SliceParams p;
    p.x = static_cast<const uint16_t*>(a.x);
    p.w = static_cast<const uint16_t*>(a.w);
    p.lam = static_cast<const uint16_t*>(a.lam);
    p.u = static_cast<const uint16_t*>(a.u);
    p.y = static_cast<uint16_t*>(a.y);
    p.B = a.B; p.C = a.C; p.H = a.H; p.W = a.W; p.Cw = a.C / a.cpw; p.cpw = a.cpw; p.groups = a.groups;
    p.dirs = a.dirs;
    // the instantiation whose LR/RL pair matches the column groups (8 columns:
    // one piece; otherwise two, which 16-column groups use)
    if (!(a.dirs & 12u) || a.W != a.groups * kColChunk)
        hipLaunchKernelGGL(slice_scan_kernel<2>, dim3((unsigned)(a.B * a.C)), dim3(kSliceThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(slice_scan_kernel<1>, dim3((unsigned)(a.B * a.C)), dim3(kSliceThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gspn

