// gspn_fused_bwd.hip -- fused backward of the GSPN line scan for grids up to
// 64 x 64.
//
// Gradients of y = u * sum_dir h_dir, h_i = w_i h_{i-1} + lam_i x_i ("Parallel
// Sequence Modeling via Generalized Spatial Propagation Network", CVPR 2025
// paper notes, "Key design 1-3"; channel-shared weights from the GSPN-2
// author response, "How Channel-shared Weight Mitigates the Concurrency
// Bottleneck?"), the exact vector-Jacobian product:
//   gu = gy * sum_d h_d;   gx = lam * sum_d g_d;   glam = x * sum_d g_d
//   g_i = gy u (line i) + w_{i+1}^T g_{i+1}   (cut at the first line of a group)
//   dL/da_t = w_t (1 - sigmoid(a_t)) (D_t - sum_v w_v D_v),
//   D_t = sum over the set's channels of g_i[p] h_{i-1}[p+t-1].
//
// Design (gfx950, wave64), one workgroup of four waves per weight set
// (b, k); wave d owns direction d, lane p position p of the line:
//  * The normalised weights of the wave's direction are computed once into
//    registers (64 lines x w0, w2; w1 = 1 - w0 - w2) and serve the forward
//    and the adjoint of every channel of the set.
//  * Per channel, LDS holds gy u and one fp32 plane per direction, which
//    starts as lam x and is overwritten in place with h; after gu = gy * sum h
//    the adjoint runs the lines backwards and overwrites h_i with g_i (h_i is
//    last read at line i+1, the step before), and gx, glam come from the sum
//    of the adjoint planes.  Nothing but the inputs and the gradients
//    crosses HBM.
//  * Only the differences E0 = sum g (h[p-1] - h[p]) and E2 = sum g (h[p+1]
//    - h[p]) are accumulated per line and position (two registers per line,
//    summed over the set's channels): because the weights sum to 1,
//    D_t - sum_v w_v D_v is a cancellation-free expression in E0, E2 and
//    the weights.
//  * The prologue also keeps, per pixel, the sum S of the sigmoids of its
//    existing taps, so that the epilogue gets sigmoid(a_t) = w_t S.  For fp32
//    gradients it forms 1 - sigmoid(a_t) as 1 - w_t S below 1/2 and as
//    exp(-a_t) w_t S above (no cancellation), reading the raw taps again; for
//    bf16 gradients, whose rounding is far coarser than that cancellation,
//    it uses 1 - w_t S and w1 = 1 - w0 - w2 and reads no tap twice.  The tap
//    gradients of the set are written once.
//  * The prologue and the epilogue take 16 slots at a time.  Column
//    directions read and write a lane's own row as 16-byte vectors; row
//    directions hold the chunk transposed (lane = slot and 16 positions) so
//    that they read and write 16-byte row vectors too.
#include "gspn_lines.h"

namespace gspn {
namespace {

constexpr int kBS = kFusedMaxSide;   // max lines and positions
// LDS planes carry a zero border line on every side: grid pixel (r, c) is at
// (r + 1) * kBPitch + (c + 1).  The odd pitch keeps both row-wise and
// column-wise scalar accesses free of bank conflicts.
constexpr int kBPitch = kBS + 3;
constexpr int kBPlane = (kBS + 2) * kBPitch;
constexpr int kBThreads = 256;
constexpr int kBDepth = 4;           // LDS reads issued this many steps ahead
// Pitch of the [slot][position] arrays of the prologue and epilogue (sigmoid
// sums, exchange area): a multiple of 4 that is not one of 64, so that 16-byte
// accesses by lanes holding consecutive slots fall into distinct banks.
constexpr int kXP = kBS + 4;

struct FusedBwdParams {
    const void* x;
    const void* w;
    const void* lam;
    const void* u;
    const void* gy;
    void* gx;
    void* gw;
    void* glam;
    void* gu;
    int B, C, H, W, Cw, cpw, groups;
    uint32_t dirs;
};

template <int B, int E, typename F>
__device__ __forceinline__ void sfor(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        sfor<B + 1, E>(f);
    }
}

// up to N consecutive elements as a 16-byte register image (zeros past nvalid)
__device__ __forceinline__ uint4 ld_row(const uint16_t* p, int nvalid, bool vec) {
    if (vec) return *reinterpret_cast<const uint4*>(p);
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 8; ++j)
        if (j < nvalid) v[j >> 1] |= (uint32_t)p[j] << ((j & 1) * 16);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 ld_row(const float* p, int nvalid, bool vec) {
    if (vec) return *reinterpret_cast<const uint4*>(p);
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 4; ++j)
        if (j < nvalid) v[j] = __float_as_uint(p[j]);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
template <typename T, int N>
__device__ __forceinline__ void st_row(T* p, const float (&v)[N], int nvalid, bool vec) {
    if (vec) {
        store16(p, v);
    } else {
        for (int j = 0; j < N; ++j)
            if (j < nvalid) p[j] = from_f32(v[j], (T*)nullptr);
    }
}

// Workgroup barrier that orders LDS only: global loads issued before it (the
// next channel's rows) and global stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-wave view of one direction in the padded static form.  Slot t = 0..63
// is line coordinate j = t (TB, LR) or j = 63 - t (BT, RL); scanning the
// slots in order visits the real lines (j < n) in scan order, and for BT/RL
// the padding lines first, whose state stays 0, so the first real line
// starts from zero.  In an LDS plane, position p of slot t is at
// off0 + t * ds, and slot -1 (the line before slot 0) is a border line of
// zeros.  Bit t of `starts` is set when slot t holds the first line of a
// local group: the state restarts there and no adjoint flows out of it.
// Register arrays are indexed by slot, a compile-time constant in the
// unrolled loops, so all four directions share one code path.
struct BwdDir {
    int off0, ds;
    uint64_t starts;
};

// Forward of one channel, in place: the plane P holds lam x on entry and h
// on exit (slot t is read kBDepth steps before it is overwritten).
//   h' = keep * (h + w0 (h[p-1] - h) + w2 (h[p+1] - h)) + lam x
// KEEP = false when no slot after slot 0 starts a group: the state before
// slot 0 is 0, so keep changes nothing there and the factor is left out.
template <bool KEEP>
__device__ __forceinline__ void fwd_scan(const BwdDir& v, float* P, const float (&w0)[kBS], const float (&w2)[kBS]) {
    // offsets advance by ds per slot; opaque here so that the compiler does
    // not hoist 64 precomputed offsets (or keep factors) out of the loop
    int o = v.off0, ds = v.ds;
    uint64_t st = v.starts;
    asm volatile("" : "+v"(o), "+s"(ds), "+s"(st));
    int ol = o;
    float xr[kBDepth];
#pragma unroll
    for (int i = 0; i < kBDepth; ++i) { xr[i] = P[ol]; ol += ds; }
    float h = 0.0f;
    sfor<0, kBS>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const float xl = xr[t % kBDepth];
        if constexpr (t + kBDepth < kBS) { xr[t % kBDepth] = P[ol]; ol += ds; }
        // keep the read issued here, kBDepth steps before its use
        __builtin_amdgcn_sched_barrier(0);
        const float dl = from_left(h) - h;
        const float dr = from_right(h) - h;
        float nv = fmaf(w0[t], dl, h);
        nv = fmaf(w2[t], dr, nv);
        if constexpr (KEEP) {
            const float keep = ((st >> t) & 1u) ? 0.0f : 1.0f;
            h = fmaf(keep, nv, xl);
        } else {
            h = nv + xl;
        }
        P[o] = h;
        o += ds;
    });
}

// Adjoint of one channel, last slot first.  P holds h on entry and g on
// exit: slot t's h is last read at slot t+1 (the step before), and the h of
// slot t-1 is read kBDepth steps ahead, before slot t-1 is written.
// E0 / E2 accumulate the tap-gradient differences of every slot.
// KEEP = false when no slot after slot 0 starts a group: the carry out of
// slot 0 is never used.
template <bool KEEP>
__device__ __forceinline__ void adj_scan(const BwdDir& v, const float* __restrict__ GH, float* __restrict__ P,
                                         const float (&w0)[kBS], const float (&w2)[kBS], float (&e0)[kBS],
                                         float (&e2)[kBS]) {
    int o = v.off0, ds = v.ds;
    uint64_t st = v.starts;
    asm volatile("" : "+v"(o), "+s"(ds), "+s"(st));
    o += (kBS - 1) * ds;                     // slot 63
    int og = o, oh = o - ds;                 // read offsets: GH of slot t, P of slot t-1
    float gr[kBDepth], hr[kBDepth];
#pragma unroll
    for (int i = 0; i < kBDepth; ++i) {
        gr[i] = GH[og]; og -= ds;
        hr[i] = P[oh]; oh -= ds;
    }
    float carry = 0.0f;
    sfor<0, kBS>([&](auto tc) {
        constexpr int t = kBS - 1 - decltype(tc)::value;
        constexpr int q = (kBS - 1 - t) % kBDepth;
        const float gh = gr[q], hp = hr[q];
        if constexpr (t - kBDepth >= 0) { gr[q] = GH[og]; og -= ds; }
        if constexpr (t - 1 - kBDepth >= -1) { hr[q] = P[oh]; oh -= ds; }
        __builtin_amdgcn_sched_barrier(0);
        const float g = gh + carry;
        const float dl = from_left(hp) - hp;
        const float dr = from_right(hp) - hp;
        e0[t] = fmaf(g, dl, e0[t]);
        e2[t] = fmaf(g, dr, e2[t]);
        const float c0 = w0[t] * g, c2 = w2[t] * g;
        carry = ((g - c0) - c2) + from_right(c0) + from_left(c2);
        if constexpr (KEEP) {
            const float keep = ((st >> t) & 1u) ? 0.0f : 1.0f;
            carry *= keep;
        }
        P[o] = g;
        o -= ds;
    });
}

template <typename T, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(kBThreads, kBThreads), amdgpu_waves_per_eu(1, 1)))
void fused_bwd_kernel(FusedBwdParams prm) {
    constexpr int N = 16 / (int)sizeof(T);
    constexpr int kIt = kBS * kBS / (kBThreads * N);
    // LDS: GH | HP[4] (channel loop) | SG[4] (sigmoid sums, [slot][position]
    // per direction).  The prologue's exact-form branch borrows 4096 floats
    // per wave of the channel-loop planes before they are zeroed.
    constexpr int kSG = kBS * kXP;
    constexpr int kLoop = (5 * kBPlane + 3) / 4 * 4;     // channel-loop planes, padded
    __shared__ __attribute__((aligned(16))) float lds[kLoop + 4 * kSG];
    float* const GH = lds;
    float* const HP = lds + kBPlane;   // + d * kBPlane

    const int H = prm.H, W = prm.W, B = prm.B, C = prm.C, Cw = prm.Cw;
    const int HW = H * W;
    const uint32_t dirs = prm.dirs;
    const int k = blockIdx.x % Cw;
    const int b = blockIdx.x / Cw;
    const int c_begin = k * prm.cpw, c_end = c_begin + prm.cpw;

    const int tid = threadIdx.x;
    const int d = uniform(tid >> 6);
    const int p = tid & 63;
    const bool is_row = d < 2;
    const bool asc = d == 0 || d == 2;
    const bool on = (dirs >> d) & 1u;
    const int n = is_row ? H : W;
    const int m = is_row ? W : H;
    const int L = n / prm.groups;
    const bool has0 = p >= 1 && p < m;
    const bool has2 = p + 1 < m;
    float* const SGw = lds + kLoop + d * kSG;      // this wave's sums, [slot][position]
    float* const SG = SGw + p;
    // per-wave exchange area for one chunk of per-slot registers (prologue
    // and epilogue only; it lies in the channel-loop planes): [value][slot]
    // [position]
    static_assert(4 * 4 * 16 * kXP <= kLoop, "exchange areas exceed the channel-loop planes");
    float* const XRw = lds + d * 4 * 16 * kXP;
    float* const XR = XRw + p;

    // slot t <-> line coordinate j
    auto line_of = [&](int t) { return asc ? t : kBS - 1 - t; };
    BwdDir v;
    {
        const int stride = is_row ? kBPitch : 1;
        const int base = is_row ? (p + 1) : (p + 1) * kBPitch;      // line coordinate -1
        v.off0 = base + (asc ? 1 : kBS) * stride;                   // slot 0
        v.ds = asc ? stride : -stride;
        // scan step s sits in slot s (TB, LR) or s + 64 - n (BT, RL)
        uint64_t st = 0;
        for (int s0 = 0; s0 < n; s0 += L) st |= 1ull << (asc ? s0 : s0 + kBS - n);
        v.starts = st;
    }
    // a group starts after slot 0 (local groups, or BT / RL shorter than
    // 64).  The fp32 instantiations always take the scans with the keep
    // factor: a second copy of the scans costs them register spills.
    const bool restarts = sizeof(T) == 4 || (v.starts & ~1ull) != 0;
    // slots whose line exists and reads the previous line (taps in use)
    uint64_t coupled = 0;
    for (int t = 0; t < kBS; ++t)
        if (line_of(t) < n && !((v.starts >> t) & 1u)) coupled |= 1ull << t;

    // raw taps of this wave's direction for weight set (b, k)
    const int dd = on ? d : __builtin_ctz(dirs);
    const int slab = __builtin_popcount(dirs & ((1u << dd) - 1u));
    const T* wd = static_cast<const T*>(prm.w) + ((size_t)(slab * B + b) * Cw + k) * 3 * (size_t)HW;
    // grid offset of position pp on line j (pp < m, j < n)
    auto pix = [&](int j, int pp) { return is_row ? j * W + pp : pp * W + j; };
    constexpr int kChunk = 16;
    constexpr int kNCh = kBS / kChunk;
    auto opaque_mask = [](bool on_) {
        uint32_t mk = on_ ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(mk));
        return mk;
    };
    // Taps of slots t0 .. t0+15 at position p (0 where the pixel does not
    // exist); all loads of a chunk are issued before any is used.  The loads
    // are unconditional, from clamped addresses, and masked afterwards with
    // a mask the compiler cannot see through (a load under a divergent
    // condition becomes a branch with a full memory-counter wait).
    // Column directions with whole-vector rows: lane p reads its own row,
    // the chunk's 16 columns as 16-byte vectors (a vector lies wholly inside
    // or outside the grid).  Slot t0+i is column c0+i (LR) or c0+15-i (RL).
    constexpr int kNV = kChunk / N;                    // vectors per tap and chunk
    const bool col_vec = VEC && !is_row;
    const int crow = min(p, m - 1);                    // clamped row of this lane
    auto chunk_col0 = [&](int t0) { return asc ? t0 : kBS - kChunk - t0; };
    auto load_taps = [&](int t0, float (&a)[3][kChunk]) __attribute__((always_inline)) {
        if (col_vec) {
            const int c0 = chunk_col0(t0);
            uint4 raw[3][kNV];
            uint32_t vm[kNV];
#pragma unroll
            for (int q = 0; q < kNV; ++q) {
                const int cq = c0 + q * N;
                const bool ok = cq < n && p < m;
                vm[q] = opaque_mask(ok);
                const size_t o = (size_t)crow * W + (ok ? cq : 0);
#pragma unroll
                for (int t = 0; t < 3; ++t) raw[t][q] = *reinterpret_cast<const uint4*>(wd + (size_t)t * HW + o);
            }
            float cols[3][kChunk];   // in column order
#pragma unroll
            for (int q = 0; q < kNV; ++q)
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    float f[N];
                    const uint4 r = raw[t][q];
                    unpack(make_uint4(r.x & vm[q], r.y & vm[q], r.z & vm[q], r.w & vm[q]), f);
#pragma unroll
                    for (int e = 0; e < N; ++e) cols[t][q * N + e] = f[e];
                }
            // to slot order; both indices are compile-time constants
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int i = 0; i < kChunk; ++i) a[t][i] = asc ? cols[t][i] : cols[t][kChunk - 1 - i];
            return;
        }
        // rows (lanes read consecutive columns) and non-vector widths
        uint32_t bits[3][kChunk], msk[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const int j = line_of(t0 + i);
            const int o = pix(min(j, n - 1), min(p, m - 1));
            msk[i] = opaque_mask(j < n && p < m);
#pragma unroll
            for (int t = 0; t < 3; ++t) bits[t][i] = __float_as_uint(to_f32(wd[(size_t)t * HW + o]));
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
#pragma unroll
            for (int t = 0; t < 3; ++t) a[t][i] = __uint_as_float(bits[t][i] & msk[i]);
    };
    // Row directions with whole-vector rows take a chunk transposed: lane p
    // holds slot t0 + (p & 15) at the 16 positions from 16 (p >> 4), so that
    // its taps are read and written as 16-byte row vectors, and its entries
    // of the [slot][position] arrays (exchange area, SG) are 16-byte vectors
    // too (the pitch kXP keeps them free of bank conflicts).  Chunk values
    // pass between the two layouts through the exchange area: a wave's LDS
    // accesses complete in order.
    const bool row_vec = VEC && is_row;
    const int qi = p & (kChunk - 1);           // transposed: slot within the chunk
    const int qpos = (p >> 4) * kChunk;        // transposed: first position
    // taps of slot t0 + qi at positions qpos .. qpos+15 (0 outside the grid)
    auto load_taps_rows = [&](int t0, float (&a)[3][kChunk]) __attribute__((always_inline)) {
        const int j = line_of(t0 + qi);
        uint4 raw[3][kNV];
        uint32_t vm[kNV];
#pragma unroll
        for (int q = 0; q < kNV; ++q) {
            const int cq = qpos + q * N;
            const bool ok = j < n && cq < m;
            vm[q] = opaque_mask(ok);
            const size_t o = (size_t)min(j, n - 1) * W + (ok ? cq : 0);
#pragma unroll
            for (int u = 0; u < 3; ++u) raw[u][q] = *reinterpret_cast<const uint4*>(wd + (size_t)u * HW + o);
        }
#pragma unroll
        for (int q = 0; q < kNV; ++q)
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                float f[N];
                const uint4 r = raw[u][q];
                unpack(make_uint4(r.x & vm[q], r.y & vm[q], r.z & vm[q], r.w & vm[q]), f);
#pragma unroll
                for (int e = 0; e < N; ++e) a[u][q * N + e] = f[e];
            }
    };

    // ---- normalised weights of every slot (0 where a slot reads no taps)
    // and the sum S of the sigmoids of its existing taps, kept for the
    // Jacobian (s_t = w_t S).
    //   With q_t = 1 + exp(-a_t): w0 = q1 q2 / D, w2 = q0 q1 / D,
    //   D = q1 q2 + q0 q2 + q0 q1 (missing taps: q = 2 and the product
    //   term dropped), S = D / (q0 q1 q2) (a missing tap's q cancels).
    //   No overflow while every tap is >= -25; a chunk with a smaller tap
    //   is redone with the exact per-tap form.
    // The work runs as a loop over chunks of 16 slots (compact code: the
    // whole kernel does not fit the instruction cache unrolled); a chunk's
    // results reach the statically indexed registers through LDS.
    float w0[kBS], w2[kBS];
    sfor<0, kBS>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        w0[t] = 0.0f;
        w2[t] = 0.0f;
    });
    if (on) {
        const float kNegLog2e = -1.44269504088896340736f;
        // One chunk in either layout.  Element e is slot t0 + e at position
        // p, or (transposed) slot t0 + qi at position qpos + e; xo(e) is its
        // entry in the exchange area.
        auto norm_chunk = [&](int t0, auto tr_tag) __attribute__((always_inline)) {
            constexpr bool TR = decltype(tr_tag)::value;
            float a[3][kChunk];
            if constexpr (TR) load_taps_rows(t0, a);
            else load_taps(t0, a);
            auto slot = [&](int e) { return TR ? t0 + qi : t0 + e; };
            auto pos = [&](int e) { return TR ? qpos + e : p; };
            auto xo = [&](int e) { return TR ? qi * kXP + qpos + e : e * kXP + p; };
            float amin = 0.0f;
#pragma unroll
            for (int e = 0; e < kChunk; ++e) {
                const int t = slot(e), ps = pos(e);
                const bool cpl = (coupled >> t) & 1u;
                const bool h0 = ps >= 1 && ps < m, h2 = ps + 1 < m;
                // unused taps (missing neighbours, unused lines) are taken as 0
                const float a0 = cpl && h0 ? a[0][e] : 0.0f;
                const float a1 = cpl ? a[1][e] : 0.0f;
                const float a2 = cpl && h2 ? a[2][e] : 0.0f;
                amin = fminf(amin, fminf(fminf(a0, a1), a2));
                const float q0 = 1.0f + fast_exp2(a0 * kNegLog2e);
                const float q1 = 1.0f + fast_exp2(a1 * kNegLog2e);
                const float q2 = 1.0f + fast_exp2(a2 * kNegLog2e);
                const float p12 = h0 ? q1 * q2 : 0.0f;
                const float p01 = h2 ? q0 * q1 : 0.0f;
                const float D = fmaf(q0, q2, p12) + p01;
                const float inv = fast_rcp(D);
                XRw[xo(e)] = cpl ? p12 * inv : 0.0f;
                XRw[kChunk * kXP + xo(e)] = cpl ? p01 * inv : 0.0f;
                SGw[t * kXP + ps] = D * fast_rcp(q0 * q1 * q2);
            }
            if (__builtin_amdgcn_ballot_w64(amin < -25.0f) != 0) {
                // exact form for this chunk
                for (int e = 0; e < kChunk; ++e) {
                    const int t = slot(e), ps = pos(e);
                    const bool cpl = (coupled >> t) & 1u;
                    const bool h0 = ps >= 1 && ps < m, h2 = ps + 1 < m;
                    float v3[3];
#pragma unroll
                    for (int u = 0; u < 3; ++u) v3[u] = a[u][0];
#pragma unroll
                    for (int ee = 1; ee < kChunk; ++ee)   // a[.][e] without a dynamic index
                        if (ee == e)
#pragma unroll
                            for (int u = 0; u < 3; ++u) v3[u] = a[u][ee];
                    const float a0 = cpl && h0 ? v3[0] : 0.0f;
                    const float a1 = cpl ? v3[1] : 0.0f;
                    const float a2 = cpl && h2 ? v3[2] : 0.0f;
                    const Taps tp = normalise_taps(a0, a1, a2, h0, h2);
                    const float s0 = h0 ? fast_rcp(1.0f + fast_exp2(a0 * kNegLog2e)) : 0.0f;
                    const float s1 = fast_rcp(1.0f + fast_exp2(a1 * kNegLog2e));
                    const float s2 = h2 ? fast_rcp(1.0f + fast_exp2(a2 * kNegLog2e)) : 0.0f;
                    SGw[t * kXP + ps] = (s0 + s1) + s2;
                    XRw[xo(e)] = cpl ? tp.w0 : 0.0f;
                    XRw[kChunk * kXP + xo(e)] = cpl ? tp.w2 : 0.0f;
                }
            }
        };
        for (int ch = 0; ch < kNCh; ++ch) {
            if (row_vec) norm_chunk(ch * kChunk, std::integral_constant<bool, true>{});
            else norm_chunk(ch * kChunk, std::integral_constant<bool, false>{});
            asm volatile("" ::: "memory");   // other lanes' entries (transposed chunks)
            // the chunk's weights into registers (one static block per chunk)
            switch (ch) {
#define GSPN_UNDUMP(CH)                                                     \
                case CH:                                                    \
                    sfor<0, kChunk>([&](auto ic) {                          \
                        constexpr int i = decltype(ic)::value;              \
                        w0[CH * kChunk + i] = XR[i * kXP];                  \
                        w2[CH * kChunk + i] = XR[(kChunk + i) * kXP];       \
                    });                                                     \
                    break;
                GSPN_UNDUMP(0) GSPN_UNDUMP(1) GSPN_UNDUMP(2) GSPN_UNDUMP(3)
#undef GSPN_UNDUMP
            }
        }
    }
    float e0[kBS], e2[kBS];
    sfor<0, kBS>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        e0[t] = 0.0f;
        e2[t] = 0.0f;
    });

    // ---- rows of x / lam / u / gy: N elements per thread
    const int tpr = (W + N - 1) / N;
    const int rpi = kBThreads / tpr;
    const int tr = tid / tpr;
    const int tcol = tid - tr * tpr;
    const int col0 = tcol * N;
    const int nvalid = min(N, W - col0);
    const bool t_active = tr < rpi;
    auto row_ok = [&](int it) { return t_active && tr + it * rpi < H; };
    // offsets are recomputed from an opaque value at each use, so that the
    // compiler does not keep them (and their per-element variants) in
    // registers across the channel loop
    auto opaque_int = [](int x) {
        asm volatile("" : "+v"(x));
        return x;
    };
    auto row_off = [&](int it) { return opaque_int(min(tr + it * rpi, H - 1) * W + col0); };   // clamped
    auto plane_off = [&](int it) { return opaque_int((tr + it * rpi + 1) * kBPitch + col0 + 1); };
    // sum of the four direction planes at LDS offset o, in the order TB, BT,
    // LR, RL (a disabled direction's plane stays zero); no branch, so the
    // reads of a phase are all in flight together
    auto plane_sum = [&](int o) {
        return ((HP[o] + HP[kBPlane + o]) + HP[2 * kBPlane + o]) + HP[3 * kBPlane + o];
    };
    // x, lam, u, gy rows of channel c (rows past H read a clamped row); the
    // slice base is uniform and the lane offset 32-bit, so the accesses use
    // a scalar base address
    auto load_channel = [&](int c, uint4 (&xr)[kIt], uint4 (&lr)[kIt], uint4 (&ur)[kIt], uint4 (&gr)[kIt]) {
        const size_t so = ((size_t)b * C + c) * (size_t)HW;
        const T* xs = static_cast<const T*>(prm.x) + so;
        const T* ls = static_cast<const T*>(prm.lam) + so;
        const T* us = static_cast<const T*>(prm.u) + so;
        const T* gs = static_cast<const T*>(prm.gy) + so;
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int o = row_off(it);
            const bool ok = VEC || row_ok(it);
            xr[it] = ok ? ld_row(xs + o, nvalid, VEC) : make_uint4(0, 0, 0, 0);
            lr[it] = ok ? ld_row(ls + o, nvalid, VEC) : make_uint4(0, 0, 0, 0);
            ur[it] = ok ? ld_row(us + o, nvalid, VEC) : make_uint4(0, 0, 0, 0);
            gr[it] = ok ? ld_row(gs + o, nvalid, VEC) : make_uint4(0, 0, 0, 0);
        }
    };

    float* const Pd = HP + d * kBPlane;
    uint4 xc[kIt], lc[kIt], uc[kIt], gc[kIt];
    load_channel(c_begin, xc, lc, uc, gc);
    lds_barrier();   // every wave has its weights: the scratch area is free
    // zero the channel loop's planes (borders and entries outside the grid stay 0)
    for (int i = tid; i < kLoop / 4; i += kBThreads)
        reinterpret_cast<float4*>(lds)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    lds_barrier();

    // 1 for an enabled direction, 0 for a disabled one (whose plane stays 0)
    float dir_on[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) dir_on[q] = ((dirs >> q) & 1u) ? 1.0f : 0.0f;

    for (int c = c_begin; c < c_end; ++c) {
        const size_t so = ((size_t)b * C + c) * (size_t)HW;
        T* const gus = static_cast<T*>(prm.gu) + so;
        T* const gxs = static_cast<T*>(prm.gx) + so;
        T* const gls = static_cast<T*>(prm.glam) + so;
        // lam * x into each enabled direction's plane (the forward then
        // overwrites it in place with h), gy * u into GH
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            if (row_ok(it)) {
                float xv[N], lv[N], uv[N], gv[N];
                unpack(xc[it], xv);
                unpack(lc[it], lv);
                unpack(uc[it], uv);
                unpack(gc[it], gv);
                const int po = plane_off(it);
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    if (VEC || e < nvalid) {
                        const float xl = xv[e] * lv[e];
#pragma unroll
                        for (int q = 0; q < 4; ++q) HP[q * kBPlane + po + e] = xl * dir_on[q];
                        GH[po + e] = gv[e] * uv[e];
                    }
                }
            }
        }
        // next channel's rows, in flight during the scans (the last channel
        // reloads itself: unconditional loads keep the counter waits exact)
        uint4 xn[kIt], ln[kIt], un[kIt], gn[kIt];
        load_channel(min(c + 1, c_end - 1), xn, ln, un, gn);
        lds_barrier();

        // ---- forward: h of every direction into its plane
        if (on) {
            if (restarts) fwd_scan<true>(v, Pd, w0, w2);
            else fwd_scan<false>(v, Pd, w0, w2);
        }
        lds_barrier();

        // ---- gu = gy * sum_d h_d
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            if (row_ok(it)) {
                float gv[N], out[N];
                unpack(gc[it], gv);
                const int po = plane_off(it);
#pragma unroll
                for (int e = 0; e < N; ++e) out[e] = gv[e] * plane_sum(po + e);
                st_row(gus + row_off(it), out, nvalid, VEC);
            }
        }
        lds_barrier();

        // ---- adjoint: g of every direction over its plane, tap sums
        if (on) {
            if (restarts) adj_scan<true>(v, GH, Pd, w0, w2, e0, e2);
            else adj_scan<false>(v, GH, Pd, w0, w2, e0, e2);
        }
        lds_barrier();

        // ---- gx = lam * G, glam = x * G
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            if (row_ok(it)) {
                float xv[N], lv[N], ox[N], ol[N];
                unpack(xc[it], xv);
                unpack(lc[it], lv);
                const int po = plane_off(it);
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float sg = plane_sum(po + e);
                    ox[e] = lv[e] * sg;
                    ol[e] = xv[e] * sg;
                }
                st_row(gxs + row_off(it), ox, nvalid, VEC);
                st_row(gls + row_off(it), ol, nvalid, VEC);
            }
        }
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            xc[it] = xn[it]; lc[it] = ln[it]; uc[it] = un[it]; gc[it] = gn[it];
        }
        lds_barrier();
    }

    // ---- tap gradients of the set (every tap of the slab is written).
    // With D_t the channel sums of g_i[p] h_{i-1}[p+t-1] and E0 = D0 - D1,
    // E2 = D2 - D1 (accumulated as such), D_t - sum_v w_v D_v expands,
    // since the weights sum to 1, into sums of products with no cancellation:
    //   t = 0: w1 E0 + w2 (E0 - E2);  t = 1: -(w0 E0 + w2 E2);
    //   t = 2: w1 E2 + w0 (E2 - E0)
    // and ga_t = w_t (1 - s_t) (D_t - sum_v w_v D_v), with s_t = w_t S.
    // fp32 gradients: every weight is formed directly (w1 = s1 / S), and
    // 1 - s_t without cancellation (1 - s_t for s_t < 1/2, else
    // exp(-a_t) s_t), so the raw taps are read again.  bf16 gradients: their
    // rounding (2^-9 relative) dwarfs what w1 = 1 - w0 - w2 and 1 - s_t as it
    // stands lose to cancellation (about one fp32 ulp of 1, absolute), so the
    // raw taps are not read again.  The chunks of 16 slots run unrolled.
    constexpr bool kReadTaps = sizeof(T) == 4;
    if (on) {
        T* gwd = static_cast<T*>(prm.gw) + ((size_t)(slab * B + b) * Cw + k) * 3 * (size_t)HW;
        const float kNegLog2e = -1.44269504088896340736f;
        // tap gradients of one pixel: raw taps a3 (used where cpl and the
        // neighbour exists), weights x0, x2, tap sums E0, E2, sigmoid sum S
        auto tap_grads = [&](bool cpl, bool h0, bool h2, const float (&a3)[3], float x0, float x2, float E0,
                             float E2, float S, float (&ga)[3]) __attribute__((always_inline)) {
            float wv[3] = {x0, 1.0f - x0 - x2, x2};
            float om[3];
            if constexpr (kReadTaps) {
                const float av[3] = {cpl && h0 ? a3[0] : 0.0f, cpl ? a3[1] : 0.0f, cpl && h2 ? a3[2] : 0.0f};
                float ex[3];
#pragma unroll
                for (int u = 0; u < 3; ++u) ex[u] = fast_exp2(av[u] * kNegLog2e);   // may be inf
                // w1 = sigmoid(a1) / S; if every sigmoid underflows, the
                // weights came from the exact form and w1 = 1 - w0 - w2
                if (S > 1e-30f) wv[1] = fast_rcp(1.0f + ex[1]) * fast_rcp(S);
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const float sg = wv[u] * S;
                    om[u] = sg < 0.5f ? 1.0f - sg : ex[u] * sg;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 3; ++u) om[u] = 1.0f - wv[u] * S;
            }
            const float r0 = fmaf(wv[1], E0, wv[2] * (E0 - E2));
            const float r1 = -fmaf(wv[0], E0, wv[2] * E2);
            const float r2 = fmaf(wv[1], E2, wv[0] * (E2 - E0));
            ga[0] = cpl ? wv[0] * om[0] * r0 : 0.0f;
            ga[1] = cpl ? wv[1] * om[1] * r1 : 0.0f;
            ga[2] = cpl ? wv[2] * om[2] * r2 : 0.0f;
        };
        sfor<0, kNCh>([&](auto cc) {
            constexpr int ch = decltype(cc)::value;
            constexpr int t0 = ch * kChunk;
            // the chunk's registers into LDS
            sfor<0, kChunk>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                XR[i * kXP] = w0[ch * kChunk + i];
                XR[(kChunk + i) * kXP] = w2[ch * kChunk + i];
                XR[(2 * kChunk + i) * kXP] = e0[ch * kChunk + i];
                XR[(3 * kChunk + i) * kXP] = e2[ch * kChunk + i];
            });
            if (row_vec) {
                asm volatile("" ::: "memory");   // other lanes' entries
                const int t = t0 + qi;
                const int j = line_of(t);
                const bool cpl = (coupled >> t) & 1u;
                float a[3][kChunk] = {};
                if constexpr (kReadTaps) load_taps_rows(t0, a);
                const float* xr = XRw + qi * kXP + qpos;
                const float* sg = SGw + t * kXP + qpos;
                float gaf[3][kChunk];
#pragma unroll
                for (int e = 0; e < kChunk; ++e) {
                    const int pos = qpos + e;
                    const float a3[3] = {a[0][e], a[1][e], a[2][e]};
                    float ga[3];
                    tap_grads(cpl, pos >= 1 && pos < m, pos + 1 < m, a3, xr[e], xr[kChunk * kXP + e],
                              xr[2 * kChunk * kXP + e], xr[3 * kChunk * kXP + e], sg[e], ga);
#pragma unroll
                    for (int u = 0; u < 3; ++u) gaf[u][e] = ga[u];
                }
#pragma unroll
                for (int q = 0; q < kNV; ++q) {
                    const int cq = qpos + q * N;
                    if (j < n && cq < m) {
#pragma unroll
                        for (int u = 0; u < 3; ++u) {
                            float f[N];
#pragma unroll
                            for (int e = 0; e < N; ++e) f[e] = gaf[u][q * N + e];
                            store16(gwd + (size_t)u * HW + (size_t)j * W + cq, f);
                        }
                    }
                }
            } else {
                float a[3][kChunk] = {};
                if constexpr (kReadTaps) load_taps(t0, a);
                float gaf[3][kChunk];
#pragma unroll
                for (int i = 0; i < kChunk; ++i) {
                    const int t = t0 + i;
                    const float a3[3] = {a[0][i], a[1][i], a[2][i]};
                    float ga[3];
                    tap_grads((coupled >> t) & 1u, has0, has2, a3, XR[i * kXP], XR[(kChunk + i) * kXP],
                              XR[(2 * kChunk + i) * kXP], XR[(3 * kChunk + i) * kXP], SG[t * kXP], ga);
#pragma unroll
                    for (int u = 0; u < 3; ++u) gaf[u][i] = ga[u];
                }
                if (col_vec) {
                    // lane p writes its row: the chunk's columns as 16-byte vectors
                    const int c0 = chunk_col0(t0);
#pragma unroll
                    for (int q = 0; q < kNV; ++q) {
                        const int cq = c0 + q * N;
                        if (cq < n && p < m) {
#pragma unroll
                            for (int u = 0; u < 3; ++u) {
                                float f[N];
#pragma unroll
                                for (int e = 0; e < N; ++e)
                                    f[e] = asc ? gaf[u][q * N + e] : gaf[u][kChunk - 1 - q * N - e];
                                store16(gwd + (size_t)u * HW + (size_t)p * W + cq, f);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kChunk; ++i) {
                        const int j = line_of(t0 + i);
                        if (j < n && p < m) {
                            const int o = pix(j, p);
#pragma unroll
                            for (int u = 0; u < 3; ++u) gwd[(size_t)u * HW + o] = from_f32(gaf[u][i], (T*)nullptr);
                        }
                    }
                }
            }
        });
    }
}

}  // namespace

hipError_t launch_fused_bwd(const GradArgs& g, hipStream_t stream) {
    const ScanArgs& a = g.fwd;
    FusedBwdParams p;
    p.x = a.x; p.w = a.w; p.lam = a.lam; p.u = a.u; p.gy = g.gy;
    p.gx = g.gx; p.gw = g.gw; p.glam = g.glam; p.gu = g.gu;
    p.B = a.B; p.C = a.C; p.H = a.H; p.W = a.W;
    p.cpw = a.cpw; p.Cw = a.C / a.cpw; p.groups = a.groups; p.dirs = a.dirs;
    const unsigned grid = (unsigned)((long)a.B * p.Cw);
    const bool vec = a.W % (a.bf16 ? 8 : 4) == 0;
    if (a.bf16) {
        if (vec) hipLaunchKernelGGL((fused_bwd_kernel<uint16_t, true>), dim3(grid), dim3(kBThreads), 0, stream, p);
        else hipLaunchKernelGGL((fused_bwd_kernel<uint16_t, false>), dim3(grid), dim3(kBThreads), 0, stream, p);
    } else {
        if (vec) hipLaunchKernelGGL((fused_bwd_kernel<float, true>), dim3(grid), dim3(kBThreads), 0, stream, p);
        else hipLaunchKernelGGL((fused_bwd_kernel<float, false>), dim3(grid), dim3(kBThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gspn
