// Integer SGD with momentum and per-group velocity ("Memory-Efficient
// Integer-Only Training of Deep Neural Networks", Figure 1b and Table 5).
//
// For every velocity group (one row = one output channel):
//   v = momentum * V + G          exact, then V' = requantised into V's group
//   w = W - lr * V'               exact, then W' = requantised into W's group
// W' takes the weights' mantissa width (|C| <= 2^w_q - 1, Table 4's B-bit
// variants); the velocity is always INT8.
// momentum and lr are (C, e) scalars.  One wave owns one row; the row's
// bytes of W, V and G stay in registers between the two steps.
//
// Exact two-term sums X*2^pa + Y*2^pb (|X|, |Y| <= 2^14): when the exponent
// gap is at most 15 the sum fits int32 at the smaller exponent.  Otherwise it
// is formed in int64; for gaps above 40 the smaller term (below 2^(P-9) in
// magnitude, P the larger term's exponent) can only decide a rounding tie
// or a sticky bit, so it is replaced by sign(Y) * 2^(P-24), which rounds
// identically at every exponent the group can take (every such exponent is
// at least P - 7 at any width, where the larger term dominates).
#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

struct Ex64 {
    long long n;
    int base;
};

__device__ __forceinline__ Ex64 combine64(int X, int pa, int Y, int pb) {
    if (X == 0) return {(long long)Y, pb};
    if (Y == 0) return {(long long)X, pa};
    int d = pa - pb;
    if (d >= 0) {
        if (d <= 40) return {((long long)X << d) + Y, pb};
        return {((long long)X << 24) + (Y > 0 ? 1 : -1), pa - 24};
    }
    d = -d;
    if (d <= 40) return {(long long)X + ((long long)Y << d), pa};
    return {((long long)Y << 24) + (X > 0 ? 1 : -1), pb - 24};
}

__device__ __forceinline__ int sbyte(uint32_t w, int j) { return (int)(int8_t)(w >> (8 * j)); }

__device__ __forceinline__ int wave_max64(int v) { return wave_max_dpp(v); }

__device__ __forceinline__ uint32_t load_dw(const int8_t *row, long long col, long long cols, int vec) {
    if (vec && col + 4 <= cols) return *(const uint32_t *)(row + col);
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j)
        if (col + j < cols) w |= (uint32_t)(uint8_t)row[col + j] << (8 * j);
    return w;
}

__device__ __forceinline__ void store_dw(int8_t *row, long long col, long long cols, int vec, uint32_t w) {
    if (vec && col + 4 <= cols) {
        *(uint32_t *)(row + col) = w;
        return;
    }
    for (int j = 0; j < 4; ++j)
        if (col + j < cols) row[col + j] = (int8_t)(w >> (8 * j));
}

// The D dwords a lane owns in a row are contiguous (bytes col0 .. col0 +
// 4 D): one vector access per four dwords when the row holds them all and is
// 4-byte aligned, else dword by dword with bounds checks.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));

template <int D>
__device__ __forceinline__ void load_dws(const int8_t *row, long long col0, long long cols, int vec, uint32_t (&w)[D]) {
    if (vec && col0 + 4 * D <= cols) {
#pragma unroll
        for (int j = 0; j < D; j += 4) {
            const int8_t *p = row + col0 + 4 * j;
            const int n = D - j < 4 ? D - j : 4;  // a compile-time constant once unrolled
            // (indices clamped so that every branch compiles for any D)
            if (n == 4) {
                const u32x4 v = *(const u32x4 *)p;
                w[j] = v.x, w[j + 1 < D ? j + 1 : j] = v.y, w[j + 2 < D ? j + 2 : j] = v.z,
                w[j + 3 < D ? j + 3 : j] = v.w;
            } else if (n == 3) {
                const u32x3 v = *(const u32x3 *)p;
                w[j] = v.x, w[j + 1 < D ? j + 1 : j] = v.y, w[j + 2 < D ? j + 2 : j] = v.z;
            } else if (n == 2) {
                const u32x2 v = *(const u32x2 *)p;
                w[j] = v.x, w[j + 1 < D ? j + 1 : j] = v.y;
            } else {
                w[j] = *(const uint32_t *)p;
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < D; ++j) w[j] = load_dw(row, col0 + 4 * j, cols, vec);
}

template <int D>
__device__ __forceinline__ void store_dws(int8_t *row, long long col0, long long cols, int vec, const uint32_t (&w)[D]) {
    if (vec && col0 + 4 * D <= cols) {
#pragma unroll
        for (int j = 0; j < D; j += 4) {
            int8_t *p = row + col0 + 4 * j;
            const int n = D - j < 4 ? D - j : 4;
            if (n == 4) {
                *(u32x4 *)p = u32x4{w[j], w[j + 1 < D ? j + 1 : j], w[j + 2 < D ? j + 2 : j], w[j + 3 < D ? j + 3 : j]};
            } else if (n == 3) {
                *(u32x3 *)p = u32x3{w[j], w[j + 1 < D ? j + 1 : j], w[j + 2 < D ? j + 2 : j]};
            } else if (n == 2) {
                *(u32x2 *)p = u32x2{w[j], w[j + 1 < D ? j + 1 : j]};
            } else {
                *(uint32_t *)p = w[j];
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < D; ++j) store_dw(row, col0 + 4 * j, cols, vec, w[j]);
}

// The wide (int64) forms are out of line: rows with exponent gaps above 15
// are rare, and inlined they raise the register pressure of every row's path
// (measured: spills and half the throughput).
__device__ __noinline__ int sum_need_wide(int X, int pa, int Y, int pb, int q) {
    Ex64 s = combine64(X, pa, Y, pb);
    return need64(s.n, s.base, q);
}

__device__ __noinline__ int sum_round_wide(int X, int pa, int Y, int pb, int e) {
    Ex64 s = combine64(X, pa, Y, pb);
    return (int)rne_shift64(s.n, e - s.base);
}

// Smallest exponent / rounding of X*2^pa + Y*2^pb, using the int32 form
// when `narrow` (|pa - pb| <= 15, uniform over the row).
__device__ __forceinline__ int sum_need(bool narrow, int X, int pa, int Y, int pb) {
    if (narrow) {
        int base = min(pa, pb);
        int n = (X << (pa - base)) + (Y << (pb - base));
        return need32(n, base);
    }
    return sum_need_wide(X, pa, Y, pb, 7);
}

__device__ __forceinline__ int sum_round(bool narrow, int X, int pa, int Y, int pb, int e) {
    if (narrow) {
        int base = min(pa, pb);
        int n = (X << (pa - base)) + (Y << (pb - base));
        return rne_shift32(n, e - base);
    }
    return sum_round_wide(X, pa, Y, pb, e);
}

// ---------------------------------------------------------------------------
// Weight decay adds a third term: v = momentum*V + G + wd*W.  Exact sums of
// three terms X*2^p (|X| < 2^15) as n * 2^base in 128 bits, terms sorted by
// exponent pa >= pb >= pc:
//   - pa - pb > 60: b and c lie below 2^(pa-45) while the sum exceeds
//     2^(pa-1), so every exponent the group can take is at least pa - 8 and
//     they only decide ties and sticky bits: a * 2^24 + sign(b 2^pb + c 2^pc)
//     at pa - 24 rounds identically;
//   - else S = a 2^(pa-pb) + b exactly (|S| < 2^75); if pb - pc > 40 and
//     S != 0, c (below 2^(pb-25) against a sum above 2^(pb-1)) is replaced
//     the same way: S * 2^24 + sign(c) at pb - 24; S == 0 leaves c exactly;
//   - otherwise S * 2^(pb-pc) + c exactly (|.| < 2^116).
// ---------------------------------------------------------------------------

struct Ex128 {
    __int128 n;
    int base;
};

__device__ __noinline__ Ex128 combine3(int X1, int p1, int X2, int p2, int X3, int p3) {
    int x[3] = {X1, X2, X3}, p[3] = {p1, p2, p3};
    // sort by exponent, descending (three compare-exchanges)
    auto cx = [&](int i, int j) {
        if (p[i] < p[j]) {
            int t = p[i]; p[i] = p[j]; p[j] = t;
            t = x[i]; x[i] = x[j]; x[j] = t;
        }
    };
    cx(0, 1);
    cx(1, 2);
    cx(0, 1);
    // zero terms drop out: the two-term form covers what is left
    if (x[0] == 0 || x[1] == 0 || x[2] == 0) {
        int k = 0, y[3], q[3];
        for (int i = 0; i < 3; ++i)
            if (x[i] != 0) {
                y[k] = x[i];
                q[k] = p[i];
                ++k;
            }
        if (k == 0) return {0, p[2]};
        if (k == 1) return {(__int128)y[0], q[0]};
        const Ex64 s = combine64(y[0], q[0], y[1], q[1]);
        return {(__int128)s.n, s.base};
    }
    const int a = x[0], b = x[1], c = x[2], pa = p[0], pb = p[1], pc = p[2];
    if (pa - pb > 60) {
        const Ex64 bc = combine64(b, pb, c, pc);
        if (bc.n == 0) return {(__int128)a, pa};
        return {((__int128)a << 24) + (bc.n > 0 ? 1 : -1), pa - 24};
    }
    const __int128 S = ((__int128)a << (pa - pb)) + b;
    if (pb - pc > 40) {
        if (S == 0) return {(__int128)c, pc};
        return {(S << 24) + (c > 0 ? 1 : -1), pb - 24};
    }
    return {(S << (pb - pc)) + c, pc};
}

// Smallest exponent of n * 2^base (NEED_NONE for n == 0): bit length - 7,
// plus one when the top eight bits are all ones.
__device__ __forceinline__ int need128(__int128 n, int base) {
    if (n == 0) return NEED_NONE;
    const unsigned __int128 m = (unsigned __int128)(n < 0 ? -n : n);
    const uint64_t hi = (uint64_t)(m >> 64), lo = (uint64_t)m;
    const int z = hi ? __clzll(hi) : 64 + __clzll(lo);  // leading zeros of m (m != 0)
    const uint32_t top = (uint32_t)((m << z) >> 120);
    return base + (128 - z) - 7 + (top == 255u ? 1 : 0);
}

// n * 2^-s rounded half to even (s <= 0: exact left shift; the result is a
// mantissa, so callers only reach it for values that fit).
__device__ __forceinline__ int rne128(__int128 n, int s) {
    if (s <= 0) return (int)(n << (-s > 126 ? 126 : -s));
    if (s >= 126) return 0;
    __int128 q = n >> s;
    const __int128 r = n - (q << s), half = (__int128)1 << (s - 1);
    if (r > half || (r == half && (q & 1))) ++q;
    return (int)q;
}

__device__ __noinline__ int sum3_need_wide(int X1, int p1, int X2, int p2, int X3, int p3) {
    const Ex128 s = combine3(X1, p1, X2, p2, X3, p3);
    return need128(s.n, s.base);
}

__device__ __noinline__ int sum3_round_wide(int X1, int p1, int X2, int p2, int X3, int p3, int e) {
    const Ex128 s = combine3(X1, p1, X2, p2, X3, p3);
    return rne128(s.n, e - s.base);
}

// Rounding of a row with one uniform shift: n * 2^-sh, half to even
// (sh <= 0: exact left shift); |n| < 2^30.
struct RneU {
    int sh;
    int hm1;
    int left;
    bool is_left;
};

__device__ __forceinline__ RneU rne_u(int sh) {
    RneU r;
    r.is_left = sh <= 0;
    r.left = sh <= 0 ? -sh : 0;
    r.sh = sh > 31 ? 31 : (sh < 1 ? 1 : sh);
    r.hm1 = (1 << (r.sh - 1)) - 1;
    return r;
}


// c = rne(n, r) for D x 4 held values; the shift direction is uniform over
// the row, so it is decided once, outside the element loops.
template <int D>
__device__ __forceinline__ void rne_rows(const int (&n)[D][4], const RneU &r, int (&c)[D][4]) {
    if (r.is_left) {
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) c[j][t] = n[j][t] << r.left;
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) c[j][t] = (n[j][t] + r.hm1 + ((n[j][t] >> r.sh) & 1)) >> r.sh;
    }
}

__device__ __forceinline__ uint32_t pack4(const int (&c)[4]) {
    return (uint32_t)(uint8_t)c[0] | ((uint32_t)(uint8_t)c[1] << 8) | ((uint32_t)(uint8_t)c[2] << 16) |
           ((uint32_t)(uint8_t)c[3] << 24);
}

// Largest |n| of D x 4 values (signed maximum and minimum, combined once).
template <int D>
__device__ __forceinline__ uint32_t absmax_rows(const int (&n)[D][4]) {
    int hi = 0, lo = 0;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        hi = max(hi, max(max(n[j][0], n[j][1]), max(n[j][2], n[j][3])));
        lo = min(lo, min(min(n[j][0], n[j][1]), min(n[j][2], n[j][3])));
    }
    return (uint32_t)max(hi, -lo);
}

__device__ __forceinline__ uint32_t umax_wave(uint32_t v) { return wave_umax_dpp(v); }

// One row of W, V, G is owned by WPR waves (WPR = 1: four rows per block;
// WPR = 4: one row per block, maxima combined through LDS).  Each lane holds D
// dwords (4 D bytes) of each tensor.
//   pass 0: whole-tensor velocity: each block stores the largest need of its
//           rows' velocities in bmax_v[block].
//   pass 1: velocity step; weight step for row-grouped W, otherwise store V'
//           and the block's largest weight need in bmax_w[block].
//   pass 2: whole-tensor weight: round W at the maximum of bmax_w.
// Whole-tensor exponents that a pass overwrites are read from snapshots taken
// by the pass before (tmp[0]: old velocity exponent, tmp[1]: old weight
// exponent).  All passes run on the same grid of nblk blocks (this block is
// blk of them).
// RR: velocity and weight both grouped by rows, so that the second pass is
// the only one (the kernel is then built for it alone).
template <int D, int WPR, bool WD = false, bool RR = false>
__device__ __forceinline__ void update_rows(const UpdateArgs &a, int pass_, int vec, int blk, int nblk) {
    const int pass = RR ? 1 : pass_;
    constexpr int RPB = 4 / WPR;  // rows per block
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % WPR;
    const long long col0 = 4ll * D * (lane + 64 * sub);  // this lane's first byte of a row
    __shared__ uint32_t red[2][4];
    __shared__ int bred[4];
    int parity = 0;
    int *bmax_v = a.tmp + 2, *bmax_w = a.tmp + 2 + UPD_MAX_BLOCKS;
    auto block_imax = [&](int v) -> int {
        v = wave_max_dpp(v);
        __syncthreads();
        if (lane == 0) bred[wave] = v;
        __syncthreads();
        return max(max(bred[0], bred[1]), max(bred[2], bred[3]));
    };
    auto max_of = [&](const int *p) -> int {
        int m = NEED_NONE;
        for (int i = threadIdx.x; i < nblk; i += 256) m = max(m, p[i]);
        return block_imax(m);
    };
    // maximum over the row (all WPR waves); every wave of the block calls it
    auto row_umax = [&](uint32_t v) -> uint32_t {
        v = umax_wave(v);
        if constexpr (WPR > 1) {
            if (lane == 0) red[parity][sub] = v;
            __syncthreads();
            v = max(max(red[parity][0], red[parity][1]), max(red[parity][2], red[parity][3]));
            parity ^= 1;
        }
        return v;
    };
    auto row_imax = [&](int v) -> int { return (int)(row_umax((uint32_t)(v ^ (int)0x80000000)) ^ 0x80000000u); };
    const bool v_tensor = !RR && a.v_row == 0, w_tensor = !RR && a.w_row == 0;
    // whole-tensor exponents of this pass (before any write of this pass)
    int ev_t = 0, ew_t = 0, evn_t = 0, ewn_t = 0;
    if (pass == 0) {
        ev_t = a.v_exp[0];
        if (WD && w_tensor) ew_t = a.w_exp[0];  // the decay term reads W before it changes
        if (blk == 0 && threadIdx.x == 0) a.tmp[0] = ev_t;
    } else if (pass == 1) {
        if (v_tensor) {
            ev_t = a.tmp[0];
            evn_t = clamp_exp_flag(max(E_MIN, max_of(bmax_v)), a.flags);
        }
        if (w_tensor) {
            ew_t = a.w_exp[0];
            if (blk == 0 && threadIdx.x == 0) a.tmp[1] = ew_t;
        }
    } else {
        ew_t = a.tmp[1];
        ewn_t = clamp_exp_flag(max(E_MIN, max_of(bmax_w)), a.flags);
    }
    int bneed = NEED_NONE;  // largest need of this block's rows (passes 0, 1)

    // Rows of this block: row, row + stride, ...  The next row's tensors and
    // exponents are loaded before the current row is worked on, so a wave
    // keeps loads in flight across its rows.  (Exponents are read with the
    // data: a read after this row's stores could not be moved ahead of them.)
    struct RowIn {
        uint32_t W[D], V[D], G[D];
        int ew, ev, eg;
    };
    auto load_row = [&](long long row, RowIn &x) {
        const long long off = row * a.cols;
        if (pass != 0 || WD) {
            load_dws<D>(a.w + off, col0, a.cols, vec, x.W);
        } else {
#pragma unroll
            for (int j = 0; j < D; ++j) x.W[j] = 0u;
        }
        load_dws<D>(a.v + off, col0, a.cols, vec, x.V);
        if (pass != 2) {
            load_dws<D>(a.g + off, col0, a.cols, vec, x.G);
        } else {
#pragma unroll
            for (int j = 0; j < D; ++j) x.G[j] = 0u;
        }
        x.ew = w_tensor ? ew_t : (int)a.w_exp[row];
        x.ev = pass == 2 ? (int)a.v_exp[v_tensor ? 0 : row] : v_tensor ? ev_t : (int)a.v_exp[row];
        x.eg = pass == 2 ? 0 : a.g_row ? (int)a.g_exp[row] : (int)a.g_exp[0];
    };
    auto process = [&](long long row, const RowIn &x) {
        const long long off = row * a.cols;
        const uint32_t(&W)[D] = x.W;
        const uint32_t(&V)[D] = x.V;
        const uint32_t(&G)[D] = x.G;
            const int ew = x.ew;

            // ---- weight step only (whole-tensor weight, second pass) ----
            if (pass == 2) {
                const int evn = x.ev;
                const int pw = a.lr_e + evn;
                const int e = ewn_t;
                if (abs(ew - pw) <= 15) {
                    // |factors| <= 2^22 and mantissas are bytes: exact 24-bit products
                    const int base = min(ew, pw);
                    const int fa = 1 << (ew - base), fb = -a.lr_m * (1 << (pw - base));
                    int n[D][4], c[D][4];
    #pragma unroll
                    for (int j = 0; j < D; ++j)
    #pragma unroll
                        for (int t = 0; t < 4; ++t) n[j][t] = __mul24(sbyte(W[j], t), fa) + __mul24(sbyte(V[j], t), fb);
                    rne_rows<D>(n, rne_u(e - base), c);
                    uint32_t o[D];
    #pragma unroll
                    for (int j = 0; j < D; ++j) o[j] = pack4(c[j]);
                    store_dws<D>(a.w + off, col0, a.cols, vec, o);
                } else {
                    uint32_t o[D];
    #pragma unroll
                    for (int j = 0; j < D; ++j) {
                        o[j] = 0;
    #pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int c = sum_round_wide(sbyte(W[j], t), ew, -a.lr_m * sbyte(V[j], t), pw, e);
                            o[j] |= (uint32_t)(uint8_t)c << (8 * t);
                        }
                    }
                    store_dws<D>(a.w + off, col0, a.cols, vec, o);
                }
                if (row == 0 && lane == 0 && sub == 0) a.w_exp[0] = (int8_t)e;
                return;
            }

            // ---- velocity: v = momentum * V + G (+ weight_decay * W) ----
            const int ev = x.ev;
            const int eg = x.eg;
            const int pa = ev + a.mom_e, pb = eg;
            const int pc = WD ? ew + a.wd_e : pa;
            const int vbase = WD ? min(min(pa, pb), pc) : min(pa, pb);
            // narrow: exact in int32 at vbase (three terms: each below 2^28)
            const bool nv = WD ? max(max(pa, pb), pc) - vbase <= 14 : abs(pa - pb) <= 15;
            int vn[D][4];
            int needv;
            if (nv) {
                // |factors| <= 2^22 and mantissas are bytes: exact 24-bit products
                const int fa = a.mom_m * (1 << (pa - vbase)), fb = 1 << (pb - vbase);
                const int fc = WD ? a.wd_m * (1 << (pc - vbase)) : 0;
    #pragma unroll
                for (int j = 0; j < D; ++j)
    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        vn[j][t] = __mul24(sbyte(V[j], t), fa) + __mul24(sbyte(G[j], t), fb);
                        if constexpr (WD) vn[j][t] += __mul24(sbyte(W[j], t), fc);
                    }
                const uint32_t mx = row_umax(absmax_rows<D>(vn));
                needv = mx ? vbase + mant_shift32(mx) : NEED_NONE;
            } else {
                int m = NEED_NONE;
    #pragma unroll
                for (int j = 0; j < D; ++j)
    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if constexpr (WD)
                            m = max(m, sum3_need_wide(a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb,
                                                      a.wd_m * sbyte(W[j], t), pc));
                        else
                            m = max(m, sum_need_wide(a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb, 7));
                    }
                needv = row_imax(m);
            }
            if (pass == 0) {
                bneed = max(bneed, needv);
                return;
            }
            const int evn = v_tensor ? evn_t : clamp_exp_flag(max(E_MIN, needv), a.flags);
            int c[D][4];
            if (nv) {
                rne_rows<D>(vn, rne_u(evn - vbase), c);
            } else {
    #pragma unroll
                for (int j = 0; j < D; ++j)
    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if constexpr (WD)
                            c[j][t] = sum3_round_wide(a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb,
                                                      a.wd_m * sbyte(W[j], t), pc, evn);
                        else
                            c[j][t] = sum_round_wide(a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb, evn);
                    }
            }
            {
                uint32_t o[D];
    #pragma unroll
                for (int j = 0; j < D; ++j) o[j] = pack4(c[j]);
                store_dws<D>(a.v + off, col0, a.cols, vec, o);
            }
            if (lane == 0 && sub == 0) {
                if (!v_tensor) a.v_exp[row] = (int8_t)evn;
                else if (row == 0) a.v_exp[0] = (int8_t)evn;
            }

            // ---- weight: w = W - lr * V' ----
            const int pw = a.lr_e + evn;
            const bool nw = abs(ew - pw) <= 15;
            int needw;
            if (nw) {
                const int base = min(ew, pw);
                const int fa = 1 << (ew - base), fb = -a.lr_m * (1 << (pw - base));
    #pragma unroll
                for (int j = 0; j < D; ++j)
    #pragma unroll
                    for (int t = 0; t < 4; ++t) vn[j][t] = __mul24(sbyte(W[j], t), fa) + __mul24(c[j][t], fb);
                const uint32_t mx = row_umax(absmax_rows<D>(vn));
                needw = mx ? base + mant_shift32(mx, a.w_q) : NEED_NONE;
            } else {
                int m = NEED_NONE;
    #pragma unroll
                for (int j = 0; j < D; ++j)
    #pragma unroll
                    for (int t = 0; t < 4; ++t)
                        m = max(m, sum_need_wide(sbyte(W[j], t), ew, -a.lr_m * c[j][t], pw, a.w_q));
                needw = row_imax(m);
            }
            if (w_tensor) {
                bneed = max(bneed, needw);
                return;
            }
            const int ewn = clamp_exp_flag(max(E_MIN, needw), a.flags);
            if (nw) {
                int cw[D][4];
                rne_rows<D>(vn, rne_u(ewn - min(ew, pw)), cw);
                uint32_t o[D];
    #pragma unroll
                for (int j = 0; j < D; ++j) o[j] = pack4(cw[j]);
                store_dws<D>(a.w + off, col0, a.cols, vec, o);
            } else {
                uint32_t o[D];
    #pragma unroll
                for (int j = 0; j < D; ++j) {
                    o[j] = 0;
    #pragma unroll
                    for (int t = 0; t < 4; ++t)
                        o[j] |= (uint32_t)(uint8_t)sum_round_wide(sbyte(W[j], t), ew, -a.lr_m * c[j][t], pw, ewn) << (8 * t);
                }
                store_dws<D>(a.w + off, col0, a.cols, vec, o);
            }
            if (lane == 0 && sub == 0) a.w_exp[row] = (int8_t)ewn;
    };
    const long long stride = (long long)nblk * RPB;
    long long row = (long long)blk * RPB + wave / WPR;  // WPR > 1: the same row in every wave of the block
    RowIn A, B;
    if (row < a.rows) load_row(row, A);
    while (row < a.rows) {
        const long long r1 = row + stride;
        if (r1 < a.rows) load_row(r1, B);
        process(row, A);
        if (r1 >= a.rows) break;
        const long long r2 = r1 + stride;
        if (r2 < a.rows) load_row(r2, A);
        process(r1, B);
        row = r2;
    }
    if (pass == 0 || (pass == 1 && w_tensor)) {
        const int m = block_imax(bneed);
        if (threadIdx.x == 0) (pass == 0 ? bmax_v : bmax_w)[blk] = m;
    }
}

template <int D, int WPR, bool WD, bool RR = false>
__global__ __launch_bounds__(256) void sgd_rows_kernel(UpdateArgs a, int pass, int vec) {
    update_rows<D, WPR, WD, RR>(a, pass, vec, blockIdx.x, gridDim.x);
}

// Several tensors of one (D, WPR) class in one launch: segment i owns blocks
// [block0[i], block0[i + 1]).
constexpr int UPD_SEGS = 12;
struct UpdSegs {
    UpdateArgs a[UPD_SEGS];
    int vec[UPD_SEGS];
    int block0[UPD_SEGS + 1];
    int n;
};

__device__ __forceinline__ int segment_of(const int *block0, int n) {
    int i = 0;
    while (i + 1 < n && (int)blockIdx.x >= block0[i + 1]) ++i;
    return __builtin_amdgcn_readfirstlane(i);  // block-uniform: keep the segment's arguments scalar
}

template <int D, int WPR, bool RR = false>
__global__ __launch_bounds__(256) void sgd_multi_kernel(UpdSegs sg, int pass) {
    const int i = segment_of(sg.block0, sg.n);
    update_rows<D, WPR, false, RR>(sg.a[i], pass, sg.vec[i], blockIdx.x - sg.block0[i],
                                   sg.block0[i + 1] - sg.block0[i]);
}

// Tensors of the narrow classes (at most 4 dwords of each tensor per lane)
// together in one launch per pass, each segment with its own class: a
// model's many small tensors then cost two or three launches in all.
constexpr int UPD_MIX = 24;
constexpr int UPD_MIX_CLASSES = 8;  // classes 0..7 of update_class
struct UpdMix {
    UpdateArgs a[UPD_MIX];
    int vec[UPD_MIX];
    int cls[UPD_MIX];
    int block0[UPD_MIX + 1];
    int n;
};
static_assert(sizeof(UpdMix) <= 4096, "kernel arguments of the mixed update");

__global__ __launch_bounds__(256) void sgd_mixed_kernel(UpdMix sg, int pass) {
    const int i = segment_of(sg.block0, sg.n);
    const int b = blockIdx.x - sg.block0[i], nb = sg.block0[i + 1] - sg.block0[i];
    switch (sg.cls[i]) {
        case 0: update_rows<1, 1>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 1: update_rows<2, 1>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 2: update_rows<3, 1>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 3: update_rows<4, 1>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 4: update_rows<1, 4>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 5: update_rows<2, 4>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 6: update_rows<3, 4>(sg.a[i], pass, sg.vec[i], b, nb); break;
        case 7: update_rows<4, 4>(sg.a[i], pass, sg.vec[i], b, nb); break;
        default: break;
    }
}

// Grid of one tensor's passes: at most UPD_MAX_BLOCKS blocks (about what
// the CUs hold at once), so that a wave walks several rows and overlaps the
// next row's loads with the current row's work.
static int update_blocks(const UpdateArgs &a, int wpr) {
    const int rpb = 4 / wpr;
    long long blocks = (a.rows + rpb - 1) / rpb;
    if (blocks > UPD_MAX_BLOCKS) blocks = UPD_MAX_BLOCKS;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

template <int D, int WPR, bool WD = false>
static hipError_t run_passes(const UpdateArgs &a, int vec, hipStream_t st) {
    const int blocks = update_blocks(a, WPR);
    hipError_t err;
    if (a.v_row && a.w_row) {
        // row groups on both: the one pass, in its own build
        prof_begin(st, 2001);
        hipLaunchKernelGGL((sgd_rows_kernel<D, WPR, WD, true>), dim3((int)blocks), dim3(256), 0, st, a, 1, vec);
        prof_end(st, 2001);
        return hipGetLastError();
    }
    for (int pass = 0; pass < 3; ++pass) {
        if (pass == 0 && a.v_row) continue;
        if (pass == 2 && a.w_row) continue;
        prof_begin(st, 2000 + pass);
        hipLaunchKernelGGL((sgd_rows_kernel<D, WPR, WD>), dim3((int)blocks), dim3(256), 0, st, a, pass, vec);
        prof_end(st, 2000 + pass);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int D, int WPR>
static hipError_t run_multi(const UpdateArgs *a, const int *vec, int n, hipStream_t st) {
    for (int pass = 0; pass < 3; ++pass) {
        UpdSegs sg;
        sg.n = 0;
        int blocks = 0;
        for (int i = 0; i < n; ++i) {
            if ((pass == 0 && a[i].v_row) || (pass == 2 && a[i].w_row)) continue;
            sg.a[sg.n] = a[i];
            sg.vec[sg.n] = vec[i];
            sg.block0[sg.n] = blocks;
            blocks += update_blocks(a[i], WPR);
            ++sg.n;
        }
        if (sg.n == 0) continue;
        sg.block0[sg.n] = blocks;
        bool rr = pass == 1;
        for (int i = 0; i < sg.n; ++i) rr = rr && sg.a[i].v_row && sg.a[i].w_row;
        prof_begin(st, 2000 + pass);
        if (rr)  // row groups on both for every tensor: the one pass's own build
            hipLaunchKernelGGL((sgd_multi_kernel<D, WPR, true>), dim3(blocks), dim3(256), 0, st, sg, pass);
        else
            hipLaunchKernelGGL((sgd_multi_kernel<D, WPR>), dim3(blocks), dim3(256), 0, st, sg, pass);
        prof_end(st, 2000 + pass);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// Launch class of a tensor: rows of 256 dwords or more put four waves on a
// row (one row per block), so a lane holds at most 8 dwords of each tensor
// up to 8192 columns.  Returns 0..9 (an index into the instantiated (D, WPR)
// pairs) or -1.
static const int CLASS_D[10] = {1, 2, 3, 4, 1, 2, 3, 4, 6, 8};
static int update_class(const UpdateArgs &a) {
    const long long dw = (a.cols + 3) / 4;
    const bool wide = dw >= 256;
    const long long per_lane = wide ? (dw + 255) / 256 : (dw + 63) / 64;
    for (int c = wide ? 4 : 0; c < (wide ? 10 : 4); ++c)
        if (per_lane <= CLASS_D[c]) return c;
    return -1;
}

static int update_vec(const UpdateArgs &a) {
    return (a.cols % 4 == 0) && ((uintptr_t)a.w % 4 == 0) && ((uintptr_t)a.v % 4 == 0) &&
           ((uintptr_t)a.g % 4 == 0);
}

// One tensor with weight decay: a launch per pass of its class's kernel.
static hipError_t run_class_wd(int c, const UpdateArgs &a, int vec, hipStream_t st) {
    switch (c) {
        case 0: return run_passes<1, 1, true>(a, vec, st);
        case 1: return run_passes<2, 1, true>(a, vec, st);
        case 2: return run_passes<3, 1, true>(a, vec, st);
        case 3: return run_passes<4, 1, true>(a, vec, st);
        case 4: return run_passes<1, 4, true>(a, vec, st);
        case 5: return run_passes<2, 4, true>(a, vec, st);
        case 6: return run_passes<3, 4, true>(a, vec, st);
        case 7: return run_passes<4, 4, true>(a, vec, st);
        case 8: return run_passes<6, 4, true>(a, vec, st);
        case 9: return run_passes<8, 4, true>(a, vec, st);
    }
    return hipErrorInvalidValue;
}

// One tensor: a launch per pass of its class's kernel.
static hipError_t run_class(int c, const UpdateArgs &a, int vec, hipStream_t st) {
    if (a.wd_m != 0) return run_class_wd(c, a, vec, st);
    switch (c) {
        case 0: return run_passes<1, 1>(a, vec, st);
        case 1: return run_passes<2, 1>(a, vec, st);
        case 2: return run_passes<3, 1>(a, vec, st);
        case 3: return run_passes<4, 1>(a, vec, st);
        case 4: return run_passes<1, 4>(a, vec, st);
        case 5: return run_passes<2, 4>(a, vec, st);
        case 6: return run_passes<3, 4>(a, vec, st);
        case 7: return run_passes<4, 4>(a, vec, st);
        case 8: return run_passes<6, 4>(a, vec, st);
        case 9: return run_passes<8, 4>(a, vec, st);
    }
    return hipErrorInvalidValue;
}

// Several tensors of one class: a launch per pass.
static hipError_t run_class_multi(int c, const UpdateArgs *a, const int *vec, int n, hipStream_t st) {
    if (n == 1) return run_class(c, a[0], vec[0], st);
    switch (c) {
        case 0: return run_multi<1, 1>(a, vec, n, st);
        case 1: return run_multi<2, 1>(a, vec, n, st);
        case 2: return run_multi<3, 1>(a, vec, n, st);
        case 3: return run_multi<4, 1>(a, vec, n, st);
        case 4: return run_multi<1, 4>(a, vec, n, st);
        case 5: return run_multi<2, 4>(a, vec, n, st);
        case 6: return run_multi<3, 4>(a, vec, n, st);
        case 7: return run_multi<4, 4>(a, vec, n, st);
        case 8: return run_multi<6, 4>(a, vec, n, st);
        case 9: return run_multi<8, 4>(a, vec, n, st);
    }
    return hipErrorInvalidValue;
}

// Mixed launches take the narrow classes' small tensors; a large tensor
// keeps its class's own kernel, which holds more waves per CU.
constexpr long long UPD_MIX_MAX_ELEMS = 1ll << 21;
static int mixed_class(const UpdateArgs &a) {
    const int c = update_class(a);
    return c >= 0 && c < UPD_MIX_CLASSES && a.rows * a.cols <= UPD_MIX_MAX_ELEMS ? c : -1;
}

// Narrow-class tensors: a launch per pass (per UPD_MIX tensors).
static hipError_t run_mixed(const UpdateArgs *a, const int *vec, const int *cls, int n, hipStream_t st) {
    for (int pass = 0; pass < 3; ++pass) {
        for (int i0 = 0; i0 < n;) {
            UpdMix sg;
            sg.n = 0;
            int blocks = 0, i = i0;
            for (; i < n && sg.n < UPD_MIX; ++i) {
                if ((pass == 0 && a[i].v_row) || (pass == 2 && a[i].w_row)) continue;
                sg.a[sg.n] = a[i];
                sg.vec[sg.n] = vec[i];
                sg.cls[sg.n] = cls[i];
                sg.block0[sg.n] = blocks;
                blocks += update_blocks(a[i], cls[i] >= 4 ? 4 : 1);
                ++sg.n;
            }
            i0 = i;
            if (sg.n == 0) continue;
            sg.block0[sg.n] = blocks;
            prof_begin(st, 2000 + pass);
            hipLaunchKernelGGL(sgd_mixed_kernel, dim3(blocks), dim3(256), 0, st, sg, pass);
            prof_end(st, 2000 + pass);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
    }
    return hipSuccess;
}

static hipError_t empty_update(const UpdateArgs &a, hipStream_t st) {
    // Empty tensor: whole-tensor groups are all-zero.
    hipError_t err;
    if (a.v_row == 0 && (err = launch_fill_i8(a.v_exp, 1, E_MIN, st)) != hipSuccess) return err;
    if (a.w_row == 0 && (err = launch_fill_i8(a.w_exp, 1, E_MIN, st)) != hipSuccess) return err;
    return hipSuccess;
}

hipError_t launch_sgd_update(const UpdateArgs &a, hipStream_t st) {
    if (a.rows <= 0) return empty_update(a, st);
    const int c = update_class(a);
    if (c < 0) return hipErrorInvalidValue;
    return run_class(c, a, update_vec(a), st);
}

hipError_t launch_sgd_update_multi(const UpdateArgs *a, int n, hipStream_t st) {
    for (int i = 0; i < n; ++i)
        if (a[i].rows > 0 && update_class(a[i]) < 0) return hipErrorInvalidValue;
    if (n > 0 && a[0].wd_m != 0) {
        // weight decay (one scalar for all): tensor by tensor
        for (int i = 0; i < n; ++i) {
            hipError_t err = launch_sgd_update(a[i], st);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }
    // small tensors of the narrow classes: all together, one launch per pass
    {
        UpdateArgs seg[UPD_MIX];
        int vec[UPD_MIX], cls[UPD_MIX];
        int k = 0;
        for (int i = 0; i <= n; ++i) {
            const int c = i < n && a[i].rows > 0 ? mixed_class(a[i]) : -1;
            if (c >= 0) {
                seg[k] = a[i];
                vec[k] = update_vec(a[i]);
                cls[k] = c;
                ++k;
            }
            if (k == UPD_MIX || (i == n && k > 0)) {
                hipError_t err = run_mixed(seg, vec, cls, k, st);
                if (err != hipSuccess) return err;
                k = 0;
            }
        }
    }
    // the others: one launch per pass for up to UPD_SEGS tensors of a class
    for (int c = 0; c < 10; ++c) {
        UpdateArgs seg[UPD_SEGS];
        int vec[UPD_SEGS];
        int k = 0;
        for (int i = 0; i <= n; ++i) {
            const bool take = i < n && a[i].rows > 0 && mixed_class(a[i]) < 0 && update_class(a[i]) == c;
            if (take) {
                seg[k] = a[i];
                vec[k] = update_vec(a[i]);
                ++k;
            }
            if (k == UPD_SEGS || (i == n && k > 0)) {
                hipError_t err = run_class_multi(c, seg, vec, k, st);
                if (err != hipSuccess) return err;
                k = 0;
            }
        }
    }
    for (int i = 0; i < n; ++i) {
        if (a[i].rows > 0) continue;
        hipError_t err = empty_update(a[i], st);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace ie
