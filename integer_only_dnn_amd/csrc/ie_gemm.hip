// int8 x int8 -> int32 contraction on CDNA4 MFMA with a fused (C, e)
// requantisation epilogue.
//
// Implements the "Product" building block ("Memory-Efficient Integer-Only
// Training of Deep Neural Networks", Table 6: convolution, linear; Figure 1a:
// forward and backward of every layer): acc = sum_k A(m,k) B(n,k) exactly in
// int32, exponent eps = e_A(m) + e_B(n), then the result group's exponent is
// the smallest that brings every |C| to 127 or less (ties to even).
//
// One workgroup (4 waves) computes a 128 x 128 tile with
// v_mfma_i32_32x32x32_i8; each wave owns 64 x 64 (2 x 2 MFMA tiles).
// Operands are staged through LDS in K-contiguous rows (double buffered);
// loaders handle the operand layouts: K-contiguous matrices, M-contiguous
// matrices (4x4 byte transposes in registers), and the implicit-GEMM views of
// a convolution (im2col, input-gradient gather, transposed im2col).
//
// Epilogues:
//   DIRECT  - the result group lies inside the tile: reduce, round, store int8.
//   RTO     - the group spans tiles: store round-to-odd int16 values at a
//             per-(row, tile) exponent two or more bits below the final one,
//             and atomically raise the group's maximum; a finalize kernel
//             then rounds half to even, which equals rounding the exact value.
//   PARTIAL - store exact int32 partial sums (split contraction) for a
//             finalize kernel that merges them in int64.
#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

constexpr int NTHR = 256;
constexpr int LDK = BK + 16;  // LDS row stride in bytes (16 B of padding)

__device__ __forceinline__ void tr4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                    uint32_t &o0, uint32_t &o1, uint32_t &o2, uint32_t &o3) {
    // Byte transpose of a 4x4 block: o_j byte i = a_i byte j.
    uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
    uint32_t t1 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
    uint32_t t2 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
    uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
    o0 = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
    o1 = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
    o2 = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
    o3 = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

__device__ __forceinline__ void put_byte(uint32_t *w, int b, int8_t v) {
    w[b >> 2] |= (uint32_t)(uint8_t)v << (8 * (b & 3));
}

// ---------------------------------------------------------------------------
// Loaders.  Each thread moves 32 bytes of a [128 x 64] operand tile per step.
// ---------------------------------------------------------------------------

template <int KIND>
struct Loader;

// K-contiguous rows: thread owns two 16-byte chunks (row, 16-byte column).
template <int KIND>
struct LoaderKRows {
    v4i reg[2];
    int kc;
    int rowc[2];

    __device__ __forceinline__ void store(int8_t *s) const {
#pragma unroll
        for (int c = 0; c < 2; ++c) *(v4i *)(s + rowc[c] * LDK + kc * 16) = reg[c];
    }
};

template <>
struct Loader<LD_K> : LoaderKRows<LD_K> {
    const int8_t *base;
    long long ld;
    int rows, vec;

    __device__ __forceinline__ void init(const Operand &op, int i0, int tid) {
        base = op.base;
        ld = op.ld;
        rows = op.rows;
        vec = op.vec;
        kc = tid & 3;
        rowc[0] = tid >> 2;
        rowc[1] = (tid + NTHR) >> 2;
    }
    __device__ __forceinline__ void load(int i0, int k0, int kend) {
        int k = k0 + kc * 16;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            int i = i0 + rowc[c];
            if (vec) {
                v4i z = {0, 0, 0, 0};
                reg[c] = (i < rows && k < kend) ? *(const v4i *)(base + (long long)i * ld + k) : z;
            } else {
                uint32_t w[4] = {0, 0, 0, 0};
                if (i < rows) {
                    const int8_t *p = base + (long long)i * ld;
                    for (int b = 0; b < 16; ++b)
                        if (k + b < kend) put_byte(w, b, p[k + b]);
                }
                reg[c] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        }
    }
};

// Convolution forward: row m = (n, p, q) output pixel, k = (r, s, c).
template <>
struct Loader<LD_IM2COL> : LoaderKRows<LD_IM2COL> {
    const int8_t *x;
    ConvGeom g;
    int rows, vec;
    int hb[2], wb[2];
    long long pix[2];
    bool ok[2];

    __device__ __forceinline__ void init(const Operand &op, int i0, int tid) {
        x = op.base;
        g = op.g;
        rows = op.rows;
        vec = op.vec;
        kc = tid & 3;
        rowc[0] = tid >> 2;
        rowc[1] = (tid + NTHR) >> 2;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            int m = i0 + rowc[c];
            ok[c] = m < rows;
            int mm = ok[c] ? m : 0;
            int pq = g.p * g.q;
            int n = mm / pq, rem = mm - n * pq;
            int p = rem / g.q, q = rem - p * g.q;
            hb[c] = p * g.stride - g.pad;
            wb[c] = q * g.stride - g.pad;
            pix[c] = (long long)n * g.h * g.w * g.c;
        }
    }
    __device__ __forceinline__ int8_t fetch(int c, int kk, int kend) const {
        if (!ok[c] || kk >= kend) return 0;
        int rs = kk / g.c, ch = kk - rs * g.c;
        int r = rs / g.s, s = rs - r * g.s;
        int h = hb[c] + r, w = wb[c] + s;
        if (h < 0 || h >= g.h || w < 0 || w >= g.w) return 0;
        return x[pix[c] + ((long long)h * g.w + w) * g.c + ch];
    }
    __device__ __forceinline__ void load(int i0, int k0, int kend) {
        int kk = k0 + kc * 16;
        if (vec) {
            int rs = kk / g.c, ch = kk - rs * g.c;
            int r = rs / g.s, s = rs - r * g.s;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                int h = hb[c] + r, w = wb[c] + s;
                bool in = ok[c] && kk < kend && h >= 0 && h < g.h && w >= 0 && w < g.w;
                v4i z = {0, 0, 0, 0};
                reg[c] = in ? *(const v4i *)(x + pix[c] + ((long long)h * g.w + w) * g.c + ch) : z;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                uint32_t w[4] = {0, 0, 0, 0};
                for (int b = 0; b < 16; ++b) put_byte(w, b, fetch(c, kk + b, kend));
                reg[c] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        }
    }
};

// Convolution input gradient: row m = (n, h, w) input pixel, k = (r, s, ko);
// element dY[n, p, q, ko] with p*stride = h + pad - r (zero unless exact).
template <>
struct Loader<LD_DGRAD> : LoaderKRows<LD_DGRAD> {
    const int8_t *dy;
    ConvGeom g;
    int rows, vec;
    int hp[2], wp[2];
    long long pix[2];
    bool ok[2];

    __device__ __forceinline__ void init(const Operand &op, int i0, int tid) {
        dy = op.base;
        g = op.g;
        rows = op.rows;
        vec = op.vec;
        kc = tid & 3;
        rowc[0] = tid >> 2;
        rowc[1] = (tid + NTHR) >> 2;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            int m = i0 + rowc[c];
            ok[c] = m < rows;
            int mm = ok[c] ? m : 0;
            int hw = g.h * g.w;
            int n = mm / hw, rem = mm - n * hw;
            int h = rem / g.w, w = rem - h * g.w;
            hp[c] = h + g.pad;
            wp[c] = w + g.pad;
            pix[c] = (long long)n * g.p * g.q * g.k;
        }
    }
    __device__ __forceinline__ bool tap(int c, int r, int s, long long &off) const {
        int a = hp[c] - r, b = wp[c] - s;
        if (a < 0 || b < 0) return false;
        int p = a / g.stride, q = b / g.stride;
        if (p * g.stride != a || q * g.stride != b || p >= g.p || q >= g.q) return false;
        off = pix[c] + ((long long)p * g.q + q) * g.k;
        return true;
    }
    __device__ __forceinline__ void load(int i0, int k0, int kend) {
        int kk = k0 + kc * 16;
        if (vec) {
            int rs = kk / g.k, ko = kk - rs * g.k;
            int r = rs / g.s, s = rs - r * g.s;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                long long off = 0;
                bool in = ok[c] && kk < kend && tap(c, r, s, off);
                v4i z = {0, 0, 0, 0};
                reg[c] = in ? *(const v4i *)(dy + off + ko) : z;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                uint32_t w[4] = {0, 0, 0, 0};
                for (int b = 0; b < 16; ++b) {
                    int kb = kk + b;
                    if (!ok[c] || kb >= kend) continue;
                    int rs = kb / g.k, ko = kb - rs * g.k;
                    int r = rs / g.s, s = rs - r * g.s;
                    long long off;
                    if (tap(c, r, s, off)) put_byte(w, b, dy[off + ko]);
                }
                reg[c] = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        }
    }
};

// M-contiguous operands: thread owns 8 rows x 4 k; loads 4 runs of 8 bytes
// (one per k) and transposes them into 8 dwords of 4 consecutive k.
template <int KIND>
struct LoaderTRows {
    uint32_t lo[4], hi[4];
    int ig, kg;

    __device__ __forceinline__ void store(int8_t *s) const {
        uint32_t o[8];
        tr4(lo[0], lo[1], lo[2], lo[3], o[0], o[1], o[2], o[3]);
        tr4(hi[0], hi[1], hi[2], hi[3], o[4], o[5], o[6], o[7]);
#pragma unroll
        for (int u = 0; u < 8; ++u) *(uint32_t *)(s + (ig * 8 + u) * LDK + kg * 4) = o[u];
    }
};

template <>
struct Loader<LD_T> : LoaderTRows<LD_T> {
    const int8_t *base;
    long long ld;
    int rows, vec;

    __device__ __forceinline__ void init(const Operand &op, int i0, int tid) {
        base = op.base;
        ld = op.ld;
        rows = op.rows;
        vec = op.vec;
        ig = tid & 15;
        kg = tid >> 4;
    }
    __device__ __forceinline__ void load(int i0, int k0, int kend) {
        int i = i0 + ig * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int k = k0 + kg * 4 + j;
            uint32_t a = 0, b = 0;
            if (k < kend) {
                const int8_t *p = base + (long long)k * ld + i;
                if (vec && i + 8 <= rows) {
                    v2i v = *(const v2i *)p;
                    a = (uint32_t)v.x;
                    b = (uint32_t)v.y;
                } else {
                    uint32_t w[2] = {0, 0};
                    for (int u = 0; u < 8; ++u)
                        if (i + u < rows) put_byte(w, u, p[u]);
                    a = w[0];
                    b = w[1];
                }
            }
            lo[j] = a;
            hi[j] = b;
        }
    }
};

// Convolution weight gradient, B side: row j = (r, s, c), k = output pixel
// (n, p, q); element X[n, p*st + r - pad, q*st + s - pad, c].
template <>
struct Loader<LD_IM2COL_T> : LoaderTRows<LD_IM2COL_T> {
    const int8_t *x;
    ConvGeom g;
    int rows, vec;
    int jr, js, jc;   // (r, s, c) of this thread's first row
    int jb;

    __device__ __forceinline__ void init(const Operand &op, int j0, int tid) {
        x = op.base;
        g = op.g;
        rows = op.rows;
        vec = op.vec;
        ig = tid & 15;
        kg = tid >> 4;
        jb = j0 + ig * 8;
        int rs = jb / g.c;
        jc = jb - rs * g.c;
        jr = rs / g.s;
        js = rs - jr * g.s;
    }
    __device__ __forceinline__ int8_t fetch(int j, int n, int p, int q) const {
        if (j >= rows) return 0;
        int rs = j / g.c, c = j - rs * g.c;
        int r = rs / g.s, s = rs - r * g.s;
        int h = p * g.stride + r - g.pad, w = q * g.stride + s - g.pad;
        if (h < 0 || h >= g.h || w < 0 || w >= g.w) return 0;
        return x[(((long long)n * g.h + h) * g.w + w) * g.c + c];
    }
    __device__ __forceinline__ void load(int j0, int k0, int kend) {
        int pq = g.p * g.q;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            int kk = k0 + kg * 4 + t;
            uint32_t a = 0, b = 0;
            if (kk < kend) {
                int n = kk / pq, rem = kk - n * pq;
                int p = rem / g.q, q = rem - p * g.q;
                if (vec && jb + 8 <= rows) {
                    int h = p * g.stride + jr - g.pad, w = q * g.stride + js - g.pad;
                    if (h >= 0 && h < g.h && w >= 0 && w < g.w) {
                        v2i v = *(const v2i *)(x + (((long long)n * g.h + h) * g.w + w) * g.c + jc);
                        a = (uint32_t)v.x;
                        b = (uint32_t)v.y;
                    }
                } else {
                    uint32_t w2[2] = {0, 0};
                    for (int u = 0; u < 8; ++u) put_byte(w2, u, fetch(jb + u, n, p, q));
                    a = w2[0];
                    b = w2[1];
                }
            }
            lo[t] = a;
            hi[t] = b;
        }
    }
};

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int exp_at(const ExpSrc &e, int idx) {
    if (e.e32) return *e.e32;
    return e.row ? (int)e.e8[idx] : (int)e.e8[0];
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off));
    return v;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int KA, int KB, int EPI>
__global__ __launch_bounds__(NTHR) void gemm_i8_kernel(Operand A, Operand B, int M, int N, int K,
                                                      int k_chunk, int TM, Epi ep) {
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * (BM + BN) * LDK];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tile_m = blockIdx.x % TM;
    const int tile_n = blockIdx.x / TM;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int z = blockIdx.z;
    const int kb = z * k_chunk;
    const int ke = min(K, kb + k_chunk);
    const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

    Loader<KA> la;
    Loader<KB> lb;
    la.init(A, m0, tid);
    lb.init(B, n0, tid);

    v16i acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    if (nk > 0) {
        la.load(m0, kb, ke);
        lb.load(n0, kb, ke);
        la.store(lds);
        lb.store(lds + BM * LDK);
        __syncthreads();
    }
    for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < nk;
        if (more) {
            la.load(m0, kb + (it + 1) * BK, ke);
            lb.load(n0, kb + (it + 1) * BK, ke);
        }
        const int8_t *sA = lds + cur * (BM + BN) * LDK;
        const int8_t *sB = sA + BM * LDK;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v4i af[2], bf[2];
            const int koff = ks * 32 + (lane >> 5) * 16;
#pragma unroll
            for (int a = 0; a < 2; ++a)
                af[a] = *(const v4i *)(sA + (wm * 64 + a * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bf[b] = *(const v4i *)(sB + (wn * 64 + b * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
        if (more) {
            int8_t *nA = lds + (cur ^ 1) * (BM + BN) * LDK;
            la.store(nA);
            lb.store(nA + BM * LDK);
        }
        __syncthreads();
    }

    // Element (a, b, r) of this lane sits at tile row / column:
    //   row = wm*64 + a*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = wn*64 + b*32 + lane%32
    if (EPI == EPI_PARTIAL) {
        int *P = ep.partial + (long long)z * ep.split_stride;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int row = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    int col = n0 + wn * 64 + b * 32 + (lane & 31);
                    if (row < M && col < N) P[(long long)row * N + col] = acc[a][b][r];
                }
        return;
    }

    int ebv[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        int col = n0 + wn * 64 + b * 32 + (lane & 31);
        ebv[b] = col < N ? exp_at(ep.eb, col) : 0;
    }
    // per-row maximum of the smallest exponents, this lane's 2 columns
    int rmax[2][16];
    int eav[2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int row = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            eav[a][r] = row < M ? exp_at(ep.ea, row) : 0;
            int n0v = need32(acc[a][0][r], eav[a][r] + ebv[0]);
            int n1v = need32(acc[a][1][r], eav[a][r] + ebv[1]);
            rmax[a][r] = max(n0v, n1v);
        }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) rmax[a][r] = max(rmax[a][r], __shfl_xor(rmax[a][r], off));

    int *red = (int *)lds;  // [2][BM] row maxima of the two column halves, then [4] wave maxima
    if ((lane & 31) == 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[wn * BM + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] = rmax[a][r];
    }
    __syncthreads();
    int tmax = NEED_NONE;  // this lane's maximum over its rows (whole-tensor groups)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int rt = wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            rmax[a][r] = max(red[rt], red[BM + rt]);
            tmax = max(tmax, rmax[a][r]);
        }
    int gmax = NEED_NONE;
    if (!ep.row_group) {
        tmax = wave_max(tmax);
        __syncthreads();
        if (lane == 0) red[2 * BM + wave] = tmax;
        __syncthreads();
        gmax = max(max(red[2 * BM + 0], red[2 * BM + 1]), max(red[2 * BM + 2], red[2 * BM + 3]));
    }

    if (EPI == EPI_DIRECT) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int row = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                int e = clamp_exp_flag(ep.row_group ? rmax[a][r] : gmax, ep.flags);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    int col = n0 + wn * 64 + b * 32 + (lane & 31);
                    if (col < N)
                        ep.out[(long long)row * N + col] =
                            (int8_t)rne_shift32(acc[a][b][r], e - (eav[a][r] + ebv[b]));
                }
                if (ep.row_group && wn == 0 && (lane & 31) == 0) ep.out_exp[row] = (int8_t)e;
            }
        if (!ep.row_group && tid == 0 && blockIdx.x == 0) ep.out_exp[0] = (int8_t)clamp_exp_flag(gmax, ep.flags);
    } else {  // EPI_RTO
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int row = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                int p = rmax[a][r] == NEED_NONE ? P_NONE : rmax[a][r] - 2;
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    int col = n0 + wn * 64 + b * 32 + (lane & 31);
                    if (col < N)
                        ep.v16[(long long)row * N + col] =
                            (int16_t)rto_shift32(acc[a][b][r], p - (eav[a][r] + ebv[b]));
                }
                if (wn == 0 && (lane & 31) == 0) {
                    ep.p16[(long long)row * ep.n_ct + tile_n] = (int16_t)p;
                    if (ep.row_group && rmax[a][r] != NEED_NONE) atomicMax(&ep.gneed[row], rmax[a][r]);
                }
            }
        if (!ep.row_group && tid == 0 && gmax != NEED_NONE) atomicMax(&ep.gneed[0], gmax);
    }
}

template <int KA, int KB, int EPI>
static hipError_t launch_t(const Operand &A, const Operand &B, int M, int N, int K, int splits,
                           int k_chunk, const Epi &ep, hipStream_t st) {
    int TM = (M + BM - 1) / BM, TN = (N + BN - 1) / BN;
    dim3 grid(TM * TN, 1, splits);
    prof_begin(st);
    hipLaunchKernelGGL((gemm_i8_kernel<KA, KB, EPI>), grid, dim3(NTHR), 0, st, A, B, M, N, K,
                       k_chunk, TM, ep);
    prof_end(st, 1000 + 100 * EPI + 10 * KA + KB);
    return hipGetLastError();
}

hipError_t launch_gemm(const Operand &A, const Operand &B, int M, int N, int K, int splits,
                       int k_chunk, int epi, const Epi &ep, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
#define IE_CASE(KA, KB, E) \
    if (A.kind == KA && B.kind == KB && epi == E) return launch_t<KA, KB, E>(A, B, M, N, K, splits, k_chunk, ep, st);
    IE_CASE(LD_K, LD_K, EPI_DIRECT)
    IE_CASE(LD_K, LD_K, EPI_RTO)
    IE_CASE(LD_IM2COL, LD_K, EPI_DIRECT)
    IE_CASE(LD_IM2COL, LD_K, EPI_RTO)
    IE_CASE(LD_DGRAD, LD_K, EPI_DIRECT)
    IE_CASE(LD_DGRAD, LD_K, EPI_RTO)
    IE_CASE(LD_T, LD_T, EPI_PARTIAL)
    IE_CASE(LD_T, LD_IM2COL_T, EPI_PARTIAL)
#undef IE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ie
