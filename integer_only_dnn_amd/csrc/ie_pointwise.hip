// Pointwise steps beside a layer's products ("Memory-Efficient Integer-Only
// Training of Deep Neural Networks", Table 6 "Sum" and Table 7 "Clip
// activations"):
//   - ReLU / ReLU6 forward act on the mantissas alone (the exponent is kept):
//     max(C, 0), and for ReLU6 min(., c6) with c6 = floor(6 * 2^-e) capped at
//     the activation's largest mantissa 2^q - 1 (127 for INT8), e the
//     element's group exponent;
//   - their backward passes mask the incoming gradient's mantissas where the
//     forward output was clipped (dY's exponents are kept);
//   - Sum is the exact elementwise A + B, rounded once (half to even) into
//     the output's groups and its mantissa width (|C| <= 2^q - 1).
// All three are HBM-bound streams: one 16-byte chunk per thread and trip.
#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

// floor(6 * 2^-e), at most 2^q - 1 (q <= 7)
__device__ __forceinline__ int relu6_cap(int e, int q) {
    if (e >= 3) return 0;
    const int c = e >= 0 ? 6 >> e : (-e >= 5 ? 192 : 6 << -e);
    return min(c, (1 << q) - 1);
}

// Walks the bytes of one 16-byte chunk of a row-major [rows x cols] buffer
// (flat byte offset f0) with the row of each byte; `row`/`next` track the
// current row and the flat offset where the next row begins.
struct RowWalk {
    long long row, next;
    long long cols;
    __device__ __forceinline__ void start(long long f0, long long cols_) {
        cols = cols_;
        row = cols ? f0 / cols : 0;
        next = (row + 1) * cols;
    }
    __device__ __forceinline__ long long at(long long f) {
        while (f >= next) {
            ++row;
            next += cols;
        }
        return row;
    }
};

__device__ __forceinline__ v4i load16(const int8_t *p, long long f, long long total, bool vec) {
    if (vec && f + 16 <= total) return *(const v4i *)(p + f);
    uint32_t w[4] = {0, 0, 0, 0};
    for (int j = 0; j < 16; ++j)
        if (f + j < total) w[j >> 2] |= (uint32_t)(uint8_t)p[f + j] << (8 * (j & 3));
    return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

__device__ __forceinline__ void store16(int8_t *p, long long f, long long total, bool vec, const v4i &v) {
    if (vec && f + 16 <= total) {
        *(v4i *)(p + f) = v;
        return;
    }
    for (int j = 0; j < 16; ++j)
        if (f + j < total) p[f + j] = (int8_t)((uint32_t)v[j >> 2] >> (8 * (j & 3)));
}

__device__ __forceinline__ int byte_at(const v4i &v, int j) { return (int)(int8_t)((uint32_t)v[j >> 2] >> (8 * (j & 3))); }

__device__ __forceinline__ void set_byte(v4i &v, int j, int c) {
    const int sh = 8 * (j & 3);
    v[j >> 2] = (int)(((uint32_t)v[j >> 2] & ~(0xffu << sh)) | ((uint32_t)(uint8_t)c << sh));
}

// Copy of `n` exponent bytes (grid-stride), skipped when in place.
__device__ __forceinline__ void copy_exps(const int8_t *src, int8_t *dst, long long n) {
    if (src == dst) return;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void relu_fwd_kernel(const int8_t *x, const int8_t *xe, int x_row, int8_t *y,
                                                       int8_t *ye, long long rows, long long cols, int relu6,
                                                       int q, int vec) {
    const long long total = rows * cols;
    copy_exps(xe, ye, x_row ? rows : 1);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long f0 = i * 16;
        v4i v = load16(x, f0, total, vec);
        if (!relu6) {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (int)relu4((uint32_t)v[k]);
        } else {
            RowWalk rw;
            rw.start(f0, cols);
            const int cap_t = relu6_cap(xe[0], q);
            for (int j = 0; j < 16 && f0 + j < total; ++j) {
                const int cap = x_row ? relu6_cap(xe[rw.at(f0 + j)], q) : cap_t;
                set_byte(v, j, min(max(byte_at(v, j), 0), cap));
            }
        }
        store16(y, f0, total, vec, v);
    }
}

__global__ __launch_bounds__(256) void relu_bwd_kernel(const int8_t *dy, const int8_t *dye, int dy_row,
                                                       const int8_t *yc, const int8_t *ye, int y_row, int8_t *dx,
                                                       int8_t *dxe, long long rows, long long cols, int relu6,
                                                       int q, int vec) {
    const long long total = rows * cols;
    copy_exps(dye, dxe, dy_row ? rows : 1);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long f0 = i * 16;
        v4i g = load16(dy, f0, total, vec);
        const v4i c = load16(yc, f0, total, vec);
        if (!relu6) {
            // keep the gradient where the forward output is positive
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t w = (uint32_t)c[k];
                // byte > 0: not negative and not zero
                const uint32_t neg = (w & 0x80808080u) >> 7;
                const uint32_t nz = ((w & 0x7f7f7f7fu) + 0x7f7f7f7fu | w) & 0x80808080u;  // bit 7 set iff byte != 0
                const uint32_t keep = (nz >> 7) & ~neg;
                g[k] = (int)((uint32_t)g[k] & (keep * 0xffu));
            }
        } else {
            RowWalk rw;
            rw.start(f0, cols);
            const int cap_t = relu6_cap(ye[0], q);
            for (int j = 0; j < 16 && f0 + j < total; ++j) {
                const int cap = y_row ? relu6_cap(ye[rw.at(f0 + j)], q) : cap_t;
                const int cv = byte_at(c, j);
                if (!(cv > 0 && cv < cap)) set_byte(g, j, 0);
            }
        }
        store16(dx, f0, total, vec, g);
    }
}

// ---------------------------------------------------------------------------
// Sum.  X * 2^pa + Y * 2^pb with |X|, |Y| <= 128 as n * 2^base: exact for
// exponent gaps up to 30; above, the smaller term (below 2^(P-23), P the
// larger exponent) only decides ties and sticky bits at every exponent the
// result can take (at least P - 7 at any width), so it is replaced by its sign at
// 2^(P-23), which rounds identically.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void sum2(int X, int pa, int Y, int pb, long long &n, int &base) {
    if (X == 0) {
        n = Y;
        base = pb;
        return;
    }
    if (Y == 0) {
        n = X;
        base = pa;
        return;
    }
    int d = pa - pb;
    if (d >= 0) {
        if (d <= 30) {
            n = ((long long)X << d) + Y;
            base = pb;
        } else {
            n = ((long long)X << 23) + (Y > 0 ? 1 : -1);
            base = pa - 23;
        }
        return;
    }
    d = -d;
    if (d <= 30) {
        n = (long long)X + ((long long)Y << d);
        base = pa;
    } else {
        n = ((long long)Y << 23) + (X > 0 ? 1 : -1);
        base = pb - 23;
    }
}

struct AddArgs {
    const int8_t *a, *ae;
    const int8_t *b, *be;
    int8_t *z, *ze;
    int a_row, b_row;
    long long rows, cols;
    int *bmax;  // [gridDim.x] block maxima (whole-tensor output)
    uint32_t *flags;
    int q;      // results have |C| <= 2^q - 1
    int vec;
};

__device__ __forceinline__ int block_max_256(int v, int *sh) {
    v = wave_max_dpp(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

// Both operands with one exponent each and at most 22 bits apart: every
// sum is exact in int32 at the smaller exponent (|n| < 2^30), and the
// largest |n| gives the need.
struct Uni {
    bool on;
    int sa, sb, base;
};

__device__ __forceinline__ Uni uni_of(const AddArgs &p) {
    Uni u{false, 0, 0, 0};
    if (p.a_row || p.b_row) return u;
    const int ea = p.ae[0], eb = p.be[0];
    if (abs(ea - eb) > 22) return u;
    u.on = true;
    u.base = min(ea, eb);
    u.sa = ea - u.base;
    u.sb = eb - u.base;
    return u;
}

__device__ __forceinline__ int sum_uni(const Uni &u, const v4i &va, const v4i &vb, int j) {
    return (byte_at(va, j) << u.sa) + (byte_at(vb, j) << u.sb);
}

// Whole-tensor output, pass 1: every block's largest need.
__global__ __launch_bounds__(256) void add_need_kernel(AddArgs p) {
    __shared__ int sh[4];
    const long long total = p.rows * p.cols;
    int m = NEED_NONE;
    const Uni u = uni_of(p);
    if (u.on) {
        int hi = 0, lo = 0;
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
             i += (long long)gridDim.x * blockDim.x) {
            const long long f0 = i * 16;
            const v4i va = load16(p.a, f0, total, p.vec), vb = load16(p.b, f0, total, p.vec);
            // bytes past the end load as zeros and add nothing
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int n = sum_uni(u, va, vb, j);
                hi = max(hi, n);
                lo = min(lo, n);
            }
        }
        const uint32_t mx = max((uint32_t)hi, 0u - (uint32_t)lo);
        m = mx ? u.base + mant_shift32(mx, p.q) : NEED_NONE;
        m = block_max_256(m, sh);
        if (threadIdx.x == 0) p.bmax[blockIdx.x] = m;
        return;
    }
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long f0 = i * 16;
        const v4i va = load16(p.a, f0, total, p.vec), vb = load16(p.b, f0, total, p.vec);
        RowWalk rw;
        rw.start(f0, p.cols);
        for (int j = 0; j < 16 && f0 + j < total; ++j) {
            const long long r = rw.at(f0 + j);
            long long n;
            int base;
            sum2(byte_at(va, j), p.ae[p.a_row ? r : 0], byte_at(vb, j), p.be[p.b_row ? r : 0], n, base);
            m = max(m, need64(n, base, p.q));
        }
    }
    m = block_max_256(m, sh);
    if (threadIdx.x == 0) p.bmax[blockIdx.x] = m;
}

// Whole-tensor output, pass 2: the tensor's exponent from the block maxima
// (every block reduces them itself), then every element rounded.
__global__ __launch_bounds__(256) void add_round_kernel(AddArgs p) {
    __shared__ int sh[4];
    int m = NEED_NONE;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += 256) m = max(m, p.bmax[i]);
    m = block_max_256(m, sh);
    const int e = clamp_exp_flag(max(E_MIN, m), p.flags);
    const long long total = p.rows * p.cols;
    const Uni u = uni_of(p);
    if (u.on) {
        // one shift for every element: n * 2^-(e - base), half to even
        const int s = e - u.base;
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
             i += (long long)gridDim.x * blockDim.x) {
            const long long f0 = i * 16;
            const v4i va = load16(p.a, f0, total, p.vec), vb = load16(p.b, f0, total, p.vec);
            v4i out = v4i{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j) set_byte(out, j, rne_shift32(sum_uni(u, va, vb, j), s));
            store16(p.z, f0, total, p.vec, out);
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) p.ze[0] = (int8_t)e;
        return;
    }
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i * 16 < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long f0 = i * 16;
        const v4i va = load16(p.a, f0, total, p.vec), vb = load16(p.b, f0, total, p.vec);
        v4i out = v4i{0, 0, 0, 0};
        RowWalk rw;
        rw.start(f0, p.cols);
        for (int j = 0; j < 16 && f0 + j < total; ++j) {
            const long long r = rw.at(f0 + j);
            long long n;
            int base;
            sum2(byte_at(va, j), p.ae[p.a_row ? r : 0], byte_at(vb, j), p.be[p.b_row ? r : 0], n, base);
            set_byte(out, j, (int)rne_shift64(n, e - base));
        }
        store16(p.z, f0, total, p.vec, out);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) p.ze[0] = (int8_t)e;
}

// Row-grouped output: one block per row (grid-stride over rows); the row's
// largest need first, then the row rounded (its second read hits L2).
__global__ __launch_bounds__(256) void add_rows_kernel(AddArgs p) {
    __shared__ int sh[4];
    for (long long r = blockIdx.x; r < p.rows; r += gridDim.x) {
        const int ea = p.ae[p.a_row ? r : 0], eb = p.be[p.b_row ? r : 0];
        const int8_t *ra = p.a + r * p.cols, *rb = p.b + r * p.cols;
        int m = NEED_NONE;
        for (long long c = threadIdx.x; c < p.cols; c += 256) {
            long long n;
            int base;
            sum2(ra[c], ea, rb[c], eb, n, base);
            m = max(m, need64(n, base, p.q));
        }
        m = block_max_256(m, sh);
        const int e = clamp_exp_flag(max(E_MIN, m), p.flags);
        int8_t *rz = p.z + r * p.cols;
        for (long long c = threadIdx.x; c < p.cols; c += 256) {
            long long n;
            int base;
            sum2(ra[c], ea, rb[c], eb, n, base);
            rz[c] = (int8_t)rne_shift64(n, e - base);
        }
        if (threadIdx.x == 0) p.ze[r] = (int8_t)e;
    }
}

static int grid_for(long long chunks, int cap) {
    long long b = (chunks + 255) / 256;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

static int vec16(const void *a, const void *b, const void *c) {
    return ((uintptr_t)a % 16 == 0) && ((uintptr_t)b % 16 == 0) && ((uintptr_t)c % 16 == 0);
}

hipError_t launch_relu_fwd(const int8_t *x, const int8_t *xe, int x_row, int8_t *y, int8_t *ye, long long rows,
                           long long cols, int relu6, int q, hipStream_t st) {
    const long long chunks = (rows * cols + 15) / 16;
    const int n_e = x_row ? (int)rows : 1;
    if (chunks == 0 && n_e == 0) return hipSuccess;
    prof_begin(st, PROF_RELU_FWD);
    hipLaunchKernelGGL(relu_fwd_kernel, dim3(grid_for(chunks, 4096)), dim3(256), 0, st, x, xe, x_row, y, ye, rows,
                       cols, relu6, q, vec16(x, y, y));
    prof_end(st, PROF_RELU_FWD);
    return hipGetLastError();
}

hipError_t launch_relu_bwd(const int8_t *dy, const int8_t *dye, int dy_row, const int8_t *yc, const int8_t *ye,
                           int y_row, int8_t *dx, int8_t *dxe, long long rows, long long cols, int relu6, int q,
                           hipStream_t st) {
    const long long chunks = (rows * cols + 15) / 16;
    const int n_e = dy_row ? (int)rows : 1;
    if (chunks == 0 && n_e == 0) return hipSuccess;
    prof_begin(st, PROF_RELU_BWD);
    hipLaunchKernelGGL(relu_bwd_kernel, dim3(grid_for(chunks, 4096)), dim3(256), 0, st, dy, dye, dy_row, yc, ye,
                       y_row, dx, dxe, rows, cols, relu6, q, vec16(dy, yc, dx));
    prof_end(st, PROF_RELU_BWD);
    return hipGetLastError();
}

hipError_t launch_add(const int8_t *a, const int8_t *ae, int a_row, const int8_t *b, const int8_t *be, int b_row,
                      int8_t *z, int8_t *ze, int z_row, long long rows, long long cols, int *bmax, uint32_t *flags,
                      int q, hipStream_t st) {
    AddArgs p{a, ae, b, be, z, ze, a_row, b_row, rows, cols, bmax, flags, q, vec16(a, b, z)};
    if (z_row) {
        if (rows == 0) return hipSuccess;
        prof_begin(st, PROF_ADD_ROWS);
        hipLaunchKernelGGL(add_rows_kernel, dim3((int)(rows < 8192 ? rows : 8192)), dim3(256), 0, st, p);
        prof_end(st, PROF_ADD_ROWS);
        return hipGetLastError();
    }
    const int g = grid_for((rows * cols + 15) / 16, ADD_MAX_BLOCKS);
    prof_begin(st, PROF_ADD_NEED);
    hipLaunchKernelGGL(add_need_kernel, dim3(g), dim3(256), 0, st, p);
    prof_end(st, PROF_ADD_NEED);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_begin(st, PROF_ADD_ROUND);
    hipLaunchKernelGGL(add_round_kernel, dim3(g), dim3(256), 0, st, p);
    prof_end(st, PROF_ADD_ROUND);
    return hipGetLastError();
}

}  // namespace ie
