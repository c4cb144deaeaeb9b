// Auxiliary kernels of the (C, e) layer step: fills, the common exponent of
// an operand aligned along a contraction axis, alignment copies, and the
// finalize passes of results whose groups span several GEMM tiles.
//
// Alignment ("Memory-Efficient Integer-Only Training of Deep Neural
// Networks", Table 6: products over operands whose exponents vary along the
// summed axis) re-expresses every row at the largest row exponent e*:
// C' = C / 2^(e* - e_row), rounded half to even.
#include <vector>

#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

// ---------------------------------------------------------------------------
// Optional kernel timing
// ---------------------------------------------------------------------------

namespace {
struct ProfRec {
    hipEvent_t start, stop;
    int kind;
};
bool g_prof_on = false;
std::vector<hipEvent_t> g_pool;
std::vector<ProfRec> g_recs;
hipEvent_t g_pending = nullptr;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

void prof_begin(hipStream_t st) {
    if (!g_prof_on) return;
    g_pending = take_event();
    if (g_pending) (void)hipEventRecord(g_pending, st);
}

void prof_end(hipStream_t st, int kind) {
    if (!g_prof_on || !g_pending) return;
    hipEvent_t e = take_event();
    if (!e) return;
    (void)hipEventRecord(e, st);
    g_recs.push_back({g_pending, e, kind});
    g_pending = nullptr;
}

void prof_enable(int on) {
    g_prof_on = on != 0;
    for (auto &r : g_recs) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_recs.clear();
}

int prof_read(float *ms, int *kind, int max) {
    int n = (int)g_recs.size();
    for (int i = 0; i < n; ++i) {
        ProfRec &r = g_recs[i];
        float t = 0.f;
        if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&t, r.start, r.stop);
        if (i < max) {
            if (ms) ms[i] = t;
            if (kind) kind[i] = r.kind;
        }
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_recs.clear();
    return n;
}

__global__ void fill_i32_kernel(int *p, long long n, int v) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void fill_i8_kernel(int8_t *p, long long n, int v) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        p[i] = (int8_t)v;
}

static int blocks_for(long long n, int per_block, int cap = 4096) {
    long long b = (n + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

hipError_t launch_fill_i32(int *p, long long n, int v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_i8(int8_t *p, long long n, int v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i8_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_zero_flags(void *ws, hipStream_t st) {
    return launch_fill_i32((int *)ws, 64, 0, st);
}

__device__ __forceinline__ void raise_max_aux(int *p, int v) {
    if (v > __atomic_load_n(p, __ATOMIC_RELAXED)) atomicMax(p, v);
}

__device__ __forceinline__ int block_wave_max(int v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ int block_max256(int v, int *sh) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

// out[0] = largest of n int8 exponents (E_MIN when n == 0).
__global__ __launch_bounds__(256) void exp_max_kernel(const int8_t *e, long long n, int *out) {
    __shared__ int sh[4];
    int m = E_MIN;
    for (long long i = threadIdx.x; i < n; i += 256) m = max(m, (int)e[i]);
    m = block_max256(m, sh);
    if (threadIdx.x == 0) out[0] = m;
}

hipError_t launch_exp_max(const int8_t *e, long long n, int *out, hipStream_t st) {
    hipLaunchKernelGGL(exp_max_kernel, dim3(1), dim3(256), 0, st, e, n, out);
    return hipGetLastError();
}

// out[i][k] = in[i][k] re-expressed at *estar (row exponents e[i]; no shift
// when estar is null), for k < cols; zeros for cols <= k < cols_p.
__global__ void pad_rows_kernel(const int8_t *in, long long rows, long long cols, const int8_t *e, int e_row,
                                const int *estar, long long cols_p, int8_t *out) {
    const int es = estar ? *estar : 0;
    const long long n = rows * cols_p;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        const long long r = i / cols_p, c = i - r * cols_p;
        int v = 0;
        if (c < cols) {
            v = in[r * cols + c];
            if (estar) v = rne_shift32(v, es - (e_row ? (int)e[r] : (int)e[0]));
        }
        out[i] = (int8_t)v;
    }
}

hipError_t launch_pad_rows(const int8_t *in, long long rows, long long cols, const int8_t *e, int e_row,
                           const int *estar, long long cols_p, int8_t *out, hipStream_t st) {
    const long long n = rows * cols_p;
    if (n <= 0) return hipSuccess;
    prof_begin(st);
    hipLaunchKernelGGL(pad_rows_kernel, dim3(blocks_for(n, 256, 16384)), dim3(256), 0, st, in, rows, cols, e,
                       e_row, estar, cols_p, out);
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// w viewed as [A][B][C] (row exponent e[a]): out[c][b][a] = w[a][b][c] at
// *estar for a < A, zero for A <= a < Ap (output pitch Ap).
__global__ __launch_bounds__(256) void align_transpose_kernel(const int8_t *w, const int8_t *e, int e_row,
                                                              const int *estar, int A, int B, int C, int Ap,
                                                              int8_t *out) {
    __shared__ int8_t tile[64][65];
    int es = *estar;
    int c0 = blockIdx.x * 64, a0 = blockIdx.y * 64, b = blockIdx.z;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int la = i >> 6, lc = i & 63;
        int a = a0 + la, c = c0 + lc;
        int8_t v = 0;
        if (a < A && c < C) {
            int ea = e_row ? (int)e[a] : (int)e[0];
            v = (int8_t)rne_shift32(w[((long long)a * B + b) * C + c], es - ea);
        }
        tile[la][lc] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        int lc = i >> 6, la = i & 63;
        int a = a0 + la, c = c0 + lc;
        if (a < Ap && c < C) out[((long long)c * B + b) * Ap + a] = tile[la][lc];
    }
}

hipError_t launch_align_transpose(const int8_t *w, const int8_t *e, int e_row, const int *estar, int A, int B,
                                  int C, int Ap, int8_t *out, hipStream_t st) {
    if (Ap <= 0 || B <= 0 || C <= 0) return hipSuccess;
    dim3 grid((C + 63) / 64, (Ap + 63) / 64, B);
    prof_begin(st);
    hipLaunchKernelGGL(align_transpose_kernel, grid, dim3(256), 0, st, w, e, e_row, estar, A, B, C, Ap, out);
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------

FastDiv make_fastdiv(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;  // l = ceil(log2 d)
    int s = 31 + l;
    uint64_t m = ((1ull << s) + d - 1) / d;
    return FastDiv{(uint32_t)m, s};
}

hipError_t launch_gemm(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                       int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (A.kind == LD_K && B.kind == LD_K) return launch_gemm_kk(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_IM2COL && B.kind == LD_K)
        return launch_gemm_im2col(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_DGRAD && B.kind == LD_K)
        return launch_gemm_dgrad(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_T) return launch_gemm_wgrad(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Second pass of the round-to-odd epilogue: C = rne(v, e_group - p).
// Each thread rounds 8 consecutive elements of a row (or 1 when the row
// length is not a multiple of 8).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t fdiv32(uint32_t n, FastDiv f) { return (uint32_t)(((uint64_t)n * f.m) >> f.s); }

__global__ __launch_bounds__(256) void rto_finalize_kernel(const int16_t *v16, const int16_t *p16,
                                                           const int *gneed, int M, int N, int bm, int bn,
                                                           int TM, int n_ct, int row_group, int8_t *out,
                                                           int8_t *out_exp, uint32_t *flags, int vw,
                                                           FastDiv dper) {
    const uint32_t per_row = N / vw;
    const uint32_t total = (uint32_t)M * per_row;
    const int eT = row_group ? 0 : clamp_exp_flag(max(E_MIN, gneed[0]), flags);
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
        const uint32_t row = fdiv32(i, dper);
        const int c0 = (int)(i - row * per_row) * vw;
        const int e = row_group ? clamp_exp_flag(max(E_MIN, gneed[row]), flags) : eT;
        const int p = row_group ? p16[(long long)row * n_ct + c0 / bn] : p16[row / bm + TM * (c0 / bn)];
        const int sh = e - p;
        const long long o = (long long)row * N + c0;
        if (vw == 8) {
            v4i v = *(const v4i *)(v16 + o);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int x = (int)(int16_t)((uint32_t)v[j] & 0xffff), y = (int)(int16_t)((uint32_t)v[j] >> 16);
                uint32_t b = ((uint32_t)(uint8_t)rne_shift32(x, sh)) | ((uint32_t)(uint8_t)rne_shift32(y, sh) << 8);
                if (j < 2) lo |= b << (16 * j);
                else hi |= b << (16 * (j - 2));
            }
            *(v2i *)(out + o) = v2i{(int)lo, (int)hi};
        } else {
            out[o] = (int8_t)rne_shift32(v16[o], sh);
        }
        if (row_group && c0 == 0) out_exp[row] = (int8_t)e;
    }
    if (!row_group && blockIdx.x == 0 && threadIdx.x == 0) out_exp[0] = (int8_t)eT;
}

hipError_t launch_rto_finalize(const int16_t *v16, const int16_t *p16, const int *gneed, int M, int N, Tile t,
                               int row_group, int8_t *out, int8_t *out_exp, uint32_t *flags, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int vw = (N % 8 == 0 && ((uintptr_t)out % 8) == 0) ? 8 : 1;
    const long long total = (long long)M * (N / vw);
    const int TM = (M + t.bm() - 1) / t.bm();
    const int n_ct = (N + t.bn() - 1) / t.bn();
    prof_begin(st);
    hipLaunchKernelGGL(rto_finalize_kernel, dim3(blocks_for(total, 256, 8192)), dim3(256), 0, st, v16, p16,
                       gneed, M, N, t.bm(), t.bn(), TM, n_ct, row_group, out, out_exp, flags, vw,
                       make_fastdiv((uint32_t)(N / vw)));
    prof_end(st, PROF_RTO_FINALIZE);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-contraction finalize.  Pass 1 sums the int32 partials of every
// element in int64 and raises its group's maximum smallest exponent; pass 2
// rounds the sums.  Each thread owns 4 consecutive elements of a row (or 1).
// ---------------------------------------------------------------------------

// Block = 64 element chunks x 4 split subsets; subset j sums splits j, j+4, ...
__global__ __launch_bounds__(256) void partial_reduce_kernel(const int *partial, int splits, long long stride,
                                                             int M, int N, ExpSrc ea, ExpSrc eb, int row_group,
                                                             long long *sums, int *gneed, int vw,
                                                             FastDiv dper) {
    __shared__ long long sh[3][64][4];
    const uint32_t per_row = N / vw;
    const uint32_t total = (uint32_t)M * per_row;
    const int sub = threadIdx.x >> 6, lc = threadIdx.x & 63;
    for (uint32_t base = blockIdx.x * 64; base < total; base += gridDim.x * 64) {
        const uint32_t i = base + lc;
        long long s0 = 0, s1 = 0, s2 = 0, s3 = 0;
        uint32_t row = 0;
        int c0 = 0;
        long long o = 0;
        if (i < total) {
            row = fdiv32(i, dper);
            c0 = (int)(i - row * per_row) * vw;
            o = (long long)row * N + c0;
            if (vw == 4) {
#pragma unroll 4
                for (int zz = sub; zz < splits; zz += 4) {
                    v4i v = *(const v4i *)(partial + zz * stride + o);
                    s0 += v[0];
                    s1 += v[1];
                    s2 += v[2];
                    s3 += v[3];
                }
            } else {
#pragma unroll 4
                for (int zz = sub; zz < splits; zz += 4) s0 += partial[zz * stride + o];
            }
        }
        if (sub > 0) {
            sh[sub - 1][lc][0] = s0;
            sh[sub - 1][lc][1] = s1;
            sh[sub - 1][lc][2] = s2;
            sh[sub - 1][lc][3] = s3;
        }
        __syncthreads();
        if (sub == 0) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                s0 += sh[j][lc][0];
                s1 += sh[j][lc][1];
                s2 += sh[j][lc][2];
                s3 += sh[j][lc][3];
            }
            int m = NEED_NONE;
            if (i < total) {
                const int er = exp_at(ea, row);
                if (vw == 4) {
                    long long *so = sums + o;
                    so[0] = s0;
                    so[1] = s1;
                    so[2] = s2;
                    so[3] = s3;
                    m = max(max(need64(s0, er + exp_at(eb, c0)), need64(s1, er + exp_at(eb, c0 + 1))),
                            max(need64(s2, er + exp_at(eb, c0 + 2)), need64(s3, er + exp_at(eb, c0 + 3))));
                } else {
                    sums[o] = s0;
                    m = need64(s0, er + exp_at(eb, c0));
                }
            }
            // wave 0 (all 64 lanes) reduces its chunks: rows of consecutive
            // chunks are non-decreasing, so segment at the first lane's row
            // (lane 0 holds the wave's first chunk; invalid lanes carry no value)
            const uint32_t r0 = __shfl((int)row, 0);
            if (i >= total) row = r0;
            const uint32_t rmax_ = (uint32_t)block_wave_max((int)row);
            if (!row_group || r0 == rmax_) {
                m = block_wave_max(m);
                if (lc == 0 && m != NEED_NONE) raise_max_aux(&gneed[row_group ? r0 : 0], m);
            } else if (per_row >= 64) {
                // 64 consecutive chunks of rows of >= 64 chunks: two rows at most
                int m0 = block_wave_max(row == r0 ? m : NEED_NONE);
                int m1 = block_wave_max(row == r0 ? NEED_NONE : m);
                if (lc == 0 && m0 != NEED_NONE) raise_max_aux(&gneed[r0], m0);
                if (lc == 0 && m1 != NEED_NONE) raise_max_aux(&gneed[rmax_], m1);
            } else if (m != NEED_NONE) {
                raise_max_aux(&gneed[row], m);
            }
        }
        __syncthreads();
    }
}

// Output [M x N]; sums [M x src_pitch]: output column j reads source column j,
// or (j / c) * cp + j % c when the source pads each group of c columns to cp.
__global__ __launch_bounds__(256) void round_sums_kernel(const long long *sums, int M, int N, int src_pitch,
                                                         int mc, int mcp, FastDiv dmc, ExpSrc ea, ExpSrc eb,
                                                         int row_group, const int *gneed, int8_t *out,
                                                         int8_t *out_exp, uint32_t *flags, int vw, FastDiv dper) {
    const uint32_t per_row = N / vw;
    const uint32_t total = (uint32_t)M * per_row;
    const int eT = row_group ? 0 : clamp_exp_flag(max(E_MIN, gneed[0]), flags);
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
        const uint32_t row = fdiv32(i, dper);
        const int c0 = (int)(i - row * per_row) * vw;
        const long long o = (long long)row * N + c0;
        const long long so = (long long)row * src_pitch;
        const int e = row_group ? clamp_exp_flag(max(E_MIN, gneed[row]), flags) : eT;
        const int er = exp_at(ea, row);
        uint32_t w = 0;
        for (int j = 0; j < vw; ++j) {
            const uint32_t col = c0 + j;
            uint32_t sc = col;
            if (mc != mcp) {
                const uint32_t g = fdiv32(col, dmc);
                sc = g * mcp + (col - g * mc);
            }
            w |= (uint32_t)(uint8_t)rne_shift64(sums[so + sc], e - (er + exp_at(eb, col))) << (8 * j);
        }
        if (vw == 4) *(uint32_t *)(out + o) = w;
        else out[o] = (int8_t)w;
        if (row_group && c0 == 0) out_exp[row] = (int8_t)e;
    }
    if (!row_group && blockIdx.x == 0 && threadIdx.x == 0) out_exp[0] = (int8_t)eT;
}

hipError_t launch_partial_reduce(const int *partial, int splits, long long split_stride, int M, int N,
                                 ExpSrc ea, ExpSrc eb, int row_group, long long *sums, int *gneed,
                                 hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    hipError_t err = launch_fill_i32(gneed, row_group ? M : 1, NEED_NONE, st);
    if (err != hipSuccess) return err;
    const int vw = (N % 4 == 0) ? 4 : 1;
    const long long total = (long long)M * (N / vw);
    prof_begin(st);
    hipLaunchKernelGGL(partial_reduce_kernel, dim3(blocks_for(total, 64, 8192)), dim3(256), 0, st, partial,
                       splits, split_stride, M, N, ea, eb, row_group, sums, gneed, vw,
                       make_fastdiv((uint32_t)(N / vw)));
    prof_end(st, PROF_PARTIAL_REDUCE);
    return hipGetLastError();
}

hipError_t launch_round_sums(const long long *sums, int M, int N, int src_pitch, int mc, int mcp, ExpSrc ea,
                             ExpSrc eb, int row_group, const int *gneed, int8_t *out, int8_t *out_exp,
                             uint32_t *flags, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int vw = (N % 4 == 0 && ((uintptr_t)out % 4) == 0) ? 4 : 1;
    const long long total = (long long)M * (N / vw);
    prof_begin(st);
    hipLaunchKernelGGL(round_sums_kernel, dim3(blocks_for(total, 256, 8192)), dim3(256), 0, st, sums, M, N,
                       src_pitch, mc, mcp, make_fastdiv((uint32_t)(mc > 0 ? mc : 1)), ea, eb, row_group, gneed,
                       out, out_exp, flags, vw, make_fastdiv((uint32_t)(N / vw)));
    prof_end(st, PROF_ROUND_SUMS);
    return hipGetLastError();
}

}  // namespace ie
