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

// out[i][k] = in[i][k] re-expressed at *estar (row exponents e[i]).
__global__ void align_rows_kernel(const int8_t *in, const int8_t *e, const int *estar, long long rows,
                                  long long cols, int8_t *out) {
    int es = *estar;
    long long n = rows * cols;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        long long r = i / cols;
        out[i] = (int8_t)rne_shift32(in[i], es - (int)e[r]);
    }
}

hipError_t launch_align_rows(const int8_t *in, const int8_t *e, const int *estar, long long rows,
                             long long cols, int8_t *out, hipStream_t st) {
    long long n = rows * cols;
    if (n <= 0) return hipSuccess;
    prof_begin(st);
    hipLaunchKernelGGL(align_rows_kernel, dim3(blocks_for(n, 256, 16384)), dim3(256), 0, st, in, e,
                       estar, rows, cols, out);
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// w viewed as [A][B][C] (row exponent e[a]): out[c][b][a] = w[a][b][c] at *estar.
__global__ __launch_bounds__(256) void align_transpose_kernel(const int8_t *w, const int8_t *e, int e_row,
                                                              const int *estar, int A, int B, int C,
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
        if (a < A && c < C) out[((long long)c * B + b) * A + a] = tile[la][lc];
    }
}

hipError_t launch_align_transpose(const int8_t *w, const int8_t *e, int e_row, const int *estar, int A,
                                  int B, int C, int8_t *out, hipStream_t st) {
    if (A <= 0 || B <= 0 || C <= 0) return hipSuccess;
    dim3 grid((C + 63) / 64, (A + 63) / 64, B);
    prof_begin(st);
    hipLaunchKernelGGL(align_transpose_kernel, grid, dim3(256), 0, st, w, e, e_row, estar, A, B, C, out);
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// Second pass of the round-to-odd epilogue: C = rne(v, e_group - p).
__global__ __launch_bounds__(256) void rto_finalize_kernel(const int16_t *v16, const int16_t *p16,
                                                           const int *gneed, int M, int N, int n_ct,
                                                           int row_group, int8_t *out, int8_t *out_exp,
                                                           uint32_t *flags) {
    for (int row = blockIdx.x; row < M; row += gridDim.x) {
        int e = clamp_exp_flag(max(E_MIN, gneed[row_group ? row : 0]), flags);
        const int16_t *v = v16 + (long long)row * N;
        int8_t *o = out + (long long)row * N;
        const int16_t *pr = p16 + (long long)row * n_ct;
        for (int col = threadIdx.x; col < N; col += 256) {
            int p = pr[col / BN];
            o[col] = (int8_t)rne_shift32(v[col], e - p);
        }
        if (threadIdx.x == 0 && (row_group || row == 0)) out_exp[row_group ? row : 0] = (int8_t)e;
    }
}

hipError_t launch_rto_finalize(const int16_t *v16, const int16_t *p16, const int *gneed, int M, int N,
                               int n_ct, int row_group, int8_t *out, int8_t *out_exp, uint32_t *flags,
                               hipStream_t st) {
    if (M <= 0) return hipSuccess;
    int blocks = M < 16384 ? M : 16384;
    prof_begin(st);
    hipLaunchKernelGGL(rto_finalize_kernel, dim3(blocks), dim3(256), 0, st, v16, p16, gneed, M, N, n_ct,
                       row_group, out, out_exp, flags);
    prof_end(st, PROF_RTO_FINALIZE);
    return hipGetLastError();
}

// Weight-gradient finalize: merge exact int32 partial sums in int64, then
// requantise per output channel (row) or over the whole tensor.
//   mode 0: row groups, one pass.  mode 1: whole tensor, raise gneed[0].
//   mode 2: whole tensor, round with gneed[0].
__global__ __launch_bounds__(256) void dw_finalize_kernel(const int *partial, int splits, long long stride,
                                                          int N, int K, const int *eps_a, const int *eps_b,
                                                          int mode, int *gneed, int8_t *out, int8_t *out_exp,
                                                          uint32_t *flags) {
    __shared__ int sh[4];
    int eps = *eps_a + *eps_b;
    for (int row = blockIdx.x; row < N; row += gridDim.x) {
        const int *p = partial + (long long)row * K;
        int e;
        if (mode != 2) {
            int m = NEED_NONE;
            for (int k = threadIdx.x; k < K; k += 256) {
                long long s = 0;
                for (int z = 0; z < splits; ++z) s += p[z * stride + k];
                m = max(m, need64(s, eps));
            }
            m = block_max256(m, sh);
            if (mode == 1) {
                if (threadIdx.x == 0 && m != NEED_NONE) atomicMax(gneed, m);
                continue;
            }
            e = clamp_exp_flag(max(E_MIN, m), flags);
        } else {
            e = clamp_exp_flag(max(E_MIN, *gneed), flags);
        }
        for (int k = threadIdx.x; k < K; k += 256) {
            long long s = 0;
            for (int z = 0; z < splits; ++z) s += p[z * stride + k];
            out[(long long)row * K + k] = (int8_t)rne_shift64(s, e - eps);
        }
        if (threadIdx.x == 0 && (mode == 0 || row == 0)) out_exp[mode == 0 ? row : 0] = (int8_t)e;
    }
}

hipError_t launch_dw_finalize(const int *partial, int splits, long long split_stride, int N, int K,
                              const int *eps_a, const int *eps_b, int row_group, int *gneed, int8_t *out,
                              int8_t *out_exp, uint32_t *flags, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    int blocks = N < 8192 ? N : 8192;
    if (row_group) {
        prof_begin(st);
        hipLaunchKernelGGL(dw_finalize_kernel, dim3(blocks), dim3(256), 0, st, partial, splits, split_stride,
                           N, K, eps_a, eps_b, 0, gneed, out, out_exp, flags);
        prof_end(st, PROF_DW_FINALIZE);
        return hipGetLastError();
    }
    hipError_t err = launch_fill_i32(gneed, 1, NEED_NONE, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dw_finalize_kernel, dim3(blocks), dim3(256), 0, st, partial, splits, split_stride, N,
                       K, eps_a, eps_b, 1, gneed, out, out_exp, flags);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(dw_finalize_kernel, dim3(blocks), dim3(256), 0, st, partial, splits, split_stride, N,
                       K, eps_a, eps_b, 2, gneed, out, out_exp, flags);
    return hipGetLastError();
}

}  // namespace ie
