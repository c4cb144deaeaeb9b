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
int g_prof_sel = 0;
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

void prof_begin(hipStream_t st, int kind) {
    if (!g_prof_on || (g_prof_sel && kind != g_prof_sel)) return;
    g_pending = take_event();
    if (g_pending) (void)hipEventRecord(g_pending, st);
}

void prof_end(hipStream_t st, int kind) {
    if (!g_prof_on || !g_pending || (g_prof_sel && kind != g_prof_sel)) return;
    hipEvent_t e = take_event();
    if (!e) return;
    (void)hipEventRecord(e, st);
    g_recs.push_back({g_pending, e, kind});
    g_pending = nullptr;
}

void prof_select(int kind) { g_prof_sel = kind; }

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

__device__ __forceinline__ uint32_t fdiv32(uint32_t n, FastDiv f) { return (uint32_t)(((uint64_t)n * f.m) >> f.s); }

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

__device__ __forceinline__ int block_wave_max(int v) { return wave_max_dpp(v); }

__device__ __forceinline__ int block_max256(int v, int *sh) {
    v = wave_max_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

// Largest of n int8 exponents (E_MIN when n == 0), by one block: four
// bytes per load when the array is 4-byte aligned.
__device__ int exp_max_block(const int8_t *e, long long n, int *sh) {
    int m = E_MIN;
    long long i0 = 0;
    if (((uintptr_t)e & 3) == 0) {
        const long long nw = n >> 2;
        const int *w = (const int *)e;
#pragma unroll 4
        for (long long i = threadIdx.x; i < nw; i += blockDim.x) {
            const int v = w[i];
            m = max(m, max(max((int)(int8_t)v, (int)(int8_t)(v >> 8)),
                           max((int)(int8_t)(v >> 16), (int)(int8_t)(v >> 24))));
        }
        i0 = nw << 2;
    }
    for (long long i = i0 + threadIdx.x; i < n; i += blockDim.x) m = max(m, (int)e[i]);
    return block_max256(m, sh);
}

__global__ __launch_bounds__(256) void exp_max2_kernel(const int8_t *e0, long long n0, int *out0, const int8_t *e1,
                                                      long long n1, int *out1) {
    __shared__ int sh[4];
    const int m = blockIdx.x == 0 ? exp_max_block(e0, n0, sh) : exp_max_block(e1, n1, sh);
    if (threadIdx.x == 0) (blockIdx.x == 0 ? out0 : out1)[0] = m;
}

hipError_t launch_exp_max2(const int8_t *e0, long long n0, int *out0, const int8_t *e1, long long n1, int *out1,
                           hipStream_t st) {
    hipLaunchKernelGGL(exp_max2_kernel, dim3(out1 ? 2 : 1), dim3(256), 0, st, e0, n0, out0, e1, n1, out1);
    return hipGetLastError();
}

// out[i][k] = in[i][k] re-expressed at *estar (row exponents e[i]; no shift
// when estar is null), for k < cols; zeros for cols <= k < cols_p.  Each
// thread writes 16 output bytes of one row (cols_p is a multiple of 16);
// the input is read 16 bytes at a time when its rows are 16-byte aligned.
__device__ __forceinline__ uint32_t rne_bytes4(uint32_t w, int sh) {
    uint32_t o = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) o |= (uint32_t)(uint8_t)rne_shift32((int)(int8_t)(w >> (8 * t)), sh) << (8 * t);
    return o;
}

// 16 bytes of a row at byte offset p of a 4-byte aligned buffer of `total`
// bytes, any alignment of p: five aligned dword loads, funnel-shifted (a
// dword reaching past `total` is read byte by byte); bytes of the row past
// `valid` (< 16) are zeroed.
__device__ __forceinline__ v4i load16_row(const int8_t *base, long long p, long long total, int valid) {
    const long long a0 = p & ~3ll;
    const int sh = (int)(p - a0) * 8;
    uint32_t d[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const long long a = a0 + 4 * k;
        if (a + 4 <= total) {
            d[k] = *(const uint32_t *)(base + a);
        } else {
            uint32_t w = 0;
            for (int j = 0; j < 4; ++j)
                if (a + j < total) w |= (uint32_t)(uint8_t)base[a + j] << (8 * j);
            d[k] = w;
        }
    }
    v4i v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t w = sh ? (d[k] >> sh) | (d[k + 1] << (32 - sh)) : d[k];
        const int nb = valid - 4 * k;
        if (nb < 4) w = nb <= 0 ? 0u : w & ((1u << (8 * nb)) - 1u);
        v[k] = (int)w;
    }
    return v;
}

__global__ __launch_bounds__(256) void pad_rows_kernel(const int8_t *in, long long rows, long long cols,
                                                       const int8_t *e, int e_row, const int *estar, long long cols_p,
                                                       int8_t *out, int vec_in, FastDiv dcpr) {
    const int es = estar ? *estar : 0;
    const uint32_t cpr = (uint32_t)(cols_p >> 4);  // 16-byte chunks per row
    const uint32_t n = (uint32_t)(rows * cpr);      // < 2^31 (checked by the launcher)
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const uint32_t r32 = (uint32_t)(((uint64_t)i * dcpr.m) >> dcpr.s);
        const long long r = r32, c0 = (long long)(i - r32 * cpr) << 4;
        const int8_t *src = in + r * cols + c0;
        v4i v;
        if (vec_in && c0 + 16 <= cols) {
            v = *(const v4i *)src;
        } else if (((uintptr_t)in & 3) == 0) {
            v = load16_row(in, r * cols + c0, rows * cols, (int)min(cols - c0, 16ll));
        } else {
            uint32_t w[4] = {0, 0, 0, 0};
            for (int j = 0; j < 16; ++j)
                if (c0 + j < cols) w[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
            v = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
        if (estar) {
            const int sh = es - (e_row ? (int)e[r] : (int)e[0]);
            if (sh != 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (int)rne_bytes4((uint32_t)v[j], sh);
            }
        }
        *(v4i *)(out + r * cols_p + c0) = v;
    }
}

hipError_t launch_pad_rows(const int8_t *in, long long rows, long long cols, const int8_t *e, int e_row,
                           const int *estar, long long cols_p, int8_t *out, hipStream_t st) {
    const long long n = rows * (cols_p >> 4);
    if (n <= 0) return hipSuccess;
    if (n >= (1ll << 31)) return hipErrorInvalidValue;
    const int vec_in = (cols % 16 == 0) && ((uintptr_t)in % 16 == 0);
    prof_begin(st, PROF_ALIGN);
    hipLaunchKernelGGL(pad_rows_kernel, dim3(blocks_for(n, 256, 8192)), dim3(256), 0, st, in, rows, cols, e, e_row,
                       estar, cols_p, out, vec_in, make_fastdiv((uint32_t)(cols_p >> 4)));
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// w viewed as [A][B][C] (row exponent e[a], or e[0]): out[c][b'][a] =
// w[a][b][c] at the largest row exponent e*, zero for A <= a < Ap (output
// pitch Ap, a multiple of 16); b' = b, or with to.st the position of filter
// tap b = (r, s) among the taps sorted by stride phase.  Every block finds
// e* itself (A bytes); block 0 stores it.  A block moves a 64 x 64 tile
// through LDS: with C a multiple of 16 (vec), each thread loads 16 bytes of
// one row a and stores 16 bytes of one output row c; otherwise bytes one at
// a time.
__global__ __launch_bounds__(256) void align_transpose_kernel(const int8_t *w, const int8_t *e, int e_row, int A,
                                                              int B, int C, int Ap, int8_t *out, int *estar_out,
                                                              int vec, TapOrder to) {
    constexpr int TP = 64 + 16;  // tile pitch
    __shared__ __attribute__((aligned(16))) int8_t tile[64 * TP];
    __shared__ int sh[4];
    const int es = e_row ? exp_max_block(e, A, sh) : (int)e[0];
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) estar_out[0] = es;
    const int c0 = blockIdx.x * 64, a0 = blockIdx.y * 64, bi = blockIdx.z;
    int b = bi;
    if (to.st) {
        // tap (r, s) of phase (ph, pw), ph = (r - pad) mod st: its (r / st, s / st)
        // in that phase's row-major block
        const int r = bi / to.s, s_ = bi - r * to.s;
        const int ph = ((r - to.pad) % to.st + to.st) % to.st, pw = ((s_ - to.pad) % to.st + to.st) % to.st;
        const int t = ph * to.st + pw;
        b = to.tap0[t] + (r / to.st) * to.sb[t] + s_ / to.st;
    }
    const int t = threadIdx.x;
    if (vec) {
        const int la = t >> 2, lc = (t & 3) * 16;
        const int a = a0 + la, c = c0 + lc;
        v4i v = v4i{0, 0, 0, 0};
        if (a < A && c < C) {
            v = *(const v4i *)(w + ((long long)a * B + bi) * C + c);
            const int s = es - (e_row ? (int)e[a] : es);
            if (s != 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = (int)rne_bytes4((uint32_t)v[k], s);
            }
        }
        *(v4i *)(tile + la * TP + lc) = v;
        __syncthreads();
        const int oc = t >> 2, oa = (t & 3) * 16;
        if (c0 + oc < C && a0 + oa < Ap) {
            uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j) d[j >> 2] |= (uint32_t)(uint8_t)tile[(oa + j) * TP + oc] << (8 * (j & 3));
            *(v4i *)(out + ((long long)(c0 + oc) * B + b) * Ap + a0 + oa) =
                v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
        }
        return;
    }
    for (int i = t; i < 64 * 64; i += 256) {
        int la = i >> 6, lc = i & 63;
        int a = a0 + la, c = c0 + lc;
        int8_t v = 0;
        if (a < A && c < C) {
            int ea = e_row ? (int)e[a] : es;
            v = (int8_t)rne_shift32(w[((long long)a * B + bi) * C + c], es - ea);
        }
        tile[la * TP + lc] = v;
    }
    __syncthreads();
    for (int i = t; i < 64 * 64; i += 256) {
        int lc = i >> 6, la = i & 63;
        int a = a0 + la, c = c0 + lc;
        if (a < Ap && c < C) out[((long long)c * B + b) * Ap + a] = tile[la * TP + lc];
    }
}

hipError_t launch_align_transpose(const int8_t *w, const int8_t *e, int e_row, int A, int B, int C, int Ap,
                                  int8_t *out, int *estar_out, hipStream_t st, const TapOrder &to) {
    if (Ap <= 0 || B <= 0 || C <= 0) return hipSuccess;
    dim3 grid((C + 63) / 64, (Ap + 63) / 64, B);
    const int vec = C % 16 == 0 && Ap % 16 == 0 && ((uintptr_t)w % 16) == 0 && ((uintptr_t)out % 16) == 0;
    prof_begin(st, PROF_ALIGN);
    hipLaunchKernelGGL(align_transpose_kernel, grid, dim3(256), 0, st, w, e, e_row, A, B, C, Ap, out, estar_out,
                       vec, to);
    prof_end(st, PROF_ALIGN);
    return hipGetLastError();
}

// Batched row alignment with padding: slice z = blockIdx.y; every block finds
// the slice's largest row exponent itself (R bytes) and block (0, z) stores
// it; each thread writes 16 output bytes of one row.
__global__ __launch_bounds__(256) void pad_rows_z_kernel(const int8_t *in, const int8_t *e, int e_row, int R,
                                                         int cols, int cols_p, int8_t *out, int *estar,
                                                         FastDiv dcpr) {
    __shared__ int sh[4];
    const int z = blockIdx.y;
    const int8_t *ez = e_row ? e + (long long)z * R : e;
    const int8_t *iz = in + (long long)z * R * cols;
    int8_t *oz = out + (long long)z * R * cols_p;
    const uint32_t cpr = (uint32_t)(cols_p >> 4);
    const uint32_t n = (uint32_t)R * cpr;
    const bool vec = (cols & 15) == 0 && ((uintptr_t)in & 15) == 0;
    // chunk i: its row, first column and 16 bytes (zeros past the row)
    auto fetch = [&](uint32_t i, uint32_t &r, int &c0) -> v4i {
        r = fdiv32(i, dcpr);
        c0 = (int)(i - r * cpr) << 4;
        const int valid = min(cols - c0, 16);
        if (vec && valid == 16) return *(const v4i *)(iz + (long long)r * cols + c0);
        if (((uintptr_t)in & 3) == 0)
            return load16_row(in, ((long long)z * R + r) * cols + c0, (long long)gridDim.y * R * cols, valid);
        const int8_t *src = iz + (long long)r * cols + c0;
        uint32_t wv[4] = {0, 0, 0, 0};
        for (int j = 0; j < valid; ++j) wv[j >> 2] |= (uint32_t)(uint8_t)src[j] << (8 * (j & 3));
        return v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    };
    // the first chunk's load goes out before the slice's largest exponent is
    // reduced, so the two memory round trips overlap
    const uint32_t i0 = blockIdx.x * 256 + threadIdx.x;
    uint32_t r0 = 0;
    int c00 = 0;
    v4i v0 = v4i{0, 0, 0, 0};
    if (i0 < n) v0 = fetch(i0, r0, c00);
    const int es = e_row ? exp_max_block(ez, R, sh) : (int)e[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) estar[z] = es;
    for (uint32_t i = i0; i < n; i += gridDim.x * 256) {
        uint32_t r = r0;
        int c0 = c00;
        v4i v = i == i0 ? v0 : fetch(i, r, c0);
        const int sh_ = e_row ? es - (int)ez[r] : 0;
        if (sh_ != 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (int)rne_bytes4((uint32_t)v[j], sh_);
        }
        *(v4i *)(oz + (long long)r * cols_p + c0) = v;
    }
}

hipError_t launch_pad_rows_z(const int8_t *in, const int8_t *e, int e_row, int Z, int R, int cols, int cols_p,
                             int8_t *out, int *estar, hipStream_t st) {
    if (Z <= 0) return hipSuccess;
    if (Z > 65535) return hipErrorInvalidValue;
    const long long n = (long long)R * (cols_p >> 4);
    if (n >= (1ll << 31)) return hipErrorInvalidValue;
    prof_begin(st, PROF_ALIGN_Z);
    hipLaunchKernelGGL(pad_rows_z_kernel, dim3(blocks_for(n > 0 ? n : 1, 1024, 64), Z), dim3(256), 0, st, in, e,
                       e_row, R, cols, cols_p, out, estar, make_fastdiv((uint32_t)(cols_p >> 4 > 0 ? cols_p >> 4 : 1)));
    prof_end(st, PROF_ALIGN_Z);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------


hipError_t launch_gemm(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                       int k_chunk, bool partial, const Epi &ep, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (A.kind == LD_K && B.kind == LD_K) return launch_gemm_kk(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_IM2COL && B.kind == LD_K)
        return launch_gemm_im2col(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_DGRAD && (B.kind == LD_K || B.kind == LD_WT))
        return launch_gemm_dgrad(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    if (A.kind == LD_T) return launch_gemm_wgrad(A, B, M, N, K, t, splits, k_chunk, partial, ep, st);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Second pass of the round-to-odd epilogue: C = rne(v, e_group - p).
// Each thread rounds 8 consecutive elements of a row (or 1 when the row
// length is not a multiple of 8).
// ---------------------------------------------------------------------------


// Whole-tensor groups: every block first takes the maximum of all tile
// needs (T values).  Row groups: a block walks runs of RB rows; the needs of
// a run (RB * n_ct values) go through LDS and one thread per row reduces them.
constexpr int FIN_NEEDS = 2048;

__device__ __forceinline__ void rto_finalize_body(const int16_t *v16, const int16_t *p16, int M, int N,
                                                           int lbm, int lbn, int TM, int n_ct, int row_group, int rb,
                                                           int8_t *out, int8_t *out_exp, uint32_t *flags, int vw,
                                                           FastDiv dper, Act act, int bid, int nblk) {
    __shared__ int sh[4];
    __shared__ int16_t needs[FIN_NEEDS];
    __shared__ int rowe[256];
    const uint32_t per_row = N / vw;
    // eight values held in registers -> eight bytes at out + o
    auto store8 = [&](long long o, const v4i &v, int sh_) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int x = (int)(int16_t)((uint32_t)v[j] & 0xffff), y = (int)(int16_t)((uint32_t)v[j] >> 16);
            uint32_t b = ((uint32_t)(uint8_t)rne_shift32(x, sh_)) | ((uint32_t)(uint8_t)rne_shift32(y, sh_) << 8);
            if (j < 2) lo |= b << (16 * j);
            else hi |= b << (16 * (j - 2));
        }
        lo = act4(lo, act, o);
        hi = act4(hi, act, o + 4);
        *(v2i *)(out + o) = v2i{(int)lo, (int)hi};
    };
    auto round8 = [&](long long o, int sh_) {
        if (vw == 8) {
            v4i v = *(const v4i *)(v16 + o);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int x = (int)(int16_t)((uint32_t)v[j] & 0xffff), y = (int)(int16_t)((uint32_t)v[j] >> 16);
                uint32_t b = ((uint32_t)(uint8_t)rne_shift32(x, sh_)) | ((uint32_t)(uint8_t)rne_shift32(y, sh_) << 8);
                if (j < 2) lo |= b << (16 * j);
                else hi |= b << (16 * (j - 2));
            }
            lo = act4(lo, act, o);
            hi = act4(hi, act, o + 4);
            *(v2i *)(out + o) = v2i{(int)lo, (int)hi};
        } else {
            out[o] = (int8_t)act1(rne_shift32(v16[o], sh_), act, o);
        }
    };
    if (!row_group) {
        // four independent chunks per thread and trip, all loads first; the
        // first trip's loads go out before the tile needs are reduced, so the
        // two memory round trips overlap
        constexpr int U = 4;
        const uint32_t total = (uint32_t)M * per_row;
        long long o[U];
        int t[U];
        v4i v[U];
        auto fetch = [&](uint32_t i0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + 256 * u;
                const uint32_t ii = i < total ? i : i0;
                const uint32_t row = fdiv32(ii, dper);
                const int c0 = (int)(ii - row * per_row) * vw;
                o[u] = (long long)row * N + c0;
                t[u] = p16[(row >> lbm) + TM * (c0 >> lbn)];
                if (vw == 8) v[u] = *(const v4i *)(v16 + o[u]);
            }
        };
        uint32_t i0 = bid * 256 * U + threadIdx.x;
        if (i0 < total) fetch(i0);
        // largest tile need, eight per 16-byte load (p16 is 16-byte aligned);
        // all-zero tiles (P_NONE) stay below every real need and E_MIN
        const int T = TM * n_ct, T8 = T >> 3;
        int m = NEED_NONE;
        for (int i = threadIdx.x; i < T8; i += 256) {
            const v4i w = *(const v4i *)(p16 + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                m = max(m, max((int)(int16_t)(w[j] & 0xffff), (int)(int16_t)((uint32_t)w[j] >> 16)));
        }
        for (int i = 8 * T8 + threadIdx.x; i < T; i += 256) m = max(m, (int)p16[i]);
        m = block_max256(m, sh);
        const int eT = clamp_exp_flag(max(E_MIN, m), flags);
        for (; i0 < total; i0 += nblk * 256 * U) {
            if (i0 != bid * 256 * U + threadIdx.x) fetch(i0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i0 + 256 * u >= total) break;
                const int sh_ = eT - (t[u] == P_NONE ? P_NONE : t[u] - 2);
                if (vw == 8) store8(o[u], v[u], sh_);
                else round8(o[u], sh_);
            }
        }
        if (bid == 0 && threadIdx.x == 0) out_exp[0] = (int8_t)eT;
        return;
    }
    const bool staged = rb * n_ct <= FIN_NEEDS;
    for (long long r0 = (long long)bid * rb; r0 < M; r0 += (long long)nblk * rb) {
        const int nr = (int)min((long long)rb, M - r0);
        const int16_t *pr = p16 + r0 * n_ct;
        if (staged) {
            for (int i = threadIdx.x; i < nr * n_ct; i += 256) needs[i] = pr[i];
            __syncthreads();
            if (threadIdx.x < nr) {
                int m = NEED_NONE;
                for (int j = 0; j < n_ct; ++j) {
                    const int v = needs[threadIdx.x * n_ct + j];
                    if (v != P_NONE) m = max(m, v);
                }
                const int e = clamp_exp_flag(max(E_MIN, m), flags);
                rowe[threadIdx.x] = e;
                out_exp[r0 + threadIdx.x] = (int8_t)e;
            }
        } else {
            // one row of more than FIN_NEEDS column tiles
            int m = NEED_NONE;
            for (int j = threadIdx.x; j < n_ct; j += 256) {
                const int v = pr[j];
                if (v != P_NONE) m = max(m, v);
            }
            m = block_max256(m, sh);
            if (threadIdx.x == 0) {
                const int e = clamp_exp_flag(max(E_MIN, m), flags);
                rowe[0] = e;
                out_exp[r0] = (int8_t)e;
            }
        }
        __syncthreads();
        const uint32_t cnt = (uint32_t)nr * per_row;
        for (uint32_t i = threadIdx.x; i < cnt; i += 256) {
            const uint32_t lr = fdiv32(i, dper);
            const int c0 = (int)(i - lr * per_row) * vw;
            const int t = staged ? needs[lr * n_ct + (c0 >> lbn)] : pr[c0 >> lbn];
            round8((r0 + lr) * N + c0, rowe[lr] - (t == P_NONE ? P_NONE : t - 2));
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void rto_finalize_kernel(const int16_t *v16, const int16_t *p16, int M, int N,
                                                           int lbm, int lbn, int TM, int n_ct, int row_group, int rb,
                                                           int8_t *out, int8_t *out_exp, uint32_t *flags, int vw,
                                                           FastDiv dper, Act act) {
    rto_finalize_body(v16, p16, M, N, lbm, lbn, TM, n_ct, row_group, rb, out, out_exp, flags, vw, dper, act,
                      blockIdx.x, gridDim.x);
}

// Arguments of a round-to-odd finalize and its grid.
struct RtoFin {
    const int16_t *v16, *p16;
    int M, N, lbm, lbn, TM, n_ct, row_group, rb;
    int8_t *out, *out_exp;
    uint32_t *flags;
    int vw;
    FastDiv dper;
    int blocks;
    Act act;
};

static RtoFin rto_fin(const int16_t *v16, const int16_t *p16, int M, int N, Tile t, int row_group, int8_t *out,
                      int8_t *out_exp, uint32_t *flags, Act act) {
    RtoFin f;
    f.v16 = v16;
    f.p16 = p16;
    f.M = M;
    f.N = N;
    f.vw = (N % 8 == 0 && ((uintptr_t)out % 8) == 0 && act_aligned(act, 8)) ? 8 : 1;
    f.TM = (M + t.bm() - 1) / t.bm();
    f.n_ct = (N + t.bn() - 1) / t.bn();
    // row runs of about 8192 elements (at most 256 rows)
    int rb = 8192 / N;
    f.rb = rb < 1 ? 1 : (rb > 256 ? 256 : rb);
    const long long total = (long long)M * (N / f.vw);
    f.blocks = row_group ? blocks_for((M + f.rb - 1) / f.rb, 1, 8192) : blocks_for(total, 256 * 4, 2048);
    auto lg = [](int v) { int l = 0; while ((1 << l) < v) ++l; return l; };  // tile sides are powers of two
    f.lbm = lg(t.bm());
    f.lbn = lg(t.bn());
    f.row_group = row_group;
    f.out = out;
    f.out_exp = out_exp;
    f.flags = flags;
    f.dper = make_fastdiv((uint32_t)(N / f.vw));
    f.act = act;
    return f;
}

hipError_t launch_rto_finalize(const int16_t *v16, const int16_t *p16, int M, int N, Tile t, int row_group,
                               int8_t *out, int8_t *out_exp, uint32_t *flags, hipStream_t st, Act act) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const RtoFin f = rto_fin(v16, p16, M, N, t, row_group, out, out_exp, flags, act);
    prof_begin(st, PROF_RTO_FINALIZE);
    hipLaunchKernelGGL(rto_finalize_kernel, dim3(f.blocks), dim3(256), 0, st, f.v16, f.p16, f.M, f.N, f.lbm, f.lbn,
                       f.TM, f.n_ct, f.row_group, f.rb, f.out, f.out_exp, f.flags, f.vw, f.dper, f.act);
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
                                                             FastDiv dper, int wq) {
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
                    m = max(max(need64(s0, er + exp_at(eb, c0), wq), need64(s1, er + exp_at(eb, c0 + 1), wq)),
                            max(need64(s2, er + exp_at(eb, c0 + 2), wq), need64(s3, er + exp_at(eb, c0 + 3), wq)));
                } else {
                    sums[o] = s0;
                    m = need64(s0, er + exp_at(eb, c0), wq);
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
                                                         int8_t *out_exp, uint32_t *flags, int vw, FastDiv dper,
                                                         Act act) {
    const uint32_t per_row = N / vw;
    const uint32_t total = (uint32_t)M * per_row;
    const int eT = row_group ? 0 : clamp_exp_flag(max(E_MIN, gneed[0]), flags);
    // exponents and sums are read before this chunk's store (out may alias
    // them as far as the compiler knows)
    const bool eb_uni = eb.e32 != nullptr || !eb.row;
    const int eb0 = exp_at(eb, 0);
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
        const uint32_t row = fdiv32(i, dper);
        const int c0 = (int)(i - row * per_row) * vw;
        const long long o = (long long)row * N + c0;
        const long long so = (long long)row * src_pitch;
        const int e = row_group ? clamp_exp_flag(max(E_MIN, gneed[row]), flags) : eT;
        const int er = exp_at(ea, row);
        long long sv[4];
        int ev[4];
        for (int j = 0; j < vw; ++j) {
            const uint32_t col = c0 + j;
            uint32_t sc = col;
            if (mc != mcp) {
                const uint32_t g = fdiv32(col, dmc);
                sc = g * mcp + (col - g * mc);
            }
            sv[j] = sums[so + sc];
            ev[j] = er + (eb_uni ? eb0 : exp_at(eb, col));
        }
        uint32_t w = 0;
        for (int j = 0; j < vw; ++j) w |= (uint32_t)(uint8_t)rne_shift64(sv[j], e - ev[j]) << (8 * j);
        if (vw == 4) *(uint32_t *)(out + o) = act4(w, act, o);
        else out[o] = (int8_t)act1((int)(int8_t)w, act, o);
        if (row_group && c0 == 0) out_exp[row] = (int8_t)e;
    }
    if (!row_group && blockIdx.x == 0 && threadIdx.x == 0) out_exp[0] = (int8_t)eT;
}

// Split-contraction finalize of row groups in one pass.  A block of 512
// threads owns one output row: the row's nch chunks of vw output columns
// are summed in int64 over the splits (when the row is short, Q subsets of
// the splits run side by side and meet in LDS), the row exponent is the
// largest need, and the row is rounded and stored.
// Short rows (at most 512 chunks) take 1024 threads, so more split subsets
// load at once; long rows take 512 threads with up to SR_MAXV chunks each.
constexpr int SR_FEW = 2;   // up to this many splits, a thread loads all of its chunks before summing

__device__ __forceinline__ int block_max_n(int v, int *sh) {
    v = wave_max_dpp(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    int m = sh[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = max(m, sh[i]);
    return m;
}

// a[j] += p[z * stride + j] over z = z0, z0 + dz, ... < n, eight loads in
// flight at a time (VW = 4: one 16-byte load per split; VW = 1: one int).
template <int VW>
__device__ __forceinline__ void sum_splits(const int *p, long long stride, int z0, int dz, int n, long long (&a)[4]) {
    int z = z0;
    for (; z + 7 * dz < n; z += 8 * dz) {
        if constexpr (VW == 4) {
            v4i x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = *(const v4i *)(p + (long long)(z + u * dz) * stride);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a[0] += x[u][0];
                a[1] += x[u][1];
                a[2] += x[u][2];
                a[3] += x[u][3];
            }
        } else {
            int x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = p[(long long)(z + u * dz) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) a[0] += x[u];
        }
    }
    for (; z < n; z += dz) {
        if constexpr (VW == 4) {
            const v4i x = *(const v4i *)(p + (long long)z * stride);
            a[0] += x[0];
            a[1] += x[1];
            a[2] += x[2];
            a[3] += x[3];
        } else {
            a[0] += p[(long long)z * stride];
        }
    }
}

// At least four waves per SIMD (two 512-thread blocks per CU, at most 128
// VGPRs), so that consecutive rows overlap.
template <int THR>
__device__ __forceinline__ void split_round_body(const int *partial, int splits, long long stride,
                                                                 int M, int Nout, int src_pitch, int mc, int mcp,
                                                                 FastDiv dmc, ExpSrc ea, ExpSrc eb, int8_t *out,
                                                                 int8_t *out_exp, uint32_t *flags, int vw, int Q, Act act,
                                                                 int wq, int bid, int nblk) {
    // short rows (THR == SR_THR_SHORT) hold at most one chunk per thread
    constexpr int MAXV = THR == SR_THR_SHORT ? 1 : SR_MAXV;
    __shared__ int sh[THR / 64];
    __shared__ long long acc[THR * 4];
    const int tid = threadIdx.x;
    const int nch = Nout / vw;
    auto src_col = [&](int col) -> int {
        if (mc == mcp) return col;
        const int g = (int)fdiv32((uint32_t)col, dmc);
        return g * mcp + (col - g * mc);
    };
    // A column exponent shared by every column (the usual case) is read once,
    // before any store: out may alias it as far as the compiler knows, and a
    // reload after each store would put a memory round trip behind every
    // element.
    const bool eb_uni = eb.e32 != nullptr || !eb.row;
    const int eb0 = exp_at(eb, 0);
    for (int row = bid; row < M; row += nblk) {
        const int er = exp_at(ea, row);
        const int *prow = partial + (long long)row * src_pitch;
        long long v[MAXV][4];
        auto eps = [&](int col) { return er + (eb_uni ? eb0 : exp_at(eb, col)); };
        int need = NEED_NONE;
        if (Q > 1) {
            // short row: chunk c = tid % nch, split subset q = tid / nch
            const int c = tid % nch, q = tid / nch;
            long long a4[4] = {0, 0, 0, 0};
            if (q < Q) {
                if (vw == 4) sum_splits<4>(prow + 4 * c, stride, q, Q, splits, a4);
                else sum_splits<1>(prow + src_col(c), stride, q, Q, splits, a4);
            }
            long long a0 = a4[0], a1 = a4[1], a2 = a4[2], a3 = a4[3];
            if (q < Q) {
                acc[4 * tid + 0] = a0;
                acc[4 * tid + 1] = a1;
                acc[4 * tid + 2] = a2;
                acc[4 * tid + 3] = a3;
            }
            __syncthreads();
            // the Q partial sums of each chunk, summed as a tree: subset q takes
            // subset q + h's while q + h < qn (log2 Q steps, all threads busy)
            for (int qn = Q; qn > 1;) {
                const int h = (qn + 1) >> 1;
                if (q + h < qn) {
                    const int t = tid + h * nch;
                    acc[4 * tid + 0] += acc[4 * t + 0];
                    acc[4 * tid + 1] += acc[4 * t + 1];
                    acc[4 * tid + 2] += acc[4 * t + 2];
                    acc[4 * tid + 3] += acc[4 * t + 3];
                }
                qn = h;
                __syncthreads();
            }
            if (tid < nch) {
                a0 = acc[4 * tid + 0];
                a1 = acc[4 * tid + 1];
                a2 = acc[4 * tid + 2];
                a3 = acc[4 * tid + 3];
                v[0][0] = a0;
                v[0][1] = a1;
                v[0][2] = a2;
                v[0][3] = a3;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j < vw) need = max(need, need64(v[0][j], eps(vw * tid + j), wq));
            }
        } else {
            if (vw == 4 && splits <= SR_FEW) {
                // few splits: every load of the row's chunks in flight at once
                v4i x[MAXV][SR_FEW];
#pragma unroll
                for (int k = 0; k < MAXV; ++k) {
                    const int c = tid + THR * k;
#pragma unroll
                    for (int z = 0; z < SR_FEW; ++z)
                        x[k][z] = c < nch && z < splits ? *(const v4i *)(prow + 4 * c + (long long)z * stride)
                                                        : v4i{0, 0, 0, 0};
                }
#pragma unroll
                for (int k = 0; k < MAXV; ++k) {
                    const int c = tid + THR * k;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        long long a = 0;
#pragma unroll
                        for (int z = 0; z < SR_FEW; ++z) a += x[k][z][j];
                        v[k][j] = a;
                        if (c < nch) need = max(need, need64(a, eps(4 * c + j), wq));
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < MAXV; ++k) {
                    const int c = tid + THR * k;
                    v[k][0] = v[k][1] = v[k][2] = v[k][3] = 0;
                    if (c < nch) {
                        if (vw == 4) sum_splits<4>(prow + 4 * c, stride, 0, 1, splits, v[k]);
                        else sum_splits<1>(prow + src_col(c), stride, 0, 1, splits, v[k]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (j < vw) need = max(need, need64(v[k][j], eps(vw * c + j), wq));
                    }
                }
            }
        }
        need = block_max_n(need, sh);
        const int e = clamp_exp_flag(max(E_MIN, need), flags);
        if (tid == 0) out_exp[row] = (int8_t)e;
        int8_t *orow = out + (long long)row * Nout;
        const int kmax = Q > 1 ? 1 : MAXV;
#pragma unroll
        for (int k = 0; k < MAXV; ++k) {
            const int c = tid + THR * k;
            if (k >= kmax || c >= nch) break;
            if (vw == 4) {
                uint32_t w = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w |= (uint32_t)(uint8_t)rne_shift64(v[k][j], e - eps(4 * c + j)) << (8 * j);
                *(uint32_t *)(orow + 4 * c) = act4(w, act, (long long)row * Nout + 4 * c);
            } else {
                const int cv = (int)rne_shift64(v[k][0], e - eps(c));
                orow[c] = (int8_t)act1(cv, act, (long long)row * Nout + c);
            }
        }
        __syncthreads();
    }
}

template <int THR>
__global__ __launch_bounds__(THR) __attribute__((amdgpu_waves_per_eu(4))) void split_round_rows_kernel(const int *partial, int splits, long long stride,
                                                                 int M, int Nout, int src_pitch, int mc, int mcp,
                                                                 FastDiv dmc, ExpSrc ea, ExpSrc eb, int8_t *out,
                                                                 int8_t *out_exp, uint32_t *flags, int vw, int Q,
                                                                 Act act, int wq) {
    split_round_body<THR>(partial, splits, stride, M, Nout, src_pitch, mc, mcp, dmc, ea, eb, out, out_exp, flags, vw, Q,
                          act, wq, blockIdx.x, gridDim.x);
}


// Arguments of a split finalize by rows and its grid.
struct SplitFin {
    const int *partial;
    int splits;
    long long stride;
    int M, Nout, src_pitch, mc, mcp;
    FastDiv dmc;
    ExpSrc ea, eb;
    int8_t *out, *out_exp;
    uint32_t *flags;
    int vw, Q, blocks;
    bool shortrow;
    Act act;
    int wq;  // results have |C| <= 2^wq - 1
};

static SplitFin split_fin(const int *partial, int splits, long long split_stride, int M, int Nout, int src_pitch,
                          int mc, int mcp, ExpSrc ea, ExpSrc eb, int8_t *out, int8_t *out_exp, uint32_t *flags,
                          int wq, Act act) {
    SplitFin f;
    f.partial = partial;
    f.splits = splits;
    f.stride = split_stride;
    f.M = M;
    f.Nout = Nout;
    f.src_pitch = src_pitch;
    f.mc = mc;
    f.mcp = mcp;
    f.ea = ea;
    f.eb = eb;
    f.out = out;
    f.out_exp = out_exp;
    f.flags = flags;
    f.vw = (mc == mcp && Nout % 4 == 0 && src_pitch % 4 == 0 && ((uintptr_t)out % 4) == 0 && act_aligned(act, 4)) ? 4
                                                                                                            : 1;
    const int nch = Nout / f.vw;
    f.shortrow = nch <= SR_THR;
    const int thr = f.shortrow ? SR_THR_SHORT : SR_THR;
    f.Q = 1;
    if (f.shortrow && nch <= thr / 2) {
        f.Q = thr / nch;
        if (f.Q > splits) f.Q = splits;
    }
    f.blocks = blocks_for(M, 1, 16384);
    f.dmc = make_fastdiv((uint32_t)(mc > 0 ? mc : 1));
    f.act = act;
    f.wq = wq;
    return f;
}

hipError_t launch_split_round_rows(const int *partial, int splits, long long split_stride, int M, int Nout,
                                   int src_pitch, int mc, int mcp, ExpSrc ea, ExpSrc eb, int8_t *out,
                                   int8_t *out_exp, uint32_t *flags, int q, hipStream_t st, Act act) {
    if (M <= 0 || Nout <= 0) return hipSuccess;
    const SplitFin f = split_fin(partial, splits, split_stride, M, Nout, src_pitch, mc, mcp, ea, eb, out, out_exp,
                                 flags, q, act);
    prof_begin(st, PROF_SPLIT_ROUND);
    if (f.shortrow)
        hipLaunchKernelGGL(split_round_rows_kernel<SR_THR_SHORT>, dim3(f.blocks), dim3(SR_THR_SHORT), 0, st,
                           f.partial, f.splits, f.stride, f.M, f.Nout, f.src_pitch, f.mc, f.mcp, f.dmc, f.ea, f.eb,
                           f.out, f.out_exp, f.flags, f.vw, f.Q, f.act, f.wq);
    else
        hipLaunchKernelGGL(split_round_rows_kernel<SR_THR>, dim3(f.blocks), dim3(SR_THR), 0, st, f.partial,
                           f.splits, f.stride, f.M, f.Nout, f.src_pitch, f.mc, f.mcp, f.dmc, f.ea, f.eb, f.out,
                           f.out_exp, f.flags, f.vw, f.Q, f.act, f.wq);
    prof_end(st, PROF_SPLIT_ROUND);
    return hipGetLastError();
}

// The two finalizes of a convolution's backward pass (input gradient by
// round-to-odd, weight gradient by split rows) in one grid: the first
// r.blocks blocks run the former on 256 of their threads, the rest the
// latter.
template <int THR>
__global__ __launch_bounds__(THR) __attribute__((amdgpu_waves_per_eu(4))) void finalize_pair_kernel(RtoFin r,
                                                                                                  SplitFin q) {
    if ((int)blockIdx.x < r.blocks) {
        if (threadIdx.x >= 256) return;
        rto_finalize_body(r.v16, r.p16, r.M, r.N, r.lbm, r.lbn, r.TM, r.n_ct, r.row_group, r.rb, r.out, r.out_exp,
                          r.flags, r.vw, r.dper, r.act, blockIdx.x, r.blocks);
    } else {
        split_round_body<THR>(q.partial, q.splits, q.stride, q.M, q.Nout, q.src_pitch, q.mc, q.mcp, q.dmc, q.ea,
                              q.eb, q.out, q.out_exp, q.flags, q.vw, q.Q, q.act, q.wq, blockIdx.x - r.blocks,
                              gridDim.x - r.blocks);
    }
}

hipError_t launch_finalize_pair(const int16_t *v16, const int16_t *p16, int M1, int N1, Tile t1, int8_t *out1,
                                int8_t *out1_exp, const int *partial, int splits, long long split_stride, int M2,
                                int Nout, int src_pitch, int mc, int mcp, ExpSrc ea, ExpSrc eb, int8_t *out2,
                                int8_t *out2_exp, uint32_t *flags, int q2, hipStream_t st, Act act1) {
    if (M1 <= 0 || N1 <= 0 || M2 <= 0 || Nout <= 0) {
        hipError_t e = launch_rto_finalize(v16, p16, M1, N1, t1, 0, out1, out1_exp, flags, st, act1);
        if (e != hipSuccess) return e;
        return launch_split_round_rows(partial, splits, split_stride, M2, Nout, src_pitch, mc, mcp, ea, eb, out2,
                                       out2_exp, flags, q2, st);
    }
    const RtoFin r = rto_fin(v16, p16, M1, N1, t1, 0, out1, out1_exp, flags, act1);
    const SplitFin q = split_fin(partial, splits, split_stride, M2, Nout, src_pitch, mc, mcp, ea, eb, out2, out2_exp,
                                 flags, q2, Act{});
    const dim3 grid(r.blocks + q.blocks);
    prof_begin(st, PROF_FIN_PAIR);
    if (q.shortrow)
        hipLaunchKernelGGL(finalize_pair_kernel<SR_THR_SHORT>, grid, dim3(SR_THR_SHORT), 0, st, r, q);
    else
        hipLaunchKernelGGL(finalize_pair_kernel<SR_THR>, grid, dim3(SR_THR), 0, st, r, q);
    prof_end(st, PROF_FIN_PAIR);
    return hipGetLastError();
}

hipError_t launch_partial_reduce(const int *partial, int splits, long long split_stride, int M, int N,
                                 ExpSrc ea, ExpSrc eb, int row_group, long long *sums, int *gneed, int q,
                                 hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int vw = (N % 4 == 0) ? 4 : 1;
    const long long total = (long long)M * (N / vw);
    prof_begin(st, PROF_PARTIAL_REDUCE);
    hipLaunchKernelGGL(partial_reduce_kernel, dim3(blocks_for(total, 64, 8192)), dim3(256), 0, st, partial,
                       splits, split_stride, M, N, ea, eb, row_group, sums, gneed, vw,
                       make_fastdiv((uint32_t)(N / vw)), q);
    prof_end(st, PROF_PARTIAL_REDUCE);
    return hipGetLastError();
}

hipError_t launch_round_sums(const long long *sums, int M, int N, int src_pitch, int mc, int mcp, ExpSrc ea,
                             ExpSrc eb, int row_group, const int *gneed, int8_t *out, int8_t *out_exp,
                             uint32_t *flags, hipStream_t st, Act act) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int vw = (N % 4 == 0 && ((uintptr_t)out % 4) == 0 && act_aligned(act, 4)) ? 4 : 1;
    const long long total = (long long)M * (N / vw);
    prof_begin(st, PROF_ROUND_SUMS);
    hipLaunchKernelGGL(round_sums_kernel, dim3(blocks_for(total, 256, 8192)), dim3(256), 0, st, sums, M, N,
                       src_pitch, mc, mcp, make_fastdiv((uint32_t)(mc > 0 ? mc : 1)), ea, eb, row_group, gneed,
                       out, out_exp, flags, vw, make_fastdiv((uint32_t)(N / vw)), act);
    prof_end(st, PROF_ROUND_SUMS);
    return hipGetLastError();
}

}  // namespace ie
