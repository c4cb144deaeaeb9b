// C ABI of the (C, e) layer-step library: argument checks, workspace layout
// and the launch sequence of every entry point.  See include/ie.h.
#include <string.h>

#include "../../include/ie.h"
#include "ie_device.h"
#include "ie_internal.h"

using namespace ie;

namespace {

constexpr size_t HEADER = 256;
constexpr long long MAX_CONTRACT = 65536;   // |acc| < 2^30 for the fused epilogue
constexpr long long SPLIT_MAX_ROWS = 65536; // exact int32 partial sums: |sum| <= 2^30
constexpr long long DIM_MAX = (1ll << 31) - 1;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump allocator over the caller's workspace.
struct Carve {
    char *base;
    size_t off;
    template <class T>
    T *take(size_t count) {
        off = align256(off);
        T *p = (T *)(base ? base + off : nullptr);
        off += count * sizeof(T);
        return p;
    }
};

int n_exps(const ie_mat *t) { return t->group == IE_GROUP_ROW ? (int)t->rows : 1; }

ie_status check_mat(const ie_mat *t) {
    if (!t) return IE_ERR_NULL;
    if (t->group != IE_GROUP_TENSOR && t->group != IE_GROUP_ROW) return IE_ERR_GROUP;
    if (t->rows < 0 || t->cols < 0 || t->rows > DIM_MAX || t->cols > DIM_MAX) return IE_ERR_SHAPE;
    if (t->rows * t->cols > 0 && !t->mant) return IE_ERR_NULL;
    if ((t->group == IE_GROUP_TENSOR || t->rows > 0) && !t->exp) return IE_ERR_NULL;
    return IE_OK;
}

ie_status hip_status(hipError_t e) { return e == hipSuccess ? IE_OK : IE_ERR_HIP; }

#define IE_TRY(x)                                   \
    do {                                            \
        hipError_t _e = (x);                        \
        if (_e != hipSuccess) return IE_ERR_HIP;    \
    } while (0)

#define IE_CHECK(x)                                 \
    do {                                            \
        ie_status _s = (x);                         \
        if (_s != IE_OK) return _s;                 \
    } while (0)

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Workspace of a product whose int8 output [M x N] may need the two-pass
// (round-to-odd) epilogue.
struct ProductWs {
    int *gneed;
    int16_t *p16;
    int16_t *v16;
};

ProductWs carve_product(Carve &c, long long M, long long N) {
    ProductWs w;
    long long n_ct = N > 0 ? cdiv(N, BN) : 1;
    w.gneed = c.take<int>(M > 0 ? M : 1);
    w.p16 = c.take<int16_t>(M * n_ct);
    w.v16 = c.take<int16_t>(M * N);
    return w;
}

// Run A(m,k) . B(n,k) over K into an int8 output, choosing the one-pass
// epilogue when every output group lies inside one tile.
ie_status run_product(const Operand &A, const Operand &B, long long M, long long N, long long K,
                      ExpSrc ea, ExpSrc eb, const ie_mat *out, const ProductWs &pw, uint32_t *flags,
                      hipStream_t st) {
    if (M == 0 || N == 0) {
        return hip_status(launch_fill_i8(out->exp, out->group == IE_GROUP_ROW ? M : 1, E_MIN, st));
    }
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.ea = ea;
    ep.eb = eb;
    ep.row_group = out->group == IE_GROUP_ROW;
    ep.out = out->mant;
    ep.out_exp = out->exp;
    ep.flags = flags;
    ep.n_ct = cdiv(N, BN);
    bool direct = ep.row_group ? (N <= BN) : (M <= BM && N <= BN);
    if (direct) {
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, 1, (int)(K > 0 ? cdiv(K, BK) * BK : BK),
                           EPI_DIRECT, ep, st));
        return IE_OK;
    }
    ep.v16 = pw.v16;
    ep.p16 = pw.p16;
    ep.gneed = pw.gneed;
    IE_TRY(launch_fill_i32(pw.gneed, ep.row_group ? M : 1, NEED_NONE, st));
    IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, 1, (int)(K > 0 ? cdiv(K, BK) * BK : BK), EPI_RTO, ep,
                       st));
    IE_TRY(launch_rto_finalize(pw.v16, pw.p16, pw.gneed, (int)M, (int)N, ep.n_ct, ep.row_group, out->mant,
                               out->exp, flags, st));
    return IE_OK;
}

// Split of a long contraction (weight gradients) into exact int32 chunks.
struct Split {
    int splits;
    int chunk;
};

Split choose_split(long long M, long long N, long long L) {
    long long tiles = (long long)cdiv(M, BM) * cdiv(N, BN);
    long long want = tiles > 0 ? (1024 + tiles - 1) / tiles : 1;
    long long s = want < 1 ? 1 : want;
    long long chunk = L > 0 ? (L + s - 1) / s : BK;
    if (chunk < 512) chunk = 512;
    chunk = (chunk + BK - 1) / BK * BK;
    if (chunk > SPLIT_MAX_ROWS) chunk = SPLIT_MAX_ROWS;
    long long splits = L > 0 ? (L + chunk - 1) / chunk : 1;
    return {(int)splits, (int)chunk};
}

struct WgradWs {
    int *partial;
    int *gneed;
    int *eps;  // [2]
};

WgradWs carve_wgrad(Carve &c, long long N, long long K, long long L) {
    WgradWs w;
    Split sp = choose_split(N, K, L);
    w.eps = c.take<int>(2);
    w.gneed = c.take<int>(1);
    w.partial = c.take<int>((size_t)sp.splits * N * K);
    return w;
}

ie_status run_wgrad(const Operand &A, const Operand &B, long long N, long long K, long long L,
                    const ie_mat *dW, const WgradWs &w, uint32_t *flags, hipStream_t st) {
    if (N == 0 || K == 0) {
        return hip_status(launch_fill_i8(dW->exp, dW->group == IE_GROUP_ROW ? N : 1, E_MIN, st));
    }
    Split sp = choose_split(N, K, L);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.partial = w.partial;
    ep.split_stride = N * K;
    ep.flags = flags;
    if (L == 0) {
        IE_TRY(launch_fill_i32(w.partial, N * K, 0, st));
    } else {
        IE_TRY(launch_gemm(A, B, (int)N, (int)K, (int)L, sp.splits, sp.chunk, EPI_PARTIAL, ep, st));
    }
    IE_TRY(launch_dw_finalize(w.partial, L == 0 ? 1 : sp.splits, N * K, (int)N, (int)K, w.eps, w.eps + 1,
                              dW->group == IE_GROUP_ROW, w.gneed, dW->mant, dW->exp, flags, st));
    return IE_OK;
}

ConvGeom geom(const ie_conv_desc *d) {
    ConvGeom g;
    g.n = d->n;
    g.h = d->h;
    g.w = d->w;
    g.c = d->c;
    g.k = d->k;
    g.r = d->r;
    g.s = d->s;
    g.stride = d->stride;
    g.pad = d->pad;
    g.p = (d->h + 2 * d->pad - d->r) / d->stride + 1;
    g.q = (d->w + 2 * d->pad - d->s) / d->stride + 1;
    return g;
}

ie_status check_conv(const ie_conv_desc *d) {
    if (!d) return IE_ERR_NULL;
    if (d->n < 0 || d->h <= 0 || d->w <= 0 || d->c <= 0 || d->k <= 0 || d->r <= 0 || d->s <= 0 ||
        d->stride <= 0 || d->pad < 0)
        return IE_ERR_SHAPE;
    if (d->h + 2 * d->pad < d->r || d->w + 2 * d->pad < d->s) return IE_ERR_SHAPE;
    long long rsc = (long long)d->r * d->s * d->c;
    if (rsc > DIM_MAX || (long long)d->n * d->h * d->w * d->c > DIM_MAX * 8ll) return IE_ERR_SHAPE;
    return IE_OK;
}

size_t linear_fwd_ws(long long M, long long N, long long K) {
    (void)K;
    Carve c{nullptr, HEADER};
    carve_product(c, M, N);
    return align256(c.off);
}

size_t linear_dx_ws(long long M, long long N, long long K) {
    Carve c{nullptr, HEADER};
    c.take<int>(1);
    c.take<int8_t>((size_t)N * K);
    carve_product(c, M, K);
    return align256(c.off);
}

size_t linear_dw_ws(long long M, long long N, long long K) {
    Carve c{nullptr, HEADER};
    c.take<int8_t>((size_t)M * N);
    c.take<int8_t>((size_t)M * K);
    carve_wgrad(c, N, K, M);
    return align256(c.off);
}

size_t conv_fwd_ws(const ie_conv_desc *d) {
    ConvGeom g = geom(d);
    Carve c{nullptr, HEADER};
    carve_product(c, (long long)g.n * g.p * g.q, g.k);
    return align256(c.off);
}

size_t conv_bwd_ws(const ie_conv_desc *d) {
    ConvGeom g = geom(d);
    long long rsc = (long long)g.r * g.s * g.c;
    Carve c{nullptr, HEADER};
    c.take<int>(1);
    c.take<int8_t>((size_t)rsc * g.k);
    carve_product(c, (long long)g.n * g.h * g.w, g.c);
    carve_wgrad(c, g.k, rsc, (long long)g.n * g.p * g.q);
    return align256(c.off);
}

}  // namespace

extern "C" {

size_t ie_linear_fwd_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return linear_fwd_ws(M, N, K);
}
size_t ie_linear_bwd_dx_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return linear_dx_ws(M, N, K);
}
size_t ie_linear_bwd_dw_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return linear_dw_ws(M, N, K);
}
size_t ie_conv_fwd_workspace(const ie_conv_desc *d) {
    if (check_conv(d) != IE_OK) return 0;
    return conv_fwd_ws(d);
}
size_t ie_conv_bwd_workspace(const ie_conv_desc *d) {
    if (check_conv(d) != IE_OK) return 0;
    return conv_bwd_ws(d);
}
size_t ie_sgd_update_workspace(int64_t rows, int64_t cols) {
    (void)rows;
    (void)cols;
    return HEADER + 256;
}

ie_status ie_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return IE_ERR_NULL;
    if (ws_bytes < HEADER) return IE_ERR_WORKSPACE;
    return hip_status(launch_zero_flags(ws, (hipStream_t)stream));
}

ie_status ie_linear_fwd(const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws, size_t ws_bytes,
                        void *stream) {
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    long long M = X->rows, K = X->cols, N = W->rows;
    if (W->cols != K || Y->rows != M || Y->cols != N) return IE_ERR_SHAPE;
    if (K > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_fwd_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    ProductWs pw = carve_product(c, M, N);
    Operand A{LD_K, X->mant, K, (int)M, (K % 16 == 0) && aligned(X->mant, 16), {}};
    Operand B{LD_K, W->mant, K, (int)N, (K % 16 == 0) && aligned(W->mant, 16), {}};
    ExpSrc ea{X->exp, nullptr, X->group == IE_GROUP_ROW};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, M, N, K, ea, eb, Y, pw, flags, st);
}

ie_status ie_linear_bwd_dx(const ie_mat *dY, const ie_mat *W, const ie_mat *dX, void *ws, size_t ws_bytes,
                           void *stream) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(dX));
    long long M = dY->rows, N = dY->cols, K = W->cols;
    if (W->rows != N || dX->rows != M || dX->cols != K) return IE_ERR_SHAPE;
    if (N > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_dx_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    int *estar = c.take<int>(1);
    int8_t *wt = c.take<int8_t>((size_t)N * K);
    ProductWs pw = carve_product(c, M, K);
    if (M == 0 || K == 0) return run_product(Operand{}, Operand{}, M, K, N, ExpSrc{}, ExpSrc{}, dX, pw, flags, st);
    IE_TRY(launch_exp_max(W->exp, n_exps(W), estar, st));
    IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, estar, (int)N, 1, (int)K, wt, st));
    Operand A{LD_K, dY->mant, N, (int)M, (N % 16 == 0) && aligned(dY->mant, 16), {}};
    Operand B{LD_K, wt, N, (int)K, (N % 16 == 0), {}};
    ExpSrc ea{dY->exp, nullptr, dY->group == IE_GROUP_ROW};
    ExpSrc eb{nullptr, estar, 0};
    return run_product(A, B, M, K, N, ea, eb, dX, pw, flags, st);
}

ie_status ie_linear_bwd_dw(const ie_mat *dY, const ie_mat *X, const ie_mat *dW, void *ws, size_t ws_bytes,
                           void *stream) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(dW));
    long long M = dY->rows, N = dY->cols, K = X->cols;
    if (X->rows != M || dW->rows != N || dW->cols != K) return IE_ERR_SHAPE;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_dw_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    int8_t *dya = c.take<int8_t>((size_t)M * N);
    int8_t *xa = c.take<int8_t>((size_t)M * K);
    WgradWs w = carve_wgrad(c, N, K, M);
    if (N == 0 || K == 0) return run_wgrad(Operand{}, Operand{}, N, K, M, dW, w, flags, st);
    // common exponents over the contraction axis (rows); align ROW operands
    IE_TRY(launch_exp_max(dY->exp, n_exps(dY), w.eps, st));
    IE_TRY(launch_exp_max(X->exp, n_exps(X), w.eps + 1, st));
    const int8_t *dys = dY->mant, *xs = X->mant;
    if (dY->group == IE_GROUP_ROW && M > 0) {
        IE_TRY(launch_align_rows(dY->mant, dY->exp, w.eps, M, N, dya, st));
        dys = dya;
    }
    if (X->group == IE_GROUP_ROW && M > 0) {
        IE_TRY(launch_align_rows(X->mant, X->exp, w.eps + 1, M, K, xa, st));
        xs = xa;
    }
    Operand A{LD_T, dys, N, (int)N, (N % 8 == 0) && aligned(dys, 8), {}};
    Operand B{LD_T, xs, K, (int)K, (K % 8 == 0) && aligned(xs, 8), {}};
    return run_wgrad(A, B, N, K, M, dW, w, flags, st);
}

ie_status ie_conv_fwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws,
                      size_t ws_bytes, void *stream) {
    IE_CHECK(check_conv(d));
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    ConvGeom g = geom(d);
    long long rsc = (long long)g.r * g.s * g.c;
    long long npq = (long long)g.n * g.p * g.q;
    if (X->rows != (long long)g.n * g.h * g.w || X->cols != g.c) return IE_ERR_SHAPE;
    if (W->rows != g.k || W->cols != rsc) return IE_ERR_SHAPE;
    if (Y->rows != npq || Y->cols != g.k) return IE_ERR_SHAPE;
    if (X->group != IE_GROUP_TENSOR) return IE_ERR_UNSUPPORTED;
    if (rsc > MAX_CONTRACT || npq > DIM_MAX) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < conv_fwd_ws(d)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    ProductWs pw = carve_product(c, npq, g.k);
    Operand A{LD_IM2COL, X->mant, g.c, (int)npq, (g.c % 16 == 0) && aligned(X->mant, 16), g};
    Operand B{LD_K, W->mant, rsc, g.k, (rsc % 16 == 0) && aligned(W->mant, 16), {}};
    ExpSrc ea{X->exp, nullptr, 0};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, npq, g.k, rsc, ea, eb, Y, pw, flags, st);
}

ie_status ie_conv_bwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *dY,
                      const ie_mat *dX, const ie_mat *dW, void *ws, size_t ws_bytes, void *stream) {
    IE_CHECK(check_conv(d));
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(dY));
    if (dX) IE_CHECK(check_mat(dX));
    if (dW) IE_CHECK(check_mat(dW));
    ConvGeom g = geom(d);
    long long rsc = (long long)g.r * g.s * g.c;
    long long npq = (long long)g.n * g.p * g.q;
    long long nhw = (long long)g.n * g.h * g.w;
    if (X->rows != nhw || X->cols != g.c) return IE_ERR_SHAPE;
    if (W->rows != g.k || W->cols != rsc) return IE_ERR_SHAPE;
    if (dY->rows != npq || dY->cols != g.k) return IE_ERR_SHAPE;
    if (dX && (dX->rows != nhw || dX->cols != g.c)) return IE_ERR_SHAPE;
    if (dW && (dW->rows != g.k || dW->cols != rsc)) return IE_ERR_SHAPE;
    if (X->group != IE_GROUP_TENSOR || dY->group != IE_GROUP_TENSOR) return IE_ERR_UNSUPPORTED;
    if ((long long)g.k * g.r * g.s > MAX_CONTRACT || nhw > DIM_MAX) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < conv_bwd_ws(d)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    int *estar = c.take<int>(1);
    int8_t *wt = c.take<int8_t>((size_t)rsc * g.k);
    ProductWs pw = carve_product(c, nhw, g.c);
    WgradWs w = carve_wgrad(c, g.k, rsc, npq);
    if (dX) {
        long long rsk = (long long)g.r * g.s * g.k;
        IE_TRY(launch_exp_max(W->exp, n_exps(W), estar, st));
        IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, estar, g.k, g.r * g.s, g.c,
                                      wt, st));
        Operand A{LD_DGRAD, dY->mant, g.k, (int)nhw, (g.k % 16 == 0) && aligned(dY->mant, 16), g};
        Operand B{LD_K, wt, rsk, g.c, (rsk % 16 == 0), {}};
        ExpSrc ea{dY->exp, nullptr, 0};
        ExpSrc eb{nullptr, estar, 0};
        IE_CHECK(run_product(A, B, nhw, g.c, rsk, ea, eb, dX, pw, flags, st));
    }
    if (dW) {
        IE_TRY(launch_exp_max(dY->exp, 1, w.eps, st));
        IE_TRY(launch_exp_max(X->exp, 1, w.eps + 1, st));
        Operand A{LD_T, dY->mant, g.k, g.k, (g.k % 8 == 0) && aligned(dY->mant, 8), {}};
        Operand B{LD_IM2COL_T, X->mant, g.c, (int)rsc, (g.c % 8 == 0) && aligned(X->mant, 8), g};
        IE_CHECK(run_wgrad(A, B, g.k, rsc, npq, dW, w, flags, st));
    }
    return IE_OK;
}

ie_status ie_sgd_update(const ie_mat *W, const ie_mat *V, const ie_mat *G, ie_scalar lr, ie_scalar momentum,
                        ie_scalar weight_decay, void *ws, size_t ws_bytes, void *stream) {
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(V));
    IE_CHECK(check_mat(G));
    if (V->rows != W->rows || V->cols != W->cols || G->rows != W->rows || G->cols != W->cols)
        return IE_ERR_SHAPE;
    if (weight_decay.mant != 0) return IE_ERR_UNSUPPORTED;
    if (W->cols > 64 * 4 * 32) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < ie_sgd_update_workspace(W->rows, W->cols)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws, HEADER};
    int *gn = c.take<int>(4);
    UpdateArgs a;
    a.w = W->mant;
    a.w_exp = W->exp;
    a.v = V->mant;
    a.v_exp = V->exp;
    a.g = G->mant;
    a.g_exp = G->exp;
    a.w_row = W->group == IE_GROUP_ROW;
    a.v_row = V->group == IE_GROUP_ROW;
    a.g_row = G->group == IE_GROUP_ROW;
    a.rows = W->rows;
    a.cols = W->cols;
    a.lr_m = lr.mant;
    a.lr_e = lr.exp;
    a.mom_m = momentum.mant;
    a.mom_e = momentum.exp;
    a.gneed_v = gn;
    a.gneed_w = gn + 1;
    a.flags = (uint32_t *)ws;
    return hip_status(launch_sgd_update(a, st));
}

ie_status ie_device_status(void *ws, void *stream, uint32_t *flags, int clear) {
    if (!ws || !flags) return IE_ERR_NULL;
    hipStream_t st = (hipStream_t)stream;
    IE_TRY(hipStreamSynchronize(st));
    IE_TRY(hipMemcpy(flags, ws, sizeof(uint32_t), hipMemcpyDeviceToHost));
    if (clear) {
        IE_TRY(launch_zero_flags(ws, st));
        IE_TRY(hipStreamSynchronize(st));
    }
    return IE_OK;
}

ie_status ie_profile_enable(int on) {
    prof_enable(on);
    return IE_OK;
}

int ie_profile_read(float *ms, int *kind, int max) { return prof_read(ms, kind, max); }

const char *ie_status_str(ie_status s) {
    switch (s) {
        case IE_OK: return "IE_OK";
        case IE_ERR_NULL: return "IE_ERR_NULL";
        case IE_ERR_SHAPE: return "IE_ERR_SHAPE";
        case IE_ERR_GROUP: return "IE_ERR_GROUP";
        case IE_ERR_WORKSPACE: return "IE_ERR_WORKSPACE";
        case IE_ERR_EXP_RANGE: return "IE_ERR_EXP_RANGE";
        case IE_ERR_UNSUPPORTED: return "IE_ERR_UNSUPPORTED";
        case IE_ERR_HIP: return "IE_ERR_HIP";
    }
    return "IE_ERR_UNKNOWN";
}

}  // extern "C"
