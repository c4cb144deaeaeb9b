// C ABI of the (C, e) layer-step library: argument checks, workspace layout
// and the launch sequence of every entry point.  See include/ie.h.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

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
    if (t->bits != 0 && (t->bits < 2 || t->bits > 8)) return IE_ERR_BITS;
    return IE_OK;
}

// Mantissa width as q: a result of t has |C| <= 2^q - 1 (bits 0 reads as 8).
int mat_q(const ie_mat *t) { return (t->bits ? t->bits : 8) - 1; }

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

// ---------------------------------------------------------------------------
// Planning: tile shape, epilogue and contraction split of a product.
// ---------------------------------------------------------------------------


// Planning rules, calibrated by timing every plan of the ResNet-18 and ViT-B
// products on an MI355X:
//  * a workgroup runs MI*NI waves' worth of 32x32 MFMA tiles and keeps its
//    loads in flight for a few steps, so small grids are latency bound: the
//    128x128 tile pays off only with at least four workgroups per CU (and a
//    full tile width), 128x64 with two, otherwise 64x64;
//  * a split contraction costs an extra pass over splits x M x N int32
//    partials, so products split only when even 64x64 tiles leave most CUs
//    idle;
//  * weight gradients (short outputs, long contractions) split into chunks
//    of at least eight steps, doubling while fewer than 2.25 workgroups per
//    CU result.
constexpr long long WG_TARGET = 576;

enum PlanMode { PLAN_DIRECT = 0, PLAN_RTO = 1, PLAN_SPLIT = 2 };

struct Plan {
    Tile t;
    int mode;
    int splits;
    int k_chunk;
};

int chunk_for(long long K, int splits) {
    long long c = (K + splits - 1) / splits;
    c = (c + BK - 1) / BK * BK;
    return (int)(c > 0 ? c : BK);
}

// Tuning override: IE_TILE="mi,ni[,mode[,splits]]" forces the plan of every
// product (mode 0 direct, 1 round-to-odd, 2 split).  Unset in normal use.
bool forced_plan(long long K, Plan &pl) {
    const char *v = getenv("IE_TILE");
    if (!v || !*v) return false;
    int mi = 0, ni = 0, mode = -1, sp = 1;
    if (sscanf(v, "%d,%d,%d,%d", &mi, &ni, &mode, &sp) < 2) return false;
    pl.t = Tile{mi, ni};
    pl.mode = mode < 0 ? PLAN_RTO : mode;
    pl.splits = sp < 1 ? 1 : sp;
    pl.k_chunk = chunk_for(K, pl.splits);
    pl.splits = (int)((K + pl.k_chunk - 1) / pl.k_chunk);
    if (pl.splits < 1) pl.splits = 1;
    return true;
}

// Diagnostics: IE_PLAN_LOG set prints every planned product to stderr.
void log_plan(const char *what, long long M, long long N, long long K, const Plan &pl) {
    static const bool on = getenv("IE_PLAN_LOG") != nullptr;
    if (!on) return;
    fprintf(stderr, "[ie plan] %s M=%lld N=%lld K=%lld tile=%dx%d mode=%d splits=%d k_chunk=%d\n", what, M, N, K,
            pl.t.bm(), pl.t.bn(), pl.mode, pl.splits, pl.k_chunk);
}

// family: 0 = dense K-major, 1 = convolution (im2col / dgrad)
Plan plan_product(long long M, long long N, long long K, int row_group, int family) {
    {
        Plan f;
        if (forced_plan(K, f)) return f;
    }
    (void)family;
    auto tiles = [&](Tile t) { return (long long)cdiv(M, t.bm()) * cdiv(N, t.bn()); };
    Tile t{1, 1};
    if (N > 64 && tiles(Tile{2, 2}) >= 4ll * NCU) t = Tile{2, 2};
    else if (tiles(Tile{2, 1}) >= 2ll * NCU) t = Tile{2, 1};
    const bool direct = row_group ? N <= t.bn() : tiles(t) == 1;
    Plan best{t, direct ? PLAN_DIRECT : PLAN_RTO, 1, chunk_for(K, 1)};
    if (!direct && tiles(Tile{1, 1}) < NCU / 2 && K >= 8 * BK) {
        const long long n11 = tiles(Tile{1, 1});
        int sp = 1;
        while (sp < 16 && n11 * sp * 2 <= WG_TARGET && K / (sp * 2) >= 4 * BK) sp *= 2;
        if (sp > 1) {
            const int kc = chunk_for(K, sp);
            best = Plan{Tile{1, 1}, PLAN_SPLIT, (int)((K + kc - 1) / kc), kc};
        }
    }
    return best;
}

// Weight gradients: always split over the contraction in chunks of at most
// 65536 rows (exact int32 partial sums).
Plan plan_wgrad(long long M, long long N, long long L) {
    if (const char *v = getenv("IE_WTILE")) {
        // tuning override: IE_WTILE="mi,ni,splits"
        int mi = 0, ni = 0, sp = 1;
        if (sscanf(v, "%d,%d,%d", &mi, &ni, &sp) == 3 && sp >= 1) {
            int kc = chunk_for(L, sp);
            if (kc <= SPLIT_MAX_ROWS) return Plan{Tile{mi, ni}, PLAN_SPLIT, (int)((L + kc - 1) / kc), kc};
        }
    }
    const long long t22 = (long long)cdiv(M, 128) * cdiv(N, 128);
    const Tile t = t22 >= 32 ? Tile{2, 2} : Tile{1, 1};
    const long long nt = (long long)cdiv(M, t.bm()) * cdiv(N, t.bn());
    const int smin = (int)((L + SPLIT_MAX_ROWS - 1) / SPLIT_MAX_ROWS);
    int sp = 1;
    while (sp < 1024 && nt * sp * 2 < WG_TARGET && L / (sp * 2) >= 8 * BK) sp *= 2;
    if (sp < smin) sp = smin;
    const int kc = chunk_for(L, sp);
    return Plan{t, PLAN_SPLIT, (int)((L + kc - 1) / kc), kc};
}

// Workspace of a product's epilogue.
struct ProductWs {
    int *gneed;
    int16_t *p16;
    int16_t *v16;
    int *partial;
    long long *sums;
};

ProductWs carve_product(Carve &c, long long M, long long N, long long K, int family) {
    ProductWs w{};
    size_t p16 = 0, v16 = 0, part = 0, sums = 0;
    for (int rg = 0; rg < 2; ++rg) {
        Plan pl = plan_product(M, N, K, rg, family);
        if (pl.mode == PLAN_RTO) {
            size_t n_p = rg ? (size_t)M * cdiv(N, pl.t.bn()) : (size_t)cdiv(M, pl.t.bm()) * cdiv(N, pl.t.bn());
            p16 = p16 > n_p ? p16 : n_p;
            v16 = (size_t)M * N;
        } else if (pl.mode == PLAN_SPLIT) {
            size_t n_part = (size_t)pl.splits * M * N;
            part = part > n_part ? part : n_part;
            sums = (size_t)M * N;
        }
    }
    w.gneed = c.take<int>(M > 0 ? M : 1);
    w.p16 = c.take<int16_t>(p16);
    w.v16 = c.take<int16_t>(v16);
    w.partial = c.take<int>(part);
    w.sums = c.take<long long>(sums);
    return w;
}

// A(m,k) . B(n,k) over K into an int8 output with the planned epilogue.
ie_status run_product(const Operand &A, const Operand &B, long long M, long long N, long long K, ExpSrc ea,
                      ExpSrc eb, const ie_mat *out, const ProductWs &pw, uint32_t *flags, int family,
                      hipStream_t st, int relu = 0) {
    if (M == 0 || N == 0) {
        return hip_status(launch_fill_i8(out->exp, out->group == IE_GROUP_ROW ? M : 1, E_MIN, st));
    }
    const int rg = out->group == IE_GROUP_ROW;
    if (K == 0) {
        // empty contraction: every result is zero, every group at E_MIN
        IE_TRY(launch_fill_i8(out->mant, M * N, 0, st));
        return hip_status(launch_fill_i8(out->exp, rg ? M : 1, E_MIN, st));
    }
    Plan pl = plan_product(M, N, K, rg, family);
    log_plan(family ? "conv" : "dense", M, N, K, pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.ea = ea;
    ep.eb = eb;
    ep.row_group = rg;
    ep.out = out->mant;
    ep.out_exp = out->exp;
    ep.flags = flags;
    ep.relu = relu;
    ep.q = mat_q(out);
    if (pl.mode == PLAN_DIRECT) {
        ep.mode = EPI_DIRECT;
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, 1, pl.k_chunk, false, ep, st));
        return IE_OK;
    }
    if (pl.mode == PLAN_RTO) {
        ep.mode = EPI_RTO;
        ep.v16 = pw.v16;
        ep.p16 = pw.p16;
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, 1, pl.k_chunk, false, ep, st));
        IE_TRY(launch_rto_finalize(pw.v16, pw.p16, (int)M, (int)N, pl.t, rg, out->mant, out->exp, flags, st, relu));
        return IE_OK;
    }
    ep.partial = pw.partial;
    ep.split_stride = M * N;
    if (rg && split_round_rows_fits((int)N, 1, 1)) {
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, pl.splits, pl.k_chunk, true, ep, st));
        IE_TRY(launch_split_round_rows(pw.partial, pl.splits, M * N, (int)M, (int)N, (int)N, 1, 1, ea, eb, out->mant,
                                       out->exp, flags, mat_q(out), st, relu));
        return IE_OK;
    }
    ep.gneed = pw.gneed;
    ep.gneed_n = rg ? (int)M : 1;
    IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, pl.splits, pl.k_chunk, true, ep, st));
    IE_TRY(launch_partial_reduce(pw.partial, pl.splits, M * N, (int)M, (int)N, ea, eb, rg, pw.sums, pw.gneed,
                                 mat_q(out), st));
    IE_TRY(launch_round_sums(pw.sums, (int)M, (int)N, (int)N, 1, 1, ea, eb, rg, pw.gneed, out->mant, out->exp, flags,
                             st, relu));
    return IE_OK;
}

struct WgradWs {
    int *partial;
    long long *sums;
    int *gneed;
    int *eps;  // [2]: common exponents of row-grouped operands
};

// Weight gradient [N x Kg] contracted over L rows; the stored output is
// [N x Kout] with column j taken from (j / mc) * mcp + j % mc of the GEMM
// columns (mc == mcp: identity).
WgradWs carve_wgrad(Carve &c, long long N, long long Kg, long long L) {
    WgradWs w;
    Plan pl = plan_wgrad(N, Kg, L);
    w.eps = c.take<int>(2);
    w.gneed = c.take<int>(N > 0 ? N : 1);
    w.partial = c.take<int>((size_t)pl.splits * N * Kg);
    w.sums = c.take<long long>((size_t)N * Kg);
    return w;
}

ie_status run_wgrad(const Operand &A, const Operand &B, long long N, long long Kg, long long Kout, int mc, int mcp,
                    long long L, ExpSrc ea, ExpSrc eb, const ie_mat *dW, const WgradWs &w, uint32_t *flags,
                    hipStream_t st) {
    if (N == 0 || Kout == 0) {
        return hip_status(launch_fill_i8(dW->exp, dW->group == IE_GROUP_ROW ? N : 1, E_MIN, st));
    }
    Plan pl = plan_wgrad(N, Kg, L);
    log_plan("wgrad", N, Kg, L, pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    const int rg = dW->group == IE_GROUP_ROW;
    const bool fused = rg && split_round_rows_fits((int)Kout, mc, mcp);
    ep.partial = w.partial;
    ep.split_stride = N * Kg;
    ep.flags = flags;
    ep.q = mat_q(dW);
    ep.gneed = w.gneed;
    ep.gneed_n = fused ? 0 : rg ? (int)N : 1;
    int splits = pl.splits;
    if (L == 0) {
        IE_TRY(launch_fill_i32(w.partial, N * Kg, 0, st));
        IE_TRY(launch_fill_i32(w.gneed, rg ? N : 1, NEED_NONE, st));
        splits = 1;
    } else {
        IE_TRY(launch_gemm(A, B, (int)N, (int)Kg, (int)L, pl.t, pl.splits, pl.k_chunk, true, ep, st));
    }
    if (fused) {
        IE_TRY(launch_split_round_rows(w.partial, splits, N * Kg, (int)N, (int)Kout, (int)Kg, mc, mcp, ea, eb,
                                       dW->mant, dW->exp, flags, mat_q(dW), st));
        return IE_OK;
    }
    IE_TRY(launch_partial_reduce(w.partial, splits, N * Kg, (int)N, (int)Kg, ea, eb, rg, w.sums, w.gneed,
                                 mat_q(dW), st));
    IE_TRY(launch_round_sums(w.sums, (int)N, (int)Kout, (int)Kg, mc, mcp, ea, eb, rg, w.gneed, dW->mant, dW->exp,
                             flags, st));
    return IE_OK;
}

long long r16(long long x) { return (x + 15) / 16 * 16; }

// A second stream per device, on which independent work of one call runs
// beside the caller's stream (fork and join through events).  Default
// priority; created on first use and kept for the life of the process.
struct AuxStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool tried = false;
};
constexpr int MAX_DEVICES = 64;
std::mutex g_aux_mu;  // guards g_aux and every fork ... join sequence
AuxStream g_aux[MAX_DEVICES];

// Caller holds g_aux_mu.  Null when no second stream can be had (the work
// then runs on the caller's stream alone).
AuxStream *aux_stream() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    AuxStream &a = g_aux[dev];
    if (!a.tried) {
        a.tried = true;
        if (hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess)
            a.s = nullptr;
    }
    return a.s ? &a : nullptr;
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
    g.dpq = make_fastdiv((uint32_t)(g.p * g.q));
    g.dq = make_fastdiv((uint32_t)g.q);
    g.dhw = make_fastdiv((uint32_t)(g.h * g.w));
    g.dw = make_fastdiv((uint32_t)g.w);
    g.cp = (int)r16(g.c);
    g.kp = (int)r16(g.k);
    g.dc = make_fastdiv((uint32_t)g.cp);
    g.ds = make_fastdiv((uint32_t)g.s);
    g.dk = make_fastdiv((uint32_t)g.kp);
    g.dst = make_fastdiv((uint32_t)g.stride);
    const int cp = g.cp, kp = g.kp, st = g.stride;
    int t = BK / cp;
    g.im_dc = BK % cp;
    g.im_ds = t % g.s;
    g.im_dr = t / g.s;
    g.im_d0 = g.im_dc + g.im_ds * cp + g.im_dr * g.w * cp;
    g.im_d1 = (g.w - g.s) * cp;
    t = BK / kp;
    g.dg_dc = BK % kp;
    g.dg_ds = t % g.s;
    g.dg_dr = t / g.s;
    const long long rsc = (long long)g.r * g.s * g.c;
    g.wt_d0 = (int)(g.dg_dc * rsc + (long long)t * g.c);
    g.wt_d1 = (int)(g.c - kp * rsc);
    const long long pq = (long long)g.p * g.q, img = (long long)g.h * g.w * cp;
    g.px_dq = BK % g.q;
    g.px_dp = (BK / g.q) % g.p;
    g.px_d0 = (int)((long long)g.px_dq * st * cp + (long long)g.px_dp * st * g.w * cp + (BK / pq) * img);
    g.px_d1 = (st * g.w - g.q * st) * cp;
    g.px_d2 = (int)(img - (long long)g.p * st * g.w * cp);
    g.px_nw = (int)(BK / pq + 2);
    g.st_inv = (65536 + st - 1) / st;
    return g;
}

// The GEMM loaders address operands through buffer descriptors of at most
// 2^30 bytes (a tile's images, a step's contraction rows) with 32-bit
// offsets, and keep filter-tap masks of 15 bits per axis.
constexpr long long WINDOW = 1ll << 30;

bool conv_fits(const ConvGeom &g) {
    if (g.r > 15 || g.s > 15 || g.h > 65535 || g.w > 65535 || g.cp > (1 << 22) || g.kp > (1 << 22)) return false;
    const long long pq = (long long)g.p * g.q, hw = (long long)g.h * g.w;
    const long long img_x = hw * g.cp, img_y = pq * g.kp;
    if ((256 / pq + 2) * img_x > WINDOW) return false;   // forward im2col rows, weight-gradient pixels
    if ((256 / hw + 2) * img_y > WINDOW) return false;   // input-gradient gather
    const long long rs = (long long)g.r * g.s;
    return 256 * rs * g.cp <= WINDOW && 256 * rs * g.kp <= WINDOW && 128ll * g.kp <= WINDOW;
}

// The in-place weight read of the input gradient spans the whole weight.
bool weight_window_fits(const ConvGeom &g) { return (long long)g.kp * g.r * g.s * g.c <= WINDOW; }

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
    Carve c{nullptr, HEADER};
    if (K != r16(K)) {
        c.take<int8_t>((size_t)M * r16(K));
        c.take<int8_t>((size_t)N * r16(K));
    }
    carve_product(c, M, N, r16(K), 0);
    return align256(c.off);
}

size_t linear_dx_ws(long long M, long long N, long long K) {
    Carve c{nullptr, HEADER};
    c.take<int>(1);
    c.take<int8_t>((size_t)K * r16(N));
    if (N != r16(N)) c.take<int8_t>((size_t)M * r16(N));
    carve_product(c, M, K, r16(N), 0);
    return align256(c.off);
}

size_t linear_dw_ws(long long M, long long N, long long K) {
    Carve c{nullptr, HEADER};
    c.take<int8_t>((size_t)M * r16(N));
    c.take<int8_t>((size_t)M * r16(K));
    carve_wgrad(c, N, K, M);
    return align256(c.off);
}

size_t conv_fwd_ws(const ie_conv_desc *d) {
    ConvGeom g = geom(d);
    Carve c{nullptr, HEADER};
    if (g.cp != g.c) {
        c.take<int8_t>((size_t)g.n * g.h * g.w * g.cp);
        c.take<int8_t>((size_t)g.k * g.r * g.s * g.cp);
    }
    carve_product(c, (long long)g.n * g.p * g.q, g.k, (long long)g.r * g.s * g.cp, 1);
    return align256(c.off);
}

size_t conv_bwd_ws(const ie_conv_desc *d) {
    ConvGeom g = geom(d);
    Carve c{nullptr, HEADER};
    c.take<int>(1);
    c.take<int8_t>((size_t)g.c * g.r * g.s * g.kp);
    if (g.kp != g.k) c.take<int8_t>((size_t)g.n * g.p * g.q * g.kp);
    if (g.cp != g.c) c.take<int8_t>((size_t)g.n * g.h * g.w * g.cp);
    carve_product(c, (long long)g.n * g.h * g.w, g.c, (long long)g.r * g.s * g.kp, 1);
    carve_wgrad(c, g.k, (long long)g.r * g.s * g.cp, (long long)g.n * g.p * g.q);
    return align256(c.off);
}

// Input and weight gradient of a convolution in one paired launch, when
// both plans allow it: the input gradient as a round-to-odd product reading
// W in place, the weight gradient as a split contraction with the fused row
// finalize.  IE_ERR_UNSUPPORTED, with nothing launched, otherwise.
ie_status conv_bwd_pair(const ConvGeom &g, const ie_mat *X, const ie_mat *W, const ie_mat *dY, const ie_mat *dX,
                        const ie_mat *dW, const int8_t *dys, int8_t *xp, const ProductWs &pw, const WgradWs &w,
                        uint32_t *flags, hipStream_t st) {
    const long long nhw = (long long)g.n * g.h * g.w, npq = (long long)g.n * g.p * g.q;
    const long long rskp = (long long)g.r * g.s * g.kp, rscp = (long long)g.r * g.s * g.cp;
    const long long rsc = (long long)g.r * g.s * g.c;
    if (W->group != IE_GROUP_TENSOR || g.c % 16 != 0 || !aligned(W->mant, 16) || !weight_window_fits(g))
        return IE_ERR_UNSUPPORTED;
    if (nhw == 0 || npq == 0 || dW->group != IE_GROUP_ROW || !split_round_rows_fits((int)rsc, g.c, g.cp))
        return IE_ERR_UNSUPPORTED;
    const Plan p1 = plan_product(nhw, g.c, rskp, 0, 1);
    if (p1.mode != PLAN_RTO) return IE_ERR_UNSUPPORTED;
    const Plan p2 = plan_wgrad(g.k, rscp, npq);
    const Operand A1{LD_DGRAD, dys, g.kp, (int)nhw, g};
    const Operand B1{LD_WT, W->mant, 0, g.c, g};
    const Operand A2{LD_T, dys, g.kp, g.k, {}};
    const Operand B2{LD_IM2COL_T, xp ? xp : X->mant, g.cp, (int)rscp, g};
    if (!gemm_pair_supported(A1, B1, p1.t, A2, B2, p2.t)) return IE_ERR_UNSUPPORTED;
    log_plan("conv", nhw, g.c, rskp, p1);
    log_plan("wgrad", g.k, rscp, npq, p2);
    if (xp) IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, xp, st));
    const ExpSrc edy{dY->exp, nullptr, 0}, ew{W->exp, nullptr, 0}, ex{X->exp, nullptr, 0};
    Epi e1;
    memset(&e1, 0, sizeof e1);
    e1.ea = edy;
    e1.eb = ew;
    e1.out = dX->mant;
    e1.out_exp = dX->exp;
    e1.flags = flags;
    e1.mode = EPI_RTO;
    e1.v16 = pw.v16;
    e1.p16 = pw.p16;
    e1.q = mat_q(dX);
    Epi e2;
    memset(&e2, 0, sizeof e2);
    e2.partial = w.partial;
    e2.split_stride = g.k * rscp;
    e2.flags = flags;
    e2.gneed = w.gneed;
    e2.gneed_n = 0;
    e2.q = mat_q(dW);
    IE_TRY(launch_gemm_pair(A1, B1, (int)nhw, g.c, (int)rskp, p1.t, p1.k_chunk, e1, A2, B2, g.k, (int)rscp,
                            (int)npq, p2.t, p2.splits, p2.k_chunk, e2, st));
    IE_TRY(launch_finalize_pair(pw.v16, pw.p16, (int)nhw, g.c, p1.t, dX->mant, dX->exp, w.partial, p2.splits,
                                g.k * rscp, g.k, (int)rsc, (int)rscp, g.c, g.cp, edy, ex, dW->mant, dW->exp, flags,
                                mat_q(dW), st));
    return IE_OK;
}

ie_status check_update(const ie_mat *W, const ie_mat *V, const ie_mat *G, ie_scalar weight_decay) {
    (void)weight_decay;  // any (C, e) scalar
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(V));
    IE_CHECK(check_mat(G));
    if (mat_q(V) != 7) return IE_ERR_BITS;  // the velocity is INT8 at every weight width
    if (V->rows != W->rows || V->cols != W->cols || G->rows != W->rows || G->cols != W->cols)
        return IE_ERR_SHAPE;
    if (W->cols > 64 * 4 * 32) return IE_ERR_UNSUPPORTED;
    return IE_OK;
}

UpdateArgs update_args(const ie_mat *W, const ie_mat *V, const ie_mat *G, ie_scalar lr, ie_scalar momentum,
                       ie_scalar weight_decay, int *tmp, void *ws) {
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
    a.wd_m = weight_decay.mant;
    a.wd_e = weight_decay.exp;
    a.w_q = mat_q(W);
    a.tmp = tmp;
    a.flags = (uint32_t *)ws;
    return a;
}

// ---------------------------------------------------------------------------
// Batched products: C_z = op(A_z) . op(B_z) over stacks of slices, row groups
// ---------------------------------------------------------------------------

enum BmmForm { BMM_NT = 0, BMM_NN = 1, BMM_TN = 2 };

// Tiles instantiated for the batched kernel: 128x128, 64x256, 128x64, 64x64
// (the 64x256 one for A . B^T only).  A row group fits one tile (direct
// epilogue, no second pass) when N <= the tile width, so rows up to 256
// wide take the 64x256 tile when there is work enough for it.  The tuning
// override of the other products does not apply here: only these choices
// are run.
Plan plan_batched(long long Z, long long M, long long N, bool kk) {
    auto tiles = [&](Tile t) { return Z * cdiv(M, t.bm()) * cdiv(N, t.bn()); };
    Tile t{1, 1};
    if (kk && N > 128 && N <= 256 && tiles(Tile{1, 4}) >= 2ll * NCU) t = Tile{1, 4};
    else if (N > 64 && tiles(Tile{2, 2}) >= 2ll * NCU) t = Tile{2, 2};
    else if (tiles(Tile{2, 1}) >= 2ll * NCU) t = Tile{2, 1};
    return Plan{t, N <= t.bn() ? PLAN_DIRECT : PLAN_RTO, 1, BK};
}

struct BmmWs {
    int8_t *a, *b;   // padded / aligned operand copies
    int *ea, *eb;    // per-slice common exponents of aligned operands
    int16_t *p16, *v16;
};

BmmWs carve_bmm(Carve &c, int form, long long Z, long long M, long long N, long long K) {
    BmmWs w{};
    const long long Kp = r16(K);
    if (form == BMM_NT) {
        if (Kp != K) {
            w.a = c.take<int8_t>((size_t)(Z * M * Kp));
            w.b = c.take<int8_t>((size_t)(Z * N * Kp));
        }
    } else if (form == BMM_NN) {
        if (Kp != K) w.a = c.take<int8_t>((size_t)(Z * M * Kp));
        w.b = c.take<int8_t>((size_t)(Z * K * r16(N)));
        w.eb = c.take<int>((size_t)(Z > 0 ? Z : 1));
    } else {
        w.a = c.take<int8_t>((size_t)(Z * K * r16(M)));
        w.b = c.take<int8_t>((size_t)(Z * K * r16(N)));
        w.ea = c.take<int>((size_t)(Z > 0 ? Z : 1));
        w.eb = c.take<int>((size_t)(Z > 0 ? Z : 1));
    }
    if (N > 64) {
        // round-to-odd: per (row, 64-wide column tile) needs and int16 values
        w.p16 = c.take<int16_t>((size_t)(Z * M * cdiv(N, 64)));
        w.v16 = c.take<int16_t>((size_t)(Z * M * N));
    }
    return w;
}

size_t bmm_ws(long long Z, long long M, long long N, long long K) {
    size_t best = HEADER;
    for (int form = 0; form < 3; ++form) {
        Carve c{nullptr, HEADER};
        carve_bmm(c, form, Z, M, N, K);
        best = best > align256(c.off) ? best : align256(c.off);
    }
    return best;
}

ie_status bmm(int form, int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C, void *ws, size_t ws_bytes,
              void *stream) {
    IE_CHECK(check_mat(A));
    IE_CHECK(check_mat(B));
    IE_CHECK(check_mat(C));
    if (batch < 0) return IE_ERR_SHAPE;
    if (batch == 0) return A->rows == 0 && B->rows == 0 && C->rows == 0 ? IE_OK : IE_ERR_SHAPE;
    if (A->rows % batch || B->rows % batch || C->rows % batch) return IE_ERR_SHAPE;
    const long long Z = batch, ra = A->rows / Z, rb = B->rows / Z;
    long long M, N, K;
    if (form == BMM_NT) {
        M = ra, K = A->cols, N = rb;
        if (B->cols != K) return IE_ERR_SHAPE;
    } else if (form == BMM_NN) {
        M = ra, K = A->cols, N = B->cols;
        if (rb != K) return IE_ERR_SHAPE;
    } else {
        K = ra, M = A->cols, N = B->cols;
        if (rb != K) return IE_ERR_SHAPE;
    }
    if (C->rows != Z * M || C->cols != N) return IE_ERR_SHAPE;
    if (C->group != IE_GROUP_ROW) return IE_ERR_UNSUPPORTED;
    if (K > MAX_CONTRACT || Z > 65535) return IE_ERR_UNSUPPORTED;
    if (r16(M) > DIM_MAX || r16(N) > DIM_MAX) return IE_ERR_UNSUPPORTED;  // padded pitches stay int
    if (form != BMM_TN && r16(K) == K && (!aligned(A->mant, 16) || (form == BMM_NT && !aligned(B->mant, 16))))
        return IE_ERR_UNSUPPORTED;
    if (form == BMM_TN && ((long long)BK * r16(M) > WINDOW || (long long)BK * r16(N) > WINDOW))
        return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < bmm_ws(Z, M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const BmmWs w = carve_bmm(c, form, Z, M, N, K);
    if (M == 0 || N == 0) return hip_status(launch_fill_i8(C->exp, Z * M, E_MIN, st));
    if (K == 0) {
        IE_TRY(launch_fill_i8(C->mant, Z * M * N, 0, st));
        return hip_status(launch_fill_i8(C->exp, Z * M, E_MIN, st));
    }
    const Plan pl = plan_batched(Z, M, N, form == BMM_NT);
    log_plan(form == BMM_NT ? "bmm_nt" : form == BMM_NN ? "bmm_nn" : "bmm_tn", Z * M, N, K, pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.row_group = 1;
    ep.out = C->mant;
    ep.out_exp = C->exp;
    ep.flags = flags;
    ep.q = mat_q(C);
    ep.mode = pl.mode == PLAN_DIRECT ? EPI_DIRECT : EPI_RTO;
    if (ep.mode == EPI_RTO) {
        ep.v16 = w.v16;
        ep.p16 = w.p16;
    }
    BatchArgs ba;
    memset(&ba, 0, sizeof ba);
    ba.Z = batch;
    ba.out = M * N;
    ba.out_exp = M;
    ba.p16 = M * cdiv(N, pl.t.bn());
    const int a_row = A->group == IE_GROUP_ROW, b_row = B->group == IE_GROUP_ROW;
    Operand Aop{}, Bop{};
    long long Kc = r16(K);
    if (form == BMM_NT || form == BMM_NN) {
        const int8_t *as = A->mant;
        if (Kc != K) {
            IE_TRY(launch_pad_rows(A->mant, Z * M, K, nullptr, 0, nullptr, Kc, w.a, st));
            as = w.a;
        }
        Aop = Operand{LD_K, as, Kc, (int)M, {}};
        ba.a = M * Kc;
        ep.ea = ExpSrc{A->exp, nullptr, a_row};
        ba.ea8 = a_row ? M : 0;
        if (form == BMM_NT) {
            const int8_t *bs = B->mant;
            if (Kc != K) {
                IE_TRY(launch_pad_rows(B->mant, Z * N, K, nullptr, 0, nullptr, Kc, w.b, st));
                bs = w.b;
            }
            Bop = Operand{LD_K, bs, Kc, (int)N, {}};
            ep.eb = ExpSrc{B->exp, nullptr, b_row};
            ba.eb8 = b_row ? N : 0;
            ba.b = N * Kc;
        } else {
            // B_z [K x N] contracted over its rows: aligned per slice, rows
            // padded to 16 bytes, read row-contiguous; A's padding columns
            // are zeroed by its loader (contraction K, not Kc)
            const long long Np = r16(N);
            IE_TRY(launch_pad_rows_z(B->mant, B->exp, b_row, batch, (int)K, (int)N, (int)Np, w.b, w.eb, st));
            Bop = Operand{LD_T, w.b, Np, (int)N, {}};
            ep.eb = ExpSrc{nullptr, w.eb, 0};
            ba.eb32 = 1;
            ba.b = K * Np;
            Kc = K;
        }
    } else {
        // both contracted over their rows: aligned per slice, rows padded to 16
        const long long Mp = r16(M), Np = r16(N);
        IE_TRY(launch_pad_rows_z(A->mant, A->exp, a_row, batch, (int)K, (int)M, (int)Mp, w.a, w.ea, st));
        IE_TRY(launch_pad_rows_z(B->mant, B->exp, b_row, batch, (int)K, (int)N, (int)Np, w.b, w.eb, st));
        Aop = Operand{LD_T, w.a, Mp, (int)M, {}};
        Bop = Operand{LD_T, w.b, Np, (int)N, {}};
        ba.a = K * Mp;
        ba.b = K * Np;
        ep.ea = ExpSrc{nullptr, w.ea, 0};
        ep.eb = ExpSrc{nullptr, w.eb, 0};
        ba.ea32 = ba.eb32 = 1;
        Kc = K;
    }
    IE_TRY(launch_gemm_batched(Aop, Bop, (int)M, (int)N, (int)Kc, pl.t, ep, ba, st));
    if (ep.mode == EPI_RTO)
        IE_TRY(launch_rto_finalize(w.v16, w.p16, (int)(Z * M), (int)N, pl.t, 1, C->mant, C->exp, flags, st));
    return IE_OK;
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
    return HEADER + align256(UPD_WS_INTS * sizeof(int));
}
size_t ie_sgd_update_multi_workspace(int32_t n) {
    if (n < 0) return 0;
    return HEADER + (size_t)(n > 0 ? n : 1) * align256(UPD_WS_INTS * sizeof(int));
}

ie_status ie_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return IE_ERR_NULL;
    if (ws_bytes < HEADER) return IE_ERR_WORKSPACE;
    return hip_status(launch_zero_flags(ws, (hipStream_t)stream));
}

static ie_status linear_fwd(const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws, size_t ws_bytes,
                            void *stream, int relu) {
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    long long M = X->rows, K = X->cols, N = W->rows;
    if (W->cols != K || Y->rows != M || Y->cols != N) return IE_ERR_SHAPE;
    if (K > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!aligned(X->mant, 16) || !aligned(W->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_fwd_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const long long Kp = r16(K);
    const int8_t *xs = X->mant, *wsrc = W->mant;
    if (Kp != K) {
        int8_t *xp = c.take<int8_t>((size_t)M * Kp), *wp = c.take<int8_t>((size_t)N * Kp);
        IE_TRY(launch_pad_rows(X->mant, M, K, nullptr, 0, nullptr, Kp, xp, st));
        IE_TRY(launch_pad_rows(W->mant, N, K, nullptr, 0, nullptr, Kp, wp, st));
        xs = xp;
        wsrc = wp;
    }
    ProductWs pw = carve_product(c, M, N, Kp, 0);
    Operand A{LD_K, xs, Kp, (int)M, {}};
    Operand B{LD_K, wsrc, Kp, (int)N, {}};
    ExpSrc ea{X->exp, nullptr, X->group == IE_GROUP_ROW};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, M, N, Kp, ea, eb, Y, pw, flags, 0, st, relu);
}

ie_status ie_linear_fwd(const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws, size_t ws_bytes,
                        void *stream) {
    return linear_fwd(X, W, Y, ws, ws_bytes, stream, 0);
}

ie_status ie_linear_fwd_act(const ie_mat *X, const ie_mat *W, const ie_mat *Y, int act, void *ws, size_t ws_bytes,
                            void *stream) {
    if (act != IE_ACT_NONE && act != IE_ACT_RELU) return IE_ERR_UNSUPPORTED;
    return linear_fwd(X, W, Y, ws, ws_bytes, stream, act == IE_ACT_RELU);
}

ie_status ie_linear_bwd_dx(const ie_mat *dY, const ie_mat *W, const ie_mat *dX, void *ws, size_t ws_bytes,
                           void *stream) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(dX));
    long long M = dY->rows, N = dY->cols, K = W->cols;
    if (W->rows != N || dX->rows != M || dX->cols != K) return IE_ERR_SHAPE;
    if (N > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!aligned(dY->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_dx_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const long long Np = r16(N);
    int *estar = c.take<int>(1);
    int8_t *wt = c.take<int8_t>((size_t)K * Np);
    int8_t *dyp = Np != N ? c.take<int8_t>((size_t)M * Np) : nullptr;
    ProductWs pw = carve_product(c, M, K, Np, 0);
    if (M == 0 || K == 0) return run_product(Operand{}, Operand{}, M, K, Np, ExpSrc{}, ExpSrc{}, dX, pw, flags, 0, st);
    IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, (int)N, 1, (int)K, (int)Np, wt, estar,
                                  st));
    const int8_t *dys = dY->mant;
    if (dyp) {
        IE_TRY(launch_pad_rows(dY->mant, M, N, nullptr, 0, nullptr, Np, dyp, st));
        dys = dyp;
    }
    Operand A{LD_K, dys, Np, (int)M, {}};
    Operand B{LD_K, wt, Np, (int)K, {}};
    ExpSrc ea{dY->exp, nullptr, dY->group == IE_GROUP_ROW};
    ExpSrc eb{nullptr, estar, 0};
    return run_product(A, B, M, K, Np, ea, eb, dX, pw, flags, 0, st);
}

ie_status ie_linear_bwd_dw(const ie_mat *dY, const ie_mat *X, const ie_mat *dW, void *ws, size_t ws_bytes,
                           void *stream) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(dW));
    long long M = dY->rows, N = dY->cols, K = X->cols;
    if (X->rows != M || dW->rows != N || dW->cols != K) return IE_ERR_SHAPE;
    if (!aligned(dY->mant, 16) || !aligned(X->mant, 16)) return IE_ERR_UNSUPPORTED;
    if ((long long)BK * r16(N) > WINDOW || (long long)BK * r16(K) > WINDOW) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < linear_dw_ws(M, N, K)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const long long Np = r16(N), Kp = r16(K);
    int8_t *dya = c.take<int8_t>((size_t)M * Np);
    int8_t *xa = c.take<int8_t>((size_t)M * Kp);
    WgradWs w = carve_wgrad(c, N, K, M);
    if (N == 0 || K == 0)
        return run_wgrad(Operand{}, Operand{}, N, K, K, 1, 1, M, ExpSrc{}, ExpSrc{}, dW, w, flags, st);
    // common exponents over the contraction axis (rows); align ROW operands,
    // pad rows to multiples of 16
    const int8_t *dys = dY->mant, *xs = X->mant;
    const bool dy_row = dY->group == IE_GROUP_ROW, x_row = X->group == IE_GROUP_ROW;
    ExpSrc ea{dY->exp, nullptr, 0}, eb{X->exp, nullptr, 0};
    if (dy_row || x_row) {
        IE_TRY(launch_exp_max2(dY->exp, n_exps(dY), w.eps, X->exp, n_exps(X), w.eps + 1, st));
        ea = ExpSrc{nullptr, w.eps, 0};
        eb = ExpSrc{nullptr, w.eps + 1, 0};
    }
    if ((dy_row || Np != N) && M > 0) {
        IE_TRY(launch_pad_rows(dY->mant, M, N, dY->exp, dy_row, dy_row ? w.eps : nullptr, Np, dya, st));
        dys = dya;
    }
    if ((x_row || Kp != K) && M > 0) {
        IE_TRY(launch_pad_rows(X->mant, M, K, X->exp, x_row, x_row ? w.eps + 1 : nullptr, Kp, xa, st));
        xs = xa;
    }
    Operand A{LD_T, dys, Np, (int)N, {}};
    Operand B{LD_T, xs, Kp, (int)K, {}};
    return run_wgrad(A, B, N, K, K, 1, 1, M, ea, eb, dW, w, flags, st);
}

static ie_status conv_fwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws,
                          size_t ws_bytes, void *stream, int relu) {
    IE_CHECK(check_conv(d));
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    ConvGeom g = geom(d);
    long long rsc = (long long)g.r * g.s * g.c;
    long long npq = (long long)g.n * g.p * g.q;
    long long nhw = (long long)g.n * g.h * g.w;
    if (X->rows != nhw || X->cols != g.c) return IE_ERR_SHAPE;
    if (W->rows != g.k || W->cols != rsc) return IE_ERR_SHAPE;
    if (Y->rows != npq || Y->cols != g.k) return IE_ERR_SHAPE;
    if (X->group != IE_GROUP_TENSOR) return IE_ERR_UNSUPPORTED;
    if (rsc > MAX_CONTRACT || npq > DIM_MAX || !conv_fits(g)) return IE_ERR_UNSUPPORTED;
    if (!aligned(X->mant, 16) || !aligned(W->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < conv_fwd_ws(d)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const int8_t *xs = X->mant, *wsrc = W->mant;
    if (g.cp != g.c) {
        int8_t *xp = c.take<int8_t>((size_t)nhw * g.cp), *wp = c.take<int8_t>((size_t)g.k * g.r * g.s * g.cp);
        IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, xp, st));
        IE_TRY(launch_pad_rows(W->mant, (long long)g.k * g.r * g.s, g.c, nullptr, 0, nullptr, g.cp, wp, st));
        xs = xp;
        wsrc = wp;
    }
    const long long kg = (long long)g.r * g.s * g.cp;
    ProductWs pw = carve_product(c, npq, g.k, kg, 1);
    Operand A{LD_IM2COL, xs, g.cp, (int)npq, g};
    Operand B{LD_K, wsrc, kg, g.k, {}};
    ExpSrc ea{X->exp, nullptr, 0};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, npq, g.k, kg, ea, eb, Y, pw, flags, 1, st, relu);
}

ie_status ie_conv_fwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws,
                      size_t ws_bytes, void *stream) {
    return conv_fwd(d, X, W, Y, ws, ws_bytes, stream, 0);
}

ie_status ie_conv_fwd_act(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *Y, int act,
                          void *ws, size_t ws_bytes, void *stream) {
    if (act != IE_ACT_NONE && act != IE_ACT_RELU) return IE_ERR_UNSUPPORTED;
    return conv_fwd(d, X, W, Y, ws, ws_bytes, stream, act == IE_ACT_RELU);
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
    if ((long long)g.k * g.r * g.s > MAX_CONTRACT || nhw > DIM_MAX || !conv_fits(g)) return IE_ERR_UNSUPPORTED;
    if (!aligned(X->mant, 16) || !aligned(dY->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < conv_bwd_ws(d)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    int *estar = c.take<int>(1);
    int8_t *wt = c.take<int8_t>((size_t)g.c * g.r * g.s * g.kp);
    int8_t *dyp = g.kp != g.k ? c.take<int8_t>((size_t)npq * g.kp) : nullptr;
    int8_t *xp = g.cp != g.c ? c.take<int8_t>((size_t)nhw * g.cp) : nullptr;
    const long long rskp = (long long)g.r * g.s * g.kp, rscp = (long long)g.r * g.s * g.cp;
    ProductWs pw = carve_product(c, nhw, g.c, rskp, 1);
    WgradWs w = carve_wgrad(c, g.k, rscp, npq);
    const int8_t *dys = dY->mant;
    if (dyp && (dX || dW)) {
        IE_TRY(launch_pad_rows(dY->mant, npq, g.k, nullptr, 0, nullptr, g.kp, dyp, st));
        dys = dyp;
    }
    auto dgrad = [&](hipStream_t s) -> ie_status {
        Operand A{LD_DGRAD, dys, g.kp, (int)nhw, g};
        ExpSrc ea{dY->exp, nullptr, 0};
        if (W->group == IE_GROUP_TENSOR && g.c % 16 == 0 && aligned(W->mant, 16) && weight_window_fits(g)) {
            // one weight exponent: nothing to align, read W in place
            Operand B{LD_WT, W->mant, 0, g.c, g};
            return run_product(A, B, nhw, g.c, rskp, ea, ExpSrc{W->exp, nullptr, 0}, dX, pw, flags, 1, s);
        }
        IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, g.k, g.r * g.s, g.c, g.kp, wt,
                                      estar, s));
        Operand B{LD_K, wt, rskp, g.c, {}};
        return run_product(A, B, nhw, g.c, rskp, ea, ExpSrc{nullptr, estar, 0}, dX, pw, flags, 1, s);
    };
    auto wgrad = [&](hipStream_t s) -> ie_status {
        const int8_t *xs = X->mant;
        if (xp) {
            IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, xp, s));
            xs = xp;
        }
        Operand A{LD_T, dys, g.kp, g.k, {}};
        Operand B{LD_IM2COL_T, xs, g.cp, (int)rscp, g};
        return run_wgrad(A, B, g.k, rscp, rsc, g.c, g.cp, npq, ExpSrc{dY->exp, nullptr, 0},
                         ExpSrc{X->exp, nullptr, 0}, dW, w, flags, s);
    };
    if (dX && dW) {
        // the two products are independent: one grid runs both when a paired
        // kernel covers their plans ...
        const ie_status sp = conv_bwd_pair(g, X, W, dY, dX, dW, dys, xp, pw, w, flags, st);
        if (sp != IE_ERR_UNSUPPORTED) return sp;
        // ... else the weight gradient runs on a second stream beside the
        // input gradient
        std::lock_guard<std::mutex> lock(g_aux_mu);
        if (AuxStream *ax = aux_stream()) {
            IE_TRY(hipEventRecord(ax->fork, st));
            IE_TRY(hipStreamWaitEvent(ax->s, ax->fork, 0));
            const ie_status sw = wgrad(ax->s);
            const hipError_t ej = hipEventRecord(ax->join, ax->s);
            const ie_status sd = dgrad(st);
            const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(st, ax->join, 0) : ej;
            if (sw != IE_OK) return sw;
            if (sd != IE_OK) return sd;
            return hip_status(ew);
        }
    }
    if (dX) IE_CHECK(dgrad(st));
    if (dW) IE_CHECK(wgrad(st));
    return IE_OK;
}

ie_status ie_sgd_update(const ie_mat *W, const ie_mat *V, const ie_mat *G, ie_scalar lr, ie_scalar momentum,
                        ie_scalar weight_decay, void *ws, size_t ws_bytes, void *stream) {
    IE_CHECK(check_update(W, V, G, weight_decay));
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < ie_sgd_update_workspace(W->rows, W->cols)) return IE_ERR_WORKSPACE;
    Carve c{(char *)ws, HEADER};
    UpdateArgs a = update_args(W, V, G, lr, momentum, weight_decay, c.take<int>(UPD_WS_INTS), ws);
    return hip_status(launch_sgd_update(a, (hipStream_t)stream));
}

ie_status ie_sgd_update_multi(int32_t n, const ie_mat *W, const ie_mat *V, const ie_mat *G, ie_scalar lr,
                              ie_scalar momentum, ie_scalar weight_decay, void *ws, size_t ws_bytes, void *stream) {
    if (n < 0) return IE_ERR_SHAPE;
    if (n == 0) return IE_OK;
    if (!W || !V || !G) return IE_ERR_NULL;
    for (int i = 0; i < n; ++i) IE_CHECK(check_update(W + i, V + i, G + i, weight_decay));
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < ie_sgd_update_multi_workspace(n)) return IE_ERR_WORKSPACE;
    Carve c{(char *)ws, HEADER};
    std::vector<UpdateArgs> a((size_t)n);
    for (int i = 0; i < n; ++i)
        a[i] = update_args(W + i, V + i, G + i, lr, momentum, weight_decay, c.take<int>(UPD_WS_INTS), ws);
    return hip_status(launch_sgd_update_multi(a.data(), n, (hipStream_t)stream));
}


// ---------------------------------------------------------------------------
// Pointwise steps
// ---------------------------------------------------------------------------

static bool same_shape(const ie_mat *a, const ie_mat *b) { return a->rows == b->rows && a->cols == b->cols; }

ie_status ie_relu_fwd(const ie_mat *X, const ie_mat *Y, int relu6, void *stream) {
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(Y));
    if (!same_shape(X, Y)) return IE_ERR_SHAPE;
    if (X->group != Y->group) return IE_ERR_GROUP;
    if (relu6 != 0 && relu6 != 1) return IE_ERR_SHAPE;
    return hip_status(launch_relu_fwd(X->mant, X->exp, X->group == IE_GROUP_ROW, Y->mant, Y->exp, X->rows, X->cols,
                                      relu6, mat_q(Y), (hipStream_t)stream));
}

ie_status ie_relu_bwd(const ie_mat *dY, const ie_mat *Y, const ie_mat *dX, int relu6, void *stream) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(Y));
    IE_CHECK(check_mat(dX));
    if (!same_shape(dY, Y) || !same_shape(dY, dX)) return IE_ERR_SHAPE;
    if (dX->group != dY->group) return IE_ERR_GROUP;
    if (relu6 != 0 && relu6 != 1) return IE_ERR_SHAPE;
    return hip_status(launch_relu_bwd(dY->mant, dY->exp, dY->group == IE_GROUP_ROW, Y->mant, Y->exp,
                                      Y->group == IE_GROUP_ROW, dX->mant, dX->exp, dY->rows, dY->cols, relu6,
                                      mat_q(Y), (hipStream_t)stream));
}

size_t ie_add_workspace(int64_t rows, int64_t cols) {
    (void)rows;
    (void)cols;
    return HEADER + (size_t)ADD_MAX_BLOCKS * sizeof(int);
}

ie_status ie_add(const ie_mat *A, const ie_mat *B, const ie_mat *Z, void *ws, size_t ws_bytes, void *stream) {
    IE_CHECK(check_mat(A));
    IE_CHECK(check_mat(B));
    IE_CHECK(check_mat(Z));
    if (!same_shape(A, B) || !same_shape(A, Z)) return IE_ERR_SHAPE;
    if (!ws) return IE_ERR_WORKSPACE;
    if (ws_bytes < ie_add_workspace(A->rows, A->cols)) return IE_ERR_WORKSPACE;
    Carve c{(char *)ws, HEADER};
    int *bmax = c.take<int>(ADD_MAX_BLOCKS);
    return hip_status(launch_add(A->mant, A->exp, A->group == IE_GROUP_ROW, B->mant, B->exp,
                                 B->group == IE_GROUP_ROW, Z->mant, Z->exp, Z->group == IE_GROUP_ROW, A->rows,
                                 A->cols, bmax, (uint32_t *)ws, mat_q(Z), (hipStream_t)stream));
}

size_t ie_bmm_workspace(int32_t batch, int64_t M, int64_t N, int64_t K) {
    if (batch < 0 || M < 0 || N < 0 || K < 0) return 0;
    return bmm_ws(batch, M, N, K);
}

ie_status ie_bmm_nt(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C, void *ws, size_t ws_bytes,
                    void *stream) {
    return bmm(BMM_NT, batch, A, B, C, ws, ws_bytes, stream);
}

ie_status ie_bmm_nn(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C, void *ws, size_t ws_bytes,
                    void *stream) {
    return bmm(BMM_NN, batch, A, B, C, ws, ws_bytes, stream);
}

ie_status ie_bmm_tn(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C, void *ws, size_t ws_bytes,
                    void *stream) {
    return bmm(BMM_TN, batch, A, B, C, ws, ws_bytes, stream);
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

ie_status ie_profile_select(int kind) {
    prof_select(kind);
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
        case IE_ERR_BITS: return "IE_ERR_BITS";
    }
    return "IE_ERR_UNKNOWN";
}

}  // extern "C"
