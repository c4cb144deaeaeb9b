// C ABI of the (C, e) layer-step library: the launch sequence of every entry
// point (argument checks, plans and workspace layouts are in ie_plan.cpp).
// See include/ie.h.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "../../include/ie.h"
#include "ie_device.h"
#include "ie_internal.h"

using namespace ie;

// Fixed device scratch of ie_linear_fwd_noalloc (one copy per GPU, held until
// the process ends).  Host code never uses this name as an address: each
// device's copy is found once with hipGetSymbolAddress.
static __device__ __align__(256) char scratch[IE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<void *> g_scratch[MAX_DEVICES];

// The current device's copy of `scratch` (looked up on the first call on that
// device; the lookup is idempotent, so racing first calls agree), or nullptr.
void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
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

// Forced plans for tests and tuning (unset in normal use; validated like
// every plan).
Force force_product() { return force_from_env("IE_TILE", false); }
Force force_wgrad() { return force_from_env("IE_WTILE", true); }

// Diagnostics: IE_PLAN_LOG set prints every planned product to stderr.
void log_plan(const char *what, long long M, long long N, long long K, const Plan &pl) {
    static const bool on = getenv("IE_PLAN_LOG") != nullptr;
    if (!on) return;
    fprintf(stderr, "[ie plan] %s M=%lld N=%lld K=%lld tile=%dx%d mode=%d splits=%d k_chunk=%d\n", what, M, N, K,
            pl.t.bm(), pl.t.bn(), pl.mode, pl.splits, pl.k_chunk);
}

int family_of(const Operand &A, const Operand &B) {
    if (A.kind == LD_K && B.kind == LD_K) return FAM_DENSE;
    if (A.kind == LD_IM2COL) return FAM_IM2COL;
    if (A.kind == LD_DGRAD) return B.kind == LD_WT ? FAM_DGRAD_WT : FAM_DGRAD;
    if (A.kind == LD_T) return B.kind == LD_T ? FAM_WGRAD : FAM_WGRAD_CONV;
    return -1;
}

// IE_ERR_UNSUPPORTED when a plan has no kernel or the workspace reserved for
// the call does not hold what its kernels write.
ie_status checked_plan(const Plan &pl, long long M, long long N, long long K, int rg, int family, const Needs &have,
                       const Needs &need) {
    if (!plan_valid(pl, M, N, K, rg, family)) return IE_ERR_UNSUPPORTED;
    if (!covers(have, need)) return IE_ERR_UNSUPPORTED;
    return IE_OK;
}

// A(m,k) . B(n,k) over K into an int8 output with the planned epilogue.
ie_status run_product(const Operand &A, const Operand &B, long long M, long long N, long long K, ExpSrc ea,
                      ExpSrc eb, const ie_mat *out, const ProductWs &pw, uint32_t *flags, hipStream_t st,
                      Act act = Act{}) {
    if (M == 0 || N == 0) {
        return hip_status(launch_fill_i8(out->exp, out->group == IE_GROUP_ROW ? M : 1, E_MIN, st));
    }
    const int rg = out->group == IE_GROUP_ROW;
    if (K == 0) {
        // empty contraction: every result is zero, every group at E_MIN
        IE_TRY(launch_fill_i8(out->mant, M * N, 0, st));
        return hip_status(launch_fill_i8(out->exp, rg ? M : 1, E_MIN, st));
    }
    const int family = family_of(A, B);
    const Plan pl = plan_product(M, N, K, rg, family, force_product());
    IE_CHECK(checked_plan(pl, M, N, K, rg, family, pw.n, product_needs(pl, M, N, K, rg)));
    log_plan(family == FAM_DENSE ? "dense" : "conv", M, N, K, pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.ea = ea;
    ep.eb = eb;
    ep.row_group = rg;
    ep.out = out->mant;
    ep.out_exp = out->exp;
    ep.flags = flags;
    ep.act = act;
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
        IE_TRY(launch_rto_finalize(pw.v16, pw.p16, (int)M, (int)N, pl.t, rg, out->mant, out->exp, flags, st, act));
        return IE_OK;
    }
    if (pl.mode == PLAN_RECOMP) {
        // group maxima first, then the product again, rounded straight to int8
        ep.tneed = pw.tneed;
        ep.tneed_n = rg ? 0 : recomp_grid(M, N, K, pl.t);
        ep.mode = EPI_MAX;
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, 1, pl.k_chunk, false, ep, st));
        ep.mode = EPI_GIVEN;
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, 1, pl.k_chunk, false, ep, st));
        return IE_OK;
    }
    ep.partial = pw.partial;
    ep.split_stride = M * N;
    if (rg && split_round_rows_fits((int)N, 1, 1)) {
        IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, pl.splits, pl.k_chunk, true, ep, st));
        IE_TRY(launch_split_round_rows(pw.partial, pl.splits, M * N, (int)M, (int)N, (int)N, 1, 1, ea, eb, out->mant,
                                       out->exp, flags, mat_q(out), st, act));
        return IE_OK;
    }
    ep.gneed = pw.gneed;
    ep.gneed_n = rg ? (int)M : 1;
    IE_TRY(launch_gemm(A, B, (int)M, (int)N, (int)K, pl.t, pl.splits, pl.k_chunk, true, ep, st));
    IE_TRY(launch_partial_reduce(pw.partial, pl.splits, M * N, (int)M, (int)N, ea, eb, rg, pw.sums, pw.gneed,
                                 mat_q(out), st));
    IE_TRY(launch_round_sums(pw.sums, (int)M, (int)N, (int)N, 1, 1, ea, eb, rg, pw.gneed, out->mant, out->exp, flags,
                             st, act));
    return IE_OK;
}

// Input gradient of a strided convolution in stride phases (the recomputed
// epilogue: group maximum over every phase, then each phase rounded
// straight to int8 at its input pixels).
ie_status run_dgrad_phased(const DgradPlan &dp, const Operand &A, const Operand &B, long long N, ExpSrc ea,
                           ExpSrc eb, const ie_mat *out, const ProductWs &pw, uint32_t *flags, hipStream_t st,
                           Act act) {
    IE_CHECK(checked_plan(dp.pl, dp.M, N, dp.K, 0, FAM_DGRAD, pw.n, product_needs(dp.pl, dp.M, N, dp.K, 0)));
    if (dp.pl.mode != PLAN_RECOMP || out->group != IE_GROUP_TENSOR || dp.ps.n == 0) return IE_ERR_UNSUPPORTED;
    log_plan("conv phased", dp.M, N, dp.K, dp.pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
    ep.ea = ea;
    ep.eb = eb;
    ep.out = out->mant;
    ep.out_exp = out->exp;
    ep.flags = flags;
    ep.q = mat_q(out);
    ep.act = act;
    ep.ph = dp.ps;
    ep.tneed = pw.tneed;
    ep.tneed_n = recomp_grid(dp.M, N, dp.K, dp.pl.t);
    ep.mode = EPI_MAX;
    IE_TRY(launch_gemm(A, B, (int)dp.M, (int)N, (int)dp.K, dp.pl.t, 1, dp.pl.k_chunk, false, ep, st));
    ep.mode = EPI_GIVEN;
    IE_TRY(launch_gemm(A, B, (int)dp.M, (int)N, (int)dp.K, dp.pl.t, 1, dp.pl.k_chunk, false, ep, st));
    return IE_OK;
}

// Weight gradient [N x Kg] contracted over L rows; the stored output is
// [N x Kout] with column j taken from (j / mc) * mcp + j % mc of the GEMM
// columns (mc == mcp: identity).
ie_status run_wgrad(const Operand &A, const Operand &B, long long N, long long Kg, long long Kout, int mc, int mcp,
                    long long L, ExpSrc ea, ExpSrc eb, const ie_mat *dW, const WgradWs &w, uint32_t *flags,
                    hipStream_t st) {
    if (N == 0 || Kout == 0) {
        return hip_status(launch_fill_i8(dW->exp, dW->group == IE_GROUP_ROW ? N : 1, E_MIN, st));
    }
    const int family = family_of(A, B);
    const int rg = dW->group == IE_GROUP_ROW;
    const Plan pl = plan_wgrad(N, Kg, L, family, force_wgrad());
    IE_CHECK(checked_plan(pl, N, Kg, L, rg, family, w.n, wgrad_needs(pl, N, Kg, Kout, mc, mcp, rg)));
    log_plan("wgrad", N, Kg, L, pl);
    Epi ep;
    memset(&ep, 0, sizeof ep);
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

// A 1x1 convolution with stride 1 and no padding: every product is a plain
// dense one (rows of the activations and gradients are pixels).
static bool conv_is_dense(const ConvGeom &g) { return g.r == 1 && g.s == 1 && g.stride == 1 && g.pad == 0; }

// Input and weight gradient of a convolution in one paired launch, when both
// plans allow it: the input gradient as a round-to-odd product, or as the
// second pass of a recomputed one (its first pass launched just before), B1
// being the weight read in place or its aligned transposed copy, already
// written; the weight gradient as a split contraction with the fused row
// finalize.  IE_ERR_UNSUPPORTED, with nothing launched, otherwise.
ie_status conv_bwd_pair(const ConvGeom &g, const DgradPlan &dp, const ie_mat *X, const Operand &B1, ExpSrc ew,
                        const ie_mat *dY, const ie_mat *dX, const ie_mat *dW, const int8_t *dys, int8_t *xp,
                        const ConvBwdWs &cw, uint32_t *flags, hipStream_t st, Act act1) {
    const long long nhw = (long long)g.n * g.h * g.w, npq = (long long)g.n * g.p * g.q;
    const long long rscp = (long long)g.r * g.s * g.cp;
    const long long rsc = (long long)g.r * g.s * g.c;
    if (nhw == 0 || npq == 0 || dX->group != IE_GROUP_TENSOR || dW->group != IE_GROUP_ROW ||
        !split_round_rows_fits((int)rsc, g.c, g.cp) || conv_is_dense(g))
        return IE_ERR_UNSUPPORTED;
    const Operand A1{LD_DGRAD, dys, g.kp, (int)nhw, g};
    const Operand A2{LD_T, dys, g.kp, g.k, {}};
    const Operand B2{LD_IM2COL_T, xp ? xp : X->mant, g.cp, (int)rscp, g};
    const int fam1 = family_of(A1, B1);
    const Plan p1 = dp.pl;
    const long long M1 = dp.M, K1 = dp.K;
    if (p1.mode != PLAN_RTO && p1.mode != PLAN_RECOMP) return IE_ERR_UNSUPPORTED;
    // a one-step input gradient runs faster in its own one-step kernels (one
    // LDS stage, twice the workgroups per CU) than inside the paired grid,
    // whose tiles keep the pipelined form (measured on ResNet-50's 1x1
    // layers with 64 and 128 output channels: 7-37 us per layer)
    if (K1 <= BK) return IE_ERR_UNSUPPORTED;
    const Plan p2 = plan_wgrad(g.k, rscp, npq, FAM_WGRAD_CONV, force_wgrad());
    if (!gemm_pair_supported(A1, B1, p1.t, A2, B2, p2.t)) return IE_ERR_UNSUPPORTED;
    if (checked_plan(p1, M1, g.c, K1, 0, fam1, cw.pw.n, product_needs(p1, M1, g.c, K1, 0)) != IE_OK ||
        checked_plan(p2, g.k, rscp, npq, 1, FAM_WGRAD_CONV, cw.w.n, wgrad_needs(p2, g.k, rscp, rsc, g.c, g.cp, 1)) !=
            IE_OK)
        return IE_ERR_UNSUPPORTED;
    log_plan(dp.ps.n ? "conv phased" : "conv", M1, g.c, K1, p1);
    log_plan("wgrad", g.k, rscp, npq, p2);
    if (xp) IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, xp, st));
    const ExpSrc edy{dY->exp, nullptr, 0}, ex{X->exp, nullptr, 0};
    Epi e1;
    memset(&e1, 0, sizeof e1);
    e1.ea = edy;
    e1.eb = ew;
    e1.out = dX->mant;
    e1.out_exp = dX->exp;
    e1.flags = flags;
    e1.mode = EPI_RTO;
    e1.v16 = cw.pw.v16;
    e1.p16 = cw.pw.p16;
    e1.q = mat_q(dX);
    e1.act = act1;
    e1.ph = dp.ps;
    if (p1.mode == PLAN_RECOMP) {
        e1.tneed = cw.pw.tneed;
        e1.tneed_n = recomp_grid(M1, g.c, K1, p1.t);
        e1.mode = EPI_MAX;
        IE_TRY(launch_gemm(A1, B1, (int)M1, g.c, (int)K1, p1.t, 1, p1.k_chunk, false, e1, st));
        e1.mode = EPI_GIVEN;
    }
    Epi e2;
    memset(&e2, 0, sizeof e2);
    e2.partial = cw.w.partial;
    e2.split_stride = g.k * rscp;
    e2.flags = flags;
    e2.gneed = cw.w.gneed;
    e2.gneed_n = 0;
    e2.q = mat_q(dW);
    IE_TRY(launch_gemm_pair(A1, B1, (int)M1, g.c, (int)K1, p1.t, p1.k_chunk, e1, A2, B2, g.k, (int)rscp,
                            (int)npq, p2.t, p2.splits, p2.k_chunk, e2, st));
    if (p1.mode == PLAN_RECOMP) {
        IE_TRY(launch_split_round_rows(cw.w.partial, p2.splits, g.k * rscp, g.k, (int)rsc, (int)rscp, g.c, g.cp, edy,
                                       ex, dW->mant, dW->exp, flags, mat_q(dW), st));
        return IE_OK;
    }
    IE_TRY(launch_finalize_pair(cw.pw.v16, cw.pw.p16, (int)nhw, g.c, p1.t, dX->mant, dX->exp, cw.w.partial,
                                p2.splits, g.k * rscp, g.k, (int)rsc, (int)rscp, g.c, g.cp, edy, ex, dW->mant, dW->exp,
                                flags, mat_q(dW), st, act1));
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
    // the round-to-odd epilogue writes v16 / p16: a plan runs only when the
    // workspace carved for this call holds them
    if (!plan_valid_batched(pl, form, M, N, K) || !covers(w.n, batched_needs(pl, Z, M, N)))
        return IE_ERR_UNSUPPORTED;
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
    return linear_fwd_ws(M, N, K, force_product());
}
size_t ie_linear_bwd_dx_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return linear_dx_ws(M, N, K, force_product());
}
size_t ie_linear_bwd_dw_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return linear_dw_ws(M, N, K, force_wgrad());
}
size_t ie_conv_fwd_workspace(const ie_conv_desc *d) {
    if (check_conv(d) != IE_OK) return 0;
    return conv_fwd_ws(geom(d), force_product());
}
size_t ie_conv_bwd_workspace(const ie_conv_desc *d) {
    if (check_conv(d) != IE_OK) return 0;
    return conv_bwd_ws(geom(d), force_product(), force_wgrad());
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
                            void *stream, int relu, uint32_t *flags_out = nullptr) {
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    long long M = X->rows, K = X->cols, N = W->rows;
    if (W->cols != K || Y->rows != M || Y->cols != N) return IE_ERR_SHAPE;
    if (K > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!aligned(X->mant, 16) || !aligned(W->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    const Force f = force_product();
    if (ws_bytes < linear_fwd_ws(M, N, K, f)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = flags_out ? flags_out : (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const LinearFwdWs w = carve_linear_fwd(c, M, N, K, f);
    const long long Kp = r16(K);
    const int8_t *xs = X->mant, *wsrc = W->mant;
    if (Kp != K) {
        IE_TRY(launch_pad_rows(X->mant, M, K, nullptr, 0, nullptr, Kp, w.xp, st));
        IE_TRY(launch_pad_rows(W->mant, N, K, nullptr, 0, nullptr, Kp, w.wp, st));
        xs = w.xp;
        wsrc = w.wp;
    }
    Operand A{LD_K, xs, Kp, (int)M, {}};
    Operand B{LD_K, wsrc, Kp, (int)N, {}};
    ExpSrc ea{X->exp, nullptr, X->group == IE_GROUP_ROW};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, M, N, Kp, ea, eb, Y, w.pw, flags, st, Act{relu, nullptr});
}

ie_status ie_linear_fwd(const ie_mat *X, const ie_mat *W, const ie_mat *Y, void *ws, size_t ws_bytes,
                        void *stream) {
    return linear_fwd(X, W, Y, ws, ws_bytes, stream, 0);
}

ie_status ie_linear_fwd_noalloc(const ie_mat *X, const ie_mat *W, const ie_mat *Y, uint32_t *flags, void *stream) {
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(Y));
    if (W->cols != X->cols || Y->rows != X->rows || Y->cols != W->rows) return IE_ERR_SHAPE;
    if (linear_fwd_ws(X->rows, W->rows, X->cols, force_product()) > IE_NOALLOC_SCRATCH_BYTES) return IE_ERR_SCRATCH;
    void *p = scratch_ptr();
    if (!p) return IE_ERR_HIP;
    // the scratch's flag header stands in for the caller's flag word when
    // none is given (nothing reads it then)
    return linear_fwd(X, W, Y, p, IE_NOALLOC_SCRATCH_BYTES, stream, 0, flags);
}

ie_status ie_linear_fwd_act(const ie_mat *X, const ie_mat *W, const ie_mat *Y, int act, void *ws, size_t ws_bytes,
                            void *stream) {
    if (act != IE_ACT_NONE && act != IE_ACT_RELU) return IE_ERR_UNSUPPORTED;
    return linear_fwd(X, W, Y, ws, ws_bytes, stream, act == IE_ACT_RELU);
}

static ie_status linear_bwd_dx(const ie_mat *dY, const ie_mat *W, const ie_mat *dX, void *ws, size_t ws_bytes,
                               void *stream, Act act) {
    IE_CHECK(check_mat(dY));
    IE_CHECK(check_mat(W));
    IE_CHECK(check_mat(dX));
    long long M = dY->rows, N = dY->cols, K = W->cols;
    if (W->rows != N || dX->rows != M || dX->cols != K) return IE_ERR_SHAPE;
    if (N > MAX_CONTRACT) return IE_ERR_UNSUPPORTED;
    if (!aligned(dY->mant, 16)) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    const Force f = force_product();
    if (ws_bytes < linear_dx_ws(M, N, K, f)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const LinearDxWs w = carve_linear_dx(c, M, N, K, f);
    const long long Np = r16(N);
    if (M == 0 || K == 0)
        return run_product(Operand{LD_K}, Operand{LD_K}, M, K, Np, ExpSrc{}, ExpSrc{}, dX, w.pw, flags, st, act);
    IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, (int)N, 1, (int)K, (int)Np, w.wt,
                                  w.estar, st));
    const int8_t *dys = dY->mant;
    if (w.dyp) {
        IE_TRY(launch_pad_rows(dY->mant, M, N, nullptr, 0, nullptr, Np, w.dyp, st));
        dys = w.dyp;
    }
    Operand A{LD_K, dys, Np, (int)M, {}};
    Operand B{LD_K, w.wt, Np, (int)K, {}};
    ExpSrc ea{dY->exp, nullptr, dY->group == IE_GROUP_ROW};
    ExpSrc eb{nullptr, w.estar, 0};
    return run_product(A, B, M, K, Np, ea, eb, dX, w.pw, flags, st, act);
}

ie_status ie_linear_bwd_dx(const ie_mat *dY, const ie_mat *W, const ie_mat *dX, void *ws, size_t ws_bytes,
                           void *stream) {
    return linear_bwd_dx(dY, W, dX, ws, ws_bytes, stream, Act{});
}

ie_status ie_linear_bwd_dx_act(const ie_mat *dY, const ie_mat *W, const ie_mat *X, const ie_mat *dX, int act,
                               void *ws, size_t ws_bytes, void *stream) {
    if (act != IE_ACT_NONE && act != IE_ACT_RELU) return IE_ERR_UNSUPPORTED;
    if (act == IE_ACT_NONE) return linear_bwd_dx(dY, W, dX, ws, ws_bytes, stream, Act{});
    IE_CHECK(check_mat(X));
    IE_CHECK(check_mat(dX));
    if (X->rows != dX->rows || X->cols != dX->cols) return IE_ERR_SHAPE;
    if (X->mant == dX->mant) return IE_ERR_UNSUPPORTED;
    return linear_bwd_dx(dY, W, dX, ws, ws_bytes, stream, Act{0, X->mant});
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
    const Force fw = force_wgrad();
    if (ws_bytes < linear_dw_ws(M, N, K, fw)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const LinearDwWs w = carve_linear_dw(c, M, N, K, fw);
    const long long Np = r16(N), Kp = r16(K);
    if (N == 0 || K == 0)
        return run_wgrad(Operand{LD_T}, Operand{LD_T}, N, K, K, 1, 1, M, ExpSrc{}, ExpSrc{}, dW, w.w, flags, st);
    // common exponents over the contraction axis (rows); align ROW operands,
    // pad rows to multiples of 16
    const int8_t *dys = dY->mant, *xs = X->mant;
    const bool dy_row = dY->group == IE_GROUP_ROW, x_row = X->group == IE_GROUP_ROW;
    ExpSrc ea{dY->exp, nullptr, 0}, eb{X->exp, nullptr, 0};
    if (dy_row || x_row) {
        IE_TRY(launch_exp_max2(dY->exp, n_exps(dY), w.w.eps, X->exp, n_exps(X), w.w.eps + 1, st));
        ea = ExpSrc{nullptr, w.w.eps, 0};
        eb = ExpSrc{nullptr, w.w.eps + 1, 0};
    }
    if ((dy_row || Np != N) && M > 0) {
        IE_TRY(launch_pad_rows(dY->mant, M, N, dY->exp, dy_row, dy_row ? w.w.eps : nullptr, Np, w.dya, st));
        dys = w.dya;
    }
    if ((x_row || Kp != K) && M > 0) {
        IE_TRY(launch_pad_rows(X->mant, M, K, X->exp, x_row, x_row ? w.w.eps + 1 : nullptr, Kp, w.xa, st));
        xs = w.xa;
    }
    Operand A{LD_T, dys, Np, (int)N, {}};
    Operand B{LD_T, xs, Kp, (int)K, {}};
    return run_wgrad(A, B, N, K, K, 1, 1, M, ea, eb, dW, w.w, flags, st);
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
    const Force f = force_product();
    if (ws_bytes < conv_fwd_ws(g, f)) return IE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const ConvFwdWs w = carve_conv_fwd(c, g, f);
    const int8_t *xs = X->mant, *wsrc = W->mant;
    if (g.cp != g.c) {
        IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, w.xp, st));
        IE_TRY(launch_pad_rows(W->mant, (long long)g.k * g.r * g.s, g.c, nullptr, 0, nullptr, g.cp, w.wp, st));
        xs = w.xp;
        wsrc = w.wp;
    }
    const long long kg = (long long)g.r * g.s * g.cp;
    // a 1x1 convolution with stride 1 and no padding is a plain product of
    // the [n h w x cp] activation (no gather)
    Operand A = conv_is_dense(g) ? Operand{LD_K, xs, g.cp, (int)npq, {}} : Operand{LD_IM2COL, xs, g.cp, (int)npq, g};
    Operand B{LD_K, wsrc, kg, g.k, {}};
    ExpSrc ea{X->exp, nullptr, 0};
    ExpSrc eb{W->exp, nullptr, W->group == IE_GROUP_ROW};
    return run_product(A, B, npq, g.k, kg, ea, eb, Y, w.pw, flags, st, Act{relu, nullptr});
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

static ie_status conv_bwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *dY,
                          const ie_mat *dX, const ie_mat *dW, void *ws, size_t ws_bytes, void *stream, int act) {
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
    if (dX && act == IE_ACT_RELU && dX->mant == X->mant) return IE_ERR_UNSUPPORTED;
    if (!ws) return IE_ERR_WORKSPACE;
    const Force f = force_product(), fw = force_wgrad();
    if (ws_bytes < conv_bwd_ws(g, f, fw)) return IE_ERR_WORKSPACE;
    // dX through the ReLU whose output is X: zero where X is not positive
    const Act act1{0, act == IE_ACT_RELU ? X->mant : nullptr};
    hipStream_t st = (hipStream_t)stream;
    uint32_t *flags = (uint32_t *)ws;
    Carve c{(char *)ws, HEADER};
    const ConvBwdWs cw = carve_conv_bwd(c, g, f, fw);
    const long long rskp = (long long)g.r * g.s * g.kp, rscp = (long long)g.r * g.s * g.cp;
    const int8_t *dys = dY->mant;
    if (cw.dyp && (dX || dW)) {
        IE_TRY(launch_pad_rows(dY->mant, npq, g.k, nullptr, 0, nullptr, g.kp, cw.dyp, st));
        dys = cw.dyp;
    }
    // B side of the input gradient: the weight read in place (one exponent,
    // 16-channel multiples, no phases), else its copy aligned over the
    // output channels and transposed to [c][r][s][kp].  The input gradient's
    // plan: stride 2 with one exponent for dX runs in stride phases, which
    // read the copy with its taps sorted by phase.
    const bool dense = conv_is_dense(g);
    const bool in_place_ok = !dense && W->group == IE_GROUP_TENSOR && g.c % 16 == 0 && aligned(W->mant, 16) &&
                             weight_window_fits(g);
    const DgradPlan dp = plan_dgrad(g, dX && dX->group == IE_GROUP_ROW, f, in_place_ok);
    const bool phased = dX && dp.ps.n > 0;
    const bool in_place = !phased && in_place_ok;
    const Operand B1 = in_place ? Operand{LD_WT, W->mant, 0, g.c, g} : Operand{LD_K, cw.wt, rskp, g.c, {}};
    const ExpSrc ew = in_place ? ExpSrc{W->exp, nullptr, 0} : ExpSrc{nullptr, cw.estar, 0};
    if (dX && !in_place && nhw > 0) {
        TapOrder to{};
        if (phased) {
            to.st = dp.ps.st;
            to.pad = g.pad;
            to.s = g.s;
            for (int t = 0; t < dp.ps.n; ++t) {
                to.tap0[t] = dp.ps.r[t].tap0;
                to.sb[t] = dp.ps.r[t].sb;
            }
        }
        IE_TRY(launch_align_transpose(W->mant, W->exp, W->group == IE_GROUP_ROW, g.k, g.r * g.s, g.c, g.kp, cw.wt,
                                      cw.estar, st, to));
    }
    if (dX && dW) {
        // the two products are independent: one grid runs both when a paired
        // kernel covers their plans, else they run one after the other
        const ie_status sp = conv_bwd_pair(g, dp, X, B1, ew, dY, dX, dW, dys, cw.xp, cw, flags, st, act1);
        if (sp != IE_ERR_UNSUPPORTED) return sp;
    }
    if (dX) {
        const Operand A = dense ? Operand{LD_K, dys, g.kp, (int)nhw, {}} : Operand{LD_DGRAD, dys, g.kp, (int)nhw, g};
        if (phased)
            IE_CHECK(run_dgrad_phased(dp, A, B1, g.c, ExpSrc{dY->exp, nullptr, 0}, ew, dX, cw.pw, flags, st, act1));
        else
            IE_CHECK(
                run_product(A, B1, nhw, g.c, rskp, ExpSrc{dY->exp, nullptr, 0}, ew, dX, cw.pw, flags, st, act1));
    }
    if (dW) {
        const int8_t *xs = X->mant;
        if (cw.xp) {
            IE_TRY(launch_pad_rows(X->mant, nhw, g.c, nullptr, 0, nullptr, g.cp, cw.xp, st));
            xs = cw.xp;
        }
        const Operand A{LD_T, dys, g.kp, g.k, {}};
        const Operand B = dense ? Operand{LD_T, xs, g.cp, (int)rscp, {}} : Operand{LD_IM2COL_T, xs, g.cp, (int)rscp, g};
        IE_CHECK(run_wgrad(A, B, g.k, rscp, rsc, g.c, g.cp, npq, ExpSrc{dY->exp, nullptr, 0},
                           ExpSrc{X->exp, nullptr, 0}, dW, cw.w, flags, st));
    }
    return IE_OK;
}

ie_status ie_conv_bwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *dY,
                      const ie_mat *dX, const ie_mat *dW, void *ws, size_t ws_bytes, void *stream) {
    return conv_bwd(d, X, W, dY, dX, dW, ws, ws_bytes, stream, IE_ACT_NONE);
}

ie_status ie_conv_bwd_act(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *dY,
                          const ie_mat *dX, const ie_mat *dW, int act, void *ws, size_t ws_bytes, void *stream) {
    if (act != IE_ACT_NONE && act != IE_ACT_RELU) return IE_ERR_UNSUPPORTED;
    return conv_bwd(d, X, W, dY, dX, dW, ws, ws_bytes, stream, act);
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
        case IE_ERR_SCRATCH: return "IE_ERR_SCRATCH";
    }
    return "IE_ERR_UNKNOWN";
}

}  // extern "C"
