// Host-only check of the library's planner and workspace layouts, built with
// address and undefined-behaviour sanitizers (tests/test_plan_host.py).
//
// For every product / weight-gradient / batched-product shape in a grid that
// crosses the tile edges (1, 63, 64, 65, 197, 256, 257, ...), and for every
// forced plan (tile x mode x splits, including tiles that are not built and
// direct epilogues that would split a group), it checks:
//   * the planner's own plans are valid and the carved workspace holds what
//     they write;
//   * a plan the library would run (valid, and covered by the carve) writes
//     only inside the buffers carved for it: the workspace is allocated at
//     the size the query returns, poisoned whole, the carved buffers are
//     unpoisoned, and every index the kernels write (modelled here from the
//     kernels' own index formulas, tile by tile) is touched -- a write outside
//     a carved buffer, including into the gap before the next one, aborts;
//   * a direct epilogue on a shape whose groups span tiles is rejected;
//   * argument checks and convolution geometry are free of undefined
//     behaviour at the extremes of their ranges.
// Exit status 0 when every check passes; the first failure is printed.
#include <sanitizer/asan_interface.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../integer_only_dnn_amd/csrc/ie_plan.h"

using namespace ie;

static long long g_checks = 0, g_runs = 0;

#define REQUIRE(cond, ...)                                                      \
    do {                                                                        \
        ++g_checks;                                                             \
        if (!(cond)) {                                                          \
            fprintf(stderr, "FAIL %s:%d: %s\n  ", __FILE__, __LINE__, #cond);   \
            fprintf(stderr, __VA_ARGS__);                                       \
            fprintf(stderr, "\n");                                              \
            exit(1);                                                            \
        }                                                                       \
    } while (0)

// A workspace of `bytes`, poisoned whole until buffers are released.
struct Arena {
    char *base;
    size_t bytes;
    explicit Arena(size_t b) : bytes(b) {
        base = (char *)aligned_alloc(256, (b + 255) / 256 * 256);
        ASAN_POISON_MEMORY_REGION(base, bytes);
    }
    ~Arena() {
        ASAN_UNPOISON_MEMORY_REGION(base, bytes);
        free(base);
    }
    template <class T>
    void open(T *p, size_t count) {
        if (p && count) ASAN_UNPOISON_MEMORY_REGION(p, count * sizeof(T));
    }
};

template <class T>
static void touch(T *p, size_t idx) {
    volatile char *c = (volatile char *)(p + idx);
    for (size_t b = 0; b < sizeof(T); ++b) c[b] = 1;
}

// ---------------------------------------------------------------------------
// What the kernels write, from their index formulas.
// ---------------------------------------------------------------------------

// The product epilogues and finalizes of plan pl on an M x N output.
static void product_writes(const Plan &pl, long long M, long long N, long long K, int rg, const ProductWs &w) {
    const int bm = pl.t.bm(), bn = pl.t.bn();
    const long long TM = (M + bm - 1) / bm, TN = (N + bn - 1) / bn;
    if (pl.mode == PLAN_RECOMP) {
        if (!rg) {
            // one running maximum per workgroup of the persistent first pass
            for (int b = 0; b < recomp_grid(M, N, K, pl.t); ++b) touch(w.tneed, (size_t)b);
        } else {
            for (long long r = 0; r < M; ++r)
                for (long long tn = 0; tn < TN; ++tn) touch(w.tneed, (size_t)(r * TN + tn));
        }
    } else if (pl.mode == PLAN_RTO) {
        for (long long tn = 0; tn < TN; ++tn)
            for (long long tm = 0; tm < TM; ++tm) {
                if (!rg) {
                    touch(w.p16, (size_t)(tm + TM * tn));  // one need per tile
                } else {
                    for (long long r = tm * bm; r < (tm + 1) * bm && r < M; ++r)
                        touch(w.p16, (size_t)(r * TN + tn));  // per (row, column tile)
                }
                // int16 values of the tile's valid rows and columns (first and
                // last column of every row)
                for (long long r = tm * bm; r < (tm + 1) * bm && r < M; ++r) {
                    touch(w.v16, (size_t)(r * N + tn * bn));
                    const long long c1 = (tn + 1) * bn < N ? (tn + 1) * bn - 1 : N - 1;
                    touch(w.v16, (size_t)(r * N + c1));
                }
            }
    } else if (pl.mode == PLAN_SPLIT) {
        for (int z = 0; z < pl.splits; ++z) {
            touch(w.partial, (size_t)((long long)z * M * N));
            touch(w.partial, (size_t)((long long)z * M * N + M * N - 1));
        }
        if (!(rg && split_round_rows_fits((int)N, 1, 1))) {
            // group maxima set empty by the split kernel; int64 sums
            for (long long i = 0; i < (rg ? M : 1); ++i) touch(w.gneed, (size_t)i);
            touch(w.sums, 0);
            touch(w.sums, (size_t)(M * N - 1));
        }
    }
}

static void wgrad_writes(const Plan &pl, long long N, long long Kg, long long Kout, int mc, int mcp, int rg,
                         long long L, const WgradWs &w) {
    const int splits = L == 0 ? 1 : pl.splits;  // empty contraction: one zeroed partial
    for (int z = 0; z < splits; ++z) {
        touch(w.partial, (size_t)((long long)z * N * Kg));
        touch(w.partial, (size_t)((long long)z * N * Kg + N * Kg - 1));
    }
    for (long long i = 0; i < (rg ? N : 1); ++i) touch(w.gneed, (size_t)i);
    if (!(rg && split_round_rows_fits((int)Kout, mc, mcp))) {
        touch(w.sums, 0);
        touch(w.sums, (size_t)(N * Kg - 1));
    }
}

static void open_product(Arena &a, const ProductWs &w) {
    a.open(w.gneed, w.n.gneed);
    a.open(w.p16, w.n.p16);
    a.open(w.v16, w.n.v16);
    a.open(w.partial, w.n.partial);
    a.open(w.sums, w.n.sums);
    a.open(w.tneed, w.n.tneed);
}

static void open_wgrad(Arena &a, const WgradWs &w) {
    a.open(w.eps, 2);
    a.open(w.gneed, w.n.gneed);
    a.open(w.partial, w.n.partial);
    a.open(w.sums, w.n.sums);
}

// ---------------------------------------------------------------------------
// Products
// ---------------------------------------------------------------------------

static const long long EDGES[] = {1, 63, 64, 65, 197, 256, 257, 1000};
static const long long EDGES_FORCED[] = {1, 64, 65, 197, 257};
static const Tile TRY_TILES[] = {{1, 1}, {1, 2}, {2, 1}, {2, 2}, {1, 4}, {4, 1}, {4, 4}, {3, 1}, {0, 1}, {1, 0}};

static void check_product_case(long long M, long long N, long long K, int family, const Force &f, bool unforced) {
    for (int rg = 0; rg < 2; ++rg) {
        const Plan pl = plan_product(M, N, K, rg, family, f);
        const bool valid = plan_valid(pl, M, N, K, rg, family);
        Carve c0{nullptr, HEADER};
        const ProductWs q = carve_product(c0, M, N, K, family, f);
        const bool cov = covers(q.n, product_needs(pl, M, N, K, rg));
        if (unforced) {
            REQUIRE(valid, "planner plan invalid: fam %d M %lld N %lld K %lld rg %d tile %dx%d mode %d", family, M, N,
                    K, rg, pl.t.mi, pl.t.ni, pl.mode);
            REQUIRE(cov, "carve short of planner plan: fam %d M %lld N %lld K %lld rg %d", family, M, N, K, rg);
        }
        if (valid && pl.mode == PLAN_DIRECT) {
            const long long tiles = (long long)cdiv(M, pl.t.bm()) * cdiv(N, pl.t.bn());
            REQUIRE(rg ? N <= pl.t.bn() : tiles == 1, "direct plan splits a group: M %lld N %lld rg %d", M, N, rg);
        }
        if (!valid || !cov) continue;  // the library returns IE_ERR_UNSUPPORTED
        Arena a(align256(c0.off));
        Carve c{a.base, HEADER};
        const ProductWs w = carve_product(c, M, N, K, family, f);
        open_product(a, w);
        product_writes(pl, M, N, K, rg, w);
        ++g_runs;
    }
}

static void check_products() {
    const long long Ks[] = {16, 128, 400, 4608};
    const int fams[] = {FAM_DENSE, FAM_IM2COL, FAM_DGRAD, FAM_DGRAD_WT};
    for (int fam : fams)
        for (long long M : EDGES)
            for (long long N : EDGES)
                for (long long K : Ks) check_product_case(M, N, K, fam, Force{0, 0, 0, 0, 1}, true);
    for (int fam : fams)
        for (long long M : EDGES_FORCED)
            for (long long N : EDGES_FORCED)
                for (long long K : Ks) {
                    for (const Tile &t : TRY_TILES)
                        for (int mode = 0; mode < 5; ++mode)
                            for (int sp : {1, 2, 3, 7}) {
                                if (mode != PLAN_SPLIT && sp != 1 && sp != 2) continue;
                                check_product_case(M, N, K, fam, Force{1, t.mi, t.ni, mode, sp}, false);
                            }
                }
    // large outputs of the benchmark workloads (planner only)
    const long long big[][3] = {{401408, 256, 64}, {401408, 64, 576}, {100352, 512, 128}, {25216, 3072, 768},
                                {25216, 768, 3072}, {50432, 576, 192}, {6272, 2048, 512}, {131072, 64, 576}};
    for (auto &s : big)
        for (int fam : fams) check_product_case(s[0], s[1], s[2], fam, Force{0, 0, 0, 0, 1}, true);
}

// Direct epilogues on groups that span tiles must be refused whatever forces them.
static void check_direct_refused() {
    for (const Tile &t : TRY_TILES) {
        if (t.mi < 1 || t.ni < 1) continue;
        const long long M = 2 * t.bm() + 1, N = t.bn() + 1;
        const Plan pl{t, PLAN_DIRECT, 1, BK};
        REQUIRE(!plan_valid(pl, M, N, 256, 0, FAM_DENSE), "direct whole-tensor plan over %lld tiles accepted",
                (long long)cdiv(M, t.bm()) * cdiv(N, t.bn()));
        REQUIRE(!plan_valid(pl, M, N, 256, 1, FAM_DENSE), "direct row plan over rows of %lld accepted", N);
    }
}

// ---------------------------------------------------------------------------
// Weight gradients
// ---------------------------------------------------------------------------

static void check_wgrad_case(long long N, long long Kg, long long Kout, int mc, int mcp, long long L, int family,
                             const Force &f, bool unforced) {
    for (int rg = 0; rg < 2; ++rg) {
        const Plan pl = plan_wgrad(N, Kg, L, family, f);
        const bool valid = plan_valid(pl, N, Kg, L, rg, family);
        Carve c0{nullptr, HEADER};
        const WgradWs q = carve_wgrad(c0, N, Kg, L, family, f);
        const bool cov = covers(q.n, wgrad_needs(pl, N, Kg, Kout, mc, mcp, rg));
        if (unforced) {
            REQUIRE(valid, "wgrad plan invalid: N %lld Kg %lld L %lld rg %d", N, Kg, L, rg);
            REQUIRE(cov, "carve short of wgrad plan: N %lld Kg %lld L %lld rg %d", N, Kg, L, rg);
            REQUIRE(pl.k_chunk <= SPLIT_MAX_ROWS, "wgrad chunk %d over the exact int32 limit", pl.k_chunk);
        }
        if (!valid || !cov) continue;
        Arena a(align256(c0.off));
        Carve c{a.base, HEADER};
        const WgradWs w = carve_wgrad(c, N, Kg, L, family, f);
        open_wgrad(a, w);
        wgrad_writes(pl, N, Kg, Kout, mc, mcp, rg, L, w);
        ++g_runs;
    }
}

static void check_wgrads() {
    const long long Ns[] = {1, 64, 65, 256, 2048};
    const long long Ks[] = {16, 64, 576, 4608};
    const long long Ls[] = {0, 1, 100, 65536, 65537, 401408};
    for (long long N : Ns)
        for (long long K : Ks)
            for (long long L : Ls) {
                check_wgrad_case(N, K, K, 1, 1, L, FAM_WGRAD, Force{0, 0, 0, 0, 1}, true);
                // a convolution with 3 channels padded to 16
                check_wgrad_case(N, 9 * 16, 27, 3, 16, L, FAM_WGRAD_CONV, Force{0, 0, 0, 0, 1}, true);
                if (L > 65537) continue;
                for (const Tile &t : TRY_TILES)
                    for (int sp : {1, 2, 5, 64})
                        check_wgrad_case(N, K, K, 1, 1, L, FAM_WGRAD, Force{1, t.mi, t.ni, PLAN_SPLIT, sp}, false);
            }
}

// ---------------------------------------------------------------------------
// Batched products
// ---------------------------------------------------------------------------

static void bmm_writes(const Plan &pl, long long Z, long long M, long long N, const BmmWs &w) {
    if (pl.mode != PLAN_RTO) return;
    const long long n_ct = (N + pl.t.bn() - 1) / pl.t.bn();
    for (long long z = 0; z < Z; z += (Z > 4 ? Z - 1 : 1))  // first and last slices
        for (long long r = 0; r < M; ++r)
            for (long long tn = 0; tn < n_ct; ++tn) {
                touch(w.p16, (size_t)(z * M * n_ct + r * n_ct + tn));
                touch(w.v16, (size_t)(z * M * N + r * N + tn * pl.t.bn()));
                touch(w.v16, (size_t)(z * M * N + r * N + N - 1));
            }
}

static void check_bmm() {
    const long long Zs[] = {1, 3, 1536};
    const long long Ks[] = {1, 64, 197};
    for (int form = 0; form < 3; ++form)
        for (long long Z : Zs)
            for (long long M : EDGES)
                for (long long N : EDGES)
                    for (long long K : Ks) {
                        if (Z * M * N > (1ll << 24)) continue;
                        Carve c0{nullptr, HEADER};
                        const BmmWs q = carve_bmm(c0, form, Z, M, N, K);
                        const size_t bytes = align256(c0.off);
                        REQUIRE(bytes <= bmm_ws(Z, M, N, K), "bmm size query short");
                        const Plan own = plan_batched(Z, M, N, form == BMM_NT);
                        REQUIRE(plan_valid_batched(own, form, M, N, K), "batched plan invalid: form %d M %lld N %lld",
                                form, M, N);
                        REQUIRE(covers(q.n, batched_needs(own, Z, M, N)), "carve short of batched plan");
                        // the planner's plan, then every other tile and epilogue: the
                        // guard in bmm() runs a plan only if the carve holds it
                        std::vector<Plan> plans{own};
                        for (const Tile &t : TRY_TILES)
                            for (int mode : {PLAN_DIRECT, PLAN_RTO}) plans.push_back(Plan{t, mode, 1, BK});
                        for (const Plan &pl : plans) {
                            if (!plan_valid_batched(pl, form, M, N, K)) continue;
                            if (!covers(q.n, batched_needs(pl, Z, M, N))) continue;
                            Arena a(bytes);
                            Carve c{a.base, HEADER};
                            const BmmWs w = carve_bmm(c, form, Z, M, N, K);
                            a.open(w.p16, w.n.p16);
                            a.open(w.v16, w.n.v16);
                            bmm_writes(pl, Z, M, N, w);
                            ++g_runs;
                        }
                    }
    // the attention workloads of a ViT-B at batch 128: scores (N = 197 on the
    // 64 x 256 tile, direct) and P . V (N = 64, direct); a round-to-odd plan
    // on P . V (the carve holds no int16 values for N <= 64) is refused
    const Plan pv = plan_batched(1536, 197, 64, false);
    REQUIRE(pv.mode == PLAN_DIRECT, "P.V at head size 64 not direct");
    Carve c0{nullptr, HEADER};
    const BmmWs q = carve_bmm(c0, BMM_NN, 1536, 197, 64, 197);
    REQUIRE(!covers(q.n, batched_needs(Plan{Tile{1, 4}, PLAN_RTO, 1, BK}, 1536, 197, 64)),
            "round-to-odd P.V would write int16 values the carve does not hold");
}

// ---------------------------------------------------------------------------
// Whole entry-point layouts at the workload shapes
// ---------------------------------------------------------------------------

static void conv_layouts(const ie_conv_desc &d) {
    REQUIRE(check_conv(&d) == IE_OK, "conv desc rejected");
    const ConvGeom g = geom(&d);
    REQUIRE(conv_fits(g), "workload conv does not fit");
    const Force off{0, 0, 0, 0, 1};
    const long long nhw = (long long)g.n * g.h * g.w, npq = (long long)g.n * g.p * g.q;
    {
        Arena a(conv_bwd_ws(g, off, off));
        Carve c{a.base, HEADER};
        const ConvBwdWs w = carve_conv_bwd(c, g, off, off);
        REQUIRE(c.off <= a.bytes, "conv bwd layout past its size");
        a.open(w.estar, 1);
        a.open(w.wt, (size_t)g.c * g.r * g.s * g.kp);
        if (w.dyp) a.open(w.dyp, (size_t)npq * g.kp);
        if (w.xp) a.open(w.xp, (size_t)nhw * g.cp);
        open_product(a, w.pw);
        open_wgrad(a, w.w);
        // aligned transposed weight [c][r s][kp], padded copies
        touch(w.wt, (size_t)g.c * g.r * g.s * g.kp - 1);
        if (w.dyp) touch(w.dyp, (size_t)npq * g.kp - 1);
        if (w.xp) touch(w.xp, (size_t)nhw * g.cp - 1);
        const long long rscp = (long long)g.r * g.s * g.cp;
        const DgradPlan dp = plan_dgrad(g, 0, off);
        product_writes(dp.pl, dp.M, g.c, dp.K, 0, w.pw);
        const Plan pw = plan_wgrad(g.k, rscp, npq, FAM_WGRAD_CONV, off);
        wgrad_writes(pw, g.k, rscp, (long long)g.r * g.s * g.c, g.c, g.cp, 1, npq, w.w);
    }
    {
        Arena a(conv_fwd_ws(g, off));
        Carve c{a.base, HEADER};
        const ConvFwdWs w = carve_conv_fwd(c, g, off);
        if (w.xp) a.open(w.xp, (size_t)nhw * g.cp);
        if (w.wp) a.open(w.wp, (size_t)g.k * g.r * g.s * g.cp);
        open_product(a, w.pw);
        if (w.xp) touch(w.xp, (size_t)nhw * g.cp - 1);
        if (w.wp) touch(w.wp, (size_t)g.k * g.r * g.s * g.cp - 1);
        product_writes(plan_product(npq, g.k, (long long)g.r * g.s * g.cp, 0, FAM_IM2COL, off), npq, g.k,
                       (long long)g.r * g.s * g.cp, 0, w.pw);
    }
    ++g_runs;
}

static void check_layouts() {
    // ResNet-18 on 32 x 32 inputs and ResNet-50 on 224 x 224 inputs, batch 128
    const ie_conv_desc descs[] = {
        {128, 32, 32, 3, 64, 3, 3, 1, 1},     {128, 32, 32, 64, 64, 3, 3, 1, 1},   {128, 32, 32, 64, 128, 3, 3, 2, 1},
        {128, 4, 4, 512, 512, 3, 3, 1, 1},    {128, 56, 56, 64, 256, 1, 1, 1, 0},  {128, 56, 56, 256, 64, 1, 1, 1, 0},
        {128, 56, 56, 64, 64, 3, 3, 1, 1},    {128, 56, 56, 128, 128, 3, 3, 2, 1}, {128, 56, 56, 256, 512, 1, 1, 2, 0},
        {128, 7, 7, 2048, 512, 1, 1, 1, 0},   {128, 14, 14, 512, 512, 3, 3, 2, 1}, {3, 5, 7, 5, 7, 3, 2, 2, 1},
    };
    for (const auto &d : descs) conv_layouts(d);
    const Force off{0, 0, 0, 0, 1};
    const long long lin[][3] = {{64, 128, 256}, {50432, 576, 192}, {25216, 3072, 768}, {25216, 768, 3072},
                                {5, 7, 9}, {200, 150, 392}};
    for (auto &s : lin) {
        const long long M = s[0], N = s[1], K = s[2];
        Arena a(linear_fwd_ws(M, N, K, off));
        Carve c{a.base, HEADER};
        const LinearFwdWs w = carve_linear_fwd(c, M, N, K, off);
        if (w.xp) a.open(w.xp, (size_t)M * r16(K));
        if (w.wp) a.open(w.wp, (size_t)N * r16(K));
        open_product(a, w.pw);
        for (int rg = 0; rg < 2; ++rg)
            product_writes(plan_product(M, N, r16(K), rg, FAM_DENSE, off), M, N, r16(K), rg, w.pw);
        Arena b(linear_dw_ws(M, N, K, off));
        Carve cb{b.base, HEADER};
        const LinearDwWs v = carve_linear_dw(cb, M, N, K, off);
        b.open(v.dya, (size_t)M * r16(N));
        b.open(v.xa, (size_t)M * r16(K));
        open_wgrad(b, v.w);
        touch(v.dya, (size_t)M * r16(N) - 1);
        touch(v.xa, (size_t)M * r16(K) - 1);
        for (int rg = 0; rg < 2; ++rg) wgrad_writes(plan_wgrad(N, K, M, FAM_WGRAD, off), N, K, K, 1, 1, rg, M, v.w);
        ++g_runs;
    }
}

// ---------------------------------------------------------------------------
// Stride phases of the input gradient
// ---------------------------------------------------------------------------

// The phases of g: their pixels cover every input pixel once (through the
// store formula of the second pass), their taps cover every filter tap once
// (through the weight copy's tap order), each phase's taps and output pixels
// are exactly those the definition p st = h + pad - r pairs with its
// pixels, and the first pass's maxima fit the carve.
static void check_phase_case(const ie_conv_desc &d, int bm, const Force &f) {
    if (check_conv(&d) != IE_OK) return;
    const ConvGeom g = geom(&d);
    if (!phases_apply(g)) return;
    const Phases ps = make_phases(g, bm);
    REQUIRE(ps.n == 4 && ps.st == 2, "stride-2 phases: n %d", ps.n);
    const long long nhw = (long long)g.n * g.h * g.w;
    // pixels: every phase row stored once, inside dX
    std::vector<unsigned char> *hits = new std::vector<unsigned char>((size_t)nhw, 0);
    unsigned char *dx = (unsigned char *)malloc((size_t)nhw);
    long long rows = 0;
    int tiles = 0, taps = 0;
    for (int t = 0; t < ps.n; ++t) {
        const PhaseRec &p = ps.r[t];
        REQUIRE(ps.tm % ps.n == 0 && cdiv(p.rows, bm) <= ps.tm / ps.n, "phase %d tile rows beyond its share", t);
        tiles = cdiv(p.rows, bm) > tiles ? cdiv(p.rows, bm) : tiles;
        REQUIRE(p.rows == (long long)g.n * p.hn * p.wn, "phase rows");
        REQUIRE(p.k0 == taps * g.kp && p.tap0 == taps && p.klen == p.ra * p.sb * g.kp, "phase columns");
        taps += p.ra * p.sb;
        REQUIRE(p.klen <= ps.kmax, "kmax below a phase");
        for (long long m = 0; m < p.rows; ++m) {
            // the kernel's formula (fast divisions) and the plain one
            const uint32_t hw = (uint32_t)(p.hn * p.wn);
            const uint32_t n = (uint32_t)(((uint64_t)m * p.dhw.m) >> p.dhw.s), rem = (uint32_t)m - n * hw;
            const uint32_t i = (uint32_t)(((uint64_t)rem * p.dw.m) >> p.dw.s), j = rem - i * (uint32_t)p.wn;
            REQUIRE(n == m / hw && i == (m % hw) / p.wn && j == (m % hw) % p.wn, "fast division of a phase row");
            const long long h = p.ph + 2ll * i, w = p.pw + 2ll * j;
            REQUIRE(h < g.h && w < g.w, "phase pixel outside the image");
            const long long phys = ((long long)n * ps.h + h) * ps.w + w;
            dx[phys] = 1;  // out of bounds aborts under the sanitizer
            (*hits)[(size_t)phys]++;
            // taps: the phase's (a, b) reach exactly the output pixels of the definition
            if (m < 64 || m + 64 > p.rows) {
                for (int r = 0; r < g.r; ++r)
                    for (int s_ = 0; s_ < g.s; ++s_) {
                        const long long ah = h + g.pad - r, aw = w + g.pad - s_;
                        const bool def = ah >= 0 && aw >= 0 && ah % 2 == 0 && aw % 2 == 0 && ah / 2 < g.p &&
                                         aw / 2 < g.q;
                        const bool mine = r % 2 == (p.ph + g.pad) % 2 && s_ % 2 == (p.pw + g.pad) % 2;
                        bool hit = false;
                        if (mine) {
                            const int a = r / 2, b = s_ / 2;
                            REQUIRE(a < p.ra && b < p.sb, "tap of the phase outside its block");
                            const long long pp = (long long)i + p.ch - a, qq = (long long)j + p.cw - b;
                            hit = pp >= 0 && pp < g.p && qq >= 0 && qq < g.q;
                            if (hit) REQUIRE(pp * 2 == ah && qq * 2 == aw, "phase tap at the wrong output pixel");
                            REQUIRE(phase_tap(ps, g, r, s_) == p.tap0 + a * p.sb + b, "tap order");
                        }
                        REQUIRE(def == hit, "phase taps differ from the definition at (%lld, %lld) tap (%d, %d)",
                                h, w, r, s_);
                    }
            }
        }
        rows += p.rows;
    }
    REQUIRE(rows == nhw && tiles * ps.n == ps.tm, "phase rows %lld of %lld", rows, nhw);
    // the kernel's tile order (tile row t: phase (t + h(t / 4)) % 4, rows
    // from (t / 4) bm) reaches every phase row exactly once
    std::vector<unsigned char> seen_rows((size_t)nhw, 0);
    for (int t = 0; t < ps.tm; ++t) {
        const int ph = (t + (int)(((uint32_t)(t >> 2) * 2654435761u) >> 30)) & 3;
        const PhaseRec &p = ps.r[ph];
        for (long long m = (long long)(t / ps.n) * bm; m < (long long)(t / ps.n + 1) * bm && m < p.rows; ++m) {
            const long long hw = (long long)p.hn * p.wn, nn = m / hw, i = (m % hw) / p.wn, j = (m % hw) % p.wn;
            seen_rows[(size_t)(((nn * ps.h) + p.ph + 2 * i) * ps.w + p.pw + 2 * j)]++;
        }
    }
    for (long long x = 0; x < nhw; ++x) REQUIRE(seen_rows[(size_t)x] == 1, "tile order stores pixel %lld %d times",
                                                 x, (int)seen_rows[(size_t)x]);
    REQUIRE(taps == g.r * g.s, "phase taps %d of %d", taps, g.r * g.s);
    for (long long x = 0; x < nhw; ++x) REQUIRE((*hits)[(size_t)x] == 1, "input pixel %lld stored %d times", x,
                                                 (int)(*hits)[(size_t)x]);
    std::vector<int> seen((size_t)(g.r * g.s), 0);
    for (int r = 0; r < g.r; ++r)
        for (int s_ = 0; s_ < g.s; ++s_) seen[(size_t)phase_tap(ps, g, r, s_)]++;
    for (int v : seen) REQUIRE(v == 1, "tap order not a permutation");
    free(dx);
    delete hits;
    // the plan and its workspace
    const DgradPlan dp = plan_dgrad(g, 0, f);
    const bool valid = plan_valid(dp.pl, dp.M, g.c, dp.K, 0, FAM_DGRAD);
    if (!f.on) REQUIRE(valid, "phased plan invalid");
    if (dp.ps.n && valid) {
        REQUIRE(dp.pl.mode == PLAN_RECOMP && dp.M == (long long)dp.ps.tm * dp.pl.t.bm() && dp.K == dp.ps.kmax,
                "phased plan");
        Arena a(conv_bwd_ws(g, f, Force{0, 0, 0, 0, 1}));
        Carve c{a.base, HEADER};
        const ConvBwdWs w = carve_conv_bwd(c, g, f, Force{0, 0, 0, 0, 1});
        open_product(a, w.pw);
        REQUIRE(covers(w.pw.n, product_needs(dp.pl, dp.M, g.c, dp.K, 0)), "carve short of the phased plan");
        product_writes(dp.pl, dp.M, g.c, dp.K, 0, w.pw);
        ++g_runs;
    }
    REQUIRE(plan_dgrad(g, 1, f).ps.n == 0, "row-grouped input gradient in phases");
}

static void check_phases() {
    const ie_conv_desc ds[] = {
        {2, 9, 9, 24, 40, 3, 3, 2, 1},  {2, 9, 9, 48, 24, 3, 3, 2, 1},  {2, 10, 10, 32, 40, 3, 3, 2, 1},
        {3, 7, 5, 16, 8, 1, 1, 2, 0},   {2, 8, 8, 16, 16, 1, 1, 2, 1},  {1, 1, 1, 16, 16, 1, 1, 2, 0},
        {2, 2, 3, 16, 16, 3, 3, 2, 1},  {2, 11, 6, 20, 30, 5, 5, 2, 2}, {2, 6, 11, 16, 16, 2, 2, 2, 0},
        {2, 12, 12, 16, 48, 4, 4, 2, 1}, {1, 3, 3, 16, 16, 3, 1, 2, 0}, {4, 5, 5, 16, 300, 3, 3, 2, 1},
        {128, 32, 32, 64, 128, 3, 3, 2, 1}, {128, 56, 56, 128, 128, 3, 3, 2, 1},
        {128, 56, 56, 256, 512, 1, 1, 2, 0}, {128, 14, 14, 512, 512, 3, 3, 2, 1},
    };
    const Force off{0, 0, 0, 0, 1};
    for (const auto &d : ds)
        for (int bm : {64, 128, 256}) {
            check_phase_case(d, bm, off);
            check_phase_case(d, bm, Force{1, bm / 64, 1, PLAN_RECOMP, 1});
            check_phase_case(d, bm, Force{1, bm / 64, 2, PLAN_RECOMP, 1});
        }
    // other strides and forced non-recomputed plans are not decomposed
    const ie_conv_desc d1{2, 9, 9, 16, 16, 3, 3, 1, 1}, d3{2, 9, 9, 16, 16, 3, 3, 3, 1};
    REQUIRE(plan_dgrad(geom(&d1), 0, off).ps.n == 0, "stride 1 in phases");
    REQUIRE(plan_dgrad(geom(&d3), 0, off).ps.n == 0, "stride 3 in phases");
    const ie_conv_desc d2{2, 9, 9, 16, 16, 3, 3, 2, 1};
    REQUIRE(plan_dgrad(geom(&d2), 0, Force{1, 2, 1, PLAN_RTO, 1}).ps.n == 0, "forced round-to-odd in phases");
    REQUIRE(plan_dgrad(geom(&d2), 0, Force{1, 2, 1, PLAN_RECOMP, 1}).ps.n == 4, "forced recompute not in phases");
}

// Argument checks and geometry at the ends of their ranges (UB-free under
// the sanitizer; shapes the kernels cannot take are refused).
static void check_extremes() {
    const int big = 2147483647;
    const ie_conv_desc ds[] = {
        {1, 65535, 65535, 16, 16, 3, 3, 1, 1}, {1, 1, 1, big, 1, 1, 1, 1, 0}, {big, 1, 1, 1, 1, 1, 1, 1, 0},
        {1, 32768, 32768, 16, 16, 1, 1, 1, 0}, {1, 8, 8, 16, 16, 3, 3, big, 1}, {1, 8, 8, 16, 16, 3, 3, 1, big / 4},
        {1, 100, 100, 4194304, 16, 1, 1, 1, 0}, {1, 7, 7, 16, 16, 15, 15, 1, 7}, {1, 7, 7, 16, 16, 16, 16, 1, 8},
        {4, 2, 2, 1, 1, 2, 2, 1, 0},
    };
    for (const auto &d : ds) {
        if (check_conv(&d) != IE_OK) continue;
        const ConvGeom g = geom(&d);
        (void)conv_fits(g);
        (void)weight_window_fits(g);
        ++g_checks;
    }
    ie_mat m{nullptr, nullptr, 0, 0, 0, 0};
    REQUIRE(check_mat(&m) == IE_ERR_NULL, "tensor group without exponent accepted");
    m.rows = -1;
    REQUIRE(check_mat(&m) == IE_ERR_SHAPE || check_mat(&m) == IE_ERR_NULL, "negative rows accepted");
    REQUIRE(check_mat(nullptr) == IE_ERR_NULL, "null matrix accepted");
    const Force bad = force_from_env("IE_PLAN_CHECK_UNSET_VARIABLE", false);
    REQUIRE(!bad.on, "unset override read as on");
}

int main() {
    check_extremes();
    check_direct_refused();
    check_products();
    check_wgrads();
    check_bmm();
    check_layouts();
    check_phases();
    printf("plan_check: %lld checks, %lld plans written into their carved workspaces\n", g_checks, g_runs);
    return 0;
}
