// Host-side planning of the (C, e) library (see ie_plan.h): argument checks,
// convolution geometry, product plans and workspace layouts.  No GPU code.
#include "ie_plan.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace ie {

// ---------------------------------------------------------------------------
// Argument checks and geometry
// ---------------------------------------------------------------------------

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

int mat_q(const ie_mat *t) { return (t->bits ? t->bits : 8) - 1; }

FastDiv make_fastdiv(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;  // l = ceil(log2 d)
    int s = 31 + l;
    uint64_t m = ((1ull << s) + d - 1) / d;
    return FastDiv{(uint32_t)m, s};
}

ie_status check_conv(const ie_conv_desc *d) {
    if (!d) return IE_ERR_NULL;
    if (d->n < 0 || d->h <= 0 || d->w <= 0 || d->c <= 0 || d->k <= 0 || d->r <= 0 || d->s <= 0 ||
        d->stride <= 0 || d->pad < 0)
        return IE_ERR_SHAPE;
    if ((long long)d->h + 2ll * d->pad < d->r || (long long)d->w + 2ll * d->pad < d->s) return IE_ERR_SHAPE;
    long long rsc = (long long)d->r * d->s * d->c;
    if (rsc > DIM_MAX || (long long)d->n * d->h * d->w * d->c > DIM_MAX * 8ll) return IE_ERR_SHAPE;
    return IE_OK;
}

// Every field is computed in checked 64-bit arithmetic; g.ok is cleared when
// an intermediate overflows or a field does not fit the 32-bit integers the
// kernels use (conv_fits then rejects the shape).
namespace {
struct Checked {
    bool ok = true;
    long long mul(long long a, long long b) {
        long long r = 0;
        if (__builtin_mul_overflow(a, b, &r)) ok = false;
        return ok ? r : 0;
    }
    long long add(long long a, long long b) {
        long long r = 0;
        if (__builtin_add_overflow(a, b, &r)) ok = false;
        return ok ? r : 0;
    }
    long long sub(long long a, long long b) {
        long long r = 0;
        if (__builtin_sub_overflow(a, b, &r)) ok = false;
        return ok ? r : 0;
    }
    int fit(long long v) {
        if (v < -(1ll << 31) || v > DIM_MAX) ok = false;
        return ok ? (int)v : 0;
    }
};
}  // namespace

ConvGeom geom(const ie_conv_desc *d) {
    ConvGeom g;
    memset(&g, 0, sizeof g);
    Checked k;
    auto fdv = [&](long long v) -> FastDiv { return make_fastdiv(v >= 1 && v <= DIM_MAX ? (uint32_t)v : 1u); };
    const long long n = d->n, h = d->h, w = d->w, c = d->c, ko = d->k, r = d->r, s = d->s, st = d->stride,
                    pad = d->pad;
    g.n = d->n;
    g.h = d->h;
    g.w = d->w;
    g.c = d->c;
    g.k = d->k;
    g.r = d->r;
    g.s = d->s;
    g.stride = d->stride;
    g.pad = d->pad;
    // check_conv guarantees h + 2 pad >= r, w + 2 pad >= s and positive sizes
    const long long p = k.sub(k.add(h, k.mul(2, pad)), r) / st + 1;
    const long long q = k.sub(k.add(w, k.mul(2, pad)), s) / st + 1;
    const long long cp = r16(c), kp = r16(ko);
    const long long pq = k.mul(p, q), hw = k.mul(h, w);
    g.p = k.fit(p);
    g.q = k.fit(q);
    g.cp = k.fit(cp);
    g.kp = k.fit(kp);
    k.fit(pq);
    k.fit(hw);
    k.fit(k.mul(n, pq));
    if (!k.ok) return g;  // g.ok stays 0
    g.dpq = fdv(pq);
    g.dq = fdv(q);
    g.dhw = fdv(hw);
    g.dw = fdv(w);
    g.dc = fdv(cp);
    g.ds = fdv(s);
    g.dk = fdv(kp);
    g.dst = fdv(st);
    long long t = BK / cp;
    g.im_dc = k.fit(BK % cp);
    g.im_ds = k.fit(t % s);
    g.im_dr = k.fit(t / s);
    g.im_d0 = k.fit(k.add(k.add(BK % cp, k.mul(t % s, cp)), k.mul(k.mul(t / s, w), cp)));
    g.im_d1 = k.fit(k.mul(w - s, cp));
    t = BK / kp;
    g.dg_dc = k.fit(BK % kp);
    g.dg_ds = k.fit(t % s);
    g.dg_dr = k.fit(t / s);
    const long long rsc = k.mul(k.mul(r, s), c);
    g.wt_d0 = k.fit(k.add(k.mul(BK % kp, rsc), k.mul(t, c)));
    g.wt_d1 = k.fit(k.sub(c, k.mul(kp, rsc)));
    const long long img = k.mul(hw, cp);
    const long long px_dq = BK % q, px_dp = (BK / q) % p;
    g.px_dq = k.fit(px_dq);
    g.px_dp = k.fit(px_dp);
    g.px_d0 = k.fit(k.add(k.add(k.mul(k.mul(px_dq, st), cp), k.mul(k.mul(k.mul(px_dp, st), w), cp)),
                          k.mul(BK / pq, img)));
    g.px_d1 = k.fit(k.mul(k.sub(k.mul(st, w), k.mul(q, st)), cp));
    g.px_d2 = k.fit(k.sub(img, k.mul(k.mul(k.mul(p, st), w), cp)));
    g.px_nw = k.fit(BK / pq + 2);
    g.st_inv = k.fit((65536 + st - 1) / st);
    k.fit(img);
    k.fit(k.mul(pq, kp));
    k.fit(k.mul(k.mul(r, s), cp));
    k.fit(k.mul(k.mul(r, s), kp));
    g.ok = k.ok ? 1 : 0;
    return g;
}

bool conv_fits(const ConvGeom &g) {
    if (!g.ok) return false;
    if (g.r > 15 || g.s > 15 || g.h > 65535 || g.w > 65535 || g.cp > (1 << 22) || g.kp > (1 << 22)) return false;
    const long long pq = (long long)g.p * g.q, hw = (long long)g.h * g.w;
    const long long img_x = hw * g.cp, img_y = pq * g.kp;
    if ((256 / pq + 2) * img_x > WINDOW) return false;  // forward im2col rows, weight-gradient pixels
    if ((256 / hw + 2) * img_y > WINDOW) return false;  // input-gradient gather
    const long long rs = (long long)g.r * g.s;
    return 256 * rs * g.cp <= WINDOW && 256 * rs * g.kp <= WINDOW && 128ll * g.kp <= WINDOW;
}

bool weight_window_fits(const ConvGeom &g) { return (long long)g.kp * g.r * g.s * g.c <= WINDOW; }

// ---------------------------------------------------------------------------
// Stride phases of the input gradient
// ---------------------------------------------------------------------------

bool phases_apply(const ConvGeom &g) {
    if (!conv_fits(g) || g.stride != 2 || g.n <= 0) return false;
    // a phase's tile of at most 256 rows spans at most 256 / (hn wn) + 2
    // output images (as the whole convolution's does)
    const long long img_y = (long long)g.p * g.q * g.kp;
    for (int ph = 0; ph < 2; ++ph)
        for (int pw = 0; pw < 2; ++pw) {
            const long long hn = (g.h - ph + 1) / 2, wn = (g.w - pw + 1) / 2;
            if (hn * wn > 0 && (256 / (hn * wn) + 2) * img_y > WINDOW) return false;
        }
    return true;
}

Phases make_phases(const ConvGeom &g, int bm) {
    Phases ps;
    memset(&ps, 0, sizeof ps);
    if (!phases_apply(g) || bm <= 0) return ps;
    const int st = g.stride;
    ps.n = st * st;
    ps.st = st;
    ps.h = g.h;
    ps.w = g.w;
    int tap = 0, tiles = 0;  // tiles: the most tile rows of one phase
    for (int t = 0; t < ps.n; ++t) {
        PhaseRec &p = ps.r[t];
        p.ph = t / st;
        p.pw = t % st;
        p.hn = g.h > p.ph ? (g.h - p.ph + st - 1) / st : 0;
        p.wn = g.w > p.pw ? (g.w - p.pw + st - 1) / st : 0;
        const int r0 = (p.ph + g.pad) % st, s0 = (p.pw + g.pad) % st;
        p.ra = g.r > r0 ? (g.r - r0 + st - 1) / st : 0;
        p.sb = g.s > s0 ? (g.s - s0 + st - 1) / st : 0;
        p.ch = (p.ph + g.pad - r0) / st;
        p.cw = (p.pw + g.pad - s0) / st;
        const int sb = p.sb > 0 ? p.sb : 1;
        p.ds = (BK / g.kp) % sb;
        p.dr = (BK / g.kp) / sb;
        p.tap0 = tap;
        p.k0 = tap * g.kp;
        p.klen = p.ra * p.sb * g.kp;
        tap += p.ra * p.sb;
        p.rows = g.n * p.hn * p.wn;
        if (cdiv(p.rows, bm) > tiles) tiles = cdiv(p.rows, bm);
        p.dhw = make_fastdiv(p.hn * p.wn > 0 ? (uint32_t)(p.hn * p.wn) : 1u);
        p.dw = make_fastdiv(p.wn > 0 ? (uint32_t)p.wn : 1u);
        p.dsb = make_fastdiv((uint32_t)sb);
        if (p.klen > ps.kmax) ps.kmax = p.klen;
    }
    ps.tm = ps.n * tiles;
    return ps;
}

int phase_tap(const Phases &ps, const ConvGeom &g, int r, int s) {
    const int st = ps.st;
    const int ph = ((r - g.pad) % st + st) % st, pw = ((s - g.pad) % st + st) % st;
    const PhaseRec &p = ps.r[ph * st + pw];
    return p.tap0 + (r / st) * p.sb + s / st;
}

// ---------------------------------------------------------------------------
// Built tiles
// ---------------------------------------------------------------------------

bool tile_built(int family, Tile t, bool partial) {
#define IE_HAS(a, b) \
    if (t.mi == a && t.ni == b) return true;
    switch (family) {
        case FAM_DENSE:
            IE_TILES_DENSE(IE_HAS)
            return false;
        case FAM_IM2COL:
        case FAM_DGRAD:
        case FAM_DGRAD_WT:
            IE_TILES_CONV(IE_HAS)
            return false;
        case FAM_WGRAD:
        case FAM_WGRAD_CONV:
            if (!partial) return false;
            IE_TILES_WGRAD(IE_HAS)
            return false;
    }
#undef IE_HAS
    return false;
}

bool pair_tiles_built(Tile t1, Tile t2) {
#define IE_HAS(a, b, c, d) \
    if (t1.mi == a && t1.ni == b && t2.mi == c && t2.ni == d) return true;
    IE_TILES_PAIR(IE_HAS)
#undef IE_HAS
    return false;
}

// ---------------------------------------------------------------------------
// Plans
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

int chunk_for(long long K, int splits) {
    long long c = (K + splits - 1) / splits;
    c = (c + BK - 1) / BK * BK;
    return (int)(c > 0 ? c : BK);
}

Force force_from_env(const char *var, bool wgrad) {
    Force f{0, 0, 0, -1, 1};
    const char *v = getenv(var);
    if (!v || !*v) return f;
    int mi = 0, ni = 0, a = -1, b = 1;
    if (wgrad) {
        if (sscanf(v, "%d,%d,%d", &mi, &ni, &b) != 3) return f;
        a = PLAN_SPLIT;
    } else if (sscanf(v, "%d,%d,%d,%d", &mi, &ni, &a, &b) < 2) {
        return f;
    }
    f.on = 1;
    f.mi = mi;
    f.ni = ni;
    f.mode = a < 0 ? PLAN_RTO : a;
    f.splits = b;
    return f;
}

static Plan forced(const Force &f, long long K) {
    Plan p;
    p.t = Tile{f.mi, f.ni};
    p.mode = f.mode;
    const int sp = f.splits < 1 ? 1 : (f.splits > 4096 ? 4096 : f.splits);
    p.k_chunk = chunk_for(K, sp);
    p.splits = (int)((K + p.k_chunk - 1) / p.k_chunk);
    if (p.splits < 1) p.splits = 1;
    return p;
}

Plan plan_product(long long M, long long N, long long K, int row_group, int family, const Force &f) {
    if (f.on) return forced(f, K);
    auto tiles = [&](Tile t) { return (long long)cdiv(M, t.bm()) * cdiv(N, t.bn()); };
    // Rows of 129..256 results: the 64 x 256 tile holds a whole row group,
    // so its epilogue rounds straight to int8 in one pass.  Measured against
    // the plans below over row-grouped products (bit-identical results): it
    // wins while its tiles need at most two workgroups per CU (M up to
    // 32768; 25216 x 192 x 192: 18.9 vs 25.5 us, x 768: 25.7 vs 29.5 us;
    // 8192 x 192 x 768: 14.6 vs 20.2 us), and loses with more rows (one
    // workgroup per CU: 50432 x 192 x 576, 46.2 vs 40.6 us).  A few tiles
    // with a long contraction keep the split plan below.
    const bool few_long = tiles(Tile{1, 1}) < NCU / 2 && K >= 8 * BK;
    if (row_group && N > 128 && N <= 256 && !few_long && tile_built(family, Tile{1, 4}, false) &&
        tiles(Tile{1, 4}) <= 2ll * NCU)
        return Plan{Tile{1, 4}, PLAN_DIRECT, 1, chunk_for(K, 1)};
    // The 128 x 128 tile for outputs wider than 64 with at least 3/4 of a
    // tile per CU (its matrix work per LDS byte and per barrier is twice the
    // 128 x 64 tile's), else 128 x 64 with 1.5 tiles per CU, else 64 x 64: a
    // sweep of every built tile over the ResNet-50 and ResNet-18 forward and
    // input-gradient products (the smallest ResNet-18 layers, 2048 rows,
    // want the 64 x 64 tile's 512 workgroups).
    Tile t{1, 1};
    if (N > 64 && tiles(Tile{2, 2}) >= 3ll * NCU / 4) t = Tile{2, 2};
    else if (tiles(Tile{2, 1}) >= 3ll * NCU / 2) t = Tile{2, 1};
    const bool direct = row_group ? N <= t.bn() : tiles(t) == 1;
    // Recompute (two passes over the operands) or round to odd (one pass, an
    // int16 round trip of the output): row groups recompute contractions up
    // to RECOMP_KMAX; a whole-tensor result recomputes one-step contractions,
    // and two-step ones whose output is at least twice as wide as the
    // contraction (measured over ResNet-50's forward and input-gradient
    // products: elsewhere the second pass's matrix work outweighs the int16
    // round trip).
    const bool recomp = row_group ? K <= RECOMP_KMAX : K <= BK || (K <= 2 * BK && N >= 2 * K);
    Plan best{t, direct ? PLAN_DIRECT : recomp ? PLAN_RECOMP : PLAN_RTO, 1, chunk_for(K, 1)};
    if (!direct && few_long) {
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

DgradPlan plan_dgrad(const ConvGeom &g, int row_group, const Force &f, bool weight_in_place) {
    DgradPlan d;
    memset(&d, 0, sizeof d);
    d.M = (long long)g.n * g.h * g.w;
    d.K = (long long)g.r * g.s * g.kp;
    d.pl = plan_product(d.M, g.c, d.K, row_group, FAM_DGRAD, f);
    const bool want = f.on ? f.mode == PLAN_RECOMP : d.pl.mode != PLAN_DIRECT && !weight_in_place;
    if (row_group || !want || d.M == 0 || !phases_apply(g)) return d;
    d.ps = make_phases(g, d.pl.t.bm());
    if (d.ps.n == 0) return d;
    d.M = (long long)d.ps.tm * d.pl.t.bm();
    d.K = d.ps.kmax;
    d.pl = Plan{d.pl.t, PLAN_RECOMP, 1, chunk_for(d.K, 1)};
    return d;
}

Plan plan_wgrad(long long M, long long N, long long L, int family, const Force &f) {
    (void)family;
    if (f.on) {
        Plan p = forced(f, L);
        p.mode = PLAN_SPLIT;
        return p;
    }
    // The 128 x 128 tile whenever both sides fill it (16 matrix instructions
    // per wave and step, against 4 for the contraction-sliced 64 x 64 one),
    // and about one workgroup per CU in all (two per CU for more than four
    // 64 x 64 tiles): measured over ResNet-50's weight gradients, longer
    // contraction chunks beat a fuller grid, as the split partials (written,
    // then summed by the finalize) shrink with the split count.
    const bool big = M >= 128 && N >= 128;
    const Tile t = big ? Tile{2, 2} : Tile{1, 1};
    const long long nt = (long long)cdiv(M, t.bm()) * cdiv(N, t.bn());
    const long long target = big || nt <= 4 ? NCU : 2 * NCU;
    const int smin = (int)((L + SPLIT_MAX_ROWS - 1) / SPLIT_MAX_ROWS);
    long long want = (target + nt / 2) / nt;  // nearest split count to the target
    const long long smax = L / (8 * BK);      // chunks of at least eight steps
    if (want > smax) want = smax;
    if (want > 1024) want = 1024;
    int sp = want > 1 ? (int)want : 1;
    if (sp < smin) sp = smin;
    const int kc = chunk_for(L, sp);
    const int n = (int)((L + kc - 1) / kc);
    return Plan{t, PLAN_SPLIT, n > 0 ? n : 1, kc};
}

// Tiles built for the batched kernel: 128x128, 64x256, 128x64, 64x64 (the
// 64x256 one for A . B^T only).  A row group fits one tile (direct epilogue,
// no second pass) when N <= the tile width, so rows up to 256 wide take the
// 64x256 tile when there is work enough for it.
Plan plan_batched(long long Z, long long M, long long N, bool kk) {
    auto tiles = [&](Tile t) { return Z * cdiv(M, t.bm()) * cdiv(N, t.bn()); };
    Tile t{1, 1};
    if (kk && N > 128 && N <= 256 && tiles(Tile{1, 4}) >= 2ll * NCU) t = Tile{1, 4};
    else if (N > 64 && tiles(Tile{2, 2}) >= 2ll * NCU) t = Tile{2, 2};
    else if (tiles(Tile{2, 1}) >= 2ll * NCU) t = Tile{2, 1};
    return Plan{t, N <= t.bn() ? PLAN_DIRECT : PLAN_RTO, 1, BK};
}

int recomp_grid(long long M, long long N, long long K, Tile t) {
    const long long tiles = (long long)cdiv(M, t.bm()) * cdiv(N, t.bn());
    // workgroups per CU of the tile's kernel (its one-step form for K <= BK)
    const long long per_cu = K <= BK ? (t.mi * t.ni <= 2 ? 4 : t.mi * t.ni == 4 ? 3 : t.mi * t.ni <= 8 ? 2 : 1)
                                     : (t.mi * t.ni == 1 ? 3 : t.mi * t.ni <= 4 ? 2 : 1);
    long long g = NCU * per_cu;
    if (tiles < g) g = tiles;
    return (int)(g > 8 ? g / 8 * 8 : g);  // a multiple of 8: item % 8 stays the XCD
}

bool plan_valid(const Plan &pl, long long M, long long N, long long K, int row_group, int family) {
    if (pl.t.mi < 1 || pl.t.ni < 1) return false;
    if (pl.mode != PLAN_DIRECT && pl.mode != PLAN_RTO && pl.mode != PLAN_SPLIT && pl.mode != PLAN_RECOMP)
        return false;
    const bool wg = family == FAM_WGRAD || family == FAM_WGRAD_CONV;
    if (wg && pl.mode != PLAN_SPLIT) return false;
    if (!tile_built(family, pl.t, pl.mode == PLAN_SPLIT)) return false;
    if (pl.splits < 1 || pl.k_chunk <= 0 || pl.k_chunk % BK != 0) return false;
    if ((long long)pl.splits * pl.k_chunk < K) return false;
    if (pl.mode != PLAN_SPLIT && pl.splits != 1) return false;
    if (pl.mode == PLAN_SPLIT && pl.k_chunk > SPLIT_MAX_ROWS) return false;
    const long long tiles = (long long)cdiv(M, pl.t.bm()) * cdiv(N, pl.t.bn());
    if (tiles * pl.splits >= (1ll << 31)) return false;
    if (pl.mode == PLAN_DIRECT && (row_group ? N > pl.t.bn() : tiles > 1)) return false;
    return true;
}

bool plan_valid_batched(const Plan &pl, int form, long long M, long long N, long long K) {
    (void)M;
    const Tile t = pl.t;
    bool built = false;
    if (form == BMM_NT) {
        built = (t.mi == 2 && t.ni == 2) || (t.mi == 1 && t.ni == 4) || (t.mi == 2 && t.ni == 1) ||
                (t.mi == 1 && t.ni == 1);
    } else {
        built = (t.mi == 2 && t.ni == 2) || (t.mi == 2 && t.ni == 1) || (t.mi == 1 && t.ni == 1);
    }
    if (!built || pl.splits != 1 || pl.k_chunk != BK || K > MAX_CONTRACT) return false;
    if (pl.mode == PLAN_DIRECT) return N <= t.bn();
    return pl.mode == PLAN_RTO;
}

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------

// One split finalize block per row: 512 threads with up to 4 chunks each.
bool split_round_rows_fits(int Nout, int mc, int mcp) {
    const int vw = (mc == mcp && Nout % 4 == 0) ? 4 : 1;
    return Nout / vw <= SR_THR * SR_MAXV;
}

static size_t mx(size_t a, size_t b) { return a > b ? a : b; }

Needs product_needs(const Plan &pl, long long M, long long N, long long K, int row_group) {
    Needs n{0, 0, 0, 0, 0, 0};
    if (pl.t.mi < 1 || pl.t.ni < 1) return n;
    if (pl.mode == PLAN_RECOMP) {
        n.tneed = row_group ? (size_t)M * cdiv(N, pl.t.bn()) : (size_t)recomp_grid(M, N, K, pl.t);
    } else if (pl.mode == PLAN_RTO) {
        n.p16 = row_group ? (size_t)M * cdiv(N, pl.t.bn()) : (size_t)cdiv(M, pl.t.bm()) * cdiv(N, pl.t.bn());
        n.v16 = (size_t)M * N;
    } else if (pl.mode == PLAN_SPLIT) {
        n.partial = (size_t)pl.splits * M * N;
        if (!(row_group && split_round_rows_fits((int)N, 1, 1))) {
            n.sums = (size_t)M * N;
            n.gneed = row_group ? (size_t)M : 1;
        }
    }
    return n;
}

Needs wgrad_needs(const Plan &pl, long long N, long long Kg, long long Kout, int mc, int mcp, int row_group) {
    Needs n{0, 0, 0, 0, 0, 0};
    n.partial = (size_t)(pl.splits < 1 ? 1 : pl.splits) * N * Kg;
    n.gneed = row_group ? (size_t)N : 1;
    if (!(row_group && split_round_rows_fits((int)Kout, mc, mcp))) n.sums = (size_t)N * Kg;
    return n;
}

Needs batched_needs(const Plan &pl, long long Z, long long M, long long N) {
    Needs n{0, 0, 0, 0, 0, 0};
    if (pl.mode == PLAN_RTO && pl.t.ni >= 1) {
        n.p16 = (size_t)Z * M * cdiv(N, pl.t.bn());
        n.v16 = (size_t)Z * M * N;
    }
    return n;
}

bool covers(const Needs &have, const Needs &need) {
    return need.gneed <= have.gneed && need.p16 <= have.p16 && need.v16 <= have.v16 &&
           need.partial <= have.partial && need.sums <= have.sums && need.tneed <= have.tneed;
}

ProductWs carve_product(Carve &c, long long M, long long N, long long K, int family, const Force &f,
                        size_t tneed_min) {
    ProductWs w{};
    Needs n{0, 0, 0, 0, 0, tneed_min};
    for (int rg = 0; rg < 2; ++rg) {
        const Needs r = product_needs(plan_product(M, N, K, rg, family, f), M, N, K, rg);
        n.gneed = mx(n.gneed, r.gneed);
        n.p16 = mx(n.p16, r.p16);
        n.v16 = mx(n.v16, r.v16);
        n.partial = mx(n.partial, r.partial);
        n.sums = mx(n.sums, r.sums);
        n.tneed = mx(n.tneed, r.tneed);
    }
    n.gneed = mx(n.gneed, M > 0 ? (size_t)M : 1);
    w.gneed = c.take<int>(n.gneed);
    w.p16 = c.take<int16_t>(n.p16);
    w.v16 = c.take<int16_t>(n.v16);
    w.partial = c.take<int>(n.partial);
    w.sums = c.take<long long>(n.sums);
    w.tneed = c.take<int>(n.tneed);
    w.n = n;
    return w;
}

WgradWs carve_wgrad(Carve &c, long long N, long long Kg, long long L, int family, const Force &f) {
    WgradWs w{};
    const Plan pl = plan_wgrad(N, Kg, L, family, f);
    Needs n{0, 0, 0, 0, 0, 0};
    n.gneed = N > 0 ? (size_t)N : 1;
    n.partial = (size_t)(pl.splits < 1 ? 1 : pl.splits) * N * Kg;
    n.sums = (size_t)N * Kg;
    w.eps = c.take<int>(2);
    w.gneed = c.take<int>(n.gneed);
    w.partial = c.take<int>(n.partial);
    w.sums = c.take<long long>(n.sums);
    w.n = n;
    return w;
}

LinearFwdWs carve_linear_fwd(Carve &c, long long M, long long N, long long K, const Force &f) {
    LinearFwdWs w{};
    const long long Kp = r16(K);
    if (Kp != K) {
        w.xp = c.take<int8_t>((size_t)M * Kp);
        w.wp = c.take<int8_t>((size_t)N * Kp);
    }
    w.pw = carve_product(c, M, N, Kp, FAM_DENSE, f);
    return w;
}

LinearDxWs carve_linear_dx(Carve &c, long long M, long long N, long long K, const Force &f) {
    LinearDxWs w{};
    const long long Np = r16(N);
    w.estar = c.take<int>(1);
    w.wt = c.take<int8_t>((size_t)K * Np);
    if (Np != N) w.dyp = c.take<int8_t>((size_t)M * Np);
    w.pw = carve_product(c, M, K, Np, FAM_DENSE, f);
    return w;
}

LinearDwWs carve_linear_dw(Carve &c, long long M, long long N, long long K, const Force &fw) {
    LinearDwWs w{};
    w.dya = c.take<int8_t>((size_t)M * r16(N));
    w.xa = c.take<int8_t>((size_t)M * r16(K));
    w.w = carve_wgrad(c, N, K, M, FAM_WGRAD, fw);
    return w;
}

ConvFwdWs carve_conv_fwd(Carve &c, const ConvGeom &g, const Force &f) {
    ConvFwdWs w{};
    if (g.cp != g.c) {
        w.xp = c.take<int8_t>((size_t)g.n * g.h * g.w * g.cp);
        w.wp = c.take<int8_t>((size_t)g.k * g.r * g.s * g.cp);
    }
    w.pw = carve_product(c, (long long)g.n * g.p * g.q, g.k, (long long)g.r * g.s * g.cp, FAM_IM2COL, f);
    return w;
}

ConvBwdWs carve_conv_bwd(Carve &c, const ConvGeom &g, const Force &f, const Force &fw) {
    ConvBwdWs w{};
    const long long nhw = (long long)g.n * g.h * g.w, npq = (long long)g.n * g.p * g.q;
    w.estar = c.take<int>(1);
    w.wt = c.take<int8_t>((size_t)g.c * g.r * g.s * g.kp);
    if (g.kp != g.k) w.dyp = c.take<int8_t>((size_t)npq * g.kp);
    if (g.cp != g.c) w.xp = c.take<int8_t>((size_t)nhw * g.cp);
    const DgradPlan dp = plan_dgrad(g, 0, f);
    const size_t tn = dp.ps.n ? product_needs(dp.pl, dp.M, g.c, dp.K, 0).tneed : 0;
    w.pw = carve_product(c, nhw, g.c, (long long)g.r * g.s * g.kp, FAM_DGRAD, f, tn);
    w.w = carve_wgrad(c, g.k, (long long)g.r * g.s * g.cp, npq, FAM_WGRAD_CONV, fw);
    return w;
}

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
    // round-to-odd values and per-(row, column tile) needs, when the plan
    // rounds in two passes
    w.n = batched_needs(plan_batched(Z, M, N, form == BMM_NT), Z, M, N);
    if (w.n.p16) {
        w.p16 = c.take<int16_t>(w.n.p16);
        w.v16 = c.take<int16_t>(w.n.v16);
    }
    return w;
}

size_t linear_fwd_ws(long long M, long long N, long long K, const Force &f) {
    Carve c{nullptr, HEADER};
    carve_linear_fwd(c, M, N, K, f);
    return align256(c.off);
}

size_t linear_dx_ws(long long M, long long N, long long K, const Force &f) {
    Carve c{nullptr, HEADER};
    carve_linear_dx(c, M, N, K, f);
    return align256(c.off);
}

size_t linear_dw_ws(long long M, long long N, long long K, const Force &fw) {
    Carve c{nullptr, HEADER};
    carve_linear_dw(c, M, N, K, fw);
    return align256(c.off);
}

size_t conv_fwd_ws(const ConvGeom &g, const Force &f) {
    Carve c{nullptr, HEADER};
    carve_conv_fwd(c, g, f);
    return align256(c.off);
}

size_t conv_bwd_ws(const ConvGeom &g, const Force &f, const Force &fw) {
    Carve c{nullptr, HEADER};
    carve_conv_bwd(c, g, f, fw);
    return align256(c.off);
}

size_t bmm_ws(long long Z, long long M, long long N, long long K) {
    size_t best = HEADER;
    for (int form = 0; form < 3; ++form) {
        Carve c{nullptr, HEADER};
        carve_bmm(c, form, Z, M, N, K);
        best = mx(best, align256(c.off));
    }
    return best;
}

}  // namespace ie
