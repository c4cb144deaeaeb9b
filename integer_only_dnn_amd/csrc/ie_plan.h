// Host-side planning of the (C, e) library: argument checks, convolution
// geometry, the execution plan of every product (workgroup tile, epilogue,
// contraction split) and the layout of each entry point's workspace.
//
// Nothing here touches a GPU or includes HIP headers, so the same source is
// compiled into libie.so and, on its own, into a host-only checker built
// with address and undefined-behaviour sanitizers, which enumerates plans
// and proves that every buffer a plan's kernels write lies inside the
// workspace the size queries promise.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ie.h"

namespace ie {

constexpr int BK = 128;                        // contraction step of a workgroup tile (bytes)
constexpr int NCU = 256;                       // compute units of an MI355X
constexpr size_t HEADER = 256;                 // sticky flags at the start of every workspace
constexpr long long MAX_CONTRACT = 65536;      // |acc| < 2^30 for the fused epilogue
constexpr long long SPLIT_MAX_ROWS = 65536;    // exact int32 partial sums: |sum| <= 2^30
constexpr long long DIM_MAX = (1ll << 31) - 1;
// The GEMM loaders address operands through buffer descriptors of at most
// 2^30 bytes (a tile's images, a step's contraction rows) with 32-bit
// offsets, and keep filter-tap masks of 15 bits per axis.
constexpr long long WINDOW = 1ll << 30;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
inline long long r16(long long x) { return (x + 15) / 16 * 16; }

// n / d = (n * m) >> s for 0 <= n < 2^31 (m = ceil(2^s / d), s = 31 + ceil(log2 d)).
struct FastDiv {
    uint32_t m;
    int s;
};
FastDiv make_fastdiv(uint32_t d);

// Convolution geometry.  cp / kp: input / output channel counts as stored in
// the operands the kernels read (rounded up to multiples of 16 with zeros);
// dc divides by cp, dk by kp, dst by the stride.
struct ConvGeom {
    int n, h, w, c, k, r, s, stride, pad, p, q, cp, kp;
    FastDiv dpq, dq, dhw, dw, dc, ds, dk, dst;
    // Advance of the contraction index by one BK step, for the loaders:
    //   (r, s, c) over cp:  im_dc = BK % cp, im_ds = (BK / cp) % s, im_dr = BK / (cp s);
    //                       the tap offset (r w + s) cp + c moves by im_d0, plus im_d1
    //                       when s wraps;
    //   (r, s, ko) over kp: dg_dc, dg_ds, dg_dr likewise; ko r s c + (r s_ + s) c moves
    //                       by wt_d0, plus wt_d1 when ko wraps;
    //   output pixels:      px_dq = BK % q, px_dp = (BK / q) % p; the NHWC offset of
    //                       tap (0, 0) moves by px_d0, plus px_d1 when q wraps and px_d2
    //                       when p wraps; px_nw images cover any BK consecutive pixels;
    //   st_inv = ceil(2^16 / stride).
    int im_dc, im_ds, im_dr, im_d0, im_d1;
    int dg_dc, dg_ds, dg_dr, wt_d0, wt_d1;
    int px_dq, px_dp, px_d0, px_d1, px_d2, px_nw;
    int st_inv;
    int ok;  // every field fits its 32-bit integer
};

// Workgroup tile: 4 waves (2 x 2), each 32*mi x 32*ni; workgroup 64*mi x 64*ni.
struct Tile {
    int mi, ni;
    int bm() const { return 64 * mi; }
    int bn() const { return 64 * ni; }
};

// Stride phases of a strided convolution's input gradient.  The input pixels
// h = ph + st i, w = pw + st j (phase (ph, pw)) are reached only by the
// filter taps r = r0 + st a, s = s0 + st b with r0 = (ph + pad) % st,
// s0 = (pw + pad) % st, at output pixel p = i + ch - a, q = j + cw - b
// (ch = (ph + pad - r0) / st, cw likewise): each phase is a stride-1
// product over its own pixels and taps, and no tap that misses an output
// pixel reaches the matrix cores.  The weight copy the phases read holds the
// taps sorted by phase: phase t's taps (a, b), a < ra, b < sb, are the
// contraction columns k0 + (a sb + b) kp + ko, k0 = tap0 kp.
constexpr int PHASES_MAX = 4;  // stride 2
struct PhaseRec {
    int ph, pw;        // the phase's first input pixel
    int hn, wn;        // its pixels per image along h and w
    int ra, sb;        // its taps along r and s
    int ch, cw;        // output pixel of its tap (0, 0) relative to pixel (i, j)
    int ds, dr;        // advance of (a, b) per contraction step (b by ds, a by dr)
    int tap0;          // its first tap in the sorted weight copy
    int k0, klen;      // its contraction columns in that copy
    int rows;          // its GEMM rows (n hn wn)
    FastDiv dhw, dw, dsb;  // divide by hn wn, wn, sb
};
// Tile row t of the product is tile row t / 4 of phase (t + h(t / 4)) % 4,
// h(x) = (x * 2654435761 mod 2^32) / 2^30: the phases interleaved, rotated
// per group of four, so that every XCD's contiguous run of tiles and every
// persistent workgroup's strided walk mixes them; tile rows past a phase's
// own count are empty.
struct Phases {
    int n;             // phases (0: the product is not decomposed)
    int st, h, w;      // stride and input image size
    int tm;            // tile rows over all phases: n times the most of one phase
    int kmax;          // longest contraction of a phase
    PhaseRec r[PHASES_MAX];
};

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------

int n_exps(const ie_mat *t);
ie_status check_mat(const ie_mat *t);
// Mantissa width as q: a result of t has |C| <= 2^q - 1 (bits 0 reads as 8).
int mat_q(const ie_mat *t);
ie_status check_conv(const ie_conv_desc *d);
ConvGeom geom(const ie_conv_desc *d);
bool conv_fits(const ConvGeom &g);
// The in-place weight read of the input gradient spans the whole weight.
bool weight_window_fits(const ConvGeom &g);
// Whether the input gradient of g is decomposed into stride phases (stride
// 2 only), and the phases for workgroup tiles of bm rows.
bool phases_apply(const ConvGeom &g);
Phases make_phases(const ConvGeom &g, int bm);
// Position of tap (r, s) in the phase-sorted weight copy.
int phase_tap(const Phases &ps, const ConvGeom &g, int r, int s);

// ---------------------------------------------------------------------------
// Kernel families and the tiles instantiated for each (one list, used by the
// launchers and by plan validation).
// ---------------------------------------------------------------------------

enum Family {
    FAM_DENSE = 0,       // K-contiguous x K-contiguous (linear forward / input gradient)
    FAM_IM2COL = 1,      // convolution forward
    FAM_DGRAD = 2,       // convolution input gradient, aligned transposed weight
    FAM_DGRAD_WT = 3,    // convolution input gradient, weight read in place
    FAM_WGRAD = 4,       // M-contiguous x M-contiguous (linear weight gradient)
    FAM_WGRAD_CONV = 5,  // convolution weight gradient
};

#define IE_TILES_DENSE(X) X(2, 2) X(4, 1) X(1, 4) X(2, 1) X(1, 2) X(1, 1)
#define IE_TILES_CONV(X) X(2, 2) X(4, 1) X(2, 1) X(1, 1)
#define IE_TILES_WGRAD(X) X(2, 2) X(1, 4) X(4, 1) X(1, 1)
// Paired convolution backward: (input-gradient tile, weight-gradient tile).
#define IE_TILES_PAIR(X) X(2, 1, 1, 1) X(2, 1, 2, 2) X(1, 1, 1, 1) X(1, 1, 2, 2) X(2, 2, 1, 1) X(2, 2, 2, 2)

// Whether a kernel of `family` with tile t is built (split contractions:
// `partial`; the weight-gradient families exist only in that form).
bool tile_built(int family, Tile t, bool partial);
bool pair_tiles_built(Tile t1, Tile t2);

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

// DIRECT: every output group lies inside one workgroup tile.
// RTO:    round-to-odd int16 values at a provisional exponent + tile needs,
//         then a rounding pass.
// SPLIT:  the contraction is split into chunks of exact int32 partial sums,
//         merged and rounded by a finalize pass.
// RECOMP: two passes of the product: the first finds the group maxima only
//         (nothing stored), the second recomputes and rounds straight to int8.
//         Cheaper than RTO when the contraction is short (the extra pass
//         reads the operands again but saves 4 bytes per output element).
enum PlanMode { PLAN_DIRECT = 0, PLAN_RTO = 1, PLAN_SPLIT = 2, PLAN_RECOMP = 3 };

// Row-grouped results with contractions of at most this many bytes (one
// step) recompute instead of two-pass rounding (RECOMP instead of RTO);
// whole-tensor results choose by contraction and width (plan_product).
// Measured on row-grouped products whose rows span several 128-wide tiles,
// round to odd against recompute: 50432 x 576 x 192 59.0 vs 64.6 us,
// 50432 x 768 x 192 71.9 vs 78.6, 25216 x 3072 x 256 133.7 vs 160.9,
// 25216 x 3072 x 512 159.0 vs 205.5.
constexpr long long RECOMP_KMAX = 128;
// Workgroups of the first pass of a recomputed whole-tensor product (a
// persistent grid; each writes one maximum).
int recomp_grid(long long M, long long N, long long K, Tile t);

struct Plan {
    Tile t;
    int mode;
    int splits;
    int k_chunk;
};

int chunk_for(long long K, int splits);

// A forced plan (tests and tuning only): tile, mode and split count.  Read
// from the environment by the library (IE_TILE="mi,ni[,mode[,splits]]",
// IE_WTILE="mi,ni,splits"); every forced plan is validated like any other.
struct Force {
    int on;
    int mi, ni, mode, splits;
};
Force force_from_env(const char *var, bool wgrad);

// Product A(m, k) B(n, k) over K into an int8 output with one exponent per
// row (row_group) or one for the whole tensor.
Plan plan_product(long long M, long long N, long long K, int row_group, int family, const Force &f);
// Input gradient of a convolution: the product's plan and, for stride 2
// with one exponent for the whole result, its stride phases (then always
// the recomputed epilogue, whose second pass stores each phase pixel at its
// input pixel).  M and K are the row count and contraction the launches
// take: with phases, tile rows over all phases times the tile height, and
// the longest phase contraction.  The phases read a weight copy with the
// taps sorted by phase; when the weight could be read in place instead
// (weight_in_place), the planner keeps the undecomposed product, whose
// saved copy outweighs the masked taps at the shapes measured, unless a
// recomputed plan is forced.
struct DgradPlan {
    Plan pl;
    Phases ps;
    long long M, K;
};
DgradPlan plan_dgrad(const ConvGeom &g, int row_group, const Force &f, bool weight_in_place = false);
// Weight gradients: always split over the contraction, chunks of at most
// 65536 rows.
Plan plan_wgrad(long long M, long long N, long long L, int family, const Force &f);
// Batched products (always row groups): tile and epilogue.  kk: A . B^T.
Plan plan_batched(long long Z, long long M, long long N, bool kk);

// A plan is valid when its kernel is built, its chunks cover the contraction
// (exact int32 partials for splits), and a direct epilogue holds every group
// in one tile.
bool plan_valid(const Plan &pl, long long M, long long N, long long K, int row_group, int family);
enum BmmForm { BMM_NT = 0, BMM_NN = 1, BMM_TN = 2 };
bool plan_valid_batched(const Plan &pl, int form, long long M, long long N, long long K);

// ---------------------------------------------------------------------------
// Workspace layout.  A bump allocator over the caller's workspace (base
// nullptr: the size query), every buffer 256-byte aligned.
// ---------------------------------------------------------------------------

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

// Split finalize by rows: SR_THR threads per row with up to SR_MAXV chunks
// each (SR_THR_SHORT threads for rows of at most SR_THR chunks).
constexpr int SR_THR = 512;
constexpr int SR_THR_SHORT = 1024;
constexpr int SR_MAXV = 4;

// Element counts of the buffers a plan's kernels write besides the output.
struct Needs {
    size_t gneed, p16, v16, partial, sums, tneed;
};
bool split_round_rows_fits(int Nout, int mc, int mcp);
Needs product_needs(const Plan &pl, long long M, long long N, long long K, int row_group);
Needs wgrad_needs(const Plan &pl, long long N, long long Kg, long long Kout, int mc, int mcp, int row_group);
Needs batched_needs(const Plan &pl, long long Z, long long M, long long N);
bool covers(const Needs &have, const Needs &need);

// Epilogue workspace of a product: sized for both output group kinds.
struct ProductWs {
    int *gneed;
    int16_t *p16;
    int16_t *v16;
    int *partial;
    long long *sums;
    int *tneed;
    Needs n;  // element counts reserved
};
// tneed_min: entries the first pass of another plan of the same call needs
// (a stride-phased input gradient).
ProductWs carve_product(Carve &c, long long M, long long N, long long K, int family, const Force &f,
                        size_t tneed_min = 0);

struct WgradWs {
    int *partial;
    long long *sums;
    int *gneed;
    int *eps;  // [2]: common exponents of row-grouped operands
    Needs n;
};
// Weight gradient [N x Kg] contracted over L rows.
WgradWs carve_wgrad(Carve &c, long long N, long long Kg, long long L, int family, const Force &f);

// Whole layouts of the entry points (the size queries and the calls carve
// the same way).
struct LinearFwdWs {
    int8_t *xp, *wp;  // 16-byte padded copies (K not a multiple of 16)
    ProductWs pw;
};
LinearFwdWs carve_linear_fwd(Carve &c, long long M, long long N, long long K, const Force &f);

struct LinearDxWs {
    int *estar;   // W's common exponent
    int8_t *wt;   // W aligned and transposed [K x r16(N)]
    int8_t *dyp;  // padded dY (N not a multiple of 16)
    ProductWs pw;
};
LinearDxWs carve_linear_dx(Carve &c, long long M, long long N, long long K, const Force &f);

struct LinearDwWs {
    int8_t *dya, *xa;  // aligned / padded operands
    WgradWs w;
};
LinearDwWs carve_linear_dw(Carve &c, long long M, long long N, long long K, const Force &fw);

struct ConvFwdWs {
    int8_t *xp, *wp;
    ProductWs pw;
};
ConvFwdWs carve_conv_fwd(Carve &c, const ConvGeom &g, const Force &f);

struct ConvBwdWs {
    int *estar;
    int8_t *wt;   // aligned transposed weight [c][r][s][kp]
    int8_t *dyp;  // padded dY
    int8_t *xp;   // padded X
    ProductWs pw;
    WgradWs w;
};
ConvBwdWs carve_conv_bwd(Carve &c, const ConvGeom &g, const Force &f, const Force &fw);

struct BmmWs {
    int8_t *a, *b;  // padded / aligned operand copies
    int *ea, *eb;   // per-slice common exponents of aligned operands
    int16_t *p16, *v16;
    Needs n;
};
BmmWs carve_bmm(Carve &c, int form, long long Z, long long M, long long N, long long K);

size_t linear_fwd_ws(long long M, long long N, long long K, const Force &f);
size_t linear_dx_ws(long long M, long long N, long long K, const Force &f);
size_t linear_dw_ws(long long M, long long N, long long K, const Force &fw);
size_t conv_fwd_ws(const ConvGeom &g, const Force &f);
size_t conv_bwd_ws(const ConvGeom &g, const Force &f, const Force &fw);
size_t bmm_ws(long long Z, long long M, long long N, long long K);

}  // namespace ie
