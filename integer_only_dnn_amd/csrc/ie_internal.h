// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ie_device.h"
#include "ie_plan.h"

namespace ie {

// Exponent of operand rows: per-row int8 array (row != 0), one int8 for the
// whole tensor (row == 0), or, when e32 is set, one int32 computed on the
// device (an aligned operand's common exponent).
struct ExpSrc {
    const int8_t *e8;
    const int *e32;
    int row;
};

#ifdef __HIPCC__
__device__ __forceinline__ int exp_at(const ExpSrc &e, int idx) {
    if (e.e32) return *e.e32;
    return e.row ? (int)e.e8[idx] : (int)e.e8[0];
}
#endif

// Epilogue modes of a contraction kernel.
//   DIRECT  - every result group lies inside the workgroup tile
//   RTO     - round-to-odd int16 values at a provisional exponent + group maxima
//   PARTIAL - exact int32 partial sums of one contraction chunk
//   MAX     - first pass of a recomputed product: group maxima only, no
//             values stored (whole tensor: one running maximum per workgroup
//             of a persistent grid; rows: one per (row, column tile))
//   GIVEN   - second pass: the product again, rounded straight to int8 at the
//             group exponents reduced from the first pass's maxima
enum EpiKind { EPI_DIRECT = 0, EPI_RTO = 1, EPI_PARTIAL = 2, EPI_MAX = 8, EPI_GIVEN = 9 };

struct Epi {
    ExpSrc ea;        // exponent of GEMM row m
    ExpSrc eb;        // exponent of GEMM column n
    int mode;         // EPI_DIRECT or EPI_RTO (PARTIAL is a template choice)
    int row_group;    // output groups: 1 = one per row m, 0 = whole tensor
    int8_t *out;      // DIRECT: int8 mantissas [M x N]
    int8_t *out_exp;  // DIRECT: exponents
    int16_t *v16;     // RTO: round-to-odd values [M x N]
    int16_t *p16;     // RTO: the tile's need per (row, column tile) or per tile
    int *gneed;       // PARTIAL: group maxima of the finalize, set empty here
    int gneed_n;      //   (count)
    int *partial;     // PARTIAL: int32 [splits][M][N]
    long long split_stride;
    uint32_t *flags;
    Act act;          // applied to the int8 results (fused ReLU or ReLU backward)
    int q;            // results have |C| <= 2^q - 1 (mantissa width q + 1 bits)
    int *tneed;       // MAX writes / GIVEN reads: group maxima of the first pass
    int tneed_n;      //   whole tensor: the first pass's grid size (entries)
    Phases ph;        // input gradient in stride phases (ph.n = 0: not decomposed);
                      //   rows are then phase pixels, stored at their input pixel
};

enum LoaderKind {
    LD_K = 0,         // element (i, k) at base[i*ld + k]
    LD_T = 1,         // element (i, k) at base[k*ld + i]
    LD_IM2COL = 2,    // convolution forward: rows = output pixels, k = (r, s, c)
    LD_DGRAD = 3,     // convolution input gradient: rows = input pixels, k = (r, s, k_out)
    LD_IM2COL_T = 4,  // convolution weight gradient: rows = (r, s, c), k = output pixels
    LD_WT = 5         // convolution input gradient, B side: rows = input channels c,
                      // k = (r, s, k_out) over kp; weight read in place [k_out][r][s][c]
};

struct Operand {
    int kind;
    const int8_t *base;
    long long ld;
    int rows;         // valid rows of this operand (GEMM M or N)
    ConvGeom g;
};

// C[m][n] = sum_k A(m, k) B(n, k) over k in [0, K), split into `splits`
// chunks of `k_chunk` (a multiple of BK), then the epilogue.
hipError_t launch_gemm(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                       int k_chunk, bool partial, const Epi &ep, hipStream_t st);
// ep.mode == EPI_MAX: the first pass of a recomputed product, on a persistent
// grid of recomp_grid(M, N, t) workgroups.
// Per-translation-unit launchers (return hipErrorInvalidValue if the
// loader / tile combination is not instantiated there).
hipError_t launch_gemm_kk(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                          int k_chunk, bool partial, const Epi &ep, hipStream_t st);
hipError_t launch_gemm_im2col(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                              int k_chunk, bool partial, const Epi &ep, hipStream_t st);
hipError_t launch_gemm_dgrad(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                             int k_chunk, bool partial, const Epi &ep, hipStream_t st);
hipError_t launch_gemm_dgrad_wt(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                                int k_chunk, bool partial, const Epi &ep, hipStream_t st);
hipError_t launch_gemm_wgrad(const Operand &A, const Operand &B, int M, int N, int K, Tile t, int splits,
                             int k_chunk, bool partial, const Epi &ep, hipStream_t st);
// Input gradient (LD_DGRAD x LD_WT, round-to-odd epilogue, tile t1) and weight
// gradient (LD_T x LD_IM2COL_T, split contraction, tile t2) in one grid.
// hipErrorInvalidValue when the combination has no kernel (nothing launched).
bool gemm_pair_supported(const Operand &A1, const Operand &B1, Tile t1, const Operand &A2, const Operand &B2,
                         Tile t2);
hipError_t launch_gemm_pair(const Operand &A1, const Operand &B1, int M1, int N1, int K1, Tile t1, int k_chunk1,
                            const Epi &ep1, const Operand &A2, const Operand &B2, int M2, int N2, int K2, Tile t2,
                            int splits2, int k_chunk2, const Epi &ep2, hipStream_t st);

// Batched products (ie_gemm_batched.hip): slice z of a stack reads A at
// A.base + z * a, B at B.base + z * b, exponents at e8 + z * e*8 or
// e32 + z * e*32, and writes its [M x N] result (row groups) at out +
// z * out (mantissas and round-to-odd values), out_exp + z * out_exp and
// p16 + z * p16.  mode: EPI_DIRECT (N within one tile) or EPI_RTO.
struct BatchArgs {
    long long a, b;
    long long ea8, eb8;
    int ea32, eb32;
    long long out, out_exp, p16;
    int Z;
};
hipError_t launch_gemm_batched(const Operand &A, const Operand &B, int M, int N, int K, Tile t, const Epi &ep,
                               const BatchArgs &ba, hipStream_t st);

// Optional kernel timing (ie_aux.hip): bracket a launch with HIP events.
void prof_begin(hipStream_t st, int kind);
void prof_end(hipStream_t st, int kind);
void prof_enable(int on);
void prof_select(int kind);
int prof_read(float *ms, int *kind, int max);
constexpr int PROF_RTO_FINALIZE = 3000;
constexpr int PROF_PARTIAL_REDUCE = 3100;
constexpr int PROF_ROUND_SUMS = 3150;
constexpr int PROF_ALIGN = 3200;
constexpr int PROF_ALIGN_Z = 3210;  // per-slice alignment of batched products
constexpr int PROF_SPLIT_ROUND = 3300;
constexpr int PROF_FIN_PAIR = 3400;
constexpr int PROF_RELU_FWD = 3500;
constexpr int PROF_RELU_BWD = 3510;
constexpr int PROF_ADD_NEED = 3520;
constexpr int PROF_ADD_ROUND = 3521;
constexpr int PROF_ADD_ROWS = 3530;

// Auxiliary kernels (ie_aux.hip).
hipError_t launch_fill_i32(int *p, long long n, int v, hipStream_t st);
hipError_t launch_fill_i8(int8_t *p, long long n, int v, hipStream_t st);
// out0[0] = max(e0[0..n0)), out1[0] = max(e1[0..n1)) (one launch; n1 may be 0).
hipError_t launch_exp_max2(const int8_t *e0, long long n0, int *out0, const int8_t *e1, long long n1, int *out1,
                           hipStream_t st);
// Copy rows into a zero-padded pitch, re-expressed at *estar when set.
hipError_t launch_pad_rows(const int8_t *in, long long rows, long long cols, const int8_t *e, int e_row,
                           const int *estar, long long cols_p, int8_t *out, hipStream_t st);
// Order of the filter taps b = r s_ + s in a transposed weight copy: as
// they come (st = 0), or sorted by stride phase (tap (r, s) of phase t =
// ph st + pw, ph = (r - pad) mod st, goes to tap0[t] + (r / st) sb[t] + s / st).
struct TapOrder {
    int st, pad, s;
    int tap0[PHASES_MAX], sb[PHASES_MAX];
};
// w viewed as [A][B][C] with row exponents e[a] (e_row) or e[0]:
// out[c][b'][a] = w[a][b][c] re-expressed at the largest row exponent, zero
// for A <= a < Ap, b' the position of b in the tap order; that exponent is
// also written to *estar_out.
hipError_t launch_align_transpose(const int8_t *w, const int8_t *e, int e_row, int A, int B, int C, int Ap,
                                  int8_t *out, int *estar_out, hipStream_t st, const TapOrder &to = TapOrder{});
// Second pass of the round-to-odd epilogue: the group exponent is the
// maximum of the tile needs in p16 (ROW groups: per (row, column tile);
// whole-tensor groups: per tile, tile_m + TM * tile_n).
hipError_t launch_rto_finalize(const int16_t *v16, const int16_t *p16, int M, int N, Tile t, int row_group,
                               int8_t *out, int8_t *out_exp, uint32_t *flags, hipStream_t st, Act act = Act{});
// Split-contraction finalize: sum int32 partials into int64 and raise the
// group maxima (set empty by the split kernel, or by launch_fill_i32 when no
// split kernel ran); then round the sums into int8.
hipError_t launch_partial_reduce(const int *partial, int splits, long long split_stride, int M, int N,
                                 ExpSrc ea, ExpSrc eb, int row_group, long long *sums, int *gneed, int q,
                                 hipStream_t st);
hipError_t launch_round_sums(const long long *sums, int M, int N, int src_pitch, int mc, int mcp, ExpSrc ea,
                             ExpSrc eb, int row_group, const int *gneed, int8_t *out, int8_t *out_exp,
                             uint32_t *flags, hipStream_t st, Act act = Act{});
// Split finalize of row groups in one pass (sums never stored): output
// [M x Nout] from partials [splits][M][src_pitch] with the column map of
// launch_round_sums.  Requires split_round_rows_fits(Nout, mc, mcp).
hipError_t launch_split_round_rows(const int *partial, int splits, long long split_stride, int M, int Nout,
                                   int src_pitch, int mc, int mcp, ExpSrc ea, ExpSrc eb, int8_t *out,
                                   int8_t *out_exp, uint32_t *flags, int q, hipStream_t st, Act act = Act{});
// A round-to-odd finalize (whole-tensor group, M1 x N1 from tile t1) and a
// split finalize by rows (the arguments of launch_split_round_rows) in one
// launch.
hipError_t launch_finalize_pair(const int16_t *v16, const int16_t *p16, int M1, int N1, Tile t1, int8_t *out1,
                                int8_t *out1_exp, const int *partial, int splits, long long split_stride, int M2,
                                int Nout, int src_pitch, int mc, int mcp, ExpSrc ea, ExpSrc eb, int8_t *out2,
                                int8_t *out2_exp, uint32_t *flags, int q2, hipStream_t st, Act act1 = Act{});
hipError_t launch_zero_flags(void *ws, hipStream_t st);

// Integer SGD update (ie_update.hip).
struct UpdateArgs {
    int8_t *w, *w_exp;
    int8_t *v, *v_exp;
    const int8_t *g, *g_exp;
    int w_row, v_row, g_row;
    long long rows, cols;
    int lr_m, lr_e, mom_m, mom_e;
    int wd_m, wd_e;    // weight decay (C, e); wd_m == 0: none
    int w_q;           // new weights have |C| <= 2^w_q - 1 (the velocity: 127)
    int *tmp;          // [UPD_WS_INTS]: exponent snapshots, per-block maxima
    uint32_t *flags;
};
constexpr int UPD_MAX_BLOCKS = 1024;  // grid of the update when a group spans the tensor
constexpr int UPD_WS_INTS = 2 + 2 * UPD_MAX_BLOCKS;
hipError_t launch_sgd_update(const UpdateArgs &a, hipStream_t st);
// The same for n tensors (each with its own tmp), in few launches.
hipError_t launch_sgd_update_multi(const UpdateArgs *a, int n, hipStream_t st);

// Pointwise steps (ie_pointwise.hip).  Whole-tensor sums keep one int per
// block in `bmax` (at most ADD_MAX_BLOCKS).
constexpr int ADD_MAX_BLOCKS = 1024;
// Batched alignment (reading R5 per slice): in [Z][R][cols] -> out
// [Z][R][cols_p] re-expressed at estar[z] (the slice's largest row exponent;
// e[0] when e_row is 0), zero past cols.
hipError_t launch_pad_rows_z(const int8_t *in, const int8_t *e, int e_row, int Z, int R, int cols, int cols_p,
                             int8_t *out, int *estar, hipStream_t st);

// relu6: the cap is min(6 * 2^-e, 2^q - 1) with q from the activation's width.
hipError_t launch_relu_fwd(const int8_t *x, const int8_t *xe, int x_row, int8_t *y, int8_t *ye, long long rows,
                           long long cols, int relu6, int q, hipStream_t st);
hipError_t launch_relu_bwd(const int8_t *dy, const int8_t *dye, int dy_row, const int8_t *yc, const int8_t *ye,
                           int y_row, int8_t *dx, int8_t *dxe, long long rows, long long cols, int relu6, int q,
                           hipStream_t st);
hipError_t launch_add(const int8_t *a, const int8_t *ae, int a_row, const int8_t *b, const int8_t *be, int b_row,
                      int8_t *z, int8_t *ze, int z_row, long long rows, long long cols, int *bmax, uint32_t *flags,
                      int q, hipStream_t st);

}  // namespace ie
