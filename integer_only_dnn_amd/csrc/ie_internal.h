// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ie {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;

// Exponent of operand rows: per-row int8 array (row != 0), one int8 for the
// whole tensor (row == 0), or, when e32 is set, one int32 computed on the
// device (an aligned operand's common exponent).
struct ExpSrc {
    const int8_t *e8;
    const int *e32;
    int row;
};

enum EpiKind { EPI_DIRECT = 0, EPI_RTO = 1, EPI_PARTIAL = 2 };

struct Epi {
    ExpSrc ea;        // exponent of GEMM row m
    ExpSrc eb;        // exponent of GEMM column n
    int row_group;    // output groups: 1 = one per row m, 0 = whole tensor
    int8_t *out;      // EPI_DIRECT: int8 mantissas [M x N]
    int8_t *out_exp;  // EPI_DIRECT: exponents
    int16_t *v16;     // EPI_RTO: round-to-odd values [M x N]
    int16_t *p16;     // EPI_RTO: provisional exponent per (row, column tile)
    int n_ct;         // number of column tiles
    int *gneed;       // EPI_RTO: group maxima of the smallest exponents
    int *partial;     // EPI_PARTIAL: int32 [splits][M][N]
    long long split_stride;
    uint32_t *flags;
};

enum LoaderKind {
    LD_K = 0,         // element (i, k) at base[i*ld + k]
    LD_T = 1,         // element (i, k) at base[k*ld + i]
    LD_IM2COL = 2,    // convolution forward: rows = output pixels, k = (r, s, c)
    LD_DGRAD = 3,     // convolution input gradient: rows = input pixels, k = (r, s, k_out)
    LD_IM2COL_T = 4   // convolution weight gradient: rows = (r, s, c), k = output pixels
};

struct ConvGeom {
    int n, h, w, c, k, r, s, stride, pad, p, q;
};

struct Operand {
    int kind;
    const int8_t *base;
    long long ld;
    int rows;         // valid rows of this operand (GEMM M or N)
    int vec;          // aligned fast path allowed
    ConvGeom g;
};

// Launch C[m][n] = sum_k A(m, k) B(n, k) over k in [0, K) (split into
// `splits` chunks of `k_chunk`, a multiple of BK), then the epilogue.
hipError_t launch_gemm(const Operand &A, const Operand &B, int M, int N, int K,
                       int splits, int k_chunk, int epi, const Epi &ep, hipStream_t st);

// Optional kernel timing (ie_aux.hip): bracket a launch with HIP events.
void prof_begin(hipStream_t st);
void prof_end(hipStream_t st, int kind);
void prof_enable(int on);
int prof_read(float *ms, int *kind, int max);
constexpr int PROF_RTO_FINALIZE = 3000;
constexpr int PROF_DW_FINALIZE = 3100;
constexpr int PROF_ALIGN = 3200;

// Auxiliary kernels (ie_aux.hip).
hipError_t launch_fill_i32(int *p, long long n, int v, hipStream_t st);
hipError_t launch_fill_i8(int8_t *p, long long n, int v, hipStream_t st);
hipError_t launch_exp_max(const int8_t *e, long long n, int *out, hipStream_t st);
hipError_t launch_align_rows(const int8_t *in, const int8_t *e, const int *estar,
                             long long rows, long long cols, int8_t *out, hipStream_t st);
hipError_t launch_align_transpose(const int8_t *w, const int8_t *e, int e_row, const int *estar,
                                  int A, int B, int C, int8_t *out, hipStream_t st);
hipError_t launch_rto_finalize(const int16_t *v16, const int16_t *p16, const int *gneed,
                               int M, int N, int n_ct, int row_group, int8_t *out,
                               int8_t *out_exp, uint32_t *flags, hipStream_t st);
hipError_t launch_dw_finalize(const int *partial, int splits, long long split_stride, int N,
                              int K, const int *eps_a, const int *eps_b, int row_group,
                              int *gneed, int8_t *out, int8_t *out_exp, uint32_t *flags,
                              hipStream_t st);
hipError_t launch_zero_flags(void *ws, hipStream_t st);

// Integer SGD update (ie_update.hip).
struct UpdateArgs {
    int8_t *w, *w_exp;
    int8_t *v, *v_exp;
    const int8_t *g, *g_exp;
    int w_row, v_row, g_row;
    long long rows, cols;
    int lr_m, lr_e, mom_m, mom_e;
    int *gneed_v;      // [1] for a whole-tensor velocity group
    int *gneed_w;      // [1] for a whole-tensor weight group
    uint32_t *flags;
};
hipError_t launch_sgd_update(const UpdateArgs &a, hipStream_t st);

}  // namespace ie
