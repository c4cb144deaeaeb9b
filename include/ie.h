/*
 * ie.h - C ABI of the integer-only (C, e) layer-step library for MI355X (gfx950).
 *
 * Every tensor is a pair (C, e): signed INT8 mantissas C and signed INT8
 * power-of-two exponents e, value C * 2^e ("Memory-Efficient Integer-Only
 * Training of Deep Neural Networks", Abstract and Figure 1).  An exponent is
 * shared by a group: the whole tensor (IE_GROUP_TENSOR) or one leading-index
 * row (IE_GROUP_ROW: a token / pixel row of an activation, an output channel of
 * a weight [N x K]; Table 5 gives one exponent byte per output channel).
 *
 * Arithmetic contract (identical for every entry point):
 *   - products are exact int8 x int8 sums, exponent e_a + e_b (Table 6,
 *     "Product"); every stored result is rounded exactly once from the exact
 *     value, right shifts rounding half to even;
 *   - a result group's exponent is the smallest e with all |C| <= 127, or
 *     -128 if the group is all zero or smaller; mantissas -128 are accepted on
 *     input and never produced;
 *   - an operand whose exponent varies along a contraction axis is first
 *     re-expressed at the largest exponent on that axis (same rounding);
 *   - an exponent above 127 sets IE_FLAG_EXP_RANGE in the workspace's sticky
 *     flags (read with ie_device_status); that output's values are undefined.
 *
 * Memory and execution:
 *   - every mantissa/exponent/workspace pointer is a DEVICE pointer owned by
 *     the caller; the library allocates no device memory, creates no stream
 *     or event (the optional kernel timing below aside) and keeps no global
 *     state apart from that timing;
 *   - matrices are row-major and contiguous; activations of convolutions are
 *     NHWC, viewed as a matrix [N*H*W x C]; weights are [K x R*S*C] (KRSC);
 *   - outputs are fully overwritten, mantissas and exponents; outputs must not
 *     alias inputs (ie_sgd_update works in place on W and V);
 *   - `ws` is a workspace of at least the size the matching *_workspace_bytes
 *     call returns; its first 256 bytes hold sticky flags and must be zeroed
 *     once (ie_workspace_init) before first use;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     runs asynchronously; calls sharing one workspace must be ordered on one
 *     stream;
 *   - argument errors are detected on the host and returned before anything
 *     is enqueued; launch failures return IE_ERR_HIP;
 *   - each product's execution plan (workgroup tile, epilogue, contraction
 *     split) is chosen from its shape.  For tests and tuning only, the
 *     environment variables IE_TILE="mi,ni[,mode[,splits]]" and
 *     IE_WTILE="mi,ni,splits" force the plans of products and of weight
 *     gradients; a forced plan without a built kernel, or one whose direct
 *     epilogue would split a group across workgroups, returns
 *     IE_ERR_UNSUPPORTED before anything is enqueued (as does any plan whose
 *     buffers the carved workspace does not hold).
 */
#ifndef IE_H
#define IE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IE_OK = 0,
    IE_ERR_NULL = 1,        /* a required pointer is NULL */
    IE_ERR_SHAPE = 2,       /* shapes do not agree or are negative */
    IE_ERR_GROUP = 3,       /* unknown group kind */
    IE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
    IE_ERR_EXP_RANGE = 5,   /* reported by ie_device_status callers */
    IE_ERR_UNSUPPORTED = 6, /* valid but outside what this library supports */
    IE_ERR_HIP = 7,         /* a HIP runtime call failed */
    IE_ERR_BITS = 8,        /* ie_mat.bits outside {0, 2..8}, or a velocity not INT8 */
    IE_ERR_SCRATCH = 9      /* the call needs more than the fixed scratch of ie_linear_fwd_noalloc */
} ie_status;

typedef enum { IE_GROUP_TENSOR = 0, IE_GROUP_ROW = 1 } ie_group;

#define IE_FLAG_EXP_RANGE 1u

/* A (C, e) matrix.  mant: rows*cols bytes, row-major.  exp: 1 byte (TENSOR)
 * or `rows` bytes (ROW).
 * bits: the mantissa width B ("Memory-Efficient Integer-Only Training of Deep
 * Neural Networks", Table 4: INT8 down to INT4), 2..8, with 0 read as 8.
 * Every step that rounds into this matrix rounds to |C| <= 2^(B-1) - 1
 * (its group exponent is the smallest that fits), and ReLU6's cap on an
 * activation is at most 2^(B-1) - 1.  Mantissas are stored one per byte
 * whatever B is, and inputs are read as the bytes they hold, so B matters
 * only on outputs and on ReLU6's activation.  The velocity of
 * ie_sgd_update must be INT8 (0 or 8). */
typedef struct {
    int8_t *mant;
    int8_t *exp;
    int64_t rows;
    int64_t cols;
    int32_t group;
    int32_t bits;
} ie_mat;

/* Convolution shape: input NHWC [n, h, w, c], weight [k, r, s, c], zero
 * padding `pad` on every side, equal strides; output [n, p, q, k] with
 * p = (h + 2 pad - r) / stride + 1, q = (w + 2 pad - s) / stride + 1. */
typedef struct {
    int32_t n, h, w, c, k, r, s, stride, pad;
} ie_conv_desc;

/* A (C, e) scalar (learning rate, momentum, weight decay): value mant * 2^exp. */
typedef struct {
    int8_t mant;
    int8_t exp;
} ie_scalar;

/* Workspace sizes (bytes) for one call of the matching entry point. */
size_t ie_linear_fwd_workspace(int64_t M, int64_t N, int64_t K);
size_t ie_linear_bwd_dx_workspace(int64_t M, int64_t N, int64_t K);
size_t ie_linear_bwd_dw_workspace(int64_t M, int64_t N, int64_t K);
size_t ie_conv_fwd_workspace(const ie_conv_desc *d);
size_t ie_conv_bwd_workspace(const ie_conv_desc *d);
size_t ie_sgd_update_workspace(int64_t rows, int64_t cols);
size_t ie_sgd_update_multi_workspace(int32_t n);

/* Zero the workspace's sticky flags (enqueued on `stream`). */
ie_status ie_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * Forward product of a linear layer, Y = X . W^T (Table 6 "Linear /
 * fully-connected -> Product"; Figure 1a).
 *   X [M x K], W [N x K], Y [M x N]; groups: X, W, Y each TENSOR or ROW.
 *   Contraction limit: K <= 65536.
 */
ie_status ie_linear_fwd(const ie_mat *X, const ie_mat *W, const ie_mat *Y,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * ie_linear_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * There is no workspace argument: the call uses a fixed scratch array of
 * IE_NOALLOC_SCRATCH_BYTES that the library keeps in device memory (one copy
 * per GPU, held until the process ends, its address looked up on the first
 * call on each device), and calls no allocating routine.  Results, limits and
 * errors are those of ie_linear_fwd, plus IE_ERR_SCRATCH (nothing enqueued)
 * when the shape needs more scratch than that (ie_linear_fwd_workspace(M, N,
 * K) > IE_NOALLOC_SCRATCH_BYTES).  flags: a device word into which the
 * exponent-range flag (IE_FLAG_EXP_RANGE) is ORed, or NULL to drop it.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind (nothing in it needs to start at any value): calls that may overlap
 * on one GPU (different streams, different host threads) race and must be
 * ordered by the caller.
 */
#define IE_NOALLOC_SCRATCH_BYTES (64u << 20)
ie_status ie_linear_fwd_noalloc(const ie_mat *X, const ie_mat *W, const ie_mat *Y,
                                uint32_t *flags, void *stream);

/*
 * Input gradient of a linear layer, dX = dY . W (Figure 1a, backward).
 *   dY [M x N], W [N x K], dX [M x K].  A ROW-grouped W is aligned over its
 *   rows (the contraction axis) first.  N <= 65536.
 */
ie_status ie_linear_bwd_dx(const ie_mat *dY, const ie_mat *W, const ie_mat *dX,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Weight gradient of a linear layer, dW = dY^T . X (Figure 1a, backward;
 * Table 5 groups: ROW = per output channel).
 *   dY [M x N], X [M x K], dW [N x K].  ROW-grouped dY or X are aligned over
 *   their rows (the contraction axis) first.  Any M (exact int32 partial sums
 *   over chunks of at most 65536 rows, merged in int64).  N and K up to 2^23
 *   (IE_ERR_UNSUPPORTED beyond: 128 rows of either operand must fit in 2^30
 *   bytes).
 */
ie_status ie_linear_bwd_dw(const ie_mat *dY, const ie_mat *X, const ie_mat *dW,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Forward convolution (Table 6 "Convolution -> Product"), implicit GEMM:
 *   Y[n,p,q,k] = sum_{r,s,c} X[n, p*st+r-pad, q*st+s-pad, c] * W[k,r,s,c].
 *   X: rows n*h*w, cols c, TENSOR.  W: rows k, cols r*s*c, TENSOR or ROW.
 *   Y: rows n*p*q, cols k, TENSOR.  r*s*c <= 65536.
 * Convolution limits (both directions; IE_ERR_UNSUPPORTED beyond): r, s <= 15;
 * h, w <= 65535; c, k <= 2^22; the images a tile of 256 output (or input)
 * pixels spans must fit in 2^30 bytes, and so must 256 rows of the weight.
 */
ie_status ie_conv_fwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W,
                      const ie_mat *Y, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward convolution ("Memory-Efficient Integer-Only Training of Deep
 * Neural Networks", Figure 1a: the backward pass of every layer; Table 6:
 * "Convolution -> Product"): the input gradient dX, the exact adjoint of
 * ie_conv_fwd in X (W aligned over its output channels first when
 * ROW-grouped), and the weight gradient dW, its adjoint in W (one exponent
 * per output channel when ROW, Table 5).  dX or dW may be NULL to skip that
 * output.  X, dY: TENSOR; dX: TENSOR, or ROW (one exponent per input
 * pixel); W, dW: TENSOR or ROW.
 * A stride-2 input gradient with one exponent is computed in stride phases
 * (each input pixel only meets the filter taps of its phase), so no tap that
 * misses an output pixel is multiplied.
 * With both outputs requested the two products run as one grid where a
 * paired kernel covers their plans (whole-tensor input gradient, row-grouped
 * weight gradient), else one after the other; all work is enqueued on
 * `stream`, and the library creates no stream or event of its own.
 * Limits as for ie_conv_fwd, with the contraction k*r*s <= 65536.
 */
ie_status ie_conv_bwd(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W,
                      const ie_mat *dY, const ie_mat *dX, const ie_mat *dW,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * Integer SGD with momentum and per-group velocity (Figure 1b; Table 5),
 * in place on W and V:
 *   V <- R_V(momentum * V + G + weight_decay * W),  W <- R_W(W - lr * V)
 * where R_x requantises into x's groups, the velocity sum is exact (the
 * decay term uses W before the step; Table 10 lists weight decay 1e-4, e.g.
 * (1, -13)), and the weight step uses the stored, rounded V.  W, V, G:
 * [rows x cols], each TENSOR or ROW.  weight_decay.mant == 0: no decay term.
 * W' rounds to W's mantissa width (W->bits); V is always INT8 (Table 4's
 * B-bit variants keep the velocity INT8), else IE_ERR_BITS.
 */
ie_status ie_sgd_update(const ie_mat *W, const ie_mat *V, const ie_mat *G,
                        ie_scalar lr, ie_scalar momentum, ie_scalar weight_decay,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * The same update for n independent (W[i], V[i], G[i]) triples (arrays of
 * n ie_mat each), e.g. every layer of a network in one optimiser step, with
 * one set of scalars.  The result equals n calls of ie_sgd_update; tensors
 * of similar row length share kernel launches (one per pass).  Every triple
 * is checked before anything is enqueued.  n >= 0.
 */
ie_status ie_sgd_update_multi(int32_t n, const ie_mat *W, const ie_mat *V, const ie_mat *G,
                              ie_scalar lr, ie_scalar momentum, ie_scalar weight_decay,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * Forward products with the activation fused into their output (Table 7:
 * the clip acts on the rounded mantissas, the exponents are those of the
 * plain product).  act: IE_ACT_NONE (same as ie_linear_fwd / ie_conv_fwd) or
 * IE_ACT_RELU; other values return IE_ERR_UNSUPPORTED.  Arguments, limits
 * and workspace sizes as for the plain entry points.
 */
#define IE_ACT_NONE 0
#define IE_ACT_RELU 1
ie_status ie_linear_fwd_act(const ie_mat *X, const ie_mat *W, const ie_mat *Y, int act,
                            void *ws, size_t ws_bytes, void *stream);
ie_status ie_conv_fwd_act(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W,
                          const ie_mat *Y, int act, void *ws, size_t ws_bytes, void *stream);

/*
 * Input gradients passed back through the activation that produced the
 * layer's input (Table 7, the ReLU backward fused into the product's
 * output).  With act = IE_ACT_RELU, X is that activation's output and
 *   dX.C = (the plain input gradient's C) where X.C > 0, else 0,
 *   dX.exp = the plain input gradient's exponents,
 * i.e. exactly ie_conv_bwd / ie_linear_bwd_dx followed by ie_relu_bwd(dX, X)
 * (relu6 = 0), in one pass over dX.  The weight gradient of ie_conv_bwd_act
 * is that of ie_conv_bwd (it does not depend on the activation).
 * act = IE_ACT_NONE: the plain entry points; other values return
 * IE_ERR_UNSUPPORTED.  ie_linear_bwd_dx_act: X [M x K] is read only for the
 * mask (any group, shape of dX, else IE_ERR_SHAPE).  dX must not be X
 * (IE_ERR_UNSUPPORTED).  Other arguments, limits and workspace sizes as for
 * the plain entry points.
 */
ie_status ie_linear_bwd_dx_act(const ie_mat *dY, const ie_mat *W, const ie_mat *X, const ie_mat *dX, int act,
                               void *ws, size_t ws_bytes, void *stream);
ie_status ie_conv_bwd_act(const ie_conv_desc *d, const ie_mat *X, const ie_mat *W, const ie_mat *dY,
                          const ie_mat *dX, const ie_mat *dW, int act, void *ws, size_t ws_bytes, void *stream);

/*
 * ReLU and ReLU6 of a (C, e) tensor (Table 7, "Clip activations"), on the
 * mantissas; the exponents are copied:
 *   relu:  Y.C = max(X.C, 0)
 *   relu6: Y.C = min(max(X.C, 0), c6),  c6 = min(floor(6 * 2^-e), 2^(B-1) - 1)
 * with e the element's group exponent (6 expressed in the group's units) and
 * B the width of Y.  X, Y: same shape and group.  Y may be X (in place).
 * relu6: 0 or 1.
 */
ie_status ie_relu_fwd(const ie_mat *X, const ie_mat *Y, int relu6, void *stream);

/*
 * Backward of ie_relu_fwd (Table 7): dX.C = dY.C where the forward output
 * Y.C > 0 (and Y.C < c6 of Y's group and width for relu6), else 0;
 * dX.exp = dY.exp.
 * dY, Y, dX: same shape; dX has dY's group.  dX may be dY (in place).
 */
ie_status ie_relu_bwd(const ie_mat *dY, const ie_mat *Y, const ie_mat *dX, int relu6, void *stream);

/*
 * Sum (Table 6, "Residual add, gradient merge -> Sum"): Z = R_Z(A + B), the
 * exact elementwise sum rounded once into Z's groups.  A, B, Z: same shape,
 * each TENSOR or ROW.  Z must not alias A or B.
 */
size_t ie_add_workspace(int64_t rows, int64_t cols);
ie_status ie_add(const ie_mat *A, const ie_mat *B, const ie_mat *Z, void *ws, size_t ws_bytes, void *stream);

/*
 * Batched products: one independent Product (Table 6: the same primitive as
 * the linear layer) per slice z of stacked operands, e.g. a ViT's attention
 * per (image, head) with batch = images * heads:
 *   ie_bmm_nt: C_z = A_z . B_z^T   A [batch*M x K], B [batch*N x K]
 *              (scores Q.K^T; dP = dO.V^T)
 *   ie_bmm_nn: C_z = A_z . B_z     A [batch*M x K], B [batch*K x N]
 *              (context P.V; dQ = dS.K)
 *   ie_bmm_tn: C_z = A_z^T . B_z   A [batch*K x M], B [batch*K x N]
 *              (dK = dS^T.Q; dV = P^T.dO)
 * C [batch*M x N]; slice z of a stack is its rows z*rows .. (z+1)*rows - 1.
 * Operands may be TENSOR (one exponent for the stack) or ROW (one per row).
 * An operand contracted over its rows (B of nn, A and B of tn) that is
 * ROW-grouped is first re-expressed, slice by slice, at the largest of that
 * slice's row exponents (round half to even), as the linear input and
 * weight gradients do.  Sums are exact (contraction K <= 65536); C must be
 * ROW (one exponent per row of every slice), else IE_ERR_UNSUPPORTED; it is
 * rounded to C->bits.  batch >= 1 (0: every stack empty), batch <= 65535,
 * and every stack's rows a multiple of batch, else IE_ERR_SHAPE.  A and B of
 * nt (A of nn) with K a multiple of 16 must be 16-byte aligned.  Workspace:
 * ie_bmm_workspace(batch, M, N, K) bytes, the same for all three forms.
 */
size_t ie_bmm_workspace(int32_t batch, int64_t M, int64_t N, int64_t K);
ie_status ie_bmm_nt(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C,
                    void *ws, size_t ws_bytes, void *stream);
ie_status ie_bmm_nn(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C,
                    void *ws, size_t ws_bytes, void *stream);
ie_status ie_bmm_tn(int32_t batch, const ie_mat *A, const ie_mat *B, const ie_mat *C,
                    void *ws, size_t ws_bytes, void *stream);

/* Wait for `stream`, then copy the workspace's sticky flags to *flags and,
 * if clear != 0, zero them. */
ie_status ie_device_status(void *ws, void *stream, uint32_t *flags, int clear);

/*
 * Kernel timing, for diagnostics and benchmarks.  While enabled, the launch
 * of every contraction, finalize and update kernel (or, after
 * ie_profile_select(kind) with kind != 0, of the kernels of that kind only)
 * is bracketed by two HIP events recorded on the launch's stream.  ie_profile_read waits for the
 * recorded events, writes up to `max` records in launch order (elapsed
 * milliseconds and a kernel-kind code: 10000*(10*mi + ni) + 1000 +
 * 100*epilogue + 10*loader_A + loader_B for contractions with a
 * (64 mi) x (64 ni) tile (epilogue 0 direct, 1 round-to-odd, 2 split, 3 the
 * paired convolution backward, 4 / 5 batched direct / round-to-odd, 6 / 7
 * the same with a one-step contraction),
 * 2000 + pass for the update, 3000 round-to-odd
 * finalize, 3100 split-sum reduction, 3150 rounding of sums, 3200 padding /
 * alignment copies, 3210 the per-slice alignment copies of batched products,
 * 3300 split rounding by rows, 3400 the paired finalize of
 * a convolution's backward pass, 3500 / 3510 ReLU forward / backward, 3520 /
 * 3521 / 3530 the Sum's maximum, rounding and row-grouped passes) and returns how
 * many were recorded since the last read; the records are then cleared.
 * The timing records (and their events) are the library's only process-wide
 * state; they are not thread-safe.
 */
ie_status ie_profile_enable(int on);
ie_status ie_profile_select(int kind);
int ie_profile_read(float *ms, int *kind, int max);

/* Human-readable name of a status code. */
const char *ie_status_str(ie_status st);

#ifdef __cplusplus
}
#endif

#endif /* IE_H */
