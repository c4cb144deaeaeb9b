// int8 x int8 -> int32 contraction on CDNA4 MFMA with a fused (C, e)
// requantisation epilogue.
//
// Implements the "Product" building block ("Memory-Efficient Integer-Only
// Training of Deep Neural Networks", Table 6: convolution, linear; Figure 1a:
// forward and backward of every layer): acc = sum_k A(m,k) B(n,k) exactly in
// int32, exponent eps = e_A(m) + e_B(n); a result group's exponent is the
// smallest that brings every |C| to 127 or less (ties to even).
//
// A workgroup of 4 waves (2 x 2) computes a (64 MI) x (64 NI) tile with
// v_mfma_i32_32x32x32_i8; each wave owns (32 MI) x (32 NI).  Operand tiles
// of BK (128) contraction bytes are staged through LDS, double buffered, with
// the next steps' buffer loads in flight during the current step's MFMAs.
//   - K-contiguous operands sit in LDS as [row][k] (16-byte pad) and are
//     read with ds_read_b128;
//   - M-contiguous operands (weight gradients) sit as [k][row] (16-byte
//     pad), written straight from coalesced 16-byte global loads, and are
//     transposed on the way out with two ds_read_b64_tr_b8 per fragment:
//     within each 16-lane group, lanes 2j and 2j+1 name the two halves of
//     row j of an 8 x 16 byte block and lane i receives its column i.
// Convolutions are implicit GEMMs: the loaders compute NHWC addresses of the
// im2col view (forward), of the input-gradient gather and of the transposed
// im2col view (weight gradient) on the fly, stepping offsets incrementally;
// zero padding loads zeros.
#pragma once

#ifndef IE_STAGES
#define IE_STAGES 4
#endif
#ifndef IE_UNROLL
#define IE_UNROLL 4
#endif
// Tuning knobs (compile time).  IE_PIPE 0 keeps the fragment reads inside
// each sub-step (measured 0.3 % slower on the ResNet-50 step).  The 128 x 128
// tile's register pipeline depth and workgroups per CU: four stages measured
// the same as three at long contractions and up to 6 % slower at short ones;
// one workgroup per CU with six stages 20-75 % slower (25216 x 3072 x K
// products, K = 6144 ... 256).
#ifndef IE_PIPE
#define IE_PIPE 1
#endif
#ifndef IE_STAGES22
#define IE_STAGES22 3
#endif
#ifndef IE_OCC22
#define IE_OCC22 2
#endif

#include <type_traits>

#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

constexpr int NTHR = 256;
// Row padding of a [k][row] LDS tile (bytes): 32 for 64-row tiles, whose
// bank conflicts it removes; 16 for wider ones, which would not fit two
// workgroups per CU with 32.
template <int ROWS>
struct TPad {
    static constexpr int value = ROWS <= 64 ? 32 : 16;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

__device__ __forceinline__ void put_byte(uint32_t *w, int b, int8_t v) {
    w[b >> 2] |= (uint32_t)(uint8_t)v << (8 * (b & 3));
}

__device__ __forceinline__ v4i pack16(const uint32_t *w) { return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]}; }

template <int KIND>
struct IsT {
    static constexpr bool value = KIND == LD_T || KIND == LD_IM2COL_T || KIND == LD_WT;
};

// LDS tile of an operand with ROWS rows (GEMM M or N side).  [row][k] tiles
// pad each row by 16 bytes, [k][row] tiles by TPad.
template <int KIND, int ROWS>
struct Lds {
    static constexpr bool T = IsT<KIND>::value;
    static constexpr int STRIDE = T ? ROWS + TPad<ROWS>::value : BK + 16;
    static constexpr int BYTES = T ? BK * STRIDE : ROWS * STRIDE;
};

// ---------------------------------------------------------------------------
// Loaders.  Every operand is read in 16-byte chunks (the host pads channel
// and contraction extents to multiples of 16) with raw buffer loads: the
// workgroup builds a buffer descriptor over the window of the operand it
// reads, and a chunk whose 32-bit offset lies at or past the window's end
// loads zeros in hardware.  Invalid chunks (padding taps, rows past the
// operand, contraction past the end) are given such an offset, so loads are
// unconditional, never fault, and no loaded register is touched before its
// stage is written to LDS.  Offsets advance from step to step by constants
// the host precomputes: the main loop holds no divisions.
//
// Windows hold at most 2^30 bytes, so a valid offset plus OOB_ROW (2^30) or
// OOB_K (2^31), or both, lies past every window.
//
// Only one operand of a product zeroes the contraction past its end (ZK);
// the other one's chunks there meet zeros, so they need only be safe to
// read, which the descriptor guarantees.  Each thread moves
// ROWS * BK / 4096 chunks per contraction step.
// ---------------------------------------------------------------------------

constexpr uint32_t OOB_ROW = 1u << 30, OOB_K = 1u << 31;

typedef __amdgpu_buffer_rsrc_t Res;

// Descriptor of `bytes` bytes at p (none when bytes <= 0; the host keeps
// every window within 2^30 bytes).  Raw buffer, no stride, 32-bit data format.
// p and bytes are the same in every lane (window bases and sizes derive from
// the workgroup's tile and step only); reading them from the first lane lets
// the descriptor live in scalar registers, as a buffer load needs.
__device__ __forceinline__ Res make_res(const int8_t *p, int bytes) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane(max(bytes, 0));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

__device__ __forceinline__ v4i bload(Res r, uint32_t off) {
    return (v4i)__builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// bits t in [0, n) with 0 <= b + t < lim (n <= 15)
__device__ __forceinline__ uint32_t span_bits(int b, int n, int lim) {
    const int lo = max(-b, 0), hi = min(n, lim - b);
    return hi > lo ? (1u << hi) - (1u << lo) : 0u;
}

// filter taps t < n that land on an output row: (b - t) a multiple of st and
// 0 <= (b - t) / st < lim
__device__ __forceinline__ uint32_t stride_bits(int b, int n, int lim, int st, FastDiv dst) {
    uint32_t m = 0;
    for (int t = 0; t < n; ++t) {
        const int a = b - t;
        if (a < 0) break;
        const int q = (int)fdiv((uint32_t)a, dst);
        if (q * st == a && q < lim) m |= 1u << t;
    }
    return m;
}

// tap bit of a filter position (r, s); masks keep rows in bits 0..14 and
// columns in bits 16..30
__device__ __forceinline__ uint32_t tap_bits(int r, int s) { return (1u << (r & 15)) | (1u << (16 + (s & 15))); }

template <int KIND, int ROWS>
struct Ld;

// [row][k] chunks: chunk c of thread tid -> tile row (tid + 256 c) / CPR,
// contraction offset ((tid + 256 c) % CPR) * 16 (the same for every c).
template <int ROWS>
struct KChunks {
    static constexpr int CPR = BK / 16;
    static constexpr int CH = ROWS * CPR / NTHR;
    static constexpr int STRIDE = BK + 16;
    __device__ __forceinline__ static int row(int c, int tid) { return (tid + NTHR * c) / CPR; }
    __device__ __forceinline__ static int col(int tid) { return (tid % CPR) * 16; }
    __device__ __forceinline__ static void store(int8_t *s, int tid, const v4i (&reg)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) *(v4i *)(s + row(c, tid) * STRIDE + col(tid)) = reg[c];
    }
};

// [k][row] chunks: ROWS/16 chunks per k-row; chunk c -> k-row (tid + 256 c) /
// (ROWS/16), row offset ((tid + 256 c) % (ROWS/16)) * 16 (the same for every c).
template <int ROWS>
struct TChunks {
    static constexpr int PER = ROWS / 16;
    static constexpr int CH = ROWS * BK / 16 / NTHR;
    static constexpr int STRIDE = ROWS + TPad<ROWS>::value;
    __device__ __forceinline__ static int krow(int c, int tid) { return (tid + NTHR * c) / PER; }
    __device__ __forceinline__ static int ic(int tid) { return tid % PER; }
    __device__ __forceinline__ static void store(int8_t *s, int tid, const v4i (&reg)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) *(v4i *)(s + krow(c, tid) * STRIDE + ic(tid) * 16) = reg[c];
    }
};

// [k][row] chunks, two threads per contraction row: thread tid takes k-row
// tid / 2 and its chunks 2 c + tid % 2, so it decodes one contraction index
// per step for all of its chunks.
template <int ROWS>
struct TPairChunks {
    static_assert(BK == 128 && NTHR == 256, "two threads per contraction row");
    static constexpr int CH = ROWS / 32;
    static constexpr int STRIDE = ROWS + TPad<ROWS>::value;
    __device__ __forceinline__ static int krow(int tid) { return tid >> 1; }
    __device__ __forceinline__ static int ic(int c, int tid) { return 2 * c + (tid & 1); }
    __device__ __forceinline__ static void store(int8_t *s, int tid, const v4i (&reg)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) *(v4i *)(s + krow(tid) * STRIDE + ic(c, tid) * 16) = reg[c];
    }
};

// Dense K-contiguous operand: element (i, k) at base[i*ld + k].  Window: the
// tile's rows.
template <int ROWS>
struct Ld<LD_K, ROWS> : KChunks<ROWS> {
    using B_ = KChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = true;
    Res res;
    uint32_t off[CH];
    int col;
    __device__ __forceinline__ void init(const Operand &op, int i0, int kb, int tid, int koff = 0) {
        (void)kb;
        col = B_::col(tid);
        const int vr = min(max(op.rows - i0, 0), ROWS);
        // koff: the contraction starts at column koff (a stride phase's taps);
        // every load stays below column koff + kend <= ld
        res = make_res(op.base + (long long)i0 * op.ld + koff, vr * (int)op.ld - koff);
#pragma unroll
        for (int c = 0; c < CH; ++c) off[c] = (uint32_t)(B_::row(c, tid) * (int)op.ld + col);
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        const uint32_t kk = k0 + col < kend ? (uint32_t)k0 : OOB_K;
#pragma unroll
        for (int c = 0; c < CH; ++c) reg[c] = bload(res, off[c] + kk);
    }
};

// Forward convolution: row m = (n, p, q), k = (r, s, c) over the padded
// channel count cp (activation [N*H*W x cp]).  Window: the images of the
// tile's rows.  Taps outside the image read zeros (mask of valid r and s
// per row); the contraction past its end is zeroed by the weight operand.
template <int ROWS>
struct Ld<LD_IM2COL, ROWS> : KChunks<ROWS> {
    using B_ = KChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = false;
    Res res;
    int pix[CH];       // offset of tap (0, 0), channel 0 of the row's pixel (may be negative)
    uint32_t msk[CH];  // valid taps of the row (tap_bits layout)
    int r, s, ch, tap; // contraction index of the next load: (r, s, ch), tap = (r W + s) cp + ch
    int cp, S, dc, ds, dr, d0, d1;
    __device__ __forceinline__ void init(const Operand &op, int i0, int kb, int tid) {
        const ConvGeom &g = op.g;
        cp = g.cp;
        S = g.s;
        dc = g.im_dc;
        ds = g.im_ds;
        dr = g.im_dr;
        d0 = g.im_d0;
        d1 = g.im_d1;
        const int last = min(i0 + ROWS, op.rows) - 1;
        const int nf = (int)fdiv((uint32_t)i0, g.dpq), nl = (int)fdiv((uint32_t)max(last, i0), g.dpq);
        const int img = g.h * g.w * g.cp;
        res = make_res(op.base + (long long)nf * img, (nl - nf + 1) * img);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int m = i0 + B_::row(c, tid);
            const bool ok = m < op.rows;
            const uint32_t mm = ok ? m : i0;
            const uint32_t n = fdiv(mm, g.dpq), rem = mm - n * (uint32_t)(g.p * g.q);
            const uint32_t p = fdiv(rem, g.dq), q = rem - p * g.q;
            const int hb = (int)p * g.stride - g.pad, wb = (int)q * g.stride - g.pad;
            pix[c] = (((int)(n - nf) * g.h + hb) * g.w + wb) * g.cp;
            msk[c] = ok ? span_bits(hb, g.r, g.h) | span_bits(wb, g.s, g.w) << 16 : 0u;
        }
        const uint32_t kk = kb + B_::col(tid);
        const uint32_t rs = fdiv(kk, g.dc);
        ch = (int)(kk - rs * g.cp);
        r = (int)fdiv(rs, g.ds);
        s = (int)rs - r * g.s;
        tap = (r * g.w + s) * g.cp + ch;
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        (void)k0;
        (void)kend;
        const uint32_t bits = tap_bits(r, s);
#pragma unroll
        for (int c = 0; c < CH; ++c) reg[c] = bload(res, (msk[c] & bits) == bits ? (uint32_t)(pix[c] + tap) : OOB_K);
        // next step: (r, s, ch) += BK over (R, S, cp)
        ch += dc;
        const bool c1 = ch >= cp;
        ch = c1 ? ch - cp : ch;
        s += ds + (int)c1;
        const bool c2 = s >= S;
        s = c2 ? s - S : s;
        r += dr + (int)c2;
        tap += c2 ? d0 + d1 : d0;
    }
};

// What the input-gradient loader reads of a geometry: the convolution's own,
// or one of its stride phases (a stride-1 gather over the phase's pixels
// h = ph + st i, w = pw + st j and taps r = r0 + st a, s = s0 + st b).
struct DgGeo {
    int kp, R, S, P, Q, hw, W, padh, padw, stride, st_inv, dc, ds, dr;
    FastDiv dhw, dw, dst, dk, dsS;
};

__device__ __forceinline__ DgGeo dg_geo(const ConvGeom &g) {
    return DgGeo{g.kp, g.r, g.s, g.p, g.q, g.h * g.w, g.w, g.pad, g.pad, g.stride, g.st_inv, g.dg_dc, g.dg_ds,
                 g.dg_dr, g.dhw, g.dw, g.dst, g.dk, g.ds};
}

__device__ __forceinline__ DgGeo dg_geo(const ConvGeom &g, const PhaseRec &p) {
    return DgGeo{g.kp, p.ra, p.sb, g.p, g.q, p.hn * p.wn, p.wn, p.ch, p.cw, 1, 65536, g.dg_dc, p.ds,
                 p.dr, p.dhw, p.dw, FastDiv{1u << 31, 31}, g.dk, p.dsb};
}

// Input gradient of a convolution: row m = (n, h, w), k = (r, s, ko) over the
// padded output-channel count kp; element dY[n, p, q, ko] with
// p * stride = h + pad - r (zero unless exact).  With h + pad = st a + b, the
// taps that hit are r = b + st j, at p = a - j = a - floor(r / st).  Window:
// the output images of the tile's rows.  For a stride phase the rows are the
// phase's pixels and the taps its own, at stride 1.
template <int ROWS>
struct Ld<LD_DGRAD, ROWS> : KChunks<ROWS> {
    using B_ = KChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = false;
    Res res;
    int pix[CH];       // offset of output pixel (a_h, a_w), channel 0
    uint32_t msk[CH];  // taps that hit an output pixel (tap_bits layout)
    int r, s, ko;      // contraction index of the next load
    int kp, S, Q, dc, ds, dr, st_inv;
    __device__ __forceinline__ void init(const Operand &op, int i0, int kb, int tid) {
        init_geo(dg_geo(op.g), op.base, op.rows, i0, kb, tid);
    }
    __device__ __forceinline__ void init_geo(const DgGeo &g, const int8_t *base, int nrows, int i0, int kb,
                                             int tid) {
        kp = g.kp;
        S = g.S;
        Q = g.Q;
        dc = g.dc;
        ds = g.ds;
        dr = g.dr;
        st_inv = g.st_inv;
        const int last = min(i0 + ROWS, nrows) - 1;
        const int nf = (int)fdiv((uint32_t)i0, g.dhw), nl = (int)fdiv((uint32_t)max(last, i0), g.dhw);
        const int img = g.P * g.Q * g.kp;
        res = make_res(base + (long long)nf * img, (nl - nf + 1) * img);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int m = i0 + B_::row(c, tid);
            const bool ok = m < nrows;
            const uint32_t mm = ok ? m : i0;
            const uint32_t n = fdiv(mm, g.dhw), rem = mm - n * (uint32_t)g.hw;
            const uint32_t h = fdiv(rem, g.dw), w = rem - h * g.W;
            const int hp = (int)h + g.padh, wp = (int)w + g.padw;
            const int ah = (int)fdiv((uint32_t)hp, g.dst), aw = (int)fdiv((uint32_t)wp, g.dst);
            pix[c] = (((int)(n - nf) * g.P + ah) * g.Q + aw) * g.kp;
            msk[c] = ok ? stride_bits(hp, g.R, g.P, g.stride, g.dst) | stride_bits(wp, g.S, g.Q, g.stride, g.dst) << 16
                        : 0u;
        }
        const uint32_t kk = kb + B_::col(tid);
        const uint32_t rs = fdiv(kk, g.dk);
        ko = (int)(kk - rs * g.kp);
        r = (int)fdiv(rs, g.dsS);
        s = (int)rs - r * g.S;
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        (void)k0;
        (void)kend;
        const uint32_t bits = tap_bits(r, s);
        // floor(r / st) for r < 16: (r * ceil(2^16 / st)) >> 16
        const int rq = (int)(__umul24((uint32_t)r, (uint32_t)st_inv) >> 16);
        const int sq = (int)(__umul24((uint32_t)s, (uint32_t)st_inv) >> 16);
        const int tap = ko - __mul24(__mul24(rq, Q) + sq, kp);
#pragma unroll
        for (int c = 0; c < CH; ++c) reg[c] = bload(res, (msk[c] & bits) == bits ? (uint32_t)(pix[c] + tap) : OOB_K);
        ko += dc;
        const bool c1 = ko >= kp;
        ko = c1 ? ko - kp : ko;
        s += ds + (int)c1;
        const bool c2 = s >= S;
        s = c2 ? s - S : s;
        r += dr + (int)c2;
    }
};

// M-contiguous dense operand: element (i, k) at base[k*ld + i]; ld >= the
// row count rounded up to 16.  Window: the step's BK contraction rows, so
// rows past the end read zeros.
template <int ROWS>
struct Ld<LD_T, ROWS> : TChunks<ROWS> {
    using B_ = TChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = true;
    const int8_t *cur;  // element (i0, k0) of the next load
    int ld, i0;
    uint32_t off[CH];
    __device__ __forceinline__ void init(const Operand &op, int i0_, int kb, int tid) {
        i0 = i0_;
        ld = (int)op.ld;
        cur = op.base + i0 + (long long)kb * ld;
        const bool iok = i0 + B_::ic(tid) * 16 < op.rows;
#pragma unroll
        for (int c = 0; c < CH; ++c) off[c] = iok ? (uint32_t)(B_::krow(c, tid) * ld + B_::ic(tid) * 16) : OOB_ROW;
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        // contraction rows left in this step (written without a min / max
        // pair against constants, which would become a vector med3)
        const int rows = min(kend - k0, BK);
        const Res res = make_res(cur, rows > 0 ? rows * ld - i0 : 0);
#pragma unroll
        for (int c = 0; c < CH; ++c) reg[c] = bload(res, off[c]);
        cur += BK * ld;
    }
};

// Weight gradient of a convolution, B side: row j = (r, s, c) over the padded
// channel count cp, k = output pixel (n, p, q); element
// X[n, p*st + r - pad, q*st + s - pad, c].  Window: the images the step's BK
// pixels fall in; the contraction past its end is zeroed by the dY operand.
template <int ROWS>
struct Ld<LD_IM2COL_T, ROWS> : TPairChunks<ROWS> {
    using B_ = TPairChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = false;
    const int8_t *win;      // the window's first image
    int img;                // bytes per image
    int n_img, nw;          // images of the tensor, images per window
    int ns, urem;           // window's first image; k0 - ns P Q
    int hb, wb, pix;        // this thread's pixel: p st - pad, q st - pad, offset from the window
    // Validity of a chunk: its filter position (jr, js) puts the pixel's tap
    // inside the image.  Up to 4 chunks per thread test it directly; more
    // share per-step masks of the valid rows and columns.
    static constexpr bool MASKS = CH > 4;
    uint32_t jbit[MASKS ? CH : 1];  // tap bits of (jr, js) (bit 15 when past the rows)
    int jr[MASKS ? 1 : CH], js[MASKS ? 1 : CH];  // (jr = 2^20 when past the rows)
    int joff[CH];           // (jr W + js) cp + jc
    int pq, u_dr, u_dn, wlim, hlim, qs, ps, dwb, dhb, st, d0, d1, d2, R, S, H, W;
    __device__ __forceinline__ void init(const Operand &op, int j0, int kb, int tid) {
        const ConvGeom &g = op.g;
        img = g.h * g.w * g.cp;
        n_img = g.n;
        nw = g.px_nw;
        pq = g.p * g.q;
        u_dr = BK % pq;
        u_dn = BK / pq;
        st = g.stride;
        qs = g.q * g.stride;
        ps = g.p * g.stride;
        wlim = qs - g.pad;
        hlim = ps - g.pad;
        dwb = g.px_dq * g.stride;
        dhb = g.px_dp * g.stride;
        d0 = g.px_d0;
        d1 = g.px_d1;
        d2 = g.px_d2;
        R = g.r;
        S = g.s;
        H = g.h;
        W = g.w;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = j0 + B_::ic(c, tid) * 16;
            const bool ok = j < op.rows;
            const uint32_t rs = fdiv(ok ? j : 0, g.dc);
            const int jc = (ok ? j : 0) - (int)rs * g.cp;
            const int r_ = (int)fdiv(rs, g.ds), s_ = (int)rs - r_ * g.s;
            if constexpr (MASKS) {
                jbit[c] = ok ? tap_bits(r_, s_) : 1u << 15;
            } else {
                jr[c] = ok ? r_ : 1 << 20;
                js[c] = s_;
            }
            joff[c] = (r_ * g.w + s_) * g.cp + jc;
        }
        ns = (int)fdiv((uint32_t)kb, g.dpq);
        urem = kb - ns * pq;
        win = op.base + (long long)ns * img;
        const uint32_t k = kb + B_::krow(tid);
        const uint32_t n = fdiv(k, g.dpq), rem = k - n * (uint32_t)pq;
        const uint32_t p = fdiv(rem, g.dq), q = rem - p * g.q;
        hb = (int)p * g.stride - g.pad;
        wb = (int)q * g.stride - g.pad;
        pix = (((int)n - ns) * g.h + hb) * g.w * g.cp + wb * g.cp;
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        (void)k0;
        (void)kend;
        const int left = min(n_img - ns, nw);
        const Res res = make_res(win, left > 0 ? left * img : 0);
        if constexpr (MASKS) {
            const uint32_t hw = span_bits(hb, R, H) | span_bits(wb, S, W) << 16;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                reg[c] = bload(res, (hw & jbit[c]) == jbit[c] ? (uint32_t)(pix + joff[c]) : OOB_K);
        } else {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const bool ok = (uint32_t)(hb + jr[c]) < (uint32_t)H && (uint32_t)(wb + js[c]) < (uint32_t)W;
                reg[c] = bload(res, ok ? (uint32_t)(pix + joff[c]) : OOB_K);
            }
        }
        // next step: the window's first image and this thread's pixel move by BK pixels
        urem += u_dr;
        const int cs = urem >= pq;
        urem = cs ? urem - pq : urem;
        const int dns = u_dn + cs;
        ns += dns;
        win += dns * img;
        wb += dwb;
        const bool c1 = wb >= wlim;
        wb = c1 ? wb - qs : wb;
        hb += c1 ? dhb + st : dhb;
        const bool c2 = hb >= hlim;
        hb = c2 ? hb - ps : hb;
        pix += d0 - dns * img + (c1 ? d1 : 0) + (c2 ? d2 : 0);
    }
};

// Input gradient of a convolution, B side, straight from the weight
// [k_out][r][s][c] (whole-tensor exponent, c a multiple of 16): row j = input
// channel, k = (r, s, ko) over the padded output-channel count kp; 16
// consecutive channels of one (r, s, ko) are contiguous.  Window: the whole
// weight, so padded output channels read zeros.
template <int ROWS>
struct Ld<LD_WT, ROWS> : TPairChunks<ROWS> {
    using B_ = TPairChunks<ROWS>;
    static constexpr int CH = B_::CH;
    static constexpr bool ZK = true;
    Res res;
    uint32_t joff[CH];
    int krow, ko, koff;     // this thread's k-row; ko of the next load and ko R S C + rs C
    int kp, dc, d0, d1;
    __device__ __forceinline__ void init(const Operand &op, int j0, int kb, int tid) {
        const ConvGeom &g = op.g;
        kp = g.kp;
        dc = g.dg_dc;
        d0 = g.wt_d0;
        d1 = g.wt_d1;
        const int rsc = g.r * g.s * g.c;
        res = make_res(op.base + j0, g.k * rsc - j0);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = j0 + B_::ic(c, tid) * 16;
            joff[c] = j < op.rows ? (uint32_t)(B_::ic(c, tid) * 16) : OOB_ROW;
        }
        krow = B_::krow(tid);
        const uint32_t kk = kb + krow;
        const uint32_t rs = fdiv(kk, g.dk);
        ko = (int)(kk - rs * g.kp);
        koff = ko * rsc + (int)rs * g.c;
    }
    __device__ __forceinline__ void load(int k0, int kend, v4i (&reg)[CH]) {
        const uint32_t kbase = k0 + krow < kend ? (uint32_t)koff : OOB_K;
#pragma unroll
        for (int c = 0; c < CH; ++c) reg[c] = bload(res, kbase + joff[c]);
        ko += dc;
        const bool c1 = ko >= kp;
        ko = c1 ? ko - kp : ko;
        koff += c1 ? d0 + d1 : d0;
    }
};

// ---------------------------------------------------------------------------
// MFMA fragments: lane l holds row (l % 32) and contraction bytes
// 16 (l / 32) .. + 15 of a 32-byte step.
// ---------------------------------------------------------------------------

template <int KIND, int ROWS>
__device__ __forceinline__ v4i frag(const int8_t *s, int rowbase, int ks, int lane) {
    constexpr int STRIDE = Lds<KIND, ROWS>::STRIDE;
    if constexpr (!IsT<KIND>::value) {
        return *(const v4i *)(s + (rowbase + (lane & 31)) * STRIDE + ks * 32 + (lane >> 5) * 16);
    } else {
        const int g = lane & 15;
        const int i = rowbase + (lane & 16) + (g & 1) * 8;
        const int k = ks * 32 + (lane >> 5) * 16 + (g >> 1);
        typedef __attribute__((address_space(3))) v2i lds_v2i;
        v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(s + k * STRIDE + i));
        v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(s + (k + 8) * STRIDE + i));
        return v4i{lo.x, lo.y, hi.x, hi.y};
    }
}

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int wave_max(int v) { return wave_max_dpp(v); }

// Maxima of 16 rows over the 32 lanes of a half-wave, transposing as it
// reduces (16 exchanges instead of 80): at each step a lane keeps half of its
// rows and takes the partner's values for them.  The lane ends with the
// maximum of row 8 b4 + 4 b3 + 2 b2 + b1 (b_i = bit i of the lane).
__device__ __forceinline__ int rows16_max(const int (&v)[16], int lane) {
    int w[8], x[4], y[2];
    const bool u16 = lane & 16, u8 = lane & 8, u4 = lane & 4, u2 = lane & 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = max(u16 ? v[i + 8] : v[i], __shfl_xor(u16 ? v[i] : v[i + 8], 16));
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = max(u8 ? w[i + 4] : w[i], __shfl_xor(u8 ? w[i] : w[i + 4], 8));
#pragma unroll
    for (int i = 0; i < 2; ++i) y[i] = max(u4 ? x[i + 2] : x[i], __shfl_xor(u4 ? x[i] : x[i + 2], 4));
    int z = max(u2 ? y[1] : y[0], __shfl_xor(u2 ? y[0] : y[1], 2));
    return max(z, __shfl_xor(z, 1));
}

__device__ __forceinline__ int rows16_row(int lane) {
    return 8 * ((lane >> 4) & 1) + 4 * ((lane >> 3) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 1) & 1);
}

// Branch-free forms of rne_shift32 / rto_shift32 (the same results, shift
// clamped to [-31, 31]): x = a * 2^L, then a right shift by R, with L or R zero.
__device__ __forceinline__ int rne_bf(int a, int s) {
    s = min(max(s, -31), 31);
    const int L = max(-s, 0), R = max(s, 0);
    const int x = a << L;
    const int hm1 = R > 0 ? (1 << (R - 1)) - 1 : 0;
    const int bit = R > 0 ? (x >> R) & 1 : 0;
    return (x + hm1 + bit) >> R;
}

__device__ __forceinline__ int rto_bf(int a, int t) {
    t = min(max(t, -31), 31);
    const int L = max(-t, 0), R = max(t, 0);
    const int x = a << L;
    const uint32_t mask = (1u << R) - 1u;
    return (x >> R) | (int)((((uint32_t)x & mask) + mask) >> R);
}

// The same roundings with the shift-dependent part computed once: a value
// shared by a column (or row) of the tile then costs four operations (shift,
// bit extract, three-input add, shift) for rne, five for rto.
struct RneP {
    int L, R, hm1, w;  // left shift, right shift, 2^(R-1) - 1, extract width (1 when R > 0)
};
__device__ __forceinline__ RneP rne_prep(int s) {
    s = min(max(s, -31), 31);
    RneP p;
    p.L = max(-s, 0);
    p.R = max(s, 0);
    p.hm1 = p.R > 0 ? (1 << (p.R - 1)) - 1 : 0;
    p.w = p.R > 0 ? 1 : 0;
    return p;
}
__device__ __forceinline__ int rne_apply(int a, const RneP &p) {
    const int x = a << p.L;
    const int bit = (int)__builtin_amdgcn_ubfe((uint32_t)x, (uint32_t)p.R, (uint32_t)p.w);
    return (x + p.hm1 + bit) >> p.R;
}
struct RtoP {
    int L, R;
    uint32_t mask;  // the R bits shifted out
};
__device__ __forceinline__ RtoP rto_prep(int t) {
    t = min(max(t, -31), 31);
    RtoP p;
    p.L = max(-t, 0);
    p.R = max(t, 0);
    p.mask = (1u << p.R) - 1u;
    return p;
}
__device__ __forceinline__ int rto_apply(int a, const RtoP &p) {
    const int x = a << p.L;
    return (x >> p.R) | (int)min((uint32_t)x & p.mask, 1u);
}

// Largest |v| over a run of values as an unsigned magnitude, from the signed
// maximum and minimum (two values per three-input max / min).
template <int N>
__device__ __forceinline__ uint32_t max_mag(const int (&v)[N]) {
    int hi = 0, lo = 0;
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        hi = max(hi, max(v[i], v[i + 1]));
        lo = min(lo, min(v[i], v[i + 1]));
    }
    return max((uint32_t)hi, 0u - (uint32_t)lo);
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

// Workgroups are dispatched to the 8 XCDs round robin (id % 8).  Work items
// are numbered so that each XCD receives a contiguous run of the logical
// order -- contraction chunk slowest, then row tile, then column tile: one
// XCD walks all column tiles of a row tile, and all tiles of a chunk, before
// the next, keeping the shared operand rows (and a chunk's rows of both
// operands) in its own L2.
__device__ __forceinline__ void work_of(int bid, int TM, int TN, int S, int &tm, int &tn, int &z) {
    const int T = TM * TN, W = T * S;
    const int q = W / 8, r = W % 8;
    const int x = bid % 8, j = bid / 8;
    const int logical = x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
    // the divisions run on the vector unit; the work item is the same in
    // every lane, so its indices go back to scalar registers
    z = __builtin_amdgcn_readfirstlane(logical / T);
    const int t = logical - z * T;
    tm = __builtin_amdgcn_readfirstlane(t / TN);
    tn = __builtin_amdgcn_readfirstlane(t - tm * TN);
}

// Stride phase of tile row t of a phase-decomposed input gradient: each
// aligned group of four tile rows holds the four phases, rotated by a hash
// of the group, so that workgroups walking the tiles at any stride (the
// persistent first pass) meet every phase, not one.
__device__ __forceinline__ int phase_of_tile(int t) {
    return (t + (int)(((uint32_t)(t >> 2) * 2654435761u) >> 30)) & 3;
}

// Register pipeline depth: 3 for the 2 x 2 tile, which runs two workgroups
// per CU and would spill at 4, and for the 64 x 64 tile.
template <int MI, int NI>
struct Stages {
    static constexpr int value = MI * NI >= 8 ? 2 : (MI == 2 && NI == 2) ? IE_STAGES22 : MI * NI == 1 ? 3 : IE_STAGES;
};

// Contraction slicing of the 64 x 64 tile: wave w takes the w-th 32-byte
// sub-step of every stage for the whole tile (four independent accumulators,
// half the fragment reads of a 2 x 2 split of the tile between the waves);
// the four partial tiles are summed through LDS after the main loop, leaving
// each wave its own quadrant as in the other tiles.
#ifndef IE_KSLICE
#define IE_KSLICE 1
#endif
template <int MI, int NI>
struct KSlice {
    static constexpr bool value = IE_KSLICE && MI == 1 && NI == 1;
};

// Workgroups per CU that a tile's register budget is sized for.
template <int MI, int NI>
struct Occ {
    static constexpr int value = MI * NI == 1 ? (KSlice<MI, NI>::value ? 3 : 4) : MI * NI < 4 ? 2 : MI * NI == 4 ? IE_OCC22 : 1;
};
// The same for the one-step form of a tile (one LDS stage, no register
// pipeline): up to four workgroups per CU.
template <int MI, int NI>
struct Occ1 {
    static constexpr int value = MI * NI <= 2 ? 4 : MI * NI == 4 ? 3 : MI * NI <= 8 ? 2 : 1;
};

// LDS of a tile: two stages of both operands (also the epilogue's staging).
template <int KA, int KB, int MI, int NI, bool PARTIAL = true>
struct TileLds {
    static constexpr int stages = 2 * (Lds<KA, 64 * MI>::BYTES + Lds<KB, 64 * NI>::BYTES);
    static constexpr int partial = 64 * MI * (64 * NI * 4 + 32);  // int32 staging of a split product
    static constexpr int epi = 64 * MI * (64 * NI * 2 + 16) + 4 * 64 * MI * 4 + 64;  // int16 staging + maxima
    static constexpr int out = PARTIAL ? partial : epi;
    static constexpr int value = stages > out ? stages : out;
};

// LDS of a tile whose contraction is one step (K <= BK): one stage, or the
// epilogue's staging and maxima if larger (no split products).
template <int KA, int KB, int MI, int NI>
struct TileLds1 {
    static constexpr int stage = Lds<KA, 64 * MI>::BYTES + Lds<KB, 64 * NI>::BYTES;
    static constexpr int epi = 64 * MI * (64 * NI * 2 + 16) + 4 * 64 * MI * 4 + 64;
    // the contraction-sliced 64 x 64 tile sums four partial tiles through LDS
    static constexpr int slices = KSlice<MI, NI>::value ? 8 * 4096 : 0;
    static constexpr int v0 = stage > epi ? stage : epi;
    static constexpr int value = v0 > slices ? v0 : slices;
};

// One workgroup's work item: bid and nblk are its index and the number of
// workgroups of its grid (or of its part of a paired grid); lds points to
// TileLds bytes of shared memory (TileLds1 when ONE: a contraction of at
// most one step, loaded once, with no pipeline and no second buffer).
// Returns the tile's group maximum in the first pass of a recomputed
// whole-tensor product (EPI_MAX), NEED_NONE otherwise.
// RG: the result groups when fixed at compile time (0: one for the whole
// tensor, 1: one per row; -1: ep.row_group decides), so that a kernel that
// only ever takes one of them carries no code for the other.  DI likewise
// for the epilogue: 1 rounds to int8 in this pass (direct, or the second
// pass of a recomputed product), 0 rounds to odd; -1: ep.mode decides.
template <int KA, int KB, int MI, int NI, bool PARTIAL, bool ONE = false, int MODE = -1, int RG = -1, int DI = -1>
__device__ __forceinline__ int gemm_tile(const Operand &A, const Operand &B, int M_, int N, int K, int k_chunk,
                                          int TM, int S, const Epi &ep, int bid, int nblk, int8_t *lds) {
    static_assert(!(ONE && PARTIAL), "one-step tiles have no split form");
    constexpr int BMt = 64 * MI, BNt = 64 * NI;
    using LA = Lds<KA, BMt>;
    using LB = Lds<KB, BNt>;
    constexpr int STAGE = LA::BYTES + LB::BYTES;
    constexpr int LDSB = ONE ? TileLds1<KA, KB, MI, NI>::value : TileLds<KA, KB, MI, NI, PARTIAL>::value;  // bytes at lds

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int TN = (N + BNt - 1) / BNt;
    int tile_m, tile_n, z;
    work_of(bid, TM, TN, S, tile_m, tile_n, z);
    int M = M_, m0 = tile_m * BMt;
    const int n0 = tile_n * BNt;
    int kb = z * k_chunk;
    int ke = min(K, kb + k_chunk);

    Ld<KA, BMt> la;
    Ld<KB, BNt> lb;
    static_assert(Ld<KA, BMt>::ZK || Ld<KB, BNt>::ZK, "one operand must zero the contraction past its end");
    // A stride phase of an input gradient (tile rows are grouped by phase,
    // the phases in order): the phase's pixels as rows, its taps as the
    // contraction, its columns of the phase-sorted weight copy.
    bool phased = false;
    PhaseRec pr{};
    if constexpr (KA == LD_DGRAD && KB == LD_K) {
        if (ep.ph.n) {
            // the phases interleave: tile row tile_m is row tile_m / 4 of phase
            // phase_of_tile(tile_m), a rotation within each aligned group of four
            pr = ep.ph.r[phase_of_tile(tile_m)];
            phased = true;
            M = pr.rows;
            m0 = (tile_m >> 2) * BMt;
            kb = 0;
            ke = pr.klen;
            static_assert(PHASES_MAX == 4, "stride-2 phases");
            if (m0 >= M) ke = 0;  // past the phase's rows: an empty tile
            // the first pass finds nothing in a phase without taps or past its rows
            if constexpr (MODE == EPI_MAX)
                if (ke == 0) return NEED_NONE;
            la.init_geo(dg_geo(A.g, pr), A.base, M, m0, 0, tid);
            lb.init(B, n0, 0, tid, pr.k0);
        }
    }
    if (!phased) {
        la.init(A, m0, kb, tid);
        lb.init(B, n0, kb, tid);
    }
    const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
    constexpr int CA = Ld<KA, BMt>::CH, CB = Ld<KB, BNt>::CH;

    // exponents of this tile's rows and columns, for the epilogue
    __shared__ int seA[PARTIAL ? 1 : BMt], seB[PARTIAL ? 1 : BNt];
    if constexpr (!PARTIAL) {
        for (int i = tid; i < BMt; i += NTHR) seA[i] = m0 + i < M ? exp_at(ep.ea, m0 + i) : 0;
        for (int i = tid; i < BNt; i += NTHR) seB[i] = n0 + i < N ? exp_at(ep.eb, n0 + i) : 0;
    } else {
        // group maxima of the split finalize start empty (it runs after this grid)
        for (int i = bid * NTHR + tid; i < ep.gneed_n; i += nblk * NTHR) ep.gneed[i] = NEED_NONE;
    }
    // second pass of a recomputed whole-tensor product: the first pass's
    // maxima, loaded now so that they land during the main loop
    int given = NEED_NONE;
    if constexpr (!PARTIAL) {
        if (ep.mode == EPI_GIVEN && !(RG >= 0 ? RG == 1 : ep.row_group))
            for (int i = tid; i < ep.tneed_n; i += NTHR) given = max(given, ep.tneed[i]);
    }

    constexpr bool KS = KSlice<MI, NI>::value;
    constexpr int AM = KS ? 2 : MI, AN = KS ? 2 : NI;  // accumulators per wave
    v16i acc[AM][AN];
#pragma unroll
    for (int a = 0; a < AM; ++a)
#pragma unroll
        for (int b = 0; b < AN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    // NS register stages in flight: stage s is loaded into register set
    // s % NS at step s - NS, written to LDS buffer s % 2 at the end of step
    // s - 1 and computed at step s, so a load has NS - 1 steps to land.
    constexpr int NS = ONE ? 1 : Stages<MI, NI>::value;
    v4i ra[NS][CA], rb[NS][CB];
    // An empty chunk issues no load at all: with an empty contraction the
    // operand pointers need not address any memory.
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            la.load(kb + s * BK, ke, ra[s]);
            lb.load(kb + s * BK, ke, rb[s]);
        }
        la.store(lds, tid, ra[0]);
        lb.store(lds + LA::BYTES, tid, rb[0]);
    }
    __syncthreads();

    auto compute = [&](const int8_t *sA) {
        const int8_t *sB = sA + LA::BYTES;
        if constexpr (KS) {
            static_assert(BK / 32 == NTHR / 64, "one contraction sub-step per wave");
            v4i af[2], bf[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) af[a] = frag<KA, BMt>(sA, a * 32, wave, lane);
#pragma unroll
            for (int b = 0; b < 2; ++b) bf[b] = frag<KB, BNt>(sB, b * 32, wave, lane);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
            return;
        }
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            v4i af[MI], bf[NI];
#pragma unroll
            for (int a = 0; a < MI; ++a) af[a] = frag<KA, BMt>(sA, wm * 32 * MI + a * 32, ks, lane);
#pragma unroll
            for (int b = 0; b < NI; ++b) bf[b] = frag<KB, BNt>(sB, wn * 32 * NI + b * 32, ks, lane);
#pragma unroll
            for (int a = 0; a < MI; ++a)
#pragma unroll
                for (int b = 0; b < NI; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
    };

    // Fragments of one 32-byte sub-step, read ahead of the MFMAs that take
    // them: sub-step ks + 1 is read while sub-step ks multiplies, and the
    // first sub-step of the next LDS buffer right after the barrier, while
    // the last sub-step of the current one multiplies.  The scheduling
    // groups interleave one fragment read with each MFMA, so that the LDS
    // latency hides under matrix work within the wave.
    constexpr int RD = (IsT<KA>::value ? 2 : 1) * MI + (IsT<KB>::value ? 2 : 1) * NI;  // LDS reads per sub-step
    constexpr int NMF = MI * NI;
    v4i fa[2][MI], fb[2][NI];
    auto rdfrag = [&](const int8_t *sA, const int ks, v4i (&af)[MI], v4i (&bf)[NI]) {
        const int8_t *sB = sA + LA::BYTES;
#pragma unroll
        for (int a = 0; a < MI; ++a) af[a] = frag<KA, BMt>(sA, wm * 32 * MI + a * 32, ks, lane);
#pragma unroll
        for (int b = 0; b < NI; ++b) bf[b] = frag<KB, BNt>(sB, wn * 32 * NI + b * 32, ks, lane);
    };
    auto mma = [&](const v4i (&af)[MI], const v4i (&bf)[NI]) {
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int b = 0; b < NI; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
    };
    // the next sub-step's reads first, then this sub-step's MFMAs: a read
    // has a whole sub-step of matrix work to land
    auto interleave = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);  // MFMAs
    };

    // Trips of NU steps with no exit inside: the loads of the next stages stay
    // in flight across the back edge (an exit inside the trip would make the
    // loop head wait for all of them).  The last nk % NU steps follow the loop.
    if constexpr (ONE) {
        // nk <= 1: the stage loaded above is the whole contraction
        if (nk > 0) compute(lds);
    } else if constexpr (IE_PIPE && !KS) {
        static_assert(BK / 32 % 2 == 0, "sub-step parity picks the fragment set");
        rdfrag(lds, 0, fa[0], fb[0]);
        auto step = [&](const int uu, const int s) {
            const int u = uu % NS;
            la.load(kb + (s + NS) * BK, ke, ra[u]);
            lb.load(kb + (s + NS) * BK, ke, rb[u]);
            __builtin_amdgcn_sched_barrier(0);
            const int8_t *cur = lds + (uu & 1) * STAGE;
#pragma unroll
            for (int ks = 0; ks + 1 < BK / 32; ++ks) {
                rdfrag(cur, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
                mma(fa[ks & 1], fb[ks & 1]);
                interleave();
                __builtin_amdgcn_sched_barrier(0);
            }
            // stage s + 1 into the other buffer, whose readers all passed
            // the previous barrier (past the end: zeros nobody reads)
            la.store(lds + ((uu + 1) & 1) * STAGE, tid, ra[(u + 1) % NS]);
            lb.store(lds + ((uu + 1) & 1) * STAGE + LA::BYTES, tid, rb[(u + 1) % NS]);
            __syncthreads();
            rdfrag(lds + ((uu + 1) & 1) * STAGE, 0, fa[0], fb[0]);
            mma(fa[1], fb[1]);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
        };
        constexpr int NU = NS % 2 ? 4 * NS : IE_UNROLL * NS;  // even: step parity picks the LDS buffer
        const int full = nk - nk % NU;
        for (int it = 0; it < full; it += NU) {
#pragma unroll
            for (int uu = 0; uu < NU; ++uu) step(uu, it + uu);
        }
#pragma unroll
        for (int uu = 0; uu < NU - 1; ++uu) {
            if (full + uu >= nk) break;
            step(uu, full + uu);
        }
    } else {
        auto step = [&](const int uu, const int s) {
            const int u = uu % NS;
            // set u held stage s, already in LDS: refill it with stage s + NS
            // (past the end: loaded, never computed)
            la.load(kb + (s + NS) * BK, ke, ra[u]);
            lb.load(kb + (s + NS) * BK, ke, rb[u]);
#ifndef IE_NO_SCHED_BARRIER
            // keep the refill ahead of the fragment reads, so that no fragment
            // lands in registers whose loads are still in flight
            __builtin_amdgcn_sched_barrier(0);
#endif
            compute(lds + (uu & 1) * STAGE);
            // stage s + 1 (past the end: zeros into a buffer nobody reads)
            la.store(lds + ((uu + 1) & 1) * STAGE, tid, ra[(u + 1) % NS]);
            lb.store(lds + ((uu + 1) & 1) * STAGE + LA::BYTES, tid, rb[(u + 1) % NS]);
            __syncthreads();
        };
        constexpr int NU = NS % 2 ? 4 * NS : IE_UNROLL * NS;  // even: step parity picks the LDS buffer
        const int full = nk - nk % NU;
        for (int it = 0; it < full; it += NU) {
#pragma unroll
            for (int uu = 0; uu < NU; ++uu) step(uu, it + uu);
        }
#pragma unroll
        for (int uu = 0; uu < NU - 1; ++uu) {
            if (full + uu >= nk) break;
            step(uu, full + uu);
        }
    }

    if constexpr (KS) {
        // Sum the four partial tiles: quadrant q = 2 a + b (rows 32 a, columns
        // 32 b) ends with wave q.  Chunk j (ints 4j..4j+3) of a lane's partial
        // quadrant sits at slot * 1024 + j * 256 + lane (in 16-byte units).
        // Phase 1: wave w posts quadrants w+1, w+2 (mod 4); phase 2: w+3.
        v4i *red = (v4i *)lds;
        const int w = __builtin_amdgcn_readfirstlane(wave);
        auto quad = [&](int q) -> v16i {
            return q == 0 ? acc[0][0] : q == 1 ? acc[0][1] : q == 2 ? acc[1][0] : acc[1][1];
        };
        auto post = [&](int slot, const v16i &v) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[slot * 256 + j * 64 + lane] = v4i{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        };
        auto take = [&](int slot, v16i &v) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i t = red[slot * 256 + j * 64 + lane];
                v[4 * j] += t[0];
                v[4 * j + 1] += t[1];
                v[4 * j + 2] += t[2];
                v[4 * j + 3] += t[3];
            }
        };
        static_assert(8 * 4096 <= LDSB, "partial tiles exceed LDS");
        v16i mine = quad(w);
        __syncthreads();  // every wave is done with the last stage
        post(2 * w, quad((w + 1) & 3));
        post(2 * w + 1, quad((w + 2) & 3));
        __syncthreads();
        take(2 * ((w + 3) & 3), mine);      // wave w - 1 posted quadrant w first
        take(2 * ((w + 2) & 3) + 1, mine);  // wave w - 2 posted it second
        __syncthreads();
        post(w, quad((w + 3) & 3));
        __syncthreads();
        take((w + 1) & 3, mine);  // wave w + 1 posted quadrant (w + 1) + 3 = w
        __syncthreads();
        acc[0][0] = mine;
    }

    // Element (a, b, r) of this lane sits at tile row / column
    //   TR = 32 MI wm + 32 a + 8 (r/4) + 4 (lane/32) + r%4,   TC = 32 NI wn + 32 b + lane%32.
    const int tr0 = wm * 32 * MI + 4 * (lane >> 5);
    const int tc0 = wn * 32 * NI + (lane & 31);
    auto TR = [&](int a, int r) { return tr0 + a * 32 + 8 * (r >> 2) + (r & 3); };
    auto TC = [&](int b) { return tc0 + b * 32; };

    // Results leave through LDS: every lane writes its values into a
    // row-major staging tile (element size ES bytes, row pitch padded so that
    // the two half-waves, four rows apart, hit different banks), then the
    // tile is written out in 16-byte row chunks.
    auto flush = [&](auto es_tag, void *dst, long long ld, bool vec) {
        constexpr int ES = decltype(es_tag)::value;
        constexpr int PITCH = BNt * ES + (ES == 4 ? 32 : 16);
        constexpr int CPR = BNt * ES / 16;  // chunks per tile row
        constexpr int EPC = 16 / ES;        // elements per chunk
#pragma unroll
        for (int q0 = 0; q0 < BMt * CPR; q0 += NTHR) {
            const int q = q0 + tid;
            const int row = q / CPR, cb = (q % CPR) * 16;
            const int gcol = n0 + cb / ES;
            int grow = m0 + row;
            if (grow >= M || gcol >= N) continue;
            if constexpr (KA == LD_DGRAD && KB == LD_K) {
                // a phase pixel (n, i, j) is input pixel (n, ph + st i, pw + st j)
                if (phased) {
                    const uint32_t n = fdiv((uint32_t)grow, pr.dhw), rem = grow - n * (uint32_t)(pr.hn * pr.wn);
                    const uint32_t i = fdiv(rem, pr.dw), j = rem - i * (uint32_t)pr.wn;
                    grow = ((int)n * ep.ph.h + pr.ph + ep.ph.st * (int)i) * ep.ph.w + pr.pw + ep.ph.st * (int)j;
                }
            }
            v4i v = *(const v4i *)(lds + row * PITCH + cb);
            if constexpr (ES == 1) {
                // the activation on the rounded bytes (mask bytes at the
                // results' own offsets)
                const long long o = (long long)grow * ld + gcol;
                if (vec && gcol + EPC <= N) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] = (int)act4((uint32_t)v[k], ep.act, o + 4 * k);
                } else if (ep.act.relu || ep.act.mask) {
                    const int n = min(16, N - gcol);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint32_t w = (uint32_t)v[k];
                        if (ep.act.relu) w = relu4(w);
                        if (ep.act.mask) {
                            uint32_t x = 0;
                            for (int j = 0; j < 4; ++j)
                                if (4 * k + j < n) x |= (uint32_t)(uint8_t)ep.act.mask[o + 4 * k + j] << (8 * j);
                            w = pos_mask4(w, x);
                        }
                        v[k] = (int)w;
                    }
                }
            }
            int8_t *g = (int8_t *)dst + ((long long)grow * ld + gcol) * ES;
            if (vec && gcol + EPC <= N) {
                *(v4i *)g = v;
            } else if constexpr (ES == 1) {
                // rows not 16-byte aligned (or a row's last chunk): bytes up to
                // the first 4-byte boundary, then whole dwords, then the rest
                const int n = min(16, N - gcol);
                auto sel = [&](int i) -> uint32_t {
                    return (uint32_t)(i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : i == 3 ? v[3] : 0);
                };
                auto byte_at_ = [&](int j) { return (int8_t)(sel(j >> 2) >> (8 * (j & 3))); };
                const int j0 = min((int)((4u - ((uint32_t)(uintptr_t)g & 3u)) & 3u), n);
                for (int j = 0; j < 3; ++j)
                    if (j < j0) g[j] = byte_at_(j);
                const int nd = (n - j0) >> 2, sh = 8 * j0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (k < nd) {
                        const int p = j0 + 4 * k;
                        const uint32_t lo = sel(p >> 2), hi = sel((p >> 2) + 1);
                        *(uint32_t *)(g + p) = sh ? (lo >> sh) | (hi << (32 - sh)) : lo;
                    }
                }
                for (int j = j0 + 4 * nd; j < n; ++j) g[j] = byte_at_(j);
            } else {
                const int8_t *b8 = (const int8_t *)&v;
                for (int j = 0; j < EPC && gcol + j < N; ++j)
                    for (int t = 0; t < ES; ++t) g[j * ES + t] = b8[j * ES + t];
            }
        }
    };
    auto stage = [&](auto es_tag, int a, int b, int r, int v) {
        constexpr int ES = decltype(es_tag)::value;
        constexpr int PITCH = BNt * ES + (ES == 4 ? 32 : 16);
        int8_t *d = lds + TR(a, r) * PITCH + TC(b) * ES;
        if constexpr (ES == 1) *d = (int8_t)v;
        else if constexpr (ES == 2) *(int16_t *)d = (int16_t)v;
        else *(int *)d = v;
    };
    using ES1 = std::integral_constant<int, 1>;
    using ES2 = std::integral_constant<int, 2>;
    using ES4 = std::integral_constant<int, 4>;

    if constexpr (PARTIAL) {
        static_assert(BMt * (BNt * 4 + 32) <= LDSB, "staging tile exceeds LDS");
#pragma unroll
        for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int b = 0; b < NI; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) stage(ES4{}, a, b, r, acc[a][b][r]);
        __syncthreads();
        flush(ES4{}, ep.partial + (long long)z * ep.split_stride, N, (N & 3) == 0);
        return NEED_NONE;
    } else {
        int *red = (int *)(lds + LDSB) - 2 * BMt;  // maxima, at the top of LDS
        int *scr = red - 16;                             // block reductions
        static_assert(BMt * (BNt * 2 + 16) + 4 * BMt * 4 + 64 <= LDSB, "staging tile exceeds LDS");
        int ebv[NI];
#pragma unroll
        for (int b = 0; b < NI; ++b) ebv[b] = seB[TC(b)];
        const bool uni = !ep.ea.row && !ep.eb.row;
        const int wq = ep.q;  // results have |C| <= 2^wq - 1
        const int ea0 = seA[0];
        const int eb0 = seB[0];
        const int mode = MODE >= 0 ? MODE : ep.mode;
        // int8 results from this pass
        const bool direct = DI >= 0 ? DI == 1 : (mode == EPI_DIRECT || mode == EPI_GIVEN);

        if (!(RG >= 0 ? RG == 1 : ep.row_group)) {
            // whole-tensor group: one maximum for the tile (or, in the second
            // pass of a recomputed product, the first pass's maxima)
            int tmax;
            if (mode == EPI_GIVEN) {
                tmax = given;
            } else if (uni) {
                // largest |acc| from the signed maximum and minimum, two
                // values per three-input max / min
                int hi = 0, lo = 0;
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int b = 0; b < NI; ++b)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) {
                            hi = max(hi, max(acc[a][b][r], acc[a][b][r + 1]));
                            lo = min(lo, min(acc[a][b][r], acc[a][b][r + 1]));
                        }
                const uint32_t mx = max((uint32_t)hi, 0u - (uint32_t)lo);
                tmax = mx ? ea0 + eb0 + mant_shift32(mx, wq) : NEED_NONE;
            } else if (!ep.ea.row) {
                // one row exponent, per-column ones: a column's largest |acc|
                // decides its need
                tmax = NEED_NONE;
#pragma unroll
                for (int b = 0; b < NI; ++b) {
                    int v[16 * MI];
#pragma unroll
                    for (int a = 0; a < MI; ++a)
#pragma unroll
                        for (int r = 0; r < 16; ++r) v[16 * a + r] = acc[a][b][r];
                    const uint32_t mx = max_mag(v);
                    tmax = max(tmax, mx ? ea0 + ebv[b] + mant_shift32(mx, wq) : NEED_NONE);
                }
            } else if (!ep.eb.row) {
                // per-row exponents, one column exponent: a row's largest |acc|
                tmax = NEED_NONE;
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int v[2 * NI];
#pragma unroll
                        for (int b = 0; b < NI; ++b) v[2 * b] = v[2 * b + 1] = acc[a][b][r];
                        const uint32_t mx = max_mag(v);
                        tmax = max(tmax, mx ? seA[TR(a, r)] + eb0 + mant_shift32(mx, wq) : NEED_NONE);
                    }
            } else {
                tmax = NEED_NONE;
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int eav = seA[TR(a, r)];
#pragma unroll
                        for (int b = 0; b < NI; ++b) tmax = max(tmax, need32(acc[a][b][r], eav + ebv[b], wq));
                    }
            }
            tmax = wave_max(tmax);
            if (lane == 0) red[wave] = tmax;
            __syncthreads();
            const int gmax = max(max(red[0], red[1]), max(red[2], red[3]));
            if (mode == EPI_MAX) return gmax;  // nothing stored in the first pass
            // the result's exponent (direct) or the round-to-odd position
            int e = 0, p = 0;
            if (direct) {
                e = clamp_exp_flag(max(E_MIN, gmax), ep.flags);
                if (tid == 0 && bid == 0) ep.out_exp[0] = (int8_t)e;
            } else {
                // round to odd two bits below the tile's own need; the tile's
                // need goes to p16, where the second pass takes the maximum
                p = gmax == NEED_NONE ? P_NONE : gmax - 2;
                if (tid == 0) ep.p16[tile_m + TM * tile_n] = (int16_t)(gmax == NEED_NONE ? P_NONE : gmax);
            }
            if (uni) {
                // one shift for the whole tile: a * 2^-t with t in [-31, 31]
                int t = (direct ? e : p) - (ea0 + eb0);
                t = t > 31 ? 31 : (t < -31 ? -31 : t);
                if (t <= 0) {
                    const int l = -t;
#pragma unroll
                    for (int a = 0; a < MI; ++a)
#pragma unroll
                        for (int b = 0; b < NI; ++b)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                if (direct) stage(ES1{}, a, b, r, acc[a][b][r] << l);
                                else stage(ES2{}, a, b, r, acc[a][b][r] << l);
                            }
                } else if (direct) {
                    const int hm1 = (1 << (t - 1)) - 1;
#pragma unroll
                    for (int a = 0; a < MI; ++a)
#pragma unroll
                        for (int b = 0; b < NI; ++b)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int v = acc[a][b][r];
                                stage(ES1{}, a, b, r, (v + hm1 + ((v >> t) & 1)) >> t);
                            }
                } else {
                    // sticky bit: any of the t bits shifted out (t in [1, 31])
                    const int tl = 32 - t;
#pragma unroll
                    for (int a = 0; a < MI; ++a)
#pragma unroll
                        for (int b = 0; b < NI; ++b)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int v = acc[a][b][r];
                                const int sticky = (int)min((uint32_t)v << tl, 1u);
                                stage(ES2{}, a, b, r, (v >> t) | sticky);
                            }
                }
            } else {
                // the shift of a value depends on its column (one row
                // exponent), on its row (one column exponent), or on both
                auto elems = [&](auto dir_tag) {
                    constexpr bool DIR = decltype(dir_tag)::value;
                    const int tgt = DIR ? e : p;
                    if (!ep.ea.row) {
#pragma unroll
                        for (int b = 0; b < NI; ++b) {
                            const int sh = tgt - ea0 - ebv[b];
                            if constexpr (DIR) {
                                const RneP q = rne_prep(sh);
#pragma unroll
                                for (int a = 0; a < MI; ++a)
#pragma unroll
                                    for (int r = 0; r < 16; ++r) stage(ES1{}, a, b, r, rne_apply(acc[a][b][r], q));
                            } else {
                                const RtoP q = rto_prep(sh);
#pragma unroll
                                for (int a = 0; a < MI; ++a)
#pragma unroll
                                    for (int r = 0; r < 16; ++r) stage(ES2{}, a, b, r, rto_apply(acc[a][b][r], q));
                            }
                        }
                    } else if (!ep.eb.row) {
#pragma unroll
                        for (int a = 0; a < MI; ++a)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int sh = tgt - seA[TR(a, r)] - eb0;
                                if constexpr (DIR) {
                                    const RneP q = rne_prep(sh);
#pragma unroll
                                    for (int b = 0; b < NI; ++b) stage(ES1{}, a, b, r, rne_apply(acc[a][b][r], q));
                                } else {
                                    const RtoP q = rto_prep(sh);
#pragma unroll
                                    for (int b = 0; b < NI; ++b) stage(ES2{}, a, b, r, rto_apply(acc[a][b][r], q));
                                }
                            }
                    } else {
#pragma unroll
                        for (int a = 0; a < MI; ++a)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int off = tgt - seA[TR(a, r)];
#pragma unroll
                                for (int b = 0; b < NI; ++b) {
                                    if constexpr (DIR) stage(ES1{}, a, b, r, rne_bf(acc[a][b][r], off - ebv[b]));
                                    else stage(ES2{}, a, b, r, rto_bf(acc[a][b][r], off - ebv[b]));
                                }
                            }
                    }
                };
                if (direct) elems(std::true_type{});
                else elems(std::false_type{});
            }
        } else {
            // row groups.  The float path (contractions of at most 1024, so
            // |acc| <= 2^24 converts to fp32 exactly, and a column-exponent
            // spread of at most 96 within the tile) compares |acc| 2^(eb - ebmin)
            // in fp32 and rounds by an exact power-of-two scaling; otherwise
            // every element's need and shift are computed in integers.
            int *rowi = scr - 2 * BMt;              // per tile row: integer offset
            float *rowf = (float *)(scr - BMt);     //   or fp32 scale
            int lo = ebv[0], hi = ebv[0];
#pragma unroll
            for (int b = 1; b < NI; ++b) {
                lo = min(lo, ebv[b]);
                hi = max(hi, ebv[b]);
            }
            lo = -wave_max(-lo);
            hi = wave_max(hi);
            if (lane == 0) {
                scr[wave] = lo;
                scr[4 + wave] = hi;
            }
            __syncthreads();
            const int ebmin = min(min(scr[0], scr[1]), min(scr[2], scr[3]));
            const int ebmax = max(max(scr[4], scr[5]), max(scr[6], scr[7]));
            const bool fpath = ke - kb <= 1024 && ebmax - ebmin <= 96;
            float cs[NI];
#pragma unroll
            for (int b = 0; b < NI; ++b) cs[b] = __builtin_ldexpf(1.0f, fpath ? ebv[b] - ebmin : 0);

            // 1. per-row maxima (fp32 bit patterns of non-negative values, or needs)
#pragma unroll
            for (int a = 0; a < MI; ++a) {
                int key[16];
                if (fpath) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float m = 0.f;
#pragma unroll
                        for (int b = 0; b < NI; ++b) m = fmaxf(m, fabsf((float)acc[a][b][r] * cs[b]));
                        key[r] = __float_as_int(m);
                    }
                } else if (!ep.eb.row) {
                    // one column exponent: the row's largest |acc| decides
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int v[2 * NI];
#pragma unroll
                        for (int b = 0; b < NI; ++b) v[2 * b] = v[2 * b + 1] = acc[a][b][r];
                        const uint32_t mx = max_mag(v);
                        key[r] = mx ? seA[TR(a, r)] + eb0 + mant_shift32(mx, wq) : NEED_NONE;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int eav = seA[TR(a, r)];
                        int m = NEED_NONE;
#pragma unroll
                        for (int b = 0; b < NI; ++b) m = max(m, need32(acc[a][b][r], eav + ebv[b], wq));
                        key[r] = m;
                    }
                }
                const int k = rows16_max(key, lane);
                if ((lane & 1) == 0) {
                    const int rr = rows16_row(lane);
                    red[wn * BMt + tr0 + a * 32 + 8 * (rr >> 2) + (rr & 3)] = k;
                }
            }
            __syncthreads();
            // 2. one thread per tile row: the row's exponent, and the offset
            //    (integer path) or scale (float path) its elements use
            const int n_ct = (N + BNt - 1) / BNt;
            bool ovf = false;
            for (int tr = tid; tr < BMt; tr += NTHR) {
                const int row = m0 + tr;
                const int kmax = max(red[tr], red[BMt + tr]);
                const int eav = seA[tr];
                int rm, s = 0;
                if (fpath) {
                    // need of m = |acc| 2^(eb - ebmin) from its fp32 exponent and top
                    // mantissa bits: bit length - wq, plus one when the top wq + 1
                    // bits are all ones (m at or above (2^(wq+1) - 1) 2^(len - wq - 1))
                    const int ones = (1 << wq) - 1;
                    s = ((kmax >> 23) - 127) - (wq - 1) + (((kmax >> (23 - wq)) & ones) == ones);
                    rm = kmax == 0 ? NEED_NONE : eav + ebmin + s;
                } else {
                    rm = kmax;
                }
                if (mode == EPI_MAX) {
                    // first pass: this (row, column tile)'s need only
                    if (row < M) ep.tneed[(long long)row * n_ct + tile_n] = rm;
                    continue;
                }
                if (mode == EPI_GIVEN) {
                    // second pass: the row's exponent from every column tile's need
                    rm = NEED_NONE;
                    if (row < M)
                        for (int j = 0; j < n_ct; ++j) rm = max(rm, ep.tneed[(long long)row * n_ct + j]);
                }
                int tgt;
                if (direct) {
                    tgt = max(E_MIN, rm);
                    ovf |= tgt > E_MAX;
                    tgt = min(tgt, E_MAX);
                    if (row < M && tile_n == 0) ep.out_exp[row] = (int8_t)tgt;
                    // an all-zero row would otherwise scale by up to 2^254
                    // (inf, and 0 * inf is NaN); its results are 0
                    rowf[tr] = rm == NEED_NONE ? 0.0f : __builtin_ldexpf(1.0f, eav + ebmin - tgt);
                } else {
                    tgt = rm == NEED_NONE ? P_NONE : rm - 2;
                    if (row < M) ep.p16[(long long)row * n_ct + tile_n] = (int16_t)(rm == NEED_NONE ? P_NONE : rm);
                    rowf[tr] = rm == NEED_NONE ? 1.0f : __builtin_ldexpf(1.0f, 2 - s);
                }
                rowi[tr] = tgt - eav;
            }
            if (ovf) atomicOr(ep.flags, 1u);
            __syncthreads();
            if (mode == EPI_MAX) return NEED_NONE;  // nothing stored in the first pass
            // 3. the elements, with the mode and the path fixed per instance
            auto elems = [&](auto dir_tag, auto fp_tag) {
                constexpr bool DIR = decltype(dir_tag)::value, FP = decltype(fp_tag)::value;
#pragma unroll
                for (int a = 0; a < MI; ++a)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int tr = TR(a, r);
                        if constexpr (FP) {
                            // acc 2^(eps - target), exact in fp32 (or below 2^-126,
                            // where the result is 0 either way)
                            const float rs = rowf[tr];
#pragma unroll
                            for (int b = 0; b < NI; ++b) {
                                const float y = (float)acc[a][b][r] * cs[b] * rs;
                                if constexpr (DIR) {
                                    stage(ES1{}, a, b, r, (int)__builtin_rintf(y));
                                } else {
                                    const float q = floorf(y);
                                    stage(ES2{}, a, b, r, (int)q | (int)(y != q));
                                }
                            }
                        } else if (!ep.eb.row) {
                            // one column exponent: one shift for the row
                            if constexpr (DIR) {
                                const RneP q = rne_prep(rowi[tr] - eb0);
#pragma unroll
                                for (int b = 0; b < NI; ++b) stage(ES1{}, a, b, r, rne_apply(acc[a][b][r], q));
                            } else {
                                const RtoP q = rto_prep(rowi[tr] - eb0);
#pragma unroll
                                for (int b = 0; b < NI; ++b) stage(ES2{}, a, b, r, rto_apply(acc[a][b][r], q));
                            }
                        } else {
                            const int off = rowi[tr];
#pragma unroll
                            for (int b = 0; b < NI; ++b) {
                                if constexpr (DIR) stage(ES1{}, a, b, r, rne_bf(acc[a][b][r], off - ebv[b]));
                                else stage(ES2{}, a, b, r, rto_bf(acc[a][b][r], off - ebv[b]));
                            }
                        }
                    }
            };
            if (direct) {
                if (fpath) elems(std::true_type{}, std::true_type{});
                else elems(std::true_type{}, std::false_type{});
            } else {
                if (fpath) elems(std::false_type{}, std::true_type{});
                else elems(std::false_type{}, std::false_type{});
            }
        }
        __syncthreads();
        if (direct)
            flush(ES1{}, ep.out, N, (N & 15) == 0 && ((uintptr_t)ep.out & 15) == 0 && act_aligned(ep.act, 16));
        else flush(ES2{}, ep.v16, N, (N & 7) == 0);
        return NEED_NONE;
    }
}

// ONE: the contraction is at most one step (K <= BK; not for split
// contractions), so the tile loads it once into a single LDS stage and more
// workgroups fit a CU.
// RG: the result groups it is built for (0 whole tensor, 1 rows); DI: its
// epilogue (1 int8 in this pass, 0 round to odd).  Split products, whose
// int32 partials have neither yet, take 0 and 0.
template <int KA, int KB, int MI, int NI, bool PARTIAL, bool ONE, int RG, int DI>
__global__ __launch_bounds__(NTHR, (ONE ? Occ1<MI, NI>::value : Occ<MI, NI>::value)) void gemm_i8_kernel(
    Operand A, Operand B, int M, int N, int K, int k_chunk, int TM, int S, Epi ep) {
    static_assert(!(ONE && PARTIAL), "one-step tiles have no split form");
    __shared__ __attribute__((aligned(16)))
    int8_t lds[ONE ? TileLds1<KA, KB, MI, NI>::value : TileLds<KA, KB, MI, NI, PARTIAL>::value];
    gemm_tile<KA, KB, MI, NI, PARTIAL, ONE, -1, RG, DI>(A, B, M, N, K, k_chunk, TM, S, ep, blockIdx.x, gridDim.x,
                                                        lds);
}

// Kind codes of kernels built for row groups: the code of the whole-tensor
// kernel plus ROW_KIND.
constexpr int ROW_KIND = 200000000;

// Kind codes of one-step kernels for the timing records: the code of the
// plain kernel plus ONE_KIND.
constexpr int ONE_KIND = 99000000;

// First pass of a recomputed product (EPI_MAX): a persistent grid walks the
// tiles (item = blockIdx.x + j * gridDim.x; gridDim.x a multiple of 8 keeps
// item % 8 on the workgroup's XCD), finding group maxima without storing
// values.  Whole-tensor groups: each workgroup writes its running maximum to
// tneed[blockIdx.x]; row groups: the tiles write tneed[row][column tile].
template <int KA, int KB, int MI, int NI, bool ONE, int RG>
__global__ __launch_bounds__(NTHR, (ONE ? Occ1<MI, NI>::value : Occ<MI, NI>::value)) void gemm_max_kernel(
    Operand A, Operand B, int M, int N, int K, int TM, int items, Epi ep) {
    __shared__ __attribute__((aligned(16)))
    int8_t lds[ONE ? TileLds1<KA, KB, MI, NI>::value : TileLds<KA, KB, MI, NI, false>::value];
    int run = NEED_NONE;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        run = max(run, gemm_tile<KA, KB, MI, NI, false, ONE, EPI_MAX, RG>(A, B, M, N, K, K, TM, 1, ep, item, items,
                                                                          lds));
        __syncthreads();  // the next item's stages reuse the LDS
    }
    if (RG == 0 && threadIdx.x == 0) ep.tneed[blockIdx.x] = run;
}

template <int KA, int KB, int MI, int NI>
hipError_t launch_max(const Operand &A, const Operand &B, int M, int N, int K, const Epi &ep, hipStream_t st) {
    const int TM = (M + 64 * MI - 1) / (64 * MI), TN = (N + 64 * NI - 1) / (64 * NI);
    const int items = TM * TN;
    const int grid = recomp_grid(M, N, K, Tile{MI, NI});
    if (grid <= 0) return hipSuccess;
    if (!ep.row_group && ep.tneed_n != grid) return hipErrorInvalidValue;
    const bool one = K <= BK;
    const int kind = 10000 * (10 * MI + NI) + 1000 + 100 * EPI_MAX + 10 * KA + KB + (one ? ONE_KIND : 0) +
                     (ep.row_group ? ROW_KIND : 0);
    prof_begin(st, kind);
    auto go = [&](auto one_tag, auto rg_tag) {
        constexpr bool O = decltype(one_tag)::value;
        constexpr int R = decltype(rg_tag)::value;
        hipLaunchKernelGGL((gemm_max_kernel<KA, KB, MI, NI, O, R>), dim3(grid), dim3(NTHR), 0, st, A, B, M, N, K,
                           TM, items, ep);
    };
    using T1 = std::true_type;
    using F1 = std::false_type;
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    if (one) {
        if (ep.row_group) go(T1{}, R1{});
        else go(T1{}, R0{});
    } else {
        if (ep.row_group) go(F1{}, R1{});
        else go(F1{}, R0{});
    }
    prof_end(st, kind);
    return hipGetLastError();
}

// Two independent products in one grid: the first part's workgroups (a
// round-to-odd or direct product), padded to a multiple of 8 so that the
// second part's work order still meets the XCDs as planned, then the second
// part's (a split contraction).  One launch instead of two streams joined
// by events.
struct PairPart {
    Operand A, B;
    int M, N, K, k_chunk, TM, S, nblk;
    Epi ep;
};

template <int KA1, int KB1, int MI1, int NI1, int KA2, int KB2, int MI2, int NI2>
__global__ __launch_bounds__(NTHR, (Occ<MI1, NI1>::value < Occ<MI2, NI2>::value ? Occ<MI1, NI1>::value
                                                                                : Occ<MI2, NI2>::value))
void gemm_pair_kernel(PairPart p1, PairPart p2, int g1) {
    constexpr int L1 = TileLds<KA1, KB1, MI1, NI1>::value, L2 = TileLds<KA2, KB2, MI2, NI2>::value;
    __shared__ __attribute__((aligned(16))) int8_t lds[L1 > L2 ? L1 : L2];
    const int b = blockIdx.x;
    if (b < g1) {
        if (b < p1.nblk)
            gemm_tile<KA1, KB1, MI1, NI1, false, false, -1, 0>(p1.A, p1.B, p1.M, p1.N, p1.K, p1.k_chunk, p1.TM,
                                                                 p1.S, p1.ep, b, p1.nblk, lds);
    } else {
        gemm_tile<KA2, KB2, MI2, NI2, true>(p2.A, p2.B, p2.M, p2.N, p2.K, p2.k_chunk, p2.TM, p2.S, p2.ep, b - g1,
                                            p2.nblk, lds);
    }
}

// Part descriptor of a product of tile (MI, NI).
inline PairPart pair_part(const Operand &A, const Operand &B, int M, int N, int K, int MI, int NI, int splits,
                          int k_chunk, const Epi &ep) {
    PairPart p;
    p.A = A;
    p.B = B;
    p.M = M;
    p.N = N;
    p.K = K;
    p.k_chunk = k_chunk;
    p.TM = (M + 64 * MI - 1) / (64 * MI);
    p.S = splits;
    p.nblk = p.TM * ((N + 64 * NI - 1) / (64 * NI)) * splits;
    p.ep = ep;
    return p;
}

template <int KA1, int KB1, int MI1, int NI1, int KA2, int KB2, int MI2, int NI2>
hipError_t launch_pair(const PairPart &p1, const PairPart &p2, hipStream_t st) {
    // the input-gradient part is built for one whole-tensor group only
    if (p1.ep.row_group) return hipErrorInvalidValue;
    const int g1 = (p1.nblk + 7) / 8 * 8;
    const int kind = 1000000 * (10 * MI2 + NI2) + 10000 * (10 * MI1 + NI1) + 1000 + 100 * 3 + 10 * KA1 + KB1;
    prof_begin(st, kind);
    hipLaunchKernelGGL((gemm_pair_kernel<KA1, KB1, MI1, NI1, KA2, KB2, MI2, NI2>), dim3(g1 + p2.nblk), dim3(NTHR), 0,
                       st, p1, p2, g1);
    prof_end(st, kind);
    return hipGetLastError();
}

// The block index that work_of (one split) maps to logical tile L of T: its
// inverse, so that a caller can pick the tile and still run gemm_tile.
__device__ __forceinline__ int block_of_tile(int L, int T) {
    const int q = T / 8, r = T % 8;
    int x, j;
    if (L < r * (q + 1)) {
        x = L / (q + 1);
        j = L - x * (q + 1);
    } else {
        const int L2 = L - r * (q + 1);  // q >= 1 here: L < T
        x = r + L2 / q;
        j = L2 - (x - r) * q;
    }
    return x + 8 * j;
}

// A stack of independent products (slice z = the batch index): the work of
// all slices is spread over the XCDs as one grid of Z * TM * TN tiles (a
// slice's tiles stay together), each workgroup shifts the operands, exponent
// sources and outputs to its slice and runs the plain tile.  ONE: the
// contraction is one step (K <= BK), so the tile needs half the LDS and twice
// the workgroups fit a CU.
template <int KA, int KB, int MI, int NI, bool ONE>
__global__ __launch_bounds__(NTHR, (Occ<MI, NI>::value)) void gemm_batched_kernel(Operand A, Operand B, int M, int N,
                                                                                int K, int TM, Epi ep, BatchArgs ba) {
    __shared__ __attribute__((aligned(16)))
    int8_t lds[ONE ? TileLds1<KA, KB, MI, NI>::value : TileLds<KA, KB, MI, NI>::value];
    const int TN = (N + 64 * NI - 1) / (64 * NI), T = TM * TN;
    int tm, tn, z;
    work_of(blockIdx.x, TM, TN, ba.Z, tm, tn, z);
    A.base += z * ba.a;
    B.base += z * ba.b;
    if (ep.ea.e8) ep.ea.e8 += z * ba.ea8;
    if (ep.ea.e32) ep.ea.e32 += z * ba.ea32;
    if (ep.eb.e8) ep.eb.e8 += z * ba.eb8;
    if (ep.eb.e32) ep.eb.e32 += z * ba.eb32;
    if (ep.out) ep.out += z * ba.out;
    if (ep.v16) ep.v16 += z * ba.out;
    if (ep.out_exp) ep.out_exp += z * ba.out_exp;
    if (ep.p16) ep.p16 += z * ba.p16;
    gemm_tile<KA, KB, MI, NI, false, ONE, -1, 1>(A, B, M, N, K, K, TM, 1, ep, block_of_tile(tm * TN + tn, T), T,
                                                 lds);
}

template <int KA, int KB, int MI, int NI, bool ONE = false>
hipError_t launch_batched_one(const Operand &A, const Operand &B, int M, int N, int K, const Epi &ep,
                              const BatchArgs &ba, hipStream_t st) {
    if (ONE && K > BK) return hipErrorInvalidValue;
    if (!ep.row_group) return hipErrorInvalidValue;  // the kernel is built for row groups only
    const int TM = (M + 64 * MI - 1) / (64 * MI), TN = (N + 64 * NI - 1) / (64 * NI);
    const long long blocks = (long long)TM * TN * ba.Z;
    if (blocks <= 0) return hipSuccess;
    if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
    const int kind = 10000 * (10 * MI + NI) + 1000 + 100 * ((ONE ? 6 : 4) + ep.mode) + 10 * KA + KB;
    prof_begin(st, kind);
    hipLaunchKernelGGL((gemm_batched_kernel<KA, KB, MI, NI, ONE>), dim3((int)blocks), dim3(NTHR), 0, st, A, B, M, N,
                       K, TM, ep, ba);
    prof_end(st, kind);
    return hipGetLastError();
}

template <int KA, int KB, int MI, int NI, bool PARTIAL>
hipError_t launch_one(const Operand &A, const Operand &B, int M, int N, int K, int splits, int k_chunk,
                      const Epi &ep, hipStream_t st) {
    const int TM = (M + 64 * MI - 1) / (64 * MI), TN = (N + 64 * NI - 1) / (64 * NI);
    dim3 grid(TM * TN * splits, 1, 1);
    const bool one = !PARTIAL && K <= BK;
    const bool rows = !PARTIAL && ep.row_group;
    const int kind = 10000 * (10 * MI + NI) + 1000 + 100 * (PARTIAL ? 2 : ep.mode) + 10 * KA + KB +
                     (one ? ONE_KIND : 0) + (rows ? ROW_KIND : 0);
    prof_begin(st, kind);
    if constexpr (!PARTIAL) {
        auto go = [&](auto one_tag, auto rg_tag, auto dir_tag) {
            constexpr bool O = decltype(one_tag)::value;
            constexpr int R = decltype(rg_tag)::value, D = decltype(dir_tag)::value;
            hipLaunchKernelGGL((gemm_i8_kernel<KA, KB, MI, NI, false, O, R, D>), grid, dim3(NTHR), 0, st, A, B, M,
                               N, K, k_chunk, TM, splits, ep);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        auto go2 = [&](auto one_tag, auto rg_tag) {
            if (ep.mode == EPI_RTO) go(one_tag, rg_tag, I0{});
            else go(one_tag, rg_tag, I1{});
        };
        if (one) {
            if (rows) go2(std::true_type{}, I1{});
            else go2(std::true_type{}, I0{});
        } else {
            if (rows) go2(std::false_type{}, I1{});
            else go2(std::false_type{}, I0{});
        }
    } else {
        hipLaunchKernelGGL((gemm_i8_kernel<KA, KB, MI, NI, true, false, 0, 0>), grid, dim3(NTHR), 0, st, A, B, M, N,
                           K, k_chunk, TM, splits, ep);
    }
    prof_end(st, kind);
    return hipGetLastError();
}

}  // namespace ie

// Dispatch over a tile list inside one translation unit.
#define IE_TILE_CASE(KA, KB, MI_, NI_)                                                                   \
    if (t.mi == MI_ && t.ni == NI_) {                                                                    \
        if (!partial && ep.mode == EPI_MAX) return launch_max<KA, KB, MI_, NI_>(A, B, M, N, K, ep, st);   \
        return partial ? launch_one<KA, KB, MI_, NI_, true>(A, B, M, N, K, splits, k_chunk, ep, st)       \
                       : launch_one<KA, KB, MI_, NI_, false>(A, B, M, N, K, splits, k_chunk, ep, st);     \
    }

#define IE_TILE_CASE_PARTIAL(KA, KB, MI_, NI_)                                                           \
    if (t.mi == MI_ && t.ni == NI_) {                                                                    \
        if (!partial) return hipErrorInvalidValue;                                                       \
        return launch_one<KA, KB, MI_, NI_, true>(A, B, M, N, K, splits, k_chunk, ep, st);               \
    }
