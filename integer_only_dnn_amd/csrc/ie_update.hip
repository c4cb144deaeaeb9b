// Integer SGD with momentum and per-group velocity ("Memory-Efficient
// Integer-Only Training of Deep Neural Networks", Figure 1b and Table 5).
//
// For every velocity group (one row = one output channel):
//   v = momentum * V + G          exact, then V' = requantised into V's group
//   w = W - lr * V'               exact, then W' = requantised into W's group
// momentum and lr are (C, e) scalars.  One wave owns one row; the row's
// bytes of W, V and G stay in registers between the two steps.
//
// Exact two-term sums X*2^pa + Y*2^pb (|X|, |Y| <= 2^14): when the exponent
// gap is at most 15 the sum fits int32 at the smaller exponent.  Otherwise it
// is formed in int64; for gaps above 40 the smaller term (below 2^(P-9) in
// magnitude, P the larger term's exponent) can only decide a rounding tie
// or a sticky bit, so it is replaced by sign(Y) * 2^(P-24), which rounds
// identically at every exponent the group can take (every such exponent is
// at least P - 7, where the larger term dominates).
#include "ie_device.h"
#include "ie_internal.h"

namespace ie {

struct Ex64 {
    long long n;
    int base;
};

__device__ __forceinline__ Ex64 combine64(int X, int pa, int Y, int pb) {
    if (X == 0) return {(long long)Y, pb};
    if (Y == 0) return {(long long)X, pa};
    int d = pa - pb;
    if (d >= 0) {
        if (d <= 40) return {((long long)X << d) + Y, pb};
        return {((long long)X << 24) + (Y > 0 ? 1 : -1), pa - 24};
    }
    d = -d;
    if (d <= 40) return {(long long)X + ((long long)Y << d), pa};
    return {((long long)Y << 24) + (X > 0 ? 1 : -1), pb - 24};
}

__device__ __forceinline__ int sbyte(uint32_t w, int j) { return (int)(int8_t)(w >> (8 * j)); }

__device__ __forceinline__ int wave_max64(int v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ uint32_t load_dw(const int8_t *row, long long col, long long cols, int vec) {
    if (vec && col + 4 <= cols) return *(const uint32_t *)(row + col);
    uint32_t w = 0;
    for (int j = 0; j < 4; ++j)
        if (col + j < cols) w |= (uint32_t)(uint8_t)row[col + j] << (8 * j);
    return w;
}

__device__ __forceinline__ void store_dw(int8_t *row, long long col, long long cols, int vec, uint32_t w) {
    if (vec && col + 4 <= cols) {
        *(uint32_t *)(row + col) = w;
        return;
    }
    for (int j = 0; j < 4; ++j)
        if (col + j < cols) row[col + j] = (int8_t)(w >> (8 * j));
}

// The wide (int64) forms are out of line: rows with exponent gaps above 15
// are rare and the inlined code would multiply the kernel size.
__device__ __noinline__ int sum_need_wide(int X, int pa, int Y, int pb) {
    Ex64 s = combine64(X, pa, Y, pb);
    return need64(s.n, s.base);
}

__device__ __noinline__ int sum_round_wide(int X, int pa, int Y, int pb, int e) {
    Ex64 s = combine64(X, pa, Y, pb);
    return (int)rne_shift64(s.n, e - s.base);
}

// Smallest exponent / rounding of X*2^pa + Y*2^pb, using the int32 form
// when `narrow` (|pa - pb| <= 15, uniform over the row).
__device__ __forceinline__ int sum_need(bool narrow, int X, int pa, int Y, int pb) {
    if (narrow) {
        int base = min(pa, pb);
        int n = (X << (pa - base)) + (Y << (pb - base));
        return need32(n, base);
    }
    return sum_need_wide(X, pa, Y, pb);
}

__device__ __forceinline__ int sum_round(bool narrow, int X, int pa, int Y, int pb, int e) {
    if (narrow) {
        int base = min(pa, pb);
        int n = (X << (pa - base)) + (Y << (pb - base));
        return rne_shift32(n, e - base);
    }
    return sum_round_wide(X, pa, Y, pb, e);
}

// pass 0: whole-tensor velocity, raise gneed_v with the velocity's needs.
// pass 1: velocity and (row-grouped) weight step; for a whole-tensor weight,
//         store V' and raise gneed_w.
// pass 2: whole-tensor weight, round W with gneed_w.
template <int D>
__global__ __launch_bounds__(256) void sgd_rows_kernel(UpdateArgs a, int pass, int vec, const int *old_ev,
                                                      const int *old_ew) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool v_tensor = a.v_row == 0, w_tensor = a.w_row == 0;
    for (long long row = (long long)blockIdx.x * 4 + wave; row < a.rows; row += (long long)gridDim.x * 4) {
        const long long off = row * a.cols;
        uint32_t W[D], V[D], G[D];
#pragma unroll
        for (int j = 0; j < D; ++j) {
            long long col = 4ll * (lane + 64 * j);
            W[j] = (pass != 0) ? load_dw(a.w + off, col, a.cols, vec) : 0u;
            V[j] = load_dw(a.v + off, col, a.cols, vec);
            G[j] = (pass != 2) ? load_dw(a.g + off, col, a.cols, vec) : 0u;
        }
        const int ew = w_tensor ? *old_ew : (int)a.w_exp[row];
        if (pass == 2) {
            // V already holds V' with its new exponent
            const int evn = v_tensor ? clamp_exp_flag(max(E_MIN, *a.gneed_v), a.flags) : (int)a.v_exp[row];
            const int pb = a.lr_e + evn;
            const bool nw = abs(ew - pb) <= 15;
            const int e = clamp_exp_flag(max(E_MIN, *a.gneed_w), a.flags);
#pragma unroll
            for (int j = 0; j < D; ++j) {
                uint32_t o = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    int c = sum_round(nw, sbyte(W[j], t), ew, -a.lr_m * sbyte(V[j], t), pb, e);
                    o |= (uint32_t)(uint8_t)c << (8 * t);
                }
                store_dw(a.w + off, 4ll * (lane + 64 * j), a.cols, vec, o);
            }
            if (row == 0 && lane == 0) a.w_exp[0] = (int8_t)e;
            continue;
        }
        const int ev = v_tensor ? *old_ev : (int)a.v_exp[row];
        const int eg = a.g_row ? (int)a.g_exp[row] : (int)a.g_exp[0];
        const int pa = ev + a.mom_e, pb = eg;
        const bool nv = abs(pa - pb) <= 15;
        int m = NEED_NONE;
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                m = max(m, sum_need(nv, a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb));
        if (pass == 0) {
            m = wave_max64(m);
            if (lane == 0 && m != NEED_NONE && m > __atomic_load_n(a.gneed_v, __ATOMIC_RELAXED)) atomicMax(a.gneed_v, m);
            continue;
        }
        int evn;
        if (v_tensor) {
            evn = clamp_exp_flag(max(E_MIN, *a.gneed_v), a.flags);
        } else {
            evn = clamp_exp_flag(max(E_MIN, wave_max64(m)), a.flags);
        }
        // V' and the weight step's needs
        const int pw = a.lr_e + evn;
        const bool nw = abs(ew - pw) <= 15;
        uint32_t Vn[D];
        int mw = NEED_NONE;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            uint32_t o = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                int c = sum_round(nv, a.mom_m * sbyte(V[j], t), pa, sbyte(G[j], t), pb, evn);
                o |= (uint32_t)(uint8_t)c << (8 * t);
                mw = max(mw, sum_need(nw, sbyte(W[j], t), ew, -a.lr_m * c, pw));
            }
            Vn[j] = o;
        }
#pragma unroll
        for (int j = 0; j < D; ++j) store_dw(a.v + off, 4ll * (lane + 64 * j), a.cols, vec, Vn[j]);
        if (lane == 0) {
            if (!v_tensor) a.v_exp[row] = (int8_t)evn;
            else if (row == 0) a.v_exp[0] = (int8_t)evn;
        }
        mw = wave_max64(mw);
        if (w_tensor) {
            if (lane == 0 && mw != NEED_NONE && mw > __atomic_load_n(a.gneed_w, __ATOMIC_RELAXED)) atomicMax(a.gneed_w, mw);
            continue;
        }
        const int ewn = clamp_exp_flag(max(E_MIN, mw), a.flags);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            uint32_t o = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                int c = sum_round(nw, sbyte(W[j], t), ew, -a.lr_m * sbyte(Vn[j], t), pw, ewn);
                o |= (uint32_t)(uint8_t)c << (8 * t);
            }
            store_dw(a.w + off, 4ll * (lane + 64 * j), a.cols, vec, o);
        }
        if (lane == 0) a.w_exp[row] = (int8_t)ewn;
    }
}

template <int D>
static hipError_t run_passes(const UpdateArgs &a, int vec, const int *old_ev, const int *old_ew, hipStream_t st) {
    long long blocks = (a.rows + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipError_t err;
    if (a.v_row == 0) {
        prof_begin(st);
        hipLaunchKernelGGL((sgd_rows_kernel<D>), dim3((int)blocks), dim3(256), 0, st, a, 0, vec, old_ev, old_ew);
        prof_end(st, 2000 + 0);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    prof_begin(st);
    hipLaunchKernelGGL((sgd_rows_kernel<D>), dim3((int)blocks), dim3(256), 0, st, a, 1, vec, old_ev, old_ew);
    prof_end(st, 2000 + 1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.w_row == 0) {
        prof_begin(st);
        hipLaunchKernelGGL((sgd_rows_kernel<D>), dim3((int)blocks), dim3(256), 0, st, a, 2, vec, old_ev, old_ew);
        prof_end(st, 2000 + 2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

// Workspace ints used here: gneed_v, gneed_w and two snapshots of the old
// whole-tensor exponents, which later passes must not read back after the
// first pass has overwritten the exponent byte.
hipError_t launch_sgd_update(const UpdateArgs &a, hipStream_t st) {
    int *old_ev = a.gneed_v + 2, *old_ew = a.gneed_v + 3;
    hipError_t err;
    if ((err = launch_fill_i32(a.gneed_v, 2, NEED_NONE, st)) != hipSuccess) return err;
    if (a.v_row == 0 && (err = launch_exp_max(a.v_exp, 1, old_ev, st)) != hipSuccess) return err;
    if (a.w_row == 0 && (err = launch_exp_max(a.w_exp, 1, old_ew, st)) != hipSuccess) return err;
    if (a.rows <= 0) {
        // Empty tensor: whole-tensor groups are all-zero.
        if (a.v_row == 0 && (err = launch_fill_i8(a.v_exp, 1, E_MIN, st)) != hipSuccess) return err;
        if (a.w_row == 0 && (err = launch_fill_i8(a.w_exp, 1, E_MIN, st)) != hipSuccess) return err;
        return hipSuccess;
    }
    int vec = (a.cols % 4 == 0) && ((uintptr_t)a.w % 4 == 0) && ((uintptr_t)a.v % 4 == 0) &&
              ((uintptr_t)a.g % 4 == 0);
    long long dw = (a.cols + 3) / 4;
    long long per_lane = (dw + 63) / 64;
    if (per_lane <= 1) return run_passes<1>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 2) return run_passes<2>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 3) return run_passes<3>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 4) return run_passes<4>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 6) return run_passes<6>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 8) return run_passes<8>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 12) return run_passes<12>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 16) return run_passes<16>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 18) return run_passes<18>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 24) return run_passes<24>(a, vec, old_ev, old_ew, st);
    if (per_lane <= 32) return run_passes<32>(a, vec, old_ev, old_ew, st);
    return hipErrorInvalidValue;
}

}  // namespace ie
