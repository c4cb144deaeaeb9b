// Device-side integer helpers of the (C, e) arithmetic, for gfx950.
//
// Number format ("Memory-Efficient Integer-Only Training of Deep Neural
// Networks", Abstract, Figure 1): value = C * 2^e, C an int8 mantissa, e an
// int8 exponent.  Every right shift rounds half to even; a group's exponent is
// the smallest one that brings every |C| to 127 or less.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ie {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int E_MIN = -128;
constexpr int E_MAX = 127;
// "No nonzero value": below every reachable exponent, above int overflow.
constexpr int NEED_NONE = -(1 << 28);
// Sentinel provisional exponent of an all-zero row tile (fits int16).
constexpr int P_NONE = -30000;

// Smallest s with |rne(m / 2^s)| <= 2^q - 1 (q = B - 1 for a B-bit mantissa,
// 7 for INT8), for m = |a| > 0 (32-bit).  With b the bit length of m, the
// answer is b - q, plus one when the top q + 1 bits of m are all ones
// (m / 2^(b-q) >= 2^q - 0.5 rounds up to 2^q).
__device__ __forceinline__ int mant_shift32(uint32_t m, int q = 7) {
    int z = __clz(m);
    uint32_t top = (m << z) >> (31 - q);
    return 32 - z - q + (top == (2u << q) - 1u ? 1 : 0);
}

__device__ __forceinline__ int mant_shift64(uint64_t m, int q = 7) {
    int z = __clzll(m);
    uint32_t top = (uint32_t)((m << z) >> (63 - q));
    return 64 - z - q + (top == (2u << q) - 1u ? 1 : 0);
}

// Smallest exponent for the exact value a * 2^eps; NEED_NONE when a == 0.
__device__ __forceinline__ int need32(int a, int eps, int q = 7) {
    uint32_t m = (uint32_t)(a < 0 ? -a : a);
    return m ? eps + mant_shift32(m, q) : NEED_NONE;
}

__device__ __forceinline__ int need64(long long a, int eps, int q = 7) {
    uint64_t m = (uint64_t)(a < 0 ? -a : a);
    return m ? eps + mant_shift64(m, q) : NEED_NONE;
}

// a * 2^-s rounded half to even, |a| < 2^30.  s <= 0 is an exact left shift
// (callers guarantee the result fits); s >= 31 gives 0.
__device__ __forceinline__ int rne_shift32(int a, int s) {
    s = s > 31 ? 31 : (s < -31 ? -31 : s);
    if (s <= 0) return a << (-s);
    int bit = (a >> s) & 1;
    return (a + (1 << (s - 1)) - 1 + bit) >> s;
}

// 64-bit version, |a| < 2^62; s >= 63 gives 0.
__device__ __forceinline__ long long rne_shift64(long long a, int s) {
    s = s > 63 ? 63 : (s < -63 ? -63 : s);
    if (s <= 0) return a << (-s);
    long long bit = (a >> s) & 1;
    return (a + (1ll << (s - 1)) - 1 + bit) >> s;
}

// Round to odd at 2^t: floor(a / 2^t) with the lowest bit forced to 1 when
// any discarded bit is nonzero.  Followed by a half-to-even rounding at least
// two bits higher, this gives the same result as rounding a directly.
__device__ __forceinline__ int rto_shift32(int a, int t) {
    t = t > 31 ? 31 : (t < -31 ? -31 : t);
    if (t <= 0) return a << (-t);
    int q = a >> t;
    int sticky = (a & (int)((1u << t) - 1u)) != 0;
    return q | sticky;
}

// ReLU of four packed int8 mantissas (Table 7: the exponent is kept): the
// negative bytes become zero.
__device__ __forceinline__ uint32_t relu4(uint32_t w) {
    const uint32_t neg = (w & 0x80808080u) >> 7;
    return w & ~(neg * 0xffu);
}

// The activation applied to rounded int8 results, their exponents kept
// (Table 7): ReLU of the results themselves (forward products), or the
// backward of a ReLU whose output is `mask`, laid out like the results
// (input gradients: a result stays where the matching mask byte is
// positive, else it becomes zero).
struct Act {
    int relu;
    const int8_t *mask;
};

// The bytes of w whose matching byte of x is positive; the others zero.
__device__ __forceinline__ uint32_t pos_mask4(uint32_t w, uint32_t x) {
    const uint32_t nz = ((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) & 0x80808080u;  // low seven bits not all zero
    return w & (((nz & ~x) >> 7) * 0xffu);                                // ... and the sign bit clear
}

// Four results at out + o (o a multiple of 4 when a.mask is set; the mask
// 4-byte aligned).
__device__ __forceinline__ uint32_t act4(uint32_t w, const Act &a, long long o) {
    if (a.relu) w = relu4(w);
    if (a.mask) w = pos_mask4(w, *(const uint32_t *)(a.mask + o));
    return w;
}

// One result at out + o.
__device__ __forceinline__ int act1(int c, const Act &a, long long o) {
    if (a.relu && c < 0) c = 0;
    if (a.mask && a.mask[o] <= 0) c = 0;
    return c;
}

// Whether 4-byte (8-byte) result groups at multiples of 4 (8) may take the
// vector forms: the mask, if any, aligned like the results.
__host__ __device__ inline bool act_aligned(const Act &a, int bytes) { return !a.mask || ((uintptr_t)a.mask % bytes) == 0; }

__device__ __forceinline__ int clamp_exp_flag(int e, uint32_t *flags) {
    if (e < E_MIN) e = E_MIN;
    if (e > E_MAX) {
        atomicOr(flags, 1u);
        e = E_MAX;
    }
    return e;
}

// Maximum over the 64 lanes of a wave, returned in every lane (all lanes
// active).  DPP row shifts by 1, 2, 4, 8 leave each 16-lane row's maximum in
// its lane 15; row broadcasts 15 and 31 carry it across the rows to lane 63,
// which is read back.  Lanes whose DPP source is outside the row keep `lo`.
__device__ __forceinline__ int wave_max_dpp(int v) {
    constexpr int lo = (int)0x80000000;
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x118, 0xf, 0xf, false));  // row_shr:8
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x142, 0xa, 0xf, false));  // row_bcast:15 -> rows 1, 3
    v = max(v, __builtin_amdgcn_update_dpp(lo, v, 0x143, 0xc, 0xf, false));  // row_bcast:31 -> rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}

// Unsigned form (flipping the sign bit maps unsigned order onto signed).
__device__ __forceinline__ uint32_t wave_umax_dpp(uint32_t v) {
    return (uint32_t)wave_max_dpp((int)(v ^ 0x80000000u)) ^ 0x80000000u;
}

}  // namespace ie
