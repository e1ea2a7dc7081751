// Device helpers shared by the HIP kernels: bf16 packing, RoPE angle reduction,
// wavefront reductions.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 2*pi split into a double and its rounding error.  The error term is -sin(fl(2*pi)):
// sin(2*pi - e) = -sin(e) = -e + O(e^3), and e ~ 2.4e-16 makes the cubic term vanish.
constexpr double kTwoPiHi = 6.283185307179586;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189535;

// sin and cos of pos*theta.  The angle is formed in double, reduced to [-pi, pi] by
// subtracting the nearest multiple of 2*pi (two-part constant), then evaluated in fp32.
// At pos ~ 1e6 the double angle carries ~1e-10 rad absolute error; fp32 sincos of the
// reduced angle adds ~1e-7.
__device__ inline void rope_sincos(int64_t pos, double theta, float* s, float* c) {
    double a = (double)pos * theta;
    double k = rint(a * kInvTwoPi);
    double r = fma(-k, kTwoPiHi, a);
    r = fma(-k, kTwoPiLo, r);
    sincosf((float)r, s, c);
}

__device__ inline float bf16_bits_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Two floats -> packed bf16 pair (round to nearest even), `lo` in the low half.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// IEEE half precision (rotated keys and queries, the operands of the q.k product).
__device__ inline float f16_bits_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ inline uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Two floats -> packed halves (round to nearest even), `lo` in the low half.
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Load 8 consecutive input elements (bf16 or fp32) as floats.
template <bool F32>
__device__ inline void load8(const void* base, int64_t idx, float* o) {
    if constexpr (F32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
        f32x4 a = p[0], b = p[1];
        o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
        o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
    } else {
        u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            o[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
    }
}

// Inputs in fp32 are rounded to bf16 on load, so every path sees bf16 values.
__device__ inline float round_bf16(float x) {
    return bf16_bits_to_f32(f32_to_bf16_bits(x));
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Window of a pair with rotation frequency theta: floor(alpha * (2*pi / theta)) in IEEE
// double, or INT32_MAX when that is not below INT32_MAX (an unbounded window; also a NaN).
// The same expression and rounding as the host's table, so per-head tables computed here give
// the decisions the host would.
__device__ inline int window_from_theta(double alpha, double theta) {
    const double t = alpha * ((2.0 * M_PI) / theta);
    return t < (double)INT32_MAX ? (int)floor(t) : INT32_MAX;
}

// First index i in [0, P) with W[i] >= x (W non-decreasing), or P.  Uniform across the
// wave; W lives in kernel arguments.
__device__ inline int first_at_least(const int32_t* W, int P, int64_t x) {
    int lo = 0, hi = P;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)W[mid] >= x) hi = mid; else lo = mid + 1;
    }
    return lo;
}

}  // namespace wpa
