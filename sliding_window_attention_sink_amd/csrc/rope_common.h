// Rotary position embedding helpers shared by the gfx950 kernels.
//
// Rotation pairs dimension j with j + d/2 and turns the pair by the angle
// position * theta_j, theta_j = base^(-2j/d) = rr^j with rr = base^(-2/d)
// (computed on the host in fp64).  Angles are formed in fp64 as a number of
// turns, position * theta_j / (2 pi), reduced to the fraction of a turn and
// handed to the hardware sine and cosine (v_sin_f32 / v_cos_f32 take turns),
// so positions up to 2^30 keep full accuracy; the rotation itself runs in
// fp32 and is rounded to bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {
namespace rope {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kInvTwoPi = 0.15915494309189535;

// rr^j for 0 <= j < 2^7 by binary powers (at most 13 fp64 products).
__device__ __forceinline__ double powi(double rr, int j) {
    double x = 1.0, b = rr;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {
        if (j & (1 << bit)) x *= b;
        b *= b;
    }
    return x;
}

// Fraction of a turn of the angle pos * theta / (2 pi); pos_turns = pos / (2 pi).
__device__ __forceinline__ float turn_frac(double pos_turns, double theta) {
    const double v = pos_turns * theta;
    return (float)(v - __builtin_floor(v));
}

// Rotate the eight pairs (lo[e], hi[e]) (packed bf16, dims j0 + e and
// j0 + e + d/2) by the angles whose turn fractions are x[e].
__device__ __forceinline__ void rot8(u32x4& lo, u32x4& hi, const float* x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t rl = 0, rh = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float c = __builtin_amdgcn_cosf(x[2 * w + h]), sn = __builtin_amdgcn_sinf(x[2 * w + h]);
            const float x0 = __builtin_bit_cast(float, (lo[w] >> (16 * h)) << 16);
            const float x1 = __builtin_bit_cast(float, (hi[w] >> (16 * h)) << 16);
            const uint32_t y0 = __builtin_bit_cast(uint16_t, (__bf16)(x0 * c - x1 * sn));
            const uint32_t y1 = __builtin_bit_cast(uint16_t, (__bf16)(x0 * sn + x1 * c));
            rl |= y0 << (16 * h);
            rh |= y1 << (16 * h);
        }
        lo[w] = rl;
        hi[w] = rh;
    }
}

// Rotate dims j0 .. j0+7 and their partners j0+d/2 .. (one 16-byte chunk of
// each half of a row) to position pos.  The angles depend only on the
// position and the lane, so inside a loop the compiler would hoist them and
// keep every cosine and sine live across it; the empty asm makes the inputs
// opaque at each call, so they are formed where they are used.
__device__ __forceinline__ void rot_chunk_pair(u32x4& lo, u32x4& hi, int j0, double pos, double rr) {
    asm volatile("" : "+v"(pos), "+v"(rr));
    const double pt = pos * kInvTwoPi;
    double th = powi(rr, j0);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = turn_frac(pt, th);
        th *= rr;
    }
    rot8(lo, hi, x);
}

}  // namespace rope
}  // namespace swa
