// RoPE re-positioning for chunked prefill over the rolling cache, gfx950.
//
// StreamingLLM keeps keys before rotation and, for every query, places the
// keys of the cache at consecutive positions 0 .. |U(t)|-1 with the query at
// |U(t)|-1 (the paragraph after eq:attn-fixed-streaming on the t6page page
// "滑窗与固定稀疏").  Rotary scores depend only on the difference of the two
// positions, so with U(t) in temporal order:
//   * a window key i >= s is |U(t)|-1 - rank(i) = t - i before the query, the
//     true distance: rotate it to i and the query to t;
//   * sink j < s is min(t, s+r-1) - j before the query: rotate it to j and,
//     for sink scores only, the query to min(t, s+r-1).
// This kernel writes those rotated copies once per call (bf16, rotated in
// fp32; the angle position * theta is formed in fp64 and reduced to its
// fraction of a turn before the fp32 sine and cosine, so positions up to
// 2^31 keep full accuracy):
//   qb  = q rotated to t,  qs = q rotated to min(t, s+r-1),
//   knr = chunk keys rotated to their position,
//   kcr = cache keys rotated to the position of the token each slot holds.
// Rotation pairs dimension j with j + d/2 and turns the pair by
// position * base^(-2j/d).
#include "swa_internal.h"

namespace swa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void rope_prepare_kernel(RopeArgs a) {
    constexpr int H2 = D / 2;
    __shared__ float cs[2][H2], sn[2][H2];

    const int item = blockIdx.x;     // [0, L): chunk row; [L, L + s + r): cache slot
    const int S = a.s + a.r;
    const int64_t L = a.L;
    int64_t pos_a, pos_b;            // positions of the two rotations this item needs
    bool is_row = item < L;
    bool slot_valid = true;
    if (is_row) {
        const int64_t t = a.pos0 + item;
        pos_a = t;
        pos_b = t < S - 1 ? t : (int64_t)(S - 1);
    } else {
        // token held by cache slot j when the cache holds tokens 0 .. pos0-1
        const int j = item - (int)L;
        const int64_t T = a.pos0;
        int64_t p;
        if (j < a.s) {
            p = j;
            slot_valid = j < T;
        } else {
            const int64_t q = j - a.s;
            if (q > T - 1) {
                slot_valid = false;
                p = 0;
            } else {
                p = (T - 1) - (((T - 1) - q) % a.r);
                slot_valid = p >= a.s;
            }
        }
        pos_a = pos_b = p;
    }
    if (!slot_valid) return;

    const int tid = threadIdx.x;
    if (tid < 2 * H2) {
        const int which = tid / H2, j = tid % H2;
        // turns per position of pair j, then the fraction of a turn at the
        // position (the hardware sine and cosine take turns)
        const double turns = exp2(-(2.0 * j / D) * log2((double)a.base)) * 0.15915494309189535;
        const double rv = (double)(which ? pos_b : pos_a) * turns;
        const float x = (float)(rv - __builtin_floor(rv));
        cs[which][j] = __builtin_amdgcn_cosf(x);
        sn[which][j] = __builtin_amdgcn_sinf(x);
    }
    __syncthreads();

    // 8 threads per row, each rotating 8 pairs (two 16-byte loads, two stores)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int TPR = H2 / 8;
    const int rows_per_pass = 256 / TPR;
    const int rsub = tid / TPR, j0 = (tid % TPR) * 8;
    auto rot_to = [&](const u32x4& lo, const u32x4& hi, __bf16* dst, int which) {
        u32x4 olo, ohi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t rl = 0, rh = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = j0 + 2 * w + h;
                const float x0 = __builtin_bit_cast(float, (lo[w] >> (16 * h)) << 16);
                const float x1 = __builtin_bit_cast(float, (hi[w] >> (16 * h)) << 16);
                const float c = cs[which][j], sv = sn[which][j];
                const uint32_t y0 = __builtin_bit_cast(uint16_t, (__bf16)(x0 * c - x1 * sv));
                const uint32_t y1 = __builtin_bit_cast(uint16_t, (__bf16)(x0 * sv + x1 * c));
                rl |= y0 << (16 * h);
                rh |= y1 << (16 * h);
            }
            olo[w] = rl;
            ohi[w] = rh;
        }
        *(u32x4*)(dst + j0) = olo;
        *(u32x4*)(dst + j0 + H2) = ohi;
    };
    // each source row is read once (non-temporal); the rotated copies are
    // read by the attention kernel right after, so they are stored normally
    auto load_row = [&](const __bf16* src, u32x4& lo, u32x4& hi) {
        lo = __builtin_nontemporal_load((const u32x4*)(src + j0));
        hi = __builtin_nontemporal_load((const u32x4*)(src + j0 + H2));
    };
    auto rot = [&](const __bf16* src, __bf16* dst, int which) {
        u32x4 lo, hi;
        load_row(src, lo, hi);
        rot_to(lo, hi, dst, which);
    };
    if (is_row) {
        // queries: B*Hq rows at chunk row `item`, read once, rotated twice
        for (int rr = rsub; rr < a.B * a.Hq; rr += rows_per_pass) {
            const size_t off = ((size_t)rr * L + item) * D;
            u32x4 lo, hi;
            load_row((const __bf16*)a.q + off, lo, hi);
            rot_to(lo, hi, (__bf16*)a.qb + off, 0);
            rot_to(lo, hi, (__bf16*)a.qsk + off, 1);
        }
        for (int rr = rsub; rr < a.B * a.Hkv; rr += rows_per_pass) {
            const size_t off = ((size_t)rr * L + item) * D;
            rot((const __bf16*)a.kn + off, (__bf16*)a.knr + off, 0);
        }
    } else {
        const int j = item - (int)L;
        for (int rr = rsub; rr < a.B * a.Hkv; rr += rows_per_pass) {
            const size_t off = ((size_t)rr * S + j) * D;
            rot((const __bf16*)a.kc + off, (__bf16*)a.kcr + off, 0);
        }
    }
}

}  // namespace

hipError_t launch_rope_prepare_bf16(const RopeArgs& a, int d, hipStream_t st) {
    const int64_t items = a.L + (a.kc ? (a.s + a.r) : 0);
    if (d == 128) {
        hipLaunchKernelGGL(rope_prepare_kernel<128>, dim3((unsigned)items), dim3(256), 0, st, a);
    } else if (d == 64) {
        hipLaunchKernelGGL(rope_prepare_kernel<64>, dim3((unsigned)items), dim3(256), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace swa
