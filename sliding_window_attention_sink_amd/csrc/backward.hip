// Backward of the windowed rows (training), bf16 inputs, fp32 gradients, gfx950.
//
// The forward row t is softmax over U(t) = {i <= t : i < s or i >= t-r+1}
// of scale * q_t . k_i, weighting v_i (hyper.ai summary of arXiv
// 2608.28444, section "带 Sink 的滑动窗口注意力"; eq:attn-fixed-streaming on
// the t6page page for the key set).  Its gradient for an upstream dO, with
// P the row's softmax weights and D_t = dO_t . O_t:
//   dV_i = sum_{t : i in U(t)} P_ti dO_t
//   dS_ti = P_ti (dO_t . v_i - D_t)
//   dQ_t = scale sum_{i in U(t)} dS_ti k_i,   dK_i = scale sum_t dS_ti q_t
// with dK and dV summed over the q-heads of a kv-head.
//
// Three kernels, one wave per row or key, fp32 vector arithmetic (this first
// backward is correct and plain, not MFMA-tiled):
//   bwd_q:   per query row, the row's log2-sum-exp over U(t) (one pass over
//            its keys, lanes over keys), D_t, then dQ_t (a second pass:
//            lanes score their keys, then lanes over dims add dS_ti k_i);
//            lse and D go to the workspace.
//   bwd_kv:  per key i, the queries t = i .. min(L-1, i+r-1) of every q-head
//            of its group (for i >= s these are all of its queries): dK_i,
//            dV_i, stored.
//   bwd_sink: per sink key i < s and segment of the queries t >= i + r (the
//            sinks are attended by every later query), the same sums, added
//            atomically after bwd_kv's stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BW = 4;               // waves per workgroup, one row or key each
constexpr int BT = 64 * BW;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x (fp32, LDS, D values) . row (bf16, global); four independent chains
// (element e goes to chain e mod 4), so the result does not depend on which
// of the two rows sits in LDS
template <int D>
__device__ __forceinline__ float dot_row(const float* x, const __bf16* row) {
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 w = *(const u32x4*)(row + 8 * c);
        const f32x4 a = *(const f32x4*)(x + 8 * c);
        const f32x4 b = *(const f32x4*)(x + 8 * c + 4);
        a0 = fmaf(a[0], bf_lo(w[0]), a0);
        a1 = fmaf(a[1], bf_hi(w[0]), a1);
        a2 = fmaf(a[2], bf_lo(w[1]), a2);
        a3 = fmaf(a[3], bf_hi(w[1]), a3);
        a0 = fmaf(b[0], bf_lo(w[2]), a0);
        a1 = fmaf(b[1], bf_hi(w[2]), a1);
        a2 = fmaf(b[2], bf_lo(w[3]), a2);
        a3 = fmaf(b[3], bf_hi(w[3]), a3);
    }
    return (a0 + a1) + (a2 + a3);
}

// lane j's value to every lane (j uniform: a scalar read, no LDS round trip)
__device__ __forceinline__ float lane_value(float x, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

// This lane's D / 64 consecutive dims of a bf16 row, as fp32.
template <int D>
__device__ __forceinline__ void lane_dims(const __bf16* row, int lane, float (&x)[D / 64]) {
    if constexpr (D == 128) {
        const uint32_t w = *(const uint32_t*)(row + 2 * lane);
        x[0] = bf_lo(w);
        x[1] = bf_hi(w);
    } else {
        x[0] = (float)row[lane];
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// LDS rows written by the wave's lanes are read by all of them next; LDS
// accesses of one wave complete in order, the clobber keeps the compiler's.
__device__ __forceinline__ void lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Stage two bf16 rows of D values into fp32 LDS rows (lanes over dims).
template <int D>
__device__ __forceinline__ void stage2(float* xa, float* xb, const __bf16* ra, const __bf16* rb, int lane) {
    for (int e = lane; e < D; e += 64) {
        xa[e] = (float)ra[e];
        xb[e] = (float)rb[e];
    }
}

template <int D>
__global__ __launch_bounds__(BT) void bwd_q_kernel(BackwardArgs a) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) float xs[BW][2][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t nrows = (int64_t)a.B * a.Hq * a.L;
    const int64_t row = (int64_t)blockIdx.x * BW + wv;     // (b * Hq + h) * L + t
    if (row >= nrows) return;
    const int t = (int)(row % a.L);
    const int64_t bh = row / a.L;
    const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq);
    const int kvh = h / (a.Hq / a.Hkv);
    const __bf16* kb = (const __bf16*)a.k + ((int64_t)b * a.Hkv + kvh) * a.L * D;
    const __bf16* vb = (const __bf16*)a.v + ((int64_t)b * a.Hkv + kvh) * a.L * D;
    const __bf16* orow = (const __bf16*)a.o + row * D;
    float* qs = xs[wv][0];
    float* gs = xs[wv][1];
    stage2<D>(qs, gs, (const __bf16*)a.q + row * D, (const __bf16*)a.dout + row * D, lane);
    lds_order();
    float dpart = 0.0f;
    for (int e = lane; e < D; e += 64) dpart += gs[e] * (float)orow[e];
    const float Dt = wave_sum(dpart);

    // U(t): sinks 0 .. ns-1, then the window wlo .. t
    const int ns = a.s < t + 1 ? a.s : t + 1;
    const int wlo = a.s > t - a.r + 1 ? a.s : t - a.r + 1;
    const int n = ns + (t >= wlo ? t - wlo + 1 : 0);
    auto key_of = [&](int j) { return j < ns ? j : wlo + (j - ns); };
    const float c = a.scale_log2e;

    // pass 1: log2-sum-exp of the row's scores (per lane, then across lanes)
    float m = -__builtin_inff(), l = 0.0f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        if (j < n) {
            const float sc = dot_row<D>(qs, kb + (int64_t)key_of(j) * D) * c;
            if (sc > m) {
                l = l * exp2f(m - sc) + 1.0f;
                m = sc;
            } else {
                l += exp2f(sc - m);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
        const float mm = fmaxf(m, m2);
        l = (m == -__builtin_inff() ? 0.0f : l * exp2f(m - mm)) + (m2 == -__builtin_inff() ? 0.0f : l2 * exp2f(m2 - mm));
        m = mm;
    }
    const float lse2 = m + log2f(l);

    // pass 2: dS of each key (lanes over keys), then dQ (lanes over dims)
    float acc[NE], acc2[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = acc2[e] = 0.0f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        float ds = 0.0f;
        if (j < n) {
            const int64_t ko = (int64_t)key_of(j) * D;
            const float p = exp2f(dot_row<D>(qs, kb + ko) * c - lse2);
            ds = p * (dot_row<D>(gs, vb + ko) - Dt);
        }
        const int cnt = n - j0 < 64 ? n - j0 : 64;
        // keys in pairs, one accumulator chain each
#pragma unroll 4
        for (int jj = 0; jj < cnt; jj += 2) {
            const bool two = jj + 1 < cnt;
            const float g0 = lane_value(ds, jj), g1 = two ? lane_value(ds, jj + 1) : 0.0f;
            float k0[NE], k1[NE];
            lane_dims<D>(kb + (int64_t)key_of(j0 + jj) * D, lane, k0);
            lane_dims<D>(kb + (int64_t)key_of(two ? j0 + jj + 1 : j0 + jj) * D, lane, k1);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                acc[e] = fmaf(g0, k0[e], acc[e]);
                acc2[e] = fmaf(g1, k1[e], acc2[e]);
            }
        }
    }
    float* dq = a.dq + row * D + NE * lane;
#pragma unroll
    for (int e = 0; e < NE; ++e) dq[e] = (acc[e] + acc2[e]) * a.scale;
    if (lane == 0) {
        a.lse2[row] = lse2;
        a.dd[row] = Dt;
    }
}

// dK, dV contributions of key i (kv-head kvh of batch b, K and V rows
// staged in ks, vs) from the queries t0 .. t0+nt-1 of every q-head of the
// group, added into dka, dva (this lane's dims).
template <int D>
__device__ __forceinline__ void kv_sums(const BackwardArgs& a, const float* ks, const float* vs, int b, int kvh,
                                        int t0, int nt, int lane, float (&dka)[D / 64], float (&dva)[D / 64]) {
    constexpr int NE = D / 64;
    const int G = a.Hq / a.Hkv;
    const int n = nt * G;
    const float c = a.scale_log2e;
    auto qrow_of = [&](int j) { return ((int64_t)b * a.Hq + kvh * G + j % G) * a.L + t0 + j / G; };
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        float p = 0.0f, ds = 0.0f;
        if (j < n) {
            const int64_t qr = qrow_of(j);
            p = exp2f(dot_row<D>(ks, (const __bf16*)a.q + qr * D) * c - a.lse2[qr]);
            ds = p * (dot_row<D>(vs, (const __bf16*)a.dout + qr * D) - a.dd[qr]);
        }
        const int cnt = n - j0 < 64 ? n - j0 : 64;
#pragma unroll 8
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = lane_value(p, jj), gj = lane_value(ds, jj);
            const int64_t qr = qrow_of(j0 + jj);
            float gx[NE], qx[NE];
            lane_dims<D>((const __bf16*)a.dout + qr * D, lane, gx);
            lane_dims<D>((const __bf16*)a.q + qr * D, lane, qx);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                dva[e] = fmaf(pj, gx[e], dva[e]);
                dka[e] = fmaf(gj, qx[e], dka[e]);
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(BT) void bwd_kv_kernel(BackwardArgs a) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) float xs[BW][2][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t nkeys = (int64_t)a.B * a.Hkv * a.L;
    const int64_t key = (int64_t)blockIdx.x * BW + wv;     // (b * Hkv + kvh) * L + i
    if (key >= nkeys) return;
    const int i = (int)(key % a.L);
    const int64_t bk = key / a.L;
    const int b = (int)(bk / a.Hkv), kvh = (int)(bk % a.Hkv);
    float* ks = xs[wv][0];
    float* vs = xs[wv][1];
    stage2<D>(ks, vs, (const __bf16*)a.k + key * D, (const __bf16*)a.v + key * D, lane);
    lds_order();
    // queries i .. i + r - 1 (all of them for i >= s; the first r for a sink)
    const int64_t tend = (int64_t)i + a.r - 1 < a.L - 1 ? (int64_t)i + a.r - 1 : a.L - 1;
    float dka[NE], dva[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) dka[e] = dva[e] = 0.0f;
    kv_sums<D>(a, ks, vs, b, kvh, i, (int)(tend - i + 1), lane, dka, dva);
    float* dk = a.dk + key * D + NE * lane;
    float* dv = a.dv + key * D + NE * lane;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        dk[e] = dka[e] * a.scale;
        dv[e] = dva[e];
    }
}

// Sink key i < s, queries i + r + seg * kSinkSeg onwards (at most kSinkSeg
// positions): added to bwd_kv's stored sums.
template <int D>
__global__ __launch_bounds__(BT) void bwd_sink_kernel(BackwardArgs a, int32_t nseg) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) float xs[BW][2][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t nitems = (int64_t)a.B * a.Hkv * a.s * nseg;
    const int64_t item = (int64_t)blockIdx.x * BW + wv;    // ((b * Hkv + kvh) * s + i) * nseg + seg
    if (item >= nitems) return;
    const int seg = (int)(item % nseg);
    const int64_t rest = item / nseg;
    const int i = (int)(rest % a.s);
    const int64_t bk = rest / a.s;
    const int b = (int)(bk / a.Hkv), kvh = (int)(bk % a.Hkv);
    const int64_t t0 = (int64_t)i + a.r + (int64_t)seg * kSinkSeg;
    if (t0 > a.L - 1) return;
    const int64_t t1 = t0 + kSinkSeg - 1 < a.L - 1 ? t0 + kSinkSeg - 1 : a.L - 1;
    const int64_t key = bk * a.L + i;
    float* ks = xs[wv][0];
    float* vs = xs[wv][1];
    stage2<D>(ks, vs, (const __bf16*)a.k + key * D, (const __bf16*)a.v + key * D, lane);
    lds_order();
    float dka[NE], dva[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) dka[e] = dva[e] = 0.0f;
    kv_sums<D>(a, ks, vs, b, kvh, (int)t0, (int)(t1 - t0 + 1), lane, dka, dva);
    float* dk = a.dk + key * D + NE * lane;
    float* dv = a.dv + key * D + NE * lane;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        atomicAdd(dk + e, dka[e] * a.scale);
        atomicAdd(dv + e, dva[e]);
    }
}

template <int D>
hipError_t launch(const BackwardArgs& a, hipStream_t st) {
    const int64_t nrows = (int64_t)a.B * a.Hq * a.L, nkeys = (int64_t)a.B * a.Hkv * a.L;
    hipLaunchKernelGGL((bwd_q_kernel<D>), dim3((unsigned)((nrows + BW - 1) / BW)), dim3(BT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kv_kernel<D>), dim3((unsigned)((nkeys + BW - 1) / BW)), dim3(BT), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.s == 0 || a.L <= a.r) return e;
    const int32_t nseg = (int32_t)((a.L - a.r + kSinkSeg - 1) / kSinkSeg);
    const int64_t nitems = (int64_t)a.B * a.Hkv * a.s * nseg;
    hipLaunchKernelGGL((bwd_sink_kernel<D>), dim3((unsigned)((nitems + BW - 1) / BW)), dim3(BT), 0, st, a, nseg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_bf16(const BackwardArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st);
    if (d == 64) return launch<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
