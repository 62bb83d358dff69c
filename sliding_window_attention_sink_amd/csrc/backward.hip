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
// Three kernels on the vector units (a plain first backward, not
// MFMA-tiled): dot products as bf16 pairs into fp32 (v_dot2c_f32_bf16, the
// inputs exact), sums in fp32.  A wave takes eight adjacent rows or keys, so
// each row a lane reads from memory serves eight dot products; the rows
// staged for the dot products and each chunk's dS (and P) go through LDS:
//   bwd_q:   per eight query rows, D_t, then one pass over the union of
//            their keys (lanes score keys, then lanes over dims add
//            dS_ti k_i) with the softmax normalised at the end, as in the
//            forward's online softmax; lse and D go to the workspace.
//   bwd_kv:  per eight keys, the queries t = i .. min(L-1, i+r-1) of each
//            key i from every q-head of its group (for i >= s these are all
//            of its queries): dK_i, dV_i, stored.
//   bwd_sink: per sink key i < s and segment of the queries t >= i + r (the
//            sinks are attended by every later query), the same sums, added
//            atomically after bwd_kv's stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "backward_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BW = 4;               // waves per workgroup
constexpr int BT = 64 * BW;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// LDS rows written by the wave's lanes are read by all of them next; LDS
// accesses of one wave complete in order, the clobber keeps the compiler's.
__device__ __forceinline__ void lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Stage two bf16 rows of D values into LDS as they are (bf16 pairs, lanes
// over pairs).
template <int D>
__device__ __forceinline__ void stage2(uint32_t* xa, uint32_t* xb, const __bf16* ra, const __bf16* rb, int lane) {
    for (int e = lane; e < D / 2; e += 64) {
        xa[e] = ((const uint32_t*)ra)[e];
        xb[e] = ((const uint32_t*)rb)[e];
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a[0] b[0] + a[1] b[1] + acc for two bf16 pairs (products exact in fp32)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// R dot products at once: x holds R bf16 rows of D values (LDS, as pairs,
// row stride D / 2 words), row is one bf16 row (global memory), read once
// for all R.  Pairs 0-1 of every 4 go to one accumulator chain and 2-3 to
// another, so the result does not depend on which operand sits in LDS.
template <int D, int R>
__device__ __forceinline__ void dot_rows(const uint32_t* x, const __bf16* row, float (&out)[R]) {
    float c0[R], c1[R];
#pragma unroll
    for (int q = 0; q < R; ++q) c0[q] = c1[q] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 w = *(const u32x4*)(row + 8 * c);
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const u32x4 a = *(const u32x4*)(x + q * (D / 2) + 4 * c);
            c0[q] = dot2(a[0], w[0], c0[q]);
            c0[q] = dot2(a[1], w[1], c0[q]);
            c1[q] = dot2(a[2], w[2], c1[q]);
            c1[q] = dot2(a[3], w[3], c1[q]);
        }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) out[q] = c0[q] + c1[q];
}

// Rows (or keys) per wave in bwd_q and bwd_kv: every K, V, Q or dout row a
// lane reads serves RW of them (8 ran 11% faster than 4 on the main
// workload's shape, at 141-179 VGPRs).
constexpr int RW = 8;

template <int D>
__global__ __launch_bounds__(BT) void bwd_q_kernel(BackwardArgs a) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) uint32_t xs[BW][2][RW * D / 2];
    __shared__ __attribute__((aligned(16))) float bc[BW][64 * RW];   // a chunk's dS, [pair][row]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t ngr = (a.L + RW - 1) / RW;                 // row groups per (b, h)
    const int64_t grp = (int64_t)blockIdx.x * BW + wv;       // (b * Hq + h) * ngr + row group
    if (grp >= (int64_t)a.B * a.Hq * ngr) return;
    const int64_t bh = grp / ngr;
    const int tb = (int)(grp % ngr) * RW;                    // rows tb .. tl
    const int nr = a.L - tb < RW ? (int)(a.L - tb) : RW;
    const int tl = tb + nr - 1;
    const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq);
    const int kvh = h / (a.Hq / a.Hkv);
    const __bf16* kb = (const __bf16*)a.k + ((int64_t)b * a.Hkv + kvh) * a.L * D;
    const __bf16* vb = (const __bf16*)a.v + ((int64_t)b * a.Hkv + kvh) * a.L * D;
    const int64_t row0 = bh * a.L + tb;
    uint32_t* qs = xs[wv][0];
    uint32_t* gs = xs[wv][1];
    // rows past the end stage row tl again (their results are not stored)
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        const int64_t rx = row0 + (x < nr ? x : nr - 1);
        stage2<D>(qs + x * (D / 2), gs + x * (D / 2), (const __bf16*)a.q + rx * D, (const __bf16*)a.dout + rx * D,
                  lane);
    }
    lds_order();
    float Dt[RW];
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        const uint32_t* orow = (const uint32_t*)((const __bf16*)a.o + (row0 + (x < nr ? x : nr - 1)) * D);
        float dpart = 0.0f;
        for (int e = lane; e < D / 2; e += 64) {
            const uint32_t gw = gs[x * (D / 2) + e], ow = orow[e];
            dpart += bf_lo(gw) * bf_lo(ow) + bf_hi(gw) * bf_hi(ow);
        }
        Dt[x] = wave_sum(dpart);
    }

    // keys of any of the rows: sinks 0 .. ns-1, then the window wlo .. tl;
    // key i is in U(tb + x) iff i <= tb + x and (i < s or i >= tb + x - r + 1)
    const int ns = a.s < tl + 1 ? a.s : tl + 1;
    const int wlo = a.s > tb - a.r + 1 ? a.s : tb - a.r + 1;
    const int n = ns + (tl >= wlo ? tl - wlo + 1 : 0);
    auto key_of = [&](int j) { return j < ns ? j : wlo + (j - ns); };
    auto in_set = [&](int x, int i) { return x < nr && i <= tb + x && (i < a.s || i >= tb + x - a.r + 1); };
    const float c = a.scale_log2e;

    // one pass over the keys, the softmax normalised at the end: per row a
    // running max m (the same in every lane), per lane a partial sum of
    // exp2(score - m), and dQ accumulated against that m, all rescaled when m
    // rises (dS_ti l_t = exp2(score - m) (dp - D_t) with l_t the row's sum)
    float m[RW], lp[RW], acc[RW][NE];
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        m[x] = -__builtin_inff();
        lp[x] = 0.0f;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[x][e] = 0.0f;
    }
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        float v[RW], dp[RW];
#pragma unroll
        for (int x = 0; x < RW; ++x) {
            v[x] = -__builtin_inff();
            dp[x] = 0.0f;
        }
        if (j < n) {
            const int i = key_of(j);
            float sc[RW];
            dot_rows<D, RW>(qs, kb + (int64_t)i * D, sc);
            dot_rows<D, RW>(gs, vb + (int64_t)i * D, dp);
#pragma unroll
            for (int x = 0; x < RW; ++x)
                if (in_set(x, i)) v[x] = sc[x] * c;
        }
        float ds[RW];
#pragma unroll
        for (int x = 0; x < RW; ++x) {
            const float mn = fmaxf(m[x], wave_max(v[x]));
            if (mn > m[x]) {
                const float alpha = exp2f(m[x] - mn);     // 0 while m is -inf
                lp[x] *= alpha;
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[x][e] *= alpha;
                m[x] = mn;
            }
            const float p = v[x] == -__builtin_inff() ? 0.0f : exp2f(v[x] - m[x]);
            lp[x] += p;
            ds[x] = p * (dp[x] - Dt[x]);
        }
        // the chunk's (unnormalised) dS through LDS: each key's RW values
        // come back as broadcast reads in the dims loop
#pragma unroll
        for (int x = 0; x < RW; ++x) bc[wv][lane * RW + x] = ds[x];
        lds_order();
        const int cnt = n - j0 < 64 ? n - j0 : 64;
#pragma unroll 2
        for (int jj = 0; jj < cnt; ++jj) {
            float kx[NE];
            lane_dims<D>(kb + (int64_t)key_of(j0 + jj) * D, lane, kx);
            const float* g = &bc[wv][jj * RW];
#pragma unroll
            for (int x = 0; x < RW; ++x) {
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[x][e] = fmaf(g[x], kx[e], acc[x][e]);
            }
        }
        lds_order();
    }
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        if (x >= nr) break;
        const float l = wave_sum(lp[x]);
        float* dq = a.dq + (row0 + x) * D + NE * lane;
#pragma unroll
        for (int e = 0; e < NE; ++e) dq[e] = acc[x][e] * (a.scale / l);
        if (lane == 0) {
            a.lse2[row0 + x] = m[x] + log2f(l);
            a.dd[row0 + x] = Dt[x];
        }
    }
}

// dK, dV contributions of R keys of kv-head kvh of batch b (K and V rows
// staged in ks, vs, row stride D) from the queries t0 .. t0+nt-1 of every
// q-head of the group, for the (key x, query t) pairs with ok(x, t); added
// into dka, dva (this lane's dims).
template <int D, int R, class Ok>
__device__ __forceinline__ void kv_sums(const BackwardArgs& a, const uint32_t* ks, const uint32_t* vs, float* bc,
                                        int b, int kvh, int t0, int nt, int lane, Ok&& ok, float (&dka)[R][D / 64],
                                        float (&dva)[R][D / 64]) {
    constexpr int NE = D / 64;
    const int G = a.Hq / a.Hkv;
    const int n = nt * G;
    const float c = a.scale_log2e;
    auto qrow_of = [&](int j) { return ((int64_t)b * a.Hq + kvh * G + j % G) * a.L + t0 + j / G; };
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        float p[R], ds[R];
#pragma unroll
        for (int x = 0; x < R; ++x) p[x] = ds[x] = 0.0f;
        if (j < n) {
            const int64_t qr = qrow_of(j);
            const int t = t0 + j / G;
            float sc[R], dp[R];
            dot_rows<D, R>(ks, (const __bf16*)a.q + qr * D, sc);
            dot_rows<D, R>(vs, (const __bf16*)a.dout + qr * D, dp);
            const float l2 = a.lse2[qr], dd = a.dd[qr];
#pragma unroll
            for (int x = 0; x < R; ++x) {
                if (!ok(x, t)) continue;
                p[x] = exp2f(sc[x] * c - l2);
                ds[x] = p[x] * (dp[x] - dd);
            }
        }
        // the chunk's P and dS through LDS ([pair][P of the R keys, dS of
        // the R keys]), read back as broadcasts in the dims loop
#pragma unroll
        for (int x = 0; x < R; ++x) {
            bc[lane * 2 * R + x] = p[x];
            bc[lane * 2 * R + R + x] = ds[x];
        }
        lds_order();
        const int cnt = n - j0 < 64 ? n - j0 : 64;
#pragma unroll 2
        for (int jj = 0; jj < cnt; ++jj) {
            const int64_t qr = qrow_of(j0 + jj);
            float gx[NE], qx[NE];
            lane_dims<D>((const __bf16*)a.dout + qr * D, lane, gx);
            lane_dims<D>((const __bf16*)a.q + qr * D, lane, qx);
            const float* pj = bc + jj * 2 * R;
#pragma unroll
            for (int x = 0; x < R; ++x) {
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    dva[x][e] = fmaf(pj[x], gx[e], dva[x][e]);
                    dka[x][e] = fmaf(pj[R + x], qx[e], dka[x][e]);
                }
            }
        }
        lds_order();
    }
}

template <int D>
__global__ __launch_bounds__(BT) void bwd_kv_kernel(BackwardArgs a) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) uint32_t xs[BW][2][RW * D / 2];
    __shared__ __attribute__((aligned(16))) float bc[BW][64 * 2 * RW];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t ngr = (a.L + RW - 1) / RW;                 // key groups per (b, kv-head)
    const int64_t grp = (int64_t)blockIdx.x * BW + wv;       // (b * Hkv + kvh) * ngr + key group
    if (grp >= (int64_t)a.B * a.Hkv * ngr) return;
    const int64_t bk = grp / ngr;
    const int ib = (int)(grp % ngr) * RW;                    // keys ib .. ib + nk - 1
    const int nk = a.L - ib < RW ? (int)(a.L - ib) : RW;
    const int b = (int)(bk / a.Hkv), kvh = (int)(bk % a.Hkv);
    const int64_t key0 = bk * a.L + ib;
    uint32_t* ks = xs[wv][0];
    uint32_t* vs = xs[wv][1];
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        const int64_t kx = key0 + (x < nk ? x : nk - 1);
        stage2<D>(ks + x * (D / 2), vs + x * (D / 2), (const __bf16*)a.k + kx * D, (const __bf16*)a.v + kx * D,
                  lane);
    }
    lds_order();
    // key ib + x takes the queries ib + x .. ib + x + r - 1 (all of them for
    // a key >= s; the first r for a sink, whose later ones bwd_sink adds)
    const int64_t last = (int64_t)ib + nk - 1 + a.r - 1;
    const int tend = (int)(last < a.L - 1 ? last : a.L - 1);
    auto ok = [&](int x, int t) { return x < nk && t >= ib + x && (int64_t)t <= (int64_t)ib + x + a.r - 1; };
    float dka[RW][NE], dva[RW][NE];
#pragma unroll
    for (int x = 0; x < RW; ++x)
#pragma unroll
        for (int e = 0; e < NE; ++e) dka[x][e] = dva[x][e] = 0.0f;
    kv_sums<D, RW>(a, ks, vs, bc[wv], b, kvh, ib, tend - ib + 1, lane, ok, dka, dva);
#pragma unroll
    for (int x = 0; x < RW; ++x) {
        if (x >= nk) break;
        float* dk = a.dk + (key0 + x) * D + NE * lane;
        float* dv = a.dv + (key0 + x) * D + NE * lane;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            dk[e] = dka[x][e] * a.scale;
            dv[e] = dva[x][e];
        }
    }
}

// Sink key i < s, queries i + r + seg * kSinkSeg onwards (at most kSinkSeg
// positions): added to bwd_kv's stored sums.
template <int D>
__global__ __launch_bounds__(BT) void bwd_sink_kernel(BackwardArgs a, int32_t nseg) {
    constexpr int NE = D / 64;
    __shared__ __attribute__((aligned(16))) uint32_t xs[BW][2][D / 2];
    __shared__ __attribute__((aligned(16))) float bc[BW][64 * 2];
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
    uint32_t* ks = xs[wv][0];
    uint32_t* vs = xs[wv][1];
    stage2<D>(ks, vs, (const __bf16*)a.k + key * D, (const __bf16*)a.v + key * D, lane);
    lds_order();
    float dka[1][NE], dva[1][NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) dka[0][e] = dva[0][e] = 0.0f;
    kv_sums<D, 1>(a, ks, vs, bc[wv], b, kvh, (int)t0, (int)(t1 - t0 + 1), lane, [](int, int) { return true; }, dka,
                  dva);
    float* dk = a.dk + key * D + NE * lane;
    float* dv = a.dv + key * D + NE * lane;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        atomicAdd(dk + e, dka[0][e] * a.scale);
        atomicAdd(dv + e, dva[0][e]);
    }
}

template <int D>
hipError_t launch(const BackwardArgs& a, hipStream_t st) {
    const int64_t ngr = (a.L + RW - 1) / RW;
    const int64_t nq = (int64_t)a.B * a.Hq * ngr, nk = (int64_t)a.B * a.Hkv * ngr;
    hipLaunchKernelGGL((bwd_q_kernel<D>), dim3((unsigned)((nq + BW - 1) / BW)), dim3(BT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_kv_kernel<D>), dim3((unsigned)((nk + BW - 1) / BW)), dim3(BT), 0, st, a);
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
