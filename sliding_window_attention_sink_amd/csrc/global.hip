// Task-bound global tokens on the banded prefill, gfx950.
//
// Longformer adds a few global tokens to the sliding window: they see the
// whole sequence and the whole sequence sees them (the Longformer section and
// the glossary entry on global tokens of the t6page page "滑窗与固定稀疏").
// In causal form, with G the sorted global positions: a row t in G attends
// every key <= t; any other row attends U(t) plus the global positions
// g <= t, each key once (a global among the sinks or inside the window is
// already there).
//
// swa_prefill_global runs
//   1. global_gather: the keys and values of G, per (batch, kv-head), into
//      a [64, d] block pair (rows past |G| zero);
//   2. the banded prefill (sinks + window), which also writes each row's
//      log-sum-exp;
//   3. global_merge (here): per row, softmax attention over the global keys
//      not already in U(t) (g >= s, g < t - r + 1, g <= t), merged into the
//      banded row through the two log-sum-exps;
//   4. the rows in G as dense causal rows: the decode kernel over keys 0 .. t.
#include "mfma_tile.h"
#include "swa_internal.h"

namespace swa {
namespace {

using namespace mt;

// Keys and values of the global positions into [B*Hkv, kMaxGlobals, d]
// (rows past ng zero).  Thread: one 16-byte chunk.
template <int D>
__global__ __launch_bounds__(256) void global_gather_kernel(GlobalArgs a) {
    constexpr int CH = D / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)a.B * a.Hkv * kMaxGlobals * CH;
    if (idx >= total) return;
    const int c = (int)(idx % CH);
    const int j = (int)((idx / CH) % kMaxGlobals);
    const int64_t bh = idx / (CH * kMaxGlobals);
    u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
    if (j < a.ng) {
        const size_t src = ((size_t)bh * a.L + a.pos[j]) * D + 8 * c;
        kx = *(const u32x4*)((const __bf16*)a.k + src);
        vx = *(const u32x4*)((const __bf16*)a.v + src);
    }
    const size_t dst = ((size_t)bh * kMaxGlobals + j) * D + 8 * c;
    *(u32x4*)((__bf16*)a.kg + dst) = kx;
    *(u32x4*)((__bf16*)a.vg + dst) = vx;
}

// Merge of the global keys into the banded rows.  Workgroup: 128 rows of one
// (batch, q-head), a wave 32 of them: S^T = K_G Q^T per 32 global keys,
// softmax over the keys that the row does not already have, O_G^T = V_G^T
// P^T, then O = (O_band 2^lse_band + O_G 2^m) / (2^lse_band + l 2^m).
template <int D>
__global__ __launch_bounds__(NT, 2) void global_merge_kernel(GlobalArgs a) {
    typedef Tile<D> TT;
    constexpr int KS = TT::KS, NDB = TT::NDB;
    constexpr int NGB = kMaxGlobals / BLK;
    __shared__ __attribute__((aligned(1024))) char kgs[NGB][TT::BYTES];
    __shared__ __attribute__((aligned(1024))) char vgs[NGB][TT::BYTES];
    __shared__ int gpos[kMaxGlobals];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int L = (int)a.L, s = a.s, r = a.r;
    const int G = a.Hq / a.Hkv;
    const int nqt = (L + 127) / 128;
    const int bid = xcd_item(blockIdx.x, gridDim.x);
    const int qt = bid % nqt;
    const int bhq = bid / nqt;                      // b * Hq + h
    const int b = bhq / a.Hq, h = bhq % a.Hq;
    const int bhk = b * a.Hkv + h / G;
    const int t0 = qt * 128, t1 = (t0 + 127) < (L - 1) ? (t0 + 127) : (L - 1);
    const int my_t = t0 + 32 * wave + l32;
    const bool my_valid = my_t <= t1;
    const size_t row = (size_t)bhq * L + (my_valid ? my_t : t1);

    const int nblk = (a.ng + BLK - 1) / BLK;
#pragma unroll
    for (int kb = 0; kb < NGB; ++kb) {
        if (kb < nblk) {
            TT::load(kgs[kb], (const __bf16*)a.kg + (size_t)bhk * kMaxGlobals * D, BLK * kb, 0, kMaxGlobals - 1,
                     wave, lane);
            TT::load(vgs[kb], (const __bf16*)a.vg + (size_t)bhk * kMaxGlobals * D, BLK * kb, 0, kMaxGlobals - 1,
                     wave, lane);
        }
    }
    if (threadIdx.x < kMaxGlobals) gpos[threadIdx.x] = (int)threadIdx.x < a.ng ? a.pos[threadIdx.x] : 0x7fffffff;
    bf16x8 qB[KS];
    {
        const __bf16* qr = (const __bf16*)a.q + row * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qB[ks] = *(const bf16x8*)(qr + 16 * ks + 8 * g);
    }
    wait_vm(0);
    __syncthreads();

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_c = -__builtin_inff(), l_part = 0.0f;
    const float c = a.scale_log2e;
    const int win_lo = (my_t - r + 1) > s ? (my_t - r + 1) : s;   // window keys start here
    for (int kb = 0; kb < nblk; ++kb) {
        f32x16 sa = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sa = mfma(TT::rowop(kgs[kb], l32, g, ks), qB[ks], sa);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int p = gpos[BLK * kb + crow(i, g)];
            const bool ok = my_valid & (p >= s) & (p < win_lo) & (p <= my_t);
            sa[i] = ok ? sa[i] : -__builtin_inff();
        }
        float mx = sa[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sa[i]);
        const float mxc = pair_max(mx) * c;
        if (mxc > m_c) {
            const float alpha = __builtin_amdgcn_exp2f(m_c - mxc);
            m_c = mxc;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
        const float mneg = m_c == -__builtin_inff() ? 0.0f : -m_c;
        bf16x8 pk[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, mneg));
            l_part += p;
            pk[i / 8][i % 8] = (__bf16)p;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mfma(TT::trop(vgs[kb], lane, db, kk), pk[kk], acc[db]);
    }
    const float l_tot = pair_sum(l_part);
    if (!my_valid || m_c == -__builtin_inff()) return;   // no global key outside U(t): the row stands
    const float lse_b = a.lse[row];
    const float M = fmaxf(lse_b, m_c);
    const float wb = __builtin_amdgcn_exp2f(lse_b - M), wgl = __builtin_amdgcn_exp2f(m_c - M);
    const float inv = 1.0f / (wb + l_tot * wgl);
    __bf16* orow = (__bf16*)a.o + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            __bf16* p = orow + 32 * db + 8 * q4 + 4 * g;
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 ob = *(const bf16x4*)p;
            bf16x4 on;
#pragma unroll
            for (int j = 0; j < 4; ++j) on[j] = (__bf16)(((float)ob[j] * wb + acc[db][4 * q4 + j] * wgl) * inv);
            *(bf16x4*)p = on;
        }
}

template <int D>
hipError_t launch(const GlobalArgs& a, hipStream_t st, int phase) {
    if (phase == 0) {
        const int64_t n = (int64_t)a.B * a.Hkv * kMaxGlobals * (D / 8);
        hipLaunchKernelGGL((global_gather_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    } else {
        const int64_t nqt = (a.L + 127) / 128;
        hipLaunchKernelGGL((global_merge_kernel<D>), dim3((unsigned)(a.B * a.Hq * nqt)), dim3(NT), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_global_gather_bf16(const GlobalArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st, 0);
    if (d == 64) return launch<64>(a, st, 0);
    return hipErrorInvalidValue;
}

hipError_t launch_global_merge_bf16(const GlobalArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st, 1);
    if (d == 64) return launch<64>(a, st, 1);
    return hipErrorInvalidValue;
}

}  // namespace swa
