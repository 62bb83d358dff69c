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
//   1. global_gather (here): the keys and values of G, per (batch,
//      kv-head), into a [64, d] block pair (rows past |G| zero), and the
//      per-row count of globals below the row's window;
//   2. the banded prefill with that block as one more key tile after the
//      band: row t keeps the globals g with s <= g < t - r + 1 (the others
//      are sinks, in the window or in the future);
//   3. the rows in G as dense causal rows: the decode kernel over keys
//      0 .. t, several positions per launch as extra query columns.
#include "mfma_tile.h"
#include "swa_internal.h"

namespace swa {
namespace {

using namespace mt;

// Keys and values of the global positions at or past the sinks into
// [B*Hkv, kMaxGlobals, d] (rows past ng zero).  Thread: one 16-byte chunk.
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

// gjb[t] = #{j : pos[j] < t - r + 1}: the gathered globals (all at or past
// the sinks) below row t's window; the prefill keeps block rows
// 0 .. gjb[t]-1 for row t.  Thread: one row.
__global__ __launch_bounds__(256) void global_rows_kernel(GlobalArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= a.L) return;
    int c = 0;
    for (int j = 0; j < a.ng; ++j) c += (int64_t)a.pos[j] < t - a.r + 1 ? 1 : 0;
    a.gjb[t] = (uint8_t)c;
}

template <int D>
hipError_t launch(const GlobalArgs& a, hipStream_t st) {
    const int64_t n = (int64_t)a.B * a.Hkv * kMaxGlobals * (D / 8);
    hipLaunchKernelGGL((global_gather_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(global_rows_kernel, dim3((unsigned)((a.L + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_global_gather_bf16(const GlobalArgs& a, int d, hipStream_t st) {
    if (d == 128) return launch<128>(a, st);
    if (d == 64) return launch<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace swa
