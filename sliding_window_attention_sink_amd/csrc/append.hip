// Rolling-cache append for sliding-window attention with sinks, gfx950.
//
// The cache keeps s sink slots and an r-slot rolling buffer: token p goes to
// slot p when p < s, else to slot s + (p mod r), overwriting the oldest recent
// token (eq:attn-fixed-rolling and eq:attn-fixed-streaming on the t6page page
// "滑窗与固定稀疏").  When one call brings more than r recent tokens, several
// of them map to the same slot; only the last survives a token-by-token
// append, so only the tokens p >= pos0 + n - r (and the sinks) are copied and
// every slot has exactly one writer.
#include "swa_internal.h"

namespace swa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int64_t n_sink, int64_t n_keep,
                                                     int64_t total) {
    const int64_t chunks = (int64_t)a.d * a.elem_bytes / 16;       // 16-byte chunks per row
    const int64_t per_head = (n_sink + n_keep) * chunks;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bh = idx / per_head;
        const int64_t rem = idx - bh * per_head;
        const int64_t ti = rem / chunks, c = rem - ti * chunks;
        const int64_t p = ti < n_sink ? a.pos0 + ti : a.first + (ti - n_sink);
        const int64_t slot = p < a.s ? p : a.s + p % a.r;
        const int64_t src = ((bh * a.n) + (p - a.pos0)) * chunks + c;
        const int64_t dst = ((bh * (a.s + a.r)) + slot) * chunks + c;
        // the new tokens are read once: non-temporal, so they do not displace
        // cache lines that are read again
        ((u32x4*)a.kc)[dst] = __builtin_nontemporal_load((const u32x4*)a.kn + src);
        ((u32x4*)a.vc)[dst] = __builtin_nontemporal_load((const u32x4*)a.vn + src);
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
    // sinks of this call: positions [pos0, min(pos0 + n, s))
    const int64_t sink_end = a.pos0 + a.n < a.s ? a.pos0 + a.n : (int64_t)a.s;
    const int64_t n_sink = sink_end > a.pos0 ? sink_end - a.pos0 : 0;
    // recent tokens that survive: [first, pos0 + n)
    const int64_t n_keep = a.pos0 + a.n - a.first;
    const int64_t chunks = (int64_t)a.d * a.elem_bytes / 16;
    const int64_t total = (int64_t)a.B * a.Hkv * (n_sink + n_keep) * chunks;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, n_sink, n_keep, total);
    return hipGetLastError();
}

}  // namespace swa
